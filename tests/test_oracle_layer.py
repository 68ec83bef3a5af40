"""Pins for the oracle's transformer-layer stages (attention, LayerNorm, GELU)
and the chained sequence-parallel layer.  Each is checked against something
other than itself:

  * attention: closed forms (zero queries give the running mean of the
    values; one row gives that row's value; two keys whose scaled scores
    differ by exactly 1 weight the second by the logistic function at 1),
    the argmax limit, and invariants (causality, shifting every key by one
    vector, head independence, outputs inside the values' range);
  * LayerNorm: a hand-derived row ([1, 2, 3, 4] -> (x - 5/2) / sqrt(5/4),
    that is +-3/sqrt(5) and +-1/sqrt(5), which fixes the population
    variance), constant rows, alternating rows, the affine map, and the
    shift/scale invariance and unit second moment of the normalised row;
  * GELU: the textbook value Phi(1) = 0.8413447460685429 of the standard
    normal distribution, gelu(x) - gelu(-x) = x, and the limits;
  * the layer: the sharded chain equals the same layer computed without
    tensor parallelism (full weights, every head at once), and a sample of
    tokens equals the same rows of the whole computation;
  * planted mistakes in the C source and in the Python chain must fail a pin.
"""
import math
import os
import subprocess
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from collective_matmul_decomposition_amd import inputs as gen


def bits(a):
    return gen.f32_to_bf16_bits(np.asarray(a, np.float32))


def vals(b):
    return gen.bf16_bits_to_f32(b).astype(np.float64)


def qkv_array(q, k, v):
    """[N, T, heads, D] arrays of small exact values -> qkv bits [N, T, 3*heads*D]."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    N, T, H, D = q.shape
    return bits(np.concatenate([a.reshape(N, T, H * D) for a in (q, k, v)], axis=2)), H


# ------------------------------------------------------------------ attention
def check_attn_zero_queries(lib):
    # every score is 0, so every weight is equal: the output is the mean of
    # the visible values (rows 0..t when causal, all rows otherwise)
    rng = np.random.default_rng(1)
    N, T, H, D = 2, 9, 3, 5
    v = rng.integers(-8, 9, (N, T, H, D))
    k = rng.integers(-3, 4, (N, T, H, D))
    qkv, heads = qkv_array(np.zeros((N, T, H, D)), k, v)
    for causal in (True, False):
        out = oracle.attention(qkv, heads, causal=causal, lib=lib).reshape(N, T, H, D)
        for r, t, h, d in np.ndindex(N, T, H, D):
            rows = range(t + 1) if causal else range(T)
            exact = Fraction(int(sum(v[r, j, h, d] for j in rows)), len(rows))
            assert abs(out[r, t, h, d] - float(exact)) <= 1e-12 * (1 + abs(float(exact)))


def check_attn_single_row(lib):
    rng = np.random.default_rng(2)
    q, k, v = (rng.integers(-3, 4, (3, 1, 2, 8)) for _ in range(3))
    qkv, heads = qkv_array(q, k, v)
    for causal in (True, False):
        out = oracle.attention(qkv, heads, causal=causal, lib=lib).reshape(3, 1, 2, 8)
        assert np.array_equal(out, v.astype(np.float64))


def check_attn_two_keys(lib):
    # D = 4, so the scale is 1/2; q . k1 = 2 and q . k0 = 0 make the scaled
    # scores 1 and 0: the weights are 1/(1+e) and e/(1+e) = logistic(1).
    logistic1 = 0.7310585786300049
    q = np.zeros((1, 2, 1, 4)); k = np.zeros((1, 2, 1, 4)); v = np.zeros((1, 2, 1, 4))
    q[0, 1, 0] = [1, 1, 0, 0]
    k[0, 1, 0] = [1, 1, 0, 0]
    v[0, 0, 0] = [0, 4, -2, 1]
    v[0, 1, 0] = [1, 0, 2, 1]
    qkv, heads = qkv_array(q, k, v)
    for causal in (True, False):
        out = oracle.attention(qkv, heads, causal=causal, lib=lib)[0, :, :]
        want1 = (1 - logistic1) * v[0, 0, 0] + logistic1 * v[0, 1, 0]
        assert np.allclose(out[1], want1, rtol=0, atol=1e-14)
    # causal row 0 sees only key 0
    out = oracle.attention(qkv, heads, causal=True, lib=lib)[0]
    assert np.array_equal(out[0], v[0, 0, 0])


def check_attn_argmax_limit(lib):
    # one key per query scores 64 above the others: the output is that key's
    # value up to exp(-64 / sqrt(D)) relative
    rng = np.random.default_rng(3)
    T, D = 6, 16
    target = rng.integers(0, T, T)
    q = np.zeros((1, T, 1, D)); k = np.zeros((1, T, 1, D))
    v = rng.integers(-4, 5, (1, T, 1, D)).astype(np.float64)
    for j in range(T):
        k[0, j, 0, j] = 16
    for t in range(T):
        q[0, t, 0, target[t]] = 16  # q.k = 256 for the target key, 0 otherwise
    qkv, heads = qkv_array(q, k, v)
    out = oracle.attention(qkv, heads, causal=False, lib=lib)[0]
    for t in range(T):
        assert np.allclose(out[t], v[0, target[t], 0], rtol=0, atol=1e-25)


def check_attn_invariants(lib):
    rng = np.random.default_rng(4)
    N, T, H, D = 2, 11, 2, 8
    q, k = (rng.integers(-3, 4, (N, T, H, D)) for _ in range(2))
    v = rng.integers(-5, 6, (N, T, H, D))
    qkv, heads = qkv_array(q, k, v)
    base, mag = oracle.attention(qkv, heads, causal=True, with_mag=True, lib=lib)
    base4 = base.reshape(N, T, H, D)
    # inside the range of the visible values; mag bounds |out|
    for r, t, h in np.ndindex(N, T, H):
        seen = v[r, :t + 1, h]
        assert (base4[r, t, h] >= seen.min(0) - 1e-12).all() and (base4[r, t, h] <= seen.max(0) + 1e-12).all()
    assert (mag >= np.abs(base) - 1e-12).all()
    # causality: later keys and values do not change earlier rows
    t0 = 5
    k2, v2 = k.copy(), v.copy()
    k2[:, t0 + 1:] = rng.integers(-3, 4, k2[:, t0 + 1:].shape)
    v2[:, t0 + 1:] = rng.integers(-5, 6, v2[:, t0 + 1:].shape)
    out2 = oracle.attention(qkv_array(q, k2, v2)[0], heads, causal=True, lib=lib)
    assert np.array_equal(out2[:, :t0 + 1], base[:, :t0 + 1])
    # adding one vector u to every key adds q.u to every score of a query
    u = rng.integers(-2, 3, D)
    out3 = oracle.attention(qkv_array(q, k + u, v)[0], heads, causal=True, lib=lib)
    assert np.allclose(out3, base, rtol=1e-12, atol=1e-12)
    # heads are independent: scrambling head 1 leaves head 0 unchanged
    q4, k4, v4 = q.copy(), k.copy(), v.copy()
    q4[:, :, 1] = rng.integers(-3, 4, q4[:, :, 1].shape)
    v4[:, :, 1] = rng.integers(-3, 4, v4[:, :, 1].shape)
    out4 = oracle.attention(qkv_array(q4, k4, v4)[0], heads, causal=True, lib=lib).reshape(N, T, H, D)
    assert np.array_equal(out4[:, :, 0], base4[:, :, 0])
    # the sampled form agrees with the full form
    ranks, hs, rows = np.array([1, 0, 1]), np.array([0, 1, 1]), np.array([10, 3, 0])
    part = oracle.attention_rows(qkv, heads, ranks, hs, rows, causal=True, lib=lib)
    for s in range(3):
        assert np.array_equal(part[s], base4[ranks[s], rows[s], hs[s]])


# ------------------------------------------------------------------ LayerNorm
def check_ln_hand_row(lib):
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    want = np.array([-3, -1, 1, 3]) / math.sqrt(5)
    assert np.allclose(oracle.layernorm(x, eps=0.0, lib=lib)[0], want, rtol=0, atol=1e-15)
    g = np.full(4, 2.0); b = np.full(4, 1.0)
    assert np.allclose(oracle.layernorm(x, 0.0, g, b, lib=lib)[0], 1 + 2 * want, rtol=0, atol=1e-14)
    # eps enters under the square root: var 5/4 + eps 3/4 = 2
    assert np.allclose(oracle.layernorm(x, eps=0.75, lib=lib)[0], np.array([-1.5, -0.5, 0.5, 1.5]) / math.sqrt(2),
                       rtol=0, atol=1e-15)


def check_ln_special_rows(lib):
    x = np.full((3, 16), 7.25)
    assert np.array_equal(oracle.layernorm(x, 1e-5, lib=lib), np.zeros_like(x))
    a = 3.0
    alt = np.tile([a, -a], (2, 8))
    y = oracle.layernorm(alt, 1e-5, lib=lib)
    assert np.allclose(y, alt / math.sqrt(a * a + 1e-5), rtol=1e-15, atol=0)


def check_ln_invariants(lib):
    x = gen.layernorm_inputs(6, 512, seed=3).astype(np.float64)
    y = oracle.layernorm(x, 0.0, lib=lib)
    assert np.allclose(y.mean(1), 0, atol=1e-12)
    assert np.allclose((y * y).mean(1), 1, atol=1e-12)
    y2 = oracle.layernorm(2.5 * x - 3.0, 0.0, lib=lib)
    assert np.allclose(y2, y, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ GELU
def check_gelu(lib):
    phi1 = 0.8413447460685429  # standard normal CDF at 1
    y = oracle.gelu(np.array([0.0, 1.0, -1.0, 10.0, -10.0]), lib=lib)
    assert y[0] == 0.0
    assert abs(y[1] - phi1) < 1e-15 and abs(y[2] + (1 - phi1)) < 1e-15
    assert y[3] == 10.0 and -1e-20 < y[4] <= 0.0
    x = np.random.default_rng(5).standard_normal(1000) * 3
    assert np.allclose(oracle.gelu(x, lib=lib) - oracle.gelu(-x, lib=lib), x, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ the layer
def dense_layer(x, wqkv, wo, w1, w2, heads, eps, lib):
    """The same layer without tensor parallelism: the full weights (every
    rank's slice put back in place) applied to the whole sequence at once."""
    N, m, d = x.shape
    HD = wqkv.shape[1] // 3
    X = vals(x).reshape(N * m, d)
    # global heads r*heads + h: query, key and value blocks of all ranks side by side
    Wq = np.concatenate([vals(wqkv[r, :HD]) for r in range(N)])
    Wk = np.concatenate([vals(wqkv[r, HD:2 * HD]) for r in range(N)])
    Wv = np.concatenate([vals(wqkv[r, 2 * HD:]) for r in range(N)])
    qkv = oracle.round_bf16(X @ np.concatenate([Wq, Wk, Wv]).T, lib)[None]
    A = vals(oracle.round_bf16(oracle.attention(qkv, N * heads, causal=True, lib=lib)[0], lib))
    Wo = np.concatenate([vals(wo[r]) for r in range(N)], axis=1)  # [d, N*HD]
    L = vals(oracle.round_bf16(oracle.layernorm(A @ Wo.T, eps, lib=lib), lib))
    W1 = np.concatenate([vals(w1[r]) for r in range(N)])  # [f, d]
    F = vals(oracle.round_bf16(oracle.gelu(L @ W1.T, lib), lib))
    W2 = np.concatenate([vals(w2[r]) for r in range(N)], axis=1)  # [d, f]
    return F @ W2.T


def layer_case(seed=0):
    N, m, d, heads, D, fN = 3, 5, 64, 2, 8, 24
    return gen.layer_inputs(N, m, d, heads, D, fN, "normal", seed), heads


def check_layer_dense_equivalence(lib, mod=oracle):
    (x, wqkv, wo, w1, w2), heads = layer_case()
    N, m, d = x.shape
    res = mod.sp_layer_rows(x, wqkv, wo, w1, w2, heads, np.arange(N * m), 1e-5, lib=lib)
    want = dense_layer(x, wqkv, wo, w1, w2, heads, 1e-5, oracle.load())
    assert np.allclose(res["out"], want, rtol=1e-9, atol=1e-9)


def check_layer_sampled_rows(lib, mod=oracle):
    (x, wqkv, wo, w1, w2), heads = layer_case(1)
    N, m, d = x.shape
    full = mod.sp_layer_rows(x, wqkv, wo, w1, w2, heads, np.arange(N * m), 1e-5, lib=lib)
    tok = np.array([7, 0, 13, 2])
    part = mod.sp_layer_rows(x, wqkv, wo, w1, w2, heads, tok, 1e-5, lib=lib)
    for key in ("out", "mag", "proj", "ln"):
        assert np.allclose(part[key], full[key][tok], rtol=1e-12, atol=1e-12), key
    assert np.allclose(part["fc1"], full["fc1"][:, tok], rtol=1e-12, atol=1e-12)


LIB_CHECKS = [check_attn_zero_queries, check_attn_single_row, check_attn_two_keys, check_attn_argmax_limit,
              check_attn_invariants, check_ln_hand_row, check_ln_special_rows, check_ln_invariants, check_gelu,
              check_layer_dense_equivalence, check_layer_sampled_rows]


@pytest.mark.parametrize("check", LIB_CHECKS, ids=lambda c: c.__name__)
def test_layer_oracle_pin(check):
    check(oracle.load())


def test_layer_generators_seeded():
    a = gen.layer_inputs(2, 4, 64, 1, 8, 16, "normal", 0)
    b = gen.layer_inputs(2, 4, 64, 1, 8, 16, "normal", 0)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    assert [t.shape for t in a] == [(2, 4, 64), (2, 24, 64), (2, 64, 8), (2, 16, 64), (2, 64, 16)]
    assert np.array_equal(gen.attention_inputs(1, 4, 2, 8, seed=1), gen.attention_inputs(1, 4, 2, 8, seed=1))
    x = gen.layernorm_inputs(4, 64)
    assert x.dtype == np.float32 and x.shape == (4, 64)


# ------------------------------------------------------------ planted mistakes
C_MUTANTS = {
    "attn_scale_1_over_d": ("const double scale = 1.0 / sqrt((double)D);", "const double scale = 1.0 / (double)D;"),
    "attn_causal_off_by_one": ("const int nk = causal ? i + 1 : T;", "const int nk = causal ? i : T;"),
    "attn_values_from_keys": ("bf16_value(base[(size_t)j * ld + (size_t)2 * H * D", "bf16_value(base[(size_t)j * ld + (size_t)H * D"),
    "attn_wrong_head": ("const uint16_t *q = base + (size_t)i * ld + (size_t)h * D;", "const uint16_t *q = base + (size_t)i * ld;"),
    "ln_sample_variance": ("sqrt(ss / cols + eps)", "sqrt(ss / (cols - 1) + eps)"),
    "ln_eps_outside": ("sqrt(ss / cols + eps)", "(sqrt(ss / cols) + eps)"),
    "gelu_no_sqrt2": ("erf(x[t] / sqrt(2.0))", "erf(x[t])"),
    "gelu_no_half": ("y[t] = 0.5 * x[t] *", "y[t] = x[t] *"),
}


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_layer_planted_mistake_is_caught(name, tmp_path):
    src = open(obuild.SRC).read()
    old, new = C_MUTANTS[name]
    assert src.count(old) == 1, "mutation site moved; update the planted-mistake table"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", *obuild.CFLAGS, str(mutated), "-o", so, "-lm"], check=True)
    lib = oracle.load(so)
    failed = []
    for check in LIB_CHECKS:
        try:
            check(lib)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "planted mistake %r passed every pin" % name


PY_MUTANTS = {
    "proj_drops_a_rank": ("    for r in range(N):\n        proj += attn_b[r]", "    for r in range(N - 1):\n        proj += attn_b[r]"),
    "ln_not_rounded": ("ln = bf16_to_f64(round_bf16(layernorm(proj, eps, lib=lib), lib))", "ln = layernorm(proj, eps, lib=lib)"),
    "no_activation": ("round_bf16(gelu(ln @ bf16_to_f64(w1[r]).T, lib), lib)", "round_bf16(ln @ bf16_to_f64(w1[r]).T, lib)"),
    "keys_of_sampled_rows_only": ("qkv[r] = round_bf16(xf[:rows_needed]", "qkv[r] = round_bf16(xf[:rows_needed][::-1]"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_layer_chain_planted_mistake_is_caught(name):
    path = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
    src = open(path).read()
    old, new = PY_MUTANTS[name]
    assert src.count(old) == 1, "mutation site moved; update the planted-mistake table"
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    lib = oracle.load()
    failed = []
    for check in (check_layer_dense_equivalence, check_layer_sampled_rows):
        try:
            check(lib, mod)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "planted mistake %r passed every pin" % name
