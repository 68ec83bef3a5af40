"""Pins for the CPU oracle: it is checked against things other than itself.

  * a hand-computed two-rank fixture (tests/golden/hand_n2.json);
  * brute force in exact Python integers / fractions on tiny shapes;
  * the N = 1 special case against numpy's float64 matmul (a library routine);
  * closed forms: all-ones, permutation weights (catch transposed operands),
    identity weights (catch concatenation order), rank-tagged rows (catch
    bucket offsets and dropped ranks);
  * the AllReduce = ReduceScatter then AllGather invariant ("Tensor
    Parallelism > Communication Patterns");
  * bf16 rounding: hand-derived ties, subnormals and overflow, plus agreement
    with the input generator's independent bias-method rounding;
  * planted mistakes: mutated copies of the oracle source must fail a pin.
"""
import itertools
import json
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from collective_matmul_decomposition_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(a):
    """Small exact values -> bf16 bit patterns (via the generator's rounding)."""
    return gen.f32_to_bf16_bits(np.asarray(a, np.float32))


def vals(b):
    return gen.bf16_bits_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------- pin checks
# Each check takes the loaded oracle library so the planted-mistake test can
# run the same checks against mutated builds.

def check_golden(lib):
    g = json.load(open(os.path.join(GOLDEN, "hand_n2.json")))
    y = oracle.ag_gemm(bits(g["ag"]["x"]), bits(g["ag"]["w"]), lib=lib)
    assert np.array_equal(y, np.array(g["ag"]["y"], np.float64))
    out = oracle.gemm_rs(bits(g["rs"]["h"]), bits(g["rs"]["w"]), lib=lib)
    assert np.array_equal(out, np.array(g["rs"]["out"], np.float64))
    ar = oracle.allreduce(bits(g["rs"]["h"]), bits(g["rs"]["w"]), lib=lib)
    assert np.array_equal(ar, np.array(g["rs"]["allreduce"], np.float64))


def _brute_ag(x, w):
    """Exact AllGather -> GEMM with Python ints: gather the shard lists, multiply."""
    N = len(x)
    gathered = [row for shard in x for row in shard]
    return [[[sum(a * b for a, b in zip(row, wrow)) for wrow in w[r]] for row in gathered] for r in range(N)]


def _brute_rs(h, w):
    """Exact GEMM -> ReduceScatter with Python ints: full partials, then sum each bucket."""
    N = len(h)
    T = len(h[0])
    m = T // N
    partial = [[[sum(a * b for a, b in zip(row, wrow)) for wrow in w[r]] for row in h[r]] for r in range(N)]
    return [[[sum(partial[r][q * m + i][j] for r in range(N)) for j in range(len(w[0]))]
             for i in range(m)] for q in range(N)]


def check_brute_force(lib):
    rng = np.random.default_rng(12345)
    for N, m, k, n in itertools.product((1, 2, 3, 5), (1, 2, 3), (1, 3, 5), (1, 2, 5)):
        xi = rng.integers(-3, 4, size=(N, m, k))
        wi = rng.integers(-3, 4, size=(N, n, k))
        hi = rng.integers(-3, 4, size=(N, N * m, k))
        y = oracle.ag_gemm(bits(xi), bits(wi), lib=lib)
        assert np.array_equal(y, np.array(_brute_ag(xi.tolist(), wi.tolist()), np.float64)), (N, m, k, n)
        out = oracle.gemm_rs(bits(hi), bits(wi), lib=lib)
        assert np.array_equal(out, np.array(_brute_rs(hi.tolist(), wi.tolist()), np.float64)), (N, m, k, n)


def check_brute_force_fractions(lib):
    """Float (bf16 N(0,1)) inputs: exact rational result vs the fp64 oracle."""
    for N, m, k, n in ((2, 2, 7, 3), (3, 1, 9, 2)):
        x, w = gen.ag_inputs(N, m, k, n, "normal", seed=3)
        h, _ = gen.rs_inputs(N, m, k, n, "normal", seed=3)
        xf = [[[Fraction(float(v)) for v in row] for row in s] for s in vals(x)]
        wf = [[[Fraction(float(v)) for v in row] for row in s] for s in vals(w)]
        hf = [[[Fraction(float(v)) for v in row] for row in s] for s in vals(h)]
        y, ymag = oracle.ag_gemm(x, w, with_mag=True, lib=lib)
        exact = np.array(_brute_ag(xf, wf), dtype=object)
        err = np.abs(y - exact.astype(np.float64))
        assert (err <= 4 * k * 2.0 ** -53 * ymag).all()
        out, omag = oracle.gemm_rs(h, w, with_mag=True, lib=lib)
        exact = np.array(_brute_rs(hf, wf), dtype=object)
        err = np.abs(out - exact.astype(np.float64))
        assert (err <= 4 * (N * k) * 2.0 ** -53 * omag).all()


def check_n1_matmul(lib):
    """N = 1: AllGather is the identity and ReduceScatter a no-op -> plain GEMM."""
    x, w = gen.ag_inputs(1, 37, 64, 29, "normal", seed=1)
    y, mag = oracle.ag_gemm(x, w, with_mag=True, lib=lib)
    ref = vals(x)[0] @ vals(w)[0].T
    assert np.all(np.abs(y[0] - ref) <= 1e-13 * mag[0])
    h, w = gen.rs_inputs(1, 21, 48, 33, "normal", seed=2)
    out, mag = oracle.gemm_rs(h, w, with_mag=True, lib=lib)
    ref = vals(h)[0] @ vals(w)[0].T
    assert np.all(np.abs(out[0] - ref) <= 1e-13 * mag[0])


def check_closed_forms(lib):
    # all ones: every output of AG is k, every output of RS is N*k
    N, m, k, n = 3, 2, 5, 4
    one = bits(np.ones(1))[0]
    y = oracle.ag_gemm(np.full((N, m, k), one, np.uint16), np.full((N, n, k), one, np.uint16), lib=lib)
    assert np.array_equal(y, np.full((N, N * m, n), float(k)))
    out = oracle.gemm_rs(np.full((N, N * m, k), one, np.uint16), np.full((N, n, k), one, np.uint16), lib=lib)
    assert np.array_equal(out, np.full((N, m, n), float(N * k)))

    # permutation weights: Y_r[i, j] = Xfull[i, perm_r[j]]  (W_r row j = e_{perm_r[j]})
    N, m, k = 4, 3, 6
    rng = np.random.default_rng(7)
    x = rng.integers(-3, 4, size=(N, m, k))
    perms = [rng.permutation(k) for _ in range(N)]
    w = np.zeros((N, k, k))
    for r in range(N):
        w[r, np.arange(k), perms[r]] = 1
    y = oracle.ag_gemm(bits(x), bits(w), lib=lib)
    xfull = x.reshape(N * m, k)
    for r in range(N):
        assert np.array_equal(y[r], xfull[:, perms[r]].astype(np.float64))

    # identity weights, rank-tagged activation rows: value(r, t, c) = 100*r + 10*t + c
    N, m = 3, 2
    T, k = N * m, 4
    h = np.array([[[100 * r + 10 * t + c for c in range(k)] for t in range(T)] for r in range(N)])
    eye = np.stack([np.eye(k)] * N)
    out = oracle.gemm_rs(bits(h), bits(eye), lib=lib)
    for q in range(N):
        expect = h[:, q * m:(q + 1) * m, :].sum(axis=0)  # sum over ranks of bucket q's rows
        assert np.array_equal(out[q], expect.astype(np.float64))
    # and AG with identity weights returns the concatenation, in rank order
    x = h[:, :m, :]
    y = oracle.ag_gemm(bits(x), bits(eye), lib=lib)
    for r in range(N):
        assert np.array_equal(y[r], np.concatenate(list(x), axis=0).astype(np.float64))


def check_allreduce_invariant(lib):
    """AllReduce == ReduceScatter followed by AllGather (concatenate the owners' rows)."""
    N, m, k, n = 4, 5, 24, 7
    h, w = gen.rs_inputs(N, m, k, n, "normal", seed=4)
    out, mag = oracle.gemm_rs(h, w, with_mag=True, lib=lib)
    ar = oracle.allreduce(h, w, lib=lib)
    assert np.array_equal(np.concatenate(list(out), axis=0), ar)
    ref = sum(vals(h)[r] @ vals(w)[r].T for r in range(N))
    assert np.all(np.abs(ar - ref) <= 1e-13 * np.concatenate(list(mag), axis=0))


def check_sampled_rows(lib):
    N, m, k, n = 3, 4, 16, 6
    x, w = gen.ag_inputs(N, m, k, n, "normal", seed=5)
    y, ymag = oracle.ag_gemm(x, w, with_mag=True, lib=lib)
    ranks, rows = np.array([0, 2, 1, 2]), np.array([11, 0, 5, 7])
    ys, ysm = oracle.ag_gemm_rows(x, w, ranks, rows, with_mag=True, lib=lib)
    assert np.array_equal(ys, y[ranks, rows]) and np.array_equal(ysm, ymag[ranks, rows])
    h, w = gen.rs_inputs(N, m, k, n, "normal", seed=5)
    out, omag = oracle.gemm_rs(h, w, with_mag=True, lib=lib)
    owners, rows = np.array([2, 0, 1]), np.array([3, 0, 2])
    os_, osm = oracle.gemm_rs_rows(h, w, owners, rows, with_mag=True, lib=lib)
    assert np.array_equal(os_, out[owners, rows]) and np.array_equal(osm, omag[owners, rows])


def check_round_bf16(lib):
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),                # tie between 1 and 1+2^-7: even (1)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),            # tie between 1+2^-7 and 1+2^-6: even
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),   # just above the tie
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (255.0 * 2.0 ** 120, 0x7F7F),             # largest finite bf16
        (2.0 ** 128 - 2.0 ** 119, 0x7F80),        # halfway past it: ties to even -> overflow
        (-(2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100), 0xFF7F),
        (2.0 ** -133, 0x0001),                    # smallest subnormal
        (2.0 ** -134, 0x0000),                    # tie between 0 and 2^-133: even (0)
        (3 * 2.0 ** -134, 0x0002),                # tie between 2^-133 and 2^-132: even
        (2.0 ** -126, 0x0080),                    # smallest normal
        (1e-50, 0x0000),
    ]
    got = oracle.round_bf16(np.array([c[0] for c in cases]), lib=lib)
    for (v, expect), g in zip(cases, got):
        assert int(g) == expect, (v, hex(int(g)), hex(expect))
    # agreement with the generator's independent bias-method rounding on finite float32s
    rng = np.random.default_rng(11)
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.integers(-2 ** 20, 2 ** 20, 5000).astype(np.float32) / 7.0])
    f = f[np.isfinite(f)].astype(np.float32)
    assert np.array_equal(oracle.round_bf16(f.astype(np.float64), lib=lib), gen.f32_to_bf16_bits(f))


def check_bf16_bucket_golden(lib):
    g = json.load(open(os.path.join(GOLDEN, "bf16_bucket_n3.json")))
    h, w = bits(g["h"]), bits(g["w"])
    for dir, key in (("uni", "out_uni"), ("bi", "out_bi")):
        out = oracle.gemm_rs_bf16_bucket(h, w, dir=dir, lib=lib)
        assert np.array_equal(out, np.array(g[key], np.float64)), (dir, out)
    assert np.array_equal(oracle.gemm_rs(h, w, lib=lib), np.array(g["out_fp32_bucket"], np.float64))


def _brute_bf16_bucket(h, w, dir):
    """Python-integer partials; the bucket rounded after every addition with the
    input generator's float32 -> bf16 rounding (exact here: small integers)."""
    N = len(h)
    m = len(h[0]) // N
    n = len(w[0])
    L, R = -(-(N - 1) // 2), (N - 1) // 2

    def z(r, q, i):
        return [sum(a * b for a, b in zip(h[r][q * m + i], w[r][j])) for j in range(n)]

    def rnd(v):
        return [int(x) for x in vals(gen.f32_to_bf16_bits(np.asarray(v, np.float32)))]

    out = []
    for q in range(N):
        rows = []
        for i in range(m):
            if dir == "uni":
                chains = [[(q + t) % N for t in range(1, N)]]
            else:
                chains = [[(q - L + t) % N for t in range(L)], [(q + R - t) % N for t in range(R)]]
            total = z(q, q, i)
            for chain in chains:
                b = [0] * n
                for r in chain:
                    b = rnd([x + y for x, y in zip(b, z(r, q, i))])
                total = [x + y for x, y in zip(total, b)]
            rows.append(total)
        out.append(rows)
    return out


def check_bf16_bucket_brute_force(lib):
    rng = np.random.default_rng(11)
    # values large enough that almost every bucket addition rounds
    for N, m, k, n in ((2, 1, 3, 2), (3, 2, 2, 3), (4, 1, 4, 2), (5, 2, 3, 2), (6, 1, 2, 3), (7, 1, 2, 4)):
        hv = rng.integers(-60, 61, (N, N * m, k))
        wv = rng.integers(-60, 61, (N, n, k))
        for dir in ("uni", "bi"):
            want = np.array(_brute_bf16_bucket(hv.tolist(), wv.tolist(), dir), np.float64)
            got = oracle.gemm_rs_bf16_bucket(bits(hv), bits(wv), dir=dir, lib=lib)
            assert np.array_equal(got, want), (N, m, k, n, dir)


def check_bf16_bucket_reductions(lib):
    """Where no rounding can act, the bf16 bucket is the fp32 definition: one
    rank (no hops), and integer data whose partial sums stay within +-256."""
    h, w = gen.rs_inputs(1, 4, 64, 8, "normal", 2)
    assert np.array_equal(oracle.gemm_rs_bf16_bucket(h, w, lib=lib), oracle.gemm_rs(h, w, lib=lib))
    rng = np.random.default_rng(5)
    for N in (2, 3, 4, 7):
        hv = rng.integers(-2, 3, (N, N * 2, 4))
        wv = rng.integers(-2, 3, (N, 5, 4))
        ref = oracle.gemm_rs(bits(hv), bits(wv), lib=lib)
        for dir in ("uni", "bi"):
            assert np.array_equal(oracle.gemm_rs_bf16_bucket(bits(hv), bits(wv), dir=dir, lib=lib), ref)


ALL_CHECKS = [check_golden, check_brute_force, check_brute_force_fractions, check_n1_matmul,
              check_closed_forms, check_allreduce_invariant, check_sampled_rows, check_round_bf16,
              check_bf16_bucket_golden, check_bf16_bucket_brute_force, check_bf16_bucket_reductions]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.load())


def test_generator_is_seeded_and_in_range():
    a = gen.ag_inputs(2, 3, 8, 4, "int", seed=0)
    b = gen.ag_inputs(2, 3, 8, 4, "int", seed=0)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    v = vals(a[0])
    assert set(np.unique(v)).issubset(set(range(-3, 4)))
    h, w = gen.rs_inputs(4, 64, 256, 256, "normal", seed=0)
    assert abs(vals(h).std() - 1.0) < 0.02 and abs(vals(w).std() - 0.02) < 0.001


# ------------------------------------------------------------ planted mistakes
MUTANTS = {
    "transposed_weight": ("acc += bf16_value(a[kk]) * bf16_value(wj[kk]);",
                          "acc += bf16_value(a[kk]) * bf16_value(w[(size_t)kk * n + j]);"),
    "dropped_rank": ("for (int r = 0; r < N; ++r) {\n    const uint16_t *hrow",
                     "for (int r = 0; r < N - 1; ++r) {\n    const uint16_t *hrow"),
    "wrong_bucket_row": ("(size_t)q * m + i) * k;", "(size_t)i * N + q) * k;"),
    "wrong_sign": ("out[j] += zrow[j];", "out[j] -= zrow[j];"),
    "reversed_shard_rows": ("int local = i % m;", "int local = m - 1 - i % m;"),
    "dropped_last_term": ("for (int kk = 0; kk < k; ++kk) acc +=", "for (int kk = 0; kk < k - 1; ++kk) acc +="),
    "round_ties_away": ("nearbyint(a / quantum)", "round(a / quantum)"),
    "bucket_unrounded": ("b[j] = bf16_round(b[j] + z[j]);", "b[j] = b[j] + z[j];"),
    "bucket_owner_first": ("if (!dir) { first = q + 1; len = N - 1; step = 1; }",
                           "if (!dir) { first = q; len = N - 1; step = 1; }"),
    "bucket_final_rounded": ("o[j] = z[j] + b0[j] + b1[j];", "o[j] = bf16_round(z[j] + b0[j] + b1[j]);"),
    "bucket_ccw_wrong_way": ("else { first = q + R; len = R; step = -1; }", "else { first = q + 1; len = R; step = 1; }"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(obuild.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation site moved; update the planted-mistake table"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", *obuild.CFLAGS, str(mutated), "-o", so, "-lm"], check=True)
    lib = oracle.load(so)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(lib)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "planted mistake %r passed every pin" % name
