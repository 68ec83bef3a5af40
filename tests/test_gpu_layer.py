"""GPU parity of the layer around the collective matmuls, through the C ABI,
against the CPU oracle.

Bars (each derived from the arithmetic the kernel does):
  (bf16 holds 8 significant bits: rounding to nearest moves a value by at
  most u = 2^-8 of its magnitude.)
  * attention: the kernel computes the scores in fp32 from bf16 operands
    (|error| <= 1e-5 * sum_d |q_d k_d| / sqrt(D), the matmul bound, which
    moves a probability by the same relative amount), rounds every
    probability to bf16 (relative u) and uses the same rounded values in the
    weighted sum and the normaliser, so each normalised weight carries a
    relative error of at most 2 eps / (1 - eps), eps = u + e_s; the fp32
    accumulation over up to 4096 keys (256 MFMA steps) and the block
    rescalings add at most 3e-5 of M; hence
        |o - ref| <= (1.01 * 2^-7 + 2.1e-5 * Sqk + 3e-5) * M + 1.01 * 2^-8 |ref|
    with M = sum_j p_j |v_j| / sum_j p_j (from the oracle) and Sqk the largest
    sum_d |q_d k_jd| / sqrt(D) of the row, and the last term the output's
    rounding to bf16;
  * LayerNorm: fp32 statistics (relative error below 1e-6 for these rows)
    and the rounding of the output to bf16:
        |y - ref| <= 1.01 * 2^-8 |ref| + 1e-5 (1 + |beta| + |gamma| (|yn| + mean|x| / std))
  * GELU epilogue: GELU is 1.13-Lipschitz, so the matmul bound carries over
    with that factor, plus fp32 erf (1e-6 |x|) and the bf16 rounding:
        |y - gelu(ref)| <= 1.13e-5 * S + 1e-6 |pre| (+ 2^-8 |gelu(ref)| for bf16)
  * the chained layer: its first stage (the QKV projection) to the matmul
    bound plus one bf16 spacing (both sides round their own values), and the
    output to a composed tolerance (see test_layer_chain): every later stage
    starts from bf16 values that may differ from the oracle's by one
    spacing, which the stage tests above do not cover.
"""
import sys

import numpy as np
import pytest

import oracle
from collective_matmul_decomposition_amd import _native as nat
from collective_matmul_decomposition_amd import buffers
from collective_matmul_decomposition_amd import inputs as gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
D = 128


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nat.lib()
    yield


def vals(bits):
    return gen.bf16_bits_to_f32(bits).astype(np.float64)


def score_mag(qkv_v, heads, r, h, t, causal):
    """max_j sum_d |q_td k_jd| / sqrt(D) over the keys query t sees."""
    HD = heads * D
    q = np.abs(qkv_v[r, t, h * D:(h + 1) * D])
    nk = t + 1 if causal else qkv_v.shape[1]
    k = np.abs(qkv_v[r, :nk, HD + h * D:HD + (h + 1) * D])
    return (k @ q).max() / np.sqrt(D)


def attn_bound(qkv_bits, heads, causal, ranks, hs, rows, ref, mag):
    qv = vals(qkv_bits)
    sqk = np.array([score_mag(qv, heads, r, h, t, causal) for r, h, t in zip(ranks, hs, rows)])[:, None]
    return (1.01 * 2.0 ** -7 + 2.1e-5 * sqk + 3e-5) * mag + 1.01 * 2.0 ** -8 * np.abs(ref) + 1e-30


def run_attention(qkv_t, N, T, heads, causal):
    o = torch.full((N, T, heads * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    say("  attention N=%d T=%d heads=%d causal=%d" % (N, T, heads, causal))
    nat.cm_attention(qkv_t, o, N, T, heads, D, causal)
    torch.cuda.synchronize()
    return o


ATTN = [(1, 1, 1, True), (2, 17, 2, True), (1, 128, 1, True), (2, 200, 3, True), (1, 300, 2, False),
        (3, 64, 1, False), (1, 513, 2, True), (2, 130, 1, False), (1, 256, 1, True), (1, 384, 2, False),
        (1, 640, 1, True)]


@pytest.mark.parametrize("N,T,heads,causal", ATTN)
def test_attention_parity(N, T, heads, causal):
    say("attention", N, T, heads, causal)
    qkv = gen.attention_inputs(N, T, heads, D, seed=T)
    o = run_attention(gen.to_torch_bf16(qkv, "cuda"), N, T, heads, causal)
    got = vals(gen.torch_bf16_to_bits(o))
    ref, mag = oracle.attention(qkv, heads, causal, with_mag=True)
    rr, tt, hh = np.meshgrid(np.arange(N), np.arange(T), np.arange(heads), indexing="ij")
    bound = attn_bound(qkv, heads, causal, rr.ravel(), hh.ravel(), tt.ravel(), ref.reshape(-1, D),
                       mag.reshape(-1, D)).reshape(ref.shape)
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert (err <= bound).all(), "worst err/bound %g" % (err / bound).max()


def test_attention_closed_forms():
    # zero queries: every visible key has the same weight, the output is the
    # running mean of the values (integers, so the mean is the oracle's exactly)
    N, T, heads = 1, 150, 2
    rng = np.random.default_rng(7)
    q = np.zeros((N, T, heads * D))
    k = rng.integers(-3, 4, (N, T, heads * D))
    v = rng.integers(-3, 4, (N, T, heads * D))
    qkv = gen.f32_to_bf16_bits(np.concatenate([q, k, v], axis=2).astype(np.float32))
    o = run_attention(gen.to_torch_bf16(qkv, "cuda"), N, T, heads, True)
    got = vals(gen.torch_bf16_to_bits(o))
    want = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    # equal weights are exactly representable: only the final rounding to bf16
    assert (np.abs(got - want) <= 2.0 ** -8 * np.abs(want) * 1.0001 + 1e-30).all()


def test_attention_repeatable():
    qkv = gen.attention_inputs(2, 257, 2, D, seed=11)
    t = gen.to_torch_bf16(qkv, "cuda")
    a = run_attention(t, 2, 257, 2, True).clone()
    b = run_attention(t, 2, 257, 2, True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_full_size_sampled():
    # the layer's attention: 8 ranks x 8 heads, 4096 tokens, head dim 128
    N, T, heads = 8, 4096, 8
    say("attention full size")
    qkv_t = gen.attention_inputs_torch(N, T, heads, D, seed=0)
    o = run_attention(qkv_t, N, T, heads, True)
    qkv = gen.torch_bf16_to_bits(qkv_t)
    got = vals(gen.torch_bf16_to_bits(o))
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 4094, 2048], rng.integers(0, T, 39)])
    ranks = rng.integers(0, N, len(rows))
    hs = rng.integers(0, heads, len(rows))
    ref, mag = oracle.attention_rows(qkv, heads, ranks, hs, rows, True, with_mag=True)
    bound = attn_bound(qkv, heads, True, ranks, hs, rows, ref, mag)
    g = np.stack([got[r, t, h * D:(h + 1) * D] for r, h, t in zip(ranks, hs, rows)])
    err = np.abs(g - ref)
    assert (err <= bound).all(), "worst err/bound %g" % (err / bound).max()


# ------------------------------------------------------------------ LayerNorm
def ln_bound(x, ref, yn, gamma, beta):
    x = x.astype(np.float64)
    std = np.sqrt(x.var(axis=1, keepdims=True) + 1e-5)
    scale = np.abs(x).mean(axis=1, keepdims=True) / std
    g = 1.0 if gamma is None else np.abs(gamma)
    b = 0.0 if beta is None else np.abs(beta)
    return 1.01 * 2.0 ** -8 * np.abs(ref) + 1e-5 * (1 + b + g * (np.abs(yn) + scale))


@pytest.mark.parametrize("rows,cols,affine", [(1, 4, False), (7, 64, True), (33, 1000, False), (256, 4096, True),
                                              (64, 8192, False), (5, 16384, True), (4096, 8192, False)])
def test_layernorm_parity(rows, cols, affine):
    say("layernorm", rows, cols, affine)
    x = gen.layernorm_inputs(rows, cols, seed=cols)
    gamma = beta = None
    if affine:
        rng = np.random.default_rng(cols)
        gamma = rng.standard_normal(cols).astype(np.float32)
        beta = rng.standard_normal(cols).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    y = torch.full((rows, cols), float("nan"), dtype=torch.bfloat16, device="cuda")
    gt = None if gamma is None else torch.from_numpy(gamma).cuda()
    bt = None if beta is None else torch.from_numpy(beta).cuda()
    nat.cm_layernorm(xt, y, rows, cols, 1e-5, gt, bt)
    torch.cuda.synchronize()
    got = vals(gen.torch_bf16_to_bits(y))
    x64 = x.astype(np.float64)
    yn = oracle.layernorm(x64, 1e-5)
    ref = yn if not affine else oracle.layernorm(x64, 1e-5, gamma.astype(np.float64), beta.astype(np.float64))
    bound = ln_bound(x, ref, yn, gamma, beta)
    err = np.abs(got - ref)
    assert (err <= bound).all(), "worst err/bound %g" % (err / bound).max()


# ------------------------------------------------------------ GELU epilogue
GELU = [(4, 64, 256, 256, "uni", 1, "normal", "bf16"), (4, 64, 256, 256, "bi", 2, "int", "f32"),
        (3, 40, 192, 320, "uni", 2, "normal", "f32"), (2, 33, 320, 960, "direct", 1, "normal", "bf16"),
        (4, 64, 256, 256, "uni", 1, "normal", "f32")]


@pytest.mark.parametrize("N,m,k,n,dir,chunks,dist,out", GELU)
@pytest.mark.parametrize("sched", ["decomposed", "naive"])
def test_gelu_epilogue(N, m, k, n, dir, chunks, dist, out, sched):
    say("gelu", N, m, k, n, dir, chunks, dist, out, sched)
    plan = nat.cm_ring_plan(op="ag", n_ranks=N, m=m, k=k, n=n, dir=dir, chunks=chunks, sched=sched, out_dtype=out,
                            n_comm=2, act="gelu")
    a, w = gen.ag_inputs(N, m, k, n, dist, seed=1)
    y, ws = buffers.alloc_outputs(plan)
    buffers.run(plan, gen.to_torch_bf16(a, "cuda"), gen.to_torch_bf16(w, "cuda"), y, ws)
    torch.cuda.synchronize()
    pre, mag = oracle.ag_gemm(a, w, with_mag=True)
    ref = oracle.gelu(pre)
    got = y.float().cpu().numpy().astype(np.float64)
    bound = 1.13e-5 * mag + 1e-6 * np.abs(pre) + (2.0 ** -8 * np.abs(ref) if out == "bf16" else 0) + 1e-30
    err = np.abs(got - ref)
    assert (err <= bound).all(), "worst err/bound %g" % (err / bound).max()


# ------------------------------------------------------------------ the layer
def layer_buffers(N, m, d, heads, ffn, dist="normal", seed=0, device_inputs=False):
    if device_inputs:
        ts = gen.layer_inputs_torch(N, m, d, heads, D, ffn, dist, seed)
        bits = [gen.torch_bf16_to_bits(t) for t in ts]
    else:
        bits = gen.layer_inputs(N, m, d, heads, D, ffn, dist, seed)
        ts = [gen.to_torch_bf16(b, "cuda") for b in bits]
    return bits, ts


def run_layer(plan, ts, N, m, d, out_dtype="f32", repeat=1):
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    comm = buffers.comm_streams(plan.desc.n_comm)
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    outs = []
    for _ in range(repeat):
        out = torch.full((N, m, d), float("nan"), dtype=odt, device="cuda")
        say("  layer forward N=%d m=%d d=%d" % (N, m, d))
        nat.cm_layer_forward(plan, *ts, out, ws, torch.cuda.current_stream(), comm)
        torch.cuda.synchronize()
        outs.append(out)
    return outs, ws


def ws_view(ws, off, shape, dtype):
    n = int(np.prod(shape))
    esz = torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n * esz].view(dtype).view(*shape)


def check_chain(plan, bits, ws, out, tokens, heads, m):
    """Compare the layer at `tokens` with the oracle, element by element at
    every stage boundary, each stage fed with the GPU's own input to it (the
    intermediates the call leaves in the workspace) and held to that stage's
    bound; then the output against the whole chain computed by the oracle."""
    x, wqkv, wo, w1, w2 = bits
    N, _, d = x.shape
    T = N * m
    HD = heads * D
    ffn = w1.shape[1]
    tokens = np.asarray(tokens)
    owners, rows = tokens // m, tokens % m
    stage = {}

    def bits_of(off, shape):
        return gen.torch_bf16_to_bits(ws_view(ws, off, shape, torch.bfloat16))

    qkv_g = bits_of(plan.off_qkv, (N, T, 3 * HD))
    attn_g = bits_of(plan.off_attn, (N, T, HD))
    proj_g = ws_view(ws, plan.off_proj, (N, m, d), torch.float32).cpu().numpy().astype(np.float64)
    ln_g = bits_of(plan.off_ln, (N, m, d))
    fc1_g = bits_of(plan.off_fc1, (N, T, ffn))

    def within(name, got, ref, bound):
        err = np.abs(got - ref)
        worst = float((err / bound).max())
        stage[name] = worst
        assert np.isfinite(got).all(), name
        assert (err <= bound).all(), "%s stage: worst err/bound %g" % (name, worst)

    # 1. AllGather -> QKV projection (bf16 out): the matmul bound plus one bf16 rounding
    R = np.repeat(np.arange(N), len(tokens))
    tt = np.tile(tokens, N)
    ref, mag = oracle.ag_gemm_rows(x, wqkv, R, tt, with_mag=True)
    within("qkv", vals(qkv_g[R, tt]), ref, 1e-5 * mag + 2.0 ** -8 * np.abs(ref) + 1e-30)
    # 2. attention of every rank's heads at the sampled queries, from the GPU's QKV
    rr = np.repeat(np.arange(N), heads * len(tokens))
    hh = np.tile(np.repeat(np.arange(heads), len(tokens)), N)
    qq = np.tile(tokens, N * heads)
    ref, mag = oracle.attention_rows(qkv_g, heads, rr, hh, qq, True, with_mag=True)
    got = np.stack([vals(attn_g[r, t, h * D:(h + 1) * D]) for r, h, t in zip(rr, hh, qq)])
    within("attention", got, ref, attn_bound(qkv_g, heads, True, rr, hh, qq, ref, mag))
    # 3. output projection -> ReduceScatter (fp32 out), from the GPU's attention output
    ref, mag = oracle.gemm_rs_rows(attn_g, wo, owners, rows, with_mag=True)
    within("projection", proj_g[owners, rows], ref, 1e-5 * mag + 1e-30)
    # 4. LayerNorm of the GPU's projection rows (bf16 out)
    xin = proj_g[owners, rows]
    ref = oracle.layernorm(xin, 1e-5)
    within("layernorm", vals(ln_g[owners, rows]), ref, ln_bound(xin, ref, ref, None, None))
    # 5. AllGather -> fc1 with GELU (bf16 out), from the GPU's LayerNorm output
    pre, mag = oracle.ag_gemm_rows(ln_g, w1, R, tt, with_mag=True)
    ref = oracle.gelu(pre)
    within("fc1", vals(fc1_g[R, tt]), ref, 1.13e-5 * mag + 1e-6 * np.abs(pre) + 2.0 ** -8 * np.abs(ref) + 1e-30)
    # 6. fc2 -> ReduceScatter, from the GPU's fc1 output
    ref, mag = oracle.gemm_rs_rows(fc1_g, w2, owners, rows, with_mag=True)
    if out.dtype == torch.float32:
        got = out.cpu().numpy().astype(np.float64)[owners, rows]
        bound = 1e-5 * mag + 1e-30
    else:
        got = vals(gen.torch_bf16_to_bits(out))[owners, rows]
        bound = 1e-5 * mag + 2.0 ** -8 * np.abs(ref) + 1e-30
    within("fc2", got, ref, bound)
    say("  stages, worst err/bound: " + ", ".join("%s %.3f" % kv for kv in stage.items()))

    # the whole chain from x alone: each side rounds its own intermediates to
    # bf16, and softmax and LayerNorm can amplify one bf16 spacing of
    # difference, so this bound is the stage bounds composed loosely
    res = oracle.sp_layer_rows(x, wqkv, wo, w1, w2, heads, tokens, 1e-5)
    got = out.float().cpu().numpy().astype(np.float64).reshape(N * m, d)[tokens]
    ref = res["out"]
    err = np.abs(got - ref)
    rel = np.linalg.norm(err) / np.linalg.norm(ref)
    worst = (err / res["mag"]).max()
    say("  chain: relative error %.3g, worst |err| / sum|F||W2| %.3g" % (rel, worst))
    assert np.isfinite(got).all()
    assert rel <= 2.0 ** -7 and worst <= 2.0 ** -6


CHAIN = [(2, 64, 256, 1, 256, "uni", "graph"), (4, 48, 512, 2, 384, "bi", "graph"),
         (3, 100, 256, 1, 192, "direct", "eager"), (1, 96, 256, 2, 128, "uni", "graph")]


@pytest.mark.parametrize("N,m,d,heads,ffn,dir,exec_mode", CHAIN)
def test_layer_chain(N, m, d, heads, ffn, dir, exec_mode):
    say("layer", N, m, d, heads, ffn, dir, exec_mode)
    plan = nat.cm_plan_layer(n_ranks=N, m=m, d=d, heads=heads, ffn=ffn, dir=dir, n_comm=2, exec_mode=exec_mode,
                             ag_chunks=1, rs_chunks=1, proj_chunks=2 if d % 128 == 0 else 1)
    bits, ts = layer_buffers(N, m, d, heads, ffn, seed=N)
    (out,), ws = run_layer(plan, ts, N, m, d)
    check_chain(plan, bits, ws, out, np.arange(N * m), heads, m)


def test_layer_repeatable_and_bf16_out():
    N, m, d, heads, ffn = 2, 64, 256, 1, 256
    bits, ts = layer_buffers(N, m, d, heads, ffn, seed=5)
    plan = nat.cm_plan_layer(n_ranks=N, m=m, d=d, heads=heads, ffn=ffn, n_comm=1, ag_chunks=1, rs_chunks=1)
    (a, b), _ = run_layer(plan, ts, N, m, d, repeat=2)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    plan16 = nat.cm_plan_layer(n_ranks=N, m=m, d=d, heads=heads, ffn=ffn, n_comm=1, ag_chunks=1, rs_chunks=1,
                               out_dtype="bf16")
    (c,), _ = run_layer(plan16, ts, N, m, d, out_dtype="bf16")
    # the same sums, rounded once to bf16 at the owner
    assert np.array_equal(gen.torch_bf16_to_bits(c), gen.torch_bf16_to_bits(a.to(torch.bfloat16)))


def test_layer_copy_engines_agree():
    """The planner's engine choice (auto) and either engine forced give the
    same layer output bit for bit: a hop copies the same bytes whichever
    engine moves it."""
    N, m, d, heads, ffn = 4, 128, 512, 2, 1024
    bits, ts = layer_buffers(N, m, d, heads, ffn, seed=9)
    outs = {}
    for ce in ("auto", "sdma", "cu"):
        plan = nat.cm_plan_layer(n_ranks=N, m=m, d=d, heads=heads, ffn=ffn, n_comm=1, ag_chunks=1, rs_chunks=1,
                                 copy_engine=ce)
        say("layer copy engine", ce, [getattr(plan, s).desc.copy_engine for s in ("qkv", "proj", "fc1", "fc2")])
        (outs[ce],), _ = run_layer(plan, ts, N, m, d)
    for ce in ("sdma", "cu"):
        assert torch.equal(outs[ce].view(torch.int32), outs["auto"].view(torch.int32)), ce


def test_layer_full_size_sampled():
    # the full sequence-parallel layer: N = 8, 4096 tokens, d = 8192, 64 heads
    # (8 per rank), ffn 28672 (3584 per rank); the configuration the bench times
    N, m, d, heads, ffn = 8, 512, 8192, 8, 3584
    say("layer full size")
    plan = nat.cm_plan_layer(n_ranks=N, m=m, d=d, heads=heads, ffn=ffn, n_comm=1, ag_chunks=1, rs_chunks=1)
    bits, ts = layer_buffers(N, m, d, heads, ffn, device_inputs=True)
    (out,), ws = run_layer(plan, ts, N, m, d)
    tokens = np.array([0, 1, 63, 64, 127, 128, 129, 255, 300, 511, 512, 515])
    check_chain(plan, bits, ws, out, tokens, heads, m)
