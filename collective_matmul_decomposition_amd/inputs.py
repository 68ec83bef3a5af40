"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random tensors
and stores them as bfloat16.  Shapes follow the library's layout:

    AllGather -> GEMM   x [N, m, k]     (sequence shards X_r)
                        w [N, n, k]     (column-parallel weight shards W_r,
                                         one output feature per row)
    GEMM -> ReduceScatter
                        h [N, N*m, k]   (rank r's activation for all T = N*m
                                         tokens, its k = f/N slice)
                        w [N, n, k]     (row-parallel weight shards, stored
                                         one output feature per row)

The transformer layer around the two ops (layer_inputs) adds the attention
and MLP weights of one sequence-parallel layer:

    x [N, m, d], wqkv [N, 3*H*D, d], wo [N, d, H*D], w1 [N, f/N, d],
    w2 [N, d, f/N]   (H heads of D dimensions per rank)

and the stand-alone attention and LayerNorm inputs (attention_inputs:
qkv [N, T, 3*H*D]; layernorm_inputs: fp32 rows), and the fp32 buckets that
stand for the ring neighbour in one rank's share of the ReduceScatter
(peer_buckets: [N-1, m, n]).

Distributions: "normal" draws activations from N(0, 1) and weights from
N(0, 0.02^2); "int" draws every element uniformly from {-3, ..., 3}, which
bf16 holds exactly and whose products and sums stay exact in fp32.

Two back ends produce the same kinds of tensors:
  * numpy (CPU): PCG64 streams from SeedSequence(seed).spawn(4) for
    (X, W1, H, W2); float32 draws rounded to bf16 by the bias method below.
  * torch (device): a torch.Generator on the target device, for sizes where
    host generation would be slow; the bf16 cast is torch's (nearest-even).
"""
import numpy as np

ACT_STD = 1.0
WEIGHT_STD = 0.02
INT_LO, INT_HI = -3, 3


def f32_to_bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Bias method on the binary32 bit pattern: add 0x7FFF plus the lowest bit
    that is kept, then drop the low 16 bits.  Inputs must be finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    return ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(seed):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(4)]


def _draw(gen, shape, dist, std):
    if dist == "int":
        return gen.integers(INT_LO, INT_HI + 1, size=shape).astype(np.float32)
    if dist == "normal":
        return (gen.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    raise ValueError("dist must be 'normal' or 'int', got %r" % (dist,))


def ag_inputs(N, m, k, n, dist="normal", seed=0):
    """(x [N,m,k], w [N,n,k]) as uint16 bf16 bit patterns (numpy, CPU)."""
    g = _streams(seed)
    x = f32_to_bf16_bits(_draw(g[0], (N, m, k), dist, ACT_STD))
    w = f32_to_bf16_bits(_draw(g[1], (N, n, k), dist, WEIGHT_STD))
    return x, w


def rs_inputs(N, m, k, n, dist="normal", seed=0):
    """(h [N,N*m,k], w [N,n,k]) as uint16 bf16 bit patterns (numpy, CPU)."""
    g = _streams(seed)
    h = f32_to_bf16_bits(_draw(g[2], (N, N * m, k), dist, ACT_STD))
    w = f32_to_bf16_bits(_draw(g[3], (N, n, k), dist, WEIGHT_STD))
    return h, w


def to_torch_bf16(bits, device="cpu"):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor (bit-identical)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def torch_bf16_to_bits(t):
    """torch.bfloat16 tensor -> numpy uint16 bit patterns (bit-identical)."""
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _torch_draw(shape, dist, std, gen, device):
    import torch
    if dist == "int":
        return torch.randint(INT_LO, INT_HI + 1, shape, generator=gen, device=device).to(torch.bfloat16)
    if dist == "normal":
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return (t * std).to(torch.bfloat16)
    raise ValueError("dist must be 'normal' or 'int', got %r" % (dist,))


def ag_inputs_torch(N, m, k, n, dist="normal", seed=0, device="cuda"):
    """(x [N,m,k], w [N,n,k]) as torch.bfloat16 on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 4 + 0)
    x = _torch_draw((N, m, k), dist, ACT_STD, g, device)
    g.manual_seed(seed * 4 + 1)
    w = _torch_draw((N, n, k), dist, WEIGHT_STD, g, device)
    return x, w


def rs_inputs_torch(N, m, k, n, dist="normal", seed=0, device="cuda"):
    """(h [N,N*m,k], w [N,n,k]) as torch.bfloat16 on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 4 + 2)
    h = _torch_draw((N, N * m, k), dist, ACT_STD, g, device)
    g.manual_seed(seed * 4 + 3)
    w = _torch_draw((N, n, k), dist, WEIGHT_STD, g, device)
    return h, w


def _layer_streams(seed):
    # independent of the (X, W1, H, W2) streams above
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence([seed, 5]).spawn(5)]


def layer_inputs(N, m, d, heads, head_dim, f_per_rank, dist="normal", seed=0):
    """(x, wqkv, wo, w1, w2) of one sequence-parallel layer as bf16 bit
    patterns (numpy, CPU): activations N(0,1), weights N(0, 0.02^2)."""
    g = _layer_streams(seed)
    HD = heads * head_dim
    x = f32_to_bf16_bits(_draw(g[0], (N, m, d), dist, ACT_STD))
    wqkv = f32_to_bf16_bits(_draw(g[1], (N, 3 * HD, d), dist, WEIGHT_STD))
    wo = f32_to_bf16_bits(_draw(g[2], (N, d, HD), dist, WEIGHT_STD))
    w1 = f32_to_bf16_bits(_draw(g[3], (N, f_per_rank, d), dist, WEIGHT_STD))
    w2 = f32_to_bf16_bits(_draw(g[4], (N, d, f_per_rank), dist, WEIGHT_STD))
    return x, wqkv, wo, w1, w2


def layer_inputs_torch(N, m, d, heads, head_dim, f_per_rank, dist="normal", seed=0, device="cuda"):
    """The same tensors drawn on `device` (torch.bfloat16), for full sizes."""
    import torch
    g = torch.Generator(device=device)
    HD = heads * head_dim
    shapes = [((N, m, d), ACT_STD), ((N, 3 * HD, d), WEIGHT_STD), ((N, d, HD), WEIGHT_STD),
              ((N, f_per_rank, d), WEIGHT_STD), ((N, d, f_per_rank), WEIGHT_STD)]
    out = []
    for i, (shape, std) in enumerate(shapes):
        g.manual_seed(seed * 8 + 100 + i)
        out.append(_torch_draw(shape, dist, std, g, device))
    return tuple(out)


def attention_inputs(N, T, heads, head_dim, std=1.8, seed=0):
    """qkv [N, T, 3*heads*head_dim] bf16 bits, N(0, std^2) (std 1.8 is the
    spread of a projection of N(0,1) activations by N(0, 0.02^2) weights over
    d = 8192: sqrt(8192) * 0.02 = 1.81)."""
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 6])))
    return f32_to_bf16_bits(_draw(gen, (N, T, 3 * heads * head_dim), "normal", std))


def attention_inputs_torch(N, T, heads, head_dim, std=1.8, seed=0, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 8 + 110)
    return _torch_draw((N, T, 3 * heads * head_dim), "normal", std, g, device)


def layernorm_inputs(rows, cols, seed=0):
    """fp32 rows x[i] = mu_i + s_i * z with z ~ N(0,1), per-row offsets
    mu_i ~ N(0, 2^2) and spreads s_i uniform in [0.25, 4] (numpy float32)."""
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    mu = gen.standard_normal((rows, 1), dtype=np.float32) * np.float32(2.0)
    sd = gen.uniform(0.25, 4.0, (rows, 1)).astype(np.float32)
    return (mu + sd * gen.standard_normal((rows, cols), dtype=np.float32)).astype(np.float32)


def backward_inputs(kind, N, m, k, n, dist="normal", seed=0):
    """Inputs of the backward of a collective matmul as bf16 bit patterns:
    kind "col" (AllGather -> GEMM): x [N, m, k], w [N, n, k], dy [N, N*m, n];
    kind "row" (GEMM -> ReduceScatter): h [N, N*m, k], w [N, n, k],
    dout [N, m, n].  Activations N(0,1), weights N(0, 0.02^2), upstream
    gradients N(0,1) (a scale-free stand-in: the ops are linear in them)."""
    g = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence([seed, 9]).spawn(3)]
    if kind == "col":
        shapes = ((N, m, k), (N, n, k), (N, N * m, n))
    else:
        shapes = ((N, N * m, k), (N, n, k), (N, m, n))
    stds = (ACT_STD, WEIGHT_STD, ACT_STD)
    return tuple(f32_to_bf16_bits(_draw(g[i], shapes[i], dist, stds[i])) for i in range(3))


def backward_inputs_torch(kind, N, m, k, n, dist="normal", seed=0, device="cuda"):
    import torch
    gen_ = torch.Generator(device=device)
    if kind == "col":
        shapes = ((N, m, k), (N, n, k), (N, N * m, n))
    else:
        shapes = ((N, N * m, k), (N, n, k), (N, m, n))
    out = []
    for i, (shape, std) in enumerate(zip(shapes, (ACT_STD, WEIGHT_STD, ACT_STD))):
        gen_.manual_seed(seed * 8 + 120 + i + (3 if kind == "row" else 0))
        out.append(_torch_draw(shape, dist, std, gen_, device))
    return tuple(out)


def peer_buckets(N, m, n, dist="normal", seed=0):
    """The buckets a ring neighbour sends to rank 0 in one rank's share of the
    ReduceScatter: fp32 [N-1, m, n].  "int": uniform over {-3, ..., 3} x 8
    (partial sums of integer products); "normal": N(0, 0.5^2), about the size of
    a partial product of the N(0, 1) x N(0, 0.02^2) inputs at k of a few
    hundred."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    shape = (max(0, N - 1), m, n)
    if dist == "int":
        return (g.integers(INT_LO, INT_HI + 1, size=shape) * 8).astype(np.float32)
    if dist == "normal":
        return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    raise ValueError("dist must be 'normal' or 'int', got %r" % (dist,))
