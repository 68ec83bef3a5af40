// The backward pass of the two collective matmuls, with bulk overlap.
//
// "Tensor Parallelism > Communication Patterns": the backward communication
// pattern is the dual of the forward one.  For the sequence-parallel linears:
//   column-parallel (forward AllGather -> GEMM, Y_r = Xfull W_r^T):
//     input gradient   dX = ReduceScatter_r(dY_r W_r)       a GEMM -> ReduceScatter
//     weight gradient  dW_r = dY_r^T Xfull                   needs the gathered X
//   row-parallel (forward GEMM -> ReduceScatter):
//     input gradient   dH_r = AllGather(dOut) W_r            an AllGather -> GEMM
//     weight gradient  dW_r = AllGather(dOut)^T H_r          needs the gathered dOut
// Section 7 of the Megatron page ("Bulk Overlap"): the AllGather that only the
// weight gradient needs is independent of the input-gradient GEMM, so it runs
// on a communication stream beside it, into a buffer the compute stream does not
// touch until an event says it is complete.
//
// Building blocks: the decomposed collective matmuls of the forward pass (with
// the transposed weights as their weight operand), the AllGather alone
// (cm_allgather), a bf16 transpose and a batched GEMM on the same MFMA kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>
#include <unordered_map>

#include "collmm.h"
#include "internal.h"
#include "kernels.h"

namespace collmm {
namespace {

// dst[b][c][r] = src[b][r][c] for r < rows, c < cols; dst[b][c][r] = 0 for
// rows <= r < ld_dst (padding).  64 x 64 tiles through LDS: reads along src
// rows and writes along dst rows are both coalesced.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *src, uint16_t *dst, int rows, int cols,
                                                         int ld_dst, size_t src_batch, size_t dst_batch) {
  __shared__ uint16_t tile[64][66];
  const uint16_t *s = src + blockIdx.z * src_batch;
  uint16_t *d = dst + blockIdx.z * dst_batch;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + ty + 4 * i, c = c0 + tx;
    tile[ty + 4 * i][tx] = (r < rows && c < cols) ? s[(size_t)r * cols + c] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + ty + 4 * i, r = r0 + tx;
    if (c < cols && r < ld_dst) d[(size_t)c * ld_dst + r] = tile[tx][ty + 4 * i];
  }
}

// The same transpose with 16-byte accesses on both sides, for cols and
// ld_dst multiples of 8 and 16-byte aligned buffers: each thread reads 8
// consecutive elements of a src row into the LDS tile, then gathers 8
// consecutive rows of one column from the tile and writes them as one
// 16-byte store along the dst row.  The tile's rows are padded by one dword
// so that the column gathers of a wave fall into different banks.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t *src, uint16_t *dst, int rows, int cols,
                                                           int ld_dst, size_t src_batch, size_t dst_batch) {
  __shared__ uint16_t tile[64][66];
  const uint16_t *s = src + blockIdx.z * src_batch;
  uint16_t *d = dst + blockIdx.z * dst_batch;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x, q = t & 7, u = t >> 3;  // q: 8-element chunk, u: row (load) or column (store)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = u + 32 * i, r = r0 + rr, c = c0 + 8 * q;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows && c < cols) v = *reinterpret_cast<const uint4 *>(s + (size_t)r * cols + c);
    uint32_t *row = reinterpret_cast<uint32_t *>(&tile[rr][8 * q]);
    row[0] = v.x;
    row[1] = v.y;
    row[2] = v.z;
    row[3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cc = u + 32 * i, c = c0 + cc, r = r0 + 8 * q;
    if (c < cols && r < ld_dst) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (uint32_t)tile[8 * q + 2 * j][cc] | ((uint32_t)tile[8 * q + 2 * j + 1][cc] << 16);
      *reinterpret_cast<uint4 *>(d + (size_t)c * ld_dst + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

cm_status hip_fail(hipError_t e, const char *what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return CM_ERR_HIP;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

cm_status check_transpose(int batch, int rows, int cols, int ld_dst) {
  if (batch < 1 || batch > 65535 || rows < 1 || cols < 1 || ld_dst < rows || (long long)ld_dst * cols > (1ll << 40) ||
      (long long)rows * cols > (1ll << 40) || (ld_dst + 63) / 64 > 65535) {
    set_error("transpose: need 1 <= batch <= 65535, rows, cols >= 1, ld_dst >= rows (got %d, %d, %d, %d)", batch, rows,
              cols, ld_dst);
    return CM_ERR_SHAPE;
  }
  return CM_OK;
}

hipError_t launch_transpose(const void *src, void *dst, int batch, int rows, int cols, int ld_dst, hipStream_t s) {
  dim3 grid((cols + 63) / 64, (ld_dst + 63) / 64, batch);
  const bool vec = cols % 8 == 0 && ld_dst % 8 == 0 && aligned16(src) && aligned16(dst);
  const uint16_t *sp = static_cast<const uint16_t *>(src);
  uint16_t *dp = static_cast<uint16_t *>(dst);
  if (vec)
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, s, sp, dp, rows, cols, ld_dst, (size_t)rows * cols,
                       (size_t)cols * ld_dst);
  else
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, sp, dp, rows, cols, ld_dst, (size_t)rows * cols,
                       (size_t)cols * ld_dst);
  return hipGetLastError();
}

// C_b = A_b . B_b^T through the job kernel, up to kMaxJobs batches per launch.
cm_status check_gemm(int batch, int M, int N, int K, int lda, int ldb, int ldc, long long sa, long long sb,
                     long long sc, int out_dtype) {
  if (batch < 1 || M < 1 || N < 1 || K < 64 || K % 64) {
    set_error("gemm: need batch, M, N >= 1 and K a positive multiple of 64 (got %d, %d, %d, %d)", batch, M, N, K);
    return CM_ERR_SHAPE;
  }
  // operands are read 16 bytes at a time; outputs are stored element by
  // element, so only each batch's C base needs 16-byte alignment
  if (lda < K || ldb < K || ldc < N || lda % 8 || ldb % 8 || sa % 8 || sb % 8 ||
      sc % (out_dtype == CM_F32 ? 4 : 8) || sa < 0 || sb < 0 || sc < 0) {
    set_error("gemm: leading dimensions must cover the rows; lda, ldb and the batch strides must keep 16-byte "
              "alignment");
    return CM_ERR_SHAPE;
  }
  if ((long long)M * lda * 2 > 0xFFFFFFFFll || (long long)N * ldb * 2 > 0xFFFFFFFFll) {
    set_error("gemm: one operand of a batch exceeds 4 GiB");
    return CM_ERR_SHAPE;
  }
  const long long esz = out_dtype == CM_F32 ? 4 : 2;
  if ((batch - 1) * sa * 2 / 16 > 0xFFFFFFFFll || (batch - 1) * sb * 2 / 16 > 0xFFFFFFFFll ||
      (batch - 1) * sc * esz / 16 > 0xFFFFFFFFll) {
    set_error("gemm: batch strides too large");
    return CM_ERR_SHAPE;
  }
  if (out_dtype != CM_F32 && out_dtype != CM_BF16) { set_error("gemm: out dtype must be CM_F32 or CM_BF16"); return CM_ERR_UNSUPPORTED; }
  return CM_OK;
}

cm_status launch_batched_gemm(int batch, int M, int N, int K, const void *a, int lda, long long sa, const void *b,
                              int ldb, long long sb, void *c, int ldc, long long sc, int out_dtype, hipStream_t s) {
  const long long esz = out_dtype == CM_F32 ? 4 : 2;
  for (int b0 = 0; b0 < batch; b0 += kMaxJobs) {
    const int nj = batch - b0 < kMaxJobs ? batch - b0 : kMaxJobs;
    int tm, tn;
    (void)choose_gemm_tile(M, N, nj, &tm, &tn);
    GemmParams p;
    std::memset(&p, 0, sizeof p);
    p.base[0] = const_cast<char *>(static_cast<const char *>(a)) + (size_t)b0 * sa * 2;
    p.base[1] = const_cast<char *>(static_cast<const char *>(b)) + (size_t)b0 * sb * 2;
    p.base[2] = static_cast<char *>(c) + (size_t)b0 * sc * esz;
    p.base[3] = p.base[2];
    p.M = M; p.N = N; p.K = K;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.ld_in = ldc;
    p.c_f32 = out_dtype == CM_F32;
    p.n_jobs = nj;
    p.tiles_m = (M + tm - 1) / tm;
    p.tiles_per_job = p.tiles_m * ((N + tn - 1) / tn);
    for (int j = 0; j < nj; ++j) {
      p.a_off[j] = (uint32_t)((size_t)j * sa * 2 / 16);
      p.b_off[j] = (uint32_t)((size_t)j * sb * 2 / 16);
      p.c_off[j] = (uint32_t)((size_t)j * sc * esz / 16);
      p.sel[j] = (uint8_t)(0u | (1u << 2) | (2u << 4));
    }
    hipError_t e = launch_gemm(p, tm, tn, s);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
  }
  return CM_OK;
}

cm_status gfx950_current() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    set_error("device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
    return CM_ERR_UNSUPPORTED;
  }
  return CM_OK;
}

// Two events per device per host thread: inputs ready (compute -> bulk) and
// gathered operand ready (bulk -> compute).
cm_status bulk_events(hipEvent_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  thread_local std::unordered_map<int, std::pair<hipEvent_t, hipEvent_t>> pool;
  auto it = pool.find(dev);
  if (it == pool.end()) {
    hipEvent_t a, b;
    if ((e = hipEventCreateWithFlags(&a, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = hipEventCreateWithFlags(&b, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    it = pool.emplace(dev, std::make_pair(a, b)).first;
  }
  static thread_local hipEvent_t pair[2];
  pair[0] = it->second.first;
  pair[1] = it->second.second;
  *out = pair;
  return CM_OK;
}

bool same_plan_desc(const cm_plan_desc &a, const cm_plan_desc &b) {
  return a.op == b.op && a.n_ranks == b.n_ranks && a.m == b.m && a.k == b.k && a.n == b.n && a.dir == b.dir &&
         a.chunks == b.chunks && a.sched == b.sched && a.in_dtype == b.in_dtype && a.out_dtype == b.out_dtype &&
         a.n_comm == b.n_comm && a.tile_m == b.tile_m && a.tile_n == b.tile_n && a.exec_mode == b.exec_mode &&
         a.copy_engine == b.copy_engine && a.bucket_bf16 == b.bucket_bf16 && a.hop_add == b.hop_add &&
         a.copy_gbps == b.copy_gbps && a.mfma_tflops == b.mfma_tflops && a.launch_us == b.launch_us && a.act == b.act &&
         a.share == b.share && a.split_k == b.split_k && a.skip == b.skip && a.stress == b.stress &&
         a.group == b.group;
}
bool same_sched(const cm_plan &a, const cm_plan &b) {
  return same_plan_desc(a.desc, b.desc) && a.chunks == b.chunks && a.n_steps == b.n_steps && a.arc_cw == b.arc_cw &&
         a.arc_ccw == b.arc_ccw && a.tile_m == b.tile_m && a.tile_n == b.tile_n && a.n_ops == b.n_ops &&
         a.n_jobs == b.n_jobs && a.n_events == b.n_events && a.ws_bytes == b.ws_bytes && a.split == b.split &&
         a.n_launches == b.n_launches && a.slots == b.slots &&
         std::memcmp(a.group_len, b.group_len, sizeof a.group_len) == 0;
}

}  // namespace
}  // namespace collmm

using namespace collmm;

extern "C" {

cm_status cm_transpose(const void *src, void *dst, int batch, int rows, int cols, int ld_dst, void *stream) {
  cm_status st = check_transpose(batch, rows, cols, ld_dst);
  if (st != CM_OK) return st;
  if (!src || !dst) { set_error("transpose: null pointer"); return CM_ERR_INVALID_ARG; }
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 1) {
    set_error("transpose: pointers must be 2-byte aligned");
    return CM_ERR_ALIGN;
  }
  if ((st = gfx950_current()) != CM_OK) return st;
  hipError_t e = launch_transpose(src, dst, batch, rows, cols, ld_dst, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CM_OK : hip_fail(e, "transpose launch");
}

cm_status cm_gemm(int batch, int M, int N, int K, const void *a, int lda, long long stride_a, const void *b, int ldb,
                  long long stride_b, void *c, int ldc, long long stride_c, int out_dtype, void *stream) {
  cm_status st = check_gemm(batch, M, N, K, lda, ldb, ldc, stride_a, stride_b, stride_c, out_dtype);
  if (st != CM_OK) return st;
  if (!a || !b || !c) { set_error("gemm: null pointer"); return CM_ERR_INVALID_ARG; }
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) { set_error("gemm: pointers must be 16-byte aligned"); return CM_ERR_ALIGN; }
  if ((st = gfx950_current()) != CM_OK) return st;
  return launch_batched_gemm(batch, M, N, K, a, lda, stride_a, b, ldb, stride_b, c, ldc, stride_c, out_dtype,
                             static_cast<hipStream_t>(stream));
}

cm_status cm_plan_backward(const cm_bwd_desc *desc, cm_bwd_plan *out) {
  if (!desc || !out) { set_error("null argument"); return CM_ERR_INVALID_ARG; }
  const cm_bwd_desc d = *desc;
  if (d.kind != CM_BWD_COL && d.kind != CM_BWD_ROW) { set_error("unknown backward kind %d", d.kind); return CM_ERR_INVALID_ARG; }
  if (d.bulk != 0 && d.bulk != 1) { set_error("bulk must be 0 or 1"); return CM_ERR_INVALID_ARG; }
  if ((d.dx_dtype != CM_F32 && d.dx_dtype != CM_BF16) || (d.dw_dtype != CM_F32 && d.dw_dtype != CM_BF16)) {
    set_error("gradient dtypes must be CM_F32 or CM_BF16");
    return CM_ERR_UNSUPPORTED;
  }
  if (d.n_ranks < 1 || d.m < 1) { set_error("need n_ranks >= 1 and m >= 1"); return CM_ERR_INVALID_ARG; }
  const long long T = (long long)d.n_ranks * d.m;
  const long long Tp = (T + 63) / 64 * 64;  // the weight gradient contracts over tokens, padded to whole K slabs
  cm_bwd_plan p;
  std::memset(&p, 0, sizeof p);
  p.desc = d;
  // the input gradient: the dual collective matmul with the transposed weights
  // (W_r^T stored [k][n]: its n is the contraction, its k the output columns)
  cm_plan_desc g;
  std::memset(&g, 0, sizeof g);
  g.op = d.kind == CM_BWD_COL ? CM_OP_GEMM_RS : CM_OP_AG_GEMM;
  g.n_ranks = d.n_ranks; g.m = d.m; g.k = d.n; g.n = d.k;
  g.dir = d.dir; g.chunks = d.chunks; g.sched = CM_SCHED_DECOMPOSED;
  g.in_dtype = CM_BF16; g.out_dtype = d.dx_dtype; g.n_comm = d.n_comm;
  g.exec_mode = d.exec_mode; g.copy_engine = d.copy_engine;
  g.hop_add = (d.kind == CM_BWD_COL && d.dir != CM_RING_DIRECT) ? 1 : 0;
  cm_status st = plan(&g, &p.dgrad);
  if (st != CM_OK) return st;
  // the bulk AllGather of the weight gradient's gathered operand (COL: x,
  // rows of k; ROW: dOut, rows of n) on one copy lane
  cm_plan_desc a;
  std::memset(&a, 0, sizeof a);
  a.op = CM_OP_ALLGATHER;
  a.n_ranks = d.n_ranks; a.m = d.m; a.k = d.kind == CM_BWD_COL ? d.k : d.n; a.n = 0;
  a.dir = CM_RING_UNI; a.sched = CM_SCHED_DECOMPOSED; a.in_dtype = CM_BF16; a.out_dtype = CM_BF16;
  // The gather's copies are one rank's shard each (the gathered arrays are
  // per rank), which the CU copy kernel moves several times faster than the
  // SDMA engines; off the SDMA engines it also leaves them to the input
  // gradient's ring hops.  So it always uses the copy kernel.
  a.n_comm = 1; a.exec_mode = d.exec_mode; a.copy_engine = CM_COPY_CU;
  if ((st = plan(&a, &p.gather)) != CM_OK) return st;
  if (Tp > 0x7FFFFFFFll || Tp * d.n * 2 > 0xFFFFFFFFll || Tp * d.k * 2 > 0xFFFFFFFFll) {
    set_error("backward: a rank's gathered operand exceeds 4 GiB");
    return CM_ERR_SHAPE;
  }
  const size_t N = d.n_ranks, A = 256;
  const size_t gk = d.kind == CM_BWD_COL ? d.k : d.n;  // row length of the gathered operand
  const size_t ok = d.kind == CM_BWD_COL ? d.n : d.k;  // row length of the other wgrad operand (dY or H)
  size_t off = 0;
  p.off_wt = off; off = round_up(off + N * d.n * d.k * 2, A);
  p.off_g = off; off = round_up(off + N * T * gk * 2, A);
  p.off_gt = off; off = round_up(off + N * gk * Tp * 2, A);
  p.off_ot = off; off = round_up(off + N * ok * Tp * 2, A);
  p.off_ops = off;
  p.ws_bytes = off + p.dgrad.ws_bytes;
  *out = p;
  return CM_OK;
}

cm_status cm_linear_backward(const cm_bwd_plan *pl, const void *act, const void *w, const void *wt, const void *grad,
                             void *dact, void *dw, void *ws, size_t ws_bytes, void *compute, void *const *comm,
                             int n_comm) {
  if (!pl) { set_error("null plan"); return CM_ERR_INVALID_ARG; }
  cm_bwd_plan canon;
  cm_status st = cm_plan_backward(&pl->desc, &canon);
  if (st != CM_OK) return st;
  if (!same_sched(canon.dgrad, pl->dgrad) || !same_sched(canon.gather, pl->gather) || canon.off_wt != pl->off_wt ||
      canon.off_g != pl->off_g || canon.off_gt != pl->off_gt || canon.off_ot != pl->off_ot ||
      canon.off_ops != pl->off_ops || canon.ws_bytes != pl->ws_bytes) {
    set_error("backward plan does not match what cm_plan_backward produces for its request");
    return CM_ERR_INVALID_ARG;
  }
  const cm_bwd_desc &d = pl->desc;
  if (!act || !w || !grad || !dact || !dw || !ws) { set_error("null buffer"); return CM_ERR_INVALID_ARG; }
  if (!aligned16(act) || !aligned16(w) || (wt && !aligned16(wt)) || !aligned16(grad) || !aligned16(dact) ||
      !aligned16(dw) || !aligned16(ws)) {
    set_error("buffers must be 16-byte aligned");
    return CM_ERR_ALIGN;
  }
  if (ws_bytes < pl->ws_bytes) {
    set_error("workspace of %zu bytes, backward plan needs %zu", ws_bytes, pl->ws_bytes);
    return CM_ERR_WORKSPACE;
  }
  if (n_comm != d.n_comm + 2 || !comm) {
    set_error("the call passes the %d comm streams of the input gradient, then the bulk stream and its copy lane "
              "(%d in all), got %d", d.n_comm, d.n_comm + 2, n_comm);
    return CM_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n_comm; ++i) {
    if (!comm[i] || comm[i] == compute) { set_error("comm stream %d is null or the compute stream", i); return CM_ERR_INVALID_ARG; }
    for (int j = 0; j < i; ++j)
      if (comm[i] == comm[j]) { set_error("comm streams %d and %d are the same stream", j, i); return CM_ERR_INVALID_ARG; }
  }
  if ((st = gfx950_current()) != CM_OK) return st;
  if ((st = refuse_capture(compute, comm, n_comm)) != CM_OK) return st;
  hipEvent_t *ev;
  if ((st = bulk_events(&ev)) != CM_OK) return st;

  const int N = d.n_ranks, m = d.m, k = d.k, n = d.n, T = N * m, Tp = (T + 63) / 64 * 64;
  const bool col = d.kind == CM_BWD_COL;
  char *W = static_cast<char *>(ws);
  char *wt_ws = W + pl->off_wt, *g = W + pl->off_g, *gt = W + pl->off_gt, *ot = W + pl->off_ot, *ops = W + pl->off_ops;
  const size_t opbytes = ws_bytes - pl->off_ops;
  hipStream_t S = static_cast<hipStream_t>(compute);
  hipStream_t B = d.bulk ? static_cast<hipStream_t>(comm[d.n_comm]) : S;  // where the weight gradient's inputs are made
  void *const *lane = comm + d.n_comm + 1;
  hipError_t e;

  // the weight gradient's operands (bulk: on their own stream, after the inputs are ready)
  if (d.bulk) {
    if ((e = hipEventRecord(ev[0], S)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(B, ev[0], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  // the input gradient: the dual collective matmul with W_r^T [k][n].  It is
  // enqueued before the weight gradient's operands, which it does not depend
  // on, so that its first GEMM is dispatched ahead of their copies.
  const void *wtp = wt;
  if (!wtp) {
    if ((e = launch_transpose(w, wt_ws, N, n, k, n, S)) != hipSuccess) return hip_fail(e, "transpose");
    wtp = wt_ws;
  }
  if (col)
    st = cm_gemm_rs(&pl->dgrad, grad, wtp, dact, ops, opbytes, compute, comm, d.n_comm, nullptr);
  else
    st = cm_ag_gemm(&pl->dgrad, grad, wtp, dact, ops, opbytes, compute, comm, d.n_comm, nullptr);
  if (st != CM_OK) return st;

  // COL: dY_r^T [n][Tp]; ROW: H_r^T [k][Tp]
  const void *other = col ? grad : act;
  const int orows = T, ocols = col ? n : k;
  if ((e = launch_transpose(other, ot, N, orows, ocols, Tp, B)) != hipSuccess) return hip_fail(e, "transpose");
  // gather (COL: x shards; ROW: dOut shards), then transpose each rank's copy
  const void *shards = col ? act : grad;
  if ((st = cm_allgather(&pl->gather, shards, g, B, lane, 1, nullptr)) != CM_OK) return st;
  const int gcols = col ? k : n;
  if ((e = launch_transpose(g, gt, N, T, gcols, Tp, B)) != hipSuccess) return hip_fail(e, "transpose");
  if (d.bulk) {
    if ((e = hipEventRecord(ev[1], B)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  }

  // the weight gradient: dW_r [n][k] = (gathered or dY)^T-major operands, K = tokens
  if (d.bulk && (e = hipStreamWaitEvent(S, ev[1], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  const void *A = col ? ot : gt;  // [n][Tp]
  const void *Bm = col ? gt : ot; // [k][Tp]
  return launch_batched_gemm(N, n, k, Tp, A, Tp, (long long)n * Tp, Bm, Tp, (long long)k * Tp, dw, k,
                             (long long)n * k, d.dw_dtype, S);
}

}  // extern "C"
