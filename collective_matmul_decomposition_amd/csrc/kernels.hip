// gfx950 kernels of the decomposed collective matmuls.
//
//  * gemm_jobs: a batch of independent partial GEMMs ("jobs") in one launch,
//      C[i][j] = sum_kk A[i][kk] * B[j][kk] (+ in0[i][j]) (+ in1[i][j]),
//    A, B bf16 with K contiguous, fp32 accumulation on the matrix cores
//    (v_mfma_f32_32x32x16_bf16).  The epilogue covers the three uses in the
//    schedules: a plain store at a row offset of Y (the slice update of the
//    AllGather loop), a read-add-write into the fp32 bucket that circulates in
//    the ReduceScatter loop, and the owner's final add of one or two arriving
//    buckets with rounding to the output type (the realigning addition of
//    the bidirectional ring).
//  * reduce_jobs: C = in0 + in1 elementwise (the add of the pipeline-chunk
//    ReduceScatter ring), fp32 in, fp32 or bf16 out.
//
// Block tile BM x BN x 64, 256 threads = 4 waves in a WM x (4/WM) grid; each
// wave owns a (BM/WM) x (BN/(4/WM)) sub-tile made of 32x32 MFMA tiles.
// Operands are staged through LDS in two buffers (the next K-slab's global
// loads are in flight while the current slab is multiplied); LDS rows are
// 128 bytes (64 bf16) with the 16-byte column chunks XOR-swizzled by row so
// that the MFMA operand reads spread over the banks.  Blocks are numbered so
// that each of the 8 XCDs (which own separate L2 caches) works on whole jobs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace collmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int BK = 64;          // K per LDS slab
constexpr int ROW_BYTES = 128;  // one LDS row: 64 bf16

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Byte offset of 16-byte chunk `chunk` of LDS row `row` (swizzled).
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * ROW_BYTES + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ int logical_block() {
  // Round-robin dispatch puts block b on XCD b % 8; renumber so that each
  // XCD gets a contiguous range of logical blocks (whole jobs when the job
  // count is a multiple of 8).
  const int G = gridDim.x, b = blockIdx.x;
  const int per = G >> 3;
  return b < per * 8 ? (b & 7) * per + (b >> 3) : b;
}

struct EpiArgs {
  char *C;
  const float *In0, *In1;
  int ldc, ld_in, M, N, row0, col0;
};

// Store one wave's accumulators: C = acc (+ in0) (+ in1), rounded to bf16
// when the output is bf16.  Fully unrolled so the accumulators stay in
// registers.
template <int TM, int TN, bool F32, bool H0, bool H1>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[TM][TN], const EpiArgs &a) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = a.col0 + j * 32;
      const bool col_ok = col < a.N;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = a.row0 + i * 32 + 8 * (e >> 2) + (e & 3);
        if (col_ok && row < a.M) {
          float v = acc[i][j][e];
          const size_t ii = (size_t)row * a.ld_in + col;
          if (H0) v += a.In0[ii];
          if (H1) v += a.In1[ii];
          const size_t oc = (size_t)row * a.ldc + col;
          if (F32)
            reinterpret_cast<float *>(a.C)[oc] = v;
          else
            reinterpret_cast<uint16_t *>(a.C)[oc] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
}

template <int BM, int BN, int WM>
__global__ __launch_bounds__(256) void gemm_jobs_kernel(const GemmParams p) {
  constexpr int WN = 4 / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // MFMA tiles per wave
  constexpr int A_LOADS = BM * 8 / 256, B_LOADS = BN * 8 / 256;
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small for 256 threads");

  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * ROW_BYTES];
  // buffer b: A rows at smem + b*(BM+BN)*ROW_BYTES, then B rows
  auto sA = [&](int b) -> char * { return smem + b * (BM + BN) * ROW_BYTES; };
  auto sB = [&](int b) -> char * { return smem + b * (BM + BN) * ROW_BYTES + BM * ROW_BYTES; };

  const int lb = logical_block();
  const int job = lb / p.tiles_per_job;
  const int tile = lb - job * p.tiles_per_job;
  const int tm0 = (tile % p.tiles_m) * BM;
  const int tn0 = (tile / p.tiles_m) * BN;
  const uint32_t sel = p.sel[job];

  const char *Abase = p.base[sel & 3] + (size_t)p.a_off[job] * 16;
  const char *Bbase = p.base[(sel >> 2) & 3] + (size_t)p.b_off[job] * 16;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Global -> register staging: thread loads chunk (tid & 7) of rows (tid >> 3) + 32 i.
  const int ld_chunk = tid & 7, ld_row = tid >> 3;
  uint4 ra[A_LOADS], rb[B_LOADS];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int r = tm0 + ld_row + 32 * i;
      if (r < p.M)
        ra[i] = *reinterpret_cast<const uint4 *>(Abase + ((size_t)r * p.lda + k0 + ld_chunk * 8) * 2);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int r = tn0 + ld_row + 32 * i;
      if (r < p.N)
        rb[i] = *reinterpret_cast<const uint4 *>(Bbase + ((size_t)r * p.ldb + k0 + ld_chunk * 8) * 2);
      else
        rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      *reinterpret_cast<uint4 *>(sA(buf) + lds_off(ld_row + 32 * i, ld_chunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      *reinterpret_cast<uint4 *>(sB(buf) + lds_off(ld_row + 32 * i, ld_chunk)) = rb[i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int KT = p.K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  // MFMA operand rows: lane owns row (lane & 31) of each 32-row tile and the
  // 8-element K group (lane >> 5) of each 16-wide K step.
  const int frow = lane & 31, fgrp = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_global((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[TM], fb[TN];
      const int chunk = ks * 2 + fgrp;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8 *>(sA(buf) + lds_off(wm * WTM + i * 32 + frow, chunk));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8 *>(sB(buf) + lds_off(wn * WTN + j * 32 + frow, chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_lds(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element e of a 32x32 tile sits at row
  // 8*(e/4) + 4*(lane/32) + e%4 and column lane%32.
  EpiArgs ea;
  ea.C = p.base[(sel >> 4) & 3] + (size_t)p.c_off[job] * 16;
  ea.In0 = reinterpret_cast<const float *>(p.base[3] + (size_t)p.in0_off[job] * 16);
  ea.In1 = reinterpret_cast<const float *>(p.base[3] + (size_t)p.in1_off[job] * 16);
  ea.ldc = p.ldc;
  ea.ld_in = p.ld_in;
  ea.M = p.M;
  ea.N = p.N;
  ea.row0 = tm0 + wm * WTM + 4 * fgrp;
  ea.col0 = tn0 + wn * WTN + (lane & 31);
  const int mode = (p.c_f32 ? 1 : 0) | (((sel >> 6) & 1) << 1) | (((sel >> 7) & 1) << 2);
  switch (mode) {
    case 0: epilogue<TM, TN, false, false, false>(acc, ea); break;
    case 1: epilogue<TM, TN, true, false, false>(acc, ea); break;
    case 2: epilogue<TM, TN, false, true, false>(acc, ea); break;
    case 3: epilogue<TM, TN, true, true, false>(acc, ea); break;
    case 6: epilogue<TM, TN, false, true, true>(acc, ea); break;
    case 7: epilogue<TM, TN, true, true, true>(acc, ea); break;
    case 4: epilogue<TM, TN, false, false, true>(acc, ea); break;
    default: epilogue<TM, TN, true, false, true>(acc, ea); break;
  }
}

// C = in0 + in1 over rows x cols per job; 4 columns per thread.
__global__ __launch_bounds__(256) void reduce_jobs_kernel(const GemmParams p) {
  const int job = blockIdx.y;
  const uint32_t sel = p.sel[job];
  const float *In0 = reinterpret_cast<const float *>(p.base[3] + (size_t)p.in0_off[job] * 16);
  const float *In1 = reinterpret_cast<const float *>(p.base[3] + (size_t)p.in1_off[job] * 16);
  char *Cbase = p.base[(sel >> 4) & 3] + (size_t)p.c_off[job] * 16;
  const int cols4 = p.N >> 2;
  const long total = (long)p.M * cols4;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (long)gridDim.x * blockDim.x) {
    const int row = (int)(t / cols4), c4 = (int)(t - (long)row * cols4) * 4;
    const float4 a = *reinterpret_cast<const float4 *>(In0 + (size_t)row * p.ld_in + c4);
    const float4 b = *reinterpret_cast<const float4 *>(In1 + (size_t)row * p.ld_in + c4);
    const float4 s = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    const size_t oc = (size_t)row * p.ldc + c4;
    if (p.c_f32) {
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(Cbase) + oc) = s;
    } else {
      uint2 o;
      o.x = f32_to_bf16_rne(s.x) | (f32_to_bf16_rne(s.y) << 16);
      o.y = f32_to_bf16_rne(s.z) | (f32_to_bf16_rne(s.w) << 16);
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(Cbase) + oc) = o;
    }
  }
}

template <int BM, int BN, int WM>
hipError_t launch_tile(const GemmParams &p, hipStream_t s) {
  const int grid = p.n_jobs * p.tiles_per_job;
  hipLaunchKernelGGL((gemm_jobs_kernel<BM, BN, WM>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool gemm_tile_supported(int tm, int tn) {
  return (tm == 256 && tn == 256) || (tm == 256 && tn == 128) || (tm == 128 && tn == 256) ||
         (tm == 128 && tn == 128) || (tm == 64 && tn == 256) || (tm == 64 && tn == 128);
}

hipError_t launch_gemm(const GemmParams &p, int tm, int tn, hipStream_t s) {
  if (tm == 256 && tn == 256) return launch_tile<256, 256, 2>(p, s);
  if (tm == 256 && tn == 128) return launch_tile<256, 128, 2>(p, s);
  if (tm == 128 && tn == 256) return launch_tile<128, 256, 2>(p, s);
  if (tm == 128 && tn == 128) return launch_tile<128, 128, 2>(p, s);
  if (tm == 64 && tn == 256) return launch_tile<64, 256, 1>(p, s);
  if (tm == 64 && tn == 128) return launch_tile<64, 128, 1>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const GemmParams &p, hipStream_t s) {
  const long per_job = (long)p.M * (p.N / 4);
  int bx = (int)((per_job + 255) / 256);
  if (bx > 1024) bx = 1024;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL(reduce_jobs_kernel, dim3(bx, p.n_jobs), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace collmm
