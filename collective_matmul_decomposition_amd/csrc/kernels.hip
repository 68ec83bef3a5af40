// gfx950 kernels of the decomposed collective matmuls.
//
//  * gemm_jobs: a batch of independent partial GEMMs ("jobs") in one launch,
//      C[i][j] = sum_kk A[i][kk] * B[j][kk] (+ in0[i][j]) (+ in1[i][j]),
//    A, B bf16 with K contiguous, fp32 accumulation on the matrix cores
//    (v_mfma_f32_32x32x16_bf16).  The epilogue covers the three uses in the
//    schedules (and, for launches without addends, an optional GELU applied
//    before the store: the MLP activation fused into the AllGather->fc1
//    slice update): a plain store at a row offset of Y (the slice update of the
//    AllGather loop), a read-add-write into the fp32 bucket that circulates in
//    the ReduceScatter loop, and the owner's final add of one or two arriving
//    buckets with rounding to the output type (the realigning addition of
//    the bidirectional ring).
//  * reduce_jobs: C = in0 + in1 elementwise (the add of the pipeline-chunk
//    ReduceScatter ring and of the add-and-forward hops), or the sum of S
//    fp32 blocks (+ in1, then optionally GELU): the split-K partials of one
//    rank's step GEMM; fp32 in, fp32 or bf16 out.
//
// Block tile BM x BN x 64, 8 MFMA waves (two per SIMD); operands are staged
// through rings of LDS slabs by direct-to-LDS buffer loads (the next K-slabs
// are in flight while the current one is multiplied).  The two largest tiles
// add 4 loader waves that issue every load, so the MFMA waves never wait on
// the vector-memory pipe, and give the weights (B, streamed from HBM) a
// deeper ring than the activations (A, mostly L2 hits).  LDS rows are 128 bytes (64
// bf16) with the 16-byte K-chunks XOR-swizzled by row so that the MFMA
// operand reads spread over the banks.  Blocks are numbered so that each of
// the 8 XCDs (which own separate L2 caches) works on whole jobs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace collmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_ptr;

namespace {


__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}


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
  const void *In0, *In1;  // fp32, or bf16 (HB)
  int ldc, ld_in, M, N, row0, col0;
};

// Store one wave's accumulators: C = acc (+ in0) (+ in1), rounded to bf16
// when the output is bf16.  Fully unrolled so the accumulators stay in
// registers.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Addend element ii of in0 or in1: fp32, or bf16 when HB.
template <bool HB>
__device__ __forceinline__ float addend(const void *p, size_t ii) {
  if (HB) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[ii]);
  return reinterpret_cast<const float *>(p)[ii];
}

// GELU, erf form: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in fp32.
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }

template <int TM, int TN, bool F32, bool H0, bool H1, bool HB, bool GELU = false>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[TM][TN], const EpiArgs &a) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = a.col0 + j * 32;
      const bool col_ok = col < a.N;
      const int colc = min(col, a.N - 1);
      // Eight elements at a time: their addends are read unconditionally
      // from clamped (in-bounds) positions before any of them is written
      // (C may be the buffer that holds in0), so the reads are in flight
      // together; only the stores are predicated.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float add[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int e = h * 8 + q;
          const int rowc = min(a.row0 + i * 32 + 8 * (e >> 2) + (e & 3), a.M - 1);
          const size_t ii = (size_t)rowc * a.ld_in + colc;
          add[q] = 0.f;
          if (H0) add[q] = addend<HB>(a.In0, ii);
          if (H1) add[q] += addend<HB>(a.In1, ii);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int e = h * 8 + q;
          const int row = a.row0 + i * 32 + 8 * (e >> 2) + (e & 3);
          if (col_ok && row < a.M) {
            float v = (H0 || H1) ? acc[i][j][e] + add[q] : acc[i][j][e];
            if (GELU) v = gelu_erf(v);
            const size_t oc = (size_t)row * a.ldc + col;
            if (F32)
              reinterpret_cast<float *>(a.C)[oc] = v;
            else
              reinterpret_cast<uint16_t *>(a.C)[oc] = (uint16_t)f32_to_bf16_rne(v);
          }
        }
      }
    }
}

// One workgroup = 8 waves (512 threads, two per SIMD) computes a BM x BN tile
// of one job; the waves form a WM x WN grid and each owns a (BM/WM) x (BN/WN)
// sub-tile of 32x32 MFMA tiles.  Operands move HBM/L2 -> LDS with the
// direct-to-LDS loads of gfx950 (global_load_lds_dwordx4: each lane's 16
// bytes land at the wave's LDS base + 16 * lane, no VGPR staging) through
// rings of LDS slabs of BK values of K (AST slabs for A, BST for B): while
// slab kt is multiplied, the following slabs are in flight.  Rows past the
// end of A or B are clamped to the last row: they only feed outputs that are
// not stored.
//
// LDS layout of a slab: rows of 2*BK bytes holding BK/8 16-byte K-chunks;
// chunk c of row r sits at position c ^ (r / R % (BK/8)) with R = 256 / (2*BK)
// rows per 256 bytes, so the 16 rows that one 16-lane phase of an MFMA
// operand read touches cover the 64 banks once.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most n (0..63) of this wave's vector-memory loads are
// outstanding; the count is an immediate, hence the switch.
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
#define CM_WAIT_CASE(k) case k: wait_vmcnt<k>(); break;
#define CM_WAIT_8(b) CM_WAIT_CASE(b) CM_WAIT_CASE(b + 1) CM_WAIT_CASE(b + 2) CM_WAIT_CASE(b + 3) \
  CM_WAIT_CASE(b + 4) CM_WAIT_CASE(b + 5) CM_WAIT_CASE(b + 6) CM_WAIT_CASE(b + 7)
    CM_WAIT_8(0) CM_WAIT_8(8) CM_WAIT_8(16) CM_WAIT_8(24) CM_WAIT_8(32) CM_WAIT_8(40) CM_WAIT_8(48) CM_WAIT_8(56)
#undef CM_WAIT_8
#undef CM_WAIT_CASE
    default: wait_vmcnt<0>(); break;
  }
}

// 16 bytes per lane from a buffer (byte offset voff + soff from its base) into
// LDS: lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, char *dst, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voff, soff, 0, 0);
}

// The epilogue variant for one job: mode bit 0 = fp32 output, 1 = in0, 2 = in1.
template <int TM, int TN, bool HB>
__device__ __forceinline__ void epilogue_mode(const f32x16 (&acc)[TM][TN], const EpiArgs &ea, int mode) {
  switch (mode) {
    case 0: epilogue<TM, TN, false, false, false, HB>(acc, ea); break;
    case 1: epilogue<TM, TN, true, false, false, HB>(acc, ea); break;
    case 2: epilogue<TM, TN, false, true, false, HB>(acc, ea); break;
    case 3: epilogue<TM, TN, true, true, false, HB>(acc, ea); break;
    case 6: epilogue<TM, TN, false, true, true, HB>(acc, ea); break;
    case 7: epilogue<TM, TN, true, true, true, HB>(acc, ea); break;
    case 4: epilogue<TM, TN, false, false, true, HB>(acc, ea); break;
    default: epilogue<TM, TN, true, false, true, HB>(acc, ea); break;
  }
}

// ADD: the launch has jobs that add in0/in1 in the epilogue.  Launches
// without addends get their own instantiation, whose register allocation
// is not sized for the addend reads.
template <int BM, int BN, int WM, int WN, int BK, int AST, int BST, int NL, bool ADD>
__global__ __launch_bounds__(64 * (WM * WN) + 64 * NL) void gemm_jobs_kernel(const GemmParams p) {
  // A (activations, shared by every tile of a job and mostly served from L2)
  // and B (weights, streamed from HBM once per launch) have separate LDS
  // rings of AST and BST slabs, so each stream gets its own prefetch depth.
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // MFMA tiles per wave
  constexpr int KS = BK / 16;                   // MFMA K steps per slab
  constexpr int ROWB = 2 * BK, CH = BK / 8, RPG = 1024 / ROWB, RPB = 256 / ROWB;
  constexpr int A_GROUPS = BM / RPG, B_GROUPS = BN / RPG;  // 1 KB load groups per slab
  constexpr int A_SLAB = BM * ROWB, B_SLAB = BN * ROWB;
  constexpr int MW = WM * WN;  // MFMA waves: 8 (two per SIMD) or 4 (one per SIMD, larger wave tiles)
  static_assert(MW == 8 || MW == 4, "four or eight MFMA waves");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
  static_assert(BK == 32 || BK == 64, "slab depth");
  // NL = 0: the eight MFMA waves also issue the loads.  NL > 0: NL extra
  // waves issue every load and the eight MFMA waves never wait on the vector
  // memory pipe (a wave that issues a load behind a full address queue
  // stalls, and with it the MFMAs queued behind the load).
  constexpr int NLW = NL > 0 ? NL : MW;  // waves that issue loads
  static_assert(NL == 0 || NL == 2 || NL == 4, "loader waves");
  static_assert(A_GROUPS % NLW == 0 && B_GROUPS % NLW == 0, "loads split evenly over the waves");
  static_assert(AST >= 2 && BST >= 2 && AST <= 6 && BST <= 6, "stages");
  static_assert(AST * A_SLAB + BST * B_SLAB <= 160 * 1024, "LDS");
  constexpr int LA = A_GROUPS / NLW, LB = B_GROUPS / NLW;  // loads per loading wave per slab
  static_assert((LA + LB) * ((AST > BST ? AST : BST) - 1) < 64, "outstanding loads within vmcnt range");

  __shared__ __attribute__((aligned(1024))) char smem[AST * A_SLAB + BST * B_SLAB];
  char *const sA = smem;
  char *const sB = smem + AST * A_SLAB;

  const int lb = logical_block();
  // Jobs come in groups of jobs_per_b that share B.  Within a group the
  // blocks run B column by B column, and for each column every job's row
  // tiles in turn, so the group's tiles that read one B panel are dispatched
  // together and the panel is fetched from HBM once.
  int job, tile;
  {
    const int jpb = p.jobs_per_b > 1 ? p.jobs_per_b : 1;
    const int gt = p.tiles_per_job * jpb;
    const int grp = lb / gt;
    int r = lb - grp * gt;
    const int per_col = jpb * p.tiles_m;
    const int col = r / per_col;
    r -= col * per_col;
    const int jj = r / p.tiles_m;
    job = grp * jpb + jj;
    tile = col * p.tiles_m + (r - jj * p.tiles_m);
  }
  const int tm0 = (tile % p.tiles_m) * BM;
  const int tn0 = (tile / p.tiles_m) * BN;
  const uint32_t sel = p.sel[job];

  const char *Abase = p.base[sel & 3] + (size_t)p.a_off[job] * 16;
  const char *Bbase = p.base[(sel >> 2) & 3] + (size_t)p.b_off[job] * 16;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const bool loader = NL == 0 || wave >= MW;  // this wave issues loads
  const int lw = NL == 0 ? wave : (wave >= MW ? wave - MW : 0);  // its index among the loading waves

  // Direct-to-LDS addressing: load i of loading wave w fills the 1 KB group
  // (NLW i + w); lane l writes position l % CH of row l / CH of the group,
  // which holds the swizzled K-chunk.
  // Byte offsets from the job's A and B base (each operand of a job spans
  // less than 4 GiB; the planner rejects larger shapes).
  uint32_t a_src[LA];
  uint32_t b_src[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int row = (i * NLW + lw) * RPG + lane / CH;
    const int chunk = (lane % CH) ^ ((row / RPB) % CH);
    a_src[i] = ((uint32_t)min(tm0 + row, p.M - 1) * (uint32_t)p.lda + chunk * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int row = (i * NLW + lw) * RPG + lane / CH;
    const int chunk = (lane % CH) ^ ((row / RPB) % CH);
    b_src[i] = ((uint32_t)min(tn0 + row, p.N - 1) * (uint32_t)p.ldb + chunk * 8) * 2;
  }
  // Buffer loads into LDS (not the FLAT global_load_lds): the compiler counts
  // them on the vector-memory counter only, so its waits for the MFMA waves'
  // own LDS fragment reads stay exact (a FLAT load that may touch LDS made it
  // drain every LDS read); measured 2-5% faster on these tiles.
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(Abase), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(Bbase), (short)0, -1, 0x00020000);
  auto issue_a = [&](int kt) {
    char *slab = sA + (kt % AST) * A_SLAB;
    const uint32_t koff = (uint32_t)kt * BK * 2;
#pragma unroll
    for (int i = 0; i < LA; ++i) lds_dma16(rA, slab + (i * NLW + lw) * 1024, a_src[i], (int)koff);
  };
  auto issue_b = [&](int kt) {
    char *slab = sB + (kt % BST) * B_SLAB;
    const uint32_t koff = (uint32_t)kt * BK * 2;
#pragma unroll
    for (int i = 0; i < LB; ++i) lds_dma16(rB, slab + (i * NLW + lw) * 1024, b_src[i], (int)koff);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Issue schedule: iteration j (j >= 0, and the prologue as j < 0) issues
  // A slab j+AST-1 and then B slab j+BST-1, so A runs AST-1 slabs ahead of
  // its use and B runs BST-1 slabs ahead.
  const int KT = p.K / BK;
  constexpr int LEAD = (AST > BST ? AST : BST) - 1;
  auto issue_iter = [&](int j) {
    if (j + AST - 1 >= 0 && j + AST - 1 < KT) issue_a(j + AST - 1);
    if (j + BST - 1 >= 0 && j + BST - 1 < KT) issue_b(j + BST - 1);
  };
  // Loads issued after both of slab kt's loads, when iteration kt starts:
  // they may stay outstanding (loads complete in issue order).
  auto younger_than = [&](int kt) -> int {
    const int ja = kt - AST + 1, jb = kt - BST + 1;  // iterations that issued A kt, B kt
    int allow = 0;
    int first;  // first iteration all of whose loads are younger
    if (ja > jb) {  // A kt is the later one; B of the same iteration follows it
      if (ja + BST - 1 < KT) allow += LB;
      first = ja + 1;
    } else {
      first = jb + 1;
    }
    for (int j = first; j < kt; ++j) {
      if (j + AST - 1 >= 0 && j + AST - 1 < KT) allow += LA;
      if (j + BST - 1 >= 0 && j + BST - 1 < KT) allow += LB;
    }
    return allow;
  };

  const int frow = lane & 31, fgrp = lane >> 5;
  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = wm * WTM + i * 32 + frow;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_row[j] = wn * WTN + j * 32 + frow;
  bf16x8 fa[2][TM], fb[2][TN];
  auto load_frags = [&](const char *slab_a, const char *slab_b, int ks, int set) {
    const int chunk = ks * 2 + fgrp;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[set][i] = *reinterpret_cast<const bf16x8 *>(slab_a + a_row[i] * ROWB + ((chunk ^ ((a_row[i] / RPB) % CH)) << 4));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[set][j] = *reinterpret_cast<const bf16x8 *>(slab_b + b_row[j] * ROWB + ((chunk ^ ((b_row[j] / RPB) % CH)) << 4));
  };
  auto wait_slab = [&](int kt) { wait_vmcnt_upto(younger_than(kt)); };
  auto compute_slab = [&](int kt) {
    const char *slab_a = sA + (kt % AST) * A_SLAB;
    const char *slab_b = sB + (kt % BST) * B_SLAB;
    load_frags(slab_a, slab_b, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load_frags(slab_a, slab_b, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0, 0, 0);
    }
  };

  // Barrier kt separates the reads of slab kt-1 (every MFMA wave is past
  // them) from the loads issued after it into that slab's buffer, and makes
  // slab kt, which every loading wave waited for before it, visible.
  if (loader) {
#pragma unroll
    for (int j = -LEAD; j < 0; ++j) issue_iter(j);
  }
  if (NL == 0) {
    for (int kt = 0; kt < KT; ++kt) {
      wait_slab(kt);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue_iter(kt);
      compute_slab(kt);
    }
  } else if (loader) {
    for (int kt = 0; kt < KT; ++kt) {
      wait_slab(kt);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue_iter(kt);
    }
    return;
  } else {
    for (int kt = 0; kt < KT; ++kt) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      compute_slab(kt);
    }
  }

  // Epilogue.  Accumulator element e of a 32x32 tile sits at row
  // 8*(e/4) + 4*(lane/32) + e%4 and column lane%32.
  EpiArgs ea;
  ea.C = p.base[(sel >> 4) & 3] + (size_t)p.c_off[job] * 16;
  ea.In0 = p.base[3] + (size_t)p.in0_off[job] * 16;
  ea.In1 = p.base[3] + (size_t)p.in1_off[job] * 16;
  ea.ldc = p.ldc;
  ea.ld_in = p.ld_in;
  ea.M = p.M;
  ea.N = p.N;
  ea.row0 = tm0 + wm * WTM + 4 * fgrp;
  ea.col0 = tn0 + wn * WTN + (lane & 31);
  const int mode = (p.c_f32 ? 1 : 0) | (((sel >> 6) & 1) << 1) | (((sel >> 7) & 1) << 2);
  if (!ADD) {
    if (p.act == 1) {
      if (mode & 1)
        epilogue<TM, TN, true, false, false, false, true>(acc, ea);
      else
        epilogue<TM, TN, false, false, false, false, true>(acc, ea);
    } else if (mode & 1) {
      epilogue<TM, TN, true, false, false, false>(acc, ea);
    } else {
      epilogue<TM, TN, false, false, false, false>(acc, ea);
    }
    return;
  }
  if (p.add_bf16)
    epilogue_mode<TM, TN, true>(acc, ea, mode);
  else
    epilogue_mode<TM, TN, false>(acc, ea, mode);
}

// C = act(B_0 + B_1 + ... + B_{S-1} (+ in1)) over rows x cols per job, added
// in that order in fp32, where B_s is the fp32 block of rows x ld_in at
// in0 + s * rows * ld_in and S = max(1, K); 4 columns per thread.  PAIR: the
// launch is C = in0 + in1 for every job (S = 1, in1 present, no activation):
// the ring's add-and-forward, in its own instantiation, with non-temporal
// loads and stores (it streams beside the step GEMMs; measured 4% faster GEMM
// launches on the GPT-3 fc2 ring than with cached accesses).
typedef float f32x4nt __attribute__((ext_vector_type(4)));  // for the non-temporal builtins

template <bool PAIR>
__global__ __launch_bounds__(256) void reduce_jobs_kernel(const GemmParams p) {
  const int job = blockIdx.y;
  const uint32_t sel = p.sel[job];
  const float *In0 = reinterpret_cast<const float *>(p.base[3] + (size_t)p.in0_off[job] * 16);
  const float *In1 = reinterpret_cast<const float *>(p.base[3] + (size_t)p.in1_off[job] * 16);
  char *Cbase = p.base[(sel >> 4) & 3] + (size_t)p.c_off[job] * 16;
  const bool has1 = PAIR || ((sel >> 7) & 1);
  const int S = PAIR ? 1 : (p.K > 1 ? p.K : 1);
  const size_t bstride = (size_t)p.M * p.ld_in;
  const int cols4 = p.N >> 2;
  const long total = (long)p.M * cols4;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (long)gridDim.x * blockDim.x) {
    const int row = (int)(t / cols4), c4 = (int)(t - (long)row * cols4) * 4;
    const size_t ii = (size_t)row * p.ld_in + c4;
    float4 v;
    if (PAIR) {
      const f32x4nt x = __builtin_nontemporal_load(reinterpret_cast<const f32x4nt *>(In0 + ii));
      v = make_float4(x[0], x[1], x[2], x[3]);
    } else {
      v = *reinterpret_cast<const float4 *>(In0 + ii);
    }
    if (!PAIR) {
      for (int b = 1; b < S; ++b) {
        const float4 a = *reinterpret_cast<const float4 *>(In0 + (size_t)b * bstride + ii);
        v = make_float4(v.x + a.x, v.y + a.y, v.z + a.z, v.w + a.w);
      }
    }
    if (has1) {
      float4 a;
      if (PAIR) {
        const f32x4nt x = __builtin_nontemporal_load(reinterpret_cast<const f32x4nt *>(In1 + ii));
        a = make_float4(x[0], x[1], x[2], x[3]);
      } else {
        a = *reinterpret_cast<const float4 *>(In1 + ii);
      }
      v = make_float4(v.x + a.x, v.y + a.y, v.z + a.z, v.w + a.w);
    }
    if (!PAIR && p.act == 1) v = make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w));
    const size_t oc = (size_t)row * p.ldc + c4;
    if (p.c_f32) {
      if (PAIR)
        __builtin_nontemporal_store((f32x4nt){v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4nt *>(reinterpret_cast<float *>(Cbase) + oc));
      else
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(Cbase) + oc) = v;
    } else {
      uint2 o;
      o.x = f32_to_bf16_rne(v.x) | (f32_to_bf16_rne(v.y) << 16);
      o.y = f32_to_bf16_rne(v.z) | (f32_to_bf16_rne(v.w) << 16);
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(Cbase) + oc) = o;
    }
  }
}

// Sleep for about units * 8 us (one wave; s_sleep 127 is 8128 clocks).
__global__ void sleep_kernel(int units) {
  for (int i = 0; i < units * 2; ++i) __builtin_amdgcn_s_sleep(127);
}

// rows x row_bytes bytes, ld_bytes apart, set to 0xFF (4 bytes per thread).
__global__ void fill_ff_kernel(char *p, long rows, long row_words, long ld_bytes) {
  const long total = rows * row_words;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (long)gridDim.x * blockDim.x) {
    const long r = t / row_words, w = t - r * row_words;
    reinterpret_cast<uint32_t *>(p + r * ld_bytes)[w] = 0xFFFFFFFFu;
  }
}

}  // namespace

hipError_t launch_sleep(int units, hipStream_t s) {
  void *args[] = {&units};
  return hipLaunchKernel(reinterpret_cast<void *>(&sleep_kernel), dim3(1), dim3(64), args, 0, s);
}

hipError_t launch_fill_ff(char *p, long rows, long row_bytes, long ld_bytes, hipStream_t s) {
  const long words = rows * (row_bytes / 4);
  if (words <= 0) return hipSuccess;
  long blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  long row_words = row_bytes / 4;
  void *args[] = {&p, &rows, &row_words, &ld_bytes};
  return hipLaunchKernel(reinterpret_cast<void *>(&fill_ff_kernel), dim3((unsigned)blocks), dim3(256), args, 0, s);
}

bool gemm_tile_supported(int tm, int tn) {
  KernelLaunch L;
  GemmParams p{};
  return gemm_launch_config(p, tm, tn, &L);
}

template <int BM, int BN, int WM, int WN, int BK, int AST, int BST, int NL>
void pick_gemm(bool add, void **f, int *threads) {
  *f = add ? reinterpret_cast<void *>(&gemm_jobs_kernel<BM, BN, WM, WN, BK, AST, BST, NL, true>)
           : reinterpret_cast<void *>(&gemm_jobs_kernel<BM, BN, WM, WN, BK, AST, BST, NL, false>);
  *threads = 64 * (WM * WN) + 64 * NL;
}

bool gemm_launch_config(const GemmParams &p, int tm, int tn, KernelLaunch *out) {
  bool add = false;  // does any job read in0 or in1?
  for (int j = 0; j < p.n_jobs && j < kMaxJobs; ++j) add = add || (p.sel[j] & 0xC0);
  void *f = nullptr;
  int threads = 0;
  if (tm == 256 && tn == 256) pick_gemm<256, 256, 2, 4, 64, 2, 3, 4>(add, &f, &threads);
  else if (tm == 256 && tn == 192) pick_gemm<256, 192, 4, 2, 64, 2, 4, 4>(add, &f, &threads);
  else if (tm == 256 && tn == 128) pick_gemm<256, 128, 4, 2, 64, 2, 5, 0>(add, &f, &threads);
  else if (tm == 128 && tn == 256) pick_gemm<128, 256, 2, 4, 64, 2, 3, 0>(add, &f, &threads);
  else if (tm == 128 && tn == 128) pick_gemm<128, 128, 2, 4, 64, 3, 4, 0>(add, &f, &threads);
  else if (tm == 64 && tn == 256) pick_gemm<64, 256, 2, 4, 64, 2, 3, 0>(add, &f, &threads);
  if (!f) return false;
  out->func = f;
  out->grid = dim3(p.n_jobs * p.tiles_per_job);
  out->block = dim3(threads);
  return true;
}

void reduce_launch_config(const GemmParams &p, KernelLaunch *out) {
  const long per_job = (long)p.M * (p.N / 4);
  int bx = (int)((per_job + 255) / 256);
  if (bx > 1024) bx = 1024;
  if (bx < 1) bx = 1;
  bool pair = p.K <= 1 && p.act == 0;  // every job: in0 + in1
  for (int j = 0; j < p.n_jobs && j < kMaxJobs; ++j) pair = pair && ((p.sel[j] >> 7) & 1);
  out->func = pair ? reinterpret_cast<void *>(&reduce_jobs_kernel<true>) : reinterpret_cast<void *>(&reduce_jobs_kernel<false>);
  out->grid = dim3(bx, p.n_jobs);
  out->block = dim3(256);
}

hipError_t launch_gemm(const GemmParams &p, int tm, int tn, hipStream_t s) {
  KernelLaunch L;
  if (!gemm_launch_config(p, tm, tn, &L)) return hipErrorInvalidValue;
  void *args[] = {const_cast<GemmParams *>(&p)};
  return hipLaunchKernel(L.func, L.grid, L.block, args, 0, s);
}

hipError_t launch_reduce(const GemmParams &p, hipStream_t s) {
  KernelLaunch L;
  reduce_launch_config(p, &L);
  void *args[] = {const_cast<GemmParams *>(&p)};
  return hipLaunchKernel(L.func, L.grid, L.block, args, 0, s);
}

}  // namespace collmm
