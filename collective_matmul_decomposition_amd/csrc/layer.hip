// The sequence-parallel transformer layer around the two decomposed
// collective matmuls: the stages between them (causal attention, LayerNorm on
// the sequence shard) and the layer forward that chains
//
//   AllGather -> QKV projection      (cm_ag_gemm, decomposed)
//   attention, every rank's heads    (attn_fwd_kernel)
//   output projection -> ReduceScatter (cm_gemm_rs, pipeline chunks)
//   LayerNorm on the [m x d] shard   (layernorm_kernel)
//   AllGather -> fc1, GELU fused     (cm_ag_gemm, decomposed)
//   fc2 -> ReduceScatter             (cm_gemm_rs, decomposed)
//
// The Megatron page's sequence parallelism places the LayerNorm on the
// sequence-sharded activation between the ReduceScatter of one block and the
// AllGather of the next; "Tensor Parallelism > Communication Patterns" notes
// the same point, between the two halves of an all-reduce.  The pages give no
// formulas for attention, LayerNorm or the activation: the kernels compute the
// textbook definitions (scaled dot-product attention with a causal mask,
// population-variance LayerNorm, GELU in its erf form).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstring>

#include "collmm.h"
#include "internal.h"

namespace collmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *attn_lds_ptr;
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------------------ attention
//
// One workgroup: 128 query rows of one head of one virtual rank; 4 waves of
// 32 query rows each.  Keys and values stream through LDS in blocks of 64.
// The scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
// keys as rows), so that every lane of a wave owns one query: the running
// maximum, the exponentials and the running sum stay in the lane (plus one
// exchange with the lane 32 away, which holds the other half of the block's
// keys for the same query).  The output is accumulated transposed as well,
// O^T += V^T P^T: the probabilities are the B operand straight from the
// score registers (rounded to bf16), and V is written to LDS transposed.
// Within a 16-key MFMA step lane group g supplies keys {4g..4g+3, 8+4g..8+4g+3}
// of P and of V^T alike; the contraction only needs the two operands to agree.
// The probabilities' bf16 values feed both the numerator and the running sum,
// so every output row is a convex combination of the value rows.  The kernel
// is held to two waves per SIMD (accumulators in VGPRs, no AGPR moves); blocks
// entirely below the causal diagonal skip the mask, and the output is
// rescaled only when some lane's running maximum outgrows the reference of
// the exponentials by more than a fixed headroom (lazy rescaling).
constexpr int kAttnD = 128;   // head dimension
constexpr int kAttnBQ = 128;  // query rows per workgroup
constexpr int kAttnBK = 64;   // keys per block (one softmax update)
constexpr float kAttnLazy = 8.f;  // headroom of the lazy rescale, base 2

struct AttnParams {
  const uint16_t *qkv;  // [N][T][3*H*D]
  uint16_t *o;          // [N][T][H*D]
  int T, H;
  int ld_qkv, ld_o;     // row strides in elements
  int causal;
  int qblocks;          // ceil(T / 128)
  float scale_log2;     // log2(e) / sqrt(D)
};

// Combine a lane's value with the one of the lane 32 away (the other half of
// the same query's keys): v_permlane32_swap exchanges the wave's two halves
// between two registers, so each lane holds both values, lower half's first;
// both lanes of a pair get the same bits.  max when `mx`, else the sum.
__device__ __forceinline__ float half_pair(float v, bool mx) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
  return mx ? fmaxf(lo, hi) : lo + hi;
}

__device__ __forceinline__ int attn_logical_block() {
  // block b runs on XCD b % 8: give each XCD a contiguous range of logical
  // blocks, so the query blocks of one head (which share its keys and values)
  // meet in one L2
  const int G = gridDim.x, b = blockIdx.x;
  const int per = G >> 3;
  return b < per * 8 ? (b & 7) * per + (b >> 3) : b;
}

// Workgroup barrier without a memory fence: this wave's LDS stores are
// complete, then s_barrier.  (__syncthreads() would also wait for every
// outstanding global load, including the next block's prefetch.)
__device__ __forceinline__ void attn_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keys and values are read by buffer loads from the rank's QKV rows: byte
// offsets from the rank's base, which the buffer's size (T rows) bounds, so
// that rows past the sequence read as zeros (the hardware's range check; their
// scores are masked, and their zero values meet zero probabilities).  Each
// thread's offsets within a block are fixed; a block adds k0 rows.
//
// One block of keys straight into its LDS buffer (a buffer load into LDS:
// lane l of a wave's load lands at the wave's 1 KB base + 16 l, no
// registers; as a buffer load the compiler counts it on the vector-memory
// counter only, so its waits for this wave's own LDS reads stay exact): load i
// of wave w fills keys 4 (4 i + w) .. +3; lane l writes position l % 16 of key
// row l / 16, which holds the row's chunk (l % 16) ^ (key % 16).
__device__ __forceinline__ void attn_k_offsets(int ld, int kcol, int wave, int lane, uint32_t (&ko)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grp = 4 * i + wave, key = 4 * grp + (lane >> 4), ch = (lane & 15) ^ (key & 15);
    ko[i] = ((uint32_t)key * (uint32_t)ld + (uint32_t)(kcol + 8 * ch)) * 2u;
  }
}
__device__ __forceinline__ void attn_load_k(__amdgpu_buffer_rsrc_t r, const uint32_t (&ko)[4], uint32_t kbytes,
                                            int wave, char *sKbuf) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (attn_lds_ptr)(sKbuf + (4 * i + wave) * 1024), 16, ko[i] + kbytes, 0,
                                             0, 0);
}

// One block of values into registers: 4 keys x 8 dims per thread.  Thread t
// takes keys 4 (t % 16) .. +3 and dims 8 (t / 16) .. +7, so that the 16 lanes
// that store to LDS together (attn_store_v) write the 16 units of one V^T row:
// 128 contiguous bytes, every bank once (with the dims spread over the lanes
// instead, the 16 lanes hit two 16-byte chunks, an 8-way bank conflict).
__device__ __forceinline__ void attn_v_offsets(int ld, int vcol, int tid, uint32_t (&vo)[4]) {
  const int dg = tid >> 4, kgp = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) vo[i] = ((uint32_t)(4 * kgp + i) * (uint32_t)ld + (uint32_t)(vcol + 8 * dg)) * 2u;
}
__device__ __forceinline__ void attn_load_v(__amdgpu_buffer_rsrc_t r, const uint32_t (&vo)[4], uint32_t kbytes,
                                            uint4 (&vr)[4]) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, vo[i] + kbytes, 0, 0);
    vr[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// Byte offset, within its 128-byte V^T row, of the 8-byte unit u (keys
// 4u .. 4u + 3) of dim row `dim`.  The units that one 16-key MFMA step reads
// together, u and u + 2 with u % 4 < 2, share a 16-byte chunk
// (u / 4 * 2 + u % 2) in that order; chunks are XOR-swizzled by dim / 2 mod 8,
// so the 16 rows that a 16-lane phase of the operand read touches cover the
// 64 banks once.
__device__ __forceinline__ int attn_vt_unit(int dim, int u) {
  const int chunk = ((u >> 2) << 1) | (u & 1), half = (u >> 1) & 1;
  return ((chunk ^ ((dim >> 1) & 7)) << 4) | (half << 3);
}

// V transposed into V^T units of 4 keys.  Unit e (dim 8 dg + e) takes the
// 16-bit half e % 2 of register word e / 2 of the four keys' loads, two keys
// per 32-bit word with one byte permute (v_perm_b32: selector bytes 0-3 pick
// bytes of the second operand, 4-7 of the first).
__device__ __forceinline__ void attn_store_v(char *sV, int tid, const uint4 (&vr)[4]) {
  const int dg = tid >> 4, kgp = tid & 15;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    auto comp = [&](int i) -> uint32_t {
      const uint4 &v = vr[i];
      return (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    };
    uint2 pk;
    pk.x = __builtin_amdgcn_perm(comp(1), comp(0), sel);
    pk.y = __builtin_amdgcn_perm(comp(3), comp(2), sel);
    const int dim = 8 * dg + e;
    *reinterpret_cast<uint2 *>(sV + dim * 128 + attn_vt_unit(dim, kgp)) = pk;
  }
}

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const AttnParams p) {
  // K block [64 keys][128 dims]: 256-byte rows of 16 chunks of 16 bytes,
  // chunk c of key row r stored at position c ^ (r % 16).
  // Two K buffers, separate objects so that the compiler can tell the next
  // block's loads into one from this block's reads of the other.
  __shared__ __attribute__((aligned(1024))) char sK0[kAttnBK * kAttnD * 2];
  __shared__ __attribute__((aligned(1024))) char sK1[kAttnBK * kAttnD * 2];
  // V^T block [128 dims][64 keys]: 128-byte rows of 16 units of 4 keys,
  // placed by attn_vt_unit.
  __shared__ __attribute__((aligned(16))) char sV[kAttnD * kAttnBK * 2];

  const int lb = attn_logical_block();
  const int bh = lb / p.qblocks;
  const int qb = p.qblocks - 1 - (lb - bh * p.qblocks);  // long (late) query blocks first
  const int rank = bh / p.H, head = bh - rank * p.H;
  const uint16_t *base = p.qkv + (size_t)rank * p.T * p.ld_qkv;
  const int qcol = head * kAttnD, kcol = (p.H + head) * kAttnD, vcol = (2 * p.H + head) * kAttnD;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int q0 = qb * kAttnBQ + wave * 32;  // the wave's first query
  const int my_q = q0 + l32;                // the lane's query

  // B operand of S^T = K Q^T: lane (query l32, group g) holds
  // Q[my_q][16 ks + 8 g .. + 8] for the 8 MFMA steps over D = 128.
  bf16x8 qf[8];
  {
    const uint16_t *qrow = base + (size_t)min(my_q, p.T - 1) * p.ld_qkv + qcol + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * ks);
  }

  f32x16 oacc[4];  // O^T tiles: dims 32 dt .. 32 dt + 31 x this wave's queries
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = p.causal ? min(p.T, (qb + 1) * kAttnBQ) : p.T;
  const int nblk = (kv_end + kAttnBK - 1) / kAttnBK;

  // Block j + 1's keys stream into the other K buffer, and its values into
  // registers, while block j is multiplied.  The wait for the values (which
  // the compiler places before their LDS store) also covers the keys, which
  // were issued before them: vector-memory loads complete in order.
  uint4 vreg[4];
  // the rank's T rows of QKV; reads past them return zeros
  const __amdgpu_buffer_rsrc_t rqkv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(base), (short)0, (int)((uint32_t)p.T * (uint32_t)p.ld_qkv * 2u), 0x00020000);
  uint32_t ko[4], vo[4];
  attn_k_offsets(p.ld_qkv, kcol, wave, lane, ko);
  attn_v_offsets(p.ld_qkv, vcol, tid, vo);
  const uint32_t blk_bytes = (uint32_t)kAttnBK * (uint32_t)p.ld_qkv * 2u;  // one block of rows
  attn_load_k(rqkv, ko, 0u, wave, sK0);
  attn_load_v(rqkv, vo, 0u, vreg);
  // one block: its keys in sKb, the next block's keys stream into sKn
  auto block = [&](const int j, const char *sKb, char *sKn) __attribute__((always_inline)) {
    const int k0 = j * kAttnBK;
    attn_barrier();  // every wave is done with block j - 1 (V^T and the other K buffer)
    attn_store_v(sV, tid, vreg);  // the compiler waits for vreg here: block j's keys are in LDS too
    if (j + 1 < nblk) {
      attn_load_k(rqkv, ko, (uint32_t)(j + 1) * blk_bytes, wave, sKn);
      attn_load_v(rqkv, vo, (uint32_t)(j + 1) * blk_bytes, vreg);
    }
    attn_barrier();  // block j's keys and values are in LDS, for every wave
    if (p.causal && k0 > q0 + 31) return;  // every key of the block is after every query of the wave
    const char *sVb = sV;

    // S^T = K Q^T for keys k0 .. k0 + 63 (two 32-key tiles).  The key
    // fragments of step ks + 1 are read from LDS while step ks multiplies.
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[t][e] = 0.f;
    bf16x8 kf[2][2];
    auto load_kf = [&](int ks, int set) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key = t * 32 + l32, ch = 2 * ks + g;
        kf[set][t] = *reinterpret_cast<const bf16x8 *>(sKb + key * 256 + ((ch ^ (key & 15)) << 4));
      }
    };
    load_kf(0, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 1 < 8) load_kf(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int t = 0; t < 2; ++t) s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks & 1][t], qf[ks], s[t], 0, 0, 0);
    }
    // keep that order through scheduling: reads of step ks + 1, then the MFMAs of step ks
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // V^T fragments of the first 16-key step of O^T += V^T P^T: they do not
    // depend on the softmax, so their reads are in flight during it.  Step
    // q = 2 t + h covers keys 32 t + 16 h .. + 15; lane group g supplies the
    // units u0 = 8 t + 4 h + g and u0 + 2 (one 16-byte chunk).
    bf16x8 vf[2][4];
    auto load_vf = [&](int q, int set) __attribute__((always_inline)) {
      const int u0 = (q >> 1) * 8 + (q & 1) * 4 + g;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dim = dt * 32 + l32;
        vf[set][dt] = *reinterpret_cast<const bf16x8 *>(sVb + dim * 128 + attn_vt_unit(dim, u0));
      }
    };
    load_vf(0, 0);
    // online softmax: element e of tile t is key k0 + 32 t + 8 (e / 4) + 4 g + e % 4.
    // The mask is needed only where a key can lie after a query of the wave or
    // past the sequence; a key is kept while its offset 32 t + 8 (e / 4) + e % 4
    // is at most `lim` (one comparison with a per-lane limit, no branch).
    const bool masked = (p.causal && k0 + kAttnBK - 1 > q0) || k0 + kAttnBK > p.T;
    if (masked) {
      const int lim = (p.causal ? min(my_q, p.T - 1) : p.T - 1) - k0 - 4 * g;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * t + 8 * (e >> 2) + (e & 3) > lim) s[t][e] = -INFINITY;
    }
    // the maximum of the raw scores: the scale is positive, and rounding is
    // monotone, so scaling the maximum gives the maximum of the scaled scores
    // (four independent chains, then the lane 32 away through a lane swap)
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) m4[e & 3] = fmaxf(m4[e & 3], s[t][e]);
    float mloc = half_pair(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])), true);
    // Lazy rescaling: the reference point of the exponentials (m_run) moves
    // only when some lane's maximum has grown past it by more than
    // kAttnLazy (base 2); until then the probabilities are taken against the
    // older, smaller reference and stay below 2^kAttnLazy.  Numerator and
    // normaliser share the reference, so it cancels in O = (P V) / l.
    const float m_cand = fmaxf(m_run, mloc * p.scale_log2);
    const bool grow = __any(!(m_cand <= m_run + kAttnLazy));
    const float m_new = grow ? m_cand : m_run;
    const float msub = m_new == -INFINITY ? 0.f : m_new;
    // exponentials with the hardware's base-2 exponential (v_exp_f32; results
    // below 2^-126 may flush to zero, far inside the error bound), the scale
    // and the subtraction of the reference in one fused multiply-add
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - msub) : 1.f;  // 0 on the first block
    // elements e, e + 1 are converted together (nearest even) into one register
    // of the B operand; the running sum adds the same bf16 values, two at a
    // time (a dot product with ones)
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 pf[2][2];
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 8 * h + 2 * q;
          const f32x2 x = {__builtin_amdgcn_exp2f(__builtin_fmaf(s[t][e], p.scale_log2, -msub)),
                           __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][e + 1], p.scale_log2, -msub))};
          const bf16x2 b = __builtin_convertvector(x, bf16x2);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(b, ones, lsum, false);
          w[q] = __builtin_bit_cast(uint32_t, b);
        }
        pf[t][h] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      }
    lsum = half_pair(lsum, false);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    if (grow) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
    }

    // O^T += V^T P^T over the block's 64 keys (four 16-key steps), the next
    // step's V^T fragments read while this one multiplies
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q + 1 < 4) load_vf(q + 1, (q + 1) & 1);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[q & 1][dt], pf[q >> 1][q & 1], oacc[dt], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
    }
  };
  for (int j = 0; j < nblk; j += 2) {
    block(j, sK0, sK1);
    if (j + 1 < nblk) block(j + 1, sK1, sK0);
  }

  if (my_q >= p.T) return;
  const float inv = 1.f / l_run;
  uint16_t *orow = p.o + ((size_t)rank * p.T + my_q) * p.ld_o + head * kAttnD;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int eg = 0; eg < 4; ++eg) {
      // elements 4 eg .. 4 eg + 3: dims 32 dt + 8 eg + 4 g .. +3, rounded to nearest even
      bf16x4 o4;
#pragma unroll
      for (int q = 0; q < 4; ++q) o4[q] = (__bf16)(oacc[dt][4 * eg + q] * inv);
      *reinterpret_cast<bf16x4 *>(orow + dt * 32 + 8 * eg + 4 * g) = o4;
    }
}

// ------------------------------------------------------------------ LayerNorm
//
// One workgroup of 256 threads per row; the row (fp32) stays in registers,
// VPT float4 per thread: the mean, then the variance about it (two passes over
// registers, fp32), then y = (x - mean) / sqrt(var + eps) * gamma + beta,
// rounded to bf16.
__device__ __forceinline__ float block_sum_256(float v, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red is reused by consecutive sums
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

template <int VPT>
__global__ __launch_bounds__(256) void layernorm_kernel(const float *x, uint16_t *y, int cols, float eps,
                                                         const float *gamma, const float *beta) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const float *xr = x + row * cols;
  uint16_t *yr = y + row * cols;
  const int c4 = cols >> 2;
  float4 v[VPT];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = threadIdx.x + 256 * i;
    v[i] = idx < c4 ? reinterpret_cast<const float4 *>(xr)[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = block_sum_256(s, red) / cols;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    if (threadIdx.x + 256 * i < c4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      ss += (a * a + b * b) + (c * c + d * d);
    }
  }
  const float rstd = 1.f / sqrtf(block_sum_256(ss, red) / cols + eps);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = threadIdx.x + 256 * i;
    if (idx >= c4) continue;
    float o[4] = {(v[i].x - mean) * rstd, (v[i].y - mean) * rstd, (v[i].z - mean) * rstd, (v[i].w - mean) * rstd};
    if (gamma) {
      const float4 gm = reinterpret_cast<const float4 *>(gamma)[idx];
      o[0] *= gm.x; o[1] *= gm.y; o[2] *= gm.z; o[3] *= gm.w;
    }
    if (beta) {
      const float4 bt = reinterpret_cast<const float4 *>(beta)[idx];
      o[0] += bt.x; o[1] += bt.y; o[2] += bt.z; o[3] += bt.w;
    }
    uint2 pk;
    pk.x = bf16_bits_rne(o[0]) | (bf16_bits_rne(o[1]) << 16);
    pk.y = bf16_bits_rne(o[2]) | (bf16_bits_rne(o[3]) << 16);
    reinterpret_cast<uint2 *>(yr)[idx] = pk;
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

cm_status hip_fail(hipError_t e, const char *what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return CM_ERR_HIP;
}

cm_status gfx950_current(void) {
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

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Field-wise equality (struct padding is not part of a plan).
bool same_desc(const cm_plan_desc &a, const cm_plan_desc &b) {
  return a.op == b.op && a.n_ranks == b.n_ranks && a.m == b.m && a.k == b.k && a.n == b.n && a.dir == b.dir &&
         a.chunks == b.chunks && a.sched == b.sched && a.in_dtype == b.in_dtype && a.out_dtype == b.out_dtype &&
         a.n_comm == b.n_comm && a.tile_m == b.tile_m && a.tile_n == b.tile_n && a.exec_mode == b.exec_mode &&
         a.copy_engine == b.copy_engine && a.bucket_bf16 == b.bucket_bf16 && a.hop_add == b.hop_add &&
         a.copy_gbps == b.copy_gbps && a.mfma_tflops == b.mfma_tflops && a.launch_us == b.launch_us && a.act == b.act &&
         a.share == b.share && a.split_k == b.split_k && a.skip == b.skip && a.stress == b.stress &&
         a.group == b.group;
}
bool same_plan(const cm_plan &a, const cm_plan &b) {
  return same_desc(a.desc, b.desc) && a.chunks == b.chunks && a.n_steps == b.n_steps && a.arc_cw == b.arc_cw &&
         a.arc_ccw == b.arc_ccw && a.tile_m == b.tile_m && a.tile_n == b.tile_n && a.n_ops == b.n_ops &&
         a.n_jobs == b.n_jobs && a.n_events == b.n_events && a.ws_bytes == b.ws_bytes && a.split == b.split &&
         a.n_launches == b.n_launches && a.slots == b.slots &&
         std::memcmp(a.group_len, b.group_len, sizeof a.group_len) == 0;
}
bool same_layer(const cm_layer_plan &a, const cm_layer_plan &b) {
  const cm_layer_desc &x = a.desc, &y = b.desc;
  return x.n_ranks == y.n_ranks && x.m == y.m && x.d == y.d && x.heads == y.heads && x.head_dim == y.head_dim &&
         x.ffn == y.ffn && x.dir == y.dir && x.n_comm == y.n_comm && x.copy_engine == y.copy_engine &&
         x.exec_mode == y.exec_mode && x.ag_chunks == y.ag_chunks && x.rs_chunks == y.rs_chunks &&
         x.proj_chunks == y.proj_chunks && x.out_dtype == y.out_dtype && x.ln_eps == y.ln_eps &&
         same_plan(a.qkv, b.qkv) && same_plan(a.proj, b.proj) && same_plan(a.fc1, b.fc1) && same_plan(a.fc2, b.fc2) &&
         a.off_qkv == b.off_qkv && a.off_attn == b.off_attn && a.off_proj == b.off_proj && a.off_ln == b.off_ln &&
         a.off_fc1 == b.off_fc1 && a.off_ops == b.off_ops && a.ws_bytes == b.ws_bytes;
}

}  // namespace

cm_status attention_check(int n_ranks, int T, int heads, int head_dim, int causal) {
  if (n_ranks < 1 || n_ranks > CM_MAX_RANKS || T < 1 || heads < 1 || (causal != 0 && causal != 1)) {
    set_error("attention: need 1 <= n_ranks <= %d, T >= 1, heads >= 1, causal 0 or 1", CM_MAX_RANKS);
    return CM_ERR_INVALID_ARG;
  }
  if (head_dim != kAttnD) {
    set_error("attention: head_dim must be %d (got %d)", kAttnD, head_dim);
    return CM_ERR_UNSUPPORTED;
  }
  const long long blocks = (long long)n_ranks * heads * ((T + kAttnBQ - 1) / kAttnBQ);
  // one rank's QKV rows, and a block of rows past them, are addressed by
  // 32-bit byte offsets
  if (blocks > (1ll << 30) || (long long)(T + kAttnBK) * 3 * heads * kAttnD * 2 > 0x7FFFFFFFll) {
    set_error("attention: problem too large");
    return CM_ERR_SHAPE;
  }
  return CM_OK;
}

cm_status layernorm_check(int rows, int cols) {
  if (rows < 1 || cols < 4 || cols % 4 || cols > 16384) {
    set_error("layernorm: need rows >= 1 and 4 <= cols <= 16384 with cols a multiple of 4 (got %d x %d)", rows, cols);
    return CM_ERR_SHAPE;
  }
  if (rows > (1 << 30)) {
    set_error("layernorm: too many rows");
    return CM_ERR_SHAPE;
  }
  return CM_OK;
}

}  // namespace collmm

using namespace collmm;

extern "C" {

cm_status cm_attention(const void *qkv, void *o, int n_ranks, int T, int heads, int head_dim, int causal,
                       void *stream) {
  cm_status st = attention_check(n_ranks, T, heads, head_dim, causal);
  if (st != CM_OK) return st;
  if (!qkv || !o) { set_error("attention: null qkv or o"); return CM_ERR_INVALID_ARG; }
  if (!aligned16(qkv) || !aligned16(o)) { set_error("attention: qkv and o must be 16-byte aligned"); return CM_ERR_ALIGN; }
  if ((st = gfx950_current()) != CM_OK) return st;
  AttnParams p;
  p.qkv = static_cast<const uint16_t *>(qkv);
  p.o = static_cast<uint16_t *>(o);
  p.T = T;
  p.H = heads;
  p.ld_qkv = 3 * heads * kAttnD;
  p.ld_o = heads * kAttnD;
  p.causal = causal;
  p.qblocks = (T + kAttnBQ - 1) / kAttnBQ;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)kAttnD));
  const unsigned blocks = (unsigned)(n_ranks * heads * p.qblocks);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return CM_OK;
}

cm_status cm_layernorm(const void *x, void *y, int rows, int cols, float eps, const void *gamma, const void *beta,
                       void *stream) {
  cm_status st = layernorm_check(rows, cols);
  if (st != CM_OK) return st;
  if (!x || !y) { set_error("layernorm: null x or y"); return CM_ERR_INVALID_ARG; }
  if (!(eps >= 0.f) || std::isinf(eps)) { set_error("layernorm: eps must be finite and >= 0"); return CM_ERR_INVALID_ARG; }
  if (!aligned16(x) || !aligned16(y) || (gamma && !aligned16(gamma)) || (beta && !aligned16(beta))) {
    set_error("layernorm: x, y, gamma and beta must be 16-byte aligned");
    return CM_ERR_ALIGN;
  }
  if ((st = gfx950_current()) != CM_OK) return st;
  const float *xf = static_cast<const float *>(x);
  uint16_t *yb = static_cast<uint16_t *>(y);
  const float *gm = static_cast<const float *>(gamma), *bt = static_cast<const float *>(beta);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int vpt = (cols / 4 + 255) / 256;
  if (vpt <= 1) hipLaunchKernelGGL(layernorm_kernel<1>, dim3(rows), dim3(256), 0, s, xf, yb, cols, eps, gm, bt);
  else if (vpt <= 2) hipLaunchKernelGGL(layernorm_kernel<2>, dim3(rows), dim3(256), 0, s, xf, yb, cols, eps, gm, bt);
  else if (vpt <= 4) hipLaunchKernelGGL(layernorm_kernel<4>, dim3(rows), dim3(256), 0, s, xf, yb, cols, eps, gm, bt);
  else if (vpt <= 8) hipLaunchKernelGGL(layernorm_kernel<8>, dim3(rows), dim3(256), 0, s, xf, yb, cols, eps, gm, bt);
  else hipLaunchKernelGGL(layernorm_kernel<16>, dim3(rows), dim3(256), 0, s, xf, yb, cols, eps, gm, bt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "layernorm launch");
  return CM_OK;
}

// ------------------------------------------------------------------ the layer
cm_status cm_plan_layer(const cm_layer_desc *desc, cm_layer_plan *out) {
  if (!desc || !out) { set_error("null argument"); return CM_ERR_INVALID_ARG; }
  cm_layer_desc d = *desc;
  if (d.proj_chunks == 0) d.proj_chunks = 4;  // the pipeline-chunk ReduceScatter's default of four
  if (d.ln_eps == 0.f) d.ln_eps = 1e-5f;
  if (!(d.ln_eps > 0.f) || std::isinf(d.ln_eps)) { set_error("ln_eps must be finite and > 0"); return CM_ERR_INVALID_ARG; }
  if (d.out_dtype != CM_F32 && d.out_dtype != CM_BF16) { set_error("out_dtype must be CM_F32 or CM_BF16"); return CM_ERR_UNSUPPORTED; }
  cm_status st = attention_check(d.n_ranks, d.n_ranks * d.m, d.heads, d.head_dim, 1);
  if (st != CM_OK) return st;
  if ((st = layernorm_check(d.n_ranks * d.m, d.d)) != CM_OK) return st;
  cm_layer_plan p;
  std::memset(&p, 0, sizeof p);
  p.desc = d;
  const int N = d.n_ranks, HD = d.heads * d.head_dim;
  auto mk = [&](int op, int k, int n, int chunks, int out_dtype, int act, int hop_add) {
    cm_plan_desc q;
    std::memset(&q, 0, sizeof q);
    q.op = op;
    q.n_ranks = N;
    q.m = d.m;
    q.k = k;
    q.n = n;
    q.dir = d.dir;
    q.chunks = chunks;
    q.sched = CM_SCHED_DECOMPOSED;
    q.in_dtype = CM_BF16;
    q.out_dtype = out_dtype;
    q.n_comm = d.n_comm;
    q.exec_mode = d.exec_mode;
    q.copy_engine = d.copy_engine;
    q.act = act;
    q.hop_add = hop_add;
    return q;
  };
  const int rs_hop_add = d.dir == CM_RING_DIRECT ? 0 : 1;
  cm_plan_desc dq = mk(CM_OP_AG_GEMM, d.d, 3 * HD, d.ag_chunks, CM_BF16, CM_ACT_NONE, 0);
  cm_plan_desc dp = mk(CM_OP_GEMM_RS_PIPE, HD, d.d, d.proj_chunks, CM_F32, CM_ACT_NONE, 1);
  dp.dir = CM_RING_UNI;  // the pipeline-chunk ReduceScatter runs its own one-way copy-and-add ring
  cm_plan_desc d1 = mk(CM_OP_AG_GEMM, d.d, d.ffn, d.ag_chunks, CM_BF16, CM_ACT_GELU, 0);
  cm_plan_desc d2 = mk(CM_OP_GEMM_RS, d.ffn, d.d, d.rs_chunks, d.out_dtype, CM_ACT_NONE, rs_hop_add);
  if ((st = plan(&dq, &p.qkv)) != CM_OK) return st;
  if ((st = plan(&dp, &p.proj)) != CM_OK) return st;
  if ((st = plan(&d1, &p.fc1)) != CM_OK) return st;
  if ((st = plan(&d2, &p.fc2)) != CM_OK) return st;
  // workspace: the intermediates, then one region the four collective
  // matmuls share (they run one after another on the same streams)
  const size_t T = (size_t)N * d.m, A = 256;
  size_t off = 0;
  p.off_qkv = off; off = round_up(off + (size_t)N * T * 3 * HD * 2, A);
  p.off_attn = off; off = round_up(off + (size_t)N * T * HD * 2, A);
  p.off_proj = off; off = round_up(off + (size_t)N * d.m * d.d * 4, A);
  p.off_ln = off; off = round_up(off + (size_t)N * d.m * d.d * 2, A);
  p.off_fc1 = off; off = round_up(off + (size_t)N * T * d.ffn * 2, A);
  p.off_ops = off;
  size_t ops = p.qkv.ws_bytes;
  if (p.proj.ws_bytes > ops) ops = p.proj.ws_bytes;
  if (p.fc1.ws_bytes > ops) ops = p.fc1.ws_bytes;
  if (p.fc2.ws_bytes > ops) ops = p.fc2.ws_bytes;
  p.ws_bytes = off + ops;
  *out = p;
  return CM_OK;
}

cm_status cm_layer_forward(const cm_layer_plan *pl, const void *x, const void *wqkv, const void *wo, const void *w1,
                           const void *w2, void *out, void *ws, size_t ws_bytes, void *compute, void *const *comm,
                           int n_comm) {
  if (!pl) { set_error("null plan"); return CM_ERR_INVALID_ARG; }
  cm_layer_plan canon;
  cm_status st = cm_plan_layer(&pl->desc, &canon);
  if (st != CM_OK) return st;
  if (!same_layer(canon, *pl)) {
    set_error("layer plan does not match what cm_plan_layer produces for its request");
    return CM_ERR_INVALID_ARG;
  }
  if (!x || !wqkv || !wo || !w1 || !w2 || !out || !ws) { set_error("null buffer"); return CM_ERR_INVALID_ARG; }
  if (!aligned16(x) || !aligned16(wqkv) || !aligned16(wo) || !aligned16(w1) || !aligned16(w2) || !aligned16(out) ||
      !aligned16(ws)) {
    set_error("buffers must be 16-byte aligned");
    return CM_ERR_ALIGN;
  }
  if (ws_bytes < pl->ws_bytes) {
    set_error("workspace of %zu bytes, layer plan needs %zu", ws_bytes, pl->ws_bytes);
    return CM_ERR_WORKSPACE;
  }
  if ((st = refuse_capture(compute, comm, n_comm)) != CM_OK) return st;
  const cm_layer_desc &d = pl->desc;
  char *w = static_cast<char *>(ws);
  char *qkv = w + pl->off_qkv, *attn = w + pl->off_attn, *proj = w + pl->off_proj, *ln = w + pl->off_ln,
       *fc1 = w + pl->off_fc1, *opws = w + pl->off_ops;
  const size_t opbytes = ws_bytes - pl->off_ops;
  if ((st = cm_ag_gemm(&pl->qkv, x, wqkv, qkv, opws, opbytes, compute, comm, n_comm, nullptr)) != CM_OK) return st;
  if ((st = cm_attention(qkv, attn, d.n_ranks, d.n_ranks * d.m, d.heads, d.head_dim, 1, compute)) != CM_OK) return st;
  if ((st = cm_gemm_rs(&pl->proj, attn, wo, proj, opws, opbytes, compute, comm, n_comm, nullptr)) != CM_OK) return st;
  if ((st = cm_layernorm(proj, ln, d.n_ranks * d.m, d.d, d.ln_eps, nullptr, nullptr, compute)) != CM_OK) return st;
  if ((st = cm_ag_gemm(&pl->fc1, ln, w1, fc1, opws, opbytes, compute, comm, n_comm, nullptr)) != CM_OK) return st;
  return cm_gemm_rs(&pl->fc2, fc1, w2, out, opws, opbytes, compute, comm, n_comm, nullptr);
}

}  // extern "C"
