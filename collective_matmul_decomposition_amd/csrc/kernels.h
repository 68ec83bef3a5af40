// Launch interface of the gfx950 kernels (host and device see this struct).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace collmm {

constexpr int kMaxJobs = 128;

// One launch: n_jobs independent jobs of the same shape (M x N outputs, K
// contraction).  Operand addresses are base[buffer] + 16 * offset, with the
// buffer of A, B and C selected per job (0 = X, 1 = W, 2 = Y, 3 = workspace);
// the optional fp32 addends in0/in1 always live in the workspace.
//   sel bits 0-1: A buffer, 2-3: B buffer, 4-5: C buffer, 6: in0 present,
//   7: in1 present.
struct GemmParams {
  char *base[4];
  int M, N, K;
  int lda, ldb, ldc, ld_in;  // row strides in elements
  int c_f32;                 // 1: C is fp32, 0: C is bf16 (round to nearest even)
  int add_bf16;              // 1: the addends in0/in1 are bf16, 0: fp32
  int act;                   // epilogue activation of launches without addends: 0 none, 1 GELU (erf form)
  int n_jobs;
  int tiles_m;               // row tiles per job
  int tiles_per_job;
  int jobs_per_b;            // >= 1: consecutive jobs that read the same B (one
                             // rank's grouped steps); their tiles of one B column
                             // run next to each other so B is read once from HBM
  uint32_t a_off[kMaxJobs], b_off[kMaxJobs], c_off[kMaxJobs], in0_off[kMaxJobs], in1_off[kMaxJobs];
  uint8_t sel[kMaxJobs];
};

bool gemm_tile_supported(int tm, int tn);

// Kernel handle and launch shape, for adding launches to a HIP graph.
struct KernelLaunch {
  void *func;
  dim3 grid, block;
};
bool gemm_launch_config(const GemmParams &p, int tm, int tn, KernelLaunch *out);
void reduce_launch_config(const GemmParams &p, KernelLaunch *out);
hipError_t launch_gemm(const GemmParams &p, int tm, int tn, hipStream_t s);
hipError_t launch_reduce(const GemmParams &p, hipStream_t s);
// Test support (the executor's stress mode): a kernel that sleeps for about
// units * 8 us, and a fill of `rows` rows of `row_bytes` bytes, `ld_bytes`
// apart, with 0xFF bytes (row_bytes and ld_bytes multiples of 4).
hipError_t launch_sleep(int units, hipStream_t s);
hipError_t launch_fill_ff(char *p, long rows, long row_bytes, long ld_bytes, hipStream_t s);

}  // namespace collmm
