// Host-only driver for the ring planner, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_plan_sanitize.py: plans and emits
// the program of every request in a grid of ops, directions, schedules,
// chunk counts, rank counts, lane counts and modes, and checks that every
// copy and every job operand lies inside the buffers the request implies.
// Exits non-zero on the first violation (the sanitizers abort on their own).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "collmm.h"

static long long g_plans = 0, g_rejected = 0;

static void fail(const char *what, const cm_plan_desc &d) {
  std::fprintf(stderr, "violation: %s (op %d N %d m %d k %d n %d dir %d c %d sched %d hop %d share %d)\n", what, d.op,
               d.n_ranks, d.m, d.k, d.n, d.dir, d.chunks, d.sched, d.hop_add, d.share);
  std::exit(1);
}

static void check(const cm_plan_desc &d) {
  cm_plan p;
  if (cm_ring_plan(&d, &p) != CM_OK) {
    ++g_rejected;
    return;
  }
  ++g_plans;
  int n_ops = 0, n_jobs = 0;
  if (cm_plan_program(&p, nullptr, 0, &n_ops, nullptr, 0, &n_jobs) != CM_OK) fail("size query", d);
  if (n_ops != p.n_ops || n_jobs != p.n_jobs) fail("program size", d);
  std::vector<cm_op_rec> ops(n_ops > 0 ? n_ops : 1);
  std::vector<cm_job_rec> jobs(n_jobs > 0 ? n_jobs : 1);
  if (cm_plan_program(&p, ops.data(), n_ops, &n_ops, jobs.data(), n_jobs, &n_jobs) != CM_OK) fail("program", d);
  const size_t N = d.n_ranks, m = d.m, k = d.k, n = d.n, T = N * m;
  const size_t R = d.share ? 1 : N;
  const size_t osz = d.out_dtype == CM_F32 ? 4 : 2;
  size_t size[4];
  if (d.op == CM_OP_ALLGATHER) {
    size[0] = N * m * k * 2;
    size[1] = size[0];
    size[2] = N * T * k * 2;
  } else if (d.op == CM_OP_AG_GEMM) {
    size[0] = N * m * k * 2;
    size[1] = R * n * k * 2;
    size[2] = R * T * n * osz;
  } else {
    size[0] = R * T * k * 2;
    size[1] = R * n * k * 2;
    size[2] = R * m * n * osz;
  }
  size[3] = p.ws_bytes;
  auto inside = [&](int buf, size_t off, size_t bytes) {
    return buf >= 0 && buf < 4 && off <= size[buf] && bytes <= size[buf] - off;
  };
  for (int i = 0; i < n_ops; ++i) {
    const cm_op_rec &o = ops[i];
    if (o.stream < 0 || o.stream > d.n_comm) fail("stream", d);
    if ((o.kind == CM_OPK_RECORD || o.kind == CM_OPK_WAIT) && (o.event < 0 || o.event >= p.n_events)) fail("event", d);
    if (o.kind == CM_OPK_COPY && !inside(o.src_buf, o.src_off, o.bytes)) fail("copy source", d);
    if (o.kind == CM_OPK_COPY && !inside(o.dst_buf, o.dst_off, o.bytes)) fail("copy destination", d);
    if (o.kind != CM_OPK_GEMM && o.kind != CM_OPK_REDUCE) continue;
    if (o.first_job < 0 || o.n_jobs < 1 || o.first_job + o.n_jobs > n_jobs) fail("job range", d);
    for (int j = o.first_job; j < o.first_job + o.n_jobs; ++j) {
      const cm_job_rec &b = jobs[j];
      const size_t rows = o.rows, cols = o.cols;
      const size_t csz = b.c_dtype == CM_F32 ? 4 : 2, asz = b.add_dtype == CM_F32 ? 4 : 2;
      if (rows == 0 || cols == 0) fail("empty launch", d);
      if (!inside(b.c_buf, b.c_off, ((rows - 1) * b.ldc + cols) * csz)) fail("C", d);
      if (o.kind == CM_OPK_GEMM) {
        const size_t depth = o.depth;
        if (!inside(b.a_buf, b.a_off, ((rows - 1) * b.lda + depth) * 2)) fail("A", d);
        if (!inside(b.b_buf, b.b_off, ((cols - 1) * b.ldb + depth) * 2)) fail("B", d);
        if (b.in0_buf >= 0 && !inside(b.in0_buf, b.in0_off, ((rows - 1) * b.ld_in + cols) * asz)) fail("in0", d);
        if (b.in1_buf >= 0 && !inside(b.in1_buf, b.in1_off, ((rows - 1) * b.ld_in + cols) * asz)) fail("in1", d);
      } else {
        const size_t S = o.depth > 1 ? o.depth : 1;
        if (!inside(b.in0_buf, b.in0_off, ((S - 1) * rows * b.ld_in + (rows - 1) * b.ld_in + cols) * 4))
          fail("reduce in0", d);
        if (b.in1_buf >= 0 && !inside(b.in1_buf, b.in1_off, ((rows - 1) * b.ld_in + cols) * 4)) fail("reduce in1", d);
      }
    }
  }
}

int main(int argc, char **argv) {
  const int Ns[] = {1, 2, 3, 4, 5, 7, 8, 16, 64};
  const int ms[] = {1, 3, 17, 64, 96};
  const int kns[][2] = {{64, 64}, {128, 320}, {256, 128}, {512, 768}};
  const int chunkss[] = {0, 1, 2, 3, 4, 16};
  const int comms[] = {1, 2, 3, 5, 32};
  const long iters = argc > 1 ? std::atol(argv[1]) : 6000;
  // a fixed-seed sample of the grid (every axis value many times over)
  unsigned long long st = 0x9E3779B97F4A7C15ull;
  auto pick = [&](int n) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (int)(st % (unsigned long long)n);
  };
  for (long it = 0; it < iters; ++it) {
    const int N = Ns[pick(9)], m = ms[pick(5)];
    const int *kn = kns[pick(4)];
    const int op = pick(4), dir = pick(3), sched = pick(3), chunks = chunkss[pick(6)], n_comm = comms[pick(5)];
    const int hop = pick(2), variant = pick(4);
    if (N == 64 && m > 17) continue;  // keep the sample quick under the sanitizers
    cm_plan_desc d{};
    d.op = op;
    d.n_ranks = N;
    d.m = m;
    d.k = kn[0];
    d.n = op == CM_OP_ALLGATHER ? 0 : kn[1];
    d.dir = op == CM_OP_ALLGATHER ? 0 : dir;
    d.sched = op == CM_OP_ALLGATHER ? 0 : sched;
    d.chunks = op == CM_OP_ALLGATHER ? 0 : chunks;
    d.in_dtype = CM_BF16;
    d.out_dtype = variant & 1 ? CM_BF16 : CM_F32;
    d.n_comm = n_comm;
    d.hop_add = op == CM_OP_ALLGATHER ? 0 : hop;
    d.bucket_bf16 = variant == 2 && op == CM_OP_GEMM_RS && !hop;
    d.act = variant == 3 && op == CM_OP_AG_GEMM ? CM_ACT_GELU : CM_ACT_NONE;
    d.skip = (variant + N) % 3;
    check(d);
    // steps grouped per launch (AllGather, add-and-forward ReduceScatter)
    for (int g : {1, 2, 3, 4}) {
      d.group = g;
      if (op <= CM_OP_GEMM_RS && (it + g) % 3 == 0) check(d);
    }
    d.group = 0;
    if (op <= CM_OP_GEMM_RS && dir == 0 && sched == 0 && chunks <= 1 && !hop) {
      d.share = 1;
      d.chunks = 0;
      d.bucket_bf16 = 0;
      for (int split : {0, 1, 2}) {
        d.split_k = split;
        check(d);
      }
    }
  }
  // invalid requests are refused without touching memory out of bounds
  cm_plan_desc bad{};
  for (int v = -3; v < 70; v += 7) {
    bad.op = v % 5;
    bad.n_ranks = v;
    bad.m = v * 3;
    bad.k = v * 64;
    bad.n = 64 - v;
    bad.dir = v % 4;
    bad.chunks = v;
    bad.n_comm = v % 40;
    bad.group = v;
    check(bad);
  }
  cm_plan_desc ag{}, rs{};
  ag.op = CM_OP_AG_GEMM;
  ag.n_ranks = rs.n_ranks = 8;
  ag.m = rs.m = 256;
  ag.k = rs.n = 12288;
  ag.n = rs.k = 6144;
  ag.n_comm = rs.n_comm = 1;
  rs.op = CM_OP_GEMM_RS;
  ag.out_dtype = rs.out_dtype = CM_BF16;
  int choice = -2;
  double save[2];
  if (cm_pick_overlap(&ag, &rs, &choice, save) != CM_OK || choice < -1 || choice > 1) fail("pick", ag);
  std::printf("plans %lld rejected %lld\n", g_plans, g_rejected);
  return 0;
}
