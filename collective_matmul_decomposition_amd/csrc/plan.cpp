// Ring planner: turns a cm_plan_desc into a schedule and the schedule into a
// program (the exact ordered list of launches, hop copies and event
// record/wait operations the executor enqueues).  Host-only C++; makes no
// HIP call, so the CPU tests can run and simulate every program.
//
// Schedules (page titles and sections in collmm.h):
//   AllGather->GEMM, decomposed ("P2P AllGather overlap"; "The idea" on the
//     decomposition page): at step s rank r multiplies the shard it holds,
//     (r - s) mod N, into the rows of Y_r that belong to that shard (the
//     slice update), while the same shard is copied to rank r + 1.  A
//     bidirectional ring forwards shards both ways: at step s >= 1 rank r
//     holds (r - s) from the clockwise arc and (r + s) from the
//     counter-clockwise arc, so ceil((N-1)/2) hops suffice.
//   GEMM->ReduceScatter, decomposed ("P2P ReduceScatter overlap"; the
//     circulating accumulator of "The idea"): the bucket owned by q starts at
//     rank q + 1, every rank adds its partial product for the bucket's rows
//     and forwards it; after N - 1 hops the owner adds its own share last.
//     Bidirectional: the bucket is split by direction (ranks q-L..q-1
//     clockwise, q+R..q+1 counter-clockwise) and the owner sums its own
//     partial with both arrivals, the realigning addition of "What it costs".
//   Pipeline-chunk ReduceScatter ("Pipeline-chunk ReduceScatter"): the
//     output columns are cut into chunks; chunk j's full partial products are
//     one launch, then a copy-and-add ring reduce-scatters chunk j on the comm
//     streams while chunk j + 1 computes.
//   Naive schedules ("Naive AllGather", "Naive ReduceScatter"): the whole
//     collective then the whole GEMM (AG), or the whole GEMM then the whole
//     collective (RS), with the same copies.
//
// Ordering rules of the programs (section 5 of the Megatron page: a bucket may
// be overwritten only after every later reader of it is finished, and a
// contribution may be read only once the GEMM that makes it is finished):
//   every read of a receive slot waits for the copy that filled it (RAW);
//   every copy into a slot waits for the last reader of the slot's previous
//   contents (WAR); every copy of a bucket waits for the GEMM that produced it.
//   Two slots per rank and direction alternate by step parity.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <string>
#include <vector>

#include "collmm.h"
#include "internal.h"

namespace collmm {

namespace {

thread_local std::string g_last_error;

int mod(int a, int n) { return ((a % n) + n) % n; }

// Default cost-model constants for MI355X, from measurements of this
// library (graph replay): the hop rate one comm lane sustains with large
// copies, the step GEMM's rate at a full, well-shaped launch, and the fixed
// cost of one graph node (kernel or copy).
constexpr double kDefaultCopyGBps = 100.0;    // one SDMA lane
constexpr double kDefaultCuCopyGBps = 1000.0; // the CU copy kernel
constexpr double kDefaultCuAddGBps = 1500.0;  // the add-and-forward launch beside a GEMM (bytes read + written)
constexpr double kDefaultMfmaTflops = 900.0;
constexpr double kDefaultLaunchUs = 20.0;
constexpr double kDefaultHbmGBps = 5000.0;    // an HBM-bound launch (bytes read + written)
// Comm lanes a program uses at most.  A process gets four hardware queues by
// default; the compute stream takes one, so up to three comm streams run
// concurrently with it.  With more, streams share queues and a GEMM can be
// queued behind copies (measured: the hidden fraction of the GPT-3 AllGather
// fell from 0.93 with one lane to 0.06 with four).
constexpr int kMaxLanes = 3;

bool is_pow2_chunk(int c) { return c == 1 || c == 2 || c == 4 || c == 8 || c == 16; }

// Tile choice: among the compiled block tiles, pick the one that wastes the
// least of the chip for `jobs` jobs of rows x cols outputs each.  Score =
// (useful outputs / launched outputs) x (fraction of the last wave of
// workgroups that is busy) x (per-tile efficiency: larger tiles re-read
// operands less).
struct TileCand { int tm, tn; double eff; };
constexpr TileCand kTiles[] = {
    {256, 256, 1.00}, {256, 192, 0.90}, {256, 128, 0.88}, {128, 256, 0.88}, {128, 128, 0.75}, {64, 256, 0.65},
};
constexpr int kCUs = 256;
constexpr int kJobCap = 128;  // jobs one launch can hold (the kernels' parameter block)

bool tile_known(int tm, int tn) {
  for (const TileCand &t : kTiles)
    if (t.tm == tm && t.tn == tn) return true;
  return false;
}

// Returns the chosen tile's score: the fraction of the chip's rate the
// launch is expected to reach relative to an ideal full launch.
double choose_tile(int rows, int cols, int jobs, int *tm, int *tn) {
  double best = -1;
  for (const TileCand &t : kTiles) {
    long tiles_m = (rows + t.tm - 1) / t.tm, tiles_n = (cols + t.tn - 1) / t.tn;
    long wgs = tiles_m * tiles_n * (long)jobs;
    double useful = (double)rows * cols / ((double)tiles_m * t.tm * tiles_n * t.tn);
    long waves = (wgs + kCUs - 1) / kCUs;
    double fill = (double)wgs / ((double)waves * kCUs);
    double score = useful * fill * t.eff;
    if (score > best + 1e-9) { best = score; *tm = t.tm; *tn = t.tn; }
  }
  return best;
}

}  // namespace

double choose_gemm_tile(int rows, int cols, int jobs, int *tm, int *tn) { return choose_tile(rows, cols, jobs, tm, tn); }

void set_error(const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

const char *last_error() { return g_last_error.c_str(); }

// ------------------------------------------------------------ workspace map
// AG decomposed: receive slots, chunk-major so that one chunk of a range of
//   ranks is contiguous:  slot[dir][p][j][r][m/c][k] bf16, p < plan.slots (2,
//   alternating by step, or one per hop when steps are grouped per launch).
// AG naive: gathered activations G[r][T][k] bf16.
// RS decomposed: buckets  bkt[dir][p][j][r][m][n/c] fp32 (bf16 with bucket_bf16),
//   p < 2; with add-and-forward hops also partial slots
//   part[dir][q][j][r][m][n/c] fp32 after them, q < plan.slots, and, when steps
//   are grouped per launch, the owners' arrival blocks arr[r][2][m][n] fp32.
// RS pipe / naive: partials P[r][j][T][n/c] fp32, then ring slots
//   R[p][r][m][n/c] fp32; with add-and-forward hops the ring slots are per
//   chunk, R[j][p][r][m][n/c].
// Whether the plan groups steps per launch (some launch covers several steps).
bool steps_grouped(const cm_plan &pl) {
  for (int i = 0; i < pl.n_launches && i < CM_MAX_RANKS; ++i)
    if (pl.group_len[i] > 1) return true;
  return false;
}

WsLayout ws_layout(const cm_plan &pl) {
  const cm_plan_desc &d = pl.desc;
  const size_t N = d.n_ranks, m = d.m, k = d.k, n = d.n, c = pl.chunks, T = N * m;
  WsLayout L{};
  const int ndir = d.dir == CM_RING_BI ? 2 : 1;
  if (d.share) {
    const size_t S = pl.split;
    if (d.op == CM_OP_AG_GEMM) {  // receive slots [2][m][k] bf16, partials [S][m][n] fp32
      L.ring = 0;
      L.partial = 2 * m * k * 2;
    } else {  // peer [N-1][m][n] at 0, receive slots [2][m][n] at ring, sent [N-1][m][n] at acc,
              // partials [S][m][n] at partial; fp32
      L.ring = (N - 1) * m * n * 4;
      L.acc = L.ring + 2 * m * n * 4;
      L.partial = L.acc + (N - 1) * m * n * 4;
    }
    L.partial_bytes = S * m * n * 4;
    L.total = L.partial + L.partial_bytes;
  } else if (d.op == CM_OP_ALLGATHER) {
    L.total = 0;
  } else if (d.op == CM_OP_AG_GEMM) {
    if (d.sched == CM_SCHED_NAIVE) {
      L.gather = 0;
      L.total = N * T * k * 2;
    } else {
      L.slot_dir_bytes = (size_t)std::max(2, pl.slots) * N * m * k * 2;
      L.total = ndir * L.slot_dir_bytes;
    }
  } else if (d.op == CM_OP_GEMM_RS && d.sched == CM_SCHED_DECOMPOSED && d.dir == CM_RING_DIRECT) {
    // send slots S[p][j][r][m][n/c], receive slots R[p][j][q][m][n/c],
    // home accumulators A[j][q][m][n/c], all fp32
    L.partial = 0;
    L.ring = 2 * N * m * n * 4;
    L.acc = 4 * N * m * n * 4;
    L.total = 5 * N * m * n * 4;
  } else if (d.op == CM_OP_GEMM_RS && d.sched == CM_SCHED_DECOMPOSED) {
    L.slot_dir_bytes = 2 * N * m * n * (d.bucket_bf16 ? 2 : 4);  // c chunks of n/c columns
    L.total = ndir * L.slot_dir_bytes;
    if (d.hop_add) {  // + partial slots part[dir][q][j][r][m][n/c] fp32
      L.partial = L.total;
      L.part_dir_bytes = (size_t)std::max(2, pl.slots) * N * m * n * 4;
      L.total += ndir * L.part_dir_bytes;
      if (steps_grouped(pl)) {  // + the owners' arrivals arr[r][2][m][n] fp32
        L.acc = L.total;
        L.total += N * 2 * m * n * 4;
      }
    }
  } else if (d.hop_add) {  // PIPE / RS naive with add-and-forward hops: ring slots per chunk
    L.partial = 0;
    L.partial_bytes = N > 1 ? N * T * n * 4 : 0;
    L.ring = L.partial_bytes;
    L.total = L.partial_bytes + (N > 1 ? 2 * N * m * n * 4 : 0);
  } else {  // PIPE, or RS naive (PIPE with one chunk)
    L.partial = 0;
    L.partial_bytes = N > 1 ? N * T * n * 4 : 0;
    L.ring = L.partial_bytes;
    L.total = L.partial_bytes + (N > 1 ? 2 * N * m * (n / c) * 4 : 0);
  }
  return L;
}

// ---------------------------------------------------------------- validation
cm_status validate_desc(const cm_plan_desc &d) {
  if (d.op < CM_OP_AG_GEMM || d.op > CM_OP_ALLGATHER) { set_error("unknown op %d", d.op); return CM_ERR_INVALID_ARG; }
  if (d.op == CM_OP_ALLGATHER) {
    if (d.n_ranks < 1 || d.n_ranks > CM_MAX_RANKS) { set_error("n_ranks %d outside 1..%d", d.n_ranks, CM_MAX_RANKS); return CM_ERR_INVALID_ARG; }
    if (d.n_comm < 1 || d.n_comm > CM_MAX_COMM) { set_error("n_comm %d outside 1..%d", d.n_comm, CM_MAX_COMM); return CM_ERR_INVALID_ARG; }
    if (d.m < 1 || d.k < 8 || d.k % 8) { set_error("AllGather: need m >= 1 and k a multiple of 8 (got m=%d k=%d)", d.m, d.k); return CM_ERR_SHAPE; }
    if ((long long)d.n_ranks * d.m > (1 << 24)) { set_error("N*m too large"); return CM_ERR_SHAPE; }
    if (d.n != 0 || d.dir != CM_RING_UNI || d.sched != CM_SCHED_DECOMPOSED || d.chunks > 1 || d.act || d.hop_add ||
        d.bucket_bf16 || d.tile_m || d.tile_n) {
      set_error("AllGather: n must be 0 and dir, sched, chunks, act, hop_add, bucket_bf16 and tile left at their defaults");
      return CM_ERR_INVALID_ARG;
    }
    if (d.in_dtype != CM_BF16) { set_error("only bf16 inputs are supported"); return CM_ERR_UNSUPPORTED; }
    if (d.exec_mode != CM_EXEC_GRAPH && d.exec_mode != CM_EXEC_EAGER) { set_error("unknown exec_mode %d", d.exec_mode); return CM_ERR_INVALID_ARG; }
    if (d.copy_engine != CM_COPY_SDMA && d.copy_engine != CM_COPY_CU) { set_error("unknown copy_engine %d", d.copy_engine); return CM_ERR_INVALID_ARG; }
    if (d.copy_gbps < 0 || d.mfma_tflops < 0 || d.launch_us < 0) { set_error("cost-model inputs must be >= 0"); return CM_ERR_INVALID_ARG; }
    if (d.skip != CM_SKIP_NONE && d.skip != CM_SKIP_HOPS && d.skip != CM_SKIP_GEMMS) {
      set_error("unknown skip mode %d", d.skip);
      return CM_ERR_INVALID_ARG;
    }
    return CM_OK;
  }
  if (d.n_ranks < 1 || d.n_ranks > CM_MAX_RANKS) { set_error("n_ranks %d outside 1..%d", d.n_ranks, CM_MAX_RANKS); return CM_ERR_INVALID_ARG; }
  if (d.dir != CM_RING_UNI && d.dir != CM_RING_BI && d.dir != CM_RING_DIRECT) { set_error("unknown ring direction %d", d.dir); return CM_ERR_INVALID_ARG; }
  if (d.sched != CM_SCHED_DECOMPOSED && d.sched != CM_SCHED_NAIVE && d.sched != CM_SCHED_AUTO) { set_error("unknown schedule %d", d.sched); return CM_ERR_INVALID_ARG; }
  if (d.n_comm < 1 || d.n_comm > CM_MAX_COMM) { set_error("n_comm %d outside 1..%d", d.n_comm, CM_MAX_COMM); return CM_ERR_INVALID_ARG; }
  if (d.in_dtype != CM_BF16) { set_error("only bf16 inputs are supported"); return CM_ERR_UNSUPPORTED; }
  if (d.out_dtype != CM_BF16 && d.out_dtype != CM_F32) { set_error("out dtype must be CM_BF16 or CM_F32"); return CM_ERR_UNSUPPORTED; }
  if (d.chunks < 0 || d.chunks > CM_MAX_CHUNKS) { set_error("chunks %d outside 0..%d", d.chunks, CM_MAX_CHUNKS); return CM_ERR_SHAPE; }
  if (d.m < 1 || d.k < 64 || d.n < 64) { set_error("need m >= 1, k >= 64, n >= 64 (got m=%d k=%d n=%d)", d.m, d.k, d.n); return CM_ERR_SHAPE; }
  if (d.k % 64 || d.n % 64) { set_error("k (%d) and n (%d) must be multiples of 64", d.k, d.n); return CM_ERR_SHAPE; }
  if ((long long)d.n_ranks * d.m > (1 << 24)) { set_error("N*m too large"); return CM_ERR_SHAPE; }
  if ((long long)d.n_ranks * d.m * d.k * 2 > 0xFFFFFFFFll || (long long)d.n * d.k * 2 > 0xFFFFFFFFll) {
    set_error("an operand of one virtual rank exceeds 4 GiB (N*m*k*2 = %lld, n*k*2 = %lld bytes)",
              (long long)d.n_ranks * d.m * d.k * 2, (long long)d.n * d.k * 2);
    return CM_ERR_SHAPE;
  }
  if (d.copy_gbps < 0 || d.mfma_tflops < 0 || d.launch_us < 0) { set_error("cost-model inputs must be >= 0"); return CM_ERR_INVALID_ARG; }
  if (d.exec_mode != CM_EXEC_GRAPH && d.exec_mode != CM_EXEC_EAGER) { set_error("unknown exec_mode %d", d.exec_mode); return CM_ERR_INVALID_ARG; }
  if (d.copy_engine != CM_COPY_SDMA && d.copy_engine != CM_COPY_CU) { set_error("unknown copy_engine %d", d.copy_engine); return CM_ERR_INVALID_ARG; }
  if (d.bucket_bf16 != 0 && d.bucket_bf16 != 1) { set_error("bucket_bf16 must be 0 or 1"); return CM_ERR_INVALID_ARG; }
  if (d.bucket_bf16 && !(d.op == CM_OP_GEMM_RS && d.sched == CM_SCHED_DECOMPOSED && d.dir != CM_RING_DIRECT)) {
    set_error("bf16 buckets exist only for the decomposed GEMM-RS on a ring");
    return CM_ERR_UNSUPPORTED;
  }
  if (d.hop_add != 0 && d.hop_add != 1) { set_error("hop_add must be 0 or 1"); return CM_ERR_INVALID_ARG; }
  if (d.hop_add && !((d.op == CM_OP_GEMM_RS || d.op == CM_OP_GEMM_RS_PIPE) && d.dir != CM_RING_DIRECT &&
                     !d.bucket_bf16)) {
    set_error("add-and-forward hops exist only for a GEMM-RS on a ring with an fp32 bucket");
    return CM_ERR_UNSUPPORTED;
  }
  if (d.dir == CM_RING_DIRECT && d.op == CM_OP_GEMM_RS_PIPE) {
    set_error("the pipeline-chunk ReduceScatter runs its own copy-and-add ring; no direct variant");
    return CM_ERR_UNSUPPORTED;
  }
  if (d.act != CM_ACT_NONE && d.act != CM_ACT_GELU) { set_error("unknown activation %d", d.act); return CM_ERR_INVALID_ARG; }
  if (d.act != CM_ACT_NONE && d.op != CM_OP_AG_GEMM) {
    set_error("an epilogue activation exists only for AllGather->GEMM");
    return CM_ERR_UNSUPPORTED;
  }
  if (d.share != 0 && d.share != 1) { set_error("share must be 0 or 1"); return CM_ERR_INVALID_ARG; }
  if (d.split_k < 0 || d.split_k > 16) { set_error("split_k %d outside 0..16", d.split_k); return CM_ERR_INVALID_ARG; }
  if (d.skip != CM_SKIP_NONE && d.skip != CM_SKIP_HOPS && d.skip != CM_SKIP_GEMMS) {
    set_error("unknown skip mode %d", d.skip);
    return CM_ERR_INVALID_ARG;
  }
  if (d.stress && d.exec_mode != CM_EXEC_EAGER) {
    set_error("the stress mode runs in the eager executor only");
    return CM_ERR_UNSUPPORTED;
  }
  if (!d.share && d.split_k) { set_error("split_k applies to one rank's share (share = 1) only"); return CM_ERR_INVALID_ARG; }
  if (d.group < 0 || d.group > CM_MAX_RANKS) { set_error("group %d outside 0..%d", d.group, CM_MAX_RANKS); return CM_ERR_INVALID_ARG; }
  if (d.share) {
    if (!(d.op == CM_OP_AG_GEMM || d.op == CM_OP_GEMM_RS) || d.dir != CM_RING_UNI || d.sched != CM_SCHED_DECOMPOSED ||
        d.chunks > 1 || d.hop_add || d.bucket_bf16) {
      set_error("one rank's share: AllGather->GEMM or decomposed GEMM->ReduceScatter on a one-way ring, one chunk, "
                "copy hops, fp32 bucket");
      return CM_ERR_UNSUPPORTED;
    }
    if (d.split_k && (d.k / 64) % d.split_k) {
      set_error("split_k %d must divide k/64 = %d", d.split_k, d.k / 64);
      return CM_ERR_SHAPE;
    }
  }
  if ((d.tile_m || d.tile_n) && !tile_known(d.tile_m, d.tile_n)) {
    set_error("no GEMM tile %dx%d (choose 256x256, 256x192, 256x128, 128x256, 128x128, 64x256 or 0x0)", d.tile_m,
              d.tile_n);
    return CM_ERR_UNSUPPORTED;
  }
  return CM_OK;
}

// ------------------------------------------------------------------ planning
namespace {

// GEMM time of one launch of `jobs` jobs of rows x cols x depth, at the
// sustained rate scaled by how well the best tile fits the launch.
double gemm_us(const cm_plan_desc &d, int jobs, double rows, double cols, double depth) {
  int tm, tn;
  double eff = choose_tile((int)rows, (int)cols, jobs, &tm, &tn);
  const double flops = 2.0 * jobs * rows * cols * depth;
  return flops / (d.mfma_tflops * 1e12 * eff) * 1e6 + d.launch_us;
}
// Hop time of one step: `copies` copies per lane over min(n_comm, lanes) lanes.
double hop_us(const cm_plan_desc &d, double bytes_total, int lanes, int copies_per_lane) {
  int streams = std::min(std::min(d.n_comm, kMaxLanes), std::max(1, lanes));
  return bytes_total / (streams * d.copy_gbps * 1e9) * 1e6 + copies_per_lane * d.launch_us;
}

// Predicted time of the decomposed op with c chunks (the reading of the
// "simple peak-rate cost model" of "Knowing when to decline": per-step GEMM
// time at a sustained rate, per-step hop time at the comm lanes' rate, and a
// fixed cost per launch and per copy).
struct Est { double total, g, h; bool hidden; };

Est estimate(const cm_plan_desc &d, int c) {
  const double N = d.n_ranks, m = d.m, k = d.k, n = d.n;
  const bool bi = d.dir == CM_RING_BI && d.n_ranks > 2;
  const int ndir = bi ? 2 : 1;
  const int lanes = d.n_ranks * ndir;
  // copies per lane per step: a lane moves a contiguous range of ranks in one
  // or two copies (AG step 0 with several chunks per shard copies rank by rank)
  const int per_lane = std::max(1, std::min(2, (int)(lanes / std::max(1, std::min(d.n_comm, kMaxLanes)))));
  Est e{};
  if (d.op == CM_OP_AG_GEMM) {
    const double g = gemm_us(d, d.n_ranks * ndir, m / c, n, k);
    const double h = hop_us(d, N * (m / c) * k * 2.0 * ndir, lanes, per_lane);
    const int steps = bi ? 1 + d.n_ranks / 2 : d.n_ranks;
    e.g = g; e.h = h;
    // hop(s) runs beside GEMM(s); GEMM(s+1) needs hop(s)
    e.total = c * steps * std::max(g, h) + std::min(g, h);
    e.hidden = h <= g;
  } else if (d.op == CM_OP_GEMM_RS && d.hop_add) {
    // add-and-forward: hop(s) (read partial, read bucket, write the next
    // rank's slot) runs beside GEMM(s+1); only the last hop is exposed
    const double g = gemm_us(d, d.n_ranks * ndir, m, n / c, k);
    const double h = N * m * (n / c) * 4.0 * 3.0 * ndir / (kDefaultCuAddGBps * 1e9) * 1e6 + d.launch_us;
    const int steps = bi ? 1 + d.n_ranks / 2 : d.n_ranks;
    e.g = g; e.h = h;
    e.total = c * steps * std::max(g, h) + h;
    e.hidden = h <= g;
  } else if (d.op == CM_OP_GEMM_RS) {
    const double g = gemm_us(d, d.n_ranks * ndir, m, n / c, k);
    const double h = hop_us(d, N * m * (n / c) * (d.bucket_bf16 ? 2.0 : 4.0) * ndir, lanes, per_lane);
    const int steps = bi ? 1 + d.n_ranks / 2 : d.n_ranks;
    e.g = g; e.h = h;
    // GEMM(s+1, j) needs hop(s, j), which starts after GEMM(s, j): a step
    // takes the longer of c GEMM chunks and one chunk's GEMM + hop.
    e.total = steps * std::max(c * g, g + h);
    e.hidden = c >= 2 && h <= (c - 1) * g;
  } else if (d.hop_add) {
    // pipeline chunks with add-and-forward hops: N - 1 add launches per
    // chunk (each reads a partial and a bucket and writes the next slot)
    const double g = gemm_us(d, d.n_ranks * d.n_ranks, m, n / c, k);
    const double h = N * m * (n / c) * 4.0 * 3.0 / (kDefaultCuAddGBps * 1e9) * 1e6 + d.launch_us;
    const double ring = (N - 1) * h;
    e.g = g; e.h = h;
    e.total = std::max(c * g + ring, g + c * ring);
    e.hidden = ring <= g;
  } else {
    const double g = gemm_us(d, d.n_ranks, N * m, n / c, k);
    const double h = hop_us(d, N * m * (n / c) * 4.0, d.n_ranks, per_lane) + d.launch_us;  // copy + add
    const double ring = (N - 1) * h;
    e.g = g; e.h = h;
    e.total = std::max(c * g + ring, g + c * ring);
    e.hidden = ring <= g;
  }
  return e;
}

// One rank's share: the K slices S of a step's GEMM ([m x k] . [k x n]) and
// the predicted time of one step (the split GEMM at the tile's expected
// rate, plus the partials written and summed at an HBM-bound rate).
// Candidates: divisors of k/64 up to 16 that leave each slice at least 8
// slabs of 64 (S = 1 always); a requested split_k is taken as it is.
double share_step_us(const cm_plan_desc &d, int S, int *tm, int *tn) {
  const double m = d.m, n = d.n, k = d.k;
  const double score = choose_tile(d.m, d.n, S, tm, tn);
  if (d.tile_m) { *tm = d.tile_m; *tn = d.tile_n; }
  const double g = 2.0 * m * n * k / (d.mfma_tflops * 1e12 * score) * 1e6;
  const double bytes = 2.0 * S * m * n * 4 + m * n * (d.op == CM_OP_GEMM_RS ? 12.0 : (d.out_dtype == CM_F32 ? 4 : 2));
  return g + bytes / (kDefaultHbmGBps * 1e9) * 1e6 + 2 * d.launch_us;
}
int share_split(const cm_plan_desc &d, int *tm, int *tn) {
  if (d.split_k) { (void)share_step_us(d, d.split_k, tm, tn); return d.split_k; }
  const int KT = d.k / 64;
  int best = 1;
  double best_t = share_step_us(d, 1, tm, tn);
  for (int S = 2; S <= 16; ++S) {
    if (KT % S || KT / S < 8) continue;
    int a, b;
    const double t = share_step_us(d, S, &a, &b);
    if (t < best_t) { best = S; best_t = t; }
  }
  (void)share_step_us(d, best, tm, tn);
  return best;
}

// Predicted time of the naive schedule: AG gathers every shard (N - 1 hop
// rounds) and then runs one GEMM over the gathered rows; RS runs the whole
// GEMM and then a copy-and-add ring of N - 1 rounds.
double estimate_naive(const cm_plan_desc &d) {
  const double N = d.n_ranks, m = d.m, k = d.k, n = d.n;
  if (d.n_ranks == 1) return gemm_us(d, 1, m, n, k);
  const int per_lane = std::max(1, std::min(2, d.n_ranks / std::max(1, std::min(d.n_comm, kMaxLanes))));
  if (d.op == CM_OP_AG_GEMM) {
    const double round = hop_us(d, N * m * k * 2.0, d.n_ranks, per_lane);
    return (N - 1) * round + gemm_us(d, d.n_ranks, N * m, n, k);
  }
  const double round = hop_us(d, N * m * n * 4.0, d.n_ranks, per_lane) + d.launch_us;  // copy + add
  return gemm_us(d, d.n_ranks, N * m, n, k) + (N - 1) * round;
}

// ------------------------------------------------- steps grouped per launch
// A launch that multiplies g steps of every rank reads each rank's weights
// once.  Its time is modelled as the part of the weight stream that the MFMA
// work does not hide plus the MFMA work at the compute-bound rate of the
// chosen tile (measured on MI355X for the GPT-3 MLP step launches: about
// 60 us of unhidden weight stream per 1.2 GB of weights, and 1.55 PFLOP/s
// scaled by the tile's efficiency).
constexpr double kGroupComputeTflops = 1550.0;
constexpr double kWeightUnhiddenGBps = 20000.0;
// A launch of one step per rank is bound by its operand bytes rather than its
// MFMA work: the GPT-3 MLP AllGather's single-step launch (8 jobs, 1.28 GB)
// takes about 335 us against about 264 us per step in a two-step launch, an
// operand stream of about 4.9 TB/s.  The launch time is the larger of the two.
constexpr double kGroupHbmGBps = 4900.0;
// Steps per launch when the model chooses: at most four.  Four steps of a
// rank read 1.3-1.4x the weight bytes from HBM (the tiles that share a
// weight column drift further apart than L2 holds), which the model does not
// see; with two copies per AllGather hop the cap was three ([1, 2, 2, 3] in
// 2251 us against 2354 us as [2, 2, 4]), with one copy per hop [1, 3, 4]
// measures 2139 us against 2183 us as [1, 2, 2, 3] (GPT-3 MLP, one box).  The
// ReduceScatter took 2368-2382 us as [4, 2, 2] against 2530-2539 us as
// [2, 2, 2, 2].
constexpr int kMaxGroupAutoAG = 4, kMaxGroupAutoRS = 4;
// The same L2 limit per weight column, in row tiles: the SP layer's
// AllGather->fc1 (512-row shards, two row tiles per step) took 1894-1946 us
// as [1, 1, 3, 3] (six row tiles per column) and 2156 us as [1, 1, 2, 4]
// (eight).
constexpr int kMaxRowTilesPerB = 6;
// Hop and add rates beside the step GEMMs, measured in the same runs (GPT-3
// MLP: a 50 MB AllGather hop step by SDMA takes about 150 us, by the CU copy
// kernel about 75 us; an add-and-forward step of 302 MB about 110 us).  They
// steer only the grouping choice, which depends on nothing else of the
// request's cost-model inputs, so that re-planning a plan's own request
// reproduces it.
constexpr double kGroupSdmaGBps = 400.0, kGroupSdmaCopyUs = 25.0;
constexpr double kGroupCuCopyGBps = 800.0, kGroupCuCopyUs = 10.0;
constexpr double kGroupAddGBps = 2750.0;

double group_launch_us(const cm_plan_desc &d, int jobs, int share, double rows, double cols, double depth) {
  int tm, tn;
  const double eff = choose_tile((int)rows, (int)cols, jobs, &tm, &tn);
  const double flops = 2.0 * jobs * rows * cols * depth;
  const double wbytes = (double)jobs / std::max(1, share) * cols * depth * 2.0;
  const double cbytes = d.op == CM_OP_AG_GEMM && d.out_dtype != CM_F32 ? 2.0 : 4.0;
  const double bytes = wbytes + (double)jobs * rows * (depth * 2.0 + cols * cbytes);
  const double compute = flops / (kGroupComputeTflops * 1e12 * eff) * 1e6;
  return d.launch_us + wbytes / (kWeightUnhiddenGBps * 1e9) * 1e6 +
         std::max(compute, bytes / (kGroupHbmGBps * 1e9) * 1e6);
}

// Jobs per rank of step s: AG step 0 multiplies the own shard only; a later
// step one shard per direction whose arc reaches it.  RS (add-and-forward):
// the owner's step one job, others one per direction that has started.
int step_dirs(const cm_plan &p, int s) {
  const cm_plan_desc &d = p.desc;
  const bool bi = d.dir == CM_RING_BI;
  if (d.op == CM_OP_AG_GEMM) {
    if (s == 0) return 1;
    return (s <= p.arc_cw ? 1 : 0) + (bi && s <= p.arc_ccw ? 1 : 0);
  }
  const int last = bi ? p.arc_cw : d.n_ranks - 1;
  if (s == last) return 1;
  return 1 + (bi && s >= p.arc_cw - p.arc_ccw ? 1 : 0);
}

// Predicted time of the op with the given launch partition (group lengths in
// step order), by a timeline: AllGather hops run back to back on the comm
// lane(s) and a launch starts when the previous one has ended and the hop
// that brings its last step's shard has arrived; ReduceScatter launches run
// back to back, each step's add-and-forward follows its launch and the
// previous add, and the owner's final launch waits for the last add.
double group_timeline(const cm_plan &p, const std::vector<int> &len) {
  const cm_plan_desc &d = p.desc;
  const int N = d.n_ranks;
  const bool bi = d.dir == CM_RING_BI;
  const int lanes = std::min(d.n_comm, kMaxLanes);
  double t = 0;
  int s = 0;
  if (d.op == CM_OP_AG_GEMM) {
    const int per_lane = 1;  // one copy per lane and hop (shard-indexed receive slots)
    const bool sdma = d.copy_engine == CM_COPY_SDMA;
    const double gbps = sdma ? kGroupSdmaGBps : kGroupCuCopyGBps;
    const double lat = sdma ? kGroupSdmaCopyUs : kGroupCuCopyUs;
    // one hop step of one direction (its lanes in parallel); both directions
    // share the lane unless there are two
    const double bytes = (double)N * d.m * d.k * 2.0 / std::max(1, std::min(lanes, N));
    const double hop = (bytes / (gbps * 1e9) * 1e6 + per_lane * lat) * (bi && lanes < 2 ? 2.0 : 1.0);
    for (int g : len) {
      const int b = s + g - 1;
      int jpr = 0;
      for (int q = s; q <= b; ++q) jpr += step_dirs(p, q);
      const double ready = b >= 1 ? std::min(b, p.arc_cw) * hop : 0.0;
      t = std::max(t, ready) + group_launch_us(d, N * jpr, jpr, d.m, d.n, d.k);
      s = b + 1;
    }
    return t;
  }
  const int last = bi ? p.arc_cw : N - 1;
  const double add1 = (double)N * d.m * d.n * 4.0 * 3.0 / (kGroupAddGBps * 1e9) * 1e6;
  // grouped: the owner's partial is an ordinary step and a final add writes
  // Out (reads the arrivals and the own partial, writes the output)
  bool final_add = false;
  for (int g : len) final_add = final_add || g > 1;
  const int ndir = bi ? 2 : 1;
  const double out_b = d.out_dtype == CM_F32 ? 4.0 : 2.0;
  // one-way ring, N >= 3: the last add-and-forward is part of the final add
  const bool fused = final_add && !bi && last >= 2;
  const double fin = (double)N * d.m * d.n * (4.0 * (fused ? 2 : ndir) + 4.0 + out_b) / (kGroupAddGBps * 1e9) * 1e6 +
                     d.launch_us;
  double adds = 0;
  for (int g : len) {
    const int b = s + g - 1;
    int jpr = 0;
    for (int q = s; q <= b; ++q) jpr += step_dirs(p, q);
    if (!final_add && b == last) t = std::max(t, adds);  // the owner's epilogue adds the arrivals
    t += group_launch_us(d, N * jpr, jpr, d.m, d.n, d.k);
    for (int q = s; q <= b && q < last - (fused ? 1 : 0); ++q)
      if (q >= 1) adds = std::max(adds, t) + (step_dirs(p, q) - (bi && q == p.arc_cw - p.arc_ccw ? 1 : 0)) * add1 + d.launch_us;
    s = b + 1;
  }
  if (final_add) t = std::max(t, adds) + fin;
  return t;
}

// Choose the launch partition: every composition of the steps into groups of
// at most gmax, or, beyond 16 steps, equal groups.  An AllGather's first
// launch is step 0 alone: it multiplies only the ranks' own shards, so the
// GEMMs start at once while the first hops are in flight (measured on the
// GPT-3 MLP: [1, 2, 2, 3] runs the op in 2251 us against 2354 us for
// [2, 2, 4], whose first launch waits for a hop).  The shortest predicted
// time wins; ties keep fewer launches.
double choose_groups(const cm_plan &p, int gmax, std::vector<int> *best) {
  const cm_plan_desc &d = p.desc;
  const bool rs = d.op != CM_OP_AG_GEMM;
  const int S = p.n_steps;
  double best_t = -1;
  auto consider = [&](const std::vector<int> &len) {
    const double t = group_timeline(p, len);
    if (best_t < 0 || t < best_t - 1e-6 || (t < best_t + 1e-6 && len.size() < best->size())) {
      best_t = t;
      *best = len;
    }
  };
  if (S <= 16) {
    std::vector<int> cur;
    // depth-first over compositions of S with parts <= gmax
    std::function<void(int)> rec = [&](int rem) {
      if (rem == 0) { consider(cur); return; }
      const int gtop = (!rs && cur.empty()) ? 1 : gmax;  // AllGather: step 0 alone
      for (int g = 1; g <= std::min(gtop, rem); ++g) {
        cur.push_back(g);
        rec(rem - g);
        cur.pop_back();
      }
    };
    rec(S);
  } else {
    for (int g = 1; g <= gmax; ++g) {
      std::vector<int> len;
      int rem = S;
      if (!rs && g > 1) { len.push_back(1); --rem; }
      while (rem > 0) { len.push_back(std::min(g, rem)); rem -= len.back(); }
      consider(len);
    }
  }
  return best_t;
}

// Engine choice (CM_COPY_AUTO): a planned op's predicted time plus what its
// hops take from the GEMMs.  SDMA copies only contend for HBM: on the GPT-3
// MLP AllGather, 352 MB of hops slowed the step GEMMs by about 83 us, the
// hop bytes read and written at about 8.5 TB/s.  The CU copy kernel also
// occupies compute units: about 0.3 of its time alone showed up in the op
// (GPT-3 MLP AllGather; the SP layer's AllGather->QKV and AllGather->fc1,
// where the SDMA hop chain outlasts the GEMMs and the CU copies won by
// 100-380 us).  Grouped-capable ring ops are timed by their launch timeline;
// the rest by the plan's estimate.
constexpr double kSdmaContendGBps = 8500.0, kCuCopyExposed = 0.3;
constexpr double kAutoCuMargin = 0.97;  // the copy kernel must win by 3%

double engine_cost(const cm_plan &p) {
  const cm_plan_desc &d = p.desc;
  if (d.op == CM_OP_ALLGATHER) return p.est_total_us;  // no GEMM to take from
  const int N = d.n_ranks;
  double t = p.est_total_us;
  if (N > 1 && p.chunks == 1 && (d.dir == CM_RING_UNI || d.dir == CM_RING_BI) && d.sched == CM_SCHED_DECOMPOSED &&
      (d.op == CM_OP_AG_GEMM || (d.op == CM_OP_GEMM_RS && d.hop_add)) && p.n_launches >= 1) {
    std::vector<int> len(p.group_len, p.group_len + std::min(p.n_launches, (int)CM_MAX_RANKS));
    t = group_timeline(p, len);
  }
  double bytes = 0;  // what the hops copy (add-and-forward hops copy nothing)
  if (d.op == CM_OP_AG_GEMM)
    bytes = (double)(N - 1) * N * d.m * d.k * 2.0;
  else if (!d.hop_add)
    bytes = (double)(N - 1) * N * d.m * d.n * (d.bucket_bf16 ? 2.0 : 4.0);
  if (d.copy_engine == CM_COPY_SDMA) return t + 2.0 * bytes / (kSdmaContendGBps * 1e9) * 1e6;
  return t + kCuCopyExposed * (bytes / (kGroupCuCopyGBps * 1e9) * 1e6 + (bytes > 0 ? (N - 1) * kGroupCuCopyUs : 0.0));
}

}  // namespace

cm_status plan(const cm_plan_desc *desc, cm_plan *out) {
  if (!desc || !out) { set_error("null argument"); return CM_ERR_INVALID_ARG; }
  if (desc->copy_engine == CM_COPY_AUTO) {
    cm_plan_desc ds = *desc, dc = *desc;
    ds.copy_engine = CM_COPY_SDMA;
    dc.copy_engine = CM_COPY_CU;
    cm_plan ps, pc;
    cm_status st = plan(&ds, &ps);
    if (st != CM_OK) return st;
    if ((st = plan(&dc, &pc)) != CM_OK) return st;
    *out = engine_cost(pc) < kAutoCuMargin * engine_cost(ps) ? pc : ps;
    return CM_OK;
  }
  cm_plan_desc d = *desc;
  if (d.copy_gbps == 0) d.copy_gbps = d.copy_engine == CM_COPY_CU ? kDefaultCuCopyGBps : kDefaultCopyGBps;
  if (d.mfma_tflops == 0) d.mfma_tflops = kDefaultMfmaTflops;
  if (d.launch_us == 0) d.launch_us = kDefaultLaunchUs;
  cm_status st = validate_desc(d);
  if (st != CM_OK) return st;
  if (d.op == CM_OP_ALLGATHER) {
    cm_plan p;
    std::memset(&p, 0, sizeof p);
    p.desc = d;
    p.chunks = 1;
    p.n_steps = 1;
    p.arc_cw = d.n_ranks - 1;
    const int per_lane = std::max(1, std::min(2, d.n_ranks / std::max(1, std::min(d.n_comm, kMaxLanes))));
    p.est_hop_us = hop_us(d, (double)d.n_ranks * d.m * d.k * 2.0, d.n_ranks, per_lane);
    p.est_total_us = (d.n_ranks - 1) * p.est_hop_us;
    p.ws_bytes = 0;
    Program prog;
    build_program(p, prog);
    p.n_ops = (int)prog.ops.size();
    p.n_jobs = (int)prog.jobs.size();
    p.n_events = prog.n_events;
    *out = p;
    return CM_OK;
  }
  if (d.share) {
    cm_plan p;
    std::memset(&p, 0, sizeof p);
    p.desc = d;
    p.chunks = 1;
    p.n_steps = d.n_ranks;
    p.arc_cw = d.n_ranks - 1;
    p.split = share_split(d, &p.tile_m, &p.tile_n);
    const double g = share_step_us(d, p.split, &p.tile_m, &p.tile_n);
    const double hop_bytes = (double)d.m * (d.op == CM_OP_AG_GEMM ? d.k * 2.0 : d.n * 4.0);
    p.est_gemm_us = g;
    p.est_hop_us = hop_bytes / (d.copy_gbps * 1e9) * 1e6 + d.launch_us;
    p.est_total_us = d.n_ranks * std::max(g, p.est_hop_us) + std::min(g, p.est_hop_us);
    p.declined = (d.n_ranks > 1 && p.est_hop_us > g) ? 1 : 0;
    p.ws_bytes = ws_layout(p).total;
    Program prog;
    build_program(p, prog);
    p.n_ops = (int)prog.ops.size();
    p.n_jobs = (int)prog.jobs.size();
    p.n_events = prog.n_events;
    *out = p;
    return CM_OK;
  }
  // A two-rank ring has one neighbour: the bidirectional ring is the uni ring;
  // one rank has no transfers at all.
  if ((d.n_ranks <= 2 && d.dir == CM_RING_BI) || d.n_ranks == 1) d.dir = CM_RING_UNI;
  // The decline gate: plan the decomposed op (best chunking) and compare its
  // predicted time with the naive schedule's.
  if (d.sched == CM_SCHED_AUTO) {
    cm_plan_desc dd = d, dn = d;
    dd.sched = CM_SCHED_DECOMPOSED;
    dn.sched = CM_SCHED_NAIVE;
    dn.chunks = 0;
    dn.hop_add = 0;
    cm_plan pd, pn;
    if ((st = plan(&dd, &pd)) != CM_OK) return st;
    if ((st = plan(&dn, &pn)) != CM_OK) return st;
    const bool decline = d.n_ranks > 1 && estimate_naive(dn) < pd.est_total_us;
    *out = decline ? pn : pd;
    out->declined = decline ? 1 : 0;
    return CM_OK;
  }
  // The naive RS is the pipeline RS with one chunk: the whole GEMM, then the
  // whole ring reduce-scatter.
  if (d.sched == CM_SCHED_NAIVE) d.dir = CM_RING_UNI;
  // The pipeline-chunk variant runs a one-directional copy-and-add ring.
  if (d.op == CM_OP_GEMM_RS_PIPE) d.dir = CM_RING_UNI;

  cm_plan p;
  std::memset(&p, 0, sizeof p);
  p.desc = d;

  auto chunk_ok = [&](int c) -> bool {
    if (c < 1 || c > CM_MAX_CHUNKS) return false;
    if (d.op == CM_OP_AG_GEMM) return d.m % c == 0;
    return d.n % c == 0 && (d.n / c) % 64 == 0;
  };

  int c = d.chunks;
  if (d.sched == CM_SCHED_NAIVE) {
    c = 1;
  } else if (c == 0) {
    // Auto: candidates 1, 2, 3, 4, 6, 8 (RS needs >= 2 for any overlap, the
    // pipeline variant starts from the pages' default of four); take the
    // smallest predicted time, preferring fewer chunks unless more chunks
    // win by at least 5%; decline (report) when nothing hides the hops.
    int best = -1;
    double best_t = 0;
    const int cands[] = {1, 2, 3, 4, 6, 8};
    for (int cc : cands) {
      if (!chunk_ok(cc)) continue;
      if (d.op == CM_OP_GEMM_RS && !d.hop_add && cc < 2 && d.n_ranks > 1) continue;
      if (d.op == CM_OP_AG_GEMM && d.m / cc < 32 && cc > 1) continue;
      Est e = estimate(d, cc);
      if (best < 0 || e.total < best_t * 0.95) { best = cc; best_t = e.total; }
    }
    if (best < 0) best = 1;
    if (d.op == CM_OP_GEMM_RS_PIPE && chunk_ok(4) && best != 4) {
      Est e4 = estimate(d, 4), eb = estimate(d, best);
      if (e4.total <= eb.total * 1.02) best = 4;
    }
    c = best;
  }
  if (!chunk_ok(c)) {
    if (d.op == CM_OP_AG_GEMM)
      set_error("chunks %d must divide m (%d)", c, d.m);
    else
      set_error("chunks %d must divide n (%d) into multiples of 64", c, d.n);
    return CM_ERR_SHAPE;
  }
  (void)is_pow2_chunk;
  p.chunks = c;
  const int N = d.n_ranks;
  const bool bi = d.dir == CM_RING_BI;
  if (d.sched == CM_SCHED_NAIVE || d.op == CM_OP_GEMM_RS_PIPE) {
    p.n_steps = 1;
    p.arc_cw = N - 1;
    p.arc_ccw = 0;
  } else if (bi) {
    p.arc_cw = N / 2;            // ceil((N-1)/2)
    p.arc_ccw = (N - 1) / 2;     // floor((N-1)/2)
    p.n_steps = 1 + p.arc_cw;
  } else {
    p.arc_cw = N - 1;
    p.arc_ccw = 0;
    p.n_steps = N;
  }
  Est e = estimate(d, c);
  p.est_gemm_us = e.g;
  p.est_hop_us = e.h;
  p.est_total_us = d.sched == CM_SCHED_NAIVE ? estimate_naive(d) : e.total;
  // Launches per chunk: one per step, or consecutive steps grouped.
  if (d.sched == CM_SCHED_DECOMPOSED && d.op != CM_OP_GEMM_RS_PIPE) {
    p.n_launches = p.n_steps;
    for (int i = 0; i < p.n_steps && i < CM_MAX_RANKS; ++i) p.group_len[i] = 1;
    p.slots = 2;
    const bool groupable = N > 1 && c == 1 && (d.dir == CM_RING_UNI || bi) &&
                           (d.op == CM_OP_AG_GEMM || (d.op == CM_OP_GEMM_RS && d.hop_add));
    if (groupable && d.group != 1) {
      const int ndir = bi ? 2 : 1;
      int gmax = d.group != 0 ? d.group : (d.op == CM_OP_AG_GEMM ? kMaxGroupAutoAG : kMaxGroupAutoRS);
      if (d.group == 0) {
        // at most kMaxRowTilesPerB row tiles read each weight column per launch
        int tm, tn;
        (void)choose_tile(d.m, d.n, N * ndir, &tm, &tn);
        const int tiles_m = (d.m + tm - 1) / tm;
        gmax = std::min(gmax, std::max(1, kMaxRowTilesPerB / tiles_m));
      }
      gmax = std::min(gmax, std::max(1, kJobCap / (N * ndir)));
      gmax = std::min(gmax, p.n_steps);
      std::vector<int> ones(p.n_steps, 1), best;
      const double t1 = group_timeline(p, ones);
      const double tb = choose_groups(p, gmax, &best);
      if (best.size() < ones.size()) {
        p.n_launches = (int)best.size();
        for (int i = 0; i < CM_MAX_RANKS; ++i) p.group_len[i] = i < p.n_launches ? best[i] : 0;
        p.slots = d.op == CM_OP_AG_GEMM ? std::max(2, p.arc_cw) : std::max(2, p.n_steps);
        // the grouped model's gain applied to the per-step estimate
        if (t1 > 0) p.est_total_us *= tb / t1;
      }
    }
  }
  p.declined = (N > 1 && !e.hidden) ? 1 : 0;
  int rows = d.op == CM_OP_AG_GEMM ? d.m / c : d.m;
  int cols = d.op == CM_OP_AG_GEMM ? d.n : d.n / c;
  if (d.tile_m) { p.tile_m = d.tile_m; p.tile_n = d.tile_n; }
  else (void)choose_tile(rows, cols, N * (bi ? 2 : 1), &p.tile_m, &p.tile_n);
  p.ws_bytes = ws_layout(p).total;

  Program prog;
  build_program(p, prog);
  p.n_ops = (int)prog.ops.size();
  p.n_jobs = (int)prog.jobs.size();
  p.n_events = prog.n_events;
  *out = p;
  return CM_OK;
}

// ------------------------------------------------------------ program build
namespace {

struct Builder {
  const cm_plan &p;
  const cm_plan_desc &d;
  Program &prog;
  WsLayout L;
  int N, c, n_comm;
  size_t m, k, n, T;
  int cur_step = -1, cur_chunk = 0;

  Builder(const cm_plan &p_, Program &pr)
      : p(p_), d(p_.desc), prog(pr), L(ws_layout(p_)), N(d.n_ranks), c(p_.chunks), n_comm(d.n_comm),
        m(d.m), k(d.k), n(d.n), T((size_t)d.n_ranks * d.m) {}

  // Vector clocks of the streams while building: a wait that the stream
  // already satisfies (through program order or an earlier wait) is left out.
  std::vector<std::vector<long>> vc;       // [stream][stream]
  std::vector<std::vector<long>> event_vc;  // [event][stream]
  void ensure_clocks() {
    if (vc.empty()) vc.assign(n_comm + 1, std::vector<long>(n_comm + 1, 0));
  }
  void tick(int stream) {
    ensure_clocks();
    vc[stream][stream]++;
  }

  int new_event() { return prog.n_events++; }
  cm_op_rec base(int kind, int stream) {
    cm_op_rec o;
    std::memset(&o, 0, sizeof o);
    o.kind = kind;
    o.stream = stream;
    o.step = cur_step;
    o.chunk = cur_chunk;
    o.src_buf = o.dst_buf = -1;
    return o;
  }
  int record(int stream) {
    int e = new_event();
    cm_op_rec o = base(CM_OPK_RECORD, stream);
    o.event = e;
    prog.ops.push_back(o);
    tick(stream);
    event_vc.push_back(vc[stream]);
    return e;
  }
  void wait(int stream, int event) {
    if (event < 0) return;
    ensure_clocks();
    const std::vector<long> &ev = event_vc[event];
    bool implied = true;
    for (int t = 0; t <= n_comm; ++t)
      if (ev[t] > vc[stream][t]) { implied = false; break; }
    if (implied) return;
    cm_op_rec o = base(CM_OPK_WAIT, stream);
    o.event = event;
    prog.ops.push_back(o);
    for (int t = 0; t <= n_comm; ++t) vc[stream][t] = std::max(vc[stream][t], ev[t]);
    tick(stream);
  }
  void copy(int stream, int sbuf, size_t soff, int dbuf, size_t doff, size_t bytes) {
    if (bytes == 0) return;
    cm_op_rec o = base(CM_OPK_COPY, stream);
    o.src_buf = sbuf; o.src_off = soff; o.dst_buf = dbuf; o.dst_off = doff; o.bytes = bytes;
    prog.ops.push_back(o);
    tick(stream);
  }
  static cm_job_rec job0() {
    cm_job_rec j;
    std::memset(&j, 0, sizeof j);
    j.a_buf = j.b_buf = j.c_buf = j.in0_buf = j.in1_buf = -1;
    j.add_dtype = CM_F32;
    return j;
  }
  void gemm(const std::vector<cm_job_rec> &jobs, int rows, int cols, int depth, int b_share = 1) {
    if (jobs.empty()) return;
    cm_op_rec o = base(CM_OPK_GEMM, 0);
    o.b_share = b_share;
    o.act = d.op == CM_OP_AG_GEMM ? d.act : CM_ACT_NONE;
    o.first_job = (int)prog.jobs.size();
    o.n_jobs = (int)jobs.size();
    o.rows = rows; o.cols = cols; o.depth = depth;
    if (d.tile_m) { o.tile_m = d.tile_m; o.tile_n = d.tile_n; }
    else (void)choose_tile(rows, cols, (int)jobs.size(), &o.tile_m, &o.tile_n);
    prog.jobs.insert(prog.jobs.end(), jobs.begin(), jobs.end());
    prog.ops.push_back(o);
    tick(0);
  }
  void reduce(int stream, const std::vector<cm_job_rec> &jobs, int rows, int cols, int blocks = 0,
              int act = CM_ACT_NONE) {
    if (jobs.empty()) return;
    cm_op_rec o = base(CM_OPK_REDUCE, stream);
    o.first_job = (int)prog.jobs.size();
    o.n_jobs = (int)jobs.size();
    o.rows = rows; o.cols = cols; o.depth = blocks; o.act = act;
    prog.jobs.insert(prog.jobs.end(), jobs.begin(), jobs.end());
    prog.ops.push_back(o);
    tick(stream);
  }

  // Comm-stream groups: the ranks of one direction are cut into contiguous
  // ranges, one range per comm stream (so a hop of a range of ranks is one
  // or two contiguous copies).  Returns the 1-based stream ids.
  struct Group { int a, b, stream; };
  std::vector<Group> groups(int dir, int ndir) {
    const int usable = std::min(n_comm, kMaxLanes);
    int avail = std::max(1, usable / ndir);
    int first = (ndir == 2 && usable >= 2) ? dir * avail : 0;
    int ng = std::min(avail, N);
    std::vector<Group> g;
    for (int i = 0; i < ng; ++i) {
      int a = (int)((long)N * i / ng), b = (int)((long)N * (i + 1) / ng);
      g.push_back({a, b, 1 + first + i});
    }
    return g;
  }
  static int group_of(const std::vector<Group> &gs, int r) {
    for (size_t i = 0; i < gs.size(); ++i)
      if (r >= gs[i].a && r < gs[i].b) return (int)i;
    return -1;
  }
  std::vector<int> comm_streams() {
    std::vector<int> s;
    for (int i = 1; i <= n_comm; ++i) s.push_back(i);
    return s;
  }

  void entry() {
    cur_step = -1; cur_chunk = 0;
    int e = record(0);
    for (int s : comm_streams()) wait(s, e);
  }
  void exit_() {
    cur_step = -1; cur_chunk = 0;
    ensure_clocks();
    for (int s : comm_streams()) {
      if (vc[0][s] >= vc[s][s]) continue;  // the compute stream already follows all of it
      int e = record(s);
      wait(0, e);
    }
  }

  // ------------------------------------------------------------ AG, decomposed
  // AG direct: for consumer ranks [a, b) copy shard (r - s - 1) of chunk j
  // from the owners' inputs into the ranks' slots (one copy per run of ranks
  // whose sources are also contiguous: only with one chunk per shard).
  void direct_fetch(int stream, int s, int j, int a, int b, size_t slot_base, size_t chunk_bytes) {
    const size_t mc = m / c;
    int r = a;
    while (r < b) {
      const int src = mod(r - s - 1, N);
      int run = 1;
      while (c == 1 && r + run < b && src + run < N) ++run;
      copy(stream, CM_BUF_X, ((size_t)src * m + (size_t)j * mc) * k * 2, CM_BUF_WS, slot_base + (size_t)r * chunk_bytes,
           chunk_bytes * run);
      r += run;
    }
  }

  void ag_decomposed() {
    if (grouped()) { ag_grouped(); return; }
    const bool direct = d.dir == CM_RING_DIRECT;
    const int ndir = d.dir == CM_RING_BI ? 2 : 1;
    const size_t mc = m / c;
    const size_t chunk_bytes = mc * k * 2;             // one rank's chunk, bf16
    auto slot_off = [&](int dir, int par, int j, int r) -> size_t {
      return dir * L.slot_dir_bytes + ((((size_t)par * c + j) * N + r) * chunk_bytes);
    };
    std::vector<std::vector<Group>> G(ndir);
    for (int dr = 0; dr < ndir; ++dr) G[dr] = groups(dr, ndir);
    // events: hop[s][j][dir][group], gemm[s][j]
    std::vector<std::vector<std::vector<std::vector<int>>>> ehop(p.n_steps,
        std::vector<std::vector<std::vector<int>>>(c, std::vector<std::vector<int>>(ndir)));
    std::vector<std::vector<int>> egemm(p.n_steps, std::vector<int>(c, -1));
    const int arcs[2] = {p.arc_cw, p.arc_ccw};
    entry();
    for (int s = 0; s < p.n_steps; ++s) {
      for (int j = 0; j < c; ++j) {
        cur_step = s; cur_chunk = j;
        auto hops = [&]() {
          // hops of step s: forward what this step multiplies
          for (int dr = 0; dr < ndir; ++dr) {
            if (s >= arcs[dr]) continue;
            const int shift = dr == 0 ? 1 : -1;
            ehop[s][j][dr].assign(G[dr].size(), -1);
            for (size_t gi = 0; gi < G[dr].size(); ++gi) {
              const Group &g = G[dr][gi];
              if (direct) {
                // owner -> consumer: rank r's slot s%2 takes shard (r - s - 1)
                // from its owner's input; WAR: GEMM(s-1, j) read that slot
                if (s >= 2) wait(g.stream, egemm[s - 1][j]);
                direct_fetch(g.stream, s, j, g.a, g.b, slot_off(0, s % 2, j, 0), chunk_bytes);
                ehop[s][j][dr][gi] = record(g.stream);
                continue;
              }
              // Ring slots are indexed by shard (as in ag_grouped): the lane
              // owns shards [a, b) at every hop and copies them in place from
              // the previous slot, so its hops depend on its own stream only.
              // WAR: the destination slot (parity s%2) was read by GEMM(s-1, j)
              // (and, as the source of hop(s-1, j), by this lane)
              if (s >= 2) wait(g.stream, egemm[s - 1][j]);
              (void)shift;
              if (s == 0 && c == 1) {
                // from the user's shards, which are laid out like the slots: one copy
                copy(g.stream, CM_BUF_X, (size_t)g.a * chunk_bytes, CM_BUF_WS, slot_off(dr, 0, 0, g.a),
                     (size_t)(g.b - g.a) * chunk_bytes);
              } else if (s == 0) {
                // from the user's shards: shard q's chunk j rows
                for (int q = g.a; q < g.b; ++q)
                  copy(g.stream, CM_BUF_X, ((size_t)q * m + (size_t)j * mc) * k * 2, CM_BUF_WS,
                       slot_off(dr, 0, j, q), chunk_bytes);
              } else {
                copy(g.stream, CM_BUF_WS, slot_off(dr, (s - 1) % 2, j, g.a), CM_BUF_WS, slot_off(dr, s % 2, j, g.a),
                     (size_t)(g.b - g.a) * chunk_bytes);
              }
              ehop[s][j][dr][gi] = record(g.stream);
            }
          }
        };
        auto step_gemm = [&]() {
          // GEMM(s, j) needs hop(s-1, j)
          if (s >= 1)
            for (int dr = 0; dr < ndir; ++dr)
              if (s - 1 < arcs[dr])
                for (int e : ehop[s - 1][j][dr]) wait(0, e);
          std::vector<cm_job_rec> jobs;
          for (int dr = 0; dr < ndir; ++dr) {
            if (s > 0 && s > arcs[dr]) continue;
            if (s == 0 && dr > 0) continue;
            for (int r = 0; r < N; ++r) {
              cm_job_rec jb = job0();
              jb.rank = r;
              jb.dir = dr;
              int shard = s == 0 ? r : (dr == 0 ? mod(r - s, N) : mod(r + s, N));
              jb.index = shard;
              if (s == 0) {
                jb.a_buf = CM_BUF_X;
                jb.a_off = ((size_t)r * m + (size_t)j * mc) * k * 2;
              } else {
                jb.a_buf = CM_BUF_WS;
                jb.a_off = slot_off(dr, (s - 1) % 2, j, direct ? r : shard);
              }
              jb.lda = (int)k;
              jb.b_buf = CM_BUF_W;
              jb.b_off = (size_t)r * n * k * 2;
              jb.ldb = (int)k;
              jb.c_buf = CM_BUF_Y;
              jb.c_dtype = d.out_dtype;
              jb.c_off = ((size_t)r * T + (size_t)shard * m + (size_t)j * mc) * n * (d.out_dtype == CM_F32 ? 4 : 2);
              jb.ldc = (int)n;
              jobs.push_back(jb);
            }
          }
          gemm(jobs, (int)mc, (int)n, (int)k);
          egemm[s][j] = record(0);
        };
        // Step 0's GEMM reads only the user's own shards. It is emitted before
        // the step's hops so that a graph dispatches it first: emitted after
        // them, it started 60-120 us late, behind the copies' dispatch
        if (s == 0) {
          step_gemm();
          hops();
        } else {
          hops();
          step_gemm();
        }
      }
    }
    exit_();
  }

  bool grouped() const { return steps_grouped(p); }

  // ---------------------------------------------- AG, steps grouped per launch
  // One chunk per shard; launch i multiplies steps [a, b] of every rank (one
  // job per rank, step and direction, rank-major so that a rank's jobs, which
  // read the same weights, are adjacent: b_share).  Every hop has a receive
  // slot of its own (slot s holds what hop s brought: the shard of step s + 1),
  // so no copy waits for a reader.  Emission order: the hops a launch needs,
  // the launch, then the hops the next launch needs (they run beside it).
  void ag_grouped() {
    const int ndir = d.dir == CM_RING_BI ? 2 : 1;
    const int P = std::max(2, p.slots);
    const size_t chunk_bytes = m * k * 2;
    // Receive slots are indexed by shard: after hop s, rank r holds shard
    // r - (s + 1) (r + s + 1 on the counter-clockwise arc) at position
    // `shard` of slot s % P.  Rank r's hop s forwards the shard it received
    // at hop s - 1, which sits at the same position of the previous slot, so
    // a hop copies a lane's shard range from one slot to the next in place:
    // one contiguous copy per lane (indexed by rank, the ring's wrap-around
    // split every hop into two copies).  A lane owns a fixed shard range for
    // every hop, so a hop's source was written by the same lane's previous
    // hop (stream order) and its slot's last copy reader was that lane too.
    auto slot_off = [&](int dir, int q, int shard) -> size_t {
      return dir * L.slot_dir_bytes + (((size_t)q * N + shard) * chunk_bytes);
    };
    std::vector<std::vector<Group>> G(ndir);
    for (int dr = 0; dr < ndir; ++dr) G[dr] = groups(dr, ndir);
    const int arcs[2] = {p.arc_cw, p.arc_ccw};
    const int max_arc = std::max(p.arc_cw, ndir == 2 ? p.arc_ccw : 0);
    std::vector<std::vector<std::vector<int>>> ehop(p.n_steps, std::vector<std::vector<int>>(ndir));
    std::vector<int> egemm(p.n_steps, -1);
    entry();
    int emitted = 0;  // hops 0 .. emitted-1 are in the program
    auto emit_hop = [&](int s) {
      cur_step = s; cur_chunk = 0;
      for (int dr = 0; dr < ndir; ++dr) {
        if (s >= arcs[dr]) continue;
        ehop[s][dr].assign(G[dr].size(), -1);
        for (size_t gi = 0; gi < G[dr].size(); ++gi) {
          const Group &g = G[dr][gi];
          // WAR: slot s % P last held hop(s - P)'s shards, read by the launch
          // of step s - P + 1 (and by this lane's hop s - P + 1)
          if (s >= P) wait(g.stream, egemm[s - P + 1]);
          // RAW: the source positions were filled by this lane's hop s - 1
          const size_t bytes = (size_t)(g.b - g.a) * chunk_bytes;
          if (s == 0)
            copy(g.stream, CM_BUF_X, (size_t)g.a * chunk_bytes, CM_BUF_WS, slot_off(dr, 0, g.a), bytes);
          else
            copy(g.stream, CM_BUF_WS, slot_off(dr, (s - 1) % P, g.a), CM_BUF_WS, slot_off(dr, s % P, g.a), bytes);
          ehop[s][dr][gi] = record(g.stream);
        }
      }
    };
    int a = 0;
    for (int li = 0; li < p.n_launches; ++li) {
      const int b = a + p.group_len[li] - 1;
      while (emitted < std::min(b, max_arc)) emit_hop(emitted++);
      cur_step = a; cur_chunk = 0;
      // RAW: every step's shard arrived with hop(step - 1); the latest hops
      // first, so the waits that they already imply are left out
      for (int s = b; s >= std::max(a, 1); --s)
        for (int dr = 0; dr < ndir; ++dr)
          if (s - 1 < arcs[dr])
            for (int e : ehop[s - 1][dr]) wait(0, e);
      std::vector<cm_job_rec> jobs;
      int per_rank = 0;
      for (int r = 0; r < N; ++r) {
        int cnt = 0;
        for (int s = a; s <= b; ++s)
          for (int dr = 0; dr < ndir; ++dr) {
            if (s > 0 && s > arcs[dr]) continue;
            if (s == 0 && dr > 0) continue;
            cm_job_rec jb = job0();
            jb.rank = r;
            jb.dir = dr;
            const int shard = s == 0 ? r : (dr == 0 ? mod(r - s, N) : mod(r + s, N));
            jb.index = shard;
            if (s == 0) {
              jb.a_buf = CM_BUF_X;
              jb.a_off = (size_t)r * m * k * 2;
            } else {
              jb.a_buf = CM_BUF_WS;
              jb.a_off = slot_off(dr, (s - 1) % P, shard);
            }
            jb.lda = (int)k;
            jb.b_buf = CM_BUF_W;
            jb.b_off = (size_t)r * n * k * 2;
            jb.ldb = (int)k;
            jb.c_buf = CM_BUF_Y;
            jb.c_dtype = d.out_dtype;
            jb.c_off = ((size_t)r * T + (size_t)shard * m) * n * (d.out_dtype == CM_F32 ? 4 : 2);
            jb.ldc = (int)n;
            jobs.push_back(jb);
            ++cnt;
          }
        per_rank = cnt;
      }
      gemm(jobs, (int)m, (int)n, (int)k, per_rank);
      const int e = record(0);
      for (int s = a; s <= b; ++s) egemm[s] = e;
      const int next_b = li + 1 < p.n_launches ? b + p.group_len[li + 1] : max_arc;
      while (emitted < std::min(next_b, max_arc)) emit_hop(emitted++);
      a = b + 1;
    }
    exit_();
  }

  // ------------------------- RS with add-and-forward hops, steps grouped
  // One chunk.  Launch i computes the partial products of steps [a, b] of
  // every rank (rank-major, b_share jobs per rank), each into a partial slot
  // of its own; the owner's own partial (step `last`) is an ordinary step of
  // the last launch.  A direction's first step stores straight into the next
  // rank's bucket slot; each later step's add-and-forward (partial + arrived
  // bucket -> the next rank's slot) follows its launch on the first comm
  // stream, in step order, and the adds of step last - 1 deliver into the
  // owners' arrival blocks arr[q][dir].  A final add on the same stream then
  // writes Out_q = (sum of arr[q][dir] over the directions) + own partial,
  // the realigning addition of the bidirectional ring, in the same fp32
  // order as an owner's epilogue would add them.
  void rs_hop_add_grouped() {
    const bool bi = d.dir == CM_RING_BI;
    const int ndir = bi ? 2 : 1;
    const int Pp = std::max(2, p.slots);
    const size_t blk = m * n * 4;
    auto bkt = [&](int dir, int par, int r) -> size_t { return dir * L.slot_dir_bytes + (((size_t)par * N + r) * blk); };
    auto part = [&](int dir, int q, int r) -> size_t {
      return L.partial + dir * L.part_dir_bytes + (((size_t)q * N + r) * blk);
    };
    auto arr = [&](int dir, int r) -> size_t { return L.acc + ((size_t)r * 2 + dir) * blk; };
    const int Lc = p.arc_cw, R = p.arc_ccw;
    const int last = bi ? Lc : N - 1;
    const int arc = bi ? Lc : N - 1;
    const int first[2] = {0, Lc - R};
    const int red = 1;
    // One-way ring with N >= 3: the add of step last - 1 and the owner's add
    // are one launch.  Rank r's arrival pair arr[r] holds the bucket that
    // reaches r at step last - 1 and r's own partial for it; the final add
    // writes Out_{r+1} = (arr[r][0] + arr[r][1]) + own partial of r + 1, the
    // fp32 additions of the ring in their order.
    const bool fused = !bi && last - 1 > first[0];
    // where the bucket that step s + 1 adds to is written (by step s's add, or
    // by a direction's first GEMM): a bucket slot, or an arrival block
    auto dest = [&](int dr, int s, int r_to) -> size_t {
      if (fused) return s + 1 == last - 1 ? arr(0, r_to) : bkt(dr, (s + 1) % 2, r_to);
      return s + 1 == last ? arr(dr, r_to) : bkt(dr, (s + 1) % 2, r_to);
    };
    int e_last_add = -1;
    entry();
    int a = 0;
    for (int li = 0; li < p.n_launches; ++li) {
      const int b = a + p.group_len[li] - 1;
      cur_step = a; cur_chunk = 0;
      for (int s = b; s >= a; --s)
        if (s >= Pp) wait(0, e_last_add);  // WAR: a reused partial slot (only with fewer slots than steps)
      std::vector<cm_job_rec> jobs;
      int per_rank = 0;
      for (int r = 0; r < N; ++r) {
        int cnt = 0;
        for (int s = a; s <= b; ++s) {
          auto mk = [&](int dr, int bucket) {
            cm_job_rec jb = job0();
            jb.rank = r; jb.dir = dr; jb.index = bucket;
            jb.a_buf = CM_BUF_X; jb.a_off = ((size_t)r * T + (size_t)bucket * m) * k * 2; jb.lda = (int)k;
            jb.b_buf = CM_BUF_W; jb.b_off = (size_t)r * n * k * 2; jb.ldb = (int)k;
            jb.ld_in = (int)n;
            jb.c_buf = CM_BUF_WS; jb.ldc = (int)n; jb.c_dtype = CM_F32;
            return jb;
          };
          if (s == last) {  // the owner's own share
            cm_job_rec jb = mk(0, r);
            jb.c_off = part(0, s % Pp, r);
            jobs.push_back(jb);
            ++cnt;
            continue;
          }
          for (int dr = 0; dr < ndir; ++dr) {
            if (s < first[dr]) continue;
            const int shift = dr == 0 ? 1 : -1;
            const int q = dr == 0 ? mod(r + (arc - s), N) : mod(r - (Lc - s), N);
            cm_job_rec jb = mk(dr, q);
            jb.c_off = s == first[dr] ? dest(dr, s, mod(r + shift, N)) : part(dr, s % Pp, r);
            if (fused && s == last - 1) jb.c_off = arr(1, r);
            jobs.push_back(jb);
            ++cnt;
          }
        }
        per_rank = cnt;
      }
      gemm(jobs, (int)m, (int)n, (int)k, per_rank);
      const int eg = record(0);
      for (int s = a; s <= b && s < last - (fused ? 1 : 0); ++s) {
        cur_step = s;
        std::vector<cm_job_rec> rj;
        for (int dr = 0; dr < ndir; ++dr) {
          if (s <= first[dr]) continue;
          const int shift = dr == 0 ? 1 : -1;
          for (int r = 0; r < N; ++r) {
            cm_job_rec jb = job0();
            jb.rank = r; jb.dir = dr;
            jb.index = dr == 0 ? mod(r + (arc - s), N) : mod(r - (Lc - s), N);
            jb.in0_buf = CM_BUF_WS; jb.in0_off = part(dr, s % Pp, r);
            jb.in1_buf = CM_BUF_WS; jb.in1_off = bkt(dr, s % 2, r);
            jb.ld_in = (int)n;
            jb.c_buf = CM_BUF_WS; jb.c_off = dest(dr, s, mod(r + shift, N)); jb.ldc = (int)n;
            jb.c_dtype = CM_F32;
            rj.push_back(jb);
          }
        }
        if (rj.empty()) continue;  // every direction's first step stored straight into the slots
        wait(red, eg);  // RAW: the partials (and, through the compute stream, earlier direct stores)
        reduce(red, rj, (int)m, (int)n);
        e_last_add = record(red);
      }
      if (b == last) {
        // the owners' final add: arr[q][0..ndir) + own partial -> Out_q (fused:
        // arr[q - 1][0..2) + own partial)
        cur_step = last;
        wait(red, eg);  // RAW: the own partials and any direct stores into arr
        std::vector<cm_job_rec> fj;
        for (int r = 0; r < N; ++r) {
          cm_job_rec jb = job0();
          jb.rank = r; jb.index = r;
          jb.in0_buf = CM_BUF_WS; jb.in0_off = fused ? arr(0, mod(r - 1, N)) : arr(0, r);
          jb.in1_buf = CM_BUF_WS; jb.in1_off = part(0, last % Pp, r);
          jb.ld_in = (int)n;
          jb.c_buf = CM_BUF_Y; jb.c_off = (size_t)r * m * n * (d.out_dtype == CM_F32 ? 4 : 2); jb.ldc = (int)n;
          jb.c_dtype = d.out_dtype;
          fj.push_back(jb);
        }
        reduce(red, fj, (int)m, (int)n, fused ? 2 : ndir);
      }
      a = b + 1;
    }
    exit_();
  }

  // --------------------------------------------------------------- AG, naive
  // The ring AllGather of the shards x[r] into every rank's gathered buffer
  // (dst_buf + r * T * k * 2, shard q at row q * m), N - 1 rounds of copies on
  // the comm streams; the compute stream then waits for all of it.
  void gather_ring(int dst_buf, size_t dst_base) {
    const size_t shard_bytes = m * k * 2;
    const size_t rank_bytes = T * k * 2;  // G[r]
    std::vector<Group> G = groups(0, 1);
    cur_step = 0; cur_chunk = 0;
    std::vector<int> prev(G.size(), -1), cur(G.size(), -1);
    // every rank's own shard into its gathered buffer (the collective's local part)
    for (size_t gi = 0; gi < G.size(); ++gi)
      for (int r = G[gi].a; r < G[gi].b; ++r)
        copy(G[gi].stream, CM_BUF_X, (size_t)r * shard_bytes, dst_buf, dst_base + (size_t)r * rank_bytes + (size_t)r * shard_bytes,
             shard_bytes);
    for (int h = 0; h < N - 1; ++h) {
      cur_step = h;
      for (size_t gi = 0; gi < G.size(); ++gi) {
        const Group &g = G[gi];
        if (h >= 1)
          for (int r = g.a; r < g.b; ++r) {
            int up = group_of(G, mod(r - 1, N));
            if (up != (int)gi) wait(g.stream, prev[up]);
          }
        for (int r = g.a; r < g.b; ++r) {
          int shard = mod(r - h, N);
          int dst = mod(r + 1, N);
          if (h == 0)
            copy(g.stream, CM_BUF_X, (size_t)r * shard_bytes, dst_buf, dst_base + (size_t)dst * rank_bytes + shard * shard_bytes,
                 shard_bytes);
          else
            copy(g.stream, dst_buf, dst_base + (size_t)r * rank_bytes + shard * shard_bytes, dst_buf,
                 dst_base + (size_t)dst * rank_bytes + shard * shard_bytes, shard_bytes);
        }
        cur[gi] = record(g.stream);
      }
      prev = cur;
    }
    cur_step = N - 1;
    // the whole gathered activation is needed before what follows
    for (size_t gi = 0; gi < G.size(); ++gi) {
      int e = prev[gi];
      if (e < 0) e = record(G[gi].stream);  // N == 1: only the local copies
      wait(0, e);
    }
  }

  // AllGather alone (the bulk collective of the backward pass): y[r] = the
  // gathered sequence for every rank r.
  void allgather() {
    entry();
    gather_ring(CM_BUF_Y, 0);
    exit_();
  }

  void ag_naive() {
    const size_t rank_bytes = T * k * 2;  // G[r]
    entry();
    gather_ring(CM_BUF_WS, 0);
    std::vector<cm_job_rec> jobs;
    for (int r = 0; r < N; ++r) {
      cm_job_rec jb = job0();
      jb.rank = r; jb.index = r;
      jb.a_buf = CM_BUF_WS; jb.a_off = (size_t)r * rank_bytes; jb.lda = (int)k;
      jb.b_buf = CM_BUF_W; jb.b_off = (size_t)r * n * k * 2; jb.ldb = (int)k;
      jb.c_buf = CM_BUF_Y; jb.c_off = (size_t)r * T * n * (d.out_dtype == CM_F32 ? 4 : 2); jb.ldc = (int)n;
      jb.c_dtype = d.out_dtype;
      jobs.push_back(jb);
    }
    gemm(jobs, (int)T, (int)n, (int)k);
    exit_();
  }

  // ------------------------------------------------------------ RS, decomposed
  void rs_decomposed() {
    if (d.hop_add) { rs_hop_add(); return; }
    const bool bi = d.dir == CM_RING_BI;
    const int ndir = bi ? 2 : 1;
    const size_t nc = n / c;
    const int bdt = d.bucket_bf16 ? CM_BF16 : CM_F32;  // bucket element type
    const size_t blk = m * nc * (d.bucket_bf16 ? 2 : 4);  // one rank's bucket chunk
    const int osz = d.out_dtype == CM_F32 ? 4 : 2;
    auto bkt = [&](int dir, int par, int j, int r) -> size_t {
      return dir * L.slot_dir_bytes + ((((size_t)par * c + j) * N + r) * blk);
    };
    std::vector<std::vector<Group>> G(ndir);
    for (int dr = 0; dr < ndir; ++dr) G[dr] = groups(dr, ndir);
    const int Lc = p.arc_cw, R = p.arc_ccw;
    // step s: clockwise contribution if s < Lc (uni: s < N-1), counter-clockwise if
    // Lc-R <= s < Lc, the owner's final add at s == last.
    const int last = bi ? Lc : N - 1;
    std::vector<std::vector<std::vector<int>>> ehop(c, std::vector<std::vector<int>>(ndir));
    entry();
    for (int s = 0; s <= last; ++s) {
      for (int j = 0; j < c; ++j) {
        cur_step = s; cur_chunk = j;
        // RAW: the buckets this step adds into arrived with hop(s-1, j)
        if (s >= 1)
          for (int dr = 0; dr < ndir; ++dr)
            for (int e : ehop[j][dr]) wait(0, e);
        std::vector<cm_job_rec> jobs;
        auto mk = [&](int r, int dr, int bucket) {
          cm_job_rec jb = job0();
          jb.rank = r; jb.dir = dr; jb.index = bucket;
          jb.a_buf = CM_BUF_X; jb.a_off = ((size_t)r * T + (size_t)bucket * m) * k * 2; jb.lda = (int)k;
          jb.b_buf = CM_BUF_W; jb.b_off = ((size_t)r * n + (size_t)j * nc) * k * 2; jb.ldb = (int)k;
          jb.ld_in = (int)nc;
          jb.add_dtype = bdt;
          return jb;
        };
        for (int r = 0; r < N; ++r) {
          if (s == last) {
            // the owner: its own partial + the arriving bucket(s) -> Out_r
            cm_job_rec jb = mk(r, 0, r);
            jb.c_buf = CM_BUF_Y; jb.c_off = ((size_t)r * m * n + (size_t)j * nc) * osz; jb.ldc = (int)n;
            jb.c_dtype = d.out_dtype;
            if (N > 1) { jb.in0_buf = CM_BUF_WS; jb.in0_off = bkt(0, s % 2, j, r); }
            if (bi && R >= 1) { jb.in1_buf = CM_BUF_WS; jb.in1_off = bkt(1, s % 2, j, r); }
            jobs.push_back(jb);
            continue;
          }
          // clockwise: bucket (r + (Lc - s)) in bi, (r - s - 1) in uni -- both
          // equal r + (arc - s) with arc = N - 1 in uni
          // Bucket slots are indexed by bucket: the bucket that rank r adds
          // into at step s is the one rank r + 1 (r - 1 counter-clockwise)
          // adds into at step s + 1, at the same position of the other slot,
          // so a hop copies a lane's bucket range in place (one copy per lane).
          int arc = bi ? Lc : N - 1;
          int q = mod(r + (arc - s), N);
          cm_job_rec jb = mk(r, 0, q);
          jb.c_buf = CM_BUF_WS; jb.c_off = bkt(0, s % 2, j, q); jb.ldc = (int)nc; jb.c_dtype = bdt;
          if (s > 0) { jb.in0_buf = CM_BUF_WS; jb.in0_off = jb.c_off; }
          jobs.push_back(jb);
          if (bi && s >= Lc - R) {
            int qq = mod(r - (Lc - s), N);
            cm_job_rec jc = mk(r, 1, qq);
            jc.c_buf = CM_BUF_WS; jc.c_off = bkt(1, s % 2, j, qq); jc.ldc = (int)nc; jc.c_dtype = bdt;
            if (s > Lc - R) { jc.in0_buf = CM_BUF_WS; jc.in0_off = jc.c_off; }
            jobs.push_back(jc);
          }
        }
        gemm(jobs, (int)m, (int)nc, (int)k);
        int eg = record(0);
        if (s == last) continue;
        for (int dr = 0; dr < ndir; ++dr) {
          ehop[j][dr].clear();
          if (dr == 1 && s < Lc - R) continue;
          const int shift = dr == 0 ? 1 : -1;
          for (const Group &g : G[dr]) {
            // RAW: the bucket was produced by GEMM(s, j).  WAR on the
            // destination slot holds through GEMM(s, j), which waited for
            // hop(s-1, j), the slot's last reader.
            wait(g.stream, eg);
            (void)shift;
            copy(g.stream, CM_BUF_WS, bkt(dr, s % 2, j, g.a), CM_BUF_WS, bkt(dr, (s + 1) % 2, j, g.a),
                 (size_t)(g.b - g.a) * blk);
            ehop[j][dr].push_back(record(g.stream));
          }
        }
      }
    }
    exit_();
  }

  // ------------------------------------------ RS, ring with add-and-forward hops
  // The ring's order and sums of rs_decomposed with the addition moved out of
  // the GEMM into the hop.  At a direction's first step the partial product is
  // stored straight into the next rank's receive slot; at later steps it is
  // stored into a partial slot, and one add launch on the first comm stream
  // writes partial + arrived bucket into the next rank's receive slot (the
  // copy and the addition in one pass over the bytes).  A step's GEMM waits
  // only for its partial slot to be free (two per rank, alternating by
  // parity), not for the previous hop.  The owner's last GEMM adds the
  // arrived bucket(s) in its epilogue as in rs_decomposed.  fp32 addition
  // commutes, so every sum equals the epilogue's bitwise.
  void rs_hop_add() {
    if (grouped()) { rs_hop_add_grouped(); return; }
    const bool bi = d.dir == CM_RING_BI;
    const int ndir = bi ? 2 : 1;
    const size_t nc = n / c;
    const size_t blk = m * nc * 4;
    const int osz = d.out_dtype == CM_F32 ? 4 : 2;
    auto bkt = [&](int dir, int par, int j, int r) -> size_t {
      return dir * L.slot_dir_bytes + ((((size_t)par * c + j) * N + r) * blk);
    };
    auto part = [&](int dir, int par, int j, int r) -> size_t {
      return L.partial + dir * L.part_dir_bytes + ((((size_t)par * c + j) * N + r) * blk);
    };
    const int Lc = p.arc_cw, R = p.arc_ccw;
    const int last = bi ? Lc : N - 1;
    const int arc = bi ? Lc : N - 1;
    // a direction contributes at steps [first, last): clockwise from 0,
    // counter-clockwise from Lc - R (bi only)
    const int first[2] = {0, Lc - R};
    const int red = 1;  // the add launches run on the first comm stream
    std::vector<std::vector<int>> ered(last + 1, std::vector<int>(c, -1));
    entry();
    for (int s = 0; s <= last; ++s) {
      for (int j = 0; j < c; ++j) {
        cur_step = s; cur_chunk = j;
        if (s == last) {
          if (s >= 1) wait(0, ered[s - 1][j]);  // RAW: the arrived buckets
        } else if (s >= 2) {
          wait(0, ered[s - 2][j]);  // WAR: partial slot s%2 was read by add(s-2, j)
        }
        std::vector<cm_job_rec> jobs;
        auto mk = [&](int r, int dr, int bucket) {
          cm_job_rec jb = job0();
          jb.rank = r; jb.dir = dr; jb.index = bucket;
          jb.a_buf = CM_BUF_X; jb.a_off = ((size_t)r * T + (size_t)bucket * m) * k * 2; jb.lda = (int)k;
          jb.b_buf = CM_BUF_W; jb.b_off = ((size_t)r * n + (size_t)j * nc) * k * 2; jb.ldb = (int)k;
          jb.ld_in = (int)nc;
          return jb;
        };
        for (int r = 0; r < N; ++r) {
          if (s == last) {
            cm_job_rec jb = mk(r, 0, r);
            jb.c_buf = CM_BUF_Y; jb.c_off = ((size_t)r * m * n + (size_t)j * nc) * osz; jb.ldc = (int)n;
            jb.c_dtype = d.out_dtype;
            if (N > 1) { jb.in0_buf = CM_BUF_WS; jb.in0_off = bkt(0, s % 2, j, r); }
            if (bi && R >= 1) { jb.in1_buf = CM_BUF_WS; jb.in1_off = bkt(1, s % 2, j, r); }
            jobs.push_back(jb);
            continue;
          }
          for (int dr = 0; dr < ndir; ++dr) {
            if (s < first[dr]) continue;
            const int shift = dr == 0 ? 1 : -1;
            const int q = dr == 0 ? mod(r + (arc - s), N) : mod(r - (Lc - s), N);
            cm_job_rec jb = mk(r, dr, q);
            jb.c_buf = CM_BUF_WS; jb.ldc = (int)nc; jb.c_dtype = CM_F32;
            jb.c_off = s == first[dr] ? bkt(dr, (s + 1) % 2, j, mod(r + shift, N)) : part(dr, s % 2, j, r);
            jobs.push_back(jb);
          }
        }
        gemm(jobs, (int)m, (int)nc, (int)k);
        const int eg = record(0);
        if (s == last) continue;
        std::vector<cm_job_rec> rj;
        for (int dr = 0; dr < ndir; ++dr) {
          if (s <= first[dr]) continue;
          const int shift = dr == 0 ? 1 : -1;
          for (int r = 0; r < N; ++r) {
            cm_job_rec jb = job0();
            jb.rank = r; jb.dir = dr;
            jb.index = dr == 0 ? mod(r + (arc - s), N) : mod(r - (Lc - s), N);
            jb.in0_buf = CM_BUF_WS; jb.in0_off = part(dr, s % 2, j, r);
            jb.in1_buf = CM_BUF_WS; jb.in1_off = bkt(dr, s % 2, j, r);
            jb.ld_in = (int)nc;
            jb.c_buf = CM_BUF_WS; jb.c_off = bkt(dr, (s + 1) % 2, j, mod(r + shift, N)); jb.ldc = (int)nc;
            jb.c_dtype = CM_F32;
            rj.push_back(jb);
          }
        }
        if (rj.empty()) continue;  // every direction's first step: the GEMM stored straight into the slots
        wait(red, eg);  // RAW: the partials (and, through the compute stream, earlier direct stores)
        reduce(red, rj, (int)m, (int)nc);
        ered[s][j] = record(red);
      }
    }
    exit_();
  }

  // ------------------------------------------------------ RS, direct to owner
  // Step s < N-1: every rank r computes its partial product for bucket
  // q = r - s - 1 (the ring's order) into its send slot, copies it straight to
  // owner q (into q's home accumulator at s = 0, else into q's receive slot),
  // and the owners add the arrivals into their accumulators (one add launch
  // per step on the first comm lane).  Step N-1: each owner's own partial
  // plus its accumulator -> Out_q.  The sum is taken in the ring's order, so
  // the result equals the one-way ring's bitwise.
  void rs_direct() {
    const size_t nc = n / c;
    const size_t blk = m * nc * 4;
    const int osz = d.out_dtype == CM_F32 ? 4 : 2;
    auto S = [&](int par, int j, int r) -> size_t { return L.partial + (((size_t)par * c + j) * N + r) * blk; };
    auto Rv = [&](int par, int j, int q) -> size_t { return L.ring + (((size_t)par * c + j) * N + q) * blk; };
    auto A = [&](int j, int q) -> size_t { return L.acc + ((size_t)j * N + q) * blk; };
    std::vector<Group> G = groups(0, 1);
    const int red_stream = G[0].stream;
    // events per (step, chunk): the GEMM, the hop groups, the add
    std::vector<std::vector<int>> eg(N, std::vector<int>(c, -1)), ered(N, std::vector<int>(c, -1));
    std::vector<std::vector<std::vector<int>>> ehop(N, std::vector<std::vector<int>>(c));
    entry();
    for (int s = 0; s < N; ++s) {
      for (int j = 0; j < c; ++j) {
        cur_step = s; cur_chunk = j;
        std::vector<cm_job_rec> jobs;
        const bool last = s == N - 1;
        if (last && s >= 1) wait(0, N >= 3 ? ered[s - 1][j] : -1);
        if (last && N == 2)
          for (int e : ehop[0][j]) wait(0, e);  // the accumulator is hop(0)'s copy
        // WAR: send slot s%2 was read by hop(s-2, j)
        if (!last && s >= 2)
          for (int e : ehop[s - 2][j]) wait(0, e);
        for (int r = 0; r < N; ++r) {
          const int q = last ? r : mod(r - s - 1, N);
          cm_job_rec jb = job0();
          jb.rank = r; jb.index = q;
          jb.a_buf = CM_BUF_X; jb.a_off = ((size_t)r * T + (size_t)q * m) * k * 2; jb.lda = (int)k;
          jb.b_buf = CM_BUF_W; jb.b_off = ((size_t)r * n + (size_t)j * nc) * k * 2; jb.ldb = (int)k;
          jb.ld_in = (int)nc;
          if (last) {
            jb.c_buf = CM_BUF_Y; jb.c_off = ((size_t)r * m * n + (size_t)j * nc) * osz; jb.ldc = (int)n;
            jb.c_dtype = d.out_dtype;
            if (N > 1) { jb.in0_buf = CM_BUF_WS; jb.in0_off = A(j, r); }
          } else {
            // send slots indexed by the owner q, so a hop copies a lane's
            // owner range in place (one copy per lane)
            jb.c_buf = CM_BUF_WS; jb.c_off = S(s % 2, j, q); jb.ldc = (int)nc; jb.c_dtype = CM_F32;
          }
          jobs.push_back(jb);
        }
        gemm(jobs, (int)m, (int)nc, (int)k);
        eg[s][j] = record(0);
        if (last) continue;
        // hop(s, j): sender ranges [a, b) -> owners r - s - 1
        std::vector<int> ecp;
        for (const Group &g : G) {
          wait(g.stream, eg[s][j]);  // RAW: the partials
          // WAR: receive slot s%2 was read by add(s-2, j) (on the add lane)
          if (s >= 2 && g.stream != red_stream) wait(g.stream, ered[s - 2][j]);
          if (s == 0)
            copy(g.stream, CM_BUF_WS, S(0, j, g.a), CM_BUF_WS, A(j, g.a), (size_t)(g.b - g.a) * blk);
          else
            copy(g.stream, CM_BUF_WS, S(s % 2, j, g.a), CM_BUF_WS, Rv(s % 2, j, g.a), (size_t)(g.b - g.a) * blk);
          const int e = record(g.stream);
          ehop[s][j].push_back(e);
          if (g.stream != red_stream) ecp.push_back(e);
        }
        if (s == 0) continue;  // the first arrivals are copied into the accumulators
        for (int e : ecp) wait(red_stream, e);
        std::vector<cm_job_rec> rj;
        for (int q = 0; q < N; ++q) {
          cm_job_rec jb = job0();
          jb.rank = q; jb.index = q;
          jb.in0_buf = CM_BUF_WS; jb.in0_off = A(j, q);
          jb.in1_buf = CM_BUF_WS; jb.in1_off = Rv(s % 2, j, q);
          jb.ld_in = (int)nc;
          jb.c_buf = CM_BUF_WS; jb.c_off = A(j, q); jb.ldc = (int)nc; jb.c_dtype = CM_F32;
          rj.push_back(jb);
        }
        reduce(red_stream, rj, (int)m, (int)nc);
        ered[s][j] = record(red_stream);
      }
    }
    exit_();
  }

  // ------------------------------- RS, pipeline chunks with add-and-forward hops
  // Chunk j's GEMM computes every rank's partial for every bucket as one job
  // per (rank, bucket); the job of rank r for bucket r - 1, which starts that
  // bucket's trip around the ring, stores straight into rank r + 1's ring
  // slot (the first hop).  Then N - 1 add launches on the first comm stream:
  // at hop t rank r adds its partial for bucket q = r - 1 - t to the bucket
  // that arrived and writes the sum into rank r + 1's slot; at t = N - 1 the
  // owner (r = q) writes Out_q.  Every chunk has its own slots, so chunk
  // j + 1's GEMM runs beside chunk j's adds and waits for none of them.  The
  // additions are those of the copy-and-add ring, in the same order.
  void rs_pipe_add() {
    const size_t nc = n / c;
    const int osz = d.out_dtype == CM_F32 ? 4 : 2;
    const size_t blk = m * nc * 4;
    auto part = [&](int r, int j, int q) -> size_t { return L.partial + (((size_t)r * c + j) * N + q) * blk; };
    auto ring = [&](int j, int par, int r) -> size_t { return L.ring + (((size_t)j * 2 + par) * N + r) * blk; };
    const int red = 1;
    const int per_launch = std::max(1, kJobCap / N);  // ranks per GEMM launch (N jobs each)
    entry();
    for (int j = 0; j < c; ++j) {
      cur_step = 0; cur_chunk = j;
      for (int a = 0; a < N; a += per_launch) {
        std::vector<cm_job_rec> jobs;
        for (int r = a; r < std::min(N, a + per_launch); ++r) {
          for (int q = 0; q < N; ++q) {
            cm_job_rec jb = job0();
            jb.rank = r; jb.index = q;
            jb.a_buf = CM_BUF_X; jb.a_off = ((size_t)r * T + (size_t)q * m) * k * 2; jb.lda = (int)k;
            jb.b_buf = CM_BUF_W; jb.b_off = ((size_t)r * n + (size_t)j * nc) * k * 2; jb.ldb = (int)k;
            jb.ld_in = (int)nc;
            if (N == 1) {
              jb.c_buf = CM_BUF_Y; jb.c_off = (size_t)j * nc * osz; jb.ldc = (int)n; jb.c_dtype = d.out_dtype;
            } else {
              jb.c_buf = CM_BUF_WS; jb.ldc = (int)nc; jb.c_dtype = CM_F32;
              jb.c_off = q == mod(r - 1, N) ? ring(j, 0, mod(r + 1, N)) : part(r, j, q);
            }
            jobs.push_back(jb);
          }
        }
        gemm(jobs, (int)m, (int)nc, (int)k);
      }
      if (N == 1) continue;
      const int eg = record(0);
      wait(red, eg);  // RAW: the partials and the first hop's slots
      for (int t = 1; t < N; ++t) {
        cur_step = t;
        std::vector<cm_job_rec> rj;
        for (int r = 0; r < N; ++r) {
          const int q = mod(r - 1 - t, N);
          cm_job_rec jb = job0();
          jb.rank = r; jb.index = q;
          jb.in0_buf = CM_BUF_WS; jb.in0_off = ring(j, (t - 1) % 2, r);
          jb.in1_buf = CM_BUF_WS; jb.in1_off = part(r, j, q);
          jb.ld_in = (int)nc;
          if (t == N - 1) {
            jb.c_buf = CM_BUF_Y; jb.c_off = ((size_t)r * m * n + (size_t)j * nc) * osz; jb.ldc = (int)n;
            jb.c_dtype = d.out_dtype;
          } else {
            jb.c_buf = CM_BUF_WS; jb.c_off = ring(j, t % 2, mod(r + 1, N)); jb.ldc = (int)nc; jb.c_dtype = CM_F32;
          }
          rj.push_back(jb);
        }
        reduce(red, rj, (int)m, (int)nc);
      }
    }
    exit_();
  }

  // ------------------------------------------------------ one rank's share
  // Virtual rank 0's steps on a one-way ring.  Step s: S split-K GEMM jobs
  // (slice i: columns [i*k/S, (i+1)*k/S) of A and B) write the partials
  // P[i] (fp32, [m][n]); one reduce launch adds them in slice order and
  // stores the step's result.  Buffers that stand for the ring neighbour
  // feed the hops.
  void share_gemm(int a_buf, size_t a_off, int lda, size_t b_off) {
    const int S = p.split;
    const size_t ks = k / S;
    std::vector<cm_job_rec> jobs;
    for (int i = 0; i < S; ++i) {
      cm_job_rec jb = job0();
      jb.rank = 0; jb.index = i;
      jb.a_buf = a_buf; jb.a_off = a_off + (size_t)i * ks * 2; jb.lda = lda;
      jb.b_buf = CM_BUF_W; jb.b_off = b_off + (size_t)i * ks * 2; jb.ldb = (int)k;
      jb.c_buf = CM_BUF_WS; jb.c_off = L.partial + (size_t)i * m * n * 4; jb.ldc = (int)n; jb.c_dtype = CM_F32;
      jobs.push_back(jb);
    }
    cm_op_rec o = base(CM_OPK_GEMM, 0);
    o.act = CM_ACT_NONE;
    o.first_job = (int)prog.jobs.size();
    o.n_jobs = S;
    o.rows = (int)m; o.cols = (int)n; o.depth = (int)ks;
    o.tile_m = p.tile_m; o.tile_n = p.tile_n;
    prog.jobs.insert(prog.jobs.end(), jobs.begin(), jobs.end());
    prog.ops.push_back(o);
    tick(0);
  }
  void share_sum(int in1_off_valid, size_t in1_off, int c_buf, size_t c_off, int ldc, int c_dtype, int act) {
    cm_job_rec jb = job0();
    jb.rank = 0;
    jb.in0_buf = CM_BUF_WS; jb.in0_off = L.partial;
    if (in1_off_valid) { jb.in1_buf = CM_BUF_WS; jb.in1_off = in1_off; }
    jb.ld_in = (int)n;
    jb.c_buf = c_buf; jb.c_off = c_off; jb.ldc = ldc; jb.c_dtype = c_dtype;
    reduce(0, {jb}, (int)m, (int)n, p.split, act);
  }

  void ag_share() {
    const size_t slot_bytes = m * k * 2;
    const int osz = d.out_dtype == CM_F32 ? 4 : 2;
    std::vector<int> ehop(N, -1), egemm(N, -1);
    entry();
    // Each step's GEMM is emitted before the step's hop (which it does not
    // depend on), so that a graph dispatches the GEMM first.
    for (int s = 0; s < N; ++s) {
      cur_step = s;
      if (s >= 1) wait(0, ehop[s - 1]);  // RAW: the shard this step multiplies
      const int c = mod(-s, N);
      if (s == 0)
        share_gemm(CM_BUF_X, 0, (int)k, 0);
      else
        share_gemm(CM_BUF_WS, (size_t)(s % 2) * slot_bytes, (int)k, 0);
      egemm[s] = record(0);
      if (s + 1 < N) {
        // hop s: the neighbour's shard (N - s - 1) arrives in slot (s + 1) % 2;
        // WAR: GEMM(s - 1) read that slot (step 0 reads rank 0's own shard
        // from x, so slot 0 is free for hop 1)
        if (s >= 2) wait(1, egemm[s - 1]);
        copy(1, CM_BUF_X, (size_t)mod(-s - 1, N) * m * k * 2, CM_BUF_WS, (size_t)((s + 1) % 2) * slot_bytes, slot_bytes);
        ehop[s] = record(1);
      }
      share_sum(0, 0, CM_BUF_Y, (size_t)c * m * n * osz, (int)n, d.out_dtype, d.act);
    }
    exit_();
  }

  void rs_share() {
    const size_t blk = m * n * 4;
    auto peer = [&](int s) -> size_t { return (size_t)s * blk; };  // the neighbour's bucket for step s + 1
    auto slot = [&](int par) -> size_t { return L.ring + (size_t)par * blk; };
    auto sent = [&](int s) -> size_t { return L.acc + (size_t)s * blk; };
    std::vector<int> ehop(N, -1), esum(N, -1);
    entry();
    // Each step's GEMM is emitted before the step's hop (which it does not
    // depend on), so that a graph dispatches the GEMM first.
    for (int s = 0; s < N; ++s) {
      cur_step = s;
      const int b = mod(-1 - s, N);
      share_gemm(CM_BUF_X, (size_t)b * m * k * 2, (int)k, 0);
      if (s + 1 < N) {
        // hop s: the bucket for step s + 1 arrives in slot (s + 1) % 2;
        // WAR: the sum of step s - 1 read that slot (step 0's sum reads none)
        if (s >= 2) wait(1, esum[s - 1]);
        copy(1, CM_BUF_WS, peer(s), CM_BUF_WS, slot((s + 1) % 2), blk);
        ehop[s] = record(1);
      }
      if (s >= 1) wait(0, ehop[s - 1]);  // RAW: the arrived bucket
      if (s + 1 < N)
        share_sum(s >= 1, slot(s % 2), CM_BUF_WS, sent(s), (int)n, CM_F32, CM_ACT_NONE);
      else
        share_sum(s >= 1, slot(s % 2), CM_BUF_Y, 0, (int)n, d.out_dtype, CM_ACT_NONE);
      esum[s] = record(0);
    }
    exit_();
  }

  // ------------------------------------------------- RS, pipeline chunks / naive
  void rs_pipe() {
    if (d.hop_add) { rs_pipe_add(); return; }
    const size_t nc = n / c;
    const int osz = d.out_dtype == CM_F32 ? 4 : 2;
    const size_t part_rank = (size_t)c * T * nc * 4;           // P[r]
    auto part = [&](int r, int j, int bucket) -> size_t {        // P[r][j] rows of `bucket`
      return L.partial + (size_t)r * part_rank + ((size_t)j * T + (size_t)bucket * m) * nc * 4;
    };
    const size_t blk = m * nc * 4;
    auto ring = [&](int par, int r) -> size_t { return L.ring + ((size_t)par * N + r) * blk; };
    std::vector<Group> G = groups(0, 1);
    const int red_stream = G[0].stream;
    entry();
    int prev_chunk_done = -1;
    for (int j = 0; j < c; ++j) {
      cur_step = 0; cur_chunk = j;
      std::vector<cm_job_rec> jobs;
      for (int r = 0; r < N; ++r) {
        cm_job_rec jb = job0();
        jb.rank = r; jb.index = j;
        jb.a_buf = CM_BUF_X; jb.a_off = (size_t)r * T * k * 2; jb.lda = (int)k;
        jb.b_buf = CM_BUF_W; jb.b_off = ((size_t)r * n + (size_t)j * nc) * k * 2; jb.ldb = (int)k;
        if (N == 1) {
          jb.c_buf = CM_BUF_Y; jb.c_off = (size_t)j * nc * osz; jb.ldc = (int)n; jb.c_dtype = d.out_dtype;
        } else {
          jb.c_buf = CM_BUF_WS; jb.c_off = part(r, j, 0); jb.ldc = (int)nc; jb.c_dtype = CM_F32;
        }
        jobs.push_back(jb);
      }
      gemm(jobs, (int)T, (int)nc, (int)k);
      int eg = record(0);
      if (N == 1) continue;
      int ered = -1;
      for (int t = 0; t < N - 1; ++t) {
        cur_step = t;
        std::vector<int> ecp;
        for (const Group &g : G) {
          if (t == 0) {
            wait(g.stream, eg);                                      // RAW on P[*][j]
            if (g.stream != red_stream) wait(g.stream, prev_chunk_done);  // WAR on the ring slots
            // ring slots are indexed by bucket: the bucket rank r holds after
            // hop t is the one rank r + 1 holds after hop t + 1, so later hops
            // copy a lane's bucket range in place (one copy per lane)
            for (int r = g.a; r < g.b; ++r)
              copy(g.stream, CM_BUF_WS, part(r, j, mod(r - 1, N)), CM_BUF_WS, ring(0, mod(r - 1, N)), blk);
          } else {
            if (g.stream != red_stream) wait(g.stream, ered);          // RAW: reduce(t-1) wrote the source
            copy(g.stream, CM_BUF_WS, ring((t - 1) % 2, g.a), CM_BUF_WS, ring(t % 2, g.a), (size_t)(g.b - g.a) * blk);
          }
          if (g.stream != red_stream) ecp.push_back(record(g.stream));
        }
        for (int e : ecp) wait(red_stream, e);
        std::vector<cm_job_rec> rj;
        for (int r = 0; r < N; ++r) {
          int q = mod(r - 2 - t, N);  // the bucket rank r received at hop t
          cm_job_rec jb = job0();
          jb.rank = r; jb.index = q;
          jb.in0_buf = CM_BUF_WS; jb.in0_off = ring(t % 2, q);
          jb.in1_buf = CM_BUF_WS; jb.in1_off = part(r, j, q);
          jb.ld_in = (int)nc;
          if (t == N - 2) {
            jb.c_buf = CM_BUF_Y; jb.c_off = ((size_t)r * m * n + (size_t)j * nc) * osz; jb.ldc = (int)n;
            jb.c_dtype = d.out_dtype;
          } else {
            jb.c_buf = CM_BUF_WS; jb.c_off = ring(t % 2, q); jb.ldc = (int)nc; jb.c_dtype = CM_F32;
          }
          rj.push_back(jb);
        }
        reduce(red_stream, rj, (int)m, (int)nc);
        ered = record(red_stream);
      }
      prev_chunk_done = ered;
    }
    exit_();
  }
};

}  // namespace

void build_program(const cm_plan &p, Program &prog) {
  prog.ops.clear();
  prog.jobs.clear();
  prog.n_events = 0;
  Builder b(p, prog);
  const cm_plan_desc &d = p.desc;
  if (d.share) {
    if (d.op == CM_OP_AG_GEMM) b.ag_share(); else b.rs_share();
  } else if (d.op == CM_OP_ALLGATHER) {
    b.allgather();
  } else if (d.op == CM_OP_AG_GEMM) {
    if (d.sched == CM_SCHED_NAIVE) b.ag_naive(); else b.ag_decomposed();
  } else if (d.op == CM_OP_GEMM_RS && d.sched == CM_SCHED_DECOMPOSED) {
    if (d.dir == CM_RING_DIRECT) b.rs_direct(); else b.rs_decomposed();
  } else {
    b.rs_pipe();
  }
}

}  // namespace collmm

// ------------------------------------------------------------------- C ABI
extern "C" {

cm_status cm_ring_plan(const cm_plan_desc *desc, cm_plan *out) { return collmm::plan(desc, out); }

cm_status cm_pick_overlap(const cm_plan_desc *ag, const cm_plan_desc *rs, int *choice, double *saving_us) {
  if (!ag || !rs || !choice) { collmm::set_error("null argument"); return CM_ERR_INVALID_ARG; }
  if (ag->op != CM_OP_AG_GEMM || (rs->op != CM_OP_GEMM_RS && rs->op != CM_OP_GEMM_RS_PIPE)) {
    collmm::set_error("cm_pick_overlap takes an AllGather-side and a ReduceScatter-side request");
    return CM_ERR_INVALID_ARG;
  }
  double save[2];
  const cm_plan_desc *cand[2] = {ag, rs};
  for (int i = 0; i < 2; ++i) {
    cm_plan_desc dd = *cand[i], dn = *cand[i];
    dd.sched = CM_SCHED_DECOMPOSED;
    dn.sched = CM_SCHED_NAIVE;
    dn.chunks = 0;
    dn.hop_add = 0;
    cm_plan pd, pn;
    cm_status st = collmm::plan(&dd, &pd);
    if (st != CM_OK) return st;
    if ((st = collmm::plan(&dn, &pn)) != CM_OK) return st;
    save[i] = pn.est_total_us - pd.est_total_us;
  }
  *choice = (save[0] <= 0 && save[1] <= 0) ? -1 : (save[0] >= save[1] ? 0 : 1);
  if (saving_us) { saving_us[0] = save[0]; saving_us[1] = save[1]; }
  return CM_OK;
}

cm_status cm_workspace_size(const cm_plan *plan, size_t *bytes) {
  if (!plan || !bytes) { collmm::set_error("null argument"); return CM_ERR_INVALID_ARG; }
  *bytes = plan->ws_bytes;
  return CM_OK;
}

cm_status cm_plan_program(const cm_plan *plan, cm_op_rec *ops, int op_cap, int *n_ops, cm_job_rec *jobs,
                          int job_cap, int *n_jobs) {
  if (!plan) { collmm::set_error("null plan"); return CM_ERR_INVALID_ARG; }
  cm_status st = collmm::validate_desc(plan->desc);
  if (st != CM_OK) return st;
  collmm::Program prog;
  collmm::build_program(*plan, prog);
  if (n_ops) *n_ops = (int)prog.ops.size();
  if (n_jobs) *n_jobs = (int)prog.jobs.size();
  if (op_cap < 0 || job_cap < 0) { collmm::set_error("negative capacity"); return CM_ERR_INVALID_ARG; }
  if ((ops == nullptr && op_cap > 0) || (jobs == nullptr && job_cap > 0)) {
    collmm::set_error("null array with non-zero capacity");
    return CM_ERR_INVALID_ARG;
  }
  if (ops == nullptr && jobs == nullptr) return CM_OK;  // size query
  if ((int)prog.ops.size() > op_cap || (int)prog.jobs.size() > job_cap) {
    collmm::set_error("program needs %zu ops and %zu jobs", prog.ops.size(), prog.jobs.size());
    return CM_ERR_CAPACITY;
  }
  std::copy(prog.ops.begin(), prog.ops.end(), ops);
  std::copy(prog.jobs.begin(), prog.jobs.end(), jobs);
  return CM_OK;
}

const char *cm_status_string(cm_status s) {
  switch (s) {
    case CM_OK: return "CM_OK";
    case CM_ERR_INVALID_ARG: return "CM_ERR_INVALID_ARG";
    case CM_ERR_SHAPE: return "CM_ERR_SHAPE";
    case CM_ERR_ALIGN: return "CM_ERR_ALIGN";
    case CM_ERR_WORKSPACE: return "CM_ERR_WORKSPACE";
    case CM_ERR_UNSUPPORTED: return "CM_ERR_UNSUPPORTED";
    case CM_ERR_HIP: return "CM_ERR_HIP";
    case CM_ERR_CAPACITY: return "CM_ERR_CAPACITY";
  }
  return "CM_ERR_UNKNOWN";
}

const char *cm_last_error(void) { return collmm::last_error(); }

const char *cm_version(void) { return "0.1.0"; }

}  // extern "C"
