// Executor and C-ABI entry points: runs a plan's program on the compute
// stream and the comm streams.
//
// Every operation of the program maps to one HIP call:
//   GEMM   -> one launch of gemm_jobs (all of the step's partial GEMMs),
//   REDUCE -> one launch of reduce_jobs,
//   COPY   -> hipMemcpyAsync(..., hipMemcpyDeviceToDeviceNoCU, comm stream):
//             the hop, executed by an SDMA engine, not by compute units,
//   RECORD -> hipEventRecord, WAIT -> hipStreamWaitEvent.
// The transfer start/done pairs of the decomposition page ("Asynchrony with
// a budget") are the copy enqueue and the event the compute stream waits on.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <list>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "collmm.h"
#include "internal.h"
#include "kernels.h"

struct cm_trace {
  int device = -1;
  int capacity = 0;
  hipEvent_t entry = nullptr;
  std::vector<hipEvent_t> ev;  // 2 per span: start, end
  std::vector<cm_span> spans;  // metadata; times filled by cm_trace_read
  int used = 0;
  bool overflow = false;
};

namespace collmm {
namespace {

// ------------------------------------------------------------ cached programs
struct Launch {
  GemmParams p;  // base[] filled per call
  int tm = 0, tn = 0;
};

struct Compiled {
  Program prog;
  std::vector<Launch> launches;  // one per GEMM / REDUCE op, in op order
  std::vector<int> launch_of_op; // op index -> launches index (-1 if none)
  hipMemcpyKind copy_kind = hipMemcpyDeviceToDeviceNoCU;  // ring hops: SDMA or the CU copy kernel
  int skip = CM_SKIP_NONE;       // measurement mode: which operations become empty
  int stress = 0;                // test mode seed (eager only): delays and poisoned destinations
  // Is program operation `o` skipped in this plan's measurement mode?  Hops are
  // the copies and the launches on comm streams; the compute stream's launches
  // are the GEMMs (and split-K reduces).
  bool skipped(const cm_op_rec &o) const {
    if (skip == CM_SKIP_HOPS) return o.kind == CM_OPK_COPY || (o.kind == CM_OPK_REDUCE && o.stream != 0);
    if (skip == CM_SKIP_GEMMS) return (o.kind == CM_OPK_GEMM || o.kind == CM_OPK_REDUCE) && o.stream == 0;
    return false;
  }
};

std::string plan_key(const cm_plan &p) {
  // Every field the program depends on (struct padding is not part of it).
  const cm_plan_desc &d = p.desc;
  char buf[512];
  std::snprintf(buf, sizeof buf,
                "%d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %a %a %a %d %d %d %d %d|%d %d %d %d %d %d %d %zu %d %d %d|",
                d.op, d.n_ranks, d.m, d.k, d.n, d.dir, d.chunks, d.sched, d.in_dtype, d.out_dtype, d.n_comm, d.tile_m,
                d.tile_n, d.exec_mode, d.copy_engine, d.bucket_bf16, d.hop_add, d.copy_gbps, d.mfma_tflops,
                d.launch_us, d.act, d.share, d.split_k, d.skip * 1000003 + d.stress, d.group, p.chunks, p.n_steps, p.arc_cw,
                p.arc_ccw, p.tile_m, p.tile_n, p.n_events, p.ws_bytes, p.split, p.n_launches, p.slots);
  std::string key = buf;
  for (int i = 0; i < p.n_launches && i < CM_MAX_RANKS; ++i) key += std::to_string(p.group_len[i]) + ",";
  return key;
}

// The caller's plan must be one that cm_ring_plan produced: re-derive it from
// its request and chunk count and compare every schedule field.
cm_status canonical_plan(const cm_plan &pl, cm_plan *canon) {
  cm_plan_desc d = pl.desc;
  d.chunks = pl.chunks;
  cm_status st = plan(&d, canon);
  if (st != CM_OK) return st;
  if (canon->chunks != pl.chunks || canon->n_steps != pl.n_steps || canon->arc_cw != pl.arc_cw ||
      canon->arc_ccw != pl.arc_ccw || canon->tile_m != pl.tile_m || canon->tile_n != pl.tile_n ||
      canon->ws_bytes != pl.ws_bytes || canon->n_ops != pl.n_ops || canon->n_jobs != pl.n_jobs ||
      canon->n_events != pl.n_events || canon->desc.dir != pl.desc.dir || canon->split != pl.split ||
      canon->n_launches != pl.n_launches || canon->slots != pl.slots ||
      std::memcmp(canon->group_len, pl.group_len, sizeof pl.group_len) != 0) {
    set_error("plan does not match what cm_ring_plan produces for its request");
    return CM_ERR_INVALID_ARG;
  }
  return CM_OK;
}

cm_status fill_params(const cm_op_rec &o, const cm_job_rec *jobs, Launch &L) {
  GemmParams &p = L.p;
  std::memset(&p, 0, sizeof p);
  if (o.n_jobs < 1 || o.n_jobs > kMaxJobs) {
    set_error("a launch has %d jobs (limit %d)", o.n_jobs, kMaxJobs);
    return CM_ERR_SHAPE;
  }
  p.M = o.rows;
  p.N = o.cols;
  p.K = o.depth;
  p.n_jobs = o.n_jobs;
  if (o.kind == CM_OPK_GEMM) {
    // the kernel maps blocks to whole runs of b_share jobs
    if (o.b_share < 0 || (o.b_share > 1 && o.n_jobs % o.b_share)) {
      set_error("a launch of %d jobs cannot be cut into runs of %d", o.n_jobs, o.b_share);
      return CM_ERR_SHAPE;
    }
    p.jobs_per_b = o.b_share > 1 ? o.b_share : 1;
  }
  const cm_job_rec &j0 = jobs[0];
  p.lda = j0.lda;
  p.ldb = j0.ldb;
  p.ldc = j0.ldc;
  p.ld_in = j0.ld_in;
  p.c_f32 = j0.c_dtype == CM_F32;
  int add_dtype = -1;  // common element type of the addends of the launch
  auto off16 = [&](size_t off, uint32_t *out) -> bool {
    if (off % 16 || off / 16 > 0xFFFFFFFFull) return false;
    *out = (uint32_t)(off / 16);
    return true;
  };
  for (int i = 0; i < o.n_jobs; ++i) {
    const cm_job_rec &j = jobs[i];
    if (j.lda != p.lda || j.ldb != p.ldb || j.ldc != p.ldc || j.ld_in != p.ld_in || (j.c_dtype == CM_F32) != (p.c_f32 != 0)) {
      set_error("jobs of one launch differ in strides or output type");
      return CM_ERR_SHAPE;
    }
    uint32_t sel = 0;
    bool ok = true;
    if (o.kind == CM_OPK_GEMM) {
      ok &= j.a_buf >= 0 && j.b_buf >= 0 && off16(j.a_off, &p.a_off[i]) && off16(j.b_off, &p.b_off[i]);
      sel |= (uint32_t)(j.a_buf & 3) | ((uint32_t)(j.b_buf & 3) << 2);
    }
    ok &= j.c_buf >= 0 && off16(j.c_off, &p.c_off[i]);
    sel |= (uint32_t)(j.c_buf & 3) << 4;
    if (j.in0_buf >= 0 || j.in1_buf >= 0) {
      if (add_dtype >= 0 && j.add_dtype != add_dtype) {
        set_error("jobs of one launch differ in addend type");
        return CM_ERR_SHAPE;
      }
      if (j.add_dtype != CM_F32 && (j.add_dtype != CM_BF16 || o.kind != CM_OPK_GEMM)) {
        set_error("bad addend type %d", j.add_dtype);
        return CM_ERR_SHAPE;
      }
      add_dtype = j.add_dtype;
    }
    if (j.in0_buf >= 0) {
      ok &= j.in0_buf == CM_BUF_WS && off16(j.in0_off, &p.in0_off[i]);
      sel |= 1u << 6;
    }
    if (j.in1_buf >= 0) {
      ok &= j.in1_buf == CM_BUF_WS && off16(j.in1_off, &p.in1_off[i]);
      sel |= 1u << 7;
    }
    if (o.kind == CM_OPK_REDUCE) ok &= j.in0_buf >= 0 && (j.in1_buf >= 0 || o.depth >= 1);
    if (!ok) {
      set_error("job %d of a launch has an unaligned, out-of-range or missing operand", i);
      return CM_ERR_SHAPE;
    }
    p.sel[i] = (uint8_t)sel;
  }
  if (o.kind == CM_OPK_GEMM) {
    if (!gemm_tile_supported(o.tile_m, o.tile_n)) {
      set_error("no kernel for tile %dx%d", o.tile_m, o.tile_n);
      return CM_ERR_UNSUPPORTED;
    }
    L.tm = o.tile_m;
    L.tn = o.tile_n;
    p.tiles_m = (p.M + L.tm - 1) / L.tm;
    p.tiles_per_job = p.tiles_m * ((p.N + L.tn - 1) / L.tn);
    if (p.K % 64) {
      set_error("K %d not a multiple of 64", p.K);
      return CM_ERR_SHAPE;
    }
  } else {
    if (p.N % 4 || p.ld_in % 4 || p.ldc % 4) {
      set_error("reduce columns must be multiples of 4");
      return CM_ERR_SHAPE;
    }
    if (o.depth < 0 || o.depth > 64) {
      set_error("a reduce sums 1..64 blocks (got %d)", o.depth);
      return CM_ERR_SHAPE;
    }
    if (o.act != CM_ACT_NONE && o.act != CM_ACT_GELU) {
      set_error("unknown activation %d", o.act);
      return CM_ERR_UNSUPPORTED;
    }
    p.act = o.act;
  }
  p.add_bf16 = add_dtype == CM_BF16;
  if (o.kind == CM_OPK_GEMM && o.act != CM_ACT_NONE) {
    if (o.act != CM_ACT_GELU || add_dtype >= 0) {
      set_error("an epilogue activation needs a launch without addends");
      return CM_ERR_UNSUPPORTED;
    }
    p.act = o.act;
  }
  return CM_OK;
}

struct GraphEntry {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  const cm_trace *trace = nullptr;
  std::vector<cm_span> spans;  // trace metadata captured with the graph
  bool overflow = false;
  // The owner makes sure no launch of the graph is still running (see
  // drop_graphs).
  ~GraphEntry() {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
  }
};

constexpr size_t kMaxGraphs = 256;

// Instantiated graphs, shared by every host thread of the process and kept in
// least-recently-used order.  A graph is keyed by the plan, the buffers and the
// trace it was built for.  A launched graph may still be running when it is
// dropped, and the only handle on its completion is the caller's stream, which
// the caller may have destroyed by then; so dropping graphs first waits for the
// device, and a full cache drops its least recently used quarter at once.
struct GraphCache {
  std::mutex mu;
  std::list<std::string> lru;  // front = most recently used
  struct Slot {
    std::unique_ptr<GraphEntry> g;
    std::list<std::string>::iterator pos;
  };
  std::unordered_map<std::string, Slot> map;
};

GraphCache &graph_cache() {
  static GraphCache *c = new GraphCache;  // never destroyed: graphs may outlive static destruction order
  return *c;
}

struct ThreadState {
  std::unordered_map<std::string, std::unique_ptr<Compiled>> programs;
  std::unordered_map<int, std::vector<hipEvent_t>> events;  // per device
  std::unordered_map<int, int> arch_ok;                     // per device: 1 ok, 0 not gfx950
};

ThreadState &tls() {
  thread_local ThreadState s;
  return s;
}

cm_status get_compiled(const cm_plan &pl, const Compiled **out) {
  ThreadState &ts = tls();
  std::string key = plan_key(pl);
  auto it = ts.programs.find(key);
  if (it != ts.programs.end()) {
    *out = it->second.get();
    return CM_OK;
  }
  cm_plan canon;
  cm_status cst = canonical_plan(pl, &canon);
  if (cst != CM_OK) return cst;
  auto c = std::make_unique<Compiled>();
  build_program(canon, c->prog);
  c->copy_kind = canon.desc.copy_engine == CM_COPY_CU ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToDeviceNoCU;
  c->skip = canon.desc.skip;
  c->stress = canon.desc.stress;
  c->launch_of_op.assign(c->prog.ops.size(), -1);
  for (size_t i = 0; i < c->prog.ops.size(); ++i) {
    const cm_op_rec &o = c->prog.ops[i];
    if (o.kind != CM_OPK_GEMM && o.kind != CM_OPK_REDUCE) continue;
    Launch L;
    cm_status st = fill_params(o, c->prog.jobs.data() + o.first_job, L);
    if (st != CM_OK) return st;
    c->launch_of_op[i] = (int)c->launches.size();
    c->launches.push_back(L);
  }
  if (ts.programs.size() > 256) ts.programs.clear();
  *out = c.get();
  ts.programs.emplace(key, std::move(c));
  return CM_OK;
}

cm_status hip_fail(hipError_t e, const char *what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return CM_ERR_HIP;
}

cm_status check_device(int *dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  ThreadState &ts = tls();
  auto it = ts.arch_ok.find(dev);
  if (it == ts.arch_ok.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    int ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    it = ts.arch_ok.emplace(dev, ok).first;
    if (!ok) set_error("device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  }
  if (!it->second) {
    set_error("current device is not gfx950");
    return CM_ERR_UNSUPPORTED;
  }
  *dev_out = dev;
  return CM_OK;
}

cm_status event_pool(int dev, int n, std::vector<hipEvent_t> **out) {
  std::vector<hipEvent_t> &v = tls().events[dev];
  while ((int)v.size() < n) {
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    v.push_back(ev);
  }
  *out = &v;
  return CM_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Which entry point a call came through.
enum Entry { kEntryAG = 0, kEntryRS = 1, kEntryGather = 2 };

cm_status validate_call(const cm_plan *pl, Entry want, const void *x, const void *w, void *y, void *ws,
                        size_t ws_bytes, void *compute, void *const *comm, int n_comm) {
  if (!pl) { set_error("null plan"); return CM_ERR_INVALID_ARG; }
  cm_status st = validate_desc(pl->desc);
  if (st != CM_OK) return st;
  const int op = pl->desc.op;
  const Entry is = op == CM_OP_AG_GEMM ? kEntryAG : op == CM_OP_ALLGATHER ? kEntryGather : kEntryRS;
  const bool is_ag = is != kEntryRS;  // row-chunked (or unchunked) ops
  if (is != want) {
    set_error(want == kEntryAG   ? "cm_ag_gemm needs a plan with op CM_OP_AG_GEMM"
              : want == kEntryRS ? "cm_gemm_rs needs a plan with op CM_OP_GEMM_RS or CM_OP_GEMM_RS_PIPE"
                                 : "cm_allgather needs a plan with op CM_OP_ALLGATHER");
    return CM_ERR_INVALID_ARG;
  }
  if (pl->chunks < 1 || pl->chunks > CM_MAX_CHUNKS) { set_error("plan has invalid chunk count"); return CM_ERR_INVALID_ARG; }
  if (is_ag ? (pl->desc.m % pl->chunks) : (pl->desc.n % pl->chunks || (pl->desc.n / pl->chunks) % 64)) {
    set_error("plan chunk count does not divide the shape");
    return CM_ERR_SHAPE;
  }
  if (ws_layout(*pl).total != pl->ws_bytes) { set_error("plan is inconsistent (workspace size)"); return CM_ERR_INVALID_ARG; }
  if (!x || !w || !y) { set_error("null x, w or y"); return CM_ERR_INVALID_ARG; }
  if (pl->ws_bytes > 0 && !ws) { set_error("null workspace"); return CM_ERR_INVALID_ARG; }
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (ws && !aligned16(ws))) {
    set_error("x, w, y and ws must be 16-byte aligned");
    return CM_ERR_ALIGN;
  }
  if (ws_bytes < pl->ws_bytes) {
    set_error("workspace of %zu bytes, plan needs %zu", ws_bytes, pl->ws_bytes);
    return CM_ERR_WORKSPACE;
  }
  if (n_comm != pl->desc.n_comm || !comm) {
    set_error("plan was built for %d comm streams, call passes %d", pl->desc.n_comm, n_comm);
    return CM_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n_comm; ++i) {
    if (!comm[i] || comm[i] == compute) { set_error("comm stream %d is null or equal to the compute stream", i); return CM_ERR_INVALID_ARG; }
    for (int j = 0; j < i; ++j)
      if (comm[j] == comm[i]) { set_error("comm streams %d and %d are the same stream", j, i); return CM_ERR_INVALID_ARG; }
  }
  return CM_OK;
}

// The stress mode (a test of the program's ordering): before operation `i`,
// maybe a sleep on its stream (chosen by a hash of the seed and `i`), then a
// fill with 0xFF bytes of every workspace region the operation is about to
// write (not the ones it also reads: an epilogue that adds into its output).
// Correct waits make both invisible in the results.
cm_status stress_before(const Compiled *cp, const cm_op_rec &o, uint32_t i, char *const base[4], hipStream_t s) {
  uint32_t h = (uint32_t)cp->stress * 0x9E3779B1u ^ (i + 1) * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0xC2B2AE3Du;
  h ^= h >> 13;
  hipError_t e;
  if ((h & 3) == 0 && (e = launch_sleep((int)((h >> 8) & 7), s)) != hipSuccess) return hip_fail(e, "stress sleep");
  if (o.kind == CM_OPK_COPY) {
    if (o.dst_buf == CM_BUF_WS && (e = launch_fill_ff(base[CM_BUF_WS] + o.dst_off, 1, (long)o.bytes, (long)o.bytes, s)) != hipSuccess)
      return hip_fail(e, "stress fill");
    return CM_OK;
  }
  if (cp->skipped(o)) return CM_OK;
  for (int j = o.first_job; j < o.first_job + o.n_jobs; ++j) {
    const cm_job_rec &jb = cp->prog.jobs[j];
    if (jb.c_buf != CM_BUF_WS) continue;
    if ((jb.in0_buf == CM_BUF_WS && jb.in0_off == jb.c_off) || (jb.in1_buf == CM_BUF_WS && jb.in1_off == jb.c_off)) continue;
    const long esz = jb.c_dtype == CM_F32 ? 4 : 2;
    if ((e = launch_fill_ff(base[CM_BUF_WS] + jb.c_off, o.rows, o.cols * esz, (long)jb.ldc * esz, s)) != hipSuccess)
      return hip_fail(e, "stress fill");
  }
  return CM_OK;
}

// Enqueue the program's operations on the streams, one HIP call each
// (eager mode).  Calls made while a stream is being captured are refused
// before this point (refuse_capture).
cm_status enqueue(const Compiled *cp, const std::vector<hipEvent_t> &ev, char *const base[4],
                  const hipStream_t *streams, cm_trace *trace) {
  hipError_t e;
  if (trace) {
    trace->used = 0;
    trace->overflow = false;
    trace->spans.clear();
    if ((e = hipEventRecord(trace->entry, streams[0])) != hipSuccess) return hip_fail(e, "hipEventRecord(trace)");
  }
  auto span_begin = [&](const cm_op_rec &o) -> int {
    if (!trace) return -1;
    if (trace->used >= trace->capacity) { trace->overflow = true; return -1; }
    int idx = trace->used++;
    cm_span sp{};
    sp.kind = o.kind;
    sp.stream = o.stream;
    sp.step = o.step;
    sp.chunk = o.chunk;
    trace->spans.push_back(sp);
    (void)hipEventRecord(trace->ev[2 * idx], streams[o.stream]);
    return idx;
  };
  auto span_end = [&](int idx, const cm_op_rec &o) {
    if (idx >= 0) (void)hipEventRecord(trace->ev[2 * idx + 1], streams[o.stream]);
  };

  const std::vector<cm_op_rec> &ops = cp->prog.ops;
  for (size_t i = 0; i < ops.size(); ++i) {
    const cm_op_rec &o = ops[i];
    hipStream_t s = streams[o.stream];
    if (cp->stress && o.kind != CM_OPK_RECORD && o.kind != CM_OPK_WAIT) {
      cm_status st = stress_before(cp, o, (uint32_t)i, base, s);
      if (st != CM_OK) return st;
    }
    switch (o.kind) {
      case CM_OPK_RECORD:
        if ((e = hipEventRecord(ev[o.event], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        break;
      case CM_OPK_WAIT:
        if ((e = hipStreamWaitEvent(s, ev[o.event], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        break;
      case CM_OPK_COPY: {
        int sp = span_begin(o);
        if (cp->skipped(o)) {
          span_end(sp, o);
          break;
        }
        e = hipMemcpyAsync(base[o.dst_buf] + o.dst_off, base[o.src_buf] + o.src_off, o.bytes,
                           cp->copy_kind, s);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (ring hop)");
        span_end(sp, o);
        break;
      }
      case CM_OPK_GEMM:
      case CM_OPK_REDUCE: {
        GemmParams p = cp->launches[cp->launch_of_op[i]].p;
        for (int b = 0; b < 4; ++b) p.base[b] = base[b];
        int sp = span_begin(o);
        if (cp->skipped(o)) {
          span_end(sp, o);
          break;
        }
        if (o.kind == CM_OPK_GEMM) {
          const Launch &L = cp->launches[cp->launch_of_op[i]];
          e = launch_gemm(p, L.tm, L.tn, s);
        } else {
          e = launch_reduce(p, s);
        }
        if (e != hipSuccess) return hip_fail(e, o.kind == CM_OPK_GEMM ? "gemm launch" : "reduce launch");
        span_end(sp, o);
        break;
      }
      default:
        set_error("corrupt program");
        return CM_ERR_INVALID_ARG;
    }
  }
  return CM_OK;
}

// Build the program as an explicit HIP graph.  Nodes are the launches and
// copies; edges are exactly the program's happens-before: each node follows
// the previous node of its stream, and a wait adds every node the waited
// event's record followed.  (Record and wait are not nodes.)  Trace events,
// when asked for, become event-record nodes around each op.
cm_status build_graph(const Compiled *cp, char *const base[4], int n_streams, cm_trace *trace, GraphEntry *g) {
  hipError_t e;
  hipGraph_t graph;
  if ((e = hipGraphCreate(&graph, 0)) != hipSuccess) return hip_fail(e, "hipGraphCreate");
  g->graph = graph;
  std::vector<std::vector<hipGraphNode_t>> frontier(n_streams);
  std::vector<std::vector<hipGraphNode_t>> event_frontier(cp->prog.n_events);
  auto add_after = [&](int s, hipGraphNode_t node) { frontier[s].assign(1, node); };
  if (trace) {
    trace->used = 0;
    trace->overflow = false;
    trace->spans.clear();
    hipGraphNode_t n;
    if ((e = hipGraphAddEventRecordNode(&n, graph, nullptr, 0, trace->entry)) != hipSuccess)
      return hip_fail(e, "hipGraphAddEventRecordNode");
    for (int s = 0; s < n_streams; ++s) add_after(s, n);
  }
  auto trace_node = [&](int s, hipEvent_t ev) -> cm_status {
    hipGraphNode_t n;
    hipError_t er = hipGraphAddEventRecordNode(&n, graph, frontier[s].data(), frontier[s].size(), ev);
    if (er != hipSuccess) return hip_fail(er, "hipGraphAddEventRecordNode");
    add_after(s, n);
    return CM_OK;
  };
  const std::vector<cm_op_rec> &ops = cp->prog.ops;
  for (size_t i = 0; i < ops.size(); ++i) {
    const cm_op_rec &o = ops[i];
    const int s = o.stream;
    if (o.kind == CM_OPK_RECORD) {
      event_frontier[o.event] = frontier[s];
      continue;
    }
    if (o.kind == CM_OPK_WAIT) {
      for (hipGraphNode_t n : event_frontier[o.event])
        if (std::find(frontier[s].begin(), frontier[s].end(), n) == frontier[s].end()) frontier[s].push_back(n);
      continue;
    }
    int span = -1;
    if (trace) {
      if (trace->used < trace->capacity) {
        span = trace->used++;
        cm_span sp{};
        sp.kind = o.kind;
        sp.stream = o.stream;
        sp.step = o.step;
        sp.chunk = o.chunk;
        trace->spans.push_back(sp);
        cm_status st = trace_node(s, trace->ev[2 * span]);
        if (st != CM_OK) return st;
      } else {
        trace->overflow = true;
      }
    }
    hipGraphNode_t node;
    if (cp->skipped(o)) {
      // the operation's place in the ordering stays; its work does not
      e = hipGraphAddEmptyNode(&node, graph, frontier[s].data(), frontier[s].size());
      if (e != hipSuccess) return hip_fail(e, "hipGraphAddEmptyNode");
    } else if (o.kind == CM_OPK_COPY) {
      e = hipGraphAddMemcpyNode1D(&node, graph, frontier[s].data(), frontier[s].size(), base[o.dst_buf] + o.dst_off,
                                  base[o.src_buf] + o.src_off, o.bytes, cp->copy_kind);
      if (e != hipSuccess) return hip_fail(e, "hipGraphAddMemcpyNode1D (ring hop)");
    } else if (o.kind == CM_OPK_GEMM || o.kind == CM_OPK_REDUCE) {
      const Launch &L = cp->launches[cp->launch_of_op[i]];
      GemmParams p = L.p;
      for (int b = 0; b < 4; ++b) p.base[b] = base[b];
      KernelLaunch kl;
      if (o.kind == CM_OPK_GEMM) {
        if (!gemm_launch_config(p, L.tm, L.tn, &kl)) { set_error("no kernel for tile"); return CM_ERR_UNSUPPORTED; }
      } else {
        reduce_launch_config(p, &kl);
      }
      void *args[] = {&p};
      hipKernelNodeParams kp{};
      kp.func = kl.func;
      kp.gridDim = kl.grid;
      kp.blockDim = kl.block;
      kp.sharedMemBytes = 0;
      kp.kernelParams = args;
      kp.extra = nullptr;
      e = hipGraphAddKernelNode(&node, graph, frontier[s].data(), frontier[s].size(), &kp);
      if (e != hipSuccess) return hip_fail(e, "hipGraphAddKernelNode");
    } else {
      set_error("corrupt program");
      return CM_ERR_INVALID_ARG;
    }
    add_after(s, node);
    if (span >= 0) {
      cm_status st = trace_node(s, trace->ev[2 * span + 1]);
      if (st != CM_OK) return st;
    }
  }
  if ((e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0)) != hipSuccess)
    return hip_fail(e, "hipGraphInstantiate");
  if (trace) {
    g->spans = trace->spans;
    g->overflow = trace->overflow;
  }
  return CM_OK;
}

std::string graph_key(const cm_plan &pl, char *const base[4], const cm_trace *trace) {
  char buf[160];
  std::snprintf(buf, sizeof buf, "|%p %p %p %p %p", (void *)base[0], (void *)base[1], (void *)base[2],
                (void *)base[3], (const void *)trace);
  return plan_key(pl) + buf;
}

cm_status run(const cm_plan *pl, Entry want, const void *x, const void *w, void *y, void *ws, size_t ws_bytes,
              void *compute, void *const *comm, int n_comm, cm_trace *trace) {
  cm_status st = validate_call(pl, want, x, w, y, ws, ws_bytes, compute, comm, n_comm);
  if (st != CM_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != CM_OK) return st;
  if (trace && trace->device != dev) { set_error("trace was created on another device"); return CM_ERR_INVALID_ARG; }
  if ((st = refuse_capture(compute, comm, n_comm)) != CM_OK) return st;
  const Compiled *cp;
  if ((st = get_compiled(*pl, &cp)) != CM_OK) return st;
  std::vector<hipEvent_t> *evp;
  if ((st = event_pool(dev, cp->prog.n_events, &evp)) != CM_OK) return st;

  char *base[4] = {const_cast<char *>(static_cast<const char *>(x)), const_cast<char *>(static_cast<const char *>(w)),
                   static_cast<char *>(y), static_cast<char *>(ws)};
  hipStream_t streams[CM_MAX_COMM + 1];
  streams[0] = static_cast<hipStream_t>(compute);
  for (int i = 0; i < n_comm; ++i) streams[i + 1] = static_cast<hipStream_t>(comm[i]);

  if (pl->desc.exec_mode == CM_EXEC_EAGER) return enqueue(cp, *evp, base, streams, trace);

  std::string key = graph_key(*pl, base, trace);
  GraphCache &gc = graph_cache();
  std::lock_guard<std::mutex> lock(gc.mu);
  auto it = gc.map.find(key);
  hipError_t e;
  if (it == gc.map.end()) {
    if (gc.map.size() >= kMaxGraphs) {
      if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "hipDeviceSynchronize (graph cache)");
      for (size_t i = 0; i < kMaxGraphs / 4 && !gc.lru.empty(); ++i) {
        gc.map.erase(gc.lru.back());
        gc.lru.pop_back();
      }
    }
    auto g = std::make_unique<GraphEntry>();
    g->trace = trace;
    if ((st = build_graph(cp, base, n_comm + 1, trace, g.get())) != CM_OK) return st;
    gc.lru.push_front(key);
    GraphCache::Slot slot;
    slot.g = std::move(g);
    slot.pos = gc.lru.begin();
    it = gc.map.emplace(key, std::move(slot)).first;
  } else {
    gc.lru.splice(gc.lru.begin(), gc.lru, it->second.pos);
  }
  GraphEntry *ge = it->second.g.get();
  if (trace) {
    trace->spans = ge->spans;
    trace->used = (int)trace->spans.size();
    trace->overflow = ge->overflow;
  }
  if ((e = hipGraphLaunch(ge->exec, streams[0])) != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return CM_OK;
}

}  // namespace

// Graphs that record a trace's events must not outlive the trace: drop them
// in every thread's view (the cache is process-wide), after the device has
// finished any launch of them.
void forget_graphs_of(const cm_trace *t) {
  GraphCache &gc = graph_cache();
  std::lock_guard<std::mutex> lock(gc.mu);
  bool any = false;
  for (const auto &kv : gc.map) any = any || kv.second.g->trace == t;
  if (!any) return;
  (void)hipDeviceSynchronize();
  for (auto it = gc.map.begin(); it != gc.map.end();) {
    if (it->second.g->trace == t) {
      gc.lru.erase(it->second.pos);
      it = gc.map.erase(it);
    } else {
      ++it;
    }
  }
}

// Calls made while the compute stream or a comm stream is being captured
// into a graph are refused: the programs are multi-stream, and the library
// builds its own graphs node by node instead of through stream capture.
cm_status refuse_capture(void *compute, void *const *comm, int n_comm) {
  auto capturing = [](void *s, bool *out) -> cm_status {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(static_cast<hipStream_t>(s), &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    *out = cs != hipStreamCaptureStatusNone;
    return CM_OK;
  };
  bool cap = false;
  cm_status st = capturing(compute, &cap);
  for (int i = 0; st == CM_OK && !cap && comm && i < n_comm; ++i) st = capturing(comm[i], &cap);
  if (st != CM_OK) return st;
  if (cap) {
    set_error("a stream passed to the call is being captured into a graph; stream capture is not supported "
              "(the library builds and caches its own graphs)");
    return CM_ERR_UNSUPPORTED;
  }
  return CM_OK;
}

}  // namespace collmm

extern "C" {

cm_status cm_ag_gemm(const cm_plan *plan, const void *x, const void *w, void *y, void *ws, size_t ws_bytes,
                     void *compute, void *const *comm, int n_comm, cm_trace *trace) {
  return collmm::run(plan, collmm::kEntryAG, x, w, y, ws, ws_bytes, compute, comm, n_comm, trace);
}

cm_status cm_gemm_rs(const cm_plan *plan, const void *x, const void *w, void *y, void *ws, size_t ws_bytes,
                     void *compute, void *const *comm, int n_comm, cm_trace *trace) {
  return collmm::run(plan, collmm::kEntryRS, x, w, y, ws, ws_bytes, compute, comm, n_comm, trace);
}

cm_status cm_allgather(const cm_plan *plan, const void *x, void *y, void *compute, void *const *comm, int n_comm,
                       cm_trace *trace) {
  // the program reads only x and writes only y; x stands in for the unused weight pointer
  return collmm::run(plan, collmm::kEntryGather, x, x, y, y, 0, compute, comm, n_comm, trace);
}

cm_status cm_trace_create(int capacity, cm_trace **out) {
  if (!out || capacity < 1 || capacity > (1 << 20)) {
    collmm::set_error("cm_trace_create: need out != NULL and 1 <= capacity <= 2^20");
    return CM_ERR_INVALID_ARG;
  }
  auto t = std::make_unique<cm_trace>();
  hipError_t e = hipGetDevice(&t->device);
  if (e != hipSuccess) return collmm::hip_fail(e, "hipGetDevice");
  t->capacity = capacity;
  if ((e = hipEventCreate(&t->entry)) != hipSuccess) return collmm::hip_fail(e, "hipEventCreate");
  t->ev.resize(2 * (size_t)capacity);
  for (auto &ev : t->ev)
    if ((e = hipEventCreate(&ev)) != hipSuccess) return collmm::hip_fail(e, "hipEventCreate");
  *out = t.release();
  return CM_OK;
}

cm_status cm_trace_destroy(cm_trace *t) {
  if (!t) return CM_OK;
  collmm::forget_graphs_of(t);
  if (t->entry) (void)hipEventDestroy(t->entry);
  for (auto &ev : t->ev)
    if (ev) (void)hipEventDestroy(ev);
  delete t;
  return CM_OK;
}

cm_status cm_trace_read(cm_trace *t, cm_span *spans, int cap, int *n_spans, double *total_us) {
  if (!t || !n_spans) { collmm::set_error("null argument"); return CM_ERR_INVALID_ARG; }
  *n_spans = t->used;
  if (t->overflow) { collmm::set_error("trace capacity %d exceeded", t->capacity); return CM_ERR_CAPACITY; }
  if (cap < t->used || (!spans && t->used > 0)) { collmm::set_error("span array too small"); return CM_ERR_CAPACITY; }
  double last = 0;
  for (int i = 0; i < t->used; ++i) {
    float a, b;
    hipError_t e = hipEventElapsedTime(&a, t->entry, t->ev[2 * i]);
    if (e != hipSuccess) return collmm::hip_fail(e, "hipEventElapsedTime (synchronise the compute stream first)");
    e = hipEventElapsedTime(&b, t->entry, t->ev[2 * i + 1]);
    if (e != hipSuccess) return collmm::hip_fail(e, "hipEventElapsedTime");
    spans[i] = t->spans[i];
    spans[i].start_us = a * 1e3;
    spans[i].end_us = b * 1e3;
    if (spans[i].end_us > last) last = spans[i].end_us;
  }
  if (total_us) *total_us = last;
  return CM_OK;
}

}  // extern "C"
