// Declarations shared by the planner and the executor (host side only).
#pragma once
#include <cstdarg>
#include <cstddef>
#include <vector>

#include "collmm.h"

namespace collmm {

// Byte offsets of the workspace regions a plan uses.
struct WsLayout {
  size_t slot_dir_bytes = 0;  // AG / RS decomposed: bytes of one direction's slots
  size_t part_dir_bytes = 0;  // RS add-and-forward: bytes of one direction's partial slots
  size_t gather = 0;          // AG naive: gathered activations
  size_t partial = 0;         // RS pipe / naive: partial products
  size_t partial_bytes = 0;
  size_t ring = 0;            // RS pipe / naive: ring slots; RS direct: receive slots
  size_t acc = 0;             // RS direct: the owners' home accumulators
  size_t total = 0;
};

struct Program {
  std::vector<cm_op_rec> ops;
  std::vector<cm_job_rec> jobs;
  int n_events = 0;
};

void set_error(const char *fmt, ...);
// The compiled GEMM block tile that fits `jobs` jobs of rows x cols outputs best.
double choose_gemm_tile(int rows, int cols, int jobs, int *tm, int *tn);
const char *last_error();
cm_status validate_desc(const cm_plan_desc &d);
cm_status plan(const cm_plan_desc *desc, cm_plan *out);
WsLayout ws_layout(const cm_plan &p);
void build_program(const cm_plan &p, Program &prog);
// CM_ERR_UNSUPPORTED if the compute stream or a comm stream is being
// captured into a graph (executor; streams are hipStream_t passed as void*).
cm_status refuse_capture(void *compute, void *const *comm, int n_comm);

}  // namespace collmm
