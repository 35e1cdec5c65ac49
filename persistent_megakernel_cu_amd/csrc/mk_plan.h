// mk_plan.h -- host-side planning: packed weight layout, task tape, LDS layout.
#ifndef MK_PLAN_H_
#define MK_PLAN_H_

#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {

struct Plan {
  // model and run dimensions
  int L = 0, H = 0, Hp = 0, NQ = 0, NKV = 0, D = 0, G = 0;
  int QD = 0, QDp = 0, KVD = 0, F = 0, Fp = 0, V = 0, S = 0, B = 0;
  int W = 0;       // persistent workgroups
  int C = 0;       // attention chunks per kv head (and sequence)
  int attn_slices = 1;  // batch 1: attention tasks per (kv head, chunk), one per query head or 1
  bool batched = false;  // B > 1: tiled weights, MFMA tasks
  bool partial = false;  // batch 1: down-projection tasks start on partial input (kRegionPartial)
  bool prefill = false;  // batched: the B rows are consecutive tokens of one sequence (one KV cache)
  int stages = 0;  // kStagesPerLayer * L + 1
  bool tied = true;

  // packed arena: per-layer matrix byte offsets
  std::vector<uint64_t> off_qkv, off_o, off_gu, off_down;
  uint64_t arena_bytes = 0;
  bool lm_borrowed = false;  // LM head read straight from the caller's matrix
  uint64_t lm_bytes = 0;     // bytes of the library-owned LM head copy (0 if borrowed)

  // tape [stage][wg]
  std::vector<Task> tape;
  int num_tasks = 0;

  // LDS layout
  int act_floats = 0, res_floats = 0, ring_units = 0;
  int lds_act = 0, lds_res = 0, lds_rope = 0, lds_misc = 0, lds_part = 0, lds_tape = 0, lds_bytes = 0, act_stride = 0;

  std::string error;
};

// Rows of each packed matrix and its padded row length (elements).
uint64_t qkv_rows(const Plan& p);

// Build the plan for cfg on W workgroups.  Returns MK_OK or an MK_E_* code
// (with p.error set).  Does not touch any GPU.
int plan_build(const mk_config& cfg, int W, Plan& p);

// Device workspace of a megakernel handle (one allocation): byte offset and
// byte size of each buffer (see Params for their layouts).
struct WsBuf {
  size_t off, bytes;
};
struct Workspace {
  WsBuf x_attn, x_ffn, q, kvcur, o, h, kpart, attn_part, attn_ctr, amax, amax_ctr, tokerr, abort_flag, status, dargs,
      tok_tag;
  size_t bytes;  // the whole allocation
};
Workspace layout_workspace(const Plan& p);

// Check the tape: stage order, exact coverage of every row pair and every
// attention (kv head, chunk), byte bounds of every task, LDS limits.
int plan_validate(const Plan& p, std::string* why);

}  // namespace mk

#endif  // MK_PLAN_H_
