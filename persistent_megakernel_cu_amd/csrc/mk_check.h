// mk_check.h -- test-support entry point of libmkcheck.so: the host-side
// address walk of a batch-1 megakernel plan (mk_check.cpp).
#ifndef MK_CHECK_H_
#define MK_CHECK_H_

#include "../../include/mk.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mkcheck_report {
  long long checks;      // index ranges checked
  long long violations;  // ranges outside their buffer (or broken structural rules)
  char first[256];       // the first violation, or the reason a plan was not walked
} mkcheck_report;

// Builds the plan of cfg on num_wgs workgroups and walks every task of its
// tape at decode position pos (0 <= pos < max_seq) through the kernels' own
// index helpers.  slack is added to every buffer limit (negative values
// tighten the check, so that the walk can be shown to catch overruns).
// Returns MK_OK with *out filled, MK_E_UNSUPPORTED for batched plans, or the
// planner's error code (out->first holds its message).
int mkcheck_walk(const mk_config* cfg, int num_wgs, int pos, long long slack, mkcheck_report* out);

#ifdef __cplusplus
}
#endif

#endif  // MK_CHECK_H_
