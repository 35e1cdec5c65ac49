// mk_inst.hip -- one instance of the persistent decode megakernel and of its
// one-stage-per-launch variant, selected at build time by MK_INST_G (query
// heads per kv head), MK_INST_D (head_dim), MK_INST_B (1: batched plans),
// MK_INST_GT (query heads per attention task, 0: chosen at run time) and
// MK_INST_F (instance flags: 1 trace stamps, 2 partial-input down projection).
// The library builds this file once per instance, in parallel.
#include "mk_device.h"

#if !defined(MK_INST_G) || !defined(MK_INST_D) || !defined(MK_INST_B) || !defined(MK_INST_GT) || !defined(MK_INST_F)
#error "build with -DMK_INST_G=<1|2|4> -DMK_INST_D=<64|128> -DMK_INST_B=<0|1> -DMK_INST_GT=<0|1|G> -DMK_INST_F=<0..3>"
#endif

#define MK_CAT10(a, b, c, d, e, f, g, h, i, j) a##b##c##d##e##f##g##h##i##j
#define MK_INSTANCE_NAME(g, d, b, gt, f) MK_CAT10(instance_, g, _, d, _, b, _, gt, _, f)
#define MK_INST_ARGS MK_INST_G, MK_INST_D, MK_INST_B != 0, MK_INST_GT, MK_INST_F

namespace mk {

template __global__ void mk_persistent<MK_INST_ARGS>(Params);
template __global__ void mk_stage<MK_INST_ARGS>(Params, int);
template __global__ void mk_persistent_steps<MK_INST_ARGS>(Params, int);

KernelPair MK_INSTANCE_NAME(MK_INST_G, MK_INST_D, MK_INST_B, MK_INST_GT, MK_INST_F)() {
  return {reinterpret_cast<const void*>(&mk_persistent<MK_INST_ARGS>),
          reinterpret_cast<const void*>(&mk_stage<MK_INST_ARGS>),
          reinterpret_cast<const void*>(&mk_persistent_steps<MK_INST_ARGS>)};
}

}  // namespace mk
