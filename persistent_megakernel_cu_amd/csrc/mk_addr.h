// mk_addr.h -- the index arithmetic of every global-memory access of the
// batch-1 executors (weight stream, activation staging, epilogue stores,
// attention K/V reads, split-KV partials and counters), written once and used
// both by the kernels in mk_device.h and by the host-side address walk
// (mk_check.cpp), which replays a plan's tape through these same functions
// and checks every index against the size of the buffer it falls in.
//
// Every helper returns an element index (or, for weights, a byte offset)
// relative to the buffer named in its comment.
#ifndef MK_ADDR_H_
#define MK_ADDR_H_

#include <stddef.h>
#include <stdint.h>

#include "mk_internal.h"

#if defined(__HIPCC__)
#define MK_HD __host__ __device__ __forceinline__
#else
#define MK_HD inline
#endif

namespace mk {
namespace addr {

// Row block of layer l in a [L][n] buffer (activations, gains).
MK_HD size_t layer_off(int l, int n) { return (size_t)l * n; }

// First element of token tok's row of the [V][H] embedding.
MK_HD size_t embed_row(int tok, int H) { return (size_t)tok * H; }

// cos/sin pairs of position pos in the [S][D] RoPE table.
MK_HD size_t rope_row(int pos, int D) { return (size_t)pos * D; }

// This step's k (which = 0) or v (which = 1) rows of layer l in kvcur [L][2][KVD].
MK_HD size_t kvcur_off(int l, int KVD, int which) { return ((size_t)l * 2 + which) * KVD; }

// Slot pos, element 0, of kv head g of layer l in a [L][NKV][S][D] cache.
MK_HD size_t kv_slot(int l, int NKV, int g, int S, int pos, int D) {
  return (((size_t)l * NKV + g) * S + pos) * D;
}
// Slot 0 of kv head g of layer l in the same cache.
MK_HD size_t kv_head(int l, int NKV, int g, int S, int D) { return ((size_t)l * NKV + g) * S * D; }

// Query head g * GQ + hq0 (its D elements) of layer l in q / o [L][QD].
MK_HD size_t head_off(int l, int QD, int g, int GQ, int hq0, int D) {
  return (size_t)l * QD + (size_t)(g * GQ + hq0) * D;
}

// Split-KV partial record of (layer l, kv head g, chunk ch) in attn_part
// [L][NKV][C][stride] (stride = GQ * (D + 2) floats: m[GQ], l[GQ], acc[GQ][D]).
MK_HD size_t attn_rec(int l, int NKV, int g, int C, int ch, int stride) {
  return (((size_t)l * NKV + g) * C + ch) * stride;
}
// Merge counter of (layer l, kv head g, head slice) in attn_ctr [L][NKV][GQ].
MK_HD size_t attn_ctr(int l, int NKV, int g, int GQ, int slice) { return ((size_t)l * NKV + g) * GQ + slice; }

// Weight stream: item `item` of a task over pairs from a0, 2^kslog items per
// pair, upi units per item: its pair, and the pair-relative index of unit u.
MK_HD uint32_t item_pair(uint32_t a0, uint32_t item, uint32_t kslog) { return a0 + (item >> kslog); }
MK_HD uint32_t item_unit(uint32_t item, uint32_t kslog, uint32_t upi, uint32_t u) {
  return (item & ((1u << kslog) - 1u)) * upi + u;
}
// Byte offset, from the matrix base (arena + wofs, or the LM head), of lane
// `lane`'s 16 bytes of unit `unit` of row pair `pair` (nu units per pair).
MK_HD uint64_t unit_byte(uint32_t pair, uint32_t nu, uint32_t unit, uint32_t lane) {
  return ((uint64_t)pair * nu + unit) * kUnitBytes + lane * 16u;
}

// LDS: first of the 8 activation floats that lane `lane` multiplies with its
// 16 bytes of activation unit `unit` (unit u covers columns 512 u .. 512 u + 511).
MK_HD int act_unit(int unit, int lane) { return unit * kUnitElems + lane * 8; }

// LDS: the attention scratch of a task of GT query heads of D dims, in floats
// from the activation base: q [GT][D], k [D], v [D], per-wave partial outputs
// [waves][GT][D], per-wave max [waves][GT], per-wave sum [waves][GT].
struct AttnLds {
  int qs, kcur, vcur, wpart, wm, wl, end;
};
MK_HD AttnLds attn_lds(int GT, int D) {
  AttnLds a;
  a.qs = 0;
  a.kcur = a.qs + GT * D;
  a.vcur = a.kcur + D;
  a.wpart = a.vcur + D;
  a.wm = a.wpart + kWaves * GT * D;
  a.wl = a.wm + kWaves * GT;
  a.end = a.wl + kWaves * GT;
  return a;
}

}  // namespace addr
}  // namespace mk

#endif  // MK_ADDR_H_
