// mk_device.h -- gfx950 device code of the persistent decode megakernel: the
// primitives, the fused executors, the stage loop and the kernel templates
// (the persistent kernel and its one-stage-per-launch variant).  Each kernel
// instance (query heads per kv head, head_dim, batched or not) is compiled in
// a translation unit of its own (mk_inst.hip) so that the instances build in
// parallel.
//
// Mechanism, after "Revolution der KI-Beschleunigung: Wie ein Low-Latency
// Megakernel den Llama-1B Turbo zuendet" (dasgeld.co) and the glossary entry
// "Megakernel" (synthszr.com, section "Wie eine ganze Rechenkette in ein
// Programm passt"):
//  * the whole forward pass runs in one kernel; every workgroup stays resident
//    on its compute unit and walks its column of a host-planned task tape;
//  * instead of kernel boundaries, a task waits until its inputs carry this
//    step's tag in device memory (the article's counters/signals in GPU main
//    memory that tell an instruction when its dependencies are met);
//  * the next weights are loaded while a task still waits: each wave keeps a
//    ring of 1 KiB weight units in LDS filled by asynchronous global->LDS
//    loads that run ahead across task boundaries (the article's paged shared
//    memory, where one load starts while another is still finishing).
//
// MI355X specifics that shape the code (measured on the part): an agent-scope
// release/acquire fence pair (L2 writeback + invalidate) costs ~20 us for a
// 256-workgroup exchange, and 256 workgroups on one counter serialise to
// ~4 us, while an agent-coherent 8-byte store/load round trip is ~0.6 us.
// So every activation element travels as one 4-byte tagged word (the fp32
// value rounded to 24 bits, the step's epoch in the low byte) written and read
// with agent-scope accesses: the consumer polls the data itself, no fence and
// no counter sits on the critical path.
#ifndef MK_DEVICE_H_
#define MK_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"
#include "mk_addr.h"
#include "mk_internal.h"

namespace mk {

typedef __attribute__((address_space(3))) const char lds_cchar;

// ---------------------------------------------------------------------------
// primitives
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t lds_byte(const void* p) { return (uint32_t)(uintptr_t)((lds_cchar*)p); }

// One 16-byte-per-lane asynchronous load of global memory into LDS at
// m0 + 16 * lane.  Issued from inline assembly so that the compiler does not
// see it: it would otherwise wait for every such load before any LDS read.
// Non-temporal (nt): every weight byte is read once per step, and a stream
// of several GB per step would otherwise keep evicting from the L2 what is
// read again soon: the kernel's code (larger than the instruction cache,
// refetched at every stage), the activations that every workgroup of an XCD
// stages, and the KV rows.
__device__ __forceinline__ void dma_unit(const char* gsrc, uint32_t lds_dst) {
  uint32_t keep;
  lds_dst = __builtin_amdgcn_readfirstlane(lds_dst);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(gsrc), "s"(lds_dst)
      : "memory");
}

// Read 16 bytes of a ring slot after at most N younger vector-memory loads
// remain outstanding (loads complete in issue order).
template <int N>
__device__ __forceinline__ uint4 ring_read(uint32_t lds_addr) {
  uint4 v;
  asm volatile("s_waitcnt vmcnt(%1)\n\tds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(v)
               : "n"(N), "v"(lds_addr)
               : "memory");
  return v;
}

__device__ __forceinline__ void wait_all_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Four LDS reads of 16 bytes issued back to back, one wait for all of them.
__device__ __forceinline__ void lds_read4(uint4 (&v)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// Tagged activation word: an fp32 value rounded to 24 high bits (relative
// error <= 2^-16) whose low byte carries the step's tag (epoch mod 256).  A
// 4-byte store is single-copy atomic, so a reader that sees this step's tag
// sees this step's value; every buffer is rewritten on every step, so the
// previous step's tag (epoch - 1) never matches.  Readers clear the tag bits,
// so values do not depend on the epoch.
typedef uint32_t tword;
__device__ __forceinline__ void st_tag(tword* p, float v, uint32_t epoch) {
  const uint32_t w = ((__float_as_uint(v) + 0x80u) & 0xFFFFFF00u) | (epoch & 0xFFu);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ tword ld_tag(const tword* p) {
  return __hip_atomic_load(const_cast<tword*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ready(tword w, uint32_t epoch) { return ((w ^ epoch) & 0xFFu) == 0; }
__device__ __forceinline__ uint32_t tag_of(tword w) { return w & 0xFFu; }
__device__ __forceinline__ float tag_value(tword w) { return __uint_as_float(w & 0xFFFFFF00u); }
// A word that is ready with value v_bits (low byte zero), for elements that need no wait.
__device__ __forceinline__ tword ready_word(uint32_t epoch, uint32_t v_bits = 0u) { return v_bits | (epoch & 0xFFu); }
// Four consecutive tagged words (16-byte aligned) in one coherent load; each
// word is checked on its own, so a load that sees some new and some old words
// is simply polled again.
typedef uint32_t tword4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const volatile tword4 gtword4;
// Two scopes for the same four words.  The volatile 16-byte load is issued at
// system scope (sc0 sc1) and is the faster one for the batch-1 path's small
// stagings (one 16-byte group per thread), which are latency-bound.  The
// batched path stages the activations of every sequence (up to 64 KB per
// workgroup, every workgroup at once) and is bound by the fabric's throughput
// for coherent loads; there the agent-scope load (sc1 alone: bypasses this
// XCD's L2, whose copy of a line that another XCD rewrote may be stale) moves
// the same bytes faster: 1328 -> 1211 us per 8-sequence step.
__device__ __forceinline__ tword4 ld_tag4(const tword* p) { return *(gtword4*)p; }
// Cache-policy operand of a gfx950 buffer load that sets sc1 alone (agent scope).
constexpr int kCachePolicyAgent = 16;
// Fourth word of a raw (untyped, unswizzled) gfx9 buffer resource.
constexpr int kBufferRsrcWord3 = 0x00020000;
// A buffer resource over the words [base, base + bytes / 4) (base wave-uniform).
// An offset past the range reads zeros: a wrong tag, polled until the watchdog
// stops the kernel, never a fault.
struct TagBuf {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ TagBuf tag_buf(const tword* base, uint32_t bytes) {
  return TagBuf{__builtin_amdgcn_make_buffer_rsrc(const_cast<tword*>(base), (short)0, (int)bytes, kBufferRsrcWord3)};
}
// Four tagged words at word offset `word` of the resource, at agent scope.
__device__ __forceinline__ tword4 ld_tag4_agent(const TagBuf& b, uint32_t word) {
  return __builtin_amdgcn_raw_buffer_load_b128(b.r, (int)(word * 4u), 0, kCachePolicyAgent);
}
// Four tagged words at p at agent scope, as two 8-byte atomic loads (for
// per-thread addresses that no single resource covers).
__device__ __forceinline__ tword4 ld_tag4_agent(const tword* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<tword*>(p));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return tword4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
__device__ __forceinline__ bool tag4_ready(tword4 w, uint32_t epoch) {
  return ((((w.x ^ epoch) | (w.y ^ epoch) | (w.z ^ epoch) | (w.w ^ epoch)) & 0xFFu) == 0);
}
__device__ __forceinline__ tword4 ready_word4(uint32_t epoch) {
  const tword r = ready_word(epoch);
  return tword4{r, r, r, r};
}
__device__ __forceinline__ float4 tag_value4(tword4 w) {
  return make_float4(tag_value(w.x), tag_value(w.y), tag_value(w.z), tag_value(w.w));
}
// Two bf16 of a KV-cache row, stored at agent scope: a multi-step launch
// reads the slot on other compute units in the next step.
__device__ __forceinline__ void st_kv(uint16_t* dst, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(dst), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_u64_agent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f32_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f32_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Cross-lane data movement within rows of 16 lanes (DPP).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Wave64 sum: butterflies inside each 16-lane row (quad_perm xor 1, xor 2,
// row_half_mirror, row_mirror) leave every lane of a row with the row total,
// then the four row totals are added in a fixed order.  Every lane returns the
// same value.  Must be called with all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// 8 bf16 weights (one lane's share of a unit) dotted with 8 fp32 activations in LDS.
__device__ __forceinline__ float dot8(const uint4 w, const float* x) {
  const float4 a = *reinterpret_cast<const float4*>(x);
  const float4 b = *reinterpret_cast<const float4*>(x + 4);
  float s = bf_lo(w.x) * a.x;
  s = fmaf(bf_hi(w.x), a.y, s);
  s = fmaf(bf_lo(w.y), a.z, s);
  s = fmaf(bf_hi(w.y), a.w, s);
  s = fmaf(bf_lo(w.z), b.x, s);
  s = fmaf(bf_hi(w.z), b.y, s);
  s = fmaf(bf_lo(w.w), b.z, s);
  s = fmaf(bf_hi(w.w), b.w, s);
  return s;
}

// Same with the 8 activations already in registers.
__device__ __forceinline__ float dot8r(const uint4 w, const float4 a, const float4 b) {
  float s = bf_lo(w.x) * a.x;
  s = fmaf(bf_hi(w.x), a.y, s);
  s = fmaf(bf_lo(w.y), a.z, s);
  s = fmaf(bf_hi(w.y), a.w, s);
  s = fmaf(bf_lo(w.z), b.x, s);
  s = fmaf(bf_hi(w.z), b.y, s);
  s = fmaf(bf_lo(w.w), b.z, s);
  s = fmaf(bf_hi(w.w), b.w, s);
  return s;
}

// Argmax key: larger key = larger value, ties -> lower index; 0 = no candidate.
// A NaN is no candidate (it never wins), and -0 is keyed as +0 (they compare
// equal, so the lower index must win between them too).
__device__ __forceinline__ uint64_t amax_key(float v, int idx) {
  if (idx < 0 || v != v) return 0;
  const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(~(uint32_t)idx);
}

// ---------------------------------------------------------------------------
// per-workgroup context
// ---------------------------------------------------------------------------

struct Ctx {
  int b;      // workgroup
  int tid, wave, lane;
  int pos;
  uint32_t epoch;
  float* act;
  float* res;
  float* rope;
  float* red;         // [kWaves] scratch
  uint64_t* red64;    // [kWaves]
  int* flags;         // [0] abort seen, [1] last-arriver, [2] token
  int* tok;           // [B] this step's input tokens (LDS)
  float* logits;      // this step's logits [B][V]
  int32_t* out_tok;   // this step's greedy tokens [B]
  float* part;        // [kMaxItems] partial sums of split items
  uint64_t* tr;       // trace record of the current stage, or null
  float rs;           // RMSNorm scale of the staged activation (1 if none)
};

// Trace stamp k of the current (workgroup, stage) record.
__device__ __forceinline__ void mark(Ctx& c, int k) {
  if (c.tr != nullptr && c.tid == 0) c.tr[k] = wall_clock64();
}
// Per-wave stamp: this wave finished its own part of the task.
__device__ __forceinline__ void mark_wave(Ctx& c) {
  if (c.tr != nullptr && c.lane == 0) c.tr[4 + c.wave] = wall_clock64();
}
// Per-wave stamp: this wave's first weight unit of the task is in registers.
__device__ __forceinline__ void mark_first(Ctx& c, bool& done) {
  if (!done && c.tr != nullptr && c.lane == 0) c.tr[4 + kWaves + c.wave] = wall_clock64();
  done = true;
}

// Latch the first device error; a timeout also stops every workgroup.
__device__ __forceinline__ void latch_error(const Params& P, int code, int stage, uint32_t detail) {
  int expected = 0;
  if (__hip_atomic_compare_exchange_strong(&P.status->code, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    P.status->stage = stage;
    P.status->wg = (int)blockIdx.x;
    P.status->detail = detail;
    __hip_atomic_store(&P.status_host->stage, stage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&P.status_host->wg, (int)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&P.status_host->detail, detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&P.status_host->code, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if (code == MK_E_TIMEOUT) __hip_atomic_store(P.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wall-clock ticks (100 MHz, 20 us) a wait runs before it checks the abort flag.
constexpr uint64_t kAbortCheckTicks = 2000;

// One poll iteration's bookkeeping; true when the wait must stop.
__device__ __forceinline__ bool poll_stop(const Params& P, uint64_t& t0, int stage, uint32_t seen) {
  const uint64_t now = wall_clock64();
  if (t0 == 0) {
    t0 = now | 1;
    return false;
  }
  if (now - t0 > P.watchdog_ticks) {
    latch_error(P, MK_E_TIMEOUT, stage, seen);
    return true;
  }
  // The abort flag is raised only by another workgroup's watchdog, long after
  // any normal wait has ended: skip its coherent load (one per wave and poll
  // round) during the first kAbortCheckTicks of a wait.
  if (now - t0 < kAbortCheckTicks) return false;
  return ld_u32_agent(P.abort_flag) != 0;
}

// A run of tagged elements to stage into LDS: dst[i] = value(src[i]) * scale.
struct Seg {
  float* dst;
  const tword* src;
  int n;
  float scale;
};

// 16-byte loads (4 tagged words) per thread issued in one staging round:
// 8192 words per round for one sequence, 16384 for a batch.
constexpr int kStageLoads = 4;
constexpr int kStageLoadsBatch = 8;

// Source of the 4-word group starting at flat index i over the segments
// (null past the end).  Segment lengths are multiples of 4.
template <int NSEG>
__device__ __forceinline__ const tword* seg_src(const Seg (&seg)[NSEG], int i) {
  const tword* r = nullptr;
#pragma unroll
  for (int k = 0; k < NSEG; ++k) {
    if (i >= 0 && i < seg[k].n) r = seg[k].src + i;
    i -= seg[k].n;
  }
  return r;
}

// Store the group of 4 values starting at flat index i into its segment's LDS destination.
template <int NSEG>
__device__ __forceinline__ void seg_store(const Seg (&seg)[NSEG], int i, tword4 w) {
#pragma unroll
  for (int k = 0; k < NSEG; ++k) {
    if (i >= 0 && i < seg[k].n) {
      const float4 v = tag_value4(w);
      const float sc = seg[k].scale;
      *reinterpret_cast<float4*>(seg[k].dst + i) = make_float4(v.x * sc, v.y * sc, v.z * sc, v.w * sc);
    }
    i -= seg[k].n;
  }
}

// Copy tagged segments into LDS as fp32 once every element carries this
// step's tag, and zero zdst[zfrom, zto).  WG-cooperative.  All loads of a
// round are issued before any is checked, and the first round's loads are in
// flight before the barrier that separates these LDS writes from the previous
// task's last LDS reads.  Ends with a barrier; false if the wait was aborted.
template <int NSEG, int NL = kStageLoads>
__device__ __forceinline__ bool stage_tagged(const Params& P, Ctx& c, const Seg (&seg)[NSEG], int stage,
                                             float* zdst = nullptr, int zfrom = 0, int zto = 0) {
  int total = 0;
#pragma unroll
  for (int k = 0; k < NSEG; ++k) total += seg[k].n;
  bool stop = false;
  for (int i0 = 0; i0 == 0 || i0 < total; i0 += 4 * kThreads * NL) {
    tword4 w[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const tword* p = seg_src(seg, i0 + 4 * (j * kThreads + c.tid));
      w[j] = p ? ld_tag4(p) : ready_word4(c.epoch);
    }
    uint64_t t0 = 0;
    while (!stop) {
      bool ready = true;
#pragma unroll
      for (int j = 0; j < NL; ++j) ready &= tag4_ready(w[j], c.epoch);
      if (ready) break;
      if (poll_stop(P, t0, stage, tag_of(w[0].x))) {
        stop = true;
        break;
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        if (!tag4_ready(w[j], c.epoch)) {
          const tword* p = seg_src(seg, i0 + 4 * (j * kThreads + c.tid));
          if (p) w[j] = ld_tag4(p);
        }
      }
    }
    if (i0 == 0) {
      __syncthreads();
      for (int i = zfrom + c.tid; i < zto; i += kThreads) zdst[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) seg_store(seg, i0 + 4 * (j * kThreads + c.tid), w[j]);
  }
  if (stop) c.flags[0] = 1;
  __syncthreads();
  return c.flags[0] == 0;
}

// Sum over the workgroup in a fixed order (every thread gets the same value).
__device__ __forceinline__ float block_sum(Ctx& c, float v) {
  v = wave_sum(v);
  if (c.lane == 0) c.red[c.wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += c.red[w];
  __syncthreads();
  return t;
}

// Stage the input x of an RMSNorm into LDS as dst[i] = x[i] * g[i] (i < n),
// zero dst[n, npad), and set c.rs = (mean(x^2) + eps)^(-1/2), so that
// W . rmsnorm(x) = c.rs * (W . dst).  x is either tagged (src) or, for the
// first layer, the bf16 embedding row of the input token (src == null).  The
// sum of squares is reduced under the barrier that ends the staging.
// WG-cooperative; false if the wait was aborted.
__device__ __forceinline__ bool stage_normed(const Params& P, Ctx& c, float* dst, const tword* src, const float* g,
                                             int n, int npad, int stage) {
  const uint16_t* emb = nullptr;
  if (src == nullptr) {
    if (c.tid == 0) {
      int tok = c.tok[0];
      if (tok < 0 || tok >= P.V) {
        latch_error(P, MK_E_TOKEN, stage, (uint32_t)tok);
        __hip_atomic_store(&P.tokerr[0], c.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tok = 0;
      }
      c.flags[2] = tok;
    }
    __syncthreads();
    emb = P.embed + addr::embed_row(c.flags[2], P.H);
  }
  // groups of 4 elements (n is a multiple of 4): one 16-byte load each
  float ss = 0.f;
  bool stop = false;
  for (int i0 = 0; i0 == 0 || i0 < n; i0 += 4 * kThreads * kStageLoads) {
    tword4 w[kStageLoads];
    float4 gv[kStageLoads];
    if (emb) {
      // in-bounds loads for every lane first (clamped index), then widen
      uint2 e16[kStageLoads];
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) {
        const int i = i0 + 4 * (j * kThreads + c.tid);
        const int ic = i < n ? i : n - 4;
        gv[j] = *reinterpret_cast<const float4*>(g + ic);
        e16[j] = *reinterpret_cast<const uint2*>(emb + ic);
      }
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j)
        w[j] = tword4{ready_word(c.epoch, e16[j].x << 16), ready_word(c.epoch, e16[j].x & 0xFFFF0000u),
                      ready_word(c.epoch, e16[j].y << 16), ready_word(c.epoch, e16[j].y & 0xFFFF0000u)};
    } else {
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) {
        const int i = i0 + 4 * (j * kThreads + c.tid);
        gv[j] = *reinterpret_cast<const float4*>(g + (i < n ? i : n - 4));
        w[j] = i < n ? ld_tag4(src + i) : ready_word4(c.epoch);
      }
    }
    uint64_t t0 = 0;
    while (!stop) {
      bool ready = true;
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) ready &= tag4_ready(w[j], c.epoch);
      if (ready) break;
      if (poll_stop(P, t0, stage, tag_of(w[0].x))) {
        stop = true;
        break;
      }
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) {
        const int i = i0 + 4 * (j * kThreads + c.tid);
        if (i < n && !tag4_ready(w[j], c.epoch)) w[j] = ld_tag4(src + i);
      }
    }
    if (i0 == 0) {
      __syncthreads();
      for (int i = n + c.tid; i < npad; i += kThreads) dst[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kStageLoads; ++j) {
      const int i = i0 + 4 * (j * kThreads + c.tid);
      if (i < n) {
        const float4 x = tag_value4(w[j]);
        ss = fmaf(x.x, x.x, ss);
        ss = fmaf(x.y, x.y, ss);
        ss = fmaf(x.z, x.z, ss);
        ss = fmaf(x.w, x.w, ss);
        *reinterpret_cast<float4*>(dst + i) =
            make_float4(x.x * gv[j].x, x.y * gv[j].y, x.z * gv[j].z, x.w * gv[j].w);
      }
    }
  }
  ss = wave_sum(ss);
  if (c.lane == 0) c.red[c.wave] = ss;
  if (stop) c.flags[0] = 1;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += c.red[w];
  c.rs = rsqrtf(t / (float)n + P.eps);
  return c.flags[0] == 0;
}

// This wave's columns [col0, col0 + 512 ug) of a tagged input vector of n
// elements (columns n and above read as 0) into act[]: lane l holds columns
// col0 + 512 u + 8 l .. + 8 of unit u.  Every word is polled until it carries
// this step's tag, up to four units (eight 16-byte loads per lane) in flight
// at a time.  Wave-level, no barrier; false if the wait gave up.
__device__ __forceinline__ bool wave_stage_cols(const Params& P, Ctx& c, const tword* src, int n, int col0, int ug,
                                                int stage) {
  for (int u0 = 0; u0 < ug; u0 += 4) {
    tword4 w[8];
    int col[8];
    bool live[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      col[j] = col0 + (u0 + (j >> 1)) * kUnitElems + c.lane * 8 + (j & 1) * 4;
      live[j] = u0 + (j >> 1) < ug && col[j] < n;
      w[j] = live[j] ? ld_tag4(src + col[j]) : ready_word4(c.epoch);
    }
    bool stop = false;
    uint64_t t0 = 0;
    while (true) {
      bool ready = true;
#pragma unroll
      for (int j = 0; j < 8; ++j) ready &= tag4_ready(w[j], c.epoch);
      if (ready) break;
      if (poll_stop(P, t0, stage, tag_of(w[0].x))) {
        stop = true;
        break;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (live[j] && !tag4_ready(w[j], c.epoch)) w[j] = ld_tag4(src + col[j]);
    }
    if (__any(stop)) return false;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (u0 + (j >> 1) < ug)
        *reinterpret_cast<float4*>(c.act + col[j]) = live[j] ? tag_value4(w[j]) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  return true;
}

// ---------------------------------------------------------------------------
// the per-wave weight stream (LDS ring, loader running ahead of the consumer)
// ---------------------------------------------------------------------------

// Task record of stage s for this workgroup, from the copy of its tape column
// that the workgroup keeps in LDS (a record read from memory by a scalar load
// can miss in the scalar cache for a microsecond, and the LDS reads of the
// weight ring would wait on that same counter).
__device__ __forceinline__ Task task_at(uint32_t tape_lds, int idx) {
  uint4 lo, hi;
  const uint32_t a = tape_lds + (uint32_t)idx * (uint32_t)sizeof(Task);
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(lo), "=&v"(hi)
               : "v"(a)
               : "memory");
  const uint32_t r0 = __builtin_amdgcn_readfirstlane(lo.x);
  Task t;
  t.op = (uint8_t)(r0 & 0xffu);
  t.region = (uint8_t)((r0 >> 8) & 0xffu);
  t.layer = (uint16_t)(r0 >> 16);
  t.a0 = __builtin_amdgcn_readfirstlane(lo.y);
  t.a1 = __builtin_amdgcn_readfirstlane(lo.z);
  t.nu = __builtin_amdgcn_readfirstlane(lo.w);
  t.wofs = (uint64_t)__builtin_amdgcn_readfirstlane(hi.x) | ((uint64_t)__builtin_amdgcn_readfirstlane(hi.y) << 32);
  t.ntasks = __builtin_amdgcn_readfirstlane(hi.z);
  t.kslog = __builtin_amdgcn_readfirstlane(hi.w);
  return t;
}

// Work items of a GEMV task for one wave: items wave, wave+8, ... of
// (a1 - a0) << kslog; item i is pair a0 + (i >> kslog), units
// [(i & (2^kslog - 1)) * upi, + upi) of that pair, upi = nu >> kslog.
struct Stream {
  uint32_t ring;  // LDS byte address of this wave's ring
  uint32_t tape;  // LDS byte address of the task record of stage s_begin
  int issued, consumed, lslot, cslot;
  int ls, s_begin, s_end, period;  // stages s_begin .. s_end - 1, the tape repeating every `period`
  uint32_t litem, lnitems, lkslog, lupi, lu, la0, lnu;
  uint32_t lc, lnc, lch;  // batched: chunk, chunks per row, tiles per chunk
  const char* lbase;
  bool ldone;
};

// Record of stage s of the stream's tape column (multi-step launches walk it repeatedly).
__device__ __forceinline__ Task stream_task(const Stream& st, int s) {
  int idx = s - st.s_begin;
  if (idx >= st.period) idx %= st.period;
  return task_at(st.tape, idx);
}

__device__ __forceinline__ void loader_seek(const Params& P, Stream& st, int s, int b, int wave) {
  for (; s < st.s_end; ++s) {
    const Task t = stream_task(st, s);
    if (op_is_gemv(t.op)) {
      const uint32_t n_items = (t.a1 - t.a0) << t.kslog;
      if ((uint32_t)wave < n_items) {
        st.ls = s;
        st.litem = (uint32_t)wave;
        st.lnitems = n_items;
        st.lkslog = t.kslog;
        st.lupi = t.nu >> t.kslog;
        st.lu = 0;
        st.la0 = t.a0;
        st.lnu = t.nu;
        st.lbase = ((t.region & kRegionLm) ? P.lm : P.arena) + t.wofs;
        return;
      }
    }
  }
  st.ls = st.s_end;
  st.ldone = true;
}

__device__ __forceinline__ void loader_issue(const Params& P, Stream& st, int b, int wave, int lane) {
  if (st.ldone) return;
  const uint32_t pair = addr::item_pair(st.la0, st.litem, st.lkslog);
  const uint32_t unit = addr::item_unit(st.litem, st.lkslog, st.lupi, st.lu);
  const char* g = st.lbase + addr::unit_byte(pair, st.lnu, unit, (uint32_t)lane);
  dma_unit(g, st.ring + (uint32_t)st.lslot * kUnitBytes);
  ++st.issued;
  st.lslot = (st.lslot + 1 == kRing) ? 0 : st.lslot + 1;
  if (++st.lu == st.lupi) {
    st.lu = 0;
    st.litem += kWaves;
    if (st.litem >= st.lnitems) loader_seek(P, st, st.ls + 1, b, wave);
  }
}

// Issue loads into free ring slots, at most `max` of them.
__device__ __forceinline__ void top_up(const Params& P, Stream& st, int b, int wave, int lane, int max) {
  while (max-- > 0 && !st.ldone && st.issued - st.consumed < kRing) loader_issue(P, st, b, wave, lane);
}

// Next unit of this wave's stream; the freed slot is refilled with the next
// unit of the stream, whatever its stage, so the ring stays full and the
// wait count is a constant (loads complete in issue order; once the stream
// has no units left the ring drains and the wait is for everything).
__device__ __forceinline__ uint4 consume_unit(const Params& P, Stream& st, int b, int wave, int lane) {
  const uint32_t a = st.ring + (uint32_t)st.cslot * kUnitBytes + (uint32_t)lane * 16u;
  const uint4 v = (st.issued - st.consumed == kRing) ? ring_read<kRing - 1>(a) : ring_read<0>(a);
  ++st.consumed;
  st.cslot = (st.cslot + 1 == kRing) ? 0 : st.cslot + 1;
  top_up(P, st, b, wave, lane, 1);
  return v;
}

// Next four units of this wave's stream: one vmcnt wait for the fourth, one
// LDS wait for all four reads, then four refills.
__device__ __forceinline__ void take4(const Params& P, Stream& st, int b, int wave, int lane, uint4 (&v)[4]) {
  if (st.issued - st.consumed == kRing)
    wait_vm<kRing - 4>();
  else
    wait_vm<0>();
  uint32_t a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int sl = st.cslot + k;
    sl = sl >= kRing ? sl - kRing : sl;
    a[k] = st.ring + (uint32_t)sl * kUnitBytes + (uint32_t)lane * 16u;
  }
  lds_read4(v, a);
  st.consumed += 4;
  st.cslot = st.cslot + 4 >= kRing ? st.cslot + 4 - kRing : st.cslot + 4;
  top_up(P, st, b, wave, lane, 4);
}

// Dot product of `n` consecutive units of the stream with act[col*512 ...]:
// batches of four, then single units.
__device__ __forceinline__ float dot_units(const Params& P, Stream& st, Ctx& c, const float* xa, int col, int n) {
  float a = 0.f;
  int j = 0;
  for (; j + 4 <= n; j += 4) {
    uint4 v[4];
    take4(P, st, c.b, c.wave, c.lane, v);
    const float* x = xa + addr::act_unit(col + j, 0);
    a += (dot8(v[0], x) + dot8(v[1], x + kUnitElems)) + (dot8(v[2], x + 2 * kUnitElems) + dot8(v[3], x + 3 * kUnitElems));
  }
  for (; j < n; ++j) a += dot8(consume_unit(P, st, c.b, c.wave, c.lane), xa + addr::act_unit(col + j, 0));
  return a;
}

// ---------------------------------------------------------------------------
// GEMV stages: prologue (stage activation), items, epilogue
// ---------------------------------------------------------------------------

// Residual input of layer l >= 1 (x after the previous layer).
__device__ __forceinline__ const tword* x_in(const Params& P, int l) {
  return P.x_ffn + addr::layer_off(l - 1, P.H);
}

template <int OP>
__device__ __forceinline__ bool gemv_prologue(const Params& P, Ctx& c, const Task& t, int s) {
  const int l = t.layer;
  c.rs = 1.f;
  if (OP == OP_QKV || OP == OP_LM) {
    const float* g = OP == OP_QKV ? P.g_attn + addr::layer_off(l, P.Hp) : P.g_final;
    // this position's cos/sin do not depend on the wait: load them first
    float rv = 0.f;
    if (OP == OP_QKV && c.tid < P.D) rv = P.rope[addr::rope_row(c.pos, P.D) + c.tid];
    if (!stage_normed(P, c, c.act, l == 0 ? nullptr : x_in(P, l), g, P.H, P.Hp, s)) return false;
    if (OP == OP_QKV) {
      if (c.tid < P.D) c.rope[c.tid] = rv;
      __syncthreads();
    }
  } else if (OP == OP_GU) {
    if (!stage_normed(P, c, c.act, P.x_attn + addr::layer_off(l, P.H), P.g_ffn + addr::layer_off(l, P.Hp), P.H, P.Hp, s))
      return false;
  } else {  // OPROJ, DOWN: plain activation + residual rows of this task
    const int n = OP == OP_OPROJ ? P.QD : P.F;
    const int np = OP == OP_OPROJ ? P.QDp : P.Fp;
    const tword* src = OP == OP_OPROJ ? P.o + addr::layer_off(l, P.QD) : P.h + addr::layer_off(l, P.F);
    const int r0 = 2 * (int)t.a0, nr = 2 * (int)(t.a1 - t.a0);
    // The residual rows were produced at least two stages earlier: read them
    // into registers before waiting for the activation (nr <= 512 rows).
    const tword* rs = OP == OP_OPROJ ? (l == 0 ? nullptr : x_in(P, l) + r0) : P.x_attn + addr::layer_off(l, P.H) + r0;
    tword rw = ready_word(c.epoch);
    if (c.tid < nr) {
      if (rs) {
        rw = ld_tag(rs + c.tid);
      } else {  // layer 0: the residual is the embedding row itself
        int tok = c.tok[0];
        tok = (tok < 0 || tok >= P.V) ? 0 : tok;
        rw |= (uint32_t)P.embed[addr::embed_row(tok, P.H) + r0 + c.tid] << 16;
      }
    }
    const Seg seg[1] = {{c.act, src, n, 1.f}};
    if (!stage_tagged(P, c, seg, s, c.act, n, np)) return false;
    if (c.tid < nr) {
      uint64_t t0 = 0;
      while (!tag_ready(rw, c.epoch)) {
        if (poll_stop(P, t0, s, tag_of(rw))) {
          c.flags[0] = 1;
          break;
        }
        rw = ld_tag(rs + c.tid);
      }
      c.res[c.tid] = tag_value(rw);
    }
    __syncthreads();
    if (c.flags[0]) return false;
  }
  return true;
}

struct LmBest {
  float v;
  int i;
};

// Outputs of row pair `pair` (rows 2*pair, 2*pair+1) with dot products v0, v1.
// w0 / w1: this thread writes the outputs that belong to row 0 / row 1.
template <int OP>
__device__ __forceinline__ void gemv_epilogue(const Params& P, Ctx& c, const Task& t, uint32_t pair, float v0, float v1,
                                              LmBest& best, bool w0, bool w1) {
  const int l = t.layer;
  const int r = 2 * (int)pair;
  const uint32_t tag = c.epoch;
  if (OP == OP_QKV || OP == OP_GU || OP == OP_LM) {
    v0 *= c.rs;
    v1 *= c.rs;
  }
  if (OP == OP_QKV) {
    if (r < P.QD + P.KVD) {  // q or k rows: rotate the pair (2i, 2i+1) of its head
      const int rr = r < P.QD ? r : r - P.QD;
      const int j = rr % P.D;
      const float cs = c.rope[j], sn = c.rope[j + 1];
      const float y0 = v0 * cs - v1 * sn;
      const float y1 = v0 * sn + v1 * cs;
      if (r < P.QD) {
        if (w0) st_tag(P.q + addr::layer_off(l, P.QD) + r, y0, tag);
        if (w1) st_tag(P.q + addr::layer_off(l, P.QD) + r + 1, y1, tag);
      } else {
        const uint16_t k0 = f32_to_bf16(y0), k1 = f32_to_bf16(y1);
        const int hk = rr / P.D;
        if (w0) {
          uint16_t* dst = P.kcache + addr::kv_slot(l, P.NKV, hk, P.S, c.pos, P.D) + j;
          st_kv(dst, (uint32_t)k0 | ((uint32_t)k1 << 16));
          st_tag(P.kvcur + addr::kvcur_off(l, P.KVD, 0) + rr, bf16_to_f32(k0), tag);
        }
        if (w1) st_tag(P.kvcur + addr::kvcur_off(l, P.KVD, 0) + rr + 1, bf16_to_f32(k1), tag);
      }
    } else {  // v rows
      const int rr = r - P.QD - P.KVD;
      const int hv = rr / P.D, j = rr % P.D;
      const uint16_t b0 = f32_to_bf16(v0), b1 = f32_to_bf16(v1);
      if (w0) {
        uint16_t* dst = P.vcache + addr::kv_slot(l, P.NKV, hv, P.S, c.pos, P.D) + j;
        st_kv(dst, (uint32_t)b0 | ((uint32_t)b1 << 16));
        st_tag(P.kvcur + addr::kvcur_off(l, P.KVD, 1) + rr, bf16_to_f32(b0), tag);
      }
      if (w1) st_tag(P.kvcur + addr::kvcur_off(l, P.KVD, 1) + rr + 1, bf16_to_f32(b1), tag);
    }
  } else if (OP == OP_OPROJ || OP == OP_DOWN) {
    tword* dst = (OP == OP_OPROJ ? P.x_attn : P.x_ffn) + addr::layer_off(l, P.H) + r;
    const int k = r - 2 * (int)t.a0;
    if (w0) st_tag(dst, c.res[k] + v0, tag);
    if (w1) st_tag(dst + 1, c.res[k + 1] + v1, tag);
  } else if (OP == OP_GU) {
    // pair = (gate row f, up row f): h_f = silu(gate) * up
    const float sg = v0 / (1.0f + __expf(-v0));
    if (w0) st_tag(P.h + addr::layer_off(l, P.F) + pair, sg * v1, tag);
  } else if (OP == OP_LM) {
    if (w0) {
      if ((((uintptr_t)(c.logits + r)) & 7u) == 0) {
        *reinterpret_cast<float2*>(c.logits + r) = make_float2(v0, v1);
      } else {
        c.logits[r] = v0;
        c.logits[r + 1] = v1;
      }
    }
    if (v0 > best.v) { best.v = v0; best.i = r; }
    if (v1 > best.v) { best.v = v1; best.i = r + 1; }
  }
}

// Argmax stage 2: every LM task publishes its key; the last to arrive picks the token.
__device__ __forceinline__ void lm_finish(const Params& P, Ctx& c, const Task& t, const LmBest& best) {
  if (c.lane == 0) c.red64[c.wave] = amax_key(best.v, best.i);
  // multi-step launches: every wave's stores of this step (the KV append
  // among them, read by the next step's attention on other CUs) complete
  // before this workgroup is counted and the next step's token is published
  if (P.tok_tag != nullptr) wait_all_vmem();
  __syncthreads();
  if (c.tid == 0) {
    uint64_t k = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) k = c.red64[w] > k ? c.red64[w] : k;
    __hip_atomic_store(&P.amax[c.b], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_all_vmem();
    const uint32_t old = __hip_atomic_fetch_add(P.amax_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    c.flags[1] = old == c.epoch * t.ntasks - 1u;
  }
  __syncthreads();
  if (c.flags[1] && c.wave == 0) {
    uint64_t k = 0;
    for (int w = c.lane; w < P.num_wgs; w += 64) {
      const uint64_t x = ld_u64_agent(P.amax + w);
      k = x > k ? x : k;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t y = __shfl_xor(k, o);
      k = y > k ? y : k;
    }
    if (c.lane == 0) {
      int idx = k ? (int)(~(uint32_t)k) : -1;
      if (ld_u32_agent(P.tokerr) == c.epoch) idx = -1;
      c.out_tok[0] = idx;
      if (P.tok_tag != nullptr)  // the next step's input token
        __hip_atomic_store(P.tok_tag, ((uint64_t)(c.epoch + 1u) << 32) | (uint32_t)idx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The down projection with partial-input start (region bit kRegionPartial):
// pairs cut into 8 items, the items of wave w all covering the same quarter
// of the row, so each wave stages and polls only that quarter of h and starts
// as soon as it is ready (the glossary entry "Megakernel", section "Wie eine
// ganze Rechenkette in ein Programm passt", and the article's paragraph on
// operations that begin on partial input); the residual rows are checked
// after the products, and the split-item sums are added in item order after
// the task's barrier, so results do not depend on arrival order.
__device__ __forceinline__ bool down_partial(const Params& P, Ctx& c, Stream& st, const Task& t, int s) {
  const int l = t.layer;
  const int nr = 2 * (int)(t.a1 - t.a0);
  const tword* rs = P.x_attn + addr::layer_off(l, P.H) + 2 * (int)t.a0;
  tword rw = c.tid < nr ? ld_tag(rs + c.tid) : ready_word(c.epoch);
  // the previous task's LDS readers (activation, partials, residual) are done
  __syncthreads();
  const uint32_t ks = 1u << t.kslog, hks = ks >> 1;
  const int upi = (int)(t.nu >> t.kslog);
  const uint32_t n_items = (t.a1 - t.a0) << t.kslog;
  const int col = (int)((uint32_t)c.wave & (hks - 1u)) * upi;  // the wave's first unit inside its row
  bool ok = true;
  if ((uint32_t)c.wave < n_items) {
    ok = wave_stage_cols(P, c, P.h + addr::layer_off(l, P.F), P.F, col * kUnitElems, upi, s);
    if (c.tr != nullptr && c.lane == 0) c.tr[4 + kWaves + c.wave] = wall_clock64();
    if (c.wave == 0) mark(c, 1);
    if (ok) {
      const float* xa = c.act + c.lane * 8;
      for (uint32_t i = (uint32_t)c.wave; i < n_items; i += kWaves) {
        const float a = wave_sum(dot_units(P, st, c, xa, col, upi));
        if (c.lane == 0) c.part[i] = a;
      }
    }
    mark_wave(c);
  }
  if (c.tid < nr) {
    uint64_t t0 = 0;
    while (!tag_ready(rw, c.epoch)) {
      if (poll_stop(P, t0, s, tag_of(rw))) {
        ok = false;
        break;
      }
      rw = ld_tag(rs + c.tid);
    }
    c.res[c.tid] = tag_value(rw);
  }
  if (!ok) c.flags[0] = 1;
  __syncthreads();
  if (c.flags[0]) return false;
  c.rs = 1.f;
  LmBest best{-__builtin_inff(), -1};
  for (uint32_t pl = (uint32_t)c.tid; pl < t.a1 - t.a0; pl += kThreads) {
    float v0 = 0.f, v1 = 0.f;
    for (uint32_t k = 0; k < hks; ++k) v0 += c.part[pl * ks + k];
    for (uint32_t k = hks; k < ks; ++k) v1 += c.part[pl * ks + k];
    gemv_epilogue<OP_DOWN>(P, c, t, t.a0 + pl, v0, v1, best, true, true);
  }
  mark(c, 2);
  return true;
}

template <int OP>
__device__ __forceinline__ bool gemv_task(const Params& P, Ctx& c, Stream& st, const Task& t, int s) {
  if (!gemv_prologue<OP>(P, c, t, s)) return false;
  mark(c, 1);
  LmBest best{-__builtin_inff(), -1};
  const float* xa = c.act + c.lane * 8;
  if (t.kslog == 0) {
    // whole pairs per wave; the wave finishes each pair
    const int half = (int)t.nu >> 1;  // units per row
    if (half == 4) {
      // rows of 2048: this lane's activation slice stays in registers for the task
      float4 xr[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xr[2 * j] = *reinterpret_cast<const float4*>(xa + addr::act_unit(j, 0));
        xr[2 * j + 1] = *reinterpret_cast<const float4*>(xa + addr::act_unit(j, 0) + 4);
      }
      bool first = false;
      for (uint32_t pair = t.a0 + (uint32_t)c.wave; pair < t.a1; pair += kWaves) {
        uint4 v[4];
        take4(P, st, c.b, c.wave, c.lane, v);
        mark_first(c, first);
        float a0 = (dot8r(v[0], xr[0], xr[1]) + dot8r(v[1], xr[2], xr[3])) +
                   (dot8r(v[2], xr[4], xr[5]) + dot8r(v[3], xr[6], xr[7]));
        take4(P, st, c.b, c.wave, c.lane, v);
        float a1 = (dot8r(v[0], xr[0], xr[1]) + dot8r(v[1], xr[2], xr[3])) +
                   (dot8r(v[2], xr[4], xr[5]) + dot8r(v[3], xr[6], xr[7]));
        a0 = wave_sum(a0);
        a1 = wave_sum(a1);
        gemv_epilogue<OP>(P, c, t, pair, a0, a1, best, c.lane == 0, c.lane == 1);
      }
    } else {
      for (uint32_t pair = t.a0 + (uint32_t)c.wave; pair < t.a1; pair += kWaves) {
        float a0 = dot_units(P, st, c, xa, 0, half);
        float a1 = dot_units(P, st, c, xa, 0, half);
        a0 = wave_sum(a0);
        a1 = wave_sum(a1);
        gemv_epilogue<OP>(P, c, t, pair, a0, a1, best, c.lane == 0, c.lane == 1);
      }
    }
    mark_wave(c);
  } else {
    // split items: row segments spread over all waves, partials added in LDS
    const uint32_t ks = 1u << t.kslog, hks = ks >> 1;
    const int upi = (int)(t.nu >> t.kslog);
    const uint32_t n_items = (t.a1 - t.a0) << t.kslog;
    for (uint32_t i = (uint32_t)c.wave; i < n_items; i += kWaves) {
      const int col = (int)(i & (hks - 1u)) * upi;  // first unit of the item inside its row
      if (i == (uint32_t)c.wave && c.tr != nullptr) {
        wait_vm<0>();
        bool f = false;
        mark_first(c, f);
      }
      float a = wave_sum(dot_units(P, st, c, xa, col, upi));
      if (c.lane == 0) c.part[i] = a;
    }
    mark_wave(c);
    __syncthreads();
    for (uint32_t pl = (uint32_t)c.tid; pl < t.a1 - t.a0; pl += kThreads) {
      float v0 = 0.f, v1 = 0.f;
      for (uint32_t k = 0; k < hks; ++k) v0 += c.part[pl * ks + k];
      for (uint32_t k = hks; k < ks; ++k) v1 += c.part[pl * ks + k];
      gemv_epilogue<OP>(P, c, t, t.a0 + pl, v0, v1, best, true, true);
    }
  }
  mark(c, 2);
  if (OP == OP_LM) lm_finish(P, c, t, best);
  return true;
}

// ---------------------------------------------------------------------------
// attention: one (kv head, chunk) per task, G query heads of D dims
// ---------------------------------------------------------------------------

// Layout: thread tid owns dims [8 * (tid % NT), +8) (one 16-byte slice of a
// K or V row, NT = D / 8 threads per row) of positions t0 + j * PPP + tid / NT
// for passes j < NPASS, PPP = 512 / NT positions per pass.  K and V of every
// owned position sit in registers (read before the task waits for this
// step's q, k and v: every slot below pos was written by an earlier step), q
// slices too, so scores and P.V need no LDS traffic.  A score is the sum of
// the NT slice dots (DPP within a row); each wave keeps its own softmax
// maximum and sum over its positions; the eight waves' {max, sum, P.V} are
// merged once, in wave order, after the only barrier.
template <int NT>
__device__ __forceinline__ float slice_sum(float a) {
  a += dpp<0xB1>(a);
  a += dpp<0x4E>(a);
  a += dpp<0x141>(a);
  if (NT == 16) a += dpp<0x140>(a);
  return a;
}

// Sum over the position groups of a wave (lanes with equal lane % NT):
// lane ^ 8 by DPP row rotation, lane ^ 16 and lane ^ 32 by the row and half
// swaps of gfx950 (v_permlane16_swap / v_permlane32_swap), all VALU.  Every
// lane ends with the same sum, formed in the same order.
template <int NT>
__device__ __forceinline__ float group_sum(float a) {
  if (NT == 8) a += dpp<0x128>(a);  // row_ror:8 == lane ^ 8 inside a row of 16
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  a = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// Merge of C chunk partials of one kv head, records of `stride` floats laid
// out {m[GQ], l[GQ], acc[GQ][D]}, for the GT heads [h0, h0 + GT): the global
// maximum first, then the rescaled sums, in chunk order.  Thread tid < GT * D
// owns output element tid.  The {m, l} table goes through LDS (2 * C * GT
// floats at tab); the accumulators are loaded KG chunks at a time into
// registers, all KG loads in flight together, and with EARLY the first KG
// issued before the table loads, so a merge costs ceil(C / KG) (EARLY) or 1 +
// ceil(C / KG) memory round trips instead of one per chunk (the batched path
// measured faster without EARLY).  Called by the whole workgroup (one barrier).
template <int GT, int D, int KG, bool EARLY>
__device__ __forceinline__ void merge_chunks(const Ctx& c, const float* base, int C, int stride, int GQ,
                                             int h0, float* tab, tword* o) {
  const bool mine = c.tid < GT * D;
  const int h = c.tid / D;
  float av[KG];
  // EARLY: the first KG chunks' accumulators are in flight with the table loads
  if (EARLY) {
#pragma unroll
    for (int u = 0; u < KG; ++u)
      av[u] = (mine && u < C) ? ld_f32_agent(base + (size_t)u * stride + 2 * GQ + h0 * D + c.tid) : 0.f;
  }
  for (int i = c.tid; i < C * GT; i += kThreads) {
    const int k = i / GT, hh = i - k * GT;
    const float* pk = base + (size_t)k * stride + h0 + hh;
    tab[2 * i] = ld_f32_agent(pk);
    tab[2 * i + 1] = ld_f32_agent(pk + GQ);
  }
  __syncthreads();
  if (!mine) return;
  float MM = -__builtin_inff();
  for (int k = 0; k < C; ++k) MM = fmaxf(MM, tab[2 * (k * GT + h)]);
  float LL = 0.f, AA = 0.f;
  for (int k0 = 0; k0 < C; k0 += KG) {
    if (!EARLY || k0 > 0) {
#pragma unroll
      for (int u = 0; u < KG; ++u)
        av[u] = k0 + u < C ? ld_f32_agent(base + (size_t)(k0 + u) * stride + 2 * GQ + h0 * D + c.tid) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const int k = k0 + u;
      if (k < C) {
        const float mk = tab[2 * (k * GT + h)];
        const float e = mk == -__builtin_inff() ? 0.f : __expf(mk - MM);
        LL = fmaf(e, tab[2 * (k * GT + h) + 1], LL);
        AA = fmaf(e, av[u], AA);
      }
    }
  }
  st_tag(o + c.tid, AA / LL, c.epoch);
}

template <int GT, int D>
__device__ __forceinline__ bool attn_task(const Params& P, Ctx& c, const Task& t, int s) {
  constexpr int NT = D / 8;                 // threads per K/V row
  constexpr int PPP = kThreads / NT;        // positions per pass
  constexpr int NPASS = kMaxChunk / PPP;    // passes over a full chunk
  const int l = t.layer, g = (int)t.a0, ch = (int)t.a1;
  const int C = P.attn_chunks;
  const int GQ = P.G;                      // query heads of the kv head
  const int slice = (int)t.kslog;          // this task's heads: [slice * GT, + GT)
  const int hq0 = slice * GT;
  const int n = c.pos + 1;
  const int len0 = (n + C - 1) / C;
  const int t0 = min(n, ch * len0), t1 = min(n, t0 + len0);

  const size_t head_off = addr::kv_head(l, P.NKV, g, P.S, D);
  const int ds = c.tid % NT;               // dim slice
  const int pg = c.tid / NT;               // position group
  // Branch-free prefetch: a position out of range, or pos itself, reads slot
  // 0 (in bounds) and is replaced or masked after the wait.
  uint4 kr[NPASS], vr[NPASS];
#pragma unroll
  for (int j = 0; j < NPASS; ++j) {
    const int tp = t0 + j * PPP + pg;
    const int tl = (tp < t1 && tp != c.pos) ? tp : 0;
    const size_t o = head_off + (size_t)tl * D + ds * 8;
    kr[j] = *reinterpret_cast<const uint4*>(P.kcache + o);
    vr[j] = *reinterpret_cast<const uint4*>(P.vcache + o);
  }

  const addr::AttnLds al = addr::attn_lds(GT, D);
  float* qs = c.act + al.qs;               // [GT][D], pre-scaled by 1/sqrt(D)
  float* kcur = c.act + al.kcur;           // [D]
  float* vcur = c.act + al.vcur;           // [D]
  float* wpart = c.act + al.wpart;         // [kWaves][GT][D]
  float* wm = c.act + al.wm;               // [kWaves][GT] per-wave max
  float* wl = c.act + al.wl;               // [kWaves][GT] per-wave sum
  {
    const Seg seg[3] = {{qs, P.q + addr::head_off(l, P.QD, g, GQ, hq0, D), GT * D, P.qscale},
                        {kcur, P.kvcur + addr::kvcur_off(l, P.KVD, 0) + (size_t)g * D, D, 1.f},
                        {vcur, P.kvcur + addr::kvcur_off(l, P.KVD, 1) + (size_t)g * D, D, 1.f}};
    if (!stage_tagged(P, c, seg, s)) return false;
  }
  mark(c, 1);

  // this step's row (bf16-exact values) goes back into the registers as bits
  {
    const float4 k0 = *reinterpret_cast<const float4*>(kcur + ds * 8);
    const float4 k1 = *reinterpret_cast<const float4*>(kcur + ds * 8 + 4);
    const float4 v0 = *reinterpret_cast<const float4*>(vcur + ds * 8);
    const float4 v1 = *reinterpret_cast<const float4*>(vcur + ds * 8 + 4);
    const uint4 kb = {pack_bf16x2(k0.x, k0.y), pack_bf16x2(k0.z, k0.w), pack_bf16x2(k1.x, k1.y), pack_bf16x2(k1.z, k1.w)};
    const uint4 vb = {pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w), pack_bf16x2(v1.x, v1.y), pack_bf16x2(v1.z, v1.w)};
#pragma unroll
    for (int j = 0; j < NPASS; ++j) {
      const bool here = t0 + j * PPP + pg == c.pos;
      kr[j].x = here ? kb.x : kr[j].x;
      kr[j].y = here ? kb.y : kr[j].y;
      kr[j].z = here ? kb.z : kr[j].z;
      kr[j].w = here ? kb.w : kr[j].w;
      vr[j].x = here ? vb.x : vr[j].x;
      vr[j].y = here ? vb.y : vr[j].y;
      vr[j].z = here ? vb.z : vr[j].z;
      vr[j].w = here ? vb.w : vr[j].w;
    }
  }

  float acc[GT][8];
  float wmax[GT], wsum[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const float4 qa = *reinterpret_cast<const float4*>(qs + h * D + ds * 8);
    const float4 qb = *reinterpret_cast<const float4*>(qs + h * D + ds * 8 + 4);
    float sc[NPASS];
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < NPASS; ++j) {
      const float a = slice_sum<NT>(dot8r(kr[j], qa, qb));
      sc[j] = t0 + j * PPP + pg < t1 ? a : -__builtin_inff();
      m = fmaxf(m, sc[j]);
    }
    m = wave_max(m);
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int j = 0; j < NPASS; ++j) {
      const float p = sc[j] == -__builtin_inff() ? 0.f : __expf(sc[j] - m);
      ls += p;
      const uint4 w = vr[j];
      acc[h][0] = fmaf(p, bf_lo(w.x), acc[h][0]);
      acc[h][1] = fmaf(p, bf_hi(w.x), acc[h][1]);
      acc[h][2] = fmaf(p, bf_lo(w.y), acc[h][2]);
      acc[h][3] = fmaf(p, bf_hi(w.y), acc[h][3]);
      acc[h][4] = fmaf(p, bf_lo(w.z), acc[h][4]);
      acc[h][5] = fmaf(p, bf_hi(w.z), acc[h][5]);
      acc[h][6] = fmaf(p, bf_lo(w.w), acc[h][6]);
      acc[h][7] = fmaf(p, bf_hi(w.w), acc[h][7]);
    }
    // every lane of a position group holds the same p: count one slice per group
    wsum[h] = wave_sum(ds == 0 ? ls : 0.f);
    wmax[h] = m;
  }
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = group_sum<NT>(acc[h][e]);
  if (c.lane < NT) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float* dst = wpart + (c.wave * GT + h) * D + ds * 8;
      *reinterpret_cast<float4*>(dst) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  if (c.lane == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      wm[c.wave * GT + h] = wmax[h];
      wl[c.wave * GT + h] = wsum[h];
    }
  }
  mark_wave(c);
  __syncthreads();
  mark(c, 2);

  // merge the waves in order: max, then rescaled sums
  const int h = c.tid / D, d = c.tid % D;
  float A = 0.f, Ls = 0.f, M = -__builtin_inff();
  if (c.tid < GT * D) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * GT + h]);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = wm[w * GT + h];
      const float e = mw == -__builtin_inff() ? 0.f : __expf(mw - M);
      A = fmaf(e, wpart[(w * GT + h) * D + d], A);
      Ls = fmaf(e, wl[w * GT + h], Ls);
    }
  }
  tword* o = P.o + addr::head_off(l, P.QD, g, GQ, hq0, D);
  if (C == 1) {
    if (c.tid < GT * D) st_tag(o + c.tid, A / Ls, c.epoch);
    return true;
  }
  // publish this chunk's partial of the task's heads into the kv head's
  // record {m[GQ], l[GQ], acc[GQ][D]}; the last chunk of (kv head, slice) merges
  const int stride = GQ * (D + 2);
  const int hg = hq0 + h;                  // head inside the kv head's group
  float* mine = P.attn_part + addr::attn_rec(l, P.NKV, g, C, ch, stride);
  if (c.tid < GT * D) st_f32_agent(mine + 2 * GQ + hq0 * D + c.tid, A);
  if (c.tid < GT * D && d == 0) {
    st_f32_agent(mine + hg, M);
    st_f32_agent(mine + GQ + hg, Ls);
  }
  wait_all_vmem();
  __syncthreads();
  if (c.tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(P.attn_ctr + addr::attn_ctr(l, P.NKV, g, GQ, slice), 1u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    c.flags[1] = old == c.epoch * (uint32_t)C - 1u;
  }
  __syncthreads();
  // the {m, l} table reuses wpart (free after the barrier above):
  // 2 * C * GT <= kWaves * GT * D because C <= 256 <= 4 * D
  if (c.flags[1])
    merge_chunks<GT, D, 32, true>(c, P.attn_part + addr::attn_rec(l, P.NKV, g, C, 0, stride), C, stride, GQ, hq0, wpart, o);
  return true;
}

// ---------------------------------------------------------------------------
// batched decode (2..8 sequences): tiled weights, bf16 MFMA with the batch
// as the N operand
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Sequence n's slice of a [B][L][len] activation buffer.
__device__ __forceinline__ size_t seq_off(const Params& P, int n, int l, int len) {
  return ((size_t)n * P.L + l) * (size_t)len;
}

// Loader of a batched stream: items wave, wave + 8, ... of (a1 - a0) << kslog
// (block a0 + (i >> kslog), part i & (2^kslog - 1)); per chunk of ch tiles a
// part covers tiles [part * upc, + upc) of the chunk, upc = ch >> kslog.
// Order: chunk, then the wave's items, then tiles.
__device__ __forceinline__ void loader_seek_b(const Params& P, Stream& st, int s, int wave) {
  for (; s < st.s_end; ++s) {
    const Task t = stream_task(st, s);
    if (op_is_gemv(t.op)) {
      const uint32_t n_items = (t.a1 - t.a0) << t.kslog;
      if ((uint32_t)wave < n_items) {
        const uint32_t ch = (uint32_t)gemm_chunk_tiles((int)t.nu, (t.region & kRegionSplit) != 0);
        st.ls = s;
        st.litem = (uint32_t)wave;
        st.lnitems = n_items;
        st.lkslog = t.kslog;
        st.lupi = ch >> t.kslog;  // tiles per part and chunk
        st.lu = 0;
        st.la0 = t.a0;
        st.lnu = t.nu;            // tiles per row
        // chunks [lc, lnc): all of them, or this task's half of a split block
        const uint32_t nc = t.nu / ch;
        st.lc = (t.region & kRegionHalf1) ? nc / 2 : 0;
        st.lnc = (t.region & kRegionSplit) ? st.lc + nc / 2 : nc;
        st.lch = ch;
        st.lbase = ((t.region & kRegionLm) ? P.lm : P.arena) + t.wofs;
        return;
      }
    }
  }
  st.ls = st.s_end;
  st.ldone = true;
}

__device__ __forceinline__ void loader_issue_b(const Params& P, Stream& st, int wave, int lane) {
  if (st.ldone) return;
  const uint32_t block = st.la0 + (st.litem >> st.lkslog);
  const uint32_t part = st.litem & ((1u << st.lkslog) - 1u);
  const uint32_t kb = st.lc * st.lch + part * st.lupi + st.lu;
  const char* g = st.lbase + ((uint64_t)block * st.lnu + kb) * kUnitBytes + (uint32_t)lane * 16u;
  dma_unit(g, st.ring + (uint32_t)st.lslot * kUnitBytes);
  ++st.issued;
  st.lslot = (st.lslot + 1 == kRingBatched) ? 0 : st.lslot + 1;
  if (++st.lu == st.lupi) {
    st.lu = 0;
    st.litem += kWaves;
    if (st.litem >= st.lnitems) {
      st.litem = (uint32_t)wave;
      if (++st.lc >= st.lnc) loader_seek_b(P, st, st.ls + 1, wave);
    }
  }
}

__device__ __forceinline__ void top_up_b(const Params& P, Stream& st, int wave, int lane, int max) {
  while (max-- > 0 && !st.ldone && st.issued - st.consumed < kRingBatched) loader_issue_b(P, st, wave, lane);
}

// Next four tiles of the stream (all issued: the ring is refilled on consume).
__device__ __forceinline__ void take4_b(const Params& P, Stream& st, int wave, int lane, uint4 (&v)[4]) {
  if (st.issued - st.consumed == kRingBatched)
    wait_vm<kRingBatched - 4>();
  else
    wait_vm<0>();
  uint32_t a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int sl = st.cslot + k;
    sl = sl >= kRingBatched ? sl - kRingBatched : sl;
    a[k] = st.ring + (uint32_t)sl * kUnitBytes + (uint32_t)lane * 16u;
  }
  lds_read4(v, a);
  st.consumed += 4;
  st.cslot = st.cslot + 4 >= kRingBatched ? st.cslot + 4 - kRingBatched : st.cslot + 4;
  top_up_b(P, st, wave, lane, 4);
}

__device__ __forceinline__ uint4 take1_b(const Params& P, Stream& st, int wave, int lane) {
  const uint32_t a = st.ring + (uint32_t)st.cslot * kUnitBytes + (uint32_t)lane * 16u;
  const uint4 v = (st.issued - st.consumed == kRingBatched) ? ring_read<kRingBatched - 1>(a) : ring_read<0>(a);
  ++st.consumed;
  st.cslot = (st.cslot + 1 == kRingBatched) ? 0 : st.cslot + 1;
  top_up_b(P, st, wave, lane, 1);
  return v;
}

// First round of stage_batch's loads (groups i = 4 (j * 512 + tid) of the B
// sequences' columns [k0, k0 + kc)), issued ahead of the staging itself.
__device__ __forceinline__ void stage_batch_issue(const Params& P, const Ctx& c, const tword* base, size_t sstride,
                                                  int k0, int kc, tword4 (&w)[kStageLoadsBatch]) {
  const int total = P.B * kc;
  // every group read lies in [base, base + (B - 1) sstride + k0 + kc)
  const TagBuf tb = tag_buf(base, (uint32_t)(((size_t)(P.B - 1) * sstride + k0 + kc) * 4));
#pragma unroll
  for (int j = 0; j < kStageLoadsBatch; ++j) {
    const int i = 4 * (j * kThreads + c.tid);
    const int n = i < total ? i / kc : 0, k = i - n * kc;
    w[j] = i < total ? ld_tag4_agent(tb, (uint32_t)((size_t)n * sstride + k0 + k)) : ready_word4(c.epoch);
  }
}

// Stage columns [k0, k0 + kc) of B tagged sequences into LDS:
// dst[n * stride + k] = src_n[k0 + k], src_n = base + n * sstride.  The first
// round's loads are in flight before the barrier that separates these LDS
// writes from the previous task's reads; `pre`, if given, holds that round's
// words already loaded by stage_batch_issue.  Ends with a barrier.
__device__ __forceinline__ bool stage_batch(const Params& P, Ctx& c, float* dst, int stride, const tword* base,
                                            size_t sstride, int k0, int kc, int kpad, int stage,
                                            const tword4 (*pre)[kStageLoadsBatch] = nullptr) {
  // groups of 4 columns (kc, k0, sstride and stride are multiples of 4)
  const int total = P.B * kc;
  // every group read below lies in [base, base + (B - 1) sstride + k0 + kc)
  const TagBuf tb = tag_buf(base, (uint32_t)(((size_t)(P.B - 1) * sstride + k0 + kc) * 4));
  bool stop = false;
  for (int i0 = 0; i0 == 0 || i0 < total; i0 += 4 * kThreads * kStageLoadsBatch) {
    tword4 w[kStageLoadsBatch];
    if (pre != nullptr && i0 == 0) {
#pragma unroll
      for (int j = 0; j < kStageLoadsBatch; ++j) w[j] = (*pre)[j];
    } else {
#pragma unroll
      for (int j = 0; j < kStageLoadsBatch; ++j) {
        const int i = i0 + 4 * (j * kThreads + c.tid);
        const int n = i < total ? i / kc : 0, k = i - n * kc;
        w[j] = i < total ? ld_tag4_agent(tb, (uint32_t)((size_t)n * sstride + k0 + k)) : ready_word4(c.epoch);
      }
    }
    uint64_t t0 = 0;
    while (!stop) {
      bool ready = true;
#pragma unroll
      for (int j = 0; j < kStageLoadsBatch; ++j) ready &= tag4_ready(w[j], c.epoch);
      if (ready) break;
      if (poll_stop(P, t0, stage, tag_of(w[0].x))) {
        stop = true;
        break;
      }
#pragma unroll
      for (int j = 0; j < kStageLoadsBatch; ++j) {
        const int i = i0 + 4 * (j * kThreads + c.tid);
        if (i < total && !tag4_ready(w[j], c.epoch)) {
          const int n = i / kc, k = i - n * kc;
          w[j] = ld_tag4_agent(tb, (uint32_t)((size_t)n * sstride + k0 + k));
        }
      }
    }
    if (i0 == 0) {
      __syncthreads();
      // zero the padding columns [kc, kpad) of every sequence
      const int padw = kpad - kc;
      for (int i = c.tid; i < P.B * padw; i += kThreads) dst[(i / padw) * stride + kc + i % padw] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kStageLoadsBatch; ++j) {
      const int i = i0 + 4 * (j * kThreads + c.tid);
      if (i < total) {
        const int n = i / kc, k = i - n * kc;
        *reinterpret_cast<float4*>(dst + n * stride + k) = tag_value4(w[j]);
      }
    }
  }
  if (stop) c.flags[0] = 1;
  __syncthreads();
  return c.flags[0] == 0;
}

// Input token of sequence n (a bad id latches MK_E_TOKEN, marks the sequence
// and reads row 0 instead).
__device__ __forceinline__ int token_of(const Params& P, const Ctx& c, int n, int stage, bool report) {
  int tok = c.tok[n];
  if (tok < 0 || tok >= P.V) {
    if (report) {
      latch_error(P, MK_E_TOKEN, stage, (uint32_t)tok);
      __hip_atomic_store(&P.tokerr[n], c.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    tok = 0;
  }
  return tok;
}

// RMSNorm of the staged batch: wave n < B computes rs[n] = (mean(x^2) +
// eps)^(-1/2) over x = dst[n][0, H) and scales dst[n][k] by the gain gl[k]
// (zeroing [H, Hp)), so that W . rmsnorm(x_n) = rs[n] * (W . dst_n).  The
// gains gl[0, H) are already in LDS (staged with the activation).
__device__ __forceinline__ void norm_batch(const Params& P, Ctx& c, float* dst, int stride, const float* gl,
                                           float* rsb) {
  // lane: 4 consecutive columns per step of 256 (H and Hp are multiples of 4)
  if (c.wave < P.B) {
    float* x = dst + c.wave * stride;
    float ss = 0.f;
    for (int k = c.lane * 4; k < P.H; k += 256) {
      const float4 v = *reinterpret_cast<const float4*>(x + k);
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    }
    ss = wave_sum(ss);
    if (c.lane == 0) rsb[c.wave] = rsqrtf(ss / (float)P.H + P.eps);
    for (int k = c.lane * 4; k < P.Hp; k += 256) {
      // padding columns [H, Hp) become zero whatever they held
      float4 v = *reinterpret_cast<float4*>(x + k);
      if (k < P.H) {
        const float4 gv = *reinterpret_cast<const float4*>(gl + k);
        v = make_float4(v.x * gv.x, v.y * gv.y, v.z * gv.z, v.w * gv.w);
      } else {
        v = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      *reinterpret_cast<float4*>(x + k) = v;
    }
  }
  __syncthreads();
}

// B operand of one tile: lane l holds sequence l % 16, columns 8 * (l / 16)
// .. +8 of the tile, as bf16 hi and lo parts (x = hi + lo to about 16
// significant bits), so two MFMAs give an fp32-accurate product with the bf16
// weights.  Lanes past the batch read sequence 0: column n of an MFMA result
// depends on column n of B alone, and the columns past the batch are never
// used.  Pairs are rounded together (one packed conversion for two hi parts,
// one for two lo parts).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void hilo_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
  __builtin_memcpy(&hi, &h, sizeof(hi));
  const float r0 = x0 - __uint_as_float(hi << 16);
  const float r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
  const bf16x2 l = __builtin_convertvector(f32x2{r0, r1}, bf16x2);
  __builtin_memcpy(&lo, &l, sizeof(lo));
}
__device__ __forceinline__ void b_operand(const float* act, int stride, int n, bool live, int col,
                                          bf16x8& hi, bf16x8& lo) {
  const float* x = act + (live ? n : 0) * stride + col;
  const float4 a = *reinterpret_cast<const float4*>(x);
  const float4 b = *reinterpret_cast<const float4*>(x + 4);
  uint4 h, l;
  hilo_pair(a.x, a.y, h.x, l.x);
  hilo_pair(a.z, a.w, h.y, l.y);
  hilo_pair(b.x, b.y, h.z, l.z);
  hilo_pair(b.z, b.w, h.w, l.w);
  __builtin_memcpy(&hi, &h, sizeof(hi));
  __builtin_memcpy(&lo, &l, sizeof(lo));
}

__device__ __forceinline__ f32x4 mfma_tile(const uint4 w, const bf16x8& hi, const bf16x8& lo, f32x4 acc) {
  bf16x8 a;
  __builtin_memcpy(&a, &w, sizeof(a));
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc, 0, 0, 0);
  return acc;
}

struct LmBestB {
  float v;
  int i;
};

// Outputs of a row pair (rows r, r+1 of the stage's matrix) of sequence n:
// QKV (RoPE pair / v values) and GU (gate, up) pairs.
template <int OP>
__device__ __forceinline__ void epi_pair_b(const Params& P, const Ctx& c, int l, int r, int n, float v0, float v1,
                                           const float* rsb) {
  const uint32_t tag = c.epoch;
  v0 *= rsb[n];
  v1 *= rsb[n];
  if (OP == OP_QKV) {
    if (r < P.QD + P.KVD) {
      const int rr = r < P.QD ? r : r - P.QD;
      const int j = rr % P.D;
      const float* rp = c.rope + (P.prefill ? n * P.D : 0);  // prefill: token n sits at position pos + n
      const float cs = rp[j], sn = rp[j + 1];
      const float y0 = v0 * cs - v1 * sn;
      const float y1 = v0 * sn + v1 * cs;
      if (r < P.QD) {
        tword* q = P.q + seq_off(P, n, l, P.QD) + r;
        st_tag(q, y0, tag);
        st_tag(q + 1, y1, tag);
      } else {
        const uint16_t k0 = f32_to_bf16(y0), k1 = f32_to_bf16(y1);
        const int hk = rr / P.D;
        // prefill: one cache, token n's slot pos + n
        uint16_t* dst = P.kcache + ((seq_off(P, P.prefill ? 0 : n, l, P.NKV) + hk) * P.S + c.pos + (P.prefill ? n : 0)) *
                                       P.D + j;
        st_kv(dst, (uint32_t)k0 | ((uint32_t)k1 << 16));
        tword* kv = P.kvcur + seq_off(P, n, l, 2 * P.KVD) + rr;
        st_tag(kv, bf16_to_f32(k0), tag);
        st_tag(kv + 1, bf16_to_f32(k1), tag);
      }
    } else {
      const int rr = r - P.QD - P.KVD;
      const int hv = rr / P.D, j = rr % P.D;
      const uint16_t b0 = f32_to_bf16(v0), b1 = f32_to_bf16(v1);
      uint16_t* dst = P.vcache + ((seq_off(P, P.prefill ? 0 : n, l, P.NKV) + hv) * P.S + c.pos + (P.prefill ? n : 0)) *
                                     P.D + j;
      st_kv(dst, (uint32_t)b0 | ((uint32_t)b1 << 16));
      tword* kv = P.kvcur + seq_off(P, n, l, 2 * P.KVD) + P.KVD + rr;
      st_tag(kv, bf16_to_f32(b0), tag);
      st_tag(kv + 1, bf16_to_f32(b1), tag);
    }
  } else {  // GU: rows (2f, 2f + 1) = (gate f, up f)
    const float sg = v0 / (1.0f + __expf(-v0));
    st_tag(P.h + seq_off(P, n, l, P.F) + (r >> 1), sg * v1, tag);
  }
}

// Output of one row r of sequence n: OPROJ / DOWN (residual add) and LM.
template <int OP>
__device__ __forceinline__ void epi_row_b(const Params& P, const Ctx& c, const Task& t, int l, int r, int n, float v,
                                          const float* rsb, LmBestB& best) {
  if (OP == OP_LM) {
    v *= rsb[n];
    c.logits[(size_t)n * P.V + r] = v;
    if (v > best.v) {
      best.v = v;
      best.i = r;
    }
  } else {
    const int nr = (int)(t.a1 - t.a0) * kTileRows;
    const int k = r - (int)t.a0 * kTileRows;
    tword* dst = (OP == OP_OPROJ ? P.x_attn : P.x_ffn) + seq_off(P, n, l, P.H) + r;
    st_tag(dst, c.res[n * nr + k] + v, c.epoch);
  }
}

// Argmax stage 2 for the batch: every LM task publishes one key per sequence;
// the last task to arrive picks each sequence's token.
__device__ __forceinline__ void lm_finish_b(const Params& P, Ctx& c, const Task& t) {
  uint64_t* keys = reinterpret_cast<uint64_t*>(c.part);  // [kWaves][16] per-wave keys, then [16] per sequence
  if (c.tid < P.B) {
    uint64_t k = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) k = keys[w * 16 + c.tid] > k ? keys[w * 16 + c.tid] : k;
    __hip_atomic_store(&P.amax[(size_t)c.tid * P.num_wgs + c.b], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_all_vmem();
  __syncthreads();
  if (c.tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(P.amax_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    c.flags[1] = old == c.epoch * t.ntasks - 1u;
  }
  __syncthreads();
  if (c.flags[1] && c.wave < P.B) {
    const int n = c.wave;
    uint64_t k = 0;
    for (int w = c.lane; w < P.num_wgs; w += 64) {
      const uint64_t x = ld_u64_agent(P.amax + (size_t)n * P.num_wgs + w);
      k = x > k ? x : k;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t y = __shfl_xor(k, o);
      k = y > k ? y : k;
    }
    if (c.lane == 0) {
      int idx = k ? (int)(~(uint32_t)k) : -1;
      if (ld_u32_agent(P.tokerr + n) == c.epoch) idx = -1;
      c.out_tok[n] = idx;
      if (P.tok_tag != nullptr)  // the next step's input token
        __hip_atomic_store(P.tok_tag + n, ((uint64_t)(c.epoch + 1u) << 32) | (uint32_t)idx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int OP>
__device__ __forceinline__ bool gemm_task(const Params& P, Ctx& c, Stream& st, const Task& t, int s) {
  const int l = t.layer;
  const int stride = P.act_stride;
  float* rsb = c.red + 16;  // [kMaxBatch] RMSNorm scales of the sequences
  // chunks [cb, ce) of every row: all, or one half of a block split over two workgroups
  const bool split = (t.region & kRegionSplit) != 0, half1 = (t.region & kRegionHalf1) != 0;
  const int kt = (int)t.nu, ch = gemm_chunk_tiles(kt, split), nc = kt / ch;
  const int cb = half1 ? nc / 2 : 0, ce = split ? cb + nc / 2 : nc;
  const int ks = 1 << t.kslog, upc = ch >> t.kslog;
  const int nitems = (int)(t.a1 - t.a0) << t.kslog;
  const int nblk = (int)(t.a1 - t.a0);

  // ---- prologue: first chunk of the activation, norms, residual rows, RoPE
  if (OP == OP_QKV || OP == OP_GU || OP == OP_LM) {
    // cos/sin of this step's position, or (prefill) of each token's position,
    // and the norm gains (H <= 2048: four per thread): loaded before the
    // activation's first poll round, so that they arrive with it rather than
    // behind the weight loads the waves issue meanwhile
    const int nrope = P.prefill ? P.B * P.D : P.D;
    float rv = 0.f;
    if (OP == OP_QKV && c.tid < nrope) rv = P.rope[addr::rope_row(c.pos + c.tid / P.D, P.D) + c.tid % P.D];
    const float* g = OP == OP_QKV ? P.g_attn + (size_t)l * P.Hp : OP == OP_GU ? P.g_ffn + (size_t)l * P.Hp : P.g_final;
    const float4 gv = 4 * c.tid < P.H ? *reinterpret_cast<const float4*>(g + 4 * c.tid) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (OP == OP_QKV && l == 0) {
      // embedding rows of the batch's tokens
      __syncthreads();
      for (int i = c.tid; i < P.B * P.H; i += kThreads) {
        const int n = i / P.H, k = i - n * P.H;
        const int tok = token_of(P, c, n, s, k == 0);
        c.act[n * stride + k] = bf16_to_f32(P.embed[(size_t)tok * P.H + k]);
      }
      __syncthreads();
    } else {
      const tword* src = OP == OP_GU ? P.x_attn + (size_t)l * P.H
                                        : P.x_ffn + (size_t)(OP == OP_LM ? P.L - 1 : l - 1) * P.H;
      if (!stage_batch(P, c, c.act, stride, src, (size_t)P.L * P.H, 0, P.H, P.H, s)) return false;
    }
    // the gains into the split-part area (free until this task's MFMA loop
    // ends; the staging above ended with a barrier)
    if (4 * c.tid < P.H) *reinterpret_cast<float4*>(c.part + 4 * c.tid) = gv;
    if (OP == OP_QKV && c.tid < nrope) c.rope[c.tid] = rv;
    __syncthreads();
    norm_batch(P, c, c.act, stride, c.part, rsb);
  } else {
    // residual rows [r0, r0 + nr) of every sequence, then the activation
    const int r0 = (int)t.a0 * kTileRows, nr = nblk * kTileRows;
    __syncthreads();
    for (int i = c.tid; i < P.B * nr; i += kThreads) {
      const int n = i / nr, k = i - n * nr;
      float v;
      if (OP == OP_OPROJ && l == 0) {
        const int tok = token_of(P, c, n, s, false);
        v = bf16_to_f32(P.embed[(size_t)tok * P.H + r0 + k]);
      } else {
        const tword* rsrc = (OP == OP_OPROJ ? P.x_ffn + seq_off(P, n, l - 1, P.H) : P.x_attn + seq_off(P, n, l, P.H)) + r0 + k;
        tword rw = ld_tag(rsrc);
        uint64_t t0 = 0;
        while (!tag_ready(rw, c.epoch)) {
          if (poll_stop(P, t0, s, tag_of(rw))) {
            c.flags[0] = 1;
            break;
          }
          rw = ld_tag(rsrc);
        }
        v = tag_value(rw);
      }
      c.res[i] = v;
    }
    const tword* src = OP == OP_OPROJ ? P.o + addr::layer_off(l, P.QD) : P.h + addr::layer_off(l, P.F);
    const int kfull = OP == OP_OPROJ ? P.QD : P.F;
    const int col0 = cb * ch * kTileCols;
    const int kc0 = max(0, min(ch * kTileCols, kfull - col0));  // 0: the half lies in the zero padding
    if (!stage_batch(P, c, c.act, stride, src, (size_t)P.L * kfull, col0, kc0, ch * kTileCols, s)) return false;
    if (c.flags[0]) return false;
    if (c.tid < P.B) rsb[c.tid] = 1.f;
    __syncthreads();
  }
  mark(c, 1);

  // ---- main loop: MFMA over the wave's tiles, chunk by chunk
  const int n_col = c.lane & 15;
  const bool live = n_col < P.B;
  const int kq = (c.lane >> 4) * 8;
  LmBestB best{-__builtin_inff(), -1};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // a later chunk's first round of loads is issued before the MFMA loop of
  // the chunk before it, so its round trip overlaps that chunk's compute
  tword4 wn[kStageLoadsBatch];
  for (int cc = cb; cc < ce; ++cc) {
    if constexpr (OP == OP_OPROJ || OP == OP_DOWN) {  // the others have one chunk (H <= 2048)
      const tword* src = OP == OP_OPROJ ? P.o + addr::layer_off(l, P.QD) : P.h + addr::layer_off(l, P.F);
      const int kfull = OP == OP_OPROJ ? P.QD : P.F;
      if (cc > cb) {  // next chunk of the activation (one item per wave: acc carries over)
        const int kcc = max(0, min(ch * kTileCols, kfull - cc * ch * kTileCols));
        if (!stage_batch(P, c, c.act, stride, src, (size_t)P.L * kfull, cc * ch * kTileCols, kcc, ch * kTileCols, s,
                         &wn))
          return false;
      }
      if (cc + 1 < ce) {
        const int kcn = max(0, min(ch * kTileCols, kfull - (cc + 1) * ch * kTileCols));
        stage_batch_issue(P, c, src, (size_t)P.L * kfull, (cc + 1) * ch * kTileCols, kcn, wn);
      }
    }
    for (int i = c.wave; i < nitems; i += kWaves) {
      if (nc == 1) acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const int col0 = (i & (ks - 1)) * upc * kTileCols;  // first column of the part inside the chunk
      int u = 0;
      for (; u + 4 <= upc; u += 4) {
        uint4 v[4];
        take4_b(P, st, c.wave, c.lane, v);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          bf16x8 hi, lo;
          b_operand(c.act, stride, n_col, live, col0 + (u + k) * kTileCols + kq, hi, lo);
          acc = mfma_tile(v[k], hi, lo, acc);
        }
      }
      for (; u < upc; ++u) {
        const uint4 w = take1_b(P, st, c.wave, c.lane);
        bf16x8 hi, lo;
        b_operand(c.act, stride, n_col, live, col0 + u * kTileCols + kq, hi, lo);
        acc = mfma_tile(w, hi, lo, acc);
      }
      if (cc != ce - 1) continue;
      const int blk = (int)t.a0 + (i >> t.kslog);
      if (ks == 1) {
        // lane: rows 4 * (lane / 16) + 0..3 of the block, sequence lane % 16
        const int r = blk * kTileRows + (c.lane >> 4) * 4;
        if (OP == OP_QKV || OP == OP_GU) {
          if (live) {
            epi_pair_b<OP>(P, c, l, r, n_col, acc[0], acc[1], rsb);
            epi_pair_b<OP>(P, c, l, r + 2, n_col, acc[2], acc[3], rsb);
          }
        } else if (OP == OP_LM) {
          // the lane's four consecutive logits of its sequence in one store
          if (live) {
            const float sc = rsb[n_col];
            const float4 v = make_float4(acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc);
            float* dst = c.logits + (size_t)n_col * P.V + r;
            if ((((uintptr_t)dst) & 15u) == 0) {
              *reinterpret_cast<float4*>(dst) = v;
            } else {
              dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
            }
            if (v.x > best.v) { best.v = v.x; best.i = r; }
            if (v.y > best.v) { best.v = v.y; best.i = r + 1; }
            if (v.z > best.v) { best.v = v.z; best.i = r + 2; }
            if (v.w > best.v) { best.v = v.w; best.i = r + 3; }
          }
        } else {
          if (live) {
#pragma unroll
            for (int q = 0; q < 4; ++q) epi_row_b<OP>(P, c, t, l, r + q, n_col, acc[q], rsb, best);
          }
        }
      } else {
        float* tile = c.part + (size_t)i * (kTileRows * kTileLd);  // [row][sequence column]
#pragma unroll
        for (int q = 0; q < 4; ++q) tile[((c.lane >> 4) * 4 + q) * kTileLd + n_col] = acc[q];
      }
    }
  }
  mark_wave(c);
  if (ks > 1) {
    // sum the parts of every block in part order, then the outputs
    __syncthreads();
    const int rows_per = (OP == OP_QKV || OP == OP_GU) ? kTileRows / 2 : kTileRows;
    const int combos = nblk * rows_per * P.B;
    // sequence-major: consecutive threads store consecutive rows of one
    // sequence's output, whole cache lines per wave (row-major order, eight
    // 32-byte pieces per store, measured 9-12 us slower per 8-sequence step)
    for (int e = c.tid; e < combos; e += kThreads) {
      const int n = e / (nblk * rows_per), rest = e % (nblk * rows_per);
      const int j = rest / rows_per, q = rest % rows_per;
      if (OP == OP_QKV || OP == OP_GU) {
        float v0 = 0.f, v1 = 0.f;
        for (int pp = 0; pp < ks; ++pp) {
          const float* tile = c.part + (size_t)(j * ks + pp) * (kTileRows * kTileLd);
          v0 += tile[(2 * q) * kTileLd + n];
          v1 += tile[(2 * q + 1) * kTileLd + n];
        }
        epi_pair_b<OP>(P, c, l, ((int)t.a0 + j) * kTileRows + 2 * q, n, v0, v1, rsb);
      } else {
        float v = 0.f;
        for (int pp = 0; pp < ks; ++pp) v += c.part[(size_t)(j * ks + pp) * (kTileRows * kTileLd) + q * kTileLd + n];
        if (OP == OP_LM) {
          // reduced values back into the first part's tile for the argmax scan
          c.part[(size_t)(j * ks) * (kTileRows * kTileLd) + q * kTileLd + n] = v * rsb[n];
          c.logits[(size_t)n * P.V + ((int)t.a0 + j) * kTileRows + q] = v * rsb[n];
        } else if (split) {
          // the second half hands its sums over; the first half adds them to its own
          tword* kp = P.kpart + seq_off(P, n, l, 2 * P.H) + (OP == OP_DOWN ? P.H : 0) + ((int)t.a0 + j) * kTileRows + q;
          if (half1) {
            st_tag(kp, v, c.epoch);
            continue;
          }
          tword w = ld_tag(kp);
          uint64_t t0 = 0;
          while (!tag_ready(w, c.epoch)) {
            if (poll_stop(P, t0, s, tag_of(w))) {
              c.flags[0] = 1;
              break;
            }
            w = ld_tag(kp);
          }
          epi_row_b<OP>(P, c, t, l, ((int)t.a0 + j) * kTileRows + q, n, v + tag_value(w), rsb, best);
        } else {
          epi_row_b<OP>(P, c, t, l, ((int)t.a0 + j) * kTileRows + q, n, v, rsb, best);
        }
      }
    }
    if ((OP == OP_OPROJ || OP == OP_DOWN) && split) {  // a watchdog stop while waiting for the second half
      __syncthreads();
      if (c.flags[0]) return false;
    }
  }
  mark(c, 2);
  if (OP == OP_LM) {
    uint64_t* keys = reinterpret_cast<uint64_t*>(c.part);
    if (ks == 1) {
      // lanes of one sequence column: n, n + 16, n + 32, n + 48
      uint64_t k = live ? amax_key(best.v, best.i) : 0;
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        const uint64_t y = __shfl_xor(k, o);
        k = y > k ? y : k;
      }
      __syncthreads();
      if (c.lane < 16) keys[c.wave * 16 + c.lane] = k;
    } else {
      __syncthreads();
      // scan the reduced logits of this task (<= 8 blocks) per sequence
      uint64_t k = 0;
      if (c.tid < P.B) {
        for (int j = 0; j < nblk; ++j)
          for (int q = 0; q < kTileRows; ++q) {
            const float v = c.part[(size_t)(j * ks) * (kTileRows * kTileLd) + q * kTileLd + c.tid];
            const uint64_t kk = amax_key(v, ((int)t.a0 + j) * kTileRows + q);
            k = kk > k ? kk : k;
          }
      }
      __syncthreads();
      if (c.wave == 0 && c.lane < 16) keys[c.lane] = k;
      if (c.wave > 0 && c.lane < 16) keys[c.wave * 16 + c.lane] = 0;
    }
    __syncthreads();
    lm_finish_b(P, c, t);
  }
  return true;
}

// Batched attention: task (sequence nu, kv head a0, chunk a1); the chunk is
// walked in blocks of kMaxChunk positions with each wave's running maximum,
// sum and P.V rescaled from block to block.  Layout per block as in attn_task.
// Prefill attention input: q of token n (G heads, scaled), then the k and v
// rows of kv head g of every token of the step, into qs[G * D], kcur[B][D],
// vcur[B][D]; element groups of 4, polled until they carry this step's tag
// (one round: G * D + 2 * B * D <= 1280 words).  Ends with a barrier; false
// if the wait was aborted.
template <int G, int D>
__device__ __forceinline__ bool stage_prefill_qkv(const Params& P, Ctx& c, int l, int g, int n, float* qs, float* kcur,
                                                  float* vcur, int stage) {
  const int total = G * D + 2 * P.B * D;
  const int i = 4 * c.tid;  // one group per thread
  const bool on = i < total;
  const tword* src = P.q + seq_off(P, n, l, P.QD) + (size_t)g * G * D + i;
  float* dst = qs + i;
  float scale = P.qscale;
  if (i >= G * D) {
    const int e = i - G * D, m = e / (2 * D), r = e - m * 2 * D;  // token m, k (r < D) or v
    src = P.kvcur + seq_off(P, on ? m : 0, l, 2 * P.KVD) + (r < D ? 0 : P.KVD) + (size_t)g * D + (r % D);
    dst = (r < D ? kcur : vcur) + m * D + (r % D);
    scale = 1.f;
  }
  tword4 w = on ? ld_tag4_agent(src) : ready_word4(c.epoch);
  uint64_t t0 = 0;
  bool stop = false;
  while (!tag4_ready(w, c.epoch)) {
    if (poll_stop(P, t0, stage, tag_of(w.x))) {
      stop = true;
      break;
    }
    w = ld_tag4_agent(src);
  }
  __syncthreads();  // the previous task's LDS readers are done
  if (on && !stop) {
    const float4 v = tag_value4(w);
    *reinterpret_cast<float4*>(dst) = make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale);
  }
  if (stop) c.flags[0] = 1;
  __syncthreads();
  return c.flags[0] == 0;
}

// Eight bf16 of a row held in LDS as bf16-exact fp32 (this step's k or v rows).
__device__ __forceinline__ uint4 pack8_bf16(const float* x) {
  const float4 a = *reinterpret_cast<const float4*>(x);
  const float4 b = *reinterpret_cast<const float4*>(x + 4);
  return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
}

// Eight fp32 in LDS as the bf16 hi and lo parts of an MFMA operand.
__device__ __forceinline__ void hilo8_lds(const float* x, bf16x8& hi, bf16x8& lo) {
  const float4 a = *reinterpret_cast<const float4*>(x);
  const float4 b = *reinterpret_cast<const float4*>(x + 4);
  uint4 h, l;
  hilo_pair(a.x, a.y, h.x, l.x);
  hilo_pair(a.z, a.w, h.y, l.y);
  hilo_pair(b.x, b.y, h.z, l.z);
  hilo_pair(b.z, b.w, h.w, l.w);
  __builtin_memcpy(&hi, &h, sizeof(hi));
  __builtin_memcpy(&lo, &l, sizeof(lo));
}

// Batched attention on MFMA: task (sequence nu, kv head a0, chunk a1); the
// chunk's positions are cut into blocks of 32, block q walked by wave q % 8,
// each wave keeping the running maximum, sum and P.V of the G query heads.
// Per block, in the 16x16x32 bf16 MFMA layout (A: lane l holds row l % 16,
// k elements 8 (l / 16) .. +8; B: column l % 16, same k; C: column l % 16,
// rows 4 (l / 16) .. +4):
//   scores S^T[position][head] = K . Q^T: A = two 16-position tiles of K rows
//     (bf16, straight from the cache), B = q in bf16 hi and lo parts, two
//     halves of head_dim 64 (8 MFMAs);
//   softmax per head over the 4 lanes holding its column;
//   O[head][d] += P . V: A = P rows (hi and lo) read back from a per-wave LDS
//     scratch, B = V transposed through a per-wave LDS scratch (rows of 32
//     positions, 80 bytes apart), four 16-wide d tiles (8 MFMAs).
// Positions from pos on take this step's k and v rows from LDS; positions past
// the chunk are masked.  The eight waves' {max, sum, P.V} are then merged as
// in attn_task.
template <int G, int D>
__device__ __forceinline__ bool attn_task_b(const Params& P, Ctx& c, const Task& t, int s) {
  static_assert(D == 64, "batched attention: head_dim 64 (two 32-wide MFMA k halves)");
  static_assert(G <= 4, "batched attention: the P.V rows of all heads in one lane group");
  constexpr int BLK = 32;  // positions per block
  constexpr int VRS = 40;  // V^T row stride in bf16 (32 positions, 8 padding)
  const int l = t.layer, g = (int)t.a0, ch = (int)t.a1, n = (int)t.nu;
  const int C = P.attn_chunks;
  // prefill: token n of one sequence, at position pos + n, sees the cache
  // below pos and this step's tokens 0..n (their k and v staged from kvcur)
  const bool pf = P.prefill != 0;
  const int npos = c.pos + (pf ? n : 0) + 1;
  const int len0 = (npos + C - 1) / C;
  const int t0 = min(npos, ch * len0), t1 = min(npos, t0 + len0);
  const int nblk = (t1 - t0 + BLK - 1) / BLK;

  const size_t head_off = (seq_off(P, pf ? 0 : n, l, P.NKV) + g) * P.S * D;
  const int r16 = c.lane & 15, q4 = c.lane >> 4;  // MFMA lane roles
  // V rows: lane loads position vp of the block, the 8-wide d chunks 2 j + vh
  // (j < 4), so that its transposed writes and the other half-wave's fall on
  // different LDS banks
  const int vp = c.lane & 31, vh = c.lane >> 5;
  // K and V of one block from the cache: positions from pos on (this step's,
  // from LDS below) and past the chunk read slot 0 (in bounds)
  uint4 kq[2][2], vq[4];
  auto load_block = [&](int base) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int p = base + 16 * mt + r16;
      const int sl = (p < t1 && p < c.pos) ? p : 0;
      const uint16_t* kr = P.kcache + head_off + (size_t)sl * D + 8 * q4;
      kq[mt][0] = *reinterpret_cast<const uint4*>(kr);
      kq[mt][1] = *reinterpret_cast<const uint4*>(kr + 32);
    }
    const int p = base + vp;
    const int sl = (p < t1 && p < c.pos) ? p : 0;
    const uint16_t* vr = P.vcache + head_off + (size_t)sl * D + 8 * vh;
#pragma unroll
    for (int j = 0; j < 4; ++j) vq[j] = *reinterpret_cast<const uint4*>(vr + 16 * j);
  };
  const int blk0 = c.wave;
  if (blk0 < nblk) load_block(t0 + blk0 * BLK);

  // LDS: q [G][D] (scaled), this step's k and v rows [nrows][D], per-wave
  // partial outputs [waves][G][D], per-wave max and sum [waves][G], then per
  // wave the block's probabilities [G][32] and V^T [D][VRS] bf16
  const int nrows = pf ? P.B : 1;  // k / v rows of this step in LDS
  float* qs = c.act;
  float* kcur = qs + G * D;
  float* vcur = kcur + nrows * D;
  float* wpart = vcur + nrows * D;
  float* wm = wpart + kWaves * G * D;
  float* wl = wm + kWaves * G;
  float* pw = wl + kWaves * G + c.wave * (G * BLK + D * VRS / 2);
  uint16_t* vt = reinterpret_cast<uint16_t*>(pw + G * BLK);
  if (!pf) {
    const Seg seg[3] = {{qs, P.q + seq_off(P, n, l, P.QD) + (size_t)g * G * D, G * D, P.qscale},
                        {kcur, P.kvcur + seq_off(P, n, l, 2 * P.KVD) + (size_t)g * D, D, 1.f},
                        {vcur, P.kvcur + seq_off(P, n, l, 2 * P.KVD) + P.KVD + (size_t)g * D, D, 1.f}};
    if (!stage_tagged(P, c, seg, s)) return false;
  } else if (!stage_prefill_qkv<G, D>(P, c, l, g, n, qs, kcur, vcur, s)) {
    return false;
  }
  mark(c, 1);

  // q as the B operand: lane: head r16 (zero past G), dims 8 q4 + 32 dh .. +8
  bf16x8 qh[2], ql[2];
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) {
    hilo8_lds(qs + (r16 < G ? r16 : 0) * D + 8 * q4 + 32 * dh, qh[dh], ql[dh]);
    if (r16 >= G) {
      qh[dh] = bf16x8{};
      ql[dh] = bf16x8{};
    }
  }
  float m = -__builtin_inff(), ls = 0.f;  // softmax state of head r16 (its 4 lanes agree)
  f32x4 ov[4];                            // O[head 4 q4 + i][d = r16 + 16 dt]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) ov[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int q = blk0; q < nblk; q += kWaves) {
    const int base = t0 + q * BLK;
    if (q != blk0) load_block(base);
    // this step's rows (bf16-exact values in LDS) for the positions from pos on
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int p = base + 16 * mt + r16;
      if (p >= c.pos && p < t1) {
        const float* kr = kcur + (p - c.pos) * D + 8 * q4;
        kq[mt][0] = pack8_bf16(kr);
        kq[mt][1] = pack8_bf16(kr + 32);
      }
    }
    {
      const int p = base + vp;
      if (p >= c.pos && p < t1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) vq[j] = pack8_bf16(vcur + (p - c.pos) * D + 8 * vh + 16 * j);
      } else if (p >= t1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) vq[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // scores of the two 16-position tiles
    f32x4 sc[2];
    float bm = -__builtin_inff();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
        bf16x8 a;
        __builtin_memcpy(&a, &kq[mt][dh], sizeof(a));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[dh], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[dh], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = base + 16 * mt + 4 * q4 + i;
        acc[i] = (p < t1 && r16 < G) ? acc[i] : -__builtin_inff();
        bm = fmaxf(bm, acc[i]);
      }
      sc[mt] = acc;
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    const float scale = m == -__builtin_inff() ? 0.f : __expf(m - mn);
    float ps = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = sc[mt][i] == -__builtin_inff() ? 0.f : __expf(sc[mt][i] - mn);
        sc[mt][i] = e;
        ps += e;
      }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    ls = fmaf(ls, scale, ps);
    m = mn;
    // P rows to LDS: lane: head r16, positions 16 mt + 4 q4 .. +4
    if (r16 < G) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        *reinterpret_cast<f32x4*>(pw + r16 * BLK + 16 * mt + 4 * q4) = sc[mt];
    }
    // V^T: position vp, dims 8 (2 j + vh) .. +8
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w4[4] = {vq[j].x, vq[j].y, vq[j].z, vq[j].w};
      uint16_t* col = vt + (8 * (2 * j + vh)) * VRS + vp;
#pragma unroll
      for (int e = 0; e < 8; ++e) col[e * VRS] = (uint16_t)((e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xFFFFu));
    }
    __builtin_amdgcn_wave_barrier();
    // the rows of O are rescaled by their head's factor (heads 0..3: lanes 0..3)
    float sh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sh[i] = lane_value(scale, i);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[dt][i] *= sh[i];
    // P as the A operand: lane: head r16 (zero past G), positions 8 q4 .. +8
    bf16x8 ph, pl;
    hilo8_lds(pw + (r16 < G ? r16 : 0) * BLK + 8 * q4, ph, pl);
    if (r16 >= G) {
      ph = bf16x8{};
      pl = bf16x8{};
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint4 vb4 = *reinterpret_cast<const uint4*>(vt + (r16 + 16 * dt) * VRS + 8 * q4);
      bf16x8 vb;
      __builtin_memcpy(&vb, &vb4, sizeof(vb));
      ov[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, ov[dt], 0, 0, 0);
      ov[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, ov[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }
  // this wave's {max, sum} (lanes 0..G-1) and P.V rows (lanes 0..15: heads i < G)
  if (q4 == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) wpart[(c.wave * G + i) * D + r16 + 16 * dt] = ov[dt][i];
  }
  if (c.lane < G) {
    wm[c.wave * G + c.lane] = m;
    wl[c.wave * G + c.lane] = ls;
  }
  mark_wave(c);
  __syncthreads();
  mark(c, 2);

  const int h = c.tid / D, d = c.tid % D;
  float A = 0.f, Ls = 0.f, M = -__builtin_inff();
  if (c.tid < G * D) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * G + h]);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = wm[w * G + h];
      const float e = mw == -__builtin_inff() ? 0.f : __expf(mw - M);
      A = fmaf(e, wpart[(w * G + h) * D + d], A);
      Ls = fmaf(e, wl[w * G + h], Ls);
    }
  }
  tword* o = P.o + seq_off(P, n, l, P.QD) + (size_t)g * G * D;
  if (C == 1) {
    if (c.tid < G * D) st_tag(o + c.tid, A / Ls, c.epoch);
    return true;
  }
  const int stride = G * (D + 2);
  const size_t head = seq_off(P, n, l, P.NKV) + g;  // (sequence, layer, kv head)
  float* mine = P.attn_part + (head * C + ch) * stride;
  if (c.tid < G * D) st_f32_agent(mine + 2 * G + c.tid, A);
  if (c.tid < G * D && d == 0) {
    st_f32_agent(mine + h, M);
    st_f32_agent(mine + G + h, Ls);
  }
  wait_all_vmem();
  __syncthreads();
  if (c.tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(P.attn_ctr + head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    c.flags[1] = old == c.epoch * (uint32_t)C - 1u;
  }
  __syncthreads();
  if (c.flags[1]) merge_chunks<G, D, 8, false>(c, P.attn_part + head * C * stride, C, stride, G, 0, wpart, o);
  return true;
}

// ---------------------------------------------------------------------------
// the stage loop shared by the persistent kernel and the per-stage kernels
// ---------------------------------------------------------------------------

// Kernel instance flags.
constexpr int kFlagTrace = 1;    // records the per-(workgroup, stage) trace stamps
constexpr int kFlagPartial = 2;  // carries the partial-input down projection

// G query heads per kv head and head_dim D are template parameters so that a
// kernel instance carries exactly one attention variant (register budget):
// GT query heads per attention task (1 or G), or GT = 0 for an instance that
// carries both and picks at run time.  FLAGS adds the trace stamps or the
// partial-input down projection; instances without them do not contain that
// code at all (the step time of this kernel moves by 5-20 us with the size of
// the code it carries: instruction-cache misses).
//
// STEPS launches run n_steps greedy steps in one launch (the glossary entry
// "Megakernel", section "Wie eine ganze Rechenkette in ein Programm passt":
// the kernel is started once and stays running): the stage loop walks the
// tape n_steps times, each step with the next epoch and position, and every
// step after the first takes its input tokens from the tagged words the
// previous step's argmax published (P.tok_tag).
template <int G, int D, bool BATCHED, int GT, int FLAGS, bool STEPS>
__device__ __forceinline__ void run_stages(const Params& P, int s_begin, int s_end, int n_steps) {
  constexpr bool PARTIAL = (FLAGS & kFlagPartial) != 0;
  constexpr bool TRACE = (FLAGS & kFlagTrace) != 0;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Ctx c;
  c.b = (int)blockIdx.x;
  c.tid = (int)threadIdx.x;
  c.wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  c.lane = (int)threadIdx.x & 63;
  if (P.dargs) {
    c.pos = P.dargs->pos;
    c.epoch = P.dargs->epoch;
  } else {
    c.pos = P.pos;
    c.epoch = P.epoch;
  }
  c.act = reinterpret_cast<float*>(smem + P.lds_act);
  c.res = reinterpret_cast<float*>(smem + P.lds_res);
  c.rope = reinterpret_cast<float*>(smem + P.lds_rope);
  c.red = reinterpret_cast<float*>(smem + P.lds_misc);
  c.red64 = reinterpret_cast<uint64_t*>(smem + P.lds_misc + 64);
  c.flags = reinterpret_cast<int*>(smem + P.lds_misc + 128);
  c.part = reinterpret_cast<float*>(smem + P.lds_part);
  c.tok = reinterpret_cast<int*>(smem + P.lds_misc + 160);
  c.logits = P.logits;
  c.out_tok = P.out_token;
  if (c.tid < 4) c.flags[c.tid] = 0;
  if (c.tid < P.B) c.tok[c.tid] = P.token[c.tid];
  c.tr = nullptr;
  // this workgroup's column of the tape, stages [s_begin, s_end), into LDS
  {
    constexpr int kWords = (int)(sizeof(Task) / 4);
    uint32_t* dst = reinterpret_cast<uint32_t*>(smem + P.lds_tape);
    for (int i = c.tid; i < (s_end - s_begin) * kWords; i += kThreads) {
      const int s = s_begin + i / kWords;
      dst[i] = reinterpret_cast<const uint32_t*>(P.tape + (size_t)s * P.num_wgs + c.b)[i % kWords];
    }
  }
  __syncthreads();

  Stream st;
  st.ring = lds_byte(smem) + (uint32_t)c.wave * (uint32_t)((BATCHED ? kRingBatched : kRing) * kUnitBytes);
  st.tape = lds_byte(smem) + (uint32_t)P.lds_tape;
  st.issued = st.consumed = st.lslot = st.cslot = 0;
  st.s_begin = s_begin;
  st.s_end = STEPS ? s_begin + n_steps * (s_end - s_begin) : s_end;
  st.period = s_end - s_begin;
  st.ldone = false;
  if constexpr (BATCHED) {
    loader_seek_b(P, st, s_begin, c.wave);
    top_up_b(P, st, c.wave, c.lane, kRingBatched);
  } else {
    loader_seek(P, st, s_begin, c.b, c.wave);
    top_up(P, st, c.b, c.wave, c.lane, kRing);
  }

  for (int gs = s_begin; gs < st.s_end; ++gs) {
    int s = gs;
    if constexpr (STEPS) {
      s = s_begin + (gs - s_begin) % st.period;
      if (s == s_begin && gs != s_begin) {
        // the next step: epoch, position, outputs, and the tokens the last one picked
        ++c.epoch;
        ++c.pos;
        c.logits += P.logits_step;
        c.out_tok += P.B;
        bool stop = false;
        if (c.tid < P.B) {
          uint64_t w = ld_u64_agent(P.tok_tag + c.tid);
          uint64_t t0 = 0;
          while ((uint32_t)(w >> 32) != c.epoch) {
            if (poll_stop(P, t0, s, (uint32_t)(w >> 32))) {
              stop = true;
              break;
            }
            w = ld_u64_agent(P.tok_tag + c.tid);
          }
          c.tok[c.tid] = (int32_t)(uint32_t)w;
        }
        if (stop) c.flags[0] = 1;
        __syncthreads();
        if (c.flags[0]) break;
      }
    }
    const Task t = task_at(st.tape, s - s_begin);
    if constexpr (TRACE)
      c.tr = (P.trace != nullptr && t.op != OP_NONE) ? P.trace + ((size_t)c.b * P.num_stages + s) * kTraceStamps
                                                     : nullptr;
    mark(c, 0);
    bool ok = true;
    if constexpr (BATCHED) {
      switch (t.op) {
        case OP_QKV: ok = gemm_task<OP_QKV>(P, c, st, t, s); break;
        case OP_OPROJ: ok = gemm_task<OP_OPROJ>(P, c, st, t, s); break;
        case OP_GU: ok = gemm_task<OP_GU>(P, c, st, t, s); break;
        case OP_DOWN: ok = gemm_task<OP_DOWN>(P, c, st, t, s); break;
        case OP_LM: ok = gemm_task<OP_LM>(P, c, st, t, s); break;
        case OP_ATTN: ok = attn_task_b<G, D>(P, c, t, s); break;
        default: break;
      }
    } else {
      switch (t.op) {
        case OP_QKV: ok = gemv_task<OP_QKV>(P, c, st, t, s); break;
        case OP_OPROJ: ok = gemv_task<OP_OPROJ>(P, c, st, t, s); break;
        case OP_GU: ok = gemv_task<OP_GU>(P, c, st, t, s); break;
        case OP_DOWN:
          if constexpr (PARTIAL)
            ok = (t.region & kRegionPartial) ? down_partial(P, c, st, t, s) : gemv_task<OP_DOWN>(P, c, st, t, s);
          else
            ok = gemv_task<OP_DOWN>(P, c, st, t, s);
          break;
        case OP_LM: ok = gemv_task<OP_LM>(P, c, st, t, s); break;
        case OP_ATTN:
          if constexpr (G == 1 || GT == 1)
            ok = attn_task<1, D>(P, c, t, s);
          else if constexpr (GT == G)
            ok = attn_task<G, D>(P, c, t, s);
          else
            ok = P.attn_gt == 1 ? attn_task<1, D>(P, c, t, s) : attn_task<G, D>(P, c, t, s);
          break;
        default: break;
      }
    }
    mark(c, 3);
    if (!ok) break;
  }
  wait_all_vmem();
}

template <int G, int D, bool BATCHED, int GT, int FLAGS>
__global__ void __launch_bounds__(kThreads, 1) mk_persistent(Params P) {
  run_stages<G, D, BATCHED, GT, FLAGS, false>(P, 0, P.num_stages, 1);
}

template <int G, int D, bool BATCHED, int GT, int FLAGS>
__global__ void __launch_bounds__(kThreads, 1) mk_stage(Params P, int s) {
  run_stages<G, D, BATCHED, GT, FLAGS, false>(P, s, s + 1, 1);
}

template <int G, int D, bool BATCHED, int GT, int FLAGS>
__global__ void __launch_bounds__(kThreads, 1) mk_persistent_steps(Params P, int n_steps) {
  run_stages<G, D, BATCHED, GT, FLAGS, true>(P, 0, P.num_stages, n_steps);
}

// Host-side handles of one kernel instance.
struct KernelPair {
  const void* persistent;
  const void* stage;
  const void* steps;
};

}  // namespace mk

#endif  // MK_DEVICE_H_
