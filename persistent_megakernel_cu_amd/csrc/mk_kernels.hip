// mk_kernels.hip -- gfx950 device code: the persistent decode megakernel and
// the per-stage kernels of the launch-per-op baseline (same executors).
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
// So every activation element travels as one 8-byte word {fp32 value, epoch}
// written and read with agent-scope (sc1) accesses: the consumer polls the
// data itself, no fence and no counter sits on the critical path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"
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
__device__ __forceinline__ void dma_unit(const char* gsrc, uint32_t lds_dst) {
  uint32_t keep;
  lds_dst = __builtin_amdgcn_readfirstlane(lds_dst);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
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

__device__ __forceinline__ void st_tag(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
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

// Argmax key: larger key = larger value, ties -> lower index; 0 = no candidate.
__device__ __forceinline__ uint64_t amax_key(float v, int idx) {
  if (idx < 0) return 0;
  const uint32_t u = __float_as_uint(v);
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
};

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

// One poll iteration's bookkeeping; true when the wait must stop.
__device__ __forceinline__ bool poll_stop(const Params& P, uint64_t& t0, int stage, uint32_t seen) {
  const uint64_t now = wall_clock64();
  if (t0 == 0) {
    t0 = now | 1;
  } else if (now - t0 > P.watchdog_ticks) {
    latch_error(P, MK_E_TIMEOUT, stage, seen);
    return true;
  }
  return ld_u32_agent(P.abort_flag) != 0;
}

// Copy n tagged elements into LDS as fp32 once every one carries this step's
// tag, and zero dst[n, zero_to).  WG-cooperative.  The first round of polls is
// issued before a barrier that separates these LDS writes from the previous
// task's last LDS reads, so the poll latency overlaps slower waves finishing.
// Ends with a barrier.  Returns false if the wait was aborted.
__device__ __forceinline__ bool stage_tagged(const Params& P, Ctx& c, float* dst, const uint64_t* src, int n, int stage,
                                             int zero_to = 0) {
  bool stop = false;
  for (int i0 = 0; i0 == 0 || i0 < n; i0 += kThreads * 4) {
    uint64_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * kThreads + c.tid;
      w[j] = i < n ? ld_tag(src + i) : ((uint64_t)c.epoch << 32);
    }
    uint64_t t0 = 0;
    while (!stop) {
      bool ready = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) ready &= (uint32_t)(w[j] >> 32) == c.epoch;
      if (ready) break;
      if (poll_stop(P, t0, stage, (uint32_t)(w[0] >> 32))) {
        stop = true;
        break;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * kThreads + c.tid;
        if (i < n && (uint32_t)(w[j] >> 32) != c.epoch) w[j] = ld_tag(src + i);
      }
    }
    if (i0 == 0) {
      __syncthreads();
      for (int i = n + c.tid; i < zero_to; i += kThreads) dst[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * kThreads + c.tid;
      if (i < n) dst[i] = __uint_as_float((uint32_t)w[j]);
    }
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

// Embedding row of the input token (bf16 -> fp32) into dst[0, H).
__device__ __forceinline__ void stage_embedding(const Params& P, Ctx& c, float* dst, int stage) {
  if (c.tid == 0) {
    int tok = P.token[0];
    if (tok < 0 || tok >= P.V) {
      latch_error(P, MK_E_TOKEN, stage, (uint32_t)tok);
      __hip_atomic_store(&P.tokerr[0], c.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      tok = 0;
    }
    c.flags[2] = tok;
  }
  __syncthreads();
  const uint16_t* row = P.embed + (size_t)c.flags[2] * P.H;
  for (int i = c.tid; i < P.H; i += kThreads) dst[i] = bf16_to_f32(row[i]);
  __syncthreads();
}

// dst[0, n) = RMSNorm(dst) * g over the first n entries; dst[n, npad) = 0.
__device__ __forceinline__ void rmsnorm_lds(const Params& P, Ctx& c, float* x, const float* g, int n, int npad) {
  float ss = 0.f;
  for (int i = c.tid; i < n; i += kThreads) ss = fmaf(x[i], x[i], ss);
  ss = block_sum(c, ss);
  const float r = rsqrtf(ss / (float)n + P.eps);
  for (int i = c.tid; i < npad; i += kThreads) x[i] = i < n ? x[i] * r * g[i] : 0.f;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// the per-wave weight stream (LDS ring, loader running ahead of the consumer)
// ---------------------------------------------------------------------------

struct Stream {
  uint32_t ring;   // LDS byte address of this wave's ring
  int issued, consumed, lslot, cslot;
  int ls, s_end;
  uint32_t lpair, lend, lnu, lu;
  const char* lbase;
  bool ldone;
};

// Task records are immutable during a launch; read them with a scalar load so
// that neither the loader nor the consumer waits on vector-memory counters.
__device__ __forceinline__ Task task_at(const Params& P, int s, int b) {
  typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
  const Task* ptr = P.tape + (size_t)s * P.num_wgs + b;
  u32x8 r;
  asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(ptr));
  Task t;
  t.op = (uint8_t)(r[0] & 0xffu);
  t.region = (uint8_t)((r[0] >> 8) & 0xffu);
  t.layer = (uint16_t)(r[0] >> 16);
  t.a0 = r[1];
  t.a1 = r[2];
  t.nu = r[3];
  t.wofs = (uint64_t)r[4] | ((uint64_t)r[5] << 32);
  t.ntasks = r[6];
  t.pad = r[7];
  return t;
}

__device__ __forceinline__ void loader_seek(const Params& P, Stream& st, int s, int b, int wave) {
  for (; s < st.s_end; ++s) {
    const Task t = task_at(P, s, b);
    if (op_is_gemv(t.op)) {
      const uint32_t p = t.a0 + (uint32_t)wave;
      if (p < t.a1) {
        st.ls = s;
        st.lpair = p;
        st.lend = t.a1;
        st.lnu = t.nu;
        st.lu = 0;
        st.lbase = (t.region ? P.lm : P.arena) + t.wofs;
        return;
      }
    }
  }
  st.ls = st.s_end;
  st.ldone = true;
}

__device__ __forceinline__ void loader_issue(const Params& P, Stream& st, int b, int wave, int lane) {
  if (st.ldone) return;
  const char* g = st.lbase + ((uint64_t)st.lpair * st.lnu + st.lu) * kUnitBytes + (uint32_t)lane * 16u;
  dma_unit(g, st.ring + (uint32_t)st.lslot * kUnitBytes);
  ++st.issued;
  st.lslot = (st.lslot + 1 == kRing) ? 0 : st.lslot + 1;
  if (++st.lu == st.lnu) {
    st.lu = 0;
    st.lpair += kWaves;
    if (st.lpair >= st.lend) loader_seek(P, st, st.ls + 1, b, wave);
  }
}

// Next unit of this wave's stream; refills the freed slot.
__device__ __forceinline__ uint4 consume_unit(const Params& P, Stream& st, int b, int wave, int lane) {
  const uint32_t a = st.ring + (uint32_t)st.cslot * kUnitBytes + (uint32_t)lane * 16u;
  uint4 v;
  if (st.issued - st.consumed == kRing)
    v = ring_read<kRing - 1>(a);
  else
    v = ring_read<0>(a);
  ++st.consumed;
  st.cslot = (st.cslot + 1 == kRing) ? 0 : st.cslot + 1;
  loader_issue(P, st, b, wave, lane);
  return v;
}

// ---------------------------------------------------------------------------
// GEMV stages: prologue (stage activation), row pairs, epilogue
// ---------------------------------------------------------------------------

// Residual input of layer l (x after the previous layer, or the embedding).
__device__ __forceinline__ const uint64_t* x_in(const Params& P, int l) {
  return P.x_ffn + (size_t)(l - 1) * P.H;
}

template <int OP>
__device__ __forceinline__ bool gemv_prologue(const Params& P, Ctx& c, const Task& t, int s) {
  const int l = t.layer;
  if (OP == OP_QKV || OP == OP_LM) {
    const float* g = OP == OP_QKV ? P.g_attn + (size_t)l * P.Hp : P.g_final;
    if (l == 0) {
      stage_embedding(P, c, c.act, s);
    } else if (!stage_tagged(P, c, c.act, x_in(P, l), P.H, s)) {
      return false;
    }
    rmsnorm_lds(P, c, c.act, g, P.H, P.Hp);
    if (OP == OP_QKV) {
      const float* rp = P.rope + (size_t)c.pos * P.D;
      for (int i = c.tid; i < P.D; i += kThreads) c.rope[i] = rp[i];
      __syncthreads();
    }
  } else if (OP == OP_GU) {
    if (!stage_tagged(P, c, c.act, P.x_attn + (size_t)l * P.H, P.H, s)) return false;
    rmsnorm_lds(P, c, c.act, P.g_ffn + (size_t)l * P.Hp, P.H, P.Hp);
  } else {  // OPROJ, DOWN: plain activation + residual rows of this task
    const int n = OP == OP_OPROJ ? P.QD : P.F;
    const int np = OP == OP_OPROJ ? P.QDp : P.Fp;
    const uint64_t* src = OP == OP_OPROJ ? P.o + (size_t)l * P.QD : P.h + (size_t)l * P.F;
    if (!stage_tagged(P, c, c.act, src, n, s, np)) return false;
    const int r0 = 2 * (int)t.a0, nr = 2 * (int)(t.a1 - t.a0);
    if (OP == OP_OPROJ && l == 0) {
      // the residual of layer 0 is the embedding row itself
      if (c.tid == 0) {
        int tok = P.token[0];
        if (tok < 0 || tok >= P.V) tok = 0;
        c.flags[2] = tok;
      }
      __syncthreads();
      const uint16_t* row = P.embed + (size_t)c.flags[2] * P.H + r0;
      for (int i = c.tid; i < nr; i += kThreads) c.res[i] = bf16_to_f32(row[i]);
      __syncthreads();
    } else {
      const uint64_t* rs = OP == OP_OPROJ ? x_in(P, l) + r0 : P.x_attn + (size_t)l * P.H + r0;
      if (!stage_tagged(P, c, c.res, rs, nr, s)) return false;
    }
  }
  return true;
}

struct LmBest {
  float v;
  int i;
};

template <int OP>
__device__ __forceinline__ void gemv_epilogue(const Params& P, Ctx& c, const Task& t, uint32_t pair, float v0, float v1,
                                              LmBest& best) {
  const int l = t.layer;
  const int r = 2 * (int)pair;
  const uint32_t tag = c.epoch;
  if (OP == OP_QKV) {
    if (r < P.QD + P.KVD) {  // q or k rows: rotate the pair (2i, 2i+1) of its head
      const int rr = r < P.QD ? r : r - P.QD;
      const int j = rr % P.D;
      const float cs = c.rope[j], sn = c.rope[j + 1];
      const float y0 = v0 * cs - v1 * sn;
      const float y1 = v0 * sn + v1 * cs;
      if (r < P.QD) {
        if (c.lane == 0) st_tag(P.q + (size_t)l * P.QD + r, y0, tag);
        if (c.lane == 1) st_tag(P.q + (size_t)l * P.QD + r + 1, y1, tag);
      } else {
        const uint16_t k0 = f32_to_bf16(y0), k1 = f32_to_bf16(y1);
        const int hk = rr / P.D;
        if (c.lane == 0) {
          uint16_t* dst = P.kcache + (((size_t)l * P.NKV + hk) * P.S + c.pos) * P.D + j;
          *reinterpret_cast<uint32_t*>(dst) = (uint32_t)k0 | ((uint32_t)k1 << 16);
          st_tag(P.kvcur + (size_t)l * 2 * P.KVD + rr, bf16_to_f32(k0), tag);
        }
        if (c.lane == 1) st_tag(P.kvcur + (size_t)l * 2 * P.KVD + rr + 1, bf16_to_f32(k1), tag);
      }
    } else {  // v rows
      const int rr = r - P.QD - P.KVD;
      const int hv = rr / P.D, j = rr % P.D;
      const uint16_t b0 = f32_to_bf16(v0), b1 = f32_to_bf16(v1);
      if (c.lane == 0) {
        uint16_t* dst = P.vcache + (((size_t)l * P.NKV + hv) * P.S + c.pos) * P.D + j;
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)b0 | ((uint32_t)b1 << 16);
        st_tag(P.kvcur + ((size_t)l * 2 + 1) * P.KVD + rr, bf16_to_f32(b0), tag);
      }
      if (c.lane == 1) st_tag(P.kvcur + ((size_t)l * 2 + 1) * P.KVD + rr + 1, bf16_to_f32(b1), tag);
    }
  } else if (OP == OP_OPROJ || OP == OP_DOWN) {
    uint64_t* dst = (OP == OP_OPROJ ? P.x_attn : P.x_ffn) + (size_t)l * P.H + r;
    const int k = r - 2 * (int)t.a0;
    if (c.lane == 0) st_tag(dst, c.res[k] + v0, tag);
    if (c.lane == 1) st_tag(dst + 1, c.res[k + 1] + v1, tag);
  } else if (OP == OP_GU) {
    // pair = (gate row f, up row f): h_f = silu(gate) * up
    const float sg = v0 / (1.0f + __expf(-v0));
    if (c.lane == 0) st_tag(P.h + (size_t)l * P.F + pair, sg * v1, tag);
  } else if (OP == OP_LM) {
    if (c.lane == 0) {
      P.logits[r] = v0;
      P.logits[r + 1] = v1;
    }
    if (v0 > best.v) { best.v = v0; best.i = r; }
    if (v1 > best.v) { best.v = v1; best.i = r + 1; }
  }
}

// Argmax stage 2: every LM task publishes its key; the last to arrive picks the token.
__device__ __forceinline__ void lm_finish(const Params& P, Ctx& c, const Task& t, const LmBest& best) {
  if (c.lane == 0) c.red64[c.wave] = amax_key(best.v, best.i);
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
      const uint64_t x = ld_tag(P.amax + w);
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
      P.out_token[0] = idx;
    }
  }
}

template <int OP>
__device__ __forceinline__ bool gemv_task(const Params& P, Ctx& c, Stream& st, const Task& t, int s) {
  if (!gemv_prologue<OP>(P, c, t, s)) return false;
  const int half = (int)t.nu >> 1;  // units per row
  LmBest best{-__builtin_inff(), -1};
  const float* xa = c.act + c.lane * 8;
  for (uint32_t pair = t.a0 + (uint32_t)c.wave; pair < t.a1; pair += kWaves) {
    float a0 = 0.f, a1 = 0.f;
    for (int j = 0; j < half; ++j) a0 += dot8(consume_unit(P, st, c.b, c.wave, c.lane), xa + j * kUnitElems);
    for (int j = 0; j < half; ++j) a1 += dot8(consume_unit(P, st, c.b, c.wave, c.lane), xa + j * kUnitElems);
    a0 = wave_sum(a0);
    a1 = wave_sum(a1);
    gemv_epilogue<OP>(P, c, t, pair, a0, a1, best);
  }
  if (OP == OP_LM) lm_finish(P, c, t, best);
  return true;
}

// ---------------------------------------------------------------------------
// attention: one (kv head, chunk) per task, G query heads, merge by last chunk
// ---------------------------------------------------------------------------

template <int G>
__device__ __forceinline__ bool attn_task(const Params& P, Ctx& c, const Task& t, int s) {
  const int l = t.layer, g = (int)t.a0, ch = (int)t.a1;
  const int D = P.D, C = P.attn_chunks;
  const int n = c.pos + 1;
  const int len = (n + C - 1) / C;
  const int t0 = min(n, ch * len), t1 = min(n, t0 + len);
  const int lmax = (P.S + C - 1) / C;
  const int NP = kThreads / D;
  float* qs = c.act;             // [G][D]
  float* kcur = qs + G * D;      // [D]
  float* vcur = kcur + D;        // [D]
  float* sc = vcur + D;          // [lmax][G]
  float* part = sc + lmax * G;   // [NP][G][D]
  float* red = part + NP * G * D;  // m[kMaxGroup], l[kMaxGroup]

  if (!stage_tagged(P, c, qs, P.q + (size_t)l * P.QD + (size_t)g * G * D, G * D, s)) return false;
  if (!stage_tagged(P, c, kcur, P.kvcur + (size_t)l * 2 * P.KVD + (size_t)g * D, D, s)) return false;
  if (!stage_tagged(P, c, vcur, P.kvcur + ((size_t)l * 2 + 1) * P.KVD + (size_t)g * D, D, s)) return false;
  for (int i = c.tid; i < G * D; i += kThreads) qs[i] *= P.qscale;
  __syncthreads();

  const size_t head_off = ((size_t)l * P.NKV + g) * P.S * D;
  const uint16_t* kc = P.kcache + head_off;
  const uint16_t* vc = P.vcache + head_off;

  // scores s[t][h] = q_h . k_t / sqrt(D)
  for (int tt = t0 + c.tid; tt < t1; tt += kThreads) {
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    if (tt == c.pos) {
      for (int d = 0; d < D; ++d) {
        const float kv = kcur[d];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(qs[h * D + d], kv, acc[h]);
      }
    } else {
      const uint4* row = reinterpret_cast<const uint4*>(kc + (size_t)tt * D);
      for (int d8 = 0; d8 < D / 8; ++d8) {
        const uint4 w = row[d8];
        const float k8[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y),
                             bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h] = fmaf(qs[h * D + d8 * 8 + e], k8[e], acc[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) sc[(tt - t0) * G + h] = acc[h];
  }
  __syncthreads();

  // per-head max and exp-sum of this chunk (wave h owns head h)
  if (c.wave < G) {
    const int h = c.wave;
    float m = -__builtin_inff();
    for (int i = c.lane; i < t1 - t0; i += 64) m = fmaxf(m, sc[i * G + h]);
    m = wave_max(m);
    float ls = 0.f;
    for (int i = c.lane; i < t1 - t0; i += 64) {
      const float p = __expf(sc[i * G + h] - m);
      sc[i * G + h] = p;
      ls += p;
    }
    ls = wave_sum(ls);
    if (c.lane == 0) {
      red[h] = m;
      red[kMaxGroup + h] = ls;
    }
  }
  __syncthreads();

  // acc[h][d] = sum_t p[t][h] v_t[d], positions split over NP partitions
  {
    const int d = c.tid % D, prt = c.tid / D;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    for (int tt = t0 + prt; tt < t1; tt += NP) {
      const float v = tt == c.pos ? vcur[d] : bf16_to_f32(vc[(size_t)tt * D + d]);
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fmaf(sc[(tt - t0) * G + h], v, acc[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) part[(prt * G + h) * D + d] = acc[h];
  }
  __syncthreads();

  const int h = c.tid / D, d = c.tid % D;
  float a = 0.f;
  if (c.tid < G * D)
    for (int p = 0; p < NP; ++p) a += part[(p * G + h) * D + d];
  uint64_t* o = P.o + (size_t)l * P.QD + (size_t)g * G * D;
  if (C == 1) {
    if (c.tid < G * D) st_tag(o + c.tid, a / red[kMaxGroup + h], c.epoch);
    return true;
  }
  // publish this chunk's partial {m[G], l[G], acc[G][D]}; the last chunk of the head merges
  const int stride = G * (D + 2);
  float* mine = P.attn_part + (((size_t)l * P.NKV + g) * C + ch) * stride;
  if (c.tid < G * D) st_f32_agent(mine + 2 * G + c.tid, a);
  if (c.tid < G) {
    st_f32_agent(mine + c.tid, red[c.tid]);
    st_f32_agent(mine + G + c.tid, red[kMaxGroup + c.tid]);
  }
  wait_all_vmem();
  __syncthreads();
  if (c.tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(P.attn_ctr + (size_t)l * P.NKV + g, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    c.flags[1] = old == c.epoch * (uint32_t)C - 1u;
  }
  __syncthreads();
  if (c.flags[1] && c.tid < G * D) {
    const float* base = P.attn_part + ((size_t)l * P.NKV + g) * C * stride;
    float M = -__builtin_inff();
    for (int k = 0; k < C; ++k) M = fmaxf(M, ld_f32_agent(base + (size_t)k * stride + h));
    float Ls = 0.f, A = 0.f;
    for (int k = 0; k < C; ++k) {
      const float* pk = base + (size_t)k * stride;
      const float mk = ld_f32_agent(pk + h);
      const float e = mk == -__builtin_inff() ? 0.f : __expf(mk - M);
      Ls = fmaf(e, ld_f32_agent(pk + G + h), Ls);
      A = fmaf(e, ld_f32_agent(pk + 2 * G + c.tid), A);
    }
    st_tag(o + c.tid, A / Ls, c.epoch);
  }
  return true;
}

// ---------------------------------------------------------------------------
// the stage loop shared by the persistent kernel and the per-stage kernels
// ---------------------------------------------------------------------------

__device__ __forceinline__ void run_stages(const Params& P, int s_begin, int s_end) {
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
  if (c.tid < 4) c.flags[c.tid] = 0;
  __syncthreads();

  Stream st;
  st.ring = lds_byte(smem) + (uint32_t)c.wave * (kRing * kUnitBytes);
  st.issued = st.consumed = st.lslot = st.cslot = 0;
  st.s_end = s_end;
  st.ldone = false;
  loader_seek(P, st, s_begin, c.b, c.wave);
  for (int i = 0; i < kRing; ++i) loader_issue(P, st, c.b, c.wave, c.lane);

  for (int s = s_begin; s < s_end; ++s) {
    const Task t = task_at(P, s, c.b);
    bool ok = true;
    switch (t.op) {
      case OP_QKV: ok = gemv_task<OP_QKV>(P, c, st, t, s); break;
      case OP_OPROJ: ok = gemv_task<OP_OPROJ>(P, c, st, t, s); break;
      case OP_GU: ok = gemv_task<OP_GU>(P, c, st, t, s); break;
      case OP_DOWN: ok = gemv_task<OP_DOWN>(P, c, st, t, s); break;
      case OP_LM: ok = gemv_task<OP_LM>(P, c, st, t, s); break;
      case OP_ATTN:
        switch (P.G) {
          case 1: ok = attn_task<1>(P, c, t, s); break;
          case 2: ok = attn_task<2>(P, c, t, s); break;
          case 4: ok = attn_task<4>(P, c, t, s); break;
          default: ok = attn_task<8>(P, c, t, s); break;
        }
        break;
      default: break;
    }
    if (!ok) break;
  }
  wait_all_vmem();
}

__global__ void __launch_bounds__(kThreads, 1) mk_persistent(Params P) { run_stages(P, 0, P.num_stages); }

__global__ void __launch_bounds__(kThreads, 1) mk_stage(Params P, int s) { run_stages(P, s, s + 1); }

__global__ void mk_set_args(StepArgs* a, int pos, uint32_t epoch) {
  a->pos = pos;
  a->epoch = epoch;
}

__global__ void mk_advance_args(StepArgs* a) {
  a->pos += 1;
  a->epoch += 1;
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------

hipError_t configure_kernels(int lds_bytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mk_persistent),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&mk_stage), hipFuncAttributeMaxDynamicSharedMemorySize,
                             lds_bytes);
}

hipError_t persistent_occupancy(int lds_bytes, int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, reinterpret_cast<const void*>(&mk_persistent),
                                                      kThreads, lds_bytes);
}

hipError_t launch_persistent(const Params& P, int lds_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(mk_persistent, dim3(P.num_wgs), dim3(kThreads), lds_bytes, stream, P);
  return hipGetLastError();
}

hipError_t launch_stage(const Params& P, int s, int lds_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(mk_stage, dim3(P.num_wgs), dim3(kThreads), lds_bytes, stream, P, s);
  return hipGetLastError();
}

hipError_t launch_set_args(StepArgs* a, int pos, uint32_t epoch, hipStream_t stream) {
  hipLaunchKernelGGL(mk_set_args, dim3(1), dim3(1), 0, stream, a, pos, epoch);
  return hipGetLastError();
}

hipError_t launch_advance_args(StepArgs* a, hipStream_t stream) {
  hipLaunchKernelGGL(mk_advance_args, dim3(1), dim3(1), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mk
