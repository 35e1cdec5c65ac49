// conv_kernels.hip -- the conventional decode path: one plain kernel launch
// per operation of the forward pass, the baseline the megakernel removes.
//
// The article "Revolution der KI-Beschleunigung: Wie ein Low-Latency
// Megakernel den Llama-1B Turbo zuendet" (dasgeld.co), paragraphs on the
// typical challenges and on mid-size models, and the glossary entry
// "Megakernel" (synthszr.com), section "Warum die Pausen zwischen den
// Rechenschritten teuer sind", describe the usual way a decode step runs: a
// long sequence of short kernels, each started by the host, with the GPU idle
// between them; streams and graphs only shorten those gaps.  This file is that
// usual way, written for gfx950 and independent of the megakernel (no shared
// kernels, helpers or layouts): per layer an RMSNorm kernel, separate Q, K and
// V GEMVs, a RoPE + KV-append kernel, split-KV attention and its merge, the O
// projection with the residual, an RMSNorm, separate gate and up GEMVs, the
// SiLU product, the down projection with the residual; then the final norm,
// the LM head and a two-kernel argmax.  Activations stay fp32 in a workspace.
//
// The position is read from device memory, so a captured hipGraph of one
// step replays at any position.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/mk.h"

namespace mkconv {

constexpr int kBlock = 256;      // threads of every kernel's block
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int kMaxBatch = 8;
constexpr int kMaxHeadDim = 128;
constexpr int kAttnChunk = 256;  // positions of one attention block (one thread each)
constexpr int kArgmaxBlocks = 256;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bf16 bits, round to nearest even; a NaN becomes a quiet NaN.
__device__ __forceinline__ uint16_t narrow(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float wave_reduce_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_reduce_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over the block (every thread gets it); red holds kWavesPerBlock floats.
__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
  v = wave_reduce_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  v = wave_reduce_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < kWavesPerBlock; ++i) t = fmaxf(t, red[i]);
  return t;
}

// Greedy-token key: a larger value gives a larger key, equal values order by
// the lower index; NaN is no candidate (key 0) and -0 is keyed as +0.
__device__ __forceinline__ uint64_t token_key(float v, int idx) {
  if (v != v) return 0;
  const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(~(uint32_t)idx);
}

__device__ __forceinline__ bool pos_ok(int pos, int S) { return pos >= 0 && pos < S; }

// ---------------------------------------------------------------------------
// kernels, one per operation
// ---------------------------------------------------------------------------

// x[b][i] = E[token_b][i]; a token outside [0, V) reads row 0 and marks tokerr[b].
__global__ void __launch_bounds__(kBlock) k_embed(const uint16_t* __restrict__ E, const int32_t* __restrict__ token,
                                                  int V, int H, float* __restrict__ x, int32_t* __restrict__ tokerr) {
  const int b = blockIdx.y;
  int tok = token[b];
  const bool bad = tok < 0 || tok >= V;
  if (bad) tok = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) tokerr[b] = bad ? 1 : 0;
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < H) x[(size_t)b * H + i] = widen(E[(size_t)tok * H + i]);
}

// y[b] = x[b] * (mean(x[b]^2) + eps)^(-1/2) * g, one block per sequence.
__global__ void __launch_bounds__(kBlock) k_rmsnorm(const float* __restrict__ x, const uint16_t* __restrict__ g,
                                                    float* __restrict__ y, int H, float eps) {
  __shared__ float red[kWavesPerBlock];
  const float* xb = x + (size_t)blockIdx.x * H;
  float* yb = y + (size_t)blockIdx.x * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += kBlock) ss = fmaf(xb[i], xb[i], ss);
  ss = block_reduce_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += kBlock) yb[i] = xb[i] * r * widen(g[i]);
}

// y[b][r] = res[b][r] (if res) + sum_k W[r][k] x[b][k] for rows r < rows and
// the NB sequences.  One wave per row, each lane 8 columns (one 16-byte weight
// load) at a time; the row sum is a wave reduction.  cols % 8 == 0 and W is
// 16-byte aligned (checked on the host).
template <int NB>
__global__ void __launch_bounds__(kBlock) k_gemv(const uint16_t* __restrict__ W, int rows, int cols,
                                                 const float* __restrict__ x, int xstride, float* y, int ystride,
                                                 const float* res) {
  const int r = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const uint16_t* wr = W + (size_t)r * cols;
  float acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = 0.f;
  for (int c = lane * 8; c < cols; c += 64 * 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(wr + c);
    const float wf[8] = {widen((uint16_t)(w.x & 0xffff)), widen((uint16_t)(w.x >> 16)),
                         widen((uint16_t)(w.y & 0xffff)), widen((uint16_t)(w.y >> 16)),
                         widen((uint16_t)(w.z & 0xffff)), widen((uint16_t)(w.z >> 16)),
                         widen((uint16_t)(w.w & 0xffff)), widen((uint16_t)(w.w >> 16))};
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const float4 a = *reinterpret_cast<const float4*>(x + (size_t)n * xstride + c);
      const float4 b = *reinterpret_cast<const float4*>(x + (size_t)n * xstride + c + 4);
      float s = acc[n];
      s = fmaf(wf[0], a.x, s);
      s = fmaf(wf[1], a.y, s);
      s = fmaf(wf[2], a.z, s);
      s = fmaf(wf[3], a.w, s);
      s = fmaf(wf[4], b.x, s);
      s = fmaf(wf[5], b.y, s);
      s = fmaf(wf[6], b.z, s);
      s = fmaf(wf[7], b.w, s);
      acc[n] = s;
    }
  }
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const float s = wave_reduce_sum(acc[n]);
    if (lane == 0) y[(size_t)n * ystride + r] = (res ? res[(size_t)n * ystride + r] : 0.f) + s;
  }
}

// Rotary embedding of q and k at position pos (pairs (2i, 2i+1) of every head,
// angle pos * theta^(-2i/D) evaluated in double), then the bf16 K and V rows
// appended at slot pos of the cache [B][L][NKV][S][D].  One thread per pair.
__global__ void __launch_bounds__(kBlock) k_rope_append(float* __restrict__ q, const float* __restrict__ k,
                                                        const float* __restrict__ v, const int32_t* __restrict__ d_pos,
                                                        uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int l,
                                                        int L, int NQ, int NKV, int D, int S, double theta) {
  const int pos = *d_pos;
  if (!pos_ok(pos, S)) return;
  const int b = blockIdx.y;
  const int half = D / 2;
  const int i = blockIdx.x * kBlock + threadIdx.x;
  const int nq = NQ * half, nk = NKV * half;
  if (i >= nq + 2 * nk) return;
  if (i < nq + nk) {
    const bool isq = i < nq;
    const int e = isq ? i : i - nq;
    const int head = e / half, j = e % half;
    const double ang = (double)pos * pow(theta, -2.0 * j / (double)D);
    const float cs = (float)cos(ang), sn = (float)sin(ang);
    if (isq) {
      float* p = q + (size_t)b * NQ * D + head * D + 2 * j;
      const float x0 = p[0], x1 = p[1];
      p[0] = x0 * cs - x1 * sn;
      p[1] = x0 * sn + x1 * cs;
    } else {
      const float* p = k + (size_t)b * NKV * D + head * D + 2 * j;
      const float x0 = p[0], x1 = p[1];
      uint16_t* dst = kc + ((((size_t)b * L + l) * NKV + head) * S + pos) * D + 2 * j;
      dst[0] = narrow(x0 * cs - x1 * sn);
      dst[1] = narrow(x0 * sn + x1 * cs);
    }
  } else {
    const int e = i - nq - nk;
    const int head = e / half, j = e % half;
    const float* p = v + (size_t)b * NKV * D + head * D + 2 * j;
    uint16_t* dst = vc + ((((size_t)b * L + l) * NKV + head) * S + pos) * D + 2 * j;
    dst[0] = narrow(p[0]);
    dst[1] = narrow(p[1]);
  }
}

// Split-KV decode attention, block (chunk c, query head h, sequence b): the
// positions [c * 256, min(pos + 1, c * 256 + 256)) of kv head h / (NQ / NKV)
// give the chunk's maximum score m, its sum l of exp(s - m) and its
// exp-weighted sum of V rows, written as {m, l, acc[D]} to part.  Chunks past
// pos return at once (the merge never reads them).
__global__ void __launch_bounds__(kBlock) k_attention(const float* __restrict__ q, const int32_t* __restrict__ d_pos,
                                                      const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                                                      float* __restrict__ part, int l, int L, int NQ, int NKV, int D,
                                                      int S, int C) {
  __shared__ float qs[kMaxHeadDim];
  __shared__ float p[kAttnChunk];
  __shared__ float red[kWavesPerBlock];
  __shared__ float accs[kBlock * 8];
  const int pos = *d_pos;
  if (!pos_ok(pos, S)) return;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = pos + 1;
  const int t0 = c * kAttnChunk;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + kAttnChunk);
  const int g = h / (NQ / NKV);
  const size_t head = (((size_t)b * L + l) * NKV + g) * S * D;
  const float scale = 1.0f / sqrtf((float)D);
  if (threadIdx.x < D) qs[threadIdx.x] = q[(size_t)b * NQ * D + h * D + threadIdx.x] * scale;
  __syncthreads();
  // one position per thread: its score
  const int t = t0 + threadIdx.x;
  float s = -INFINITY;
  if (t < t1) {
    const uint16_t* kr = kc + head + (size_t)t * D;
    float a = 0.f;
    for (int d = 0; d < D; d += 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(kr + d);
      a = fmaf(widen((uint16_t)(w.x & 0xffff)), qs[d + 0], a);
      a = fmaf(widen((uint16_t)(w.x >> 16)), qs[d + 1], a);
      a = fmaf(widen((uint16_t)(w.y & 0xffff)), qs[d + 2], a);
      a = fmaf(widen((uint16_t)(w.y >> 16)), qs[d + 3], a);
      a = fmaf(widen((uint16_t)(w.z & 0xffff)), qs[d + 4], a);
      a = fmaf(widen((uint16_t)(w.z >> 16)), qs[d + 5], a);
      a = fmaf(widen((uint16_t)(w.w & 0xffff)), qs[d + 6], a);
      a = fmaf(widen((uint16_t)(w.w >> 16)), qs[d + 7], a);
    }
    s = a;
  }
  const float m = block_reduce_max(s, red);
  const float e = t < t1 ? expf(s - m) : 0.f;
  p[threadIdx.x] = e;
  const float lsum = block_reduce_sum(e, red);  // its barriers also publish p
  // weighted V: thread = (8-dim group dg, position group tg)
  const int ngrp = D / 8;
  const int dg = threadIdx.x % ngrp, tg = threadIdx.x / ngrp, ntg = kBlock / ngrp;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int tt = t0 + tg; tt < t1; tt += ntg) {
    const uint4 w = *reinterpret_cast<const uint4*>(vc + head + (size_t)tt * D + dg * 8);
    const float pv = p[tt - t0];
    acc[0] = fmaf(pv, widen((uint16_t)(w.x & 0xffff)), acc[0]);
    acc[1] = fmaf(pv, widen((uint16_t)(w.x >> 16)), acc[1]);
    acc[2] = fmaf(pv, widen((uint16_t)(w.y & 0xffff)), acc[2]);
    acc[3] = fmaf(pv, widen((uint16_t)(w.y >> 16)), acc[3]);
    acc[4] = fmaf(pv, widen((uint16_t)(w.z & 0xffff)), acc[4]);
    acc[5] = fmaf(pv, widen((uint16_t)(w.z >> 16)), acc[5]);
    acc[6] = fmaf(pv, widen((uint16_t)(w.w & 0xffff)), acc[6]);
    acc[7] = fmaf(pv, widen((uint16_t)(w.w >> 16)), acc[7]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) accs[tg * D + dg * 8 + k] = acc[k];
  __syncthreads();
  float* out = part + ((((size_t)b * NQ) + h) * C + c) * (D + 2);
  if (threadIdx.x < D) {
    float a = 0.f;
    for (int k = 0; k < ntg; ++k) a += accs[k * D + threadIdx.x];
    out[2 + threadIdx.x] = a;
  }
  if (threadIdx.x == 0) {
    out[0] = m;
    out[1] = lsum;
  }
}

// o[b][h] = sum_c exp(m_c - M) acc_c / sum_c exp(m_c - M) l_c over the chunks
// of [0, pos], M the largest m_c.  Block (h, b), thread d < D.
__global__ void __launch_bounds__(kMaxHeadDim) k_attention_merge(const float* __restrict__ part,
                                                                 const int32_t* __restrict__ d_pos,
                                                                 float* __restrict__ o, int NQ, int D, int S, int C) {
  const int pos = *d_pos;
  if (!pos_ok(pos, S)) return;
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  if (d >= D) return;
  const int nc = (pos + 1 + kAttnChunk - 1) / kAttnChunk;
  const float* base = part + (((size_t)b * NQ) + h) * C * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[(size_t)c * (D + 2)]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float* pc = base + (size_t)c * (D + 2);
    const float e = expf(pc[0] - M);
    den = fmaf(e, pc[1], den);
    num = fmaf(e, pc[2 + d], num);
  }
  o[(size_t)b * NQ * D + h * D + d] = num / den;
}

// hid = silu(gate) * up, elementwise over the batch.
__global__ void __launch_bounds__(kBlock) k_silu_mul(const float* __restrict__ gate, const float* __restrict__ up,
                                                     float* __restrict__ hid, int n) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < n) {
    const float z = gate[i];
    hid[i] = z / (1.0f + expf(-z)) * up[i];
  }
}

// Greedy token, first stage: block (j, b) keys the largest logit (lowest index
// on ties) of its slice of [0, V).
__global__ void __launch_bounds__(kBlock) k_argmax_partial(const float* __restrict__ logits, int V,
                                                           uint64_t* __restrict__ keys) {
  __shared__ uint64_t red[kWavesPerBlock];
  const int j = blockIdx.x, b = blockIdx.y;
  const int per = (V + kArgmaxBlocks - 1) / kArgmaxBlocks;
  const int i0 = j * per, i1 = min(V, i0 + per);
  uint64_t k = 0;
  for (int i = i0 + threadIdx.x; i < i1; i += kBlock) {
    const uint64_t kk = token_key(logits[(size_t)b * V + i], i);
    k = kk > k ? kk : k;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = __shfl_xor(k, o);
    k = y > k ? y : k;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = red[0];
    for (int w = 1; w < kWavesPerBlock; ++w) t = red[w] > t ? red[w] : t;
    keys[(size_t)b * kArgmaxBlocks + j] = t;
  }
}

// Second stage: the largest key of the sequence's blocks gives out_token
// (-1 for a bad input token or when no logit is a number).
__global__ void __launch_bounds__(kBlock) k_argmax_final(const uint64_t* __restrict__ keys,
                                                         const int32_t* __restrict__ tokerr,
                                                         int32_t* __restrict__ out_token) {
  __shared__ uint64_t red[kWavesPerBlock];
  const int b = blockIdx.x;
  uint64_t k = 0;
  for (int j = threadIdx.x; j < kArgmaxBlocks; j += kBlock) {
    const uint64_t kk = keys[(size_t)b * kArgmaxBlocks + j];
    k = kk > k ? kk : k;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = __shfl_xor(k, o);
    k = y > k ? y : k;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = red[0];
    for (int w = 1; w < kWavesPerBlock; ++w) t = red[w] > t ? red[w] : t;
    out_token[b] = (t == 0 || tokerr[b]) ? -1 : (int32_t)(~(uint32_t)t);
  }
}

__global__ void k_set_pos(int32_t* d_pos, int pos) { *d_pos = pos; }
__global__ void k_advance_pos(int32_t* d_pos) { *d_pos += 1; }

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct Dims {
  int L, H, NQ, NKV, D, QD, KVD, F, V, S, B, C;
  float eps;
  double theta;
  bool tied;
};

// Workspace layout (bytes from the base, 256-byte aligned pieces).
struct Layout {
  size_t x, xn, q, k, v, att, gate, up, hid, part, keys, tokerr, bytes;
};

size_t take(size_t& cur, size_t bytes) {
  const size_t at = cur;
  cur = (cur + bytes + 255) / 256 * 256;
  return at;
}

int dims_of(const mk_config* c, Dims* d) {
  if (!c) return MK_E_INVAL;
  if (c->n_layers < 0 || c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->ffn <= 0 || c->vocab <= 0 || c->max_seq <= 0 || c->batch <= 0)
    return MK_E_INVAL;
  if (c->n_heads % c->n_kv_heads != 0 || c->head_dim % 8 != 0 || c->hidden % 8 != 0 || c->ffn % 8 != 0)
    return MK_E_INVAL;
  if (!(c->rms_eps >= 0.0f) || !(c->rope_theta > 0.0)) return MK_E_INVAL;
  if (c->head_dim > kMaxHeadDim || c->batch > kMaxBatch) return MK_E_UNSUPPORTED;
  // the attention block splits its threads into (8-dim group, position group) pairs
  if (kBlock % (c->head_dim / 8) != 0) return MK_E_UNSUPPORTED;
  d->L = c->n_layers;
  d->H = c->hidden;
  d->NQ = c->n_heads;
  d->NKV = c->n_kv_heads;
  d->D = c->head_dim;
  d->QD = c->n_heads * c->head_dim;
  d->KVD = c->n_kv_heads * c->head_dim;
  d->F = c->ffn;
  d->V = c->vocab;
  d->S = c->max_seq;
  d->B = c->batch;
  d->C = (c->max_seq + kAttnChunk - 1) / kAttnChunk;
  d->eps = c->rms_eps;
  d->theta = c->rope_theta;
  d->tied = c->tie_embeddings != 0;
  return MK_OK;
}

Layout layout_of(const Dims& d) {
  Layout w{};
  size_t cur = 0;
  const size_t B = d.B;
  w.x = take(cur, B * d.H * 4);
  w.xn = take(cur, B * d.H * 4);
  w.q = take(cur, B * d.QD * 4);
  w.k = take(cur, B * d.KVD * 4);
  w.v = take(cur, B * d.KVD * 4);
  w.att = take(cur, B * d.QD * 4);
  w.gate = take(cur, B * d.F * 4);
  w.up = take(cur, B * d.F * 4);
  w.hid = take(cur, B * d.F * 4);
  w.part = take(cur, B * d.NQ * (size_t)d.C * (d.D + 2) * 4);
  w.keys = take(cur, B * kArgmaxBlocks * 8);
  w.tokerr = take(cur, B * 4);
  w.bytes = cur;
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_weights(const Dims& d, const mk_weights* w) {
  if (!w || !w->embed || !w->final_norm) return MK_E_INVAL;
  if (d.tied != (w->lm_head == nullptr)) return MK_E_INVAL;
  if (d.L > 0 && !w->layers) return MK_E_INVAL;
  if (!aligned16(d.tied ? w->embed : w->lm_head)) return MK_E_INVAL;
  for (int l = 0; l < d.L; ++l) {
    const mk_layer_weights& lw = w->layers[l];
    if (!lw.attn_norm || !lw.ffn_norm) return MK_E_INVAL;
    const void* m[7] = {lw.wq, lw.wk, lw.wv, lw.wo, lw.w_gate, lw.w_up, lw.w_down};
    for (const void* p : m)
      if (!p || !aligned16(p)) return MK_E_INVAL;
  }
  return MK_OK;
}

hipError_t gemv(const uint16_t* W, int rows, int cols, const float* x, int xstride, float* y, int ystride,
                const float* res, int B, hipStream_t s) {
  const dim3 grid((unsigned)((rows + kWavesPerBlock - 1) / kWavesPerBlock));
  switch (B) {
    case 1: hipLaunchKernelGGL(k_gemv<1>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
    case 2: hipLaunchKernelGGL(k_gemv<2>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
    case 3: hipLaunchKernelGGL(k_gemv<3>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
    case 4: hipLaunchKernelGGL(k_gemv<4>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
    case 5: hipLaunchKernelGGL(k_gemv<5>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
    case 6: hipLaunchKernelGGL(k_gemv<6>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
    case 7: hipLaunchKernelGGL(k_gemv<7>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
    default: hipLaunchKernelGGL(k_gemv<8>, grid, dim3(kBlock), 0, s, W, rows, cols, x, xstride, y, ystride, res); break;
  }
  return hipGetLastError();
}

// The launches of one decode step.  Every pointer has been checked.
int run_step(const Dims& d, const mk_weights* w, const int32_t* d_token, const int32_t* d_pos, const mk_kv* kv,
             float* logits, int32_t* out_token, char* ws, hipStream_t s) {
  const Layout lo = layout_of(d);
  float* x = reinterpret_cast<float*>(ws + lo.x);
  float* xn = reinterpret_cast<float*>(ws + lo.xn);
  float* q = reinterpret_cast<float*>(ws + lo.q);
  float* k = reinterpret_cast<float*>(ws + lo.k);
  float* v = reinterpret_cast<float*>(ws + lo.v);
  float* att = reinterpret_cast<float*>(ws + lo.att);
  float* gate = reinterpret_cast<float*>(ws + lo.gate);
  float* up = reinterpret_cast<float*>(ws + lo.up);
  float* hid = reinterpret_cast<float*>(ws + lo.hid);
  float* part = reinterpret_cast<float*>(ws + lo.part);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + lo.keys);
  int32_t* tokerr = reinterpret_cast<int32_t*>(ws + lo.tokerr);
  const int B = d.B;
  auto blocks = [](size_t n) { return (unsigned)((n + kBlock - 1) / kBlock); };
  hipLaunchKernelGGL(k_embed, dim3(blocks(d.H), B), dim3(kBlock), 0, s, w->embed, d_token, d.V, d.H, x, tokerr);
  for (int l = 0; l < d.L; ++l) {
    const mk_layer_weights& lw = w->layers[l];
    hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(kBlock), 0, s, x, lw.attn_norm, xn, d.H, d.eps);
    if (gemv(lw.wq, d.QD, d.H, xn, d.H, q, d.QD, nullptr, B, s) != hipSuccess) return MK_E_HIP;
    if (gemv(lw.wk, d.KVD, d.H, xn, d.H, k, d.KVD, nullptr, B, s) != hipSuccess) return MK_E_HIP;
    if (gemv(lw.wv, d.KVD, d.H, xn, d.H, v, d.KVD, nullptr, B, s) != hipSuccess) return MK_E_HIP;
    hipLaunchKernelGGL(k_rope_append, dim3(blocks((size_t)(d.NQ + 2 * d.NKV) * d.D / 2), B), dim3(kBlock), 0, s, q,
                       k, v, d_pos, kv->k, kv->v, l, d.L, d.NQ, d.NKV, d.D, d.S, d.theta);
    hipLaunchKernelGGL(k_attention, dim3(d.C, d.NQ, B), dim3(kBlock), 0, s, q, d_pos, kv->k, kv->v, part, l, d.L,
                       d.NQ, d.NKV, d.D, d.S, d.C);
    hipLaunchKernelGGL(k_attention_merge, dim3(d.NQ, B), dim3(kMaxHeadDim), 0, s, part, d_pos, att, d.NQ, d.D, d.S,
                       d.C);
    if (gemv(lw.wo, d.H, d.QD, att, d.QD, x, d.H, x, B, s) != hipSuccess) return MK_E_HIP;
    hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(kBlock), 0, s, x, lw.ffn_norm, xn, d.H, d.eps);
    if (gemv(lw.w_gate, d.F, d.H, xn, d.H, gate, d.F, nullptr, B, s) != hipSuccess) return MK_E_HIP;
    if (gemv(lw.w_up, d.F, d.H, xn, d.H, up, d.F, nullptr, B, s) != hipSuccess) return MK_E_HIP;
    hipLaunchKernelGGL(k_silu_mul, dim3(blocks((size_t)B * d.F)), dim3(kBlock), 0, s, gate, up, hid, B * d.F);
    if (gemv(lw.w_down, d.H, d.F, hid, d.F, x, d.H, x, B, s) != hipSuccess) return MK_E_HIP;
  }
  hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(kBlock), 0, s, x, w->final_norm, xn, d.H, d.eps);
  if (gemv(d.tied ? w->embed : w->lm_head, d.V, d.H, xn, d.H, logits, d.V, nullptr, B, s) != hipSuccess)
    return MK_E_HIP;
  hipLaunchKernelGGL(k_argmax_partial, dim3(kArgmaxBlocks, B), dim3(kBlock), 0, s, logits, d.V, keys);
  hipLaunchKernelGGL(k_argmax_final, dim3(B), dim3(kBlock), 0, s, keys, tokerr, out_token);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_E_HIP;
}

int check_step_args(const Dims& d, const int32_t* d_token, const int32_t* d_pos, const mk_kv* kv, const float* logits,
                    const int32_t* out_token) {
  if (!d_token || !d_pos || !kv || !logits || !out_token) return MK_E_INVAL;
  if (d.L > 0 && (!kv->k || !kv->v)) return MK_E_INVAL;
  if (((uintptr_t)kv->k | (uintptr_t)kv->v) & 15u) return MK_E_INVAL;  // 16-byte K/V row reads
  if (((uintptr_t)logits | (uintptr_t)out_token | (uintptr_t)d_token | (uintptr_t)d_pos) & 3u) return MK_E_INVAL;
  return MK_OK;
}

// ---------------------------------------------------------------------------
// the allocation-free variant: a fixed device buffer instead of a workspace
// ---------------------------------------------------------------------------

// Workspace of mk_conv_decode_step_static.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code this name is only a
// stand-in for the symbol: the device address of a GPU's copy comes from
// hipGetSymbolAddress with that GPU current (static_scratch below), and only
// that address is ever handed to a kernel.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch, looked up once per device.
int static_scratch(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return MK_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return MK_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return MK_E_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return MK_OK;
}

}  // namespace mkconv

// ---------------------------------------------------------------------------
// launchers used by the library's handle modes (mk_api.cpp)
// ---------------------------------------------------------------------------

namespace mk {
hipError_t conv_launch_set_pos(int32_t* d_pos, int pos, hipStream_t s) {
  hipLaunchKernelGGL(mkconv::k_set_pos, dim3(1), dim3(1), 0, s, d_pos, pos);
  return hipGetLastError();
}
hipError_t conv_launch_advance_pos(int32_t* d_pos, hipStream_t s) {
  hipLaunchKernelGGL(mkconv::k_advance_pos, dim3(1), dim3(1), 0, s, d_pos);
  return hipGetLastError();
}
}  // namespace mk

extern "C" {

int mk_conv_workspace_size(const mk_config* cfg, size_t* bytes) {
  mkconv::Dims d{};
  if (!bytes) return MK_E_INVAL;
  const int rc = mkconv::dims_of(cfg, &d);
  if (rc != MK_OK) return rc;
  *bytes = mkconv::layout_of(d).bytes;
  return MK_OK;
}

int mk_conv_decode_step(const mk_config* cfg, const mk_weights* w, const int32_t* d_token, const int32_t* d_pos,
                        const mk_kv* kv, float* out_logits, int32_t* out_token, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  mkconv::Dims d{};
  int rc = mkconv::dims_of(cfg, &d);
  if (rc != MK_OK) return rc;
  if ((rc = mkconv::check_weights(d, w)) != MK_OK) return rc;
  if ((rc = mkconv::check_step_args(d, d_token, d_pos, kv, out_logits, out_token)) != MK_OK) return rc;
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < mkconv::layout_of(d).bytes) return MK_E_INVAL;
  return mkconv::run_step(d, w, d_token, d_pos, kv, out_logits, out_token, static_cast<char*>(workspace), stream);
}

int mk_conv_decode_step_static(const mk_config* cfg, const mk_weights* w, const int32_t* d_token,
                               const int32_t* d_pos, const mk_kv* kv, float* out_logits, int32_t* out_token,
                               hipStream_t stream) {
  mkconv::Dims d{};
  int rc = mkconv::dims_of(cfg, &d);
  if (rc != MK_OK) return rc;
  if ((rc = mkconv::check_weights(d, w)) != MK_OK) return rc;
  if ((rc = mkconv::check_step_args(d, d_token, d_pos, kv, out_logits, out_token)) != MK_OK) return rc;
  if (mkconv::layout_of(d).bytes > mkconv::kStaticScratchBytes) return MK_E_TOOBIG;
  char* ws = nullptr;
  if ((rc = mkconv::static_scratch(&ws)) != MK_OK) return rc;
  // every workspace element a step reads was written earlier in the same
  // step, so nothing left by a previous call needs clearing
  return mkconv::run_step(d, w, d_token, d_pos, kv, out_logits, out_token, ws, stream);
}

}  // extern "C"
