// w2a8.hip -- gfx950 W2A8 matrix-vector product: ternary weights stored in
// two bits, int8 activations, after the page "BitNet 1.58bit GPU Inference
// Kernel: Revolutionaere Effizienz fuer KI-Modelle mit W2A8-Quantisierung"
// (dasgeld.co, body): weights of three values packed 16 to a 32-bit word so
// that one shift and one mask expose four of them as bytes, and the products
// formed by 4-wide int8 dot products (v_dot4_i32_i8 on CDNA).
//
//   quantize:  s = 127 / max(max_k |x_k|, 1e-5),  q_k = clamp(rint(x_k s), -128, 127)
//   gemv:      y_r = (float(sum_k Q_rk q_k) * gamma_r) / s
//
// Packed layout (mk_w2a8_pack): row r is cols / 16 words; word w holds the
// codes c = Q + 1 (0, 1, 2) of columns 16 w .. 16 w + 15, column
// 16 w + 4 k + m at bits 8 m + 2 k .. 8 m + 2 k + 1.  So (word >> 2k) &
// 0x03030303 holds columns 16 w + 4 k .. + 3 as four bytes, in the byte order
// of the four int8 activation codes of those columns read as one 32-bit word,
// and sum_k Q_rk q_k = sum_k c_rk q_k - sum_k q_k.
//
// The GEMV streams each row once: lane l of a wave reads 16 bytes (64
// columns) per 4096-column chunk j, columns 4096 j + 64 l .. + 63, and keeps
// the int8 activation codes of those columns in registers for all its rows;
// per row the lane sums 16 dot4 products per chunk, subtracts the sum of its
// activation codes, and the wave adds the 64 lane sums (integers: the order
// does not change the result).  It is bound by HBM bandwidth: rows * cols / 4
// bytes of weights per call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>

#include "../../include/mk.h"

namespace {

constexpr int kGemvThreads = 256;           // 4 waves
constexpr int kChunkCols = 4096;             // columns one wave-wide 16-byte load covers
constexpr int kMaxCols = 4 * kChunkCols;     // activation codes of 4 chunks stay in registers
constexpr int kQuantThreads = 1024;

// Wave64 integer sum: DPP within rows of 16 lanes, then the four row totals.
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// 16 packed codes (one word) against the 16 activation codes of their columns.
__device__ __forceinline__ int dot16(uint32_t w, const uint4 x, int acc) {
  acc = __builtin_amdgcn_sdot4((int)(w & 0x03030303u), (int)x.x, acc, false);
  acc = __builtin_amdgcn_sdot4((int)((w >> 2) & 0x03030303u), (int)x.y, acc, false);
  acc = __builtin_amdgcn_sdot4((int)((w >> 4) & 0x03030303u), (int)x.z, acc, false);
  acc = __builtin_amdgcn_sdot4((int)((w >> 6) & 0x03030303u), (int)x.w, acc, false);
  return acc;
}

// The int8 code of x * s: rounded half to even, clamped to [-128, 127].
__device__ __forceinline__ uint32_t code_byte(float v, float s) {
  const float q = fminf(fmaxf(rintf(v * s), -128.f), 127.f);
  return (uint32_t)(int)q & 0xFFu;
}

// Loads of the U rows from r0, every lane and row unconditionally (so that
// the compiler's wait counts stay exact): rows past the end read the last
// row, and lanes past the end of a row read its first 64 columns; their
// activation codes are zero, so they add nothing, and rows past the end are
// not stored.
template <int J, int U>
__device__ __forceinline__ void load_rows(uint4 (&wv)[U][J], const uint4* __restrict__ w, int r0, int rows, size_t row16,
                                          const int (&col16)[J]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = r0 + u < rows ? r0 + u : rows - 1;
#pragma unroll
    for (int j = 0; j < J; ++j) wv[u][j] = w[(size_t)r * row16 + col16[j]];
  }
}

// The U rows' lane sums (the activation-code sum already subtracted), added
// over the wave; lane u < U stores row r0 + u.
template <int J, int U>
__device__ __forceinline__ void finish_rows(const uint4 (&wv)[U][J], const uint4 (&xa)[J][4], int xsum, int r0, int rows,
                                            float g, float s, float* __restrict__ y, int lane) {
  int tot[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int acc = -xsum;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      acc = dot16(wv[u][j].x, xa[j][0], acc);
      acc = dot16(wv[u][j].y, xa[j][1], acc);
      acc = dot16(wv[u][j].z, xa[j][2], acc);
      acc = dot16(wv[u][j].w, xa[j][3], acc);
    }
    tot[u] = wave_sum_i32(acc);
  }
  int t = tot[0];
#pragma unroll
  for (int u = 1; u < U; ++u) t = lane == u ? tot[u] : t;
  const int r = r0 + lane;
  if (lane < U && r < rows) y[r] = ((float)t * g) / s;
}

// y[r] for every row; J chunks of 4096 columns (the last one may be partial).
// The workgroup first puts the activation codes of the whole vector into LDS:
// FUSED, it quantises the float32 input x itself (the largest |x| over the
// vector, then every code), so that one launch does the whole product;
// otherwise it copies the codes xq of mk_w2a8_quantize.  Both give the same
// codes and scale.  Each lane then keeps the codes of its own columns in
// registers, and every wave takes U rows at a time: U * J 16-byte loads per
// lane, one wait, the dot products, U wave sums.  Latency is hidden by the
// other waves of the compute unit.
template <int J, int U, bool FUSED>
__global__ void __launch_bounds__(kGemvThreads) w2a8_gemv_kernel(const uint4* __restrict__ w, const float* __restrict__ gamma,
                                                                  const int8_t* __restrict__ xq,
                                                                  const float* __restrict__ scale,
                                                                  const float* __restrict__ x, float* __restrict__ y,
                                                                  int rows, int cols) {
  __shared__ float red[kGemvThreads / 64];
  __shared__ __attribute__((aligned(16))) uint32_t codes[kMaxCols / 4];
  const int lane = (int)threadIdx.x & 63;
  const int tid = (int)threadIdx.x;
  const int gwave = (int)blockIdx.x * (kGemvThreads / 64) + (tid >> 6);
  const int nwaves = (int)gridDim.x * (kGemvThreads / 64);
  const size_t row16 = (size_t)cols / 64;  // 16-byte groups per packed row
  int col16[J];
  bool live[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    live[j] = j * kChunkCols + 64 * lane < cols;
    col16[j] = live[j] ? j * 64 + lane : 0;
  }

  // the activation codes into LDS (straight-line loads, the last group of
  // the vector read again by threads past its end)
  float s;
  if constexpr (FUSED) {
    float4 xv[4 * J];
#pragma unroll
    for (int k = 0; k < 4 * J; ++k) {
      const int i = tid * 4 + k * kGemvThreads * 4;
      xv[k] = *reinterpret_cast<const float4*>(x + (i < cols ? i : cols - 4));
    }
    float m = 0.f;  // max is exact and order-free
#pragma unroll
    for (int k = 0; k < 4 * J; ++k)
      m = fmaxf(fmaxf(m, fmaxf(fabsf(xv[k].x), fabsf(xv[k].y))), fmaxf(fabsf(xv[k].z), fabsf(xv[k].w)));
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) red[tid >> 6] = m;
    __syncthreads();
    m = 0.f;
#pragma unroll
    for (int k = 0; k < kGemvThreads / 64; ++k) m = fmaxf(m, red[k]);
    s = 127.0f / fmaxf(m, 1e-5f);
#pragma unroll
    for (int k = 0; k < 4 * J; ++k) {
      const int i = tid * 4 + k * kGemvThreads * 4;
      if (i < cols)
        codes[i / 4] = code_byte(xv[k].x, s) | (code_byte(xv[k].y, s) << 8) | (code_byte(xv[k].z, s) << 16) |
                       (code_byte(xv[k].w, s) << 24);
    }
  } else {
    uint4 cv[J];
#pragma unroll
    for (int k = 0; k < J; ++k) {
      const int i = tid * 16 + k * kGemvThreads * 16;
      cv[k] = *reinterpret_cast<const uint4*>(xq + (i < cols ? i : cols - 16));
    }
    s = *scale;
#pragma unroll
    for (int k = 0; k < J; ++k) {
      const int i = tid * 16 + k * kGemvThreads * 16;
      if (i < cols) *reinterpret_cast<uint4*>(&codes[i / 4]) = cv[k];
    }
  }
  __syncthreads();
  uint4 xa[J][4];
  int xsum = 0;
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xa[j][q] = live[j] ? *reinterpret_cast<const uint4*>(&codes[(j * kChunkCols + 64 * lane + 16 * q) / 4])
                         : uint4{0u, 0u, 0u, 0u};
      xsum = __builtin_amdgcn_sdot4((int)xa[j][q].x, 0x01010101, xsum, false);
      xsum = __builtin_amdgcn_sdot4((int)xa[j][q].y, 0x01010101, xsum, false);
      xsum = __builtin_amdgcn_sdot4((int)xa[j][q].z, 0x01010101, xsum, false);
      xsum = __builtin_amdgcn_sdot4((int)xa[j][q].w, 0x01010101, xsum, false);
    }

  // the row scales of a pass are read one pass ahead, so that they are in
  // flight with the weights instead of waited for after the dot products
  const int stride = nwaves * U;
  int r0 = gwave * U;
  float g = gamma[r0 + lane % U < rows ? r0 + lane % U : rows - 1];
  for (; r0 < rows; r0 += stride) {
    const int rn = r0 + stride + lane % U;
    const float gn = gamma[rn < rows ? rn : rows - 1];
    uint4 wv[U][J];
    load_rows<J, U>(wv, w, r0, rows, row16, col16);
    __builtin_amdgcn_sched_barrier(0);  // every load of the pass before the first use
    finish_rows<J, U>(wv, xa, xsum, r0, rows, g, s, y, lane);
    g = gn;
  }
}

// Outputs of a product over zero columns: (0 * gamma_r) / s.
__global__ void w2a8_no_cols_kernel(const float* __restrict__ gamma, const float* __restrict__ scale, float* __restrict__ y,
                                    int rows) {
  const int r = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const float s = scale ? *scale : 127.0f / 1e-5f;
  if (r < rows) y[r] = (0.0f * gamma[r]) / s;
}

// One workgroup: the largest |x|, the scale, the codes.
__global__ void __launch_bounds__(kQuantThreads) w2a8_quantize_kernel(const float* __restrict__ x, int cols,
                                                                       int8_t* __restrict__ xq, float* __restrict__ scale) {
  __shared__ float red[kQuantThreads / 64];
  float m = 0.f;
  for (int i = (int)threadIdx.x; i < cols; i += kQuantThreads) m = fmaxf(m, fabsf(x[i]));
  // max is exact and order-free
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0.f;
#pragma unroll
  for (int k = 0; k < kQuantThreads / 64; ++k) m = fmaxf(m, red[k]);
  const float s = 127.0f / fmaxf(m, 1e-5f);
  for (int i = (int)threadIdx.x; i < cols; i += kQuantThreads) xq[i] = (int8_t)code_byte(x[i], s);
  if (threadIdx.x == 0) *scale = s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int mk_w2a8_pack(const int8_t* codes, int rows, int cols, uint32_t* packed) {
  if (rows < 0 || cols < 0 || cols % 64 != 0) return MK_E_INVAL;
  if ((size_t)rows * cols > 0 && (!codes || !packed)) return MK_E_INVAL;
  const int words = cols / 16;
  for (int r = 0; r < rows; ++r)
    for (int wd = 0; wd < words; ++wd) {
      uint32_t v = 0;
      for (int k = 0; k < 4; ++k)
        for (int m = 0; m < 4; ++m) {
          const int c = codes[(size_t)r * cols + 16 * wd + 4 * k + m];
          if (c < -1 || c > 1) return MK_E_INVAL;
          v |= (uint32_t)(c + 1) << (8 * m + 2 * k);
        }
      packed[(size_t)r * words + wd] = v;
    }
  return MK_OK;
}

extern "C" int mk_w2a8_quantize(const float* d_x, int cols, int8_t* d_xq, float* d_scale, hipStream_t stream) {
  if (cols < 0 || cols > kMaxCols || cols % 64 != 0 || !d_scale) return MK_E_INVAL;
  if (cols > 0 && (!d_x || !d_xq)) return MK_E_INVAL;
  hipLaunchKernelGGL(w2a8_quantize_kernel, dim3(1), dim3(kQuantThreads), 0, stream, d_x, cols, d_xq, d_scale);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_E_HIP;
}

namespace {

#ifndef MK_W2A8_MAX_BLOCKS
#define MK_W2A8_MAX_BLOCKS 512
#endif

int launch_gemv(bool fused, const uint32_t* d_packed, const float* d_gamma, int rows, int cols, const int8_t* d_xq,
                const float* d_scale, const float* d_x, float* d_y, hipStream_t stream) {
  if (cols == 0) {
    hipLaunchKernelGGL(w2a8_no_cols_kernel, dim3((rows + 255) / 256), dim3(256), 0, stream, d_gamma,
                       fused ? nullptr : d_scale, d_y, rows);
    return hipGetLastError() == hipSuccess ? MK_OK : MK_E_HIP;
  }
  // U rows per wave and pass: 8 while the lane's loads stay few (one or two
  // column chunks), else 4; one pass per wave while that needs at most
  // MK_W2A8_MAX_BLOCKS workgroups, several passes beyond
  const int J = (cols + kChunkCols - 1) / kChunkCols;
  const int U = J <= 2 ? 8 : 4;
  const int waves_needed = (rows + U - 1) / U;
  const int per_block = kGemvThreads / 64;
  int blocks = (waves_needed + per_block - 1) / per_block;
  if (blocks > MK_W2A8_MAX_BLOCKS) blocks = MK_W2A8_MAX_BLOCKS;
  const uint4* w = reinterpret_cast<const uint4*>(d_packed);
  const dim3 g(blocks), b(kGemvThreads);
#define MK_W2A8_LAUNCH(JJ, UU)                                                                                     \
  do {                                                                                                            \
    if (fused)                                                                                                    \
      hipLaunchKernelGGL((w2a8_gemv_kernel<JJ, UU, true>), g, b, 0, stream, w, d_gamma, d_xq, d_scale, d_x, d_y, \
                         rows, cols);                                                                             \
    else                                                                                                          \
      hipLaunchKernelGGL((w2a8_gemv_kernel<JJ, UU, false>), g, b, 0, stream, w, d_gamma, d_xq, d_scale, d_x, d_y, \
                         rows, cols);                                                                             \
  } while (0)
  switch (J) {
    case 1: MK_W2A8_LAUNCH(1, 8); break;
    case 2: MK_W2A8_LAUNCH(2, 8); break;
    case 3: MK_W2A8_LAUNCH(3, 4); break;
    default: MK_W2A8_LAUNCH(4, 4); break;
  }
#undef MK_W2A8_LAUNCH
  (void)U;
  return hipGetLastError() == hipSuccess ? MK_OK : MK_E_HIP;
}

}  // namespace

extern "C" int mk_w2a8_gemv(const uint32_t* d_packed, const float* d_gamma, int rows, int cols, const int8_t* d_xq,
                            const float* d_scale, float* d_y, hipStream_t stream) {
  if (rows < 0 || cols < 0 || cols > kMaxCols || cols % 64 != 0) return MK_E_INVAL;
  if (rows == 0) return MK_OK;
  if (!d_gamma || !d_scale || !d_y) return MK_E_INVAL;
  if (cols > 0 && (!d_packed || !d_xq || !aligned16(d_packed) || !aligned16(d_xq))) return MK_E_INVAL;
  return launch_gemv(false, d_packed, d_gamma, rows, cols, d_xq, d_scale, nullptr, d_y, stream);
}

extern "C" int mk_w2a8_linear(const uint32_t* d_packed, const float* d_gamma, int rows, int cols, const float* d_x,
                              float* d_y, hipStream_t stream) {
  if (rows < 0 || cols < 0 || cols > kMaxCols || cols % 64 != 0) return MK_E_INVAL;
  if (rows == 0) return MK_OK;
  if (!d_gamma || !d_y) return MK_E_INVAL;
  if (cols > 0 && (!d_packed || !d_x || !aligned16(d_packed) || !aligned16(d_x))) return MK_E_INVAL;
  return launch_gemv(true, d_packed, d_gamma, rows, cols, nullptr, nullptr, d_x, d_y, stream);
}
