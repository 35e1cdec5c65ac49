// mk_kernels.hip -- gfx950 load-time and step-argument kernels and the host
// launchers of the persistent decode megakernel and its one-stage-per-launch
// variant (the kernel templates are in mk_device.h, their instances in the
// builds of mk_inst.hip).
#include "mk_device.h"

namespace mk {

// Load-time repack for batched plans: source row r (< nsrc) of a bf16 matrix
// (row stride sstride elements, kcols columns) becomes row row0 + r * rstep
// of a tiled [rows][kp] matrix (16 x 32 tiles, 1 KiB each, in MFMA A-operand
// lane order); columns kcols..kp-1 are zero.  One thread per 8 columns.
__global__ void mk_tile_rows(const uint16_t* __restrict__ src, size_t sstride, int nsrc, int kcols,
                             uint16_t* __restrict__ dst, int kp, int row0, int rstep) {
  const int groups = kp / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)nsrc * groups) return;
  const int r = (int)(idx / groups), k = (int)(idx % groups) * 8;
  const int dr = row0 + r * rstep;
  const int lane = (dr % kTileRows) + kTileRows * ((k % kTileCols) / 8);
  const size_t tile = (size_t)(dr / kTileRows) * (kp / kTileCols) + (size_t)(k / kTileCols);
  uint4 v = {0u, 0u, 0u, 0u};
  if (k + 8 <= kcols) v = *reinterpret_cast<const uint4*>(src + (size_t)r * sstride + k);
  *reinterpret_cast<uint4*>(dst + (tile * 64 + lane) * 8) = v;
}

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

// Kernel instances, each defined in its own build of mk_inst.hip, named
// instance_<G>_<D>_<batched>_<GT>_<flags> (see run_stages).  Batch 1, head_dim
// 64: one attention variant per instance (GT = 1 or G), plain, with the
// partial-input down projection, or traced (both attention variants);
// head_dim 128: both variants; batched plans: plain or traced.
KernelPair instance_1_64_0_1_0();
KernelPair instance_2_64_0_1_0();
KernelPair instance_2_64_0_2_0();
KernelPair instance_4_64_0_1_0();
KernelPair instance_4_64_0_4_0();
KernelPair instance_1_64_0_1_2();
KernelPair instance_2_64_0_1_2();
KernelPair instance_2_64_0_2_2();
KernelPair instance_4_64_0_1_2();
KernelPair instance_4_64_0_4_2();
KernelPair instance_1_64_0_0_1();
KernelPair instance_2_64_0_0_1();
KernelPair instance_4_64_0_0_1();
KernelPair instance_1_128_0_0_0();
KernelPair instance_2_128_0_0_0();
KernelPair instance_4_128_0_0_0();
KernelPair instance_1_64_1_0_0();
KernelPair instance_2_64_1_0_0();
KernelPair instance_4_64_1_0_0();
KernelPair instance_1_64_1_0_1();
KernelPair instance_2_64_1_0_1();
KernelPair instance_4_64_1_0_1();

namespace {

// The instance for a plan: G query heads per kv head, head_dim D, batched or
// not, gt query heads per attention task, trace stamps, partial-input down
// projection.  {nullptr, nullptr} when no instance is built for the mix.
KernelPair kernels_for(int G, int D, bool batched, int gt, bool trace, bool partial) {
  const KernelPair none{nullptr, nullptr, nullptr};
  if (batched) {
    if (D != 64 || partial) return none;
    if (trace) return G == 1 ? instance_1_64_1_0_1() : G == 2 ? instance_2_64_1_0_1() : instance_4_64_1_0_1();
    return G == 1 ? instance_1_64_1_0_0() : G == 2 ? instance_2_64_1_0_0() : instance_4_64_1_0_0();
  }
  if (D == 128) {
    if (trace || partial) return none;
    return G == 1 ? instance_1_128_0_0_0() : G == 2 ? instance_2_128_0_0_0() : instance_4_128_0_0_0();
  }
  if (trace) {
    if (partial) return none;
    return G == 1 ? instance_1_64_0_0_1() : G == 2 ? instance_2_64_0_0_1() : instance_4_64_0_0_1();
  }
  const bool one = gt == 1;
  if (partial) {
    if (G == 1) return instance_1_64_0_1_2();
    if (G == 2) return one ? instance_2_64_0_1_2() : instance_2_64_0_2_2();
    return one ? instance_4_64_0_1_2() : instance_4_64_0_4_2();
  }
  if (G == 1) return instance_1_64_0_1_0();
  if (G == 2) return one ? instance_2_64_0_1_0() : instance_2_64_0_2_0();
  return one ? instance_4_64_0_1_0() : instance_4_64_0_4_0();
}

KernelPair kernels_of(const Params& P) {
  return kernels_for(P.G, P.D, P.B > 1, P.attn_gt, P.trace != nullptr, P.partial != 0);
}

}  // namespace

bool kernels_exist(int G, int D, bool batched, int gt, bool trace, bool partial) {
  return kernels_for(G, D, batched, gt, trace, partial).persistent != nullptr;
}

hipError_t configure_kernels(int G, int D, bool batched, int gt, bool trace, bool partial, int lds_bytes) {
  const KernelPair k = kernels_for(G, D, batched, gt, trace, partial);
  hipError_t e = hipFuncSetAttribute(k.persistent, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e == hipSuccess) e = hipFuncSetAttribute(k.stage, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e == hipSuccess) e = hipFuncSetAttribute(k.steps, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  return e;
}

hipError_t persistent_occupancy(int G, int D, bool batched, int gt, bool trace, bool partial, int lds_bytes,
                                int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks_per_cu, kernels_for(G, D, batched, gt, trace, partial).persistent, kThreads, lds_bytes);
}

hipError_t launch_persistent(const Params& P, int lds_bytes, hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&P)};
  return hipLaunchKernel(kernels_of(P).persistent, dim3(P.num_wgs), dim3(kThreads), args, lds_bytes, stream);
}

hipError_t launch_steps(const Params& P, int n_steps, int lds_bytes, hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&P), &n_steps};
  return hipLaunchKernel(kernels_of(P).steps, dim3(P.num_wgs), dim3(kThreads), args, lds_bytes, stream);
}

hipError_t launch_stage(const Params& P, int s, int lds_bytes, hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&P), &s};
  return hipLaunchKernel(kernels_of(P).stage, dim3(P.num_wgs), dim3(kThreads), args, lds_bytes, stream);
}

hipError_t launch_tile_rows(const uint16_t* src, size_t sstride, int nsrc, int kcols, uint16_t* dst, int kp, int row0,
                            int rstep) {
  const size_t n = (size_t)nsrc * (kp / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mk_tile_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, 0, src, sstride, nsrc, kcols, dst,
                     kp, row0, rstep);
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

