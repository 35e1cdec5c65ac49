// mk_api.cpp -- the C ABI (include/mk.h): load, decode step, reset, status.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"
#include "mk_plan.h"

namespace mk {
hipError_t configure_kernels(int G, int D, bool batched, int gt, bool trace, bool partial, int lds_bytes);
bool kernels_exist(int G, int D, bool batched, int gt, bool trace, bool partial);
hipError_t launch_tile_rows(const uint16_t* src, size_t sstride, int nsrc, int kcols, uint16_t* dst, int kp, int row0,
                            int rstep);
hipError_t persistent_occupancy(int G, int D, bool batched, int gt, bool trace, bool partial, int lds_bytes,
                                int* blocks_per_cu);
hipError_t launch_persistent(const Params& P, int lds_bytes, hipStream_t stream);
hipError_t launch_stage(const Params& P, int s, int lds_bytes, hipStream_t stream);
hipError_t launch_steps(const Params& P, int n_steps, int lds_bytes, hipStream_t stream);
hipError_t launch_set_args(StepArgs* a, int pos, uint32_t epoch, hipStream_t stream);
hipError_t launch_advance_args(StepArgs* a, hipStream_t stream);
hipError_t conv_launch_set_pos(int32_t* d_pos, int pos, hipStream_t s);
hipError_t conv_launch_advance_pos(int32_t* d_pos, hipStream_t s);
}  // namespace mk

using mk::Params;
using mk::Plan;
using mk::Workspace;
using mk::layout_workspace;

namespace {

// Step tags restart (with a workspace clear) before epoch * tasks-per-stage could wrap a u32.
constexpr uint32_t kEpochLimit = 1u << 20;

}  // namespace

struct mk_handle {
  mk_config cfg{};
  Plan plan;
  int device = 0;
  char* arena = nullptr;
  char* lm_copy = nullptr;
  const char* lm = nullptr;
  const uint16_t* embed = nullptr;
  float* gains = nullptr;  // g_attn [L][Hp] | g_ffn [L][Hp] | g_final [Hp]
  float* rope = nullptr;
  mk::Task* tape = nullptr;
  char* ws = nullptr;
  uint64_t* trace = nullptr;  // [W][stages][4] when cfg.trace
  int clock_khz = 0;
  Workspace wl{};
  mk::DevStatus* status_host = nullptr;     // pinned, host-mapped
  mk::DevStatus* status_host_dev = nullptr; // its device address
  hipStream_t capture_stream = nullptr;
  hipStream_t last_stream = nullptr;
  bool used = false;
  uint32_t epoch = 0;
  uint64_t watchdog_ticks = 0;
  // graph mode
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  const void* g_ptrs[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  int shadow_pos = -1;
  uint32_t shadow_epoch = 0;
  // conventional modes: the caller's weights (layers copied), fp32 workspace, device position
  bool conv = false;
  mk_weights conv_w{};
  std::vector<mk_layer_weights> conv_layers;
  char* conv_ws = nullptr;
  size_t conv_ws_bytes = 0;
  int32_t* conv_pos = nullptr;
  // logits of multi-step calls made without an output buffer: [batch][vocab]
  float* logits_scratch = nullptr;
};

namespace {

void release(mk_handle* h) {
  if (!h) return;
  if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  if (h->capture_stream) (void)hipStreamDestroy(h->capture_stream);
  if (h->arena) (void)hipFree(h->arena);
  if (h->lm_copy) (void)hipFree(h->lm_copy);
  if (h->gains) (void)hipFree(h->gains);
  if (h->rope) (void)hipFree(h->rope);
  if (h->tape) (void)hipFree(h->tape);
  if (h->ws) (void)hipFree(h->ws);
  if (h->trace) (void)hipFree(h->trace);
  if (h->conv_ws) (void)hipFree(h->conv_ws);
  if (h->conv_pos) (void)hipFree(h->conv_pos);
  if (h->logits_scratch) (void)hipFree(h->logits_scratch);
  if (h->status_host) (void)hipHostFree(h->status_host);
  delete h;
}

Params make_params(mk_handle* h) {
  const Plan& p = h->plan;
  Params P{};
  P.tape = h->tape;
  P.num_wgs = p.W;
  P.num_stages = p.stages;
  P.L = p.L; P.H = p.H; P.Hp = p.Hp; P.QD = p.QD; P.QDp = p.QDp; P.KVD = p.KVD;
  P.F = p.F; P.Fp = p.Fp; P.V = p.V; P.NQ = p.NQ; P.NKV = p.NKV; P.D = p.D; P.G = p.G; P.S = p.S; P.B = p.B;
  P.eps = h->cfg.rms_eps;
  P.qscale = (float)(1.0 / std::sqrt((double)p.D));
  P.attn_chunks = p.C;
  P.attn_gt = p.G / p.attn_slices;
  P.arena = h->arena;
  P.lm = h->lm;
  P.embed = h->embed;
  P.g_attn = h->gains;
  P.g_ffn = h->gains + (size_t)p.L * p.Hp;
  P.g_final = h->gains + 2 * (size_t)p.L * p.Hp;
  P.rope = h->rope;
  char* ws = h->ws;
  const Workspace& w = h->wl;
  P.x_attn = reinterpret_cast<uint32_t*>(ws + w.x_attn.off);
  P.x_ffn = reinterpret_cast<uint32_t*>(ws + w.x_ffn.off);
  P.q = reinterpret_cast<uint32_t*>(ws + w.q.off);
  P.kvcur = reinterpret_cast<uint32_t*>(ws + w.kvcur.off);
  P.o = reinterpret_cast<uint32_t*>(ws + w.o.off);
  P.h = reinterpret_cast<uint32_t*>(ws + w.h.off);
  P.kpart = reinterpret_cast<uint32_t*>(ws + w.kpart.off);
  P.attn_part = reinterpret_cast<float*>(ws + w.attn_part.off);
  P.attn_ctr = reinterpret_cast<uint32_t*>(ws + w.attn_ctr.off);
  P.amax = reinterpret_cast<uint64_t*>(ws + w.amax.off);
  P.amax_ctr = reinterpret_cast<uint32_t*>(ws + w.amax_ctr.off);
  P.tokerr = reinterpret_cast<uint32_t*>(ws + w.tokerr.off);
  P.abort_flag = reinterpret_cast<uint32_t*>(ws + w.abort_flag.off);
  P.status = reinterpret_cast<mk::DevStatus*>(ws + w.status.off);
  P.status_host = h->status_host_dev;
  P.lds_act = p.lds_act;
  P.lds_res = p.lds_res;
  P.lds_rope = p.lds_rope;
  P.lds_misc = p.lds_misc;
  P.lds_part = p.lds_part;
  P.lds_tape = p.lds_tape;
  P.act_stride = p.act_stride;
  P.act_floats = p.act_floats;
  P.res_floats = p.res_floats;
  P.watchdog_ticks = h->watchdog_ticks;
  P.trace = h->trace;
  P.partial = p.partial ? 1 : 0;
  P.prefill = p.prefill ? 1 : 0;
  return P;
}

#define HIP_OR(call)                  \
  do {                                \
    if ((call) != hipSuccess) {       \
      (void)hipGetLastError();        \
      release(h);                     \
      return MK_E_HIP;                \
    }                                 \
  } while (0)

// bf16 gains (device) -> fp32 zero-padded rows (host staging)
bool widen_gain(const uint16_t* dsrc, int n, float* hdst) {
  std::vector<uint16_t> tmp(n);
  if (hipMemcpy(tmp.data(), dsrc, (size_t)n * 2, hipMemcpyDeviceToHost) != hipSuccess) return false;
  for (int i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)tmp[i] << 16;
    std::memcpy(&hdst[i], &u, 4);
  }
  return true;
}

int clear_workspace(mk_handle* h, hipStream_t s) {
  if (hipMemsetAsync(h->ws, 0, h->wl.bytes, s) != hipSuccess) return MK_E_HIP;
  return MK_OK;
}

int capture_graph(mk_handle* h, const Params& base) {
  if (h->gexec) { (void)hipGraphExecDestroy(h->gexec); h->gexec = nullptr; }
  if (h->graph) { (void)hipGraphDestroy(h->graph); h->graph = nullptr; }
  Params P = base;
  P.dargs = reinterpret_cast<mk::StepArgs*>(h->ws + h->wl.dargs.off);
  hipStream_t cs = h->capture_stream;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) return MK_E_HIP;
  bool ok = true;
  for (int s = 0; s < h->plan.stages && ok; ++s) ok = mk::launch_stage(P, s, h->plan.lds_bytes, cs) == hipSuccess;
  if (ok) ok = mk::launch_advance_args(const_cast<mk::StepArgs*>(P.dargs), cs) == hipSuccess;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(cs, &g);
  if (!ok || e != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    (void)hipGetLastError();
    return MK_E_HIP;
  }
  if (hipGraphInstantiate(&h->gexec, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    h->gexec = nullptr;
    return MK_E_HIP;
  }
  h->graph = g;
  h->shadow_pos = -1;
  return MK_OK;
}

// Conventional hipGraph mode: one step of per-operation launches plus the
// position advance, captured once and replayed.
int capture_conv_graph(mk_handle* h, const int32_t* d_token, const mk_kv* kv, float* logits, int32_t* tok) {
  if (h->gexec) { (void)hipGraphExecDestroy(h->gexec); h->gexec = nullptr; }
  if (h->graph) { (void)hipGraphDestroy(h->graph); h->graph = nullptr; }
  hipStream_t cs = h->capture_stream;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) return MK_E_HIP;
  int rc = mk_conv_decode_step(&h->cfg, &h->conv_w, d_token, h->conv_pos, kv, logits, tok, h->conv_ws,
                               h->conv_ws_bytes, cs);
  bool ok = rc == MK_OK && mk::conv_launch_advance_pos(h->conv_pos, cs) == hipSuccess;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(cs, &g);
  if (!ok || e != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    (void)hipGetLastError();
    return rc != MK_OK ? rc : MK_E_HIP;
  }
  if (hipGraphInstantiate(&h->gexec, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    h->gexec = nullptr;
    return MK_E_HIP;
  }
  h->graph = g;
  h->shadow_pos = -1;
  return MK_OK;
}

// mk_load for MK_MODE_CONV / MK_MODE_CONV_GRAPH: no plan and no repack; the
// caller's weights are read in place by the per-operation kernels.
int load_conv(const mk_config* cfg, const mk_weights* w, mk_handle** out) {
  if (cfg->prefill) return MK_E_UNSUPPORTED;
  size_t bytes = 0;
  int rc = mk_conv_workspace_size(cfg, &bytes);
  if (rc != MK_OK) return rc;
  if (!w->embed || !w->final_norm || (cfg->n_layers > 0 && !w->layers)) return MK_E_INVAL;
  mk_handle* h = new (std::nothrow) mk_handle();
  if (!h) return MK_E_NOMEM;
  h->cfg = *cfg;
  h->conv = true;
  h->conv_layers.assign(w->layers, w->layers + cfg->n_layers);
  h->conv_w = *w;
  h->conv_w.layers = h->conv_layers.data();
  HIP_OR(hipGetDevice(&h->device));
  if (hipMalloc(&h->conv_ws, bytes) != hipSuccess) { (void)hipGetLastError(); release(h); return MK_E_NOMEM; }
  h->conv_ws_bytes = bytes;
  HIP_OR(hipMalloc(&h->conv_pos, 256));
  HIP_OR(hipMemset(h->conv_pos, 0, 256));
  HIP_OR(hipHostMalloc(reinterpret_cast<void**>(&h->status_host), sizeof(mk::DevStatus), hipHostMallocMapped));
  std::memset(h->status_host, 0, sizeof(mk::DevStatus));
  HIP_OR(hipStreamCreateWithFlags(&h->capture_stream, hipStreamNonBlocking));
  HIP_OR(hipMalloc(&h->logits_scratch, (size_t)cfg->batch * cfg->vocab * 4));
  HIP_OR(hipDeviceSynchronize());
  *out = h;
  return MK_OK;
}

int decode_conv(mk_handle* h, const int32_t* d_token, int32_t pos, const mk_kv* kv, float* logits, int32_t* tok,
                hipStream_t stream) {
  if (pos < 0 || pos >= h->cfg.max_seq) return MK_E_RANGE;
  int rc = MK_OK;
  if (h->cfg.exec_mode == MK_MODE_CONV) {
    if (mk::conv_launch_set_pos(h->conv_pos, pos, stream) != hipSuccess) return MK_E_HIP;
    rc = mk_conv_decode_step(&h->cfg, &h->conv_w, d_token, h->conv_pos, kv, logits, tok, h->conv_ws,
                             h->conv_ws_bytes, stream);
  } else {
    const void* ptrs[5] = {d_token, kv->k, kv->v, logits, tok};
    if (!h->gexec || std::memcmp(ptrs, h->g_ptrs, sizeof(ptrs)) != 0) {
      if ((rc = capture_conv_graph(h, d_token, kv, logits, tok)) != MK_OK) return rc;
      std::memcpy(h->g_ptrs, ptrs, sizeof(ptrs));
    }
    hipError_t e = hipSuccess;
    if (h->shadow_pos != pos) e = mk::conv_launch_set_pos(h->conv_pos, pos, stream);
    if (e == hipSuccess) e = hipGraphLaunch(h->gexec, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return MK_E_HIP;
    }
    h->shadow_pos = pos + 1;
  }
  if (rc == MK_OK) {
    h->last_stream = stream;
    h->used = true;
  }
  return rc;
}

}  // namespace

extern "C" {

const char* mk_error_string(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_E_INVAL: return "invalid argument";
    case MK_E_RANGE: return "position out of range";
    case MK_E_HIP: return "HIP runtime error";
    case MK_E_STATE: return "a device error is latched (see mk_status; call mk_reset)";
    case MK_E_TIMEOUT: return "dependency wait exceeded the watchdog budget";
    case MK_E_TOKEN: return "input token id out of range";
    case MK_E_NOMEM: return "out of memory";
    case MK_E_UNSUPPORTED: return "configuration not supported";
    case MK_E_DEVICE: return "device cannot host the persistent launch";
    case MK_E_TOOBIG: return "the step needs a larger workspace than the static scratch buffer";
    default: return "unknown error";
  }
}

int mk_plan_describe(const mk_config* cfg, int32_t num_wgs, mk_plan_info* out) {
  if (!cfg || !out) return MK_E_INVAL;
  Plan p;
  int rc = mk::plan_build(*cfg, num_wgs > 0 ? num_wgs : 256, p);
  if (rc != MK_OK) return rc;
  std::string why;
  rc = mk::plan_validate(p, &why);
  if (rc != MK_OK) return rc;
  std::memset(out, 0, sizeof(*out));
  out->num_wgs = p.W;
  out->num_stages = p.stages;
  out->num_tasks = p.num_tasks;
  out->attn_chunks = p.C;
  out->weight_bytes = (int64_t)(p.arena_bytes + p.lm_bytes);
  out->workspace_bytes = (int64_t)layout_workspace(p).bytes + (int64_t)p.tape.size() * 32;
  out->lds_bytes = p.lds_bytes;
  out->ring_units = p.ring_units;
  return MK_OK;
}

int mk_load(const mk_config* cfg, const mk_weights* w, mk_handle** out) {
  if (out) *out = nullptr;
  if (!cfg || !w || !out || !w->embed || !w->final_norm) return MK_E_INVAL;
  if (cfg->exec_mode == MK_MODE_CONV || cfg->exec_mode == MK_MODE_CONV_GRAPH) return load_conv(cfg, w, out);
  if ((cfg->tie_embeddings != 0) != (w->lm_head == nullptr)) return MK_E_INVAL;
  if (cfg->n_layers > 0 && !w->layers) return MK_E_INVAL;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const mk_layer_weights& lw = w->layers[l];
    if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.ffn_norm || !lw.w_gate || !lw.w_up || !lw.w_down)
      return MK_E_INVAL;
  }
  mk_handle* h = new (std::nothrow) mk_handle();
  if (!h) return MK_E_NOMEM;
  h->cfg = *cfg;
  HIP_OR(hipGetDevice(&h->device));
  hipDeviceProp_t prop;
  HIP_OR(hipGetDeviceProperties(&prop, h->device));
  const int ncu = prop.multiProcessorCount;
  const int W = cfg->num_wgs > 0 ? cfg->num_wgs : ncu;
  if (W > ncu) { release(h); return MK_E_DEVICE; }
  int rc = mk::plan_build(*cfg, W, h->plan);
  if (rc != MK_OK) { release(h); return rc; }
  std::string why;
  if (mk::plan_validate(h->plan, &why) != MK_OK) { release(h); return MK_E_INVAL; }
  const Plan& p = h->plan;
  // Plans outside the envelope that has run on the GPU are refused: the
  // first run of a shape with head_dim 128, hidden 4096 and a 14 GB weight
  // arena (32 layers) ended in a GPU memory fault whose cause is not found
  // yet; the host-side address walk of that plan finds every index in
  // bounds.  So head_dim 128, hidden > 2048 and packed weights of 4 GiB or
  // more are refused until the cause is known.  Such plans still build and
  // validate on the host.
  if (p.D != 64 || p.H > 2048 || p.arena_bytes + p.lm_bytes >= (4ull << 30)) {
    release(h);
    return MK_E_UNSUPPORTED;
  }
  // the kernels' rings are kRing (batch 1) or kRingBatched units deep
  if (p.ring_units != (p.batched ? mk::kRingBatched : mk::kRing)) {
    release(h);
    return MK_E_UNSUPPORTED;
  }

  // persistent residency: one workgroup per compute unit must fit
  const int gt = p.G / p.attn_slices;
  if (!mk::kernels_exist(p.G, p.D, p.batched, gt, cfg->trace != 0, p.partial)) {
    release(h);
    return MK_E_UNSUPPORTED;
  }
  HIP_OR(mk::configure_kernels(p.G, p.D, p.batched, gt, cfg->trace != 0, p.partial, p.lds_bytes));
  int per_cu = 0;
  HIP_OR(mk::persistent_occupancy(p.G, p.D, p.batched, gt, cfg->trace != 0, p.partial, p.lds_bytes, &per_cu));
  if (per_cu < 1) { release(h); return MK_E_DEVICE; }

  // packed weights
  if (hipMalloc(&h->arena, p.arena_bytes) != hipSuccess) { (void)hipGetLastError(); release(h); return MK_E_NOMEM; }
  HIP_OR(hipMemset(h->arena, 0, p.arena_bytes));
  const size_t H2 = (size_t)p.H * 2, Hp2 = (size_t)p.Hp * 2;
  if (p.batched) {
    // tiled matrices (16 x 32 tiles in MFMA A-operand lane order); rows are
    // read 16 bytes at a time, so every source must be 16-byte aligned
    auto aligned = [](const void* q) { return ((uintptr_t)q & 15u) == 0; };
    for (int l = 0; l < p.L; ++l) {
      const mk_layer_weights& lw = w->layers[l];
      if (!aligned(lw.wq) || !aligned(lw.wk) || !aligned(lw.wv) || !aligned(lw.wo) || !aligned(lw.w_gate) ||
          !aligned(lw.w_up) || !aligned(lw.w_down)) {
        release(h);
        return MK_E_INVAL;
      }
    }
    const uint16_t* lm_src = p.tied ? w->embed : w->lm_head;
    if (!aligned(lm_src)) { release(h); return MK_E_INVAL; }
    uint16_t* A = reinterpret_cast<uint16_t*>(h->arena);
    for (int l = 0; l < p.L; ++l) {
      const mk_layer_weights& lw = w->layers[l];
      uint16_t* q = A + p.off_qkv[l] / 2;
      HIP_OR(mk::launch_tile_rows(lw.wq, p.H, p.QD, p.H, q, p.Hp, 0, 1));
      HIP_OR(mk::launch_tile_rows(lw.wk, p.H, p.KVD, p.H, q, p.Hp, p.QD, 1));
      HIP_OR(mk::launch_tile_rows(lw.wv, p.H, p.KVD, p.H, q, p.Hp, p.QD + p.KVD, 1));
      HIP_OR(mk::launch_tile_rows(lw.wo, p.QD, p.H, p.QD, A + p.off_o[l] / 2, p.QDp, 0, 1));
      HIP_OR(mk::launch_tile_rows(lw.w_gate, p.H, p.F, p.H, A + p.off_gu[l] / 2, p.Hp, 0, 2));
      HIP_OR(mk::launch_tile_rows(lw.w_up, p.H, p.F, p.H, A + p.off_gu[l] / 2, p.Hp, 1, 2));
      HIP_OR(mk::launch_tile_rows(lw.w_down, p.F, p.H, p.F, A + p.off_down[l] / 2, p.Fp, 0, 1));
    }
    if (hipMalloc(&h->lm_copy, p.lm_bytes) != hipSuccess) { (void)hipGetLastError(); release(h); return MK_E_NOMEM; }
    HIP_OR(mk::launch_tile_rows(lm_src, p.H, p.V, p.H, reinterpret_cast<uint16_t*>(h->lm_copy), p.Hp, 0, 1));
    h->lm = h->lm_copy;
  }
  for (int l = 0; l < p.L && !p.batched; ++l) {
    const mk_layer_weights& lw = w->layers[l];
    char* q = h->arena + p.off_qkv[l];
    HIP_OR(hipMemcpy2D(q, Hp2, lw.wq, H2, H2, p.QD, hipMemcpyDeviceToDevice));
    HIP_OR(hipMemcpy2D(q + (size_t)p.QD * Hp2, Hp2, lw.wk, H2, H2, p.KVD, hipMemcpyDeviceToDevice));
    HIP_OR(hipMemcpy2D(q + (size_t)(p.QD + p.KVD) * Hp2, Hp2, lw.wv, H2, H2, p.KVD, hipMemcpyDeviceToDevice));
    HIP_OR(hipMemcpy2D(h->arena + p.off_o[l], (size_t)p.QDp * 2, lw.wo, (size_t)p.QD * 2, (size_t)p.QD * 2, p.H,
                       hipMemcpyDeviceToDevice));
    // gate row f -> packed row 2f, up row f -> packed row 2f+1
    HIP_OR(hipMemcpy2D(h->arena + p.off_gu[l], 2 * Hp2, lw.w_gate, H2, H2, p.F, hipMemcpyDeviceToDevice));
    HIP_OR(hipMemcpy2D(h->arena + p.off_gu[l] + Hp2, 2 * Hp2, lw.w_up, H2, H2, p.F, hipMemcpyDeviceToDevice));
    HIP_OR(hipMemcpy2D(h->arena + p.off_down[l], (size_t)p.Fp * 2, lw.w_down, (size_t)p.F * 2, (size_t)p.F * 2, p.H,
                       hipMemcpyDeviceToDevice));
  }
  const uint16_t* lm_src = p.tied ? w->embed : w->lm_head;
  if (p.batched) {
    // tiled above
  } else if (p.lm_borrowed) {
    h->lm = reinterpret_cast<const char*>(lm_src);
  } else {
    if (hipMalloc(&h->lm_copy, p.lm_bytes) != hipSuccess) { (void)hipGetLastError(); release(h); return MK_E_NOMEM; }
    HIP_OR(hipMemset(h->lm_copy, 0, p.lm_bytes));
    HIP_OR(hipMemcpy2D(h->lm_copy, Hp2, lm_src, H2, H2, p.V, hipMemcpyDeviceToDevice));
    h->lm = h->lm_copy;
  }
  h->embed = w->embed;

  // norm gains as fp32, zero-padded to Hp
  {
    std::vector<float> g((size_t)(2 * p.L + 1) * p.Hp, 0.f);
    for (int l = 0; l < p.L; ++l) {
      if (!widen_gain(w->layers[l].attn_norm, p.H, &g[(size_t)l * p.Hp]) ||
          !widen_gain(w->layers[l].ffn_norm, p.H, &g[(size_t)(p.L + l) * p.Hp])) {
        release(h);
        return MK_E_HIP;
      }
    }
    if (!widen_gain(w->final_norm, p.H, &g[(size_t)2 * p.L * p.Hp])) { release(h); return MK_E_HIP; }
    HIP_OR(hipMalloc(&h->gains, g.size() * 4));
    HIP_OR(hipMemcpy(h->gains, g.data(), g.size() * 4, hipMemcpyHostToDevice));
  }

  // RoPE table: angle p * theta^(-2i/d_h) and its cos/sin in double, stored as float
  {
    std::vector<float> t((size_t)p.S * p.D);
    for (int pos = 0; pos < p.S; ++pos)
      for (int i = 0; i < p.D / 2; ++i) {
        const double ang = (double)pos * std::pow(cfg->rope_theta, -2.0 * i / (double)p.D);
        t[(size_t)pos * p.D + 2 * i] = (float)std::cos(ang);
        t[(size_t)pos * p.D + 2 * i + 1] = (float)std::sin(ang);
      }
    HIP_OR(hipMalloc(&h->rope, t.size() * 4));
    HIP_OR(hipMemcpy(h->rope, t.data(), t.size() * 4, hipMemcpyHostToDevice));
  }

  // tape
  HIP_OR(hipMalloc(&h->tape, p.tape.size() * sizeof(mk::Task)));
  HIP_OR(hipMemcpy(h->tape, p.tape.data(), p.tape.size() * sizeof(mk::Task), hipMemcpyHostToDevice));

  // workspace
  h->wl = layout_workspace(p);
  if (hipMalloc(&h->ws, h->wl.bytes) != hipSuccess) { (void)hipGetLastError(); release(h); return MK_E_NOMEM; }
  HIP_OR(hipMemset(h->ws, 0, h->wl.bytes));

  // status mirror in pinned host memory mapped into the device
  HIP_OR(hipHostMalloc(reinterpret_cast<void**>(&h->status_host), sizeof(mk::DevStatus), hipHostMallocMapped));
  std::memset(h->status_host, 0, sizeof(mk::DevStatus));
  HIP_OR(hipHostGetDevicePointer(reinterpret_cast<void**>(&h->status_host_dev), h->status_host, 0));

  HIP_OR(hipStreamCreateWithFlags(&h->capture_stream, hipStreamNonBlocking));
  HIP_OR(hipMalloc(&h->logits_scratch, (size_t)p.B * p.V * 4));
  if (cfg->trace) {
    const size_t tb = (size_t)p.W * p.stages * mk::kTraceStamps * sizeof(uint64_t);
    HIP_OR(hipMalloc(&h->trace, tb));
    HIP_OR(hipMemset(h->trace, 0, tb));
  }
  int wclk_khz = 0;
  HIP_OR(hipDeviceGetAttribute(&wclk_khz, hipDeviceAttributeWallClockRate, h->device));
  h->clock_khz = wclk_khz > 0 ? wclk_khz : 100000;
  if (cfg->watchdog_ms < 0) {
    // a budget of -watchdog_ms device clock ticks: lets tests drive the timeout path
    h->watchdog_ticks = (uint64_t)(-(int64_t)cfg->watchdog_ms);
  } else {
    const uint64_t ms = cfg->watchdog_ms > 0 ? (uint64_t)cfg->watchdog_ms : 2000ull;
    h->watchdog_ticks = (uint64_t)(wclk_khz > 0 ? wclk_khz : 100000) * ms;
  }
  HIP_OR(hipDeviceSynchronize());
  *out = h;
  return MK_OK;
}

int mk_decode_step(mk_handle* h, const int32_t* d_token, int32_t pos, const mk_kv* kv, float* out_logits,
                   int32_t* out_token, hipStream_t stream) {
  if (!h || !d_token || !kv || !out_logits || !out_token) return MK_E_INVAL;
  if (h->plan.L > 0 && (!kv->k || !kv->v)) return MK_E_INVAL;  // a 0-layer model has no cache
  if ((reinterpret_cast<uintptr_t>(kv->k) | reinterpret_cast<uintptr_t>(kv->v)) & 3u) return MK_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(out_logits) | reinterpret_cast<uintptr_t>(out_token) |
       reinterpret_cast<uintptr_t>(d_token)) & 3u)
    return MK_E_INVAL;
  if (h->conv) return decode_conv(h, d_token, pos, kv, out_logits, out_token, stream);
  // prefill: the call covers positions pos .. pos + B - 1
  if (pos < 0 || (int64_t)pos + (h->plan.prefill ? h->plan.B : 1) > h->plan.S) return MK_E_RANGE;
  if (reinterpret_cast<volatile int32_t*>(&h->status_host->code)[0] != MK_OK) return MK_E_STATE;
  if (h->epoch + 1 >= kEpochLimit) {
    if (clear_workspace(h, stream) != MK_OK) return MK_E_HIP;
    h->epoch = 0;
    h->shadow_pos = -1;
  }
  const uint32_t epoch = ++h->epoch;
  Params P = make_params(h);
  P.token = d_token;
  P.kcache = kv->k;
  P.vcache = kv->v;
  P.logits = out_logits;
  P.out_token = out_token;
  P.pos = pos;
  P.epoch = epoch;
  hipError_t e = hipSuccess;
  switch (h->cfg.exec_mode) {
    case MK_MODE_MEGA:
      e = mk::launch_persistent(P, h->plan.lds_bytes, stream);
      break;
    case MK_MODE_MULTI:
      for (int s = 0; s < h->plan.stages && e == hipSuccess; ++s) e = mk::launch_stage(P, s, h->plan.lds_bytes, stream);
      break;
    case MK_MODE_GRAPH: {
      const void* ptrs[5] = {d_token, kv->k, kv->v, out_logits, out_token};
      if (!h->gexec || std::memcmp(ptrs, h->g_ptrs, sizeof(ptrs)) != 0) {
        if (capture_graph(h, P) != MK_OK) return MK_E_HIP;
        std::memcpy(h->g_ptrs, ptrs, sizeof(ptrs));
      }
      auto* dargs = reinterpret_cast<mk::StepArgs*>(h->ws + h->wl.dargs.off);
      if (h->shadow_pos != pos || h->shadow_epoch != epoch) e = mk::launch_set_args(dargs, pos, epoch, stream);
      if (e == hipSuccess) e = hipGraphLaunch(h->gexec, stream);
      h->shadow_pos = pos + 1;
      h->shadow_epoch = epoch + 1;
      break;
    }
    default:
      return MK_E_INVAL;
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MK_E_HIP;
  }
  h->last_stream = stream;
  h->used = true;
  return MK_OK;
}

int mk_decode_steps(mk_handle* h, const int32_t* d_token, int32_t pos, int32_t n_steps, const mk_kv* kv,
                    float* out_logits, int32_t* out_tokens, hipStream_t stream) {
  if (!h || !d_token || !kv || !out_tokens || n_steps < 1) return MK_E_INVAL;
  if (!h->conv && h->plan.prefill) return MK_E_UNSUPPORTED;  // a prefill handle runs one call per chunk
  const int B = h->cfg.batch, V = h->cfg.vocab;
  if (pos < 0 || (int64_t)pos + n_steps > (int64_t)h->cfg.max_seq) return MK_E_RANGE;
  if (h->conv || h->cfg.exec_mode != MK_MODE_MEGA) {
    // every other mode: one step at a time, the tokens chained on the device
    for (int i = 0; i < n_steps; ++i) {
      const int32_t* tin = i == 0 ? d_token : out_tokens + (size_t)(i - 1) * B;
      float* lg = out_logits ? out_logits + (size_t)i * B * V : h->logits_scratch;
      const int rc = mk_decode_step(h, tin, pos + i, kv, lg, out_tokens + (size_t)i * B, stream);
      if (rc != MK_OK) return rc;
    }
    return MK_OK;
  }
  if (h->plan.L > 0 && (!kv->k || !kv->v)) return MK_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(kv->k) | reinterpret_cast<uintptr_t>(kv->v)) & 3u) return MK_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(out_logits) | reinterpret_cast<uintptr_t>(out_tokens) |
       reinterpret_cast<uintptr_t>(d_token)) & 3u)
    return MK_E_INVAL;
  if (reinterpret_cast<volatile int32_t*>(&h->status_host->code)[0] != MK_OK) return MK_E_STATE;
  if ((uint64_t)h->epoch + (uint64_t)n_steps + 1 >= kEpochLimit) {
    if (clear_workspace(h, stream) != MK_OK) return MK_E_HIP;
    h->epoch = 0;
    h->shadow_pos = -1;
  }
  Params P = make_params(h);
  P.token = d_token;
  P.kcache = kv->k;
  P.vcache = kv->v;
  P.logits = out_logits ? out_logits : h->logits_scratch;
  P.logits_step = out_logits ? (int64_t)B * V : 0;
  P.out_token = out_tokens;
  P.pos = pos;
  P.epoch = h->epoch + 1;
  P.tok_tag = reinterpret_cast<uint64_t*>(h->ws + h->wl.tok_tag.off);
  h->epoch += (uint32_t)n_steps;
  if (mk::launch_steps(P, n_steps, h->plan.lds_bytes, stream) != hipSuccess) {
    (void)hipGetLastError();
    return MK_E_HIP;
  }
  h->last_stream = stream;
  h->used = true;
  return MK_OK;
}

int mk_reset(mk_handle* h) {
  if (!h) return MK_E_INVAL;
  // wait for the handle's own work only: the last stream a step ran on
  if (h->used && hipStreamSynchronize(h->last_stream) != hipSuccess) {
    (void)hipGetLastError();
    return MK_E_HIP;
  }
  if (h->conv) {  // no dependency state: the workspace is rewritten by every step
    h->shadow_pos = -1;
    return MK_OK;
  }
  // the clear runs on the capture stream (never captured) and is waited for
  if (hipMemsetAsync(h->ws, 0, h->wl.bytes, h->capture_stream) != hipSuccess ||
      hipStreamSynchronize(h->capture_stream) != hipSuccess) {
    (void)hipGetLastError();
    return MK_E_HIP;
  }
  std::memset(h->status_host, 0, sizeof(mk::DevStatus));
  h->epoch = 0;
  h->shadow_pos = -1;
  return MK_OK;
}

void mk_free(mk_handle* h) {
  if (!h) return;
  (void)hipDeviceSynchronize();
  release(h);
}

int mk_trace_copy(mk_handle* h, uint64_t* out, int64_t capacity_words, int64_t* words_written, int32_t* clock_khz) {
  if (!h || !out || !h->trace) return MK_E_INVAL;
  const int64_t n = (int64_t)h->plan.W * h->plan.stages * mk::kTraceStamps;
  if (capacity_words < n) return MK_E_INVAL;
  if (hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    return MK_E_HIP;
  }
  if (hipMemcpy(out, h->trace, (size_t)n * sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess) return MK_E_HIP;
  if (words_written) *words_written = n;
  if (clock_khz) *clock_khz = h->clock_khz;
  return MK_OK;
}

int mk_status(mk_handle* h, mk_status_t* out) {
  if (!h || !out) return MK_E_INVAL;
  volatile mk::DevStatus* s = h->status_host;
  out->code = s->code;
  out->stage = s->stage;
  out->wg = s->wg;
  out->detail = s->detail;
  return MK_OK;
}

}  // extern "C"
