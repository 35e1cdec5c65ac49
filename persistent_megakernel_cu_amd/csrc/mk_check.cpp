// mk_check.cpp -- host-side address walk of a batch-1 megakernel plan.
//
// Replays every task of a plan's tape, for one decode position, through the
// index helpers of mk_addr.h that the kernels themselves use, and checks each
// global index against the size of the buffer it falls in (the packed weight
// arena or LM head, the embedding, gains, RoPE table, KV caches, the
// workspace buffers as laid out by layout_workspace, the logits) and each LDS
// index against the plan's LDS regions.  The loops follow the kernel's
// (which waves take which items, which threads stage which words); the index
// arithmetic is the kernel's own.  Test support: built into its own library
// (libmkcheck.so), never linked into libmk.
#include "mk_check.h"

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>

#include "mk_addr.h"
#include "mk_plan.h"

namespace mk {
namespace {

struct Walker {
  const Plan& p;
  int pos;
  int64_t slack;  // elements (or bytes, for weights) added to every limit: < 0 tightens the check
  uint64_t checks = 0, violations = 0;
  std::string first;
  int cur_stage = -1, cur_wg = -1;

  Walker(const Plan& plan, int position, int64_t sl) : p(plan), pos(position), slack(sl) {}

  // [idx, idx + count) must lie inside [0, limit)
  void in(const char* what, uint64_t idx, uint64_t count, uint64_t limit) {
    ++checks;
    const int64_t lim = (int64_t)limit + slack;
    if ((int64_t)(idx + count) > lim) fail(what, idx + count, limit);
  }
  void fail(const char* what, uint64_t end, uint64_t limit) {
    ++violations;
    if (first.empty()) {
      char b[256];
      std::snprintf(b, sizeof b, "stage %d wg %d: %s ends at %llu, limit %llu", cur_stage, cur_wg, what,
                    (unsigned long long)end, (unsigned long long)limit);
      first = b;
    }
  }
  void rule(bool ok, const char* what) {
    ++checks;
    if (!ok) fail(what, 0, 0);
  }
};

// Every element the staging of a plain tagged vector of n words reads and
// writes (stage_tagged / stage_normed: groups of 4 per thread, 512 threads).
void walk_staging(Walker& w, const char* what, uint64_t src_off, uint64_t src_limit, int n, int npad,
                  uint64_t gain_off = ~0ull, uint64_t gain_limit = 0) {
  const int per_round = 4 * kThreads * 4;
  for (int i0 = 0; i0 == 0 || i0 < n; i0 += per_round)
    for (int j = 0; j < 4; ++j)
      for (int tid = 0; tid < kThreads; ++tid) {
        const int i = i0 + 4 * (j * kThreads + tid);
        if (gain_off != ~0ull) w.in("gain", gain_off + (i < n ? i : n - 4), 4, gain_limit);
        if (i < n) {
          w.in(what, src_off + i, 4, src_limit);
          w.in("LDS activation", i, 4, w.p.act_floats);
        }
      }
  w.in("LDS activation (zero pad)", 0, npad, w.p.act_floats);
}

void walk_gemv(Walker& w, const Task& t, const Workspace& ws, uint64_t region_bytes) {
  const Plan& p = w.p;
  const int l = t.layer;
  const int L = p.L, V = p.V;
  const uint64_t gains = (uint64_t)(2 * L + 1) * p.Hp;
  const uint64_t x_words = ws.x_attn.bytes / 4, h_words = ws.h.bytes / 4, q_words = ws.q.bytes / 4,
                 o_words = ws.o.bytes / 4, kv_words = ws.kvcur.bytes / 4;
  const uint64_t cache = (uint64_t)p.B * L * p.NKV * p.S * p.D;
  const int op = t.op;
  const bool partial = (t.region & kRegionPartial) != 0;

  // prologue
  if (op == OP_QKV || op == OP_LM) {
    const uint64_t g = op == OP_QKV ? addr::layer_off(l, p.Hp) : 2 * (uint64_t)L * p.Hp;
    if (l == 0)
      walk_staging(w, "embedding row", addr::embed_row(V - 1, p.H), (uint64_t)V * p.H, p.H, p.Hp, g, gains);
    else
      walk_staging(w, "x_ffn (layer input)", addr::layer_off(l - 1, p.H), x_words, p.H, p.Hp, g, gains);
    if (op == OP_QKV) {
      w.in("RoPE table", addr::rope_row(w.pos, p.D), p.D, (uint64_t)p.S * p.D);
      w.in("LDS rope", 0, p.D, (uint64_t)((p.D + 3) / 4 * 4));
    }
  } else if (op == OP_GU) {
    walk_staging(w, "x_attn", addr::layer_off(l, p.H), x_words, p.H, p.Hp, (uint64_t)L * p.Hp + addr::layer_off(l, p.Hp),
                 gains);
  } else if (!partial) {
    const int n = op == OP_OPROJ ? p.QD : p.F, np = op == OP_OPROJ ? p.QDp : p.Fp;
    walk_staging(w, op == OP_OPROJ ? "o" : "h", addr::layer_off(l, op == OP_OPROJ ? p.QD : p.F),
                 op == OP_OPROJ ? o_words : h_words, n, np);
  }
  if (op == OP_OPROJ || op == OP_DOWN) {
    const int r0 = 2 * (int)t.a0, nr = 2 * (int)(t.a1 - t.a0);
    w.rule(nr <= kThreads, "residual rows fit one per thread");
    if (op == OP_OPROJ && l == 0)
      w.in("embedding (residual)", addr::embed_row(V - 1, p.H) + r0, nr, (uint64_t)V * p.H);
    else if (op == OP_OPROJ)
      w.in("x_ffn (residual)", addr::layer_off(l - 1, p.H) + r0, nr, x_words);
    else
      w.in("x_attn (residual)", addr::layer_off(l, p.H) + r0, nr, x_words);
    w.in("LDS residual", 0, nr, p.res_floats);
  }

  // weight stream (per wave: items wave, wave + 8, ...) and the LDS reads of its consumer
  const uint32_t ks = 1u << t.kslog, hks = ks >> 1;
  const uint32_t upi = t.nu >> t.kslog;
  const uint32_t n_items = (t.a1 - t.a0) << t.kslog;
  w.rule(upi * ks == t.nu && t.nu % 2 == 0, "units per item divide the pair");
  uint64_t units = 0;
  for (int wave = 0; wave < kWaves; ++wave)
    for (uint32_t i = (uint32_t)wave; i < n_items; i += kWaves) {
      const uint32_t pair = addr::item_pair(t.a0, i, t.kslog);
      w.rule(pair < t.a1, "item inside the task's pairs");
      for (uint32_t u = 0; u < upi; ++u) {
        const uint32_t unit = addr::item_unit(i, t.kslog, upi, u);
        w.rule(unit < t.nu, "unit inside its pair");
        for (uint32_t lane : {0u, 63u}) w.in("weight unit", t.wofs + addr::unit_byte(pair, t.nu, unit, lane), 16, region_bytes);
        ++units;
      }
      // consumer: activation columns of the item
      if (t.kslog == 0) {
        const int half = (int)t.nu >> 1;
        for (int j = 0; j < half; ++j) w.in("LDS activation (dot)", addr::act_unit(j, 63), 8, p.act_floats);
      } else {
        const int col = (int)(i & (hks - 1u)) * (int)upi;
        for (int j = 0; j < (int)upi; ++j) w.in("LDS activation (dot)", addr::act_unit(col + j, 63), 8, p.act_floats);
      }
    }
  w.rule(units == (uint64_t)(t.a1 - t.a0) * t.nu, "stream covers the task's units once");
  if (t.kslog > 0) w.in("LDS split partials", 0, n_items, (uint64_t)std::max(kMaxItems, kWaves * kTileRows * kTileLd));
  if (partial) {
    // down_partial: each wave stages only its columns of h
    for (int wave = 0; wave < kWaves && (uint32_t)wave < n_items; ++wave) {
      const int col0 = (int)(((uint32_t)wave & (hks - 1u)) * upi) * kUnitElems;
      for (int u0 = 0; u0 < (int)upi; u0 += 4)
        for (int j = 0; j < 8; ++j)
          for (int lane : {0, 63}) {
            const int col = col0 + (u0 + (j >> 1)) * kUnitElems + lane * 8 + (j & 1) * 4;
            if (u0 + (j >> 1) >= (int)upi) continue;
            if (col < p.F) w.in("h (partial staging)", addr::layer_off(l, p.F) + col, 4, h_words);
            w.in("LDS activation (partial staging)", col, 4, p.act_floats);
          }
    }
  }

  // epilogue of every pair
  for (uint32_t pair = t.a0; pair < t.a1; ++pair) {
    const int r = 2 * (int)pair;
    if (op == OP_QKV) {
      if (r < p.QD + p.KVD) {
        const int rr = r < p.QD ? r : r - p.QD;
        const int j = rr % p.D;
        w.in("LDS rope (pair)", j, 2, p.D);
        if (r < p.QD) {
          w.in("q", addr::layer_off(l, p.QD) + r, 2, q_words);
        } else {
          const int hk = rr / p.D;
          w.in("k cache (append)", addr::kv_slot(l, p.NKV, hk, p.S, w.pos, p.D) + j, 2, cache);
          w.in("kvcur (k)", addr::kvcur_off(l, p.KVD, 0) + rr, 2, kv_words);
        }
      } else {
        const int rr = r - p.QD - p.KVD;
        w.rule(rr + 1 < p.KVD, "v row inside KVD");
        const int hv = rr / p.D, j = rr % p.D;
        w.in("v cache (append)", addr::kv_slot(l, p.NKV, hv, p.S, w.pos, p.D) + j, 2, cache);
        w.in("kvcur (v)", addr::kvcur_off(l, p.KVD, 1) + rr, 2, kv_words);
      }
    } else if (op == OP_OPROJ || op == OP_DOWN) {
      w.in(op == OP_OPROJ ? "x_attn (out)" : "x_ffn (out)", addr::layer_off(l, p.H) + r, 2, x_words);
      w.in("LDS residual (epilogue)", r - 2 * t.a0, 2, p.res_floats);
    } else if (op == OP_GU) {
      w.in("h (out)", addr::layer_off(l, p.F) + pair, 1, h_words);
    } else if (op == OP_LM) {
      w.in("logits", r, 2, (uint64_t)p.B * V);
    }
  }
  if (op == OP_LM) {
    w.in("argmax keys", (uint64_t)w.cur_wg, 1, ws.amax.bytes / 8);
    w.in("argmax keys (winner scan)", 0, p.W, ws.amax.bytes / 8);
  }
}

void walk_attn(Walker& w, const Task& t, const Workspace& ws) {
  const Plan& p = w.p;
  const int l = t.layer, g = (int)t.a0, ch = (int)t.a1, slice = (int)t.kslog;
  const int GQ = p.G, GT = p.G / p.attn_slices, D = p.D, C = p.C;
  const int hq0 = slice * GT;
  const int NT = D / 8, PPP = kThreads / NT, NPASS = kMaxChunk / PPP;
  const int n = w.pos + 1;
  const int len0 = (n + C - 1) / C;
  const int t0 = std::min(n, ch * len0), t1 = std::min(n, t0 + len0);
  const uint64_t cache = (uint64_t)p.B * p.L * p.NKV * p.S * D;
  w.rule(t1 - t0 <= NPASS * PPP, "chunk fits the task's register passes");
  w.rule(g < p.NKV && hq0 + GT <= GQ && ch < C, "task indices");
  const size_t head = addr::kv_head(l, p.NKV, g, p.S, D);
  for (int j = 0; j < NPASS; ++j)
    for (int pg = 0; pg < PPP; ++pg) {
      const int tp = t0 + j * PPP + pg;
      const int tl = (tp < t1 && tp != w.pos) ? tp : 0;
      for (int ds : {0, NT - 1}) w.in("k/v cache (attention)", head + (size_t)tl * D + ds * 8, 8, cache);
    }
  const addr::AttnLds al = addr::attn_lds(GT, D);
  w.in("LDS attention scratch", 0, al.end, p.act_floats);
  w.in("q (attention)", addr::head_off(l, p.QD, g, GQ, hq0, D), GT * D, ws.q.bytes / 4);
  w.in("kvcur k (attention)", addr::kvcur_off(l, p.KVD, 0) + (size_t)g * D, D, ws.kvcur.bytes / 4);
  w.in("kvcur v (attention)", addr::kvcur_off(l, p.KVD, 1) + (size_t)g * D, D, ws.kvcur.bytes / 4);
  w.in("o (attention out)", addr::head_off(l, p.QD, g, GQ, hq0, D), GT * D, ws.o.bytes / 4);
  if (C == 1) return;
  const int stride = GQ * (D + 2);
  const uint64_t parts = ws.attn_part.bytes / 4;
  const size_t mine = addr::attn_rec(l, p.NKV, g, C, ch, stride);
  w.in("attention partial (acc)", mine + 2 * GQ + (size_t)hq0 * D, GT * D, parts);
  w.rule(2 * GQ + hq0 * D + GT * D <= stride, "partial stays inside its record");
  w.in("attention partial (m, l)", mine + GQ + hq0, GT, parts);
  w.in("attention merge counter", addr::attn_ctr(l, p.NKV, g, GQ, slice), 1, ws.attn_ctr.bytes / 4);
  const size_t base = addr::attn_rec(l, p.NKV, g, C, 0, stride);
  for (int k = 0; k < C; ++k) {
    w.in("attention merge (m, l)", base + (size_t)k * stride + hq0, GQ + GT, parts);
    w.in("attention merge (acc)", base + (size_t)k * stride + 2 * GQ + (size_t)hq0 * D, GT * D, parts);
  }
  w.in("LDS merge table", al.wpart + 0, 2 * C * GT, al.wpart + kWaves * GT * D);
}

}  // namespace
}  // namespace mk

extern "C" int mkcheck_walk(const mk_config* cfg, int num_wgs, int pos, long long slack, mkcheck_report* out) {
  using namespace mk;
  if (!cfg || !out) return MK_E_INVAL;
  std::memset(out, 0, sizeof(*out));
  Plan p;
  int rc = plan_build(*cfg, num_wgs, p);
  if (rc != MK_OK) {
    std::snprintf(out->first, sizeof out->first, "plan: %s", p.error.c_str());
    return rc;
  }
  if (p.batched) {
    std::snprintf(out->first, sizeof out->first, "batched plans are not walked");
    return MK_E_UNSUPPORTED;
  }
  if (pos < 0 || pos >= p.S) return MK_E_INVAL;
  const Workspace ws = layout_workspace(p);
  Walker w(p, pos, slack);
  // LDS regions in order, inside the 160 KiB of a workgroup
  w.rule(ring_bytes(p.ring_units) <= p.lds_act && p.lds_act + 4 * p.act_floats <= p.lds_res && p.lds_res + 4 * p.res_floats <= p.lds_rope &&
             p.lds_rope + 4 * p.D <= p.lds_misc && p.lds_misc + 256 <= p.lds_part && p.lds_tape + p.stages * 32 <= p.lds_bytes &&
             p.lds_bytes <= 160 * 1024,
         "LDS layout");
  const uint64_t lm_region = p.lm_borrowed ? (uint64_t)p.V * p.H * 2 : p.lm_bytes;
  for (int s = 0; s < p.stages; ++s)
    for (int b = 0; b < p.W; ++b) {
      const Task& t = p.tape[(size_t)s * p.W + b];
      if (t.op == OP_NONE) continue;
      w.cur_stage = s;
      w.cur_wg = b;
      if (t.op == OP_ATTN)
        walk_attn(w, t, ws);
      else
        walk_gemv(w, t, ws, (t.region & kRegionLm) ? lm_region : p.arena_bytes);
    }
  out->checks = (long long)w.checks;
  out->violations = (long long)w.violations;
  std::snprintf(out->first, sizeof out->first, "%s", w.first.c_str());
  return MK_OK;
}
