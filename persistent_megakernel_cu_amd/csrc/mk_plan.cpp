// mk_plan.cpp -- the host planner.
//
// The article "Revolution der KI-Beschleunigung: Wie ein Low-Latency
// Megakernel den Llama-1B Turbo zuendet" (dasgeld.co) describes a GPU
// interpreter that receives the forward pass as instruction sequences planned
// on the host and reused, unchanged, for every forward pass.  Here the plan is
// a [stage][workgroup] tape: every matrix op of every layer is cut into
// contiguous row-pair ranges, one per workgroup, so each workgroup streams a
// disjoint slice of every weight matrix exactly once per token.
#include "mk_plan.h"

#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

namespace mk {

namespace {

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }
inline uint64_t round_up64(uint64_t x, uint64_t m) { return (x + m - 1) / m * m; }

int fail(Plan& p, int code, const char* msg) {
  p.error = msg;
  return code;
}

// Split of each row pair into 2^k items shared by the 8 waves of a
// workgroup.  One item per row (k = 1) whenever every wave gets at least one
// row and the items fit the partial-sum area: measured on MI355X against the
// split that minimises the units of the busiest wave, rows were faster for
// every Llama-1B stage (gate/up: rows against whole pairs -18 us per step,
// against half rows -21, against quarter rows -63; QKV: rows against half
// rows -3 us; O-proj and down: rows against whole pairs -9 / -60 us, against
// half rows -7 / -5 us).  Otherwise minimise the units of the busiest wave,
// fewer splits on ties.  Items must stay inside one row.
uint32_t split_log2(uint32_t pairs, uint32_t nu) {
  if (nu >= 2 && 2ull * pairs >= (uint64_t)kWaves && 2ull * pairs <= (uint64_t)kMaxItems) return 1;
  uint32_t best = 0;
  uint64_t best_cost = ~0ull;
  for (uint32_t k = 0; (1u << k) <= nu; ++k) {
    const uint32_t ks = 1u << k;
    if (ks > 1 && ((nu / 2) % (ks / 2)) != 0) break;
    if ((uint64_t)pairs * ks > (uint64_t)kMaxItems && ks > 1) break;
    const uint64_t items = (uint64_t)pairs * ks;
    const uint64_t cost = (items + kWaves - 1) / kWaves * (nu / ks);
    if (cost < best_cost) {
      best_cost = cost;
      best = k;
    }
  }
  return best;
}

}  // namespace

uint64_t qkv_rows(const Plan& p) { return (uint64_t)p.QD + 2ull * p.KVD; }

int plan_build(const mk_config& c, int W, Plan& p) {
  p = Plan();
  if (c.n_layers < 0 || c.hidden <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 || c.ffn <= 0 ||
      c.vocab <= 0 || c.max_seq <= 0 || c.batch <= 0)
    return fail(p, MK_E_INVAL, "dimensions must be positive (n_layers >= 0)");
  if (c.n_heads % c.n_kv_heads != 0) return fail(p, MK_E_INVAL, "n_heads must be a multiple of n_kv_heads");
  if (c.head_dim != 64 && c.head_dim != 128) return fail(p, MK_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c.hidden % 4 != 0 || c.ffn % 4 != 0 || c.vocab % 2 != 0)
    return fail(p, MK_E_UNSUPPORTED, "hidden and ffn must be multiples of 4, vocab even");
  {
    const int grp = c.n_heads / c.n_kv_heads;
    if (grp != 1 && grp != 2 && grp != 4) return fail(p, MK_E_UNSUPPORTED, "1, 2 or 4 query heads per kv head");
  }
  if (c.batch > kMaxBatch) return fail(p, MK_E_UNSUPPORTED, "at most 8 sequences per batch");
  if (c.batch > 1) {
    if (c.head_dim != 64) return fail(p, MK_E_UNSUPPORTED, "batched decode needs head_dim 64");
    if (c.hidden % kTileRows != 0 || c.vocab % kTileRows != 0 || c.ffn % (kTileRows / 2) != 0)
      return fail(p, MK_E_UNSUPPORTED, "batched decode needs hidden and vocab multiples of 16, ffn of 8");
  }
  if (!(c.rms_eps >= 0.0f) || !(c.rope_theta > 0.0)) return fail(p, MK_E_INVAL, "rms_eps >= 0 and rope_theta > 0");
  if (c.exec_mode < MK_MODE_MEGA || c.exec_mode > MK_MODE_GRAPH) return fail(p, MK_E_INVAL, "unknown exec_mode");
  if (W <= 0 || W > 4096) return fail(p, MK_E_INVAL, "workgroup count out of range");

  p.L = c.n_layers;
  p.H = c.hidden;
  p.NQ = c.n_heads;
  p.NKV = c.n_kv_heads;
  p.D = c.head_dim;
  p.G = c.n_heads / c.n_kv_heads;
  p.QD = c.n_heads * c.head_dim;
  p.KVD = c.n_kv_heads * c.head_dim;
  p.F = c.ffn;
  p.V = c.vocab;
  p.S = c.max_seq;
  p.B = c.batch;
  p.W = W;
  p.tied = c.tie_embeddings != 0;
  p.Hp = round_up(p.H, kRowAlign);
  p.QDp = round_up(p.QD, kRowAlign);
  p.Fp = round_up(p.F, kRowAlign);
  p.batched = p.B > 1;
  if (c.partial_input && (p.batched || p.D != 64))
    return fail(p, MK_E_UNSUPPORTED, "partial-input starts need batch 1 and head_dim 64");
  p.partial = c.partial_input != 0;
  if (c.prefill && (!p.batched || c.exec_mode > MK_MODE_GRAPH))
    return fail(p, MK_E_UNSUPPORTED, "prefill needs batch 2..8 and a megakernel mode");
  p.prefill = c.prefill != 0;
  if (p.batched && (p.Hp > kChunkCols || p.QDp > kChunkCols))
    return fail(p, MK_E_UNSUPPORTED, "batched decode needs hidden and n_heads * head_dim <= 2048");

  // Attention split: chunks of at most kMaxChunk positions (batched plans
  // walk longer chunks in blocks), at most one task per workgroup.
  const int seqs_kv = p.B * p.NKV;  // (sequence, kv head) pairs
  int C = c.attn_chunks;
  if (C <= 0) C = (p.S + kMaxChunk - 1) / kMaxChunk;
  C = std::max(1, std::min(C, p.S));
  if ((int64_t)C * seqs_kv > W) C = std::max(1, W / seqs_kv);
  if ((int64_t)C * seqs_kv > W) return fail(p, MK_E_UNSUPPORTED, "more (sequence, kv head) pairs than workgroups");
  // the merge keeps a {max, sum} pair per chunk and head in the LDS that
  // held the eight waves' partial outputs
  C = std::min(C, kWaves * p.D / 2);
  p.C = C;
  // Batch 1: when there are workgroups to spare, every query head of a kv
  // head gets its own attention task (no merge: heads are independent).
  p.attn_slices = (!p.batched && (int64_t)seqs_kv * p.G * C <= W) ? p.G : 1;
  const int lmax = (p.S + C - 1) / C;  // longest chunk
  if (!p.batched && lmax > kMaxChunk) return fail(p, MK_E_UNSUPPORTED, "attention chunk longer than 256 positions");

  // ---- packed arena layout: per layer [Wq;Wk;Wv] | Wo | [gate/up interleaved] | Wd
  const uint64_t align = 4096;
  uint64_t off = 0;
  p.off_qkv.resize(p.L);
  p.off_o.resize(p.L);
  p.off_gu.resize(p.L);
  p.off_down.resize(p.L);
  for (int l = 0; l < p.L; ++l) {
    p.off_qkv[l] = off;
    off = round_up64(off + qkv_rows(p) * p.Hp * 2, align);
    p.off_o[l] = off;
    off = round_up64(off + (uint64_t)p.H * p.QDp * 2, align);
    p.off_gu[l] = off;
    off = round_up64(off + 2ull * p.F * p.Hp * 2, align);
    p.off_down[l] = off;
    off = round_up64(off + (uint64_t)p.H * p.Fp * 2, align);
  }
  p.arena_bytes = std::max<uint64_t>(off, align);
  p.lm_borrowed = !p.batched && (p.Hp == p.H);  // tiled plans always repack
  p.lm_bytes = p.lm_borrowed ? 0 : (uint64_t)p.V * p.Hp * 2;

  // ---- tape
  p.stages = kStagesPerLayer * p.L + 1;
  p.tape.assign((size_t)p.stages * W, Task{});
  int max_res_rows = 0;
  // Which workgroup streams which part of a matrix.  Workgroup b runs on XCD
  // b mod 8.  The gate/up stage streams 256 KB per workgroup (batch 1: 32 row
  // pairs of 8 KB; batched: 4 blocks of 64 KB).  Measured on MI355X with the
  // batched stage's whole blocks (and the batch-1 stage's whole pairs, before
  // it took row items), the step is 6-8 us faster when workgroup i of the
  // stage takes range i + 1 (or i + 5) instead of range i, and 7-8 us slower
  // with i + 3; even offsets change nothing, nor do offsets of the other
  // stages or, with row items, any offset at batch 1.  The cause is not
  // established (a streaming probe shows no XCD-to-address affinity).
  auto range_rotation = [&](Op op, int nw) { return op == OP_GU && nw > 1 ? 1 : 0; };
  // Row pairs of a GEMV stage in contiguous, balanced ranges over workgroups
  // [b0, W), range (i + rotation) mod nw on workgroup b0 + i.
  auto gemv_stage = [&](int s, Op op, int layer, uint64_t pairs, uint32_t nu, uint64_t wofs, uint8_t region,
                        int b0 = 0) {
    const int nw = W - b0;
    const int rot = range_rotation(op, nw);
    uint32_t n = 0;
    for (int i = 0; i < nw; ++i) {
      uint64_t a0 = pairs * (uint64_t)i / nw, a1 = pairs * (uint64_t)(i + 1) / nw;
      if (a1 > a0) ++n;
    }
    for (int i = 0; i < nw; ++i) {
      const int b = b0 + i, j = (i + rot) % nw;
      uint64_t a0 = pairs * (uint64_t)j / nw, a1 = pairs * (uint64_t)(j + 1) / nw;
      Task& t = p.tape[(size_t)s * W + b];
      if (a1 == a0) continue;
      t.op = op;
      t.region = region;
      t.layer = (uint16_t)layer;
      t.a0 = (uint32_t)a0;
      t.a1 = (uint32_t)a1;
      t.nu = nu;
      t.wofs = wofs;
      t.ntasks = n;
      t.kslog = op == OP_LM ? 0u : split_log2((uint32_t)(a1 - a0), nu);
      // Partial-input plans (cfg.partial_input): the down projection's input
      // (ffn wide) is produced by the gate/up stage, whose straggler tail is
      // the longest.  Cut every pair into 8 items of nu / 8 units: the items
      // of wave w all cover the same quarter of the row's columns, so each
      // wave stages only that quarter of h and starts as soon as it carries
      // this step's tag, without waiting for the rest of h.
      if (p.partial && op == OP_DOWN && (nu / 2) % 4 == 0 && (a1 - a0) * 8 <= (uint64_t)kMaxItems) {
        t.kslog = 3;
        t.region |= kRegionPartial;
      }
      if (op == OP_OPROJ || op == OP_DOWN) max_res_rows = std::max(max_res_rows, (int)(2 * (a1 - a0)));
    }
  };
  // Batched plans: row blocks of 16 rows over workgroups [b0, W); a task's
  // blocks are cut into 2^kslog parts so that at least 8 (block, part) items
  // keep the waves busy (parts split the columns of every chunk).
  auto gemm_stage = [&](int s, Op op, int layer, uint64_t rows, uint32_t ktiles, uint64_t wofs, uint8_t region,
                        int b0 = 0) {
    const uint64_t blocks = rows / kTileRows;
    const int nw = W - b0;
    const uint32_t ch = std::min<uint32_t>(ktiles, kChunkTiles);
    const uint32_t sch = (uint32_t)gemm_chunk_tiles((int)ktiles, true);
    const uint32_t snc = ktiles / sch;
    if ((op == OP_DOWN || op == OP_OPROJ) && b0 == 0 && 2 * blocks <= (uint64_t)W && snc % 2 == 0 &&
        sch % kWaves == 0 && ktiles % sch == 0) {
      // two workgroups per block, one per half of the row's chunks
      const uint32_t ch = sch;
      uint32_t k = 0;
      while ((2u << k) <= (uint32_t)kWaves && (ch >> (k + 1)) > 0 && ch % (2u << k) == 0) ++k;
      for (uint64_t i = 0; i < 2 * blocks; ++i) {
        Task& t = p.tape[(size_t)s * W + i];
        t.op = op;
        t.region = (uint8_t)(region | kRegionSplit | ((i & 1) ? kRegionHalf1 : 0));
        t.layer = (uint16_t)layer;
        t.a0 = (uint32_t)(i / 2);
        t.a1 = t.a0 + 1;
        t.nu = ktiles;
        t.wofs = wofs;
        t.ntasks = (uint32_t)(2 * blocks);
        t.kslog = k;
        max_res_rows = std::max(max_res_rows, kTileRows);
      }
      return;
    }
    uint32_t n = 0;
    for (int i = 0; i < nw; ++i) n += blocks * (uint64_t)(i + 1) / nw > blocks * (uint64_t)i / nw;
    const int rot = range_rotation(op, nw);
    for (int i = 0; i < nw; ++i) {
      const int j = (i + rot) % nw;
      const uint64_t a0 = blocks * (uint64_t)j / nw, a1 = blocks * (uint64_t)(j + 1) / nw;
      if (a1 == a0) continue;
      Task& t = p.tape[(size_t)s * W + b0 + i];
      t.op = op;
      t.region = region;
      t.layer = (uint16_t)layer;
      t.a0 = (uint32_t)a0;
      t.a1 = (uint32_t)a1;
      t.nu = ktiles;
      t.wofs = wofs;
      t.ntasks = n;
      uint32_t k = 0;
      while ((a1 - a0) << (k + 1) <= (uint64_t)kWaves && (ch >> (k + 1)) > 0 && ch % (2u << k) == 0) ++k;
      t.kslog = k;
      if (op == OP_OPROJ || op == OP_DOWN) max_res_rows = std::max(max_res_rows, (int)((a1 - a0) * kTileRows));
    }
  };
  for (int l = 0; l < p.L; ++l) {
    const int s0 = kStagesPerLayer * l;
    if (p.batched)
      gemm_stage(s0 + 0, OP_QKV, l, qkv_rows(p), (uint32_t)(p.Hp / kTileCols), p.off_qkv[l], 0);
    else
      gemv_stage(s0 + 0, OP_QKV, l, qkv_rows(p) / 2, (uint32_t)(2 * p.Hp / kUnitElems), p.off_qkv[l], 0);
    // attention: task i = (sequence, kv head, query-head slice, chunk) on workgroup i
    const int sl = p.attn_slices;
    for (int i = 0; i < seqs_kv * sl * C; ++i) {
      Task& t = p.tape[(size_t)(s0 + 1) * W + i];
      t.op = OP_ATTN;
      t.layer = (uint16_t)l;
      t.nu = (uint32_t)(i / (p.NKV * sl * C));
      t.a0 = (uint32_t)((i / (sl * C)) % p.NKV);
      t.kslog = (uint32_t)((i / C) % sl);
      t.a1 = (uint32_t)(i % C);
      t.ntasks = (uint32_t)(seqs_kv * sl * C);
    }
    if (p.batched) {
      const int gu_b0 = (seqs_kv * C * 8 <= W) ? seqs_kv * C : 0;  // batched plans have one slice
      gemm_stage(s0 + 2, OP_OPROJ, l, p.H, (uint32_t)(p.QDp / kTileCols), p.off_o[l], 0);
      gemm_stage(s0 + 3, OP_GU, l, 2ull * p.F, (uint32_t)(p.Hp / kTileCols), p.off_gu[l], 0, gu_b0);
      gemm_stage(s0 + 4, OP_DOWN, l, p.H, (uint32_t)(p.Fp / kTileCols), p.off_down[l], 0);
      continue;
    }
    gemv_stage(s0 + 2, OP_OPROJ, l, p.H / 2, (uint32_t)(2 * p.QDp / kUnitElems), p.off_o[l], 0);
    // When attention occupies very few workgroups (at most 1/16 of them) they
    // sit out the gate/up stage: they reach it last (after attention and
    // O-proj), and the down projection waits for the slowest gate/up task.
    const int gu_b0 = (p.NKV * sl * C * 16 <= W) ? p.NKV * sl * C : 0;
    gemv_stage(s0 + 3, OP_GU, l, p.F, (uint32_t)(2 * p.Hp / kUnitElems), p.off_gu[l], 0, gu_b0);
    gemv_stage(s0 + 4, OP_DOWN, l, p.H / 2, (uint32_t)(2 * p.Fp / kUnitElems), p.off_down[l], 0);
  }
  if (p.batched)
    gemm_stage(p.stages - 1, OP_LM, p.L, p.V, (uint32_t)(p.Hp / kTileCols), 0, 1);
  else
    gemv_stage(p.stages - 1, OP_LM, p.L, p.V / 2, (uint32_t)(2 * p.Hp / kUnitElems), 0, 1);
  p.num_tasks = 0;
  for (const Task& t : p.tape) p.num_tasks += t.op != OP_NONE;

  // ---- LDS layout
  // attention scratch: q [G][D], k and v of this step [D] each, per-wave
  // partial outputs [waves][G][D], per-wave max and sum [waves][G] each
  // (prefill: the k and v rows of all B tokens of the step); batched plans
  // add per wave the MFMA path's probabilities [G][32] and V^T [D][40] bf16
  const int kv_rows = p.prefill ? p.B : 1;
  const int attn_floats = p.G * p.D + 2 * kv_rows * p.D + kWaves * p.G * p.D + 2 * kWaves * p.G +
                          (p.batched ? kWaves * (p.G * 32 + p.D * 20) : 0);
  if (p.batched) {
    p.act_stride = std::max(std::max(p.Hp, p.QDp), std::min(p.Fp, kChunkCols));
    p.act_floats = round_up(std::max(p.B * p.act_stride, attn_floats), 4);
    p.res_floats = round_up(std::max(p.B * max_res_rows, 4), 4);
  } else {
    p.act_floats = round_up(std::max(std::max(p.Hp, p.QDp), std::max(p.Fp, attn_floats)), 4);
    p.res_floats = round_up(std::max(max_res_rows, 4), 4);
  }
  if (max_res_rows > kThreads) return fail(p, MK_E_UNSUPPORTED, "more than 512 residual rows per workgroup");
  auto lay_out = [&](int ring_units) {
    p.ring_units = ring_units;
    p.lds_act = ring_bytes(ring_units);
    p.lds_res = p.lds_act + p.act_floats * 4;
    p.lds_rope = p.lds_res + p.res_floats * 4;
    p.lds_misc = p.lds_rope + round_up(p.D * kv_rows, 4) * 4;  // cos/sin of each token's position
    p.lds_part = p.lds_misc + 256;
    // split-item sums; batched: one 16x16 fp32 tile per wave
    p.lds_tape = p.lds_part + std::max(kMaxItems, kWaves * kTileRows * kTileLd) * 4;
    p.lds_bytes = p.lds_tape + p.stages * (int)sizeof(Task);
  };
  lay_out(p.batched ? kRingBatched : kRing);
  if (!p.batched && p.lds_bytes > 160 * 1024) lay_out(kRingMin);
  if (p.lds_bytes > 160 * 1024) return fail(p, MK_E_UNSUPPORTED, "LDS plan exceeds 160 KiB per workgroup");
  return MK_OK;
}

Workspace layout_workspace(const Plan& p) {
  Workspace w{};
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const WsBuf b{cur, bytes};
    cur = (cur + bytes + 255) / 256 * 256;
    return b;
  };
  const size_t L = std::max(p.L, 1), B = p.B;
  w.x_attn = take(B * L * p.H * 4);
  w.x_ffn = take(B * L * p.H * 4);
  w.q = take(B * L * p.QD * 4);
  w.kvcur = take(B * L * 2 * p.KVD * 4);
  w.o = take(B * L * p.QD * 4);
  w.h = take(B * L * p.F * 4);
  w.kpart = take(B * L * 2 * p.H * 4);
  w.attn_part = take(B * L * p.NKV * p.C * p.G * (p.D + 2) * 4);
  w.attn_ctr = take(B * L * p.NKV * p.G * 4);
  w.amax = take(B * p.W * 8);
  w.amax_ctr = take(B * 4);
  w.tokerr = take(B * 4);
  w.abort_flag = take(4);
  w.status = take(sizeof(DevStatus));
  w.dargs = take(sizeof(StepArgs));
  w.tok_tag = take(B * 8);
  w.bytes = cur;
  return w;
}

// True when the half-open ranges cover [0, total) exactly once.
static bool tiles_exactly(std::vector<std::pair<uint64_t, uint64_t>> r, uint64_t total) {
  std::sort(r.begin(), r.end());
  uint64_t next = 0;
  for (const auto& x : r) {
    if (x.first != next || x.second <= x.first) return false;
    next = x.second;
  }
  return next == total;
}

int plan_validate(const Plan& p, std::string* why) {
  auto bad = [&](const std::string& m) {
    if (why) *why = m;
    return MK_E_INVAL;
  };
  const int W = p.W;
  if ((int)p.tape.size() != p.stages * W) return bad("tape size");
  {
    // the batched staging addresses a tagged buffer with 32-bit byte offsets
    const Workspace w = layout_workspace(p);
    if (w.kpart.off + w.kpart.bytes - w.x_attn.off >= (1ull << 31)) return bad("tagged activations exceed 2 GiB");
  }
  for (int s = 0; s < p.stages; ++s) {
    const bool lm = s == p.stages - 1;
    const int kind = lm ? OP_LM : 1 + (s % kStagesPerLayer);
    const int layer = lm ? p.L : s / kStagesPerLayer;
    uint64_t pairs = 0, nu = 0, wofs = 0, region_bytes = 0;
    switch (kind) {
      case OP_QKV:
        pairs = qkv_rows(p) / 2; nu = 2 * p.Hp / kUnitElems; wofs = p.off_qkv[layer];
        region_bytes = qkv_rows(p) * p.Hp * 2; break;
      case OP_OPROJ:
        pairs = p.H / 2; nu = 2 * p.QDp / kUnitElems; wofs = p.off_o[layer];
        region_bytes = (uint64_t)p.H * p.QDp * 2; break;
      case OP_GU:
        pairs = p.F; nu = 2 * p.Hp / kUnitElems; wofs = p.off_gu[layer];
        region_bytes = 2ull * p.F * p.Hp * 2; break;
      case OP_DOWN:
        pairs = p.H / 2; nu = 2 * p.Fp / kUnitElems; wofs = p.off_down[layer];
        region_bytes = (uint64_t)p.H * p.Fp * 2; break;
      case OP_LM:
        pairs = p.V / 2; nu = 2 * p.Hp / kUnitElems; wofs = 0;
        region_bytes = (uint64_t)p.V * p.Hp * 2; break;
      default: break;
    }
    uint32_t count = 0;
    for (int b = 0; b < W; ++b) count += p.tape[(size_t)s * W + b].op != OP_NONE;
    if (kind == OP_ATTN) {
      const int sl = p.attn_slices;
      if (2 * p.C > kWaves * p.D) return bad("more attention chunks than the merge table holds");
      std::vector<int> seen((size_t)p.B * p.NKV * sl * p.C, 0);
      for (int b = 0; b < W; ++b) {
        const Task& t = p.tape[(size_t)s * W + b];
        if (t.op == OP_NONE) continue;
        if (t.op != OP_ATTN || t.layer != layer) return bad("attention stage holds another op");
        if ((int)t.a0 >= p.NKV || (int)t.a1 >= p.C || (int)t.nu >= p.B || (int)t.kslog >= sl)
          return bad("attention task out of range");
        if (seen[(((size_t)t.nu * p.NKV + t.a0) * sl + t.kslog) * p.C + t.a1]++) return bad("attention task repeated");
        if (t.ntasks != count) return bad("attention task count");
      }
      for (int v : seen)
        if (v != 1) return bad("attention task missing");
      continue;
    }
    if (p.batched) {
      // GEMM: row blocks [a0, a1) must tile [0, rows / 16) exactly
      uint64_t rows = 0, kt = 0;
      switch (kind) {
        case OP_QKV: rows = qkv_rows(p); kt = p.Hp / kTileCols; break;
        case OP_OPROJ: rows = p.H; kt = p.QDp / kTileCols; break;
        case OP_GU: rows = 2ull * p.F; kt = p.Hp / kTileCols; break;
        case OP_DOWN: rows = p.H; kt = p.Fp / kTileCols; break;
        default: rows = p.V; kt = p.Hp / kTileCols; break;
      }
      const uint64_t ch = std::min<uint64_t>(kt, kChunkTiles);
      uint64_t next = 0;
      std::vector<std::pair<uint64_t, uint64_t>> whole;  // unsplit blocks' ranges, in any workgroup order
      int half0 = -1;  // workgroup holding the first half of a split block, until its second half
      for (int b = 0; b < W; ++b) {
        const Task& t = p.tape[(size_t)s * W + b];
        if (t.op == OP_NONE) continue;
        if (t.op != kind || t.layer != layer) return bad("stage holds another op");
        if (t.region & kRegionSplit) {
          // split block: the first half, then the second half on the next workgroup
          const uint64_t sch = (uint64_t)gemm_chunk_tiles((int)kt, true);
          if ((kind != OP_DOWN && kind != OP_OPROJ) || t.a1 != t.a0 + 1 || t.kslog == 0 || kt % sch != 0 ||
              (kt / sch) % 2 != 0 || sch % (1ull << t.kslog) != 0)
            return bad("split task geometry");
          if (!(t.region & kRegionHalf1)) {
            if (half0 >= 0 || t.a0 != next) return bad("split blocks not tiled exactly");
            half0 = b;
          } else {
            const Task& f = p.tape[(size_t)s * W + (half0 < 0 ? 0 : half0)];
            if (half0 != b - 1 || f.a0 != t.a0) return bad("split block without its first half");
            half0 = -1;
            next = t.a1;
          }
        } else {
          if (half0 >= 0) return bad("split block without its second half");
          if (t.a1 <= t.a0) return bad("row blocks not tiled exactly");
          whole.push_back({t.a0, t.a1});
        }
        if (t.nu != kt || t.wofs != wofs) return bad("task geometry");
        if ((uint64_t)t.a1 * kt * kUnitBytes > region_bytes) return bad("task reads past its matrix");
        if (t.ntasks != count) return bad("task count");
        if ((t.region & kRegionLm) != (kind == OP_LM ? kRegionLm : 0)) return bad("weight region");
        const uint64_t ks = 1ull << t.kslog, items = (uint64_t)(t.a1 - t.a0) * ks;
        if (kt % ch != 0 || (!(t.region & kRegionSplit) && ch % ks != 0)) return bad("parts do not divide the chunks");
        if (ks > 1 && items > (uint64_t)kWaves) return bad("split blocks need one item per wave");
        if (kt > ch && items > (uint64_t)kWaves) return bad("chunked rows need one item per wave");
        if ((kind == OP_OPROJ || kind == OP_DOWN) && (uint64_t)p.B * (t.a1 - t.a0) * kTileRows > (uint64_t)p.res_floats)
          return bad("residual rows exceed LDS");
      }
      if (half0 >= 0) return bad("split block without its second half");
      if (!whole.empty() && next != 0) return bad("split and unsplit blocks in one stage");
      if (!whole.empty() && !tiles_exactly(whole, rows / kTileRows)) return bad("row blocks not tiled exactly");
      if (whole.empty() && next != rows / kTileRows) return bad("row blocks not covered");
      continue;
    }
    // GEMV: ranges must tile [0, pairs) exactly (in any workgroup order)
    std::vector<std::pair<uint64_t, uint64_t>> ranges;
    for (int b = 0; b < W; ++b) {
      const Task& t = p.tape[(size_t)s * W + b];
      if (t.op == OP_NONE) continue;
      if (t.op != kind || t.layer != layer) return bad("stage holds another op");
      if (t.a1 <= t.a0) return bad("row pairs not tiled exactly");
      ranges.push_back({t.a0, t.a1});
      if (t.nu != nu || t.wofs != wofs) return bad("task geometry");
      if ((uint64_t)t.a1 * t.nu * kUnitBytes > region_bytes) return bad("task reads past its matrix");
      if (t.ntasks != count) return bad("task count");
      if ((kind == OP_OPROJ || kind == OP_DOWN) && 2 * (t.a1 - t.a0) > (uint32_t)p.res_floats)
        return bad("residual rows exceed LDS");
      if (t.region & kRegionPartial) {
        if (kind != OP_DOWN || t.kslog != 3 || (t.nu / 2) % 4 != 0) return bad("partial-input task geometry");
      } else if (t.region != (kind == OP_LM ? 1 : 0)) {
        return bad("weight region");
      }
      if (t.kslog > 0) {
        const uint32_t ks = 1u << t.kslog;
        if (kind == OP_LM) return bad("LM head is never split");
        if ((t.nu / 2) % (ks / 2) != 0) return bad("split item crosses a row");
        if ((uint64_t)(t.a1 - t.a0) * ks > (uint64_t)kMaxItems) return bad("too many split items");
      }
    }
    if (!tiles_exactly(ranges, pairs)) return bad("row pairs not tiled exactly");
  }
  if (p.lds_bytes > 160 * 1024) return bad("LDS");
  if (p.batched ? p.ring_units != kRingBatched : (p.ring_units != kRing && p.ring_units != kRingMin))
    return bad("ring depth");
  return MK_OK;
}

}  // namespace mk
