// mk_internal.h -- structures shared by the host planner and the gfx950 kernels.
//
// The task tape is the "instruction sequences planned on the host once and
// reused for every forward pass" of the article "Revolution der
// KI-Beschleunigung: Wie ein Low-Latency Megakernel den Llama-1B Turbo
// zuendet" (dasgeld.co): a [stage][workgroup] table of fixed-size task records.
#ifndef MK_INTERNAL_H_
#define MK_INTERNAL_H_

#include <stdint.h>

namespace mk {

// Workgroup shape: 8 wave64s, one persistent workgroup per compute unit.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
// A weight "unit" is 1 KiB: one 16-byte load per lane of a wave64.
constexpr int kUnitBytes = 1024;
constexpr int kUnitElems = kUnitBytes / 2;  // bf16 elements per unit
// Rows are padded to a multiple of one unit.
constexpr int kRowAlign = kUnitElems;
// Per-wave LDS ring of weight units kept in flight: 14 KiB per wave (112 KiB
// per workgroup) on the batch-1 path, 10 KiB per wave on the batched path,
// whose activation tiles take more LDS.  Compile-time depths keep every wait
// count an immediate.  The planner lays out batch-1 plans whose LDS does not
// fit beside the deep ring with kRingMin, for the host-side description and
// address walk only: the library refuses to run them.
constexpr int kRing = 14;
constexpr int kRingMin = 8;
constexpr int kRingBatched = 10;
// Largest group of query heads sharing one KV head.
constexpr int kMaxGroup = 8;
// Largest number of split items (pairs << kslog) of one task (LDS partials).
constexpr int kMaxItems = 256;
// Positions one attention task holds in registers at a time; a task of a
// batched plan walks its chunk in blocks of this many positions.
constexpr int kMaxChunk = 256;

// Batched decode (2..kMaxBatch sequences): every matrix is stored as tiles of
// kTileRows rows x kTileCols columns, one 1 KiB unit per tile in the lane
// order of a 16x16x32 bf16 MFMA A operand (lane l holds row l % 16, columns
// 8 * (l / 16) .. +8); activations of the batch form the B operand.
constexpr int kMaxBatch = 8;
constexpr int kTileRows = 16;
// LDS row stride (floats) of a split item's [row][sequence] partial tile:
// one past the 16 sequence columns, so that reads along the rows do not
// fall on one bank.
constexpr int kTileLd = 17;
constexpr int kTileCols = 32;
// Columns of an activation chunk held in LDS at once (per sequence).
constexpr int kChunkCols = 2048;
constexpr int kChunkTiles = kChunkCols / kTileCols;

// Stage kinds, in their order within a layer; the LM head closes the tape.
enum Op : uint8_t {
  OP_NONE = 0,
  OP_QKV = 1,    // attn RMSNorm + [Wq;Wk;Wv] GEMV + RoPE + KV append
  OP_ATTN = 2,   // split-KV GQA decode attention (+ merge by the last chunk)
  OP_OPROJ = 3,  // Wo GEMV + residual
  OP_GU = 4,     // ffn RMSNorm + interleaved [gate;up] GEMV + SiLU*mul
  OP_DOWN = 5,   // Wd GEMV + residual
  OP_LM = 6,     // final RMSNorm + LM-head GEMV + argmax stage 1 (+ stage 2 by the last task)
};

inline constexpr bool op_is_gemv(int op) { return op == OP_QKV || op == OP_OPROJ || op == OP_GU || op == OP_DOWN || op == OP_LM; }

constexpr int kStagesPerLayer = 5;

// One tape entry (32 bytes, read with scalar loads).
//  GEMV ops: row pairs [a0, a1) of the op's packed matrix; pair p occupies
//            nu units starting at byte wofs + p * nu * kUnitBytes of the
//            weight region selected by `region` (0 = arena, 1 = LM head).
//            Each pair is cut into 2^kslog work items: with kslog == 0 an item
//            is the whole pair and one wave finishes it; otherwise an item is
//            a run of nu >> kslog units inside one row, and the partial sums
//            of a pair's items are added in LDS in item order.
//  OP_ATTN : a0 = kv head, a1 = chunk index, nu = sequence of the batch,
//            kslog = slice of the kv head's query heads (batch 1).
//  Batched plans: GEMM tasks cover row blocks [a0, a1) of 16 rows; nu is the
//            number of 32-column tiles of a row; each block's tiles are cut
//            into 2^kslog parts (split over waves, summed in LDS).  A down
//            or down projection with at most half as many blocks as
//            workgroups gives each block to two workgroups (region bit
//            kRegionSplit), each walking half of the row's chunks (a row of
//            one chunk is walked as two half-width chunks); the second half
//            (kRegionHalf1) hands its partial sums to the first, which adds
//            them in that order.
// Activation columns of a batched GEMM chunk: kChunkTiles tiles, or half of
// a single-chunk row that is split over two workgroups.
inline constexpr int gemm_chunk_tiles(int ktiles, bool split) {
  return ktiles > kChunkTiles ? kChunkTiles : (split ? ktiles / 2 : ktiles);
}

// Bits of Task::region.
constexpr uint8_t kRegionLm = 1;      // weights are the LM head, not the arena
constexpr uint8_t kRegionSplit = 2;   // batched: the block's chunks are split over two workgroups
constexpr uint8_t kRegionHalf1 = 4;   // batched: this task walks the second half of the chunks
constexpr uint8_t kRegionPartial = 8; // batch 1 down projection: every wave stages only its items' columns of h

struct Task {
  uint8_t op;
  uint8_t region;
  uint16_t layer;
  uint32_t a0;
  uint32_t a1;
  uint32_t nu;
  uint64_t wofs;
  uint32_t ntasks;  // tasks in this stage (argmax / merge participants)
  uint32_t kslog;
};
static_assert(sizeof(Task) == 32, "task record must stay 32 bytes");

// Step arguments read from device memory by graph-captured launches.
struct StepArgs {
  int32_t pos;
  uint32_t epoch;
};

// Device status (first error wins).  Mirrored into host-mapped memory.
struct DevStatus {
  int32_t code;
  int32_t stage;
  int32_t wg;
  uint32_t detail;
};

// Kernel parameters (passed by value).
struct Params {
  const Task* tape;      // [num_stages][num_wgs]
  int32_t num_wgs;
  int32_t num_stages;

  // model
  int32_t L, H, Hp, QD, QDp, KVD, F, Fp, V, NQ, NKV, D, G, S, B;
  float eps;
  float qscale;          // 1 / sqrt(head_dim)
  int32_t attn_chunks;
  int32_t attn_gt;       // query heads per attention task (G, or 1 when each head has its own task)

  // weights
  const char* arena;     // packed bf16 matrices (byte base)
  const char* lm;        // LM-head matrix [V][Hp] (byte base)
  const uint16_t* embed; // caller's [V][H] embedding
  const float* g_attn;   // [L][Hp]
  const float* g_ffn;    // [L][Hp]
  const float* g_final;  // [Hp]
  const float* rope;     // [S][D/2][2] cos, sin

  // tagged activations: one 32-bit word per element, the fp32 value's 24
  // high bits and the step's tag (epoch mod 256) in the low byte
  uint32_t* x_attn;      // [B][L][H]   residual after attention
  uint32_t* x_ffn;       // [B][L][H]   residual after FFN
  uint32_t* q;           // [B][L][QD]  rotated queries
  uint32_t* kvcur;       // [B][L][2][KVD] this step's bf16-rounded k, v
  uint32_t* o;           // [B][L][QD]  attention output
  uint32_t* h;           // [B][L][F]   SwiGLU hidden
  uint32_t* kpart;       // [B][L][2][H] second-half partial sums of split O-proj / down tasks
  float* attn_part;      // [B][L][NKV][C][G*(D+2)] split-KV partials
  uint32_t* attn_ctr;    // [B][L][NKV][G] merge counters per head slice (epoch * C per step)
  uint64_t* amax;        // [B][num_wgs] argmax keys
  uint32_t* amax_ctr;    // [B] argmax counters (epoch * tasks per step)
  uint32_t* tokerr;      // [B] epoch of the last bad input token
  uint32_t* abort_flag;  // non-zero: every workgroup stops
  DevStatus* status;     // device copy of the status
  DevStatus* status_host;// host-mapped mirror

  // LDS layout (bytes from the dynamic LDS base)
  int32_t lds_act;       // fp32 activation vector / attention scratch
  int32_t lds_res;       // residual rows of the task
  int32_t lds_rope;      // cos/sin of this position
  int32_t lds_misc;      // reductions and flags
  int32_t lds_part;      // [kMaxItems] partial sums of split items
  int32_t lds_tape;      // this workgroup's task records, one per stage
  int32_t act_stride;    // batched: floats per sequence in the activation chunk
  int32_t act_floats;
  int32_t res_floats;

  uint64_t watchdog_ticks;  // wall-clock ticks (100 MHz on MI355X)
  uint64_t* trace;          // [num_wgs][num_stages][kTraceStamps] stamps, or null

  // per step
  const int32_t* token;  // [B]
  uint16_t* kcache;      // [B][L][NKV][S][D]
  uint16_t* vcache;
  float* logits;         // [B][V]
  int32_t* out_token;    // [B]
  int32_t pos;
  uint32_t epoch;
  const StepArgs* dargs; // non-null: read pos and epoch from here (graph mode)
  int32_t partial;       // the plan has partial-input down-projection tasks (selects the kernel instance)
  int32_t prefill;       // batched plans: the B "sequences" are tokens pos .. pos + B - 1 of one sequence
  // multi-step launches: step i's greedy tokens are published as 64-bit words
  // (epoch of step i + 1 in the high half, the token in the low half) that
  // step i + 1 polls before its first stage; the full epoch cannot match a
  // word left by an earlier launch
  uint64_t* tok_tag;     // [B], or null for single-step launches
  int64_t logits_step;   // floats between the logits of consecutive steps (0: one buffer reused)
};

// Trace record of one (workgroup, stage): entered, inputs ready, compute done,
// left, then for each of the kWaves waves the time it finished its own work,
// then for each wave the time its first weight unit of the task was in hand.
constexpr int kTraceStamps = 4 + 2 * kWaves;

// LDS bytes of the per-wave rings of a given depth.
constexpr int ring_bytes(int units) { return kWaves * units * kUnitBytes; }

}  // namespace mk

#endif  // MK_INTERNAL_H_
