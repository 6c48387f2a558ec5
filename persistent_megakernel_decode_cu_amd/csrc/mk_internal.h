// Internal definitions shared by the host task-graph builder, the runtime and
// the device interpreter.  Not part of the public ABI (include/mk.h is).
#pragma once
#include <stdint.h>

namespace mk {

// ---- opcodes of the on-GPU interpreter ----------------------------------------
enum Op : uint8_t {
    OP_END = 0,       // end of a queue
    OP_QKV = 1,       // RMSNorm + fused QKV GEMV tile + RoPE + KV-cache append
    OP_ATTN = 2,      // GQA decode attention over one KV chunk -> (m, l, o) partials
    OP_OPROJ = 3,     // merge attention partials of one KV group + O-proj K-slice + residual (atomic)
    OP_GATEUP = 4,    // RMSNorm + gate/up GEMV tile + SiLU * up
    OP_DOWN = 5,      // down-proj K-slice tile + residual (atomic)
    OP_LMHEAD = 6,    // final RMSNorm + LM-head tile + argmax (packed 64-bit atomic max)
    // mixture-of-experts FFN (several sequences): routing decided inside the step
    OP_ROUTE = 7,     // RMSNorm + router GEMV rows: router logits of up to 16 experts
    OP_EGU = 8,       // RMSNorm + one expert's gate/up rows + SiLU * up
    OP_EDOWN = 9,     // routing weights (top-k + softmax) + one expert's down-proj rows, weighted, + residual (atomic)
    // the prompt (prefill) megakernel: the T tokens of one sequence's prompt per launch
    OP_PNORM = 10,    // RMSNorm of 16 tokens' residual rows -> matrix-core operands (+ the residual carried on)
    OP_PQKV = 11,     // Q/K/V rows x a token block + RoPE -> query operands and K/V cache rows
    OP_PATTN = 12,    // causal attention of 16 query tokens for the heads of one KV group
    OP_POPROJ = 13,   // O-proj rows x a token block over one K slice, added to the residual (atomic)
    OP_PGU = 14,      // gate/up rows x a token block + SiLU * up -> down-projection operands
    OP_PDOWN = 15,    // down-proj rows x a token block over one K slice, added to the residual (atomic)
    OP_PLM = 16,      // final RMSNorm'd last token x LM-head rows + argmax
    OP_COUNT = 17
};

constexpr uint32_t NONE = 0xFFFFFFFFu;

// Device-side capacities the tiling must respect.
constexpr int MAX_TILE_ROWS = 1024;  // rows x sequences of one GEMV tile (LDS row-result buffer)
constexpr int GROUP_SEQS = 16;       // sequences per column group (columns of one matrix-core operand)
constexpr int MAX_BATCH = 64;
// Argmax keys per sequence and step parity: LM-head tile i folds its maximum into slot i % KEY_SLOTS
// (one 64-bit atomic max per tile and sequence; spreading them keeps the tiles that finish together
// from queueing on one word), and the step's last tile reduces the slots.
constexpr int KEY_SLOTS = 16;
// Counter words per event with many producers (a task record's nsub of 8): producers add to one of
// CTR_SUBS words (by their XCD, then by workgroup), each on its own 128-byte line, and consumers sum
// them; events with few producers use word 0 alone.  (Measured on the 1B shape: 16 words against 8,
// 807.0 -> 800.3 us per step at batch 1 and 1530.3 -> 1518.3 us at batch 16; 32 words no better:
// the increments that end a phase arrive together and queue on their word.)
#ifndef MK_CTR_SUBS
#define MK_CTR_SUBS 16
#endif
constexpr int CTR_SUBS = MK_CTR_SUBS;
constexpr int CTR_LINE = 32;  // 32-bit words per counter line
static_assert(CTR_SUBS == 8 || CTR_SUBS == 16 || CTR_SUBS == 32 || CTR_SUBS == 64, "8..64 counter words per event");        // sequences per step: GEMV tiles run once per column group
constexpr int MAX_ACT = 4096;        // floats of one staged activation vector (LDS)

// Several-sequence QKV and gate/up tiles with K = 2048 are packed in two halves of K
// (chunk by chunk of halves_chunk_rows rows: all row groups of columns 0..1023, then
// of 1024..2047), so that their GEMV holds the operands of one half at a time.
constexpr int halves_chunk_rows(int B) { return (MAX_TILE_ROWS / (B < GROUP_SEQS ? B : GROUP_SEQS)) / 64 * 64; }
constexpr bool halves_packed(bool batched, int op, int kt) { return batched && kt == 2048 && (op == OP_QKV || op == OP_GATEUP); }

// The several-sequence path (batched GEMV tiles over column groups of sequences,
// attention chunk slots dealt per step and merged by the last chunk, operand regions) runs
// every step of more than one sequence and every mixture-of-experts step: expert
// routing is implemented there only, so one sequence with experts is a column group
// of one.
constexpr bool batched_path(int B, int E) { return B > 1 || E > 0; }

// Attention partials per (sequence, KV group): at most 16 chunks are merged; on the
// several-sequence path a sequence may take up to 16 of its group's chunk slots.
constexpr int ATTN_MAX_CHUNKS = 16;
constexpr int part_chunks(bool batched, int splits) { return batched ? ATTN_MAX_CHUNKS : splits; }

// One instruction of the interpreter: 48 bytes, read by the loader wave into LDS.
struct Task {
    uint8_t op;
    uint8_t wait_nsub;     // counter words of the awaited event: 1, or 8 for CTR_SUBS words
    uint8_t sig_nsub;      // counter words of the signalled event: 1, or 8 for CTR_SUBS words
    uint8_t flags;         // TaskFlags
    uint16_t layer;
    uint16_t part;         // QKV: head slot; ATTN/OPROJ: KV group; DOWN: K block; EGU/EDOWN: expert
    uint32_t row0;         // first output row (QKV: first RoPE pair; ATTN: chunk index)
    uint32_t nrows;        // output rows of the tile (QKV: pairs)
    uint32_t wait_ev;      // awaited event or NONE
    uint32_t wait_target;  // producers of the awaited event (per step)
    uint32_t sig_ev;       // signalled event or NONE
    uint32_t wbytes;       // bytes of weights streamed into LDS pages for this task
    uint64_t wofs;         // byte offset of those weights in the packed weight buffer
    uint32_t seq;          // ATTN: sequence (batch index); GEMV tiles: column group of 16 sequences
    uint32_t id;           // global task index (topological order)
};
static_assert(sizeof(Task) == 48, "task record is 48 bytes");

enum TaskFlags : uint8_t {
    TF_RESID = 1,    // OPROJ / DOWN: this tile also adds the residual input
    TF_SIGRANGE = 2, // ROUTE: signals the E consecutive events sig_ev .. sig_ev + E - 1
    TF_NGW2 = 4      // prompt GEMM tiles: two token groups of 16 per compute wave (128-token blocks), else one
};

// Prompt GEMM tiles: the tile's weights (rows x K slice) are stored page by page, each
// 16 KiB page holding every row of the tile over a 16 / (rows / 16) x 32-column stretch
// of K, as 16 x 32 matrix-core blocks in (column block, row group) order.
constexpr int PF_GEMMS = 4;  // QKV, O-proj, gate/up, down
constexpr int PF_MAX_SLICES = 4;  // K slices of the O- and down projections (their partials meet in the RMSNorm tasks)
constexpr int pf_kbp(int rows) { return 16 / (rows / 16); }  // 32-column blocks per page

// Tiling of one model on W workgroups (computed once on the host).
struct Tiling {
    int32_t L, h, nq, nkv, d, f, V, B, C, W;
    int32_t grp;          // query heads per KV head
    int32_t qkv_pairs;    // RoPE pairs per QKV tile (rows = 2 * pairs)
    int32_t attn_splits;  // KV chunks per (sequence, KV group)
    int32_t o_rows;       // O-proj tile rows (tile columns = grp * d)
    int32_t g_rows;       // gate rows per gate/up tile (same number of up rows)
    int32_t kd;           // down-proj K block (columns of m per tile)
    int32_t d_rows;       // down-proj tile rows
    int32_t lm_rows;      // LM-head rows per tile
    int32_t n_qkv_tiles, n_attn_tiles, n_o_tiles, n_gu_tiles, n_down_tiles, n_lm_tiles;  // per layer / total LM
    // mixture of experts (E = 0: dense FFN): E experts of expert_ffn fe rows, top-k
    // routing; expert gate/up tiles of r_gu rows of m (gate and up rows interleaved in
    // blocks of 32), expert down tiles of r_dn rows
    int32_t E, topk, fe, r_gu, r_dn;
    // prompt graph (mk_build_prefill; pf_T = 0 for a decode graph): tokens per launch, then per
    // GEMM (QKV, O-proj, gate/up, down): rows per tile (64 or 128; gate/up: half gate, half up
    // rows), token groups of 16 per compute wave (tokens per task: 64 ngw), K slices
    int32_t pf_T;
    int32_t pf_rows[PF_GEMMS], pf_ngw[PF_GEMMS], pf_slices[PF_GEMMS];
};

// Byte layout of the handle-owned packed weight buffer.
struct Layout {
    uint64_t gains;       // (2L+1) x h bf16: attn_norm[l], ffn_norm[l] (l = 0..L-1), final
    uint64_t embed;       // V x h
    uint64_t lm;          // LM-head tiles (a copy of its own even when tied to the embedding)
    uint64_t layer0;      // start of layer 0
    uint64_t layer_bytes; // bytes per layer
    uint64_t qkv, o, gu, down;  // offsets within a layer (dense FFN)
    uint64_t router, egu, edown;  // offsets within a layer (mixture of experts)
    uint64_t total;
};

// Export image (mk_export_graph / mk_plan_graph): header, then
// Task[n_tasks], uint32 target[n_events], uint32 nsub[n_events],
// uint32 queue_off[W+1], uint32 queue[n_tasks], uint32 order[n_tasks].
struct ExportHeader {
    uint32_t magic;       // 'MKG1'
    uint32_t version;     // 1
    uint32_t n_tasks, n_events, W, sched;
    int32_t L, h, nq, nkv, d, f, V, B, C;
    int32_t grp, qkv_pairs, attn_splits, o_rows, g_rows, kd, d_rows, lm_rows;
    uint32_t record_bytes;
    int32_t E, topk, fe, r_gu, r_dn;
    uint32_t reserved[2];
};
constexpr uint32_t EXPORT_MAGIC = 0x31474B4Du;

}  // namespace mk
