// Kernel parameter block and launch glue shared by the runtime (host) and the
// megakernel (device).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

// control words in Params::state (uint32 index; each on its own 128-byte line)
constexpr uint32_t ST_EPOCH = 0;    // step number of the next launch (starts at 1)
constexpr uint32_t ST_EXIT = 32;    // workgroups that finished (monotonic)
constexpr uint32_t ST_HEAD = 64;    // dynamic queue head (monotonic)
constexpr uint32_t ST_ABORT = 96;   // set when any wave gives up
constexpr uint32_t ST_ERR = 128;    // error record: code, workgroup, task, event, seen, target
constexpr uint32_t ST_TAIL = 160;   // event-driven dispatch: ready-queue slots reserved (monotonic)
constexpr uint32_t ST_WORDS = 192;

// per task: workgroup, fetch, inputs ready, staged, computed, end (signalled), results acknowledged, last
// page held, first page, last wave's epilogue issued, last wave's stores acknowledged, wave 0's epilogue
// issued, 4 reserved
constexpr int TRACE_WORDS = 16;

enum ErrCode : uint32_t { ERR_NONE = 0, ERR_TIMEOUT_EVENT = 1, ERR_TIMEOUT_LDS = 2, ERR_INPUT = 3 };

// Per-step pointers, passed by value with every launch.
struct StepArgs {
    const int32_t* tokens;    // [B]
    const int32_t* positions; // [B]
    uint16_t* kc;             // K cache [L][B][n_kv][C][d]
    uint16_t* vc;             // V cache
    float* logits;            // [B][V] or null (prompt launch: [V] of the last token)
    int32_t pos0;             // prompt launch: position of the first prompt token (tokens: [T])
};

// Everything else the kernel reads, resident in device memory for the life of the handle.
struct Params {
    const Task* tasks;
    const uint32_t* queue_off;
    const uint32_t* queue;
    uint32_t n_tasks;
    uint32_t sched;           // 0 static queues, 1 dynamic (atomic pop), 2 event-driven, 3 event-driven
                              // with scheduler waves
    // event-driven dispatch: producers per event, each event's dependents (CSR), the ready
    // queue [n_tasks] (the first n_init slots: the tasks that wait on no event, written once)
    // and the step that filled each of its slots
    const uint32_t* ev_target;
    const uint32_t* cons_off;
    const uint32_t* cons;
    uint32_t* rq;
    uint32_t* rq_stamp;
    uint32_t n_init;
    // scheduler waves (sched 3): the step that activated each event [n_events]; event ev
    // is in the activated-event queue of workgroup ev % W, which dispatches it
    uint32_t* aeq_stamp;
    uint32_t n_events;
    uint32_t* ctr;            // event counters [n_events][8 sub-counters][32 words]
    uint32_t* state;          // control words
    const uint8_t* w;         // packed weights
    const float2* rope;       // [max_ctx][head_dim/2] (cos, sin)
    float* q;                 // [B][n_q*d]
    float* part;              // [B][n_kv][S][grp][d+2]
    float* m;                 // [B][f]
    float* acc;               // [2][2L+1][B][h] residual accumulators (by step parity)
    // batch > 1: inputs of the O-projection and down-projection of all sequences as
    // matrix-core B operands, bf16 parts hi/lo of 16 x 32 column blocks (lane l:
    // sequence l % 16, columns 8 (l / 16) .. +7)
    uint16_t* xop;            // [L][2][nq*d/32][64][8] (merged attention), then [L][2][f/32][64][8] (SiLU(gate) * up)
    uint32_t* aticket;        // batch > 1: [2][L][B][n_kv] finished attention partials per step parity
    float* rlogit;            // MoE: [L][B][E] router logits
    int32_t* eids;            // MoE: [L][B][top_k] selected experts, in selection order
    float* hidden;            // [B][h]
    unsigned long long* key;  // [2][KEY_SLOTS][B] packed argmax keys
    uint32_t* ticket;         // [B]
    int32_t* next;            // [B]
    uint32_t* task_count;     // [n_tasks] or null
    unsigned long long* trace;  // [n_tasks][TRACE_WORDS] or null
    Tiling T;
    Layout lay;
    float eps;
    uint32_t drop_task;
    unsigned long long timeout;  // ticks of the 100 MHz device clock
};

// One strided copy of the weight repacking: rows x row_bytes from src (row pitch
// src_pitch) to dst + dst_off (rows contiguous).  row_bytes is a multiple of 16.
struct CopyOp {
    const uint8_t* src;
    uint64_t dst_off;
    uint64_t src_pitch;
    uint32_t rows, row_bytes;
};
hipError_t launch_repack(const CopyOp* ops, uint32_t n_ops, uint8_t* dst, hipStream_t stream);

// One GEMV weight tile of the repacking: `rows` rows (a multiple of 16) of kt
// bf16 columns, row r read from rowsrc[row_base + r] (null: zeros), written to
// dst + dst_off either row by row (blocked = 0) or as 16 x 32 matrix-core blocks
// (blocked = 1; block b = (row group b / (kt/32), column block b % (kt/32)),
// lane l of a block holds row 16*rg + l%16, columns 32*kb + 8*(l/16) .. +7).
struct TileOp {
    uint64_t dst_off;
    uint32_t row_base, rows, kt, blocked;  // blocked: 0 row-major, 1 matrix-core blocks, 2 the same in K halves,
                                           // 3 prompt GEMM pages (page, then column block, then row group)
    uint32_t chunk_rows;                   // blocked == 2: rows per chunk
};
hipError_t launch_repack_tiles(const TileOp* ops, uint32_t n_ops, const uint8_t* const* rowsrc, uint8_t* dst,
                               hipStream_t stream);

hipError_t launch_step(const Params* dparams, const StepArgs& a, uint32_t grid, hipStream_t stream, bool cooperative);
// the prompt megakernel: same interpreter, prompt operations
hipError_t launch_prefill(const Params* dparams, const StepArgs& a, uint32_t grid, hipStream_t stream, bool cooperative);

// Fill spans (poison mode, and the allocation-free step's clears): up to MAX_SPANS spans of
// 32-bit words, each filled with a pattern before a step.
constexpr int MAX_SPANS = 12;
struct PoisonSpans {
    void* ptr[MAX_SPANS];
    uint64_t words[MAX_SPANS];
    uint32_t pattern[MAX_SPANS];
    int32_t n;
};
hipError_t launch_poison(const PoisonSpans& s, hipStream_t stream);

// The allocation-free step: its scratch is a file-scope device array of this many bytes, one per GPU.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
constexpr int MAX_DEVICES = 64;
// Device address of the current device's copy of that array (`device` is the current device's id),
// looked up once per device and kept.
hipError_t noalloc_scratch_base(int device, uint8_t** out);
int step_threads();
size_t step_lds_bytes();
const void* step_kernel_ptr();
const void* prefill_kernel_ptr();

}  // namespace mk
