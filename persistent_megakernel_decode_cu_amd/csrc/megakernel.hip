// Persistent decode megakernel for gfx950 (MI355X).
//
// One launch runs one decode step.  Each workgroup owns one CU (the ~150 KiB of
// LDS it declares leaves room for no second one) and runs an interpreter over
// a queue of tile tasks (koas-w.github.io megakernel notes, "on-GPU
// interpreter / persistent kernel"; Hazy Research megakernel news page,
// section 4, "fusion big bang").  The workgroup has six waves:
//
//   waves 4-5 (loaders): fetch task records (static: the workgroup's queue;
//     dynamic: an atomic pop from one global queue, koas-w.github.io notes,
//     "static and dynamic scheduling"; event-driven: slots of a ready queue)
//     into an LDS FIFO (wave 4), and stream every task's weights (attention:
//     its KV-cache chunk) into a ring of eight 16 KiB LDS pages with
//     global_load_lds_dwordx4, each loader wave issuing half of every page.  Weights never depend on activations, so the
//     loader runs ahead of the compute waves as far as free pages allow: the
//     next tasks' weights arrive while the current task still waits on its
//     inputs (Hazy page, section 4, "shared memory to remove memory bubbles":
//     paged shared memory; pages released by one instruction are handed to the
//     next one so it can start its loads early).  The loader keeps its vector
//     memory counter for the page loads alone: task records and parameters are
//     read with scalar loads, control words through LDS.
//   waves 0-3 (compute): wait for the task's event counter, stage its
//     activations into LDS, run the op out of the LDS pages, store results and
//     add one to the event the task completes (Hazy page, section 4,
//     "synchronisation"; MPK news page, part 2: fetch, execute, trigger event).
//
// Cross-CU data (activations, partial sums, counters) is written with
// device-scope (sc1) stores or atomics, waited for with s_waitcnt, and read
// with device-scope loads; no L2 write-back or invalidate is issued inside the
// step.  Weights and the KV-cache prefix come from earlier launches and use
// ordinary (LDS-DMA) loads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mk_internal.h"
#include "runtime.h"

namespace mk {

constexpr int NCW = 4;                 // compute waves
constexpr int NLW = 2;                 // loader waves; each issues every NLW-th 1 KiB load of every page
constexpr int NTHREADS = (NCW + NLW) * 64;
constexpr int PAGE = 16384;            // LDS page (bytes)
constexpr int NPAGES = 8;              // ring of 8 pages = 128 KiB
constexpr int FIFO = 16;               // task records in flight in LDS
constexpr int XS = MAX_ACT;            // activation staging (floats)
constexpr int ROWRES = MAX_TILE_ROWS;  // per-task row results (floats)
constexpr int LPP = 16 / NLW;          // loads per page per loader wave
// Pages in flight per loader wave: two, i.e. 32 KiB per CU and 8 MiB over the chip.  That keeps HBM
// busy; every deeper queue only adds queueing delay to the small latency-critical loads and stores
// between dependent tasks, which share the CU's memory pipeline with the page loads (measured: 3 -> 2
// pages saved 4 us per step at batch 1 and 8 us at batch 16; 4 cost 2 us).
#ifndef MK_MAX_INFLIGHT
#define MK_MAX_INFLIGHT 2
#endif
constexpr int MAX_INFLIGHT = MK_MAX_INFLIGHT;
// Pages in flight per loader wave while it streams an attention task's KV rows.
#ifndef MK_ATTN_INFLIGHT
#define MK_ATTN_INFLIGHT MK_MAX_INFLIGHT
#endif
constexpr int ATTN_INFLIGHT = MK_ATTN_INFLIGHT;
#ifndef MK_PF_INFLIGHT
#define MK_PF_INFLIGHT 6
#endif
constexpr int PF_INFLIGHT = MK_PF_INFLIGHT;  // the prompt megakernel's loader depth
static_assert(PF_INFLIGHT >= 1 && PF_INFLIGHT < NPAGES && LPP * PF_INFLIGHT <= 63, "vmcnt range");
static_assert(ATTN_INFLIGHT >= 1 && ATTN_INFLIGHT <= NPAGES && LPP * ATTN_INFLIGHT <= 63, "vmcnt range");
constexpr int DYNQ = 64;               // popped task ids shared between the loader waves (dynamic queue)
constexpr int MAXB = 64;               // sequences per step held in LDS

struct __attribute__((aligned(16))) Smem {
    float xs[XS];
    float rowres[ROWRES];
    Task fifo[FIFO];
    float wsc[NCW][256];  // attention: softmax weights of up to 4 pages per wave
    int32_t pos[MAXB];
    int32_t tok[MAXB];
    StepArgs args;
    uint32_t fifo_first_page[FIFO];
    uint32_t fifo_ready[FIFO];
    uint32_t fifo_free[FIFO];
    uint32_t page_ready[NLW][NPAGES];  // per loader wave: uses of the slot it has published
    uint32_t page_free[NPAGES];   // compute-wave releases (NCW per use of the slot)
    uint32_t dyn_tid[DYNQ];
    uint32_t dyn_ready, dyn_ack;
    uint32_t go, cbar, done, abort;
    uint32_t cgen[NCW];  // compute-wave barrier generation (per wave)
    float ssq[NCW];      // per-wave partial sums of squares of the staged activation
    float ssqb[NCW][GROUP_SEQS];  // batch > 1: per-wave, per-sequence partial sums of squares
    float rwb[GROUP_SEQS];        // expert down tiles: the expert's routing weight per sequence
    int32_t rtop[GROUP_SEQS];     // expert down tiles: 1 if the expert is the sequence's first choice
    uint32_t t_ready_lo, t_ready_hi;
    uint32_t tm[4];  // trace: low 32 bits of the clock after staging / after the GEMV
    uint32_t tw_epi[NCW], tw_ack[NCW];  // trace: per wave, epilogue issued / its stores acknowledged
    uint32_t trace_on;                  // 1 when the handle records a trace: the clock is read only then
    // trace, loader wave 0: per FIFO slot, when the task's first and last pages were issued and when
    // its last page was published; per ring slot, the FIFO slot of the task whose page it holds
    uint32_t tl_issue0[FIFO], tl_issue1[FIFO], tl_pub[FIFO];
    uint32_t pg_fslot[NPAGES];
    // several sequences: this step's deal of every KV group's attention slots (attn_deal)
    uint32_t amap[MAX_BATCH * ATTN_MAX_CHUNKS];  // slot -> sequence << 8 | chunk, 0xffff: empty
    uint32_t alen[MAX_BATCH];                    // chunk length of each sequence (positions)
    uint32_t anch[MAX_BATCH];                    // non-empty chunks of each sequence
    uint32_t adealt;                             // 1 once loader wave 0 has dealt this step's slots
};

__shared__ Smem S;
// The page ring is its own LDS object so that LDS accesses of the loader to the
// control words can be told apart from its in-flight LDS-DMA writes.
__shared__ __attribute__((aligned(16))) uint8_t ring[NPAGES][PAGE];

typedef const __attribute__((address_space(4))) Params CParams;
typedef __attribute__((address_space(3))) volatile uint32_t lds_u32;
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) unsigned long long g_u64;
typedef __attribute__((address_space(1))) uint16_t g_u16;

// ---- small device helpers -----------------------------------------------------

__device__ __forceinline__ uint64_t rtc() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 7u; }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
// A pointer every lane holds the same value of (say, read from LDS), made visibly
// wave-uniform: a buffer resource built from it then needs no per-lane loop.
template <class T>
__device__ __forceinline__ T* uni_ptr(T* ptr) {
    const uint64_t v = (uint64_t)ptr;
    return (T*)(((uint64_t)uni((uint32_t)(v >> 32)) << 32) | (uint64_t)uni((uint32_t)v));
}

// Params are read through the constant address space with a wave-uniform pointer: scalar loads.
__device__ __forceinline__ CParams& P(const Params* pp) {
    uint64_t v = (uint64_t)pp;
    uint32_t lo = uni((uint32_t)v), hi = uni((uint32_t)(v >> 32));
    return *(CParams*)(((uint64_t)hi << 32) | lo);
}

// Plain global loads/stores through the global address space (generic pointers
// would give flat instructions, which also count against lgkmcnt).
template <class T>
__device__ __forceinline__ T gld(const T* ptr) {
    return *(const __attribute__((address_space(1))) T*)ptr;
}
template <class T>
__device__ __forceinline__ void gst(T* ptr, T v) {
    *(__attribute__((address_space(1))) T*)ptr = v;
}
// vector types (HIP's uint4/float2 are classes): load through clang vector types
__device__ __forceinline__ uint4 gld_u4(const void* ptr) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = *(const __attribute__((address_space(1))) v4u*)ptr;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float2 gld_f2(const void* ptr) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const v2f v = *(const __attribute__((address_space(1))) v2f*)ptr;
    return make_float2(v.x, v.y);
}

__device__ __forceinline__ uint32_t lds_ld(const uint32_t& x) { return *(lds_u32*)&x; }
__device__ __forceinline__ void lds_st(uint32_t& x, uint32_t v) { *(lds_u32*)&x = v; }
__device__ __forceinline__ void lds_add(uint32_t& x, uint32_t v) {
    __hip_atomic_fetch_add(&x, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load((g_u32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ldf_dev(const float* p) { return __uint_as_float(ld_dev((const uint32_t*)p)); }
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stf_dev(float* p, float v) { st_dev((uint32_t*)p, __float_as_uint(v)); }
__device__ __forceinline__ void addf_dev(float* p, float v) {
    __hip_atomic_fetch_add((g_f32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t addu_dev(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-bit device-scope store (a plain store with the sc1 bit; each lane its own address)
__device__ __forceinline__ void st16_dev(uint16_t* p, uint16_t v) {
    __hip_atomic_store((g_u16*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cross-check build of the synchronisation protocol (-DMK_FENCED=1): agent-scope release fences before
// every signal (counter, ticket or ready-queue stamp) and agent-scope acquire fences after every wait
// that a signal ends, as the memory model's generic sequences would have them.  The default build
// issues none: every datum read across CUs is written and read with device-scope (sc1) accesses, and a
// producer waits for its stores to be acknowledged before it signals.
#ifndef MK_FENCED
#define MK_FENCED 0
#endif
__device__ __forceinline__ void release_fence() {
    if constexpr (MK_FENCED) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void acquire_fence() {
    if constexpr (MK_FENCED) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void lgkm_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float dot8(uint4 w, const float* x, float a) {
    a = fmaf(bf16lo(w.x), x[0], a);
    a = fmaf(bf16hi(w.x), x[1], a);
    a = fmaf(bf16lo(w.y), x[2], a);
    a = fmaf(bf16hi(w.y), x[3], a);
    a = fmaf(bf16lo(w.z), x[4], a);
    a = fmaf(bf16hi(w.z), x[5], a);
    a = fmaf(bf16lo(w.w), x[6], a);
    a = fmaf(bf16hi(w.w), x[7], a);
    return a;
}

// Sum over each row of 16 lanes with DPP (every lane of the row gets the row sum).
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true)); // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true)); // row_ror:8
    return v;
}
// Sum over the wave, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true)));
    const float a = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)));
    const float b = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
    return fmaxf(a, b);
}
// Top-k routing of one sequence, lane j holding the router logit v of expert j (j < E):
// expert j's rank is the number of experts with a larger logit, or an equal one and a
// lower id; the k of rank < k are selected, in rank order, and weighted by the softmax
// over the selected logits.  Returns the weight of expert e (0 if not selected) and
// sets slot to its rank (-1 if not selected).  Wave-uniform results.  Expert e's own
// rank takes one ballot; only if e is selected are all ranks counted for the softmax.
__device__ __forceinline__ float route_weight(float v, int lane, int E, int K, int e, int& slot) {
    const float ve = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), e));
    const int rank_e = __popcll(__ballot(lane < E && (v > ve || (v == ve && lane < e))));
    slot = -1;
    if (rank_e >= K) return 0.f;
    slot = rank_e;
    int rank = 0;
    for (int j = 0; j < E; ++j) {
        const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
        rank += (vj > v || (vj == v && j < lane)) ? 1 : 0;
    }
    const bool sel = lane < E && rank < K;
    const float top = wave_max(lane < E ? v : -INFINITY);
    const float ex = sel ? __expf(v - top) : 0.f;
    const float z = wave_sum(ex);
    return __expf(ve - top) / z;
}
// Sum over aligned segments of W lanes (W = 8, 16, 32); every lane gets its segment's sum.
template <int W>
__device__ __forceinline__ float seg_sum(float v) {
    if constexpr (W >= 16) {
        v = row16_sum(v);
        if constexpr (W == 32) v += __shfl_xor(v, 16, 64);
    } else {
#pragma unroll
        for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    }
    return v;
}

__device__ __forceinline__ uint32_t ctr_index(uint32_t ev, uint32_t sub) { return (ev * CTR_SUBS + sub) * CTR_LINE; }
// The counter words a consumer sums (a task record's nsub is 1 or 8)
__device__ __forceinline__ uint32_t ctr_words(uint32_t nsub) { return nsub == 8u ? (uint32_t)CTR_SUBS : 1u; }
// One poll: lane i < ctr_words(nsub) reads word i, the wave sums them
__device__ __forceinline__ uint32_t ctr_sum(const uint32_t* ctr, uint32_t ev, uint32_t nsub, int lane) {
    uint32_t v = (uint32_t)lane < ctr_words(nsub) ? ld_dev(&ctr[ctr_index(ev, lane)]) : 0u;
#pragma unroll
    for (int o = 1; o < CTR_SUBS; o <<= 1) v += __shfl_xor(v, o, 64);
    return __builtin_amdgcn_readfirstlane(v);
}

// ---- error path -------------------------------------------------------------------

__device__ __noinline__ void raise_error(const Params* pp, uint32_t code, uint32_t task, uint32_t ev, uint32_t seen,
                                         uint32_t target) {
    CParams& p = P(pp);
    uint32_t* st = p.state;
    uint32_t expected = 0u;
    if (__hip_atomic_compare_exchange_strong((g_u32*)&st[ST_ERR], &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
        st_dev(&st[ST_ERR + 1], blockIdx.x);
        st_dev(&st[ST_ERR + 2], task);
        st_dev(&st[ST_ERR + 3], ev);
        st_dev(&st[ST_ERR + 4], seen);
        st_dev(&st[ST_ERR + 5], target);
    }
    st_dev(&st[ST_ABORT], 1u);
    lds_st(S.abort, 1u);
}

// Spin until an LDS word reaches v.  Returns false on abort or timeout.
__device__ __noinline__ bool lds_wait_slow(const uint32_t& w, uint32_t v, const Params* pp, uint32_t task) {
    uint64_t t0 = 0;
    uint32_t it = 0;
    while (lds_ld(w) < v) {
        if (lds_ld(S.abort)) return false;
        if ((++it & 255u) == 0u) {
            CParams& p = P(pp);
            const uint64_t now = rtc();
            if (t0 == 0) {
                t0 = now;
            } else if (now - t0 > 2 * p.timeout) {  // longer than an event wait: the stalled event is reported first
                raise_error(pp, ERR_TIMEOUT_LDS, task, NONE, lds_ld(w), v);
                return false;
            }
            if (ld_dev(&p.state[ST_ABORT])) {
                lds_st(S.abort, 1u);
                return false;
            }
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}

__device__ __forceinline__ bool lds_wait_ge(const uint32_t& w, uint32_t v, const Params* pp, uint32_t task) {
    if (lds_ld(w) >= v) return true;
    return uni(lds_wait_slow(w, v, pp, task)) != 0;
}

// Compute wave 0: wait until the event's sub-counters sum to `want`.
__device__ __noinline__ bool wait_event(const Params* pp, uint32_t ev, uint32_t nsub, uint32_t want, uint32_t task) {
    CParams& p = P(pp);
    const int lane = threadIdx.x & 63;
    const uint64_t t0 = rtc();
    uint32_t it = 0;
    const uint32_t* ctr = p.ctr;
    for (;;) {
        const uint32_t sum = ctr_sum(ctr, ev, nsub, lane);
        if (sum >= want) return true;
        if (lds_ld(S.abort)) return false;
        if ((++it & 63u) == 0u) {
            if (ld_dev(&p.state[ST_ABORT])) {
                lds_st(S.abort, 1u);
                return false;
            }
            if (rtc() - t0 > p.timeout) {
                raise_error(pp, ERR_TIMEOUT_EVENT, task, ev, sum, want);
                return false;
            }
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// ---- geometry shared by loader and compute -------------------------------------------

struct Chunk {
    int32_t c0, c1, P;  // chunk positions [c0, c1) of 0..P; prefix rows in LDS are [c0, min(c1, P))
};
// Chunk c of the one context 0..P at batch 1: one of `splits` equal parts of it.
__device__ __forceinline__ Chunk attn_chunk(int32_t splits, int32_t P, uint32_t c) {
    const int32_t n = P + 1;
    const int32_t lc = (n + splits - 1) / splits;
    Chunk ch;
    ch.P = P;
    ch.c0 = min(n, (int32_t)c * lc);
    ch.c1 = min(n, ch.c0 + lc);
    return ch;
}
// one page holds 8 KiB of K rows then 8 KiB of V rows of consecutive positions
__device__ __forceinline__ int32_t attn_block_rows(int32_t d) { return 4096 / d; }
// attention on the matrix cores (head_dim 64, at most 4 query heads per KV head), whose
// K pages are row-major with XOR-swizzled 16-byte chunks
__device__ __forceinline__ bool attn_kswizzle(int32_t d, int32_t grp) { return d == 64 && grp <= 4; }

__device__ __forceinline__ int32_t seq_pos(uint32_t b) { return (int32_t)lds_ld(*(const uint32_t*)&S.pos[b]); }

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 64; o *= 2) v += (uint32_t)__shfl_xor((int)v, o, 64);
    return uni(v);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 64; o *= 2) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return uni(v);
}

// Several sequences: the B x S attention tasks of each KV group and layer (task slot
// j = seq * S + chunk of the record) are dealt to the sequences in proportion to their
// contexts, at every step, so that the step's attention tasks carry about the same
// number of positions whatever the mix of context lengths (split-KV decode load
// balance).  The chunk length L is the smallest whole number of pages with
// sum_b ceil(n_b / L) <= B S and at most 16 chunks per sequence (n_b = P_b + 1);
// sequence b takes s_b = ceil(n_b / L) consecutive slots in sequence order, with chunks
// of len_b = ceil(n_b / s_b) rounded up to whole pages, and the slots past the last
// non-empty chunk stay empty.  Every workgroup computes the same deal from the
// positions; loader wave 0 does it (one wave, lane = sequence) before it hands the
// first attention task of the step to the compute waves.
__device__ __noinline__ void attn_deal(CParams& p, int lane) {
    const int B = p.T.B, T = B * p.T.attn_splits;
    const uint32_t pb = (uint32_t)(4096 / p.T.d);
    const bool mine = lane < B;
    const uint32_t n = mine ? (uint32_t)min(max(seq_pos((uint32_t)lane) + 1, 1), p.T.C) : 0u;
    const uint32_t nmax = wave_max_u32(n);
    uint32_t lo = max(1u, (nmax + ATTN_MAX_CHUNKS * pb - 1) / (ATTN_MAX_CHUNKS * pb)), hi = (nmax + pb - 1) / pb;
    while (lo < hi) {  // wave-uniform bisection over the chunk length in pages
        const uint32_t mid = (lo + hi) / 2, L = mid * pb;
        if (wave_sum_u32(mine ? (n + L - 1) / L : 0u) <= (uint32_t)T) hi = mid;
        else lo = mid + 1;
    }
    const uint32_t L = lo * pb;
    const uint32_t sl = mine ? (n + L - 1) / L : 0u;
    const uint32_t len = mine ? ((n + sl - 1) / sl + pb - 1) / pb * pb : 0u;
    const uint32_t nch = mine ? (n + len - 1) / len : 0u;
    uint32_t incl = sl;  // inclusive prefix sum of the slots over the sequences
#pragma unroll
    for (int o = 1; o < 64; o *= 2) {
        const uint32_t t = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += t;
    }
    const uint32_t base = incl - sl, used = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (mine) {
        S.alen[lane] = len;
        S.anch[lane] = nch;
        for (uint32_t c = 0; c < sl; ++c) S.amap[base + c] = c < nch ? (((uint32_t)lane << 8) | c) : 0xffffu;
    }
    for (uint32_t j = used + (uint32_t)lane; j < (uint32_t)T; j += 64) S.amap[j] = 0xffffu;
}

// The chunk of attention task k: batch 1, chunk row0 of the one context; several
// sequences, the slot the deal gave it (an empty slot: b = 0 and c0 = c1 = P + 1).
struct AttnTask {
    int32_t b, c, nch;  // sequence, chunk, non-empty chunks of the sequence (several sequences)
    Chunk ch;
};
__device__ __forceinline__ AttnTask attn_task(CParams& p, const Task& k) {
    AttnTask a;
    if (!batched_path(p.T.B, p.T.E)) {
        a.b = (int32_t)k.seq;
        a.c = (int32_t)k.row0;
        a.nch = p.T.attn_splits;
        a.ch = attn_chunk(p.T.attn_splits, seq_pos(k.seq), k.row0);
        return a;
    }
    const uint32_t e = lds_ld(S.amap[k.seq * (uint32_t)p.T.attn_splits + k.row0]);
    if (e == 0xffffu) {
        a.b = 0;
        a.c = 0;
        a.nch = 0;
        a.ch.P = seq_pos(0);
        a.ch.c0 = a.ch.c1 = a.ch.P + 1;
        return a;
    }
    a.b = (int32_t)uni(e >> 8);
    a.c = (int32_t)uni(e & 0xffu);
    a.nch = (int32_t)uni(lds_ld(S.anch[a.b]));
    const int32_t len = (int32_t)uni(lds_ld(S.alen[a.b]));
    a.ch.P = (int32_t)uni((uint32_t)seq_pos((uint32_t)a.b));
    a.ch.c0 = min(a.ch.P + 1, a.c * len);
    a.ch.c1 = min(a.ch.P + 1, a.ch.c0 + len);
    return a;
}

__device__ __forceinline__ uint32_t task_pages(CParams& p, const Task& k, int32_t d) {
    if (k.op == OP_ATTN) {
        const Chunk ch = attn_task(p, k).ch;
        const int32_t npre = max(0, min(ch.c1, ch.P) - ch.c0);
        const int32_t pb = attn_block_rows(d);
        return (uint32_t)((npre + pb - 1) / pb);
    }
    return (k.wbytes + PAGE - 1) / PAGE;
}

// ---- loader wave ---------------------------------------------------------------------

// 16 bytes per lane from global memory straight into LDS, non-temporal: weights
// and KV rows are read once per step, so they are marked evict-first in L2.
constexpr int CPOL_NT = 2;
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, CPOL_NT);
}

// The LPP loads of loader wave lw for page kp of task k into ring slot `slot`.
__device__ __forceinline__ void issue_page(CParams& p, const Task& k, uint32_t kp, uint32_t slot, int lane, int lw) {
    uint8_t* const dst = &ring[slot][0];
    if (k.op == OP_ATTN) {
        const int32_t d = p.T.d;
        const AttnTask at = attn_task(p, k);
        const Chunk ch = at.ch;
        const int32_t pb = attn_block_rows(d);
        const int32_t p0 = ch.c0 + (int32_t)kp * pb;
        const int32_t rows = min(pb, min(ch.c1, ch.P) - p0);
        const uint32_t valid = (uint32_t)rows * (uint32_t)d * 2u;
        const uint64_t row = (((uint64_t)k.layer * p.T.B + (uint32_t)at.b) * p.T.nkv + k.part) * (uint64_t)p.T.C + (uint64_t)p0;
        const uint8_t* kb = (const uint8_t*)S.args.kc + row * d * 2;
        const uint8_t* vb = (const uint8_t*)S.args.vc + row * d * 2;
        // K: for the matrix-core attention (head_dim 64, up to 4 heads per group) rows stay
        // row-major with the 16-byte chunks of row r XOR-swizzled by r % 8, so every load
        // reads 1 KiB of consecutive K rows and the operand reads (16 rows, one chunk) hit
        // distinct banks; otherwise 16-byte-column-major order (column chunk c of all pb
        // rows, then c + 1, ...: a lane per position reads its chunk without bank
        // conflicts).  V stays row-major.  Rows past the valid ones repeat the last valid row.
        const bool swz = attn_kswizzle(p.T.d, p.T.grp);
#pragma unroll
        for (int i = 0; i < LPP; ++i) {
            const int j = i * NLW + lw;  // 1 KiB load j of the page: K for j < 8, V after
            uint32_t off;
            if (j < 8) {
                const uint32_t e = (uint32_t)(j * 64 + lane);  // 16-byte element of the K block
                if (swz) {
                    const uint32_t r = e / 8u, c = (e % 8u) ^ (r & 7u);
                    off = min(r, (uint32_t)rows - 1u) * (uint32_t)d * 2u + c * 16u;
                } else {
                    const uint32_t c = e / (uint32_t)pb, r = min(e % (uint32_t)pb, (uint32_t)rows - 1u);
                    off = r * (uint32_t)d * 2u + c * 16u;
                }
            } else {
                off = min((uint32_t)((j - 8) * 1024 + lane * 16), valid - 16u);
            }
            dma16((j < 8 ? kb : vb) + off, dst + j * 1024);
        }
    } else {
        const uint8_t* base = p.w + k.wofs + (uint64_t)kp * PAGE;
        const uint32_t valid = min((uint32_t)PAGE, k.wbytes - kp * PAGE);
#pragma unroll
        for (int i = 0; i < LPP; ++i) {
            const int j = i * NLW + lw;
            const uint32_t off = min((uint32_t)(j * 1024 + lane * 16), valid - 16u);
            dma16(base + off, dst + j * 1024);
        }
    }
}

// ---- event-driven dispatch --------------------------------------------------------------

// Wait until slot `slot` of the ready queue has been filled in step `epoch`.
__device__ __noinline__ bool wait_ready_slot(const Params* pp, uint32_t slot, uint32_t epoch) {
    CParams& p = P(pp);
    const uint64_t t0 = rtc();
    for (uint32_t it = 1;; ++it) {
        if (uni(ld_dev(&p.rq_stamp[slot])) == epoch) {
            acquire_fence();
            return true;
        }
        if (lds_ld(S.abort)) return false;
        if ((it & 63u) == 0u) {
            if (ld_dev(&p.state[ST_ABORT])) {
                lds_st(S.abort, 1u);
                return false;
            }
            if (rtc() - t0 > p.timeout) {
                raise_error(pp, ERR_TIMEOUT_EVENT, NONE, NONE, slot, epoch);
                return false;
            }
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// The activated event ev launches its dependents: the whole wave appends them to the
// ready queue (ids first, then, once those are stored, the step number of each slot).
__device__ __noinline__ void launch_dependents(const Params* pp, uint32_t ev, uint32_t epoch, int lane) {
    CParams& p = P(pp);
    const uint32_t c0 = p.cons_off[ev], n = p.cons_off[ev + 1] - c0;
    if (n == 0) return;
    uint32_t base = 0;
    if (lane == 0) base = addu_dev(&p.state[ST_TAIL], n);
    base = uni(base) - (epoch - 1u) * (p.n_tasks - p.n_init) + p.n_init;
    if (base < p.n_init || base + n > p.n_tasks) {  // an event activated twice in a step: never expected
        if (lane == 0) raise_error(pp, ERR_TIMEOUT_EVENT, NONE, ev, base, p.n_tasks);
        return;
    }
    for (uint32_t j = (uint32_t)lane; j < n; j += 64) st_dev(&p.rq[base + j], p.cons[c0 + j]);
    vm_wait_all();
    release_fence();
    for (uint32_t j = (uint32_t)lane; j < n; j += 64) st_dev(&p.rq_stamp[base + j], epoch);
    vm_wait_all();
}

// Scheduler waves (sched 3; MPK news page, part 2: scheduler units with activated-event
// queues that hand the dependents of each activated event to the workers).  The worker
// whose count activates an event posts it (stamps it with the step); event ev sits in the
// activated-event queue of workgroup ev % W, whose second loader wave is that queue's
// scheduler: it takes its events in id order (a topological order) and launches each
// one's dependents into the ready queue the workers pop.  It serves its queue while it
// waits for its next task and, after its last one, until every event of its queue has
// been dispatched.
//
// One pass over the queue without blocking: dispatch the events that have been posted,
// in order, up to the first that has not.
__device__ __forceinline__ void serve_events(const Params* pp, uint32_t epoch, int lane, uint32_t& next_ev) {
    CParams& p = P(pp);
    while (next_ev < p.n_events && uni(ld_dev(&p.aeq_stamp[next_ev])) == epoch) {
        acquire_fence();
        launch_dependents(pp, next_ev, epoch, lane);
        next_ev += gridDim.x;
    }
}
// Serve the queue until the LDS word w reaches v (the next task handed over), bounded in time.
__device__ __noinline__ bool serve_until(const Params* pp, uint32_t epoch, int lane, uint32_t& next_ev,
                                         const uint32_t& w, uint32_t v) {
    CParams& p = P(pp);
    const uint64_t t0 = rtc();
    for (uint32_t it = 1;; ++it) {
        if (uni(lds_ld(w)) >= v) return true;
        serve_events(pp, epoch, lane, next_ev);
        if (lds_ld(S.abort)) return false;
        if ((it & 63u) == 0u) {
            if (ld_dev(&p.state[ST_ABORT])) {
                lds_st(S.abort, 1u);
                return false;
            }
            if (rtc() - t0 > 2 * p.timeout) {
                raise_error(pp, ERR_TIMEOUT_LDS, NONE, NONE, lds_ld(w), v);
                return false;
            }
        }
        __builtin_amdgcn_s_sleep(1);
    }
}
// After the scheduler's last task: dispatch the rest of its queue, bounded in time.
__device__ __noinline__ void serve_rest(const Params* pp, uint32_t epoch, int lane, uint32_t& next_ev) {
    CParams& p = P(pp);
    const uint64_t t0 = rtc();
    for (uint32_t it = 1; next_ev < p.n_events; ++it) {
        serve_events(pp, epoch, lane, next_ev);
        if (next_ev >= p.n_events || lds_ld(S.abort)) return;
        if ((it & 63u) == 0u) {
            if (ld_dev(&p.state[ST_ABORT])) {
                lds_st(S.abort, 1u);
                return;
            }
            if (rtc() - t0 > p.timeout) {
                raise_error(pp, ERR_TIMEOUT_EVENT, NONE, next_ev, 0, epoch);
                return;
            }
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

typedef const __attribute__((address_space(4))) uint32_t c_u32;
typedef const __attribute__((address_space(4))) Task c_task;

// Loader wave lw of NLW.  All loader waves walk the same task sequence and the
// same page sequence; each issues its share of every page and publishes it with
// an LDS add.  Wave 0 also feeds the compute waves' task FIFO and, for the
// dynamic queue, pops task ids and hands them to the other loader waves.  Every
// wait first drains and publishes the loads in flight, so a page a consumer
// waits for is never held back by a waiting loader.
// INFL: pages in flight per loader wave before it waits for the oldest (the decode step: MAX_INFLIGHT;
// the prompt megakernel's GEMM tiles consume pages faster and keep more in flight)
template <int INFL>
__device__ __noinline__ void loader(const Params* pp, uint32_t epoch, int lw) {
    CParams& p = P(pp);
    lw = (int)uni((uint32_t)lw);
    const int lane = threadIdx.x & 63;
    const uint32_t W = gridDim.x;
    c_u32* qoff = (c_u32*)p.queue_off;
    c_u32* queue = (c_u32*)p.queue;
    c_task* tasks = (c_task*)p.tasks;
    const uint32_t sched = p.sched;
    const uint32_t n_tasks = p.n_tasks;
    const int32_t hd = p.T.d;
    const bool deal = batched_path(p.T.B, p.T.E);
    bool dealt = false;
    uint32_t qbeg = 0, qend = 0;
    if (sched == 0) {
        qbeg = qoff[blockIdx.x];
        qend = qoff[blockIdx.x + 1];
    }
    uint32_t pseq = 0, pub = 0;  // next page to issue / to publish
    const bool tr = lw == 0 && uni(lds_ld(S.trace_on)) != 0;
    uint32_t next_ev = blockIdx.x;  // scheduler waves: the next event of this workgroup's queue

    auto publish_one = [&]() {
        if (lane == 0) lds_st(S.page_ready[lw][pub % NPAGES], pub / NPAGES + 1);
        if (tr && lane == 0) lds_st(S.tl_pub[lds_ld(S.pg_fslot[pub % NPAGES])], (uint32_t)rtc());
        ++pub;
    };
    auto drain = [&]() {
        vm_wait_all();
        while (pub < pseq) publish_one();
    };

    for (uint32_t t = 0;; ++t) {
        bool end;
        uint32_t ti;
        if (sched == 0) {
            end = qbeg + t >= qend;
            ti = end ? 0u : queue[qbeg + t];
        } else if (lw == 0) {
            drain();
            uint32_t old = 0;
            if (lane == 0) old = addu_dev(&p.state[ST_HEAD], 1u);
            old = uni(old);
            const uint32_t rel = old - (epoch - 1u) * (n_tasks + W);
            end = rel >= n_tasks;
            ti = end ? NONE : rel;
            if (sched >= 2 && !end) {
                // event-driven: slot rel of the ready queue, once a completed event has filled it
                if (rel >= p.n_init && !wait_ready_slot(pp, rel, epoch)) break;
                ti = uni(ld_dev(&p.rq[rel]));
            }
            if (NLW > 1) {
                if (lds_ld(S.dyn_ack) + DYNQ < t + 1 && !uni(lds_wait_ge(S.dyn_ack, t + 1 - DYNQ, pp, ti))) break;
                if (lane == 0) lds_st(S.dyn_tid[t % DYNQ], ti);
                lgkm_wait_all();
                if (lane == 0) lds_st(S.dyn_ready, t + 1);
            }
            if (end) ti = 0u;
        } else {
            if (lds_ld(S.dyn_ready) < t + 1) {
                drain();
                if (sched == 3) {
                    if (!uni(serve_until(pp, epoch, lane, next_ev, S.dyn_ready, t + 1))) break;
                } else if (!uni(lds_wait_ge(S.dyn_ready, t + 1, pp, NONE))) {
                    break;
                }
            }
            ti = uni(lds_ld(S.dyn_tid[t % DYNQ]));
            lgkm_wait_all();
            if (lane == 0 && lw == 1) lds_st(S.dyn_ack, t + 1);
            end = ti == NONE;
            if (end) ti = 0u;
        }
        ti = uni(ti);
        Task k;
        if (!end) {
            c_u32* src = (c_u32*)&tasks[ti];
#pragma unroll
            for (int i = 0; i < 12; ++i) ((uint32_t*)&k)[i] = src[i];
        } else {
            k = Task();
            k.op = OP_END;
        }
        if (deal && !dealt && !end && k.op == OP_ATTN) {
            // this step's deal of the attention slots, before the first attention task
            // reaches the compute waves or its pages are issued
            if (lw == 0) {
                attn_deal(p, lane);
                lgkm_wait_all();
                if (lane == 0) lds_st(S.adealt, 1u);
            } else if (lds_ld(S.adealt) == 0u) {
                drain();  // publish this wave's pages in flight before it waits
                if (!uni(lds_wait_ge(S.adealt, 1u, pp, ti))) break;
            }
            dealt = true;
        }
        if (lw == 0) {
            const uint32_t slot = t % FIFO;
            if (lds_ld(S.fifo_free[slot]) < t / FIFO) {
                drain();
                if (!uni(lds_wait_ge(S.fifo_free[slot], t / FIFO, pp, ti))) break;
            }
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < 12; ++i) lds_st(((uint32_t*)&S.fifo[slot])[i], ((const uint32_t*)&k)[i]);
                lds_st(S.fifo_first_page[slot], pseq);
                if (tr) {
                    lds_st(S.tl_issue0[slot], 0u);
                    lds_st(S.tl_issue1[slot], 0u);
                    lds_st(S.tl_pub[slot], 0u);
                }
            }
            lgkm_wait_all();
            if (lane == 0) lds_st(S.fifo_ready[slot], t + 1);
        }
        if (end) break;
        const uint32_t np = task_pages(p, k, hd);
        for (uint32_t kp = 0; kp < np; ++kp) {
            const uint32_t ps = pseq % NPAGES;
            const uint32_t need = NCW * (pseq / NPAGES);
            while (lds_ld(S.page_free[ps]) < need) {
                drain();
                if (!uni(lds_wait_ge(S.page_free[ps], need, pp, ti))) goto out;
            }
            issue_page(p, k, kp, ps, lane, lw);
            if (tr && lane == 0) {
                const uint32_t now = (uint32_t)rtc(), fs = t % FIFO;
                lds_st(S.pg_fslot[ps], fs);
                if (kp == 0) lds_st(S.tl_issue0[fs], now);
                lds_st(S.tl_issue1[fs], now);
            }
            ++pseq;
            if constexpr (ATTN_INFLIGHT == INFL) {
                if (pseq - pub == INFL) {
                    vm_wait<LPP * (INFL - 1)>();
                    publish_one();
                }
            } else if (k.op == OP_ATTN) {
                if (pseq - pub >= (uint32_t)ATTN_INFLIGHT) {
                    vm_wait<LPP * (ATTN_INFLIGHT - 1)>();
                    while (pseq - pub > (uint32_t)ATTN_INFLIGHT - 1u) publish_one();
                }
            } else if (pseq - pub >= (uint32_t)INFL) {
                // (after an attention task's deeper queue: every page but the newest INFL - 1)
                vm_wait<LPP * (INFL - 1)>();
                while (pseq - pub > (uint32_t)INFL - 1u) publish_one();
            }
        }
    }
out:
    drain();
    if (sched == 3 && lw == 1) serve_rest(pp, epoch, lane, next_ev);
}

// ---- compute-wave primitives -------------------------------------------------------

constexpr uint32_t RSRC_FLAGS = 0x00020000;  // raw buffer, 32-bit data format
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

struct Ctx {
    int wave, lane, tid;  // compute wave, lane, thread index among the compute lanes
    uint32_t t;           // task sequence number of this workgroup
    uint32_t epoch, parity;
    bool tr;              // tracing: take time stamps (a clock read stalls wave 0 on the scalar memory path)
};

// The task record of FIFO slot `slot`, read from LDS into wave-uniform registers.
__device__ __forceinline__ Task fifo_task(uint32_t slot) {
    Task k;
#pragma unroll
    for (int i = 0; i < 12; ++i) ((uint32_t*)&k)[i] = uni(lds_ld(((const uint32_t*)&S.fifo[uni(slot)])[i]));
    return k;
}
__device__ __forceinline__ Ctx make_ctx(uint32_t t, uint32_t epoch) {
    Ctx c;
    c.wave = (int)uni(threadIdx.x >> 6);
    c.lane = threadIdx.x & 63;
    c.tid = c.wave * 64 + c.lane;
    c.t = uni(t);
    c.epoch = uni(epoch);
    c.parity = c.epoch & 1u;
    c.tr = uni(lds_ld(S.trace_on)) != 0;
    return c;
}

__device__ __forceinline__ bool cbarrier(const Params* pp, Ctx& c, uint32_t task) {
    const uint32_t gen = uni(lds_ld(S.cgen[c.wave])) + NCW;
    if (c.lane == 0) lds_st(S.cgen[c.wave], gen);
    lgkm_wait_all();
    if (c.lane == 0) lds_add(S.cbar, 1u);
    return lds_wait_ge(S.cbar, gen, pp, task);
}

__device__ __forceinline__ bool page_acquire(const Params* pp, uint32_t seq, uint32_t task) {
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
        const uint32_t& w = S.page_ready[lw][seq % NPAGES];
        const uint32_t want = seq / NPAGES + 1;
        // short waits spin here: the out-of-line wait (timeouts, abort) is a call, around
        // which a GEMV holding many operand registers would save and restore them
        uint32_t it = 0;
        while (lds_ld(w) < want && ++it < 512u) __builtin_amdgcn_s_sleep(1);
        if (it == 512u && !lds_wait_ge(w, want, pp, task)) return false;
    }
    return true;
}
// Traced wave 0: page_acquire, its waiting time added to tm[3] (ticks).
__device__ __forceinline__ bool page_acquire_tr(const Params* pp, uint32_t seq, uint32_t task, bool tr, int lane) {
    if (!tr) return page_acquire(pp, seq, task);
    const uint32_t t0 = (uint32_t)rtc();
    const bool ok = page_acquire(pp, seq, task);
    if (lane == 0) lds_st(S.tm[3], lds_ld(S.tm[3]) + ((uint32_t)rtc() - t0));
    return ok;
}
__device__ __forceinline__ void page_release(uint32_t seq, int lane) {
    lgkm_wait_all();
    if (lane == 0) lds_add(S.page_free[seq % NPAGES], 1u);
}
__device__ __forceinline__ void page_skip(uint32_t seq, int lane) {
    if (lane == 0) lds_add(S.page_free[seq % NPAGES], 1u);
}

__device__ __forceinline__ void tmark(const Ctx& c, int i) {
    if (c.tr && c.wave == 0 && c.lane == 0) lds_st(S.tm[i], (uint32_t)rtc());
}

// One poll of an event: do its sub-counters sum to `want`?
__device__ __forceinline__ bool event_ready(CParams& p, uint32_t ev, uint32_t nsub, uint32_t want, int lane) {
    return ctr_sum(p.ctr, ev, nsub, lane) >= want;
}

// Compute wave 0 waits for the task's event and releases the other compute waves.
__device__ __forceinline__ bool await_inputs(const Params* pp, const Task& k, Ctx& c) {
    if (c.wave == 0) {
        if (k.wait_ev != NONE) {
            CParams& p = P(pp);
            const uint32_t want = c.epoch * k.wait_target;
            if (!event_ready(p, k.wait_ev, k.wait_nsub, want, c.lane) &&
                !uni(wait_event(pp, k.wait_ev, k.wait_nsub, want, k.id)))
                return false;
        }
        acquire_fence();
        if (c.tr) {
            const uint64_t tr = rtc();
            if (c.lane == 0) {
                lds_st(S.t_ready_lo, (uint32_t)tr);
                lds_st(S.t_ready_hi, (uint32_t)(tr >> 32));
            }
        }
        if (c.lane == 0) lds_st(S.go, c.t + 1);
        return true;
    }
    const bool ok = lds_wait_ge(S.go, c.t + 1, pp, k.id);
    acquire_fence();
    return ok;
}

// Device-scope (sc1) loads of data written by other workgroups in this step,
// through a bounds-checked buffer resource (offsets past `bytes` read 0).  Unlike
// atomic loads, the compiler keeps many of these in flight before a single wait.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, RSRC_FLAGS);
}
__device__ __forceinline__ float ldb_dev(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 16));
}

// n floats (n a multiple of 4) from src, read with device-scope 16-byte loads spread
// over the compute lanes (all issued before any is used), into LDS xs[dst + i].
template <int MAXQ>
__device__ __forceinline__ void stage_f32(int dst, const float* src, int n, int tid) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, n * 4, RSRC_FLAGS);
    u32x4 v[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) v[q] = __builtin_amdgcn_raw_buffer_load_b128(r, (tid + q * NCW * 64) * 16, 0, 16);
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
        const int i = (tid + q * NCW * 64) * 4;
        if (i < n) *(u32x4*)&S.xs[dst + i] = v[q];
    }
}
// n bf16 values (n a multiple of 8) from src (ordinary loads) into LDS xs[dst + i] as floats
__device__ __forceinline__ void stage_bf16(int dst, const uint16_t* src, int n, int tid) {
    uint4 v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = (tid + q * NCW * 64) * 8;
        v[q] = i < n ? gld_u4(src + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = (tid + q * NCW * 64) * 8;
        if (i < n) {
            *(float4*)&S.xs[dst + i] = make_float4(bf16lo(v[q].x), bf16hi(v[q].x), bf16lo(v[q].y), bf16hi(v[q].y));
            *(float4*)&S.xs[dst + i + 4] = make_float4(bf16lo(v[q].z), bf16hi(v[q].z), bf16lo(v[q].w), bf16hi(v[q].w));
        }
    }
}

// This lane's slice of xs[xo + column] in GEMV order, times `scale` and the bf16
// gains gw (already loaded: KT/512 words of 8 gains; null = no gains).
template <int KT>
__device__ __forceinline__ void load_x(int xo, int lane, float scale, const uint4* gw, float* x) {
    if constexpr (KT >= 512) {
#pragma unroll
        for (int j = 0; j < KT / 512; ++j) {
            const float4 a = *(const float4*)&S.xs[xo + j * 512 + lane * 8];
            const float4 b = *(const float4*)&S.xs[xo + j * 512 + lane * 8 + 4];
            float g[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
            if (gw) {
                g[0] = bf16lo(gw[j].x); g[1] = bf16hi(gw[j].x); g[2] = bf16lo(gw[j].y); g[3] = bf16hi(gw[j].y);
                g[4] = bf16lo(gw[j].z); g[5] = bf16hi(gw[j].z); g[6] = bf16lo(gw[j].w); g[7] = bf16hi(gw[j].w);
            }
            x[j * 8 + 0] = a.x * scale * g[0]; x[j * 8 + 1] = a.y * scale * g[1];
            x[j * 8 + 2] = a.z * scale * g[2]; x[j * 8 + 3] = a.w * scale * g[3];
            x[j * 8 + 4] = b.x * scale * g[4]; x[j * 8 + 5] = b.y * scale * g[5];
            x[j * 8 + 6] = b.z * scale * g[6]; x[j * 8 + 7] = b.w * scale * g[7];
        }
    } else {
        constexpr int LPROW = KT / 8;
        const float4 a = *(const float4*)&S.xs[xo + (lane % LPROW) * 8];
        const float4 b = *(const float4*)&S.xs[xo + (lane % LPROW) * 8 + 4];
        x[0] = a.x * scale; x[1] = a.y * scale; x[2] = a.z * scale; x[3] = a.w * scale;
        x[4] = b.x * scale; x[5] = b.y * scale; x[6] = b.z * scale; x[7] = b.w * scale;
    }
}
// gains of this lane's GEMV columns (KT >= 512 only)
template <int KT>
__device__ __forceinline__ void load_gains(const uint16_t* g, int lane, uint4* gw) {
#pragma unroll
    for (int j = 0; j < KT / 512; ++j) gw[j] = gld_u4(g + j * 512 + lane * 8);
}

// 1/sqrt(mean(xs[0..n)^2) + eps), computed by each wave from LDS
__device__ __forceinline__ float rms_scale(int n, float eps, int lane) {
    float ss = 0.f;
    for (int i = lane * 4; i < n; i += 256) {
        const float4 a = *(const float4*)&S.xs[i];
        ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
    return 1.0f / sqrtf(wave_sum(ss) / (float)n + eps);
}

// ---- GEMV over LDS pages --------------------------------------------------------------

// y[r] = W[r, :] . x over the task's rows, rows of KT = 4096 bf16 (two rows per
// 16 KiB page, stored row by row); wave w computes the pages pg = w (mod NCW).
// Results in S.rowres[r].  Each wave releases every page of the task once.
template <int KT>
__device__ __forceinline__ bool gemv_pages(const Params* pp, int wave, int lane, uint32_t page0, uint32_t nrows,
                                           uint32_t wbytes, const float* x, uint32_t task) {
    static_assert(KT >= 4096, "row-major GEMV pages are used for K = 4096 only");
    const bool trace_pages = wave == 0 && uni(lds_ld(S.trace_on)) != 0;
    const uint32_t npages = (wbytes + PAGE - 1) / PAGE;
    constexpr int RPP = PAGE / (2 * KT);  // rows per page
    constexpr int LPR = KT / 512;         // 1 KiB wave loads per row
    for (uint32_t pg = 0; pg < npages; ++pg) {
        if ((int)(pg % NCW) != wave) {
            page_skip(page0 + pg, lane);
            continue;
        }
        if (!page_acquire(pp, page0 + pg, task)) return false;
        if (trace_pages && wave == 0 && lane == 0) lds_st(S.tm[2], (uint32_t)rtc());
        const uint32_t slot = (page0 + pg) % NPAGES;
        uint4 wv[RPP * LPR];
#pragma unroll
        for (int i = 0; i < RPP * LPR; ++i) wv[i] = *(const uint4*)&ring[slot][i * 1024 + lane * 16];
        page_release(page0 + pg, lane);
#pragma unroll
        for (int rr = 0; rr < RPP; ++rr) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int j = 0; j < LPR; j += 2) {
                a = dot8(wv[rr * LPR + j], x + j * 8, a);
                b = dot8(wv[rr * LPR + j + 1], x + (j + 1) * 8, b);
            }
            const float sum = wave_sum(a + b);
            const uint32_t r = pg * RPP + rr;
            if (lane == 0 && r < nrows) S.rowres[r] = sum;
        }
    }
    return true;
}

// ---- matrix-core GEMV (128 <= K <= 2048) --------------------------------------------------
//
// The activation x (fp32) is split exactly into three bf16 parts, x = hi + mid +
// lo (8 significant bits each), kept in LDS as three bf16 arrays.  These are the
// first three columns of the B operand of v_mfma_f32_16x16x32_bf16 (the other 13
// are zero) and the weights the A operand, so D[m][0] + D[m][1] + D[m][2] is the
// dot product of weight row m with x: products exact, fp32 accumulation.  The
// weight tile is stored as 1 KiB blocks of 16 rows x 32 columns in operand order
// (lane l: row l % 16, columns 8 (l / 16) .. +7); blocks row-group-major, 16 per
// page; compute wave w owns the column blocks kb = w (mod 4), so every page holds
// four blocks of every wave.  The waves' partial rows meet in S.rowres through
// LDS float atomics.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t* split_arrays() { return (uint16_t*)&S.xs[0]; }

// exact split of v: hi = v truncated to bf16, mid = the remainder truncated, lo = the rest
__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t uh = __float_as_uint(v) & 0xffff0000u;
    const float r1 = v - __uint_as_float(uh);
    const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(um);
    hi = uh >> 16;
    mid = um >> 16;
    lo = __float_as_uint(r2) >> 16;
}
// columns c .. c+7 of x (c a multiple of 8) into the split arrays of a K = KT activation
template <int KT>
__device__ __forceinline__ void put_split8(int c, const float* v) {
    uint32_t hh[4], mm[4], ll[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h0, m0, l0, h1, m1, l1;
        split3(v[2 * i], h0, m0, l0);
        split3(v[2 * i + 1], h1, m1, l1);
        hh[i] = h0 | (h1 << 16);
        mm[i] = m0 | (m1 << 16);
        ll[i] = l0 | (l1 << 16);
    }
    uint16_t* sp = split_arrays();
    *(u32x4v*)(sp + c) = u32x4v{hh[0], hh[1], hh[2], hh[3]};
    *(u32x4v*)(sp + KT + c) = u32x4v{mm[0], mm[1], mm[2], mm[3]};
    *(u32x4v*)(sp + 2 * KT + c) = u32x4v{ll[0], ll[1], ll[2], ll[3]};
}
template <int KT>
__device__ __forceinline__ void put_split1(int c, float v) {
    uint32_t h0, m0, l0;
    split3(v, h0, m0, l0);
    uint16_t* sp = split_arrays();
    sp[c] = (uint16_t)h0;
    sp[KT + c] = (uint16_t)m0;
    sp[2 * KT + c] = (uint16_t)l0;
}

// Stage x (columns 8 tid .. +7 per lane) into the split arrays: from bf16 (srcb,
// ordinary loads: the embedding) or fp32 written by other workgroups (srcf,
// device-scope loads).  With gains (gp) x is multiplied by them; the sum of
// squares of the unscaled x goes to S.ssq[wave] when wanted.
template <int KT>
__device__ __forceinline__ void stage_split(const uint16_t* srcb, const float* srcf, bool use_gains, uint4 gp,
                                            bool want_ss, int tid, int wave, int lane) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
    const bool act = tid * 8 < KT;
    if (srcb) {
        if (act) {
            const uint4 w = gld_u4(srcb + tid * 8);
            v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
            v[4] = bf16lo(w.z); v[5] = bf16hi(w.z); v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
        }
    } else {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)srcf, 0, KT * 4, RSRC_FLAGS);
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 32, 0, 16);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 32 + 16, 0, 16);
        if (act) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = __uint_as_float(a[i]);
                v[4 + i] = __uint_as_float(b[i]);
            }
        }
    }
    if (want_ss) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
        ss = wave_sum(ss);
        if (lane == 0) S.ssq[wave] = ss;
    }
    if (use_gains) {
        v[0] *= bf16lo(gp.x); v[1] *= bf16hi(gp.x); v[2] *= bf16lo(gp.y); v[3] *= bf16hi(gp.y);
        v[4] *= bf16lo(gp.z); v[5] *= bf16hi(gp.z); v[6] *= bf16lo(gp.w); v[7] *= bf16hi(gp.w);
    }
    if (act) put_split8<KT>(tid * 8, v);
}
// 1 / RMS of the staged activation from the per-wave partial sums (after a barrier)
__device__ __forceinline__ float rms_from_ssq(int n, float eps) {
    const float ss = (S.ssq[0] + S.ssq[1]) + (S.ssq[2] + S.ssq[3]);
    return 1.0f / sqrtf(ss / (float)n + eps);
}
__device__ __forceinline__ void zero_rowres(int tid) { *(float4*)&S.rowres[tid * 4] = make_float4(0.f, 0.f, 0.f, 0.f); }

// The B operands of this wave (column blocks kb = 4 i + wave): lanes 0..2 of each
// 16-lane row carry hi, mid, lo of columns 32 kb + 8 (lane / 16) .. +7, the others zero.
template <int KT>
__device__ __forceinline__ void load_bop(int wave, int lane, u32x4v* B) {
    const int n = lane % 16, kq = lane / 16;
    const uint16_t* sp = split_arrays();
#pragma unroll
    for (int i = 0; i < KT / 128; ++i) {
        const int col = (4 * i + wave) * 32 + kq * 8;
        B[i] = n < 3 ? *(const u32x4v*)(sp + n * KT + col) : u32x4v{0u, 0u, 0u, 0u};
    }
}

// Row group rg of the tile: add D[m][0] + D[m][1] + D[m][2] of this wave to S.rowres.
__device__ __forceinline__ void flush_rows(f32x4v acc, uint32_t rg, int lane) {
    const int n = lane % 16, kq = lane / 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float v = acc[i];
        const float s1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
        const float s2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
        const float t = v + s1 + s2;  // row_shr 1 and 2: lane n = 2 sums columns 0, 1, 2
        if (n == 2 && rg * 16 < (uint32_t)ROWRES)
            __hip_atomic_fetch_add(&S.rowres[rg * 16 + kq * 4 + i], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

template <int KT>
__device__ __forceinline__ bool gemv_mfma(const Params* pp, int wave, int lane, uint32_t page0, uint32_t wbytes,
                                          const u32x4v* B, uint32_t task) {
    static_assert(KT >= 128 && KT <= 2048, "matrix-core GEMV covers 128 <= K <= 2048");
    constexpr int NKB = KT / 32;  // column blocks
    const bool trace_pages = wave == 0 && uni(lds_ld(S.trace_on)) != 0;
    const uint32_t npages = (wbytes + PAGE - 1) / PAGE;
    if constexpr (NKB >= 16) {
        constexpr int PPR = NKB / 16;  // pages per row group
        const uint32_t nrg = npages / PPR;
        for (uint32_t rg = 0; rg < nrg; ++rg) {
            // four independent accumulators (block slot j) keep the matrix core busy
            f32x4v acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < PPR; ++s) {
                const uint32_t pg = rg * PPR + s;
                if (!page_acquire(pp, page0 + pg, task)) return false;
                if (trace_pages && wave == 0 && lane == 0) lds_st(S.tm[2], (uint32_t)rtc());
                const uint32_t slot = (page0 + pg) % NPAGES;
                u32x4v a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = *(const u32x4v*)&ring[slot][(4 * j + wave) * 1024 + lane * 16];
                page_release(page0 + pg, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a[j]),
                                                                     __builtin_bit_cast(bf16x8v, B[4 * s + j]), acc[j], 0,
                                                                     0, 0);
            }
            flush_rows((acc[0] + acc[1]) + (acc[2] + acc[3]), rg, lane);
        }
    } else {
        constexpr int RPG = 16 / NKB;  // row groups per page
        constexpr int BPR = 4 / RPG;   // blocks per row group and wave
        for (uint32_t pg = 0; pg < npages; ++pg) {
            if (!page_acquire(pp, page0 + pg, task)) return false;
            if (trace_pages && wave == 0 && lane == 0) lds_st(S.tm[2], (uint32_t)rtc());
            const uint32_t slot = (page0 + pg) % NPAGES;
            u32x4v a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = *(const u32x4v*)&ring[slot][(4 * j + wave) * 1024 + lane * 16];
            page_release(page0 + pg, lane);
#pragma unroll
            for (int rr = 0; rr < RPG; ++rr) {
                f32x4v acc[BPR];
#pragma unroll
                for (int jj = 0; jj < BPR; ++jj)
                    acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a[rr * BPR + jj]),
                                                                      __builtin_bit_cast(bf16x8v, B[jj]),
                                                                      f32x4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                f32x4v sum = acc[0];
#pragma unroll
                for (int jj = 1; jj < BPR; ++jj) sum += acc[jj];
                flush_rows(sum, pg * RPG + rr, lane);
            }
        }
    }
    return true;
}

__device__ __forceinline__ float* acc_buf(CParams& p, uint32_t parity, int idx, int b) {
    return p.acc + (((size_t)parity * (2 * p.T.L + 1) + idx) * p.T.B + b) * p.T.h;
}
__device__ __forceinline__ const uint16_t* gains(CParams& p, int idx) {
    return (const uint16_t*)(p.w + p.lay.gains) + (size_t)idx * p.T.h;
}
__device__ __forceinline__ const uint16_t* embed_row(CParams& p, int b) {
    return (const uint16_t*)(p.w + p.lay.embed) + (size_t)S.tok[b] * p.T.h;
}

// Residual stream entering layer l (l == L: the final one) into xs[0..h)
template <int H4>
__device__ __forceinline__ void stage_x(CParams& p, int l, uint32_t parity, int tid) {
    if (l == 0) stage_bf16(0, embed_row(p, 0), p.T.h, tid);
    else stage_f32<H4>(0, acc_buf(p, parity, 2 * l - 1, 0), p.T.h, tid);
}

// Residual rows row0 + tid + 256 q of a residual-adding tile (zeros otherwise):
// accumulator idx (device-scope loads) or, for idx < 0, the embedding row.
__device__ __forceinline__ void load_residual(CParams& p, const Task& k, int idx, uint32_t parity, int tid, float* res) {
#pragma unroll
    for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) res[q] = 0.f;
    if (!(k.flags & TF_RESID)) return;
    if (idx < 0) {
        const uint16_t* e = embed_row(p, 0) + k.row0;
#pragma unroll
        for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) {
            const uint32_t i = (uint32_t)(tid + q * NCW * 64);
            if (i < k.nrows) res[q] = bf16f(gld(e + i));
        }
    } else {
        const __amdgpu_buffer_rsrc_t r = dev_rsrc(acc_buf(p, parity, idx, 0) + k.row0, k.nrows * 4);
#pragma unroll
        for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) res[q] = ldb_dev(r, (uint32_t)(tid + q * NCW * 64) * 4);
    }
}

// ---- several sequences: matrix-core operands in global memory -------------------------
//
// On the several-sequence path (B > 1, or any B with experts), the inputs of the O-projection (merged attention) and of the
// down-projection (SiLU(gate) * up) are written once per step as matrix-core B operands
// (columns = sequences) by their producers, with device-scope stores, and read with
// device-scope loads by every tile that consumes them.  Each fp32 input is carried as
// two bf16 parts, hi = its truncation to bf16 and lo = the remainder rounded to bf16,
// so hi + lo is within 2^-16 of it (relative); both parts go through the same weights.

constexpr int NPART = 2;
constexpr int OPS_PER_COL = NPART * GROUP_SEQS;  // bf16 elements per column of an operand region

// operand regions of layer l and column group sg (sequences 16 sg .. 16 sg + 15)
__device__ __forceinline__ int n_col_groups(CParams& p) { return (p.T.B + GROUP_SEQS - 1) / GROUP_SEQS; }
__device__ __forceinline__ uint16_t* opr_attn(CParams& p, int l, int sg) {
    return p.xop + ((size_t)l * n_col_groups(p) + sg) * p.T.nq * p.T.d * OPS_PER_COL;
}
__device__ __forceinline__ uint16_t* opr_m(CParams& p, int l, int sg) {
    return p.xop + ((size_t)p.T.L * n_col_groups(p) * p.T.nq * p.T.d + ((size_t)l * n_col_groups(p) + sg) * p.T.f) *
                       OPS_PER_COL;
}
// expert e's m rows (mixture of experts), after the attention and dense-FFN regions
__device__ __forceinline__ uint16_t* opr_me(CParams& p, int l, int e, int sg) {
    const size_t ng = (size_t)n_col_groups(p);
    return p.xop + ((size_t)p.T.L * ng * p.T.nq * p.T.d + (size_t)p.T.L * ng * p.T.f +
                    (((size_t)l * p.T.E + e) * ng + sg) * p.T.fe) * OPS_PER_COL;
}
// element of (part, column c, sequence b) in a region of nkb 32-column blocks: block
// (part, c / 32) holds 64 lanes x 8 elements, lane = 16 ((c % 32) / 8) + b
__device__ __forceinline__ uint32_t opr_index(int nkb, int part, int c, int b) {
    return ((uint32_t)(part * nkb + (c >> 5)) * 64u + (uint32_t)(((c & 31) >> 3) * 16 + b)) * 8u + (uint32_t)(c & 7);
}
// hi = v truncated to bf16; lo = the (exact) remainder rounded to nearest even bf16,
// branch-free (the remainder of a finite input is finite)
__device__ __forceinline__ void split2(float v, uint32_t& hi, uint32_t& lo) {
    const uint32_t uh = __float_as_uint(v) & 0xffff0000u;
    const uint32_t r = __float_as_uint(v - __uint_as_float(uh));
    hi = uh >> 16;
    lo = (r + 0x7fffu + ((r >> 16) & 1u)) >> 16;
}
// the parts of 8 consecutive inputs as two B-operand registers (hi, lo)
__device__ __forceinline__ void split8(const float* v, u32x4v& hi, u32x4v& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h0, l0, h1, l1;
        split2(v[2 * i], h0, l0);
        split2(v[2 * i + 1], h1, l1);
        hi[i] = h0 | (h1 << 16);
        lo[i] = l0 | (l1 << 16);
    }
}
// x[c .. c+7] of sequence b (c a multiple of 8) into region R
__device__ __forceinline__ void put_op8(uint16_t* R, int nkb, int c, int b, const float* v) {
    u32x4v hh, ll;
    split8(v, hh, ll);
    const __amdgpu_buffer_rsrc_t r = dev_rsrc(R, (uint32_t)nkb * NPART * 1024u);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hh), r, opr_index(nkb, 0, c, b) * 2, 0, 16);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ll), r, opr_index(nkb, 1, c, b) * 2, 0, 16);
}
__device__ __forceinline__ void put_op1(uint16_t* R, int nkb, int c, int b, float v) {
    uint32_t h0, l0;
    split2(v, h0, l0);
    const __amdgpu_buffer_rsrc_t r = dev_rsrc(R, (uint32_t)nkb * NPART * 1024u);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)h0, r, opr_index(nkb, 0, c, b) * 2, 0, 16);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)l0, r, opr_index(nkb, 1, c, b) * 2, 0, 16);
}

// One wave merges the nch attention chunks of (layer, sequence b, KV group g) into the
// O-projection's operands: a = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
// Lane = (query head, 8-dimension chunk).
__device__ __noinline__ void merge_chunks(const Params* pp, int layer_, int b_, int g_, int nch_, int lane) {
    CParams& p = P(pp);
    // wave-uniform arguments (a call passes them in vector registers)
    const int layer = (int)uni((uint32_t)layer_), b = (int)uni((uint32_t)b_), g = (int)uni((uint32_t)g_),
              nch = (int)uni((uint32_t)nch_);
    const int D = p.T.d, G = p.T.grp, Sp = ATTN_MAX_CHUNKS;  // partials: ATTN_MAX_CHUNKS chunks per (b, g)
    const uint32_t cs = (uint32_t)G * (D + 2);  // floats per chunk
    uint16_t* R = opr_attn(p, layer, b / GROUP_SEQS);
    const int nkb = p.T.nq * D / 32;
    for (int idx = lane; idx < G * (D / 8); idx += 64) {
        const int head = idx / (D / 8), c8 = idx % (D / 8);
        // one wave-uniform resource over the (b, g) partials; this lane's head at offset head (D + 2)
        const __amdgpu_buffer_rsrc_t r = dev_rsrc(p.part + (((size_t)b * p.T.nkv + g) * Sp) * cs, (uint32_t)(Sp * cs) * 4);
        const uint32_t ho = (uint32_t)head * (uint32_t)(D + 2);
        float mc[16], lc[16];
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            mc[cc] = cc < nch ? ldb_dev(r, (uint32_t)(cc * cs + ho) * 4) : -INFINITY;
            lc[cc] = cc < nch ? ldb_dev(r, (uint32_t)(cc * cs + ho + 1) * 4) : 0.f;
        }
        float Mx = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) Mx = fmaxf(Mx, mc[cc]);
        float den = 0.f, num[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) num[e] = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < 16; c4 += 4) {
            if (c4 >= nch) break;
            float oc[4][8];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    oc[cc][e] = c4 + cc < nch ? ldb_dev(r, (uint32_t)((c4 + cc) * cs + ho + 2 + c8 * 8 + e) * 4) : 0.f;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const float m = mc[c4 + cc];
                const float sc = m == -INFINITY ? 0.f : __expf(m - Mx);
                den = fmaf(sc, lc[c4 + cc], den);
#pragma unroll
                for (int e = 0; e < 8; ++e) num[e] = fmaf(sc, oc[cc][e], num[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) num[e] /= den;
        put_op8(R, nkb, (g * G + head) * D + c8 * 8, b % GROUP_SEQS, num);
    }
}

// The LM-head tiles also publish the final residual (hidden output): tile i copies
// its share [i * per, (i + 1) * per) of the B x h values, per = ceil(B h / tiles).
__device__ __forceinline__ void copy_hidden_share(CParams& p, const Task& k, uint32_t parity, int tid) {
    const int h = p.T.h, total = p.T.B * h, nt = p.T.n_lm_tiles;
    const int per = (total + nt - 1) / nt, ti = (int)(k.row0 / (uint32_t)p.T.lm_rows);
    const int e0 = ti * per, e1 = min(total, e0 + per);
    for (int e = e0 + tid; e < e1; e += NCW * 64) {
        float v;
        if (p.T.L == 0) v = bf16f(gld((const uint16_t*)(p.w + p.lay.embed) + (size_t)S.tok[e / h] * h + e % h));
        else v = ldf_dev(acc_buf(p, parity, 2 * p.T.L - 1, 0) + e);
        gst(p.hidden + e, v);
    }
}

// ---- ops ---------------------------------------------------------------------------------

// RMSNorm + QKV tile + RoPE + K/V append.  Tile rows [0, n) are the first halves
// (j0 + i) of n RoPE pairs of one head, rows [n, 2n) the second halves (j0 + i + d/2).
template <int KT>
__device__ __noinline__ bool op_qkv(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, tid = c.tid;
    const uint32_t n = k.nrows, slot = k.part;
    const int half = p.T.d / 2, nq = p.T.nq, nkv = p.T.nkv;
    const int32_t P0 = S.pos[0];
    float2 cs = make_float2(1.f, 0.f);
    if ((uint32_t)tid < n && slot < (uint32_t)(nq + nkv)) cs = gld_f2(p.rope + (size_t)P0 * half + k.row0 + tid);
    float r = 1.0f;  // 1/RMS, applied to the results (matrix-core path) or to x (K = 4096)
    if constexpr (KT <= 2048) {
        const uint4 gp = tid * 8 < KT ? gld_u4(gains(p, 2 * k.layer) + tid * 8) : make_uint4(0, 0, 0, 0);
        if (!await_inputs(pp, k, c)) return false;
        stage_split<KT>(k.layer == 0 ? embed_row(p, 0) : nullptr,
                        k.layer == 0 ? nullptr : acc_buf(p, c.parity, 2 * k.layer - 1, 0), true, gp, true, tid, c.wave,
                        lane);
        zero_rowres(tid);
        if (!cbarrier(pp, c, k.id)) return false;
        tmark(c, 0);
        r = rms_from_ssq(KT, p.eps);
        u32x4v B[KT / 128];
        load_bop<KT>(c.wave, lane, B);
        if (!gemv_mfma<KT>(pp, c.wave, lane, page0, k.wbytes, B, k.id)) return false;
    } else {
        uint4 gw[KT / 512];
        load_gains<KT>(gains(p, 2 * k.layer), lane, gw);
        if (!await_inputs(pp, k, c)) return false;
        stage_x<(MAX_ACT + 1023) / 1024>(p, k.layer, c.parity, tid);
        if (!cbarrier(pp, c, k.id)) return false;
        tmark(c, 0);
        float x[KT / 64];
        load_x<KT>(0, lane, rms_scale(KT, p.eps, lane), gw, x);
        if (!gemv_pages<KT>(pp, c.wave, lane, page0, 2 * n, k.wbytes, x, k.id)) return false;
    }
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 1);
    if ((uint32_t)tid < n) {
        const int j = (int)k.row0 + tid;
        float lo = S.rowres[tid] * r, hi = S.rowres[n + tid] * r;
        if (slot < (uint32_t)(nq + nkv)) {
            const float a = lo * cs.x - hi * cs.y;
            const float b = lo * cs.y + hi * cs.x;
            lo = a;
            hi = b;
        }
        if (slot < (uint32_t)nq) {
            float* q = p.q + (size_t)slot * p.T.d;
            stf_dev(q + j, lo);
            stf_dev(q + j + half, hi);
        } else {
            const bool is_k = slot < (uint32_t)(nq + nkv);
            const int g = is_k ? (int)slot - nq : (int)slot - nq - nkv;
            uint16_t* base = (is_k ? S.args.kc : S.args.vc) +
                             (((size_t)k.layer * p.T.B + 0) * nkv + g) * (size_t)p.T.C * p.T.d + (size_t)P0 * p.T.d;
            st16_dev(base + j, f2bf16(lo));
            st16_dev(base + j + half, f2bf16(hi));
        }
    }
    return true;
}

// Attention over one chunk of the context of (sequence, KV group): one wave per
// query head, softmax over 64-position pages taken in batches of up to four
// (one running maximum and sum per batch; the split of the context into chunks
// merged afterwards is the usual split-KV decode).  Scores: lane = position, K
// read column-chunk-major.  P.V: lane = (8-dimension chunk, position group), V
// read row-major; the position groups' partial sums are added through LDS.
template <int D>
__device__ __noinline__ bool op_attn(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, wave = c.wave;
    const AttnTask at = attn_task(p, k);
    const int b = at.b, g = k.part;
    const Chunk ch = at.ch;
    constexpr int PB = 4096 / D;      // positions per page (64 or 32)
    constexpr int NC = D / 8;         // 16-byte chunks per row (8 or 16)
    constexpr int NPG = 64 / NC;      // position groups in P.V (8 or 4)
    constexpr int IT = PB / NPG;      // positions per lane and page in P.V (8)
    constexpr int BATCH = 4;          // pages per softmax batch
    const int32_t pre_end = min(ch.c1, ch.P);
    const int32_t npre = max(0, pre_end - ch.c0);
    const uint32_t npages = (uint32_t)((npre + PB - 1) / PB);
    const float scale = 1.0f / sqrtf((float)D);
    const int G = p.T.grp;
    const int nh = (G - wave + NCW - 1) / NCW;  // heads of this wave: wave, wave + NCW, ...
    const bool has_cur = ch.c0 <= ch.P && ch.P < ch.c1;
    const int cl = lane % NC, pgl = lane / NC;  // P.V: dimension chunk and position group of this lane
    // an empty slot (several sequences; the merge reads only the non-empty chunks):
    // no pages, no partials, no wait for the event.  It still takes the
    // workgroup's start-of-task handshake: without it the waves that have no work
    // would run ahead into later tasks and count their completions early.  At batch 1
    // every chunk writes its partials.
    if (batched_path(p.T.B, p.T.E) && ch.c0 > ch.P) {
        Task none = k;
        none.wait_ev = NONE;
        return await_inputs(pp, none, c);
    }
    if (!await_inputs(pp, k, c)) return false;
    // each wave stages the query rows of its own heads, and the current token's K/V chunk
    float kc8[8], vc8[8];
    {
        const __amdgpu_buffer_rsrc_t qr = dev_rsrc(p.q + (size_t)b * p.T.nq * D + (size_t)g * G * D, G * D * 4);
        float qv[4][D / 64];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
#pragma unroll
            for (int ee = 0; ee < D / 64; ++ee)
                qv[hh][ee] = hh < nh ? ldb_dev(qr, ((wave + hh * NCW) * D + lane + 64 * ee) * 4) : 0.f;
        if (has_cur) {
            const size_t row = (((size_t)k.layer * p.T.B + b) * p.T.nkv + g) * (size_t)p.T.C + (size_t)ch.P;
            const __amdgpu_buffer_rsrc_t kr = dev_rsrc(uni_ptr(S.args.kc) + row * D, D * 2);
            const __amdgpu_buffer_rsrc_t vr = dev_rsrc(uni_ptr(S.args.vc) + row * D, D * 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wk = __float_as_uint(ldb_dev(kr, cl * 16 + i * 4));
                const uint32_t wv = __float_as_uint(ldb_dev(vr, cl * 16 + i * 4));
                kc8[2 * i] = bf16lo(wk);
                kc8[2 * i + 1] = bf16hi(wk);
                vc8[2 * i] = bf16lo(wv);
                vc8[2 * i + 1] = bf16hi(wv);
            }
        }
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
#pragma unroll
            for (int ee = 0; ee < D / 64; ++ee)
                if (hh < nh) S.xs[(wave + hh * NCW) * D + lane + 64 * ee] = qv[hh][ee];
        lgkm_wait_all();
    }
    tmark(c, 0);
    float M[4], Ls[4], o[4][8];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
        M[hh] = -INFINITY;
        Ls[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
    }
    float* const wsc = S.wsc[wave];
    for (uint32_t pb0 = 0; pb0 < npages; pb0 += BATCH) {
        const uint32_t nb = min((uint32_t)BATCH, npages - pb0);
        for (uint32_t i = 0; i < nb; ++i)
            if (!page_acquire(pp, page0 + pb0 + i, k.id)) return false;
        tmark(c, 2);
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            if (hh >= nh) break;
            const int hw = wave + hh * NCW;
            // scores of the batch: lane = position within each page
            float sc[BATCH];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                sc[i] = -INFINITY;
                if ((uint32_t)i < nb) {
                    const uint32_t slot = (page0 + pb0 + i) % NPAGES;
                    const int32_t rows = min(PB, pre_end - (ch.c0 + (int32_t)(pb0 + i) * PB));
                    if (lane < rows) {
                        float a0 = 0.f, a1 = 0.f;
#pragma unroll
                        for (int cc = 0; cc < NC; cc += 2) {
                            const uint4 k0 = *(const uint4*)&ring[slot][cc * (PB * 16) + lane * 16];
                            const uint4 k1 = *(const uint4*)&ring[slot][(cc + 1) * (PB * 16) + lane * 16];
                            a0 = dot8(k0, &S.xs[hw * D + cc * 8], a0);
                            a1 = dot8(k1, &S.xs[hw * D + (cc + 1) * 8], a1);
                        }
                        sc[i] = (a0 + a1) * scale;
                    }
                    mx = fmaxf(mx, sc[i]);
                }
            }
            const float mn = fmaxf(M[hh], wave_max(mx));
            const float corr = __expf(M[hh] - mn);
            float es = 0.f;
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const float e = sc[i] == -INFINITY ? 0.f : __expf(sc[i] - mn);
                es += e;
                // weights stored so that lane (chunk, group) finds its IT positions contiguous;
                // with fewer positions per page than lanes (head_dim 128) only the position
                // lanes store, the others would land on the same slots
                if ((uint32_t)i < nb && lane < PB) wsc[i * 64 + (lane % NPG) * IT + lane / NPG] = e;
            }
            Ls[hh] = Ls[hh] * corr + wave_sum(es);
            M[hh] = mn;
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) o[hh][ee] *= corr;
            lgkm_wait_all();
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                if ((uint32_t)i >= nb) break;
                const uint32_t slot = (page0 + pb0 + i) % NPAGES;
                float wgt[IT];
#pragma unroll
                for (int q = 0; q < IT; q += 4) {
                    const float4 w4 = *(const float4*)&wsc[i * 64 + pgl * IT + q];
                    wgt[q] = w4.x;
                    wgt[q + 1] = w4.y;
                    wgt[q + 2] = w4.z;
                    wgt[q + 3] = w4.w;
                }
#pragma unroll
                for (int r = 0; r < IT; ++r) {
                    const uint4 w = *(const uint4*)&ring[slot][8192 + (pgl + NPG * r) * (2 * D) + cl * 16];
                    o[hh][0] = fmaf(wgt[r], bf16lo(w.x), o[hh][0]);
                    o[hh][1] = fmaf(wgt[r], bf16hi(w.x), o[hh][1]);
                    o[hh][2] = fmaf(wgt[r], bf16lo(w.y), o[hh][2]);
                    o[hh][3] = fmaf(wgt[r], bf16hi(w.y), o[hh][3]);
                    o[hh][4] = fmaf(wgt[r], bf16lo(w.z), o[hh][4]);
                    o[hh][5] = fmaf(wgt[r], bf16hi(w.z), o[hh][5]);
                    o[hh][6] = fmaf(wgt[r], bf16lo(w.w), o[hh][6]);
                    o[hh][7] = fmaf(wgt[r], bf16hi(w.w), o[hh][7]);
                }
            }
            lgkm_wait_all();
        }
        for (uint32_t i = 0; i < nb; ++i) page_release(page0 + pb0 + i, lane);
    }
    // add the position groups' partial sums through LDS (xs above the staged queries)
    float* const red = &S.xs[MAX_ACT / 2 + wave * 512];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
        if (hh >= nh) break;
        *(float4*)&red[lane * 8] = make_float4(o[hh][0], o[hh][1], o[hh][2], o[hh][3]);
        *(float4*)&red[lane * 8 + 4] = make_float4(o[hh][4], o[hh][5], o[hh][6], o[hh][7]);
        lgkm_wait_all();
        if (pgl == 0) {
#pragma unroll
            for (int gg = 1; gg < NPG; ++gg) {
                const float4 a = *(const float4*)&red[(gg * NC + cl) * 8];
                const float4 bb = *(const float4*)&red[(gg * NC + cl) * 8 + 4];
                o[hh][0] += a.x; o[hh][1] += a.y; o[hh][2] += a.z; o[hh][3] += a.w;
                o[hh][4] += bb.x; o[hh][5] += bb.y; o[hh][6] += bb.z; o[hh][7] += bb.w;
            }
        }
        lgkm_wait_all();
    }
    if (has_cur) {
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            if (hh >= nh) break;
            const int hw = wave + hh * NCW;
            // q . k_cur: the lanes of position group 0 hold the NC chunks
            float a = 0.f;
            if (pgl == 0) {
#pragma unroll
                for (int ee = 0; ee < 8; ++ee) a = fmaf(S.xs[hw * D + cl * 8 + ee], kc8[ee], a);
            }
            const float sc = wave_sum(a) * scale;
            const float mn = fmaxf(M[hh], sc);
            const float corr = __expf(M[hh] - mn);
            const float e = __expf(sc - mn);
            Ls[hh] = Ls[hh] * corr + e;
            M[hh] = mn;
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) o[hh][ee] = fmaf(e, vc8[ee], o[hh][ee] * corr);
        }
    }
    tmark(c, 1);
    // partials (m, l, o) -> part[b][g][chunk][head][D + 2]
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
        if (hh >= nh) break;
        const int hw = wave + hh * NCW;
        float* dst = p.part + ((((size_t)b * p.T.nkv + g) * part_chunks(batched_path(p.T.B, p.T.E), p.T.attn_splits) +
                               (size_t)at.c) * G + hw) * (D + 2);
        if (lane == 0) {
            stf_dev(dst, M[hh]);
            stf_dev(dst + 1, Ls[hh]);
        }
        if (pgl == 0) {
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) stf_dev(dst + 2 + cl * 8 + ee, o[hh][ee]);
        }
    }
    if (batched_path(p.T.B, p.T.E) && nh > 0) {
        // several sequences: every wave with heads counts its finished partials on the
        // step's ticket of (sequence, group); the wave completing the count over the
        // non-empty chunks merges them all
        vm_wait_all();  // this wave's partials are stored
        const uint32_t want = (uint32_t)at.nch * (uint32_t)min(G, NCW);
        uint32_t old = 0;
        release_fence();
        if (lane == 0)
            old = addu_dev(&p.aticket[(((size_t)c.parity * p.T.L + k.layer) * p.T.B + b) * p.T.nkv + g], 1u);
        old = uni(old);
        if (old + 1u == want) {
            acquire_fence();
            merge_chunks(pp, k.layer, b, g, at.nch, lane);
        }
    }
    return true;
}

// GQA decode attention over one KV chunk on the matrix cores (head_dim 64, up to four
// query heads per KV head).  Wave w takes positions 16 w .. 16 w + 15 of every page, for
// all heads.  Scores: S^T = K q^T on v_mfma_f32_16x16x32_bf16 with the K rows as the A
// operand (one 16-byte chunk of a row per lane) and the query in
// the B operand split exactly into three bf16 parts, column n holding part n / 4 of head
// n % 4 (part 3 zero): summing a row's columns of one head gives the fp32-exact dot
// product.  The probabilities (in [0, 1]) go in as two parts, within 2^-16 of them.  The output layout puts, in lane (n, kq), the scores of positions 4 kq .. +3
// for head n % 4 -- exactly the positions and head whose probabilities that lane feeds to
// O^T += V^T P^T (v_mfma_f32_16x16x16_bf16), so the probabilities
// never move between lanes.  Each wave keeps its own running max, sum and output per head;
// the four are merged through LDS at the end, together with the current token's K/V.
// The page's K rows are row-major with 16-byte chunk c of row r stored at chunk c ^ (r % 8).
typedef short s16x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// Part `part` (0 hi, 1 mid, 2 lo, 3 zero) of the exact split of v, chosen with the lane's
// masks pm[i] = 0xffff if part == i else 0 (no branches: part differs between lanes).
__device__ __forceinline__ uint32_t split_part(float v, const uint32_t (&pm)[3]) {
    const uint32_t uh = __float_as_uint(v) & 0xffff0000u;
    const float r1 = v - __uint_as_float(uh);
    const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(um);
    return ((uh >> 16) & pm[0]) | ((um >> 16) & pm[1]) | ((__float_as_uint(r2) >> 16) & pm[2]);
}
// Part `part` of a two-part split of v in [0, 1]: hi = v truncated to bf16, lo = the
// remainder rounded to nearest even (v - hi - lo within 2^-16 of v); part 2 and 3 zero.
__device__ __forceinline__ uint32_t split_part2(float v, const uint32_t (&pm)[3]) {
    const uint32_t uh = __float_as_uint(v) & 0xffff0000u;
    const uint32_t r = __float_as_uint(v - __uint_as_float(uh));
    const uint32_t lo = (r + 0x7fffu + ((r >> 16) & 1u)) >> 16;
    return ((uh >> 16) & pm[0]) | (lo & pm[1]);
}
// sum over the four columns n, n +- 4, n +- 8 of a 16-lane row (the parts of one head)
__device__ __forceinline__ float sum_parts(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));  // row_ror:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true));  // row_ror:4
    return v;
}

__device__ __noinline__ bool op_attn_mfma(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_,
                                          uint32_t epoch_) {
    constexpr int D = 64, PB = 4096 / D, BATCH = 4, MW = 8 + 4 * D;  // merge record: M[4], L[4], O[4][D]
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, wave = c.wave;
    const AttnTask at = attn_task(p, k);
    const int b = at.b, g = k.part, G = p.T.grp;
    Chunk ch = at.ch;
    ch.c0 = (int32_t)uni((uint32_t)ch.c0);  // wave-uniform: scalar loop bounds and branches
    ch.c1 = (int32_t)uni((uint32_t)ch.c1);
    ch.P = (int32_t)uni((uint32_t)ch.P);
    const int32_t pre_end = min(ch.c1, ch.P);
    const int32_t npre = max(0, pre_end - ch.c0);
    const uint32_t npages = (uint32_t)((npre + PB - 1) / PB);
    const float scale = 1.0f / sqrtf((float)D);
    const bool has_cur = ch.c0 <= ch.P && ch.P < ch.c1;
    // an empty chunk slot (several sequences): no pages, no partials, but the start-of-task
    // handshake (see op_attn)
    if (batched_path(p.T.B, p.T.E) && ch.c0 > ch.P) {
        Task none = k;
        none.wait_ev = NONE;
        return await_inputs(pp, none, c);
    }
    if (!await_inputs(pp, k, c)) return false;
    const int n = lane % 16, kq = lane / 16, hq = n % 4, part = n / 4;
    const uint32_t pm[3] = {part == 0 ? 0xffffu : 0u, part == 1 ? 0xffffu : 0u, part == 2 ? 0xffffu : 0u};
    const __amdgpu_buffer_rsrc_t qr = dev_rsrc(p.q + (size_t)b * p.T.nq * D + (size_t)g * G * D, (uint32_t)(G * D * 4));
    // for the merge (wave = head, lane = dimension): q and the current token's K and V,
    // loaded now so that they arrive during the page loop
    float qd = 0.f, kcur = 0.f, vcur = 0.f;
    if (wave < G) {
        qd = ldb_dev(qr, (wave * D + lane) * 4);
        if (has_cur) {
            const size_t row = (((size_t)k.layer * p.T.B + b) * p.T.nkv + g) * (size_t)p.T.C + (size_t)ch.P;
            const uint32_t wk = __float_as_uint(ldb_dev(dev_rsrc(uni_ptr(S.args.kc) + row * D, D * 2), (lane / 2) * 4));
            const uint32_t wv = __float_as_uint(ldb_dev(dev_rsrc(uni_ptr(S.args.vc) + row * D, D * 2), (lane / 2) * 4));
            kcur = (lane & 1) ? bf16hi(wk) : bf16lo(wk);
            vcur = (lane & 1) ? bf16hi(wv) : bf16lo(wv);
        }
    }
    // B operand of the scores: part `part` of q[head hq][32 ks + 8 kq .. +7]
    u32x4v qb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        u32x4v raw = u32x4v{0u, 0u, 0u, 0u};
        if (hq < G) raw = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(qr, (hq * D + 32 * ks + 8 * kq) * 4, 0, 16));
        u32x4v raw2 = u32x4v{0u, 0u, 0u, 0u};
        if (hq < G) raw2 = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(qr, (hq * D + 32 * ks + 8 * kq + 4) * 4, 0, 16));
        const float qv[8] = {__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z), __uint_as_float(raw.w),
                             __uint_as_float(raw2.x), __uint_as_float(raw2.y), __uint_as_float(raw2.z), __uint_as_float(raw2.w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) qb[ks][i] = split_part(qv[2 * i], pm) | (split_part(qv[2 * i + 1], pm) << 16);
    }
    tmark(c, 0);
    f32x4v oacc[D / 16];  // O^T accumulators: operand t, rows d = 16 kq + 4 r + t, column n
#pragma unroll
    for (int dg = 0; dg < D / 16; ++dg) oacc[dg] = f32x4v{0.f, 0.f, 0.f, 0.f};
    float M = -INFINITY, L = 0.f;  // running max and this lane's sum (head hq, its positions)
    for (uint32_t pb0 = 0; pb0 < npages; pb0 += BATCH) {
        const uint32_t nb = min((uint32_t)BATCH, npages - pb0);
        for (uint32_t i = 0; i < nb; ++i)
            if (!page_acquire_tr(pp, page0 + pb0 + i, k.id, c.tr && wave == 0, lane)) return false;
        tmark(c, 2);
        // this wave's K operands and V words of the batch's pages into registers, then the
        // pages go back to the loader, which refills them during the arithmetic below
        u32x4v ka[BATCH][2];
        u32x2v vw4[BATCH][4];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if ((uint32_t)i >= nb) break;
            const uint32_t slot = (page0 + pb0 + i) % NPAGES;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int pos = 16 * wave + n, cix = (4 * ks + kq) ^ (pos & 7);
                ka[i][ks] = *(const u32x4v*)&ring[slot][pos * (2 * D) + cix * 16];
            }
            // V of positions 4 kq + j (j = 0..3) of this wave's 16, dimensions 4 n .. 4 n + 3
            const uint16_t* vrow = (const uint16_t*)&ring[slot][8192] + (16 * wave + 4 * kq) * D + 4 * n;
#pragma unroll
            for (int j = 0; j < 4; ++j) vw4[i][j] = *(const u32x2v*)(vrow + j * D);
        }
        for (uint32_t i = 0; i < nb; ++i) page_release(page0 + pb0 + i, lane);  // (waits for the reads)
        float sc[BATCH][4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[i][r] = -INFINITY;
            if ((uint32_t)i < nb) {
                const int32_t rows = min(PB, pre_end - (ch.c0 + (int32_t)(pb0 + i) * PB));
                const int32_t lim = rows - 16 * wave - 4 * kq;  // this lane's valid positions: r < lim
                f32x4v acc = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, ka[i][ks]),
                                                                   __builtin_bit_cast(bf16x8v, qb[ks]), acc, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // every lane takes part in the row sums; positions past the page's rows get -inf
                    sc[i][r] = sum_parts(acc[r]) * scale + (r < lim ? 0.f : -INFINITY);
                    mx = fmaxf(mx, sc[i][r]);
                }
            }
        }
        // this wave's max for head hq: over the four lane rows (the part columns agree)
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(M, mx);
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float corr = __expf(M - mref);
        L *= corr;
#pragma unroll
        for (int dg = 0; dg < D / 16; ++dg) oacc[dg] *= corr;
        M = mn;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if ((uint32_t)i >= nb) break;
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[r] = __expf(sc[i][r] - mref);
                L += pr[r];
            }
            // B operand: part `part` of p at positions 4 kq + r (r = 0..3), head hq
            const s16x4v pbv = __builtin_bit_cast(
                s16x4v, u32x2v{split_part2(pr[0], pm) | (split_part2(pr[1], pm) << 16),
                               split_part2(pr[2], pm) | (split_part2(pr[3], pm) << 16)});
            // A operand t is V^T with row n standing for dimension d = 4 n + t (V words read above)
            const u32x2v* vw = vw4[i];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = t / 2;
                const uint32_t a01 = (t & 1) ? (vw[0][c] >> 16) | (vw[1][c] & 0xffff0000u)
                                             : (vw[0][c] & 0xffffu) | (vw[1][c] << 16);
                const uint32_t a23 = (t & 1) ? (vw[2][c] >> 16) | (vw[3][c] & 0xffff0000u)
                                             : (vw[2][c] & 0xffffu) | (vw[3][c] << 16);
                oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4v, u32x2v{a01, a23}), pbv,
                                                                     oacc[t], 0, 0, 0);
            }
        }
    }
    // this wave's record for the merge: M and L per head, O[head][d]
    float* const mrec = &S.xs[MAX_ACT / 2 + wave * MW];
    float Lh = part == 0 ? L : 0.f;  // the part columns hold copies of the same sums
    Lh += __shfl_xor(Lh, 16, 64);
    Lh += __shfl_xor(Lh, 32, 64);
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float o = sum_parts(oacc[t][r]);
            if (part == 0) mrec[8 + hq * D + 16 * kq + 4 * r + t] = o;
        }
    if (part == 0 && kq == 0) {
        mrec[hq] = M;
        mrec[4 + hq] = Lh;
    }
    if (!cbarrier(pp, c, k.id)) return false;  // every wave's record is in LDS
    tmark(c, 1);
    if (wave < G) {
        // head `wave`: merge the four waves' records (lane = dimension), then the current token
        const int h = wave;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NCW; ++w) Mx = fmaxf(Mx, S.xs[MAX_ACT / 2 + w * MW + h]);
        const float mref = Mx == -INFINITY ? 0.f : Mx;
        float Lt = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < NCW; ++w) {
            const float* rec = &S.xs[MAX_ACT / 2 + w * MW];
            const float a = __expf(rec[h] - mref);
            Lt += a * rec[4 + h];
            o += a * rec[8 + h * D + lane];
        }
        if (has_cur) {
            const float sc = wave_sum(qd * kcur) * scale;
            const float mn = fmaxf(Mx, sc);
            const float corr = __expf(Mx - mn);
            const float e = __expf(sc - mn);
            Lt = Lt * corr + e;
            o = fmaf(e, vcur, o * corr);
            Mx = mn;
        }
        // partials (m, l, o) -> part[b][g][chunk][head][D + 2]
        float* dst = p.part + ((((size_t)b * p.T.nkv + g) * part_chunks(batched_path(p.T.B, p.T.E), p.T.attn_splits) +
                               (size_t)at.c) * G + h) * (D + 2);
        if (lane == 0) {
            stf_dev(dst, Mx);
            stf_dev(dst + 1, Lt);
        }
        stf_dev(dst + 2 + lane, o);
        if (batched_path(p.T.B, p.T.E)) {
            // several sequences: count this head's partial on the step's ticket of
            // (sequence, group); the wave completing the count merges the chunks
            vm_wait_all();
            const uint32_t want = (uint32_t)at.nch * (uint32_t)min(G, NCW);
            uint32_t old = 0;
            release_fence();
            if (lane == 0)
                old = addu_dev(&p.aticket[(((size_t)c.parity * p.T.L + k.layer) * p.T.B + b) * p.T.nkv + g], 1u);
            old = uni(old);
            if (old + 1u == want) {
                acquire_fence();
                merge_chunks(pp, k.layer, b, g, at.nch, lane);
            }
        }
    }
    return true;
}

// Merge of the attention partials of one KV group, O-proj K-slice, residual (atomic add).
template <int KT>
__device__ __noinline__ bool op_oproj(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    static_assert(KT <= 2048, "K of the O-projection slice is grp * head_dim <= 2048");
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, tid = c.tid, wave = c.wave;
    if (!await_inputs(pp, k, c)) return false;
    const int D = p.T.d, Sp = p.T.attn_splits, G = p.T.grp;
    // a = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c, one wave per query head
    const __amdgpu_buffer_rsrc_t pr = dev_rsrc(p.part + (size_t)k.part * Sp * G * (D + 2), Sp * G * (D + 2) * 4);
    for (int hw = wave; hw < G; hw += NCW) {
        const uint32_t cs = (uint32_t)G * (D + 2) * 4, h0 = (uint32_t)hw * (D + 2) * 4;
        float mc[16], lc[16], oc[16][2];
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            mc[cc] = ldb_dev(pr, h0 + cc * cs);
            lc[cc] = ldb_dev(pr, h0 + cc * cs + 4);
            oc[cc][0] = ldb_dev(pr, h0 + cc * cs + (2 + lane) * 4);
            oc[cc][1] = D == 128 ? ldb_dev(pr, h0 + cc * cs + (2 + 64 + lane) * 4) : 0.f;
        }
        float Mx = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc)
            if (cc < Sp) Mx = fmaxf(Mx, mc[cc]);
        float den = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            if (cc < Sp) {
                const float sc = mc[cc] == -INFINITY ? 0.f : __expf(mc[cc] - Mx);
                den = fmaf(sc, lc[cc], den);
                n0 = fmaf(sc, oc[cc][0], n0);
                n1 = fmaf(sc, oc[cc][1], n1);
            }
        }
        put_split1<KT>(hw * D + lane, n0 / den);
        if (D == 128) put_split1<KT>(hw * D + 64 + lane, n1 / den);
    }
    zero_rowres(tid);
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 0);
    // residual rows of this lane's epilogue (in flight during the GEMV)
    float res[MAX_TILE_ROWS / (NCW * 64)];
    load_residual(p, k, k.layer == 0 ? -1 : 2 * k.layer - 1, c.parity, tid, res);
    {
        u32x4v B[KT / 128];
        load_bop<KT>(wave, lane, B);
        if (!gemv_mfma<KT>(pp, wave, lane, page0, k.wbytes, B, k.id)) return false;
    }
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 1);
    float* dst = acc_buf(p, c.parity, 2 * k.layer, 0);
#pragma unroll
    for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) {
        const uint32_t i = (uint32_t)(tid + q * NCW * 64);
        if (i < k.nrows) addf_dev(dst + k.row0 + i, S.rowres[i] + res[q]);
    }
    return true;
}

// RMSNorm + gate/up tile + SiLU(gate) * up.  Tile rows [0, n) gate, [n, 2n) up.
template <int KT>
__device__ __noinline__ bool op_gateup(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, tid = c.tid;
    float r = 1.0f;
    if constexpr (KT <= 2048) {
        const uint4 gp = tid * 8 < KT ? gld_u4(gains(p, 2 * k.layer + 1) + tid * 8) : make_uint4(0, 0, 0, 0);
        if (!await_inputs(pp, k, c)) return false;
        stage_split<KT>(nullptr, acc_buf(p, c.parity, 2 * k.layer, 0), true, gp, true, tid, c.wave, lane);
        zero_rowres(tid);
        if (!cbarrier(pp, c, k.id)) return false;
        tmark(c, 0);
        r = rms_from_ssq(KT, p.eps);
        u32x4v B[KT / 128];
        load_bop<KT>(c.wave, lane, B);
        if (!gemv_mfma<KT>(pp, c.wave, lane, page0, k.wbytes, B, k.id)) return false;
    } else {
        uint4 gw[KT / 512];
        load_gains<KT>(gains(p, 2 * k.layer + 1), lane, gw);
        if (!await_inputs(pp, k, c)) return false;
        stage_f32<(MAX_ACT + 1023) / 1024>(0, acc_buf(p, c.parity, 2 * k.layer, 0), p.T.h, tid);
        if (!cbarrier(pp, c, k.id)) return false;
        tmark(c, 0);
        float x[KT / 64];
        load_x<KT>(0, lane, rms_scale(KT, p.eps, lane), gw, x);
        if (!gemv_pages<KT>(pp, c.wave, lane, page0, 2 * k.nrows, k.wbytes, x, k.id)) return false;
    }
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 1);
    for (uint32_t i = (uint32_t)tid; i < k.nrows; i += NCW * 64) {
        const float gt = S.rowres[i] * r, up = S.rowres[k.nrows + i] * r;
        stf_dev(p.m + k.row0 + i, gt / (1.0f + __expf(-gt)) * up);
    }
    return true;
}

// Down-proj K-slice tile + residual (atomic add).
template <int KT>
__device__ __noinline__ bool op_down(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    static_assert(KT <= 2048, "down-projection K blocks are at most 1024 columns");
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, tid = c.tid;
    if (!await_inputs(pp, k, c)) return false;
    stage_split<KT>(nullptr, p.m + (size_t)k.part * KT, false, make_uint4(0, 0, 0, 0), false, tid, c.wave, lane);
    zero_rowres(tid);
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 0);
    // residual rows of this lane's epilogue (in flight during the GEMV)
    float res[MAX_TILE_ROWS / (NCW * 64)];
    load_residual(p, k, 2 * k.layer, c.parity, tid, res);
    {
        u32x4v B[KT / 128];
        load_bop<KT>(c.wave, lane, B);
        if (!gemv_mfma<KT>(pp, c.wave, lane, page0, k.wbytes, B, k.id)) return false;
    }
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 1);
    float* dst = acc_buf(p, c.parity, 2 * k.layer + 1, 0);
#pragma unroll
    for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) {
        const uint32_t i = (uint32_t)(tid + q * NCW * 64);
        if (i < k.nrows) addf_dev(dst + k.row0 + i, S.rowres[i] + res[q]);
    }
    return true;
}

// Final RMSNorm + LM-head tile + argmax (packed 64-bit atomic max).
template <int KT>
__device__ __noinline__ bool op_lmhead(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, tid = c.tid;
    const int L = p.T.L;
    float r = 1.0f;
    if constexpr (KT <= 2048) {
        const uint4 gp = tid * 8 < KT ? gld_u4(gains(p, 2 * L) + tid * 8) : make_uint4(0, 0, 0, 0);
        if (!await_inputs(pp, k, c)) return false;
        stage_split<KT>(L == 0 ? embed_row(p, 0) : nullptr, L == 0 ? nullptr : acc_buf(p, c.parity, 2 * L - 1, 0), true,
                        gp, true, tid, c.wave, lane);
        zero_rowres(tid);
        if (!cbarrier(pp, c, k.id)) return false;
        tmark(c, 0);
        r = rms_from_ssq(KT, p.eps);
        u32x4v B[KT / 128];
        load_bop<KT>(c.wave, lane, B);
        if (!gemv_mfma<KT>(pp, c.wave, lane, page0, k.wbytes, B, k.id)) return false;
    } else {
        uint4 gw[KT / 512];
        load_gains<KT>(gains(p, 2 * L), lane, gw);
        if (!await_inputs(pp, k, c)) return false;
        stage_x<(MAX_ACT + 1023) / 1024>(p, L, c.parity, tid);
        if (!cbarrier(pp, c, k.id)) return false;
        tmark(c, 0);
        float x[KT / 64];
        load_x<KT>(0, lane, rms_scale(KT, p.eps, lane), gw, x);
        if (!gemv_pages<KT>(pp, c.wave, lane, page0, k.nrows, k.wbytes, x, k.id)) return false;
    }
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 1);
    float bv = -INFINITY;
    uint32_t bi = 0xffffffffu;
    float* logits = S.args.logits;
    for (uint32_t i = (uint32_t)tid; i < k.nrows; i += NCW * 64) {
        const float val = S.rowres[i] * r;
        if (logits) gst(logits + k.row0 + i, val);
        if (val > bv) {  // rows visited in increasing order: the first maximum is kept
            bv = val;
            bi = k.row0 + i;
        }
    }
    // pack (order-preserving value bits, inverted index): the largest key is the
    // largest value at the lowest index
    const uint32_t ub = __float_as_uint(bv);
    const uint32_t ord = (ub & 0x80000000u) ? ~ub : (ub | 0x80000000u);
    unsigned long long key = bi == 0xffffffffu ? 0ull : (((unsigned long long)ord << 32) | (0xffffffffu - bi));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(key, o, 64);
        key = other > key ? other : key;
    }
    if (lane == 0 && key)
        __hip_atomic_fetch_max((g_u64*)&p.key[(c.parity * KEY_SLOTS + k.row0 / (uint32_t)p.T.lm_rows % KEY_SLOTS) * p.T.B],
                               key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    copy_hidden_share(p, k, c.parity, tid);
    return true;
}

// ---- batched GEMV tiles (B > 1, or experts) ------------------------------------------
//
// One pass over a weight tile serves all sequences: the tile's 16 x 32 blocks are the
// A operands, the inputs of the 16 sequences the B operands (two bf16 parts, one MFMA
// each).  Each compute wave owns the column blocks kb = 4 i + wave and keeps the B
// operands of all of them in registers for the whole task.  Its products go to a
// wave-private slice of S.xs (row-major rows x B); the epilogue adds the 4 slices.

// Inputs of the normalised GEMVs: the fp32 residual rows of the sequences (or their
// bf16 embedding rows) for this wave's column blocks 4 i + wave, lane (kq = lane / 16,
// sequence n = lane % 16) holding columns 8 kq .. 8 kq + 7 of each block; rows past
// the batch read zeros (offsets outside the buffer range).  The 8 fp32 values of block
// i land in bo[i] as raw bits, to be turned into the block's operands in place.
template <int NBW>
__device__ __forceinline__ void load_rows(u32x4v (*bo)[NPART], __amdgpu_buffer_rsrc_t r, bool emb, uint32_t row_ofs,
                                          int wave, int lane, int c0 = 0) {
    const int kq = lane / 16;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const uint32_t col = (uint32_t)(c0 + 32 * (4 * i + wave) + 8 * kq);
        if (emb) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, (row_ofs + col) * 2, 0, 0);
            bo[i][0] = u32x4v{w[0] << 16, w[0] & 0xffff0000u, w[1] << 16, w[1] & 0xffff0000u};
            bo[i][1] = u32x4v{w[2] << 16, w[2] & 0xffff0000u, w[3] << 16, w[3] & 0xffff0000u};
        } else {
            bo[i][0] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, (row_ofs + col) * 4, 0, 16));
            bo[i][1] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, (row_ofs + col) * 4 + 16, 0, 16));
        }
    }
}
// Block i's inputs (raw fp32 bits in bo) times the RMSNorm gains staged in LDS (bf16,
// in S.rowres), split into the two B-operand parts in place; the sum of squares of the
// unscaled inputs is accumulated into ss.
__device__ __forceinline__ void ops_of_row_block(u32x4v* bo, int i, int wave, int lane, float& ss, int c0 = 0) {
    const uint16_t* gl = (const uint16_t*)S.rowres;
    const uint4 gw = *(const uint4*)&gl[c0 + 32 * (4 * i + wave) + 8 * (lane / 16)];
    const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float v0 = __uint_as_float(bo[e / 2][(e % 2) * 2]), v1 = __uint_as_float(bo[e / 2][(e % 2) * 2 + 1]);
        ss = fmaf(v0, v0, ss);
        ss = fmaf(v1, v1, ss);
        x[2 * e] = v0 * bf16lo(gg[e]);
        x[2 * e + 1] = v1 * bf16hi(gg[e]);
    }
    split8(x, bo[0], bo[1]);
}
// B operands read from an operand region (nkb_total column blocks, this tile's first at kb_off)
template <int NBW>
__device__ __forceinline__ void bops_from_region(u32x4v (*bo)[NPART], __amdgpu_buffer_rsrc_t r, int nkb_total,
                                                 int kb_off, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int pt = 0; pt < NPART; ++pt)
            bo[i][pt] = __builtin_bit_cast(
                u32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                            r, ((uint32_t)(pt * nkb_total + kb_off + 4 * i + wave) * 64u + (uint32_t)lane) * 16u, 0,
                            16));
}
__device__ __forceinline__ f32x4v mfma_parts(u32x4v a, const u32x4v* b2, f32x4v acc) {
#pragma unroll
    for (int pt = 0; pt < NPART; ++pt)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b2[pt]),
                                                      acc, 0, 0, 0);
    return acc;
}
// the 16 x 16 result block of row group rg into this wave's slice (first visit: store)
__device__ __forceinline__ void slice_put(float* sl, f32x4v acc, uint32_t rg, int lane, int B, bool first) {
    const int n = lane % 16, kq = lane / 16;
    if (n < B) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t at = (rg * 16 + kq * 4 + i) * (uint32_t)B + n;
            if (at < 1024u) sl[at] = first ? acc[i] : sl[at] + acc[i];
        }
    }
}
// row i, sequence b of the tile's result: the sum of the four waves' slices
__device__ __forceinline__ float tile_res(int i, int b, int B) {
    const int at = i * B + b;
    return (S.xs[at] + S.xs[1024 + at]) + (S.xs[2048 + at] + S.xs[3072 + at]);
}
// 1 / RMS of sequence b from the per-wave sums of squares
__device__ __forceinline__ float rs_seq(int b, int n, float eps) {
    const float ss = (S.ssqb[0][b] + S.ssqb[1][b]) + (S.ssqb[2][b] + S.ssqb[3][b]);
    return 1.0f / sqrtf(ss / (float)n + eps);
}

// The tile's pages in the batch-1 order (row group by row group; a page holds K = 512
// columns of one row group, or 16 / (K / 32) whole row groups for K <= 256); bo holds
// this wave's B operands for all of K (column blocks 4 i + wave).  Row group rg's
// products are summed over its pages in two accumulators (one per part) and stored
// once into this wave's slice.
template <int KT>
__device__ __forceinline__ bool gemv_mfma_b(const Params* pp, int wave, int lane, uint32_t page0, uint32_t nrg,
                                            const u32x4v (*bo)[NPART], int B, uint32_t task, bool first = true) {
    static_assert(KT >= 128 && KT <= 2048, "matrix-core GEMV covers 128 <= K <= 2048");
    constexpr int NKB = KT / 32;
    const bool trace_pages = wave == 0 && uni(lds_ld(S.trace_on)) != 0;
    float* const sl = &S.xs[wave * 1024];
    auto mfma = [](u32x4v a, u32x4v b, f32x4v acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b),
                                                       acc, 0, 0, 0);
    };
    if constexpr (NKB >= 16) {
        constexpr int PPR = NKB / 16;  // pages per row group
        for (uint32_t rg = 0; rg < nrg; ++rg) {
            f32x4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < PPR; ++s) {
                const uint32_t pg = rg * PPR + s;
                if (!page_acquire_tr(pp, page0 + pg, task, trace_pages, lane)) return false;
                if (trace_pages && wave == 0 && lane == 0) lds_st(S.tm[2], (uint32_t)rtc());
                const uint32_t slot = (page0 + pg) % NPAGES;
                u32x4v a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = *(const u32x4v*)&ring[slot][(4 * j + wave) * 1024 + lane * 16];
                page_release(page0 + pg, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc0 = mfma(a[j], bo[4 * s + j][0], acc0);
                    acc1 = mfma(a[j], bo[4 * s + j][1], acc1);
                }
            }
            slice_put(sl, acc0 + acc1, rg, lane, B, first);
        }
    } else {
        constexpr int RPG = 16 / NKB;  // row groups per page
        constexpr int BPR = 4 / RPG;   // blocks per row group and wave
        const uint32_t npages = (nrg + RPG - 1) / RPG;
        for (uint32_t pg = 0; pg < npages; ++pg) {
            if (!page_acquire_tr(pp, page0 + pg, task, trace_pages, lane)) return false;
            if (trace_pages && wave == 0 && lane == 0) lds_st(S.tm[2], (uint32_t)rtc());
            const uint32_t slot = (page0 + pg) % NPAGES;
            u32x4v a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = *(const u32x4v*)&ring[slot][(4 * j + wave) * 1024 + lane * 16];
            page_release(page0 + pg, lane);
#pragma unroll
            for (int rr = 0; rr < RPG; ++rr) {
                f32x4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jj = 0; jj < BPR; ++jj) {
                    acc0 = mfma(a[rr * BPR + jj], bo[jj][0], acc0);
                    acc1 = mfma(a[rr * BPR + jj], bo[jj][1], acc1);
                }
                slice_put(sl, acc0 + acc1, pg * RPG + rr, lane, B, true);
            }
        }
    }
    return true;
}

// Batched GEMV task (QKV, O-proj, gate/up, down, LM head, router, expert gate/up and down)
// on the several-sequence path.  QKV,
// gate/up and LM head read the residual rows themselves and apply RMSNorm (gains on
// the inputs, 1/RMS per sequence on the results); O-proj and down read the operand
// regions their producers wrote.
template <int KT, bool NORMED, int OPK>
__device__ __noinline__ bool op_gemv_b(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    Task k = fifo_task(slot_);
    k.op = (uint8_t)OPK;  // one instance per operation: the other operations' code folds away
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, tid = c.tid, wave = c.wave;
    // this tile's column group: sequences gb0 .. gb0 + B - 1 of the Btot in the step
    const int Btot = p.T.B, gb0 = (int)k.seq * GROUP_SEQS, B = min(GROUP_SEQS, Btot - gb0);
    const int L = p.T.L, l = k.layer, D = p.T.d, h = p.T.h;
    constexpr bool normed = NORMED;  // QKV, gate/up, LM head
    // normalised inputs: gains slot and source residual (-1: the embedding)
    const bool ffn_in = k.op == OP_GATEUP || k.op == OP_ROUTE || k.op == OP_EGU;  // the FFN's normalised input
    const int gslot = k.op == OP_QKV ? 2 * l : (ffn_in ? 2 * l + 1 : 2 * L);
    const int src = ffn_in ? 2 * l : (l == 0 ? -1 : 2 * l - 1);
    uint4 gpre = make_uint4(0, 0, 0, 0);
    if (normed && tid * 8 < h) gpre = gld_u4(gains(p, gslot) + tid * 8);
    if (!await_inputs(pp, k, c)) return false;
    // QKV and gate/up tiles of K = 2048 are packed in K halves: the operands of one half at a time
    constexpr bool HV = NORMED && KT == 2048 && (OPK == OP_QKV || OPK == OP_GATEUP);
    constexpr int NBW = HV ? KT / 256 : KT / 128;
    u32x4v bo[NBW][NPART];
    __amdgpu_buffer_rsrc_t nr;  // normalised inputs: the residual rows, or the embedding rows
    uint32_t nrow_ofs = 0;
    bool nemb = false;
    float ss = 0.f;
    if constexpr (NORMED) {
        if (tid * 8 < h) *(uint4*)&((uint16_t*)S.rowres)[tid * 8] = gpre;
        const int n = lane % 16;
        nemb = src < 0;
        if (nemb) {
            nr = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w + p.lay.embed), 0, (uint32_t)((uint64_t)p.T.V * h * 2),
                                                   RSRC_FLAGS);
            nrow_ofs = n < B ? (uint32_t)S.tok[gb0 + n] * (uint32_t)h : (uint32_t)p.T.V * (uint32_t)h;
        } else {
            nr = dev_rsrc(acc_buf(p, c.parity, src, gb0), (uint32_t)(B * h * 4));
            nrow_ofs = (uint32_t)(n * h);  // sequences past B read zeros (out of the buffer's range)
        }
        if constexpr (!HV) load_rows<NBW>(bo, nr, nemb, nrow_ofs, wave, lane);
        if (!cbarrier(pp, c, k.id)) return false;  // gains staged
        if constexpr (!HV) {
#pragma unroll
            for (int i = 0; i < NBW; ++i) ops_of_row_block(bo[i], i, wave, lane, ss);
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            if (lane < GROUP_SEQS) S.ssqb[wave][lane] = ss;
        }
    } else {
        const uint16_t* R = k.op == OP_OPROJ ? opr_attn(p, l, (int)k.seq)
                            : k.op == OP_EDOWN ? opr_me(p, l, k.part, (int)k.seq)
                                               : opr_m(p, l, (int)k.seq);
        const int nkb_total = k.op == OP_OPROJ ? p.T.nq * D / 32 : k.op == OP_EDOWN ? p.T.fe / 32 : p.T.f / 32;
        const int kb_off = k.op == OP_OPROJ ? k.part * p.T.grp * D / 32 : k.op == OP_EDOWN ? 0 : k.part * p.T.kd / 32;
        // expert down tiles: the router logits of this wave's sequences, loaded ahead of the
        // operands so that the routing is computed while those are in flight
        const int E = p.T.E;
        float rlv[GROUP_SEQS / NCW];
#pragma unroll
        for (int j = 0; j < GROUP_SEQS / NCW; ++j) {
            const int b = wave + j * NCW;
            rlv[j] = -INFINITY;
            if (k.op == OP_EDOWN && b < B && lane < E)
                rlv[j] = ldb_dev(dev_rsrc(p.rlogit + ((size_t)l * Btot + gb0 + b) * E, (uint32_t)E * 4u),
                                 (uint32_t)lane * 4u);
        }
        bops_from_region<NBW>(bo, dev_rsrc(R, (uint32_t)nkb_total * NPART * 1024u), nkb_total, kb_off, wave, lane);
        if (k.op == OP_EDOWN) {
            // the routing weight of this expert for each sequence, from all router logits
            // (the expert's event also counts every router tile); its selection slot too
            const int K = p.T.topk, e = k.part;
#pragma unroll
            for (int j = 0; j < GROUP_SEQS / NCW; ++j) {
                const int b = wave + j * NCW;
                if (b >= B) break;
                int slot;
                const float wgt = route_weight(rlv[j], lane, E, K, e, slot);
                if (lane == 0) {
                    S.rwb[b] = wgt;
                    S.rtop[b] = slot == 0;
                    if (k.row0 == 0 && slot >= 0) gst(p.eids + ((size_t)l * Btot + gb0 + b) * K + slot, (int32_t)e);
                }
            }
            if (!cbarrier(pp, c, k.id)) return false;  // routing of every sequence staged
        }
    }
    tmark(c, 0);
    // residual (rows x sequences) of residual-adding tiles, in flight during the GEMV.
    // Element idx of an O-projection or down tile's results is row idx % rows of sequence
    // idx / rows, so the lanes of one residual load or atomic touch consecutive rows of
    // one sequence.  (Expert down tiles, where most sequences add nothing, keep
    // sequence-minor order: measured faster there.)
    const bool resid = (k.op == OP_OPROJ || k.op == OP_DOWN) && (k.flags & TF_RESID);
    float res[MAX_TILE_ROWS / (NCW * 64)];
#pragma unroll
    for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) {
        res[q] = 0.f;
        const int idx = tid + q * NCW * 64;
        if (resid && idx < (int)k.nrows * B) {
            const int i = idx % (int)k.nrows, b = idx / (int)k.nrows, row = (int)k.row0 + i;
            const int rsrc_i = k.op == OP_DOWN ? 2 * l : (l == 0 ? -1 : 2 * l - 1);
            res[q] = rsrc_i < 0 ? bf16f(gld((const uint16_t*)(p.w + p.lay.embed) + (size_t)S.tok[gb0 + b] * h + row))
                                : ldb_dev(dev_rsrc(acc_buf(p, c.parity, rsrc_i, gb0), (uint32_t)(B * h) * 4u),
                                          (uint32_t)(b * h + row) * 4u);
        }
    }
    // the tile's rows in chunks of whole row groups whose results fit the slices
    // (one chunk except for LM-head tiles)
    constexpr int NKB = KT / 32;
    const bool expert = k.op == OP_EGU || k.op == OP_EDOWN;
    const int CR = expert ? 64 : HV ? halves_chunk_rows(Btot) : MAX_TILE_ROWS / B / 64 * 64;  // expert chunks: 32 gate + 32 up rows / 64 down rows
    static_assert(64 * GROUP_SEQS <= MAX_TILE_ROWS, "an expert chunk's results (and residual rows) fit res[] and the slices");
    const int rows_pad = (int)(k.wbytes / (KT * 2));
    float lm_bv[GROUP_SEQS / NCW];
    uint32_t lm_bi[GROUP_SEQS / NCW];
#pragma unroll
    for (int j = 0; j < GROUP_SEQS / NCW; ++j) {
        lm_bv[j] = -INFINITY;
        lm_bi[j] = 0xffffffffu;
    }
    for (int c0 = 0; c0 < rows_pad; c0 += CR) {
        const uint32_t nrg = (uint32_t)min(CR, rows_pad - c0) / 16;
        const uint32_t pbase = page0 + (NKB >= 16 ? (uint32_t)(c0 / 16) * (NKB / 16) : (uint32_t)(c0 / 16) / (16 / NKB));
        if (c0 > 0 && !cbarrier(pp, c, k.id)) return false;  // the previous chunk's results are consumed
        // expert down tiles: the residual rows of the chunk (64 x up to 16 sequences, in
        // res[]) of the sequences whose first choice is this expert, in flight during its
        // GEMV; so each sequence's residual is added exactly once, with that expert's output
        if (k.op == OP_EDOWN) {
            const int nr = min(CR, (int)k.nrows - c0);
#pragma unroll
            for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) {
                const int idx = tid + q * NCW * 64, i = idx / B, b = idx % B;
                res[q] = i < nr && S.rtop[b]
                             ? ldb_dev(dev_rsrc(acc_buf(p, c.parity, 2 * l, gb0), (uint32_t)(B * h) * 4u),
                                       (uint32_t)(b * h + (int)k.row0 + c0 + i) * 4u)
                             : 0.f;
            }
        }
        if constexpr (HV) {
            // the chunk's rows over columns 0 .. K/2 - 1, then K/2 .. K - 1 (added); the sums
            // of squares of the inputs from the first chunk's two halves
#pragma unroll 1
            for (int hh = 0; hh < 2; ++hh) {
                load_rows<NBW>(bo, nr, nemb, nrow_ofs, wave, lane, hh * (KT / 2));
                float ssh = 0.f;
#pragma unroll
                for (int i = 0; i < NBW; ++i) ops_of_row_block(bo[i], i, wave, lane, ssh, hh * (KT / 2));
                if (c0 == 0) ss += ssh;
                if (!gemv_mfma_b<KT / 2>(pp, wave, lane, pbase + (uint32_t)hh * nrg * (KT / 1024), nrg, bo, B, k.id,
                                         hh == 0))
                    return false;
            }
            if (c0 == 0) {
                ss += __shfl_xor(ss, 16, 64);
                ss += __shfl_xor(ss, 32, 64);
                if (lane < GROUP_SEQS) S.ssqb[wave][lane] = ss;
            }
        } else {
            if (!gemv_mfma_b<KT>(pp, wave, lane, pbase, nrg, bo, B, k.id)) return false;
        }
        if (!cbarrier(pp, c, k.id)) return false;
        if (k.op == OP_EGU) {  // m = SiLU(gate) * up, rows row0 + c0 / 2 .. + 31
            uint16_t* Rm = opr_me(p, l, k.part, (int)k.seq);
            for (int idx = tid; idx < 32 * B; idx += NCW * 64) {
                const int i = idx / B, b = idx % B;
                const float rb = rs_seq(b, h, p.eps);
                const float gt = tile_res(i, b, B) * rb, up = tile_res(32 + i, b, B) * rb;
                put_op1(Rm, p.T.fe / 32, (int)k.row0 + c0 / 2 + i, b, gt / (1.0f + __expf(-gt)) * up);
            }
        } else if (k.op == OP_EDOWN) {  // weighted residual accumulation of the chunk's rows
            // (sequences that did not select the expert add nothing)
            const int nr = min(CR, (int)k.nrows - c0);
#pragma unroll
            for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) {
                const int idx = tid + q * NCW * 64, i = idx / B, b = idx % B;
                if (i >= nr) break;
                const float wb = S.rwb[b];
                if (wb == 0.f) continue;
                addf_dev(acc_buf(p, c.parity, 2 * l + 1, gb0 + b) + k.row0 + c0 + i, tile_res(i, b, B) * wb + res[q]);
            }
        } else if (k.op == OP_LMHEAD) {  // logits of the chunk, running argmax per sequence
            float* logits = S.args.logits;
            const int nr = min(CR, (int)k.nrows - c0);
#pragma unroll
            for (int j = 0; j < GROUP_SEQS / NCW; ++j) {
                const int b = wave + j * NCW;
                if (b >= B) break;
                const float rb = rs_seq(b, h, p.eps);
                for (int i = lane; i < nr; i += 64) {
                    const float val = tile_res(i, b, B) * rb;
                    if (logits) gst(logits + (size_t)(gb0 + b) * p.T.V + k.row0 + c0 + i, val);
                    if (val > lm_bv[j]) {  // rows visited in increasing order per lane: the first maximum is kept
                        lm_bv[j] = val;
                        lm_bi[j] = k.row0 + (uint32_t)(c0 + i);
                    }
                }
            }
        }
    }
    tmark(c, 1);
    if (k.op == OP_QKV) {
        const uint32_t n = k.nrows, slot = k.part;
        const int half = D / 2, nq = p.T.nq, nkv = p.T.nkv;
        const int b = tid / (int)n, i = tid % (int)n;
        if (b < B) {
            const float rb = rs_seq(b, h, p.eps);
            const int32_t Pb = S.pos[gb0 + b];
            const int j = (int)k.row0 + i;
            float lo = tile_res(i, b, B) * rb, hi = tile_res((int)n + i, b, B) * rb;
            if (slot < (uint32_t)(nq + nkv)) {
                const float2 cs = gld_f2(p.rope + (size_t)Pb * half + j);
                const float x0 = lo * cs.x - hi * cs.y, x1 = lo * cs.y + hi * cs.x;
                lo = x0;
                hi = x1;
            }
            if (slot < (uint32_t)nq) {
                float* q = p.q + (size_t)(gb0 + b) * nq * D + (size_t)slot * D;
                stf_dev(q + j, lo);
                stf_dev(q + j + half, hi);
            } else {
                const bool is_k = slot < (uint32_t)(nq + nkv);
                const int g = is_k ? (int)slot - nq : (int)slot - nq - nkv;
                uint16_t* base = (is_k ? S.args.kc : S.args.vc) +
                                 (((size_t)l * Btot + gb0 + b) * nkv + g) * (size_t)p.T.C * D + (size_t)Pb * D;
                st16_dev(base + j, f2bf16(lo));
                st16_dev(base + j + half, f2bf16(hi));
            }
        }
    } else if (k.op == OP_ROUTE) {  // router logits of experts row0 .. row0 + nrows - 1
        for (int idx = tid; idx < (int)k.nrows * B; idx += NCW * 64) {
            const int i = idx / B, b = idx % B;
            stf_dev(p.rlogit + ((size_t)l * Btot + gb0 + b) * p.T.E + k.row0 + i, tile_res(i, b, B) * rs_seq(b, h, p.eps));
        }
    } else if (k.op == OP_GATEUP) {
        uint16_t* Rm = opr_m(p, l, (int)k.seq);
        for (int idx = tid; idx < (int)k.nrows * B; idx += NCW * 64) {
            const int i = idx / B, b = idx % B;
            const float rb = rs_seq(b, h, p.eps);
            const float gt = tile_res(i, b, B) * rb, up = tile_res((int)k.nrows + i, b, B) * rb;
            put_op1(Rm, p.T.f / 32, (int)k.row0 + i, b, gt / (1.0f + __expf(-gt)) * up);
        }
    } else if (k.op == OP_LMHEAD) {
#pragma unroll
        for (int j = 0; j < GROUP_SEQS / NCW; ++j) {
            const int b = wave + j * NCW;
            if (b >= B) break;
            const float bv = lm_bv[j];
            const uint32_t bi = lm_bi[j];
            const uint32_t ub = __float_as_uint(bv);
            const uint32_t ord = (ub & 0x80000000u) ? ~ub : (ub | 0x80000000u);
            unsigned long long key = bi == 0xffffffffu ? 0ull : (((unsigned long long)ord << 32) | (0xffffffffu - bi));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const unsigned long long other = __shfl_xor(key, o, 64);
                key = other > key ? other : key;
            }
            if (lane == 0 && key)
                __hip_atomic_fetch_max(
                    (g_u64*)&p.key[(c.parity * KEY_SLOTS + k.row0 / (uint32_t)p.T.lm_rows % KEY_SLOTS) * Btot + gb0 + b],
                    key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (k.seq == 0) copy_hidden_share(p, k, c.parity, tid);  // once, by the first column group's tiles
    } else if (k.op == OP_OPROJ || k.op == OP_DOWN) {  // residual accumulation (expert tiles did theirs per chunk)
        const int dst = k.op == OP_DOWN ? 2 * l + 1 : 2 * l;
#pragma unroll
        for (int q = 0; q < MAX_TILE_ROWS / (NCW * 64); ++q) {
            const int idx = tid + q * NCW * 64;
            if (idx < (int)k.nrows * B) {
                const int i = idx % (int)k.nrows, b = idx / (int)k.nrows;
                addf_dev(acc_buf(p, c.parity, dst, gb0 + b) + k.row0 + i, tile_res(i, b, B) + res[q]);
            }
        }
    }
    return true;
}

// The several-sequence GEMV of operation OPK: normalised input (n) or operand region (r)
template <int OPK>
struct GemvB {
    template <int KT>
    static __device__ __forceinline__ bool n(const Params* pp, uint32_t slot, uint32_t page0, uint32_t t, uint32_t epoch) {
        return op_gemv_b<KT, true, OPK>(pp, slot, page0, t, epoch);
    }
    template <int KT>
    static __device__ __forceinline__ bool r(const Params* pp, uint32_t slot, uint32_t page0, uint32_t t, uint32_t epoch) {
        return op_gemv_b<KT, false, OPK>(pp, slot, page0, t, epoch);
    }
};

// After the last LM-head tile of the step: publish the argmax (the LM-head tiles
// have published the final residual).
__device__ __noinline__ void finish_step(const Params* pp, uint32_t epoch, uint32_t parity) {
    CParams& p = P(pp);
    const int lane = threadIdx.x & 63;
    uint32_t old = 0;
    release_fence();
    if (lane == 0) old = addu_dev(&p.ticket[0], 1u);
    old = uni(old);
    if (old + 1u != epoch * (uint32_t)(p.T.n_lm_tiles * n_col_groups(p))) return;
    acquire_fence();
    const int B = p.T.B;
    for (int b = lane; b < B; b += 64) {
        unsigned long long key = 0ull;
#pragma unroll
        for (int s = 0; s < KEY_SLOTS; ++s) {
            const unsigned long long ks = __hip_atomic_load((g_u64*)&p.key[(parity * KEY_SLOTS + s) * B + b],
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            key = ks > key ? ks : key;
        }
        gst(p.next + b, (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffu)));
    }
}

#include "prefill_ops.h"

#define MK_KT_DISPATCH(fn, kt, ...)                                      \
    ((kt) == 128    ? fn<128>(__VA_ARGS__)                               \
     : (kt) == 256  ? fn<256>(__VA_ARGS__)                               \
     : (kt) == 512  ? fn<512>(__VA_ARGS__)                               \
     : (kt) == 1024 ? fn<1024>(__VA_ARGS__)                              \
     : (kt) == 2048 ? fn<2048>(__VA_ARGS__)                              \
                    : fn<4096>(__VA_ARGS__))
#define MK_KT_DISPATCH_2K(fn, kt, ...)                                   \
    ((kt) == 128    ? fn<128>(__VA_ARGS__)                               \
     : (kt) == 256  ? fn<256>(__VA_ARGS__)                               \
     : (kt) == 512  ? fn<512>(__VA_ARGS__)                               \
     : (kt) == 1024 ? fn<1024>(__VA_ARGS__)                              \
                    : fn<2048>(__VA_ARGS__))

// ---- compute-wave main loop ---------------------------------------------------------------

// PF: the prompt megakernel's operations (else the decode step's)
template <bool PF>
__device__ __noinline__ void compute(const Params* pp, uint32_t epoch, int wave) {
    Ctx c;
    c.wave = (int)uni((uint32_t)wave);
    c.lane = threadIdx.x & 63;
    c.tid = c.wave * 64 + c.lane;
    c.epoch = epoch;
    c.parity = epoch & 1u;
    CParams& p0 = P(pp);
    const int h = p0.T.h, okt = p0.T.grp * p0.T.d, dkt = p0.T.kd, hd = p0.T.d;
    const bool tracing = uni(lds_ld(S.trace_on)) != 0;  // clock reads only when tracing
    // what the completion of every task reads, loaded once (not a scalar-load round trip per task between
    // the workgroup's done barrier and its signal)
    uint32_t* const ctr = p0.ctr;
    const uint32_t drop_task = p0.drop_task, sched = p0.sched, n_exp = (uint32_t)p0.T.E;
    uint32_t* const task_count = p0.task_count;
    const bool batched = batched_path(p0.T.B, p0.T.E);
    for (uint32_t t = 0;; ++t) {
        const uint32_t slot = t % FIFO;
        if (!lds_wait_ge(S.fifo_ready[slot], t + 1, pp, NONE)) return;
        const Task k = fifo_task(slot);
        const uint32_t page0 = uni(lds_ld(S.fifo_first_page[slot]));
        if (k.op == OP_END) return;
        const uint64_t t_fetch = tracing ? rtc() : 0;
        c.t = t;
        bool ok = true;
        // single-sequence operations referenced first: their functions are emitted next
        // to the loader, ahead of the several-sequence GEMV instances
        if constexpr (PF) {
            const bool w2 = (k.flags & TF_NGW2) != 0, r128 = k.nrows == 128;
#define MK_PF_GEMM(OPK)                                                                  \
    (r128 ? (w2 ? op_pgemm<OPK, 8, 2>(pp, slot, page0, t, epoch) : op_pgemm<OPK, 8, 1>(pp, slot, page0, t, epoch)) \
          : op_pgemm<OPK, 4, 1>(pp, slot, page0, t, epoch))
            switch (k.op) {
                case OP_PNORM: ok = op_pnorm(pp, slot, page0, t, epoch); break;
                case OP_PQKV: ok = MK_PF_GEMM(OP_PQKV); break;
                case OP_PATTN: ok = op_pattn(pp, slot, page0, t, epoch); break;
                case OP_POPROJ: ok = MK_PF_GEMM(OP_POPROJ); break;
                case OP_PGU: ok = MK_PF_GEMM(OP_PGU); break;
                case OP_PDOWN: ok = MK_PF_GEMM(OP_PDOWN); break;
                case OP_PLM: ok = MK_KT_DISPATCH_2K(op_plm, h, pp, slot, page0, t, epoch); break;
                default: break;
            }
#undef MK_PF_GEMM
        } else if (!batched) {
            switch (k.op) {
                case OP_QKV: ok = MK_KT_DISPATCH(op_qkv, h, pp, slot, page0, t, epoch); break;
                case OP_ATTN: ok = attn_kswizzle(p0.T.d, p0.T.grp) ? op_attn_mfma(pp, slot, page0, t, epoch)
                                   : hd == 64 ? op_attn<64>(pp, slot, page0, t, epoch)
                                              : op_attn<128>(pp, slot, page0, t, epoch);
                    break;
                case OP_OPROJ: ok = MK_KT_DISPATCH_2K(op_oproj, okt, pp, slot, page0, t, epoch); break;
                case OP_GATEUP: ok = MK_KT_DISPATCH(op_gateup, h, pp, slot, page0, t, epoch); break;
                case OP_DOWN: ok = MK_KT_DISPATCH_2K(op_down, dkt, pp, slot, page0, t, epoch); break;
                case OP_LMHEAD: ok = MK_KT_DISPATCH(op_lmhead, h, pp, slot, page0, t, epoch); break;
                default: break;
            }
        } else {
            switch (k.op) {
                case OP_QKV: ok = MK_KT_DISPATCH_2K(GemvB<OP_QKV>::template n, h, pp, slot, page0, t, epoch); break;
                case OP_GATEUP: ok = MK_KT_DISPATCH_2K(GemvB<OP_GATEUP>::template n, h, pp, slot, page0, t, epoch); break;
                case OP_LMHEAD: ok = MK_KT_DISPATCH_2K(GemvB<OP_LMHEAD>::template n, h, pp, slot, page0, t, epoch); break;
                case OP_OPROJ: ok = MK_KT_DISPATCH_2K(GemvB<OP_OPROJ>::template r, okt, pp, slot, page0, t, epoch); break;
                case OP_DOWN: ok = MK_KT_DISPATCH_2K(GemvB<OP_DOWN>::template r, dkt, pp, slot, page0, t, epoch); break;
                case OP_ROUTE: ok = MK_KT_DISPATCH_2K(GemvB<OP_ROUTE>::template n, h, pp, slot, page0, t, epoch); break;
                case OP_EGU: ok = MK_KT_DISPATCH_2K(GemvB<OP_EGU>::template n, h, pp, slot, page0, t, epoch); break;
                case OP_EDOWN:
                    ok = MK_KT_DISPATCH_2K(GemvB<OP_EDOWN>::template r, p0.T.fe, pp, slot, page0, t, epoch);
                    break;
                case OP_ATTN: ok = attn_kswizzle(p0.T.d, p0.T.grp) ? op_attn_mfma(pp, slot, page0, t, epoch)
                               : hd == 64 ? op_attn<64>(pp, slot, page0, t, epoch)
                                          : op_attn<128>(pp, slot, page0, t, epoch);
                break;
                default: break;
            }
        }
        if (!uni(ok)) return;
        // ---- completion: every wave's stores are done, then wave 0 signals ----
        if (tracing && c.lane == 0) lds_st(S.tw_epi[c.wave], (uint32_t)rtc());
        vm_wait_all();
        if (tracing && c.lane == 0) lds_st(S.tw_ack[c.wave], (uint32_t)rtc());
        release_fence();  // (fenced build) this wave's results before the workgroup's signal
        lgkm_wait_all();
        if (c.lane == 0) lds_add(S.done, 1u);
        if (c.wave == 0) {
            if (!lds_wait_ge(S.done, NCW * (t + 1), pp, k.id)) return;
            const uint64_t t_stored = tracing ? rtc() : 0;  // every wave's results acknowledged by memory
            release_fence();
            CParams& p = P(pp);
            const uint32_t n_sig = (k.flags & TF_SIGRANGE) ? n_exp : 1u;  // router tiles: every expert's event
            bool activated = false;
            if (k.sig_ev != NONE && k.id != drop_task && (uint32_t)c.lane < n_sig) {
                const uint32_t ev = k.sig_ev + (uint32_t)c.lane;
                const uint32_t sub = k.sig_nsub == 8 ? xcc_id() + 8u * ((blockIdx.x >> 3) % (uint32_t)(CTR_SUBS / 8)) : 0u;
                const uint32_t old = addu_dev(&ctr[ctr_index(ev, sub)], 1u);
                // event-driven dispatch: the count that reaches the event's threshold activates it
                activated = sched >= 2 && old + 1u == epoch * p.ev_target[ev];
            }
            if (sched == 2) {
                uint64_t act = __ballot(activated);
                while (act) {
                    const int l = __ffsll((unsigned long long)act) - 1;
                    act &= act - 1;
                    launch_dependents(pp, k.sig_ev + (uint32_t)l, epoch, c.lane);
                }
            } else if (sched == 3 && activated) {
                // post the event to its scheduler's activated-event queue
                st_dev(&p.aeq_stamp[k.sig_ev + (uint32_t)c.lane], epoch);
            }
            if (k.op == OP_LMHEAD || (PF && k.op == OP_PLM)) finish_step(pp, epoch, c.parity);
            if (task_count && c.lane == 0) addu_dev(&task_count[k.id], 1u);
            if (tracing && c.lane == 0) {
                unsigned long long* tr = p.trace + (size_t)k.id * TRACE_WORDS;
                const uint64_t t_ready = ((unsigned long long)lds_ld(S.t_ready_hi) << 32) | lds_ld(S.t_ready_lo);
                const uint64_t hi = t_ready & ~0xffffffffull;
                gst(tr + 0, (unsigned long long)blockIdx.x);
                gst(tr + 1, (unsigned long long)t_fetch);
                gst(tr + 2, (unsigned long long)t_ready);
                gst(tr + 3, (unsigned long long)(hi | lds_ld(S.tm[0])));
                gst(tr + 4, (unsigned long long)(hi | lds_ld(S.tm[1])));
                gst(tr + 5, (unsigned long long)rtc());
                gst(tr + 6, (unsigned long long)t_stored);
                gst(tr + 7, (unsigned long long)(hi | lds_ld(S.tm[2])));
                gst(tr + 8, (unsigned long long)page0);
                uint32_t we = 0, wa = 0;  // the last wave to finish its epilogue / to have its stores acknowledged
#pragma unroll
                for (int w = 0; w < NCW; ++w) {
                    we = max(we, lds_ld(S.tw_epi[w]) - (uint32_t)t_fetch);
                    wa = max(wa, lds_ld(S.tw_ack[w]) - (uint32_t)t_fetch);
                }
                gst(tr + 9, (unsigned long long)(t_fetch + we));
                gst(tr + 10, (unsigned long long)(t_fetch + wa));
                gst(tr + 11, (unsigned long long)(hi | lds_ld(S.tw_epi[0])));
                // the loader's stamps (0: the task has no pages)
                const uint32_t i0 = lds_ld(S.tl_issue0[slot]), i1 = lds_ld(S.tl_issue1[slot]), pb_ = lds_ld(S.tl_pub[slot]);
                gst(tr + 12, i0 ? (unsigned long long)(hi | i0) : 0ull);
                gst(tr + 13, i1 ? (unsigned long long)(hi | i1) : 0ull);
                gst(tr + 14, pb_ ? (unsigned long long)(hi | pb_) : 0ull);
                gst(tr + 15, (unsigned long long)lds_ld(S.tm[3]));  // wave 0's page waits (ticks)
                if (c.lane == 0) {
                    lds_st(S.tm[2], 0u);
                    lds_st(S.tm[3], 0u);
                }
            }
            vm_wait_all();
            if (c.lane == 0) lds_add(S.fifo_free[slot], 1u);
        }
    }
}

// ---- the kernel --------------------------------------------------------------------------

__global__ void __launch_bounds__(NTHREADS, 1) mk_step_kernel(const Params* pp, StepArgs a) {
    const int wave = threadIdx.x >> 6;
    CParams& p = P(pp);
    if (threadIdx.x < FIFO) {
        S.fifo_ready[threadIdx.x] = 0;
        S.fifo_free[threadIdx.x] = 0;
    }
    if (threadIdx.x < NPAGES) {
        for (int lw = 0; lw < NLW; ++lw) S.page_ready[lw][threadIdx.x] = 0;
        S.page_free[threadIdx.x] = 0;
    }
    if (threadIdx.x < NCW) S.cgen[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        S.go = 0;
        S.cbar = 0;
        S.done = 0;
        S.abort = 0;
        S.dyn_ready = 0;
        S.dyn_ack = 0;
        S.trace_on = p.trace != nullptr ? 1u : 0u;
        S.adealt = 0;
        S.tm[2] = 0;
        S.tm[3] = 0;
        S.args = a;
    }
    const uint32_t epoch = p.state[ST_EPOCH];
    const uint32_t parity = epoch & 1u;
    const int B = p.T.B;
    for (int b = threadIdx.x; b < B; b += NTHREADS) {
        S.tok[b] = a.tokens[b];
        S.pos[b] = a.positions[b];
    }
    __syncthreads();
    bool bad = false;
    for (int b = 0; b < B; ++b) {
        if (S.tok[b] < 0 || S.tok[b] >= p.T.V) bad = true;
        if (S.pos[b] < 0 || S.pos[b] >= p.T.C) bad = true;
    }
    if (bad) {
        if (blockIdx.x == 0 && threadIdx.x == 0) raise_error(pp, ERR_INPUT, 0, 0, 0, 0);
    } else {
        // clear the other parity's accumulators and argmax keys for the next step (read only after this launch)
        const size_t nacc = (size_t)(2 * p.T.L + 1) * B * p.T.h;
        float* other = p.acc + (size_t)(parity ^ 1u) * nacc;
        for (size_t i = (size_t)blockIdx.x * NTHREADS + threadIdx.x; i < nacc; i += (size_t)gridDim.x * NTHREADS)
            other[i] = 0.f;
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < KEY_SLOTS * B; i += NTHREADS) p.key[(parity ^ 1u) * KEY_SLOTS * B + i] = 0ull;
        if (p.aticket) {
            const size_t nt = (size_t)p.T.L * B * p.T.nkv;
            for (size_t i = (size_t)blockIdx.x * NTHREADS + threadIdx.x; i < nt; i += (size_t)gridDim.x * NTHREADS)
                p.aticket[(parity ^ 1u) * nt + i] = 0u;
        }
        if (wave >= NCW) loader<MAX_INFLIGHT>(pp, epoch, wave - NCW);
        else compute<false>(pp, epoch, wave);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = addu_dev(&p.state[ST_EXIT], 1u);
        if (old + 1u == epoch * gridDim.x) st_dev(&p.state[ST_EPOCH], epoch + 1u);
    }
}

hipError_t launch_step(const Params* dparams, const StepArgs& a, uint32_t grid, hipStream_t stream, bool cooperative) {
    if (cooperative) {
        StepArgs ac = a;
        const Params* pc = dparams;
        void* args[] = {(void*)&pc, (void*)&ac};
        return hipLaunchCooperativeKernel((const void*)mk_step_kernel, dim3(grid), dim3(NTHREADS), args, 0, stream);
    }
    hipLaunchKernelGGL(mk_step_kernel, dim3(grid), dim3(NTHREADS), 0, stream, dparams, a);
    return hipGetLastError();
}

// The prompt megakernel: the same interpreter (loader waves, LDS ring, queues, events) over a
// prompt graph.  Input check: every prompt token in [0, vocab) (pos0 is checked on the host).
__global__ void __launch_bounds__(NTHREADS, 1) mk_prefill_kernel(const Params* pp, StepArgs a) {
    const int wave = threadIdx.x >> 6;
    CParams& p = P(pp);
    if (threadIdx.x < FIFO) {
        S.fifo_ready[threadIdx.x] = 0;
        S.fifo_free[threadIdx.x] = 0;
    }
    if (threadIdx.x < NPAGES) {
        for (int lw = 0; lw < NLW; ++lw) S.page_ready[lw][threadIdx.x] = 0;
        S.page_free[threadIdx.x] = 0;
    }
    if (threadIdx.x < NCW) S.cgen[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        S.go = 0;
        S.cbar = 0;
        S.done = 0;
        S.abort = 0;
        S.dyn_ready = 0;
        S.dyn_ack = 0;
        S.trace_on = p.trace != nullptr ? 1u : 0u;
        S.adealt = 0;
        S.tm[2] = 0;
        S.tm[3] = 0;
        S.args = a;
    }
    const uint32_t epoch = p.state[ST_EPOCH];
    const uint32_t parity = epoch & 1u;
    int bad = 0;
    for (int t = threadIdx.x; t < p.T.pf_T; t += NTHREADS) {
        const int32_t v = a.tokens[t];
        if (v < 0 || v >= p.T.V) bad = 1;
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        if (blockIdx.x == 0 && threadIdx.x == 0) raise_error(pp, ERR_INPUT, 0, 0, 0, 0);
    } else {
        // the other parity's argmax key, for the next launch (read only after this one)
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < KEY_SLOTS * p.T.B; i += NTHREADS) p.key[(parity ^ 1u) * KEY_SLOTS * p.T.B + i] = 0ull;
        if (wave >= NCW) loader<PF_INFLIGHT>(pp, epoch, wave - NCW);
        else compute<true>(pp, epoch, wave);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = addu_dev(&p.state[ST_EXIT], 1u);
        if (old + 1u == epoch * gridDim.x) st_dev(&p.state[ST_EPOCH], epoch + 1u);
    }
}

hipError_t launch_prefill(const Params* dparams, const StepArgs& a, uint32_t grid, hipStream_t stream, bool cooperative) {
    if (cooperative) {
        StepArgs ac = a;
        const Params* pc = dparams;
        void* args[] = {(void*)&pc, (void*)&ac};
        return hipLaunchCooperativeKernel((const void*)mk_prefill_kernel, dim3(grid), dim3(NTHREADS), args, 0, stream);
    }
    hipLaunchKernelGGL(mk_prefill_kernel, dim3(grid), dim3(NTHREADS), 0, stream, dparams, a);
    return hipGetLastError();
}

// Poison mode: fill each span with its pattern (NaN for floats and bf16 pairs, -1 for expert ids).
__global__ void __launch_bounds__(256) poison_kernel(PoisonSpans s) {
    for (int i = 0; i < s.n; ++i) {
        uint32_t* w = (uint32_t*)s.ptr[i];
        for (uint64_t j = (uint64_t)blockIdx.x * 256 + threadIdx.x; j < s.words[i]; j += (uint64_t)gridDim.x * 256)
            w[j] = s.pattern[i];
    }
}

hipError_t launch_poison(const PoisonSpans& s, hipStream_t stream) {
    hipLaunchKernelGGL(poison_kernel, dim3(256), dim3(256), 0, stream, s);
    return hipGetLastError();
}

// ---- the allocation-free step's scratch ----------------------------------------------------
//
// mk_decode_step_noalloc keeps the step's scratch (event counters, control words, residual
// accumulators, query rows, attention partials, m rows, operand regions, argmax keys, tickets) in
// this file-scope array instead of handle-owned buffers.  Each GPU holds its own copy from the
// moment the library's code object is loaded on it until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device array: only the address hipGetSymbolAddress returns
// for the current device may be handed to kernels or copies.
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch_base(int device, uint8_t** out) {
    static std::mutex mu;
    static void* addr[MAX_DEVICES] = {};
    if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));  // the current device's copy
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        addr[device] = ptr;
    }
    *out = (uint8_t*)addr[device];
    return hipSuccess;
}

// Weight repacking at build time: one workgroup per copy operation.
__global__ void __launch_bounds__(256) repack_kernel(const CopyOp* ops, uint8_t* dst) {
    const CopyOp op = ops[blockIdx.x];
    const uint32_t n16 = op.row_bytes / 16;
    for (uint32_t r = 0; r < op.rows; ++r) {
        const uint4* s = (const uint4*)(op.src + (uint64_t)r * op.src_pitch);
        uint4* d = (uint4*)(dst + op.dst_off + (uint64_t)r * op.row_bytes);
        for (uint32_t i = threadIdx.x; i < n16; i += 256) d[i] = s[i];
    }
}

// GEMV tiles: one workgroup per tile, one 16-byte element per thread and step.
__global__ void __launch_bounds__(256) repack_tiles_kernel(const TileOp* ops, const uint8_t* const* rowsrc, uint8_t* dst) {
    const TileOp op = ops[blockIdx.x];
    const uint32_t n16 = op.rows * (op.kt / 8);
    const uint32_t nkb = op.kt / 32;
    for (uint32_t e = threadIdx.x; e < n16; e += 256) {
        uint32_t row, col;
        if (op.blocked == 2) {  // chunk, then K half, then row group, then column block of the half
            const uint32_t b = e / 64, l = e % 64;
            const uint32_t nrg = op.rows / 16, cr = op.chunk_rows / 16, hb = nkb / 2;
            const uint32_t c = b / (cr * nkb), w = b - c * cr * nkb;
            const uint32_t rgs = min(cr, nrg - c * cr);
            const uint32_t half = w / (rgs * hb), w2 = w % (rgs * hb);
            row = (c * cr + w2 / hb) * 16 + l % 16;
            col = (half * hb + w2 % hb) * 32 + (l / 16) * 8;
        } else if (op.blocked == 3) {  // prompt GEMM pages: page, then column block, then row group
            const uint32_t b = e / 64, l = e % 64;
            const uint32_t nrg = op.rows / 16, kbp = 16 / nrg;
            const uint32_t pg = b / 16, w = b % 16;
            row = (w % nrg) * 16 + l % 16;
            col = (pg * kbp + w / nrg) * 32 + (l / 16) * 8;
        } else if (op.blocked) {  // row-group major: block b = (row group, column block)
            const uint32_t b = e / 64, l = e % 64;
            row = (b / nkb) * 16 + l % 16;
            col = (b % nkb) * 32 + (l / 16) * 8;
        } else {
            row = e / (op.kt / 8);
            col = (e % (op.kt / 8)) * 8;
        }
        const uint8_t* src = rowsrc[op.row_base + row];
        const uint4 v = src ? *(const uint4*)(src + (uint64_t)col * 2) : make_uint4(0, 0, 0, 0);
        *(uint4*)(dst + op.dst_off + (uint64_t)e * 16) = v;
    }
}

hipError_t launch_repack_tiles(const TileOp* ops, uint32_t n_ops, const uint8_t* const* rowsrc, uint8_t* dst,
                               hipStream_t stream) {
    if (n_ops == 0) return hipSuccess;
    hipLaunchKernelGGL(repack_tiles_kernel, dim3(n_ops), dim3(256), 0, stream, ops, rowsrc, dst);
    return hipGetLastError();
}

hipError_t launch_repack(const CopyOp* ops, uint32_t n_ops, uint8_t* dst, hipStream_t stream) {
    if (n_ops == 0) return hipSuccess;
    hipLaunchKernelGGL(repack_kernel, dim3(n_ops), dim3(256), 0, stream, ops, dst);
    return hipGetLastError();
}

int step_threads() { return NTHREADS; }
size_t step_lds_bytes() { return sizeof(Smem); }
const void* step_kernel_ptr() { return (const void*)mk_step_kernel; }
const void* prefill_kernel_ptr() { return (const void*)mk_prefill_kernel; }

}  // namespace mk
