// C ABI of the megakernel library: handle lifecycle, weight repacking, graph
// upload and the one-launch decode step (declarations in include/mk.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "graph.h"
#include "runtime.h"

using namespace mk;

struct mk_handle {
    int device = 0;
    int W = 0;
    bool cooperative = false;  // plain launch unless asked (mk_options.cooperative)
    bool poison = false;       // fill the step's scratch with NaN before every step (mk_options.poison)
    int prompt = 0;            // a prompt (prefill) handle: tokens per launch (mk_build_prefill); 0: decode
    size_t xop_bytes = 0;
    // the allocation-free step: the same parameters with the step's scratch in the per-GPU static
    // array (null when this handle's scratch does not fit it)
    Params p_na;
    Params* dparams_na = nullptr;
    size_t na_bytes = 0;  // scratch this handle's steps need
    // the handle's last step was an allocation-free one: only then is the error record in the
    // per-GPU array its own (the array holds another handle's scratch after that one's steps)
    bool na_last = false;
    bool tied = true;
    Graph g;
    Params p;           // host copy
    Params* dparams = nullptr;  // device copy read by the kernel
    size_t n_events = 0;
    size_t acc_bytes = 0;
    // device allocations owned by the handle
    std::vector<void*> allocs;
};

namespace {

mk_status hip_fail(hipError_t e) {
    (void)e;
    return e == hipErrorOutOfMemory ? MK_E_NOMEM : MK_E_HIP;
}

#define HIPCHK(x)                                        \
    do {                                                 \
        hipError_t e_ = (x);                             \
        if (e_ != hipSuccess) return hip_fail(e_);       \
    } while (0)

template <typename T>
mk_status dalloc(mk_handle* h, T** out, size_t bytes, bool zero) {
    void* p = nullptr;
    if (bytes == 0) bytes = 256;
    HIPCHK(hipMalloc(&p, bytes));
    h->allocs.push_back(p);
    if (zero) HIPCHK(hipMemset(p, 0, bytes));
    *out = (T*)p;
    return MK_OK;
}

Dims dims_of(const mk_model_desc* d) {
    Dims dm;
    dm.L = d->n_layers;
    dm.h = d->hidden;
    dm.nq = d->n_q_heads;
    dm.nkv = d->n_kv_heads;
    dm.d = d->head_dim;
    dm.f = d->ffn_dim;
    dm.V = d->vocab;
    dm.n_experts = d->n_experts;
    dm.top_k = d->top_k;
    dm.fe = d->expert_ffn_dim;
    return dm;
}

mk_status plan(const mk_model_desc* desc, int32_t batch, int32_t max_ctx, const mk_options* opt, int W, Graph* g,
               bool* tied) {
    if (!desc) return MK_E_INVALID;
    mk_options o;
    memset(&o, 0, sizeof(o));
    if (opt) o = *opt;
    if (o.sched < 0 || o.sched > 3 || o.policy < 0 || o.policy > 1) return MK_E_INVALID;
    if (o.page_kib != 0 && o.page_kib != 16) return MK_E_INVALID;  // the page size is part of the weight layout
    if (o.poison < 0 || o.poison > 1) return MK_E_INVALID;
    PlanOptions po;
    po.attn_splits = o.attn_splits;
    Tiling T;
    std::string err;
    Dims dm = dims_of(desc);
    if (dm.n_experts < 0 || batch < 1) return MK_E_INVALID;
    if (batch > MAX_BATCH || (batched_path(batch, dm.n_experts) && dm.h > 2048)) return MK_E_UNSUPPORTED;
    if (plan_tiling(dm, batch, max_ctx, W, po, &T, &err) != 0) return MK_E_INVALID;
    Layout Ly;
    *tied = desc->tied_lm_head != 0;
    plan_layout(T, *tied, &Ly);
    build_graph(T, Ly, o.sched, o.policy, g);
    return MK_OK;
}

mk_status plan_prefill(const mk_model_desc* desc, int32_t n_tokens, int32_t max_ctx, const mk_options* opt, int W,
                       Graph* g, bool* tied) {
    if (!desc) return MK_E_INVALID;
    mk_options o;
    memset(&o, 0, sizeof(o));
    if (opt) o = *opt;
    if (o.sched < 0 || o.sched > 3 || o.policy < 0 || o.policy > 1) return MK_E_INVALID;
    if (o.page_kib != 0 && o.page_kib != 16) return MK_E_INVALID;
    if (o.poison < 0 || o.poison > 1 || o.attn_splits < 0 || o.attn_splits > 16) return MK_E_INVALID;
    Tiling T;
    std::string err;
    bool unsup = false;
    if (plan_prefill_tiling(dims_of(desc), n_tokens, max_ctx, W, &T, &err, &unsup) != 0)
        return unsup ? MK_E_UNSUPPORTED : MK_E_INVALID;
    Layout Ly;
    *tied = desc->tied_lm_head != 0;
    plan_layout(T, *tied, &Ly);
    build_prefill_graph(T, Ly, o.sched, o.policy, g);
    return MK_OK;
}

// Copy the caller's weights into the packed layout: gains and embedding row by
// row (CopyOp), then every GEMV tile in task order (TileOp): rows of the tile
// come from a host-built table of row addresses (null = a zero row of padding),
// and tiles with 128 <= K <= 2048 are stored as 16 x 32 matrix-core blocks.
mk_status repack(mk_handle* h, const mk_model_desc* d, uint8_t* wd) {
    const Tiling& T = h->g.T;
    const Layout& Ly = h->g.lay;
    const uint64_t rowb = (uint64_t)T.h * 2;
    std::vector<CopyOp> ops;
    auto add = [&](const void* src, uint64_t dst_off, uint64_t rows, uint64_t row_bytes, uint64_t pitch) {
        // split large contiguous copies so one workgroup moves at most ~1 MiB
        const uint64_t per = row_bytes >= (1u << 20) ? 1 : std::max<uint64_t>(1, (1u << 20) / row_bytes);
        for (uint64_t r = 0; r < rows; r += per) {
            CopyOp o;
            o.src = (const uint8_t*)src + r * pitch;
            o.dst_off = dst_off + r * row_bytes;
            o.src_pitch = pitch;
            o.rows = (uint32_t)std::min<uint64_t>(per, rows - r);
            o.row_bytes = (uint32_t)row_bytes;
            ops.push_back(o);
        }
    };
    for (int l = 0; l < T.L; ++l) {
        add(d->layers[l].attn_norm, Ly.gains + (uint64_t)(2 * l) * rowb, 1, rowb, rowb);
        add(d->layers[l].ffn_norm, Ly.gains + (uint64_t)(2 * l + 1) * rowb, 1, rowb, rowb);
    }
    add(d->final_norm, Ly.gains + (uint64_t)(2 * T.L) * rowb, 1, rowb, rowb);
    add(d->tok_embed, Ly.embed, (uint64_t)T.V, rowb, rowb);

    std::vector<TileOp> tiles;
    std::vector<const uint8_t*> rows;
    const int half = T.d / 2, P = T.qkv_pairs;
    const uint8_t* lm = (const uint8_t*)(h->tied ? d->tok_embed : d->lm_head);
    for (const Task& k : h->g.tasks) {
        if (k.op == OP_ATTN || k.wbytes == 0 || k.seq != 0) continue;  // column groups (token blocks) share the tiles
        const mk_layer_weights& lw = d->layers[k.layer < T.L ? k.layer : 0];
        TileOp t;
        t.dst_off = k.wofs;
        t.row_base = (uint32_t)rows.size();
        uint32_t kt = (uint32_t)T.h;
        if (k.op == OP_QKV) {
            const uint8_t* src;
            int hrow;
            if (k.part < T.nq) {
                src = (const uint8_t*)lw.wq;
                hrow = k.part * T.d;
            } else if (k.part < T.nq + T.nkv) {
                src = (const uint8_t*)lw.wk;
                hrow = (k.part - T.nq) * T.d;
            } else {
                src = (const uint8_t*)lw.wv;
                hrow = (k.part - T.nq - T.nkv) * T.d;
            }
            for (int i = 0; i < P; ++i) rows.push_back(src + (uint64_t)(hrow + k.row0 + i) * rowb);
            for (int i = 0; i < P; ++i) rows.push_back(src + (uint64_t)(hrow + k.row0 + half + i) * rowb);
        } else if (k.op == OP_OPROJ) {
            kt = (uint32_t)(T.grp * T.d);
            const uint64_t pitch = (uint64_t)T.nq * T.d * 2;
            for (uint32_t i = 0; i < k.nrows; ++i)
                rows.push_back((const uint8_t*)lw.wo + (uint64_t)(k.row0 + i) * pitch + (uint64_t)k.part * kt * 2);
        } else if (k.op == OP_GATEUP) {
            for (uint32_t i = 0; i < k.nrows; ++i) rows.push_back((const uint8_t*)lw.w_gate + (uint64_t)(k.row0 + i) * rowb);
            for (uint32_t i = 0; i < k.nrows; ++i) rows.push_back((const uint8_t*)lw.w_up + (uint64_t)(k.row0 + i) * rowb);
        } else if (k.op == OP_DOWN) {
            kt = (uint32_t)T.kd;
            const uint64_t pitch = (uint64_t)T.f * 2;
            for (uint32_t i = 0; i < k.nrows; ++i)
                rows.push_back((const uint8_t*)lw.w_down + (uint64_t)(k.row0 + i) * pitch + (uint64_t)k.part * kt * 2);
        } else if (k.op == OP_LMHEAD) {
            for (uint32_t i = 0; i < k.nrows; ++i) rows.push_back(lm + (uint64_t)(k.row0 + i) * rowb);
        } else if (k.op == OP_ROUTE) {
            for (uint32_t i = 0; i < k.nrows; ++i) rows.push_back((const uint8_t*)lw.router + (uint64_t)(k.row0 + i) * rowb);
        } else if (k.op == OP_EGU) {
            // m rows row0 .. row0 + nrows of expert `part`, gate and up interleaved in blocks of 32
            const uint64_t e0 = (uint64_t)k.part * T.fe;
            for (uint32_t q = 0; q < k.nrows; q += 32) {
                for (uint32_t i = 0; i < 32; ++i) rows.push_back((const uint8_t*)lw.exp_gate + (e0 + k.row0 + q + i) * rowb);
                for (uint32_t i = 0; i < 32; ++i) rows.push_back((const uint8_t*)lw.exp_up + (e0 + k.row0 + q + i) * rowb);
            }
        } else if (k.op == OP_PQKV) {
            // rows row0 .. of the stacked [Wq; Wk; Wv]
            const uint32_t nqd = (uint32_t)(T.nq * T.d), nkd = (uint32_t)(T.nkv * T.d);
            for (uint32_t i = 0; i < k.nrows; ++i) {
                const uint32_t r = k.row0 + i;
                rows.push_back(r < nqd         ? (const uint8_t*)lw.wq + (uint64_t)r * rowb
                               : r < nqd + nkd ? (const uint8_t*)lw.wk + (uint64_t)(r - nqd) * rowb
                                               : (const uint8_t*)lw.wv + (uint64_t)(r - nqd - nkd) * rowb);
            }
        } else if (k.op == OP_POPROJ || k.op == OP_PDOWN) {
            // rows row0 .. of W_o or W_d over K slice `part`
            const uint64_t kfull = k.op == OP_POPROJ ? (uint64_t)T.nq * T.d : (uint64_t)T.f;
            kt = (uint32_t)(kfull / (uint64_t)T.pf_slices[k.op == OP_POPROJ ? 1 : 3]);
            const uint8_t* src = (const uint8_t*)(k.op == OP_POPROJ ? lw.wo : lw.w_down);
            for (uint32_t i = 0; i < k.nrows; ++i)
                rows.push_back(src + (uint64_t)(k.row0 + i) * kfull * 2 + (uint64_t)k.part * kt * 2);
        } else if (k.op == OP_PGU) {
            // m rows row0 .. row0 + nrows/2: their gate rows, then their up rows
            for (uint32_t i = 0; i < k.nrows / 2; ++i) rows.push_back((const uint8_t*)lw.w_gate + (uint64_t)(k.row0 + i) * rowb);
            for (uint32_t i = 0; i < k.nrows / 2; ++i) rows.push_back((const uint8_t*)lw.w_up + (uint64_t)(k.row0 + i) * rowb);
        } else if (k.op == OP_PLM) {
            for (uint32_t i = 0; i < k.nrows; ++i) rows.push_back(lm + (uint64_t)(k.row0 + i) * rowb);
        } else if (k.op == OP_EDOWN) {
            kt = (uint32_t)T.fe;
            const uint64_t pitch = (uint64_t)T.fe * 2;
            for (uint32_t i = 0; i < k.nrows; ++i)
                rows.push_back((const uint8_t*)lw.exp_down + ((uint64_t)k.part * T.h + k.row0 + i) * pitch);
        }
        t.kt = kt;
        t.rows = (uint32_t)(k.wbytes / (kt * 2));
        while (rows.size() < (size_t)t.row_base + t.rows) rows.push_back(nullptr);
        t.blocked = kt <= 2048 ? 1u : 0u;
        if (k.op == OP_PQKV || k.op == OP_POPROJ || k.op == OP_PGU || k.op == OP_PDOWN) t.blocked = 3u;
        t.chunk_rows = 0;
        if (halves_packed(batched_path(T.B, T.E), k.op, (int)kt)) {
            t.blocked = 2u;
            t.chunk_rows = (uint32_t)halves_chunk_rows(T.B);
        }
        tiles.push_back(t);
    }
    CopyOp* dops = nullptr;
    TileOp* dtiles = nullptr;
    const uint8_t** drows = nullptr;
    hipError_t e = hipMalloc(&dops, std::max<size_t>(1, ops.size()) * sizeof(CopyOp));
    if (e == hipSuccess) e = hipMalloc(&dtiles, std::max<size_t>(1, tiles.size()) * sizeof(TileOp));
    if (e == hipSuccess) e = hipMalloc(&drows, std::max<size_t>(1, rows.size()) * sizeof(void*));
    if (e == hipSuccess) e = hipMemcpy(dops, ops.data(), ops.size() * sizeof(CopyOp), hipMemcpyHostToDevice);
    if (e == hipSuccess && !tiles.empty())
        e = hipMemcpy(dtiles, tiles.data(), tiles.size() * sizeof(TileOp), hipMemcpyHostToDevice);
    if (e == hipSuccess && !rows.empty()) e = hipMemcpy(drows, rows.data(), rows.size() * sizeof(void*), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = launch_repack(dops, (uint32_t)ops.size(), wd, nullptr);
    if (e == hipSuccess) e = launch_repack_tiles(dtiles, (uint32_t)tiles.size(), drows, wd, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    (void)hipFree(dops);
    (void)hipFree(dtiles);
    (void)hipFree(drows);
    HIPCHK(e);
    return MK_OK;
}

mk_status rearm(mk_handle* h) {
    const Tiling& T = h->g.T;
    Params& p = h->p;
    HIPCHK(hipMemset(p.ctr, 0, h->n_events * CTR_SUBS * CTR_LINE * 4));
    std::vector<uint32_t> st(ST_WORDS, 0);
    st[ST_EPOCH] = 1;
    HIPCHK(hipMemcpy(p.state, st.data(), ST_WORDS * 4, hipMemcpyHostToDevice));
    HIPCHK(hipMemset(p.acc, 0, h->acc_bytes));
    if (p.aticket) HIPCHK(hipMemset(p.aticket, 0, (size_t)2 * T.L * T.B * T.nkv * 4));
    if (p.rq_stamp) HIPCHK(hipMemset(p.rq_stamp, 0, h->g.tasks.size() * 4));
    if (p.aeq_stamp) HIPCHK(hipMemset(p.aeq_stamp, 0, h->n_events * 4));
    HIPCHK(hipMemset(p.key, 0, sizeof(unsigned long long) * 2 * KEY_SLOTS * T.B));
    HIPCHK(hipMemset(p.ticket, 0, 4 * T.B));
    HIPCHK(hipDeviceSynchronize());
    return MK_OK;
}

mk_status enqueue_poison(mk_handle* h, const Params& p, float* logits, hipStream_t stream);

bool desc_ok(const mk_model_desc* d) {
    if (!d || !d->tok_embed || !d->final_norm || (!d->tied_lm_head && !d->lm_head)) return false;
    if (d->n_layers > 0 && !d->layers) return false;
    for (int l = 0; l < d->n_layers; ++l) {
        const mk_layer_weights& w = d->layers[l];
        if (!w.attn_norm || !w.wq || !w.wk || !w.wv || !w.wo || !w.ffn_norm) return false;
        if (d->n_experts == 0 && (!w.w_gate || !w.w_up || !w.w_down)) return false;
        if (d->n_experts != 0 && (!w.router || !w.exp_gate || !w.exp_up || !w.exp_down)) return false;
    }
    return true;
}

}  // namespace

extern "C" {

const char* mk_status_str(mk_status s) {
    switch (s) {
        case MK_OK: return "ok";
        case MK_E_INVALID: return "invalid argument";
        case MK_E_UNSUPPORTED: return "unsupported";
        case MK_E_NOMEM: return "out of memory";
        case MK_E_HIP: return "HIP runtime error";
        case MK_E_NOT_RESIDENT: return "persistent grid cannot be co-resident";
        case MK_E_DEVICE: return "device-side error";
        case MK_E_NO_DEVICE: return "no GPU";
    }
    return "unknown status";
}

mk_status mk_plan_graph(const mk_model_desc* desc, int32_t batch, int32_t max_ctx, const mk_options* opt,
                        int32_t n_workgroups, void* buf, size_t cap, size_t* need) {
    if (!desc || n_workgroups < 1) return MK_E_INVALID;
    Graph g;
    bool tied;
    mk_status st = plan(desc, batch, max_ctx, opt, n_workgroups, &g, &tied);
    if (st != MK_OK) return st;
    size_t n = export_size(g);
    if (need) *need = n;
    if (!buf || cap < n) return MK_E_INVALID;
    export_graph(g, buf, cap);
    return MK_OK;
}

}  // extern "C"

namespace {

// A decode handle (prompt = 0) or a prompt handle (prompt = tokens per launch, batch 1).
mk_status build_handle(const mk_model_desc* desc, int32_t batch, int32_t max_ctx, const mk_options* opt, int32_t prompt,
                       mk_handle** out) {
    if (!out) return MK_E_INVALID;
    *out = nullptr;
    if (!desc_ok(desc)) return MK_E_INVALID;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return MK_E_NO_DEVICE;
    mk_options o;
    memset(&o, 0, sizeof(o));
    if (opt) o = *opt;
    mk_handle* h = new mk_handle();
    h->cooperative = o.cooperative != 0;
    h->poison = o.poison != 0;
    HIPCHK(hipGetDevice(&h->device));
    hipDeviceProp_t prop;
    HIPCHK(hipGetDeviceProperties(&prop, h->device));
    int per_cu = 0;
    HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prompt ? prefill_kernel_ptr() : step_kernel_ptr(),
                                                         step_threads(), 0));
    const int max_resident = per_cu * prop.multiProcessorCount;
    h->W = o.n_workgroups > 0 ? o.n_workgroups : prop.multiProcessorCount;
    if (h->W > max_resident) {
        delete h;
        return MK_E_NOT_RESIDENT;
    }
    h->prompt = prompt;
    mk_status st = prompt ? plan_prefill(desc, prompt, max_ctx, &o, h->W, &h->g, &h->tied)
                          : plan(desc, batch, max_ctx, &o, h->W, &h->g, &h->tied);
    if (st != MK_OK) {
        delete h;
        return st;
    }
    const Tiling& T = h->g.T;
    Params& p = h->p;
    memset(&p, 0, sizeof(p));
    p.T = T;
    p.lay = h->g.lay;
    p.eps = desc->rms_eps;
    p.sched = (uint32_t)o.sched;
    p.n_tasks = (uint32_t)h->g.tasks.size();
    p.drop_task = o.debug_drop_signal > 0 ? (uint32_t)(o.debug_drop_signal - 1) : NONE;
    const double ms = o.debug_timeout_ms > 0 ? o.debug_timeout_ms : 2000.0;
    p.timeout = (unsigned long long)(ms * 1e5);  // 100 MHz clock
    h->n_events = h->g.target.size();
    p.n_events = (uint32_t)h->n_events;
#define ALLOC(ptr, bytes, zero)                                   \
    do {                                                          \
        mk_status s_ = dalloc(h, &(ptr), (bytes), (zero));        \
        if (s_ != MK_OK) {                                        \
            mk_destroy(h);                                        \
            return s_;                                            \
        }                                                         \
    } while (0)
#define ALLOC2(ptr, bytes) ALLOC(ptr, bytes, false)
    uint8_t* wd;
    ALLOC(wd, h->g.lay.total, false);
    p.w = wd;
    st = repack(h, desc, wd);
    if (st != MK_OK) {
        mk_destroy(h);
        return st;
    }
    Task* td;
    ALLOC(td, h->g.tasks.size() * sizeof(Task), false);
    p.tasks = td;
    uint32_t *qo, *qq;
    ALLOC(qo, h->g.queue_off.size() * 4, false);
    ALLOC(qq, h->g.queue.size() * 4, false);
    p.queue_off = qo;
    p.queue = qq;
    ALLOC(p.ctr, h->n_events * CTR_SUBS * CTR_LINE * 4, true);
    if (o.sched >= 2) {
        uint32_t *evt, *co, *cs, *rq;
        ALLOC(evt, h->n_events * 4, false);
        ALLOC(co, h->g.cons_off.size() * 4, false);
        ALLOC(cs, std::max<size_t>(1, h->g.cons.size()) * 4, false);
        ALLOC(rq, h->g.tasks.size() * 4, true);
        ALLOC(p.rq_stamp, h->g.tasks.size() * 4, true);
        if (o.sched == 3) ALLOC(p.aeq_stamp, h->n_events * 4, true);
        p.ev_target = evt;
        p.cons_off = co;
        p.cons = cs;
        p.rq = rq;
        p.n_init = (uint32_t)h->g.init.size();
        if (hipMemcpy(evt, h->g.target.data(), h->n_events * 4, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(co, h->g.cons_off.data(), h->g.cons_off.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
            (!h->g.cons.empty() &&
             hipMemcpy(cs, h->g.cons.data(), h->g.cons.size() * 4, hipMemcpyHostToDevice) != hipSuccess) ||
            (!h->g.init.empty() &&
             hipMemcpy(rq, h->g.init.data(), h->g.init.size() * 4, hipMemcpyHostToDevice) != hipSuccess)) {
            mk_destroy(h);
            return MK_E_HIP;
        }
    }
    ALLOC(p.state, ST_WORDS * 4, true);
    float2* rope;
    const int half = T.d / 2;
    ALLOC(rope, (size_t)T.C * half * sizeof(float2), false);
    p.rope = rope;
    if (prompt) {
        // prompt buffers: query operands, the residual rows (input of a layer, after its attention) and
        // the K-slice partial outputs of the O- and down projections, and the matrix-core operand regions (normalised inputs, attention output, SiLU(gate) * up, final
        // normalised last token), all zero at first (the columns of the tokens past the prompt in its
        // last group of 16 stay zero or finite)
        const size_t ntg = (size_t)(T.pf_T + 15) / 16;
        ALLOC(p.q, ntg * T.nq * (T.d / 32) * 2048, true);
        ALLOC(p.part, 256, true);
        ALLOC(p.m, 256, true);
        h->acc_bytes = (2 + (size_t)T.pf_slices[1] + (size_t)T.pf_slices[3]) * ntg * 16 * T.h * 4;
        ALLOC(p.acc, h->acc_bytes, true);
        h->xop_bytes = (ntg * ((size_t)T.h + (size_t)T.nq * T.d + (size_t)T.f) + T.h) / 32 * 2048;
        ALLOC(p.xop, h->xop_bytes, true);
    } else {
    ALLOC(p.q, (size_t)T.B * T.nq * T.d * 4, true);
    ALLOC(p.part, (size_t)T.B * T.nkv * part_chunks(batched_path(T.B, T.E), T.attn_splits) * T.grp * (T.d + 2) * 4, true);
    ALLOC(p.m, (size_t)T.B * T.f * 4, true);
    h->acc_bytes = (size_t)2 * (2 * T.L + 1) * T.B * T.h * 4;
    ALLOC(p.acc, h->acc_bytes, true);
    }
    if (!prompt && batched_path(T.B, T.E)) {
        // matrix-core operands of the O- and down-projection inputs: 2 bf16 parts x 16
        // sequences per column (columns of absent sequences stay zero for the handle's life)
        const size_t n_sg = (size_t)(T.B + GROUP_SEQS - 1) / GROUP_SEQS;
        // (then, for a mixture of experts, every expert's m rows)
        const size_t xop_elems =
            ((size_t)T.L * T.nq * T.d + (size_t)T.L * T.f + (size_t)T.L * T.E * T.fe) * n_sg * 32;
        h->xop_bytes = xop_elems * 2;
        ALLOC(p.xop, xop_elems * 2, true);
        ALLOC(p.aticket, (size_t)2 * T.L * T.B * T.nkv * 4, true);
        if (T.E) {
            ALLOC(p.rlogit, (size_t)T.L * T.B * T.E * 4, true);
            ALLOC(p.eids, (size_t)T.L * T.B * T.topk * 4, true);
        }
    }
    if (prompt) p.hidden = p.acc + (size_t)(T.pf_T + 15) / 16 * 16 * T.h;  // the residual after the last layer
    else ALLOC(p.hidden, (size_t)T.B * T.h * 4, true);
    ALLOC(p.key, sizeof(unsigned long long) * 2 * KEY_SLOTS * T.B, true);
    ALLOC(p.ticket, 4 * T.B, true);
    ALLOC(p.next, 4 * T.B, true);
    if (o.trace) {
        ALLOC(p.task_count, h->g.tasks.size() * 4, true);
        ALLOC(p.trace, h->g.tasks.size() * 8 * TRACE_WORDS, true);
    }
    auto up = [&](void* dst, const void* src, size_t n) { return hipMemcpy(dst, src, n, hipMemcpyHostToDevice); };
    if (up(td, h->g.tasks.data(), h->g.tasks.size() * sizeof(Task)) != hipSuccess ||
        up(qo, h->g.queue_off.data(), h->g.queue_off.size() * 4) != hipSuccess ||
        up(qq, h->g.queue.data(), h->g.queue.size() * 4) != hipSuccess) {
        mk_destroy(h);
        return MK_E_HIP;
    }
    // RoPE table: angle = pos * theta^(-2j/d), evaluated in double, stored as float (cos, sin)
    std::vector<float2> tab((size_t)T.C * half);
    for (int pos = 0; pos < T.C; ++pos)
        for (int j = 0; j < half; ++j) {
            double a = (double)pos * std::pow((double)desc->rope_theta, -2.0 * j / (double)T.d);
            tab[(size_t)pos * half + j] = make_float2((float)std::cos(a), (float)std::sin(a));
        }
    if (up(rope, tab.data(), tab.size() * sizeof(float2)) != hipSuccess) {
        mk_destroy(h);
        return MK_E_HIP;
    }
    if (!prompt) {
        // the allocation-free step: the same buffers laid out in this GPU's static scratch array
        // (tasks, queues, weights, RoPE table, outputs and the event-driven lists stay the handle's)
        size_t at = 0;
        auto take = [&](size_t bytes) {  // 256-byte aligned, at least 256 bytes (as dalloc)
            const size_t o = at;
            at += std::max<size_t>(256, (bytes + 255) / 256 * 256);
            return o;
        };
        const size_t o_ctr = take(h->n_events * CTR_SUBS * CTR_LINE * 4), o_state = take(ST_WORDS * 4);
        const size_t o_q = take((size_t)T.B * T.nq * T.d * 4);
        const size_t o_part = take((size_t)T.B * T.nkv * part_chunks(batched_path(T.B, T.E), T.attn_splits) * T.grp * (T.d + 2) * 4);
        const size_t o_m = take((size_t)T.B * T.f * 4), o_acc = take(h->acc_bytes);
        const size_t o_xop = batched_path(T.B, T.E) ? take(h->xop_bytes) : 0;
        const size_t o_at = batched_path(T.B, T.E) ? take((size_t)2 * T.L * T.B * T.nkv * 4) : 0;
        const size_t o_rl = T.E ? take((size_t)T.L * T.B * T.E * 4) : 0;
        const size_t o_key = take(sizeof(unsigned long long) * 2 * KEY_SLOTS * T.B), o_ticket = take(4 * (size_t)T.B);
        const size_t o_rqs = o.sched >= 2 ? take(h->g.tasks.size() * 4) : 0;
        const size_t o_aeq = o.sched == 3 ? take(h->n_events * 4) : 0;
        h->na_bytes = at;
        if (at <= NOALLOC_SCRATCH_BYTES) {
            uint8_t* base = nullptr;
            const hipError_t e = noalloc_scratch_base(h->device, &base);
            if (e != hipSuccess) {
                mk_destroy(h);
                return hip_fail(e);
            }
            Params q = p;
            q.ctr = (uint32_t*)(base + o_ctr);
            q.state = (uint32_t*)(base + o_state);
            q.q = (float*)(base + o_q);
            q.part = (float*)(base + o_part);
            q.m = (float*)(base + o_m);
            q.acc = (float*)(base + o_acc);
            q.xop = batched_path(T.B, T.E) ? (uint16_t*)(base + o_xop) : nullptr;
            q.aticket = batched_path(T.B, T.E) ? (uint32_t*)(base + o_at) : nullptr;
            q.rlogit = T.E ? (float*)(base + o_rl) : nullptr;
            q.key = (unsigned long long*)(base + o_key);
            q.ticket = (uint32_t*)(base + o_ticket);
            q.rq_stamp = o.sched >= 2 ? (uint32_t*)(base + o_rqs) : nullptr;
            q.aeq_stamp = o.sched == 3 ? (uint32_t*)(base + o_aeq) : nullptr;
            h->p_na = q;
            Params* dq;
            ALLOC2(dq, sizeof(Params));
            h->dparams_na = dq;
            if (up(dq, &q, sizeof(Params)) != hipSuccess) {
                mk_destroy(h);
                return MK_E_HIP;
            }
        }
    }
    Params* dp;
    ALLOC2(dp, sizeof(Params));
    h->dparams = dp;
    if (up(dp, &p, sizeof(Params)) != hipSuccess) {
        mk_destroy(h);
        return MK_E_HIP;
    }
    st = rearm(h);
    if (st != MK_OK) {
        mk_destroy(h);
        return st;
    }
    *out = h;
    return MK_OK;
#undef ALLOC2
#undef ALLOC
}

}  // namespace

extern "C" {

mk_status mk_build_graph(const mk_model_desc* desc, int32_t batch, int32_t max_ctx, const mk_options* opt,
                         mk_handle** out) {
    return build_handle(desc, batch, max_ctx, opt, 0, out);
}

mk_status mk_build_prefill(const mk_model_desc* desc, int32_t n_tokens, int32_t max_ctx, const mk_options* opt,
                           mk_handle** out) {
    if (n_tokens < 1) {
        if (out) *out = nullptr;
        return MK_E_INVALID;
    }
    return build_handle(desc, 1, max_ctx, opt, n_tokens, out);
}

mk_status mk_plan_prefill(const mk_model_desc* desc, int32_t n_tokens, int32_t max_ctx, const mk_options* opt,
                          int32_t n_workgroups, void* buf, size_t cap, size_t* need) {
    if (!desc || n_workgroups < 1 || n_tokens < 1) return MK_E_INVALID;
    Graph g;
    bool tied;
    mk_status st = plan_prefill(desc, n_tokens, max_ctx, opt, n_workgroups, &g, &tied);
    if (st != MK_OK) return st;
    size_t n = export_size(g);
    if (need) *need = n;
    if (!buf || cap < n) return MK_E_INVALID;
    export_graph(g, buf, cap);
    return MK_OK;
}

mk_status mk_prefill(mk_handle* h, const int32_t* tokens, int32_t pos0, void* kv_cache, float* logits, void* stream) {
    if (!h || !h->prompt || !tokens || !kv_cache) return MK_E_INVALID;
    const Tiling& T = h->g.T;
    if (pos0 < 0 || pos0 > T.C - T.pf_T) return MK_E_INVALID;
    StepArgs a;
    a.tokens = tokens;
    a.positions = nullptr;
    a.kc = (uint16_t*)kv_cache;
    a.vc = (uint16_t*)kv_cache + (size_t)T.L * T.B * T.nkv * (size_t)T.C * T.d;
    a.logits = logits;
    a.pos0 = pos0;
    if (h->poison) {
        const mk_status st = enqueue_poison(h, h->p, logits, (hipStream_t)stream);
        if (st != MK_OK) return st;
    }
    h->na_last = false;
    hipError_t e = launch_prefill(h->dparams, a, (uint32_t)h->W, (hipStream_t)stream, h->cooperative);
    if (e == hipErrorCooperativeLaunchTooLarge) return MK_E_NOT_RESIDENT;
    return e == hipSuccess ? MK_OK : MK_E_HIP;
}

size_t mk_kv_cache_bytes(const mk_handle* h) {
    if (!h) return 0;
    const Tiling& T = h->g.T;
    return (size_t)2 * T.L * T.B * T.nkv * (size_t)T.C * T.d * 2;
}

mk_status mk_decode_step(mk_handle* h, const int32_t* tokens, const int32_t* positions, void* kv_cache, float* logits,
                         void* stream) {
    if (!h || h->prompt || !tokens || !positions || (!kv_cache && h->g.T.L > 0)) return MK_E_INVALID;
    const Tiling& T = h->g.T;
    StepArgs a;
    a.tokens = tokens;
    a.positions = positions;
    a.kc = (uint16_t*)kv_cache;
    a.vc = (uint16_t*)kv_cache + (size_t)T.L * T.B * T.nkv * (size_t)T.C * T.d;
    a.logits = logits;
    a.pos0 = 0;
    if (h->poison) {
        const mk_status st = enqueue_poison(h, h->p, logits, (hipStream_t)stream);
        if (st != MK_OK) return st;
    }
    h->na_last = false;
    hipError_t e = launch_step(h->dparams, a, (uint32_t)h->W, (hipStream_t)stream, h->cooperative);
    if (e == hipErrorCooperativeLaunchTooLarge) return MK_E_NOT_RESIDENT;
    return e == hipSuccess ? MK_OK : MK_E_HIP;
}

mk_status mk_decode_step_noalloc(mk_handle* h, const int32_t* tokens, const int32_t* positions, void* kv_cache,
                                 float* logits, void* stream) {
    if (!h || h->prompt || !tokens || !positions || (!kv_cache && h->g.T.L > 0)) return MK_E_INVALID;
    if (!h->dparams_na) return MK_E_UNSUPPORTED;  // this handle's scratch exceeds the static array
    const Tiling& T = h->g.T;
    const Params& p = h->p_na;
    // This GPU's array keeps whatever the last call (of any handle) left in it: clear what must start
    // at zero and start the step at epoch 1 (parity 1), with a fill kernel (no memset, no allocation).
    PoisonSpans cs;
    memset(&cs, 0, sizeof(cs));
    bool too_many = false;  // (more spans than the fill kernel takes: a build error, never expected)
    auto span = [&](void* ptr, size_t bytes, uint32_t pattern) {
        if (!ptr || !bytes) return;
        if (cs.n >= MAX_SPANS) {
            too_many = true;
            return;
        }
        cs.ptr[cs.n] = ptr;
        cs.words[cs.n] = bytes / 4;
        cs.pattern[cs.n] = pattern;
        ++cs.n;
    };
    const size_t nacc = (size_t)(2 * T.L + 1) * T.B * T.h, nat = (size_t)T.L * T.B * T.nkv;
    span(p.ctr, h->n_events * CTR_SUBS * CTR_LINE * 4, 0u);
    span(p.state + 1, (ST_WORDS - 1) * 4, 0u);
    span(p.state + ST_EPOCH, 4, 1u);  // ST_EPOCH is word 0
    span(p.acc + nacc, nacc * 4, 0u);  // parity 1
    span(p.key + (size_t)KEY_SLOTS * T.B, (size_t)KEY_SLOTS * T.B * 8, 0u);
    span(p.ticket, (size_t)T.B * 4, 0u);
    span(p.aticket ? p.aticket + nat : nullptr, nat * 4, 0u);
    span(p.rq_stamp, h->g.tasks.size() * 4, 0u);
    span(p.aeq_stamp, h->n_events * 4, 0u);
    if (too_many) return MK_E_INVALID;
    hipError_t e = launch_poison(cs, (hipStream_t)stream);
    if (e != hipSuccess) return MK_E_HIP;
    if (h->poison) {
        const mk_status st = enqueue_poison(h, p, logits, (hipStream_t)stream);
        if (st != MK_OK) return st;
    }
    StepArgs a;
    a.tokens = tokens;
    a.positions = positions;
    a.kc = (uint16_t*)kv_cache;
    a.vc = (uint16_t*)kv_cache + (size_t)T.L * T.B * T.nkv * (size_t)T.C * T.d;
    a.logits = logits;
    a.pos0 = 0;
    h->na_last = true;
    e = launch_step(h->dparams_na, a, (uint32_t)h->W, (hipStream_t)stream, h->cooperative);
    if (e == hipErrorCooperativeLaunchTooLarge) return MK_E_NOT_RESIDENT;
    return e == hipSuccess ? MK_OK : MK_E_HIP;
}

}  // extern "C"

namespace {
// Poison mode: everything a producer of the step overwrites, so a task that read it first would see NaN.
mk_status enqueue_poison(mk_handle* h, const Params& p, float* logits, hipStream_t stream) {
    const Tiling& T = h->g.T;
    {
        PoisonSpans ps;
        memset(&ps, 0, sizeof(ps));
        auto span = [&](void* ptr, size_t bytes, uint32_t pattern) {
            if (!ptr || !bytes || ps.n >= MAX_SPANS) return;  // (8 spans at most are named below)
            ps.ptr[ps.n] = ptr;
            ps.words[ps.n] = bytes / 4;
            ps.pattern[ps.n] = pattern;
            ++ps.n;
        };
        const uint32_t fnan = 0x7fc00000u, bnan2 = 0x7fc07fc0u, neg1 = 0xffffffffu;
        if (h->prompt) {
            // query operands, operand regions, residual rows and logits (each written before it is read;
            // columns of tokens past the prompt only ever meet other such columns)
            span(p.q, (size_t)(T.pf_T + 15) / 16 * T.nq * (T.d / 32) * 2048, fnan);
            span(p.xop, h->xop_bytes, bnan2);
            span(p.acc, h->acc_bytes, fnan);
            span(logits, (size_t)T.V * 4, fnan);
            hipError_t e = launch_poison(ps, stream);
            return e == hipSuccess ? MK_OK : MK_E_HIP;
        }
        span(p.q, (size_t)T.B * T.nq * T.d * 4, fnan);
        span(p.part, (size_t)T.B * T.nkv * part_chunks(batched_path(T.B, T.E), T.attn_splits) * T.grp * (T.d + 2) * 4, fnan);
        span(p.m, (size_t)T.B * T.f * 4, fnan);
        span(p.xop, h->xop_bytes, bnan2);
        span(p.rlogit, (size_t)T.L * T.B * T.E * 4, fnan);
        span(p.eids, (size_t)T.L * T.B * T.topk * 4, neg1);
        span(p.hidden, (size_t)T.B * T.h * 4, fnan);
        span(logits, (size_t)T.B * T.V * 4, fnan);
        hipError_t e = launch_poison(ps, stream);
        if (e != hipSuccess) return MK_E_HIP;
    }
    return MK_OK;
}
}  // namespace

extern "C" {

const int32_t* mk_next_tokens(const mk_handle* h) { return h ? h->p.next : nullptr; }
const float* mk_hidden_out(const mk_handle* h) { return h ? h->p.hidden : nullptr; }
const int32_t* mk_expert_ids(const mk_handle* h) { return h ? h->p.eids : nullptr; }

mk_status mk_check_device_error(mk_handle* h, char* msg, size_t cap) {
    if (!h) return MK_E_INVALID;
    HIPCHK(hipDeviceSynchronize());
    uint32_t rec[8];
    HIPCHK(hipMemcpy(rec, h->p.state + ST_ERR, sizeof(rec), hipMemcpyDeviceToHost));
    if (rec[0] == ERR_NONE && h->dparams_na && h->na_last) {
        // this handle's last step was allocation-free: its record is in the per-GPU array (kept
        // until the next allocation-free step on this GPU clears it)
        HIPCHK(hipMemcpy(rec, h->p_na.state + ST_ERR, sizeof(rec), hipMemcpyDeviceToHost));
        if (rec[0] != ERR_NONE) {
            const uint32_t zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            HIPCHK(hipMemcpy(h->p_na.state + ST_ERR, zero, sizeof(zero), hipMemcpyHostToDevice));
        }
    }
    if (rec[0] == ERR_NONE) return MK_OK;
    if (msg && cap) {
        const char* what = rec[0] == ERR_TIMEOUT_EVENT ? "timeout waiting for an event counter"
                           : rec[0] == ERR_TIMEOUT_LDS ? "timeout waiting inside a workgroup"
                           : rec[0] == ERR_INPUT     ? "token or position out of range"
                                                     : "unknown device error";
        snprintf(msg, cap, "%s (workgroup %u, task %u, event %u, seen %u, target %u)", what, rec[1], rec[2], rec[3],
                 rec[4], rec[5]);
    }
    mk_status st = rearm(h);
    return st == MK_OK ? MK_E_DEVICE : st;
}

mk_status mk_export_graph(const mk_handle* h, void* buf, size_t cap, size_t* need) {
    if (!h) return MK_E_INVALID;
    size_t n = export_size(h->g);
    if (need) *need = n;
    if (!buf || cap < n) return MK_E_INVALID;
    export_graph(h->g, buf, cap);
    return MK_OK;
}

mk_status mk_read_counters(mk_handle* h, uint32_t* host, size_t n, uint32_t* epoch) {
    if (!h || (!host && n)) return MK_E_INVALID;
    HIPCHK(hipDeviceSynchronize());
    std::vector<uint32_t> raw(h->n_events * CTR_SUBS * CTR_LINE);
    HIPCHK(hipMemcpy(raw.data(), h->p.ctr, raw.size() * 4, hipMemcpyDeviceToHost));
    for (size_t e = 0; e < n && e < h->n_events; ++e) {
        uint32_t s = 0;
        for (int k = 0; k < CTR_SUBS; ++k) s += raw[(e * CTR_SUBS + k) * CTR_LINE];
        host[e] = s;
    }
    if (epoch) {
        uint32_t ep;
        HIPCHK(hipMemcpy(&ep, h->p.state + ST_EPOCH, 4, hipMemcpyDeviceToHost));
        *epoch = ep - 1;  // steps completed since the last re-arm
    }
    return MK_OK;
}

mk_status mk_read_task_counts(mk_handle* h, uint32_t* host, size_t n) {
    if (!h || !host) return MK_E_INVALID;
    if (!h->p.task_count) return MK_E_UNSUPPORTED;
    HIPCHK(hipDeviceSynchronize());
    size_t m = n < h->g.tasks.size() ? n : h->g.tasks.size();
    HIPCHK(hipMemcpy(host, h->p.task_count, m * 4, hipMemcpyDeviceToHost));
    return MK_OK;
}

mk_status mk_read_trace(mk_handle* h, uint64_t* host, size_t n) {
    if (!h || !host) return MK_E_INVALID;
    if (!h->p.trace) return MK_E_UNSUPPORTED;
    HIPCHK(hipDeviceSynchronize());
    size_t m = n < h->g.tasks.size() * TRACE_WORDS ? n : h->g.tasks.size() * TRACE_WORDS;
    HIPCHK(hipMemcpy(host, h->p.trace, m * 8, hipMemcpyDeviceToHost));
    return MK_OK;
}

void mk_destroy(mk_handle* h) {
    if (!h) return;
    (void)hipDeviceSynchronize();
    for (void* a : h->allocs) (void)hipFree(a);
    delete h;
}

}  // extern "C"
