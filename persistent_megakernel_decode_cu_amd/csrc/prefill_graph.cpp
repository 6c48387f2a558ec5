// Host builder of the prompt (prefill) graph (pure C++, no GPU calls): the tile planner of
// its GEMMs and the task list, events and queues of one prompt launch.
#include <algorithm>
#include <cstring>
#include <vector>

#include "graph.h"

namespace mk {

static int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }

// ---- the prompt (prefill) graph -----------------------------------------------------------
//
// One launch runs the T tokens of one sequence's prompt through the decoder: the prefill
// pass that runs once per request, before decoding (knowledge-base digest "megakernel
// boundary selection", list of first-used concepts; its planner gives Llama-1B a second
// megakernel for it, Figure 4).  The projections are GEMMs over token blocks on the matrix
// cores (rows x 64 or 128 tokens per task); between them sit RMSNorm tasks of 4 tokens and
// causal attention tasks of 16 query tokens x one KV group.  Events, queues and the
// interpreter are those of the decode graph.

int plan_prefill_tiling(const Dims& dm, int Tn, int C, int W, Tiling* t, std::string* err, bool* unsupported) {
    auto fail = [&](const char* m, bool unsup = false) {
        if (err) *err = m;
        if (unsupported) *unsupported = unsup;
        return -1;
    };
    if (dm.n_experts) return fail("the prompt megakernel covers dense models", true);
    if (dm.L < 1 || dm.h <= 0 || dm.nq <= 0 || dm.nkv <= 0 || dm.d <= 0 || dm.V <= 0 || dm.f <= 0)
        return fail("non-positive model dimension");
    if (Tn < 1 || C < Tn || W < 1) return fail("1 <= prompt tokens <= max_ctx and workgroups >= 1");
    if (dm.nq % dm.nkv) return fail("n_q_heads must be a multiple of n_kv_heads");
    if (dm.d != 64) return fail("the prompt attention tiles are written for head_dim 64", true);
    if (dm.h % 512 || dm.h > 2048) return fail("the prompt graph needs hidden a multiple of 512, at most 2048", true);
    if (dm.f % 128 || (dm.nq * dm.d) % 128) return fail("ffn_dim and n_q*head_dim must be multiples of 128", true);
    if (dm.nq / dm.nkv > 16) return fail("more than 16 query heads per KV head");
    Tiling& T = *t;
    memset(&T, 0, sizeof(T));
    T.L = dm.L; T.h = dm.h; T.nq = dm.nq; T.nkv = dm.nkv; T.d = dm.d; T.f = dm.f; T.V = dm.V;
    T.B = 1; T.C = C; T.W = W; T.grp = dm.nq / dm.nkv;
    T.attn_splits = 1;
    T.pf_T = Tn;
    // per GEMM: (output rows, K) and whether its K may be sliced (the residual-adding ones)
    const int64_t N[PF_GEMMS] = {(int64_t)(dm.nq + 2 * dm.nkv) * dm.d, dm.h, 2ll * dm.f, dm.h};
    const int64_t K[PF_GEMMS] = {dm.h, (int64_t)dm.nq * dm.d, dm.h, dm.f};
    for (int op = 0; op < PF_GEMMS; ++op) {
        // the shape whose estimated time is least: rounds of W tasks x pages per task x the time
        // of a page, the larger of its matrix-core work (512 ngw cycles: 16 blocks x ngw token
        // groups x 2 parts per wave) and its L2 reads at about 64 bytes a cycle (the 16 KiB page
        // plus 4 waves x ngw x its column blocks x 2 KiB of operands); ties to the fewest tasks
        int64_t best_cost = -1, best_tasks = 0;
        const int shapes[3][2] = {{128, 2}, {128, 1}, {64, 1}};
        for (const auto& sh : shapes) {
            const int rows = sh[0], ngw = sh[1];
#ifdef MK_PF_ONLY_SHAPE  // (tuning builds: one tile shape only, 0, 1 or 2 of the list)
            if (&sh != &shapes[MK_PF_ONLY_SHAPE]) continue;
#endif
            if (N[op] % rows) continue;
            if (op == 2 && dm.f % (rows / 2)) continue;
            const int64_t page_cols = 32ll * pf_kbp(rows);
            for (int S = 1; S <= (op == 1 || op == 3 ? PF_MAX_SLICES : 1); S *= 2) {
                if (K[op] % (S * page_cols) || K[op] / S < 256) continue;
                const int64_t tasks = N[op] / rows * ((Tn + 64 * ngw - 1) / (64 * ngw)) * S;
                const int64_t pages = rows * (K[op] / S) * 2 / 16384;
                const int64_t page_time = std::max<int64_t>(512ll * ngw, 256 + 128ll * ngw * pf_kbp(rows));
                const int64_t cost = (tasks + W - 1) / W * pages * page_time;
                if (best_cost < 0 || cost < best_cost || (cost == best_cost && tasks < best_tasks)) {
                    best_cost = cost;
                    best_tasks = tasks;
                    T.pf_rows[op] = rows;
                    T.pf_ngw[op] = ngw;
                    T.pf_slices[op] = S;
                }
            }
        }
        if (best_cost < 0) return fail("no prompt GEMM tile divides the projection", true);
    }
    T.lm_rows = (int)std::min<int64_t>(MAX_TILE_ROWS, round16((dm.V + W - 1) / W));
    T.n_lm_tiles = (dm.V + T.lm_rows - 1) / T.lm_rows;
    return 0;
}

int build_prefill_graph(const Tiling& T, const Layout& Ly, int sched, int policy, Graph* G) {
    Graph& g = *G;
    g.T = T;
    g.lay = Ly;
    g.sched = (uint32_t)sched;
    g.tasks.clear();
    g.target.clear();
    g.nsub.clear();
    const uint64_t h = T.h;
    const int L = T.L, ntg = (T.pf_T + 15) / 16;
    auto add = [&](Task k) {
        k.id = (uint32_t)g.tasks.size();
        g.tasks.push_back(k);
        if (k.sig_ev != NONE) g.target[k.sig_ev] += 1;
    };
    auto blank = [](uint8_t op, int layer, uint32_t wait, uint32_t sig) {
        Task k;
        memset(&k, 0, sizeof(k));
        k.op = op;
        k.layer = (uint16_t)layer;
        k.wait_ev = wait;
        k.sig_ev = sig;
        k.wait_nsub = 1;
        k.sig_nsub = 1;
        return k;
    };
    // RMSNorm tasks of 4 tokens each (kind 0: attention input, 1: FFN input, 2: the final residual),
    // which also add the previous projection's K-slice partials to the residual
    // RMSNorm tasks: of one token while the prompt has no more tokens than there are workgroups
    // (a phase of one round, each task's loads a quarter of a four-token task's), else of four
    const int tpn = T.pf_T <= T.W ? 1 : 4, nnorm = (T.pf_T + tpn - 1) / tpn;
    auto norms = [&](int l, int kind, uint32_t wait, uint32_t sig) {
        for (int q = 0; q < nnorm; ++q) {
            Task k = blank(OP_PNORM, l, wait, sig);
            k.part = (uint16_t)kind;
            k.seq = (uint32_t)q;
            k.nrows = (uint32_t)tpn;  // tokens tpn q .. tpn q + tpn - 1
            add(k);
        }
    };
    // GEMM tiles of projection `op`, listed tile by tile (a tile's K slices and token blocks together)
    // and placed so that, under round-robin queues, each run of W/8 consecutive tiles-and-blocks falls
    // on the workgroups of one XCD in the same round (workgroup w runs on XCD w mod 8): the token
    // blocks of one weight tile run at the same time on one XCD and read its weights through one L2
    const uint8_t opc[PF_GEMMS] = {OP_PQKV, OP_POPROJ, OP_PGU, OP_PDOWN};
    const int64_t N[PF_GEMMS] = {(int64_t)(T.nq + 2 * T.nkv) * T.d, T.h, 2ll * T.f, T.h};
    const int64_t K[PF_GEMMS] = {T.h, (int64_t)T.nq * T.d, T.h, T.f};
    auto gemms = [&](int l, int op, uint64_t region, uint32_t wait, uint32_t sig) {
        const int rows = T.pf_rows[op], ngw = T.pf_ngw[op], S = T.pf_slices[op];
        const int ntb = (T.pf_T + 64 * ngw - 1) / (64 * ngw);
        const int64_t nrt = N[op] / rows;
        const uint32_t wbytes = (uint32_t)(rows * (K[op] / S) * 2);
        std::vector<Task> list;
        for (int64_t r = 0; r < nrt; ++r)
            for (int s = 0; s < S; ++s)
                for (int tb = 0; tb < ntb; ++tb) {
                    Task k = blank(opc[op], l, wait, sig);
                    k.part = (uint16_t)s;
                    k.row0 = (uint32_t)(op == 2 ? r * rows / 2 : r * rows);  // gate/up: the first m row
                    k.nrows = (uint32_t)rows;
                    k.seq = (uint32_t)tb;
                    k.flags = ngw == 2 ? TF_NGW2 : 0;
                    k.wbytes = wbytes;
                    k.wofs = Ly.layer0 + (uint64_t)l * Ly.layer_bytes + region + ((uint64_t)s * nrt + r) * wbytes;
                    list.push_back(k);
                }
        const size_t n = list.size(), Wn = (size_t)T.W;
        if (Wn % 8 == 0) {
            // round r holds m = min(W, n - r W) tasks; when m is a multiple of 8, its i-th task goes to
            // XCD i / (m / 8), slot i mod (m / 8), i.e. position 8 slot + XCD of the round
            std::vector<Task> placed(list);
            for (size_t r0 = 0; r0 < n; r0 += Wn) {
                const size_t m = std::min(Wn, n - r0), G = m / 8;
                if (m % 8) continue;
                for (size_t i = 0; i < m; ++i) placed[r0 + 8 * (i % G) + i / G] = list[r0 + i];
            }
            list.swap(placed);
        }
        for (const Task& k : list) add(k);
    };
    uint32_t ev_x = NONE;
    for (int l = 0; l < L; ++l) {
        const uint32_t ev_n1 = g.new_event(), ev_q = g.new_event(), ev_a = g.new_event(), ev_o = g.new_event();
        const uint32_t ev_n2 = g.new_event(), ev_g = g.new_event(), ev_d = g.new_event();
        norms(l, 0, ev_x, ev_n1);
        gemms(l, 0, Ly.qkv, ev_n1, ev_q);
        // attention: the longest (last) query groups first
        for (int qg = ntg - 1; qg >= 0; --qg)
            for (int gi = 0; gi < T.nkv; ++gi) {
                Task k = blank(OP_PATTN, l, ev_q, ev_a);
                k.part = (uint16_t)gi;
                k.seq = (uint32_t)qg;
                k.nrows = (uint32_t)T.grp;
                add(k);
            }
        gemms(l, 1, Ly.o, ev_a, ev_o);
        norms(l, 1, ev_o, ev_n2);
        gemms(l, 2, Ly.gu, ev_n2, ev_g);
        gemms(l, 3, Ly.down, ev_g, ev_d);
        ev_x = ev_d;
    }
    // the final residual of every token (the last one also normalised for the LM head), LM head + argmax
    const uint32_t ev_f = g.new_event();
    norms(L, 2, ev_x, ev_f);
    for (int t = 0; t < T.n_lm_tiles; ++t) {
        Task k = blank(OP_PLM, L, ev_f, NONE);
        k.row0 = (uint32_t)(t * T.lm_rows);
        k.nrows = (uint32_t)std::min<int64_t>(T.lm_rows, (int64_t)T.V - (int64_t)t * T.lm_rows);
        k.wbytes = (uint32_t)((uint64_t)round16(k.nrows) * h * 2);
        k.wofs = Ly.lm + (uint64_t)k.row0 * h * 2;
        add(k);
    }
    finish_graph(g, sched, policy);
    return 0;
}

}  // namespace mk
