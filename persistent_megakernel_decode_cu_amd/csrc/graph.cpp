// Host task-graph builder and queue scheduler (pure C++, no GPU calls).
//
// The graph follows the SM-level task graph of the pages (koas-w.github.io
// megakernel notes, "SM-level task graph": nodes are tasks that run on one
// SM/CU, edges are tile-level dependencies; MPK news page, part 1: tasks and
// events, a trigger edge from each task to the event it completes, a
// dependency edge from an event to the tasks it releases).  Events are integer
// counters: a task adds one to its event when done, and a task waits until the
// counter of its event reaches the number of producers (Hazy Research
// megakernel news page, section 4, "synchronisation").
//
// Static scheduling gives every workgroup a private queue fixed before launch;
// dynamic scheduling lets workgroups claim tasks from one global queue
// (koas-w.github.io notes, "static and dynamic scheduling").  Both queue kinds
// are subsequences of one topological order, so the task that is lowest in
// that order among the unfinished ones can always run: no deadlock.
//
// Event-driven dispatch follows the MPK runtime (MPK news page, part 2: a task
// completes by counting its event; the event is activated when the count reaches
// its threshold, and the scheduling unit then launches every task that depends on
// it).  Here (sched 2) the task whose count activates an event appends the event's
// dependents to one global ready queue, or (sched 3) posts the event to the
// activated-event queue of one workgroup, whose scheduler wave appends them; either
// way workgroups take tasks from that queue in the order they became ready.  The
// builder lists each event's dependents and the tasks that depend on nothing; every
// event has one counter (the count that activates it has to be seen by one producer).
#include "graph.h"

#include <algorithm>
#include <array>
#include <cstring>
#include <numeric>

namespace mk {

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
static int64_t pow2_floor(int64_t x) {
    int64_t p = 1;
    while (p * 2 <= x) p *= 2;
    return p;
}
static int64_t pow2_ceil(int64_t x) {
    int64_t p = 1;
    while (p < x) p *= 2;
    return p;
}
static uint64_t pad256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// A GEMV tile whose rows have KT bf16 columns is consumed from 16 KiB LDS
// pages.  128 <= KT <= 2048: pages hold 16 x 32 blocks of matrix-core operands,
// and every compute wave owns a quarter of the 32-column blocks; KT = 4096: two
// whole rows per page.
static bool gemv_k_ok(int64_t kt) { return is_pow2(kt) && kt >= 128 && kt <= 4096; }
static int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }

int plan_tiling(const Dims& dm, int B, int C, int W, const PlanOptions& o, Tiling* t, std::string* err) {
    auto fail = [&](const char* m) {
        if (err) *err = m;
        return -1;
    };
    if (dm.L < 0 || dm.h <= 0 || dm.nq <= 0 || dm.nkv <= 0 || dm.d <= 0 || dm.V <= 0) return fail("non-positive model dimension");
    if (B < 1 || C < 1 || W < 1) return fail("batch, max_ctx and workgroups must be >= 1");
    if (dm.d != 64 && dm.d != 128) return fail("head_dim must be 64 or 128");
    if (dm.nq % dm.nkv) return fail("n_q_heads must be a multiple of n_kv_heads");
    const bool moe = dm.n_experts != 0;
    if (B > MAX_BATCH) return fail("batch is limited to 64 sequences per step");
    const bool batched = batched_path(B, dm.n_experts);
    if (batched && dm.h > 2048) return fail("batch > 1 and experts need hidden <= 2048");
    if (moe) {
        if (dm.n_experts < 1 || dm.n_experts > 64) return fail("1..64 experts");
        if (dm.top_k < 1 || dm.top_k > dm.n_experts) return fail("top_k must be in [1, n_experts]");
        if (!gemv_k_ok(dm.fe) || dm.fe > 2048) return fail("expert_ffn must be a power of two in [128, 2048]");
    } else if (dm.f <= 0) {
        return fail("ffn_dim must be positive");
    }
    if (!gemv_k_ok(dm.h) || dm.h > MAX_ACT) return fail("hidden must be a power of two in [128, 4096]");
    const int grp = dm.nq / dm.nkv;
    if (grp > 16) return fail("more than 16 query heads per KV head");
    if (!gemv_k_ok((int64_t)grp * dm.d) || (int64_t)grp * dm.d > 2048)
        return fail("query heads per KV head times head_dim must be a power of two in [128, 2048]");
    Tiling& T = *t;
    memset(&T, 0, sizeof(T));
    T.L = dm.L; T.h = dm.h; T.nq = dm.nq; T.nkv = dm.nkv; T.d = dm.d; T.f = dm.f; T.V = dm.V;
    T.B = B; T.C = C; T.W = W; T.grp = grp;
    T.qkv_pairs = 8;
    T.n_qkv_tiles = (dm.nq + 2 * dm.nkv) * (dm.d / 2) / T.qkv_pairs;
    int S = o.attn_splits;
    if (S > 16) return fail("attn_splits must be at most 16 (the merge reads up to 16 chunk partials)");
    if (S <= 0) {
        // one sequence: 256-position chunks of its context.  The several-sequence path
        // (slots dealt per step in proportion to the contexts): up to two sequences,
        // about one attention task per workgroup and layer, at most 8 slots; more
        // sequences, about two, at most 4 slots (each task carries a fixed cost of a few
        // microseconds; measured at 2..32 sequences of the 1B shape)
        const int64_t per_wg = batched && B > 2 ? 2 : 1, cap = batched && B > 2 ? 4 : 8;
        S = !batched ? (int)std::max<int64_t>(1, std::min<int64_t>(16, (C + 255) / 256))
                   : (int)std::max<int64_t>(1, std::min<int64_t>(cap, pow2_floor(std::max<int64_t>(
                                                                     1, per_wg * W / ((int64_t)B * dm.nkv)))));
    }
    if (S > C) S = C;
    T.attn_splits = S;
    T.n_attn_tiles = B * dm.nkv * S;
    // rows x sequences (of one column group) of a tile fit the LDS row-result buffer;
    // a power of two, so that every tile height derived from it divides its matrix
    const int64_t max_rows = pow2_floor(MAX_TILE_ROWS / std::min<int64_t>(B, GROUP_SEQS));
    // O-proj: tiles (KV group g, rows) with K = grp*d columns; about W tiles per layer
    T.o_rows = (int)std::min<int64_t>(std::min<int64_t>(dm.h, max_rows),
                                      std::max<int64_t>(16, pow2_floor((int64_t)dm.h * dm.nkv / W)));
    T.n_o_tiles = dm.nkv * (dm.h / T.o_rows);
    if (moe) {
        // about one expert gate/up tile and one expert down tile per workgroup and layer;
        // gate/up tiles hold whole 32-row blocks of m, down tiles whole 64-row chunks
        T.E = dm.n_experts;
        T.topk = dm.top_k;
        T.fe = dm.fe;
        T.r_gu = (int)std::min<int64_t>(dm.fe, std::max<int64_t>(32, pow2_floor((int64_t)dm.n_experts * dm.fe / W)));
        T.r_dn = (int)std::min<int64_t>(dm.h, std::max<int64_t>(64, pow2_floor((int64_t)dm.n_experts * dm.h / W)));
    } else {
    // down-proj K blocks of kd columns of m; gate/up tiles feed whole K blocks
    T.kd = (int)std::min<int64_t>(1024, dm.f);
    if (dm.f % T.kd || !gemv_k_ok(T.kd)) return fail("ffn_dim must be a multiple of 1024 (or a power of two in [128, 1024))");
    const int64_t n_kb = dm.f / T.kd;
    T.d_rows = (int)std::min<int64_t>(std::min<int64_t>(dm.h, max_rows),
                                      std::max<int64_t>(16, pow2_floor((int64_t)dm.h * n_kb / W)));
    T.n_down_tiles = (int)(n_kb * (dm.h / T.d_rows));
    T.g_rows = (int)std::max<int64_t>(8, pow2_ceil((dm.f + W - 1) / W));
    if (T.g_rows > T.kd) T.g_rows = T.kd;
    if (T.g_rows > max_rows / 2) T.g_rows = (int)(max_rows / 2);
    if (T.kd % T.g_rows) return fail("gate/up tile does not divide the down-proj K block");
    T.n_gu_tiles = dm.f / T.g_rows;
    }
    // LM head: about one tile per workgroup (with several sequences the device takes a
    // tile in chunks of whole row groups within the row-result bound)
    T.lm_rows = (int)std::min<int64_t>(MAX_TILE_ROWS, round16((dm.V + W - 1) / W));
    T.n_lm_tiles = (dm.V + T.lm_rows - 1) / T.lm_rows;
    return 0;
}

void plan_layout(const Tiling& T, bool tied, Layout* out) {
    Layout& Ly = *out;
    memset(&Ly, 0, sizeof(Ly));
    const uint64_t h = T.h;
    uint64_t at = 0;
    Ly.gains = at;
    at = pad256(at + (uint64_t)(2 * T.L + 1) * h * 2);
    Ly.embed = at;
    at = pad256(at + (uint64_t)T.V * h * 2);
    // the LM head has its own copy even when tied to the embedding: its tiles
    // are stored in GEMV page order, the embedding row by row for the gather
    (void)tied;
    Ly.lm = at;
    at = pad256(at + (uint64_t)T.n_lm_tiles * T.lm_rows * h * 2);
    Ly.layer0 = at;
    uint64_t l = 0;
    Ly.qkv = l;
    l = pad256(l + (uint64_t)(T.nq + 2 * T.nkv) * T.d * h * 2);
    Ly.o = l;
    l = pad256(l + h * (uint64_t)T.nq * T.d * 2);
    if (T.E == 0) {
        Ly.gu = l;
        l = pad256(l + 2ull * T.f * h * 2);
        Ly.down = l;
        l = pad256(l + h * (uint64_t)T.f * 2);
    } else {
        Ly.router = l;  // E rows padded to 16
        l = pad256(l + (uint64_t)round16(T.E) * h * 2);
        Ly.egu = l;
        l = pad256(l + 2ull * T.E * T.fe * h * 2);
        Ly.edown = l;
        l = pad256(l + (uint64_t)T.E * h * T.fe * 2);
    }
    Ly.layer_bytes = l;
    Ly.total = Ly.layer0 + (uint64_t)T.L * l;
}

uint32_t Graph::new_event() {
    target.push_back(0);
    nsub.push_back(1);
    return (uint32_t)target.size() - 1;
}

static uint64_t task_cost(const Task& k) { return (uint64_t)k.wbytes + 8192; }

// Sub-counters, event dependents and the queues of a graph whose tasks and targets are built.
void finish_graph(Graph& g, int sched, int policy) {
    // counter words: events with more than 4 producers spread their increments over the device's
    // CTR_SUBS words (nsub 8); measured on the 1B shape at batch 1 against more than 32 / 16: 799 / 786
    // -> 780 us per step (event-driven dispatch: one counter per event, which tells its last producer)
    for (size_t e = 0; e < g.target.size(); ++e) g.nsub[e] = sched < 2 && g.target[e] > 4 ? 8 : 1;
    // dependents of every event, and the tasks that wait on none
    g.cons_off.assign(g.target.size() + 1, 0);
    g.cons.clear();
    g.init.clear();
    for (const auto& k : g.tasks)
        if (k.wait_ev != NONE) ++g.cons_off[k.wait_ev + 1];
        else g.init.push_back(k.id);
    for (size_t e = 0; e < g.target.size(); ++e) g.cons_off[e + 1] += g.cons_off[e];
    g.cons.resize(g.cons_off.back());
    {
        std::vector<uint32_t> fill(g.cons_off.begin(), g.cons_off.end() - 1);
        for (const auto& k : g.tasks)
            if (k.wait_ev != NONE) g.cons[fill[k.wait_ev]++] = k.id;
    }
    for (auto& k : g.tasks) {
        if (k.wait_ev != NONE) {
            k.wait_target = g.target[k.wait_ev];
            k.wait_nsub = (uint8_t)g.nsub[k.wait_ev];
        }
        if (k.sig_ev != NONE) k.sig_nsub = (uint8_t)g.nsub[k.sig_ev];
    }
    // queues
    const int W = g.T.W;
    const size_t n = g.tasks.size();
    g.order.resize(n);
    std::iota(g.order.begin(), g.order.end(), 0u);
    std::vector<std::vector<uint32_t>> per(W);
    if (policy == 0) {
        for (size_t i = 0; i < n; ++i) per[i % W].push_back((uint32_t)i);
    } else {
        std::vector<uint64_t> load(W, 0);
        for (size_t i = 0; i < n; ++i) {
            int best = 0;
            for (int w = 1; w < W; ++w)
                if (load[w] < load[best]) best = w;
            load[best] += task_cost(g.tasks[i]);
            per[best].push_back((uint32_t)i);
        }
    }
    g.queue_off.assign(W + 1, 0);
    g.queue.clear();
    for (int w = 0; w < W; ++w) {
        g.queue_off[w] = (uint32_t)g.queue.size();
        g.queue.insert(g.queue.end(), per[w].begin(), per[w].end());
    }
    g.queue_off[W] = (uint32_t)g.queue.size();
}

int build_graph(const Tiling& T, const Layout& Ly, int sched, int policy, Graph* G) {
    Graph& g = *G;
    g.T = T;
    g.lay = Ly;
    g.sched = (uint32_t)sched;
    g.tasks.clear();
    g.target.clear();
    g.nsub.clear();
    const uint64_t h = T.h;
    const int L = T.L, grp = T.grp, half = T.d / 2;
    const int pair_blocks = half / T.qkv_pairs;
    const int n_kb = T.E ? 0 : T.f / T.kd;
    const int n_sg = (T.B + GROUP_SEQS - 1) / GROUP_SEQS;  // column groups of the batched GEMV tiles

    auto add = [&](Task k) {
        k.id = (uint32_t)g.tasks.size();
        g.tasks.push_back(k);
        if (k.sig_ev != NONE) {
            const int n_sig = (k.flags & TF_SIGRANGE) ? T.E : 1;
            for (int i = 0; i < n_sig; ++i) g.target[k.sig_ev + i] += 1;
        }
    };
    auto blank = [](uint8_t op, int layer) {
        Task k;
        memset(&k, 0, sizeof(k));
        k.op = op;
        k.layer = (uint16_t)layer;
        k.wait_ev = NONE;
        k.sig_ev = NONE;
        k.wait_nsub = 1;
        k.sig_nsub = 1;
        return k;
    };

    uint32_t ev_x = NONE;  // residual stream ready for the current layer (NONE for layer 0: embedding)
    for (int l = 0; l < L; ++l) {
        const uint64_t lbase = Ly.layer0 + (uint64_t)l * Ly.layer_bytes;
        std::vector<uint32_t> ev_qkv(T.nkv), ev_attn(T.nkv), ev_m(n_kb);
        for (int gi = 0; gi < T.nkv; ++gi) ev_qkv[gi] = g.new_event();
        for (int gi = 0; gi < T.nkv; ++gi) ev_attn[gi] = g.new_event();
        const uint32_t ev_xb = g.new_event();
        for (int kb = 0; kb < n_kb; ++kb) ev_m[kb] = g.new_event();
        // mixture of experts: one event per expert, raised by its gate/up tiles and by every
        // router tile (the expert's down tiles need both the expert's m and all router logits)
        std::vector<uint32_t> ev_me(T.E);
        for (int e = 0; e < T.E; ++e) ev_me[e] = g.new_event();
        const uint32_t ev_next = g.new_event();

        // fused RMSNorm + QKV + RoPE tiles, grouped by KV head: q heads of the group, then its k and v head
        // (more than 16 sequences: every GEMV tile once per column group of 16, on the same weights)
        for (int sg = 0; sg < n_sg; ++sg) {
            uint64_t tile = 0;
            for (int gi = 0; gi < T.nkv; ++gi) {
                for (int s = 0; s < grp + 2; ++s) {
                    int slot = s < grp ? gi * grp + s : (s == grp ? T.nq + gi : T.nq + T.nkv + gi);
                    for (int pb = 0; pb < pair_blocks; ++pb, ++tile) {
                        Task k = blank(OP_QKV, l);
                        k.part = (uint16_t)slot;
                        k.row0 = (uint32_t)(pb * T.qkv_pairs);
                        k.nrows = (uint32_t)T.qkv_pairs;
                        k.seq = (uint32_t)sg;
                        k.wait_ev = ev_x;
                        k.sig_ev = ev_qkv[gi];
                        k.wbytes = (uint32_t)(2 * T.qkv_pairs * h * 2);
                        k.wofs = lbase + Ly.qkv + tile * k.wbytes;
                        add(k);
                    }
                }
            }
        }
        // attention tasks per (sequence, KV group, chunk).  One sequence: chunks in order
        // per group.  Several sequences (or experts): the B x S tasks of a group are slots
        // j = seq * S + chunk that the device deals to the sequences at every step, in
        // proportion to their contexts; the last chunk of a (sequence, group) to finish
        // merges the chunks.  The records go in slot-chunk order 0, 1, .., S/2 - 1, then
        // S - 1, .., S/2, so that round-robin queues give a workgroup slots c and S - 1 - c.
        std::vector<int> corder;
        for (int c = 0; c < (T.attn_splits + 1) / 2; ++c) corder.push_back(c);
        for (int c = T.attn_splits - 1; c >= (T.attn_splits + 1) / 2; --c) corder.push_back(c);
        std::vector<std::array<int, 3>> attn;  // (sequence, group, chunk)
        if (batched_path(T.B, T.E)) {
            for (int c : corder)
                for (int b = 0; b < T.B; ++b)
                    for (int gi = 0; gi < T.nkv; ++gi) attn.push_back({b, gi, c});
        } else {
            for (int gi = 0; gi < T.nkv; ++gi)
                for (int c = 0; c < T.attn_splits; ++c) attn.push_back({0, gi, c});
        }
        for (const auto& a : attn) {
            const int b = a[0], gi = a[1], c = a[2];
            Task k = blank(OP_ATTN, l);
            k.part = (uint16_t)gi;
            k.row0 = (uint32_t)c;
            k.nrows = (uint32_t)grp;
            k.seq = (uint32_t)b;
            k.wait_ev = ev_qkv[gi];
            k.sig_ev = ev_attn[gi];
            add(k);
        }
        // O-proj K slices: tile (group, row block)
        const int o_kt = grp * T.d;
        for (int sg = 0; sg < n_sg; ++sg)
        for (int gi = 0; gi < T.nkv; ++gi)
            for (int rb = 0; rb < T.h / T.o_rows; ++rb) {
                Task k = blank(OP_OPROJ, l);
                k.part = (uint16_t)gi;
                k.row0 = (uint32_t)(rb * T.o_rows);
                k.nrows = (uint32_t)T.o_rows;
                k.seq = (uint32_t)sg;
                k.flags = gi == 0 ? TF_RESID : 0;
                k.wait_ev = ev_attn[gi];
                k.sig_ev = ev_xb;
                k.wbytes = (uint32_t)((uint64_t)T.o_rows * o_kt * 2);
                k.wofs = lbase + Ly.o + ((uint64_t)gi * (T.h / T.o_rows) + rb) * k.wbytes;
                add(k);
            }
        if (T.E) {
            // router: tiles of 16 experts' logits per column group, each raising every expert's
            // event; then every expert's gate/up tiles (m rows row0 .. row0 + r_gu), which need
            // only the normalised residual, and its down tiles (h rows), which apply the routing
            for (int sg = 0; sg < n_sg; ++sg)
                for (int r0 = 0; r0 < T.E; r0 += 16) {
                    Task k = blank(OP_ROUTE, l);
                    k.row0 = (uint32_t)r0;
                    k.nrows = (uint32_t)std::min(16, T.E - r0);
                    k.seq = (uint32_t)sg;
                    k.flags = TF_SIGRANGE;
                    k.wait_ev = ev_xb;
                    k.sig_ev = ev_me[0];
                    k.wbytes = (uint32_t)(16 * h * 2);
                    k.wofs = lbase + Ly.router + (uint64_t)r0 * h * 2;
                    add(k);
                }
            const int gu_per_e = T.fe / T.r_gu, dn_per_e = T.h / T.r_dn;
            for (int sg = 0; sg < n_sg; ++sg)
                for (int e = 0; e < T.E; ++e)
                    for (int t = 0; t < gu_per_e; ++t) {
                        Task k = blank(OP_EGU, l);
                        k.part = (uint16_t)e;
                        k.row0 = (uint32_t)(t * T.r_gu);
                        k.nrows = (uint32_t)T.r_gu;
                        k.seq = (uint32_t)sg;
                        k.wait_ev = ev_xb;
                        k.sig_ev = ev_me[e];
                        k.wbytes = (uint32_t)(2ull * T.r_gu * h * 2);
                        k.wofs = lbase + Ly.egu + ((uint64_t)e * gu_per_e + t) * k.wbytes;
                        add(k);
                    }
            for (int sg = 0; sg < n_sg; ++sg)
                for (int e = 0; e < T.E; ++e)
                    for (int rb = 0; rb < dn_per_e; ++rb) {
                        Task k = blank(OP_EDOWN, l);
                        k.part = (uint16_t)e;
                        k.row0 = (uint32_t)(rb * T.r_dn);
                        k.nrows = (uint32_t)T.r_dn;
                        k.seq = (uint32_t)sg;
                        k.wait_ev = ev_me[e];
                        k.sig_ev = ev_next;
                        k.wbytes = (uint32_t)((uint64_t)T.r_dn * T.fe * 2);
                        k.wofs = lbase + Ly.edown + ((uint64_t)e * dn_per_e + rb) * k.wbytes;
                        add(k);
                    }
            ev_x = ev_next;
            continue;
        }
        // RMSNorm + gate/up + SiLU tiles
        for (int sg = 0; sg < n_sg; ++sg)
        for (int t = 0; t < T.n_gu_tiles; ++t) {
            Task k = blank(OP_GATEUP, l);
            k.row0 = (uint32_t)(t * T.g_rows);
            k.nrows = (uint32_t)T.g_rows;
            k.seq = (uint32_t)sg;
            k.wait_ev = ev_xb;
            k.sig_ev = ev_m[(t * T.g_rows) / T.kd];
            k.wbytes = (uint32_t)(2ull * T.g_rows * h * 2);
            k.wofs = lbase + Ly.gu + (uint64_t)t * k.wbytes;
            add(k);
        }
        // down-proj K slices: tile (K block, row block)
        for (int sg = 0; sg < n_sg; ++sg)
        for (int kb = 0; kb < n_kb; ++kb)
            for (int rb = 0; rb < T.h / T.d_rows; ++rb) {
                Task k = blank(OP_DOWN, l);
                k.part = (uint16_t)kb;
                k.row0 = (uint32_t)(rb * T.d_rows);
                k.nrows = (uint32_t)T.d_rows;
                k.seq = (uint32_t)sg;
                k.flags = kb == 0 ? TF_RESID : 0;
                k.wait_ev = ev_m[kb];
                k.sig_ev = ev_next;
                k.wbytes = (uint32_t)((uint64_t)T.d_rows * T.kd * 2);
                k.wofs = lbase + Ly.down + ((uint64_t)kb * (T.h / T.d_rows) + rb) * k.wbytes;
                add(k);
            }
        ev_x = ev_next;
    }
    // final RMSNorm + LM head + argmax
    for (int sg = 0; sg < n_sg; ++sg)
    for (int t = 0; t < T.n_lm_tiles; ++t) {
        Task k = blank(OP_LMHEAD, L);
        k.seq = (uint32_t)sg;
        k.row0 = (uint32_t)(t * T.lm_rows);
        k.nrows = (uint32_t)std::min<int64_t>(T.lm_rows, (int64_t)T.V - (int64_t)t * T.lm_rows);
        k.wait_ev = ev_x;
        k.wbytes = (uint32_t)((uint64_t)round16(k.nrows) * h * 2);
        k.wofs = Ly.lm + (uint64_t)k.row0 * h * 2;
        add(k);
    }
    finish_graph(g, sched, policy);
    return 0;
}


size_t export_size(const Graph& g) {
    return sizeof(ExportHeader) + g.tasks.size() * sizeof(Task) + g.target.size() * 8 + g.queue_off.size() * 4 +
           g.queue.size() * 4 + g.order.size() * 4;
}

size_t export_graph(const Graph& g, void* buf, size_t cap) {
    size_t need = export_size(g);
    if (!buf || cap < need) return need;
    ExportHeader hd;
    memset(&hd, 0, sizeof(hd));
    hd.magic = EXPORT_MAGIC;
    hd.version = 1;
    hd.n_tasks = (uint32_t)g.tasks.size();
    hd.n_events = (uint32_t)g.target.size();
    hd.W = (uint32_t)g.T.W;
    hd.sched = g.sched;
    const Tiling& T = g.T;
    hd.L = T.L; hd.h = T.h; hd.nq = T.nq; hd.nkv = T.nkv; hd.d = T.d; hd.f = T.f; hd.V = T.V; hd.B = T.B; hd.C = T.C;
    hd.grp = T.grp; hd.qkv_pairs = T.qkv_pairs; hd.attn_splits = T.attn_splits; hd.o_rows = T.o_rows;
    hd.g_rows = T.g_rows; hd.kd = T.kd; hd.d_rows = T.d_rows; hd.lm_rows = T.lm_rows;
    hd.E = T.E; hd.topk = T.topk; hd.fe = T.fe; hd.r_gu = T.r_gu; hd.r_dn = T.r_dn;
    hd.record_bytes = sizeof(Task);
    uint8_t* p = (uint8_t*)buf;
    memcpy(p, &hd, sizeof(hd));
    p += sizeof(hd);
    auto put = [&](const void* src, size_t bytes) {
        if (bytes) memcpy(p, src, bytes);
        p += bytes;
    };
    put(g.tasks.data(), g.tasks.size() * sizeof(Task));
    put(g.target.data(), g.target.size() * 4);
    put(g.nsub.data(), g.nsub.size() * 4);
    put(g.queue_off.data(), g.queue_off.size() * 4);
    put(g.queue.data(), g.queue.size() * 4);
    put(g.order.data(), g.order.size() * 4);
    return need;
}

}  // namespace mk
