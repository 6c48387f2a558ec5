"""ORACLE — test infrastructure only.

A CPU "fake device" that executes a task graph record by record: every task of
the graph (the oracle builder's, or the library planner's export) computes just
its own tile, reads the step's shared buffers as they are at the moment it
runs, and counts its event; a seeded scheduler runs the workgroups' queues (or
the dynamic order) in a random interleaving, a task starting only once its
event has reached its target.  The result of the whole step is then compared
with the plain definition of the step (oracle.decode_step) by the tests.

This is the runtime loop of the pages taken literally on the CPU: fetch a task,
wait for its event, execute it, trigger the event it completes (MPK news page,
part 2; Hazy Research megakernel news page, section 4, counters that tasks
increment and wait on).  It checks what the structural checker in taskgraph.py
cannot: that the tiles, as the records describe them (head slot and RoPE-pair
block of a QKV tile, chunk of an attention task, KV-group K slice and row block
of an O-projection tile, rows of a gate/up tile, K block and row block of a
down tile, experts of a router tile, ...), compose into the decode step, and
that a task never needs a value its event does not guarantee.  Buffers a task
writes start as NaN each step, so a premature read shows up as a NaN or wrong
result rather than as a plausible stale one.

Arithmetic in double precision, in numpy, from the tile semantics (not from the
GPU code): per task a few dot products, RMSNorm, RoPE at the sequence's
position, a softmax chunk (max, sum, weighted values) and the max-rescaled
merge of chunks, SiLU, top-k routing with ties to the lower expert id and
softmax over the selected logits (taken on float-rounded logits, as the oracle
does).
"""
import numpy as np

from . import taskgraph as tg

NONE = tg.NONE


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_bits(x):
    """double -> float (nearest even) -> bf16 (nearest even), as the cache write."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


class FakeDevice:
    """One decode step of `cfg` for B sequences, executed task by task."""

    def __init__(self, cfg, w, B, C, attn_splits):
        self.cfg, self.B, self.C, self.S = cfg, B, C, attn_splits
        self.W = {k: _f64(v) for k, v in w.items()}
        self.grp = cfg.n_q // cfg.n_kv

    # ---- tile semantics --------------------------------------------------------------

    def _seqs(self, k):
        """The sequences of a GEMV tile's column group (16 per group)."""
        return range(16 * k["seq"], min(16 * k["seq"] + 16, self.B))

    def _x_in(self, l, b):
        """Residual stream entering layer l (l == L: the final one)."""
        return self.W["tok_embed"][self.tok[b]] if l == 0 else self.acc[2 * l - 1][b]

    def _norm(self, x, gain):
        return x / np.sqrt(np.mean(x * x) + self.cfg.eps) * gain

    def _several(self):
        return self.B > 1 or self.cfg.n_experts > 0

    def _deal(self):
        """Several sequences: the B S attention slots of a KV group dealt to the sequences in proportion to
        their contexts.  L = the smallest whole number of pages (pb positions each) with at most 16 chunks
        per sequence and sum_b ceil(n_b / L) <= B S; sequence b takes ceil(n_b / L) consecutive slots (in
        sequence order) of chunks of ceil(n_b / s_b) positions rounded up to whole pages.
        Returns {slot: (b, c)} for the non-empty chunks, and per sequence (chunk length, chunks)."""
        B, T, pb = self.B, self.B * self.S, 4096 // self.cfg.head_dim
        n = [int(p) + 1 for p in self.pos]
        m = max(1, -(-max(n) // (16 * pb)))
        while sum(-(-x // (m * pb)) for x in n) > T:
            m += 1
        slots, per, j = {}, [], 0
        for b in range(B):
            s = -(-n[b] // (m * pb))
            ln = -(-(-(-n[b] // s)) // pb) * pb
            nch = -(-n[b] // ln)
            per.append((ln, nch))
            for c in range(nch):
                slots[j + c] = (b, c)
            j += s
        assert j <= T
        return slots, per

    def _qkv(self, k):
        cfg, l, slot, d = self.cfg, k["layer"], k["part"], self.cfg.head_dim
        half, nq, nkv = d // 2, cfg.n_q, cfg.n_kv
        if slot < nq:
            W, off = self.W[f"l{l}.wq"], slot * d
        elif slot < nq + nkv:
            W, off = self.W[f"l{l}.wk"], (slot - nq) * d
        else:
            W, off = self.W[f"l{l}.wv"], (slot - nq - nkv) * d
        for b in self._seqs(k):
            xn = self._norm(self._x_in(l, b), self.W[f"l{l}.attn_norm"])
            P = self.pos[b]
            for i in range(k["nrows"]):
                j = k["row0"] + i
                lo, hi = W[off + j] @ xn, W[off + j + half] @ xn
                if slot < nq + nkv:  # RoPE pair (j, j + d/2) at the sequence's position
                    a = P * cfg.rope_theta ** (-2.0 * j / d)
                    lo, hi = lo * np.cos(a) - hi * np.sin(a), lo * np.sin(a) + hi * np.cos(a)
                if slot < nq:
                    self.q[b][slot * d + j], self.q[b][slot * d + j + half] = lo, hi
                else:
                    cache = self.kc if slot < nq + nkv else self.vc
                    g = (slot - nq) % nkv
                    cache[l, b, g, P, j], cache[l, b, g, P, j + half] = _bf16_bits(lo), _bf16_bits(hi)

    def _attn(self, k):
        d, l, g = self.cfg.head_dim, k["layer"], k["part"]
        if self._several():  # the slot the step's deal gave this record; an empty slot does nothing
            slot = k["seq"] * self.S + k["row0"]
            if slot not in self.slots:
                return
            b, c = self.slots[slot]
            ln = self.per[b][0]
        else:  # one sequence: chunk row0 of S equal parts of its context
            b, c = k["seq"], k["row0"]
            ln = -(-(self.pos[b] + 1) // self.S)
        P = self.pos[b]
        c0 = min(P + 1, c * ln)
        c1 = min(P + 1, c0 + ln)
        K = _f64(self.kc[l, b, g, c0:c1])
        V = _f64(self.vc[l, b, g, c0:c1])
        parts = []
        for hh in range(self.grp):
            i = g * self.grp + hh
            if c1 <= c0:
                parts.append((-np.inf, 0.0, np.zeros(d)))
                continue
            s = K @ self.q[b][i * d:(i + 1) * d] / np.sqrt(d)
            m = s.max()
            e = np.exp(s - m)
            parts.append((m, e.sum(), e @ V))
        self.part[(l, b, g, c)] = parts

    def _merged(self, l, b, g):
        """Attention output of the group's query heads: the chunks' partials merged with max rescaling."""
        d = self.cfg.head_dim
        out = np.empty(self.grp * d)
        nch = self.per[b][1] if self._several() else self.S
        for hh in range(self.grp):
            ps = [self.part[(l, b, g, c)][hh] for c in range(nch)]  # KeyError: a chunk not yet run
            M = max(p[0] for p in ps)
            num, den = np.zeros(d), 0.0
            for m, s, o in ps:
                if m != -np.inf:  # an empty chunk adds nothing; a NaN (a read before a write) spreads
                    num, den = num + np.exp(m - M) * o, den + np.exp(m - M) * s
            out[hh * d:(hh + 1) * d] = num / den if den != 0.0 else np.nan
        return out

    def _oproj(self, k):
        l, g, r0, n = k["layer"], k["part"], k["row0"], k["nrows"]
        kg = self.grp * self.cfg.head_dim
        Wo = self.W[f"l{l}.wo"][r0:r0 + n, g * kg:(g + 1) * kg]
        for b in self._seqs(k):
            add = Wo @ self._merged(l, b, g)
            if k["flags"] & tg.TF_RESID:
                add = add + self._x_in(l, b)[r0:r0 + n]
            self.acc[2 * l][b][r0:r0 + n] += add

    def _gateup(self, k):
        l, r0, n = k["layer"], k["row0"], k["nrows"]
        for b in self._seqs(k):
            xn = self._norm(self.acc[2 * l][b], self.W[f"l{l}.ffn_norm"])
            gt = self.W[f"l{l}.w_gate"][r0:r0 + n] @ xn
            up = self.W[f"l{l}.w_up"][r0:r0 + n] @ xn
            self.m[b][r0:r0 + n] = gt / (1.0 + np.exp(-gt)) * up

    def _down(self, k, kd):
        l, kb, r0, n = k["layer"], k["part"], k["row0"], k["nrows"]
        Wd = self.W[f"l{l}.w_down"][r0:r0 + n, kb * kd:(kb + 1) * kd]
        for b in self._seqs(k):
            add = Wd @ self.m[b][kb * kd:(kb + 1) * kd]
            if k["flags"] & tg.TF_RESID:
                add = add + self.acc[2 * l][b][r0:r0 + n]
            self.acc[2 * l + 1][b][r0:r0 + n] += add

    def _route(self, k):
        l, r0, n = k["layer"], k["row0"], k["nrows"]
        for b in self._seqs(k):
            xn = self._norm(self.acc[2 * l][b], self.W[f"l{l}.ffn_norm"])
            self.rlogit[b][r0:r0 + n] = self.W[f"l{l}.router"][r0:r0 + n] @ xn

    def _egu(self, k):
        l, e, r0, n = k["layer"], k["part"], k["row0"], k["nrows"]
        for b in self._seqs(k):
            xn = self._norm(self.acc[2 * l][b], self.W[f"l{l}.ffn_norm"])
            gt = self.W[f"l{l}.exp_gate"][e, r0:r0 + n] @ xn
            up = self.W[f"l{l}.exp_up"][e, r0:r0 + n] @ xn
            self.me[b][e][r0:r0 + n] = gt / (1.0 + np.exp(-gt)) * up

    def _edown(self, k):
        cfg, l, e, r0, n = self.cfg, k["layer"], k["part"], k["row0"], k["nrows"]
        for b in self._seqs(k):
            lg = self.rlogit[b].astype(np.float32).astype(np.float64)  # the choice is taken on float logits
            assert np.isfinite(lg).all(), "routing before every router tile ran"
            order = sorted(range(cfg.n_experts), key=lambda j: (-lg[j], j))[:cfg.top_k]
            if e not in order:
                continue
            sel = np.array([self.rlogit[b][j] for j in order])  # weights: softmax of the selected logits
            wgt = np.exp(sel - sel.max())
            wgt /= wgt.sum()
            if k["row0"] == 0:
                self.experts[l, b, order.index(e)] = e
            add = wgt[order.index(e)] * (self.W[f"l{l}.exp_down"][e, r0:r0 + n] @ self.me[b][e])
            if order[0] == e:  # each sequence's residual rides on its first-choice expert
                add = add + self.acc[2 * l][b][r0:r0 + n]
            self.acc[2 * l + 1][b][r0:r0 + n] += add

    def _lmhead(self, k):
        L, r0, n = self.cfg.n_layers, k["row0"], k["nrows"]
        Wlm = self.W["tok_embed" if self.cfg.tied else "lm_head"]
        for b in self._seqs(k):
            xn = self._norm(self._x_in(L, b), self.W["final_norm"])
            self.logits[b][r0:r0 + n] = Wlm[r0:r0 + n] @ xn

    # ---- the step -------------------------------------------------------------------

    def run(self, g, tokens, positions, k_cache, v_cache, seed=0, dynamic=False, event=False, slow=None):
        """Executes graph g (taskgraph dict form) once; returns (hidden, logits, next, experts, tasks run)
        and leaves the K/V writes in k_cache / v_cache.

        Static queues by default; dynamic: workgroups claim the next task of the global order one at a
        time; event: they claim the next slot of a ready queue that starts with the tasks waiting on no
        event and grows by an event's dependents when its count completes.  slow: a workgroup that only
        moves when no other can (an adversarial interleaving)."""
        cfg, B = self.cfg, self.B
        L, h, f = cfg.n_layers, cfg.hidden, cfg.ffn
        self.tok, self.pos = np.asarray(tokens), np.asarray(positions)
        self.kc, self.vc = k_cache, v_cache
        if self._several():
            self.slots, self.per = self._deal()
        nan = np.nan
        self.acc = np.zeros((2 * L + 1, B, h))
        self.q = np.full((B, cfg.n_q * cfg.head_dim), nan)
        self.part = {}
        self.m = np.full((B, max(f, 1)), nan)
        E = cfg.n_experts
        self.rlogit = np.full((B, max(E, 1)), nan)
        self.me = np.full((B, max(E, 1), max(cfg.expert_ffn, 1)), nan)
        self.experts = np.full((L, B, max(cfg.top_k, 1)), -1, np.int32)
        self.logits = np.full((B, cfg.vocab), nan)
        kd = g["tiling"].get("kd", 0)
        ops = {tg.OP_QKV: self._qkv, tg.OP_ATTN: self._attn, tg.OP_OPROJ: self._oproj, tg.OP_GATEUP: self._gateup,
               tg.OP_DOWN: lambda k: self._down(k, kd), tg.OP_LMHEAD: self._lmhead, tg.OP_ROUTE: self._route,
               tg.OP_EGU: self._egu, tg.OP_EDOWN: self._edown}
        tasks = g["tasks"]
        ctr = [0] * len(g["target"])
        rng = np.random.default_rng(seed)
        W = len(g["queues"])
        if event:  # the ready queue: filled slots, in the order their events completed
            dynamic = True
            cons = [[] for _ in g["target"]]
            for k in tasks:
                if k["wait_ev"] != NONE:
                    cons[k["wait_ev"]].append(k["id"])
            order = [k["id"] for k in tasks if k["wait_ev"] == NONE]
        elif dynamic:  # one global order
            order = list(g["order"])
        if dynamic:  # claimed one task (slot) at a time by whichever workgroup is free
            held = [None] * W
            nxt = 0
        else:
            queues = [list(q) for q in g["queues"]]
            at = [0] * W
        ran = 0
        while True:
            moves = []
            for wg in range(W):
                if dynamic:
                    if held[wg] is None:
                        if nxt < len(tasks):
                            moves.append((wg, "claim"))
                        continue
                    if held[wg] >= len(order):  # a ready-queue slot not filled yet
                        continue
                    i = order[held[wg]]
                else:
                    if at[wg] >= len(queues[wg]):
                        continue
                    i = queues[wg][at[wg]]
                k = tasks[i]
                if k["wait_ev"] == NONE or ctr[k["wait_ev"]] >= g["target"][k["wait_ev"]]:
                    moves.append((wg, "run"))
            if not moves:
                break
            if slow is not None and any(m[0] != slow for m in moves):
                moves = [m for m in moves if m[0] != slow]
            wg, what = moves[rng.integers(len(moves))]
            if what == "claim":
                held[wg] = nxt
                nxt += 1
                continue
            if dynamic:
                i, held[wg] = order[held[wg]], None
            else:
                i = queues[wg][at[wg]]
                at[wg] += 1
            k = tasks[i]
            ops[k["op"]](k)
            for ev in tg.signals(k, E):
                ctr[ev] += 1
                if event and ctr[ev] == g["target"][ev]:
                    order.extend(cons[ev])
            ran += 1
        hidden = np.stack([self._x_in(L, b) for b in range(B)])
        nxt_tok = np.array([int(np.argmax(self.logits[b].astype(np.float32))) for b in range(B)], np.int32)
        return hidden, self.logits.copy(), nxt_tok, (self.experts if E else None), ran
