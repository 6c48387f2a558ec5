"""ORACLE — test infrastructure only.

The CPU fake device of the prompt (prefill) graph: every task record of a prompt launch
(the library planner's export, mk_plan_prefill) computes just its own tile, in double
precision, from the record's fields, reading the launch's shared buffers as they stand
when it runs, and counts its event; a seeded scheduler interleaves the workgroups' static
queues (or the dynamic order, or holds one workgroup back), a task starting only once its
event has reached its target.  The tests compare the outcome with the oracle's causal
prefill (oracle/prefill.py).  This checks what the GPU parity tests cannot isolate: that the
tiles as the records describe them (rows of a stacked Q/K/V tile and the heads in it, the
token block a GEMM tile covers and whether it holds one or two token groups per wave, the
K slice of an O- or down-projection tile and the partial it writes, the m rows of a gate/up
tile, the query group and KV group of an attention task, the tokens of an RMSNorm task and
which residual it completes) compose into the prompt's forward pass, and that no task
needs a value its event does not guarantee: every buffer a task writes starts as NaN.

Tile semantics, as the prompt graph defines them (the knowledge-base digest "megakernel
boundary selection" defines prefill as the pass over the whole prompt, once per request):
  RMSNorm (part = kind, seq = q, nrows = n tokens, 1 or 4): tokens nq .. nq+n-1; kind 0 of layer l: x = R_a + the down
    partials (layer 0: the embedding row) -> R_b, normalised -> X; kind 1: x = R_b + the
    O-projection partials -> R_a, normalised -> X; kind 2: x = R_a + the down partials -> R_b
    (the hidden output), the last token normalised with the final gains -> LM.
  QKV (row0, nrows, seq = token block): rows row0 .. of [Wq; Wk; Wv] for the block's tokens,
    each 64-row head rotated (pairs j, j + d/2 at the token's position); query rows -> Q,
    key and value rows -> the bf16 cache at the token's position.
  attention (part = g, seq = query group): the group's heads for tokens 16 qg .. 16 qg + 15,
    over cache slots 0 .. the token's position -> O.
  O-projection / down (row0, nrows, part = slice s, seq = token block): rows row0 .. over
    the K slice s of S -> partial s.
  gate/up (row0 = first m row, nrows = gate + up rows): m rows row0 .. row0 + nrows/2 -> M.
  LM head (row0, nrows): logits of the last token, running argmax (lowest index on ties,
    over float-rounded logits, as the oracle).
"""
import numpy as np

NONE = 0xFFFFFFFF
OP_PNORM, OP_PQKV, OP_PATTN, OP_POPROJ, OP_PGU, OP_PDOWN, OP_PLM = range(10, 17)
TF_NGW2 = 4


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_bits(x):
    """double -> float (nearest even) -> bf16 (nearest even), as the cache write."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


class PromptDevice:
    """One prompt launch of `cfg` for T tokens, executed task by task."""

    def __init__(self, cfg, w, T):
        self.cfg, self.T = cfg, T
        self.W = {k: _f64(v) for k, v in w.items()}
        self.grp = cfg.n_q // cfg.n_kv
        L = cfg.n_layers
        self.Wqkv = [np.concatenate([self.W[f"l{l}.wq"], self.W[f"l{l}.wk"], self.W[f"l{l}.wv"]]) for l in range(L)]

    # ---- tile semantics --------------------------------------------------------------

    def _norm(self, x, gain):
        return x / np.sqrt(np.mean(x * x) + self.cfg.eps) * gain

    def _block(self, k):
        """Tokens of a GEMM tile's block (64 per token group of each of the 4 compute waves)."""
        n = 128 if k["flags"] & TF_NGW2 else 64
        return range(n * k["seq"], min(n * k["seq"] + n, self.T))

    def _pnorm(self, k):
        cfg, l, kind, n = self.cfg, k["layer"], k["part"], k["nrows"]
        assert n in (1, 4), "an RMSNorm task covers one or four tokens"
        for t in range(n * k["seq"], min(n * k["seq"] + n, self.T)):
            if kind == 0:
                x = self.W["tok_embed"][self.tok[t]] if l == 0 else self.Ra[t] + self.Pd[:, t].sum(axis=0)
                self.Rb[t] = x
                self.X[t] = self._norm(x, self.W[f"l{l}.attn_norm"])
            elif kind == 1:
                x = self.Rb[t] + self.Po[:, t].sum(axis=0)
                self.Ra[t] = x
                self.X[t] = self._norm(x, self.W[f"l{l}.ffn_norm"])
            else:
                x = self.Ra[t] + self.Pd[:, t].sum(axis=0)
                self.Rb[t] = x
                if t == self.T - 1:
                    self.LM = self._norm(x, self.W["final_norm"])

    def _pqkv(self, k):
        cfg, l = self.cfg, k["layer"]
        d = cfg.head_dim
        half = d // 2
        nq, nkv = cfg.n_q, cfg.n_kv
        r0, nr = k["row0"], k["nrows"]
        assert r0 % d == 0 and nr % d == 0, "a QKV tile holds whole heads"
        for t in self._block(k):
            out = self.Wqkv[l][r0:r0 + nr] @ self.X[t]
            pos = self.pos0 + t
            for hb in range(nr // d):
                head = r0 // d + hb
                v = out[hb * d:(hb + 1) * d].copy()
                if head < nq + nkv:  # queries and keys turn; values do not
                    j = np.arange(half)
                    a = pos * np.power(float(cfg.rope_theta), -2.0 * j / d)
                    c, s = np.cos(a), np.sin(a)
                    v = np.concatenate([v[:half] * c - v[half:] * s, v[:half] * s + v[half:] * c])
                if head < nq:
                    self.Q[t, head * d:(head + 1) * d] = v
                elif head < nq + nkv:
                    self.kc[l, 0, head - nq, pos] = _bf16_bits(v)
                else:
                    self.vc[l, 0, head - nq - nkv, pos] = _bf16_bits(v)

    def _pattn(self, k):
        cfg, l, g = self.cfg, k["layer"], k["part"]
        d = cfg.head_dim
        for t in range(16 * k["seq"], min(16 * k["seq"] + 16, self.T)):
            n = self.pos0 + t + 1
            K, V = _f64(self.kc[l, 0, g, :n]), _f64(self.vc[l, 0, g, :n])
            for i in range(g * self.grp, (g + 1) * self.grp):
                s = K @ self.Q[t, i * d:(i + 1) * d] / np.sqrt(d)
                p = np.exp(s - s.max())
                self.O[t, i * d:(i + 1) * d] = (p / p.sum()) @ V

    def _slice(self, k, op):
        """The K slice of an O-projection or down tile: (first column, width)."""
        kfull = self.cfg.n_q * self.cfg.head_dim if op == OP_POPROJ else self.cfg.ffn
        S = self.So if op == OP_POPROJ else self.Sd
        return k["part"] * (kfull // S), kfull // S

    def _poproj(self, k):
        l, r0, nr = k["layer"], k["row0"], k["nrows"]
        c0, kw = self._slice(k, OP_POPROJ)
        for t in self._block(k):
            self.Po[k["part"], t, r0:r0 + nr] = self.W[f"l{l}.wo"][r0:r0 + nr, c0:c0 + kw] @ self.O[t, c0:c0 + kw]

    def _pgu(self, k):
        l, r0, nm = k["layer"], k["row0"], k["nrows"] // 2
        for t in self._block(k):
            gt = self.W[f"l{l}.w_gate"][r0:r0 + nm] @ self.X[t]
            up = self.W[f"l{l}.w_up"][r0:r0 + nm] @ self.X[t]
            self.M[t, r0:r0 + nm] = gt / (1.0 + np.exp(-gt)) * up

    def _pdown(self, k):
        l, r0, nr = k["layer"], k["row0"], k["nrows"]
        c0, kw = self._slice(k, OP_PDOWN)
        for t in self._block(k):
            self.Pd[k["part"], t, r0:r0 + nr] = self.W[f"l{l}.w_down"][r0:r0 + nr, c0:c0 + kw] @ self.M[t, c0:c0 + kw]

    def _plm(self, k):
        lm = self.W["tok_embed"] if self.cfg.tied else self.W["lm_head"]
        r0, nr = k["row0"], k["nrows"]
        self.logits[r0:r0 + nr] = lm[r0:r0 + nr] @ self.LM

    # ---- the launch --------------------------------------------------------------------

    def run(self, g, tokens, pos0, k_cache, v_cache, seed=0, dynamic=False, slow=None):
        """Executes graph g (taskgraph dict form, from_export) once; returns (hidden [T][h], logits [V],
        next, tasks run) and leaves the K/V writes in k_cache / v_cache."""
        cfg, T = self.cfg, self.T
        h, f, nqd = cfg.hidden, cfg.ffn, cfg.n_q * cfg.head_dim
        tasks = g["tasks"]
        self.So = 1 + max(k["part"] for k in tasks if k["op"] == OP_POPROJ)
        self.Sd = 1 + max(k["part"] for k in tasks if k["op"] == OP_PDOWN)
        self.tok, self.pos0 = np.asarray(tokens), int(pos0)
        self.kc, self.vc = k_cache, v_cache
        nan = np.nan
        self.Ra, self.Rb = np.full((T, h), nan), np.full((T, h), nan)
        self.Po, self.Pd = np.full((self.So, T, h), nan), np.full((self.Sd, T, h), nan)
        self.X, self.Q, self.O, self.M = (np.full((T, h), nan), np.full((T, nqd), nan), np.full((T, nqd), nan),
                                          np.full((T, f), nan))
        self.LM = np.full(h, nan)
        self.logits = np.full(cfg.vocab, nan)
        ops = {OP_PNORM: self._pnorm, OP_PQKV: self._pqkv, OP_PATTN: self._pattn, OP_POPROJ: self._poproj,
               OP_PGU: self._pgu, OP_PDOWN: self._pdown, OP_PLM: self._plm}
        ctr = [0] * len(g["target"])
        rng = np.random.default_rng(seed)
        W = len(g["queues"])
        if dynamic:
            order, nxt, held = list(g["order"]), 0, [None] * W
        else:
            queues, at = [list(q) for q in g["queues"]], [0] * W
        ran = 0
        while True:
            moves = []
            for wg in range(W):
                if dynamic:
                    if held[wg] is None:
                        if nxt < len(order):
                            moves.append((wg, "claim"))
                        continue
                    i = held[wg]
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
                held[wg], nxt = order[nxt], nxt + 1
                continue
            if dynamic:
                i, held[wg] = held[wg], None
            else:
                i = queues[wg][at[wg]]
                at[wg] += 1
            k = tasks[i]
            ops[k["op"]](k)
            if k["sig_ev"] != NONE:
                ctr[k["sig_ev"]] += 1
            ran += 1
        fl = self.logits.astype(np.float32)
        nxt_tok = int(np.argmax(fl)) if np.isfinite(fl).all() else -1
        return self.Rb.copy(), self.logits.copy(), nxt_tok, ran
