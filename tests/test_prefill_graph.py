"""Host-side tests (no GPU) of the prompt (prefill) graph that mk_plan_prefill exports: every
GEMM output (rows x K slice x token block), attention block and RMSNorm token is covered exactly
once per layer; each phase waits for the phase before it; event targets equal the producers; the
weight tiles of one projection tile the layer's weights without overlap; the graph completes
under random and adversarial interleavings of static and dynamic queues (no deadlock); the
planner's shape limits."""
import collections

import numpy as np
import pytest

import persistent_megakernel_decode_cu_amd as mk
import synth
from oracle import taskgraph as tg
from test_graph import _Fake

TINY_PF, LLAMA_1B = synth.configs.TINY_PF, synth.configs.LLAMA_1B
OPS = (mk.OP_PNORM, mk.OP_PQKV, mk.OP_PATTN, mk.OP_POPROJ, mk.OP_PGU, mk.OP_PDOWN, mk.OP_PLM)


def plan_prefill(cfg, W, T, C, sched=0, policy=0):
    names = ["tok_embed", "final_norm"] + ([] if cfg.tied else ["lm_head"])
    for l in range(cfg.n_layers):
        ffn = ("router", "exp_gate", "exp_up", "exp_down") if cfg.n_experts else ("w_gate", "w_up", "w_down")
        names += [f"l{l}.{n}" for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm") + ffn]
    model = mk.Model(cfg, {n: _Fake() for n in names})
    return mk.parse_export(mk.mk_plan_prefill(model.desc, T, C, mk.options(sched=sched, policy=policy), W))


CASES = [(TINY_PF, 16, 40), (TINY_PF, 4, 150), (TINY_PF, 37, 1), (LLAMA_1B, 256, 128), (LLAMA_1B, 256, 1024)]


@pytest.mark.parametrize("cfg,W,T", CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_prompt_graph_covers_every_output_once(cfg, W, T):
    ex = plan_prefill(cfg, W, T, max(T, 256))
    t = ex["tasks"]
    L, h, d, f = cfg.n_layers, cfg.hidden, cfg.head_dim, cfg.ffn
    ntg = (T + 15) // 16
    tpn = 1 if T <= W else 4  # tokens per RMSNorm task

    def norm_tokens(nt):
        assert set(int(n) for n in nt["nrows"]) == {tpn}
        cov = collections.Counter(t for q in nt["seq"] for t in range(tpn * int(q), min(tpn * int(q) + tpn, T)))
        return sorted(cov) == list(range(T)) and max(cov.values()) == 1 and len(nt) == (T + tpn - 1) // tpn
    assert set(int(o) for o in t["op"]) == set(OPS)
    assert list(t["id"]) == list(range(len(t)))
    rows_of = {mk.OP_PQKV: (cfg.n_q + 2 * cfg.n_kv) * d, mk.OP_POPROJ: h, mk.OP_PGU: f, mk.OP_PDOWN: h}
    k_of = {mk.OP_PQKV: h, mk.OP_POPROJ: cfg.n_q * d, mk.OP_PGU: h, mk.OP_PDOWN: f}
    for l in range(L):
        lt = t[t["layer"] == l]
        for kind in (0, 1):
            assert norm_tokens(lt[(lt["op"] == mk.OP_PNORM) & (lt["part"] == kind)])
        at = lt[lt["op"] == mk.OP_PATTN]
        assert sorted(zip(at["part"], at["seq"])) == sorted((g, q) for g in range(cfg.n_kv) for q in range(ntg))
        for op, N in rows_of.items():
            gt = lt[lt["op"] == op]
            rows = int(gt["nrows"][0])
            assert set(gt["nrows"]) == {rows} and rows in (64, 128)
            ngw = 2 if gt["flags"][0] & 4 else 1
            ntb = (T + 64 * ngw - 1) // (64 * ngw)
            S = len(set(gt["part"]))
            step = rows // 2 if op == mk.OP_PGU else rows  # gate/up tiles hold rows/2 m rows
            cells = collections.Counter((int(r0), int(s), int(b)) for r0, s, b in zip(gt["row0"], gt["part"], gt["seq"]))
            want = {(r0, s, b) for r0 in range(0, N, step) for s in range(S) for b in range(ntb)}
            assert set(cells) == want and max(cells.values()) == 1, op
            # weights: one tile per (row tile, slice), the layer's K x N exactly once, within the packed buffer
            tiles = {(int(r0), int(s)): (int(o), int(wb)) for r0, s, o, wb in zip(gt["row0"], gt["part"], gt["wofs"], gt["wbytes"])}
            assert sum(wb for _, wb in tiles.values()) == (2 if op == mk.OP_PGU else 1) * N * k_of[op] * 2
            spans = sorted(tiles.values())
            assert all(a[0] + a[1] <= b[0] for a, b in zip(spans, spans[1:]))
            assert all(wb % 16384 == 0 for _, wb in tiles.values())
    # the final residual of every token, then the LM head over the whole vocabulary
    assert norm_tokens(t[(t["op"] == mk.OP_PNORM) & (t["part"] == 2)])
    lm = t[t["op"] == mk.OP_PLM]
    cov = np.zeros(cfg.vocab, int)
    for r0, n in zip(lm["row0"], lm["nrows"]):
        cov[r0:r0 + n] += 1
    assert (cov == 1).all()


def _phase(k, L):
    """(layer, phase) of a prompt task: per layer 0 attention-input norms, 1 QKV, 2 attention, 3 O-proj,
    4 FFN-input norms, 5 gate/up, 6 down; after the last layer (L, 0) the final norms, (L, 1) the LM head."""
    op, l = int(k["op"]), int(k["layer"])
    if op == mk.OP_PNORM:
        return (l, {0: 0, 1: 4}[int(k["part"])]) if int(k["part"]) < 2 else (L, 0)
    if op == mk.OP_PLM:
        return (L, 1)
    return (l, {mk.OP_PQKV: 1, mk.OP_PATTN: 2, mk.OP_POPROJ: 3, mk.OP_PGU: 5, mk.OP_PDOWN: 6}[op])


@pytest.mark.parametrize("cfg,W,T", CASES[:4], ids=lambda x: getattr(x, "name", str(x)))
def test_prompt_graph_events_chain_the_phases(cfg, W, T):
    ex = plan_prefill(cfg, W, T, max(T, 256))
    t = ex["tasks"]
    target = ex["target"]
    L = cfg.n_layers
    # targets are the producers' counts; one phase raises each event
    prod = collections.Counter(int(e) for e in t["sig_ev"] if e != tg.NONE)
    assert all(prod[e] == target[e] for e in range(len(target)))
    ev_phase = {}
    for k in t:
        if k["sig_ev"] != tg.NONE:
            ev_phase.setdefault(int(k["sig_ev"]), set()).add(_phase(k, L))
    assert all(len(v) == 1 for v in ev_phase.values())
    # every task waits for exactly the phase before it (and for all of it: wait_target = target)
    for k in t:
        l, ph = _phase(k, L)
        if k["wait_ev"] == tg.NONE:
            assert (l, ph) == (0, 0)
            continue
        (got,) = ev_phase[int(k["wait_ev"])]
        want = (l - 1, 6) if ph == 0 else (l, ph - 1)
        if l == L:
            want = (L - 1, 6) if ph == 0 else (L, 0)
        assert got == want, (int(k["op"]), l, ph, got)
        assert k["wait_target"] == target[k["wait_ev"]]
    assert all(k["sig_ev"] == tg.NONE for k in t if k["op"] == mk.OP_PLM)


@pytest.mark.parametrize("cfg,W,T", [(TINY_PF, 16, 40), (TINY_PF, 5, 77), (LLAMA_1B, 256, 128)],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_prompt_graph_runs_to_completion(cfg, W, T):
    g = tg.from_export(plan_prefill(cfg, W, T, max(T, 256)))
    n = len(g["tasks"])
    for seed in range(3):
        assert tg.simulate(g, W, seed=seed) == n
        assert tg.simulate(g, W, seed=seed, dynamic=True) == n
        assert tg.simulate(g, W, seed=seed, slow=seed % W) == n


def test_prompt_planner_limits():
    for cfg, T, C, status in [
        (TINY_PF.with_(head_dim=128, n_q=4, n_kv=1), 16, 64, mk.MK_E_UNSUPPORTED),   # head_dim 128
        (TINY_PF.with_(hidden=256), 16, 64, mk.MK_E_UNSUPPORTED),                     # hidden not a multiple of 512
        (synth.configs.TINY_MOE.with_(hidden=512), 16, 64, mk.MK_E_UNSUPPORTED),      # mixture of experts
        (synth.configs.LLAMA_8B, 16, 64, mk.MK_E_UNSUPPORTED),                        # hidden 4096
        (TINY_PF, 65, 64, mk.MK_E_INVALID),                                           # prompt longer than the cache
        (TINY_PF, 0, 64, mk.MK_E_INVALID),
    ]:
        with pytest.raises(mk.MkError) as e:
            plan_prefill(cfg, 16, T, C)
        assert e.value.status == status, (cfg.name, T, C)
