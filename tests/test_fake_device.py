"""The task graph executed record by record on the CPU fake device equals the decode step.

oracle/fake_device.py runs every task of a graph as its own tile (the tile named
by the record's fields), reading shared buffers as they stand when it runs and
raising its event when done, under seeded random interleavings of the static
queues, the dynamic queue and the event-driven ready queue.  Both the oracle's
own graph and the library planner's export (planning only, no GPU) must give
the oracle's decode step: hidden state and logits to 1e-9 relative, the next
token, the routed experts and every K/V cache byte exactly.  Planted mistakes in
a graph (a lost residual flag, a missing head tile, an early wait, a low target)
must break the result.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import fake_device as fd
from oracle import taskgraph as tg

from test_graph import plan

TINY, TINY_MOE = synth.configs.TINY, synth.configs.TINY_MOE


def _case(cfg, B, C, lo, hi):
    w = synth.make_weights(cfg, gain_std=0.1)
    k, v = synth.make_kv(cfg, B, C)
    return w, synth.make_tokens(cfg, B), synth.make_positions(B, lo, hi), k, v


def _expect(cfg, w, tok, pos, k, v):
    kk, vv = k.copy(), v.copy()
    r = oracle.decode_step(cfg, w, tok, pos, kk, vv)
    return r, kk, vv


def _run(cfg, g, case, B, C, S, **kw):
    w, tok, pos, k, v = case
    kk, vv = k.copy(), v.copy()
    dev = fd.FakeDevice(cfg, w, B, C, S)
    out = dev.run(g, tok, pos, kk, vv, **kw)
    return out, kk, vv


def _agrees(cfg, out, kk, vv, want):
    r, wk, wv = want
    hidden, logits, nxt, experts, _ = out
    if not (np.isfinite(hidden).all() and np.isfinite(logits).all()):
        return False
    ok = np.allclose(hidden, r["hidden"], rtol=1e-9, atol=1e-12) and \
        np.allclose(logits, r["logits"], rtol=1e-9, atol=1e-12)
    ok = ok and np.array_equal(nxt, r["next"]) and np.array_equal(kk, wk) and np.array_equal(vv, wv)
    if cfg.n_experts:
        ok = ok and np.array_equal(experts, r["experts"])
    return ok


# (config, batch, max context, workgroups, context range) -- one sequence, several, and more than 16
# (two column groups of sequences on the same tiles)
CASES = [
    (TINY, 1, 512, 16, (300, 300)),
    (TINY, 1, 700, 5, (520, 520)),  # three chunks, the last one ragged
    (TINY, 3, 256, 16, (3, 200)),
    (TINY, 17, 64, 32, (1, 60)),
    (TINY_MOE, 1, 300, 16, (200, 200)),
    (TINY_MOE, 2, 128, 16, (5, 100)),
    (TINY_MOE, 17, 32, 24, (0, 30)),
]


@pytest.mark.parametrize("cfg,B,C,W,ctx", CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_oracle_graph_on_the_fake_device_equals_the_decode_step(cfg, B, C, W, ctx):
    case = _case(cfg, B, C, *ctx)
    want = _expect(cfg, *case)
    g = tg.build(cfg, B, C, W)
    S = g["tiling"]["S"]
    n = len(g["tasks"])
    for seed, mode in ((0, {}), (1, {"dynamic": True}), (2, {"event": True}), (3, {"slow": 0})):
        out, kk, vv = _run(cfg, g, case, B, C, S, seed=seed, **mode)
        assert out[4] == n, mode
        assert _agrees(cfg, out, kk, vv, want), mode


@pytest.mark.parametrize("cfg,B,C,W,ctx", CASES[:1] + CASES[3:5] + CASES[6:], ids=lambda x: getattr(x, "name", str(x)))
@pytest.mark.parametrize("policy", [0, 1])
def test_library_plan_on_the_fake_device_equals_the_decode_step(cfg, B, C, W, ctx, policy):
    case = _case(cfg, B, C, *ctx)
    want = _expect(cfg, *case)
    ex = plan(cfg, W, B=B, C=C, policy=policy)
    g = tg.from_export(ex)
    S = ex["header"]["attn_splits"]
    for seed, mode in ((5, {}), (6, {"event": True}), (7, {"slow": W - 1})):
        out, kk, vv = _run(cfg, g, case, B, C, S, seed=seed, **mode)
        assert out[4] == len(g["tasks"])
        assert _agrees(cfg, out, kk, vv, want), mode


def _find(g, **kw):
    return next(k for k in g["tasks"] if all(k[a] == b for a, b in kw.items()))


def test_planted_mistakes_break_the_result():
    """A graph that is wrong in its tiles or its events gives a wrong or unfinished step."""
    cfg, B, C, W = TINY, 1, 512, 8
    case = _case(cfg, B, C, 300, 300)
    want = _expect(cfg, *case)
    S = tg.build(cfg, B, C, W)["tiling"]["S"]

    def broken(edit, seeds=range(6)):
        for seed in seeds:
            g = tg.build(cfg, B, C, W)
            edit(g)
            try:
                out, kk, vv = _run(cfg, g, case, B, C, S, seed=seed, slow=seed % W)
            except (KeyError, AssertionError, IndexError):
                return True
            if out[4] < len(g["tasks"]) or not _agrees(cfg, out, kk, vv, want):
                return True
        return False

    assert not broken(lambda g: None)  # the unedited graph passes

    def no_resid(g):
        _find(g, op=tg.OP_OPROJ, layer=1, part=0, row0=0)["flags"] = 0

    def head_twice(g):  # the last pair block of query head 1 recomputes head 0's block instead
        k = _find(g, op=tg.OP_QKV, layer=0, part=1, row0=24)
        k["part"] = 0

    def oproj_waits_on_qkv(g):  # an O-projection tile that does not wait for attention
        k = _find(g, op=tg.OP_OPROJ, layer=0, part=1, row0=64)
        k["wait_ev"] = _find(g, op=tg.OP_QKV, layer=0, part=0)["sig_ev"]

    def low_target(g):  # the FFN output event of layer 0 released one producer early
        ev = _find(g, op=tg.OP_DOWN, layer=0)["sig_ev"]
        g["target"][ev] -= 1

    def chunk_twice(g):  # attention chunk 1 of group 0 replaced by a second chunk 0
        _find(g, op=tg.OP_ATTN, layer=1, part=0, row0=1)["row0"] = 0

    for edit in (no_resid, head_twice, oproj_waits_on_qkv, low_target, chunk_twice):
        assert broken(edit), edit.__name__


def _deal_of(pos, S, C=1 << 20, d=64):
    dev = fd.FakeDevice(TINY.with_(head_dim=d), {}, len(pos), C, S)
    dev.pos = np.asarray(pos)
    return dev._deal()


@pytest.mark.parametrize("seed", range(40))
def test_attention_deal_is_the_min_max_split_by_brute_force(seed):
    """The deal covers every context exactly once with at most B S chunks (16 per sequence at most), and its
    longest chunk, in pages, is the smallest any split of the contexts into that many chunks can reach
    (all allocations of chunks to sequences enumerated)."""
    import itertools
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    S = int(rng.integers(1, 5))
    pos = rng.integers(0, 1200, B)
    pb = 64
    slots, per = _deal_of(pos, S)
    n = pos + 1
    for b in range(B):
        ln, nch = per[b]
        assert ln % pb == 0 and 1 <= nch <= 16
        got = sorted(c for (bb, c) in slots.values() if bb == b)
        assert got == list(range(nch))
        assert (nch - 1) * ln < n[b] <= nch * ln  # chunks [c ln, (c + 1) ln) clipped to n cover 0..n-1
    assert len(slots) <= B * S and max(slots) < B * S
    best = min(max(-(-(-(-n[b] // s[b])) // pb) for b in range(B))
               for s in itertools.product(range(1, min(16, B * S) + 1), repeat=B) if sum(s) <= B * S)
    assert max(per[b][0] // pb for b in range(B)) == best


def test_attention_deal_worked_example():
    """Two sequences at positions 4095 and 299 (n = 4096 and 300) share 2 x 8 slots: L = 5 pages (320
    positions: 13 + 1 chunks fit 16, 4 pages would need 16 + 2); sequence 0 takes 13 slots of 320 positions
    (the last chunk 256), sequence 1 one slot of 320; slots 14 and 15 stay empty."""
    slots, per = _deal_of([4095, 299], 8)
    assert per == [(320, 13), (320, 1)]
    assert slots == {**{c: (0, c) for c in range(13)}, 13: (1, 0)}
