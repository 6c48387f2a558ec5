"""The prompt graph executed record by record on the CPU fake device equals the oracle's causal prefill.

oracle/fake_prefill.py runs every task of the library planner's prompt graph (mk_plan_prefill, planning
only, no GPU) as its own tile under seeded interleavings of the static queues and of the dynamic order,
with every buffer a task writes starting as NaN.  The result must equal oracle/prefill.py: every prompt
token's final residual and the last token's logits to 1e-9 relative, the next token, and every K/V byte.
Planted mistakes in a graph (a head tile computed twice, a K slice left out, a gate/up tile that does not
wait for its RMSNorm, a norm of the wrong kind, an attention task of the wrong query group) must break it.
"""
import copy

import numpy as np
import pytest

import synth
from oracle import fake_prefill as fp
from oracle import prefill as oprefill
from oracle import taskgraph as tg
from test_prefill_graph import plan_prefill

CFG = synth.configs.TINY_PF


def _inputs(T, pos0, C, seed=0):
    w = synth.make_weights(CFG, gain_std=0.1)
    kc, vc = synth.make_kv(CFG, 1, C)
    toks = synth.make_prompt(CFG, T, seed=seed)
    return w, kc, vc, toks


def _expect(w, kc, vc, toks, pos0):
    kk, vv = kc.copy(), vc.copy()
    r = oprefill.prefill(CFG, w, toks, pos0, kk, vv)
    return r, kk, vv


def _run(g, w, kc, vc, toks, pos0, **kw):
    kk, vv = kc.copy(), vc.copy()
    dev = fp.PromptDevice(CFG, w, len(toks))
    out = dev.run(g, toks, pos0, kk, vv, **kw)
    return out, kk, vv


def _agrees(out, kk, vv, want):
    r, wk, wv = want
    hidden, logits, nxt, _ = out
    if not (np.isfinite(hidden).all() and np.isfinite(logits).all()):
        return False
    return (np.allclose(hidden, r["hidden"], rtol=1e-9, atol=1e-12) and
            np.allclose(logits, r["logits"], rtol=1e-9, atol=1e-12) and nxt == r["next"] and
            np.array_equal(kk, wk) and np.array_equal(vv, wv))


# (prompt tokens, pos0, max ctx, workgroups): ragged prompts, earlier context, the three tile shapes,
# RMSNorm tasks of four tokens and of one (prompts no longer than the workgroup count)
CASES = [(40, 0, 64, 16), (77, 13, 128, 16), (150, 0, 256, 4), (1, 5, 32, 7), (20, 3, 64, 32)]


@pytest.mark.parametrize("T,pos0,C,W", CASES)
def test_prompt_graph_on_the_fake_device_equals_the_prefill(T, pos0, C, W):
    w, kc, vc, toks = _inputs(T, pos0, C)
    want = _expect(w, kc, vc, toks, pos0)
    g = tg.from_export(plan_prefill(CFG, W, T, C))
    n = len(g["tasks"])
    for seed, mode in ((0, {}), (1, {"dynamic": True}), (2, {"slow": 0}), (3, {"slow": W - 1})):
        out, kk, vv = _run(g, w, kc, vc, toks, pos0, seed=seed, **mode)
        assert out[3] == n, mode
        assert _agrees(out, kk, vv, want), mode


def _find(g, **kw):
    return next(k for k in g["tasks"] if all(k[a] == b for a, b in kw.items()))


def test_planted_mistakes_break_the_prompt():
    T, pos0, C, W = 40, 0, 64, 8
    w, kc, vc, toks = _inputs(T, pos0, C)
    want = _expect(w, kc, vc, toks, pos0)
    base = tg.from_export(plan_prefill(CFG, W, T, C))

    def broken(edit, seeds=range(4)):
        for seed in seeds:
            g = copy.deepcopy(base)
            edit(g)
            try:
                out, kk, vv = _run(g, w, kc, vc, toks, pos0, seed=seed, slow=seed % W)
            except (KeyError, AssertionError, IndexError, ValueError):
                return True
            if out[3] < len(g["tasks"]) or not _agrees(out, kk, vv, want):
                return True
        return False

    assert not broken(lambda g: None)  # the unedited graph passes

    def head_twice(g):  # a QKV tile recomputes the tile before it (its own heads never computed)
        k = next(t for t in g["tasks"] if t["op"] == fp.OP_PQKV and t["layer"] == 1 and t["row0"] > 0)
        k["row0"] -= k["nrows"]

    def slice_missing(g):  # one K slice of a down tile dropped (its event's target recounted)
        k = _find(g, op=fp.OP_PDOWN, layer=0, part=1)
        g["tasks"].remove(k)
        g["target"][k["sig_ev"]] -= 1
        for t in g["tasks"]:
            if t["wait_ev"] == k["sig_ev"]:
                t["wait_target"] -= 1
        for q in g["queues"]:
            if k["id"] in q:
                q.remove(k["id"])
        ids = {t["id"]: i for i, t in enumerate(g["tasks"])}
        g["queues"] = [[ids[i] for i in q] for q in g["queues"]]
        g["order"] = [ids[i] for i in g["order"] if i in ids]
        for i, t in enumerate(g["tasks"]):
            t["id"] = i

    def gu_waits_on_attention(g):  # a gate/up tile that does not wait for the FFN-input norms
        k = _find(g, op=fp.OP_PGU, layer=1)
        a = _find(g, op=fp.OP_PATTN, layer=1)
        k["wait_ev"], k["wait_target"] = a["sig_ev"], g["target"][a["sig_ev"]]

    def norm_kind_swapped(g):  # an attention-input norm that completes the FFN's residual instead
        _find(g, op=fp.OP_PNORM, layer=1, part=0, seq=2)["part"] = 1

    def wrong_query_group(g):  # attention for query group 0 of KV group 1 replaced by group 1's
        _find(g, op=fp.OP_PATTN, layer=0, part=1, seq=0)["seq"] = 1

    for edit in (head_twice, slice_missing, gu_waits_on_attention, norm_kind_swapped, wrong_query_group):
        assert broken(edit), edit.__name__
