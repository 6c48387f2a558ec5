"""Poison mode (mk_options.poison): before every step the step's scratch that producers
overwrite (query rows, attention partials, SiLU(gate)*up rows, matrix-core operand regions,
router logits, selected experts) and the logits and hidden outputs are filled with NaN (expert
ids with -1).  A task that read any of them before its producer wrote it would carry NaN (or an
impossible expert id) into the outputs, so results equal to the oracle's under poison show that
no task reads ahead of its producers, for one sequence, for several, with experts, and over a
chain of steps.  Checks against the oracle through the C ABI, as every GPU parity test."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Runner, compare_step, TOL_HIDDEN_REL, TOL_LOGIT_ABS

pytestmark = pytest.mark.gpu

TINY = synth.configs.TINY
TINY_MOE = synth.configs.TINY_MOE
LLAMA_1B = synth.configs.LLAMA_1B


def _poisoned_step(cfg, B, C, positions, **opt):
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, B, C)
    tok = synth.make_tokens(cfg, B)
    pos = np.asarray(positions, np.int32)
    print(f"case {cfg.name} B={B} C={C} positions={pos.tolist()} poison opt={opt}", flush=True)
    run = Runner(cfg, w, B, C, kc, vc, poison=1, **opt)
    run.step(tok, pos)
    run.check()
    logits = run.logits.cpu().numpy()
    hidden = run.hidden().cpu().numpy()
    nxt = run.next_tokens().cpu().numpy()
    eids = None
    if cfg.n_experts:
        import persistent_megakernel_decode_cu_amd as mk
        from gpu_util import _copy_from_ptr
        out = torch.empty(cfg.n_layers * B * cfg.top_k, dtype=torch.int32, device="cuda")
        eids = _copy_from_ptr(mk.mk_expert_ids(run.h), out).cpu().numpy().reshape(cfg.n_layers, B, cfg.top_k)
    run.close()
    assert np.isfinite(logits).all() and np.isfinite(hidden).all()
    ref = oracle.decode_step(cfg, w, tok, pos, kc.copy(), vc.copy())
    res = compare_step(cfg, ref, logits, hidden, nxt)
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL
    assert res["max_dlogit"] <= TOL_LOGIT_ABS
    assert res["argmax_equal"], (nxt, ref["next"])
    if eids is not None:
        assert (eids >= 0).all()
        np.testing.assert_array_equal(eids, ref["experts"])


def test_poison_tiny_one_sequence():
    _poisoned_step(TINY, 1, 512, [128])


@pytest.mark.parametrize("sched", [0, 1, 2, 3], ids=["static", "dynamic", "event", "scheduler"])
def test_poison_tiny_five_sequences(sched):
    pos = synth.make_positions(5, 0, 511)
    pos[0] = 0
    _poisoned_step(TINY, 5, 512, pos, sched=sched)


def test_poison_tiny_moe():
    pos = synth.make_positions(5, 0, 511)
    _poisoned_step(TINY_MOE, 5, 512, pos)


def test_poison_tiny_moe_one_sequence():
    _poisoned_step(TINY_MOE, 1, 512, [300])


def test_poison_llama1b_one_sequence():
    _poisoned_step(LLAMA_1B, 1, 2048, [1024])


def test_poison_llama1b_sixteen_sequences():
    """The several-sequence path at scale under poison: dealt attention chunks, column-group operands."""
    _poisoned_step(LLAMA_1B, 16, 4352, synth.make_positions(16, 256, 4096))


def test_poison_tiny_greedy_chain():
    """Eight chained steps with poison before each one equal eight oracle steps."""
    cfg, C, P0, n = TINY, 512, 100, 8
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, 1, C)
    tok = synth.make_tokens(cfg, 1)
    run = Runner(cfg, w, 1, C, kc, vc, poison=1)
    toks = []
    t = torch.tensor(np.asarray(tok, np.int32), device="cuda")
    for s in range(n):
        run.step(t, [P0 + s])
        t = run.next_tokens().clone()
        toks.append(int(t.cpu()[0]))
    run.check()
    run.close()
    k2, v2 = kc.copy(), vc.copy()
    tt = np.asarray(tok, np.int32)
    ref = []
    for s in range(n):
        r = oracle.decode_step(cfg, w, tt, [P0 + s], k2, v2)
        tt = r["next"].astype(np.int32)
        ref.append(int(tt[0]))
    assert toks == ref
