"""GPU parity of the one-kernel-per-op baseline against the oracle: one sequence
(vector-ALU GEMVs) and several (matrix-core projections over all sequences, split-K
epilogues, attention chunks per sequence and KV group)."""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_decode_cu_amd as mk
import synth
from gpu_util import compare_step, dev_weights, _copy_from_ptr, TOL_HIDDEN_REL, TOL_LOGIT_ABS

pytestmark = pytest.mark.gpu

SMALL = synth.configs.ModelConfig("small", 2, 512, 8, 2, 64, 1024, 4096, True, 10000.0)


def _run_baseline(cfg, C, positions, steps=1, w=None, kc=None, vc=None, tok=None):
    B = len(positions)
    if w is None:
        w = synth.make_weights(cfg, gain_std=0.1)
        kc, vc = synth.make_kv(cfg, B, C)
        tok = synth.make_tokens(cfg, B)
    wd = dev_weights(w)
    model = mk.Model(cfg, wd)
    h = mk.mkb_create(model.desc, B, C)
    kv = torch.from_numpy(np.concatenate([kc.reshape(-1), vc.reshape(-1)]).view(np.int16)).cuda()
    t = torch.tensor(tok, dtype=torch.int32, device="cuda")
    p = torch.tensor(np.asarray(positions, np.int32), device="cuda")
    logits = torch.zeros(B, cfg.vocab, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    toks = []
    for _ in range(steps):
        mk.mkb_decode_step(h, t.data_ptr(), p.data_ptr(), kv.data_ptr(), logits.data_ptr(), s, 1)
        torch.cuda.synchronize()
        toks.append(t.cpu().numpy().copy())
    hidden = _copy_from_ptr(mk.mkb_hidden_out(h), torch.empty(B, cfg.hidden, device="cuda")).cpu().numpy()
    nxt = _copy_from_ptr(mk.mkb_next_tokens(h), torch.empty(B, dtype=torch.int32, device="cuda")).cpu().numpy()
    launches = mk.mkb_launches_per_step(h)
    lg = logits.cpu().numpy()
    kvh = kv.cpu().numpy().view(np.uint16)
    mk.mkb_destroy(h)
    return dict(w=w, kc=kc, vc=vc, tok=tok, logits=lg, hidden=hidden, next=nxt, toks=np.array(toks),
                pos_end=p.cpu().numpy(), launches=launches, kv=kvh)


def _check_one_step(cfg, C, positions):
    print(f"case baseline {cfg.name} B={len(positions)} C={C} positions={list(positions)}", flush=True)
    r = _run_baseline(cfg, C, positions)
    pos = np.asarray(positions, np.int32)
    kc2, vc2 = r["kc"].copy(), r["vc"].copy()
    ref = oracle.decode_step(cfg, r["w"], r["tok"], pos, kc2, vc2)
    res = compare_step(cfg, ref, r["logits"], r["hidden"], r["next"])
    print(res, "launches", r["launches"])
    assert res["hidden_rel"] <= TOL_HIDDEN_REL and res["max_dlogit"] <= TOL_LOGIT_ABS and res["argmax_equal"]
    np.testing.assert_array_equal(r["toks"][-1], r["next"])
    np.testing.assert_array_equal(r["pos_end"], pos + 1)
    # the cache: only each sequence's own slot changes
    n = r["kc"].size
    kg, vg = r["kv"][:n].reshape(r["kc"].shape), r["kv"][n:].reshape(r["vc"].shape)
    for a0, ag in ((r["kc"], kg), (r["vc"], vg)):
        for b, P in enumerate(pos):
            mask = np.ones(a0.shape[3], bool)
            mask[P] = False
            np.testing.assert_array_equal(ag[:, b][:, :, mask], a0[:, b][:, :, mask])
    return r


@pytest.mark.parametrize("cfg,C,P", [(SMALL, 512, 300), (synth.configs.LLAMA_1B, 2048, 1024)])
def test_baseline_one_step(cfg, C, P):
    r = _check_one_step(cfg, C, [P])
    # embedding, 11 per layer, final norm, LM head, two argmax stages
    assert r["launches"] == 11 * cfg.n_layers + 5


@pytest.mark.parametrize("B", [3, 20, 50])
def test_baseline_batch_small(B):
    # ragged batches: one column group with padding, two groups with the second ragged, four
    # groups (50 sequences: the fourth holds 2); contexts from 1 to the last slot
    pos = synth.make_positions(B, 0, 511)
    pos[0], pos[-1] = 0, 511
    _check_one_step(SMALL, 512, pos)


def test_baseline_batch_llama1b():
    """16 sequences at the 1B shape, contexts uniform in [256, 4096]."""
    _check_one_step(synth.configs.LLAMA_1B, 4352, synth.make_positions(16, 256, 4096))


def test_baseline_greedy_chain():
    cfg, C, steps = SMALL, 512, 12
    r = _run_baseline(cfg, C, [200], steps)
    ref = oracle.greedy(cfg, r["w"], r["tok"], [200], r["kc"].copy(), r["vc"].copy(), steps)
    np.testing.assert_array_equal(r["toks"][:, 0], ref["tokens"][:, 0])
    assert r["pos_end"][0] == 200 + steps


def test_baseline_batch_greedy_chain():
    cfg, C, steps = SMALL, 512, 12
    P0 = np.array([5, 200, 480], np.int32)
    r = _run_baseline(cfg, C, P0, steps)
    ref = oracle.greedy(cfg, r["w"], r["tok"], P0, r["kc"].copy(), r["vc"].copy(), steps)
    np.testing.assert_array_equal(r["toks"], ref["tokens"])
    np.testing.assert_array_equal(r["pos_end"], P0 + steps)
