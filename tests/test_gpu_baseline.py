"""GPU parity of the one-kernel-per-op baseline against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_decode_cu_amd as mk
import synth
from gpu_util import compare_step, dev_kv, dev_weights, _copy_from_ptr, TOL_HIDDEN_REL, TOL_LOGIT_ABS

pytestmark = pytest.mark.gpu

SMALL = synth.configs.ModelConfig("small", 2, 512, 8, 2, 64, 1024, 4096, True, 10000.0)


def _run_baseline(cfg, C, P, steps=1):
    w = synth.make_weights(cfg, gain_std=0.1)
    kc, vc = synth.make_kv(cfg, 1, C)
    tok = synth.make_tokens(cfg, 1)
    wd = dev_weights(w)
    model = mk.Model(cfg, wd)
    h = mk.mkb_create(model.desc, 1, C)
    kv = dev_kv(kc, vc)
    t = torch.tensor(tok, dtype=torch.int32, device="cuda")
    p = torch.tensor([P], dtype=torch.int32, device="cuda")
    logits = torch.zeros(cfg.vocab, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    toks = []
    for _ in range(steps):
        mk.mkb_decode_step(h, t.data_ptr(), p.data_ptr(), kv.data_ptr(), logits.data_ptr(), s, 1)
        torch.cuda.synchronize()
        toks.append(int(t.cpu()[0]))
    hidden = _copy_from_ptr(mk.mkb_hidden_out(h), torch.empty(1, cfg.hidden, device="cuda")).cpu().numpy()
    lg = logits.cpu().numpy()
    mk.mkb_destroy(h)
    return w, kc, vc, tok, lg, hidden, toks, int(p.cpu()[0])


@pytest.mark.parametrize("cfg,C,P", [(SMALL, 512, 300), (synth.configs.LLAMA_1B, 2048, 1024)])
def test_baseline_one_step(cfg, C, P):
    print(f"case baseline {cfg.name} P={P}", flush=True)
    w, kc, vc, tok, lg, hidden, toks, pend = _run_baseline(cfg, C, P)
    ref = oracle.decode_step(cfg, w, tok, [P], kc.copy(), vc.copy())
    res = compare_step(cfg, ref, lg[None], hidden, np.array(toks[-1:], np.int32))
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL and res["max_dlogit"] <= TOL_LOGIT_ABS and res["argmax_equal"]
    assert pend == P + 1


def test_baseline_greedy_chain():
    cfg, C, P, steps = SMALL, 512, 200, 12
    w, kc, vc, tok, lg, hidden, toks, pend = _run_baseline(cfg, C, P, steps)
    ref = oracle.greedy(cfg, w, tok, [P], kc.copy(), vc.copy(), steps)
    assert toks == ref["tokens"][:, 0].tolist()
    assert pend == P + steps
