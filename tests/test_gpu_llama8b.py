"""GPU parity at the full Llama-3-8B shape (32 layers, hidden 4096, heads of 128, SwiGLU 14336,
untied LM head) at batch 1 with a KV cache of 8192 positions, in the launch configuration of
the benchmark (one workgroup per CU, static queues), against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_decode_cu_amd as mk
import synth
from gpu_util import Runner, compare_step, TOL_HIDDEN_REL, TOL_LOGIT_ABS

pytestmark = pytest.mark.gpu

CFG = synth.configs.LLAMA_8B
C, P0, STEPS = 8448, 8192, 4


@pytest.fixture(scope="module")
def model():
    w = synth.make_weights(CFG)
    kc, vc = synth.make_kv(CFG, 1, C)
    tok = synth.make_tokens(CFG, 1)
    return w, kc, vc, tok


def test_llama8b_first_step_and_greedy(model):
    w, kc, vc, tok = model
    print(f"case llama8b P0={P0} steps={STEPS}", flush=True)
    run = Runner(CFG, w, 1, C, kc, vc)
    t0 = torch.tensor(tok, dtype=torch.int32, device="cuda")
    positions = torch.arange(P0, P0 + STEPS, dtype=torch.int32, device="cuda")
    nxt = mk.mk_next_tokens(run.h)
    got = []
    for s in range(STEPS):
        mk.mk_decode_step(run.h, t0.data_ptr() if s == 0 else nxt, positions[s:s + 1].data_ptr(), run.kv.data_ptr(),
                          run.logits.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got.append(int(run.next_tokens().cpu()[0]))
        if s == 0:
            logits = run.logits.cpu().numpy()
            hidden = run.hidden().cpu().numpy()
            first_next = run.next_tokens().cpu().numpy()
    run.check()
    run.close()
    ref = oracle.greedy(CFG, w, tok, [P0], kc.copy(), vc.copy(), STEPS, keep_logits=True)
    r0 = dict(hidden=None, logits=ref["logits"][0], next=ref["tokens"][0])
    dlog = float(np.abs(logits.astype(np.float64) - r0["logits"]).max())
    print({"max_dlogit": dlog, "tokens": got, "oracle": ref["tokens"][:, 0].tolist(), "gaps": ref["gaps"][:, 0].tolist()})
    assert dlog <= TOL_LOGIT_ABS
    assert int(first_next[0]) == int(r0["next"][0])
    assert got == ref["tokens"][:, 0].tolist()


def test_llama8b_first_step_hidden(model):
    w, kc, vc, tok = model
    run = Runner(CFG, w, 1, C, kc, vc, sched=1)
    run.step(tok, [P0])
    run.check()
    res = compare_step(CFG, oracle.decode_step(CFG, w, tok, [P0], kc.copy(), vc.copy()), run.logits.cpu().numpy(),
                       run.hidden().cpu().numpy(), run.next_tokens().cpu().numpy())
    run.close()
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL and res["max_dlogit"] <= TOL_LOGIT_ABS and res["argmax_equal"]
