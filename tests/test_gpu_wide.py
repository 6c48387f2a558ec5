"""GPU parity of the code paths of the larger shapes on small models: hidden 4096 (row-major
VALU GEMV pages for K = 4096) and head_dim 128 (attention pages of 32 positions, O-projection
K = 512), at batch 1 and, for head_dim 128, with several sequences."""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_decode_cu_amd as mk
import synth
from gpu_util import Runner, compare_step, kv_to_host, TOL_HIDDEN_REL, TOL_LOGIT_ABS

pytestmark = pytest.mark.gpu

# 2 layers, hidden 4096, 8 Q / 2 KV heads of 128, SwiGLU 1024, vocab 4096
WIDE = synth.configs.ModelConfig("wide", 2, 4096, 8, 2, 128, 1024, 4096, False, 10000.0)
# hidden 2048 (matrix-core path), heads of 128, for the batched path with head_dim 128
WIDE_B = synth.configs.ModelConfig("wide-b", 2, 2048, 8, 2, 128, 1024, 4096, True, 10000.0)


def _run(cfg, B, C, pos, steps=1, check_kv=True, **opt):
    w = synth.make_weights(cfg, gain_std=0.1)
    kc, vc = synth.make_kv(cfg, B, C)
    tok = synth.make_tokens(cfg, B)
    pos = np.asarray(pos, np.int32)
    print(f"case {cfg.name} B={B} C={C} positions={pos.tolist()} steps={steps} opt={opt}", flush=True)
    run = Runner(cfg, w, B, C, kc, vc, **opt)
    t0 = torch.tensor(tok, dtype=torch.int32, device="cuda")
    positions = torch.tensor(np.stack([pos + s for s in range(steps)]), dtype=torch.int32, device="cuda")
    nxt = mk.mk_next_tokens(run.h)
    got = []
    for s in range(steps):
        mk.mk_decode_step(run.h, t0.data_ptr() if s == 0 else nxt, positions[s].data_ptr(), run.kv.data_ptr(),
                          run.logits.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got.append(run.next_tokens().cpu().numpy().copy())
        if s == 0:
            logits = run.logits.cpu().numpy()
            hidden = run.hidden().cpu().numpy()
            kg, vg = kv_to_host(run.kv, kc.shape)
    run.check()
    run.close()
    k2, v2 = kc.copy(), vc.copy()
    ref = oracle.decode_step(cfg, w, tok, pos, k2, v2)
    res = compare_step(cfg, ref, logits, hidden, got[0])
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL
    assert res["max_dlogit"] <= TOL_LOGIT_ABS
    assert res["argmax_equal"]
    if check_kv:
        for a_ref, a_gpu, a0 in zip((k2, v2), (kg, vg), (kc, vc)):
            for b, P in enumerate(pos):
                mask = np.ones(a0.shape[3], bool)
                mask[P] = False
                np.testing.assert_array_equal(a_gpu[:, b][:, :, mask], a0[:, b][:, :, mask])
                r = oracle.bf16_to_f64(a_ref[:, b, :, P])
                g = oracle.bf16_to_f64(a_gpu[:, b, :, P])
                # batch 1: exact three-part inputs, one bf16 ulp; batches: two-part inputs (see test_gpu_batch)
                tol = np.abs(r) * 2.0 ** -7 + (0 if B == 1 else 2.0 ** -10 * np.abs(r).max(axis=2, keepdims=True))
                assert np.all(np.abs(g - r) <= tol + 1e-30), (b, P)
    if steps > 1:
        ref = oracle.greedy(cfg, w, tok, pos, kc.copy(), vc.copy(), steps)
        np.testing.assert_array_equal(np.array(got), ref["tokens"])


@pytest.mark.parametrize("P", [0, 31, 32, 100, 511])
def test_wide_one_step(P):
    _run(WIDE, 1, 512, [P])


def test_wide_greedy_chain():
    _run(WIDE, 1, 512, [200], steps=12)


def test_wide_dynamic_queue():
    _run(WIDE, 1, 512, [300], sched=1)


def test_head_dim_128_batch():
    _run(WIDE_B, 3, 512, [5, 300, 511])


def test_head_dim_128_batch_greedy_chain():
    _run(WIDE_B, 4, 1024, [40, 700, 1000, 63], steps=6)
