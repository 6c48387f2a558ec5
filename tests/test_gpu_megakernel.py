"""GPU parity of the persistent megakernel against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_decode_cu_amd as mk
import synth
from gpu_util import Runner, compare_step, kv_to_host, TOL_HIDDEN_REL, TOL_LOGIT_ABS

pytestmark = pytest.mark.gpu


def _setup(cfg, C, P, gain_std=0.0):
    w = synth.make_weights(cfg, gain_std=gain_std)
    kc, vc = synth.make_kv(cfg, 1, C)
    tok = synth.make_tokens(cfg, 1)
    return w, kc, vc, tok, np.array([P], np.int32)


def _one_step(cfg, C, P, gain_std=0.0, **opt):
    w, kc, vc, tok, pos = _setup(cfg, C, P, gain_std)
    print(f"case {cfg.name} C={C} P={P} opt={opt}", flush=True)
    run = Runner(cfg, w, 1, C, kc, vc, **opt)
    run.step(tok, pos)
    run.check()
    k2, v2 = kc.copy(), vc.copy()
    ref = oracle.decode_step(cfg, w, tok, pos, k2, v2)
    res = compare_step(cfg, ref, run.logits.cpu().numpy(), run.hidden().cpu().numpy(), run.next_tokens().cpu().numpy())
    kg, vg = kv_to_host(run.kv, kc.shape)
    run.close()
    return ref, res, (kc, vc), (k2, v2), (kg, vg)


def _check_kv(orig, ref, gpu, P):
    kc, vc = orig
    for a_ref, a_gpu, a0 in zip(ref, gpu, orig):
        # every slot except P untouched, slot P within one bf16 ulp of the oracle's rounding
        mask = np.ones(a0.shape[3], bool)
        mask[P] = False
        np.testing.assert_array_equal(a_gpu[:, :, :, mask], a0[:, :, :, mask])
        r = oracle.bf16_to_f64(a_ref[:, :, :, P])
        g = oracle.bf16_to_f64(a_gpu[:, :, :, P])
        assert np.all(np.abs(g - r) <= np.abs(r) * 2.0 ** -7 + 1e-30)


@pytest.mark.parametrize("P", [0, 1, 63, 64, 128, 511])
def test_tiny_one_step(P):
    cfg = synth.configs.TINY
    ref, res, orig, refkv, gkv = _one_step(cfg, 512, P)
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL
    assert res["max_dlogit"] <= TOL_LOGIT_ABS
    assert res["argmax_equal"]
    _check_kv(orig, refkv, gkv, P)


def test_tiny_one_step_gains_untied():
    cfg = synth.configs.TINY.with_(tied=False)
    ref, res, orig, refkv, gkv = _one_step(cfg, 256, 200, gain_std=0.2)
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL and res["max_dlogit"] <= TOL_LOGIT_ABS and res["argmax_equal"]
    _check_kv(orig, refkv, gkv, 200)


@pytest.mark.parametrize("W", [1, 4, 37])
def test_tiny_few_workgroups(W):
    cfg = synth.configs.TINY
    ref, res, orig, refkv, gkv = _one_step(cfg, 512, 128, n_workgroups=W)
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL and res["max_dlogit"] <= TOL_LOGIT_ABS and res["argmax_equal"]


def test_tiny_greedy_chain_and_counters():
    cfg = synth.configs.TINY
    C, P0, steps = 512, 128, 32
    w, kc, vc, tok, pos = _setup(cfg, C, P0)
    run = Runner(cfg, w, 1, C, kc, vc, trace=1)
    toks = torch.tensor(tok, dtype=torch.int32, device="cuda")
    positions = torch.arange(P0, P0 + steps, dtype=torch.int32, device="cuda")
    nxt_ptr = mk.mk_next_tokens(run.h)
    got = []
    for s in range(steps):
        if s == 0:
            run.step(toks, positions[0:1])
        else:
            mk.mk_decode_step(run.h, nxt_ptr, positions[s:s + 1].data_ptr(), run.kv.data_ptr(),
                              run.logits.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got.append(int(run.next_tokens().cpu()[0]))
    run.check()
    counts = mk.mk_read_task_counts(run.h, len(run.graph["tasks"]))
    ctr, epoch = mk.mk_read_counters(run.h, run.graph["header"]["n_events"])
    assert epoch == steps
    np.testing.assert_array_equal(counts, np.full(len(counts), steps, np.uint32))
    np.testing.assert_array_equal(ctr, run.graph["target"] * steps)
    run.close()
    ref = oracle.greedy(cfg, w, tok, [P0], kc.copy(), vc.copy(), steps)
    assert got == ref["tokens"][:, 0].tolist(), (got, ref["tokens"][:, 0].tolist(), ref["gaps"][:, 0])


@pytest.mark.parametrize("sched", [1, 2, 3], ids=["dynamic", "event", "scheduler"])
def test_tiny_dynamic_queue_greedy(sched):
    """Greedy chain with tasks taken from one global queue: in task order (1) or in the order their
    events activated them (2: the activating worker appends the dependents; 3: scheduler waves append
    them from activated-event queues); every task runs once per step, counters = k x target."""
    cfg = synth.configs.TINY
    C, P0, steps = 512, 100, 16
    w, kc, vc, tok, pos = _setup(cfg, C, P0)
    print(f"case tiny greedy sched={sched}", flush=True)
    run = Runner(cfg, w, 1, C, kc, vc, sched=sched, trace=1)
    positions = torch.arange(P0, P0 + steps, dtype=torch.int32, device="cuda")
    t0 = torch.tensor(tok, dtype=torch.int32, device="cuda")
    nxt = mk.mk_next_tokens(run.h)
    got = []
    for s in range(steps):
        mk.mk_decode_step(run.h, t0.data_ptr() if s == 0 else nxt, positions[s:s + 1].data_ptr(), run.kv.data_ptr(),
                          run.logits.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got.append(int(run.next_tokens().cpu()[0]))
    run.check()
    counts = mk.mk_read_task_counts(run.h, len(run.graph["tasks"]))
    np.testing.assert_array_equal(counts, np.full(len(counts), steps, np.uint32))
    ctr, epoch = mk.mk_read_counters(run.h, run.graph["header"]["n_events"])
    assert epoch == steps
    np.testing.assert_array_equal(ctr, run.graph["target"] * steps)
    run.close()
    ref = oracle.greedy(cfg, w, tok, [P0], kc.copy(), vc.copy(), steps)
    assert got == ref["tokens"][:, 0].tolist()


@pytest.mark.parametrize("sched", [2, 3], ids=["event", "scheduler"])
@pytest.mark.parametrize("W", [1, 5, 37])
def test_tiny_event_driven_few_workgroups(W, sched):
    ref, res, orig, refkv, gkv = _one_step(synth.configs.TINY, 512, 300, sched=sched, n_workgroups=W)
    print(res)
    assert res["hidden_rel"] <= TOL_HIDDEN_REL and res["max_dlogit"] <= TOL_LOGIT_ABS and res["argmax_equal"]
    _check_kv(orig, refkv, gkv, 300)


def test_tiny_cooperative_launch_greedy():
    """The same greedy chain with the runtime's cooperative launch instead of the default plain one."""
    cfg = synth.configs.TINY
    C, P0, steps = 512, 77, 12
    w, kc, vc, tok, pos = _setup(cfg, C, P0)
    run = Runner(cfg, w, 1, C, kc, vc, cooperative=1)
    positions = torch.arange(P0, P0 + steps, dtype=torch.int32, device="cuda")
    t0 = torch.tensor(tok, dtype=torch.int32, device="cuda")
    nxt = mk.mk_next_tokens(run.h)
    got = []
    for s in range(steps):
        mk.mk_decode_step(run.h, t0.data_ptr() if s == 0 else nxt, positions[s:s + 1].data_ptr(), run.kv.data_ptr(),
                          run.logits.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got.append(int(run.next_tokens().cpu()[0]))
    run.check()
    run.close()
    ref = oracle.greedy(cfg, w, tok, [P0], kc.copy(), vc.copy(), steps)
    assert got == ref["tokens"][:, 0].tolist()


def test_bad_token_is_a_device_error_not_a_hang():
    cfg = synth.configs.TINY
    w, kc, vc, tok, pos = _setup(cfg, 256, 10)
    run = Runner(cfg, w, 1, 256, kc, vc)
    run.step(np.array([cfg.vocab], np.int32), pos)
    torch.cuda.synchronize()
    err = mk.mk_check_device_error(run.h)
    assert err is not None and "out of range" in err
    run.step(np.array([cfg.vocab - 1], np.int32), np.array([256], np.int32))
    err = mk.mk_check_device_error(run.h)
    assert err is not None and "out of range" in err
    # the handle is re-armed: a valid step works afterwards
    run.step(tok, pos)
    run.check()
    run.close()


def test_dropped_signal_is_reported_with_its_event():
    cfg = synth.configs.TINY
    w, kc, vc, tok, pos = _setup(cfg, 256, 10)
    # plan once to pick a task in the middle of layer 1 that signals an event
    probe = Runner(cfg, w, 1, 256, kc, vc)
    tasks = probe.graph["tasks"]
    probe.close()
    victim = int(np.nonzero((tasks["layer"] == 1) & (tasks["op"] == mk.OP_OPROJ))[0][0])
    run = Runner(cfg, w, 1, 256, kc, vc, drop_signal_of_task=victim, debug_timeout_ms=20)
    run.step(tok, pos)
    torch.cuda.synchronize()
    err = mk.mk_check_device_error(run.h)
    print(err)
    assert err is not None and "timeout" in err
    assert f"event {int(tasks['sig_ev'][victim])}" in err
    run.close()


def test_grid_larger_than_the_device_is_refused():
    cfg = synth.configs.TINY
    w, kc, vc, tok, pos = _setup(cfg, 256, 10)
    with pytest.raises(mk.MkError) as ei:
        Runner(cfg, w, 1, 256, kc, vc, n_workgroups=100000)
    assert ei.value.status == mk.MK_E_NOT_RESIDENT
