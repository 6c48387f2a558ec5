"""The allocation-free entry point (mk_decode_step_noalloc) against the ordinary one
(mk_decode_step): the same handle, the same inputs on separate copies of the KV cache, to the
parity bar of the GPU tests (hidden relative error, max |delta logit|, identical next tokens, the
written K/V slots within one bf16 ulp of each other).  Two allocation-free calls in a row on
one GPU, the second with a smaller input (five sequences, then one), so the second starts from
whatever the first left in the shared static scratch; then a greedy chain of allocation-free
steps; and a handle whose scratch exceeds the array is refused."""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_decode_cu_amd as mk
import synth
from gpu_util import Runner, kv_to_host, TOL_HIDDEN_REL, TOL_LOGIT_ABS

pytestmark = pytest.mark.gpu

TINY = synth.configs.TINY
LLAMA_1B = synth.configs.LLAMA_1B
TINY_MOE = synth.configs.TINY_MOE


class Case:
    """A handle, its inputs, and two copies of the KV cache: one for each entry point."""

    def __init__(self, cfg, B, C, positions, **opt):
        self.cfg, self.B = cfg, B
        w = synth.make_weights(cfg)
        kc, vc = synth.make_kv(cfg, B, C)
        self.shape = kc.shape
        self.tok = torch.tensor(np.asarray(synth.make_tokens(cfg, B), np.int32), device="cuda")
        self.pos = torch.tensor(np.asarray(positions, np.int32), device="cuda")
        self.run = Runner(cfg, w, B, C, kc, vc, **opt)
        self.kv_na = self.run.kv.clone()
        self.logits_na = torch.zeros_like(self.run.logits)

    def step(self, noalloc, tok=None):
        sp = torch.cuda.current_stream().cuda_stream
        t = self.tok if tok is None else tok
        if noalloc:
            mk.mk_decode_step_noalloc(self.run.h, t.data_ptr(), self.pos.data_ptr(), self.kv_na.data_ptr(),
                                      self.logits_na.data_ptr(), sp)
        else:
            mk.mk_decode_step(self.run.h, t.data_ptr(), self.pos.data_ptr(), self.run.kv.data_ptr(),
                              self.run.logits.data_ptr(), sp)

    def outputs(self, noalloc):
        self.run.check()
        logits = (self.logits_na if noalloc else self.run.logits).cpu().numpy().astype(np.float64)
        return logits, self.run.hidden().cpu().numpy().astype(np.float64), self.run.next_tokens().cpu().numpy()


def _same(ref, got, kv_ref, kv_got, shape):
    (l0, h0, n0), (l1, h1, n1) = ref, got
    rel = np.linalg.norm(h1 - h0, axis=1) / np.linalg.norm(h0, axis=1)
    dl = float(np.abs(l1 - l0).max())
    print(f"hidden rel {rel.max():.2e}, max |dlogit| {dl:.2e}, next {n0.tolist()} / {n1.tolist()}")
    assert rel.max() <= TOL_HIDDEN_REL and dl <= TOL_LOGIT_ABS
    np.testing.assert_array_equal(n0, n1)
    for name, a, b in zip("KV", kv_to_host(kv_ref, shape), kv_to_host(kv_got, shape)):
        fa, fb = oracle.bf16_to_f64(a), oracle.bf16_to_f64(b)
        # the K/V bar of the parity tests: one bf16 ulp plus 2^-10 of the head vector's largest magnitude
        # (the fp32 residual is summed with device atomics in a varying order, and a K/V element far
        # smaller than its head can land on the other side of a rounding step)
        head_max = np.abs(fa).max(axis=-1, keepdims=True)
        bad = np.argwhere(~(np.abs(fa - fb) <= np.abs(fa) * 2.0 ** -7 + 2.0 ** -10 * head_max + 1e-30))
        for i in bad[:8]:
            t = tuple(i)
            print(f"{name} (layer, seq, group, slot, dim) {t}: ordinary {fa[t]!r} allocation-free {fb[t]!r}")
        assert len(bad) == 0, (name, len(bad))


def test_noalloc_equals_the_ordinary_step_two_calls_in_a_row_second_smaller():
    pos5 = synth.make_positions(5, 0, 511)
    pos5[0] = 0
    big = Case(TINY, 5, 512, pos5)
    small = Case(TINY, 1, 512, [128])
    print("case tiny B=5 then tiny B=1, ordinary steps", flush=True)
    big.step(False)
    ref_big = big.outputs(False)
    small.step(False)
    ref_small = small.outputs(False)
    print("allocation-free: B=5 then B=1, back to back", flush=True)
    big.step(True)
    small.step(True)  # starts from what the five-sequence call left in the static scratch
    torch.cuda.synchronize()
    got_small = small.outputs(True)
    _same(ref_small, got_small, small.run.kv, small.kv_na, small.shape)
    # the five-sequence handle's outputs (its own buffers) are still those of its allocation-free call
    got_big = big.outputs(True)
    _same(ref_big, got_big, big.run.kv, big.kv_na, big.shape)
    big.run.close()
    small.run.close()


@pytest.mark.parametrize("sched", [2, 3], ids=["event", "scheduler"])
def test_noalloc_event_driven_two_calls_in_a_row(sched):
    """Event-driven dispatch (the ready queue's step stamps, and with scheduler waves the activated-event
    stamps, live in the static scratch and are cleared by each call): five sequences, then one."""
    pos5 = synth.make_positions(5, 0, 511)
    big = Case(TINY, 5, 512, pos5, sched=sched)
    small = Case(TINY, 1, 512, [300], sched=sched)
    print(f"case tiny B=5 then B=1, sched {sched}", flush=True)
    big.step(False)
    ref_big = big.outputs(False)
    small.step(False)
    ref_small = small.outputs(False)
    big.step(True)
    small.step(True)
    torch.cuda.synchronize()
    _same(ref_small, small.outputs(True), small.run.kv, small.kv_na, small.shape)
    _same(ref_big, big.outputs(True), big.run.kv, big.kv_na, big.shape)
    big.run.close()
    small.run.close()


def test_noalloc_llama1b_and_a_greedy_chain():
    case = Case(LLAMA_1B, 1, 2048, [1024])
    print("case 1B B=1: ordinary then allocation-free, 3 chained steps each", flush=True)
    refs, gots = [], []
    for noalloc, out in ((False, refs), (True, gots)):
        tok = case.tok
        pos0 = int(case.pos.cpu()[0])
        for s in range(3):
            case.pos.fill_(pos0 + s)
            case.step(noalloc, tok)
            o = case.outputs(noalloc)
            out.append(o)
            tok = torch.tensor(o[2].astype(np.int32), device="cuda")
        case.pos.fill_(pos0)
    for r, g in zip(refs, gots):
        _same(r, g, case.run.kv, case.kv_na, case.shape)
    case.run.close()


def test_noalloc_refuses_a_handle_whose_scratch_exceeds_the_array():
    cfg, B, C = LLAMA_1B, 32, 1100
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, B, C)
    run = Runner(cfg, w, B, C, kc, vc)
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    pos = torch.full((B,), 8, dtype=torch.int32, device="cuda")
    with pytest.raises(mk.MkError) as ei:
        mk.mk_decode_step_noalloc(run.h, tok.data_ptr(), pos.data_ptr(), run.kv.data_ptr(), run.logits.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert ei.value.status == mk.MK_E_UNSUPPORTED
    run.close()


def test_error_check_after_another_handles_allocation_free_steps():
    """A handle whose steps were all ordinary reports no device error after another handle's
    allocation-free steps have left that handle's counters in the per-GPU array (the check
    consults the array's error record only when the handle's own last step used it)."""
    case = Case(LLAMA_1B, 1, 2048, [1024])
    print("case 1B B=1: 3 allocation-free steps, then a tiny MoE handle's ordinary step", flush=True)
    for _ in range(3):
        case.step(True)
    torch.cuda.synchronize()
    assert mk.mk_check_device_error(case.run.h) is None
    other = Case(TINY_MOE, 1, 512, [100])
    other.step(False)
    torch.cuda.synchronize()
    assert mk.mk_check_device_error(other.run.h) is None
    other.run.close()
    case.run.close()
