"""GPU parity of the prompt (prefill) megakernel against the oracle's causal prefill
(oracle/prefill.py, pinned to sequential decode steps): every K/V cache byte the prompt
writes, every prompt token's final residual, the last token's logits and next token; the
cache slots outside the prompt untouched; a decode handle continuing from the prompt's
cache.  Small shapes cover ragged prompts (not a multiple of 16), earlier context
(pos0 > 0), all three GEMM tile shapes, K-sliced projections and the four schedulers;
the Llama-3.2-1B shape runs at the benchmark's prompt lengths."""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_decode_cu_amd as mk
import synth
from gpu_util import dev_weights, dev_kv, kv_to_host, _copy_from_ptr, TOL_HIDDEN_REL, TOL_LOGIT_ABS
from oracle import prefill as oprefill

pytestmark = pytest.mark.gpu

CFG = synth.configs.TINY_PF
# K/V bar.  Layer 0 (whose K/V depend on the token and the layer's weights only): as for the decode
# step's batched path (tests/test_gpu_batch.py), one bf16 ulp of the oracle's value plus 2^-10 of the
# head vector's largest magnitude (the projections carry each fp32 input as two bf16 parts, so a
# projected value is off by up to about 2^-16 sum_i |w_i x_i| before its rounding).  Deeper layers:
# a prompt's contexts are short, so each K/V rounding that the device takes the other way from the
# oracle passes almost unaveraged into the next layers, and the prompt amplifies it: the oracle itself,
# run with the prompt's K/V unrounded instead of rounded (a perturbation of at most half an ulp), keeps
# only 23-42 % of the deeper layers' K bit-exact and moves the final residual by 0.75 % (median) at the
# Llama-1B shape with 128 tokens.  There the K/V of each layer are held, as a whole, to the relative
# error of the residual (TOL_HIDDEN_REL), and every token's residual and the logits to the decode bars.
KV_HEAD_REL = 2.0 ** -10


def check_kv_slots(got, want, positions, label, layers=1):
    """got/want: uint16 [L][1][nkv][C][d].  Layer 0 of every listed slot within the tight bound; each
    of the first `layers` layers within TOL_HIDDEN_REL relative error (L2 over the listed slots)."""
    pos = np.asarray(list(positions))
    r = oracle.bf16_to_f64(want[:1, 0][:, :, pos])
    g = oracle.bf16_to_f64(got[:1, 0][:, :, pos])
    head_max = np.abs(r).max(axis=3, keepdims=True)
    bad = np.argwhere(np.abs(g - r) > np.abs(r) * 2.0 ** -7 + KV_HEAD_REL * head_max + 1e-30)
    for i in bad[:4]:
        t = tuple(i)
        print(f"{label} layer 0 (group, slot, dim) {t[1:]}: oracle {r[t]!r} gpu {g[t]!r}", flush=True)
    assert len(bad) == 0, (label, len(bad))
    for l in range(layers):
        r = oracle.bf16_to_f64(want[l, 0][:, pos])
        g = oracle.bf16_to_f64(got[l, 0][:, pos])
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        if l in (0, layers - 1):
            print(f"{label} layer {l}: relative error {rel:.3g}, bit-exact {float((g == r).mean()):.4f}", flush=True)
        assert rel <= TOL_HIDDEN_REL, (label, l, rel)


class Prompt:
    """A prompt handle plus the device copies of its inputs."""

    def __init__(self, cfg, w, n_tokens, max_ctx, kc, vc, **opt):
        self.cfg = cfg
        wd = dev_weights(w)
        model = mk.Model(cfg, wd)
        opts = dict(debug_timeout_ms=4000)
        opts.update(opt)
        self.h = mk.mk_build_prefill(model.desc, n_tokens, max_ctx, mk.options(**opts))
        del wd, model
        self.kv = dev_kv(kc, vc)
        assert self.kv.numel() * 2 == mk.mk_kv_cache_bytes(self.h)
        self.T = n_tokens
        self.shape = kc.shape
        self.logits = torch.full((cfg.vocab,), float("nan"), dtype=torch.float32, device="cuda")
        self.graph = mk.parse_export(mk.mk_export_graph(self.h))

    def run(self, tokens, pos0):
        t = torch.tensor(np.asarray(tokens, np.int32), device="cuda")
        mk.mk_prefill(self.h, t.data_ptr(), int(pos0), self.kv.data_ptr(), self.logits.data_ptr(),
                      torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        err = mk.mk_check_device_error(self.h)
        assert err is None, err
        return t

    def hidden(self):
        Tp = (self.T + 15) // 16 * 16
        out = torch.empty(Tp, self.cfg.hidden, dtype=torch.float32, device="cuda")
        return _copy_from_ptr(mk.mk_hidden_out(self.h), out)[:self.T].cpu().numpy()

    def next_token(self):
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        return int(_copy_from_ptr(mk.mk_next_tokens(self.h), out).cpu().numpy()[0])

    def close(self):
        mk.mk_destroy(self.h)
        self.h = None


def check_prompt(cfg, run, toks, pos0, kc, vc, ref, kk, vv, label):
    T = len(toks)
    gk, gv = kv_to_host(run.kv, run.shape)
    sl = slice(pos0, pos0 + T)
    for name, got, want, orig in (("K", gk, kk, kc), ("V", gv, vv, vc)):
        check_kv_slots(got, want, range(pos0, pos0 + T), f"{label} {name}", layers=cfg.n_layers)
        # slots outside the prompt untouched
        mask = np.ones(got.shape[3], bool)
        mask[sl] = False
        np.testing.assert_array_equal(got[:, :, :, mask], orig[:, :, :, mask])
    hid = run.hidden().astype(np.float64)
    rel = np.linalg.norm(hid - ref["hidden"], axis=1) / np.linalg.norm(ref["hidden"], axis=1)
    lg = run.logits.cpu().numpy().astype(np.float64)
    dl = float(np.abs(lg - ref["logits"]).max())
    nxt = run.next_token()
    print(f"{label}: hidden rel max {rel.max():.3g}, max |dlogit| {dl:.3g}, next {nxt} (oracle {ref['next']}, "
          f"top-2 gap {oracle.top2_gap(ref['logits']):.3g})", flush=True)
    assert rel.max() <= TOL_HIDDEN_REL
    assert dl <= TOL_LOGIT_ABS
    if oracle.top2_gap(ref["logits"]) > 2 * TOL_LOGIT_ABS:
        assert nxt == ref["next"]
    assert nxt == int(np.argmax(lg.astype(np.float32)))


# (prompt tokens, pos0, max ctx, workgroups (0: one per CU), scheduler)
CASES = [
    (16, 0, 64, 0, 0),
    (40, 0, 128, 0, 0),     # ragged last token group
    (77, 13, 128, 0, 0),    # earlier context, ragged
    (1, 5, 32, 0, 0),       # one token: a decode step through the prompt graph
    (150, 0, 256, 4, 0),    # four workgroups: the 128-row tiles of two token groups per wave
    (40, 7, 128, 0, 1),
    (40, 7, 128, 0, 2),
    (40, 7, 128, 0, 3),
    (64, 64, 128, 0, 0),    # the prompt ends at the cache's last slot
    (96, 0, 96, 0, 0),      # the prompt is the whole cache
    (300, 0, 512, 0, 0),    # more tokens than workgroups: RMSNorm tasks of four tokens
]


@pytest.fixture(scope="module")
def weights():
    return synth.make_weights(CFG, gain_std=0.1)


@pytest.mark.parametrize("T,pos0,C,W,sched", CASES)
def test_prompt_matches_oracle(weights, T, pos0, C, W, sched):
    label = f"case tiny prompt T={T} pos0={pos0} C={C} W={W} sched={sched}"
    print(label, flush=True)
    kc, vc = synth.make_kv(CFG, 1, C)
    toks = synth.make_prompt(CFG, T)
    run = Prompt(CFG, weights, T, C, kc, vc, n_workgroups=W, sched=sched)
    run.run(toks, pos0)
    kk, vv = kc.copy(), vc.copy()
    ref = oprefill.prefill(CFG, weights, toks, pos0, kk, vv)
    check_prompt(CFG, run, toks, pos0, kc, vc, ref, kk, vv, label)
    # a second launch on the same handle (the next chunk of a longer prompt): the oracle continues
    # from the device's cache of the first chunk, so the chunk is compared on its own
    if pos0 + 2 * T <= C:
        toks2 = synth.make_prompt(CFG, T, seed=7)
        k1, v1 = kv_to_host(run.kv, run.shape)
        k1, v1 = k1.copy(), v1.copy()
        run.run(toks2, pos0 + T)
        kk, vv = k1.copy(), v1.copy()
        ref2 = oprefill.prefill(CFG, weights, toks2, pos0 + T, kk, vv)
        check_prompt(CFG, run, toks2, pos0 + T, k1, v1, ref2, kk, vv, label + " second chunk")
    run.close()


def test_prompt_poison_mode(weights):
    """Every scratch buffer a producer overwrites starts as NaN: nothing reads before its producer."""
    T, pos0, C = 40, 3, 128
    print("case tiny prompt poison", flush=True)
    kc, vc = synth.make_kv(CFG, 1, C)
    toks = synth.make_prompt(CFG, T)
    run = Prompt(CFG, weights, T, C, kc, vc, poison=1)
    run.run(toks, pos0)
    kk, vv = kc.copy(), vc.copy()
    ref = oprefill.prefill(CFG, weights, toks, pos0, kk, vv)
    check_prompt(CFG, run, toks, pos0, kc, vc, ref, kk, vv, "poison")
    run.close()


def test_decode_continues_from_the_prompt_cache(weights):
    """A batch-1 decode handle with the same max_ctx takes over the prompt handle's cache."""
    T, C = 40, 128
    print("case tiny prompt then decode", flush=True)
    kc, vc = synth.make_kv(CFG, 1, C)
    toks = synth.make_prompt(CFG, T)
    run = Prompt(CFG, weights, T, C, kc, vc)
    run.run(toks, 0)
    first = run.next_token()
    from gpu_util import Runner
    dec = Runner(CFG, weights, 1, C, kc, vc)
    dec.kv.copy_(run.kv)
    run.close()
    kk, vv = kc.copy(), vc.copy()
    ref = oprefill.prefill(CFG, weights, toks, 0, kk, vv)
    assert first == ref["next"] or oracle.top2_gap(ref["logits"]) <= 2 * TOL_LOGIT_ABS
    tok = ref["next"]
    for s in range(4):
        dec.step([tok], [T + s])
        dec.check()
        r = oracle.decode_step(CFG, weights, [tok], [T + s], kk, vv)
        got = dec.next_tokens().cpu().numpy()
        hid = dec.hidden().cpu().numpy()[0]
        rel = np.linalg.norm(hid - r["hidden"][0]) / np.linalg.norm(r["hidden"][0])
        print(f"decode step {s}: hidden rel {rel:.3g}", flush=True)
        assert rel <= TOL_HIDDEN_REL
        if oracle.top2_gap(r["logits"][0]) > 2 * TOL_LOGIT_ABS:
            assert int(got[0]) == int(r["next"][0])
        tok = int(r["next"][0])
    dec.close()


def test_prompt_rejects_bad_inputs(weights):
    T, C = 16, 64
    kc, vc = synth.make_kv(CFG, 1, C)
    run = Prompt(CFG, weights, T, C, kc, vc)
    t = torch.zeros(T, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for pos0 in (-1, C - T + 1):
        with pytest.raises(mk.MkError):
            mk.mk_prefill(run.h, t.data_ptr(), pos0, run.kv.data_ptr(), 0, s)
    # a token outside the vocabulary: a device error, then the handle works again
    bad = torch.full((T,), CFG.vocab, dtype=torch.int32, device="cuda")
    mk.mk_prefill(run.h, bad.data_ptr(), 0, run.kv.data_ptr(), 0, s)
    torch.cuda.synchronize()
    err = mk.mk_check_device_error(run.h)
    assert err is not None and "out of range" in err
    toks = synth.make_prompt(CFG, T)
    run.run(toks, 0)
    # decode entry points refuse a prompt handle
    with pytest.raises(mk.MkError):
        mk.mk_decode_step(run.h, t.data_ptr(), t.data_ptr(), run.kv.data_ptr(), 0, s)
    run.close()


# ---- the Llama-3.2-1B shape -------------------------------------------------------------------

CFG1B = synth.configs.LLAMA_1B


@pytest.fixture(scope="module")
def weights1b():
    return synth.make_weights(CFG1B)


def test_llama1b_prompt_128(weights1b):
    """The benchmark's short prompt: every output against the oracle's full prefill."""
    T, C = 128, 2048
    print("case llama1b prompt T=128", flush=True)
    kc, vc = synth.make_kv(CFG1B, 1, C)
    toks = synth.make_prompt(CFG1B, T)
    run = Prompt(CFG1B, weights1b, T, C, kc, vc)
    run.run(toks, 0)
    kk, vv = kc.copy(), vc.copy()
    ref = oprefill.prefill(CFG1B, weights1b, toks, 0, kk, vv)
    check_prompt(CFG1B, run, toks, 0, kc, vc, ref, kk, vv, "llama1b T=128")
    run.close()


def test_llama1b_prompt_1024_against_sampled_outputs(weights1b):
    """The benchmark's long prompt: layer-0 K/V of all 1024 tokens against the oracle (they depend on
    each token and layer 0 only), and the first 128 tokens' K/V and residuals against the
    oracle's 128-token prefill (causality: later tokens cannot change them)."""
    T, C = 1024, 2048
    print("case llama1b prompt T=1024", flush=True)
    kc, vc = synth.make_kv(CFG1B, 1, C)
    toks = synth.make_prompt(CFG1B, T)
    run = Prompt(CFG1B, weights1b, T, C, kc, vc)
    run.run(toks, 0)
    gk, gv = kv_to_host(run.kv, run.shape)
    hid = run.hidden()
    run.close()
    # layer 0 of every token
    cfg1 = CFG1B.with_(n_layers=1)
    k1, v1 = kc[:1].copy(), vc[:1].copy()
    oprefill.prefill(cfg1, weights1b, toks, 0, k1, v1)
    for name, got, want in (("K", gk[:1], k1), ("V", gv[:1], v1)):
        check_kv_slots(got, want, range(T), f"layer 0 {name}")
    # the first 128 tokens through every layer
    kk, vv = kc.copy(), vc.copy()
    ref = oprefill.prefill(CFG1B, weights1b, toks[:128], 0, kk, vv)
    for name, got, want in (("K", gk, kk), ("V", gv, vv)):
        check_kv_slots(got, want, range(128), f"first 128 {name}", layers=CFG1B.n_layers)
    rel = np.linalg.norm(hid[:128] - ref["hidden"], axis=1) / np.linalg.norm(ref["hidden"], axis=1)
    print(f"first 128 hidden rel max {rel.max():.3g}", flush=True)
    assert rel.max() <= TOL_HIDDEN_REL
