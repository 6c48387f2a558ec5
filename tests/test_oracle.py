"""Pins of the CPU oracle against what mathematics and independent libraries fix.

None of these re-types the oracle's own formulas: each compares with a library
routine (torch, numpy, HF transformers' Llama / Mixtral), a closed form, an
invariant, or a special case whose answer is known without the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

RNG = np.random.default_rng(1234)


def bf16_bits_from_torch(x):
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, std=1.0):
    return bf16_bits_from_torch(RNG.normal(0.0, std, size=shape).astype(np.float32))


# ---- scalar rounding --------------------------------------------------------

def test_bf16_rounding_matches_torch():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even; the oracle rounds
    # double -> float -> bf16, so on float32 inputs the two must agree bit for bit.
    vals = RNG.normal(0, 3, 20000).astype(np.float32)
    vals = np.concatenate([vals, np.float32([0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 65504.0,
                                             1e-38, 3.0e38])])
    ref = bf16_bits_from_torch(vals)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)
    # ties go to even: 1 + 2^-8 -> 1.0 (0x3F80), 1 + 3*2^-8 -> 0x3F82
    assert oracle.f64_to_bf16(1 + 2 ** -8) == 0x3F80
    assert oracle.f64_to_bf16(1 + 3 * 2 ** -8) == 0x3F82


def test_bf16_decode_exact():
    bits = rand_bf16(1000)
    ref = torch.tensor(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.bf16_to_f64(bits), ref)


# ---- RMSNorm ------------------------------------------------------------------

def test_rmsnorm_unit_rms_before_gain():
    x = RNG.normal(0, 2.5, 2048)
    ones = np.full(2048, synth.BF16_ONE, np.uint16)
    eps = 1e-5
    xn = oracle.rmsnorm(x, ones, eps)
    mu = np.mean(x * x)
    assert abs(np.mean(xn * xn) - mu / (mu + eps)) < 1e-13
    # scale covariance: rmsnorm(c x; eps) = rmsnorm(x; eps / c^2)
    xn2 = oracle.rmsnorm(1000.0 * x, ones, eps)
    np.testing.assert_allclose(xn2, oracle.rmsnorm(x, ones, eps * 1e-6), rtol=1e-13, atol=0)


def test_rmsnorm_matches_torch_with_gain():
    x = RNG.normal(0, 1, 256)
    g = bf16_bits_from_torch(1 + 0.1 * RNG.normal(size=256))
    gw = torch.tensor(oracle.bf16_to_f64(g))
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (256,), weight=gw, eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 1e-5), ref, rtol=1e-13, atol=1e-15)


# ---- GEMV / SiLU / argmax ------------------------------------------------------

def test_gemv_matches_numpy():
    W = rand_bf16((96, 300), 0.05)
    x = RNG.normal(size=300)
    np.testing.assert_allclose(oracle.gemv(W, x), oracle.bf16_to_f64(W) @ x, rtol=1e-12, atol=1e-13)


def test_gemv_identity_rows():
    W = np.zeros((8, 8), np.uint16)
    for i in range(8):
        W[i, i] = synth.BF16_ONE
    x = RNG.normal(size=8)
    np.testing.assert_array_equal(oracle.gemv(W, x), x)


def test_silu_matches_torch():
    z = np.concatenate([RNG.normal(0, 4, 1000), [0.0, 50.0, -50.0]])
    ref = torch.nn.functional.silu(torch.tensor(z)).numpy()
    got = np.array([oracle.silu(v) for v in z])
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) / 40.0 - 1.0) < 1e-15


def test_argmax_lowest_index_and_float_decision():
    v = np.array([0.5, 2.0, -1.0, 2.0, 1.9])
    assert oracle.argmax_f32(v) == 1
    # distinct in double, equal once rounded to float: the lower index wins
    a = 1.0 + 2 ** -30
    v = np.array([0.0, 1.0, a])
    assert np.float32(a) == np.float32(1.0)
    assert oracle.argmax_f32(v) == 1
    assert oracle.argmax_f32(np.array([0.0, np.nan, 1.0])) == -1
    r = RNG.normal(size=5000)
    assert oracle.argmax_f32(r) == int(np.argmax(r.astype(np.float32)))


def test_topk_softmax_against_torch():
    for _ in range(20):
        lg = RNG.normal(0, 1, 64)
        ids, w = oracle.topk_softmax(lg, 8)
        f = torch.tensor(lg.astype(np.float32))
        top = torch.topk(f, 8)
        assert set(ids.tolist()) == set(top.indices.tolist())
        ref = torch.softmax(torch.tensor(lg)[ids.tolist()], 0).numpy()
        np.testing.assert_allclose(w, ref, rtol=1e-14)
        # equivalently: softmax over all, keep the 8, renormalise
        p = torch.softmax(torch.tensor(lg), 0).numpy()[ids]
        np.testing.assert_allclose(w, p / p.sum(), rtol=1e-12)
    ids, _ = oracle.topk_softmax(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), 2)
    assert ids.tolist() == [1, 2]


# ---- RoPE ---------------------------------------------------------------------

def test_rope_is_complex_rotation():
    d, nh, theta = 64, 3, 500000.0
    for pos in (0, 1, 17, 1279, 8191):
        u = RNG.normal(size=nh * d)
        got = oracle.rope(u, nh, d, pos, theta).reshape(nh, d)
        z = u.reshape(nh, d)[:, : d // 2] + 1j * u.reshape(nh, d)[:, d // 2:]
        j = np.arange(d // 2)
        rot = z * np.exp(1j * pos * theta ** (-2.0 * j / d))
        np.testing.assert_allclose(got[:, : d // 2], rot.real, rtol=0, atol=1e-12)
        np.testing.assert_allclose(got[:, d // 2:], rot.imag, rtol=0, atol=1e-12)


def test_rope_invariants():
    d, theta = 128, 10000.0
    q, k = RNG.normal(size=d), RNG.normal(size=d)
    np.testing.assert_array_equal(oracle.rope(q, 1, d, 0, theta), q)  # position 0 is the identity
    for m, n in ((5, 2), (300, 41), (1000, 999)):
        lhs = oracle.rope(q, 1, d, m, theta) @ oracle.rope(k, 1, d, n, theta)
        rhs = oracle.rope(q, 1, d, m - n, theta) @ k
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))
        r = oracle.rope(q, 1, d, m, theta)
        np.testing.assert_allclose(r[: d // 2] ** 2 + r[d // 2:] ** 2, q[: d // 2] ** 2 + q[d // 2:] ** 2,
                                   rtol=1e-12)


def test_rope_matches_transformers():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    d, nh, theta = 64, 4, 500000.0
    cfg = LlamaConfig(hidden_size=nh * d, num_attention_heads=nh, head_dim=d, rope_theta=theta,
                      max_position_embeddings=8192)
    emb = LlamaRotaryEmbedding(cfg)
    emb.inv_freq = 1.0 / (theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    x = torch.tensor(RNG.normal(size=(1, nh, 1, d)))
    for pos in (0, 3, 1023, 4095):
        cos, sin = emb(x, torch.tensor([[pos]]))
        qr, _ = apply_rotary_pos_emb(x, x, cos, sin)
        got = oracle.rope(x.numpy().reshape(-1), nh, d, pos, theta)
        # transformers forms the angles in float32, so agreement is to float32 angle precision
        np.testing.assert_allclose(got, qr.numpy().reshape(-1), rtol=0, atol=1e-7 * (pos + 1))


# ---- attention ---------------------------------------------------------------

def test_attention_matches_sdpa():
    d = 64
    for n in (1, 2, 65, 300):
        q = RNG.normal(size=d)
        K, V = rand_bf16((n, d)), rand_bf16((n, d))
        got = oracle.attention_head(q, K, V)
        Kt = torch.tensor(oracle.bf16_to_f64(K))[None, None]
        Vt = torch.tensor(oracle.bf16_to_f64(V))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q)[None, None, None], Kt, Vt)
        np.testing.assert_allclose(got, ref.numpy().reshape(-1), rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    d = 64
    q = RNG.normal(size=d)
    K, V = rand_bf16((1, d)), rand_bf16((1, d))
    np.testing.assert_array_equal(oracle.attention_head(q, K, V), oracle.bf16_to_f64(V[0]))  # one position
    K = np.tile(rand_bf16((1, d)), (37, 1))  # identical keys -> plain mean of the values
    V = rand_bf16((37, d))
    np.testing.assert_allclose(oracle.attention_head(q, K, V), oracle.bf16_to_f64(V).mean(0), rtol=1e-12,
                               atol=1e-14)
    # a dominant score picks its value row
    K = np.zeros((10, d), np.uint16)
    K[4] = bf16_bits_from_torch(np.full(d, 100.0))
    V = rand_bf16((10, d))
    np.testing.assert_allclose(oracle.attention_head(np.ones(d), K, V), oracle.bf16_to_f64(V[4]), atol=1e-12)
    # cur_k / cur_v replace the last row only
    K, V = rand_bf16((5, d)), rand_bf16((5, d))
    ck, cv = RNG.normal(size=d), RNG.normal(size=d)
    Kt = torch.tensor(oracle.bf16_to_f64(K)); Kt[-1] = torch.tensor(ck)
    Vt = torch.tensor(oracle.bf16_to_f64(V)); Vt[-1] = torch.tensor(cv)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q)[None, None, None], Kt[None, None],
                                                           Vt[None, None]).numpy().reshape(-1)
    np.testing.assert_allclose(oracle.attention_head(q, K, V, ck, cv), ref, rtol=1e-12, atol=1e-13)


# ---- whole decode step against HF transformers (fp64) ------------------------

def _hf_llama(cfg, w):
    from transformers import LlamaConfig, LlamaForCausalLM
    hc = LlamaConfig(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.ffn,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_q, num_key_value_heads=cfg.n_kv,
                     head_dim=cfg.head_dim, rms_norm_eps=cfg.eps, rope_theta=cfg.rope_theta,
                     tie_word_embeddings=cfg.tied, max_position_embeddings=1 << 16, attention_bias=False,
                     mlp_bias=False)
    hc._attn_implementation = "eager"
    m = LlamaForCausalLM(hc).double().eval()
    f = oracle.bf16_to_f64
    sd = {"model.embed_tokens.weight": f(w["tok_embed"]), "model.norm.weight": f(w["final_norm"])}
    if not cfg.tied:
        sd["lm_head.weight"] = f(w["lm_head"])
    for l in range(cfg.n_layers):
        p, q = f"l{l}.", f"model.layers.{l}."
        sd[q + "input_layernorm.weight"] = f(w[p + "attn_norm"])
        sd[q + "post_attention_layernorm.weight"] = f(w[p + "ffn_norm"])
        for a, b in (("wq", "self_attn.q_proj"), ("wk", "self_attn.k_proj"), ("wv", "self_attn.v_proj"),
                     ("wo", "self_attn.o_proj"), ("w_gate", "mlp.gate_proj"), ("w_up", "mlp.up_proj"),
                     ("w_down", "mlp.down_proj")):
            sd[q + b + ".weight"] = f(w[p + a])
    sd = {k: torch.tensor(v) for k, v in sd.items()}
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("lm_head" in k for k in missing), (missing, unexpected)
    if cfg.tied:
        m.tie_weights()
    d = cfg.head_dim
    m.model.rotary_emb.inv_freq = 1.0 / (cfg.rope_theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    return m


def _hf_step(m, cfg, kc, vc, token, pos):
    """One decode step of HF's model with the cache prefilled from kc/vc (layer-major, batch 1)."""
    from transformers.cache_utils import DynamicCache
    cache = DynamicCache()
    for l in range(cfg.n_layers):
        k = torch.tensor(oracle.bf16_to_f64(kc[l, 0, :, :pos]))[None]
        v = torch.tensor(oracle.bf16_to_f64(vc[l, 0, :, :pos]))[None]
        cache.update(k, v, l)
    resid = {}
    h = m.model.layers[-1].register_forward_hook(lambda mod, i, o: resid.__setitem__("x", o[0] if isinstance(o, tuple) else o))
    with torch.no_grad():
        out = m(input_ids=torch.tensor([[token]]), position_ids=torch.tensor([[pos]]), past_key_values=cache,
                use_cache=True, cache_position=torch.tensor([pos]))
    h.remove()
    newk = [cache.layers[l].keys[0, :, pos].numpy() for l in range(cfg.n_layers)]
    return out.logits[0, 0].numpy(), resid["x"][0, 0].numpy(), newk


@pytest.mark.parametrize("tied,gain_std", [(True, 0.0), (True, 0.2), (False, 0.2)])
def test_decode_step_matches_transformers_llama(tied, gain_std):
    cfg = synth.configs.TINY.with_(tied=tied)
    w = synth.make_weights(cfg, gain_std=gain_std)
    P, C = 128, 256
    kc, vc = synth.make_kv(cfg, 1, C)
    tok = int(synth.make_tokens(cfg, 1)[0])
    m = _hf_llama(cfg, w)
    ref_logits, ref_x, ref_k = _hf_step(m, cfg, kc, vc, tok, P)
    k2, v2 = kc.copy(), vc.copy()
    r = oracle.decode_step(cfg, w, [tok], [P], k2, v2, kv_round=False)
    # HF normalises in float32 internally, so agreement is to ~1e-7 relative
    np.testing.assert_allclose(r["hidden"][0], ref_x, rtol=0, atol=2e-6 * np.abs(ref_x).max())
    np.testing.assert_allclose(r["logits"][0], ref_logits, rtol=0, atol=2e-6 * np.abs(ref_logits).max())
    assert r["next"][0] == int(np.argmax(ref_logits.astype(np.float32)))
    for l in range(cfg.n_layers):
        got = oracle.bf16_to_f64(k2[l, 0, :, P])
        ulp = np.abs(got) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(got - ref_k[l]) <= ulp), l
    # the step wrote slot P only
    mask = np.ones(C, bool)
    mask[P] = False
    np.testing.assert_array_equal(k2[:, :, :, mask], kc[:, :, :, mask])
    np.testing.assert_array_equal(v2[:, :, :, mask], vc[:, :, :, mask])


def test_decode_step_identity_blocks_predict_from_embedding():
    # With W_o = W_d = 0 the residual never moves: x = E[t], so the next token is
    # argmax_v <E_v, rmsnorm(E_t)> (brute force over the vocabulary).
    cfg = synth.configs.TINY
    w = synth.make_weights(cfg)
    for l in range(cfg.n_layers):
        w[f"l{l}.wo"][:] = 0
        w[f"l{l}.w_down"][:] = 0
    kc, vc = synth.make_kv(cfg, 1, 256)
    for tok in (0, 17, 4095):
        r = oracle.decode_step(cfg, w, [tok], [100], kc.copy(), vc.copy())
        E = oracle.bf16_to_f64(w["tok_embed"])
        np.testing.assert_array_equal(r["hidden"][0], E[tok])
        xn = E[tok] / math.sqrt(np.mean(E[tok] ** 2) + cfg.eps)
        brute = E @ xn
        assert r["next"][0] == int(np.argmax(brute.astype(np.float32)))
        np.testing.assert_allclose(r["logits"][0], brute, rtol=1e-12, atol=1e-14)


def test_decode_step_zero_layers():
    cfg = synth.configs.TINY.with_(n_layers=0)
    w = synth.make_weights(cfg)
    kc = np.zeros((0, 1, cfg.n_kv, 8, cfg.head_dim), np.uint16)
    r = oracle.decode_step(cfg, w, [7], [0], kc, kc.copy())
    E = oracle.bf16_to_f64(w["tok_embed"])
    xn = E[7] / math.sqrt(np.mean(E[7] ** 2) + cfg.eps)
    np.testing.assert_allclose(r["logits"][0], E @ xn, rtol=1e-12, atol=1e-14)


def test_decode_step_batch_is_independent_sequences():
    cfg = synth.configs.TINY
    w = synth.make_weights(cfg)
    B, C = 3, 256
    kc, vc = synth.make_kv(cfg, B, C)
    toks = np.array([5, 900, 4000], np.int32)
    pos = np.array([0, 37, 255], np.int32)
    rb = oracle.decode_step(cfg, w, toks, pos, kc.copy(), vc.copy())
    for b in range(B):
        k1 = np.ascontiguousarray(kc[:, b:b + 1])
        v1 = np.ascontiguousarray(vc[:, b:b + 1])
        r1 = oracle.decode_step(cfg, w, toks[b:b + 1], pos[b:b + 1], k1, v1)
        np.testing.assert_array_equal(rb["logits"][b], r1["logits"][0])


def test_decode_step_rejects_bad_inputs():
    cfg = synth.configs.TINY
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, 1, 16)
    with pytest.raises(ValueError):
        oracle.decode_step(cfg, w, [cfg.vocab], [0], kc, vc)
    with pytest.raises(ValueError):
        oracle.decode_step(cfg, w, [0], [16], kc, vc)


def test_moe_step_matches_transformers_mixtral():
    from transformers import MixtralConfig, MixtralForCausalLM
    from transformers.cache_utils import DynamicCache
    cfg = synth.configs.ModelConfig("moe-tiny", 2, 128, 4, 2, 32, 0, 512, True, 10000.0,
                                    n_experts=8, top_k=2, expert_ffn=64)
    w = synth.make_weights(cfg, gain_std=0.1)
    hc = MixtralConfig(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.expert_ffn,
                       num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_q, num_key_value_heads=cfg.n_kv,
                       head_dim=cfg.head_dim, num_local_experts=cfg.n_experts, num_experts_per_tok=cfg.top_k,
                       rms_norm_eps=cfg.eps, rope_theta=cfg.rope_theta, tie_word_embeddings=True,
                       max_position_embeddings=4096)
    hc._attn_implementation = "eager"
    hc._experts_implementation = "eager"
    m = MixtralForCausalLM(hc).double().eval()
    f = oracle.bf16_to_f64
    sd = {"model.embed_tokens.weight": f(w["tok_embed"]), "model.norm.weight": f(w["final_norm"])}
    for l in range(cfg.n_layers):
        p, q = f"l{l}.", f"model.layers.{l}."
        sd[q + "input_layernorm.weight"] = f(w[p + "attn_norm"])
        sd[q + "post_attention_layernorm.weight"] = f(w[p + "ffn_norm"])
        for a, b in (("wq", "self_attn.q_proj"), ("wk", "self_attn.k_proj"), ("wv", "self_attn.v_proj"),
                     ("wo", "self_attn.o_proj"), ("router", "mlp.gate")):
            sd[q + b + ".weight"] = f(w[p + a])
        sd[q + "mlp.experts.gate_up_proj"] = np.concatenate([f(w[p + "exp_gate"]), f(w[p + "exp_up"])], axis=1)
        sd[q + "mlp.experts.down_proj"] = f(w[p + "exp_down"])
    sd = {k: torch.tensor(v) for k, v in sd.items()}
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("lm_head" in k for k in missing), (missing, unexpected)
    m.tie_weights()
    d = cfg.head_dim
    m.model.rotary_emb.inv_freq = 1.0 / (cfg.rope_theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    P, C = 40, 64
    kc, vc = synth.make_kv(cfg, 1, C)
    cache = DynamicCache()
    for l in range(cfg.n_layers):
        cache.update(torch.tensor(f(kc[l, 0, :, :P]))[None], torch.tensor(f(vc[l, 0, :, :P]))[None], l)
    with torch.no_grad():
        out = m(input_ids=torch.tensor([[3]]), position_ids=torch.tensor([[P]]), past_key_values=cache,
                use_cache=True, cache_position=torch.tensor([P]), output_router_logits=True)
    ref = out.logits[0, 0].numpy()
    r = oracle.decode_step(cfg, w, [3], [P], kc.copy(), vc.copy(), kv_round=False)
    np.testing.assert_allclose(r["logits"][0], ref, rtol=0, atol=2e-6 * np.abs(ref).max())
    # router logits of every layer, and the experts they select
    for l in range(cfg.n_layers):
        rl = out.router_logits[l].reshape(-1).numpy()
        np.testing.assert_allclose(r["router"][l, 0], rl, rtol=0, atol=1e-6 * np.abs(rl).max())
        np.testing.assert_array_equal(np.sort(r["experts"][l, 0]), np.sort(np.argsort(-rl)[:cfg.top_k]))


# ---- the pages' own arithmetic ------------------------------------------------

def test_page_arithmetic_fixtures():
    """Arithmetic the pages state, kept as golden fixtures (tests/golden/page_facts.txt)."""
    import os
    from oracle import taskgraph
    facts = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                facts[k.strip()] = [int(t) for t in v.split(",")]
    n_blocks, n_sms, idle = facts["tail_effect_blocks_sms_idle"]
    assert taskgraph.idle_units_in_last_wave(n_blocks, n_sms) == idle
    n_pages, page_kib, total = facts["paged_smem_pages_kib_bytes"]
    assert n_pages * page_kib * 1024 == total


# ---- causal prefill (oracle/prefill.py) ----------------------------------------

from oracle import prefill as oprefill  # noqa: E402


def _prefill_case(cfg, T, pos0, C, gain_std=0.1, seed=0):
    w = synth.make_weights(cfg, gain_std=gain_std)
    kc, vc = synth.make_kv(cfg, 1, C)
    toks = np.random.default_rng(seed).integers(0, cfg.vocab, T)
    return w, kc, vc, toks


@pytest.mark.parametrize("T,pos0", [(1, 0), (7, 0), (19, 33)])
def test_prefill_equals_sequential_decode_steps(T, pos0):
    # Causal prefill of T tokens is T decode steps over the same tokens (the C decode-step
    # definition, pinned above against transformers): every K/V byte equal, every token's
    # final residual and the last token's logits to rounding.
    cfg = synth.configs.TINY
    w, kc, vc, toks = _prefill_case(cfg, T, pos0, 64)
    k1, v1 = kc.copy(), vc.copy()
    r = oprefill.prefill(cfg, w, toks, pos0, k1, v1)
    k2, v2 = kc.copy(), vc.copy()
    for t in range(T):
        s = oracle.decode_step(cfg, w, [int(toks[t])], [pos0 + t], k2, v2)
        np.testing.assert_allclose(r["hidden"][t], s["hidden"][0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["logits"], s["logits"][0], rtol=1e-10, atol=1e-12)
    assert r["next"] == int(s["next"][0])
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
    # slots outside pos0 .. pos0 + T - 1 untouched
    mask = np.ones(64, bool)
    mask[pos0:pos0 + T] = False
    np.testing.assert_array_equal(k1[:, :, :, mask], kc[:, :, :, mask])


def test_prefill_matches_transformers_llama_causal_forward():
    # HF's Llama run over the whole prompt at once (its causal mask, its RoPE, its cache of
    # the earlier context), unrounded K/V on both sides
    from transformers.cache_utils import DynamicCache
    cfg = synth.configs.TINY.with_(tied=False)
    T, P, C = 12, 40, 64
    w, kc, vc, toks = _prefill_case(cfg, T, P, C, gain_std=0.2, seed=3)
    m = _hf_llama(cfg, w)
    cache = DynamicCache()
    for l in range(cfg.n_layers):
        cache.update(torch.tensor(oracle.bf16_to_f64(kc[l, 0, :, :P]))[None],
                     torch.tensor(oracle.bf16_to_f64(vc[l, 0, :, :P]))[None], l)
    resid = {}
    hk = m.model.layers[-1].register_forward_hook(
        lambda mod, i, o: resid.__setitem__("x", o[0] if isinstance(o, tuple) else o))
    with torch.no_grad():
        out = m(input_ids=torch.tensor(toks)[None], position_ids=torch.arange(P, P + T)[None],
                past_key_values=cache, use_cache=True, cache_position=torch.arange(P, P + T))
    hk.remove()
    r = oprefill.prefill(cfg, w, toks, P, kc.copy(), vc.copy(), kv_round=False)
    ref_x = resid["x"][0].numpy()
    np.testing.assert_allclose(r["hidden"], ref_x, rtol=0, atol=2e-6 * np.abs(ref_x).max())
    ref_logits = out.logits[0, -1].numpy()
    np.testing.assert_allclose(r["logits"], ref_logits, rtol=0, atol=2e-6 * np.abs(ref_logits).max())


def test_prefill_chunks_compose():
    # a prompt prefilled in two calls (the second continuing at pos0 = T1) equals one call
    cfg = synth.configs.TINY
    w, kc, vc, toks = _prefill_case(cfg, 23, 0, 32, seed=5)
    k1, v1 = kc.copy(), vc.copy()
    r = oprefill.prefill(cfg, w, toks, 0, k1, v1)
    k2, v2 = kc.copy(), vc.copy()
    oprefill.prefill(cfg, w, toks[:9], 0, k2, v2)
    r2 = oprefill.prefill(cfg, w, toks[9:], 9, k2, v2)
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
    np.testing.assert_allclose(r2["hidden"], r["hidden"][9:], rtol=1e-10, atol=1e-12)
    assert r2["next"] == r["next"]
