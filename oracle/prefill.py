"""ORACLE — test infrastructure only (tests, the smoke check, the CPU-baseline leg
of the benchmark).  The GPU path never imports this module.

Causal prefill of one prompt: the prompt's T tokens at positions pos0 .. pos0+T-1
of one sequence go through the decoder together, each attending to the cache
slots 0 .. its own position.  The knowledge-base digest "megakernel boundary
selection" defines prefill, in its list of first-used concepts, as the pass over
the whole input context that runs once per request, and reports (Figure 4,
Table IV) that its planner gives Llama-1B two megakernels, the first-token
latency counting as megakernel-stable.  The pages do
not spell out prefill arithmetic; the plain reading taken here is that prefill
of T tokens equals T decode steps over the same tokens, with the same readings
as oracle.c (the decode-step definition), written in matrix form:

    X = E[tokens]                                       (T x h, one row per token)
    per layer:  Xn = rmsnorm(X, g1) row by row
                Q, K, V = Xn Wq^T, Xn Wk^T, Xn Wv^T     (rotated by RoPE at each row's position)
                K, V rows stored into the bf16 cache slots pos0 .. pos0+T-1
                A[t] = softmax(Q_i[t] K_g^T / sqrt(d)) V_g over cache slots 0 .. pos0+t
                X = X + A Wo^T
                Xn = rmsnorm(X, g2);  X = X + (silu(Xn Wg^T) * (Xn Wu^T)) Wd^T
    hidden = X;  logits = Wlm rmsnorm(X[T-1], gf);  next = argmax(logits)

Precision as oracle.c: activations, products and softmax sums in double (numpy
float64; its matrix products sum in their own order, which changes results by
rounding only), a cache write rounds double -> float -> bf16 to nearest even,
and the argmax is taken over logits rounded to float, lowest index on ties.
Every cache slot read in attention (the prompt's own included) is the stored
bf16 value, as the decode step reads the current token's K/V as stored.

Pinned in tests/test_oracle.py against T sequential calls of oracle.decode_step
(the C definition, pinned on its own), so a mistake in the matrix form (a
transposed weight, an off-by-one causal mask, a wrong RoPE pair) fails there.
Dense models only.
"""
import numpy as np

from . import bf16_to_f64


def _f64_to_bf16_bits(x):
    """double -> float -> bf16, round to nearest even (finite inputs)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _rmsnorm_rows(X, g_bits, eps):
    g = bf16_to_f64(g_bits)
    ms = np.mean(X * X, axis=1, keepdims=True)
    return X / np.sqrt(ms + eps) * g


def _rope_rows(M, n_heads, d, positions, theta):
    """RoPE on every row of M (rows = tokens, columns = n_heads x d): pairs (j, j + d/2) of each head
    turned by the angle position * theta^(-2j/d)."""
    half = d // 2
    j = np.arange(half, dtype=np.float64)
    ang = positions.astype(np.float64)[:, None] * np.power(float(theta), -2.0 * j / d)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    out = M.reshape(M.shape[0], n_heads, d).copy()
    x0 = out[:, :, :half].copy()
    x1 = out[:, :, half:].copy()
    out[:, :, :half] = x0 * c[:, None, :] - x1 * s[:, None, :]
    out[:, :, half:] = x0 * s[:, None, :] + x1 * c[:, None, :]
    return out.reshape(M.shape)


def _w(w, name):
    return bf16_to_f64(w[name])


def prefill(cfg, w, tokens, pos0, k_cache, v_cache, kv_round=True):
    """Causal prefill of one sequence's prompt; writes cache slots pos0 .. pos0 + T - 1 in place.

    w: dict from synth.make_weights (dense); tokens: T token ids; k_cache, v_cache: uint16
    [L][1][n_kv][C][d] whose slots 0 .. pos0 - 1 hold the earlier context.  kv_round: the
    prompt's own K/V enter attention as stored (bf16, the definition) or, when False,
    unrounded (only to compare with double-precision references that keep them so).
    Returns dict(hidden [T][h] (final residual of every prompt token), logits [V] of the last
    token, next (int), layers [L][T][h] residual after each layer).
    """
    assert not cfg.n_experts, "the prefill definition covers dense models"
    tokens = np.asarray(tokens, dtype=np.int64)
    T = tokens.size
    L, h, nq, nkv, d = cfg.n_layers, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim
    grp = nq // nkv
    C = k_cache.shape[3]
    assert k_cache.shape == (L, 1, nkv, C, d) and v_cache.shape == k_cache.shape
    assert T >= 1 and pos0 >= 0 and pos0 + T <= C
    pos = pos0 + np.arange(T)
    n_ctx = pos0 + T
    X = bf16_to_f64(w["tok_embed"][tokens])
    layers = np.empty((L, T, h))
    scale = 1.0 / np.sqrt(d)
    for l in range(L):
        p = f"l{l}."
        Xn = _rmsnorm_rows(X, w[p + "attn_norm"], cfg.eps)
        Q = _rope_rows(Xn @ _w(w, p + "wq").T, nq, d, pos, cfg.rope_theta)
        K = _rope_rows(Xn @ _w(w, p + "wk").T, nkv, d, pos, cfg.rope_theta)
        V = Xn @ _w(w, p + "wv").T
        for g in range(nkv):
            k_cache[l, 0, g, pos0:n_ctx, :] = _f64_to_bf16_bits(K[:, g * d:(g + 1) * d])
            v_cache[l, 0, g, pos0:n_ctx, :] = _f64_to_bf16_bits(V[:, g * d:(g + 1) * d])
        A = np.empty((T, nq * d))
        Kc = bf16_to_f64(k_cache[l, 0, :, :n_ctx, :])
        Vc = bf16_to_f64(v_cache[l, 0, :, :n_ctx, :])
        if not kv_round:
            for g in range(nkv):
                Kc[g, pos0:] = K[:, g * d:(g + 1) * d]
                Vc[g, pos0:] = V[:, g * d:(g + 1) * d]
        # token t (position pos0 + t) sees slots 0 .. pos0 + t
        mask = np.arange(n_ctx)[None, :] > pos[:, None]
        for i in range(nq):
            g = i // grp
            Kg, Vg = Kc[g], Vc[g]
            s = Q[:, i * d:(i + 1) * d] @ Kg.T * scale
            s[mask] = -np.inf
            s = np.exp(s - s.max(axis=1, keepdims=True))
            A[:, i * d:(i + 1) * d] = (s / s.sum(axis=1, keepdims=True)) @ Vg
        X = X + A @ _w(w, p + "wo").T
        Xn = _rmsnorm_rows(X, w[p + "ffn_norm"], cfg.eps)
        G = Xn @ _w(w, p + "w_gate").T
        U = Xn @ _w(w, p + "w_up").T
        X = X + (G / (1.0 + np.exp(-G)) * U) @ _w(w, p + "w_down").T
        layers[l] = X
    lm = w["tok_embed"] if cfg.tied else w["lm_head"]
    xl = _rmsnorm_rows(X[-1:], w["final_norm"], cfg.eps)[0]
    logits = np.empty(cfg.vocab)
    step = 16384  # the LM head in row blocks (its double copy would be large at real vocabularies)
    for r0 in range(0, cfg.vocab, step):
        logits[r0:r0 + step] = bf16_to_f64(lm[r0:r0 + step]) @ xl
    f = logits.astype(np.float32)
    nxt = int(np.argmax(f))  # numpy's argmax returns the first (lowest-index) maximum
    return dict(hidden=X, logits=logits, next=nxt, layers=layers)
