"""ORACLE — test infrastructure only (tests, the smoke check, the CPU-baseline leg
of the benchmark).  The GPU path never imports this package.

Python front end of oracle.c: a plain, sequential double-precision evaluation
of one Llama-style decode step, plus its building blocks for the pin tests.
See oracle.c for the definition and the readings it takes where the pages are
silent.  `taskgraph.py` beside it is the independent definition of the task
graph and event counters.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "hidden", "n_q", "n_kv", "head_dim", "ffn", "vocab",
                                               "n_experts", "top_k", "expert_ffn")] + \
               [("eps", ctypes.c_double), ("theta", ctypes.c_double)]


class _Layer(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                                  "router", "exp_gate", "exp_up", "exp_down")]


def build():
    """Compile liboracle.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = ctypes.c_double
        lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_rmsnorm.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_double, _P]
        lib.orc_gemv.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, _P]
        lib.orc_rope.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
        lib.orc_attention_head.argtypes = [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
        lib.orc_argmax_f32.argtypes = [_P, ctypes.c_int32]
        lib.orc_argmax_f32.restype = ctypes.c_int32
        lib.orc_topk_softmax.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, _P]
        lib.orc_decode_step.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Layer), _P, _P, _P, ctypes.c_int32,
                                        _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P]
        lib.orc_decode_step.restype = ctypes.c_int32
        _lib = lib
    return _lib


def _ptr(a, dtype):
    assert a.dtype == dtype and a.flags.c_contiguous, (a.dtype, dtype)
    return a.ctypes.data


# ---- building blocks --------------------------------------------------------

def bf16_to_f64(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    return _load().orc_f64_to_bf16(float(x))


def silu(z):
    return _load().orc_silu(float(z))


def rmsnorm(x, g_bits, eps):
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    out = np.empty_like(x)
    _load().orc_rmsnorm(_ptr(x, np.float64), _ptr(g, np.uint16), x.size, eps, out.ctypes.data)
    return out


def gemv(W_bits, x):
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(W.shape[0], dtype=np.float64)
    _load().orc_gemv(_ptr(W, np.uint16), W.shape[0], W.shape[1], _ptr(x, np.float64), y.ctypes.data)
    return y


def rope(v, n_heads, d, pos, theta):
    v = np.array(v, dtype=np.float64, copy=True).reshape(-1)
    _load().orc_rope(v.ctypes.data, n_heads, d, pos, theta)
    return v


def attention_head(q, K_bits, V_bits, cur_k=None, cur_v=None):
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K_bits, dtype=np.uint16)
    V = np.ascontiguousarray(V_bits, dtype=np.uint16)
    n_pos, d = K.shape
    ck = None if cur_k is None else np.ascontiguousarray(cur_k, dtype=np.float64)
    cv = None if cur_v is None else np.ascontiguousarray(cur_v, dtype=np.float64)
    out = np.empty(d, dtype=np.float64)
    _load().orc_attention_head(q.ctypes.data, K.ctypes.data, V.ctypes.data, d, n_pos,
                               None if ck is None else ck.ctypes.data, None if cv is None else cv.ctypes.data,
                               out.ctypes.data)
    return out


def argmax_f32(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    return int(_load().orc_argmax_f32(v.ctypes.data, v.size))


def topk_softmax(logits, k):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    _load().orc_topk_softmax(logits.ctypes.data, logits.size, k, ids.ctypes.data, w.ctypes.data)
    return ids, w


# ---- decode step ------------------------------------------------------------

def _cfg_struct(cfg):
    return _Cfg(cfg.n_layers, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn, cfg.vocab,
                cfg.n_experts, cfg.top_k, cfg.expert_ffn, cfg.eps, cfg.rope_theta)


def decode_step(cfg, w, tokens, positions, k_cache, v_cache, kv_round=True, want_layers=False):
    """One decode step for every sequence of the batch; updates k_cache/v_cache in place.

    w: dict from synth.make_weights; k_cache, v_cache: uint16 [L][B][n_kv][C][d].
    Returns dict(hidden [B][h], logits [B][V] (float64), next [B] int32,
                 layers [L][B][h] or None, experts [L][B][top_k] or None,
                 router [L][B][n_experts] router logits or None).
    """
    lib = _load()
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    B = tokens.size
    L = cfg.n_layers
    assert k_cache.shape == (L, B, cfg.n_kv, k_cache.shape[3], cfg.head_dim) and v_cache.shape == k_cache.shape
    C = k_cache.shape[3]
    layers = (_Layer * L)()
    keep = []
    for l in range(L):
        p = f"l{l}."
        names = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                 "router", "exp_gate", "exp_up", "exp_down"]
        for n in names:
            a = w.get(p + n)
            if a is not None:
                keep.append(a)
                setattr(layers[l], n, _ptr(a, np.uint16))
    cs = _cfg_struct(cfg)
    lm = w["tok_embed"] if cfg.tied else w["lm_head"]
    hidden = np.empty((B, cfg.hidden), dtype=np.float64)
    logits = np.empty((B, cfg.vocab), dtype=np.float64)
    nxt = np.empty(B, dtype=np.int32)
    lay = np.empty((L, B, cfg.hidden), dtype=np.float64) if want_layers else None
    exp = np.empty((L, B, cfg.top_k), dtype=np.int32) if cfg.n_experts else None
    rl = np.empty((L, B, cfg.n_experts), dtype=np.float64) if cfg.n_experts else None
    rc = lib.orc_decode_step(ctypes.byref(cs), layers, _ptr(w["tok_embed"], np.uint16), _ptr(lm, np.uint16),
                             _ptr(w["final_norm"], np.uint16), B, tokens.ctypes.data, positions.ctypes.data,
                             _ptr(k_cache, np.uint16), _ptr(v_cache, np.uint16), C, 1 if kv_round else 0,
                             hidden.ctypes.data, logits.ctypes.data, nxt.ctypes.data,
                             None if lay is None else lay.ctypes.data, None if exp is None else exp.ctypes.data,
                             None if rl is None else rl.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle decode_step rejected its input (code {rc})")
    return dict(hidden=hidden, logits=logits, next=nxt, layers=lay, experts=exp, router=rl)


def top2_gap(logits_row):
    """Gap between the largest and second-largest float-rounded logit."""
    f = np.asarray(logits_row, dtype=np.float64).astype(np.float32)
    part = np.partition(f, -2)[-2:]
    return float(part[1] - part[0])


def greedy(cfg, w, tokens, positions, k_cache, v_cache, steps, keep_logits=False):
    """Free-running greedy decode for `steps` steps from (tokens, positions).

    Returns dict(tokens [steps][B] (the token chosen at each step), gaps [steps][B],
    hidden (last step), logits list (if keep_logits)).
    """
    toks = np.array(tokens, dtype=np.int32)
    pos = np.array(positions, dtype=np.int32)
    out_t, gaps, lg = [], [], []
    r = None
    for _ in range(steps):
        r = decode_step(cfg, w, toks, pos, k_cache, v_cache)
        out_t.append(r["next"].copy())
        gaps.append([top2_gap(r["logits"][b]) for b in range(toks.size)])
        if keep_logits:
            lg.append(r["logits"])
        toks = r["next"].copy()
        pos = pos + 1
    return dict(tokens=np.array(out_t), gaps=np.array(gaps), hidden=r["hidden"], logits=lg)
