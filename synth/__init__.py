"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Holds no decode arithmetic: it only names tensors, fixes their shapes and
draws their values (bf16 bits from N(0, std), integers from U[lo, hi]) with a
counter-based generator (see synth.c), so the same (seed, name, index) gives
the same value on every machine and thread count.
"""
import ctypes
import os
import subprocess

import numpy as np

from .configs import ModelConfig, CONFIGS  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED_WEIGHTS = 1
SEED_KV = 2
SEED_TOKENS = 3


def build():
    """Compile libsynth.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_char_p, ctypes.c_double, ctypes.c_uint64,
                                          ctypes.c_void_p, ctypes.c_int64]
        lib.synth_uniform_int.argtypes = [ctypes.c_uint64, ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64]
        lib.synth_normal_at.argtypes = [ctypes.c_uint64, ctypes.c_char_p, ctypes.c_uint64]
        lib.synth_normal_at.restype = ctypes.c_double
        lib.synth_fnv_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        lib.synth_fnv_bytes.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def normal_bf16(seed, name, std, shape, offset=0, out=None):
    """bf16 bits (uint16 array of `shape`) of std * N(0,1), element i = stream index offset+i."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_bf16(seed, name.encode(), float(std), offset, out.ctypes.data, n)
    return out


def normal_at(seed, name, i):
    """The unrounded normal deviate number i of stream (seed, name)."""
    return _load().synth_normal_at(seed, name.encode(), i)


def uniform_int(seed, name, lo, hi, n, offset=0):
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_int(seed, name.encode(), int(lo), int(hi), offset, out.ctypes.data, n)
    return out


def fnv(arr):
    arr = np.ascontiguousarray(arr)
    return int(_load().synth_fnv_bytes(arr.ctypes.data, arr.nbytes))


BF16_ONE = 0x3F80


def _gain(cfg, seed, name, gain_std):
    if gain_std == 0.0:
        return np.full(cfg.hidden, BF16_ONE, dtype=np.uint16)
    # 1 + gain_std * N(0,1), then bf16: draw gain_std*N as bf16 and add 1 in float32 before rounding
    dev = normal_bf16(seed, name, gain_std, (cfg.hidden,))
    f = (dev.astype(np.uint32) << 16).view(np.float32) + np.float32(1.0)
    u = f.view(np.uint32)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def make_weights(cfg, seed=SEED_WEIGHTS, std=0.02, gain_std=0.0):
    """All weights of `cfg` as a dict of bf16-bit arrays in [out][in] layout.

    Keys: tok_embed [V][h], lm_head [V][h] (absent when tied), final_norm [h],
    and per layer l: 'l{l}.attn_norm', '.wq' [nq*d][h], '.wk', '.wv' [nkv*d][h],
    '.wo' [h][nq*d], '.ffn_norm', and either '.w_gate', '.w_up' [f][h], '.w_down' [h][f]
    or (MoE) '.router' [E][h], '.exp_gate', '.exp_up' [E][fe][h], '.exp_down' [E][h][fe].
    """
    h, d = cfg.hidden, cfg.head_dim
    w = {"tok_embed": normal_bf16(seed, "tok_embed", std, (cfg.vocab, h))}
    if not cfg.tied:
        w["lm_head"] = normal_bf16(seed, "lm_head", std, (cfg.vocab, h))
    w["final_norm"] = _gain(cfg, seed, "final_norm", gain_std)
    for l in range(cfg.n_layers):
        p = f"l{l}."
        w[p + "attn_norm"] = _gain(cfg, seed, p + "attn_norm", gain_std)
        w[p + "ffn_norm"] = _gain(cfg, seed, p + "ffn_norm", gain_std)
        w[p + "wq"] = normal_bf16(seed, p + "wq", std, (cfg.n_q * d, h))
        w[p + "wk"] = normal_bf16(seed, p + "wk", std, (cfg.n_kv * d, h))
        w[p + "wv"] = normal_bf16(seed, p + "wv", std, (cfg.n_kv * d, h))
        w[p + "wo"] = normal_bf16(seed, p + "wo", std, (h, cfg.n_q * d))
        if cfg.n_experts == 0:
            w[p + "w_gate"] = normal_bf16(seed, p + "w_gate", std, (cfg.ffn, h))
            w[p + "w_up"] = normal_bf16(seed, p + "w_up", std, (cfg.ffn, h))
            w[p + "w_down"] = normal_bf16(seed, p + "w_down", std, (h, cfg.ffn))
        else:
            E, fe = cfg.n_experts, cfg.expert_ffn
            w[p + "router"] = normal_bf16(seed, p + "router", std, (E, h))
            w[p + "exp_gate"] = normal_bf16(seed, p + "exp_gate", std, (E, fe, h))
            w[p + "exp_up"] = normal_bf16(seed, p + "exp_up", std, (E, fe, h))
            w[p + "exp_down"] = normal_bf16(seed, p + "exp_down", std, (E, h, fe))
    return w


def make_kv(cfg, batch, max_ctx, seed=SEED_KV):
    """bf16 K and V caches [L][B][n_kv][max_ctx][d], every slot N(0,1).

    Slots below each sequence's position are the prefilled context; slots at or
    above it hold values the decode step must never read before writing them.
    """
    shape = (cfg.n_layers, batch, cfg.n_kv, max_ctx, cfg.head_dim)
    return normal_bf16(seed, "kv.k", 1.0, shape), normal_bf16(seed, "kv.v", 1.0, shape)


def make_tokens(cfg, batch, seed=SEED_TOKENS):
    return uniform_int(seed, "tokens", 0, cfg.vocab - 1, batch)


def make_prompt(cfg, n, seed=SEED_TOKENS):
    """n prompt token ids, uniform over the vocabulary (a stream of their own)."""
    return uniform_int(seed, "prompt", 0, cfg.vocab - 1, n)


def make_positions(batch, lo, hi, seed=SEED_TOKENS):
    """Per-sequence context lengths, uniform in [lo, hi]."""
    if lo == hi:
        return np.full(batch, lo, dtype=np.int32)
    return uniform_int(seed, "positions", lo, hi, batch)
