"""Python binding of the MI355X persistent decode megakernel (libmk.so).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libmk.so.  The names mirror the C ABI in include/mk.h.  PyTorch is
used by callers for device memory and streams; this module passes raw device
pointers (tensor.data_ptr()) and stream handles (stream.cuda_stream).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MK_LIBRARY: path of another build of the library (a variant built with build.build(out=...)) to load instead
LIB_PATH = os.environ.get("MK_LIBRARY") or os.path.join(_HERE, "libmk.so")
_lib = None

MK_OK, MK_E_INVALID, MK_E_UNSUPPORTED, MK_E_NOMEM, MK_E_HIP, MK_E_NOT_RESIDENT, MK_E_DEVICE, MK_E_NO_DEVICE = range(8)

# opcodes of the interpreter (mirrors csrc/mk_internal.h)
OP_END, OP_QKV, OP_ATTN, OP_OPROJ, OP_GATEUP, OP_DOWN, OP_LMHEAD, OP_ROUTE, OP_EGU, OP_EDOWN = range(10)
# the prompt (prefill) graph's operations
OP_PNORM, OP_PQKV, OP_PATTN, OP_POPROJ, OP_PGU, OP_PDOWN, OP_PLM = range(10, 17)
OP_NAMES = {OP_QKV: "qkv_rope", OP_ATTN: "attention", OP_OPROJ: "oproj_residual", OP_GATEUP: "gateup_silu",
            OP_DOWN: "down_residual", OP_LMHEAD: "lmhead_argmax", OP_ROUTE: "router_topk",
            OP_EGU: "expert_gateup_silu", OP_EDOWN: "expert_down_residual",
            OP_PNORM: "prompt_rmsnorm", OP_PQKV: "prompt_qkv_rope", OP_PATTN: "prompt_attention",
            OP_POPROJ: "prompt_oproj_residual", OP_PGU: "prompt_gateup_silu", OP_PDOWN: "prompt_down_residual",
            OP_PLM: "prompt_lmhead_argmax"}
NONE = 0xFFFFFFFF

_P = ctypes.c_void_p


class MkError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})" if what else status_str(status))


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                                  "router", "exp_gate", "exp_up", "exp_down")]


class ModelDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim",
                                               "vocab", "n_experts", "top_k", "expert_ffn_dim")] + \
               [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("tied_lm_head", ctypes.c_int32),
                ("tok_embed", _P), ("lm_head", _P), ("final_norm", _P), ("layers", ctypes.POINTER(LayerWeights))]


class Options(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("sched", "n_workgroups", "policy", "attn_splits", "debug_timeout_ms",
                                               "debug_drop_signal", "trace", "cooperative", "page_kib", "poison")] + \
               [("reserved", ctypes.c_int32 * 6)]


def options(sched=0, n_workgroups=0, policy=0, attn_splits=0, debug_timeout_ms=0, drop_signal_of_task=None,
            trace=0, cooperative=0, page_kib=0, poison=0):
    """mk_options; drop_signal_of_task: index of a task that skips its signal (tests of the timeout path)."""
    drop = 0 if drop_signal_of_task is None else drop_signal_of_task + 1
    return Options(sched, n_workgroups, policy, attn_splits, debug_timeout_ms, drop, trace, cooperative, page_kib,
                   poison)


# task record (48 bytes, mirrors mk::Task)
TASK_DTYPE = np.dtype([("op", "u1"), ("wait_nsub", "u1"), ("sig_nsub", "u1"), ("flags", "u1"), ("layer", "<u2"),
                       ("part", "<u2"), ("row0", "<u4"), ("nrows", "<u4"), ("wait_ev", "<u4"),
                       ("wait_target", "<u4"), ("sig_ev", "<u4"), ("wbytes", "<u4"), ("wofs", "<u8"),
                       ("seq", "<u4"), ("id", "<u4")])
assert TASK_DTYPE.itemsize == 48

HEADER_FIELDS = ["magic", "version", "n_tasks", "n_events", "W", "sched", "L", "h", "nq", "nkv", "d", "f", "V", "B",
                 "C", "grp", "qkv_pairs", "attn_splits", "o_rows", "g_rows", "kd", "d_rows", "lm_rows",
                 "record_bytes", "E", "topk", "fe", "r_gu", "r_dn"]
HEADER_BYTES = 4 * (len(HEADER_FIELDS) + 2)


def load():
    """Load libmk.so; raises if the HIP library has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with persistent_megakernel_decode_cu_amd/build.py "
                           "(the decode path has no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mk_status_str.argtypes = [ctypes.c_int]
    lib.mk_status_str.restype = ctypes.c_char_p
    lib.mk_build_graph.argtypes = [ctypes.POINTER(ModelDesc), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(Options), ctypes.POINTER(_P)]
    lib.mk_build_graph.restype = ctypes.c_int
    lib.mk_plan_graph.argtypes = [ctypes.POINTER(ModelDesc), ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(Options),
                                  ctypes.c_int32, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
    lib.mk_plan_graph.restype = ctypes.c_int
    if hasattr(lib, "mk_prefill"):  # (older variant builds loaded through MK_LIBRARY lack it)
        lib.mk_build_prefill.argtypes = [ctypes.POINTER(ModelDesc), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(Options), ctypes.POINTER(_P)]
        lib.mk_build_prefill.restype = ctypes.c_int
        lib.mk_plan_prefill.argtypes = [ctypes.POINTER(ModelDesc), ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(Options), ctypes.c_int32, _P, ctypes.c_size_t,
                                        ctypes.POINTER(ctypes.c_size_t)]
        lib.mk_plan_prefill.restype = ctypes.c_int
        lib.mk_prefill.argtypes = [_P, _P, ctypes.c_int32, _P, _P, _P]
        lib.mk_prefill.restype = ctypes.c_int
    lib.mk_kv_cache_bytes.argtypes = [_P]
    lib.mk_kv_cache_bytes.restype = ctypes.c_size_t
    lib.mk_decode_step.argtypes = [_P, _P, _P, _P, _P, _P]
    lib.mk_decode_step.restype = ctypes.c_int
    if hasattr(lib, "mk_decode_step_noalloc"):  # (older variant builds loaded through MK_LIBRARY lack it)
        lib.mk_decode_step_noalloc.argtypes = [_P, _P, _P, _P, _P, _P]
        lib.mk_decode_step_noalloc.restype = ctypes.c_int
    for n in ("mk_next_tokens", "mk_hidden_out", "mk_expert_ids"):
        getattr(lib, n).argtypes = [_P]
        getattr(lib, n).restype = _P
    lib.mk_check_device_error.argtypes = [_P, ctypes.c_char_p, ctypes.c_size_t]
    lib.mk_check_device_error.restype = ctypes.c_int
    lib.mk_export_graph.argtypes = [_P, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
    lib.mk_export_graph.restype = ctypes.c_int
    lib.mk_read_counters.argtypes = [_P, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint32)]
    lib.mk_read_counters.restype = ctypes.c_int
    lib.mk_read_task_counts.argtypes = [_P, _P, ctypes.c_size_t]
    lib.mk_read_task_counts.restype = ctypes.c_int
    lib.mk_read_trace.argtypes = [_P, _P, ctypes.c_size_t]
    lib.mk_read_trace.restype = ctypes.c_int
    lib.mk_destroy.argtypes = [_P]
    lib.mk_destroy.restype = None
    lib.mkb_create.argtypes = [ctypes.POINTER(ModelDesc), ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_P)]
    lib.mkb_create.restype = ctypes.c_int
    lib.mkb_decode_step.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_int32]
    lib.mkb_decode_step.restype = ctypes.c_int
    for n in ("mkb_next_tokens", "mkb_hidden_out"):
        getattr(lib, n).argtypes = [_P]
        getattr(lib, n).restype = _P
    lib.mkb_launches_per_step.argtypes = [_P]
    lib.mkb_launches_per_step.restype = ctypes.c_int32
    lib.mkb_destroy.argtypes = [_P]
    lib.mkb_destroy.restype = None
    _F = ctypes.POINTER(ctypes.c_float)
    _I = ctypes.POINTER(ctypes.c_int32)
    lib.mkm_launch_latency.argtypes = [ctypes.c_int32, _F, _F]
    lib.mkm_pingpong.argtypes = [ctypes.c_int32, ctypes.c_int32, _F, _I, _I]
    lib.mkm_barrier.argtypes = [ctypes.c_int32, _F]
    lib.mkm_lds_fill.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, _F]
    lib.mkm_stream_read.argtypes = [ctypes.c_uint64, _F]
    for n in ("mkm_launch_latency", "mkm_pingpong", "mkm_barrier", "mkm_lds_fill", "mkm_stream_read"):
        getattr(lib, n).restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(s):
    try:
        return load().mk_status_str(int(s)).decode()
    except RuntimeError:
        return f"status {s}"


def _check(st, what):
    if st != MK_OK:
        raise MkError(st, what)


# ---- entry points (same names as the C ABI) -------------------------------------

def mk_build_graph(desc, batch, max_ctx, opt=None):
    h = _P()
    st = load().mk_build_graph(ctypes.byref(desc), batch, max_ctx, ctypes.byref(opt) if opt is not None else None,
                               ctypes.byref(h))
    _check(st, "mk_build_graph")
    return h


def mk_plan_graph(desc, batch, max_ctx, opt, n_workgroups):
    lib = load()
    need = ctypes.c_size_t(0)
    o = ctypes.byref(opt) if opt is not None else None
    st = lib.mk_plan_graph(ctypes.byref(desc), batch, max_ctx, o, n_workgroups, None, 0, ctypes.byref(need))
    if st not in (MK_OK, MK_E_INVALID) or need.value == 0:
        _check(st, "mk_plan_graph")
    buf = ctypes.create_string_buffer(need.value)
    _check(lib.mk_plan_graph(ctypes.byref(desc), batch, max_ctx, o, n_workgroups, buf, need.value,
                             ctypes.byref(need)), "mk_plan_graph")
    return buf.raw


def mk_build_prefill(desc, n_tokens, max_ctx, opt=None):
    """A prompt (prefill) handle for prompts of n_tokens tokens of one sequence."""
    h = _P()
    st = load().mk_build_prefill(ctypes.byref(desc), n_tokens, max_ctx,
                                 ctypes.byref(opt) if opt is not None else None, ctypes.byref(h))
    _check(st, "mk_build_prefill")
    return h


def mk_plan_prefill(desc, n_tokens, max_ctx, opt, n_workgroups):
    lib = load()
    need = ctypes.c_size_t(0)
    o = ctypes.byref(opt) if opt is not None else None
    st = lib.mk_plan_prefill(ctypes.byref(desc), n_tokens, max_ctx, o, n_workgroups, None, 0, ctypes.byref(need))
    if st not in (MK_OK, MK_E_INVALID) or need.value == 0:
        _check(st, "mk_plan_prefill")
    buf = ctypes.create_string_buffer(need.value)
    _check(lib.mk_plan_prefill(ctypes.byref(desc), n_tokens, max_ctx, o, n_workgroups, buf, need.value,
                               ctypes.byref(need)), "mk_plan_prefill")
    return buf.raw


def mk_prefill(h, tokens_ptr, pos0, kv_ptr, logits_ptr, stream_ptr):
    _check(load().mk_prefill(h, tokens_ptr, pos0, kv_ptr, logits_ptr, stream_ptr), "mk_prefill")


def mk_kv_cache_bytes(h):
    return int(load().mk_kv_cache_bytes(h))


def mk_decode_step(h, tokens_ptr, positions_ptr, kv_ptr, logits_ptr, stream_ptr):
    _check(load().mk_decode_step(h, tokens_ptr, positions_ptr, kv_ptr, logits_ptr, stream_ptr), "mk_decode_step")


def mk_decode_step_noalloc(h, tokens_ptr, positions_ptr, kv_ptr, logits_ptr, stream_ptr):
    """The allocation-free step (scratch in the library's static per-GPU array)."""
    _check(load().mk_decode_step_noalloc(h, tokens_ptr, positions_ptr, kv_ptr, logits_ptr, stream_ptr),
           "mk_decode_step_noalloc")


def mk_next_tokens(h):
    return load().mk_next_tokens(h)


def mk_hidden_out(h):
    return load().mk_hidden_out(h)


def mk_expert_ids(h):
    return load().mk_expert_ids(h)


def mk_check_device_error(h):
    """Returns None if no device error is recorded, else the message (the handle is re-armed)."""
    buf = ctypes.create_string_buffer(512)
    st = load().mk_check_device_error(h, buf, 512)
    if st == MK_OK:
        return None
    if st == MK_E_DEVICE:
        return buf.value.decode()
    raise MkError(st, "mk_check_device_error")


def mk_export_graph(h):
    lib = load()
    need = ctypes.c_size_t(0)
    lib.mk_export_graph(h, None, 0, ctypes.byref(need))
    buf = ctypes.create_string_buffer(need.value)
    _check(lib.mk_export_graph(h, buf, need.value, ctypes.byref(need)), "mk_export_graph")
    return buf.raw


def mk_read_counters(h, n_events):
    out = np.zeros(n_events, dtype=np.uint32)
    ep = ctypes.c_uint32(0)
    _check(load().mk_read_counters(h, out.ctypes.data, n_events, ctypes.byref(ep)), "mk_read_counters")
    return out, int(ep.value)


def mk_read_task_counts(h, n_tasks):
    out = np.zeros(n_tasks, dtype=np.uint32)
    _check(load().mk_read_task_counts(h, out.ctypes.data, n_tasks), "mk_read_task_counts")
    return out


TRACE_WORDS = 16


def mk_read_trace(h, n_tasks):
    out = np.zeros((n_tasks, TRACE_WORDS), dtype=np.uint64)
    _check(load().mk_read_trace(h, out.ctypes.data, out.size), "mk_read_trace")
    return out


def mk_destroy(h):
    if h:
        load().mk_destroy(h)


# ---- one-kernel-per-op baseline -------------------------------------------------

def mkb_create(desc, batch, max_ctx):
    h = _P()
    _check(load().mkb_create(ctypes.byref(desc), batch, max_ctx, ctypes.byref(h)), "mkb_create")
    return h


def mkb_decode_step(h, tokens_ptr, positions_ptr, kv_ptr, logits_ptr, stream_ptr, advance=0):
    _check(load().mkb_decode_step(h, tokens_ptr, positions_ptr, kv_ptr, logits_ptr, stream_ptr, advance),
           "mkb_decode_step")


def mkb_next_tokens(h):
    return load().mkb_next_tokens(h)


def mkb_hidden_out(h):
    return load().mkb_hidden_out(h)


def mkb_launches_per_step(h):
    return int(load().mkb_launches_per_step(h))


def mkb_destroy(h):
    if h:
        load().mkb_destroy(h)


# ---- export image ------------------------------------------------------------------

def parse_export(buf):
    """Split an export image into its header, task records, event targets,
    sub-counter counts, static queues and dynamic order."""
    hdr_words = np.frombuffer(buf, dtype="<i4", count=len(HEADER_FIELDS))
    hdr = {k: int(v) for k, v in zip(HEADER_FIELDS, hdr_words)}
    hdr["magic"] &= 0xFFFFFFFF
    assert hdr["magic"] == 0x31474B4D, "not a task-graph export"
    off = HEADER_BYTES
    n, e, W = hdr["n_tasks"], hdr["n_events"], hdr["W"]
    tasks = np.frombuffer(buf, dtype=TASK_DTYPE, count=n, offset=off)
    off += n * TASK_DTYPE.itemsize

    def take(cnt):
        nonlocal off
        a = np.frombuffer(buf, dtype="<u4", count=cnt, offset=off)
        off += 4 * cnt
        return a

    target = take(e)
    nsub = take(e)
    queue_off = take(W + 1)
    queue = take(int(queue_off[-1]))
    order = take(n)
    return dict(header=hdr, tasks=tasks, target=target, nsub=nsub, queue_off=queue_off, queue=queue, order=order)


# ---- convenience: a model held in torch device tensors -------------------------------

class Model:
    """Owns the ctypes description of a model whose weights live in torch device tensors.

    weights: dict name -> torch tensor (int16/uint16 bf16 bits or bfloat16) on the GPU, with the
    names of synth.make_weights.  The tensors must stay alive until mk_build_graph returns
    (the handle keeps its own packed copy).
    """

    def __init__(self, cfg, weights):
        self.cfg = cfg
        self._keep = weights
        L = cfg.n_layers
        self.layers = (LayerWeights * max(L, 1))()
        for l in range(L):
            p = f"l{l}."
            for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                      "router", "exp_gate", "exp_up", "exp_down"):
                t = weights.get(p + n)
                if t is not None:
                    setattr(self.layers[l], n, t.data_ptr())
        self.desc = ModelDesc(L, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn, cfg.vocab, cfg.n_experts,
                              cfg.top_k, cfg.expert_ffn, cfg.eps, cfg.rope_theta, 1 if cfg.tied else 0,
                              weights["tok_embed"].data_ptr(),
                              0 if cfg.tied else weights["lm_head"].data_ptr(),
                              weights["final_norm"].data_ptr(), self.layers)


# ---- measurement microbenchmarks (synchronous; each allocates and frees its own buffers) ----

def mkm_launch_latency(n=2000):
    """(us per empty kernel launched on a stream, us per kernel replayed from a HIP graph)."""
    a, b = ctypes.c_float(), ctypes.c_float()
    _check(load().mkm_launch_latency(n, ctypes.byref(a), ctypes.byref(b)), "mkm_launch_latency")
    return a.value, b.value


def mkm_pingpong(rounds=20000, same_xcd=False):
    """(ns per one-way hop between two workgroups through device memory, XCD of each workgroup)."""
    ns, xa, xb = ctypes.c_float(), ctypes.c_int32(), ctypes.c_int32()
    _check(load().mkm_pingpong(rounds, 1 if same_xcd else 0, ctypes.byref(ns), ctypes.byref(xa), ctypes.byref(xb)),
           "mkm_pingpong")
    return ns.value, xa.value, xb.value


def mkm_barrier(n=100000):
    """ns per workgroup barrier of 384 threads."""
    ns = ctypes.c_float()
    _check(load().mkm_barrier(n, ctypes.byref(ns)), "mkm_barrier")
    return ns.value


def mkm_lds_fill(bytes_per_wg=8 << 20, n_wg=256, depth=8):
    """GB/s of n_wg workgroups streaming bytes_per_wg each from device memory straight into LDS."""
    g = ctypes.c_float()
    _check(load().mkm_lds_fill(bytes_per_wg, n_wg, depth, ctypes.byref(g)), "mkm_lds_fill")
    return g.value


def mkm_stream_read(nbytes=4 << 30):
    """GB/s of a plain streaming read of nbytes of device memory."""
    g = ctypes.c_float()
    _check(load().mkm_stream_read(nbytes, ctypes.byref(g)), "mkm_stream_read")
    return g.value
