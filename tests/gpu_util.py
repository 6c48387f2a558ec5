"""Helpers of the GPU tests: move synthetic inputs to the device and run the
megakernel through the C ABI binding.  Expected values always come from the
oracle, never from the GPU path."""
import numpy as np
import torch

import persistent_megakernel_decode_cu_amd as mk
import synth

TOL_HIDDEN_REL = 1e-2   # relative L2 error of the final residual
TOL_LOGIT_ABS = 5e-2    # max |delta logit|


def dev_weights(w):
    return {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in w.items()}


def dev_kv(kc, vc):
    flat = np.concatenate([kc.reshape(-1), vc.reshape(-1)]).view(np.int16)
    return torch.from_numpy(flat).cuda()


def kv_to_host(kv, shape):
    a = kv.cpu().numpy().view(np.uint16)
    n = int(np.prod(shape))
    return a[:n].reshape(shape), a[n:].reshape(shape)


class Runner:
    """One megakernel handle plus device copies of the inputs."""

    def __init__(self, cfg, w, batch, max_ctx, kc, vc, **opt):
        self.cfg = cfg
        self.wd = dev_weights(w)
        self.model = mk.Model(cfg, self.wd)
        opts = dict(debug_timeout_ms=2000)
        opts.update(opt)
        self.opt = mk.options(**opts)
        self.h = mk.mk_build_graph(self.model.desc, batch, max_ctx, self.opt)
        self.wd = None  # the handle holds a packed copy
        self.model = None
        self.kv = dev_kv(kc, vc)
        assert self.kv.numel() * 2 == mk.mk_kv_cache_bytes(self.h)
        self.shape = kc.shape
        self.B = batch
        self.logits = torch.zeros(batch, cfg.vocab, dtype=torch.float32, device="cuda")
        self.graph = mk.parse_export(mk.mk_export_graph(self.h))

    def step(self, tokens, positions, stream=None):
        t = tokens if torch.is_tensor(tokens) else torch.tensor(np.asarray(tokens, np.int32), device="cuda")
        p = positions if torch.is_tensor(positions) else torch.tensor(np.asarray(positions, np.int32), device="cuda")
        s = torch.cuda.current_stream() if stream is None else stream
        mk.mk_decode_step(self.h, t.data_ptr(), p.data_ptr(), self.kv.data_ptr(), self.logits.data_ptr(),
                          s.cuda_stream)
        return t, p

    def check(self):
        torch.cuda.synchronize()
        err = mk.mk_check_device_error(self.h)
        assert err is None, err

    def next_tokens(self):
        out = torch.empty(self.B, dtype=torch.int32, device="cuda")
        return _copy_from_ptr(mk.mk_next_tokens(self.h), out)

    def hidden(self):
        out = torch.empty(self.B, self.cfg.hidden, dtype=torch.float32, device="cuda")
        return _copy_from_ptr(mk.mk_hidden_out(self.h), out)

    def close(self):
        mk.mk_destroy(self.h)
        self.h = None


def _copy_from_ptr(ptr, out):
    """Copy out.numel() elements from the device pointer ptr into `out` (device-to-device)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    torch.cuda.synchronize()
    rc = hip.hipMemcpy(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ptr), out.numel() * out.element_size(), 3)
    assert rc == 0, rc
    return out


def compare_step(cfg, r_oracle, logits_gpu, hidden_gpu, next_gpu):
    """Parity bar of one step: hidden relative error, max |delta logit|, argmax."""
    h_ref = r_oracle["hidden"]
    h = hidden_gpu.astype(np.float64)
    rel = np.linalg.norm(h - h_ref, axis=1) / np.linalg.norm(h_ref, axis=1)
    dlog = np.abs(logits_gpu.astype(np.float64) - r_oracle["logits"]).max()
    return dict(hidden_rel=float(rel.max()), max_dlogit=float(dlog),
                argmax_equal=bool(np.array_equal(next_gpu, r_oracle["next"])))
