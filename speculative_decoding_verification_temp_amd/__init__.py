"""Python binding of libspecverify (batched speculative-decoding verification
on MI355X).

Argument marshalling only: every step of verification runs in the HIP
kernels of the shared library. torch provides device memory and the stream
the work is ordered on. torch is imported before the library is loaded so
that the library binds to the same HIP runtime instance as torch.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB as LIB_PATH

SV_DTYPE_F32, SV_DTYPE_BF16 = 0, 1
MODES = {"stochastic": 0, "greedy": 1, "margin": 2}
SV_OK, SV_EINVAL, SV_EUNSUPPORTED, SV_ENOMEM, SV_EHIP = 0, -1, -2, -3, -4
_ERRNAMES = {-1: "SV_EINVAL", -2: "SV_EUNSUPPORTED", -3: "SV_ENOMEM", -4: "SV_EHIP"}

EXPORTED = (
    "spec_verify_init", "spec_verify", "spec_verify_destroy", "spec_verify_set_aux",
    "spec_verify_set_stops", "spec_verify_set_truncation", "spec_verify_set_policy",
    "spec_verify_set_residual", "spec_verify_set_walk_order",
    "spec_verify_get_ema", "spec_verify_set_ema", "spec_verify_reset_ema",
    "spec_verify_get_stats", "spec_verify_profile", "spec_verify_profile_read",
    "spec_verify_last_error", "spec_verify_version", "spec_verify_read_probe",
    "spec_verify_noalloc",
)


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERRNAMES.get(code, code)}: {msg}")
        self.code = code


class Stats(ctypes.Structure):
    _fields_ = [("sequences", ctypes.c_uint64), ("invalid", ctypes.c_uint64),
                ("zero_q_accepts", ctypes.c_uint64), ("z0_fallbacks", ctypes.c_uint64),
                ("calls", ctypes.c_uint64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing; build it first (python -m "
            "speculative_decoding_verification_temp_amd.build)")
    L = ctypes.CDLL(path)
    vp, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
    L.spec_verify_init.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, f64]
    L.spec_verify.argtypes = [vp, i32, vp, vp, vp, vp, f32, i32, f32, vp, vp, vp, vp]
    L.spec_verify_destroy.argtypes = [vp]
    L.spec_verify_set_aux.argtypes = [vp, vp, vp, vp, vp]
    L.spec_verify_set_stops.argtypes = [vp, i32, vp, vp]
    L.spec_verify_set_truncation.argtypes = [vp, vp, vp]
    L.spec_verify_set_policy.argtypes = [vp, vp, ctypes.c_double, vp, vp]
    L.spec_verify_set_residual.argtypes = [vp, i32, vp, vp]
    L.spec_verify_set_walk_order.argtypes = [vp, i32]
    L.spec_verify_get_ema.argtypes = [vp, vp, vp, vp]
    L.spec_verify_set_ema.argtypes = [vp, vp, vp, vp]
    L.spec_verify_reset_ema.argtypes = [vp, vp]
    L.spec_verify_get_stats.argtypes = [vp, ctypes.POINTER(Stats), i32, vp]
    L.spec_verify_profile.argtypes = [vp, i32]
    L.spec_verify_profile_read.argtypes = [vp, ctypes.POINTER(f64), ctypes.POINTER(f64),
                                           ctypes.POINTER(i32)]
    L.spec_verify_last_error.argtypes = [vp]
    L.spec_verify_last_error.restype = ctypes.c_char_p
    L.spec_verify_version.restype = ctypes.c_char_p
    L.spec_verify_read_probe.argtypes = [vp, ctypes.c_size_t, vp, vp]
    L.spec_verify_noalloc.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, f32, i32, f32,
                                      vp, vp, vp, vp]
    for name in EXPORTED:
        if name not in ("spec_verify_last_error", "spec_verify_version"):
            getattr(L, name).restype = i32
    _lib = L
    return L


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_out(out, B: int, K: int, device):
    """The caller's output tensors: int32, contiguous, on `device`, shaped
    [B, K+1], [B] and [K+1] (the kernels write exactly these)."""
    if not isinstance(out, (tuple, list)) or len(out) != 3:
        raise SpecVerifyError(SV_EINVAL, "out: expected (tokens, accept_len, hist)")
    for t, shape, name in zip(out, ((B, K + 1), (B,), (K + 1,)),
                              ("tokens", "accept_len", "hist")):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.device != device
                or tuple(t.shape) != shape or not t.is_contiguous()):
            raise SpecVerifyError(SV_EINVAL, f"out {name}: expected a contiguous int32 tensor "
                                             f"of shape {list(shape)} on {device}")


def _check_inputs(target, draft, tokens, uniforms, mode, K, V, dtype, device):
    """Shapes, dtypes, devices and contiguity of one call's inputs; returns B
    and the (draft, uniforms) the mode reads (None for greedy and margin)."""
    if mode not in MODES:
        raise SpecVerifyError(SV_EINVAL, f"unknown mode {mode!r}")
    B = int(target.shape[0])

    def logits(t, rows, name):
        if t.device != device or t.dtype != dtype:
            raise SpecVerifyError(SV_EINVAL, f"{name}: expected {dtype} on {device}")
        if tuple(t.shape) != (B, rows, V) or not t.is_contiguous():
            raise SpecVerifyError(SV_EINVAL, f"{name}: expected contiguous [B, {rows}, {V}]")

    logits(target, K + 1, "target")
    if mode == "stochastic":
        if draft is None or uniforms is None:
            raise SpecVerifyError(SV_EINVAL, "stochastic mode needs draft and uniforms")
        logits(draft, K, "draft")
        if (uniforms.dtype != torch.float32 or tuple(uniforms.shape) != (B, K + 1)
                or not uniforms.is_contiguous() or uniforms.device != device):
            raise SpecVerifyError(SV_EINVAL, "uniforms: expected contiguous float32 [B, K+1]")
    else:
        draft = None
        uniforms = None
    if (tokens.dtype != torch.int32 or tuple(tokens.shape) != (B, K)
            or not tokens.is_contiguous() or tokens.device != device):
        raise SpecVerifyError(SV_EINVAL, "tokens: expected contiguous int32 [B, K]")
    return B, draft, uniforms


def verify_noalloc(target, draft, tokens, uniforms, temperature: float, mode: str, tau: float,
                   out) -> None:
    """One verification through spec_verify_noalloc: no handle, no device
    allocation by the library, its workspace in the library's fixed per-GPU
    scratch array. The caller passes the inputs and the outputs out =
    (tokens [B, K+1], accept_len [B], hist [K+1]), all int32 device tensors;
    work is ordered on the current stream of the inputs' device. No EMA and
    no side outputs are kept. Calls that overlap on one GPU race."""
    L = load_library()
    device = target.device
    B, K, V = int(target.shape[0]), int(target.shape[1]) - 1, int(target.shape[2])
    if target.dtype not in (torch.float32, torch.bfloat16):
        raise SpecVerifyError(SV_EUNSUPPORTED, f"logit dtype {target.dtype}")
    B, draft, uniforms = _check_inputs(target, draft, tokens, uniforms, mode, K, V,
                                       target.dtype, device)
    _check_out(out, B, K, device)
    ot, ol, oh = out
    code = SV_DTYPE_F32 if target.dtype == torch.float32 else SV_DTYPE_BF16
    with torch.cuda.device(device):
        rc = L.spec_verify_noalloc(B, K, V, code, _ptr(target), _ptr(draft), _ptr(tokens),
                                   _ptr(uniforms), float(temperature), MODES[mode], float(tau),
                                   _ptr(ot), _ptr(ol), _ptr(oh), _stream(device))
    if rc != SV_OK:
        msg = L.spec_verify_last_error(None)
        raise SpecVerifyError(rc, f"spec_verify_noalloc: {msg.decode() if msg else ''}")


def read_probe(buf: "torch.Tensor", sink: "torch.Tensor") -> None:
    """One plain streaming read of `buf` (a contiguous device tensor, 16-byte
    aligned, size a multiple of 16 bytes) on the current stream: the
    achievable-bandwidth reference for the streaming pass."""
    L = load_library()
    rc = L.spec_verify_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                  _stream(buf.device))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "read_probe")


class SpecVerifier:
    """One verification handle: fixed K, V and logit dtype, batches up to
    max_batch, with its own workspace and per-slot acceptance EMA."""

    def __init__(self, max_batch: int, K: int, V: int, dtype=torch.bfloat16,
                 ema_decay: float = 0.99, device=None):
        self.lib = load_library()
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        if dtype not in (torch.float32, torch.bfloat16):
            raise SpecVerifyError(SV_EUNSUPPORTED, f"logit dtype {dtype}")
        self.max_batch, self.K, self.V, self.dtype = int(max_batch), int(K), int(V), dtype
        self.ema_decay = float(ema_decay)
        h = ctypes.c_void_p()
        code = SV_DTYPE_F32 if dtype == torch.float32 else SV_DTYPE_BF16
        with torch.cuda.device(self.device):
            rc = self.lib.spec_verify_init(ctypes.byref(h), self.max_batch, self.K, self.V,
                                           code, self.ema_decay)
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_init failed")
        self._h = h
        self._aux = None
        self._stops = (None, None)

    # -- lifetime --
    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            with torch.cuda.device(self.device):
                self.lib.spec_verify_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc: int, what: str):
        if rc != SV_OK:
            msg = self.lib.spec_verify_last_error(self._h)
            raise SpecVerifyError(rc, f"{what}: {msg.decode() if msg else ''}")

    # -- side outputs --
    def enable_aux(self) -> dict:
        """Allocate and register the per-call side outputs (p(d), q(d), Z, argmax)."""
        B, K = self.max_batch, self.K
        dev = self.device
        self._aux = dict(
            p_d=torch.empty((B, K), dtype=torch.float64, device=dev),
            q_d=torch.empty((B, K), dtype=torch.float64, device=dev),
            z=torch.empty((B,), dtype=torch.float64, device=dev),
            argmax=torch.empty((B, K + 1), dtype=torch.int32, device=dev))
        a = self._aux
        self._check(self.lib.spec_verify_set_aux(self._h, _ptr(a["p_d"]), _ptr(a["q_d"]),
                                                 _ptr(a["z"]), _ptr(a["argmax"])), "set_aux")
        return a

    def disable_aux(self):
        self._check(self.lib.spec_verify_set_aux(self._h, None, None, None, None), "set_aux")
        self._aux = None

    @property
    def aux(self):
        return self._aux

    # -- stopping rules --
    def set_stops(self, eos: int = -1, draft_len=None, max_emit=None):
        """End-of-sequence token, per-sequence draft counts [max_batch] and
        emission budgets [max_batch] (int32 device tensors, or None) for later
        calls. The tensors are kept referenced here while they are in use."""
        for t in (draft_len, max_emit):
            if t is not None and (t.dtype != torch.int32 or t.device != self.device
                                  or t.numel() < self.max_batch or not t.is_contiguous()):
                raise ValueError("stop arrays must be contiguous int32 device tensors "
                                 "of at least max_batch entries")
        self._check(self.lib.spec_verify_set_stops(
            self._h, int(eos), None if draft_len is None else _ptr(draft_len),
            None if max_emit is None else _ptr(max_emit)), "set_stops")
        self._stops = (draft_len, max_emit)

    def clear_stops(self):
        self.set_stops(-1, None, None)

    def set_truncation(self, top_k=None, top_p=None):
        """Per-sequence top-k [max_batch] (int32) and top-p [max_batch]
        (float32) device tensors, or None, for later stochastic calls (bf16
        or float32 logits). The tensors are kept referenced here while they
        are in use."""
        for t, dt, name in ((top_k, torch.int32, "top_k"), (top_p, torch.float32, "top_p")):
            if t is not None and (t.dtype != dt or t.device != self.device or not t.is_contiguous()
                                  or t.numel() < self.max_batch):
                raise ValueError(f"{name} must be a contiguous {dt} device tensor of "
                                 f"at least max_batch entries")
        self._check(self.lib.spec_verify_set_truncation(
            self._h, None if top_k is None else _ptr(top_k),
            None if top_p is None else _ptr(top_p)), "set_truncation")
        self._trunc = (top_k, top_p)

    def clear_truncation(self):
        self.set_truncation(None, None)

    def set_residual(self, m: int = 32):
        """Draft residual side output for later stochastic calls. m = 0
        turns it off. Returns (support [max_batch, K, m] int32, residual
        [max_batch, K, m] float64), device tensors the calls write."""
        if m == 0:
            self._check(self.lib.spec_verify_set_residual(self._h, 0, None, None),
                        "set_residual")
            self._residual = None
            return None
        sup = torch.full((self.max_batch, self.K, m), -1, dtype=torch.int32, device=self.device)
        res = torch.full((self.max_batch, self.K, m), float("nan"), dtype=torch.float64,
                         device=self.device)
        self._check(self.lib.spec_verify_set_residual(self._h, int(m), _ptr(sup), _ptr(res)),
                    "set_residual")
        self._residual = (sup, res)
        return sup, res

    def set_walk_order(self, on: bool = True):
        """Walk-order reading for later greedy, margin and stochastic calls
        (not with the residual side output): rows
        past each sequence's first rejection are not read (and so not
        checked); p(d), q(d) or the margin ratio past it are NaN, the per-row
        argmax -1."""
        self._check(self.lib.spec_verify_set_walk_order(self._h, 1 if on else 0),
                    "set_walk_order")

    def set_policy(self, draft_conf, d: float = 0.5, want_dcs: bool = False):
        """Tree-shape policy for later calls: draft_conf is a float32 device
        tensor of at least max_batch draft top-1 probabilities (or None to
        turn the policy off). Returns (shape [max_batch, 3] int32, dcs
        [max_batch] float64 or None), device tensors the calls write."""
        if draft_conf is None:
            self._check(self.lib.spec_verify_set_policy(self._h, None, 1.0, None, None),
                        "set_policy")
            self._policy = None
            return None
        if (draft_conf.dtype != torch.float32 or draft_conf.device != self.device
                or not draft_conf.is_contiguous() or draft_conf.numel() < self.max_batch):
            raise ValueError("draft_conf must be a contiguous float32 device tensor of at least "
                             "max_batch entries")
        shape = torch.full((self.max_batch, 3), -1, dtype=torch.int32, device=self.device)
        dcs = (torch.full((self.max_batch,), float("nan"), dtype=torch.float64,
                          device=self.device) if want_dcs else None)
        self._check(self.lib.spec_verify_set_policy(self._h, _ptr(draft_conf), float(d),
                                                    _ptr(shape),
                                                    None if dcs is None else _ptr(dcs)),
                    "set_policy")
        self._policy = (draft_conf, shape, dcs)
        return shape, dcs

    # -- verification --
    def verify(self, target, draft, tokens, uniforms=None, temperature: float = 1.0,
               mode: str = "stochastic", tau: float = 0.0, out=None):
        """Verify a batch. Returns (tokens [B, K+1] int32, accept_len [B] int32,
        hist [K+1] int32 holding uint32 counts), ordered on the current stream.
        out, when given, is the (tokens, accept_len, hist) tensors to write."""
        K = self.K
        B, draft, uniforms = _check_inputs(target, draft, tokens, uniforms, mode, K, self.V,
                                           self.dtype, self.device)
        if out is None:
            out = (torch.empty((B, K + 1), dtype=torch.int32, device=self.device),
                   torch.empty((B,), dtype=torch.int32, device=self.device),
                   torch.empty((K + 1,), dtype=torch.int32, device=self.device))
        else:
            _check_out(out, B, K, self.device)
        ot, ol, oh = out
        with torch.cuda.device(self.device):
            rc = self.lib.spec_verify(self._h, B, _ptr(target), _ptr(draft), _ptr(tokens),
                                      _ptr(uniforms), float(temperature), MODES[mode],
                                      float(tau), _ptr(ot), _ptr(ol), _ptr(oh),
                                      _stream(self.device))
        self._check(rc, "spec_verify")
        return ot, ol, oh

    # -- EMA and counters --
    def ema(self):
        e = torch.empty((self.max_batch,), dtype=torch.float64, device=self.device)
        s = torch.empty((self.max_batch,), dtype=torch.int32, device=self.device)
        self._check(self.lib.spec_verify_get_ema(self._h, _ptr(e), _ptr(s),
                                                 _stream(self.device)), "get_ema")
        return e, s

    def set_ema(self, ema, steps):
        ema = ema.to(device=self.device, dtype=torch.float64).contiguous()
        steps = steps.to(device=self.device, dtype=torch.int32).contiguous()
        if ema.numel() != self.max_batch or steps.numel() != self.max_batch:
            raise SpecVerifyError(SV_EINVAL, "set_ema: need max_batch entries")
        self._check(self.lib.spec_verify_set_ema(self._h, _ptr(ema), _ptr(steps),
                                                 _stream(self.device)), "set_ema")
        torch.cuda.current_stream(self.device).synchronize()

    def reset_ema(self):
        self._check(self.lib.spec_verify_reset_ema(self._h, _stream(self.device)), "reset_ema")

    def stats(self, reset: bool = False) -> dict:
        s = Stats()
        self._check(self.lib.spec_verify_get_stats(self._h, ctypes.byref(s), int(reset),
                                                   _stream(self.device)), "get_stats")
        return {k: int(getattr(s, k)) for k, _ in Stats._fields_}


    # -- profiling --
    def profile(self, enable: bool = True, call_end: bool = False):
        """Record HIP events around the streaming pass of later calls (and after
        each call when call_end is set)."""
        flag = (1 | (2 if call_end else 0)) if enable else 0
        self._check(self.lib.spec_verify_profile(self._h, flag), "profile")

    def profile_read(self):
        """(streaming-pass ms, whole-call ms, calls) summed since the last read."""
        a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
        self._check(self.lib.spec_verify_profile_read(self._h, ctypes.byref(a), ctypes.byref(b),
                                                      ctypes.byref(n)), "profile_read")
        return a.value, b.value, n.value


def version() -> str:
    return load_library().spec_verify_version().decode()


__all__ = ["SpecVerifier", "SpecVerifyError", "load_library", "version", "verify_noalloc",
           "MODES", "EXPORTED"]
