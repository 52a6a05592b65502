"""SambaY cross-decoder decode path for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libsambay.so`` (C ABI in ``include/sambay.h``).
It only checks and marshals arguments — device, dtype, shape, contiguity —
and passes torch's device memory and current HIP stream to the library;
every step of the computation runs in the library's HIP kernels.  There is
no CPU fallback: if the library is missing the import fails.

Calls (same names as the C ABI):
    gmu_forward(M, X, W1, W2, out=None)            -> Y
    xattn_decode(q, kcache, vcache, out=None, scale=None) -> out
    crossdecoder_step(h, M, kcache, vcache, layers, scale=None) -> h (in place)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsambay.so")

SB_OK, SB_EINVAL, SB_EUNSUPPORTED, SB_EWORKSPACE, SB_EHIP = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "SB_OK", 1: "SB_EINVAL", 2: "SB_EUNSUPPORTED", 3: "SB_EWORKSPACE", 4: "SB_EHIP"}
SB_F32, SB_BF16 = 0, 1
SB_LAYER_XATTN, SB_LAYER_GMU = 0, 1
SB_SELF_MAMBA, SB_SELF_SWA, SB_SELF_ATTN = 0, 1, 2

# Every function the header declares, for load-time checking.
EXPORTS = ("sb_last_error", "sb_version", "gmu_workspace_bytes", "gmu_forward", "xattn_workspace_bytes",
           "xattn_decode", "crossdecoder_workspace_bytes", "crossdecoder_step", "sb_timing_enable",
           "sb_timing_collect", "sb_probe_stream_read", "sb_probe_mfma", "sb_probe_mfma_flops",
           "xattn_decode_varlen", "crossdecoder_ex_workspace_bytes", "crossdecoder_step_ex",
           "diffattn_workspace_bytes", "diffattn_decode", "selfattn_workspace_bytes", "selfattn_decode",
           "mamba_workspace_bytes", "mamba_decode_step", "attn_prefill_workspace_bytes", "attn_prefill",
           "mamba_prefill_workspace_bytes", "mamba_prefill", "sambay_prefill_workspace_bytes", "sambay_prefill",
           "sambay_decode_workspace_bytes", "sambay_decode_step", "xattn_decode_noalloc")
SB_TIME_XATTN_SPLIT, SB_TIME_XATTN_MERGE, SB_TIME_SKINNY, SB_TIME_GEMM, SB_TIME_GMU_F32, SB_TIME_PROBE = \
    1, 2, 4, 8, 16, 32
SB_TIME_DIFF_SPLIT, SB_TIME_DIFF_MERGE, SB_TIME_PREFILL = 64, 128, 256


class SbLayer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("w_a", ctypes.c_void_p), ("w_b", ctypes.c_void_p)]


class SbMambaWeights(ctypes.Structure):
    _fields_ = [("w_in", ctypes.c_void_p), ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p),
                ("w_x", ctypes.c_void_p), ("w_dt", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("a_log", ctypes.c_void_p), ("d_skip", ctypes.c_void_p), ("w_out", ctypes.c_void_p)]


class SbLayerEx(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("w_a", ctypes.c_void_p), ("w_b", ctypes.c_void_p),
                ("norm1", ctypes.c_void_p), ("norm2", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class SbSelfLayer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("mamba", SbMambaWeights), ("conv_state", ctypes.c_void_p),
                ("ssm_state", ctypes.c_void_p), ("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p),
                ("wv", ctypes.c_void_p), ("wo", ctypes.c_void_p), ("kring", ctypes.c_void_p),
                ("vring", ctypes.c_void_p), ("norm1", ctypes.c_void_p), ("norm2", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class SambayError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s: %s: %s" % (fn, STATUS_NAMES.get(status, str(status)), msg))
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libsambay.so not built at %s; run `python attention_decoding_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.sb_last_error.restype = ctypes.c_char_p
    lib.sb_version.restype = ctypes.c_char_p
    lib.gmu_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.gmu_workspace_bytes.restype = sz
    lib.gmu_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp, sz, vp]
    lib.gmu_forward.restype = ctypes.c_int
    lib.xattn_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.xattn_workspace_bytes.restype = sz
    lib.xattn_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp, sz, vp]
    lib.xattn_decode.restype = ctypes.c_int
    lib.xattn_decode_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp]
    lib.xattn_decode_noalloc.restype = ctypes.c_int
    lib.crossdecoder_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64]
    lib.crossdecoder_workspace_bytes.restype = sz
    lib.crossdecoder_step.argtypes = [vp, vp, vp, vp, ctypes.POINTER(SbLayer), i32, i64, i64, i64, i64, i64, i64,
                                      i64, ctypes.c_float, vp, sz, vp]
    lib.crossdecoder_step.restype = ctypes.c_int
    lib.xattn_decode_varlen.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp, sz, vp]
    lib.xattn_decode_varlen.restype = ctypes.c_int
    lib.crossdecoder_ex_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64]
    lib.crossdecoder_ex_workspace_bytes.restype = sz
    lib.crossdecoder_step_ex.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(SbLayerEx), i32, i64, i64, i64, i64, i64,
                                         i64, i64, i64, ctypes.c_float, ctypes.c_float, vp, sz, vp]
    lib.crossdecoder_step_ex.restype = ctypes.c_int
    lib.diffattn_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.diffattn_workspace_bytes.restype = sz
    lib.diffattn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, ctypes.c_float,
                                    ctypes.c_float, ctypes.c_float, vp, sz, vp]
    lib.diffattn_decode.restype = ctypes.c_int
    lib.selfattn_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.selfattn_workspace_bytes.restype = sz
    lib.selfattn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float, vp, sz,
                                    vp]
    lib.selfattn_decode.restype = ctypes.c_int
    lib.mamba_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.mamba_workspace_bytes.restype = sz
    lib.mamba_decode_step.argtypes = [vp, ctypes.POINTER(SbMambaWeights), vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                      i64, vp, sz, vp]
    lib.mamba_decode_step.restype = ctypes.c_int
    lib.attn_prefill_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_prefill_workspace_bytes.restype = sz
    lib.attn_prefill.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float, vp, sz, vp]
    lib.attn_prefill.restype = ctypes.c_int
    lib.mamba_prefill_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64]
    lib.mamba_prefill_workspace_bytes.restype = sz
    lib.mamba_prefill.argtypes = [vp, ctypes.POINTER(SbMambaWeights), vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  i64, vp, sz, vp]
    lib.mamba_prefill.restype = ctypes.c_int
    lib.sambay_prefill_workspace_bytes.argtypes = [i64] * 12
    lib.sambay_prefill_workspace_bytes.restype = sz
    lib.sambay_prefill.argtypes = [vp, vp, vp, ctypes.POINTER(SbSelfLayer), i32, ctypes.POINTER(SbLayerEx), i32, vp,
                                   vp] + [i64] * 13 + [ctypes.c_float, ctypes.c_float, vp, sz, vp]
    lib.sambay_prefill.restype = ctypes.c_int
    lib.sambay_decode_workspace_bytes.argtypes = [i64] * 12
    lib.sambay_decode_workspace_bytes.restype = sz
    lib.sambay_decode_step.argtypes = [vp, vp, ctypes.POINTER(SbSelfLayer), i32, ctypes.POINTER(SbLayerEx), i32, vp,
                                       vp, vp] + [i64] * 12 + [ctypes.c_float, ctypes.c_float, vp, sz, vp]
    lib.sambay_decode_step.restype = ctypes.c_int
    lib.sb_timing_enable.argtypes = [ctypes.c_uint32]
    lib.sb_timing_enable.restype = ctypes.c_int
    lib.sb_timing_collect.argtypes = [ctypes.c_uint32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    lib.sb_timing_collect.restype = ctypes.c_int
    lib.sb_probe_stream_read.argtypes = [vp, sz, vp, vp]
    lib.sb_probe_stream_read.restype = ctypes.c_int
    lib.sb_probe_mfma.argtypes = [i64, vp, vp]
    lib.sb_probe_mfma.restype = ctypes.c_int
    lib.sb_probe_mfma_flops.argtypes = [i64]
    lib.sb_probe_mfma_flops.restype = ctypes.c_double
    return lib


lib = _load()


def version() -> str:
    return lib.sb_version().decode()


def built_source_hash() -> str:
    """The source hash the loaded library was built from (from its version string)."""
    return version().rsplit(" ", 1)[-1]


def current_source_hash() -> str:
    """The hash of the kernel and header sources as they are on disk now."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("sambay_build", os.path.join(os.path.dirname(__file__), "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.source_hash()


def timing_enable(mask: int) -> None:
    """Bracket later launches of the kernel kinds in `mask` (SB_TIME_* bits)
    with HIP events on their own stream; 0 turns recording off."""
    _check("sb_timing_enable", lib.sb_timing_enable(int(mask)))


def timing_collect(mask: int):
    """(launches, total milliseconds) of the recorded launches of `mask`; forgets them."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check("sb_timing_collect", lib.sb_timing_collect(int(mask), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def probe_stream_read_gbps(buf: torch.Tensor, reps: int = 5) -> float:
    """Rate (GB/s) of a plain streaming read of `buf` (a GPU tensor) by the library's probe kernel."""
    dev = _check_device(buf, "buf")
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    st = _stream(dev)
    _check("sb_probe_stream_read", lib.sb_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), st))
    timing_enable(SB_TIME_PROBE)
    for _ in range(reps):
        _check("sb_probe_stream_read", lib.sb_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), st))
    timing_enable(0)
    n, ms = timing_collect(SB_TIME_PROBE)
    return nbytes / (ms / n / 1e3) / 1e9


_probe_sinks: dict = {}


def probe_stream_read_raw(buf: torch.Tensor) -> None:
    """Enqueue one plain streaming read of `buf` (no timing)."""
    dev = _check_device(buf, "buf")
    sink = _probe_sinks.get(dev)
    if sink is None:
        sink = _probe_sinks[dev] = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    _check("sb_probe_stream_read", lib.sb_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(dev)))


def probe_mfma_tflops(device, iters: int = 20000, reps: int = 3) -> float:
    """Rate (TFLOP/s) of the library's register-only bf16 32x32x16 MFMA loop."""
    dev = torch.device(device)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    st = _stream(dev)
    _check("sb_probe_mfma", lib.sb_probe_mfma(100, sink.data_ptr(), st))
    timing_enable(SB_TIME_PROBE)
    for _ in range(reps):
        _check("sb_probe_mfma", lib.sb_probe_mfma(iters, sink.data_ptr(), st))
    timing_enable(0)
    n, ms = timing_collect(SB_TIME_PROBE)
    return lib.sb_probe_mfma_flops(iters) / (ms / n / 1e3) / 1e12


def _check(fn: str, status: int):
    if status != SB_OK:
        raise SambayError(fn, status, lib.sb_last_error().decode())


def _dev_ptr(t: torch.Tensor, name: str, dtype: torch.dtype, device: torch.device) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_ws_cache: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A device byte buffer of at least nbytes, cached per device and stream
    (reused only by calls ordered on that stream)."""
    key = (device, _stream(device))
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _check_device(t: torch.Tensor, name: str) -> torch.device:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (the library has no CPU path)" % name)
    return t.device


def gmu_forward(M: torch.Tensor, X: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = (M ⊙ SiLU(X W1^T)) W2^T.  M [rows, d_inner], X [rows, d_model],
    W1 [d_inner, d_model], W2 [d_model, d_inner]; all bf16 or all fp32."""
    dev = _check_device(X, "X")
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("X must be bfloat16 or float32")
    dt = X.dtype
    if X.dim() != 2 or M.dim() != 2 or W1.dim() != 2 or W2.dim() != 2:
        raise ValueError("gmu_forward expects 2-D tensors")
    rows, d_model = X.shape
    d_inner = W1.shape[0]
    if M.shape != (rows, d_inner) or W1.shape != (d_inner, d_model) or W2.shape != (d_model, d_inner):
        raise ValueError("gmu_forward shape mismatch: M %s X %s W1 %s W2 %s" % (tuple(M.shape), tuple(X.shape),
                                                                              tuple(W1.shape), tuple(W2.shape)))
    if out is None:
        out = torch.empty((rows, d_model), dtype=dt, device=dev)
    elif out.shape != (rows, d_model):
        raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (rows, d_model)))
    code = SB_BF16 if dt == torch.bfloat16 else SB_F32
    nb = lib.gmu_workspace_bytes(rows, d_model, d_inner, code)
    ws = _workspace(dev, nb)
    st = lib.gmu_forward(_dev_ptr(M, "M", dt, dev), _dev_ptr(X, "X", dt, dev), _dev_ptr(W1, "W1", dt, dev),
                         _dev_ptr(W2, "W2", dt, dev), _dev_ptr(out, "out", dt, dev), rows, d_model, d_inner, code,
                         ws.data_ptr(), ws.numel(), _stream(dev))
    _check("gmu_forward", st)
    return out


def xattn_decode(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, out: torch.Tensor | None = None,
                 scale: float | None = None, lens: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention of q [B, Hq, D] over the shared cache kcache/vcache
    [B, Hkv, L, D]; bf16 in and out.  lens (optional, [B] int32 on the same
    GPU): sequence b attends to its first lens[b] positions only."""
    dev = _check_device(q, "q")
    bf = torch.bfloat16
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and kcache [B, Hkv, L, D]")
    B, Hq, D = q.shape
    B2, Hkv, L, D2 = kcache.shape
    if B2 != B or D2 != D or vcache.shape != kcache.shape:
        raise ValueError("xattn_decode shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(kcache.shape),
                                                                       tuple(vcache.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=bf, device=dev)
    elif out.shape != (B, Hq, D):
        raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (B, Hq, D)))
    nb = lib.xattn_workspace_bytes(B, Hq, Hkv, D, L)
    ws = _workspace(dev, nb)
    args = (_dev_ptr(q, "q", bf, dev), _dev_ptr(kcache, "kcache", bf, dev), _dev_ptr(vcache, "vcache", bf, dev))
    tail = (B, Hq, Hkv, D, L, float(scale), ws.data_ptr(), ws.numel(), _stream(dev))
    if lens is None:
        _check("xattn_decode", lib.xattn_decode(*args, _dev_ptr(out, "out", bf, dev), *tail))
    else:
        if lens.shape != (B,):
            raise ValueError("lens must have shape [B]")
        lp = _dev_ptr(lens, "lens", torch.int32, dev)
        _check("xattn_decode_varlen", lib.xattn_decode_varlen(*args, lp, _dev_ptr(out, "out", bf, dev), *tail))
    return out


def xattn_decode_noalloc(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, out: torch.Tensor,
                         scale: float | None = None) -> torch.Tensor:
    """xattn_decode whose partials live in the library's own per-GPU scratch
    array: the call allocates nothing (the caller passes out).  Calls that
    overlap on one GPU race (one array per GPU)."""
    dev = _check_device(q, "q")
    bf = torch.bfloat16
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and kcache [B, Hkv, L, D]")
    B, Hq, D = q.shape
    B2, Hkv, L, D2 = kcache.shape
    if B2 != B or D2 != D or vcache.shape != kcache.shape or out.shape != (B, Hq, D):
        raise ValueError("xattn_decode_noalloc shape mismatch: q %s k %s v %s out %s" %
                         (tuple(q.shape), tuple(kcache.shape), tuple(vcache.shape), tuple(out.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check("xattn_decode_noalloc",
           lib.xattn_decode_noalloc(_dev_ptr(q, "q", bf, dev), _dev_ptr(kcache, "kcache", bf, dev),
                                    _dev_ptr(vcache, "vcache", bf, dev), _dev_ptr(out, "out", bf, dev), B, Hq, Hkv, D,
                                    L, float(scale), _stream(dev)))
    return out


def diffattn_decode(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, lam: float, lam_init: float,
                    gamma: torch.Tensor | None = None, lens: torch.Tensor | None = None, eps: float = 1e-5,
                    out: torch.Tensor | None = None, scale: float | None = None) -> torch.Tensor:
    """Differential attention decode: each D-wide row of q [B, Hq, D] and of
    kcache [B, Hkv, L, D] is two halves, one per softmax map; out [B, Hq, D]
    = (1 - lam_init) * RMSNorm(map1 @ V - lam * map2 @ V) * gamma per head.
    scale defaults to 1/sqrt(D/2); gamma ([D] bf16) to all ones; lens as in
    xattn_decode.  bf16 in and out."""
    dev = _check_device(q, "q")
    bf = torch.bfloat16
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and kcache [B, Hkv, L, D]")
    B, Hq, D = q.shape
    B2, Hkv, L, D2 = kcache.shape
    if B2 != B or D2 != D or vcache.shape != kcache.shape:
        raise ValueError("diffattn_decode shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(kcache.shape),
                                                                          tuple(vcache.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(D // 2)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=bf, device=dev)
    elif out.shape != (B, Hq, D):
        raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (B, Hq, D)))
    if lens is not None and lens.shape != (B,):
        raise ValueError("lens must have shape [B]")
    if gamma is not None and gamma.shape != (D,):
        raise ValueError("gamma must have shape [D]")
    ws = _workspace(dev, lib.diffattn_workspace_bytes(B, Hq, Hkv, D, L))
    lp = None if lens is None else _dev_ptr(lens, "lens", torch.int32, dev)
    gp = None if gamma is None else _dev_ptr(gamma, "gamma", bf, dev)
    _check("diffattn_decode", lib.diffattn_decode(
        _dev_ptr(q, "q", bf, dev), _dev_ptr(kcache, "kcache", bf, dev), _dev_ptr(vcache, "vcache", bf, dev), lp, gp,
        _dev_ptr(out, "out", bf, dev), B, Hq, Hkv, D, L, float(scale), float(lam), float(lam_init), float(eps),
        ws.data_ptr(), ws.numel(), _stream(dev)))
    return out


def selfattn_decode(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, kcache: torch.Tensor,
                    vcache: torch.Tensor, pos: torch.Tensor, window: int = 0, out: torch.Tensor | None = None,
                    scale: float | None = None) -> torch.Tensor:
    """One self-decoder attention decode step: store k_new, v_new [B, Hkv, D]
    at position pos[b] of kcache/vcache [B, Hkv, L, D] (window 0) or in ring
    slot pos[b] % window (a cache of window slots), then attend q [B, Hq, D]
    over the visible positions.  The cache is updated in place; pos is [B]
    int32 on the same GPU (pos[b] < 0: inactive)."""
    dev = _check_device(q, "q")
    bf = torch.bfloat16
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and kcache [B, Hkv, L, D]")
    B, Hq, D = q.shape
    B2, Hkv, L, D2 = kcache.shape
    if B2 != B or D2 != D or vcache.shape != kcache.shape:
        raise ValueError("selfattn_decode shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(kcache.shape),
                                                                          tuple(vcache.shape)))
    if k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D):
        raise ValueError("k_new and v_new must be [B, Hkv, D]")
    if pos.shape != (B,):
        raise ValueError("pos must have shape [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=bf, device=dev)
    elif out.shape != (B, Hq, D):
        raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (B, Hq, D)))
    ws = _workspace(dev, lib.selfattn_workspace_bytes(B, Hq, Hkv, D, L))
    _check("selfattn_decode", lib.selfattn_decode(
        _dev_ptr(q, "q", bf, dev), _dev_ptr(k_new, "k_new", bf, dev), _dev_ptr(v_new, "v_new", bf, dev),
        _dev_ptr(kcache, "kcache", bf, dev), _dev_ptr(vcache, "vcache", bf, dev), _dev_ptr(pos, "pos", torch.int32, dev),
        _dev_ptr(out, "out", bf, dev), B, Hq, Hkv, D, L, int(window), float(scale), ws.data_ptr(), ws.numel(),
        _stream(dev)))
    return out


def _mamba_weights(w: dict, dev, d_model: int):
    bf, f32 = torch.bfloat16, torch.float32
    if w["conv_w"].dim() != 2 or w["A_log"].dim() != 2 or w["W_dt"].dim() != 2:
        raise ValueError("conv_w, A_log and W_dt must be 2-D")
    d_inner, d_conv = w["conv_w"].shape
    d_state, dt_rank = w["A_log"].shape[1], w["W_dt"].shape[1]
    shapes = {"W_in": (2 * d_inner, d_model), "W_x": (dt_rank + 2 * d_state, d_inner), "W_dt": (d_inner, dt_rank),
              "W_out": (d_model, d_inner), "conv_b": (d_inner,), "dt_bias": (d_inner,), "A_log": (d_inner, d_state),
              "D": (d_inner,)}
    for k, shp in shapes.items():
        if tuple(w[k].shape) != shp:
            raise ValueError("%s has shape %s, expected %s" % (k, tuple(w[k].shape), shp))
    sw = SbMambaWeights(
        _dev_ptr(w["W_in"], "W_in", bf, dev), _dev_ptr(w["conv_w"], "conv_w", f32, dev),
        _dev_ptr(w["conv_b"], "conv_b", f32, dev), _dev_ptr(w["W_x"], "W_x", bf, dev),
        _dev_ptr(w["W_dt"], "W_dt", bf, dev), _dev_ptr(w["dt_bias"], "dt_bias", f32, dev),
        _dev_ptr(w["A_log"], "A_log", f32, dev), _dev_ptr(w["D"], "D", f32, dev), _dev_ptr(w["W_out"], "W_out", bf, dev))
    return sw, d_inner, d_state, dt_rank, d_conv


def mamba_prefill(x: torch.Tensor, w: dict, conv_state: torch.Tensor, ssm_state: torch.Tensor,
                  M_out: torch.Tensor | None = None, y_out: torch.Tensor | None = None):
    """The Mamba layer over T prompt tokens, x [B, T, d_model] (bf16), weights
    as for mamba_decode_step; conv_state and ssm_state (float32) are read as
    the states before the prompt and overwritten with those after it.
    Returns (M [B, T, d_inner], y [B, T, d_model]), bf16."""
    dev = _check_device(x, "x")
    bf = torch.bfloat16
    if x.dim() != 3:
        raise ValueError("x must be [B, T, d_model]")
    B, T, d_model = x.shape
    sw, d_inner, d_state, dt_rank, d_conv = _mamba_weights(w, dev, d_model)
    if conv_state.shape != (B, d_inner, d_conv - 1) or ssm_state.shape != (B, d_inner, d_state):
        raise ValueError("state shape mismatch")
    if M_out is None:
        M_out = torch.empty((B, T, d_inner), dtype=bf, device=dev)
    if y_out is None:
        y_out = torch.empty((B, T, d_model), dtype=bf, device=dev)
    ws = _workspace(dev, lib.mamba_prefill_workspace_bytes(B, T, d_model, d_inner, d_state, dt_rank, d_conv))
    _check("mamba_prefill", lib.mamba_prefill(
        _dev_ptr(x, "x", bf, dev), ctypes.byref(sw), _dev_ptr(conv_state, "conv_state", torch.float32, dev),
        _dev_ptr(ssm_state, "ssm_state", torch.float32, dev), _dev_ptr(M_out, "M_out", bf, dev),
        _dev_ptr(y_out, "y_out", bf, dev), B, T, d_model, d_inner, d_state, dt_rank, d_conv, ws.data_ptr(),
        ws.numel(), _stream(dev)))
    return M_out, y_out


def mamba_decode_step(x: torch.Tensor, w: dict, conv_state: torch.Tensor, ssm_state: torch.Tensor,
                      M_out: torch.Tensor | None = None, y_out: torch.Tensor | None = None):
    """One decode step of the self-decoder's Mamba layer for x [B, d_model]
    (bf16).  w: W_in [2 d_inner, d_model], W_x [dt_rank + 2 d_state, d_inner],
    W_dt [d_inner, dt_rank], W_out [d_model, d_inner] (bf16); conv_w
    [d_inner, d_conv], conv_b, dt_bias, D [d_inner], A_log [d_inner, d_state]
    (float32).  conv_state [B, d_inner, d_conv - 1] and ssm_state [B, d_inner,
    d_state] (float32) are updated in place.  Returns (M [B, d_inner], y
    [B, d_model]), bf16: the memory readout and the layer's output."""
    dev = _check_device(x, "x")
    bf, f32 = torch.bfloat16, torch.float32
    if x.dim() != 2:
        raise ValueError("x must be [B, d_model]")
    B, d_model = x.shape
    if w["conv_w"].dim() != 2 or w["A_log"].dim() != 2 or w["W_dt"].dim() != 2:
        raise ValueError("conv_w, A_log and W_dt must be 2-D")
    d_inner, d_conv = w["conv_w"].shape
    d_state, dt_rank = w["A_log"].shape[1], w["W_dt"].shape[1]
    shapes = {"W_in": (2 * d_inner, d_model), "W_x": (dt_rank + 2 * d_state, d_inner), "W_dt": (d_inner, dt_rank),
              "W_out": (d_model, d_inner), "conv_b": (d_inner,), "dt_bias": (d_inner,), "A_log": (d_inner, d_state),
              "D": (d_inner,)}
    for k, shp in shapes.items():
        if tuple(w[k].shape) != shp:
            raise ValueError("%s has shape %s, expected %s" % (k, tuple(w[k].shape), shp))
    if conv_state.shape != (B, d_inner, d_conv - 1) or ssm_state.shape != (B, d_inner, d_state):
        raise ValueError("state shape mismatch")
    if M_out is None:
        M_out = torch.empty((B, d_inner), dtype=bf, device=dev)
    if y_out is None:
        y_out = torch.empty((B, d_model), dtype=bf, device=dev)
    if M_out.shape != (B, d_inner) or y_out.shape != (B, d_model):
        raise ValueError("output shape mismatch")
    sw = SbMambaWeights(
        _dev_ptr(w["W_in"], "W_in", bf, dev), _dev_ptr(w["conv_w"], "conv_w", f32, dev),
        _dev_ptr(w["conv_b"], "conv_b", f32, dev), _dev_ptr(w["W_x"], "W_x", bf, dev),
        _dev_ptr(w["W_dt"], "W_dt", bf, dev), _dev_ptr(w["dt_bias"], "dt_bias", f32, dev),
        _dev_ptr(w["A_log"], "A_log", f32, dev), _dev_ptr(w["D"], "D", f32, dev), _dev_ptr(w["W_out"], "W_out", bf, dev))
    ws = _workspace(dev, lib.mamba_workspace_bytes(B, d_model, d_inner, d_state, dt_rank, d_conv))
    _check("mamba_decode_step", lib.mamba_decode_step(
        _dev_ptr(x, "x", bf, dev), ctypes.byref(sw), _dev_ptr(conv_state, "conv_state", f32, dev),
        _dev_ptr(ssm_state, "ssm_state", f32, dev), _dev_ptr(M_out, "M_out", bf, dev), _dev_ptr(y_out, "y_out", bf, dev),
        B, d_model, d_inner, d_state, dt_rank, d_conv, ws.data_ptr(), ws.numel(), _stream(dev)))
    return M_out, y_out


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int = 0, out: torch.Tensor | None = None,
                 scale: float | None = None) -> torch.Tensor:
    """Causal prefill attention over the prompt: q [B, T, Hq, D], k, v
    [B, T, Hkv, D] (bf16) -> out [B, T, Hq, D]; query i sees keys j <= i and,
    with window > 0, j > i - window."""
    dev = _check_device(q, "q")
    bf = torch.bfloat16
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, T, Hq, D] and k [B, T, Hkv, D]")
    B, T, Hq, D = q.shape
    if k.shape[:2] != (B, T) or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("attn_prefill shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                                       tuple(v.shape)))
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=bf, device=dev)
    elif out.shape != (B, T, Hq, D):
        raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (B, T, Hq, D)))
    ws = _workspace(dev, lib.attn_prefill_workspace_bytes(B, T, Hkv, D))
    _check("attn_prefill", lib.attn_prefill(_dev_ptr(q, "q", bf, dev), _dev_ptr(k, "k", bf, dev),
                                            _dev_ptr(v, "v", bf, dev), _dev_ptr(out, "out", bf, dev), B, T, Hq, Hkv,
                                            D, int(window), float(scale), ws.data_ptr(), ws.numel(), _stream(dev)))
    return out


def _layer_array(layers: Sequence, dev: torch.device, d_model: int, d_inner: int):
    arr = (SbLayer * max(len(layers), 1))()
    bf = torch.bfloat16
    for i, layer in enumerate(layers):
        kind, wa, wb = layer
        if kind in ("xattn", SB_LAYER_XATTN):
            k, sa, sb = SB_LAYER_XATTN, (d_model, d_model), (d_model, d_model)
        elif kind in ("gmu", SB_LAYER_GMU):
            k, sa, sb = SB_LAYER_GMU, (d_inner, d_model), (d_model, d_inner)
        else:
            raise ValueError("layer %d: kind must be 'xattn' or 'gmu'" % i)
        if tuple(wa.shape) != sa or tuple(wb.shape) != sb:
            raise ValueError("layer %d (%s): weights %s, %s; expected %s, %s" % (i, kind, tuple(wa.shape),
                                                                               tuple(wb.shape), sa, sb))
        arr[i].kind = k
        arr[i].w_a = _dev_ptr(wa, "layer %d w_a" % i, bf, dev)
        arr[i].w_b = _dev_ptr(wb, "layer %d w_b" % i, bf, dev)
    return arr


class CrossDecoderStep:
    """Prepared argument block for repeated cross-decoder steps on the same
    tensors (what a decode loop or a HIP graph capture calls): the layer array
    and workspace are built once; __call__ only enqueues."""

    def __init__(self, h, M, kcache, vcache, layers: Sequence, scale: float | None = None):
        dev = _check_device(h, "h")
        bf = torch.bfloat16
        if h.dim() != 2 or M.dim() != 2 or kcache.dim() != 4:
            raise ValueError("h [B, d_model], M [B, d_inner], kcache [B, Hkv, L, D]")
        B, d_model = h.shape
        d_inner = M.shape[1]
        B2, Hkv, L, D = kcache.shape
        if M.shape[0] != B or B2 != B or vcache.shape != kcache.shape:
            raise ValueError("crossdecoder_step shape mismatch")
        if d_model % D != 0:
            raise ValueError("d_model must be a multiple of the head dim")
        self.Hq = d_model // D
        self.dims = (B, d_model, d_inner, self.Hq, Hkv, D, L)
        self.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
        self.tensors = (h, M, kcache, vcache, layers)
        self.ptrs = (_dev_ptr(h, "h", bf, dev), _dev_ptr(M, "M", bf, dev), _dev_ptr(kcache, "kcache", bf, dev),
                     _dev_ptr(vcache, "vcache", bf, dev))
        self.arr = _layer_array(layers, dev, d_model, d_inner)
        self.n_layers = len(layers)
        nb = lib.crossdecoder_workspace_bytes(B, d_model, d_inner, self.Hq, Hkv, D, L)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.device = dev

    def __call__(self):
        st = lib.crossdecoder_step(*self.ptrs, self.arr, self.n_layers, *self.dims, self.scale, self.ws.data_ptr(),
                                   self.ws.numel(), _stream(self.device))
        _check("crossdecoder_step", st)
        return self.tensors[0]


def crossdecoder_step(h: torch.Tensor, M: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                      layers: Sequence, scale: float | None = None) -> torch.Tensor:
    """One cross-decoder decode step; h [B, d_model] bf16 is updated in place.
    layers: sequence of (kind, w_a, w_b), kind "xattn" (Wq, Wo) or "gmu" (W1, W2)."""
    return CrossDecoderStep(h, M, kcache, vcache, layers, scale)()


_EX_KEYS = ("norm1", "norm2", "w_gate", "w_up", "w_down")


def _mlp_width(layers: Sequence) -> int:
    d_ff = 0
    for ly in layers:
        if ly.get("w_gate") is not None:
            d_ff = ly["w_gate"].shape[0]
    return d_ff


def _set_norms_mlp(arr_i, ly: dict, i: int, dev, d_model: int, d_ff: int, what: str) -> None:
    shapes = {"norm1": (d_model,), "norm2": (d_model,), "w_gate": (d_ff, d_model), "w_up": (d_ff, d_model),
              "w_down": (d_model, d_ff)}
    for key in _EX_KEYS:
        t = ly.get(key)
        if t is None:
            continue
        if tuple(t.shape) != shapes[key]:
            raise ValueError("%s %d %s has shape %s, expected %s" % (what, i, key, tuple(t.shape), shapes[key]))
        setattr(arr_i, key, _dev_ptr(t, "%s %d %s" % (what, i, key), torch.bfloat16, dev))


def _layer_ex_array(layers: Sequence, dev, d_model: int, d_inner: int, d_ff: int):
    arr = (SbLayerEx * max(len(layers), 1))()
    base = _layer_array([(ly["kind"], ly["w_a"], ly["w_b"]) for ly in layers], dev, d_model, d_inner)
    for i, ly in enumerate(layers):
        arr[i].kind, arr[i].w_a, arr[i].w_b = base[i].kind, base[i].w_a, base[i].w_b
        _set_norms_mlp(arr[i], ly, i, dev, d_model, d_ff, "layer")
    return arr


class CrossDecoderStepEx:
    """Prepared complete-layer decode step (pre-RMSNorm mixer, optional
    pre-RMSNorm SwiGLU MLP, optional ragged cache lengths).  layers: sequence of
    dicts with keys kind, w_a, w_b and optional norm1, norm2, w_gate, w_up,
    w_down (None: absent).  lens: None or [B] int32 on the same GPU."""

    def __init__(self, h, M, kcache, vcache, layers: Sequence, lens: torch.Tensor | None = None,
                 eps: float = 1e-5, scale: float | None = None):
        dev = _check_device(h, "h")
        bf = torch.bfloat16
        if h.dim() != 2 or M.dim() != 2 or kcache.dim() != 4:
            raise ValueError("h [B, d_model], M [B, d_inner], kcache [B, Hkv, L, D]")
        B, d_model = h.shape
        d_inner = M.shape[1]
        B2, Hkv, L, D = kcache.shape
        if M.shape[0] != B or B2 != B or vcache.shape != kcache.shape:
            raise ValueError("crossdecoder_step_ex shape mismatch")
        if d_model % D != 0:
            raise ValueError("d_model must be a multiple of the head dim")
        Hq = d_model // D
        d_ff = _mlp_width(layers)
        arr = _layer_ex_array(layers, dev, d_model, d_inner, d_ff)
        if lens is not None and lens.shape != (B,):
            raise ValueError("lens must have shape [B]")
        self.lens_ptr = _dev_ptr(lens, "lens", torch.int32, dev) if lens is not None else None
        self.dims = (B, d_model, d_inner, d_ff, Hq, Hkv, D, L)
        self.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
        self.eps = float(eps)
        self.tensors = (h, M, kcache, vcache, layers, lens)
        self.ptrs = (_dev_ptr(h, "h", bf, dev), _dev_ptr(M, "M", bf, dev), _dev_ptr(kcache, "kcache", bf, dev),
                     _dev_ptr(vcache, "vcache", bf, dev))
        self.arr = arr
        self.n_layers = len(layers)
        nb = lib.crossdecoder_ex_workspace_bytes(*self.dims)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.device = dev

    def __call__(self):
        st = lib.crossdecoder_step_ex(*self.ptrs, self.lens_ptr, self.arr, self.n_layers, *self.dims, self.scale,
                                      self.eps, self.ws.data_ptr(), self.ws.numel(), _stream(self.device))
        _check("crossdecoder_step_ex", st)
        return self.tensors[0]


def crossdecoder_step_ex(h: torch.Tensor, M: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                         layers: Sequence, lens: torch.Tensor | None = None, eps: float = 1e-5,
                         scale: float | None = None) -> torch.Tensor:
    """One complete-layer cross-decoder decode step; h is updated in place."""
    return CrossDecoderStepEx(h, M, kcache, vcache, layers, lens, eps, scale)()


_SELF_KINDS = {"mamba": SB_SELF_MAMBA, "swa": SB_SELF_SWA, "attn": SB_SELF_ATTN}


def _self_layer_array(self_layers: Sequence, cross_layers: Sequence, dev, B: int, d_model: int, Hkv: int, D: int,
                      window: int):
    """sb_self_layer descriptors for the self-decoder layer dicts (see
    SambayPrefill); returns (array, (d_inner, d_state, dt_rank, d_conv), d_ff)."""
    bf, f32 = torch.bfloat16, torch.float32
    mamba = [ly for ly in self_layers if ly["kind"] == "mamba"]
    if mamba:
        _, d_inner, d_state, dt_rank, d_conv = _mamba_weights(mamba[0]["w"], dev, d_model)
    else:  # no SSM layer: any supported SSM shape sizes the (unused) memory
        d_inner, d_state, dt_rank, d_conv = 64, 8, 64, 1
        for ly in cross_layers:
            if ly["kind"] == "gmu":
                d_inner = ly["w_a"].shape[0]
    d_ff = max(_mlp_width(self_layers), _mlp_width(cross_layers))
    arr = (SbSelfLayer * max(len(self_layers), 1))()
    for i, ly in enumerate(self_layers):
        kind = ly["kind"]
        if kind not in _SELF_KINDS:
            raise ValueError("self layer kind must be 'mamba', 'swa' or 'attn'")
        arr[i].kind = _SELF_KINDS[kind]
        if kind == "mamba":
            sw, di, ds, dr, dc = _mamba_weights(ly["w"], dev, d_model)
            if (di, ds, dr, dc) != (d_inner, d_state, dt_rank, d_conv):
                raise ValueError("every SSM layer must have the same shape")
            if ly["ssm_state"].shape != (B, d_inner, d_state) or \
                    (d_conv > 1 and ly["conv_state"].shape != (B, d_inner, d_conv - 1)):
                raise ValueError("self layer %d: state shape mismatch" % i)
            arr[i].mamba = sw
            arr[i].ssm_state = _dev_ptr(ly["ssm_state"], "ssm_state", f32, dev)
            if d_conv > 1:
                arr[i].conv_state = _dev_ptr(ly["conv_state"], "conv_state", f32, dev)
        else:
            shapes = {"wq": (d_model, d_model), "wk": (Hkv * D, d_model), "wv": (Hkv * D, d_model),
                      "wo": (d_model, d_model)}
            for key, shp in shapes.items():
                if tuple(ly[key].shape) != shp:
                    raise ValueError("self layer %d %s has shape %s, expected %s" %
                                     (i, key, tuple(ly[key].shape), shp))
                setattr(arr[i], key, _dev_ptr(ly[key], "self layer %d %s" % (i, key), bf, dev))
            if kind == "swa":
                for key in ("kring", "vring"):
                    if tuple(ly[key].shape) != (B, Hkv, window, D):
                        raise ValueError("self layer %d %s must be [B, Hkv, window, D]" % (i, key))
                    setattr(arr[i], key, _dev_ptr(ly[key], "self layer %d %s" % (i, key), bf, dev))
        _set_norms_mlp(arr[i], ly, i, dev, d_model, d_ff, "self layer")
    return arr, (d_inner, d_state, dt_rank, d_conv), d_ff


class SambayPrefill:
    """Prepared YOCO-style prefill: the self-decoder over the prompt x [B, T,
    d_model] (bf16), its final full-attention layer writing the shared cache
    kcache / vcache [B, Hkv, L, D] at positions 0 .. T-1, then the
    cross-decoder on the last prompt token.

    self_layers: sequence of dicts, kind "mamba" (key "w": the weights dict of
    mamba_decode_step; "conv_state", "ssm_state": float32 states, in and
    out), "swa" (wq, wk, wv, wo; "kring", "vring": [B, Hkv, window, D] ring
    caches, written) or "attn" (wq, wk, wv, wo); each with optional norm1,
    norm2, w_gate, w_up, w_down.  cross_layers: as crossdecoder_step_ex.
    Calling it returns (h_out [B, d_model], M_last [B, d_inner]), bf16."""

    def __init__(self, x, self_layers: Sequence, cross_layers: Sequence, kcache, vcache, window: int = 0,
                 eps: float = 1e-5, scale: float | None = None, h_out=None, M_out=None):
        dev = _check_device(x, "x")
        bf = torch.bfloat16
        if x.dim() != 3 or kcache.dim() != 4 or vcache.shape != kcache.shape:
            raise ValueError("x [B, T, d_model], kcache and vcache [B, Hkv, L, D]")
        B, T, d_model = x.shape
        B2, Hkv, L, D = kcache.shape
        if B2 != B or d_model % D != 0:
            raise ValueError("sambay_prefill shape mismatch")
        Hq = d_model // D
        arr, (d_inner, d_state, dt_rank, d_conv), d_ff = _self_layer_array(self_layers, cross_layers, dev, B, d_model,
                                                                           Hkv, D, window)
        self.cross = _layer_ex_array(cross_layers, dev, d_model, d_inner, d_ff)
        self.self_arr = arr
        self.h_out = h_out if h_out is not None else torch.empty((B, d_model), dtype=bf, device=dev)
        self.M_out = M_out if M_out is not None else torch.empty((B, d_inner), dtype=bf, device=dev)
        self.tensors = (x, self_layers, cross_layers, kcache, vcache)
        self.ptrs = (_dev_ptr(x, "x", bf, dev), _dev_ptr(self.h_out, "h_out", bf, dev),
                     _dev_ptr(self.M_out, "M_out", bf, dev))
        self.kv = (_dev_ptr(kcache, "kcache", bf, dev), _dev_ptr(vcache, "vcache", bf, dev))
        self.n = (len(self_layers), len(cross_layers))
        self.dims = (B, T, d_model, d_inner, d_state, dt_rank, d_conv, d_ff, Hq, Hkv, D, L)
        self.window = int(window)
        self.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
        self.eps = float(eps)
        nb = lib.sambay_prefill_workspace_bytes(*self.dims)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.device = dev

    def __call__(self):
        st = lib.sambay_prefill(*self.ptrs, self.self_arr, self.n[0], self.cross, self.n[1], *self.kv, *self.dims,
                                self.window, self.scale, self.eps, self.ws.data_ptr(), self.ws.numel(),
                                _stream(self.device))
        _check("sambay_prefill", st)
        return self.h_out, self.M_out


def sambay_prefill(x, self_layers: Sequence, cross_layers: Sequence, kcache, vcache, window: int = 0,
                   eps: float = 1e-5, scale: float | None = None):
    """YOCO-style prefill (see SambayPrefill); returns (h_out, M_last)."""
    return SambayPrefill(x, self_layers, cross_layers, kcache, vcache, window, eps, scale)()


class SambayDecodeStep:
    """Prepared whole-model decode step (after sambay_prefill): h [B, d_model]
    bf16 holds each sequence's new token row and receives its last hidden
    state; pos [B] int32 (device) the token positions.  Layers, caches and
    states as for SambayPrefill (the same dicts).  Calling it returns
    (h, M_last)."""

    def __init__(self, h, pos, self_layers: Sequence, cross_layers: Sequence, kcache, vcache, window: int = 0,
                 eps: float = 1e-5, scale: float | None = None, M_out=None):
        dev = _check_device(h, "h")
        bf = torch.bfloat16
        if h.dim() != 2 or kcache.dim() != 4 or vcache.shape != kcache.shape:
            raise ValueError("h [B, d_model], kcache and vcache [B, Hkv, L, D]")
        B, d_model = h.shape
        B2, Hkv, L, D = kcache.shape
        if B2 != B or d_model % D != 0 or pos.shape != (B,):
            raise ValueError("sambay_decode_step shape mismatch")
        Hq = d_model // D
        arr, (d_inner, d_state, dt_rank, d_conv), d_ff = _self_layer_array(self_layers, cross_layers, dev, B, d_model,
                                                                           Hkv, D, window)
        self.cross = _layer_ex_array(cross_layers, dev, d_model, d_inner, d_ff)
        self.self_arr = arr
        self.M_out = M_out if M_out is not None else torch.empty((B, d_inner), dtype=bf, device=dev)
        self.tensors = (h, pos, self_layers, cross_layers, kcache, vcache)
        self.ptrs = (_dev_ptr(h, "h", bf, dev), _dev_ptr(self.M_out, "M_out", bf, dev))
        self.kv = (_dev_ptr(kcache, "kcache", bf, dev), _dev_ptr(vcache, "vcache", bf, dev),
                   _dev_ptr(pos, "pos", torch.int32, dev))
        self.n = (len(self_layers), len(cross_layers))
        self.dims = (B, d_model, d_inner, d_state, dt_rank, d_conv, d_ff, Hq, Hkv, D, L)
        self.window = int(window)
        self.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
        self.eps = float(eps)
        nb = lib.sambay_decode_workspace_bytes(*self.dims, self.window)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.device = dev

    def __call__(self):
        st = lib.sambay_decode_step(*self.ptrs, self.self_arr, self.n[0], self.cross, self.n[1], *self.kv,
                                    *self.dims, self.window, self.scale, self.eps, self.ws.data_ptr(),
                                    self.ws.numel(), _stream(self.device))
        _check("sambay_decode_step", st)
        return self.tensors[0], self.M_out


def sambay_decode_step(h, pos, self_layers: Sequence, cross_layers: Sequence, kcache, vcache, window: int = 0,
                       eps: float = 1e-5, scale: float | None = None):
    """Whole-model decode step (see SambayDecodeStep); returns (h, M_last)."""
    return SambayDecodeStep(h, pos, self_layers, cross_layers, kcache, vcache, window, eps, scale)()


__all__ = ["gmu_forward", "xattn_decode", "diffattn_decode", "selfattn_decode", "mamba_decode_step",
           "attn_prefill", "mamba_prefill", "sambay_prefill", "SambayPrefill", "sambay_decode_step",
           "SambayDecodeStep",
           "crossdecoder_step", "CrossDecoderStep", "crossdecoder_step_ex",
           "CrossDecoderStepEx", "SambayError", "version", "lib",
           "EXPORTS", "LIB_PATH", "timing_enable", "timing_collect", "probe_stream_read_gbps", "probe_mfma_tflops",
           "probe_stream_read_raw"]
