"""Plain fp64 CPU oracle for the SambaY cross-decoder step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use this package; the product library never does.  It
shares no code with the HIP path.  The arithmetic lives in ``oracle.c``
(plain double-precision loops, one function per definition on the pages);
this module only builds it with gcc, marshals numpy/torch CPU arrays and
returns float64 numpy arrays.

Accepted input arrays: numpy float64 / float32, numpy uint16 holding raw
bfloat16 bit patterns, or CPU torch tensors of dtype float64 / float32 /
bfloat16.  bfloat16 and float32 values are widened exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16 = 0, 1, 2
CATEGORIES = ("kv_cache", "state_in", "state_out", "weights")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.oracle_gmu.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i64, i64, i64, vp]
    lib.oracle_gmu.restype = ctypes.c_int
    lib.oracle_xattn.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i64, i64, i64, i64, i64, dbl, vp]
    lib.oracle_xattn.restype = ctypes.c_int
    lib.oracle_xattn_chunked.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i64, i64, i64, i64, i64, dbl,
                                         i64]
    lib.oracle_xattn_chunked.restype = ctypes.c_int
    lib.oracle_crossdecoder.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i32,
                                        i64, i64, i64, i64, i64, i64, i64, dbl, ctypes.c_int, vp, vp]
    lib.oracle_crossdecoder.restype = ctypes.c_int
    lib.oracle_xattn_varlen.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, i64, i64, i64, i64, i64, dbl]
    lib.oracle_xattn_varlen.restype = ctypes.c_int
    lib.oracle_rmsnorm.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64, dbl, vp]
    lib.oracle_rmsnorm.restype = ctypes.c_int
    lib.oracle_swiglu.argtypes = [vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
    lib.oracle_swiglu.restype = ctypes.c_int
    lib.oracle_crossdecoder_ex.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp,
                                           vp, vp, ctypes.c_int, i32, i64, i64, i64, i64, i64, i64, i64, i64, dbl,
                                           dbl, ctypes.c_int, vp]
    lib.oracle_crossdecoder_ex.restype = ctypes.c_int
    lib.oracle_diffattn.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i64, i64,
                                    i64, i64, i64, dbl, dbl, dbl, dbl]
    lib.oracle_diffattn.restype = ctypes.c_int
    lib.oracle_selfattn.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                    i64, i64, i64, i64, i64, i64, dbl]
    lib.oracle_selfattn.restype = ctypes.c_int
    lib.oracle_mamba_step.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp,
                                      ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64]
    lib.oracle_mamba_step.restype = ctypes.c_int
    lib.oracle_attn_prefill.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i64, i64, i64, i64, i64, i64,
                                        dbl]
    lib.oracle_attn_prefill.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [dbl]
    lib.oracle_round_bf16.restype = dbl
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _as_input(a):
    """Return (contiguous numpy array, dtype code) for an accepted input."""
    if not isinstance(a, np.ndarray):
        import torch  # only for CPU tensors handed in by the tests / bench

        if not isinstance(a, torch.Tensor):
            a = np.asarray(a, dtype=np.float64)
        else:
            t = a.detach()
            if t.device.type != "cpu":
                raise ValueError("oracle inputs must be CPU arrays")
            t = t.contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            if t.dtype == torch.float32:
                return t.numpy(), F32
            if t.dtype == torch.float64:
                return t.numpy(), F64
            raise TypeError("unsupported oracle input dtype %s" % t.dtype)
    a = np.ascontiguousarray(a)
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("unsupported oracle input dtype %s" % a.dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc == -1:
        raise ValueError("oracle %s: invalid arguments" % what)
    if rc != 0:
        raise MemoryError("oracle %s: allocation failed (%d)" % (what, rc))


def _bytes_dict(arr):
    return {c: int(arr[i]) for i, c in enumerate(CATEGORIES)}


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def round_bf16(x) -> np.ndarray:
    """Round each value of x (float64) to the nearest bfloat16, ties to even."""
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_round_bf16(float(flat_in[i]))
    return out


def gmu(M, X, W1, W2, count_bytes: bool = False):
    """Y = (M ⊙ SiLU(X W1^T)) W2^T in fp64.  M [rows, d_inner], X [rows, d_model],
    W1 [d_inner, d_model], W2 [d_model, d_inner].  M and X share a dtype."""
    lib = _load()
    m, dm = _as_input(M)
    x, dx = _as_input(X)
    w1, dw1 = _as_input(W1)
    w2, dw2 = _as_input(W2)
    if dm != dx or dw1 != dw2:
        raise TypeError("M/X and W1/W2 must share dtypes")
    rows, d_model = x.shape
    d_inner = w1.shape[0]
    if m.shape != (rows, d_inner) or w1.shape != (d_inner, d_model) or w2.shape != (d_model, d_inner):
        raise ValueError("gmu shape mismatch")
    y = np.empty((rows, d_model), dtype=np.float64)
    nb = np.zeros(4, dtype=np.int64)
    rc = lib.oracle_gmu(_ptr(m), _ptr(x), dm, _ptr(w1), _ptr(w2), dw1, _ptr(y), rows, d_model, d_inner,
                        _ptr(nb) if count_bytes else None)
    _check(rc, "gmu")
    return (y, _bytes_dict(nb)) if count_bytes else y


def _xattn_shapes(q, k, v):
    B, Hq, D = q.shape
    B2, Hkv, L, D2 = k.shape
    if v.shape != k.shape or B2 != B or D2 != D:
        raise ValueError("xattn shape mismatch")
    return B, Hq, Hkv, D, L


def xattn(q, K, V, scale: float | None = None, count_bytes: bool = False):
    """out[B, Hq, D] = softmax(scale q K^T) V over all L positions; K, V [B, Hkv, L, D]."""
    lib = _load()
    qa, dq = _as_input(q)
    ka, dk = _as_input(K)
    va, dv = _as_input(V)
    if dk != dv:
        raise TypeError("K and V must share a dtype")
    B, Hq, Hkv, D, L = _xattn_shapes(qa, ka, va)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    nb = np.zeros(4, dtype=np.int64)
    rc = lib.oracle_xattn(_ptr(qa), dq, _ptr(ka), _ptr(va), dk, _ptr(out), B, Hq, Hkv, D, L, float(scale),
                          _ptr(nb) if count_bytes else None)
    _check(rc, "xattn")
    return (out, _bytes_dict(nb)) if count_bytes else out


def xattn_chunked(q, K, V, S: int, scale: float | None = None):
    """The same attention as S key chunks merged by log-sum-exp."""
    lib = _load()
    qa, dq = _as_input(q)
    ka, dk = _as_input(K)
    va, dv = _as_input(V)
    B, Hq, Hkv, D, L = _xattn_shapes(qa, ka, va)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = lib.oracle_xattn_chunked(_ptr(qa), dq, _ptr(ka), _ptr(va), dk, _ptr(out), B, Hq, Hkv, D, L, float(scale),
                                  int(S))
    _check(rc, "xattn_chunked")
    return out


XATTN, GMU = 0, 1


def crossdecoder(h, M, K, V, layers: Sequence, Hq: int, scale: float | None = None, round_bf16: bool = True,
                 count_bytes: bool = False):
    """One cross-decoder decode step.  layers: sequence of (kind, w_a, w_b) with
    kind "xattn" (w_a = Wq, w_b = Wo, [d_model, d_model]) or "gmu"
    (w_a = W1 [d_inner, d_model], w_b = W2 [d_model, d_inner]).
    h [B, d_model], M [B, d_inner], K, V [B, Hkv, L, D]; Hq·D == d_model.
    Returns the final h (float64) and, with count_bytes, a per-layer list of
    byte dicts."""
    lib = _load()
    ha, dh = _as_input(h)
    ma, dm = _as_input(M)
    ka, dk = _as_input(K)
    va, dv = _as_input(V)
    if dh != dm or dk != dv:
        raise TypeError("h/M and K/V must share dtypes")
    B, d_model = ha.shape
    d_inner = ma.shape[1]
    B2, Hkv, L, D = ka.shape
    if B2 != B or ma.shape[0] != B or va.shape != ka.shape or Hq * D != d_model:
        raise ValueError("crossdecoder shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    n = len(layers)
    kinds = np.zeros(max(n, 1), dtype=np.int32)
    keep, wa_p, wb_p = [], (ctypes.c_void_p * max(n, 1))(), (ctypes.c_void_p * max(n, 1))()
    dw = None
    for i, (kind, wa, wb) in enumerate(layers):
        if kind not in ("xattn", "gmu"):
            raise ValueError("layer kind must be 'xattn' or 'gmu'")
        kinds[i] = XATTN if kind == "xattn" else GMU
        a, da = _as_input(wa)
        b, db = _as_input(wb)
        if dw is None:
            dw = da
        if da != dw or db != dw:
            raise TypeError("all layer weights must share a dtype")
        if kind == "xattn":
            ok = a.shape == (d_model, d_model) and b.shape == (d_model, d_model)
        else:
            ok = a.shape == (d_inner, d_model) and b.shape == (d_model, d_inner)
        if not ok:
            raise ValueError("layer %d weight shape mismatch" % i)
        keep += [a, b]
        wa_p[i] = a.ctypes.data
        wb_p[i] = b.ctypes.data
    out = np.empty((B, d_model), dtype=np.float64)
    nb = np.zeros((max(n, 1), 4), dtype=np.int64)
    rc = lib.oracle_crossdecoder(_ptr(ha), _ptr(ma), dh, _ptr(ka), _ptr(va), dk, _ptr(kinds),
                                 ctypes.cast(wa_p, ctypes.c_void_p), ctypes.cast(wb_p, ctypes.c_void_p),
                                 dw if dw is not None else F64, n, B, d_model, d_inner, Hq, Hkv, D, L, float(scale),
                                 1 if round_bf16 else 0, _ptr(out), _ptr(nb) if count_bytes else None)
    _check(rc, "crossdecoder")
    if count_bytes:
        return out, [_bytes_dict(nb[i]) for i in range(n)]
    return out


def _lens_array(lens, B: int, L: int) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(lens.cpu() if hasattr(lens, "cpu") else lens), dtype=np.int32)
    if a.shape != (B,):
        raise ValueError("lens must have one entry per sequence")
    if a.min(initial=0) < 0 or a.max(initial=0) > L:
        raise ValueError("lens must lie in [0, L]")
    return a


def xattn_varlen(q, K, V, lens, scale: float | None = None):
    """Ragged-batch attention: sequence b attends to its first lens[b] of the L
    cached positions (lens[b] == 0 gives zeros).  K, V [B, Hkv, L, D]."""
    lib = _load()
    qa, dq = _as_input(q)
    ka, dk = _as_input(K)
    va, dv = _as_input(V)
    if dk != dv:
        raise TypeError("K and V must share a dtype")
    B, Hq, Hkv, D, L = _xattn_shapes(qa, ka, va)
    la = _lens_array(lens, B, L)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = lib.oracle_xattn_varlen(_ptr(qa), dq, _ptr(ka), _ptr(va), dk, _ptr(la), _ptr(out), B, Hq, Hkv, D, L,
                                 float(scale))
    _check(rc, "xattn_varlen")
    return out


def diffattn(q, K, V, lam: float, lam_init: float, gamma=None, lens=None, eps: float = 1e-5,
             scale: float | None = None):
    """Differential attention decode over a shared GQA cache.

    Each D-wide query / key row is two halves (q1 | q2), (k1 | k2); value rows
    keep all D.  out = (1 - lam_init) * RMSNorm(softmax(scale q1 k1^T) V
    - lam * softmax(scale q2 k2^T) V) * gamma per head; scale defaults to
    1/sqrt(D/2); gamma None means ones; lens as in xattn_varlen."""
    lib = _load()
    qa, dq = _as_input(q)
    ka, dk = _as_input(K)
    va, dv = _as_input(V)
    if dk != dv:
        raise TypeError("K and V must share a dtype")
    B, Hq, Hkv, D, L = _xattn_shapes(qa, ka, va)
    la = None if lens is None else _lens_array(lens, B, L)
    ga, dg = (None, F64) if gamma is None else _as_input(gamma)
    if ga is not None and ga.shape != (D,):
        raise ValueError("gamma must have D entries")
    if scale is None:
        scale = 1.0 / np.sqrt(D // 2)
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = lib.oracle_diffattn(_ptr(qa), dq, _ptr(ka), _ptr(va), dk, None if la is None else _ptr(la),
                             None if ga is None else _ptr(ga), dg, _ptr(out), B, Hq, Hkv, D, L, float(scale),
                             float(lam), float(lam_init), float(eps))
    _check(rc, "diffattn")
    return out


def selfattn(q, k_new, v_new, K, V, pos, window: int = 0, scale: float | None = None):
    """One decode step of a self-decoder attention layer: store each active
    sequence's new key/value rows (k_new, v_new [B, Hkv, D]) at position
    pos[b] (window 0: cache [B, Hkv, L, D] with room for L positions) or in
    ring slot pos[b] % window (cache of window slots), then attend over the
    visible positions (0 .. pos[b], or the window most recent tokens).
    pos[b] < 0: inactive (nothing stored, zero output).  Returns (out, K_out,
    V_out), the updated cache in float64."""
    lib = _load()
    qa, dq = _as_input(q)
    ka, dk = _as_input(K)
    va, dv = _as_input(V)
    kn, dn = _as_input(k_new)
    vn, dn2 = _as_input(v_new)
    if dk != dv or dn != dn2:
        raise TypeError("K and V (and k_new and v_new) must share a dtype")
    B, Hq, Hkv, D, L = _xattn_shapes(qa, ka, va)
    if kn.shape != (B, Hkv, D) or vn.shape != (B, Hkv, D):
        raise ValueError("k_new and v_new must be [B, Hkv, D]")
    pa = np.ascontiguousarray(np.asarray(pos.cpu() if hasattr(pos, "cpu") else pos), dtype=np.int32)
    if pa.shape != (B,):
        raise ValueError("pos must have one entry per sequence")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    Ko = np.empty((B, Hkv, L, D), dtype=np.float64)
    Vo = np.empty((B, Hkv, L, D), dtype=np.float64)
    rc = lib.oracle_selfattn(_ptr(qa), dq, _ptr(kn), _ptr(vn), dn, _ptr(ka), _ptr(va), dk, _ptr(pa), _ptr(out),
                             _ptr(Ko), _ptr(Vo), B, Hq, Hkv, D, L, int(window), float(scale))
    _check(rc, "selfattn")
    return out, Ko, Vo


MAMBA_KEYS = ("W_in", "W_x", "W_dt", "W_out", "conv_w", "conv_b", "dt_bias", "A_log", "D")


def mamba_step(x, w: dict, conv_state, ssm_state):
    """One decode step of a Mamba layer for B sequences.

    x [B, d_model]; w: W_in [2 d_inner, d_model], W_x [R + 2N, d_inner],
    W_dt [d_inner, R], W_out [d_model, d_inner] (one dtype), conv_w
    [d_inner, K], conv_b, dt_bias, D [d_inner], A_log [d_inner, N] (one dtype);
    conv_state [B, d_inner, K - 1], ssm_state [B, d_inner, N].
    Returns (M [B, d_inner], y [B, d_model], conv_state', ssm_state'), float64."""
    lib = _load()
    xa, dx = _as_input(x)
    arr = {k: _as_input(w[k]) for k in MAMBA_KEYS}
    dw = {arr[k][1] for k in ("W_in", "W_x", "W_dt", "W_out")}
    dp = {arr[k][1] for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D")}
    if len(dw) != 1 or len(dp) != 1:
        raise TypeError("matrices must share a dtype, and so must the per-channel parameters")
    ca, dc = _as_input(conv_state)
    sa, ds = _as_input(ssm_state)
    if dc != ds:
        raise TypeError("states must share a dtype")
    B, d_model = xa.shape
    d_inner, K = arr["conv_w"][0].shape
    N = arr["A_log"][0].shape[1]
    R = arr["W_dt"][0].shape[1]
    shapes = {"W_in": (2 * d_inner, d_model), "W_x": (R + 2 * N, d_inner), "W_dt": (d_inner, R),
              "W_out": (d_model, d_inner), "conv_b": (d_inner,), "dt_bias": (d_inner,), "A_log": (d_inner, N),
              "D": (d_inner,)}
    for k, shp in shapes.items():
        if arr[k][0].shape != shp:
            raise ValueError("%s has shape %s, expected %s" % (k, arr[k][0].shape, shp))
    if ca.shape != (B, d_inner, K - 1) or sa.shape != (B, d_inner, N):
        raise ValueError("state shape mismatch")
    M = np.empty((B, d_inner), dtype=np.float64)
    y = np.empty((B, d_model), dtype=np.float64)
    co = np.empty((B, d_inner, K - 1), dtype=np.float64)
    so = np.empty((B, d_inner, N), dtype=np.float64)
    a = {k: _ptr(arr[k][0]) for k in MAMBA_KEYS}
    rc = lib.oracle_mamba_step(_ptr(xa), dx, a["W_in"], a["W_x"], a["W_dt"], a["W_out"], dw.pop(), a["conv_w"],
                               a["conv_b"], a["dt_bias"], a["A_log"], a["D"], dp.pop(), _ptr(ca), _ptr(sa), dc,
                               _ptr(co), _ptr(so), _ptr(M), _ptr(y), B, d_model, d_inner, N, R, K)
    _check(rc, "mamba_step")
    return M, y, co, so


def attn_prefill(q, k, v, window: int = 0, scale: float | None = None):
    """Causal (window 0) or sliding-window causal attention of T prompt
    tokens: q [B, T, Hq, D], k, v [B, T, Hkv, D] -> out [B, T, Hq, D]; query i
    sees keys j <= i (and j > i - window when window > 0)."""
    lib = _load()
    qa, dq = _as_input(q)
    ka, dk = _as_input(k)
    va, dv = _as_input(v)
    if dk != dv:
        raise TypeError("k and v must share a dtype")
    B, T, Hq, D = qa.shape
    if ka.shape[:2] != (B, T) or ka.shape[3] != D or va.shape != ka.shape:
        raise ValueError("attn_prefill shape mismatch")
    Hkv = ka.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, T, Hq, D), dtype=np.float64)
    rc = lib.oracle_attn_prefill(_ptr(qa), dq, _ptr(ka), _ptr(va), dk, _ptr(out), B, T, Hq, Hkv, D, int(window),
                                 float(scale))
    _check(rc, "attn_prefill")
    return out


def mamba_prefill(x, w: dict, conv_state, ssm_state):
    """The Mamba layer over T tokens, x [B, T, d_model]: by definition T
    successive mamba_step calls from the given states.  Returns (M [B, T,
    d_inner], y [B, T, d_model], conv_state', ssm_state'), float64."""
    xa, _ = _as_input(x)
    if xa.ndim != 3:
        raise ValueError("x must be [B, T, d_model]")
    B, T, _ = xa.shape
    conv, ssm = conv_state, ssm_state
    Ms, ys = [], []
    for t in range(T):
        M, y, conv, ssm = mamba_step(np.ascontiguousarray(xa[:, t]), w, conv, ssm)
        Ms.append(M)
        ys.append(y)
    if T == 0:
        raise ValueError("T must be positive")
    return np.stack(Ms, axis=1), np.stack(ys, axis=1), conv, ssm


def rmsnorm(x, g, eps: float = 1e-5):
    """Row-wise RMSNorm: x / sqrt(mean(x^2) + eps) * g over the last axis."""
    lib = _load()
    xa, dx = _as_input(x)
    ga, dg = _as_input(g)
    n = xa.shape[-1]
    if ga.shape != (n,):
        raise ValueError("gain shape mismatch")
    out = np.empty(xa.shape, dtype=np.float64)
    rc = lib.oracle_rmsnorm(_ptr(xa), dx, _ptr(ga), dg, xa.size // n, n, float(eps), _ptr(out))
    _check(rc, "rmsnorm")
    return out


def swiglu(x, Wg, Wu, Wd):
    """Row-wise SwiGLU MLP: (SiLU(x Wg^T) * (x Wu^T)) Wd^T."""
    lib = _load()
    xa, dx = _as_input(x)
    ga, dg = _as_input(Wg)
    ua, du = _as_input(Wu)
    da, dd = _as_input(Wd)
    if not (dg == du == dd):
        raise TypeError("MLP weights must share a dtype")
    rows, d_model = xa.shape
    d_ff = ga.shape[0]
    if ga.shape != (d_ff, d_model) or ua.shape != (d_ff, d_model) or da.shape != (d_model, d_ff):
        raise ValueError("MLP weight shape mismatch")
    out = np.empty((rows, d_model), dtype=np.float64)
    rc = lib.oracle_swiglu(_ptr(xa), dx, _ptr(ga), _ptr(ua), _ptr(da), dg, rows, d_model, d_ff, _ptr(out))
    _check(rc, "swiglu")
    return out


def crossdecoder_ex(h, M, K, V, layers: Sequence, Hq: int, lens=None, eps: float = 1e-5,
                    scale: float | None = None, round_bf16: bool = True):
    """One decode step of the complete cross-decoder (pre-RMSNorm mixer, optional
    pre-RMSNorm SwiGLU MLP, ragged cache lengths).  layers: sequence of dicts with
    keys kind ("xattn" or "gmu"), w_a, w_b and optional norm1, norm2, w_gate,
    w_up, w_down (absent or None: no norm / no MLP).  lens: None or [B] ints in
    [0, L].  Returns the final h (float64)."""
    lib = _load()
    ha, dh = _as_input(h)
    ma, dm = _as_input(M)
    ka, dk = _as_input(K)
    va, dv = _as_input(V)
    if dh != dm or dk != dv:
        raise TypeError("h/M and K/V must share dtypes")
    B, d_model = ha.shape
    d_inner = ma.shape[1]
    B2, Hkv, L, D = ka.shape
    if B2 != B or ma.shape[0] != B or va.shape != ka.shape or Hq * D != d_model:
        raise ValueError("crossdecoder shape mismatch")
    la = _lens_array(lens, B, L) if lens is not None else None
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    n = len(layers)
    N = max(n, 1)
    kinds = np.zeros(N, dtype=np.int32)
    ptrs = {k: (ctypes.c_void_p * N)() for k in ("w_a", "w_b", "norm1", "norm2", "w_gate", "w_up", "w_down")}
    keep, dw, d_ff = [], None, 0
    for i, ly in enumerate(layers):
        kind = ly["kind"]
        if kind not in ("xattn", "gmu"):
            raise ValueError("layer kind must be 'xattn' or 'gmu'")
        kinds[i] = XATTN if kind == "xattn" else GMU
        for key in ptrs:
            t = ly.get(key)
            if t is None:
                continue
            a, da = _as_input(t)
            if dw is None:
                dw = da
            if da != dw:
                raise TypeError("all layer weights must share a dtype")
            if key == "w_gate":
                if d_ff and a.shape[0] != d_ff:
                    raise ValueError("all MLPs must share d_ff")
                d_ff = a.shape[0]
            keep.append(a)
            ptrs[key][i] = a.ctypes.data
    out = np.empty((B, d_model), dtype=np.float64)
    c = lambda k: ctypes.cast(ptrs[k], ctypes.c_void_p)
    rc = lib.oracle_crossdecoder_ex(_ptr(ha), _ptr(ma), dh, _ptr(ka), _ptr(va), dk,
                                    _ptr(la) if la is not None else None, _ptr(kinds), c("w_a"), c("w_b"),
                                    c("norm1"), c("norm2"), c("w_gate"), c("w_up"), c("w_down"),
                                    dw if dw is not None else F64, n, B, d_model, d_inner, d_ff, Hq, Hkv, D, L,
                                    float(scale), float(eps), 1 if round_bf16 else 0, _ptr(out))
    _check(rc, "crossdecoder_ex")
    return out


def round_bf16_array(x) -> np.ndarray:
    """round_bf16 for whole arrays: the nearest value with an 8-bit
    significand (1 + 7 stored bits), ties to even; for the O(1) magnitudes of
    activations (no bfloat16 overflow or subnormal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m · 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def _f64(a) -> np.ndarray:
    """An accepted input widened exactly to float64 (bfloat16 bit patterns
    become the values they encode: the high half of a float32)."""
    arr, code = _as_input(a)
    if code == BF16:
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.array(arr, dtype=np.float64)


def sambay_prefill(x, self_layers: Sequence, cross_layers: Sequence, Hq: int, Hkv: int, window: int = 0,
                   eps: float = 1e-5, scale: float | None = None, round_h: bool = True) -> dict:
    """YOCO-style prefill ([Notes] 整体框架): the self-decoder over the prompt
    x [B, T, d_model], its final full-attention layer's keys and values as
    the shared cache, then the cross-decoder on the last prompt token.

    Self-decoder layer (plain pre-norm reading, as the complete
    cross-decoder layer): x = RMSNorm(h; norm1) or h; kind "mamba": (M, y)
    = mamba_prefill(x) from the layer's states, h = h + y; "swa" / "attn":
    q, k, v = x Wq^T, x Wk^T, x Wv^T, o = attn_prefill(q, k, v, window or
    0), h = h + o Wo^T; then, with an MLP, h = h + swiglu(RMSNorm(h; norm2)).
    round_h: round h to bfloat16 after every residual add (the bf16
    residual stream), also inside the cross-decoder.  Dict keys of the
    layers as in the library's binding (tensors on the CPU); D = d_model /
    Hq.

    Returns a dict: h_out [B, d_model] (the last token after the
    cross-decoder), h_last (the same token after the self-decoder), M_last
    [B, d_inner] (the last SSM layer's memory at that token), K, V [B, Hkv,
    T, D] (the cache rows the last full-attention layer writes), per layer
    "layers": {"k", "v"} token-major for attention layers or {"conv_state",
    "ssm_state"} for SSM layers, all float64."""
    h = _f64(x)
    if h.ndim != 3:
        raise ValueError("x must be [B, T, d_model]")
    B, T, dm = h.shape
    D = dm // Hq
    if Hq * D != dm or Hq % Hkv != 0:
        raise ValueError("head shape mismatch")
    rnd = round_bf16_array if round_h else (lambda a: a)
    h = rnd(h)
    M_mem, K, V, per_layer = None, None, None, []
    for ly in self_layers:
        kind = ly["kind"]
        xin = rmsnorm(h.reshape(B * T, dm), ly["norm1"], eps).reshape(B, T, dm) if ly.get("norm1") is not None else h
        if kind == "mamba":
            M, y, conv, ssm = mamba_prefill(xin, ly["w"], ly["conv_state"], ly["ssm_state"])
            h = rnd(h + y)
            M_mem = M
            per_layer.append({"conv_state": conv, "ssm_state": ssm})
        elif kind in ("swa", "attn"):
            q = (xin @ _f64(ly["wq"]).T).reshape(B, T, Hq, D)
            k = (xin @ _f64(ly["wk"]).T).reshape(B, T, Hkv, D)
            v = (xin @ _f64(ly["wv"]).T).reshape(B, T, Hkv, D)
            o = attn_prefill(q, k, v, window if kind == "swa" else 0, scale)
            h = rnd(h + o.reshape(B, T, dm) @ _f64(ly["wo"]).T)
            per_layer.append({"k": k, "v": v})
            if kind == "attn":
                K, V = np.ascontiguousarray(k.transpose(0, 2, 1, 3)), np.ascontiguousarray(v.transpose(0, 2, 1, 3))
        else:
            raise ValueError("self layer kind must be 'mamba', 'swa' or 'attn'")
        if ly.get("w_gate") is not None:
            xm = rmsnorm(h.reshape(B * T, dm), ly["norm2"], eps) if ly.get("norm2") is not None \
                else h.reshape(B * T, dm)
            h = rnd(h + swiglu(xm, ly["w_gate"], ly["w_up"], ly["w_down"]).reshape(B, T, dm))
    h_last = np.ascontiguousarray(h[:, T - 1])
    M_last = np.ascontiguousarray(M_mem[:, T - 1]) if M_mem is not None else None
    h_out = h_last
    if cross_layers:
        h_out = crossdecoder_ex(h_last, M_last if M_last is not None else np.zeros((B, 1)), K, V, cross_layers, Hq,
                                eps=eps, scale=scale, round_bf16=round_h)
    return {"h_out": h_out, "h_last": h_last, "M_last": M_last, "K": K, "V": V, "layers": per_layer}


def sambay_decode_step(x, self_layers: Sequence, cross_layers: Sequence, Hq: int, Hkv: int, pos, K, V,
                       window: int = 0, eps: float = 1e-5, scale: float | None = None, round_h: bool = True) -> dict:
    """One decode step of the whole model: the new token rows x [B, d_model]
    at positions pos [B] through the self-decoder's layers, one step each
    (the layers of sambay_prefill: mamba_step on the layer's states, selfattn
    on its ring of `window` slots or on the shared cache K, V [B, Hkv, L,
    D]), then crossdecoder_ex with cache lengths min(pos + 1, L).  Layer
    dicts as for sambay_prefill, with each SSM layer's conv_state /
    ssm_state and each sliding-window layer's kring / vring (CPU arrays)
    as the state before the step.

    Returns a dict: h_out [B, d_model], h_self (after the self-decoder),
    M_last, K, V (the shared cache after the step), per layer "layers":
    {conv_state, ssm_state} or {kring, vring} after the step, float64."""
    h = _f64(x)
    if h.ndim != 2:
        raise ValueError("x must be [B, d_model]")
    B, dm = h.shape
    D = dm // Hq
    rnd = round_bf16_array if round_h else (lambda a: a)
    h = rnd(h)
    pa = np.ascontiguousarray(np.asarray(pos.cpu() if hasattr(pos, "cpu") else pos), dtype=np.int32)
    Kc, Vc = _f64(K), _f64(V)
    L = Kc.shape[2]
    M_mem, per_layer = None, []
    for ly in self_layers:
        kind = ly["kind"]
        xin = rmsnorm(h, ly["norm1"], eps) if ly.get("norm1") is not None else h
        if kind == "mamba":
            M, y, cs, ss = mamba_step(xin, ly["w"], ly["conv_state"], ly["ssm_state"])
            h = rnd(h + y)
            M_mem = M
            per_layer.append({"conv_state": cs, "ssm_state": ss})
        elif kind in ("swa", "attn"):
            q = (xin @ _f64(ly["wq"]).T).reshape(B, Hq, D)
            kn = (xin @ _f64(ly["wk"]).T).reshape(B, Hkv, D)
            vn = (xin @ _f64(ly["wv"]).T).reshape(B, Hkv, D)
            if kind == "swa":
                o, kr, vr = selfattn(q, kn, vn, ly["kring"], ly["vring"], pa, window=window, scale=scale)
                per_layer.append({"kring": kr, "vring": vr})
            else:
                o, Kc, Vc = selfattn(q, kn, vn, Kc, Vc, pa, window=0, scale=scale)
                per_layer.append({})
            h = rnd(h + o.reshape(B, dm) @ _f64(ly["wo"]).T)
        else:
            raise ValueError("self layer kind must be 'mamba', 'swa' or 'attn'")
        if ly.get("w_gate") is not None:
            xm = rmsnorm(h, ly["norm2"], eps) if ly.get("norm2") is not None else h
            h = rnd(h + swiglu(xm, ly["w_gate"], ly["w_up"], ly["w_down"]))
    h_self = h
    h_out = h
    if cross_layers:
        lens = np.minimum(np.maximum(pa.astype(np.int64) + 1, 0), L)
        h_out = crossdecoder_ex(h, M_mem if M_mem is not None else np.zeros((B, 1)), Kc, Vc, cross_layers, Hq,
                                lens=lens, eps=eps, scale=scale, round_bf16=round_h)
    return {"h_out": h_out, "h_self": h_self, "M_last": M_mem, "K": Kc, "V": Vc, "layers": per_layer}
