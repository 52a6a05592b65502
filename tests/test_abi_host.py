"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function include/sambay.h declares, and
reject every invalid argument with the documented status before touching the
device.  Fake device addresses are used only on paths that fail validation,
so nothing is dereferenced or enqueued.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sambay.h")


@pytest.fixture(scope="module")
def sb():
    path = os.path.join(ROOT, "attention_decoding_amd", "libsambay.so")
    if not os.path.exists(path):
        import importlib.util
        spec = importlib.util.spec_from_file_location("sambay_build", os.path.join(ROOT, "attention_decoding_amd",
                                                                                   "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import attention_decoding_amd as sb
    return sb


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("gmu_forward", "xattn_decode", "crossdecoder_step", "gmu_workspace_bytes", "xattn_workspace_bytes",
              "crossdecoder_workspace_bytes", "sb_last_error", "sb_version"):
        assert n in names


def test_every_declared_symbol_is_exported(sb):
    raw = ctypes.CDLL(sb.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(raw, n), "symbol %s declared in sambay.h but not exported" % n
    assert sorted(sb.EXPORTS) == _declared_functions()


def test_version(sb):
    assert "gfx950" in sb.version()


A = 1 << 20  # fake, 16-byte aligned device addresses (never dereferenced)


def _addr(i):
    return A * (i + 1)


def _gmu(sb, M=_addr(0), X=_addr(1), W1=_addr(2), W2=_addr(3), Y=_addr(4), rows=4, dm=64, di=128, dt=1,
         ws=_addr(8), wsb=1 << 30):
    return sb.lib.gmu_forward(M, X, W1, W2, Y, rows, dm, di, dt, ws, wsb, None)


def test_gmu_validation(sb):
    lib = sb.lib
    assert _gmu(sb, rows=-1) == sb.SB_EINVAL
    assert _gmu(sb, dm=-64) == sb.SB_EINVAL
    assert _gmu(sb, dt=7) == sb.SB_EINVAL
    assert _gmu(sb, M=None) == sb.SB_EINVAL
    assert "null" in lib.sb_last_error().decode()
    assert _gmu(sb, Y=None) == sb.SB_EINVAL
    assert _gmu(sb, X=_addr(1) + 2) == sb.SB_EINVAL          # misaligned
    assert _gmu(sb, dm=0) == sb.SB_EINVAL
    assert _gmu(sb, Y=_addr(1)) == sb.SB_EINVAL              # Y aliases X
    assert "overlap" in lib.sb_last_error().decode()
    assert _gmu(sb, dm=96) == sb.SB_EUNSUPPORTED             # bf16 needs multiples of 64
    assert _gmu(sb, di=100) == sb.SB_EUNSUPPORTED
    assert _gmu(sb, ws=None) == sb.SB_EWORKSPACE
    need = lib.gmu_workspace_bytes(4, 64, 128, 1)
    assert need > 0
    assert _gmu(sb, wsb=need - 1) == sb.SB_EWORKSPACE
    assert _gmu(sb, ws=_addr(2), wsb=need) == sb.SB_EINVAL   # workspace overlaps W1
    # rows == 0 is a successful no-op, even with null pointers.
    assert _gmu(sb, rows=0, M=None, X=None) == sb.SB_OK
    assert lib.sb_last_error().decode() == ""


def test_gmu_workspace_sizes(sb):
    lib = sb.lib
    assert lib.gmu_workspace_bytes(0, 64, 128, 1) == 0
    assert lib.gmu_workspace_bytes(64, 64, 128, 0) >= 64 * 128 * 4          # fp32 H
    assert lib.gmu_workspace_bytes(8192, 2560, 5120, 1) >= 8192 * 5120 * 2  # bf16 H for prefill
    assert lib.gmu_workspace_bytes(32, 3072, 6144, 1) >= 32 * 6144 * 2


def _xa(sb, q=_addr(0), k=_addr(1) * 16, v=_addr(2) * 64, out=_addr(3), B=2, Hq=24, Hkv=8, D=128, L=300, scale=0.088,
        ws=_addr(4) * 512, wsb=1 << 30):
    return sb.lib.xattn_decode(q, k, v, out, B, Hq, Hkv, D, L, scale, ws, wsb, None)


def test_xattn_validation(sb):
    assert _xa(sb, B=-1) == sb.SB_EINVAL
    assert _xa(sb, L=0) == sb.SB_EINVAL
    assert _xa(sb, Hq=25) == sb.SB_EINVAL                     # Hq % Hkv != 0
    assert _xa(sb, Hkv=0) == sb.SB_EINVAL
    assert _xa(sb, D=64) == sb.SB_EUNSUPPORTED
    assert _xa(sb, Hq=136, Hkv=8) == sb.SB_EUNSUPPORTED       # group of 17 heads
    assert _xa(sb, L=1 << 31) == sb.SB_EUNSUPPORTED
    assert _xa(sb, q=None) == sb.SB_EINVAL
    assert _xa(sb, out=_addr(0)) == sb.SB_EINVAL              # out aliases q
    assert _xa(sb, k=_addr(1) * 16 + 8) == sb.SB_EINVAL       # misaligned
    assert _xa(sb, scale=float("nan")) == sb.SB_EINVAL
    assert _xa(sb, scale=float("inf")) == sb.SB_EINVAL
    assert _xa(sb, ws=None) == sb.SB_EWORKSPACE
    need = sb.lib.xattn_workspace_bytes(2, 24, 8, 128, 300)
    assert need > 0
    assert _xa(sb, wsb=need - 1) == sb.SB_EWORKSPACE
    assert _xa(sb, B=0, q=None, k=None) == sb.SB_OK


def test_xattn_workspace_sizes(sb):
    lib = sb.lib
    assert lib.xattn_workspace_bytes(16, 24, 8, 128, 34816) >= 16 * 24 * (128 + 2) * 4
    assert lib.xattn_workspace_bytes(16, 24, 8, 64, 34816) == 0
    assert lib.xattn_workspace_bytes(0, 24, 8, 128, 34816) == 0


def _step(sb, layers, n=None, h=_addr(0), M=_addr(1), k=_addr(2) * 16, v=_addr(3) * 64, B=2, dm=3072, di=6144, Hq=24,
          Hkv=8, D=128, L=300, ws=_addr(5) * 512, wsb=1 << 34):
    arr = (sb.SbLayer * max(len(layers), 1))()
    for i, (kind, wa, wb) in enumerate(layers):
        arr[i].kind, arr[i].w_a, arr[i].w_b = kind, wa, wb
    return sb.lib.crossdecoder_step(h, M, k, v, arr if layers is not None else None, len(layers) if n is None else n,
                                    B, dm, di, Hq, Hkv, D, L, 0.088, ws, wsb, None)


def test_crossdecoder_validation(sb):
    W = [(0, _addr(9) * 1024, _addr(10) * 1024), (1, _addr(11) * 1024, _addr(12) * 1024)]
    assert _step(sb, W, B=-1) == sb.SB_EINVAL
    assert _step(sb, W, n=-1) == sb.SB_EINVAL
    assert _step(sb, W, dm=3000) == sb.SB_EINVAL              # Hq*D != d_model
    assert _step(sb, W, di=6000) == sb.SB_EUNSUPPORTED
    assert _step(sb, W, D=64, dm=24 * 64) == sb.SB_EUNSUPPORTED
    assert _step(sb, [(2, _addr(9) * 1024, _addr(10) * 1024)]) == sb.SB_EINVAL   # unknown kind
    assert _step(sb, [(0, None, _addr(10) * 1024)]) == sb.SB_EINVAL              # null weight
    assert _step(sb, [(1, _addr(9) * 1024 + 4, _addr(10) * 1024)]) == sb.SB_EINVAL  # misaligned weight
    assert _step(sb, [(1, _addr(0), _addr(10) * 1024)]) == sb.SB_EINVAL          # weight overlaps h
    assert _step(sb, W, h=None) == sb.SB_EINVAL
    assert _step(sb, W, M=_addr(0)) == sb.SB_EINVAL           # h overlaps M
    assert _step(sb, W, ws=None) == sb.SB_EWORKSPACE
    need = sb.lib.crossdecoder_workspace_bytes(2, 3072, 6144, 24, 8, 128, 300)
    assert need > 0
    assert _step(sb, W, wsb=need - 1) == sb.SB_EWORKSPACE
    assert _step(sb, W, B=0) == sb.SB_OK
    assert _step(sb, [], n=0) == sb.SB_OK


def test_python_binding_refuses_cpu_tensors(sb):
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sb.gmu_forward(torch.zeros(4, 128, dtype=torch.bfloat16), x, torch.zeros(128, 64, dtype=torch.bfloat16),
                       torch.zeros(64, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        sb.xattn_decode(torch.zeros(1, 3, 128, dtype=torch.bfloat16), torch.zeros(1, 1, 5, 128, dtype=torch.bfloat16),
                        torch.zeros(1, 1, 5, 128, dtype=torch.bfloat16))


def _xav(sb, lens=_addr(6) * 8, q=_addr(0), out=_addr(3), B=2, **kw):
    k, v = kw.pop("k", _addr(1) * 16), kw.pop("v", _addr(2) * 64)
    return sb.lib.xattn_decode_varlen(q, k, v, lens, out, B, 24, 8, 128, kw.pop("L", 300), 0.088, _addr(4) * 512,
                                      1 << 30, None)


def test_xattn_varlen_validation(sb):
    assert _xav(sb, lens=None) == sb.SB_EINVAL                     # null lens
    assert _xav(sb, lens=_addr(6) * 8 + 2) == sb.SB_EINVAL         # misaligned lens
    assert _xav(sb, out=_addr(6) * 8) == sb.SB_EINVAL              # out overlaps lens
    assert "lens" in sb.lib.sb_last_error().decode()
    assert _xav(sb, L=0) == sb.SB_EINVAL
    assert _xav(sb, B=0, lens=None, q=None) == sb.SB_OK


def _step_ex(sb, layers, lens=None, B=2, dm=3072, di=6144, dff=8192, eps=1e-5, ws=_addr(5) * 512, wsb=1 << 36,
             h=_addr(0)):
    arr = (sb.SbLayerEx * max(len(layers), 1))()
    for i, ly in enumerate(layers):
        for key, val in ly.items():
            setattr(arr[i], key, val)
    return sb.lib.crossdecoder_step_ex(h, _addr(1), _addr(2) * 16, _addr(3) * 64, lens, arr, len(layers), B, dm, di,
                                       dff, 24, 8, 128, 300, 0.088, eps, ws, wsb, None)


def test_crossdecoder_ex_validation(sb):
    base = dict(kind=0, w_a=_addr(9) * 1024, w_b=_addr(10) * 1024)
    mlp = dict(base, norm1=_addr(13) * 1024, norm2=_addr(14) * 1024, w_gate=_addr(15) * 1024,
               w_up=_addr(16) * 1024, w_down=_addr(17) * 1024)
    assert _step_ex(sb, [mlp], dff=8040) == sb.SB_EUNSUPPORTED      # d_ff not a multiple of 64
    assert _step_ex(sb, [mlp], dff=0) == sb.SB_EINVAL                # MLP without d_ff
    assert _step_ex(sb, [dict(mlp, w_up=None)]) == sb.SB_EINVAL      # incomplete MLP
    assert _step_ex(sb, [dict(mlp, norm1=_addr(13) * 1024 + 2)]) == sb.SB_EINVAL   # misaligned gain
    assert _step_ex(sb, [dict(mlp, norm2=_addr(0))]) == sb.SB_EINVAL  # gain overlaps h
    assert _step_ex(sb, [mlp], eps=-1.0) == sb.SB_EINVAL
    assert _step_ex(sb, [mlp], eps=float("nan")) == sb.SB_EINVAL
    assert _step_ex(sb, [mlp], lens=_addr(6) * 8 + 1) == sb.SB_EINVAL   # misaligned lens
    assert _step_ex(sb, [mlp], lens=_addr(0)) == sb.SB_EINVAL        # lens overlaps h
    assert _step_ex(sb, [dict(base, kind=3)]) == sb.SB_EINVAL
    assert _step_ex(sb, [mlp], ws=None) == sb.SB_EWORKSPACE
    need = sb.lib.crossdecoder_ex_workspace_bytes(2, 3072, 6144, 8192, 24, 8, 128, 300)
    assert need > sb.lib.crossdecoder_workspace_bytes(2, 3072, 6144, 24, 8, 128, 300)
    assert _step_ex(sb, [mlp], wsb=need - 1) == sb.SB_EWORKSPACE
    assert _step_ex(sb, [mlp], B=0) == sb.SB_OK
    assert sb.lib.crossdecoder_ex_workspace_bytes(2, 3072, 6144, 8192, 24, 8, 128, 0) == 0


def _diff(sb, B=2, Hq=24, Hkv=8, D=128, L=300, lens=_addr(6) * 8, gamma=_addr(7) * 8, out=_addr(3), lam=0.8,
          lam_init=0.8, eps=1e-5, wsb=1 << 30):
    return sb.lib.diffattn_decode(_addr(0), _addr(1) * 16, _addr(2) * 64, lens, gamma, out, B, Hq, Hkv, D, L, 0.125,
                                  lam, lam_init, eps, _addr(4) * 512, wsb, None)


def test_diffattn_validation(sb):
    """Every call here fails validation (or is the B == 0 no-op), so the fake
    addresses are never used."""
    assert _diff(sb, Hkv=2) == sb.SB_EUNSUPPORTED                  # 2·G = 24 score columns > 16
    assert "two maps" in sb.lib.sb_last_error().decode()
    assert _diff(sb, D=64) == sb.SB_EUNSUPPORTED
    assert _diff(sb, lam=float("nan")) == sb.SB_EINVAL
    assert _diff(sb, lam_init=float("inf")) == sb.SB_EINVAL
    assert _diff(sb, eps=-1.0) == sb.SB_EINVAL
    assert _diff(sb, gamma=_addr(7) * 8 + 2) == sb.SB_EINVAL       # misaligned gamma
    assert _diff(sb, lens=_addr(6) * 8 + 2) == sb.SB_EINVAL        # misaligned lens
    assert _diff(sb, out=_addr(7) * 8) == sb.SB_EINVAL             # out overlaps gamma
    assert "gamma" in sb.lib.sb_last_error().decode()
    assert _diff(sb, wsb=16) == sb.SB_EWORKSPACE
    assert _diff(sb, L=0) == sb.SB_EINVAL
    assert _diff(sb, B=0) == sb.SB_OK


def test_diffattn_workspace_sizes(sb):
    lib = sb.lib
    # Two score columns per head: the partials of a plain decode with twice the heads.
    assert lib.diffattn_workspace_bytes(16, 24, 8, 128, 34816) == lib.xattn_workspace_bytes(16, 48, 8, 128, 34816)
    assert lib.diffattn_workspace_bytes(16, 24, 8, 64, 34816) == 0
    assert lib.diffattn_workspace_bytes(16, 24, 7, 128, 34816) == 0


def _self(sb, B=2, Hq=24, Hkv=8, D=128, L=300, window=0, pos=_addr(6) * 8, out=_addr(3), knew=_addr(7) * 8,
          kc=_addr(1) * 16, wsb=1 << 30):
    return sb.lib.selfattn_decode(_addr(0), knew, _addr(7) * 8 + 65536, kc, _addr(2) * 64, pos, out, B, Hq, Hkv, D,
                                  L, window, 0.088, _addr(4) * 512, wsb, None)


def test_selfattn_validation(sb):
    """Every call here fails validation (or is the B == 0 no-op)."""
    assert _self(sb, window=-1) == sb.SB_EINVAL
    assert _self(sb, window=8) == sb.SB_EINVAL                      # L (300) != window
    assert "window" in sb.lib.sb_last_error().decode()
    assert _self(sb, pos=None) == sb.SB_EINVAL
    assert _self(sb, pos=_addr(6) * 8 + 2) == sb.SB_EINVAL          # misaligned pos
    assert _self(sb, out=_addr(1) * 16 + 4096) == sb.SB_EINVAL      # out inside the cache
    assert _self(sb, knew=_addr(1) * 16) == sb.SB_EINVAL            # new rows inside the cache
    assert "k_new" in sb.lib.sb_last_error().decode()
    assert _self(sb, wsb=16) == sb.SB_EWORKSPACE
    assert _self(sb, D=64) == sb.SB_EUNSUPPORTED
    assert _self(sb, L=0) == sb.SB_EINVAL
    assert _self(sb, B=0) == sb.SB_OK


def test_selfattn_workspace_sizes(sb):
    lib = sb.lib
    assert lib.selfattn_workspace_bytes(32, 24, 8, 128, 256) > 256
    assert lib.selfattn_workspace_bytes(32, 24, 8, 128, 34816) >= lib.xattn_workspace_bytes(32, 24, 8, 128, 34816)
    assert lib.selfattn_workspace_bytes(32, 24, 8, 64, 256) == 0


def _mamba(sb, B=4, dm=3072, di=6144, N=16, R=192, K=4, w_over=None, M=None, y=None, wsb=1 << 34, null=None):
    G = 1 << 30          # fake, far-apart, 16-byte aligned addresses (never dereferenced)
    w = sb.SbMambaWeights(*[(i + 10) * G for i in range(9)])
    for k, v in (w_over or {}).items():
        setattr(w, k, v)
    if null:
        setattr(w, null, None)
    return sb.lib.mamba_decode_step(1 * G, ctypes.byref(w), 2 * G, 3 * G, M if M is not None else 4 * G,
                                    y if y is not None else 5 * G, B, dm, di, N, R, K, 6 * G, wsb, None)


def test_mamba_validation(sb):
    """Every call here fails validation (or is the B == 0 no-op)."""
    assert _mamba(sb, N=12) == sb.SB_EUNSUPPORTED
    assert _mamba(sb, R=191) == sb.SB_EUNSUPPORTED
    assert _mamba(sb, R=196) == sb.SB_EUNSUPPORTED                  # not a multiple of 8
    assert _mamba(sb, R=320) == sb.SB_EUNSUPPORTED
    assert _mamba(sb, K=9) == sb.SB_EUNSUPPORTED
    assert _mamba(sb, dm=100) == sb.SB_EUNSUPPORTED
    assert _mamba(sb, null="w_dt") == sb.SB_EINVAL
    assert _mamba(sb, w_over={"a_log": (15 << 30) + 4}) == sb.SB_EINVAL          # misaligned
    assert _mamba(sb, M=(3 << 30) + 256) == sb.SB_EINVAL                           # M inside ssm_state
    assert "overlaps" in sb.lib.sb_last_error().decode()
    assert _mamba(sb, y=(18 << 30) + 1024) == sb.SB_EINVAL                         # y inside w_out
    assert _mamba(sb, wsb=16) == sb.SB_EWORKSPACE
    assert _mamba(sb, dm=0) == sb.SB_EINVAL
    assert _mamba(sb, B=0) == sb.SB_OK


def test_mamba_workspace_sizes(sb):
    lib = sb.lib
    assert lib.mamba_workspace_bytes(32, 3072, 6144, 16, 192, 4) > 32 * 2 * 6144 * 4
    # token groups of at most 64 sequences reuse one workspace
    assert lib.mamba_workspace_bytes(200, 3072, 6144, 16, 192, 4) == lib.mamba_workspace_bytes(64, 3072, 6144, 16,
                                                                                                  192, 4)
    assert lib.mamba_workspace_bytes(32, 3072, 6144, 12, 192, 4) == 0


def test_attn_prefill_validation(sb):
    """Every call here fails validation (or is a no-op)."""
    lib = sb.lib
    G = 1 << 30
    call = lambda **kw: lib.attn_prefill(kw.get("q", 1 * G), 2 * G, 3 * G, kw.get("out", 4 * G), kw.get("B", 2),
                                         kw.get("T", 2048), kw.get("Hq", 24), kw.get("Hkv", 8), kw.get("D", 128),
                                         kw.get("W", 256), kw.get("scale", 0.088), kw.get("ws", 5 * G),
                                         kw.get("wsb", 1 << 30), None)
    assert call(D=64) == sb.SB_EUNSUPPORTED
    assert call(Hkv=7) == sb.SB_EINVAL
    assert call(W=-1) == sb.SB_EINVAL
    assert call(q=None) == sb.SB_EINVAL
    assert call(out=1 * G + 1024) == sb.SB_EINVAL                  # out overlaps q
    assert call(out=4 * G + 8) == sb.SB_EINVAL                     # misaligned
    assert call(scale=float("inf")) == sb.SB_EINVAL
    assert call(wsb=1024) == sb.SB_EWORKSPACE
    assert call(ws=2 * G + 4096) == sb.SB_EINVAL                   # workspace overlaps k
    assert call(T=0) == sb.SB_OK and call(B=0) == sb.SB_OK
    assert lib.attn_prefill_workspace_bytes(4, 2048, 8, 128) == 4 * 8 * 128 * 2048 * 2
    assert lib.attn_prefill_workspace_bytes(1, 33, 1, 128) == 128 * 64 * 2      # 33 keys padded to 64


def test_mamba_prefill_validation(sb):
    """Every call here fails validation (or is a no-op)."""
    G = 1 << 30
    w = sb.SbMambaWeights(*[(i + 10) * G for i in range(9)])
    call = lambda **kw: sb.lib.mamba_prefill(1 * G, ctypes.byref(w), 2 * G, 3 * G, kw.get("M", 4 * G), 5 * G,
                                             kw.get("B", 4), kw.get("T", 2048), 3072, 6144, 16, kw.get("R", 192), 4,
                                             6 * G, kw.get("wsb", 1 << 34), None)
    assert call(R=184) == sb.SB_EUNSUPPORTED           # a multiple of 8 but not of 64
    assert call(M=5 * G + 64) == sb.SB_EINVAL           # M overlaps y
    assert call(wsb=1 << 20) == sb.SB_EWORKSPACE
    assert call(T=0) == sb.SB_OK and call(B=0) == sb.SB_OK
    assert sb.lib.mamba_prefill_workspace_bytes(4, 2048, 3072, 6144, 16, 192, 4) > 4 * 2048 * 6144 * 8


def test_sambay_prefill_validation(sb):
    """Every call here fails validation (or is a no-op); no pointer is touched."""
    G = 1 << 30
    mw = sb.SbMambaWeights(*[(i + 10) * G for i in range(9)])
    mam = sb.SbSelfLayer(kind=sb.SB_SELF_MAMBA, mamba=mw, conv_state=30 * G, ssm_state=31 * G)
    att = sb.SbSelfLayer(kind=sb.SB_SELF_ATTN, wq=32 * G, wk=33 * G, wv=34 * G, wo=35 * G)
    swa = sb.SbSelfLayer(kind=sb.SB_SELF_SWA, wq=36 * G, wk=37 * G, wv=38 * G, wo=39 * G, kring=40 * G,
                         vring=41 * G)
    cross = (sb.SbLayerEx * 2)()
    cross[0].kind, cross[0].w_a, cross[0].w_b = sb.SB_LAYER_XATTN, 42 * G, 43 * G
    cross[1].kind, cross[1].w_a, cross[1].w_b = sb.SB_LAYER_GMU, 44 * G, 45 * G

    def call(layers=(mam, swa, att), ncross=2, T=2048, L=4096, window=256, kc=4 * G, hout=2 * G, wsb=1 << 36,
             B=4, R=192):
        arr = (sb.SbSelfLayer * max(len(layers), 1))(*layers)
        return sb.lib.sambay_prefill(1 * G, hout, 3 * G, arr, len(layers), cross, ncross, kc, 6 * G, B, T, 3072, 6144,
                                     16, R, 4, 0, 24, 8, 128, L, window, 0.088, 1e-5, 50 * G, wsb, None)

    assert call(B=0) == sb.SB_OK
    assert call(T=0) == sb.SB_EINVAL                      # no last token
    assert call(T=5000) == sb.SB_EUNSUPPORTED             # T > L
    assert call(R=184) == sb.SB_EUNSUPPORTED              # dt_rank not a multiple of 64
    assert call(window=0) == sb.SB_EUNSUPPORTED           # a sliding-window layer needs a window
    assert call(layers=(mam, swa)) == sb.SB_EINVAL        # cross-attention without a cache writer
    assert call(layers=(swa, att)) == sb.SB_EINVAL        # a GMU without an SSM layer
    assert call(hout=1 * G + 64) == sb.SB_EINVAL          # h_out overlaps x
    assert call(kc=6 * G) == sb.SB_EINVAL                 # the two caches overlap
    assert call(wsb=1 << 20) == sb.SB_EWORKSPACE
    bad = sb.SbSelfLayer(kind=7)
    assert call(layers=(mam, bad, att)) == sb.SB_EINVAL
    noring = sb.SbSelfLayer(kind=sb.SB_SELF_SWA, wq=36 * G, wk=37 * G, wv=38 * G, wo=39 * G)
    assert call(layers=(mam, noring, att)) == sb.SB_EINVAL
    lib = sb.lib
    need = lib.sambay_prefill_workspace_bytes(4, 2048, 3072, 6144, 16, 192, 4, 8192, 24, 8, 128, 36864)
    assert need > 4 * 2048 * (2 * 3072 + 6144) * 2       # h, x-norm and M rows at least
    assert lib.sambay_prefill_workspace_bytes(4, 0, 3072, 6144, 16, 192, 4, 0, 24, 8, 128, 36864) == 0
    assert lib.sambay_prefill_workspace_bytes(4, 2048, 3072, 6144, 16, 192, 4, 0, 24, 8, 64, 36864) == 0


def test_sambay_decode_validation(sb):
    """Every call here fails validation (or is a no-op); no pointer is touched."""
    G = 1 << 30
    mw = sb.SbMambaWeights(*[(i + 60) * G for i in range(9)])
    mam = sb.SbSelfLayer(kind=sb.SB_SELF_MAMBA, mamba=mw, conv_state=70 * G, ssm_state=71 * G)
    att = sb.SbSelfLayer(kind=sb.SB_SELF_ATTN, wq=72 * G, wk=73 * G, wv=74 * G, wo=75 * G)
    swa = sb.SbSelfLayer(kind=sb.SB_SELF_SWA, wq=76 * G, wk=77 * G, wv=78 * G, wo=79 * G, kring=80 * G,
                         vring=81 * G)
    cross = (sb.SbLayerEx * 2)()
    cross[0].kind, cross[0].w_a, cross[0].w_b = sb.SB_LAYER_XATTN, 82 * G, 83 * G
    cross[1].kind, cross[1].w_a, cross[1].w_b = sb.SB_LAYER_GMU, 84 * G, 85 * G

    def call(layers=(mam, swa, att), pos=5 * G, window=256, wsb=1 << 36, B=32, Hkv=8, kc=20 * G):
        arr = (sb.SbSelfLayer * max(len(layers), 1))(*layers)
        return sb.lib.sambay_decode_step(1 * G, 3 * G, arr, len(layers), cross, 2, kc, 30 * G, pos, B, 3072, 6144,
                                         16, 192, 4, 0, 24, Hkv, 128, 34816, window, 0.088, 1e-5, 100 * G, wsb, None)

    assert call(B=0) == sb.SB_OK
    assert call(pos=None) == sb.SB_EINVAL
    assert call(pos=5 * G + 2) == sb.SB_EINVAL            # misaligned positions
    assert call(layers=(mam, att, att)) == sb.SB_EINVAL   # two layers writing the shared cache
    assert call(layers=(mam, swa)) == sb.SB_EINVAL        # cross-attention without a cache writer
    assert call(window=0) == sb.SB_EUNSUPPORTED
    assert call(Hkv=5) == sb.SB_EUNSUPPORTED              # 24 % 5 != 0
    assert call(kc=29 * G) == sb.SB_EINVAL                # the caches overlap
    assert call(wsb=1 << 20) == sb.SB_EWORKSPACE
    need = sb.lib.sambay_decode_workspace_bytes(32, 3072, 6144, 16, 192, 4, 8192, 24, 8, 128, 34816, 256)
    assert need > sb.lib.crossdecoder_ex_workspace_bytes(32, 3072, 6144, 8192, 24, 8, 128, 34816)
    assert sb.lib.sambay_decode_workspace_bytes(32, 3072, 6144, 16, 192, 4, 8192, 24, 8, 64, 34816, 256) == 0


def test_noalloc_attention_rejects_requests_beyond_its_scratch(sb):
    """xattn_decode_noalloc checks shapes and its 16 MiB scratch limit before
    it touches the device: 4096 sequences x 128 query heads need 545 MB of
    partials."""
    lib = sb.lib
    assert lib.xattn_decode_noalloc(_addr(0), _addr(1), _addr(2), _addr(3), 4096, 128, 16, 128, 34816, 0.088,
                                    None) == sb.SB_EWORKSPACE
    assert "scratch" in lib.sb_last_error().decode()
    assert lib.xattn_decode_noalloc(_addr(0), _addr(1), _addr(2), _addr(3), 2, 24, 8, 64, 100, 0.1,
                                    None) == sb.SB_EUNSUPPORTED          # D != 128
    assert lib.xattn_decode_noalloc(_addr(0), _addr(1), _addr(2), _addr(3), -1, 24, 8, 128, 100, 0.1,
                                    None) == sb.SB_EINVAL
    assert lib.xattn_decode_noalloc(_addr(0), _addr(1), _addr(2), _addr(3), 0, 24, 8, 128, 100, 0.1,
                                    None) == sb.SB_OK                    # nothing to do
