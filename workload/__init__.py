"""Seeded synthetic inputs for the SambaY cross-decoder step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no GMU, no attention), so both the HIP path and the
oracle can be fed from it.  Every tensor is drawn in float32 from its own
seeded ``torch.Generator`` on the requested device and then rounded to the
storage dtype (bfloat16: round-to-nearest-even).  The same seed on the same
device type gives the same values.

The shapes follow the pages' long-generation workload (2K-token prompt plus
32K generated tokens, so a 34816-position shared KV cache) and the model
widths below.  Values: activations and the KV cache ~ N(0, 1), weights
~ N(0, 0.02^2).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED_BASE = 20250716

# ----------------------------------------------------------------- workloads

TINY_GMU = dict(rows=64, d_model=64, d_inner=128)                       # fp32
GMU_PREFILL = dict(batch=4, seq=2048, d_model=2560, d_inner=5120)        # bf16
GMU_DECODE = dict(batches=(1, 8, 32, 64), d_model=3072, d_inner=6144)    # bf16
XATTN_DECODE = dict(B=16, Hq=24, Hkv=8, D=128, L=34816)                  # bf16
CROSSDECODER = dict(B=32, d_model=3072, d_inner=6144, Hq=24, Hkv=8, D=128, L=34816, n_layers=16)  # bf16
# Ragged serving batch: every sequence has its 2048-token prompt and is somewhere
# in its 32K-token generation, so cache lengths are uniform in [2048, 34816].
XATTN_VARLEN = dict(B=32, Hq=24, Hkv=8, D=128, L=34816, min_len=2048)    # bf16
# The complete layer adds a pre-RMSNorm SwiGLU MLP (d_ff = 8192, about 8/3 of
# d_model) and pre-RMSNorms to the same stack, over the ragged batch.
CROSSDECODER_EX = dict(B=32, d_model=3072, d_inner=6144, d_ff=8192, Hq=24, Hkv=8, D=128, L=34816, n_layers=16,
                       min_len=2048)
WEIGHT_STD = 0.02
NORM_GAIN_STD = 0.1


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _seed(cfg: int, tensor: int, extra: int = 0) -> int:
    return SEED_BASE + cfg + 1_000_003 * tensor + 7_919 * extra


def normal(shape, *, std: float = 1.0, seed: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """float32 N(0, std^2) draws from a generator seeded with `seed`, rounded to dtype."""
    x = torch.randn(tuple(shape), generator=_gen(device, seed), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x if dtype == torch.float32 else x.to(dtype)


# ------------------------------------------------------------ tiny GMU (fp32)

@dataclass
class TinyGMU:
    X: torch.Tensor    # [T, d_model] fp32
    V: torch.Tensor    # [T, d_inner] fp32, token values mixed by A
    A: torch.Tensor    # [T, T] float64, causal row-stochastic mixing matrix
    M: torch.Tensor    # [T, d_inner] fp32, M = A·V rounded to fp32
    W1: torch.Tensor   # [d_inner, d_model] fp32
    W2: torch.Tensor   # [d_model, d_inner] fp32


def tiny_gmu(seed: int = 0, rows: int = 64, d_model: int = 64, d_inner: int = 128) -> TinyGMU:
    """The small fp32 GMU case: an explicit causal (lower-triangular) mixing
    matrix A whose rows are softmax-normalised N(0,1) logits over j <= i, token
    values V ~ N(0,1), and the memory M = A·V that a token-mixing layer would
    produce; X ~ N(0,1); W1, W2 ~ N(0, 0.02^2).  CPU tensors."""
    s = SEED_BASE + 1000 * seed
    X = normal((rows, d_model), seed=s + 1, dtype=torch.float32)
    V = normal((rows, d_inner), seed=s + 2, dtype=torch.float32)
    logits = normal((rows, rows), seed=s + 3, dtype=torch.float32).double()
    causal = torch.ones(rows, rows, dtype=torch.bool).tril()
    logits = logits.masked_fill(~causal, float("-inf"))
    A = torch.softmax(logits, dim=1)                # row i: weights over tokens j <= i
    M = (A @ V.double()).float()
    W1 = normal((d_inner, d_model), std=WEIGHT_STD, seed=s + 4, dtype=torch.float32)
    W2 = normal((d_model, d_inner), std=WEIGHT_STD, seed=s + 5, dtype=torch.float32)
    return TinyGMU(X=X, V=V, A=A, M=M, W1=W1, W2=W2)


# -------------------------------------------------------------- GMU (bf16)

@dataclass
class GMUInputs:
    M: torch.Tensor    # [rows, d_inner]
    X: torch.Tensor    # [rows, d_model]
    W1: torch.Tensor   # [d_inner, d_model]
    W2: torch.Tensor   # [d_model, d_inner]


def gmu_inputs(rows: int, d_model: int, d_inner: int, *, seed: int = 0, device="cpu",
               dtype=torch.bfloat16, weight_set: int = 0) -> GMUInputs:
    """M, X ~ N(0,1) rows; W1, W2 ~ N(0, 0.02^2).  `weight_set` selects one of
    several independent weight draws (the benchmark rotates them so that the
    weights are streamed from HBM rather than served from the last-level cache)."""
    M = normal((rows, d_inner), seed=_seed(seed, 1), device=device, dtype=dtype)
    X = normal((rows, d_model), seed=_seed(seed, 2), device=device, dtype=dtype)
    W1 = normal((d_inner, d_model), std=WEIGHT_STD, seed=_seed(seed, 3, weight_set), device=device, dtype=dtype)
    W2 = normal((d_model, d_inner), std=WEIGHT_STD, seed=_seed(seed, 4, weight_set), device=device, dtype=dtype)
    return GMUInputs(M=M, X=X, W1=W1, W2=W2)


# ------------------------------------------------- cross-attention (bf16)

@dataclass
class XAttnInputs:
    q: torch.Tensor    # [B, Hq, D]
    K: torch.Tensor    # [B, Hkv, L, D]
    V: torch.Tensor    # [B, Hkv, L, D]


def xattn_inputs(B: int, Hq: int, Hkv: int, D: int, L: int, *, seed: int = 0, device="cpu",
                 dtype=torch.bfloat16) -> XAttnInputs:
    """q, K, V ~ N(0,1): one decode query per sequence against a shared cache
    of L positions (all positions visible)."""
    q = normal((B, Hq, D), seed=_seed(seed, 11), device=device, dtype=dtype)
    K = normal((B, Hkv, L, D), seed=_seed(seed, 12), device=device, dtype=dtype)
    V = normal((B, Hkv, L, D), seed=_seed(seed, 13), device=device, dtype=dtype)
    return XAttnInputs(q=q, K=K, V=V)


# ------------------------------------------------------ cross-decoder step

@dataclass
class CrossDecoderInputs:
    h: torch.Tensor                 # [B, d_model] residual stream entering the cross-decoder
    M: torch.Tensor                 # [B, d_inner] memory readout shared by every GMU layer
    K: torch.Tensor                 # [B, Hkv, L, D] the single shared KV cache
    V: torch.Tensor
    layers: list = field(default_factory=list)   # [(kind, w_a, w_b)]


def layer_kinds(n_layers: int, first: str = "xattn") -> list:
    """Alternating layer kinds, starting with `first` ("xattn" or "gmu")."""
    other = "gmu" if first == "xattn" else "xattn"
    return [first if i % 2 == 0 else other for i in range(n_layers)]


def crossdecoder_inputs(B: int, d_model: int, d_inner: int, Hq: int, Hkv: int, D: int, L: int, n_layers: int, *,
                        seed: int = 0, device="cpu", dtype=torch.bfloat16, kinds=None) -> CrossDecoderInputs:
    """h, M, K, V ~ N(0,1); per-layer weights ~ N(0, 0.02^2): (Wq, Wo) of shape
    [d_model, d_model] for cross-attention, (W1 [d_inner, d_model],
    W2 [d_model, d_inner]) for GMU layers."""
    if kinds is None:
        kinds = layer_kinds(n_layers)
    h = normal((B, d_model), seed=_seed(seed, 21), device=device, dtype=dtype)
    M = normal((B, d_inner), seed=_seed(seed, 22), device=device, dtype=dtype)
    K = normal((B, Hkv, L, D), seed=_seed(seed, 23), device=device, dtype=dtype)
    V = normal((B, Hkv, L, D), seed=_seed(seed, 24), device=device, dtype=dtype)
    layers = []
    for i, kind in enumerate(kinds):
        if kind == "xattn":
            wa = normal((d_model, d_model), std=WEIGHT_STD, seed=_seed(seed, 30, 2 * i), device=device, dtype=dtype)
            wb = normal((d_model, d_model), std=WEIGHT_STD, seed=_seed(seed, 30, 2 * i + 1), device=device,
                        dtype=dtype)
        elif kind == "gmu":
            wa = normal((d_inner, d_model), std=WEIGHT_STD, seed=_seed(seed, 30, 2 * i), device=device, dtype=dtype)
            wb = normal((d_model, d_inner), std=WEIGHT_STD, seed=_seed(seed, 30, 2 * i + 1), device=device,
                        dtype=dtype)
        else:
            raise ValueError(kind)
        layers.append((kind, wa, wb))
    return CrossDecoderInputs(h=h, M=M, K=K, V=V, layers=layers)


# ------------------------------------------ ragged batch, complete layer

def ragged_lens(B: int, L: int, *, seed: int = 0, min_len: int = 1, device="cpu") -> torch.Tensor:
    """int32 cache lengths, uniform over [min_len, L] (seeded)."""
    g = _gen("cpu", _seed(seed, 41))
    lens = torch.randint(min_len, L + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    return lens.to(device)


@dataclass
class CrossDecoderExInputs:
    h: torch.Tensor
    M: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor
    lens: torch.Tensor | None       # [B] int32 or None (all L positions)
    layers: list = field(default_factory=list)   # dicts: kind, w_a, w_b, norm1, norm2, w_gate, w_up, w_down


def crossdecoder_ex_inputs(B: int, d_model: int, d_inner: int, d_ff: int, Hq: int, Hkv: int, D: int, L: int,
                           n_layers: int, *, seed: int = 0, device="cpu", dtype=torch.bfloat16, kinds=None,
                           lens="ragged", min_len: int = 1, norms: bool = True, mlp: bool = True
                           ) -> CrossDecoderExInputs:
    """The cross-decoder inputs plus, per layer, RMSNorm gains 1 + N(0, 0.1^2)
    (norm1 before the mixer, norm2 before the MLP) and SwiGLU weights
    ~ N(0, 0.02^2): w_gate, w_up [d_ff, d_model], w_down [d_model, d_ff].
    lens: "ragged" (uniform in [min_len, L]), None, or an explicit list."""
    base = crossdecoder_inputs(B, d_model, d_inner, Hq, Hkv, D, L, n_layers, seed=seed, device=device, dtype=dtype,
                               kinds=kinds)
    if isinstance(lens, str):
        lens_t = ragged_lens(B, L, seed=seed, min_len=min_len, device=device)
    elif lens is None:
        lens_t = None
    else:
        lens_t = torch.tensor(list(lens), dtype=torch.int32, device=device)
    layers = []
    for i, (kind, wa, wb) in enumerate(base.layers):
        ly = dict(kind=kind, w_a=wa, w_b=wb, norm1=None, norm2=None, w_gate=None, w_up=None, w_down=None)
        if norms:
            for j, key in enumerate(("norm1", "norm2")):
                gsd = normal((d_model,), std=NORM_GAIN_STD, seed=_seed(seed, 50, 2 * i + j), device=device,
                             dtype=torch.float32)
                ly[key] = (1.0 + gsd).to(dtype)
        if mlp:
            ly["w_gate"] = normal((d_ff, d_model), std=WEIGHT_STD, seed=_seed(seed, 60, 3 * i), device=device,
                                  dtype=dtype)
            ly["w_up"] = normal((d_ff, d_model), std=WEIGHT_STD, seed=_seed(seed, 60, 3 * i + 1), device=device,
                                dtype=dtype)
            ly["w_down"] = normal((d_model, d_ff), std=WEIGHT_STD, seed=_seed(seed, 60, 3 * i + 2), device=device,
                                  dtype=dtype)
        layers.append(ly)
    return CrossDecoderExInputs(h=base.h, M=base.M, K=base.K, V=base.V, lens=lens_t, layers=layers)


# ------------------------------------------------ differential attention (bf16)

# The same cache and query shapes as the plain decode; each 128-wide query and
# key row is two 64-wide halves, one per attention map.  lambda starts at
# lambda_init in the published definition, and lambda_init tends to 0.8 in deep
# layers; the per-head normalisation gain is 1 + N(0, 0.1^2).
DIFFATTN_DECODE = dict(B=16, Hq=24, Hkv=8, D=128, L=34816, lam=0.8, lam_init=0.8, eps=1e-5)  # bf16


@dataclass
class DiffAttnInputs:
    q: torch.Tensor      # [B, Hq, D], rows (q1 | q2)
    K: torch.Tensor      # [B, Hkv, L, D], rows (k1 | k2)
    V: torch.Tensor      # [B, Hkv, L, D]
    gamma: torch.Tensor  # [D]


def diffattn_gain(D: int, *, seed: int = 0, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """The per-head normalisation gain, 1 + N(0, 0.1^2)."""
    gsd = normal((D,), std=NORM_GAIN_STD, seed=_seed(seed, 70), device=device, dtype=torch.float32)
    return (1.0 + gsd).to(dtype)


def diffattn_inputs(B: int, Hq: int, Hkv: int, D: int, L: int, *, seed: int = 0, device="cpu",
                    dtype=torch.bfloat16) -> DiffAttnInputs:
    """q, K, V ~ N(0,1) as for the plain decode (same seed, same values), plus the gain."""
    x = xattn_inputs(B, Hq, Hkv, D, L, seed=seed, device=device, dtype=dtype)
    return DiffAttnInputs(q=x.q, K=x.K, V=x.V, gamma=diffattn_gain(D, seed=seed, device=device, dtype=dtype))


# ------------------------------------------- self-decoder attention (bf16)

# The self-decoder's attention layers at decode: the final full-attention
# layer appends to the shared cache (room for 34816 positions, the ragged
# serving batch's positions), the sliding-window layers to a ring of 256
# slots (full once 256 tokens have been generated).
SELFATTN_FULL = dict(B=32, Hq=24, Hkv=8, D=128, L=34816, min_len=2048)   # bf16
SELFATTN_SWA = dict(B=32, Hq=24, Hkv=8, D=128, window=256, min_len=2048)  # bf16


@dataclass
class SelfAttnInputs:
    q: torch.Tensor      # [B, Hq, D]
    k_new: torch.Tensor  # [B, Hkv, D]
    v_new: torch.Tensor  # [B, Hkv, D]
    K: torch.Tensor      # [B, Hkv, L, D] cache contents before the step
    V: torch.Tensor


def selfattn_inputs(B: int, Hq: int, Hkv: int, D: int, L: int, *, seed: int = 0, device="cpu",
                    dtype=torch.bfloat16) -> SelfAttnInputs:
    """q, the new key/value rows and the cache contents, all ~ N(0,1)."""
    x = xattn_inputs(B, Hq, Hkv, D, L, seed=seed, device=device, dtype=dtype)
    k_new = normal((B, Hkv, D), seed=_seed(seed, 80), device=device, dtype=dtype)
    v_new = normal((B, Hkv, D), seed=_seed(seed, 81), device=device, dtype=dtype)
    return SelfAttnInputs(q=x.q, k_new=k_new, v_new=v_new, K=x.K, V=x.V)


# --------------------------------------------- SSM decode step (Mamba layer)

# The self-decoder's SSM layer at the model width: d_inner = 2 d_model, 16
# states per channel, a 4-tap causal convolution, a step projection of rank
# ceil(d_model / 16) = 192.
MAMBA_DECODE = dict(B=32, d_model=3072, d_inner=6144, d_state=16, dt_rank=192, d_conv=4)


@dataclass
class MambaInputs:
    x: torch.Tensor            # [B, d_model] layer input
    w: dict                    # W_in, W_x, W_dt, W_out (dtype); conv_w, conv_b, dt_bias, A_log, D (float32)
    conv_state: torch.Tensor   # [B, d_inner, d_conv - 1] float32
    ssm_state: torch.Tensor    # [B, d_inner, d_state] float32


def _uniform(shape, lo: float, hi: float, *, seed: int, device) -> torch.Tensor:
    u = torch.rand(tuple(shape), generator=_gen(device, seed), device=device, dtype=torch.float32)
    return u * (hi - lo) + lo


def mamba_inputs(B: int, d_model: int, d_inner: int, d_state: int, dt_rank: int, d_conv: int, *, seed: int = 0,
                 device="cpu", dtype=torch.bfloat16) -> MambaInputs:
    """x ~ N(0,1); the four matrices ~ N(0, 0.02^2); the layer's usual
    initialisation for the rest: conv taps and bias ~ U(-1/sqrt(d_conv),
    1/sqrt(d_conv)), dt_bias = softplus^-1(dt) with log dt ~ U(log 1e-3,
    log 1e-1), A_log[c, n] = log(n + 1), D = 1; conv_state ~ N(0, 1.2^2)
    (past branch inputs), ssm_state ~ N(0, 1)."""
    s = lambda t: _seed(seed, 90 + t)
    x = normal((B, d_model), seed=s(0), device=device, dtype=dtype)
    w = {
        "W_in": normal((2 * d_inner, d_model), std=WEIGHT_STD, seed=s(1), device=device, dtype=dtype),
        "W_x": normal((dt_rank + 2 * d_state, d_inner), std=WEIGHT_STD, seed=s(2), device=device, dtype=dtype),
        "W_dt": normal((d_inner, dt_rank), std=WEIGHT_STD, seed=s(3), device=device, dtype=dtype),
        "W_out": normal((d_model, d_inner), std=WEIGHT_STD, seed=s(4), device=device, dtype=dtype),
    }
    bound = 1.0 / d_conv ** 0.5
    w["conv_w"] = _uniform((d_inner, d_conv), -bound, bound, seed=s(5), device=device)
    w["conv_b"] = _uniform((d_inner,), -bound, bound, seed=s(6), device=device)
    dt = torch.exp(_uniform((d_inner,), -6.907755278982137, -2.302585092994046, seed=s(7), device=device))
    w["dt_bias"] = dt + torch.log(-torch.expm1(-dt))
    w["A_log"] = torch.log(torch.arange(1, d_state + 1, device=device, dtype=torch.float32)).repeat(d_inner, 1)
    w["D"] = torch.ones(d_inner, device=device, dtype=torch.float32)
    conv_state = normal((B, d_inner, d_conv - 1), std=1.2, seed=s(8), device=device, dtype=torch.float32)
    ssm_state = normal((B, d_inner, d_state), seed=s(9), device=device, dtype=torch.float32)
    return MambaInputs(x=x, w=w, conv_state=conv_state, ssm_state=ssm_state)


# ---------------------------------------------- prefill attention (bf16)

# The pages' prompt length: 2048 tokens, four sequences, the model's head
# shape; the self-decoder's sliding window of 256 tokens.
ATTN_PREFILL = dict(B=4, T=2048, Hq=24, Hkv=8, D=128, window=256)   # bf16


@dataclass
class PrefillInputs:
    q: torch.Tensor    # [B, T, Hq, D]
    k: torch.Tensor    # [B, T, Hkv, D]
    v: torch.Tensor


def prefill_inputs(B: int, T: int, Hq: int, Hkv: int, D: int, *, seed: int = 0, device="cpu",
                   dtype=torch.bfloat16) -> PrefillInputs:
    """q, k, v ~ N(0, 1), token-major as the projections write them."""
    return PrefillInputs(q=normal((B, T, Hq, D), seed=_seed(seed, 100), device=device, dtype=dtype),
                         k=normal((B, T, Hkv, D), seed=_seed(seed, 101), device=device, dtype=dtype),
                         v=normal((B, T, Hkv, D), seed=_seed(seed, 102), device=device, dtype=dtype))


# ------------------------------------------------- YOCO-style prefill (bf16)

# The whole prefill of the pages' model shape: a 2048-token prompt for four
# sequences through a 16-layer Samba self-decoder (SSM layers alternating with
# 256-token sliding-window attention, the last layer full attention, each
# with a SwiGLU MLP) and the 16-layer cross-decoder on the last token; the
# shared cache has room for the 2K prompt + 32K generated tokens.
SAMBAY_PREFILL = dict(B=4, T=2048, d_model=3072, d_inner=6144, d_state=16, dt_rank=192, d_conv=4, d_ff=8192,
                      Hq=24, Hkv=8, D=128, window=256, L=34816, n_self=16, n_cross=16)


def self_layer_kinds(n: int) -> list:
    """Samba order: SSM, sliding window, SSM, ... with the last layer full attention."""
    return ["attn" if i == n - 1 else ("mamba" if i % 2 == 0 else "swa") for i in range(n)]


@dataclass
class SambayPrefillInputs:
    x: torch.Tensor                  # [B, T, d_model]
    self_layers: list                # dicts as the binding takes them
    cross_layers: list
    kcache: torch.Tensor             # [B, Hkv, L, D]
    vcache: torch.Tensor


def sambay_prefill_inputs(B: int, T: int, d_model: int, d_inner: int, d_state: int, dt_rank: int, d_conv: int,
                          d_ff: int, Hq: int, Hkv: int, D: int, window: int, L: int, self_kinds: list,
                          cross_kinds: list, *, seed: int = 0, device="cpu", fresh: bool = True,
                          mlp: bool = True, norms: bool = True, dtype=torch.bfloat16) -> SambayPrefillInputs:
    """x ~ N(0, 1); every matrix ~ N(0, 0.02^2); RMSNorm gains 1 + N(0, 0.1^2);
    the SSM layers' own parameters as mamba_inputs (one seed per layer);
    fresh: zero SSM states (a new prompt), else mamba_inputs' states.  The
    caches start as zeros."""
    x = normal((B, T, d_model), seed=_seed(seed, 120), device=device, dtype=dtype)
    w = lambda shape, t, i: normal(shape, std=WEIGHT_STD, seed=_seed(seed, t, i), device=device, dtype=dtype)

    def norms_mlp(ly, i, base):
        if norms:
            for j, key in enumerate(("norm1", "norm2")):
                gsd = normal((d_model,), std=NORM_GAIN_STD, seed=_seed(seed, base, 2 * i + j), device=device,
                             dtype=torch.float32)
                ly[key] = (1.0 + gsd).to(dtype)
        if mlp:
            ly["w_gate"] = w((d_ff, d_model), base + 1, 3 * i)
            ly["w_up"] = w((d_ff, d_model), base + 1, 3 * i + 1)
            ly["w_down"] = w((d_model, d_ff), base + 1, 3 * i + 2)
        return ly

    self_layers = []
    for i, kind in enumerate(self_kinds):
        ly = {"kind": kind}
        if kind == "mamba":
            m = mamba_inputs(B, d_model, d_inner, d_state, dt_rank, d_conv, seed=_seed(seed, 121, i), device=device,
                             dtype=dtype)
            ly["w"] = m.w
            ly["conv_state"] = torch.zeros_like(m.conv_state) if fresh else m.conv_state
            ly["ssm_state"] = torch.zeros_like(m.ssm_state) if fresh else m.ssm_state
        else:
            ly["wq"] = w((Hq * D, d_model), 122, 4 * i)
            ly["wk"] = w((Hkv * D, d_model), 122, 4 * i + 1)
            ly["wv"] = w((Hkv * D, d_model), 122, 4 * i + 2)
            ly["wo"] = w((d_model, Hq * D), 122, 4 * i + 3)
            if kind == "swa":
                ly["kring"] = torch.zeros((B, Hkv, window, D), device=device, dtype=dtype)
                ly["vring"] = torch.zeros((B, Hkv, window, D), device=device, dtype=dtype)
        self_layers.append(norms_mlp(ly, i, 123))
    cross_layers = []
    for i, kind in enumerate(cross_kinds):
        ly = {"kind": kind}
        if kind == "xattn":
            ly["w_a"], ly["w_b"] = w((d_model, d_model), 125, 2 * i), w((d_model, d_model), 125, 2 * i + 1)
        else:
            ly["w_a"], ly["w_b"] = w((d_inner, d_model), 125, 2 * i), w((d_model, d_inner), 125, 2 * i + 1)
        cross_layers.append(norms_mlp(ly, i, 126))
    kc = torch.zeros((B, Hkv, L, D), device=device, dtype=dtype)
    return SambayPrefillInputs(x=x, self_layers=self_layers, cross_layers=cross_layers, kcache=kc,
                               vcache=torch.zeros_like(kc))
