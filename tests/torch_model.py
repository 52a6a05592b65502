"""The whole model composed from torch fp64 library routines, for pinning the
oracle's own compositions (test infrastructure, no test functions here).

This is a second, independent statement of the same readings the oracle
follows, written in a different form:
- the SSM layer in its parallel form (materialised token-mixing matrix with
  decays from cumulative sums of Δ·A, F.conv1d over the whole input history
  for the causal convolution), not the per-token recurrence;
- attention over the prompt with torch's scaled_dot_product_attention and
  an explicit boolean mask (causal, optionally the last `window` keys),
  grouped-query heads by repeating the KV heads;
- RMSNorm, SwiGLU and the products as F.linear / plain tensor arithmetic.

Layer composition (Paper-Notes reading notes on "Decoder-Hybrid-Decoder
Architecture for Efficient Reasoning with Long Generation", section 整体框架:
a Samba self-decoder of SSM and sliding-window layers that ends in one full
attention layer whose keys and values become the single shared cache, then a
cross-decoder whose GMU layers reuse the memory M of the last SSM layer,
section 关键设计): every layer is pre-norm, h = h + mixer(RMSNorm(h; g1)),
then, with an MLP, h = h + SwiGLU(RMSNorm(h; g2)); h is rounded to bfloat16
after every residual add when round_h is set (the bf16 residual stream).

Sequences are processed one at a time, so a decode step at any position p is
the full forward over the p + 1 tokens of that sequence: no ring, no cache
slot arithmetic and no carried state are involved.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def t64(a) -> torch.Tensor:
    """Any accepted array (numpy, torch of any float dtype) as a float64 tensor."""
    if isinstance(a, torch.Tensor):
        return a.detach().cpu().double()
    return torch.as_tensor(np.asarray(a, np.float64))


def mamba_parallel(xs, w, conv0, s0):
    """T tokens of one sequence through the Mamba layer in parallel form:
    xs [T, d_model], conv0 [d_inner, K-1] (the K-1 branch inputs before the
    first token, oldest first), s0 [d_inner, N].  Returns M [T, d_inner]
    (the SSM output C·s + D·u), y [T, d_model], the final convolution
    window [d_inner, K-1] and the final state [d_inner, N], as float64
    numpy arrays."""
    W = {k: t64(v) for k, v in w.items()}
    xs, conv0, s0 = t64(xs), t64(conv0), t64(s0)
    T = xs.shape[0]
    d_inner, K = W["conv_w"].shape
    N = W["A_log"].shape[1]
    R = W["W_dt"].shape[1]
    xz = F.linear(xs, W["W_in"])                                       # [T, 2 d_inner]
    xi, z = xz[:, :d_inner], xz[:, d_inner:]
    hist = torch.cat([conv0, xi.T], dim=1)                             # [d_inner, K-1+T], oldest first
    u = F.silu(F.conv1d(hist[None], W["conv_w"][:, None, :], W["conv_b"], groups=d_inner)[0].T)   # [T, d_inner]
    xd = F.linear(u, W["W_x"])
    delta, Bv, Cv = xd[:, :R], xd[:, R:R + N], xd[:, R + N:]
    dt = F.softplus(F.linear(delta, W["W_dt"]) + W["dt_bias"])          # [T, d_inner]
    A = -torch.exp(W["A_log"])                                          # [d_inner, N]
    la = dt[:, :, None] * A[None]                                       # log decay per step [T, d_inner, N]
    cum = torch.cumsum(la, dim=0)                                       # sum over k <= t of log a_k
    # mixing: L[t, j] = exp(cum[t] - cum[j]) for j <= t (the decay from step j+1 to t)
    Lmix = torch.exp(cum[:, None] - cum[None, :])                       # [T, T, d_inner, N]
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    Lmix = torch.where(causal[:, :, None, None], Lmix, torch.zeros((), dtype=torch.float64))
    inp = dt[:, :, None] * Bv[:, None, :] * u[:, :, None]               # Δ_j B_j u_j  [T, d_inner, N]
    S = torch.einsum("tjcn,jcn->tcn", Lmix, inp) + torch.exp(cum) * s0[None]
    M = torch.einsum("tcn,tn->tc", S, Cv) + W["D"][None] * u
    y = F.linear(M * F.silu(z), W["W_out"])
    return M.numpy(), y.numpy(), hist[:, T:].numpy(), S[-1].numpy()


def rms(t: torch.Tensor, g, eps: float) -> torch.Tensor:
    if g is None:
        return t
    return t / torch.sqrt((t * t).mean(-1, keepdim=True) + eps) * t64(g)


def swiglu(t: torch.Tensor, ly) -> torch.Tensor:
    a = F.linear(t, t64(ly["w_gate"]))
    b = F.linear(t, t64(ly["w_up"]))
    return F.linear(F.silu(a) * b, t64(ly["w_down"]))


def rounder(round_h: bool):
    """bfloat16 rounding of the residual stream by the oracle's scalar
    definition (pinned on its own), or the identity."""
    if not round_h:
        return lambda t: t
    return lambda t: torch.from_numpy(oracle.round_bf16(t.numpy()))


def prompt_attention(q, k, v, window: int, scale=None) -> torch.Tensor:
    """q [T, Hq, D], k, v [T, Hkv, D]: query i sees keys j <= i (and
    j > i - window when window > 0)."""
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = j <= i
    if window > 0:
        mask = mask & (j > i - window)
    kk = k.transpose(0, 1).repeat_interleave(G, 0)                      # [Hq, T, D]
    vv = v.transpose(0, 1).repeat_interleave(G, 0)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), kk, vv, attn_mask=mask, scale=scale)
    return o.transpose(0, 1)                                            # [T, Hq, D]


def self_decoder(x, self_layers, Hq: int, Hkv: int, window: int, eps: float = 1e-5, scale=None,
                 round_h: bool = True, seq: int = 0) -> dict:
    """The self-decoder over the tokens x [T, d_model] of sequence `seq`
    (its initial SSM states are row `seq` of each SSM layer's states).
    Returns h [T, d_model] after the last layer, the memory M [T, d_inner]
    of the last SSM layer, and per layer its keys and values [T, Hkv, D]
    (attention layers) or its final conv window and SSM state (SSM
    layers)."""
    rnd = rounder(round_h)
    h = rnd(t64(x))
    T, dm = h.shape
    D = dm // Hq
    M_mem, per_layer = None, []
    for ly in self_layers:
        t = rms(h, ly.get("norm1"), eps)
        if ly["kind"] == "mamba":
            M, y, cw, s = mamba_parallel(t, ly["w"], t64(ly["conv_state"])[seq], t64(ly["ssm_state"])[seq])
            h = rnd(h + torch.from_numpy(y))
            M_mem = torch.from_numpy(M)
            per_layer.append({"conv_state": cw, "ssm_state": s})
        else:
            q = F.linear(t, t64(ly["wq"])).view(T, Hq, D)
            k = F.linear(t, t64(ly["wk"])).view(T, Hkv, D)
            v = F.linear(t, t64(ly["wv"])).view(T, Hkv, D)
            o = prompt_attention(q, k, v, window if ly["kind"] == "swa" else 0, scale)
            h = rnd(h + F.linear(o.reshape(T, dm), t64(ly["wo"])))
            per_layer.append({"k": k, "v": v})
        if ly.get("w_gate") is not None:
            h = rnd(h + swiglu(rms(h, ly.get("norm2"), eps), ly))
    return {"h": h, "M": M_mem, "layers": per_layer}


def cross_decoder(h, M, K, V, lens, cross_layers, Hq: int, eps: float = 1e-5, scale=None,
                  round_h: bool = True) -> torch.Tensor:
    """One token per sequence through the cross-decoder: h [B, d_model], M
    [B, d_inner] (shared by every GMU layer), K, V [B, Hkv, L, D] (shared by
    every cross-attention layer), sequence b seeing its first lens[b]
    positions."""
    rnd = rounder(round_h)
    h, M, K, V = t64(h), t64(M), t64(K), t64(V)
    B, dm = h.shape
    Hkv, D = K.shape[1], K.shape[3]
    G = Hq // Hkv
    for ly in cross_layers:
        t = rms(h, ly.get("norm1"), eps)
        if ly["kind"] == "xattn":
            q = F.linear(t, t64(ly["w_a"])).view(B, Hq, D)
            o = torch.zeros(B, Hq, D, dtype=torch.float64)
            for b in range(B):
                n = int(lens[b])
                if n == 0:
                    continue
                k = K[b, :, :n].repeat_interleave(G, 0)
                v = V[b, :, :n].repeat_interleave(G, 0)
                o[b] = F.scaled_dot_product_attention(q[b].unsqueeze(1), k, v, scale=scale).squeeze(1)
            y = F.linear(o.view(B, dm), t64(ly["w_b"]))
        else:
            y = F.linear(M * F.silu(F.linear(t, t64(ly["w_a"]))), t64(ly["w_b"]))
        h = rnd(h + y)
        if ly.get("w_gate") is not None:
            h = rnd(h + swiglu(rms(h, ly.get("norm2"), eps), ly))
    return h
