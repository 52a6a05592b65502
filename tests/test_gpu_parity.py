"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Error measure (both dtypes): err = max|y_gpu - y_ref| / max|y_ref|, with
y_ref from the oracle on the same seeded inputs.  Bars: 1e-5 for the fp32
path, 2e-2 for bf16 storage with fp32 accumulation.  Small shapes are
checked element by element and span several tiles plus ragged tails; the
full workload shapes are checked on sampled rows / sequences that the oracle
computes one by one (rows and sequences are independent in every call).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workload

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
DEV = "cuda:0"


@pytest.fixture(scope="module")
def sb():
    import attention_decoding_amd as sb
    return sb


def err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape
    assert np.all(np.isfinite(y)), "non-finite GPU output"
    return float(np.max(np.abs(y - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def report(name, e, tol):
    print("PARITY %-48s err=%.3e tol=%.0e" % (name, e, tol), flush=True)
    assert e <= tol, "%s: err %.3e > %.0e" % (name, e, tol)


def cpu(t):
    return t.detach().to("cpu")


def f64(t):
    return cpu(t).double().numpy()


# ------------------------------------------------------------------ GMU

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gmu_tiny_fp32(sb, seed):
    """The small fp32 case: T = 64 tokens, d_model 64, d_inner 128, causal mixing memory."""
    c = workload.tiny_gmu(seed)
    Y = sb.gmu_forward(c.M.to(DEV), c.X.to(DEV), c.W1.to(DEV), c.W2.to(DEV))
    torch.cuda.synchronize()
    report("gmu fp32 tiny seed=%d" % seed, err(f64(Y), oracle.gmu(c.M, c.X, c.W1, c.W2)), TOL_F32)


@pytest.mark.parametrize("rows,dm,di", [(1, 64, 128), (3, 64, 64), (5, 192, 320), (16, 256, 512), (17, 128, 640),
                                        (33, 320, 192), (64, 512, 256), (7, 3072, 6144)])
def test_gmu_decode_bf16_small(sb, rows, dm, di):
    g = workload.gmu_inputs(rows, dm, di, seed=rows + dm, device=DEV)
    Y = sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    torch.cuda.synchronize()
    ref = oracle.gmu(cpu(g.M), cpu(g.X), cpu(g.W1), cpu(g.W2))
    report("gmu bf16 rows=%d %dx%d" % (rows, dm, di), err(f64(Y), ref), TOL_BF16)


@pytest.mark.parametrize("B", workload.GMU_DECODE["batches"] + (2, 5, 17, 20, 33, 40, 50))
def test_gmu_decode_full_width(sb, B):
    """One decode step of B sequences at d_model 3072, d_inner 6144 (all rows
    checked); 2 and 5 tokens leave most of the 16 token columns of the
    LDS-streaming product's tile to the repeated last token; 17, 20, 33, 40
    and 50 tokens end in a part-filled 16-token tile (of the hidden's tiled
    layout up to 32 tokens, of the K-slab product's token slab above)."""
    c = workload.GMU_DECODE
    g = workload.gmu_inputs(B, c["d_model"], c["d_inner"], seed=100 + B, device=DEV)
    Y = sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    torch.cuda.synchronize()
    ref = oracle.gmu(cpu(g.M), cpu(g.X), cpu(g.W1), cpu(g.W2))
    report("gmu decode B=%d" % B, err(f64(Y), ref), TOL_BF16)


@pytest.mark.parametrize("rows,dm,di", [(65, 64, 128), (130, 192, 256), (300, 256, 320), (257, 512, 1024)])
def test_gmu_prefill_bf16_small(sb, rows, dm, di):
    g = workload.gmu_inputs(rows, dm, di, seed=rows, device=DEV)
    Y = sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    torch.cuda.synchronize()
    ref = oracle.gmu(cpu(g.M), cpu(g.X), cpu(g.W1), cpu(g.W2))
    report("gmu prefill rows=%d %dx%d" % (rows, dm, di), err(f64(Y), ref), TOL_BF16)


def test_gmu_prefill_full_sampled_rows(sb):
    """Prefill at 4 x 2048 tokens, d_model 2560, d_inner 5120; the oracle checks
    64 sampled rows (tile edges, the last rows, and random rows)."""
    c = workload.GMU_PREFILL
    rows = c["batch"] * c["seq"]
    g = workload.gmu_inputs(rows, c["d_model"], c["d_inner"], seed=7, device=DEV)
    Y = sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([[0, 1, 127, 128, 255, 4095, 4096, rows - 2, rows - 1],
                                    rng.choice(rows, 55, replace=False)]))
    ii = torch.from_numpy(idx).to(DEV)
    ref = oracle.gmu(cpu(g.M[ii]), cpu(g.X[ii]), cpu(g.W1), cpu(g.W2))
    report("gmu prefill 8192x2560x5120 (%d rows)" % len(idx), err(f64(Y[ii]), ref), TOL_BF16)


@pytest.mark.parametrize("rows,d_model,d_inner", [(4000, 1024, 4096), (4000, 1024, 2048), (4000, 1024, 4992),
                                                  (4000, 3008, 1024)])
def test_gmu_prefill_wide_tiles(sb, rows, d_model, d_inner):
    """Each GEMM tile shape: the gate product of d_inner 4096 runs on 256x256
    tiles, d_inner 2048 on 128x128, d_inner 4992 on 256x320 (last column
    tile 192 wide) and the output product of d_model 3008 on 256x192 (last
    column tile 128 wide); 4000 rows leave a ragged last row tile.  The
    oracle checks 64 sampled rows."""
    g = workload.gmu_inputs(rows, d_model, d_inner, seed=8, device=DEV)
    Y = sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 3839, 3840, rows - 2, rows - 1],
                                    rng.choice(rows, 54, replace=False)]))
    ii = torch.from_numpy(idx).to(DEV)
    ref = oracle.gmu(cpu(g.M[ii]), cpu(g.X[ii]), cpu(g.W1), cpu(g.W2))
    report("gmu prefill %dx%dx%d (%d rows)" % (rows, d_model, d_inner, len(idx)), err(f64(Y[ii]), ref), TOL_BF16)


def test_gmu_zero_rows_is_noop(sb):
    g = workload.gmu_inputs(1, 64, 128, device=DEV)
    out = torch.full((0, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    Y = sb.gmu_forward(g.M[:0], g.X[:0], g.W1, g.W2, out=out)
    assert Y.shape == (0, 64)


# ------------------------------------------------------ cross-attention

@pytest.mark.parametrize("B,Hq,Hkv,L", [(1, 3, 1, 1), (2, 6, 2, 31), (1, 1, 1, 33), (2, 24, 8, 300), (3, 16, 1, 1000),
                                        (1, 8, 8, 4097), (2, 48, 3, 777), (4, 24, 8, 2049)])
def test_xattn_small(sb, B, Hq, Hkv, L):
    x = workload.xattn_inputs(B, Hq, Hkv, 128, L, seed=B * 1000 + L, device=DEV)
    out = sb.xattn_decode(x.q, x.K, x.V)
    torch.cuda.synchronize()
    ref = oracle.xattn(cpu(x.q), cpu(x.K), cpu(x.V), 1.0 / math.sqrt(128))
    report("xattn B=%d Hq=%d Hkv=%d L=%d" % (B, Hq, Hkv, L), err(f64(out), ref), TOL_BF16)


def test_xattn_peaked_logits(sb):
    """Large query norms make the softmax nearly one-hot (as deep layers do)."""
    x = workload.xattn_inputs(2, 6, 2, 128, 999, seed=3, device=DEV)
    q = (x.q.float() * 12.0).to(torch.bfloat16)
    out = sb.xattn_decode(q, x.K, x.V)
    torch.cuda.synchronize()
    ref = oracle.xattn(cpu(q), cpu(x.K), cpu(x.V))
    report("xattn peaked", err(f64(out), ref), TOL_BF16)


def test_xattn_special_cases(sb):
    x = workload.xattn_inputs(2, 6, 2, 128, 300, seed=4, device=DEV)
    # q = 0: uniform weights, out = mean over positions of V.
    out = sb.xattn_decode(torch.zeros_like(x.q), x.K, x.V)
    ref = x.V.double().mean(dim=2).repeat_interleave(3, dim=1)
    report("xattn q=0 -> mean V", err(f64(out), cpu(ref).numpy()), TOL_BF16)
    # L = 1: out equals the single value row (exact up to bf16 output rounding).
    out = sb.xattn_decode(x.q, x.K[:, :, :1].contiguous(), x.V[:, :, :1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out, x.V[:, :, 0].repeat_interleave(3, dim=1))
    # Scale argument: scale 0 is uniform attention as well.
    out = sb.xattn_decode(x.q, x.K, x.V, scale=0.0)
    report("xattn scale=0 -> mean V", err(f64(out), cpu(ref).numpy()), TOL_BF16)


def test_xattn_full_sampled_sequences(sb):
    """16 sequences, 24 query / 8 KV heads, 34816 cached positions; the oracle
    checks every head of three sequences."""
    c = workload.XATTN_DECODE
    x = workload.xattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["L"], seed=11, device=DEV)
    out = sb.xattn_decode(x.q, x.K, x.V)
    torch.cuda.synchronize()
    for b in (0, 7, c["B"] - 1):
        ref = oracle.xattn(cpu(x.q[b:b + 1]), cpu(x.K[b:b + 1]), cpu(x.V[b:b + 1]))
        report("xattn full seq b=%d" % b, err(f64(out[b:b + 1]), ref), TOL_BF16)
    del x, out
    torch.cuda.empty_cache()


def test_xattn_cache_past_2_31_elements(sb):
    """64 sequences at 34816 cached positions: the K and V caches hold 2.28 G
    elements each (9.1 GB together), so the last sequences' rows sit past
    2^31 elements; the plain and the lengths path against the oracle on the
    first and the last two sequences."""
    B, Hq, Hkv, D, L = 64, 24, 8, 128, 34816
    assert B * Hkv * L * D > 2 ** 31
    x = workload.xattn_inputs(B, Hq, Hkv, D, L, seed=12, device=DEV)
    out = sb.xattn_decode(x.q, x.K, x.V)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    lens[B - 1] = L - 1000
    out_l = sb.xattn_decode(x.q, x.K, x.V, lens=lens)
    torch.cuda.synchronize()
    for b in (0, B - 2, B - 1):
        ref = oracle.xattn(cpu(x.q[b:b + 1]), cpu(x.K[b:b + 1]), cpu(x.V[b:b + 1]))
        report("xattn 64 x 34816 seq %d" % b, err(f64(out[b:b + 1]), ref), TOL_BF16)
        n = int(lens[b])
        ref_l = oracle.xattn_varlen(cpu(x.q[b:b + 1]), cpu(x.K[b:b + 1]), cpu(x.V[b:b + 1]), [n])
        report("xattn lengths 64 x 34816 seq %d (%d positions)" % (b, n), err(f64(out_l[b:b + 1]), ref_l), TOL_BF16)
    del x, out, out_l
    torch.cuda.empty_cache()


# -------------------------------------------------------- cross-decoder

def _step_inputs(B, Hq, Hkv, L, d_inner, n_layers, seed, first="xattn", D=128):
    d_model = Hq * D
    kinds = workload.layer_kinds(n_layers, first)
    return workload.crossdecoder_inputs(B, d_model, d_inner, Hq, Hkv, D, L, n_layers, seed=seed, device=DEV,
                                        kinds=kinds)


def _oracle_step(x, rows, Hq):
    layers = [(k, cpu(a), cpu(b)) for k, a, b in x.layers]
    return oracle.crossdecoder(cpu(x.h[rows]), cpu(x.M[rows]), cpu(x.K[rows]), cpu(x.V[rows]), layers, Hq)


@pytest.mark.parametrize("B,Hq,Hkv,L,d_inner,n,first", [(1, 3, 1, 40, 768, 2, "xattn"), (3, 3, 1, 100, 768, 4, "gmu"),
                                                         (5, 6, 2, 333, 512, 4, "xattn"),
                                                         (2, 24, 8, 257, 6144, 2, "xattn")])
def test_crossdecoder_small(sb, B, Hq, Hkv, L, d_inner, n, first):
    x = _step_inputs(B, Hq, Hkv, L, d_inner, n, seed=B + L, first=first)
    h0 = x.h.clone()
    sb.crossdecoder_step(x.h, x.M, x.K, x.V, x.layers)
    torch.cuda.synchronize()
    x.h, hg = h0, x.h
    ref = _oracle_step(x, slice(None), Hq)
    report("crossdecoder B=%d Hq=%d L=%d n=%d %s-first" % (B, Hq, L, n, first), err(f64(hg), ref), TOL_BF16)


def test_crossdecoder_batch_above_64(sb):
    """More than 64 sequences: the decode products run in groups of 64 rows."""
    x = _step_inputs(70, 3, 1, 50, 256, 4, seed=70)
    h0 = x.h.clone()
    sb.crossdecoder_step(x.h, x.M, x.K, x.V, x.layers)
    torch.cuda.synchronize()
    x.h, hg = h0, x.h
    ref = _oracle_step(x, slice(None), 3)
    report("crossdecoder B=70 (two row groups)", err(f64(hg), ref), TOL_BF16)


def test_crossdecoder_full_sampled_sequences(sb):
    """16 layers (8 cross-attention + 8 GMU), 32 sequences, d_model 3072,
    d_inner 6144, 34816 shared cache positions; the oracle replays two whole
    sequences through all 16 layers."""
    c = workload.CROSSDECODER
    x = workload.crossdecoder_inputs(c["B"], c["d_model"], c["d_inner"], c["Hq"], c["Hkv"], c["D"], c["L"],
                                     c["n_layers"], seed=5, device=DEV)
    h0 = x.h.clone()
    sb.crossdecoder_step(x.h, x.M, x.K, x.V, x.layers)
    torch.cuda.synchronize()
    hg = x.h
    x.h = h0
    for b in (0, c["B"] - 1):
        ref = _oracle_step(x, slice(b, b + 1), c["Hq"])
        report("crossdecoder full seq b=%d" % b, err(f64(hg[b:b + 1]), ref), TOL_BF16)
    del x, hg
    torch.cuda.empty_cache()


def test_crossdecoder_teacher_forced_layers(sb):
    """Per-layer diagnostic at the full decode-step width: each GPU layer is fed
    the GPU's own bf16 h of the previous layer and compared with the oracle's
    single layer on that same input.  Every layer must meet the bar on its
    own, so an end-to-end error is accumulated rounding, not a wrong layer."""
    c = workload.CROSSDECODER
    B, L = 2, 4096
    x = workload.crossdecoder_inputs(B, c["d_model"], c["d_inner"], c["Hq"], c["Hkv"], c["D"], L, c["n_layers"],
                                     seed=9, device=DEV)
    h = x.h.clone()
    worst = 0.0
    for i, layer in enumerate(x.layers):
        h_in = h.clone()
        sb.crossdecoder_step(h, x.M, x.K, x.V, [layer])
        torch.cuda.synchronize()
        ref = oracle.crossdecoder(cpu(h_in), cpu(x.M), cpu(x.K), cpu(x.V), [(layer[0], cpu(layer[1]), cpu(layer[2]))],
                                  c["Hq"])
        e = err(f64(h), ref)
        worst = max(worst, e)
        assert e <= TOL_BF16, "layer %d (%s): err %.3e" % (i, layer[0], e)
    report("crossdecoder teacher-forced, worst of 16 layers", worst, TOL_BF16)


def test_crossdecoder_single_sequence_full_width(sb):
    """B = 1 at the full widths (d_model 3072, d_inner 6144): every product of
    the step takes the one-token dot-product path (fp32 query, hi + lo attention
    output into Wo, GMU gate with hi + lo H, residual adds)."""
    c = workload.CROSSDECODER
    x = workload.crossdecoder_inputs(1, c["d_model"], c["d_inner"], c["Hq"], c["Hkv"], c["D"], 3000, 16, seed=17,
                                     device=DEV)
    h0 = x.h.clone()
    sb.crossdecoder_step(x.h, x.M, x.K, x.V, x.layers)
    torch.cuda.synchronize()
    ref = oracle.crossdecoder(cpu(h0), cpu(x.M), cpu(x.K), cpu(x.V), [(k, cpu(a), cpu(b)) for k, a, b in x.layers],
                              c["Hq"])
    report("crossdecoder B=1 full width, 16 layers", err(f64(x.h), ref), TOL_BF16)
    # The complete layer at one token: MLP down-projection has K = 8192.
    e = workload.crossdecoder_ex_inputs(1, c["d_model"], c["d_inner"], 8192, c["Hq"], c["Hkv"], c["D"], 3000, 2,
                                        seed=18, device=DEV, lens=[2500])
    h0 = e.h.clone()
    sb.crossdecoder_step_ex(e.h, e.M, e.K, e.V, e.layers, lens=e.lens)
    torch.cuda.synchronize()
    layers = [{k: (cpu(v) if isinstance(v, torch.Tensor) else v) for k, v in ly.items()} for ly in e.layers]
    ref = oracle.crossdecoder_ex(cpu(h0), cpu(e.M), cpu(e.K), cpu(e.V), layers, c["Hq"], lens=[2500])
    report("complete step B=1 full width, 2 layers", err(f64(e.h), ref), TOL_BF16)
