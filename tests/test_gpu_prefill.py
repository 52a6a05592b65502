"""GPU parity of the prefill attention (causal, optionally sliding-window)
against the fp64 oracle, through the C ABI.  Tolerance: the bf16 bar,
max |gpu - oracle| / max |oracle| <= 2e-2."""
import numpy as np
import pytest
import torch

import oracle
import workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def sb():
    import attention_decoding_amd as sb
    return sb


def err(y, ref):
    y, ref = np.asarray(y, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(y - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def f64(t):
    return t.detach().double().cpu().numpy()


def report(name, e, tol):
    print("%-60s err %.3e (tol %.0e)" % (name, e, tol), flush=True)
    assert e <= tol, "%s: %.3e > %.0e" % (name, e, tol)


@pytest.mark.parametrize("B,T,Hq,Hkv,W", [
    (2, 100, 6, 2, 0),        # causal, a ragged last tile
    (1, 300, 24, 8, 64),      # window shorter than the tile span
    (2, 65, 24, 8, 256),      # window longer than the prompt: plain causal
    (1, 1, 3, 1, 0),          # one token
    (1, 257, 8, 8, 33),       # window not a multiple of the key block
    (3, 130, 4, 1, 0),        # four query heads per KV head
])
def test_prefill_small(sb, B, T, Hq, Hkv, W):
    x = workload.prefill_inputs(B, T, Hq, Hkv, 128, seed=T + W, device=DEV)
    out = sb.attn_prefill(x.q, x.k, x.v, window=W)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), W)
    report("prefill B=%d T=%d %d/%d W=%d" % (B, T, Hq, Hkv, W), err(f64(out), ref), TOL_BF16)


def test_prefill_window_one_is_the_own_value(sb):
    x = workload.prefill_inputs(1, 129, 6, 2, 128, seed=3, device=DEV)
    out = sb.attn_prefill(x.q, x.k, x.v, window=1)
    torch.cuda.synchronize()
    assert torch.equal(out, x.v.repeat_interleave(3, dim=2))


def test_prefill_full_size_window(sb):
    """4 prompts of 2048 tokens, 24 query / 8 KV heads, window 256."""
    c = workload.ATTN_PREFILL
    x = workload.prefill_inputs(c["B"], c["T"], c["Hq"], c["Hkv"], c["D"], seed=4, device=DEV)
    out = sb.attn_prefill(x.q, x.k, x.v, window=c["window"])
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), c["window"])
    report("prefill 4 x 2048, window 256", err(f64(out), ref), TOL_BF16)


def test_prefill_full_size_causal(sb):
    """One prompt of 2048 tokens attending causally over all of it."""
    c = workload.ATTN_PREFILL
    x = workload.prefill_inputs(1, c["T"], c["Hq"], c["Hkv"], c["D"], seed=5, device=DEV)
    out = sb.attn_prefill(x.q, x.k, x.v, window=0)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), 0)
    report("prefill 1 x 2048 causal", err(f64(out), ref), TOL_BF16)


def test_prefill_window_beyond_prompt_equals_causal(sb):
    x = workload.prefill_inputs(2, 200, 6, 2, 128, seed=6, device=DEV)
    a = sb.attn_prefill(x.q, x.k, x.v, window=0)
    b = sb.attn_prefill(x.q, x.k, x.v, window=200)
    c = sb.attn_prefill(x.q, x.k, x.v, window=10000)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


# Heads per workgroup that divide each case's group of query heads.
_HEADS_CASES = [(heads,) + case for case in [
    (2, 100, 6, 2, 0),        # causal, a ragged last tile
    (1, 300, 24, 8, 64),      # window shorter than the tile span
    (3, 130, 12, 2, 0),       # six query heads per KV head
] for heads in (1, 2, 3) if (case[2] // case[3]) % heads == 0]


@pytest.mark.parametrize("heads,B,T,Hq,Hkv,W", _HEADS_CASES)
def test_prefill_heads_per_workgroup(sb, monkeypatch, heads, B, T, Hq, Hkv, W):
    """One workgroup serving 1, 2 or 3 query heads of a KV head (forced by
    SAMBAY_PREFILL_HEADS), against the oracle."""
    monkeypatch.setenv("SAMBAY_PREFILL_HEADS", str(heads))
    x = workload.prefill_inputs(B, T, Hq, Hkv, 128, seed=7 * T + W + heads, device=DEV)
    out = sb.attn_prefill(x.q, x.k, x.v, window=W)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), W)
    report("prefill %d heads/wg B=%d T=%d %d/%d W=%d" % (heads, B, T, Hq, Hkv, W), err(f64(out), ref), TOL_BF16)


def test_prefill_full_size_causal_three_heads(sb, monkeypatch):
    """The 2048-token causal prompt with three query heads per workgroup."""
    monkeypatch.setenv("SAMBAY_PREFILL_HEADS", "3")
    c = workload.ATTN_PREFILL
    x = workload.prefill_inputs(1, c["T"], c["Hq"], c["Hkv"], c["D"], seed=8, device=DEV)
    out = sb.attn_prefill(x.q, x.k, x.v, window=0)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), 0)
    report("prefill 1 x 2048 causal, 3 heads per workgroup", err(f64(out), ref), TOL_BF16)
