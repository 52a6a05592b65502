"""GPU parity of the self-decoder attention decode step (cache append, then
attention over the visible positions; full cache or sliding-window ring)
against the fp64 oracle, through the C ABI.

The stored cache rows are byte work: the updated cache must equal the
oracle's bit for bit.  The attention output is held to the bf16 bar,
max |gpu - oracle| / max |oracle| <= 2e-2.
"""
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


def cpu(t):
    return t.detach().cpu()


def f64(t):
    return t.detach().double().cpu().numpy()


def report(name, e, tol):
    print("%-60s err %.3e (tol %.0e)" % (name, e, tol), flush=True)
    assert e <= tol, "%s: %.3e > %.0e" % (name, e, tol)


def _check(sb, x, pos, window, name, rows=None):
    B = x.q.shape[0]
    rows = list(range(B)) if rows is None else rows
    idx = torch.tensor(rows, device=DEV)
    q, kn, vn = cpu(x.q[idx]), cpu(x.k_new[idx]), cpu(x.v_new[idx])
    K0, V0 = cpu(x.K[idx]), cpu(x.V[idx])
    pt = torch.tensor(pos, dtype=torch.int32, device=DEV)
    out = sb.selfattn_decode(x.q, x.k_new, x.v_new, x.K, x.V, pt, window=window)
    torch.cuda.synchronize()
    ref, Kr, Vr = oracle.selfattn(q, kn, vn, K0, V0, [pos[r] for r in rows], window=window)
    assert np.array_equal(f64(x.K[idx]), Kr), "%s: key cache differs from the oracle's" % name
    assert np.array_equal(f64(x.V[idx]), Vr), "%s: value cache differs from the oracle's" % name
    for i, r in enumerate(rows):
        if pos[r] < 0:
            assert torch.count_nonzero(out[r]).item() == 0
        else:
            report("%s seq %d pos %d" % (name, r, pos[r]), err(f64(out[r]), ref[i]), TOL_BF16)


@pytest.mark.parametrize("B,L,pos", [
    (3, 777, [776, 30, -1]),          # last position, block boundary, inactive
    (2, 5000, [0, 4096]),             # first position, chunk boundary
])
def test_selfattn_full_cache_small(sb, B, L, pos):
    x = workload.selfattn_inputs(B, 24, 8, 128, L, seed=L, device=DEV)
    _check(sb, x, pos, 0, "selfattn full L=%d" % L)


@pytest.mark.parametrize("W,pos", [(256, [0, 100, 255, 5000]), (32, [31, 32, 33, 95]), (256, [-1, 1, 300, 511])])
def test_selfattn_window_small(sb, W, pos):
    x = workload.selfattn_inputs(len(pos), 24, 8, 128, W, seed=W + len(pos), device=DEV)
    _check(sb, x, pos, W, "selfattn window %d" % W)


def test_selfattn_ring_step_by_step(sb):
    """Twenty decode steps through an 8-slot ring, GPU and oracle each
    carrying their own cache; every step's output and the final caches agree."""
    B, Hq, Hkv, D, W = 2, 6, 2, 128, 8
    x = workload.selfattn_inputs(B, Hq, Hkv, D, W, seed=21, device=DEV)
    Ko, Vo = cpu(x.K).double().numpy(), cpu(x.V).double().numpy()
    for t in range(20):
        s = workload.selfattn_inputs(B, Hq, Hkv, D, 1, seed=100 + t, device=DEV)
        pos = [t, t + 3]
        out = sb.selfattn_decode(s.q, s.k_new, s.v_new, x.K, x.V, torch.tensor(pos, dtype=torch.int32, device=DEV),
                                 window=W)
        torch.cuda.synchronize()
        ref, Ko, Vo = oracle.selfattn(cpu(s.q), cpu(s.k_new), cpu(s.v_new), Ko, Vo, pos, window=W)
        assert err(f64(out), ref) <= TOL_BF16, "step %d" % t
    assert np.array_equal(f64(x.K), Ko) and np.array_equal(f64(x.V), Vo)


def test_selfattn_full_size_sampled(sb):
    """32 sequences appending to the 34816-position shared cache at positions
    2047 .. 34815; every appended row is checked, the oracle runs 3 sequences."""
    c = workload.SELFATTN_FULL
    x = workload.selfattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["L"], seed=22, device=DEV)
    lens = workload.ragged_lens(c["B"], c["L"], seed=22, min_len=c["min_len"])
    pos = [int(n) - 1 for n in lens]
    _check(sb, x, pos, 0, "selfattn full 32x34816", rows=[int(np.argmin(pos)), int(np.argmax(pos)), 9])
    b = torch.arange(c["B"], device=DEV)
    p = torch.tensor(pos, device=DEV, dtype=torch.long)
    assert torch.equal(x.K[b, :, p], x.k_new) and torch.equal(x.V[b, :, p], x.v_new)


def test_selfattn_window_full_size(sb):
    c = workload.SELFATTN_SWA
    x = workload.selfattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["window"], seed=23, device=DEV)
    lens = workload.ragged_lens(c["B"], 34816, seed=23, min_len=c["min_len"])
    _check(sb, x, [int(n) - 1 for n in lens], c["window"], "selfattn window 256, 32 sequences")


def test_selfattn_equals_append_then_ragged_attention(sb):
    """The step's attention is the ragged decode over the updated cache with
    lengths pos + 1: same kernels and plan, same bits."""
    x = workload.selfattn_inputs(4, 24, 8, 128, 3000, seed=24, device=DEV)
    pos = torch.tensor([2999, 0, 1234, 77], dtype=torch.int32, device=DEV)
    a = sb.selfattn_decode(x.q, x.k_new, x.v_new, x.K, x.V, pos)
    b = sb.xattn_decode(x.q, x.K, x.V, lens=pos + 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_selfattn_position_past_the_cache_is_clamped(sb):
    """window 0, pos >= L: nothing is stored and all L positions are visible."""
    x = workload.selfattn_inputs(2, 24, 8, 128, 500, seed=25, device=DEV)
    K0, V0 = x.K.clone(), x.V.clone()
    a = sb.selfattn_decode(x.q, x.k_new, x.v_new, x.K, x.V, torch.tensor([500, 9000], dtype=torch.int32, device=DEV))
    b = sb.xattn_decode(x.q, K0, V0, lens=torch.full((2,), 500, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(x.K, K0) and torch.equal(x.V, V0)
    assert torch.equal(a, b)
