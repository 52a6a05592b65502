"""GPU parity of the fused differential-attention decode against the fp64
oracle (through the C ABI), plus invariants of the fused kernel.

Tolerance: the bf16 bar, max |gpu - oracle| / max |oracle| <= 2e-2.  The
output is normalised per head (RMS 1 times the gain), so the bar is relative
to O(1) values.
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


@pytest.mark.parametrize("B,Hq,Hkv,L,lens,lam,lam_init", [
    (2, 24, 8, 5000, None, 0.8, 0.8),                      # several chunks, ragged last block
    (3, 24, 8, 777, [777, 31, 0], 0.8, 0.2),               # block boundaries, an empty sequence
    (2, 6, 3, 40000, [40000, 2048], -0.4, 0.5),            # two heads per group, long cache, lambda < 0
    (2, 16, 2, 300, [1, 300], 0.6, 0.8),                   # eight heads per group: all 16 score columns
    (1, 4, 4, 1, None, 0.5, 0.1),                          # one position, one head per group
])
def test_diffattn_small(sb, B, Hq, Hkv, L, lens, lam, lam_init):
    x = workload.diffattn_inputs(B, Hq, Hkv, 128, L, seed=L + Hq, device=DEV)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = sb.diffattn_decode(x.q, x.K, x.V, lam, lam_init, gamma=x.gamma, lens=lt)
    torch.cuda.synchronize()
    ref = oracle.diffattn(cpu(x.q), cpu(x.K), cpu(x.V), lam, lam_init, gamma=cpu(x.gamma), lens=lens)
    for b in range(B):
        if lens is not None and lens[b] == 0:
            assert torch.count_nonzero(out[b]).item() == 0
        else:
            report("diffattn B=%d Hq=%d Hkv=%d L=%d seq %d" % (B, Hq, Hkv, L, b), err(f64(out[b]), ref[b]), TOL_BF16)


def test_diffattn_without_gain(sb):
    x = workload.diffattn_inputs(2, 24, 8, 128, 1000, seed=9, device=DEV)
    out = sb.diffattn_decode(x.q, x.K, x.V, 0.7, 0.6)
    torch.cuda.synchronize()
    ref = oracle.diffattn(cpu(x.q), cpu(x.K), cpu(x.V), 0.7, 0.6)
    report("diffattn without gain", err(f64(out), ref), TOL_BF16)


def test_diffattn_full_size_sampled(sb):
    """16 sequences x 24 heads over 34816 cached positions (the plain decode's
    cache); the oracle checks 3 sequences (sequences are independent)."""
    c = workload.DIFFATTN_DECODE
    x = workload.diffattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["L"], seed=11, device=DEV)
    out = sb.diffattn_decode(x.q, x.K, x.V, c["lam"], c["lam_init"], gamma=x.gamma, eps=c["eps"])
    torch.cuda.synchronize()
    rows = [0, 7, 15]
    idx = torch.tensor(rows, device=DEV)
    ref = oracle.diffattn(cpu(x.q[idx]), cpu(x.K[idx]), cpu(x.V[idx]), c["lam"], c["lam_init"], gamma=cpu(x.gamma),
                          eps=c["eps"])
    report("diffattn 16x24x34816 (3 sampled sequences)", err(f64(out[idx]), ref), TOL_BF16)


def test_diffattn_ragged_full_size_sampled(sb):
    c = workload.DIFFATTN_DECODE
    B = 32
    x = workload.diffattn_inputs(B, c["Hq"], c["Hkv"], c["D"], c["L"], seed=12, device=DEV)
    lens = workload.ragged_lens(B, c["L"], seed=12, min_len=2048, device=DEV)
    out = sb.diffattn_decode(x.q, x.K, x.V, c["lam"], c["lam_init"], gamma=x.gamma, lens=lens, eps=c["eps"])
    torch.cuda.synchronize()
    ln = cpu(lens).numpy()
    rows = sorted(set([int(np.argmin(ln)), int(np.argmax(ln)), 5]))
    idx = torch.tensor(rows, device=DEV)
    ref = oracle.diffattn(cpu(x.q[idx]), cpu(x.K[idx]), cpu(x.V[idx]), c["lam"], c["lam_init"], gamma=cpu(x.gamma),
                          lens=ln[rows], eps=c["eps"])
    report("diffattn ragged 32x34816 (%d sampled sequences)" % len(rows), err(f64(out[idx]), ref), TOL_BF16)


def test_diffattn_lambda_zero_ignores_second_map(sb):
    """At lambda = 0 the second map's query and key halves cannot change a bit."""
    x = workload.diffattn_inputs(2, 24, 8, 128, 2000, seed=13, device=DEV)
    a = sb.diffattn_decode(x.q, x.K, x.V, 0.0, 0.5, gamma=x.gamma)
    q2, K2 = x.q.clone(), x.K.clone()
    q2[..., 64:] = -3.0 * q2[..., 64:]
    K2[..., 64:] = torch.flip(K2[..., 64:], dims=[2])
    b = sb.diffattn_decode(q2, K2, x.V, 0.0, 0.5, gamma=x.gamma)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_diffattn_never_reads_past_the_length(sb):
    x = workload.diffattn_inputs(3, 24, 8, 128, 3000, seed=14, device=DEV)
    lens_l = [100, 2999, 1]
    lens = torch.tensor(lens_l, dtype=torch.int32, device=DEV)
    a = sb.diffattn_decode(x.q, x.K, x.V, 0.8, 0.8, gamma=x.gamma, lens=lens)
    K, V = x.K.clone(), x.V.clone()
    for b, n in enumerate(lens_l):
        K[b, :, n:] = float("nan")
        V[b, :, n:] = float("nan")
    b2 = sb.diffattn_decode(x.q, K, V, 0.8, 0.8, gamma=x.gamma, lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(a, b2)


def test_diffattn_full_lengths_equal_no_lengths(sb, monkeypatch):
    """With the same chunking, lengths equal to L give the same bits as no lengths."""
    monkeypatch.setenv("SAMBAY_XATTN_SPLITS", "3")
    x = workload.diffattn_inputs(4, 24, 8, 128, 9000, seed=15, device=DEV)
    a = sb.diffattn_decode(x.q, x.K, x.V, 0.8, 0.8, gamma=x.gamma)
    b = sb.diffattn_decode(x.q, x.K, x.V, 0.8, 0.8, gamma=x.gamma,
                           lens=torch.full((4,), 9000, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_plain_decode_unchanged_by_the_differential_mode(sb):
    """The plain decode still matches its oracle after the kernel gained the
    differential mode (same instantiation path, DIFF = false)."""
    x = workload.xattn_inputs(2, 24, 8, 128, 4000, seed=16, device=DEV)
    out = sb.xattn_decode(x.q, x.K, x.V)
    torch.cuda.synchronize()
    report("plain decode next to the differential mode", err(f64(out), oracle.xattn(cpu(x.q), cpu(x.K), cpu(x.V))),
           TOL_BF16)
