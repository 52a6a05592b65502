"""GPU parity of the SSM decode step (the Mamba layer producing the GMU
memory M) against the fp64 oracle, through the C ABI.

Tolerances: M and y (bf16 outputs) are held to the bf16 bar, max |gpu -
oracle| / max |oracle| <= 2e-2.  The fp32 states are held to 1e-4 (max-abs
normalised): every quantity they depend on accumulates in fp32 (products
of bf16 weights with fp32 or bf16 hi + lo operands, ~1e-6 relative), so a
wrong index or a dropped term is far above it while rounding is far below.
The shifted part of the convolution window is moved, not computed: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BF16 = 2e-2
TOL_STATE = 1e-4


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


def _cpu_w(m):
    return {k: v.cpu() for k, v in m.w.items()}


def _run(sb, m, name, rows=None):
    B = m.x.shape[0]
    rows = list(range(B)) if rows is None else rows
    assert 0 <= min(rows) and max(rows) < B, "sampled rows outside the batch"  # checked before any GPU gather
    idx = torch.tensor(rows, device=DEV)
    conv0, ssm0 = m.conv_state[idx].cpu(), m.ssm_state[idx].cpu()
    M, y = sb.mamba_decode_step(m.x, m.w, m.conv_state, m.ssm_state)
    torch.cuda.synchronize()
    rM, ry, rc, rs = oracle.mamba_step(m.x[idx].cpu(), _cpu_w(m), conv0, ssm0)
    report("%s M" % name, err(f64(M[idx]), rM), TOL_BF16)
    report("%s y" % name, err(f64(y[idx]), ry), TOL_BF16)
    report("%s ssm_state" % name, err(f64(m.ssm_state[idx]), rs), TOL_STATE)
    if rc.shape[-1] > 0:
        report("%s conv_state" % name, err(f64(m.conv_state[idx]), rc), TOL_STATE)
        assert np.array_equal(f64(m.conv_state[idx])[:, :, :-1], conv0.double().numpy()[:, :, 1:])


@pytest.mark.parametrize("B,dm,di,N,R,K", [
    (3, 128, 256, 16, 64, 4),
    (5, 256, 512, 8, 32, 2),
    (2, 128, 256, 32, 16, 1),       # no stored window
    (4, 64, 128, 64, 256, 8),       # widest state, longest rank and window
])
def test_mamba_small(sb, B, dm, di, N, R, K):
    m = workload.mamba_inputs(B, dm, di, N, R, K, seed=B + dm + N, device=DEV)
    _run(sb, m, "mamba B=%d %dx%d N=%d R=%d K=%d" % (B, dm, di, N, R, K))


@pytest.mark.parametrize("B", [1, 17, 32, 33, 70])
def test_mamba_full_width(sb, B):
    """d_model 3072, d_inner 6144, 16 states, rank 192, 4 taps: one token (the
    one-token product path), 17 and 33 tokens (one past a 16-token tile), the
    32-sequence batch, two token groups."""
    c = workload.MAMBA_DECODE
    m = workload.mamba_inputs(B, c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"], c["d_conv"], seed=B,
                              device=DEV)
    rows = None if B <= 33 else [0, 31, 63, 64, B - 1]   # every row up to 33; sampled across both groups above
    _run(sb, m, "mamba full width B=%d" % B, rows)


def test_mamba_several_steps(sb):
    """Six steps, the GPU and the oracle each carrying their own states."""
    m = workload.mamba_inputs(3, 128, 256, 16, 64, 4, seed=40, device=DEV)
    conv, ssm = m.conv_state.cpu(), m.ssm_state.cpu()
    w = _cpu_w(m)
    for t in range(6):
        x = workload.normal((3, 128), seed=500 + t, device=DEV)
        M, y = sb.mamba_decode_step(x, m.w, m.conv_state, m.ssm_state)
        torch.cuda.synchronize()
        rM, ry, conv, ssm = oracle.mamba_step(x.cpu(), w, conv, ssm)
        report("mamba step %d M" % t, err(f64(M), rM), TOL_BF16)
        report("mamba step %d y" % t, err(f64(y), ry), TOL_BF16)
    report("mamba after 6 steps ssm_state", err(f64(m.ssm_state), ssm), TOL_STATE)
    report("mamba after 6 steps conv_state", err(f64(m.conv_state), conv), TOL_STATE)


def test_mamba_batch_rows_are_independent(sb):
    """A sequence's results do not depend on the rest of the batch (same
    product plans: both batches in one token group of the same size)."""
    m = workload.mamba_inputs(8, 128, 256, 16, 64, 4, seed=41, device=DEV)
    c0, s0 = m.conv_state.clone(), m.ssm_state.clone()
    M1, y1 = sb.mamba_decode_step(m.x, m.w, m.conv_state, m.ssm_state)
    x2 = m.x.clone()
    x2[1:] = -x2[1:]
    c2, s2 = c0.clone(), s0.clone()
    c2[1:] += 1.0
    M2, y2 = sb.mamba_decode_step(x2, m.w, c2, s2)
    torch.cuda.synchronize()
    assert torch.equal(M1[0], M2[0]) and torch.equal(y1[0], y2[0])
    assert torch.equal(m.ssm_state[0], s2[0]) and torch.equal(m.conv_state[0], c2[0])
