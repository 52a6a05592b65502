"""GPU parity of the SSM layer over the prompt (mamba_prefill) against the
oracle's definition, T successive fp64 steps.

Tolerances: M and y take the bf16 bar (2e-2, max-abs normalised).  The
final states are held to 2e-2 too: unlike the decode step, the prompt's
projections run as GEMMs with bf16 operands and outputs (xz, u, δ, B, C are
stored bf16), each a 2^-9 relative rounding that the state integrates.
The convolution window after the prompt holds bf16-rounded inputs: within
one bf16 step (2^-7 relative) of the oracle's values at the largest.
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


def f64(t):
    return t.detach().double().cpu().numpy()


def report(name, e, tol):
    print("%-60s err %.3e (tol %.0e)" % (name, e, tol), flush=True)
    assert e <= tol, "%s: %.3e > %.0e" % (name, e, tol)


def _run(sb, B, T, dm, di, N, R, K, seed, name, rows=None):
    m = workload.mamba_inputs(B, dm, di, N, R, K, seed=seed, device=DEV)
    x = workload.normal((B, T, dm), seed=seed + 1000, device=DEV)
    rows = list(range(B)) if rows is None else rows
    idx = torch.tensor(rows, device=DEV)
    conv0, ssm0 = m.conv_state[idx].cpu(), m.ssm_state[idx].cpu()
    M, y = sb.mamba_prefill(x, m.w, m.conv_state, m.ssm_state)
    torch.cuda.synchronize()
    rM, ry, rc, rs = oracle.mamba_prefill(x[idx].cpu(), {k: v.cpu() for k, v in m.w.items()}, conv0, ssm0)
    report("%s M" % name, err(f64(M[idx]), rM), TOL_BF16)
    report("%s y" % name, err(f64(y[idx]), ry), TOL_BF16)
    report("%s ssm_state" % name, err(f64(m.ssm_state[idx]), rs), TOL_BF16)
    if K > 1:
        report("%s conv_state" % name, err(f64(m.conv_state[idx]), rc), 2.0 ** -7)


@pytest.mark.parametrize("B,T,dm,di,N,R,K", [
    (2, 37, 128, 256, 16, 64, 4),     # one partial 64-token chunk of the scan
    (2, 200, 128, 256, 16, 64, 4),    # four chunks, the last ragged
    (1, 130, 64, 128, 64, 64, 4),     # three chunks at 64 states
    (3, 2, 256, 512, 8, 64, 4),       # fewer tokens than the window: the old window shifts
    (1, 65, 64, 128, 32, 64, 1),      # no stored window
    (2, 16, 128, 256, 64, 128, 8),
])
def test_mamba_prefill_small(sb, B, T, dm, di, N, R, K):
    _run(sb, B, T, dm, di, N, R, K, seed=B * T + N, name="prefill B=%d T=%d N=%d K=%d" % (B, T, N, K))


def test_mamba_prefill_full_length(sb):
    """A 2048-token prompt (32 chunks of the scan) at a narrow width."""
    _run(sb, 1, 2048, 128, 256, 16, 64, 4, seed=11, name="prefill full length 1 x 2048")


def test_mamba_prefill_full_width(sb):
    """d_model 3072, d_inner 6144 over 96 prompt tokens of 2 sequences."""
    c = workload.MAMBA_DECODE
    _run(sb, 2, 96, c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"], c["d_conv"], seed=7,
         name="prefill full width 2 x 96")


def test_mamba_prefill_then_decode_continues(sb):
    """A prompt of T tokens then one decode step equals a prompt of T + 1
    tokens (last token's outputs and the states), within the bf16 bar."""
    m = workload.mamba_inputs(2, 128, 256, 16, 64, 4, seed=8, device=DEV)
    x = workload.normal((2, 21, 128), seed=9, device=DEV)
    c1, s1 = m.conv_state.clone(), m.ssm_state.clone()
    M_all, y_all = sb.mamba_prefill(x, m.w, c1, s1)
    c2, s2 = m.conv_state.clone(), m.ssm_state.clone()
    sb.mamba_prefill(x[:, :20].contiguous(), m.w, c2, s2)
    M1, y1 = sb.mamba_decode_step(x[:, 20].contiguous(), m.w, c2, s2)
    torch.cuda.synchronize()
    assert err(f64(M1), f64(M_all[:, 20])) <= TOL_BF16
    assert err(f64(y1), f64(y_all[:, 20])) <= TOL_BF16
    assert err(f64(s2), f64(s1)) <= TOL_BF16
