"""xattn_decode_noalloc: the cross-attention decode with its partials in the
library's own per-GPU scratch array (no workspace, nothing allocated) against
xattn_decode with a caller workspace, through the C ABI.

Both run the same kernels with the same chunk plan, so their outputs must be
bit-identical; the bf16 bar against the fp64 oracle (max-abs normalised,
2e-2) is checked as well.  Two calls in a row, the second smaller, show that
what the first call left in the array does not leak into the second.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def sb():
    import attention_decoding_amd as sb
    return sb


def _err(y, ref):
    y, ref = np.asarray(y, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def test_noalloc_matches_the_workspace_entry_point_twice(sb):
    shapes = [(16, 34816, 41), (3, 777, 42)]          # (B, L, seed): the second call smaller
    for B, L, seed in shapes:
        print("no-alloc case B=%d L=%d" % (B, L), flush=True)
        x = workload.xattn_inputs(B, 24, 8, 128, L, seed=seed, device=DEV)
        ref = sb.xattn_decode(x.q, x.K, x.V)
        got = torch.full_like(ref, float("nan"))
        sb.xattn_decode_noalloc(x.q, x.K, x.V, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "B=%d L=%d: differs from xattn_decode" % (B, L)
        rows = [0, B - 1]
        o = oracle.xattn(x.q[rows].cpu(), x.K[rows].cpu(), x.V[rows].cpu(), 1.0 / math.sqrt(128))
        assert _err(got[rows].double().cpu().numpy(), o) <= 2e-2
        del x

