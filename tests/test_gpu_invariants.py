"""GPU invariants of the HIP path: determinism, batch-permutation
equivariance, independence from the launch plan (split counts, K splits,
prefill vs decode kernels), and the structural special cases of the layer
array (all-GMU, as in the pages' all-GMU ablation; all-attention)."""
import os

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


class _env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def test_determinism(sb):
    x = workload.xattn_inputs(4, 24, 8, 128, 5000, seed=1, device=DEV)
    a, b = sb.xattn_decode(x.q, x.K, x.V), sb.xattn_decode(x.q, x.K, x.V)
    g = workload.gmu_inputs(32, 3072, 6144, seed=2, device=DEV)
    y1, y2 = sb.gmu_forward(g.M, g.X, g.W1, g.W2), sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    p = workload.gmu_inputs(300, 256, 512, seed=3, device=DEV)
    z1, z2 = sb.gmu_forward(p.M, p.X, p.W1, p.W2), sb.gmu_forward(p.M, p.X, p.W1, p.W2)
    s = workload.crossdecoder_inputs(3, 384, 768, 3, 1, 128, 500, 4, seed=4, device=DEV)
    h0 = s.h.clone()
    sb.crossdecoder_step(s.h, s.M, s.K, s.V, s.layers)
    h1 = s.h.clone()
    s.h.copy_(h0)
    sb.crossdecoder_step(s.h, s.M, s.K, s.V, s.layers)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(y1, y2) and torch.equal(z1, z2) and torch.equal(h1, s.h)


def test_batch_permutation_equivariance(sb):
    """Sequences are independent: permuting them permutes the outputs bit for bit."""
    x = workload.xattn_inputs(6, 24, 8, 128, 1000, seed=5, device=DEV)
    perm = torch.tensor([3, 0, 5, 1, 4, 2], device=DEV)
    out = sb.xattn_decode(x.q, x.K, x.V)
    outp = sb.xattn_decode(x.q[perm].contiguous(), x.K[perm].contiguous(), x.V[perm].contiguous())
    g = workload.gmu_inputs(40, 3072, 6144, seed=6, device=DEV)
    pg = torch.randperm(40, generator=torch.Generator().manual_seed(0)).to(DEV)
    y = sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    yp = sb.gmu_forward(g.M[pg].contiguous(), g.X[pg].contiguous(), g.W1, g.W2)
    torch.cuda.synchronize()
    assert torch.equal(out[perm], outp)
    assert torch.equal(y[pg], yp)


@pytest.mark.parametrize("L", [33, 4097, 34816])
def test_split_count_invariance(sb, L):
    """Any chunking of the cache gives the same attention up to fp32 rounding."""
    x = workload.xattn_inputs(2, 24, 8, 128, L, seed=L, device=DEV)
    outs = []
    for S in (1, 3, 8, 64):
        with _env(SAMBAY_XATTN_SPLITS=S):
            outs.append(sb.xattn_decode(x.q, x.K, x.V).double().cpu().numpy())
    ref = oracle.xattn(x.q.cpu(), x.K.cpu(), x.V.cpu())
    for o in outs:
        assert err(o, ref) <= TOL_BF16
        assert err(o, outs[0]) <= 1e-2


def test_k_split_invariance(sb):
    g = workload.gmu_inputs(32, 3072, 6144, seed=8, device=DEV)
    outs = []
    for ks in (1, 2, 4):
        with _env(SAMBAY_SKINNY_KSPLIT=ks):
            outs.append(sb.gmu_forward(g.M, g.X, g.W1, g.W2).double().cpu().numpy())
    ref = oracle.gmu(g.M.cpu(), g.X.cpu(), g.W1.cpu(), g.W2.cpu())
    for o in outs:
        assert err(o, ref) <= TOL_BF16
        assert err(o, outs[0]) <= 1e-2


def test_prefill_rows_match_decode_rows(sb):
    """The MFMA GEMM path (rows > 64) and the decode path (rows <= 64) agree."""
    g = workload.gmu_inputs(128, 512, 1024, seed=9, device=DEV)
    full = sb.gmu_forward(g.M, g.X, g.W1, g.W2)
    parts = torch.cat([sb.gmu_forward(g.M[i:i + 64].contiguous(), g.X[i:i + 64].contiguous(), g.W1, g.W2)
                       for i in (0, 64)])
    torch.cuda.synchronize()
    assert err(full.double().cpu().numpy(), parts.double().cpu().numpy()) <= 1e-2


@pytest.mark.parametrize("kind", ["gmu", "xattn"])
def test_uniform_layer_arrays(sb, kind):
    """All-GMU (the pages' all-GMU ablation, structurally) and all-attention stacks."""
    s = workload.crossdecoder_inputs(4, 384, 768, 3, 1, 128, 300, 4, seed=10, device=DEV, kinds=[kind] * 4)
    h0 = s.h.clone()
    sb.crossdecoder_step(s.h, s.M, s.K, s.V, s.layers)
    torch.cuda.synchronize()
    ref = oracle.crossdecoder(h0.cpu(), s.M.cpu(), s.K.cpu(), s.V.cpu(),
                              [(k, a.cpu(), b.cpu()) for k, a, b in s.layers], 3)
    assert err(s.h.double().cpu().numpy(), ref) <= TOL_BF16


def test_zero_batch_is_noop(sb):
    s = workload.crossdecoder_inputs(1, 384, 768, 3, 1, 128, 10, 2, seed=11, device=DEV)
    h = s.h[:0]
    sb.crossdecoder_step(h, s.M[:0], s.K[:0], s.V[:0], s.layers)
    q = torch.zeros(0, 3, 128, dtype=torch.bfloat16, device=DEV)
    assert sb.xattn_decode(q, s.K[:0], s.V[:0]).shape == (0, 3, 128)


def test_step_object_reuse_and_stream(sb):
    """A prepared step replays identically, also on a side stream."""
    s = workload.crossdecoder_inputs(2, 384, 768, 3, 1, 128, 200, 2, seed=12, device=DEV)
    h0 = s.h.clone()
    step = sb.CrossDecoderStep(s.h, s.M, s.K, s.V, s.layers)
    step()
    torch.cuda.synchronize()
    first = s.h.clone()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        s.h.copy_(h0)
        step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    assert torch.equal(first, s.h)


def test_ceiling_probes_run(sb):
    """The benchmark probes run and report rates within physical limits."""
    buf = torch.ones(64 << 20, dtype=torch.float32, device=DEV)
    gbps = sb.probe_stream_read_gbps(buf)
    tf = sb.probe_mfma_tflops(DEV, iters=200)
    assert 100.0 < gbps < 8000.0 * 1.05
    assert 10.0 < tf < 2500.0 * 1.05


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("complete", [False, True])
def test_step_replays_from_a_hip_graph(sb, complete):
    """The prepared steps enqueue only kernels (no memset, no allocation), so a
    captured HIP graph replays them bit-identically, also with eager work and
    synchronisations between replays."""
    if complete:
        x = workload.crossdecoder_ex_inputs(40, 384, 768, 512, 3, 1, 128, 300, 4, seed=13, device=DEV,
                                            lens=[300, 1, 77] + [200] * 37)
        step = sb.CrossDecoderStepEx(x.h, x.M, x.K, x.V, x.layers, lens=x.lens)
    else:
        x = workload.crossdecoder_inputs(40, 384, 768, 3, 1, 128, 300, 4, seed=13, device=DEV)
        step = sb.CrossDecoderStep(x.h, x.M, x.K, x.V, x.layers)
    h_in = x.h.clone()

    def run():
        x.h.copy_(h_in)
        step()

    run()
    torch.cuda.synchronize()
    ref = x.h.clone()
    g = _capture(run)
    for _ in range(4):
        x.h.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x.h, ref)
        run()
        torch.cuda.synchronize()
        assert torch.equal(x.h, ref)
