#!/usr/bin/env python3
"""Benchmark of the SambaY cross-decoder decode step on one MI355X.

Workload (synthetic, seeded, shaped like the pages' 2K-prompt + 32K-generation
decode): one step of a 16-layer cross-decoder — 8 cross-attention layers over
the single shared KV cache alternating with 8 GMU layers — for B = 32
sequences, d_model 3072, d_inner 6144, 24 query / 8 KV heads of 128, and
34816 cached positions.  Every input is resident in HBM before timing.

A step = refresh the residual stream h from the step's input (the token's
self-decoder output) and run crossdecoder_step through the C ABI.  value =
B / (seconds per step), in tokens/s.

Also reported on the same JSON line:
  roofline      the split-K attention kernel (the dominant one): algorithmic
                bytes per launch (the KV cache it must read) / its mean launch
                time, measured with HIP events on its own stream inside the
                timed region; peak 8 TB/s; `traffic` = measured HBM bytes per
                launch from the committed rocprofv3 counter summary when it
                matches the current kernel source, else null.
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
                (a few whole sequences through all 16 layers), on the host.
  kernels       per-kernel-kind times and rates from a short extra pass.
  graph_replay  the same step replayed from a captured HIP graph (host launch
                cost removed), checked bitwise against the eager step.
  configs       the other workloads in compact form: the tiny fp32 GMU against
                the oracle, GMU prefill (TFLOP/s), GMU decode at 1/8/32/64
                tokens and the 16-sequence cross-attention decode (GB/s).
  library       the version string of the loaded library, with the hash of
                the sources it was built from and of the sources present.

The timed steps carry no instrumentation; the split kernel's launch time for
`roofline` comes from the same number of steps run again with the library's
HIP-event brackets on that kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs] [--all]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "cross-decoder decode tokens/s @34K ctx; GMU & XA achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "xattn_split_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "attention_decoding_amd", "csrc", f) for f in ("xattn.hip", "device.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def step_bytes(c) -> dict:
    """Algorithmic HBM bytes of one step: what the method must read or write."""
    B, dm, di, Hkv, D, L = c["B"], c["d_model"], c["d_inner"], c["Hkv"], c["D"], c["L"]
    n_x = n_g = c["n_layers"] // 2
    kv = B * Hkv * L * D * 2 * 2
    xa_w, gmu_w = 2 * dm * dm * 2, 2 * dm * di * 2
    xa_state, gmu_state = B * 2 * dm * 2, B * (dm + di + dm) * 2
    return dict(kv=n_x * kv, kv_per_layer=kv, xattn_weights=n_x * xa_w, gmu_weights=n_g * gmu_w,
                state=n_x * xa_state + n_g * gmu_state,
                total=n_x * (kv + xa_w + xa_state) + n_g * (gmu_w + gmu_state))


def traffic_for_current_kernel():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(h_in, x, c, n_seq: int):
    """Times the fp64 oracle on the first n_seq sequences of the step's input, on
    all host threads and (one sequence) on one thread.  Returns the report and the
    oracle's output for those sequences."""
    import oracle

    layers = [(k, a.cpu(), b.cpu()) for k, a, b in x.layers]
    rows = slice(0, n_seq)
    h, M, K, V = h_in[rows].cpu(), x.M[rows].cpu(), x.K[rows].cpu(), x.V[rows].cpu()
    cores = oracle.max_threads()
    t0 = time.perf_counter()
    ref = oracle.crossdecoder(h, M, K, V, layers, c["Hq"])
    dt = time.perf_counter() - t0
    oracle.set_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.crossdecoder(h[:1], M[:1], K[:1], V[:1], layers, c["Hq"])
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_threads(cores)
    rep = {"value": n_seq / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": "%d of %d sequences, one decode token each, through all %d layers at %d cached positions "
                     "(fp64 oracle, sequences are independent); %.1f s" % (n_seq, c["B"], c["n_layers"], c["L"], dt),
           "single_core_value": 1.0 / dt1, "single_core_sample": "1 sequence on 1 thread; %.1f s" % dt1}
    return rep, ref


def time_calls(fn, n: int, warmup: int = 3) -> float:
    """Mean milliseconds per call of fn() over n calls (HIP events on the current stream)."""
    import torch

    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def time_graph(fn, n: int, reps: int = 10) -> float:
    """Mean milliseconds per call of fn() replayed from a HIP graph of n calls
    (no host launch cost: for calls whose kernels take a few microseconds)."""
    import torch

    fn(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fn(0)                      # any workspace the binding keeps per stream is made outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n)


WORKLOAD_GROUPS = ("gmu_prefill", "gmu_decode", "attention", "ragged", "mamba_decode", "mamba_prefill",
                   "sambay_prefill", "sambay_decode", "attn_prefill", "crossdecoder_ex")


def other_workloads(sb, workload, dev, read_gbps: float, mfma_tflops: float, only=None) -> dict:
    """Kernel-level rates of the other workloads (not part of `value`);
    `only`: a subset of WORKLOAD_GROUPS to run (None: all)."""
    import torch

    res = {}
    want = lambda name: only is None or name in only
    if want("gmu_prefill"):
        # GMU prefill: 4 x 2048 rows, 2560 -> 5120 -> 2560.
        c = workload.GMU_PREFILL
        rows = c["batch"] * c["seq"]
        g = workload.gmu_inputs(rows, c["d_model"], c["d_inner"], seed=1, device=dev)
        Y = torch.empty(rows, c["d_model"], dtype=torch.bfloat16, device=dev)
        # MFMA-bound: 20 warm-up calls let the clocks settle first (the first
        # calls of a process read up to ~20% slow).
        ms = time_calls(lambda i: sb.gmu_forward(g.M, g.X, g.W1, g.W2, out=Y), 20, warmup=20)
        flops = 4.0 * rows * c["d_model"] * c["d_inner"]
        # Context only: the same two products through torch's bf16 matmul (the
        # vendor BLAS), unfused, with the SiLU·M product as separate elementwise
        # work — what a caller without this library would run.
        F = torch.nn.functional
        ms_lib = time_calls(lambda i: F.linear(g.M * F.silu(F.linear(g.X, g.W1)), g.W2), 20, warmup=10)
        ms_lib_gemms = time_calls(lambda i: (F.linear(g.X, g.W1), F.linear(g.M, g.W2)), 20, warmup=10)
        res["gmu_prefill_8192x2560x5120"] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                                             "frac_of_bf16_peak": round(flops / ms / 1e9 / 2500.0, 4),
                                             "frac_of_measured_mfma_loop": round(flops / ms / 1e9 / mfma_tflops, 4),
                                             "context_torch_gmu_ms": round(ms_lib, 4),
                                             "context_torch_two_matmuls_ms": round(ms_lib_gemms, 4),
                                             "context_torch_two_matmuls_tflops": round(flops / ms_lib_gemms / 1e9, 1)}
        del g, Y
    if want("gmu_decode"):
        # GMU decode: B in {1, 8, 32, 64}, 3072 -> 6144 -> 3072, 8 rotating weight sets (604 MB).
        c = workload.GMU_DECODE
        sets = [workload.gmu_inputs(1, c["d_model"], c["d_inner"], seed=2, device=dev, weight_set=k) for k in range(8)]
        for B in c["batches"]:
            gi = workload.gmu_inputs(B, c["d_model"], c["d_inner"], seed=3 + B, device=dev)
            Y = torch.empty(B, c["d_model"], dtype=torch.bfloat16, device=dev)
            ms = time_calls(lambda i: sb.gmu_forward(gi.M, gi.X, sets[i % 8].W1, sets[i % 8].W2, out=Y), 64)
            nbytes = 2 * c["d_model"] * c["d_inner"] * 2 + B * (2 * c["d_model"] + c["d_inner"]) * 2
            gbps = nbytes / ms / 1e6
            res["gmu_decode_B%d" % B] = {"us_per_call": round(1e3 * ms, 2), "gbps": round(gbps, 1),
                                         "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                                         "frac_of_stream_read": round(gbps / read_gbps, 4)}
        # Context: two streaming reads of the same two weight matrices (the
        # library's read probe, same rotation), i.e. what a perfect kernel pair
        # could approach at this size with two launches.
        def plain_reads(i):
            sb.probe_stream_read_raw(sets[i % 8].W1)
            sb.probe_stream_read_raw(sets[i % 8].W2)

        pr = time_calls(plain_reads, 64)
        for B in c["batches"]:
            res["gmu_decode_B%d" % B]["two_plain_reads_us"] = round(1e3 * pr, 2)
            res["gmu_decode_B%d" % B]["frac_of_two_plain_reads"] = round(pr / (res["gmu_decode_B%d" % B]["us_per_call"]
                                                                              / 1e3), 4)
        del sets
    if want("attention"):
        # Attention alone: 16 x 24 q heads, 8 KV heads, 34816 positions.
        c = workload.XATTN_DECODE
        x = workload.xattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["L"], seed=4, device=dev)
        out = torch.empty(c["B"], c["Hq"], c["D"], dtype=torch.bfloat16, device=dev)
        ms = time_calls(lambda i: sb.xattn_decode(x.q, x.K, x.V, out=out), 20)
        nbytes = c["B"] * c["Hkv"] * c["L"] * c["D"] * 4
        res["xattn_decode_B16_L34816"] = {"us_per_call": round(1e3 * ms, 1), "gbps": round(nbytes / ms / 1e6, 1),
                                          "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                                          "frac_of_stream_read": round(nbytes / ms / 1e6 / read_gbps, 4)}
        # Differential attention on the same cache: both maps in one pass, against
        # two plain decode passes over it (the cache bytes that an implementation
        # running one attention pass per map reads).
        c = workload.DIFFATTN_DECODE
        gain = workload.diffattn_gain(c["D"], seed=4, device=dev)
        ms_d = time_calls(lambda i: sb.diffattn_decode(x.q, x.K, x.V, c["lam"], c["lam_init"], gamma=gain,
                                                       eps=c["eps"], out=out), 20)

        def two_passes(i):
            sb.xattn_decode(x.q, x.K, x.V, out=out)
            sb.xattn_decode(x.q, x.K, x.V, out=out)

        ms_2 = time_calls(two_passes, 10)
        res["diffattn_decode_B16_L34816"] = {
            "us_per_call": round(1e3 * ms_d, 1), "gbps": round(nbytes / ms_d / 1e6, 1),
            "frac_of_hbm_peak": round(nbytes / ms_d / 1e6 / HBM_PEAK_GBS, 4),
            "frac_of_stream_read": round(nbytes / ms_d / 1e6 / read_gbps, 4),
            "two_plain_passes_us": round(1e3 * ms_2, 1), "speedup_vs_two_passes": round(ms_2 / ms_d, 3)}
        del x
    if want("ragged"):
        # Ragged batch: 32 sequences, room for 34816 positions, lengths uniform in [2048, 34816].
        c = workload.XATTN_VARLEN
        x = workload.xattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["L"], seed=6, device=dev)
        lens = workload.ragged_lens(c["B"], c["L"], seed=6, min_len=c["min_len"], device=dev)
        out = torch.empty(c["B"], c["Hq"], c["D"], dtype=torch.bfloat16, device=dev)
        ms = time_calls(lambda i: sb.xattn_decode(x.q, x.K, x.V, out=out, lens=lens), 20)
        nbytes = int(lens.sum().item()) * c["Hkv"] * c["D"] * 4
        res["xattn_decode_varlen_B32_L34816_ragged"] = {
            "us_per_call": round(1e3 * ms, 1), "cached_positions": int(lens.sum().item()),
            "gbps": round(nbytes / ms / 1e6, 1), "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
            "frac_of_stream_read": round(nbytes / ms / 1e6 / read_gbps, 4)}
        # Self-decoder attention steps: the final full-attention layer appends each
        # sequence's new row to the same cache at position lens - 1 and attends over
        # lens positions; a sliding-window layer does the same on a 256-slot ring.
        kn = workload.normal((c["B"], c["Hkv"], c["D"]), seed=60, device=dev)
        vn = workload.normal((c["B"], c["Hkv"], c["D"]), seed=61, device=dev)
        pos = (lens - 1).to(torch.int32)
        ms = time_calls(lambda i: sb.selfattn_decode(x.q, kn, vn, x.K, x.V, pos, out=out), 20)
        nbytes = int(lens.sum().item()) * c["Hkv"] * c["D"] * 4 + c["B"] * c["Hkv"] * c["D"] * 4
        res["selfattn_decode_full_B32_L34816_ragged"] = {
            "us_per_call": round(1e3 * ms, 1), "gbps": round(nbytes / ms / 1e6, 1),
            "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
        del x
        torch.cuda.empty_cache()
        W = workload.SELFATTN_SWA["window"]
        r = workload.selfattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], W, seed=62, device=dev)
        call = lambda i: sb.selfattn_decode(r.q, r.k_new, r.v_new, r.K, r.V, pos, window=W, out=out)
        ms_eager = time_calls(call, 50)
        ms = time_graph(call, 20)
        nbytes = c["B"] * c["Hkv"] * W * c["D"] * 4 + c["B"] * c["Hkv"] * c["D"] * 4
        res["selfattn_decode_window256_B32"] = {
            "us_per_call": round(1e3 * ms, 2), "timing": "HIP graph replay of 20 calls",
            "us_per_call_eager": round(1e3 * ms_eager, 2), "gbps": round(nbytes / ms / 1e6, 1),
            "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
        del r
    if want("mamba_decode"):
        # SSM decode step (the Mamba layer producing M): 4 rotating weight sets
        # (4 x 118 MB, more than the 256 MB last-level cache) so that the weights
        # stream from HBM as they would layer after layer.
        c = workload.MAMBA_DECODE
        dm, di, N, R, K = c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"], c["d_conv"]
        msets = [workload.mamba_inputs(1, dm, di, N, R, K, seed=70 + k, device=dev).w for k in range(4)]
        wbytes = (2 * di * dm + (R + 2 * N) * di + di * R + dm * di) * 2 + (di * K + 3 * di + di * N) * 4
        for B in (1, 32):
            m = workload.mamba_inputs(B, dm, di, N, R, K, seed=80 + B, device=dev)
            Mo = torch.empty(B, di, dtype=torch.bfloat16, device=dev)
            yo = torch.empty(B, dm, dtype=torch.bfloat16, device=dev)
            ms = time_calls(lambda i: sb.mamba_decode_step(m.x, msets[i % 4], m.conv_state, m.ssm_state, Mo, yo), 40)
            nbytes = wbytes + B * di * (N + K - 1) * 4 * 2 + B * (2 * dm + di) * 2
            res["mamba_decode_B%d" % B] = {
                "us_per_call": round(1e3 * ms, 2), "hbm_bytes": nbytes, "gbps": round(nbytes / ms / 1e6, 1),
                "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                "frac_of_stream_read": round(nbytes / ms / 1e6 / read_gbps, 4)}
            del m
        del msets
    if want("mamba_prefill"):
        # SSM layer over the prompt: 4 x 2048 tokens at the model width.
        c = workload.MAMBA_DECODE
        dm, di, N, R, K = c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"], c["d_conv"]
        Bp, Tp = workload.ATTN_PREFILL["B"], workload.ATTN_PREFILL["T"]
        m = workload.mamba_inputs(Bp, dm, di, N, R, K, seed=95, device=dev)
        xs = workload.normal((Bp, Tp, dm), seed=96, device=dev)
        Mo = torch.empty(Bp, Tp, di, dtype=torch.bfloat16, device=dev)
        yo = torch.empty(Bp, Tp, dm, dtype=torch.bfloat16, device=dev)
        ms = time_calls(lambda i: sb.mamba_prefill(xs, m.w, m.conv_state, m.ssm_state, Mo, yo), 10, warmup=6)
        rows = Bp * Tp
        flops = 2.0 * rows * (2 * di * dm + ((R + 2 * N + 63) // 64 * 64) * di + di * R + dm * di)
        res["mamba_prefill_B%d_T%d" % (Bp, Tp)] = {
            "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
            "frac_of_bf16_peak": round(flops / ms / 1e9 / 2500.0, 4)}
        del m, xs, Mo, yo
    if want("sambay_prefill"):
        # YOCO-style prefill of the whole model: 4 x 2048 prompt tokens through the
        # 16-layer self-decoder, then the 16-layer cross-decoder on the last token;
        # the self-decoder alone timed beside it (the cross-decoder's share is the
        # difference).
        c = workload.SAMBAY_PREFILL
        yp = workload.sambay_prefill_inputs(c["B"], c["T"], c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"],
                                            c["d_conv"], c["d_ff"], c["Hq"], c["Hkv"], c["D"], c["window"], c["L"],
                                            workload.self_layer_kinds(c["n_self"]), workload.layer_kinds(c["n_cross"]),
                                            seed=97, device=dev)
        full = sb.SambayPrefill(yp.x, yp.self_layers, yp.cross_layers, yp.kcache, yp.vcache, window=c["window"])
        selfonly = sb.SambayPrefill(yp.x, yp.self_layers, [], yp.kcache, yp.vcache, window=c["window"])
        ms_full = time_calls(lambda i: full(), 5, warmup=2)
        ms_self = time_calls(lambda i: selfonly(), 5, warmup=1)
        rows = c["B"] * c["T"]
        res["sambay_prefill_B%d_T%d" % (c["B"], c["T"])] = {
            "ms": round(ms_full, 3), "prompt_tokens_per_s": round(rows / ms_full * 1e3, 1),
            "self_decoder_ms": round(ms_self, 3), "cross_decoder_last_token_ms": round(ms_full - ms_self, 3),
            "layers": "16 self (8 SSM, 7 sliding-window 256, 1 full attention) + 16 cross (8 attention, 8 GMU), "
                      "SwiGLU d_ff 8192 in every layer"}
        del yp, full, selfonly
        torch.cuda.empty_cache()
        # One sequence at growing prompt lengths: the prefill stays linear in T
        # (only windowed attention and the SSM recurrence run over the prompt).
        scaling = {}
        for T in (2048, 8192, 32768):
            ys = workload.sambay_prefill_inputs(1, T, c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"],
                                                c["d_conv"], c["d_ff"], c["Hq"], c["Hkv"], c["D"], c["window"], T,
                                                workload.self_layer_kinds(c["n_self"]),
                                                workload.layer_kinds(c["n_cross"]), seed=102, device=dev)
            run = sb.SambayPrefill(ys.x, ys.self_layers, ys.cross_layers, ys.kcache, ys.vcache, window=c["window"])
            ms_t = time_calls(lambda i: run(), 3, warmup=1)
            scaling["T%d" % T] = {"ms": round(ms_t, 3), "prompt_tokens_per_s": round(T / ms_t * 1e3, 1),
                                  "us_per_token": round(1e3 * ms_t / T, 3)}
            del ys, run
            torch.cuda.empty_cache()
        res["sambay_prefill_B1_length_scaling"] = scaling
    if want("sambay_decode"):
        # Whole-model decode step: 32 sequences, each at the last of 34,816
        # cache positions (2K prompt + 32K generated), through the 16-layer
        # self-decoder (SSM steps, sliding-window ring appends, the shared
        # cache append) and the 16-layer cross-decoder; the self-decoder alone
        # timed beside it.
        c = workload.SAMBAY_PREFILL
        B, L = 32, c["L"]
        yd = workload.sambay_prefill_inputs(B, 1, c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"],
                                            c["d_conv"], c["d_ff"], c["Hq"], c["Hkv"], c["D"], c["window"], L,
                                            workload.self_layer_kinds(c["n_self"]), workload.layer_kinds(c["n_cross"]),
                                            seed=98, device=dev, fresh=False)
        yd.kcache.copy_(workload.normal(tuple(yd.kcache.shape), seed=99, device=dev))
        yd.vcache.copy_(workload.normal(tuple(yd.vcache.shape), seed=100, device=dev))
        for ly in yd.self_layers:
            if ly["kind"] == "swa":
                ly["kring"].normal_()
                ly["vring"].normal_()
        pos = torch.full((B,), L - 1, dtype=torch.int32, device=dev)
        x0 = workload.normal((B, c["d_model"]), seed=101, device=dev)
        h = x0.clone()
        full = sb.SambayDecodeStep(h, pos, yd.self_layers, yd.cross_layers, yd.kcache, yd.vcache, window=c["window"])
        selfonly = sb.SambayDecodeStep(h, pos, yd.self_layers, [], yd.kcache, yd.vcache, window=c["window"])

        def run_full(i):
            h.copy_(x0)
            full()

        def run_self(i):
            h.copy_(x0)
            selfonly()

        ms_full = time_calls(run_full, 10)
        ms_self = time_calls(run_self, 10)
        # The same step replayed from a HIP graph (host launch cost removed).
        ms_graph = time_graph(run_full, 1, reps=10)
        res["sambay_decode_B%d_L%d" % (B, L)] = {
            "ms_per_step": round(ms_full, 4), "tokens_per_s": round(B / ms_full * 1e3, 1),
            "ms_per_step_graph_replay": round(ms_graph, 4),
            "self_decoder_ms": round(ms_self, 4), "cross_decoder_ms": round(ms_full - ms_self, 4),
            "layers": "16 self (8 SSM, 7 sliding-window 256, 1 full attention) + 16 cross (8 attention, 8 GMU), "
                      "SwiGLU d_ff 8192 in every layer"}
        del yd, full, selfonly
        torch.cuda.empty_cache()
    if want("attn_prefill"):
        # Prefill attention over the prompt: 4 x 2048 tokens, window 256 (the
        # self-decoder's sliding-window layers), and plain causal at 1 x 2048.
        c = workload.ATTN_PREFILL
        for B, W in ((c["B"], c["window"]), (1, 0)):
            x = workload.prefill_inputs(B, c["T"], c["Hq"], c["Hkv"], c["D"], seed=90 + W, device=dev)
            o = torch.empty_like(x.q)
            ms = time_calls(lambda i: sb.attn_prefill(x.q, x.k, x.v, window=W, out=o), 20)
            T, D = c["T"], c["D"]
            keys = sum(min(i + 1, W) if W else i + 1 for i in range(T))        # visible (query, key) pairs per head
            flops = 4.0 * D * keys * c["Hq"] * B
            nbytes = B * T * (2 * c["Hq"] + 2 * c["Hkv"]) * D * 2
            res["attn_prefill_B%d_T%d_window%d" % (B, T, W)] = {
                "us_per_call": round(1e3 * ms, 2), "tflops": round(flops / ms / 1e9, 1),
                "frac_of_bf16_peak": round(flops / ms / 1e9 / 2500.0, 4), "gbps": round(nbytes / ms / 1e6, 1),
                "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
            del x, o
    if want("crossdecoder_ex"):
        # Complete cross-decoder layer step (pre-RMSNorm mixer + pre-RMSNorm SwiGLU MLP, d_ff 8192) on that ragged batch.
        c = workload.CROSSDECODER_EX
        x = workload.crossdecoder_ex_inputs(c["B"], c["d_model"], c["d_inner"], c["d_ff"], c["Hq"], c["Hkv"], c["D"],
                                            c["L"], c["n_layers"], seed=7, device=dev, lens="ragged",
                                            min_len=c["min_len"])
        h_in = x.h.clone()
        step = sb.CrossDecoderStepEx(x.h, x.M, x.K, x.V, x.layers, lens=x.lens)

        def run(i):
            x.h.copy_(h_in)
            step()

        ms = time_calls(run, 10)
        n_x = c["n_layers"] // 2
        dm, di, dff = c["d_model"], c["d_inner"], c["d_ff"]
        kv = int(x.lens.sum().item()) * c["Hkv"] * c["D"] * 4
        nbytes = (n_x * kv + n_x * 2 * dm * dm * 2 + (c["n_layers"] - n_x) * 2 * dm * di * 2
                  + c["n_layers"] * (3 * dm * dff + 2 * dm) * 2)
        res["crossdecoder_ex_B32_ragged_dff8192"] = {
            "ms_per_step": round(ms, 4), "tokens_per_s": round(c["B"] / (ms / 1e3), 1), "hbm_bytes_per_step": nbytes,
            "gbps": round(nbytes / ms / 1e6, 1), "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
        del step, x
        torch.cuda.empty_cache()
    return res


def configs_block(sb, workload, dev, oracle_ok: bool) -> dict:
    """The five workloads of this path, compact: the tiny fp32 GMU against the
    oracle (correctness only), GMU prefill (TFLOP/s and fraction of the bf16
    MFMA peak), GMU decode per batch size (8 rotating weight sets, so every
    call reads its weights from HBM; us per call and fraction of 8 TB/s),
    and the cross-attention decode alone (us and fraction of 8 TB/s).  The
    16-layer step is the headline value itself."""
    import torch

    out = {}
    if oracle_ok:
        import numpy as np

        import oracle

        t = workload.tiny_gmu(seed=0)
        Y = sb.gmu_forward(t.M.to(dev), t.X.to(dev), t.W1.to(dev), t.W2.to(dev))
        torch.cuda.synchronize()
        ref = oracle.gmu(t.M, t.X, t.W1, t.W2)
        err = float(np.max(np.abs(Y.double().cpu().numpy() - ref)) / np.max(np.abs(ref)))
        out["tiny_gmu_fp32_T64_64x128"] = {"rel_err_vs_oracle": err, "tolerance": 1e-5, "pass": err <= 1e-5}
    c = workload.GMU_PREFILL
    rows = c["batch"] * c["seq"]
    g = workload.gmu_inputs(rows, c["d_model"], c["d_inner"], seed=1, device=dev)
    Y = torch.empty(rows, c["d_model"], dtype=torch.bfloat16, device=dev)
    ms = time_calls(lambda i: sb.gmu_forward(g.M, g.X, g.W1, g.W2, out=Y), 20, warmup=20)
    tf = 4.0 * rows * c["d_model"] * c["d_inner"] / ms / 1e9
    out["gmu_prefill_B4_T2048_2560x5120"] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                              "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    del g, Y
    c = workload.GMU_DECODE
    sets = [workload.gmu_inputs(1, c["d_model"], c["d_inner"], seed=2, device=dev, weight_set=k) for k in range(8)]
    for B in c["batches"]:
        gi = workload.gmu_inputs(B, c["d_model"], c["d_inner"], seed=3 + B, device=dev)
        Y = torch.empty(B, c["d_model"], dtype=torch.bfloat16, device=dev)
        ms = time_calls(lambda i: sb.gmu_forward(gi.M, gi.X, sets[i % 8].W1, sets[i % 8].W2, out=Y), 64)
        nbytes = 2 * c["d_model"] * c["d_inner"] * 2 + B * (2 * c["d_model"] + c["d_inner"]) * 2
        out["gmu_decode_B%d_3072x6144" % B] = {"us": round(1e3 * ms, 2), "gbps": round(nbytes / ms / 1e6, 1),
                                               "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
        del gi, Y
    del sets
    torch.cuda.empty_cache()
    c = workload.XATTN_DECODE
    x = workload.xattn_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["L"], seed=4, device=dev)
    o = torch.empty(c["B"], c["Hq"], c["D"], dtype=torch.bfloat16, device=dev)
    ms = time_calls(lambda i: sb.xattn_decode(x.q, x.K, x.V, out=o), 20)
    nbytes = c["B"] * c["Hkv"] * c["L"] * c["D"] * 4 + 2 * c["B"] * c["Hq"] * c["D"] * 2
    out["xattn_decode_B16_L34816_24q8kv"] = {"us": round(1e3 * ms, 1), "gbps": round(nbytes / ms / 1e6, 1),
                                             "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del x, o
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the compact per-workload block")
    ap.add_argument("--cpu-seqs", type=int, default=32, help="sequences in the oracle CPU sample")
    ap.add_argument("--all", action="store_true",
                    help="also time the other workloads (GMU prefill, GMU decode per batch, attention alone)")
    ap.add_argument("--only", default="", metavar="GROUPS",
                    help="with --all: only these comma-separated workload groups (%s)" % ", ".join(WORKLOAD_GROUPS))
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="only run a plain device copy of MB megabytes 5 times (reference for HBM counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (asked for %d GPUs, world size %d)."
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_decoding_amd as sb
    import workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 4 * n, "launches": 5}), flush=True)
        return
    c = dict(workload.CROSSDECODER)
    log("bench: generating inputs (B=%d, L=%d, %d layers)" % (c["B"], c["L"], c["n_layers"]))
    x = workload.crossdecoder_inputs(c["B"], c["d_model"], c["d_inner"], c["Hq"], c["Hkv"], c["D"], c["L"],
                                     c["n_layers"], seed=0, device=dev)
    h_in = x.h.clone()
    step = sb.CrossDecoderStep(x.h, x.M, x.K, x.V, x.layers)
    nbytes = step_bytes(c)

    def run_step():
        x.h.copy_(h_in)
        step()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    log("bench: warmup done, timing %d steps" % args.steps)

    # The timed steps: no per-kernel instrumentation.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        run_step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))

    def pct(q):
        return per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    ms_step = max(ms_step, 1e3 * wall / args.steps)
    tokens_per_s = c["B"] / (ms_step / 1e3)

    # The same number of steps again with the split kernel's launches bracketed
    # by HIP events that the library records on the launch's own stream: its
    # mean launch duration, for the roofline entry.
    sb.timing_enable(sb.SB_TIME_XATTN_SPLIT)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        run_step()
    e1.record()
    torch.cuda.synchronize()
    sb.timing_enable(0)
    ms_step_instr = e0.elapsed_time(e1) / args.steps
    n_split, ms_split = sb.timing_collect(sb.SB_TIME_XATTN_SPLIT)
    split_ms = ms_split / max(n_split, 1)
    achieved = nbytes["kv_per_layer"] / (split_ms / 1e3) / 1e9
    log("bench: %.3f ms/step, %.0f tokens/s; split kernel %.1f us/launch over %d launches" %
        (ms_step, tokens_per_s, 1e3 * split_ms, n_split))

    # The step replayed from a HIP graph (the input refresh and every launch of
    # the step captured once): what the host's launch cost is worth.
    h_eager = None
    graph = None
    try:
        run_step()
        torch.cuda.synchronize()
        h_eager = x.h.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            run_step()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                run_step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(x.h, h_eager))
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_g = e0.elapsed_time(e1) / args.steps
        graph = {"ms_per_step": round(ms_g, 4), "tokens_per_s": round(c["B"] / (ms_g / 1e3), 1),
                 "eager_over_graph": round(ms_step / ms_g, 4), "bitwise_equal_to_eager": same}
        del g
        log("bench: graph replay %.3f ms/step (eager %.3f)" % (ms_g, ms_step))
    except Exception as exc:  # a failed capture is reported, not fatal
        graph = {"error": str(exc)[:200]}

    # Per-kernel breakdown on a few extra steps (not part of the timed value).
    kinds = {"xattn_split": sb.SB_TIME_XATTN_SPLIT, "xattn_merge": sb.SB_TIME_XATTN_MERGE,
             "skinny_products": sb.SB_TIME_SKINNY}
    sb.timing_enable(sum(kinds.values()))
    nb = 3
    for _ in range(nb):
        run_step()
    torch.cuda.synchronize()
    sb.timing_enable(0)
    kern = {}
    for name, bit in kinds.items():
        n, ms = sb.timing_collect(bit)
        kern[name] = {"launches_per_step": n // nb, "ms_per_step": round(ms / nb, 4)}
    w_bytes = nbytes["xattn_weights"] + nbytes["gmu_weights"] + nbytes["state"]
    sk = kern["skinny_products"]["ms_per_step"]
    kern["skinny_products"]["gbps"] = round(w_bytes / (sk / 1e3) / 1e9, 1) if sk > 0 else None
    kern["skinny_products"]["frac_of_peak"] = round(w_bytes / (sk / 1e3) / 1e9 / HBM_PEAK_GBS, 4) if sk > 0 else None
    kern["xattn_split"]["gbps"] = round(nbytes["kv"] / (kern["xattn_split"]["ms_per_step"] / 1e3) / 1e9, 1)
    kern["xattn_split"]["frac_of_peak"] = round(kern["xattn_split"]["gbps"] / HBM_PEAK_GBS, 4)

    # Practical ceilings of this machine, by the library's probe kernels: a plain
    # streaming read of the K cache and a register-only bf16 MFMA loop.
    read_gbps = sb.probe_stream_read_gbps(x.K)
    mfma_tf = sb.probe_mfma_tflops(dev, iters=10000)
    log("bench: probes: streaming read %.0f GB/s, bf16 MFMA loop %.0f TFLOP/s" % (read_gbps, mfma_tf))

    configs = None
    if not args.no_configs:
        log("bench: timing the per-workload block")
        configs = configs_block(sb, workload, dev, oracle_ok=not args.no_cpu_baseline)
        configs["crossdecoder_step_B32_L34816_16_layers"] = {"ms": round(ms_step, 4),
                                                             "tokens_per_s": round(tokens_per_s, 1),
                                                             "frac_of_hbm_peak": round(nbytes["total"] / (ms_step / 1e3)
                                                                                       / 1e9 / HBM_PEAK_GBS, 4)}

    cpu = parity = None
    if not args.no_cpu_baseline:
        import numpy as np

        log("bench: timing the fp64 oracle on %d sequences" % args.cpu_seqs)
        cpu, ref = cpu_baseline(h_in, x, c, args.cpu_seqs)
        log("bench: oracle %.3f tokens/s on %d threads, %.3f on one" %
            (cpu["value"], cpu["cores"], cpu["single_core_value"]))
        # The step's own output on the timed inputs against the oracle's.
        run_step()
        torch.cuda.synchronize()
        got = x.h[:args.cpu_seqs].double().cpu().numpy()
        err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        big = np.abs(ref) > 1e-3 * np.max(np.abs(ref))
        rel = np.abs(got - ref)[big] / np.abs(ref)[big]
        parity = {"sequences": args.cpu_seqs, "max_abs_err_over_max_abs_ref": err, "tolerance": 2e-2,
                  "pass": err <= 2e-2,
                  "elementwise_rel_err_where_ref_above_1e-3_max": {"median": float(np.median(rel)),
                                                                   "p99": float(np.quantile(rel, 0.99)),
                                                                   "max": float(np.max(rel))}}
        log("bench: parity of the timed step against the oracle: %.3e (tolerance 2e-2)" % err)

    workloads = None
    if args.all:
        log("bench: timing the other workloads")
        del step
        only = [g for g in args.only.split(",") if g] or None
        if only and any(g not in WORKLOAD_GROUPS for g in only):
            raise SystemExit("--only: unknown group in %r (known: %s)" % (args.only, ", ".join(WORKLOAD_GROUPS)))
        workloads = other_workloads(sb, workload, dev, read_gbps, mfma_tf, only=only)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_median_p90": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and KV cache, N(0,0.02^2) weights)",
        "config": {"workload": "cross-decoder decode step: 16 layers alternating cross-attention over one shared "
                               "KV cache and GMU, one new token per sequence",
                   "batch": c["B"], "layers": c["n_layers"], "layer_order": "xattn,gmu,...", "d_model": c["d_model"],
                   "d_inner": c["d_inner"], "q_heads": c["Hq"], "kv_heads": c["Hkv"], "head_dim": c["D"],
                   "kv_len": c["L"]},
        "hbm_bytes_per_step": nbytes["total"],
        "step_gbps": round(nbytes["total"] / (ms_step / 1e3) / 1e9, 1),
        "step_frac_of_hbm_peak": round(nbytes["total"] / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "xattn_split_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": nbytes["kv_per_layer"], "us_per_launch": round(1e3 * split_ms, 2),
                     "traffic": traffic_for_current_kernel()},
        "measured_ceilings": {"stream_read_gbps": round(read_gbps, 1), "bf16_mfma_tflops": round(mfma_tf, 1),
                              "split_frac_of_stream_read": round(achieved / read_gbps, 4)},
        "ms_per_step_with_split_events": round(ms_step_instr, 4),
        "graph_replay": graph,
        "kernels": kern,
        "configs": configs,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "library": {"version": sb.version(), "built_from_sources": sb.built_source_hash(),
                    "sources_now": sb.current_source_hash(),
                    "matches": sb.built_source_hash() == sb.current_source_hash()},
    }
    if workloads is not None:
        out["workloads"] = workloads
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
