#!/usr/bin/env python3
"""Benchmark of the layout-aware GEMM hot path on one MI355X.

One step = one tgemm_run call of the NT down-projection GEMM
Y[768,5120] = X[768,13824] . W[5120,13824]^T (X viewed from [384,2,13824], W
read in its stored [N,K] layout, no transposed copy), inputs resident in HBM.
Three copies of (X, W) are rotated so the 256 MB last-level cache cannot
hold the operands between steps.  The same run also times the fused
cross-entropy GEMM (4096 x 32000 x 4096, loss only and loss + gradient), the
4096^3 layout sweep and the K=1 RoPE table, reported as secondary figures.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU (published 2.5 PF)
PEAK_HBM_GBS = 8000.0       # HBM3E, 8 TB/s
PEAK_FP8_TFLOPS = 5033.2    # dense fp8: twice the bf16 rate per clock (published 5.0 PF)
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "nt_gemm_768x5120x13824_hbm_traffic.md")
KERNEL_SOURCES = ["gemm_kernel.h", "gemm_nt.hip", "tgemm_internal.h", "dispatch.hip", "ce_grad.h",
                  "splitk.hip", "bf16_cvt.h"]
COPY_CAL_BYTES = 2 ** 30  # plain device copy used to calibrate the HBM byte counters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "layout_aware_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when the NT kernel's sources changed since it was taken."""
    try:
        text = open(PROFILE_COUNTERS).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def time_stream(fn, steps, warmup, rotate, probe=None):
    """Average ms per call, HIP events on the current stream (the one tgemm
    launches on), bracketed by synchronisation.  With ``probe`` (an int64[3]
    device tensor) the shader-clock probe is enqueued right after the end
    event, outside the timed region, and reads the clock the region ended at."""
    import torch

    from layout_aware_gemm_amd import tgemm

    for i in range(warmup):
        fn(i % rotate)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i % rotate)
    end.record()
    if probe is not None:
        tgemm.clock_probe(out=probe)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def step_times(fn, steps, rotate):
    """Per-call ms for ``steps`` calls, one HIP event between consecutive
    calls on the current stream (a separate pass, after the timed region)."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn(i % rotate)
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def cpu_baseline(budget_s=12.0):
    """The oracle as it stands, on the host, on a bounded sample of the NT
    workload: whole output rows of op(A).op(B) for the first rows of X."""
    import numpy as np

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    w = workloads.nt_mlp()
    M, N, K = 768, 5120, 13824
    Xb = workloads.bf16_bits(w["X"]).reshape(-1)
    Wb = workloads.bf16_bits(w["W"]).reshape(-1)
    rows_done, t_total, n = 0, 0.0, 0
    rows = np.arange(0, 96)
    while t_total < budget_s and n < 20:
        t0 = time.perf_counter()
        oracle.gemm("N", "T", M, N, K, Xb, K, Wb, K, rows=rows)
        t_total += time.perf_counter() - t0
        rows_done += len(rows)
        n += 1
    flops = 2.0 * rows_done * N * K
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n} x fp64 oracle GEMM of 96 of 768 rows (768x5120x13824 NT, decode + "
                      f"explicit transpose + BLAS matmul), {t_total:.1f} s"}


def cpu_oracle_secondary(budget_s=6.0):
    """The oracle on bounded samples of the other workloads, for the
    secondary figures: fused CE (whole rows of the 4096x32000x4096 logits,
    then the per-row loss) and the K=1 RoPE table (4096 positions)."""
    import numpy as np

    import oracle
    import workloads

    out = {}
    cv = workloads.ce_vocab()
    Hb = workloads.bf16_bits(cv["H"]).reshape(-1)
    Wb = workloads.bf16_bits(cv["W"]).reshape(-1)
    lab = cv["labels"].numpy()
    rows, t, n = np.arange(0, 8), 0.0, 0
    while t < budget_s and n < 8:
        r = rows + 8 * n
        t0 = time.perf_counter()
        logits = oracle.gemm("N", "T", 4096, 32000, 4096, Hb, 4096, Wb, 4096, rows=r)
        oracle.cross_entropy(logits, lab[r])
        t += time.perf_counter() - t0
        n += 1
    out["cpu_oracle_ce_rows_per_s"] = round(8 * n / t, 2)
    out["cpu_oracle_ce_sample"] = f"{8 * n} rows of 4096x32000x4096 (fp64 logits + loss), {t:.1f} s"
    r = workloads.rope()
    pos, inv = r["pos"].numpy(), r["inv_freq"].numpy()
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 1.0:
        oracle.rope_tables(pos, inv)
        reps += 1
    tr = time.perf_counter() - t0
    out["cpu_oracle_rope_GBps"] = round(reps * (2 * 4096 * 128 * 2 + 4096 * 8) / tr / 1e9, 4)
    out["cpu_oracle_rope_sample"] = f"{reps} x 4096-position table, {tr:.1f} s"
    return out


def layout_sweep(steps, warmup):
    """The 4096^3 GEMM in the four layouts (same logical operands, each
    stored in its layout's order): TFLOP/s per layout."""
    import torch

    import workloads
    from layout_aware_gemm_amd import tgemm

    dev = torch.device("cuda:0")
    out = {}
    ls = workloads.layout_sweep()
    for ta, tb in [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]:
        sa, lda = workloads.store_operand(ls["opA"], ta)
        sb, ldb = workloads.store_operand(ls["opB"], tb)
        A, B = sa.to(dev), sb.to(dev)
        C = torch.empty(4096, 4096, dtype=torch.bfloat16, device=dev)
        msl = time_stream(lambda i: tgemm.run(ta, tb, 4096, 4096, 4096, A, lda, B, ldb, C,
                                              4096, tgemm.EPI_STORE_BF16), steps, warmup, 1)
        out[f"sweep_{ta}{tb}_tflops"] = round(2.0 * 4096 ** 3 / (msl * 1e-3) / 1e12, 2)
        out[f"sweep_{ta}{tb}_us"] = round(msl * 1e3, 2)
        del A, B, C
    return out


def fused_ce(steps, warmup):
    """The fused CE GEMM 4096x32000x4096 (inputs rotated between two
    copies), loss only and loss + gradient.  Returns its figures and the
    device tensors (H copies, W copies, gradient) for the backward GEMMs."""
    import torch

    import workloads
    from layout_aware_gemm_amd import tgemm

    dev = torch.device("cuda:0")
    Mc, Nc, Kc = 4096, 32000, 4096
    cv = workloads.ce_vocab()
    Hs = [cv["H"].to(dev) for _ in range(2)]
    Wv = [cv["W"].to(dev) for _ in range(2)]
    lab = cv["labels"].to(dev)
    del cv
    loss = torch.empty(Mc, dtype=torch.float32, device=dev)

    def ce_step(i, g=None):
        tgemm.run("N", "T", Mc, Nc, Kc, Hs[i], Kc, Wv[i], Kc, None, Nc, tgemm.EPI_CE,
                  labels=lab, out_loss=loss, out_grad=g)

    log("timing fused CE 4096x32000x4096 ...")
    probe = torch.zeros(3, dtype=torch.int64, device=dev)
    ms_ce = time_stream(ce_step, steps, warmup, 2, probe=probe)
    sclk_ce = tgemm.clock_ghz(probe)
    g = torch.empty(Mc, Nc, dtype=torch.bfloat16, device=dev)
    ms_ceg = time_stream(lambda i: ce_step(i, g), steps, warmup, 2)
    ce_fl = 2.0 * Mc * Nc * Kc
    out = {
        "ce_loss_rows_per_s": round(Mc / (ms_ce * 1e-3), 1),
        "ce_loss_tflops": round(ce_fl / (ms_ce * 1e-3) / 1e12, 2),
        "ce_loss_frac_of_peak": round(ce_fl / (ms_ce * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ce_loss_ms": round(ms_ce, 4),
        "ce_loss_sclk_ghz_end_of_timed": round(sclk_ce, 3),
        "ce_grad_rows_per_s": round(Mc / (ms_ceg * 1e-3), 1),
        "ce_grad_ms": round(ms_ceg, 4),
    }
    return out, Hs, Wv, g, lab


def rope_tables(steps, warmup):
    """The K=1 RoPE table (cos and sin, bf16 [P, 128]) for 4096 positions
    and for 256 x 4096 positions, and the whole RoPE region (tables plus the
    query's widened head-major copy) at 4096 positions x 32 heads x 128:
    time, GB/s, fraction of HBM peak."""
    import torch

    import workloads
    from layout_aware_gemm_amd import tgemm

    dev = torch.device("cuda:0")
    out = {}
    for name, r in (("rope_4096", workloads.rope()), ("rope_256x4096", workloads.rope_batched(256))):
        pos, inv = r["pos"].to(dev), r["inv_freq"].to(dev)
        P = pos.numel()
        cos = torch.empty(P, 128, dtype=torch.bfloat16, device=dev)
        sin = torch.empty_like(cos)
        msr = time_stream(lambda i: tgemm.run("N", "N", P, 64, 1, pos, 1, inv, 64, cos, 128,
                                              tgemm.EPI_ROPE_COSSIN, out_grad=sin), steps, warmup, 1)
        byts = 2 * P * 128 * 2 + P * 8 + 64 * 4
        out[f"{name}_us"] = round(msr * 1e3, 2)
        out[f"{name}_GBps"] = round(byts / (msr * 1e-3) / 1e9, 1)
        out[f"{name}_frac_of_hbm"] = round(byts / (msr * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        if name == "rope_4096":
            # the 2 MB table is launch-bound: the same call replayed from a
            # captured HIP graph of 20 calls (one launch per replay) shows
            # the rate without the host's per-call cost; the replays must
            # leave the eager call's bits
            ref_c, ref_s = cos.clone(), sin.clone()
            cos.zero_()
            sin.zero_()
            reps = 20
            call = lambda: tgemm.run("N", "N", P, 64, 1, pos, 1, inv, 64, cos, 128,
                                     tgemm.EPI_ROPE_COSSIN, out_grad=sin)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    call()
            msg = time_stream(lambda i: g.replay(), steps, warmup, 1) / reps
            out["rope_4096_graph_us"] = round(msg * 1e3, 2)
            out["rope_4096_graph_GBps"] = round(byts / (msg * 1e-3) / 1e9, 1)
            out["rope_4096_graph_same_bits"] = bool(torch.equal(cos, ref_c) and
                                                    torch.equal(sin, ref_s))
            del g
        del pos, inv, cos, sin
    # the whole region of the listing in one launch: the tables plus the
    # query [4096, 32*128] widened and permuted to fp32 [32, 4096, 128]
    rr = workloads.rope_region()
    q, pos, inv = rr["q"].to(dev), rr["pos"].to(dev), rr["inv_freq"].to(dev)
    P, HD = rr["q"].shape
    H = rr["heads"]
    D = HD // H
    q_out = torch.empty(H, P, D, dtype=torch.float32, device=dev)
    cos = torch.empty(P, D, dtype=torch.bfloat16, device=dev)
    sin = torch.empty_like(cos)
    msq = time_stream(lambda i: tgemm.run_rope_region(q, HD, P, H, D, pos, 1, inv, cos, sin, D,
                                                      q_out), steps, warmup, 1)
    byts = P * HD * 2 + P * HD * 4 + 2 * P * D * 2 + P * 8 + (D // 2) * 4
    out["rope_region_4096x32x128_us"] = round(msq * 1e3, 2)
    out["rope_region_4096x32x128_GBps"] = round(byts / (msq * 1e-3) / 1e9, 1)
    out["rope_region_4096x32x128_frac_of_hbm"] = round(byts / (msq * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    del q, pos, inv, q_out, cos, sin
    return out


def ce_forward_backward(K_, W_):
    """The fused CE GEMM (``fused_ce``), then the GEMMs that consume its
    gradient, operands read as stored: dH = G . W (NN, K = 32000) and
    dW = G^T . H (TN, K = 4096), on the finished gradient and with the
    gradient finished on load (the fused CE without its rescale pass, the
    scale table instead, then dH and dW reading the unscaled gradient)."""
    import torch

    from layout_aware_gemm_amd import tgemm

    dev = torch.device("cuda:0")
    Mc, Nc, Kc = 4096, 32000, 4096
    out, Hs, Wv, g, lab_ce = fused_ce(max(5, K_ // 5), max(2, W_ // 5))
    ce_fl = 2.0 * Mc * Nc * Kc
    nst = max(5, K_ // 5)
    dH = torch.empty(Mc, Kc, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(Nc, Kc, dtype=torch.bfloat16, device=dev)
    ms_dh = time_stream(lambda i: tgemm.run("N", "N", Mc, Kc, Nc, g, Nc, Wv[0], Kc, dH, Kc,
                                            tgemm.EPI_STORE_BF16), nst, 2, 1)
    ms_dw = time_stream(lambda i: tgemm.run("T", "N", Nc, Kc, Mc, g, Nc, Hs[0], Kc, dW, Kc,
                                            tgemm.EPI_STORE_BF16), nst, 2, 1)
    out["ce_bwd_dH_NN_tflops"] = round(ce_fl / (ms_dh * 1e-3) / 1e12, 2)
    out["ce_bwd_dW_TN_tflops"] = round(ce_fl / (ms_dw * 1e-3) / 1e12, 2)
    lossd = torch.empty(Mc, dtype=torch.float32, device=dev)
    sc = torch.empty((Nc + 63) // 64, Mc, dtype=torch.float32, device=dev)
    ms_ced = time_stream(lambda i: tgemm.run_ce_deferred("N", "T", Mc, Nc, Kc, Hs[0], Kc, Wv[0],
                                                         Kc, lab_ce, lossd, g, Nc, sc), nst, 2, 1)
    ms_dh2 = time_stream(lambda i: tgemm.run_ce_grad("N", "N", Mc, Kc, Nc, g, Nc, sc, lab_ce,
                                                     Wv[0], Kc, dH, Kc, tgemm.EPI_STORE_BF16),
                         nst, 2, 1)
    ms_dw2 = time_stream(lambda i: tgemm.run_ce_grad("T", "N", Nc, Kc, Mc, g, Nc, sc, lab_ce,
                                                     Hs[0], Kc, dW, Kc, tgemm.EPI_STORE_BF16),
                         nst, 2, 1)
    out["ce_bwd_onload_dH_NN_tflops"] = round(ce_fl / (ms_dh2 * 1e-3) / 1e12, 2)
    out["ce_bwd_onload_dW_TN_tflops"] = round(ce_fl / (ms_dw2 * 1e-3) / 1e12, 2)
    out["ce_fwd_bwd_rescale_pass_route_us"] = round((out["ce_grad_ms"] + ms_dh + ms_dw) * 1e3, 1)
    out["ce_fwd_bwd_on_load_route_us"] = round((ms_ced + ms_dh2 + ms_dw2) * 1e3, 1)
    del Hs, Wv, g, dH, dW, sc, lossd
    return out


def torch_context(steps, warmup):
    """Context only, not this library: the same products through torch (its
    GEMM library) on the same inputs, and a plain fill of the RoPE table's
    bytes.  NT 768x5120x13824 and 4096^3 NT as ``linear`` (X . W^T), the
    gemv 1x5120x13824, the dot product of 10^8, a 537 MB fill."""
    import torch
    import torch.nn.functional as F

    import workloads

    dev = torch.device("cuda:0")
    out = {}
    w = workloads.nt_mlp()
    X, W = w["X"].reshape(-1, 13824).to(dev), w["W"].to(dev)
    ms = time_stream(lambda i: F.linear(X, W), steps, warmup, 1)
    out["torch_nt_768x5120x13824_us"] = round(ms * 1e3, 2)
    out["torch_nt_768x5120x13824_tflops"] = round(2.0 * 768 * 5120 * 13824 / (ms * 1e-3) / 1e12, 1)
    x1 = X[:1].contiguous()
    msg = time_stream(lambda i: F.linear(x1, W), steps, warmup, 1)
    out["torch_gemv_1x5120x13824_us"] = round(msg * 1e3, 2)
    del X, W, x1, w
    ls = workloads.layout_sweep()
    A, Bt = ls["opA"].to(dev), ls["opB"].t().contiguous().to(dev)
    ms4 = time_stream(lambda i: F.linear(A, Bt), steps, warmup, 1)
    out["torch_nt_4096_us"] = round(ms4 * 1e3, 2)
    out["torch_nt_4096_tflops"] = round(2.0 * 4096 ** 3 / (ms4 * 1e-3) / 1e12, 1)
    del A, Bt, ls
    Kd = 10 ** 8
    gdot = torch.Generator(device="cpu").manual_seed(5)
    av = torch.randn(Kd, generator=gdot).to(torch.bfloat16).to(dev)
    bv = torch.randn(Kd, generator=gdot).to(torch.bfloat16).to(dev)
    msd = time_stream(lambda i: torch.dot(av, bv), steps, warmup, 1)
    out["torch_dot_1e8_us"] = round(msd * 1e3, 2)
    del av, bv
    nbytes = 2 * 256 * 4096 * 128 * 2
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    msf = time_stream(lambda i: buf.fill_(1.0), steps, warmup, 1)
    out["fill_537MB_us"] = round(msf * 1e3, 2)
    out["fill_537MB_frac_of_hbm"] = round(nbytes / (msf * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    del buf
    return out


def mfma_ceiling(steps=20, warmup=40):
    """The matrix-core ceiling (tgemm_mfma_ceiling): one workgroup per compute
    unit, one wave per SIMD, MFMAs on register operands only -- the GEMM
    loops' matrix-core work without loads, LDS or barriers -- for bf16
    (32x32x16) and fp8 (32x32x64).  ``warmup`` launches first, then ``steps``
    timed ones; the clock probe reads the clock at the end."""
    import torch

    from layout_aware_gemm_amd import tgemm

    buf = torch.zeros(256 * 4, dtype=torch.float32, device="cuda")
    probe = torch.zeros(3, dtype=torch.int64, device="cuda")
    out = {}
    for kind, name, per, peak, iters in ((0, "32x32x16", 524288.0, PEAK_BF16_TFLOPS, 8192),
                                         (1, "fp8_32x32x64", 2097152.0, PEAK_FP8_TFLOPS, 4096)):
        flop = 256 * 4 * iters * per
        ms = time_stream(lambda i: tgemm.mfma_ceiling(iters, buf, kind=kind), steps, warmup, 1,
                         probe=probe)
        tf = flop / (ms * 1e-3) / 1e12
        out[f"mfma_ceiling_{name}_tflops"] = round(tf, 1)
        out[f"mfma_ceiling_{name}_frac_of_peak"] = round(tf / peak, 4)
        out[f"mfma_ceiling_{name}_sclk_ghz_end"] = round(tgemm.clock_ghz(probe), 3)
    return out


def fp8_linear(K_, W_):
    """The float8 linear 4096x3072x4096 through tgemm_run_fp8 (cast passes
    plus the fp8 matrix-core GEMM), the weight read in place (NT) and from
    its transposed storage (NN); the bf16 product of the same shape; and
    torch's unfused cast and transposed copy of the input, for context."""
    import torch

    import workloads
    from layout_aware_gemm_amd import tgemm

    dev = torch.device("cuda:0")
    secondary = {}
    wf = workloads.fp8_linear()
    Xf, Wf = wf["X"].to(dev), wf["W"].to(dev)              # [4096, 4096], [3072, 4096]
    Wft = wf["W"].t().contiguous().to(dev)                 # [4096, 3072]
    sx, sw = wf["scale_x"], wf["scale_w"]
    sc = torch.tensor([sx, sw, 1.0 / (sx * sw)], dtype=torch.float32, device=dev)
    del wf
    Yf = torch.empty(4096, 3072, dtype=torch.bfloat16, device=dev)
    f8fl = 2.0 * 4096 * 3072 * 4096
    for name, tb_, Bm, ldb_ in (("fp8_linear_4096x3072x4096_NT", "T", Wf, 4096),
                                ("fp8_linear_4096x3072x4096_NN", "N", Wft, 3072)):
        msf = time_stream(lambda i: tgemm.run_fp8("N", tb_, 4096, 3072, 4096, Xf, 4096, Bm,
                                                  ldb_, Yf, 3072, tgemm.EPI_STORE_BF16, sc),
                          K_, W_, 1)
        secondary[f"{name}_us"] = round(msf * 1e3, 2)
        secondary[f"{name}_tflops"] = round(f8fl / (msf * 1e-3) / 1e12, 2)
        # the packed route: cast passes plus the GEMM on the fp8 matrix cores
        secondary[f"{name}_frac_of_fp8_peak"] = round(
            f8fl / (msf * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)
    # the same product in bf16 (the unquantized operands), for comparison
    msb = time_stream(lambda i: tgemm.run("N", "T", 4096, 3072, 4096, Xf, 4096, Wf, 4096, Yf,
                                          3072, tgemm.EPI_STORE_BF16), K_, W_, 1)
    secondary["bf16_linear_4096x3072x4096_NT_us"] = round(msb * 1e3, 2)
    # context: the page's unfused pattern (scale, clamp and cast, then the
    # transposed fp8 copy) for the input alone, in torch, before any GEMM
    sxt = sc[0:1]

    def unfused_cast(i):
        t = (Xf * sxt).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        return t.t().contiguous().t()

    msu = time_stream(unfused_cast, K_, W_, 1)
    secondary["fp8_cast_and_transposed_copy_torch_us"] = round(msu * 1e3, 2)
    del Xf, Wf, Wft, Yf, sc

    return secondary


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-nt", action="store_true",
                    help="time only the NT GEMM with rotated inputs (the profiled command)")
    ap.add_argument("--only-sweep", action="store_true",
                    help="time only the 4096^3 layout sweep (NN, NT, TN, TT) and print its "
                         "figures (a profiling command; no headline line)")
    ap.add_argument("--only-ce", action="store_true",
                    help="time only the fused CE GEMM 4096x32000x4096, loss only then loss + "
                         "gradient, and print its figures (a profiling command; no headline line)")
    ap.add_argument("--only-rope", action="store_true",
                    help="time only the K=1 RoPE table (4096 and 256 x 4096 positions) and print "
                         "its figures (a profiling command; no headline line)")
    ap.add_argument("--only-fp8", action="store_true",
                    help="time only the fp8 linear 4096x3072x4096 (NT, NN) and the bf16 product "
                         "of its shape, and print the figures (a profiling command)")
    ap.add_argument("--only-ce-backward", action="store_true",
                    help="time only the fused CE and the backward GEMMs on both gradient routes, "
                         "and print the figures (a profiling command)")
    ap.add_argument("--only-torch-context", action="store_true",
                    help="time only torch's own kernels on the same products (context figures, "
                         "not this library) and a plain fill, and print the figures")
    ap.add_argument("--only-mfma-ceiling", action="store_true",
                    help="time only the matrix-core ceiling kernel (bf16 and fp8 MFMAs on "
                         "register operands) and print the figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, 5 times (the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE; "
                         "4x the last-level cache, so it streams from HBM)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding is described, not built); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import workloads
    from layout_aware_gemm_amd import tgemm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    tgemm.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        x = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        log(f"copied {COPY_CAL_BYTES} bytes 5 times")
        return 0
    K_, W_ = args.steps, args.warmup
    if args.only_rope:
        print(json.dumps(rope_tables(K_, W_)), flush=True)
        return 0
    if args.only_ce:
        out, *_ = fused_ce(K_, W_)
        print(json.dumps(out), flush=True)
        return 0
    if args.only_fp8:
        print(json.dumps(fp8_linear(K_, W_)), flush=True)
        return 0
    if args.only_mfma_ceiling:
        print(json.dumps(mfma_ceiling()), flush=True)
        return 0
    if args.only_ce_backward:
        print(json.dumps(ce_forward_backward(K_, W_)), flush=True)
        return 0
    if args.only_torch_context:
        print(json.dumps(torch_context(K_, W_)), flush=True)
        return 0
    if args.only_sweep:
        log("timing the 4096^3 layout sweep ...")
        print(json.dumps(layout_sweep(K_, W_)), flush=True)
        return 0

    # ---- NT down-projection: the headline step --------------------------
    M, N, K = 768, 5120, 13824
    flops = 2.0 * M * N * K
    w = workloads.nt_mlp()
    copies = 3
    Xs = [w["X"].to(dev) for _ in range(copies)]
    Ws = [w["W"].to(dev) for _ in range(copies)]
    del w
    Ys = [torch.empty(384, 2, 5120, dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    Xv = [x.view(M, K) for x in Xs]

    def nt_step(i):
        tgemm.run("N", "T", M, N, K, Xv[i], K, Ws[i], K, Ys[i], N, tgemm.EPI_STORE_BF16)

    log("timing NT 768x5120x13824 ...")
    # shader clock of the idle device, then at the end of the timed region
    sclk_idle = tgemm.clock_ghz(tgemm.clock_probe())
    probe = torch.zeros(3, dtype=torch.int64, device=dev)
    ms = time_stream(nt_step, K_, W_, copies, probe=probe)
    sclk_end = tgemm.clock_ghz(probe)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"NT: {ms * 1e3:.1f} us/step ({tflops:.1f} TFLOP/s); shader clock {sclk_idle:.2f} GHz "
        f"idle, {sclk_end:.2f} GHz at the end of the timed steps")
    secondary = {}
    # the same steps once more, right after the timed ones (so at the
    # sustained clock), with one event between calls: the spread of the
    # per-step times (median, min, max); the median gives the sustained
    # fraction of peak next to the burst average of the timed region
    per = sorted(step_times(nt_step, max(K_, 20), copies))
    ms_median = per[len(per) // 2]
    secondary["nt_step_us_median"] = round(ms_median * 1e3, 2)
    secondary["nt_step_us_min"] = round(per[0] * 1e3, 2)
    secondary["nt_step_us_max"] = round(per[-1] * 1e3, 2)
    if not args.only_nt:
        # the same operands every step (they stay in the last-level cache)
        ms_warm = time_stream(lambda i: nt_step(0), K_, W_, 1)
        secondary["nt_same_inputs_us"] = round(ms_warm * 1e3, 2)
        secondary["nt_same_inputs_tflops"] = round(flops / (ms_warm * 1e-3) / 1e12, 2)
    del Xs, Ws, Ys, Xv

    if not args.only_nt:
        # ---- fused cross-entropy GEMM and the backward GEMMs ---------------
        secondary.update(ce_forward_backward(K_, W_))

        # ---- layout sweep 4096^3 ------------------------------------------
        secondary.update(layout_sweep(K_, W_))

        # ---- matrix-vector and dot products (M = 1 or N = 1) ---------------
        wm = workloads.nt_mlp()
        Wd = wm["W"].to(dev)                                  # [5120, 13824]
        Wn = wm["W"].t().contiguous().to(dev)                 # [13824, 5120]
        xd = wm["X"].reshape(-1, 13824)[:1].contiguous().to(dev)
        del wm
        yd = torch.empty(1, 5120, dtype=torch.bfloat16, device=dev)
        gb = 5120 * 13824 * 2 + 13824 * 2 + 5120 * 2
        for name, ta_, tb_, Bm, ldb_ in (("gemv_1x5120x13824_NT", "N", "T", Wd, 13824),
                                          ("gemv_1x5120x13824_NN", "N", "N", Wn, 5120)):
            msg = time_stream(lambda i: tgemm.run(ta_, tb_, 1, 5120, 13824, xd, 13824, Bm, ldb_, yd,
                                                  5120, tgemm.EPI_STORE_BF16), K_, W_, 1)
            secondary[f"{name}_us"] = round(msg * 1e3, 2)
            secondary[f"{name}_frac_of_hbm"] = round(gb / (msg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        del Wd, Wn, xd, yd
        Kd = 10 ** 8
        gdot = torch.Generator(device="cpu").manual_seed(5)
        av = torch.randn(Kd, generator=gdot).to(torch.bfloat16).to(dev)
        bv = torch.randn(Kd, generator=gdot).to(torch.bfloat16).to(dev)
        cd = torch.empty(1, 1, dtype=torch.float32, device=dev)
        msd = time_stream(lambda i: tgemm.run("N", "N", 1, 1, Kd, av, Kd, bv, 1, cd, 1,
                                              tgemm.EPI_STORE_F32), K_, W_, 1)
        secondary["dot_1e8_us"] = round(msd * 1e3, 2)
        secondary["dot_1e8_frac_of_hbm"] = round(4 * Kd / (msd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        del av, bv, cd

        secondary.update(fp8_linear(K_, W_))

        # ---- K=1 RoPE table --------------------------------------------------
        secondary.update(rope_tables(K_, W_))

        # ---- matrix-core ceiling (no loads, LDS or barriers) -----------------
        secondary.update(mfma_ceiling())

    traffic = measured_traffic()
    out = {
        "metric": "TFLOP/s and % of MFMA bf16 peak, NT 768x5120x13824; CE-fused GEMM rows/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": W_,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded randn, bf16)",
        "config": {"workload": "nt_down_projection_768x5120x13824",
                   "X": "bf16[384,2,13824] viewed [768,13824]", "W": "bf16[5120,13824] read as 'T'",
                   "rotated_input_copies": copies},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     # the per-step median right after the timed region, one event
                     # between calls (the chip's sustained clock)
                     "frac_sustained": round(flops / (ms_median * 1e-3) / 1e12 /
                                             PEAK_BF16_TFLOPS, 4)},
        # the clock-adjusted view: the same rate against the peak at the shader
        # clock read right after the timed steps (the chip lowers its clock
        # under sustained matrix-core load)
        "clock": {"sclk_ghz_idle": round(sclk_idle, 3),
                  "sclk_ghz_end_of_timed": round(sclk_end, 3),
                  "peak_at_that_sclk": round(PEAK_BF16_TFLOPS * sclk_end / 2.4, 1),
                  "frac_at_that_sclk": round(tflops / (PEAK_BF16_TFLOPS * sclk_end / 2.4), 4)},
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample ...")
        out["cpu_baseline"] = cpu_baseline()
        if not args.only_nt:
            out["secondary"].update(cpu_oracle_secondary())
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
