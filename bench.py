#!/usr/bin/env python
"""Throughput of the fused attention hot path on one MI355X.

One step is the whole path once: the forward kernel (O, LSE), then the three
backward stages (row pass, key-block pass for dK/dV, query-block pass for
dQ), on causal
attention with B=4, H=16, N=4096, d=128 in bf16 (the forward+backward
workload; Q, K, V, dO i.i.d. N(0, 1) from a fixed seed, already resident in
HBM before timing starts).

Work convention: forward 4*B*H*N^2*d flop, halved for causal; backward 2.5x
the forward.  ``value`` is (forward + backward flop) / wall time per step, in
TFLOP/s.  Per-kernel times come from HIP events recorded on the stream the
kernels run on (torch's current stream, which the binding passes to the
library), and the dominant kernel's roofline uses the chip's published dense
bf16 MFMA peak of 2.5 PFLOP/s.

``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the same
step (40 whole heads of 64, forward + backward) on this host's cores.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["fa_common.h", "fa_launch.h", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip"]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 100 untimed steps (about 0.15 s): shorter warmups measure the GPU
    # before its clock has settled and read about 5% low
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="c5", help="named workload (default c5: fwd+bwd)")
    ap.add_argument("--cpu-heads", type=int, default=40,
                    help="heads of the step the CPU oracle times (0 = skip cpu_baseline)")
    ap.add_argument("--splitkv", type=int, default=0,
                    help="also time the forward on small-grid shapes (c2's, and few heads with "
                         "long sequences) plain and split-KV with this many key ranges "
                         "(0 = skip); reported under 'splitkv'")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="also time the fwd+bwd step with dropout of this probability next to\n"
                         "the plain step (0 = skip); reported under 'dropout'")
    ap.add_argument("--fp8", action="store_true",
                    help="also time the FP8 (E4M3) forward next to the bf16 forward on the\n"
                         "fwd+bwd and long-context shapes; reported under 'fp8_forward'")
    ap.add_argument("--naive", action="store_true",
                    help="also time the materialise-S forward in bf16 torch ops on the same inputs")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing every named workload on its own (reported under "
                         "'configs', each with the oracle timed on a sample of it)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step split-KV timings (reported under 'decode')")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters); not timed")
    return ap.parse_args()


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_flash_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when there are none or the kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(kernel)
    if not rec or rec.get("source_sha") != sha:
        return None
    return float(rec["fetch_bytes"]) + float(rec["write_bytes"])


def host_blas():
    """(BLAS library description, its thread count) of this process's numpy."""
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = sum(int(p.get("num_threads", 1)) for p in pools) or 1
        blas = ", ".join(f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
                         for p in pools) or "unknown"
        return blas, threads
    except Exception:  # pragma: no cover
        return "unknown", None


def cpu_model_name() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        return "unknown"


def cpu_baseline(x, wl, causal: bool, n_heads: int) -> dict:
    """The fp64 oracle on ``n_heads`` whole heads of the step, timed here."""
    import numpy as np
    import oracle
    blas, blas_threads = host_blas()
    cores = len(os.sched_getaffinity(0))
    cpu_model = cpu_model_name()
    n_heads = min(n_heads, wl.B * wl.H)
    stride = max(1, (wl.B * wl.H) // n_heads)
    heads = [divmod(i * stride, wl.H) for i in range(n_heads)]
    t0 = time.perf_counter()
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attention_forward(x["q"][sl], x["k"][sl], x["v"][sl], wl.scale, causal)
        oracle.attention_backward(x["q"][sl], x["k"][sl], x["v"][sl], x["do"][sl], wl.scale, causal)
    dt = time.perf_counter() - t0
    per_head = (wl.flops_fwd(causal) + wl.flops_bwd(causal)) / (wl.B * wl.H)
    return {
        "value": round(len(heads) * per_head / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "cpu_model": cpu_model,
        "blas": blas,
        "blas_threads": blas_threads,
        "parallelism": "heads one after another, each with the BLAS library's own threads",
        "sample": (f"{len(heads)} of {wl.B * wl.H} heads of one step (forward + backward, "
                   f"N={wl.N}, d={wl.d}, {'causal' if causal else 'full'}), float64 numpy, "
                   f"{dt:.2f} s; "
                   f"same flop convention as value"),
    }


# Split-KV comparison shapes (B, H, N, d, causal, seed): c2's shape (64
# workgroups for 256 CUs) and few heads with long sequences.
SPLITKV_SHAPES = [(2, 8, 1024, 64, True, 2000), (1, 2, 16384, 128, True, 7001),
                  (1, 4, 8192, 128, False, 7002)]


def splitkv_measure(fa, make_inputs, splits: int, iters: int = 20) -> list:
    """Forward on small-grid shapes, plain and split-KV, timed with HIP
    events on the current stream (average over `iters` launches each)."""
    import numpy as np
    import torch
    out = []
    stream = torch.cuda.current_stream()

    def avg(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    for B, H, N, d, causal, seed in SPLITKV_SHAPES:
        x = make_inputs(B, H, N, d, seed=seed)
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).view(
            torch.bfloat16).cuda() for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        ws = torch.empty(fa.flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, splits),
                         dtype=torch.uint8, device=q.device)
        plain = avg(lambda: fa.flash_attn_fwd(q, k, v, causal=causal, out=o, lse=lse))
        split = avg(lambda: fa.flash_attn_fwd_splitkv(q, k, v, splits, causal=causal, out=o,
                                                      lse=lse, workspace=ws))
        f = 4.0 * B * H * N * N * d / (2 if causal else 1)
        out.append({"shape": f"{'causal' if causal else 'full'} fwd B={B} H={H} N={N} d={d}",
                    "num_splits": splits, "plain_ms": round(plain, 4),
                    "split_ms": round(split, 4), "plain_tflops": round(f / plain / 1e9, 2),
                    "split_tflops": round(f / split / 1e9, 2)})
    return out


# FP8 forward shapes (B, H, N, d, causal, seed): the fwd+bwd workload's and
# the long-context workload's shapes.
FP8_SHAPES = [(4, 16, 4096, 128, True, 5100), (1, 16, 16384, 128, True, 4100)]


def fp8_measure(fa, make_inputs, make_inputs_fp8, iters: int = 50) -> list:
    """FP8 forward next to the bf16 forward on the same shapes, timed with
    HIP events on the current stream: the median of `iters` launches after
    the warm-up of ``_event_times`` (the inputs are encoded on the host
    first, which leaves the GPU idle for seconds; 20 untimed launches alone
    read the FP8 forward on C5's shape 12% slow)."""
    import numpy as np
    import torch
    out = []
    stream = torch.cuda.current_stream()

    def avg(fn):
        t = _event_times(fn, iters, 20)
        return t[len(t) // 2]

    for B, H, N, d, causal, seed in FP8_SHAPES:
        x8 = make_inputs_fp8(B, H, N, d, seed=seed)
        q8, k8, v8 = (torch.from_numpy(x8[n]).cuda().contiguous() for n in ("q", "k", "v"))
        x = make_inputs(B, H, N, d, seed=seed)
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).view(
            torch.bfloat16).cuda() for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        t8 = avg(lambda: fa.flash_attn_fwd_fp8(q8, k8, v8, x8["descale_q"], x8["descale_k"],
                                               x8["descale_v"], causal=causal, out=o, lse=lse))
        t16 = avg(lambda: fa.flash_attn_fwd(q, k, v, causal=causal, out=o, lse=lse))
        f = 4.0 * B * H * N * N * d / (2 if causal else 1)
        # quantising Q with incoherent processing (rotation by a random-sign
        # Hadamard matrix): two passes over the bf16 input, one write of the
        # codes, 5 bytes per element of algorithmic traffic
        signs = torch.from_numpy(np.random.default_rng(seed).choice([-1.0, 1.0], d)
                                 .astype(np.float32)).cuda()
        codes = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
        dsc = torch.empty(1, dtype=torch.float32, device=q.device)
        wsq = torch.empty(fa.QUANT_WORKSPACE_BYTES // 4, dtype=torch.float32, device=q.device)
        fa.flash_attn_quantize_fp8(q, signs, codes=codes, descale=dsc, workspace=wsq)  # validates
        # straight through the C ABI with the arguments prepared once: the
        # two launches take less GPU time than the binding's argument checks
        lib = fa.load_library()
        qargs = (q.data_ptr(), codes.data_ptr(), dsc.data_ptr(), wsq.data_ptr(),
                 fa.QUANT_WORKSPACE_BYTES, q.numel() // d, d)
        sptr = int(stream.cuda_stream)
        def quant(sgn):
            if lib.flash_attn_quantize_fp8(*qargs, sgn, sptr) != 0:
                raise RuntimeError("flash_attn_quantize_fp8 failed")
        sgp = signs.data_ptr()
        tq = avg(lambda: quant(sgp))
        tp = avg(lambda: quant(None))
        qbytes = 5.0 * q.numel()
        out.append({"shape": f"{'causal' if causal else 'full'} fwd B={B} H={H} N={N} d={d}",
                    "quantize_rotated_ms": round(tq, 4),
                    "quantize_rotated_gbs": round(qbytes / tq / 1e6, 1),
                    "quantize_plain_ms": round(tp, 4),
                    "quantize_plain_gbs": round(qbytes / tp / 1e6, 1),
                    "fp8_ms": round(t8, 4), "fp8_tflops": round(f / t8 / 1e9, 2),
                    "fp8_frac_of_fp8_peak": round(f / t8 / 1e9 / PEAK_FP8_TFLOPS, 4),
                    "bf16_ms": round(t16, 4), "bf16_tflops": round(f / t16 / 1e9, 2),
                    "speedup": round(t16 / t8, 3)})
    return out


def _event_times(fn, iters: int, warmup: int, warm_s: float = 0.25) -> list:
    """Per-launch times (ms) of ``fn`` from HIP events on the current stream,
    after at least ``warmup`` untimed launches and ``warm_s`` seconds of them:
    the timed legs follow host-side work (input encoding, the oracle's
    samples) that leaves the GPU idle, and its clock takes a few hundred
    milliseconds of load to settle."""
    import time
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in evs)


def _oracle_sample(x, wl, causal: bool, q_mult: float) -> dict:
    """The fp64 oracle's forward on a bounded sample of one workload,
    timed here, with the whole workload's time extrapolated from it."""
    import numpy as np
    import oracle
    BH = wl.B * wl.H
    if wl.N <= 4096:
        n = {"c1": 1, "c2": 4, "c3": 4}.get(wl.name, 2)
        heads = [divmod(i * max(1, BH // n), wl.H) for i in range(min(n, BH))]
        t0 = time.perf_counter()
        for b, h in heads:
            sl = (slice(b, b + 1), slice(h, h + 1))
            oracle.attention_forward(x["q"][sl], x["k"][sl], x["v"][sl], wl.scale, causal)
        dt = time.perf_counter() - t0
        frac = len(heads) / BH
        what = f"{len(heads)} of {BH} whole heads"
    else:
        rows = np.linspace(0, wl.N - 1, 512).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attention_forward_rows(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], wl.scale, causal,
                                      rows)
        dt = time.perf_counter() - t0
        frac = len(rows) / (BH * wl.N)
        what = f"{len(rows)} evenly spaced query rows of 1 of {BH} heads"
    f_sample = wl.flops_fwd(causal) * frac
    return {"sample": f"{what}, forward, float64 numpy, full score rows", "sample_s": round(dt, 4),
            "est_full_config_s": round(dt / frac, 4),
            "tflops": round(f_sample / dt / 1e12, 6)}


def configs_measure(fa, make_inputs, with_oracle: bool, iters: int = 50) -> list:
    """Every named workload's forward (and, where it has one, backward)
    timed on its own with HIP events on the current stream: median and
    minimum per launch, TFLOP/s and % of the bf16 peak by the metric's flop
    convention; beside it the fp64 oracle on a sample of the same inputs."""
    import numpy as np
    import torch
    from exact_attention_flash_amd.inputs import WORKLOADS
    out = []

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda().contiguous()

    for name, wl in WORKLOADS.items():
        B, H, N, d = wl.B, wl.H, wl.N, wl.d
        for causal in wl.causal:
            for q_mult in wl.q_mults:
                x = make_inputs(B, H, N, d, seed=wl.seed, q_mult=q_mult, with_dout=wl.backward)
                q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
                o = torch.empty_like(q)
                lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
                fwd = _event_times(lambda: fa.flash_attn_fwd(q, k, v, causal=causal,
                                                             softmax_scale=wl.scale, out=o,
                                                             lse=lse), iters, 20)
                f_fwd = wl.flops_fwd(causal)
                tag = (f"{name}: {'causal' if causal else 'full'} B={B} H={H} N={N} d={d}"
                       + (f", Q x {q_mult:g}" if q_mult != 1.0 else ""))
                rec = {"workload": tag, "pass": "fwd",
                       "median_ms": round(fwd[len(fwd) // 2], 4), "min_ms": round(fwd[0], 4),
                       "tflops": round(f_fwd / (fwd[len(fwd) // 2] * 1e-3) / 1e12, 2)}
                rec["pct_of_bf16_peak"] = round(100 * rec["tflops"] / PEAK_BF16_TFLOPS, 2)
                if wl.backward:
                    do = dev(x["do"])
                    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                    ws = torch.empty(fa.flash_attn_bwd_workspace_bytes(B, H, N, d),
                                     dtype=torch.uint8, device=q.device)
                    bwd = _event_times(lambda: fa.flash_attn_bwd(
                        do, q, k, v, o, lse, causal=causal, softmax_scale=wl.scale, dq=dq, dk=dk,
                        dv=dv, workspace=ws), iters, 10)
                    f_bwd = wl.flops_bwd(causal)
                    bm = bwd[len(bwd) // 2]
                    rec.update({"pass": "fwd, bwd", "bwd_median_ms": round(bm, 4),
                                "bwd_min_ms": round(bwd[0], 4),
                                "bwd_tflops": round(f_bwd / (bm * 1e-3) / 1e12, 2),
                                "fwd_bwd_tflops": round((f_fwd + f_bwd) / (
                                    (fwd[len(fwd) // 2] + bm) * 1e-3) / 1e12, 2)})
                    rec["fwd_bwd_pct_of_bf16_peak"] = round(
                        100 * rec["fwd_bwd_tflops"] / PEAK_BF16_TFLOPS, 2)
                if with_oracle:
                    rec["oracle"] = _oracle_sample(x, wl, causal, q_mult)
                out.append(rec)
                del q, k, v, o, lse
    return out


# Decode shapes (B, H, N_kv, d): one new query per head against a long key /
# value cache, full attention.
DECODE_SHAPES = [(1, 16, 16384, 128), (1, 16, 65536, 128), (8, 8, 16384, 128)]
DECODE_SPLITS = [1, 4, 8, 16, 32, 64, 128]


def decode_measure(fa, make_inputs, iters: int = 50) -> list:
    """The split-KV forward on decode steps (N_q = 1): one range per head
    (the plain forward's grid, B * H workgroups) against the key tiles cut
    into num_splits ranges, timed with HIP events on the current stream.
    K and V are the step's compulsory traffic; their bytes per median time
    are reported against the 8 TB/s HBM peak."""
    import numpy as np
    import torch
    out = []

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda().contiguous()

    for B, H, Nk, d in DECODE_SHAPES:
        xq = make_inputs(B, H, 1, d, seed=8000 + Nk)
        xk = make_inputs(B, H, Nk, d, seed=8001 + Nk)
        q, k, v = dev(xq["q"]), dev(xk["k"]), dev(xk["v"])
        o = torch.empty_like(q)
        lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
        kv_bytes = 2.0 * B * H * Nk * d * 2
        rec = {"shape": f"decode B={B} H={H} N_q=1 N_kv={Nk} d={d}", "by_splits": {}}
        for S in DECODE_SPLITS:
            ws = torch.empty(fa.flash_attn_fwd_splitkv_workspace_bytes(B, H, 1, d, S),
                             dtype=torch.uint8, device=q.device)
            t = _event_times(lambda: fa.flash_attn_fwd_splitkv(q, k, v, S, causal=False, out=o,
                                                               lse=lse, workspace=ws), iters, 5)
            med = t[len(t) // 2]
            rec["by_splits"][str(S)] = {"median_ms": round(med, 4), "min_ms": round(t[0], 4),
                                        "kv_gbs": round(kv_bytes / (med * 1e-3) / 1e9, 1)}
        plain = rec["by_splits"]["1"]["median_ms"]
        best = min(rec["by_splits"], key=lambda s: rec["by_splits"][s]["median_ms"])
        rec.update({"plain_ms": plain, "best_splits": int(best),
                    "best_ms": rec["by_splits"][best]["median_ms"],
                    "speedup": round(plain / rec["by_splits"][best]["median_ms"], 2),
                    "best_kv_frac_of_hbm_peak": round(
                        rec["by_splits"][best]["kv_gbs"] / PEAK_HBM_GBS, 4)})
        out.append(rec)
    return out


def dropout_measure(fa, tensors, wl, causal: bool, p: float, iters: int = 10) -> dict:
    """The fwd+bwd step with dropout (probability p) next to the plain one on
    the bench workload, timed with HIP events on the current stream."""
    import torch
    q, k, v, do, o, lse, dq, dk, dv, ws = tensors
    scale = wl.scale
    stream = torch.cuda.current_stream()
    seed = 0x5EED

    def run(drop: bool, evs=None):
        if evs:
            evs[0].record(stream)
        if drop:
            fa.flash_attn_fwd_dropout(q, k, v, p, seed, 0, causal=causal, softmax_scale=scale,
                                      out=o, lse=lse)
        else:
            fa.flash_attn_fwd(q, k, v, causal=causal, softmax_scale=scale, out=o, lse=lse)
        if evs:
            evs[1].record(stream)
        if drop:
            fa.flash_attn_bwd_dropout(do, q, k, v, o, lse, p, seed, 0, causal=causal,
                                      softmax_scale=scale, dq=dq, dk=dk, dv=dv, workspace=ws)
        else:
            fa.flash_attn_bwd(do, q, k, v, o, lse, causal=causal, softmax_scale=scale, dq=dq,
                              dk=dk, dv=dv, workspace=ws)
        if evs:
            evs[2].record(stream)

    out = {"p": p}
    f_fwd, f_bwd = wl.flops_fwd(causal), wl.flops_bwd(causal)
    for name, drop in (("plain", False), ("dropout", True)):
        for _ in range(3):
            run(drop)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(iters)]
        torch.cuda.synchronize()
        for e in evs:
            run(drop, e)
        torch.cuda.synchronize()
        fwd = sum(e[0].elapsed_time(e[1]) for e in evs) / iters
        bwd = sum(e[1].elapsed_time(e[2]) for e in evs) / iters
        out[name] = {"fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
                     "fwd_tflops": round(f_fwd / fwd / 1e9, 2),
                     "fwd_bwd_tflops": round((f_fwd + f_bwd) / (fwd + bwd) / 1e9, 2)}
    return out


def naive_measure(q, k, v, o_fused, scale: float, causal: bool, f_fwd: float,
                  iters: int = 5) -> dict:
    """The materialise-S forward (the pages' plain PyTorch fallback: scores,
    mask, softmax, product with V, each a separate kernel writing its full
    N x N result) in bf16 torch ops on the GPU, timed with HIP events on the
    current stream, for comparison with the fused forward on the same inputs.
    Work is counted by the fused forward's convention."""
    import torch
    stream = torch.cuda.current_stream()
    # torch's batched bf16 product is given a contiguous right operand, not a
    # transposed view
    kt = k.transpose(-1, -2).contiguous()
    N = q.shape[-2]
    mask = torch.ones(N, N, dtype=torch.bool, device=q.device).triu(1) if causal else None

    def run():
        s = torch.matmul(q, kt)
        s.mul_(scale)
        if causal:
            s.masked_fill_(mask, float("-inf"))
        p = torch.softmax(s, dim=-1)
        del s
        return torch.matmul(p, v)

    o = run()
    torch.cuda.synchronize()
    diff = float((o.float() - o_fused.float()).abs().max())
    del o
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    return {"ms": round(ms, 4), "tflops": round(f_fwd / (ms * 1e-3) / 1e12, 2),
            "max_abs_diff_vs_fused": round(diff, 5),
            "note": "scores, mask, softmax and P V as separate bf16 torch kernels (N x N "
                    "scores and probabilities written and read in HBM); forward only"}


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only; --gpus N > 1 is not supported "
              "(the path shards over (batch, head) with no exchange between GPUs)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    from exact_attention_flash_amd import binding as fa
    from exact_attention_flash_amd.inputs import WORKLOADS, make_inputs

    fa.load_library()  # fails loudly if the HIP library is missing
    wl = WORKLOADS[args.workload]
    causal = wl.causal[-1]
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    scale = wl.scale
    x = make_inputs(B, H, N, d, seed=wl.seed, with_dout=True)

    import numpy as np

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda().contiguous()

    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.flash_attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                     device=q.device)
    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.flash_attn_fwd(q, k, v, causal=causal, softmax_scale=scale, out=o, lse=lse)
        if evs:
            evs[1].record(stream)
        fa.flash_attn_bwd_preprocess(do, o, lse, ws)
        if evs:
            evs[2].record(stream)
        fa.flash_attn_bwd_kv_blocks(do, q, k, v, dk, dv, ws, causal=causal, softmax_scale=scale)
        if evs:
            evs[3].record(stream)
        fa.flash_attn_bwd_q_blocks(do, q, k, v, dq, ws, causal=causal, softmax_scale=scale)
        if evs:
            evs[4].record(stream)

    for _ in range(args.warmup):
        step()
    if args.calib_copy_mb > 0:
        src = torch.empty(args.calib_copy_mb << 20, dtype=torch.uint8, device=q.device).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    names = ["fa_fwd", "fa_bwd_pre", "fa_bwd_kv", "fa_bwd_q"]
    times = {n: sorted(e[j].elapsed_time(e[j + 1]) for e in events) for j, n in enumerate(names)}
    avg_ms = {n: sum(t) / args.steps for n, t in times.items()}
    rows = B * H * N
    f_fwd, f_bwd = wl.flops_fwd(causal), wl.flops_bwd(causal)
    # (bound, algorithmic work per launch).  The backward's 2.5 x forward flop
    # convention is five N^2 d products per head: the key-block pass does four
    # of them (S, dP, dV, dK) and the query-block pass the fifth (dQ) plus a
    # recompute of S and dP that the convention does not count.
    work = {
        "fa_fwd": ("mfma", f_fwd),
        "fa_bwd_pre": ("hbm", rows * d * 2 * 2 + rows * 4 + rows * 4 * 2),
        "fa_bwd_kv": ("mfma", f_bwd * 4 / 5),
        "fa_bwd_q": ("mfma", f_bwd * 1 / 5),
    }
    kernels = {}
    for n in names:
        bound, w = work[n]
        t = avg_ms[n] * 1e-3
        ach = w / t / (1e12 if bound == "mfma" else 1e9)
        kernels[n] = {"avg_ms": round(avg_ms[n], 4),
                      "median_ms": round(times[n][len(times[n]) // 2], 4),
                      "min_ms": round(times[n][0], 4), "bound": bound,
                      "achieved": round(ach, 2), "unit": "TFLOP/s" if bound == "mfma" else "GB/s"}
    dom = max(names, key=lambda n: avg_ms[n])
    bound, w = work[dom]
    peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
    achieved = w / (avg_ms[dom] * 1e-3) / (1e12 if bound == "mfma" else 1e9)
    roofline = {
        "bound": bound,
        "kernel": dom,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
        "frac": round(achieved / peak, 4),
        "traffic": load_traffic(dom, kernel_source_sha()),
        "work_per_launch": w,
    }
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = f_fwd / (avg_ms["fa_fwd"] * 1e-3) / 1e12
    bwd_ms = avg_ms["fa_bwd_pre"] + avg_ms["fa_bwd_kv"] + avg_ms["fa_bwd_q"]
    line = {
        "metric": "attention TFLOP/s (fwd+bwd) at 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{'causal' if causal else 'full'} attention fwd+bwd "
                               f"B={B} H={H} N={N} d={d}",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if args.naive:
        line["naive_fwd"] = naive_measure(q, k, v, o, scale, causal, f_fwd)
        line["naive_fwd"]["fused_fwd_ms"] = round(avg_ms["fa_fwd"], 4)
    if args.splitkv > 0:
        line["splitkv"] = splitkv_measure(fa, make_inputs, args.splitkv)
    if args.dropout > 0:
        line["dropout"] = dropout_measure(fa, (q, k, v, do, o, lse, dq, dk, dv, ws), wl, causal,
                                          args.dropout)
    if args.fp8:
        from exact_attention_flash_amd.inputs import make_inputs_fp8
        line["fp8_forward"] = fp8_measure(fa, make_inputs, make_inputs_fp8)
    if not args.no_configs:
        line["configs"] = configs_measure(fa, make_inputs, with_oracle=args.cpu_heads > 0)
    if not args.no_decode:
        line["decode"] = decode_measure(fa, make_inputs)
    if args.cpu_heads > 0:
        line["cpu_baseline"] = cpu_baseline(x, wl, causal, args.cpu_heads)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
