"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fine_swiglu]

One step is one moe_forward call over one batch: gate GEMM + gate epilogue
(noise, top-k, softmax, importance/load), dispatch (histogram, scan,
permutation, gather), the two grouped expert GEMMs, combine and the aux
losses.  The default workload is the largest single-GPU one, the
fine-grained layer (T=4096, d=7168, 256 SwiGLU experts of hidden 2048,
top-8, Zipf-skewed routing); --workload picks another preset.  Inputs and
weights are seeded synthetic tensors already resident in HBM.  Prints one
JSON line:
  value        tokens/s over K back-to-back steps (host clock around the
               synchronised loop); the per-step HIP-event medians with and
               without a cache flush before each step are in `timing`;
  roofline     the dominant kernel's algorithmic bytes (or flops) per launch
               over its average duration, measured with HIP events recorded
               on the library's stream (moe_profile_*) around every launch of
               the timed eager steps, against the MI355X
               peak (HBM 8 TB/s, bf16 MFMA 2.5 PFLOP/s, fp32 157.3 TFLOP/s);
               `traffic` is the kernel's HBM bytes per launch from the
               rocprofv3 counter summary under profiles/, reported only while
               the kernel's source is the one the counters were taken on;
  side_by_side where the bf16 experts split by size run their two grouped
               GEMMs side by side on shares of the CUs: the shares, and per
               phase (first GEMM, second GEMM) both kernels' algorithmic
               bytes and flops over the longer duration; the 256 x 256
               kernels' entries also carry their rate against their share of
               the matrix-unit peak (frac_cu_share);
  kernels      the same figures for every kernel of the step;
  timing       also per-step HIP-event medians, p10 and p90, warm (back to
               back) and cold (a 512 MiB write before each step evicts L2
               and the Infinity Cache);
  peaks_measured  attainable HBM (a 1 GiB read stream, moe_probe_hbm_read,
               and a 1 GiB device copy) and MFMA (moe_probe_mfma) rates;
               every roofline entry also carries its fraction of these
               (frac_measured: HBM-bound kernels against the read stream);
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload
               (its first tokens: gate, dispatch, every expert they reach,
               combine, losses; each expert's weights are copied to the host
               outside the timed parts) on this host's cores;
  check        the GPU output on that sample against the oracle.

    python bench.py --backward [--steps K] [--warmup W] [--workload lm_layer]

times moe_backward instead (one step: the forward's routing and activations
recomputed, then every gradient) and prints one JSON line of the same shape,
its cpu_baseline the oracle's backward on a bounded token sample.

    python bench.py --train [--steps K] [--warmup W] [--workload lm_layer]

times a training step: moe_forward_train (the forward, y and losses, keeping
its intermediates) then moe_backward_saved (every gradient from them); same
line shape, same cpu_baseline (the oracle's backward includes its forward).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec at 1 GPU; expert-GEMM % MFMA peak; routing % HBM BW"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
DEFAULT_WORKLOAD = "fine_swiglu"
# Gate GEMMs computed as fp32 contractions from six bf16 products per term.
SPLIT_GATE_KERNELS = ("gate_gemm_bf16x6", "gate2_gemm_bf16x6", "bwd_gate_dx")


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` at `workload` from the committed
    rocprofv3 summary profiles/<workload>_ggemm_traffic.txt: FETCH_SIZE and
    WRITE_SIZE (separate --pmc runs, KiB per dispatch), each scaled by what
    the same counter reads for a plain copy of known size.  A summary line
      # traffic_bytes <kernel> <bytes> source <file> sha256 <hex>
    carries the hash of the kernel's source file when the counters were
    taken; a different source today (the kernel changed) gives None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_ggemm_traffic.txt")
    if not os.path.exists(path):
        return None
    pat = re.compile(r"^# traffic_bytes (\S+) (\d+) source (\S+) sha256 ([0-9a-f]+)$")
    for line in open(path):
        m = pat.match(line.strip())
        if not m or m.group(1) != kernel:
            continue
        src = os.path.join(ROOT, m.group(3))
        if not os.path.exists(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != m.group(4):
            return None
        return int(m.group(2))
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def launch_experts(name, cfg, counts):
    """(rows, non-empty experts) one launch of a routed-expert GEMM covers:
    all of them, or -- where the library splits the experts by size
    (moe_expert_split_rows) -- those below the split for the 128-row kernel
    (ggemm_bf16_*, ggemm_fp8_*) and the rest for the 256 x 256 one
    (ggemm_big_*)."""
    import sparsely_gated_mixture_amd as moe
    c = np.asarray(counts)
    c = c[c > 0]
    split = moe.moe_expert_split_rows(cfg) if name.startswith("ggemm_") else 0
    if split > 0:
        c = c[c >= split] if name.startswith("ggemm_big_") else c[c < split]
    return int(c.sum()), int(len(c))


def side_by_side(cfg, counts, kernels):
    """The two expert GEMM classes run side by side on shares of the CUs
    (moe_expert_cu_split, one share per product): each such kernel entry
    gets its CU count, the
    256 x 256 kernels their rate against their share of the matrix-unit
    peak, and the result describes each phase (first GEMM, second GEMM) as a
    whole: both kernels' algorithmic bytes and flops over the longer of the
    two durations (they start together).  None when they run one after the
    other."""
    import sparsely_gated_mixture_amd as moe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shares = [moe.moe_expert_cu_split(cfg, np.asarray(counts, np.int32), cus, prod)
              for prod in (0, 1)]
    if not all(0 < s < cus for s in shares):
        return None
    out = {"cus_total": cus, "cus_big": shares, "cus_small": [cus - s for s in shares],
           "phases": []}
    for big_name, small_name, prod in (("ggemm_big_swiglu", "ggemm_bf16_swiglu", 0),
                                       ("ggemm_big_relu", "ggemm_bf16_relu", 0),
                                       ("ggemm_big_out", "ggemm_bf16_out", 1)):
        b, sm = kernels.get(big_name), kernels.get(small_name)
        if not b or not sm:
            continue
        share = shares[prod]
        b["cus"], sm["cus"] = share, cus - share
        rl = b.get("roofline")
        if rl and rl["bound"] == "mfma":
            rl["peak_cu_share"] = rl["peak"] * share / cus
            rl["frac_cu_share"] = rl["achieved"] / rl["peak_cu_share"]
        t = max(b["avg_us"], sm["avg_us"]) * 1e-6
        byt = b["algo_bytes"] + sm["algo_bytes"]
        fl = b.get("flops", 0) + sm.get("flops", 0)
        ph = {"kernels": [big_name, small_name], "us": t * 1e6, "algo_bytes": byt, "flops": fl,
              "GB_s": byt / t / 1e9, "TFLOP_s": fl / t / 1e12}
        if byt / PEAK_HBM_GBS / 1e9 >= fl / PEAK_TFLOPS["bf16"] / 1e12:
            ph.update(bound="hbm", frac=ph["GB_s"] / PEAK_HBM_GBS)
        else:
            ph.update(bound="mfma", frac=ph["TFLOP_s"] / PEAK_TFLOPS["bf16"])
        out["phases"].append(ph)
    return out


def kernel_work(name, cfg, rows, nonempty, T, fwd=True):
    """(algorithmic bytes, flops, dtype) of one launch of kernel `name` for
    this step's realised routing (rows and non-empty experts of the
    launch).  fwd: the layer forward, whose bf16 / FP8 experts write their
    output rows in bf16 (the training forward keeps them in fp32)."""
    d, h, n, k = cfg.d_model, cfg.d_hidden, cfg.n_experts, cfg.k
    bf = cfg.expert_dtype != 0
    wsz = 2 if bf else 4
    ysz = 2 if bf and fwd else 4  # bytes per element of the expert output rows
    noisy = cfg.noisy
    ng = cfg.n_groups if cfg.hierarchical else n  # the flat or primary gate's width
    ncols = 2 * ng if noisy else ng
    if cfg.hierarchical:
        # the two-level secondary gate: T*k1 rows of 2b logits (grouped split-bf16
        # GEMM: six bf16 products per term)
        r2, c2 = T * cfg.k_groups, (2 if noisy else 1) * cfg.b
        if name == "gate2_gemm_bf16x6":
            return (r2 * d * 4 + cfg.n_groups * c2 * d * 4 + r2 * c2 * 4,
                    2.0 * r2 * c2 * d, "f32")
        if name == "gate_topk_grouped":
            return (r2 * c2 * 4 + (r2 * cfg.b * 4 if noisy else 0) + T * k * 8, 0.0, "f32")
    if name in ("ggemm_bf16_relu", "ggemm_big_relu"):
        return (nonempty * h * d * 2 + rows * d * 2 + rows * h * 2, 2.0 * rows * h * d, "bf16")
    if name in ("ggemm_bf16_swiglu", "ggemm_big_swiglu"):
        return (nonempty * 2 * h * d * 2 + rows * d * 2 + rows * h * 2, 4.0 * rows * h * d,
                "bf16")
    if name in ("ggemm_bf16_out", "ggemm_big_out"):
        return (nonempty * d * h * 2 + rows * h * 2 + rows * d * ysz, 2.0 * rows * d * h, "bf16")
    # FP8 experts: one byte per weight plus one fp32 scale per weight row
    if name in ("ggemm_fp8_relu", "ggemm_big_fp8_relu"):
        return (nonempty * (h * d + 4 * h) + rows * d * 2 + rows * h * 2, 2.0 * rows * h * d,
                "bf16")
    if name in ("ggemm_fp8_swiglu", "ggemm_big_fp8_swiglu"):
        return (nonempty * 2 * (h * d + 4 * h) + rows * d * 2 + rows * h * 2,
                4.0 * rows * h * d, "bf16")
    if name in ("ggemm_fp8_out", "ggemm_big_fp8_out"):
        return (nonempty * (d * h + 4 * d) + rows * h * 2 + rows * d * ysz, 2.0 * rows * d * h,
                "bf16")
    hs = cfg.d_hidden_shared
    if name in ("shared_bf16_relu", "shared_big_relu"):
        return (hs * d * 2 + T * d * 2 + T * hs * 2, 2.0 * T * hs * d, "bf16")
    if name in ("shared_bf16_swiglu", "shared_big_swiglu"):
        return (2 * hs * d * 2 + T * d * 2 + T * hs * 2, 4.0 * T * hs * d, "bf16")
    if name in ("shared_bf16_out", "shared_big_out"):
        return (d * hs * 2 + T * hs * 2 + T * d * 4, 2.0 * T * d * hs, "bf16")
    if name == "gate_gemm_bf16x6":
        # The method's work is one fp32 contraction (2*T*d*ncols flops, graded
        # against the fp32 peak); the kernel reaches fp32 accuracy with six
        # bf16 products per term (their rate is reported beside it).  In the
        # flat layer with bf16 or FP8 experts it also writes x in bf16.
        xb = T * d * 2 if bf and not cfg.hierarchical and T * d * 2 <= 1 << 30 else 0
        return (T * d * 4 + ncols * d * 4 + T * ncols * 4 + xb, 2.0 * T * ncols * d, "f32")
    if name.startswith("gemm_f32"):
        return (T * d * 4 + ncols * d * 4 + T * ncols * 4, 2.0 * T * ncols * d, "f32")
    if name == "gate_topk":
        return (T * ncols * 4 + (T * ng * 4 if noisy else 0) + T * k * 8, 0.0, "f32")
    if name == "dispatch_gather_bf16":  # x once in token order (experts read rows via perm)
        return (T * d * 4 + T * d * 2, 0.0, "f32")
    if name == "dispatch_gather":
        return (T * d * 4 + rows * d * wsz + rows * 4 + (T * d * 2 if hs else 0), 0.0, "f32")
    if name == "combine":
        return (rows * d * ysz + T * d * 4 + T * k * 8 + (T * d * 4 if hs else 0), 0.0, "f32")
    if name == "dispatch_permute":
        return (T * k * 4 * 2 + rows * 4, 0.0, "i32")
    w = 16 if (cfg.n_groups or n) <= 512 else 8
    rpb = max(w, -(-((T + 255) // 256) // w) * w)
    nparts = (T + rpb - 1) // rpb
    if name == "dispatch_hist":
        # the flat layer's launch also sums the gate's Importance / Load partials
        sums = 0 if cfg.n_groups else (nparts * n * 4 + n * 4) * (2 if noisy else 1)
        return (T * k * 4 + ((T * k + 255) // 256) * n * 4 + sums, 0.0, "i32")
    if name == "gate_colsum":
        return (nparts * n * 4 + n * 4, 0.0, "f32")
    if name == "dispatch_colscan":
        return (((T * k + 255) // 256) * n * 8 + n * 4, 0.0, "i32")
    if name == "dispatch_scan_finalize":  # the column scan, then the finalize in its last block
        return (((T * k + 255) // 256) * n * 8 + n * 4 + n * 12, 0.0, "i32")
    if name in ("dispatch_finalize", "dispatch_offsets", "ffn_tilemap", "aux_loss"):
        return (n * 12, 0.0, "i32")
    return (0.0, 0.0, "")


def bwd_kernel_work(name, cfg, rows, nonempty, T):
    """(algorithmic bytes, flops, dtype) of one launch of a backward kernel."""
    d, h, n, k = cfg.d_model, cfg.d_hidden, cfg.n_experts, cfg.k
    sw = cfg.act == 1
    hw = 2 * h if sw else h
    ng = cfg.n_groups if cfg.hierarchical else n
    M = 2 * ng if cfg.noisy else ng
    hs = cfg.d_hidden_shared
    hws = 2 * hs if sw else hs
    if name == "bwd_ggemm_preact":   # x W1^T and x W3^T kept in fp32 (SwiGLU)
        return (nonempty * h * d * 2 + rows * d * 2 + rows * h * 4, 2.0 * rows * h * d, "bf16")
    if name == "bwd_shared_preact":
        return (hs * d * 2 + T * d * 2 + T * hs * 4, 2.0 * T * hs * d, "bf16")
    if name == "bwd_swiglu_hidden":
        return (0.0, 0.0, "")  # rows differ between the routed and shared launches
    if name == "bwd_ggemm_dhidden":
        aux = rows * h * (8 if sw else 2)
        return (nonempty * d * h * 2 + rows * d * 2 + aux + rows * hw * 2, 2.0 * rows * d * h,
                "bf16")
    if name == "bwd_ggemm_dinput":
        return (nonempty * hw * d * 2 + rows * hw * 2 + rows * d * 4, 2.0 * rows * hw * d, "bf16")
    if name == "bwd_ggemm_dw2":
        return (rows * h * 2 + rows * d * 2 + n * d * h * 4, 2.0 * rows * d * h, "bf16")
    if name == "bwd_ggemm_dw1":
        return (rows * d * 2 + rows * hw * 2 + n * hw * d * 4, 2.0 * rows * hw * d, "bf16")
    if name == "bwd_shared_dhidden":
        aux = T * hs * (8 if sw else 2)
        return (d * hs * 2 + T * d * 2 + aux + T * hws * 2, 2.0 * T * d * hs, "bf16")
    if name == "bwd_shared_dinput":
        return (hws * d * 2 + T * hws * 2 + T * d * 4, 2.0 * T * hws * d, "bf16")
    if name == "bwd_shared_dw2":
        return (T * hs * 2 + T * d * 2 + d * hs * 4, 2.0 * T * d * hs, "bf16")
    if name == "bwd_shared_dw1":
        return (T * d * 2 + T * hws * 2 + hws * d * 4, 2.0 * T * hws * d, "bf16")
    if name == "bwd_gate_wgrad":
        return (T * d * 4 + T * M * 4 + M * d * 4, 2.0 * T * M * d, "f32")
    if name == "bwd_gate_dx":  # an fp32 contraction (split-bf16 GEMM: six bf16 products per term)
        return (T * M * 4 + M * d * 4 + T * d * 4, 2.0 * T * M * d, "f32")
    if name == "bwd_combine":
        return (T * d * 4 + rows * d * 4 + rows * d * 2 + T * k * 12, 0.0, "f32")
    if name == "bwd_gate":
        if cfg.hierarchical:
            return (0.0, 0.0, "")  # the primary and secondary gates share the name
        return (T * M * 4 + (T * n * 4 if cfg.noisy else 0) + T * k * 12 + T * M * 4, 0.0,
                "f32")
    if name in ("bwd_gate2_wgrad", "bwd_gate2_dx"):
        r2, c2 = T * cfg.k_groups, (2 if cfg.noisy else 1) * cfg.b
        wbytes = cfg.n_groups * c2 * d * 4
        return (r2 * d * 4 + r2 * c2 * 4 + wbytes, 2.0 * r2 * c2 * d, "f32")
    if name == "bwd_dx_gather":
        return (T * d * 4 + rows * d * 4 + (T * d * 4 if hs else 0) + T * d * 4, 0.0, "f32")
    return kernel_work(name, cfg, rows, nonempty, T, fwd=False)


def gate_text(cfg):
    if cfg.gate == 1:
        return "Switch top-1 softmax, fp32"
    if cfg.gate == 2:
        return "sigmoid top-k with selection-only bias, fp32"
    return ("noisy " if cfg.noisy else "") + "top-k softmax, fp32"


def roofline_entry(bytes_, flops, dtype, avg_s):
    t_hbm = bytes_ / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (PEAK_TFLOPS.get(dtype, 1e30) * 1e12) if flops else 0.0
    gbs = bytes_ / avg_s / 1e9 if avg_s > 0 else 0.0
    tfs = flops / avg_s / 1e12 if avg_s > 0 else 0.0
    if t_mfma > t_hbm:
        return dict(bound="mfma", achieved=tfs, peak=PEAK_TFLOPS[dtype], unit="TFLOP/s",
                    frac=tfs / PEAK_TFLOPS[dtype]), gbs, tfs
    return dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s",
                frac=gbs / PEAK_HBM_GBS), gbs, tfs


def event_percentiles(fn, reps, flush=None):
    """Per-step device time of fn (HIP events on the current stream, which is
    the library's stream), optionally after a cache flush outside the timed
    interval: median, p10 and p90 in microseconds."""
    pairs = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    return {"median_us": float(np.median(us)), "p10_us": float(np.percentile(us, 10)),
            "p90_us": float(np.percentile(us, 90)), "reps": reps}


def measure_peaks():
    """Attainable peaks on this device, measured beside the datasheet ones:
    HBM from a plain device copy of 1 GiB into another 1 GiB (bytes read +
    written over the time), the matrix units from the library's MFMA loop
    probe (moe_probe_mfma: register operands only)."""
    import sparsely_gated_mixture_amd as moe
    out = {}
    n = 256 << 20  # fp32 elements: 1 GiB
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    r = event_percentiles(lambda: dst.copy_(src), 5)
    out["hbm_copy_GB_s"] = 2 * n * 4 / (r["median_us"] * 1e-6) / 1e9
    del dst
    blocks, iters = 2048, 1000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    moe.moe_probe_hbm_read(src, n * 4, blocks, sink)
    r = event_percentiles(lambda: moe.moe_probe_hbm_read(src, n * 4, blocks, sink), 5)
    out["hbm_read_GB_s"] = n * 4 / (r["median_us"] * 1e-6) / 1e9
    del src
    for name, dt in (("bf16", moe.MOE_BF16), ("f32", moe.MOE_F32)):
        flops = moe.moe_probe_mfma(dt, blocks, iters, sink)
        r = event_percentiles(lambda: moe.moe_probe_mfma(dt, blocks, iters, sink), 5)
        out[f"mfma_{name}_TFLOP_s"] = flops / (r["median_us"] * 1e-6) / 1e12
    out["method"] = ("HBM: torch copy_ of 1 GiB fp32 (read + write bytes / median of 5) and "
                     "moe_probe_hbm_read over 1 GiB (2048 blocks, eight 16-byte loads in flight "
                     "per thread; read bytes / median of 5); "
                     "MFMA: moe_probe_mfma, 2048 blocks x 4 waves x 1000 iterations of 4 "
                     "independent 32x32 MFMAs (median of 5)")
    torch.cuda.synchronize()
    return out


def cpu_baseline(cfg, inp, y_gpu, idx_gpu, sample_tokens, seconds):
    """The CPU oracle on the first S tokens of the batch, stage by stage: the
    gate (flat or two-level), dispatch, every expert those tokens reach (and
    the shared expert), combine and the losses, all in float64.  Each
    expert's weights are copied to the host outside the timed parts, so the
    figure is the oracle's own compute.  Without `sample_tokens`, S doubles
    from 16 until a pass takes a quarter of `seconds`, then grows so that one
    pass takes about half of it (all of it where the weights do not fit on
    the host and the pass does not repeat).  Where the
    weights fit on the host (at most 16 GiB in float64) they are kept and the
    pass repeats until `seconds` have passed; the same oracle also runs on
    one core on a smaller sample.  The GPU's y on the sample is checked
    against the oracle's on every token the two route alike."""
    import oracle
    from sparsely_gated_mixture_amd.workloads import to_numpy64
    oracle.lib()
    T, d, n, k = cfg.T, cfg.d_model, cfg.n_experts, cfg.k
    bf = cfg.expert_dtype != 0
    hk = {key: to_numpy64(inp.get(key)) for key in ("w_gate", "b_gate", "w_noise", "w_gate2",
                                                    "w_noise2", "ws1", "ws3", "ws2")}
    names = [nm for nm in ("w1", "w3", "w2", "b1", "b2") if inp.get(nm) is not None]
    per_expert = sum(inp[nm][0].numel() * 8 for nm in names)
    keep = n * per_expert <= (16 << 30)
    cache = {}

    def weights(e):
        if e in cache:
            return cache[e]
        w = {nm: (inp[nm][e].to(torch.float64).cpu().numpy() if nm in names else None)
             for nm in ("w1", "w3", "w2", "b1", "b2")}
        if cfg.expert_dtype == 2:  # FP8: the values the codes stand for
            for nm in ("w1", "w3", "w2"):
                if w[nm] is not None:
                    w[nm] = oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(w[nm]))
        if keep:
            cache[e] = w
        return w

    def one_pass(S):
        """(seconds of oracle compute, topk_idx, y) for the first S tokens."""
        x = to_numpy64(inp["x"][:S])
        noise = to_numpy64(inp["noise"][:S]) if inp.get("noise") is not None else None
        spent = 0.0
        t0 = time.perf_counter()
        if cfg.hierarchical:
            noise2 = to_numpy64(inp["noise2"][:S]) if inp.get("noise2") is not None else None
            gh = oracle.gate_hier(x, hk["w_gate"], hk["w_noise"], noise, cfg.k_groups,
                                  hk["w_gate2"], hk["w_noise2"], noise2, cfg.k2,
                                  b_gate=hk["b_gate"])
            idx, w, imp, ld = gh["topk_idx"], gh["topk_w"], gh["importance"], gh["load"]
            zsum, entsum = gh["zsum"], gh["entsum"]
        else:
            gr = oracle.gate(x, hk["w_gate"], k, hk["b_gate"], hk["w_noise"], noise, cfg.gate)
            idx, w, imp, ld, zsum, entsum = (gr.topk_idx, gr.topk_w, gr.importance, gr.load,
                                             gr.zsum, gr.entsum)
        disp = oracle.dispatch(idx, n, cfg.capacity_factor)
        spent += time.perf_counter() - t0
        off, perm = disp["offsets"], disp["perm"]
        y_perm = np.zeros((disp["rows"], d))
        for e in range(n):
            lo, hi = int(off[e]), int(off[e + 1])
            if hi == lo:
                continue
            we = weights(e)
            t0 = time.perf_counter()
            y_perm[lo:hi] = oracle.expert_ffn(x[perm[lo:hi]], we["w1"], we["w2"], b1=we["b1"],
                                              w3=we["w3"], b2=we["b2"], act=cfg.act, bf16=bf)
            spent += time.perf_counter() - t0
        t0 = time.perf_counter()
        y = oracle.combine(y_perm, disp["slot_pos"], w, d)
        if cfg.d_hidden_shared:
            y = y + oracle.expert_ffn(x, hk["ws1"], hk["ws2"], w3=hk["ws3"], act=cfg.act,
                                      bf16=bf)
        oracle.aux(S, k, imp, ld, disp["counts_pre"], cfg.w_importance, cfg.w_load,
                   cfg.alpha_switch, zsum, entsum, cfg.w_z, cfg.w_entropy)
        spent += time.perf_counter() - t0
        return spent, idx, y

    sized = sample_tokens is None
    S = min(T, 16 if sized else sample_tokens)
    dt, idx, y = one_pass(S)
    while sized and S < T and dt < seconds / 4:   # more rows per expert: more threads busy
        S = min(T, 2 * S)
        dt, idx, y = one_pass(S)
    # one pass of about half of `seconds` when it repeats, else one of about `seconds`
    target = seconds / 2 if keep else seconds
    if sized and S < T and dt < target:
        S = int(min(T, S * target / max(dt, 1e-3)))
        dt, idx, y = one_pass(S)
    reps = 1
    while keep and dt < seconds:
        d1, _, _ = one_pass(S)
        dt += d1
        reps += 1
    cores = oracle.num_threads()
    base = {"value": S * reps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {S} of {T} tokens of the {cfg.name} workload (gate, dispatch, "
                      f"the experts they reach, combine, losses in float64; expert weights "
                      f"copied to the host outside the timed parts), {reps} pass(es), "
                      f"{dt:.2f} s of oracle compute on {cores} OpenMP threads"}
    if keep:
        S1 = min(512, S)
        oracle.set_num_threads(1)
        try:
            reps1, dt1 = 0, 0.0
            while reps1 == 0 or dt1 < seconds / 2:
                d1, _, _ = one_pass(S1)
                dt1 += d1
                reps1 += 1
        finally:
            oracle.set_num_threads(cores)
        base["single_core"] = {"value": S1 * reps1 / dt1, "unit": "tokens/s", "cores": 1,
                               "sample": f"first {S1} tokens, {reps1} passes, {dt1:.2f} s"}
    same = np.all(idx_gpu[:S] == idx, axis=1)
    scale = np.max(np.abs(y[same])) if same.any() else 1.0
    err = float(np.max(np.abs(y_gpu[:S][same] - y[same])) / scale) if same.any() else None
    check = {"tokens": S, "routing_match": float(same.mean()), "y_max_abs_norm_err": err,
             "tolerance": 2e-2 if bf else 1e-4}
    return base, check


def calibrate_copy():
    """A plain elementwise device copy (y = -x, fp32) of 256 MiB, five
    launches: the reference kernel against which the rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings of the layer's kernels are scaled."""
    n = 64 << 20
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "neg copy", "read_bytes": n * 4, "write_bytes": n * 4,
                      "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens of the CPU oracle's sample (default: the workload's first "
                         "tokens, as many as about --cpu-seconds of oracle work takes)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target oracle compute time of the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (default: also replay a HIP graph)")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward (forward recompute + every gradient)")
    ap.add_argument("--train", action="store_true",
                    help="time moe_forward_train + moe_backward_saved (one training step)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (256 MiB read, "
                         "256 MiB written, 5 launches) for scaling HBM byte counters")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer is built and "
              "measured on a single MI355X, with no collectives.", file=sys.stderr)
        sys.exit(2)

    import sparsely_gated_mixture_amd as moe
    from sparsely_gated_mixture_amd.workloads import PRESETS, make_inputs

    cfg = PRESETS[args.workload]
    torch.cuda.set_device(0)
    if args.backward or args.train:
        bench_backward(args, cfg, train=args.train)
        return
    log(f"[bench] workload {cfg.name}: T={cfg.T} d={cfg.d_model} h={cfg.d_hidden} "
        f"n={cfg.n_experts} k={cfg.k}")
    inp = make_inputs(cfg, device="cuda")
    torch.cuda.synchronize()
    layer = moe.MoELayer(cfg, inp)
    T, n, k = cfg.T, cfg.n_experts, cfg.k
    i32 = dict(dtype=torch.int32, device="cuda")
    diag = {"topk_idx": torch.empty((T, k), **i32), "counts": torch.empty(n, **i32),
            "offsets": torch.empty(n + 1, **i32)}
    y = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
    losses = torch.empty(moe.N_LOSSES, dtype=torch.float32, device="cuda")

    for _ in range(args.warmup):
        layer.forward(inp["x"], inp.get("noise"), inp.get("noise2"), y=y, losses=losses)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")

    def timed(step_fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step_fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def eager_step():
        layer.forward(inp["x"], inp.get("noise"), inp.get("noise2"), y=y, losses=losses)

    # Fill the library's event pool with one untimed profiled pass, so that
    # the timed pass below creates no events.
    moe.moe_profile_enable(True)
    for _ in range(args.steps):
        eager_step()
    torch.cuda.synchronize()
    moe.moe_profile_enable(False)
    moe.moe_profile_collect()

    # Timed region 1: eager launches, nothing else on the stream.
    eager_elapsed = timed(eager_step)
    log(f"[bench] eager: {eager_elapsed / args.steps * 1e6:.1f} us/step, "
        f"{T * args.steps / eager_elapsed / 1e6:.2f} M tokens/s")

    # Timed region 2: the same K eager steps with every kernel bracketed by
    # two HIP events recorded on the library's stream; the per-kernel
    # durations (and the roofline) come from these steps.  The events add a
    # few microseconds between launches, so this region does not set `value`.
    moe.moe_profile_enable(True)
    prof_elapsed = timed(eager_step)
    moe.moe_profile_enable(False)
    nk = moe.moe_profile_collect()
    stats = [moe.moe_profile_entry(i) for i in range(nk)]
    log(f"[bench] eager with per-kernel events: {prof_elapsed / args.steps * 1e6:.1f} us/step")
    mode, elapsed = "eager launches", eager_elapsed
    graph = None
    if not args.eager:
        # The whole forward captured once as a HIP graph and replayed: the
        # same kernels, with the per-launch host and queue overhead removed.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            eager_step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()
        for _ in range(args.warmup):
            graph.replay()
        graph_elapsed = timed(graph.replay)
        log(f"[bench] graph: {graph_elapsed / args.steps * 1e6:.1f} us/step, "
            f"{T * args.steps / graph_elapsed / 1e6:.2f} M tokens/s")
        if graph_elapsed < elapsed:
            mode, elapsed = "HIP graph replay of the whole forward", graph_elapsed
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = T * args.steps / elapsed

    # Realised routing of this batch (identical every step).
    layer.forward(inp["x"], inp.get("noise"), inp.get("noise2"), y=y, losses=losses, diag=diag)
    torch.cuda.synchronize()
    counts = diag["counts"].cpu().numpy()
    rows = int(counts.sum())
    nonempty = int((counts > 0).sum())

    kernels = {}
    dominant = None
    for name, total_ms, launches in stats:
        avg_s = total_ms / launches / 1e3
        b, f, dt = kernel_work(name, cfg, *launch_experts(name, cfg, counts), T)
        entry = {"avg_us": avg_s * 1e6, "launches_per_step": launches / args.steps}
        if b:
            rl, gbs, tfs = roofline_entry(b, f, dt, avg_s)
            entry.update({"algo_bytes": b, "GB_s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS})
            if f:
                entry.update({"flops": f, "TFLOP_s": tfs, "mfma_frac": tfs / PEAK_TFLOPS[dt],
                              "ai_flop_per_byte": f / b})
                if name in SPLIT_GATE_KERNELS:
                    entry["split_bf16_products"] = {
                        "TFLOP_s": 6 * tfs, "frac_of_bf16_peak": 6 * tfs / PEAK_TFLOPS["bf16"],
                        "note": "the six bf16 products per fp32 term the kernel issues"}
            entry["roofline"] = rl
        kernels[name] = entry
        if dominant is None or total_ms > dominant[1]:
            dominant = (name, total_ms)
    for name, e in sorted(kernels.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["launches_per_step"]):
        log(f"[bench]   {name:22s} {e['avg_us']:9.1f} us x{e['launches_per_step']:.0f}"
            + (f"  {e['GB_s']:8.1f} GB/s" if "GB_s" in e else "")
            + (f"  {e['TFLOP_s']:7.1f} TFLOP/s" if "TFLOP_s" in e else ""))
    # Per-step device time, warm (back to back) and cold (a 512 MiB buffer
    # written before each step, outside its events, evicts L2 and the 256 MB
    # Infinity Cache).
    warm = event_percentiles(eager_step, args.steps)
    flush_buf = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    cold = event_percentiles(eager_step, args.steps, flush=lambda: flush_buf.fill_(1.0))
    del flush_buf
    log(f"[bench] per-step events: warm median {warm['median_us']:.1f} us "
        f"(p10 {warm['p10_us']:.1f}, p90 {warm['p90_us']:.1f}); cold median "
        f"{cold['median_us']:.1f} us (p10 {cold['p10_us']:.1f}, p90 {cold['p90_us']:.1f})")
    peaks = measure_peaks()
    log(f"[bench] measured peaks: read {peaks['hbm_read_GB_s']:.0f} GB/s, "
        f"copy {peaks['hbm_copy_GB_s']:.0f} GB/s, bf16 MFMA "
        f"{peaks['mfma_bf16_TFLOP_s']:.0f} TFLOP/s, fp32 MFMA {peaks['mfma_f32_TFLOP_s']:.1f} "
        f"TFLOP/s")
    for e in kernels.values():
        rl = e.get("roofline")
        if rl:
            mp = (peaks["hbm_read_GB_s"] if rl["bound"] == "hbm" else
                  peaks["mfma_bf16_TFLOP_s"] if rl["peak"] == PEAK_TFLOPS["bf16"] else
                  peaks["mfma_f32_TFLOP_s"])
            rl["peak_measured"] = mp
            rl["frac_measured"] = rl["achieved"] / mp
    side = side_by_side(cfg, counts, kernels)
    dname = dominant[0]
    dk = kernels[dname]
    roofline = dict(dk["roofline"])
    roofline["kernel"] = dname
    roofline["traffic"] = measured_traffic(cfg.name, dname)
    roofline["algo_bytes_per_launch"] = dk["algo_bytes"]
    roofline["avg_us"] = dk["avg_us"]
    if side:
        roofline["cus"] = dk.get("cus")
        roofline["side_by_side"] = side

    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "d_model": cfg.d_model,
                   "d_hidden": cfg.d_hidden, "n_experts": n, "k": k,
                   "gate": gate_text(cfg),
                   "experts": {0: "fp32 ", 1: "bf16 ", 2: "FP8 E4M3 weights, bf16 activations, "}[
                       cfg.expert_dtype]
                   + ("SwiGLU" if cfg.act == 1 else "ReLU") + " FFN, fp32 accumulate"
                   + (f", shared expert h={cfg.d_hidden_shared}" if cfg.d_hidden_shared else ""),
                   "rows": rows, "nonempty_experts": nonempty, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "side_by_side": side,
        "kernels": kernels,
        "timing": {"value_basis": "K back-to-back steps, host clock around the synchronised "
                                  "loop (the next step may find data of the previous one in "
                                  "the 256 MB Infinity Cache); cold_events flushes it first",
                   "mode": mode, "eager_us_per_step": eager_elapsed / args.steps * 1e6,
                   "eager_with_events_us_per_step": prof_elapsed / args.steps * 1e6,
                   "graph_us_per_step": (graph_elapsed / args.steps * 1e6) if graph else None,
                   "warm_events": warm, "cold_events": cold},
        "peaks_measured": peaks,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle on a sample of the first tokens")
        yh = y.cpu().double().numpy()
        ih = diag["topk_idx"].cpu().numpy()
        base, check = cpu_baseline(cfg, inp, yh, ih, args.cpu_sample_tokens, args.cpu_seconds)
        result["cpu_baseline"] = base
        result["check"] = check
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def bench_backward(args, cfg, train=False):
    """moe_backward (train: moe_forward_train + moe_backward_saved) timed
    like the forward (eager launches; per-kernel events in a second pass),
    one JSON line."""
    import sparsely_gated_mixture_amd as moe
    from sparsely_gated_mixture_amd.workloads import make_grad_inputs, make_inputs
    what = "training step" if train else "backward"
    log(f"[bench] {what}, workload {cfg.name}: T={cfg.T} d={cfg.d_model} h={cfg.d_hidden} "
        f"n={cfg.n_experts} k={cfg.k}")
    inp = make_inputs(cfg, device="cuda")
    dy, dl = make_grad_inputs(cfg, device="cuda")
    torch.cuda.synchronize()
    layer = moe.MoELayer(cfg, inp)
    T, n, k = cfg.T, cfg.n_experts, cfg.k

    y = torch.empty((T, cfg.d_model), dtype=torch.float32, device="cuda")
    losses = torch.empty(moe.N_LOSSES, dtype=torch.float32, device="cuda")
    x, noise, noise2 = inp["x"], inp.get("noise"), inp.get("noise2")

    def step():
        if train:
            layer.forward_train(x, noise, noise2, y=y, losses=losses)
        return layer.backward(x, dy, dl, noise, noise2, saved=train)

    for _ in range(args.warmup):
        grads = step()
    torch.cuda.synchronize()
    # gradient buffers allocated once, reused by the timed steps
    g = moe.make_grads(**grads)

    def eager_step():
        if train:
            moe.moe_forward_train(layer.c, layer.w, x, noise, noise2, y, losses, layer.ws_bwd)
            moe.moe_backward_saved(layer.c, layer.w, x, noise, noise2, dy, dl, g, layer.ws_bwd)
        else:
            moe.moe_backward(layer.c, layer.w, x, noise, noise2, dy, dl, g, layer.ws_bwd)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    moe.moe_profile_enable(True)
    for _ in range(args.steps):
        eager_step()
    torch.cuda.synchronize()
    moe.moe_profile_enable(False)
    moe.moe_profile_collect()
    elapsed = timed(eager_step)
    log(f"[bench] {what} eager: {elapsed / args.steps * 1e6:.1f} us/step, "
        f"{T * args.steps / elapsed / 1e6:.2f} M tokens/s")
    moe.moe_profile_enable(True)
    prof_elapsed = timed(eager_step)
    moe.moe_profile_enable(False)
    nk = moe.moe_profile_collect()
    stats = [moe.moe_profile_entry(i) for i in range(nk)]

    i32 = dict(dtype=torch.int32, device="cuda")
    diag = {"topk_idx": torch.empty((T, k), **i32), "counts": torch.empty(n, **i32)}
    layer.forward(inp["x"], inp.get("noise"), inp.get("noise2"), diag=diag)
    torch.cuda.synchronize()
    counts = diag["counts"].cpu().numpy()
    rows = int(counts.sum())
    nonempty = int((counts > 0).sum())
    kernels, dominant = {}, None
    for name, total_ms, launches in stats:
        avg_s = total_ms / launches / 1e3
        b, f, dt = bwd_kernel_work(name, cfg, rows, nonempty, T)
        entry = {"avg_us": avg_s * 1e6, "launches_per_step": launches / args.steps}
        if b:
            rl, gbs, tfs = roofline_entry(b, f, dt, avg_s)
            entry.update({"algo_bytes": b, "GB_s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS})
            if f:
                entry.update({"flops": f, "TFLOP_s": tfs, "mfma_frac": tfs / PEAK_TFLOPS[dt]})
            entry["roofline"] = rl
        kernels[name] = entry
        if b and (dominant is None or total_ms > dominant[1]):
            dominant = (name, total_ms)
    for name, e in sorted(kernels.items(),
                          key=lambda kv: -kv[1]["avg_us"] * kv[1]["launches_per_step"]):
        log(f"[bench]   {name:24s} {e['avg_us']:9.1f} us x{e['launches_per_step']:.0f}"
            + (f"  {e['GB_s']:8.1f} GB/s" if "GB_s" in e else "")
            + (f"  {e['TFLOP_s']:7.1f} TFLOP/s" if "TFLOP_s" in e else ""))
    dname = dominant[0]
    roofline = dict(kernels[dname]["roofline"])
    roofline.update(kernel=dname, traffic=measured_traffic(
                        cfg.name + ("_train" if train else "_bwd"), dname),
                    algo_bytes_per_launch=kernels[dname]["algo_bytes"],
                    avg_us=kernels[dname]["avg_us"])
    metric = ("MoE-layer training step (forward + all gradients) tokens/sec at 1 GPU" if train
              else "MoE-layer backward (forward recompute + all gradients) tokens/sec at 1 GPU")
    result = {
        "metric": metric,
        "value": T * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + (" training step" if train else " backward"), "T": T,
                   "d_model": cfg.d_model,
                   "d_hidden": cfg.d_hidden, "n_experts": n, "k": k, "gate": gate_text(cfg),
                   "gradients": "fp32; expert products bf16 MFMA with fp32 accumulation",
                   "rows": rows, "nonempty_experts": nonempty, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kernels": kernels,
        "timing": {"mode": "eager launches",
                   "eager_with_events_us_per_step": prof_elapsed / args.steps * 1e6},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_backward(cfg, inp, dy, dl, args.cpu_sample_tokens,
                                                       args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def cpu_baseline_backward(cfg, inp, dy, dl, sample_tokens, seconds):
    """The oracle's backward (its forward recompute included) on the first
    tokens of the batch, repeated for about `seconds`."""
    import oracle
    from sparsely_gated_mixture_amd.workloads import to_numpy64
    wbytes = sum(v.numel() * 8 for key, v in inp.items()
                 if v is not None and key in ("w1", "w3", "w2"))
    if wbytes > (16 << 30):
        return {"value": None, "unit": "tokens/s", "cores": None, "kind": "oracle",
                "sample": f"not run: the oracle's backward holds every expert weight in "
                          f"float64 ({wbytes / 2**30:.0f} GiB) on the host"}
    S = min(sample_tokens or 8192, cfg.T)
    h = {k: to_numpy64(v) for k, v in inp.items() if v is not None}
    x = h["x"][:S]
    noise = h["noise"][:S] if "noise" in h else None
    dyh = to_numpy64(dy)[:S]
    dlh = to_numpy64(dl)
    oracle.lib()
    reps, dt = 0, 0.0
    bf16 = cfg.expert_dtype != 0
    while reps == 0 or dt < seconds:
        t0 = time.perf_counter()
        if cfg.hierarchical:
            oracle.backward_hier(x, h["w_gate"], h.get("w_noise"), noise, cfg.k_groups,
                                 h["w_gate2"], h.get("w_noise2"),
                                 h["noise2"][:S] if "noise2" in h else None, cfg.k2, h["w1"],
                                 h["w2"], dyh, dlh, b1=h.get("b1"), b2=h.get("b2"), bf16=bf16,
                                 w_importance=cfg.w_importance, w_load=cfg.w_load,
                                 alpha=cfg.alpha_switch, w_z=cfg.w_z, w_entropy=cfg.w_entropy)
        else:
            oracle.backward(x, h["w_gate"], cfg.k, h["w1"], h["w2"], dyh, dlh,
                            b_gate=h.get("b_gate"), w_noise=h.get("w_noise"), noise=noise,
                            b1=h.get("b1"), w3=h.get("w3"), b2=h.get("b2"), mode=cfg.gate,
                            act=cfg.act, bf16=bf16, capacity_factor=cfg.capacity_factor,
                            w_importance=cfg.w_importance, w_load=cfg.w_load,
                            alpha=cfg.alpha_switch, w_z=cfg.w_z, w_entropy=cfg.w_entropy,
                            ws1=h.get("ws1"), ws3=h.get("ws3"), ws2=h.get("ws2"))
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": S * reps / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens of the {cfg.name} workload (forward "
                      f"recompute and every gradient in float64), {reps} runs in {dt:.2f} s"}


def report_children():
    """The run starts no process of its own (the oracle and the library are
    loaded in-process); list any child process still alive at exit on
    stderr, so a leftover would show in the log."""
    try:
        import psutil
    except ImportError:
        return
    kids = psutil.Process().children(recursive=True)
    log(f"[bench] child processes at exit: {len(kids)}"
        + "".join(f"\n[bench]   pid {k.pid}: {' '.join(k.cmdline()[:4])}" for k in kids))


if __name__ == "__main__":
    main()
    report_children()
