#!/usr/bin/env python3
"""Benchmark of the pair-interaction hot path on one MI355X.

One step = the whole path over one batch of synthetic jets at the kernel
benchmark shape of the ml4sci_cms_e2e26 README ("Results", table "ParT
Kernels": N=128 jets, P=128 slots, H=8, D=16): pair_embed (features + pair MLP
-> U, float32) then pair_bias_attention (masked softmax(QK^T/sqrt(D) + U) V).
Inputs are resident on the GPU before the timed region.  Prints ONE JSON line.

  value            = B * P^2 slot pairs per second of the whole step (K steps
                     bracketed by synchronize() and events at the two ends),
                     after >= 60 ms of untimed steps (the GPU's clocks leave
                     idle only under ~40 ms of load) and the W warmup steps
  roofline         = the pair-embed kernel (the dominant one) against the
                     float32 MFMA peak, algorithmic flops = unique real pairs
                     n(n+1)/2 per jet x 17,920 flop, over its warm median
                     duration (HIP events on the launch stream)
  attention_roofline, workloads.*.rooflines
                   = every other kernel of every workload, each with warm and
                     cold (L2 and MALL evicted by a 512 MiB write before each
                     rep) medians and p10/p90, and the rocprofv3 counters
                     committed under profiles/ for the same kernel source
  cpu_baseline     = the CPU oracle on the same workload (host threads); each
                     other workload carries its own oracle timing on a sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --profile WORKLOAD [--reps R]   (kernels only, for rocprofv3)
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("pairs/s fused PairEmbed+MLP and µs biased attn at B=128 P=128 H=8 D=16; "
          "%roofline")
MLP_FLOP_PER_PAIR = 2 * (4 * 64 + 64 * 64 + 64 * 64 + 64 * 8)  # 17,920
ATTN_FLOP_PER_PAIR_HEAD = 2 * 2 * 16                           # QK^T and PV at D=16
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_INT8_MFMA_TOPS = 5000.0
INT8_CALIB = os.path.join(ROOT, "tests", "golden", "int8_calibration.json")
PEAK_HBM_GBS = 8000.0
# non-packed VALU issue: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s
PEAK_VALU_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12
COLD_BYTES = 512 << 20
CSRC = os.path.join(ROOT, "pair_interaction_particle_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# kernel -> (profile summary file, sources whose sha256 it was taken on)
KERNELS = {
    "pair_embed_f32": ("pair_embed_f32_kernel_B128_P128.md",
                       ["pair_embed.hip", "pip_packed.h", "pip_device.h", "pip_mlp.h"]),
    "attention_f32": ("attention_f32_kernel_B128_P128.md",
                      ["attention.hip", "pip_attn_core.h", "pip_attn.h", "pip_device.h"]),
    "pair_embed_bf16": ("pair_embed_bf16_large_B64_P256.md",
                        ["pair_embed.hip", "pip_packed.h", "pip_device.h", "pip_mlp.h"]),
    "attention_bf16": ("attention_bf16_large_B64_P256.md",
                       ["attention.hip", "pip_attn_core.h", "pip_attn.h", "pip_device.h"]),
    "fused_f32": ("pair_embed_attention_f32_fused512_B512_P128.md",
                  ["fused.hip", "pip_mlp.h", "pip_attn.h", "pip_device.h"]),
    "block_stack_f32": ("block_stack_f32_stack8_B128_P128_C128_L8.md",
                        ["block_stack.hip", "pip_attn_core.h", "pip_attn.h", "pip_device.h"]),
    "attention_bwd_f32": ("attention_backward_f32_kernel_B128_P128.md",
                          ["attention_bwd.hip", "pip_attn.h", "pip_device.h"]),
    "pair_mlp_bwd_f32": ("pair_mlp_backward_f32_kernel_B128_P128.md",
                         ["mlp_bwd.hip", "pip_device.h", "pip_mlp.h"]),
    "pair_embed_int8": ("pair_embed_int8_kernel_B128_P128.md",
                        ["pair_embed.hip", "pip_packed.h", "pip_device.h", "pip_mlp.h"]),
    "attention_bf16_kernel": ("attention_bf16_kernel_B128_P128.md",
                              ["attention.hip", "pip_attn_core.h", "pip_attn.h",
                               "pip_device.h"]),
    "pair_embed_packed_f32": ("pair_embed_packed_f32_kernel_B128_n20-128.md",
                              ["pair_embed.hip", "pip_packed.h", "pip_device.h", "pip_mlp.h"]),
    "attention_packed_f32": ("attention_packed_f32_kernel_B128_n20-128.md",
                             ["attention.hip", "pip_attn_core.h", "pip_attn.h",
                              "pip_device.h"]),
    "equilinear_f32": ("lgatr_equilinear_f32_B128_items128_mv8_s16.md",
                       ["lgatr.hip", "pip_device.h"]),
    "geometric_product_f32": ("lgatr_geometric_product_f32_B128_items128_mv8.md",
                              ["lgatr.hip", "pip_device.h"]),
}
# L-GATr kernel shape ("Results", table "L-GATr Kernels"): B=128 jets x 128
# items, 8 multivector channels (16 components) and 16 scalar channels
LGATR_B, LGATR_ITEMS, LGATR_MV, LGATR_S = 128, 128, 8, 16


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_profile(kernel):
    """Figures from the committed rocprofv3 summary of `kernel` (the
    'key: value' lines at its end), or None when the summary is absent or was
    taken on different kernel sources."""
    fname, srcs = KERNELS[kernel]
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ", "\t")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_hash(srcs):
        return None
    out = {"file": "profiles/" + fname}
    for k, v in vals.items():
        try:
            out[k] = float(v)
        except ValueError:
            pass
    return out


def pair_counts(mask):
    import numpy as np
    n = (mask != 0).sum(axis=1).astype(np.int64)
    return int((n * (n + 1) // 2).sum()), int((n * n).sum()), n


def attention_bytes(mask, H, P, D, elt):
    """Algorithmic bytes of one attention launch: real Q/K/V rows and real U
    pairs read, the full O written (padding zeros are part of the result)."""
    import numpy as np
    n = (mask != 0).sum(axis=1).astype(np.int64)
    B = mask.shape[0]
    return int(H * (3 * n.sum() * D + (n * n).sum()) * elt + B * H * P * D * elt)


def stats(ts_ms):
    import numpy as np
    a = np.asarray(ts_ms, np.float64) * 1e3
    return {"median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "mean_us": float(a.mean()), "reps": len(a)}


CLOCK_SETTLE_MS = 60.0


def settle_clocks(step, min_ms=CLOCK_SETTLE_MS):
    """Untimed steps until at least min_ms of wall time has passed: the GPU
    needs ~40 ms of continuous load to leave its idle clocks, and a short
    --warmup would otherwise time the ramp.  Returns the number of steps."""
    import torch
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    return n


def time_steps(step, reps, warmup):
    """Wall and device time (ms) per step of `reps` back-to-back steps, after
    `warmup` untimed ones, bracketed by synchronize() on both sides and events
    at the two ends only."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    for _ in range(reps):
        step()
    e.record()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / reps, s.elapsed_time(e) / reps


def time_kernel(fn, reps, warmup, cold=None):
    """Per-launch device duration (ms) of fn() from HIP events recorded on the
    current stream (the stream the binding launches on) right around each
    launch.  A spin kernel before each rep keeps the GPU busy while the host
    enqueues the events and the launch, so the events bracket the kernel and
    not the host (they still add the event packets' own few microseconds).
    cold: a buffer of COLD_BYTES written before each rep, which evicts L2 and
    the MALL (the write itself is outside the events)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = []
    for r in range(reps):
        if cold is not None:
            cold.fill_(float(r & 7))
        torch.cuda._sleep(100000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_bursts(fn, bursts, per_burst, warmup):
    """Mean device duration (ms) per launch of `per_burst` back-to-back
    launches between two events, one figure per burst.  A spin kernel long
    enough for the host to enqueue the whole burst runs first, so the launches
    reach the GPU queued and the figure is the kernel's own back-to-back time
    (launch gaps included, no host time)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(bursts):
        torch.cuda._sleep(per_burst * 120000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(per_burst):
            fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / per_burst for a, b in evs]


def roofline(kind, work, warm, cold, prof, peak, extra=None):
    """One roofline block: work (flop or bytes per launch) over the warm
    median duration, with the cold figures and the counters beside it."""
    def rate(us):
        return work / (us * 1e-6) / (1e12 if kind == "mfma" else 1e9)
    achieved = rate(warm["median_us"])
    out = {"bound": kind, "achieved": achieved, "peak": peak,
           "unit": "TFLOP/s" if kind == "mfma" else "GB/s", "frac": achieved / peak,
           "traffic": prof.get("hbm_bytes_per_launch") if prof else None,
           "warm": warm, "cold": cold,
           "cold_frac": rate(cold["single_launch"]["median_us"]) / peak,
           "warm_single_frac": rate(cold["warm_single_launch"]["median_us"]) / peak}
    if prof:
        out["counters"] = {k: prof[k] for k in (
            "rocprof_avg_us", "mfma_busy_pct", "valu_busy_pct", "valu_issue_pct",
            "valu_lane_ops_per_launch", "mfma_mops_f16", "mfma_mops_bf16", "mfma_mops_f32",
            "hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch") if k in prof}
        # which unit the counters say is busiest: MFMA pipes, VALU issue, or
        # HBM (counted bytes over the profiled duration)
        util = {"mfma": prof.get("mfma_busy_pct", 0.0), "valu": prof.get("valu_issue_pct", 0.0)}
        if prof.get("hbm_bytes_per_launch") and prof.get("rocprof_avg_us"):
            util["hbm"] = 100.0 * prof["hbm_bytes_per_launch"] / (
                prof["rocprof_avg_us"] * 1e-6) / (PEAK_HBM_GBS * 1e9)
        out["counters"]["hbm_pct_of_peak"] = util.get("hbm")
        out["counter_bound"] = max(util, key=util.get)
        out["profile"] = prof["file"]
    if extra:
        out.update(extra)
    return out


def valu_roofline(block, prof, warm):
    """When the counters of a roofline block say VALU issue is the busiest
    unit (GELU, softmax, operand splits), whatever its matrix-core or HBM
    fraction: the profile's issued VALU lane-ops per launch over the warm
    median, against the non-packed VALU issue peak.  None otherwise."""
    if not prof or block.get("counter_bound") != "valu" or \
            "valu_lane_ops_per_launch" not in prof:
        return None
    lane_rate = prof["valu_lane_ops_per_launch"] / (warm["median_us"] * 1e-6) / 1e12
    return {"bound": "alu", "achieved": lane_rate, "peak": PEAK_VALU_TLANEOPS,
            "unit": "T lane-ops/s (issued)", "frac": lane_rate / PEAK_VALU_TLANEOPS}


def to_dev(x, dtype=None):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t if dtype is None else t.to(dtype)


# ---------------------------------------------------------------- workloads
def setup(pip, synth, name):
    """Device inputs of a workload and its kernels as callables, in step order."""
    import numpy as np
    import torch
    if name == "lgatr":
        return setup_lgatr(pip, synth)
    d = synth.make_workload("kernel" if name in ("packed", "backward", "int8") else name)
    B, P = d["mask"].shape
    mask = to_dev(d["mask"])
    mlp = pip.PairMLP(d["mlp"])
    k = {"d": d, "mlp": mlp}
    if name in ("kernel", "large_bf16"):
        bf = name == "large_bf16"
        tdt = torch.bfloat16 if bf else torch.float32
        p4 = to_dev(d["p4"])
        q, kk, v = (to_dev(d[x], tdt) for x in ("q", "k", "v"))
        U = torch.empty((B, 8, P, P), device="cuda", dtype=tdt)
        O = torch.empty_like(q)
        dt = "bf16" if bf else "f32"
        k["fns"] = [("pair_embed_" + dt, lambda: pip.pair_embed(p4, mask, mlp, dt, out=U)),
                    ("attention_" + dt, lambda: pip.pair_bias_attention(q, kk, v, U, mask,
                                                                        out=O))]
    elif name == "fused512":
        p4 = to_dev(d["p4"])
        q, kk, v = (to_dev(d[x]) for x in ("q", "k", "v"))
        O = torch.empty_like(q)
        k["fns"] = [("fused_f32", lambda: pip.pair_embed_attention(p4, mask, mlp, q, kk, v,
                                                                   out=O))]
    elif name == "packed":
        # the kernel workload's jets packed back to back (no padding)
        m = d["mask"]
        cu = to_dev(synth.cu_seqlens(m))
        p4 = to_dev(synth.pack_rows(d["p4"], m))
        q, kk, v = (to_dev(synth.pack_heads(d[x], m)) for x in ("q", "k", "v"))
        U, uoff = pip.pair_embed_packed(p4, cu, mlp)
        O = torch.empty_like(q)
        mx = int(d["n"].max())
        k["fns"] = [("pair_embed_packed_f32",
                     lambda: pip.pair_embed_packed(p4, cu, mlp, u_offsets=uoff, max_n=mx, out=U)),
                    ("attention_packed_f32",
                     lambda: pip.pair_bias_attention_packed(q, kk, v, U, cu, uoff, max_n=mx,
                                                            out=O))]
    elif name == "int8":
        # the kernel workload through the int8 MLP (U bf16) and the bf16
        # attention; activation quantisation from the committed calibration
        c = json.load(open(INT8_CALIB))["kernel"]
        p4 = to_dev(d["p4"])
        q, kk, v = (to_dev(synth.bf16_round(d[x]), torch.bfloat16) for x in ("q", "k", "v"))
        U = torch.empty((B, 8, P, P), device="cuda", dtype=torch.bfloat16)
        O = torch.empty_like(q)
        S, Z = c["act_scale"], c["act_zero"]
        k["fns"] = [("pair_embed_int8", lambda: pip.pair_embed_int8(p4, mask, mlp, S, Z, out=U)),
                    ("attention_bf16_kernel",
                     lambda: pip.pair_bias_attention(q, kk, v, U, mask, out=O))]
    elif name == "backward":
        # the kernel workload's backward: dO -> dQ, dK, dV, dU -> MLP gradient
        p4 = to_dev(d["p4"])
        q, kk, v = (to_dev(d[x]) for x in ("q", "k", "v"))
        U = pip.pair_embed(p4, mask, mlp)
        dO = to_dev(np.random.default_rng(7).normal(0, 1, size=d["q"].shape).astype("float32"))
        dq, dk, dv, du = pip.pair_bias_attention_backward(q, kk, v, U, mask, dO)
        ws = torch.empty(pip.lib().pip_pair_mlp_backward_workspace_bytes(B, P) // 4,
                         device="cuda")
        k["fns"] = [("attention_bwd_f32",
                     lambda: pip.pair_bias_attention_backward(q, kk, v, U, mask, dO)),
                    ("pair_mlp_bwd_f32",
                     lambda: pip.pair_mlp_backward(p4, mask, mlp, du, workspace=ws))]
    elif name == "stack8":
        U = pip.pair_embed(to_dev(d["p4"]), mask, mlp)
        X = to_dev(d["x0"])
        w = [to_dev(d[x]) for x in ("wq", "wk", "wv", "wo")]
        ws = torch.empty(pip.block_stack_workspace_bytes(B, P, 128, 8) // 4, device="cuda")
        # X is updated in place; re-applying the stack to the running X does
        # the same work every time (the stack has no data-dependent work)
        k["fns"] = [("block_stack_f32", lambda: pip.block_stack(X, *w, U, mask, workspace=ws))]
    return k


def setup_lgatr(pip, synth):
    """The L-GATr kernels at their table shape: the equivariant linear layer
    (8 -> 8 multivector, 16 -> 16 scalar channels) on B x items tokens and
    the geometric product of two (B, items, 8) multivector tensors."""
    import numpy as np
    import torch
    rng = np.random.default_rng(2024)
    n = LGATR_B * LGATR_ITEMS
    p = synth.equilinear_params(LGATR_MV, LGATR_MV, LGATR_S, LGATR_S, rng)
    x_mv = synth.multivectors((n, LGATR_MV), rng)
    x_s = rng.normal(size=(n, LGATR_S)).astype(np.float32)
    y = synth.multivectors((n, LGATR_MV), rng)
    layer = pip.EquiLinear(in_s=LGATR_S, out_s=LGATR_S, **p)
    gx, gs, gy = to_dev(x_mv), to_dev(x_s), to_dev(y)
    o_mv = torch.empty_like(gx)
    o_s = torch.empty_like(gs)
    z = torch.empty_like(gx)
    d = {"lgatr": True, "n": n, "params": p, "x_mv": x_mv, "x_s": x_s, "y": y}
    return {"d": d, "layer": layer,
            "fns": [("equilinear_f32", lambda: layer(gx, gs, y_mv=o_mv, y_s=o_s)),
                    ("geometric_product_f32", lambda: pip.geometric_product(gx, gy, out=z))]}


def work_of(kernel, d):
    """(roofline kind, algorithmic work per launch, peak) of one kernel."""
    if kernel == "equilinear_f32":
        # x_mv, x_s read and y_mv, y_s written once; W_eff's nonzero blocks
        # (8 blocks of 16 x 16, plus the scalar rows and columns) read once
        n = d["n"]
        io = n * 2 * (LGATR_MV * 16 + LGATR_S) * 4
        w = (8 * (2 * LGATR_MV) ** 2 + 2 * LGATR_MV * LGATR_S + LGATR_S * (2 * LGATR_MV + LGATR_S)
             + LGATR_MV + LGATR_S) * 4
        return "hbm", io + w, PEAK_HBM_GBS
    if kernel == "geometric_product_f32":
        return "hbm", d["n"] * LGATR_MV * 3 * 16 * 4, PEAK_HBM_GBS
    mask = d["mask"]
    B, P = mask.shape
    uniq, ordered, n = pair_counts(mask)
    if kernel == "pair_embed_f32":
        return "mfma", uniq * MLP_FLOP_PER_PAIR, PEAK_FP32_MFMA_TFLOPS
    if kernel == "pair_embed_bf16":
        return "mfma", uniq * MLP_FLOP_PER_PAIR, PEAK_BF16_MFMA_TFLOPS
    if kernel == "attention_f32":
        return "hbm", attention_bytes(mask, 8, P, 16, 4), PEAK_HBM_GBS
    if kernel == "attention_bf16":
        return "hbm", attention_bytes(mask, 8, P, 16, 2), PEAK_HBM_GBS
    if kernel == "pair_embed_int8":
        # int8 MFMA operations of layers 2, 3, 4 per unique real pair
        return "mfma", uniq * 2 * (64 * 64 * 2 + 64 * 8), PEAK_INT8_MFMA_TOPS
    if kernel == "attention_bf16_kernel":
        return "hbm", attention_bytes(mask, 8, P, 16, 2), PEAK_HBM_GBS
    if kernel == "attention_bwd_f32":
        # reads: real Q, K, V, dO rows and real U pairs; writes: dQ, dK, dV
        # and dU in full (padding zeros are part of the result)
        return ("hbm", int(8 * (4 * n.sum() * 16 + (n * n).sum()) * 4
                           + B * 8 * P * (3 * 16 + P) * 4), PEAK_HBM_GBS)
    if kernel == "pair_mlp_bwd_f32":
        # per unique real pair: the forward (17,920 flop), the backward chain
        # 2 (8*64 + 2*64*64) and the weight gradients 2 (64*4 + 2*64*64 + 8*64)
        per = MLP_FLOP_PER_PAIR + 2 * (8 * 64 + 2 * 64 * 64) + 2 * (64 * 4 + 2 * 64 * 64 + 8 * 64)
        return "mfma", uniq * per, PEAK_FP32_MFMA_TFLOPS
    if kernel == "pair_embed_packed_f32":
        return "mfma", uniq * MLP_FLOP_PER_PAIR, PEAK_FP32_MFMA_TFLOPS
    if kernel == "attention_packed_f32":
        # real Q, K, V rows and real U pairs read, real O rows written
        return "hbm", int(8 * (4 * n.sum() * 16 + (n * n).sum()) * 4), PEAK_HBM_GBS
    if kernel == "fused_f32":
        return ("mfma", uniq * MLP_FLOP_PER_PAIR + ordered * 8 * ATTN_FLOP_PER_PAIR_HEAD,
                PEAK_FP32_MFMA_TFLOPS)
    if kernel == "block_stack_f32":
        nr = int((mask != 0).sum())
        return ("mfma", 8 * (nr * 128 * 128 * 2 * 4 + ordered * 8 * ATTN_FLOP_PER_PAIR_HEAD),
                PEAK_FP32_MFMA_TFLOPS)
    raise KeyError(kernel)


def measure(k, reps, warmup, cold):
    """Warm and cold duration statistics and roofline blocks of each kernel."""
    out = {}
    for name, fn in k["fns"]:
        # warm: back-to-back bursts (the roofline figure); cold: single
        # launches after a 512 MiB write, next to warm single launches timed
        # the same way (both carry the events' own overhead)
        warm = stats(time_bursts(fn, max(5, reps // 10), 20, warmup))
        cld = {"single_launch": stats(time_kernel(fn, max(10, reps // 2), 2, cold=cold)),
               "warm_single_launch": stats(time_kernel(fn, max(10, reps // 2), 2))}
        kind, work, peak = work_of(name, k["d"])
        prof = read_profile(name)
        extra = {"algorithmic_%s_per_launch" % ("flop" if kind == "mfma" else "bytes"): work}
        out[name] = roofline(kind, work, warm, cld, prof, peak, extra)
        vb = valu_roofline(out[name], prof, warm)
        if vb:
            out[name]["valu"] = vb
        if name == "pair_embed_int8":
            out[name]["unit"] = "TOP/s"
    return out


# ---------------------------------------------------------------- CPU oracle
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(d, budget_s):
    """The oracle (fp64, OpenMP over jets) on the whole kernel workload,
    repeated until about budget_s seconds of wall time have passed."""
    import oracle
    B, P = d["mask"].shape
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 1000:
        t = time.perf_counter()
        U = oracle.pair_embed(d["p4"], d["mask"], d["mlp"])
        oracle.attention(d["q"], d["k"], d["v"], U, d["mask"])
        t_total += time.perf_counter() - t
        reps += 1
    return {"value": B * P * P * reps / t_total, "unit": "slot-pairs/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "whole kernel workload (B=128 jets, P=128) run %d time(s): float64 pair "
                      "embed + attention, %.1f s wall" % (reps, t_total)}


def cpu_sample(name, d, jets):
    """The oracle on the first `jets` jets of another workload, once; the
    rate is scaled to the whole workload."""
    import oracle
    if name == "lgatr":
        p = d["params"]
        items = jets * LGATR_ITEMS
        t = time.perf_counter()
        oracle.equilinear(d["x_mv"][:items], d["x_s"][:items], **p)
        oracle.geometric_product(d["x_mv"][:items], d["y"][:items])
        dt = time.perf_counter() - t
        return {"value": items / dt, "unit": "items/s (equilinear + geometric product)",
                "us_per_workload_call": dt * 1e6 * LGATR_B / jets,
                "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
                "sample": "first %d of %d jets (%d items): float64 equivariant linear layer "
                          "8->8 mv, 16->16 s, then the geometric product of 8 channel pairs, "
                          "%.2f s wall" % (jets, LGATR_B, items, dt)}
    B, P = d["mask"].shape
    s = slice(0, jets)
    t = time.perf_counter()
    if name == "fused512":
        oracle.pair_embed_attention(d["p4"][s], d["mask"][s], d["mlp"], d["q"][s], d["k"][s],
                                    d["v"][s])
        what = "pair embed + attention"
    elif name == "large_bf16":
        U = oracle.pair_embed(d["p4"][s], d["mask"][s], d["mlp"])
        oracle.attention(d["q"][s], d["k"][s], d["v"][s], U, d["mask"][s])
        what = "pair embed + attention (bf16-rounded inputs, float64 arithmetic)"
    else:
        U = oracle.pair_embed(d["p4"][s], d["mask"][s], d["mlp"]).astype("float32")
        oracle.block_stack(d["x0"][s], d["wq"], d["wk"], d["wv"], d["wo"], U, d["mask"][s])
        what = "8-layer block stack (U precomputed)"
    dt = time.perf_counter() - t
    return {"value": jets * P * P / dt, "unit": "slot-pairs/s",
            "us_per_workload_call": dt * 1e6 * B / jets, "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "first %d of %d jets, float64 %s, %.2f s wall" % (jets, B, what, dt)}


SHAPES = {
    "int8": "kernel workload, int8 MLP: B=128 P=128 n~U{20..128} H=8 D=16; int8 inputs to "
            "layers 2-4 (calibrated zero points), U bf16, bf16 attention",
    "backward": "kernel workload backward: B=128 P=128 n~U{20..128} H=8 D=16 fp32; "
                "attention dO -> dQ, dK, dV, dU, then pair-MLP parameter gradient",
    "packed": "kernel workload packed: B=128 jets back to back, n~U{20..128} (N=%d), H=8, "
              "D=16, fp32",
    "large_bf16": "B=64 P=256 n~U{60..256} H=8 D=16 bf16",
    "fused512": "B=512 P=128 n~U{20..128} H=8 D=16 fp32, 5% massive",
    "stack8": "B=128 P=128 C=128 H=8 D=16 L=8 fp32",
    "lgatr": "L-GATr kernels: B=128 x items=128, equivariant linear 8->8 multivectors + "
             "16->16 scalars, geometric product of (128, 128, 8) multivector pairs, fp32",
}
CPU_JETS = {"large_bf16": 16, "fused512": 128, "stack8": 32, "lgatr": 128}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU needs ~40 ms of continuous load to reach its steady clocks
    # (pair_embed runs ~75 us per call in the first milliseconds, ~64 us
    # after); 500 warmup steps are ~45 ms.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--reps", type=int, default=100,
                    help="per-kernel timed reps (warm; cold takes half)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--profile", default=None, metavar="WORKLOAD",
                    help="only run WORKLOAD's kernels (--warmup untimed, then --reps) and "
                         "exit: the command rocprofv3 wraps for profiles/")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (use --gpus 1): the path shards over jets with "
              "no exchange, and only the single-MI355X kernel is implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    from pair_interaction_particle_amd import binding as pip
    from pair_interaction_particle_amd import synth

    torch.cuda.set_device(0)
    if args.profile:
        k = setup(pip, synth, args.profile)
        for _ in range(args.warmup):
            for _, fn in k["fns"]:
                fn()
        torch.cuda.synchronize()
        for _ in range(args.reps):
            for _, fn in k["fns"]:
                fn()
        torch.cuda.synchronize()
        print(json.dumps({"profile": args.profile, "reps": args.reps,
                          "kernels": [n for n, _ in k["fns"]]}))
        return

    k = setup(pip, synth, "kernel")
    d = k["d"]
    B, P = d["mask"].shape
    H, D = 8, 16
    (_, embed), (_, attn) = k["fns"]
    # clock settling (untimed), then the W warmup steps, then the timed
    # region: K steps bracketed only at the ends
    settle = settle_clocks(lambda: (embed(), attn()))
    ms_per_step, gpu_ms_per_step = time_steps(lambda: (embed(), attn()), args.steps,
                                              args.warmup)
    cold = torch.empty(COLD_BYTES // 4, device="cuda")
    per = measure(k, args.reps, 20, cold)
    slot_pairs = B * P * P
    uniq, ordered, n = pair_counts(d["mask"])
    pe, at = per["pair_embed_f32"], per["attention_f32"]
    res = {
        "metric": METRIC,
        "value": slot_pairs / (ms_per_step * 1e-3),
        "unit": "slot-pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": gpu_ms_per_step,
        "clock_settle": {"steps": settle, "min_ms": CLOCK_SETTLE_MS,
                         "note": "untimed steps before the warmup, so that a short --warmup "
                                 "does not time the GPU's clock ramp"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "kernel: B=128 jets, P=128 slots, real n~U{20..128}, H=8, "
                               "D=16, fp32; step = pair_embed + pair_bias_attention",
                   "B": B, "P": P, "H": H, "D": D, "global_batch": B, "seq_len": P,
                   "parallelism": "single GPU"},
        "roofline": dict(pe, kernel="pair_embed_kernel<kMlpF16x2> (fp32 path)",
                         unique_real_pairs=uniq),
        "pair_embed_us": pe["warm"]["median_us"],
        "pair_embed_slot_pairs_per_s": slot_pairs / (pe["warm"]["median_us"] * 1e-6),
        "attention_us": at["warm"]["median_us"],
        "attention_roofline": dict(at, kernel="attention_kernel<f32>"),
        "real_ordered_pairs": ordered,
    }
    if not args.no_extra:
        res["workloads"] = {}
        for name in ("packed", "int8", "backward", "lgatr", "fused512", "large_bf16", "stack8"):
            kw = setup(pip, synth, name)
            shape = SHAPES[name] % int(kw["d"]["n"].sum()) if name == "packed" else SHAPES[name]
            res["workloads"][name] = {"shape": shape,
                                      "rooflines": measure(kw, args.reps, 20, cold)}
            if not args.no_cpu_baseline and name in CPU_JETS:
                res["workloads"][name]["cpu_oracle"] = cpu_sample(name, kw["d"],
                                                                  CPU_JETS[name])
            del kw
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(d, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
