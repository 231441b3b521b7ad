#!/usr/bin/env python3
"""Benchmark of the MI355X attention forward (one JSON line on stdout).

A step is one attn_fwd call on the headline workload -- causal attention,
batch 4, 32 heads, L 4096, head dim 128, bf16 -- with Q, K, V already resident
in HBM.  `value` is its throughput in algorithmic TFLOP/s (4*D FLOPs per visible
(query, key) pair).  The same run also times the block-diagonal workload at
scale (batch 8, 32 heads, N 16384, D 128, fp16, block 64 and 128) in GB/s of
algorithmic traffic (Q, K, V read once, O written once) against the HBM peak,
and the two remaining workloads for context.

The oracle leg (skipped with --no-cpu-baseline) runs the fp64 numpy oracle on the
host cores: `cpu_baseline` times it on a bounded sample of the headline workload,
`cpu_baseline_by_workload` on a bounded sample of every workload, and
`max_abs_err` compares sampled output rows of every timed workload with it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
HEADLINE = "causal_b4_h32_l4096_d128_bf16"
KERNEL_SOURCES = [os.path.join(ROOT, "attention_forward_06_amd", "csrc", f)
                  for f in ("attn_kernel.h", "attn_kernel_rows64.h", "attn_fwd.hip", "attn_fwd_d256.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU clock settles over the first ~50 back-to-back launches of the headline workload
    # (power management); 100 untimed launches put the timed ones in the steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (e.g. under a profiler)")
    ap.add_argument("--only", default=None, help="time only this workload name")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle sample of the headline workload")
    ap.add_argument("--cpu-seconds-other", type=float, default=2.5,
                    help="target wall time of the oracle sample of each other workload")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured MFMA / HBM ceilings (e.g. under a counter profiler)")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="no GPU work: turn the rocprofv3 CSV output of the profiling passes under "
                         "DIR (prof_trace, pmc_fetch, pmc_write, pmc_mfma, pmc_lds; optionally the stall passes) into the "
                         "summaries in profiles/")
    return ap.parse_args()


def source_digest():
    """sha256 of the kernel sources with comments and whitespace removed: the counters stay valid
    across comment-only edits and are dropped on any code change."""
    import re
    text = ""
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text += f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def visible_pairs(mode, L, block_size):
    """(query, key) pairs that take part in the softmax, per head (the counting rule of the
    measurement: 4 * D FLOPs per visible pair)."""
    if mode == "none":
        return L * L
    if mode == "causal":
        return L * (L + 1) // 2
    return L * block_size


def load_traffic(name):
    """HBM bytes per launch measured by counters, if they were taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_digest():
        return None
    w = t.get("workloads", {}).get(name)
    if not w:
        return None
    return w.get("hbm_bytes_per_launch")


def parity_rows(L, seed=7, n_edge=64, n_rand=64):
    """Output rows compared with the oracle: the first and last n_edge rows and n_rand seeded
    random ones."""
    import numpy as np
    rng = np.random.default_rng(seed)
    rows = set(range(min(n_edge, L))) | set(range(max(0, L - n_edge), L))
    rows |= set(int(r) for r in rng.integers(0, L, size=n_rand))
    return np.array(sorted(rows), dtype=np.int64)


def time_workload(name, steps, warmup):
    import torch
    from attention_forward_06_amd import binding
    from attention_forward_06_amd.inputs import WORKLOADS, make_qkv, default_scale

    w = WORKLOADS[name]
    B, H, L, D = w["B"], w["H"], w["L"], w["D"]
    q, k, v = make_qkv(B, H, L, D, w["dtype"], seed=42, device="cuda")
    o = torch.empty_like(q)
    scale = default_scale(D)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, L, D, scale, w["mode"],
            w["block_size"], w["dtype"], sptr)
    for _ in range(warmup):
        st = binding.attn_fwd_raw(*args)
        if st != 0:
            raise RuntimeError(f"{name}: {binding.status_str(st)}")
    torch.cuda.synchronize()
    # the timed region: one event before the first launch and one after the last, on the stream
    # the kernel runs on (events between launches would add gaps to the short kernels)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        binding.attn_fwd_raw(*args)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    # then, untimed, the same number of launches each between its own two events: how the launch
    # time moves from launch to launch (the clock under sustained load)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        binding.attn_fwd_raw(*args)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    flops = 4 * D * visible_pairs(w["mode"], L, w["block_size"]) * B * H
    vb = 1 if w["dtype"].endswith("_v_e5m2") else 2
    nbytes = B * H * L * D * (2 + 2 + vb + 2)
    ms = total_ms / steps
    # rows kept for the oracle comparison: the first and the last (batch, head)
    rows = parity_rows(L)
    rt = torch.as_tensor(rows, device="cuda")
    sample = dict(rows=rows, heads=[(0, 0), (B - 1, H - 1)],
                  q=[q[b, h].index_select(0, rt).float().cpu() for b, h in ((0, 0), (B - 1, H - 1))],
                  k=[k[b, h].float().cpu() for b, h in ((0, 0), (B - 1, H - 1))],
                  v=[v[b, h].float().cpu() for b, h in ((0, 0), (B - 1, H - 1))],
                  o=[o[b, h].index_select(0, rt).float().cpu() for b, h in ((0, 0), (B - 1, H - 1))])
    del q, k, v, o, rt
    torch.cuda.empty_cache()
    srt = sorted(per)
    return dict(name=name, ms=ms, wall_s=wall, min_ms=srt[0], median_ms=srt[len(srt) // 2],
                per_launch_ms=per, flops=flops, bytes=nbytes, tflops=flops / (ms * 1e-3) / 1e12,
                gbs=nbytes / (ms * 1e-3) / 1e9, mode=w["mode"], dtype=w["dtype"], sample=sample,
                shape=dict(B=B, H=H, L=L, D=D, block_size=w["block_size"]))


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def measured_ceilings():
    """What the chip sustains on the two bounding resources, measured after the timed workloads
    (so they cannot disturb them): back-to-back bf16 MFMAs with random operands, and HBM streaming
    in the block-diagonal mix (three arrays read, one written)."""
    from attention_forward_06_amd import binding
    mfma = binding.ceiling_mfma_bf16(warmup=2000, launches=4000)
    hbm = binding.ceiling_hbm_3r1w(warmup=5, launches=40, bytes_per_array=512 << 20)
    return {"mfma_bf16_TFLOP_per_s": round(mfma, 1), "hbm_3read_1write_GB_per_s": round(hbm, 1),
            "how": "mfma: v_mfma_f32_32x32x16_bf16 back to back, 2 waves per SIMD on every CU, "
                   "random operands changing every MFMA, 4000 launches after 2000 warm-up; hbm: "
                   "d = a ^ b ^ c over 512 MiB arrays, 16-byte non-temporal accesses, 40 launches "
                   "after 5 warm-up"}


# Tolerances of the comparison with the oracle (max abs error, by V's type).
TOLERANCE = {"f16": 2e-3, "bf16": 1e-2, "bf16_v_e5m2": 5e-2, "f16_v_e5m2": 5e-2}


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


def parity(r):
    """Max |GPU - oracle| over the sampled rows of the first and last (batch, head), against the
    plain definition (with P rounded to e5m2 where V is e5m2, the unnormalised weights in the
    final-max frame); for e5m2 V the error against exact P is reported too."""
    import numpy as np
    import oracle
    from attention_forward_06_amd.inputs import default_scale
    smp, sh = r["sample"], r["shape"]
    L, D = sh["L"], sh["D"]
    fp8 = r["dtype"].endswith("_v_e5m2")
    err, err_exact = 0.0, 0.0
    for q, k, v, o in zip(smp["q"], smp["k"], smp["v"], smp["o"]):
        # the sampled query rows sit at their own positions: embed them in a full-size Q
        qf = np.zeros((1, 1, L, D))
        qf[0, 0, smp["rows"]] = q.double().numpy()
        kf, vf = k.double().numpy()[None, None], v.double().numpy()[None, None]
        ref = oracle.attn_ref(qf, kf, vf, r["mode"], default_scale(D), sh["block_size"],
                              rows=smp["rows"], p_round="e5m2" if fp8 else None)[0, 0]
        err = max(err, float(np.abs(o.double().numpy() - ref).max()))
        if fp8:
            ex = oracle.attn_ref(qf, kf, vf, r["mode"], default_scale(D), sh["block_size"],
                                 rows=smp["rows"])[0, 0]
            err_exact = max(err_exact, float(np.abs(o.double().numpy() - ex).max()))
    out = {"max_abs_err": err, "tol": TOLERANCE[r["dtype"]], "pass": err <= TOLERANCE[r["dtype"]],
           "compared": f"{len(smp['rows'])} rows x 2 heads (first/last 64 + 64 seeded random rows "
                       f"of (b,h) = {smp['heads'][0]} and {smp['heads'][1]})",
           "oracle": "plain definition, fp64" + (", P rounded to e5m2 in the final-max frame" if fp8 else "")}
    if fp8:
        out["max_abs_err_exact_p"] = err_exact
    return out


def cpu_baseline_workload(name, target_s):
    """The oracle as it stands, on the host cores, on a bounded sample of one workload.

    none / causal: whole (batch, head) slices; the causal L = 32768 workload (one head is
    ~1.1e13 FLOPs) on a row subset of one head -- rows 0..1023, 1024 seeded random rows, the
    last 256 -- whose rate extrapolates to the workload by its exact visible-pair count;
    block_diag: whole heads, each diagonal block through the oracle on its own slice (the
    block-diagonal result equals attention restricted to each block, a pinned property)."""
    import numpy as np
    import oracle
    from attention_forward_06_amd.inputs import WORKLOADS, make_qkv, default_scale
    w = WORKLOADS[name]
    L, D, bs, mode = w["L"], w["D"], w["block_size"], w["mode"]
    scale = default_scale(D)
    flops, nbytes, elapsed, units = 0, 0, 0.0, 0
    extrapolated = False
    vb = 1 if w["dtype"].endswith("_v_e5m2") else 2
    while elapsed < target_s and units < w["B"] * w["H"]:
        q, k, v = make_qkv(1, 1, L, D, w["dtype"], seed=1000 + units)
        qn, kn, vn = (t.float().double().numpy() for t in (q, k, v))
        p_round = "e5m2" if vb == 1 else None
        if mode == "block_diag":
            t0 = time.perf_counter()
            for b0 in range(0, L, bs):
                sl = slice(b0, b0 + bs)
                oracle.attn_ref(qn[:, :, sl], kn[:, :, sl], vn[:, :, sl], "none", scale)
            elapsed += time.perf_counter() - t0
            flops += 4 * D * L * bs
            nbytes += L * D * (2 + 2 + vb + 2)
        elif L > 8192:
            rng = np.random.default_rng(units)
            rows = np.unique(np.concatenate([np.arange(1024), rng.integers(0, L, 1024),
                                             np.arange(L - 256, L)]))
            t0 = time.perf_counter()
            oracle.attn_ref(qn, kn, vn, mode, scale, rows=rows, p_round=p_round)
            elapsed += time.perf_counter() - t0
            flops += 4 * D * int((rows + 1).sum() if mode == "causal" else rows.size * L)
            nbytes += rows.size * D * 4 + L * D * (2 + vb)
            extrapolated = True
        else:
            t0 = time.perf_counter()
            oracle.attn_ref(qn, kn, vn, mode, scale, p_round=p_round)
            elapsed += time.perf_counter() - t0
            flops += 4 * D * visible_pairs(mode, L, bs)
            nbytes += L * D * (2 + 2 + vb + 2)
        units += 1
    unit_name = ("row subsets, each of one (batch, head)," if extrapolated
                 else "whole (batch, head) slices")
    if mode == "block_diag":
        value, unit = nbytes / elapsed / 1e9, "GB/s"
    else:
        value, unit = flops / elapsed / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": oracle_threads(), "kind": "oracle",
            "extrapolated": extrapolated,
            "sample": f"{units} {unit_name} of {name}, fp64 numpy, {elapsed:.1f} s"
                      + ("; rows 0-1023, 1024 seeded random rows, the last 256, rate over their "
                         "visible pairs (extrapolated to the workload by its visible-pair count)"
                         if extrapolated else "")
                      + f"; affinity cores {len(os.sched_getaffinity(0))}, os.cpu_count {os.cpu_count()}"}



# ---- rocprofv3 summaries ------------------------------------------------------------------------
BENCH_WORKLOADS = [HEADLINE, "blockdiag_b1_h2_n256_d128_bs64_f16", "blockdiag_b8_h32_n16384_d128_bs64_f16",
                   "blockdiag_b8_h32_n16384_d128_bs128_f16", "dense_b4_h16_l2048_d64_f16",
                   "causal_b1_h16_l32768_d256_bf16_ve5m2", "causal_b1_h16_l32768_d256_f16_ve5m2",
                   "dense_b4_h16_l2048_d32_f16", "causal_b4_h32_l4096_d16_bf16"]
PROFILE_COMMANDS = {
    "prof_trace": "rocprofv3 --kernel-trace --stats -d gpurun_out/prof_trace -o run --output-format csv "
                  "-- python3 bench.py --steps 30 --no-cpu-baseline --no-ceilings",
    "pmc_fetch": "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o run --output-format csv -- python3 "
                 "bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-ceilings --copy-calibration",
    "pmc_write": "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o run --output-format csv -- python3 "
                 "bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-ceilings --copy-calibration",
    "pmc_mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 "
                "SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE -d gpurun_out/pmc_mfma -o run --output-format csv "
                "-- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-ceilings",
    "pmc_lds": "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_MFMA "
               "SQ_WAVE_CYCLES GRBM_GUI_ACTIVE -d gpurun_out/pmc_lds -o run --output-format csv -- python3 "
               "bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-ceilings",
    "pmc_stall_a": "rocprofv3 --pmc SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
                   "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_INST_LDS "
                   "GRBM_GUI_ACTIVE -d gpurun_out/pmc_stall_a -o run --output-format csv -- python3 bench.py "
                   "--steps 2 --warmup 1 --no-cpu-baseline --no-ceilings",
    "pmc_stall_b": "rocprofv3 --pmc SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_MISC "
                   "SQ_ACTIVE_INST_VALU2 SQ_IFETCH SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_BUSY_CU_CYCLES "
                   "GRBM_GUI_ACTIVE -d gpurun_out/pmc_stall_b -o run --output-format csv -- python3 bench.py "
                   "--steps 2 --warmup 1 --no-cpu-baseline --no-ceilings",
    "pmc_icache": "rocprofv3 --pmc SQC_ICACHE_HITS SQC_ICACHE_MISSES SQC_ICACHE_MISSES_DUPLICATE SQC_ICACHE_REQ "
                  "SQC_ICACHE_INPUT_VALID_READYB SQC_ICACHE_BUSY_CYCLES SQ_INSTS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE "
                  "-d gpurun_out/pmc_icache -o run --output-format csv -- python3 bench.py --steps 2 --warmup 1 "
                  "--no-cpu-baseline --no-ceilings",
    "pmc_ldslat": "rocprofv3 --pmc LdsLatency -d gpurun_out/pmc_ldslat -o run --output-format csv -- python3 "
                  "bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-ceilings",
    "pmc_vmemlat": "rocprofv3 --pmc VmemLatency -d gpurun_out/pmc_vmemlat -o run --output-format csv -- python3 "
                   "bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-ceilings",
}
DT_CODE = {"f16": 0, "bf16": 1, "bf16_v_e5m2": 2, "f16_v_e5m2": 3}
MODE_CODE = {"none": 0, "causal": 1, "block_diag": 2}


def kernel_of(name):
    """(kernel name as rocprofv3 prints it, grid size in work-items) of a bench workload."""
    from attention_forward_06_amd.inputs import WORKLOADS
    w = WORKLOADS[name]
    if w["D"] <= 64 and w["mode"] in ("none", "causal"):
        # head dims 16-64, none and causal: 64 query rows per wave, 256 per workgroup
        kname = f"attn_fwd_rows64_kernel<{w['D']}, {DT_CODE[w['dtype']]}, {MODE_CODE[w['mode']]}, false>"
        return kname, -(-w["L"] // 256) * w["B"] * w["H"] * 256
    bn, kw = (128, w["block_size"]) if w["mode"] == "block_diag" else (64, 64)
    kname = (f"attn_fwd_kernel<{w['D']}, {DT_CODE[w['dtype']]}, {MODE_CODE[w['mode']]}, 4, {bn}, {kw}, "
             "false>")
    blocks = -(-w["L"] // 128) * w["B"] * w["H"]
    return kname, blocks * 256


def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _counters(d, counter):
    """{(kernel name, grid): [value per dispatch]} of one counter from a rocprofv3 PMC CSV."""
    out = {}
    for row in _csv(os.path.join(d, "run_counter_collection.csv")):
        if row["Counter_Name"] != counter:
            continue
        key = (row["Kernel_Name"], int(row["Grid_Size"]))
        out.setdefault(key, []).append(float(row["Counter_Value"]))
    return out


def _lookup(table, name):
    kname, grid = kernel_of(name)
    for (k, g), vals in table.items():
        if kname in k and g == grid:
            return vals
    return None


def summarize_profiles(d, out=None):
    """Write traffic.json and the markdown summaries from the rocprofv3 CSV output under d into
    out (default: profiles/ of the repository)."""
    from attention_forward_06_amd.inputs import WORKLOADS
    prof = out or os.path.join(ROOT, "profiles")
    digest = source_digest()
    # --- HBM traffic: FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by a 1 GiB copy
    fetch = _counters(os.path.join(d, "pmc_fetch"), "FETCH_SIZE")
    write = _counters(os.path.join(d, "pmc_write"), "WRITE_SIZE")
    cf = [v for (k, g), vals in fetch.items() if "copyBuffer" in k for v in vals if v > 1e5]
    cw = [v for (k, g), vals in write.items() if "copyBuffer" in k for v in vals if v > 1e5]
    gib_kib = float(1 << 20)
    f_scale = gib_kib / (sum(cf) / len(cf))
    w_scale = gib_kib / (sum(cw) / len(cw))
    traffic = {"kernel_source_sha256": digest, "fetch_scale": f_scale, "write_scale": w_scale,
               "workloads": {}}
    rows = []
    for n in BENCH_WORKLOADS:
        fv, wv = _lookup(fetch, n), _lookup(write, n)
        if not fv or not wv:
            continue
        w = WORKLOADS[n]
        vb = 1 if w["dtype"].endswith("_v_e5m2") else 2
        alg = w["B"] * w["H"] * w["L"] * w["D"] * (2 + 2 + vb + 2)
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        hbm = int(round((fk * f_scale + wk * w_scale) * 1024))
        traffic["workloads"][n] = {"hbm_bytes_per_launch": hbm, "fetch_kib": fk, "write_kib": wk,
                                   "algorithmic_bytes": alg}
        rows.append(f"| {n} | `{kernel_of(n)[0]}` | {fk:.1f} | {wk:.1f} | {hbm / 2**20:.1f} MiB | "
                    f"{alg / 2**20:.1f} MiB | {hbm / alg:.3f} |")
    with open(os.path.join(prof, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    with open(os.path.join(prof, "attn_fwd_hbm_traffic_all_workloads.md"), "w") as f:
        f.write("# HBM traffic per launch from rocprofv3 PMC counters\n\n"
                "Two runs, one counter each (repo root, on one MI355X):\n\n```\n"
                + PROFILE_COMMANDS["pmc_fetch"] + "\n" + PROFILE_COMMANDS["pmc_write"] + "\n```\n\n"
                f"Summarised by `python3 bench.py --summarize-profiles gpurun_out`. Kernel source digest "
                f"(sha256, comments and whitespace removed, as bench.source_digest): `{digest}`.\n\n"
                f"Calibration: a plain 1 GiB device copy (`--copy-calibration`) reads FETCH_SIZE = "
                f"{sum(cf) / len(cf):.1f} KiB and WRITE_SIZE = {sum(cw) / len(cw):.1f} KiB per dispatch, "
                f"against 1048576 KiB moved each way. Scale factors: fetch x{f_scale:.4f}, write "
                f"x{w_scale:.4f}. The counters sit at the L2's memory side, so a fetch the MALL serves "
                "counts too: the figure bounds HBM bytes from above.\n\n"
                "| workload | kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled HBM bytes | "
                "algorithmic bytes | ratio |\n|---|---|---|---|---|---|---|\n" + "\n".join(rows) + "\n")
    # --- kernel trace: per-kernel statistics and the averages of the timed launches
    stats = _csv(os.path.join(d, "prof_trace", "run_kernel_stats.csv"))
    trace = _csv(os.path.join(d, "prof_trace", "run_kernel_trace.csv"))
    lines = []
    for n in BENCH_WORKLOADS:
        kname, grid = kernel_of(n)
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                if kname in r["Kernel_Name"] and int(r["Grid_Size_X"]) == grid]
        if not durs:
            continue
        timed = 5 if "l32768" in n else 30
        t = durs[-timed:]
        lines.append(f"| `{kname}` | {n} | {len(durs)} | {sum(durs) / len(durs):.1f} | {min(durs):.1f} | "
                     f"{max(durs):.1f} | {sum(t) / len(t):.1f} ({len(t)} launches) |")
    others = [f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} |" for r in stats
              if "attn_fwd_kernel<" not in r["Name"] and "attn_fwd_rows64_kernel<" not in r["Name"]][:8]
    with open(os.path.join(prof, "attn_fwd_kernel_trace_all_workloads.md"), "w") as f:
        f.write("# rocprofv3 kernel-trace statistics: the attention kernels, the workloads of bench.py\n\n"
                "Command (repo root, on one MI355X):\n\n```\n" + PROFILE_COMMANDS["prof_trace"] + "\n```\n\n"
                f"Summarised by `python3 bench.py --summarize-profiles gpurun_out`; kernel source digest "
                f"`{digest}`. All calls include the untimed warm-up launches (100, or 10 for L = 32768); "
                "the last column averages only the launches bench.py times (with --steps 30: 30, or 5 for L = 32768).\n\n"
                "| kernel | workload | calls | average (us) | min (us) | max (us) | timed launches: "
                "average (us) |\n|---|---|---|---|---|---|---|\n" + "\n".join(lines) + "\n\n"
                "Other kernels of the run (input generation, copies of sampled rows):\n\n"
                "| kernel | calls | average (us) |\n|---|---|---|\n" + "\n".join(others) + "\n\n"
                "Template arguments: attn_fwd_kernel<head dim, dtype (0 f16, 1 bf16, 2 bf16 with e5m2 V, "
                "3 f16 with e5m2 V), mask (0 none, 1 causal, 2 block_diag), waves per workgroup, keys per "
                "tile, keys per wave, writes the log-normaliser>; attn_fwd_rows64_kernel<head dim, dtype, "
                "mask, writes the log-normaliser> (64 query rows per wave, 4 waves per workgroup, 64-key "
                "tiles).\n")
    # --- MFMA and LDS counters
    mf = {c: _counters(os.path.join(d, "pmc_mfma"), c) for c in
          ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
           "SQ_INSTS_VALU_MFMA_MOPS_F8", "GRBM_GUI_ACTIVE")}
    ld = {c: _counters(os.path.join(d, "pmc_lds"), c) for c in
          ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA",
           "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")}
    mean = lambda t, n: (lambda v: sum(v) / len(v) if v else float("nan"))(_lookup(t, n) or [])
    lines = []
    for n in BENCH_WORKLOADS:
        w = WORKLOADS[n]
        gui = mean(mf["GRBM_GUI_ACTIVE"], n) / 8
        if gui != gui:
            continue
        busy = mean(mf["SQ_VALU_MFMA_BUSY_CYCLES"], n) / (gui * 1024)
        mops16 = mean(mf["SQ_INSTS_VALU_MFMA_MOPS_BF16"], n) + mean(mf["SQ_INSTS_VALU_MFMA_MOPS_F16"], n)
        mops8 = mean(mf["SQ_INSTS_VALU_MFMA_MOPS_F8"], n)
        alg = 4 * w["D"] * visible_pairs(w["mode"], w["L"], w["block_size"]) * w["B"] * w["H"]
        issued = (mops16 + mops8) * 512
        gui_l = mean(ld["GRBM_GUI_ACTIVE"], n) / 8
        lds_act, lds_conf = mean(ld["SQ_LDS_IDX_ACTIVE"], n), mean(ld["SQ_LDS_BANK_CONFLICT"], n)
        n_mfma, n_valu, n_lds = (mean(ld["SQ_INSTS_MFMA"], n), mean(ld["SQ_INSTS_VALU"], n),
                                 mean(ld["SQ_INSTS_LDS"], n))
        lines.append(f"| {n} | {gui:,.0f} | {100 * busy:.1f}% | {issued / alg:.3f} | "
                     f"{mops16 * 512 / (gui * 1024):.0f} / {mops8 * 512 / (gui * 1024):.0f} | "
                     f"{100 * lds_act / (gui_l * 256):.1f}% | "
                     f"{lds_conf / max(lds_act - lds_conf, 1):.3f} | {n_valu / n_mfma:.2f} | "
                     f"{n_lds / n_mfma:.2f} |")
    with open(os.path.join(prof, "attn_fwd_mfma_lds_counters_all_workloads.md"), "w") as f:
        f.write("# MFMA and LDS activity per launch from rocprofv3 PMC counters\n\n"
                "Two runs (repo root, on one MI355X; counters serialise the dispatches, so clocks are per "
                "launch):\n\n```\n" + PROFILE_COMMANDS["pmc_mfma"] + "\n" + PROFILE_COMMANDS["pmc_lds"]
                + "\n```\n\n"
                f"Summarised by `python3 bench.py --summarize-profiles gpurun_out`; kernel source digest "
                f"`{digest}`. GRBM_GUI_ACTIVE is summed over the 8 XCDs, so a launch's clock count is "
                "GUI = GRBM_GUI_ACTIVE / 8.\n\n"
                "* MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI x 1024 SIMDs).\n"
                "* MFMA FLOPs = (MOPS_BF16 + MOPS_F16 + MOPS_F8) x 512; issued / algorithmic counts the "
                "masked halves of diagonal subtiles (and the D = 16 padding).\n"
                "* FLOP per clock per SIMD: the dense 16-bit peak is 1024 (2048 for fp8).\n"
                "* LDS busy = SQ_LDS_IDX_ACTIVE / (GUI x 256 CUs); bank conflicts = SQ_LDS_BANK_CONFLICT / "
                "(SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT).\n"
                "* VALU and LDS instructions per wave; SQ_INSTS_VALU includes the MFMAs.\n\n"
                "| workload | GUI clocks | MFMA busy | MFMA FLOPs issued / algorithmic | FLOP per clock per "
                "SIMD (16-bit / fp8) | LDS busy | LDS bank conflicts | VALU instr per MFMA | LDS instr per "
                "MFMA |\n|---|---|---|---|---|---|---|---|---|\n" + "\n".join(lines) + "\n")
    if all(os.path.isdir(os.path.join(d, x)) for x in STALL_PASSES):
        summarize_stalls(d, digest, prof)
    print(f"wrote {prof} from {d}", flush=True)


STALL_PASSES = ("pmc_stall_a", "pmc_stall_b", "pmc_icache", "pmc_ldslat", "pmc_vmemlat")


def summarize_stalls(d, digest, prof):
    """Where a wave's cycles go: issue, waits for issue, waits on dependencies, per workload."""
    names = {"pmc_stall_a": ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                             "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_COEXEC_CYCLES",
                             "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE"),
             "pmc_stall_b": ("SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_MISC"),
             "pmc_icache": ("SQC_ICACHE_MISSES", "SQC_ICACHE_REQ", "SQ_INSTS", "SQ_WAVE_CYCLES"),
             "pmc_ldslat": ("LdsLatency",), "pmc_vmemlat": ("VmemLatency",)}
    tab = {(pas, c): _counters(os.path.join(d, pas), c) for pas, cs in names.items() for c in cs}
    mean = lambda pas, c, n: (lambda v: sum(v) / len(v) if v else float("nan"))(_lookup(tab[(pas, c)], n) or [])
    lines = []
    for n in BENCH_WORKLOADS:
        gui = mean("pmc_stall_a", "GRBM_GUI_ACTIVE", n) / 8
        if gui != gui:
            continue
        wc = mean("pmc_stall_a", "SQ_WAVE_CYCLES", n)      # quad-cycles summed over waves
        fa = lambda c: mean("pmc_stall_a", c, n) / wc
        fb = lambda c: mean("pmc_stall_b", c, n) / wc
        insts = mean("pmc_icache", "SQ_INSTS", n) / (4 * mean("pmc_icache", "SQ_WAVE_CYCLES", n))
        miss = mean("pmc_icache", "SQC_ICACHE_MISSES", n) / mean("pmc_icache", "SQC_ICACHE_REQ", n)
        lines.append(f"| {n} | {4 * wc / gui / 1024:.2f} | {fa('SQ_ACTIVE_INST_ANY'):.2f} | "
                     f"{fa('SQ_WAIT_INST_ANY'):.2f} | {fa('SQ_WAIT_ANY'):.2f} | {fa('SQ_ACTIVE_INST_VALU'):.2f} | "
                     f"{fa('SQ_ACTIVE_INST_LDS'):.3f} | {fb('SQ_ACTIVE_INST_SCA'):.3f} | "
                     f"{fb('SQ_ACTIVE_INST_VMEM'):.3f} | "
                     f"{mean('pmc_stall_a', 'SQ_VALU_MFMA_COEXEC_CYCLES', n) / (gui * 1024):.2f} | "
                     f"{insts:.3f} | {miss:.5f} | {mean('pmc_ldslat', 'LdsLatency', n):.0f} | "
                     f"{mean('pmc_vmemlat', 'VmemLatency', n):.0f} |")
    cmds = "\n".join(PROFILE_COMMANDS[x] for x in STALL_PASSES)
    with open(os.path.join(prof, "attn_fwd_issue_and_wait_counters_all_workloads.md"), "w") as f:
        f.write("# Where the waves' cycles go: issue, waits for issue, waits on dependencies\n\n"
                "Five runs (repo root, on one MI355X):\n\n```\n" + cmds + "\n```\n\n"
                f"Summarised by `python3 bench.py --summarize-profiles gpurun_out`; kernel source digest "
                f"`{digest}`. The SQ cycle counters count per wave in units of 4 cycles; every column "
                "below except the last four is a fraction of the waves' resident cycles "
                "(SQ_WAVE_CYCLES), so issue + waits can exceed 1 (a wave can wait on a dependency while "
                "its last instruction executes).\n\n"
                "* waves per SIMD = 4 x SQ_WAVE_CYCLES / (GUI x 1024), GUI = GRBM_GUI_ACTIVE / 8;\n"
                "* issuing = SQ_ACTIVE_INST_ANY; waiting for issue (an instruction ready, its unit taken) = "
                "SQ_WAIT_INST_ANY; waiting on dependencies (s_waitcnt, barrier, operand) = SQ_WAIT_ANY;\n"
                "* VALU, LDS, scalar, vector memory: SQ_ACTIVE_INST_* by instruction class (VALU includes "
                "MFMA issue);\n"
                "* MFMA co-issue = cycles in which the MFMA pipe was busy and a VALU instruction issued, "
                "per SIMD cycle;\n"
                "* instructions per wave cycle = SQ_INSTS / (4 x SQ_WAVE_CYCLES); I-cache miss rate = "
                "SQC_ICACHE_MISSES / SQC_ICACHE_REQ;\n"
                "* LDS and vector-memory latency (cycles per instruction, rocprofv3's derived LdsLatency and "
                "VmemLatency; the vector-memory instructions are the K/V DMA and the Q loads).\n\n"
                "| workload | waves per SIMD | issuing | waiting for issue | waiting on dependencies | "
                "VALU | LDS | scalar | vector memory | MFMA co-issue | instructions per wave cycle | "
                "I-cache miss rate | LDS latency | vector-memory latency |\n"
                "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|\n" + "\n".join(lines) + "\n")


def main():
    a = parse()
    if a.summarize_profiles:
        summarize_profiles(a.summarize_profiles)
        return
    if a.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {a.gpus} is not supported (the "
              "attention forward is measured on one MI355X; the work is independent per "
              "(batch, head), so G GPUs would each run the same kernel on their slice)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from attention_forward_06_amd import binding
    binding.load_library()

    if a.copy_calibration:
        copy_calibration()
    names = [HEADLINE, "blockdiag_b1_h2_n256_d128_bs64_f16", "blockdiag_b8_h32_n16384_d128_bs64_f16",
             "blockdiag_b8_h32_n16384_d128_bs128_f16", "dense_b4_h16_l2048_d64_f16",
             "causal_b1_h16_l32768_d256_bf16_ve5m2", "causal_b1_h16_l32768_d256_f16_ve5m2",
             "dense_b4_h16_l2048_d32_f16", "causal_b4_h32_l4096_d16_bf16"]
    if a.only:
        names = [a.only]
    res = {}
    for n in names:
        # the L = 32768 launches are ~13x longer than the headline's: a tenth of the launches,
        # but at least 3 warm-up and 5 timed ones (context figures, not the timed step)
        long_seq = "l32768" in n
        steps = max(5, a.steps // 10) if long_seq else a.steps
        warmup = max(3, a.warmup // 10) if long_seq else a.warmup
        res[n] = time_workload(n, steps, warmup)
        print(f"# {n}: {res[n]['ms']:.4f} ms/launch  {res[n]['tflops']:.1f} TFLOP/s  "
              f"{res[n]['gbs']:.1f} GB/s", file=sys.stderr, flush=True)

    head = res.get(HEADLINE) or next(iter(res.values()))
    traffic = load_traffic(head["name"])
    line = {
        "metric": "attn fwd TFLOP/s + % MFMA peak (causal L=4096); block-diag GB/s % HBM peak",
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["name"], "mask": head["mode"], **head["shape"],
                   "inputs": "seeded N(0,1), resident in HBM"},
        "roofline": {"bound": "mfma", "achieved": round(head["tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(head["tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    bd = {}
    for n, r in res.items():
        if r["mode"] == "block_diag" and r["shape"]["L"] >= 4096:
            bd[f"bs{r['shape']['block_size']}"] = {
                "workload": n, "GB_per_s": round(r["gbs"], 1), "peak_GB_per_s": PEAK_HBM_GBS,
                "frac": round(r["gbs"] / PEAK_HBM_GBS, 4), "ms": round(r["ms"], 5),
                "traffic": load_traffic(n)}
    if bd:
        line["block_diag"] = bd
    others = {}
    for n, r in res.items():
        if n == head["name"] or n in [b["workload"] for b in bd.values()]:
            continue
        if r["mode"] == "block_diag":
            # the pages' quick-check size: 0.5 MiB per launch, bound by launch latency
            others[n] = {"GB_per_s": round(r["gbs"], 1), "ms": round(r["ms"], 5),
                         "note": "report only: launch-latency bound"}
        else:
            others[n] = {"TFLOP_per_s": round(r["tflops"], 2),
                         "frac_bf16_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
                         "ms": round(r["ms"], 5)}
    if others:
        line["other_workloads"] = others
    per = head["per_launch_ms"]
    line["launch_ms_after_timed_region"] = {
        "min": round(head["min_ms"], 5), "median": round(head["median_ms"], 5),
        "first_5": [round(x, 4) for x in per[:5]], "last_5": [round(x, 4) for x in per[-5:]]}
    if not a.no_ceilings:
        ceil = measured_ceilings()
        # secondary figures: against what this chip sustains, not the published peaks the
        # roofline fractions use
        ceil["headline_frac_of_measured_secondary"] = round(
            head["tflops"] / ceil["mfma_bf16_TFLOP_per_s"], 4)
        for key, b in bd.items():
            ceil[f"block_diag_{key}_frac_of_measured_secondary"] = round(
                b["GB_per_s"] / ceil["hbm_3read_1write_GB_per_s"], 4)
        line["measured_ceilings"] = ceil
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_workload(HEADLINE, a.cpu_seconds)
        line["cpu_baseline_by_workload"] = {
            n: cpu_baseline_workload(n, a.cpu_seconds_other) for n in res if n != HEADLINE}
        line["max_abs_err"] = {n: parity(r) for n, r in res.items()}
        print("# oracle leg done", file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
