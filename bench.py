"""Benchmark of the deterministic FP32 per-step d_u update on one MI355X.

One benchmark step is one pass of the whole hot path over the workload: the prepared multi-step driver running all T
steps of the workload (by default as one fused launch; --driver per-step issues one launch per step). Inputs are
synthetic, seeded and resident in device memory before timing starts. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--driver fused|per-step|graph] [--cold]
                  [--plan ...] [--no-cpu] [--cpu-seconds S]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0               # MI355X HBM3E, published
# FP32 vector peak, published (157.3 TFLOP/s): 256 CUs x 4 SIMDs x 32 FMA lanes per clock x 2 flop x 2.4 GHz. On
# gfx950 plain VOP2 v_fmac_f32 with all-VGPR operands issues at this double rate (no packed FP32 needed); an SGPR
# operand halves it.
VALU_FP32_PEAK_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12
METRIC = "GFLOP/s and HBM GB/s per gx_gemm step (fraction of roofline), bit-exact"
KERNEL_SOURCES = ("deterministic_fp32_gemm_amd/csrc/gx_gemm_kernel.hip", "deterministic_fp32_gemm_amd/csrc/gx_gemm_mfma.hip")


def kernel_hash() -> str:
    """Hash of the kernel sources' code: line comments removed and whitespace collapsed, so that an edit of comments
    alone keeps a committed counter measurement valid, and any change of code does not."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            code = re.sub(r"\s+", " ", re.sub(r"//[^\n]*", "", f.read()))
        h.update(code.encode())
    return h.hexdigest()[:16]


PLAN_KEYS = ("engine", "rows_per_wave", "cols_per_lane", "waves_per_wg", "staging", "xcd_remap", "slab_rows",
             "mf_row_waves", "mf_col_waves", "mf_stages", "mf_reg_slabs", "mf_loader_waves", "mf_workgroups",
             "mf_du_at_end", "mf_block", "mf_stream_du")


def kernel_name(plan: dict) -> str:
    if plan.get("engine") != 1:
        return "gx_chain_kernel"
    return "gx_mfma_dma_kernel" if plan.get("mf_reg_slabs") == 0 else "gx_mfma_kernel"


def measured_traffic(workload_key: int, driver: str, plan: dict):
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled as the
    copy calibration in profiles/ states), or None unless it was taken on the current kernel source and plan."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_name(plan)}_workload{workload_key}_{driver}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_sha256_16") != kernel_hash():
        return None
    if any(d.get("plan", {}).get(k) != plan.get(k) for k in PLAN_KEYS):
        return None
    return d.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=(1, 2, 3, 4, 5))
    ap.add_argument("--driver", default="fused", choices=("fused", "per-step", "graph"),
                    help="fused: one launch for all T steps; per-step: T launches; graph: one replay of a HIP graph "
                         "holding the T per-step launches")
    ap.add_argument("--cold", action="store_true", help="flush the caches before every timed launch (adds a field)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--plan", default=None,
                    help="override: valu:RI,RC,WAVES,STAGING,XCD[,SLAB] or mfma:ROW_WAVES,COL_WAVES,STAGES,REG_SLABS,"
                         "LOADER_WAVES[,WORKGROUPS[,DU_AT_END[,BLOCK[,SLAB_ROWS[,STREAM_DU]]]]] "
                         "(REG_SLABS 0: slabs straight to LDS; BLOCK 16 or 32 columns per wavefront)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); the update shards over "
              "chunks with no exchange, so N GPUs run N independent copies of this benchmark", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import deterministic_fp32_gemm_amd as g
    from deterministic_fp32_gemm_amd import inputs
    from deterministic_fp32_gemm_amd.step import aligned_empty

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    g.load()                                           # fails loudly if the HIP library is not built
    dev = torch.cuda.current_device()
    props = torch.cuda.get_device_properties(dev)
    w = inputs.WORKLOADS[args.workload]
    N, P, C, hd, ld, T = w.N, w.P, w.C, w.hd, w.ld, w.T

    # ---- inputs in HBM -------------------------------------------------------------------------------------------
    x_h, dv_h, du_h = inputs.workload_inputs(w, "normal")
    x = aligned_empty(x_h.size, 0)
    dv = aligned_empty(dv_h.size, w.base_offset_bytes)
    du = aligned_empty(du_h.size, w.base_offset_bytes)
    x.copy_(torch.from_numpy(x_h.reshape(-1)))
    dv.copy_(torch.from_numpy(dv_h.reshape(-1)))
    du.copy_(torch.from_numpy(du_h.reshape(-1)))
    x3, dv3, du3 = x.view(N, C, C), dv.view(N, C, ld)[:, :, :hd], du.view(N, C, ld)[:, :, :hd]
    plan = None
    if args.plan:
        engine, _, fields = args.plan.partition(":")
        f = [int(v) for v in fields.split(",")]
        plan = g.make_mfma_plan(*f) if engine == "mfma" else g.make_plan(*f)
    step = g.make_step(du3, x3, dv3, P, plan)
    stream = torch.cuda.current_stream()

    graph = step.graph(0, T, g.SDM_GX_STEPS_FORWARD) if args.driver == "graph" else None

    def one_pass():
        if args.driver == "fused":
            step.fused(0, T, stream)
        elif args.driver == "graph":
            graph.launch(stream)
        else:
            for ti in range(T):
                step(ti, stream)

    launches_per_pass = 1 if args.driver == "fused" else T
    bytes_per_pass = T * w.bytes_per_step
    flops_per_pass = T * w.flops_per_step
    bytes_per_launch = bytes_per_pass / launches_per_pass

    # ---- one pass of the timed configuration from the pristine d_u, kept for the CPU leg's bitwise check ----------
    one_pass()
    torch.cuda.synchronize()
    gpu_one_pass = du.cpu().numpy().reshape(du_h.shape)
    du.copy_(torch.from_numpy(du_h.reshape(-1)))

    # ---- warm timing: the whole region, and every launch between its own events -------------------------------------
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    region_ms = t0.elapsed_time(t1)
    ms_per_step = region_ms / args.steps

    # Average launch duration: the timed region over the launches it holds (back-to-back launches on one stream, so
    # this is the kernel's own duration plus the dispatch gap, the figure a kernel trace reports as its average).
    launch_ms_mean = region_ms / (args.steps * launches_per_pass)

    # Per-launch spread: an event pair around each launch (adds the events' own overhead, ~2 us, to each figure).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(args.steps, 200) * (1 if args.driver == "graph" else launches_per_pass))]
    k = 0
    for _ in range(min(args.steps, 200)):
        if args.driver in ("fused", "graph"):
            ev[k][0].record(stream)
            one_pass()
            ev[k][1].record(stream)
            k += 1
        else:
            for ti in range(T):
                ev[k][0].record(stream)
                step(ti, stream)
                ev[k][1].record(stream)
                k += 1
    torch.cuda.synchronize()
    bracketed = sorted(a.elapsed_time(b) for a, b in ev)
    bracketed_median = bracketed[len(bracketed) // 2]

    # ---- cold timing (optional): 1 GiB written between launches, outside the event pair -----------------------------
    cold = None
    if args.cold:
        flush = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
        cms = []
        for i in range(min(args.steps, 50)):
            flush.fill_(float(i))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            one_pass()
            b.record(stream)
            torch.cuda.synchronize()
            cms.append(a.elapsed_time(b))
        cms.sort()
        cmed = cms[len(cms) // 2]
        cold = {"ms_per_step_median": cmed, "gflops": flops_per_pass / (cmed * 1e-3) / 1e9,
                "hbm_gbps": bytes_per_pass / (cmed * 1e-3) / 1e9,
                "frac": bytes_per_pass / (cmed * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del flush

    # ---- CPU baseline: the oracle on whole passes of the same workload, on the host cores --------------------------
    # The first oracle pass also checks the GPU's single pass bit for bit (NaN results by class, padding by bits).
    cpu = None
    bit_exact = None
    if not args.no_cpu:
        import oracle
        threads = min(16, len(os.sched_getaffinity(0)))
        work = du_h.copy()
        passes, t_start = 0, time.perf_counter()
        while True:
            used = oracle.gx_gemm_chunks(work, x_h, dv_h, 0, N, hd, threads=threads)
            passes += 1
            if passes == 1:
                t_check = time.perf_counter()
                same = (gpu_one_pass.view(np.uint32) == work.view(np.uint32)) | (
                    np.isnan(gpu_one_pass) & np.isnan(work))
                bit_exact = bool(same.all())
                t_start += time.perf_counter() - t_check
            if time.perf_counter() - t_start >= args.cpu_seconds:
                break
        el = time.perf_counter() - t_start
        cpu = {"value": round(passes * flops_per_pass / el / 1e9, 3), "unit": "GFLOP/s", "cores": used,
               "kind": "oracle",
               "sample": f"{passes} full passes of the workload ({T} steps x {P} chunks) in {el:.1f} s, chunks "
                         f"split over {used} host threads, scalar fmaf chain",
               "hbm_gbps_equiv": round(passes * bytes_per_pass / el / 1e9, 3)}

    # ---- roofline of the dominant kernel ------------------------------------------------------------------------------
    t_hbm = bytes_per_launch / (HBM_PEAK_GBS * 1e9)
    t_alu = (flops_per_pass / launches_per_pass) / (VALU_FP32_PEAK_TFLOPS * 1e12)
    launch_s = launch_ms_mean * 1e-3
    if t_hbm >= t_alu:
        roof = {"bound": "hbm", "achieved": bytes_per_launch / launch_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "alu", "achieved": flops_per_pass / launches_per_pass / launch_s / 1e12,
                "peak": VALU_FP32_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.key, args.driver, step.geom["fused" if args.driver == "fused" else "step"])
    roof["kernel"] = kernel_name(step.geom["fused" if args.driver == "fused" else "step"])
    roof["algorithmic_bytes_per_launch"] = bytes_per_launch
    roof["algorithmic_flops_per_launch"] = flops_per_pass / launches_per_pass
    roof["launch_ms_mean"] = launch_ms_mean
    roof["bracketed_launch_ms_median"] = bracketed_median
    roof["bracketed_launch_ms_min"] = bracketed[0]

    gflops = flops_per_pass / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"workload {w.key}: {w.description}", "T": T, "P": P, "N": N, "C": C, "hd": hd,
                   "ld": ld, "base_offset_bytes": w.base_offset_bytes, "driver": args.driver, "pattern": "normal",
                   "plan": step.geom["fused" if args.driver == "fused" else "step"]},
        "hbm_gbps": round(bytes_per_pass / (ms_per_step * 1e-3) / 1e9, 3),
        "bit_exact": bit_exact,
        "roofline": roof,
        "cpu_baseline": cpu,
        "cold": cold,
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
