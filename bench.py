"""Benchmark of the deterministic FP32 per-step d_u update on one MI355X.

One benchmark step is one pass of the whole hot path over one workload: the prepared multi-step driver running all
T gx_gemm steps of the workload (by default as one fused launch; --driver per-step issues one launch per step). The
headline workload is workload 5 (T=2 x P=512 chunks, C=64, hd=256, row stride 260, d_u and d_dv bases at +4 B), the
largest of the five. Inputs are synthetic, seeded and resident in device memory before any timing starts. Prints ONE
JSON line.

What the line holds:
  value / ms_per_step / roofline   the headline workload, warm: K passes back to back on one stream between two
                                   HIP events (the figure a kernel trace of back-to-back launches averages to)
  cold                             the same pass with every cache flushed first: batches of (read 1 GiB, pass)
                                   minus batches of (read 1 GiB), per pass; d_u's write-back is charged to the pass
  per_step_driver                  the same pass as T launches, one per gx_gemm step
  workloads                        workloads 2-5: both engines warm, the default engine cold and per step, each
                                   pass checked bit for bit against the CPU oracle; and a device copy of the same
                                   bytes (half read, half written) warm and cold, as a streaming yardstick
  phase_a                          Phase A, the consumer of the updated d_u, on synthetic records shaped like workloads
                                   3 and 5 (T steps, one launch each), warm and cold, checked against its oracle
  cpu_baseline                     the CPU oracle, unchanged, on this host's cores (and on one core)

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--driver fused|per-step|graph]
                  [--plan ...] [--only] [--no-cpu] [--cpu-seconds S] [--profile warm|cold]
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
FLUSH_BYTES = 1 << 30               # larger than the 256 MB Infinity Cache and the 8 x 4 MB of L2


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
             "mf_du_at_end", "mf_block", "mf_stream_du", "mf_aln")


def kernel_name(plan: dict) -> str:
    if plan.get("engine") != 1:
        return "gx_chain_kernel"
    return "gx_mfma_dma_kernel" if plan.get("mf_reg_slabs") == 0 else "gx_mfma_kernel"


def measured_traffic(workload_key: int, driver: str, plan: dict):
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE of cold-cache
    launches, scaled as the copy calibration in profiles/ states), or None unless it was taken on the current kernel
    source and plan."""
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


def host_cpus():
    """(CPUs this process may run on: the affinity set within the cgroup's CPU quota, affinity count, quota or None,
    CPU model)."""
    aff = len(os.sched_getaffinity(0))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
        if q != "max":
            quota = max(1, int(int(q) // int(period)))
    except (OSError, ValueError):
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return (min(aff, quota) if quota else aff), aff, quota, model


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed passes (benchmark steps) of the headline workload")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=(1, 2, 3, 4, 5), help="headline workload")
    ap.add_argument("--driver", default="fused", choices=("fused", "per-step", "graph"),
                    help="headline driver. fused: one launch for all T steps; per-step: T launches; graph: one replay "
                         "of a HIP graph holding the T per-step launches")
    ap.add_argument("--only", action="store_true", help="the headline workload alone (no per-workload table)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the threaded CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle (no baseline, no bit-exact check)")
    ap.add_argument("--no-phase-a", action="store_true", help="skip the Phase A leg")
    ap.add_argument("--phase-a", default=None, choices=("a3", "a5"),
                    help="with --profile: profile this Phase A workload's pass instead of the update")
    ap.add_argument("--profile", choices=("warm", "graph", "cold"), default=None,
                    help="profiling run of the headline workload's launch alone: warm = W + K passes launched back to "
                         "back from the host, as the benchmark times them; graph = K passes replayed from a graph of "
                         "20 (after one warm-up replay); cold = K flush-read + pass pairs")
    ap.add_argument("--plan", default=None,
                    help="headline override: valu:RI,RC,WAVES,STAGING,XCD[,SLAB] or mfma:ROW_WAVES,COL_WAVES,STAGES,"
                         "REG_SLABS,LOADER_WAVES[,WORKGROUPS[,DU_AT_END[,BLOCK[,SLAB_ROWS[,STREAM_DU]]]]] "
                         "(REG_SLABS 0: slabs straight to LDS; BLOCK 16 or 32 columns per wavefront)")
    return ap.parse_args()


class Bench:
    """Device buffers of one workload and the timing of its passes."""

    def __init__(self, g, inputs, torch, w, flush, sink):
        from deterministic_fp32_gemm_amd.step import aligned_empty
        self.g, self.torch, self.w = g, torch, w
        self.flush, self.sink = flush, sink
        self.x_h, self.dv_h, self.du_h = inputs.workload_inputs(w, "normal")
        self.x = aligned_empty(self.x_h.size, 0)
        self.dv = aligned_empty(self.dv_h.size, w.base_offset_bytes)
        self.du = aligned_empty(self.du_h.size, w.base_offset_bytes)
        self.x.copy_(torch.from_numpy(self.x_h.reshape(-1)))
        self.dv.copy_(torch.from_numpy(self.dv_h.reshape(-1)))
        self.reset()
        N, C, hd, ld = w.N, w.C, w.hd, w.ld
        self.views = (self.du.view(N, C, ld)[:, :, :hd], self.x.view(N, C, C), self.dv.view(N, C, ld)[:, :, :hd])
        self.stream = torch.cuda.current_stream()

    def reset(self):
        self.du.copy_(self.torch.from_numpy(self.du_h.reshape(-1)))
        self.torch.cuda.synchronize()

    def step(self, plan=None):
        du, x, dv = self.views
        return self.g.make_step(du, x, dv, self.w.P, plan)

    def pass_fn(self, step, driver, stream=None):
        T, s = self.w.T, (self.stream if stream is None else stream)
        if driver == "fused":
            return lambda: step.fused(0, T, s)
        if driver == "graph":
            graph = step.graph(0, T, self.g.SDM_GX_STEPS_FORWARD)
            return lambda: graph.launch(s)
        return lambda: [step(ti, s) for ti in range(T)]

    def one_pass_result(self, one_pass):
        """d_u after one pass from the pristine inputs (host copy); d_u is reset afterwards."""
        self.reset()
        one_pass()
        self.torch.cuda.synchronize()
        out = self.du.cpu().numpy().reshape(self.du_h.shape)
        self.reset()
        return out

    def warm_ms(self, one_pass, passes, warmup):
        """Milliseconds per pass: `passes` passes back to back between two events on the launch stream."""
        torch = self.torch
        for _ in range(warmup):
            one_pass()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(passes):
            one_pass()
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / passes

    def flush_read(self):
        self.torch.sum(self.flush, dim=0, out=self.sink)   # reads FLUSH_BYTES, writes one float

    def cold_ms(self, one_pass, batch=25, pairs=7):
        """Milliseconds per pass with cold caches: the median over `pairs` of (batch of [flush read, pass]) minus
        (batch of [flush read]), divided by the batch size. No event sits between a flush and its pass."""
        torch = self.torch

        def timed(with_pass):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(self.stream)
            for _ in range(batch):
                self.flush_read()
                if with_pass:
                    one_pass()
            t1.record(self.stream)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1)

        timed(True)
        timed(False)                                     # warm-up of both batch kinds
        est = []
        for _ in range(pairs):
            a = timed(True)
            b = timed(False)
            est.append((a - b) / batch)
        est.sort()
        return est[len(est) // 2], est


class Pa2Bench:
    """Phase A (the consumer of the updated d_u) on one synthetic record workload: device buffers, one pass = the T
    steps in order, one launch each (steps are sequential: a step reads grad rows earlier steps wrote)."""

    def __init__(self, g, torch, key):
        import numpy as np

        from deterministic_fp32_gemm_amd import pa2_inputs as PI
        from deterministic_fp32_gemm_amd.step import aligned_empty
        self.g, self.torch = g, torch
        self.w = w = PI.PA2_WORKLOADS[key]
        self.h = h = PI.inputs(w, "normal")
        self.grad = torch.from_numpy(h["grad"]).cuda()
        self.bank = torch.from_numpy(h["bank"]).cuda()
        self.snap = torch.from_numpy(h["snap"]).cuda()
        du = aligned_empty(h["du"].size, w.du_offset_bytes)
        du.copy_(torch.from_numpy(h["du"].reshape(-1)))
        self.du = du.view(h["du"].shape)
        self.beta = torch.from_numpy(h["beta"]).cuda()
        self.kpay = torch.from_numpy(h["kpay"]).cuda()
        self.rec = torch.from_numpy(h["rec"]).cuda()
        self.bpre = torch.from_numpy(h["bpre"]).cuda() if h["ssr"] < 0 else None
        self.eff = torch.zeros((h["planes"], w.N * w.n), dtype=torch.float32, device="cuda")
        self.gout = torch.zeros_like(self.eff)
        self.args = g.pa2_args(self.grad, self.bank, self.snap, h["ssr"], self.du, self.beta, self.kpay, self.rec,
                               self.bpre, self.eff, self.gout, w.P, w.C, w.W, w.hd, ld_u=w.ld_u)
        self.plan = g.sdm_pa2_plan_for(self.args, torch.cuda.get_device_properties(0).multi_processor_count)
        self.stream = torch.cuda.current_stream()
        # algorithmic bytes and flops of a pass, from the records: each record (16 bytes) and output (4 bytes per
        # plane, two outputs) once, the token rows and beta once per chunk, a grad row and a snapshot row read per
        # valid FIRST, a grad row and a bank row written per valid LAST
        pay = h["kpay"].view(np.uint32)
        valid = (pay & np.uint32(0x20000)) == 0
        vfirst = int(((pay & np.uint32(0x80000000)) != 0)[valid].sum())
        vlast = int(((pay & np.uint32(0x40000000)) != 0)[valid].sum())
        recs = w.N * w.n
        self.bytes_pass = (recs * (16 + 8 * h["planes"]) + w.N * w.C * (w.hd + 1) * 4 +
                           (vfirst + vlast) * 2 * w.hd * 4)
        self.flops_pass = recs * w.hd * 4 + (vfirst + vlast) * w.hd * 2 + recs * w.nsl * 2 * 31

    def one_pass(self):
        self.g.sdm_pa2_steps(self.args, 0, self.w.T, self.g.SDM_GX_STEPS_FORWARD, self.plan, self.stream)

    def reset(self):
        self.grad.copy_(self.torch.from_numpy(self.h["grad"]))
        self.bank.copy_(self.torch.from_numpy(self.h["bank"]))
        self.torch.cuda.synchronize()

    def result(self):
        self.torch.cuda.synchronize()
        return self.grad.cpu().numpy(), self.bank.cpu().numpy(), self.eff.cpu().numpy(), self.gout.cpu().numpy()

    def rates(self, ms):
        s = ms * 1e-3
        return {"ms_per_pass": ms, "ms_per_step": ms / self.w.T, "gflops": self.flops_pass / s / 1e9,
                "hbm_gbps": self.bytes_pass / s / 1e9, "frac": self.bytes_pass / s / 1e9 / HBM_PEAK_GBS}


def rates(w, ms_per_pass, launches_per_pass):
    bytes_pass, flops_pass = w.T * w.bytes_per_step, w.T * w.flops_per_step
    s = ms_per_pass * 1e-3
    return {"ms_per_pass": ms_per_pass, "ms_per_gx_gemm_step": ms_per_pass / w.T,
            "ms_per_launch": ms_per_pass / launches_per_pass,
            "gflops": flops_pass / s / 1e9, "hbm_gbps": bytes_pass / s / 1e9,
            "frac": bytes_pass / s / 1e9 / HBM_PEAK_GBS}


def b_warm(torch, one_pass, stream, passes, warmup):
    """Milliseconds per pass: `passes` passes back to back between two events on the launch stream."""
    for _ in range(warmup):
        one_pass()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(passes):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / passes


class pb_cold_shim:
    """The attributes Bench.cold_ms uses, for a Phase A workload."""

    def __init__(self, pb, torch, flush, sink):
        self.torch, self.stream, self.flush, self.sink = torch, pb.stream, flush, sink

    def flush_read(self):
        self.torch.sum(self.flush, dim=0, out=self.sink)


def same_bits(np, a, b):
    return bool(((a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))).all())


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the update shards over "
              "chunks with no exchange, so N GPUs would run N independent copies of this benchmark", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import deterministic_fp32_gemm_amd as g
    from deterministic_fp32_gemm_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    g.load()                                           # fails loudly if the HIP library is not built
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    head = inputs.WORKLOADS[args.workload]

    plan_override = None
    if args.plan:
        engine, _, fields = args.plan.partition(":")
        f = [int(v) for v in fields.split(",")]
        plan_override = g.make_mfma_plan(*f) if engine == "mfma" else g.make_plan(*f)

    # ---- profiling runs: the headline launch alone ------------------------------------------------------------------
    if args.profile and args.phase_a:
        pb = Pa2Bench(g, torch, args.phase_a)
        if args.profile == "cold":
            shim = pb_cold_shim(pb, torch, flush, sink)
            for _ in range(args.steps):
                shim.flush_read()
                pb.one_pass()
            torch.cuda.synchronize()
            ms = None
        else:
            ms = b_warm(torch, pb.one_pass, pb.stream, args.steps, args.warmup)
        print(json.dumps({"profile": args.profile, "phase_a": args.phase_a, "passes": args.steps,
                          "ms_per_pass_warm": ms, "plan": pb.plan.as_dict()}), flush=True)
        return 0
    if args.profile:
        b = Bench(g, inputs, torch, head, flush, sink)
        step = b.step(plan_override)
        one_pass = b.pass_fn(step, args.driver)
        if args.profile == "warm":                      # the benchmark's own launches: back to back from the host
            ms = b.warm_ms(one_pass, args.steps, args.warmup)
        elif args.profile == "graph":
            # launches captured in a HIP graph (torch's stream capture of the library's kernel launches), so that the
            # traced dispatches run back to back whatever the profiler's per-launch host cost
            if args.driver == "graph":
                raise SystemExit("bench.py: --profile graph takes the fused or per-step driver")
            per_graph = 20
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn = b.pass_fn(step, args.driver, torch.cuda.current_stream())
                for _ in range(per_graph):
                    fn()
            graph.replay()                               # warm-up: one replay
            torch.cuda.synchronize()
            reps = max(1, -(-args.steps // per_graph))
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(reps):
                graph.replay()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / (reps * per_graph)
        else:
            for _ in range(args.steps):
                b.flush_read()
                one_pass()
            torch.cuda.synchronize()
            ms = None
        print(json.dumps({"profile": args.profile, "workload": head.key, "passes": args.steps,
                          "ms_per_pass_warm": ms, "plan": step.geom["fused" if args.driver == "fused" else "step"]}),
              flush=True)
        return 0

    # ---- CPU oracle (reference passes for the bit-exact checks, and the baseline) -------------------------------------
    cpus, aff, quota, model = host_cpus()
    oracle = None
    if not args.no_cpu:
        import oracle as _oracle
        oracle = _oracle

    def oracle_pass(b, threads):
        want = b.du_h.copy()
        t = time.perf_counter()
        oracle.gx_gemm_chunks(want, b.x_h, b.dv_h, 0, b.w.N, b.w.hd, threads=threads)
        return want, time.perf_counter() - t

    # ---- per-workload table (headline included) ------------------------------------------------------------------------
    keys = [head.key] if args.only else sorted({2, 3, 4, 5, head.key})
    table = {}
    headline = None
    for key in keys:
        w = inputs.WORKLOADS[key]
        b = Bench(g, inputs, torch, w, flush, sink)
        want = oracle_pass(b, cpus)[0] if oracle else None
        row = {"description": w.description}
        passes = max(20, args.steps if key == head.key else min(args.steps, 200))
        for name in ("default", "valu"):
            if name == "valu" and key == head.key and plan_override is not None:
                continue
            if name == "default":
                step = b.step(plan_override if key == head.key else None)
            else:                                          # the vector-ALU engine's plan for the fused launch
                step = b.step(g.sdm_gx_plan(w.N, w.C, w.hd, w.ld, w.ld, 0, w.base_offset_bytes % 16,
                                            g.SDM_GX_ENGINE_VALU))
            fused = b.pass_fn(step, "fused")
            e = {"plan": step.geom["fused"], "kernel": kernel_name(step.geom["fused"])}
            got = b.one_pass_result(fused)
            e["bit_exact"] = same_bits(np, got, want) if want is not None else None
            e["warm"] = rates(w, b.warm_ms(fused, passes, args.warmup), 1)
            b.reset()
            if name == "default":
                cms, est = b.cold_ms(fused)
                e["cold"] = rates(w, cms, 1)
                e["cold"]["per_pair_ms"] = est
                b.reset()
                per = b.pass_fn(step, "per-step")
                got = b.one_pass_result(per)
                e["per_step_driver"] = rates(w, b.warm_ms(per, max(20, passes // 4), 5), w.T)
                e["per_step_driver"]["plan"] = step.geom["step"]
                e["per_step_driver"]["bit_exact"] = same_bits(np, got, want) if want is not None else None
                b.reset()
                if key == head.key:
                    one_pass = b.pass_fn(step, args.driver)
                    if args.driver != "fused":
                        got = b.one_pass_result(one_pass)
                        hb = same_bits(np, got, want) if want is not None else None
                    else:
                        hb = e["bit_exact"]
                    launches = 1 if args.driver == "fused" else w.T
                    ms = b.warm_ms(one_pass, args.steps, args.warmup) if args.driver != "fused" else \
                        e["warm"]["ms_per_pass"]
                    headline = dict(b=b, step=step, ms=ms, launches=launches, bit_exact=hb, cold=e["cold"],
                                    per_step=e["per_step_driver"],
                                    plan=step.geom["fused" if args.driver == "fused" else "step"])
            row[name] = e
            print(f"bench: workload {key} {name}: {e['kernel']} warm {e['warm']['ms_per_pass'] * 1e3:.2f} us/pass "
                  f"(frac {e['warm']['frac']:.3f})" + (f", cold {e['cold']['ms_per_pass'] * 1e3:.2f} us/pass "
                                                      f"(frac {e['cold']['frac']:.3f})" if "cold" in e else "")
                  + f", bit_exact {e['bit_exact']}", file=sys.stderr, flush=True)
        # yardstick: a device copy moving the pass's algorithmic bytes (half read, half written), same cold protocol
        src = torch.empty(w.T * w.bytes_per_step // 8, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        copy = lambda: dst.copy_(src)                  # noqa: E731
        row["copy_yardstick"] = {"bytes": w.T * w.bytes_per_step,
                                 "warm": rates(w, b.warm_ms(copy, passes, args.warmup), 1),
                                 "cold": rates(w, b.cold_ms(copy)[0], 1)}
        del src, dst
        table[str(key)] = row
        if key != head.key:
            del b

    # ---- Phase A: the consumer of the updated d_u, per-step launches -------------------------------------------------
    phase_a = {}
    if not args.no_phase_a:
        for key in ("a3", "a5"):
            pb = Pa2Bench(g, torch, key)
            e = {"description": pb.w.description, "plan": pb.plan.as_dict(),
                 "kernel": "gx_pa2_staged_kernel" if pb.plan.stage_out else "gx_pa2_kernel",
                 "algorithmic_bytes_per_pass": pb.bytes_pass, "algorithmic_flops_per_pass": pb.flops_pass}
            pb.one_pass()
            got = pb.result()
            if oracle:
                h, w = pb.h, pb.w
                grad, bank = h["grad"].copy(), h["bank"].copy()
                eff = np.zeros((h["planes"], w.N * w.n), np.float32)
                gout = eff.copy()
                t = time.perf_counter()
                for ti in range(w.T):
                    oracle.pa2_step(grad, bank, h["snap"], h["ssr"], h["du"], h["beta"], h["rec"], eff, gout, ti,
                                    w.P, w.C, w.W, w.hd)
                e["oracle_pass_s"] = time.perf_counter() - t
                e["bit_exact"] = all(same_bits(np, a, b) for a, b in zip(got, (grad, bank, eff, gout)))
            else:
                e["bit_exact"] = None
            pb.reset()
            e["warm"] = pb.rates(b_warm(torch, pb.one_pass, pb.stream, max(20, args.steps // 4), 5))
            pb.reset()
            e["cold"] = pb.rates(Bench.cold_ms(pb_cold_shim(pb, torch, flush, sink), pb.one_pass)[0])
            pb.reset()
            phase_a[key] = e
            print(f"bench: phase A {key}: warm {e['warm']['ms_per_pass'] * 1e3:.2f} us/pass (frac "
                  f"{e['warm']['frac']:.3f}), cold {e['cold']['ms_per_pass'] * 1e3:.2f} us/pass (frac "
                  f"{e['cold']['frac']:.3f}), bit_exact {e['bit_exact']}", file=sys.stderr, flush=True)
            del pb

    # ---- CPU baseline: the oracle on whole passes of the headline workload ---------------------------------------------
    cpu = None
    if oracle:
        b = headline["b"]
        passes, el = 0, 0.0
        while el < args.cpu_seconds:
            el += oracle_pass(b, cpus)[1]
            passes += 1
        flops_pass, bytes_pass = head.T * head.flops_per_step, head.T * head.bytes_per_step
        # one thread, the scalar oracle as it stands, over as many whole chunks as fit about a fifth of the budget
        n1, el1 = 0, 0.0
        sub = b.du_h.copy()
        while el1 < args.cpu_seconds / 5 and n1 < head.N:
            k = min(head.P, head.N - n1)
            t = time.perf_counter()
            oracle.gx_gemm_chunks(sub, b.x_h, b.dv_h, n1, n1 + k, head.hd, threads=1)
            el1 += time.perf_counter() - t
            n1 += k
        flops_chunk = flops_pass / head.N
        cpu = {"value": round(passes * flops_pass / el / 1e9, 3), "unit": "GFLOP/s", "cores": cpus, "kind": "oracle",
               "sample": f"{passes} full passes of workload {head.key} ({head.T} steps x {head.P} chunks) in "
                         f"{el:.1f} s, chunks split over {cpus} host threads (one per CPU this process may use), "
                         f"the unchanged scalar fmaf chain",
               "hbm_gbps_equiv": round(passes * bytes_pass / el / 1e9, 3),
               "single_thread": {"value": round(n1 * flops_chunk / el1 / 1e9, 3), "unit": "GFLOP/s",
                                 "sample": f"{n1} chunks of workload {head.key} in {el1:.1f} s on one thread"},
               "host": {"cpu_model": model, "affinity_cpus": aff, "cgroup_cpu_quota": quota}}

    # ---- headline line ----------------------------------------------------------------------------------------------------
    w = head
    launches = headline["launches"]
    ms_pass = headline["ms"]
    bytes_launch = w.T * w.bytes_per_step / launches
    flops_launch = w.T * w.flops_per_step / launches
    launch_s = ms_pass / launches * 1e-3
    t_hbm = bytes_launch / (HBM_PEAK_GBS * 1e9)
    t_alu = flops_launch / (VALU_FP32_PEAK_TFLOPS * 1e12)
    plan = headline["plan"]
    if t_hbm >= t_alu:
        roof = {"bound": "hbm", "achieved": bytes_launch / launch_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "alu", "achieved": flops_launch / launch_s / 1e12, "peak": VALU_FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.key, args.driver, plan)
    roof["kernel"] = kernel_name(plan)
    roof["algorithmic_bytes_per_launch"] = bytes_launch
    roof["algorithmic_flops_per_launch"] = flops_launch
    roof["launch_ms_mean"] = ms_pass / launches
    roof["cold_frac"] = headline["cold"]["frac"] if launches == 1 else None
    gflops = w.T * w.flops_per_step / (ms_pass * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_pass,
        "ms_per_gx_gemm_step": ms_pass / w.T,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"workload {w.key}: {w.description}", "T": w.T, "P": w.P, "N": w.N, "C": w.C,
                   "hd": w.hd, "ld": w.ld, "base_offset_bytes": w.base_offset_bytes, "driver": args.driver,
                   "pattern": "normal", "bench_step": f"one pass over the workload: its {w.T} gx_gemm steps",
                   "plan": plan},
        "hbm_gbps": round(w.T * w.bytes_per_step / (ms_pass * 1e-3) / 1e9, 3),
        "bit_exact": headline["bit_exact"],
        "roofline": roof,
        "cold": headline["cold"],
        "per_step_driver": headline["per_step"],
        "workloads": table,
        "phase_a": phase_a,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
