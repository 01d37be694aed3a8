"""Throughput of the per-expert mixed-precision MoE expert layer on one MI355X.

Default run (one JSON line): decode on the coarse MoE layer, E=8,
d_model=4096, d_ff=14336 SwiGLU, top-2, 16 tokens per step, bit-widths from
the exact allocator at an average of 4.5 bits/weight with Zipf(1.0)
importance. A step is one pw_moe_forward: route, group, fused dequant +
gate/up + SwiGLU, dequant + down, combine. Batches of 1 and 4 tokens are
reported in "sweep"; the other workloads (the fine-grained decode layer, the
same layer with importance-skewed routing, prefill on the matrix cores, the
dynamic re-precision schedule) in "workloads", each with its tokens/s and
its dominant kernels' fraction of the roofline.

Inputs are resident in HBM before timing starts. Each step reads a
different copy of the packed pool (several contexts over the same masters)
so that weights come from HBM, not from the 256 MB Infinity Cache.

roofline: the gate/up kernel (two thirds of the packed bytes), algorithmic
bytes = packed W1 + W3 bytes of the experts the step routes to, divided by
the kernel's mean duration from HIP events on the forward's stream.
cpu_baseline: the plain C++ CPU oracle (float64) timed on a bounded sample,
on all host cores and single-threaded.

One workload alone: --workload decode_fine | skewed | bitplane | prefill | dynamic | kvtrace | swap | tiny.
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

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s + achieved packed-weight HBM GB/s (% of peak), 1×MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 500 untimed forwards (about 75 ms at 16 decode tokens, 0.5 s of prefill)
    # bring the GPU to its steady clocks; after 5 the timed region still
    # started below them (decode 97k against 109k tokens/s)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="decode_coarse",
                    choices=["decode_coarse", "decode_fine", "skewed", "bitplane", "prefill", "dynamic", "kvtrace",
                             "swap", "tiny"])
    ap.add_argument("--tokens", type=int, default=None, help="batch for the main line")
    ap.add_argument("--pools", type=int, default=4, help="rotating packed pools")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="default run: only the decode_coarse line (no other workloads)")
    ap.add_argument("--no-profile", action="store_true",
                    help="time without the per-kernel events (no roofline)")
    ap.add_argument("--event-every-step", action="store_true",
                    help="timing events on every forward of the timed region (default: on the forwards of "
                         "the first rotated pool only, every len(pools)-th step)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (reference for HBM counters)")
    return ap.parse_args()


def kernel_source_hash(workload: str) -> str:
    """Hash of the sources of the workload's gate/up kernel (the roofline
    kernel): the matrix-core kernels for prefill, the streaming kernels for
    the decode workloads. Comments and blank lines are left out, so that
    edits of the prose alone keep the counters valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixed_precision_weight_page_amd", "csrc")
    srcs = ("kernels_gemm.hip",) if workload == "prefill" else ("kernels_ffn.hip", "route_dev.h")
    for f in srcs + ("pw_internal.h", "dequant.h", "xscale.h"):
        text = open(os.path.join(csrc, f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, T: int):
    """HBM bytes per gate/up launch from the committed PMC summary, or None
    if there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"gate_up_{workload}_T{T}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash(workload):
        return None
    return float(t.group(1))


class Bench:
    def __init__(self, wl, max_tokens, npools, log, bias=None, layout="eq2"):
        """bias: added to every batch's logits (None: N(0, 1) logits as the
        workload specifies); layout: "eq2" or "bitplane" pages."""
        import torch

        import synth
        from mixed_precision_weight_page_amd import PagedMoELayer
        self.torch = torch
        self.wl = wl
        self.bias = bias
        t0 = time.time()
        self.masters = synth.expert_weights(wl, device="cuda", seed=0)
        torch.cuda.synchronize()
        log(f"{wl.name}: masters on device ({time.time() - t0:.1f}s)")
        self.layers, self.pools = [], []
        bits = None
        for i in range(npools):
            layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=max_tokens,
                                  renorm=wl.renorm, master_dtype=wl.master, layout=layout)
            layer.bind_masters(*self.masters)
            pool = layer.alloc_pool(layer.pool_bytes_for_bits([8] * wl.E))
            layer.alloc_workspace()
            if wl.bits is not None:
                bits = list(wl.bits)
                layer.quantize_experts(bits)
            elif bits is None:
                bits = layer.set_budget(wl.budget_bits(), synth.importance(wl)).tolist()
            else:
                layer.quantize_experts(bits)
            self.layers.append(layer)
            self.pools.append(pool)
        torch.cuda.synchronize()
        self.bits = bits
        log(f"{wl.name}: bits {bits} ({time.time() - t0:.1f}s)")

    def release(self):
        self.layers, self.pools, self.masters = [], [], None
        self.torch.cuda.empty_cache()

    def batches(self, T, n, seed=1):
        import synth
        out = []
        for i in range(n):
            x, lg = synth.tokens(self.wl, T=T, device="cuda", seed=seed, step=i)
            if self.bias is not None:
                lg = (lg + self.bias).contiguous()
            out.append((x, lg))
        return out

    def routed_bytes(self, logits):
        """Packed bytes (W1+W3, W2) of the experts the batch routes to, and
        the most tokens any expert receives."""
        _, _, counts = self.layers[0].route(logits)
        c = counts.cpu()
        active = (c > 0).nonzero().flatten().tolist()
        wl = self.wl
        gu = sum(2 * wl.F * wl.d * self.bits[e] // 8 for e in active)
        dn = sum(wl.d * wl.F * self.bits[e] // 8 for e in active)
        return gu, dn, len(active), int(c.max())

    def run(self, T, steps, warmup, profile=2, sample=False):
        """profile: kernel mask timed with events; sample: events only on the
        forwards of the first rotated context (every len(layers)-th step)."""
        torch = self.torch
        nb = 8
        batches = self.batches(T, nb)
        ys = [torch.empty((T, self.wl.d), dtype=torch.float32, device="cuda") for _ in range(nb)]
        bytes_gu, bytes_dn, n_act, tmax = [], [], [], []
        for x, lg in batches:
            a, b, c, m = self.routed_bytes(lg)
            bytes_gu.append(a)
            bytes_dn.append(b)
            n_act.append(c)
            tmax.append(m)
        L = len(self.layers)
        for i in range(warmup):
            x, lg = batches[i % nb]
            self.layers[i % L].moe_forward(x, lg, ys[i % nb])
        torch.cuda.synchronize()
        # a layer whose profiling is off keeps the records of its last timed
        # run: read only the layers timed in this one
        timed_layers = [j for j in range(L) if profile and (j == 0 or not sample)]
        for j, layer in enumerate(self.layers):
            layer.profile(profile if j in timed_layers else 0)
        t0 = time.perf_counter()
        for i in range(steps):
            x, lg = batches[i % nb]
            self.layers[i % L].moe_forward(x, lg, ys[i % nb])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        prof = {"gate_up_ms": 0.0, "down_ms": 0.0, "route_ms": 0.0, "combine_ms": 0.0}
        timed = 0
        if profile:
            for j in timed_layers:
                p = self.layers[j].profile_read()
                self.layers[j].profile(0)
                timed += p["forwards"]
                for k in prof:
                    prof[k] += p[k]
        # per-forward kernel times, averaged over the forwards that carried events
        prof = {k: (v / timed if timed else 0.0) for k, v in prof.items()}
        tot_gu = sum(bytes_gu[i % nb] for i in range(steps))
        # packed W1+W3 bytes of the forwards that carried events
        gu_timed = sum(bytes_gu[i % nb] for i in range(steps) if not sample or i % L == 0)
        tot_dn = sum(bytes_dn[i % nb] for i in range(steps))
        return dict(T=T, steps=steps, timed_forwards=timed, bytes_gu_timed=gu_timed, elapsed=elapsed, prof=prof,
                    bytes_gu=tot_gu, bytes_dn=tot_dn,
                    mean_active=sum(n_act[i % nb] for i in range(steps)) / steps,
                    max_tokens_per_expert=max(tmax))


def cpu_model() -> str:
    """The host CPU's model name (Linux), for the CPU baseline's record."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(bench, T, log, min_seconds=10.0, max_batches=4):
    """The plain C++ oracle (float64, from the fp32 masters) on T-token
    batches of the same layer: each batch routes its tokens, quantizes the
    experts they route to and runs the forward.

    All host threads (up to 16, the machine's CPU share per GPU): whole batches
    one after another until min_seconds or max_batches (experts quantized
    one per thread, tokens spread over the threads). One thread: the first
    batch, whole."""
    from oracle import c_oracle
    nproc = os.cpu_count() or 1
    batches = bench.batches(T, max_batches, seed=99)
    w = [m.cpu() for m in bench.masters]   # host copies of the masters, not timed

    def one_batch(x, lg, threads):
        t0 = time.time()
        y = c_oracle.moe_forward_quantized(x, lg, bench.wl.k, *w, bench.bits, bool(bench.wl.renorm),
                                           nthreads=threads)
        return time.time() - t0, y

    threads = min(16, nproc)
    total, done, n_exp, y0 = 0.0, 0, [], None
    for x, lg in batches:
        x, lg = x.cpu(), lg.cpu()
        ids, _ = c_oracle.route(lg, bench.wl.k)
        n_exp.append(len(set(ids.reshape(-1).tolist())))
        dt, y = one_batch(x, lg, threads)
        total += dt
        done += 1
        y0 = y if y0 is None else y0
        if total >= min_seconds:
            break
    log(f"oracle, {threads} threads: {done} batches of {T} tokens in {total:.1f}s")
    x, lg = batches[0]
    t1, _ = one_batch(x.cpu(), lg.cpu(), 1)
    log(f"oracle, 1 thread: one batch of {T} tokens in {t1:.1f}s")
    import torch
    return {"value": T * done / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": nproc, "cpu_model": cpu_model(),
            "sample": f"the plain C++ oracle: {done} batch(es) of {T} tokens of the same layer, each routing its "
                      f"tokens, quantizing the experts they route to ({', '.join(map(str, n_exp))}) from the fp32 "
                      f"masters and running the float64 forward (host copies of the masters excluded), "
                      f"{threads} threads; {cpu_model()}, nproc {nproc}",
            "single_thread": {"value": T / t1, "unit": "tokens/s", "cores": 1,
                              "sample": f"the first of those batches ({n_exp[0]} experts), whole, one thread"}}, \
        torch.from_numpy(y0)


def parity_line(bench, T, y_ref):
    """The library's y on the oracle's first batch (the same seeded tokens
    and logits as cpu_baseline's) against the oracle's float64 y: normwise
    error and largest error over the largest |y|, with the bounds the
    parity tests use."""
    import torch
    x, lg = bench.batches(T, 1, seed=99)[0]
    y = bench.layers[0].moe_forward(x, lg)
    torch.cuda.synchronize()
    d = y.double().cpu() - y_ref
    return {"normwise": float(d.norm() / y_ref.norm()), "max_abs_over_max_y": float(d.abs().max() / y_ref.abs().max()),
            "bounds": [2e-3, 1e-2], "sample": f"the oracle's first {T}-token batch"}


HBM = "GB/s"


def kernel_line(name, ms, work, unit):
    """Achieved rate of a kernel class and its fraction of the roofline:
    work in bytes (unit GB/s) or flops (unit TFLOP/s) per launch."""
    if not ms:
        return {f"{name}_us": None}
    if unit == HBM:
        rate = work / (ms * 1e-3) / 1e9
        peak = HBM_PEAK_GBPS
    else:
        rate = work / (ms * 1e-3) / 1e12
        peak = MFMA_F16_PEAK_TFLOPS
    return {f"{name}_us": 1e3 * ms, f"{name}_{'GBps' if unit == HBM else 'TFLOPs'}": rate,
            f"{name}_frac": rate / peak}


def measure(wl, T, args, log, npools, bias=None, bench=None, layout="eq2"):
    """One workload's summary: tokens/s over the timed steps (events on the
    gate/up kernel of the first rotated context), then a second pass timing
    every kernel class for the breakdown and the down kernel's rate."""
    b = bench or Bench(wl, T, npools, log, bias, layout)
    r = b.run(T, args.steps, args.warmup, profile=2, sample=True)
    r_all = b.run(T, args.steps, 0, profile=15)
    out = {"tokens_per_s": T * r["steps"] / r["elapsed"], "ms_per_step": 1e3 * r["elapsed"] / r["steps"],
           "tokens": T, "bits_per_weight": sum(b.bits) / len(b.bits), "mean_active_experts": r["mean_active"],
           "max_tokens_per_expert": r["max_tokens_per_expert"]}
    gu_bytes = r["bytes_gu_timed"] / max(1, r["timed_forwards"])
    dn_bytes = r_all["bytes_dn"] / r_all["steps"]
    if wl.name == "prefill":
        flops = 2.0 * T * wl.k * wl.d * wl.F           # per matrix: 2 flops per weight per pair
        out.update(kernel_line("gate_up", r["prof"]["gate_up_ms"], 2 * flops, "TFLOP/s"))
        out.update(kernel_line("down", r_all["prof"]["down_ms"], flops, "TFLOP/s"))
    else:
        out.update(kernel_line("gate_up", r["prof"]["gate_up_ms"], gu_bytes, HBM))
        out.update(kernel_line("down", r_all["prof"]["down_ms"], dn_bytes, HBM))
    out["route_us"] = 1e3 * r_all["prof"]["route_ms"]
    out["combine_us"] = 1e3 * r_all["prof"]["combine_ms"]
    out["packed_weight_GBps"] = (r["bytes_gu"] + r["bytes_dn"]) / r["elapsed"] / 1e9
    out["packed_weight_frac_of_hbm"] = out["packed_weight_GBps"] / HBM_PEAK_GBPS
    if layout == "bitplane":
        out["layout"] = "bitplane pages (depths from Eq. 1 over 3, 4, 8)"
        out.update(plane_reprecision(b, log))
    if bench is None:
        b.release()
    return out, r, r_all, gu_bytes


def plane_reprecision(b, log, reps=5):
    """Re-precision of a bitplane layer by plane count: every expert's depth
    halved (the pages lose their last planes in place: a table upload, no
    master reads), then restored (the missing planes written from the
    masters where the pages were). Wall time per change, synchronised."""
    import torch
    layer = b.layers[0]
    full = list(b.bits)
    low = [max(1, x // 2) for x in full]
    t_low = t_high = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        layer.quantize_experts(low)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        layer.quantize_experts(full)
        torch.cuda.synchronize()
        t_high += time.perf_counter() - t1
        t_low += t1 - t0
    wl = b.wl
    written = sum((f - l) for f, l in zip(full, low)) * wl.W_e / 8
    log(f"bitplane re-precision: lower {1e3 * t_low / reps:.3f} ms, raise {1e3 * t_high / reps:.3f} ms")
    return {"lower_depths_ms": 1e3 * t_low / reps, "raise_depths_ms": 1e3 * t_high / reps,
            "raise_plane_bytes_written": written,
            "raise_GBps": written / (t_high / reps) / 1e9 if t_high else None}


def skew_bias(wl):
    """Logits bias log p_e: experts routed in proportion to their importance
    (Zipf), so the most important experts take most of the tokens."""
    import numpy as np
    import torch

    import synth
    p = np.asarray(synth.importance(wl), dtype=np.float64)
    return torch.tensor(np.log(p), dtype=torch.float32, device="cuda")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              f"multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n} bytes")
        del src, dst
    if args.workload == "kvtrace":
        return bench_kvtrace(args, synth.WORKLOADS["dynamic"], log)
    if args.workload == "swap":
        return bench_swap(args, synth.WORKLOADS["decode_fine"], log)
    if args.workload == "dynamic":
        print(json.dumps(bench_dynamic(args, synth.WORKLOADS["dynamic"], log)), flush=True)
        return
    if args.workload == "bitplane":
        wl = synth.WORKLOADS["decode_fine"]
        res, _, _, gu_bytes = measure(wl, wl.T, args, log, args.pools, layout="bitplane")
        # planes read per gate/up launch (depth x W1, W3 bits of the routed
        # experts) and the counters' HBM bytes (null once the kernels changed)
        res["gate_up_code_bytes_per_launch"] = gu_bytes
        traffic = traffic_from_profiles("bitplane", wl.T)
        res["gate_up_traffic_bytes"] = traffic
        if traffic:
            res["gate_up_traffic_over_code_bytes"] = traffic / gu_bytes
        print(json.dumps({"metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                          "data": "synthetic",
                          "config": {"workload": "decode_fine layer (E=128, d_model=2048, d_ff=768, top-8, 64 "
                                                 "tokens) in bitplane pages, avg 4 bits/weight"},
                          **res}), flush=True)
        return
    skewed = args.workload == "skewed"
    wl = synth.WORKLOADS["decode_fine" if skewed else args.workload]
    T = args.tokens or wl.T
    default_run = args.workload == "decode_coarse"
    sweep_T = [t for t in synth.DECODE_COARSE_BATCHES if t != T] if default_run else []
    max_tokens = max([T] + sweep_T)
    npools = args.pools if args.workload != "prefill" else 2
    b = Bench(wl, max_tokens, npools, log, skew_bias(wl) if skewed else None)
    # timed region: events only on the gate/up kernel (the roofline kernel);
    # a second pass of the same steps times every kernel for the breakdown
    sample = not args.event_every_step
    r = b.run(T, args.steps, args.warmup, profile=0 if args.no_profile else 2, sample=sample)
    r_all = b.run(T, args.steps, 0, profile=15) if not args.no_profile else None
    tokens_per_s = T * r["steps"] / r["elapsed"]
    ms = 1e3 * r["elapsed"] / r["steps"]
    gu_ms = r["prof"]["gate_up_ms"]
    # packed W1+W3 bytes per launch: of the forwards that carried events, or
    # of all timed forwards when none did (--no-profile)
    gu_bytes = (r["bytes_gu_timed"] / r["timed_forwards"] if r["timed_forwards"]
                else r["bytes_gu"] / r["steps"])
    gu_gbps = gu_bytes / (gu_ms * 1e-3) / 1e9 if gu_ms > 0 else None
    fwd_gbps = (r["bytes_gu"] + r["bytes_dn"]) / r["elapsed"] / 1e9
    traffic = traffic_from_profiles(args.workload, T)
    if args.workload == "prefill":
        pairs = T * wl.k
        flops = 2.0 * pairs * 2 * wl.d * wl.F          # gate/up: 2 flops per weight per pair
        achieved = flops / (gu_ms * 1e-3) / 1e12 if gu_ms > 0 else None
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": (achieved or 0) / MFMA_F16_PEAK_TFLOPS, "traffic": traffic,
                "kernel": "gate_up (fused dequant + W1/W3 + SwiGLU)"}
    else:
        roof = {"bound": "hbm", "achieved": gu_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": (gu_gbps or 0) / HBM_PEAK_GBPS, "traffic": traffic,
                "kernel": "gate_up (fused dequant + W1/W3 + SwiGLU)",
                "bytes_per_launch": gu_bytes,
                "launches_timed": r["timed_forwards"],
                "launch_ms": gu_ms}
    name = "decode_fine, importance-skewed routing" if skewed else wl.name
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{name}: E={wl.E}, d_model={wl.d}, d_ff={wl.F} SwiGLU, "
                               f"top-{wl.k}, {T} tokens per step, "
                               + (f"avg {wl.budget_avg} bits/weight" if wl.budget_avg else f"bits {list(wl.bits)}"),
                   "E": wl.E, "d_model": wl.d, "d_ff": wl.F, "top_k": wl.k, "tokens": T,
                   "bits": b.bits, "pools_rotated": npools},
        "packed_weight_GBps": fwd_gbps,
        "packed_weight_frac_of_hbm": fwd_gbps / HBM_PEAK_GBPS,
        "kernels_ms_per_step": (dict(r_all["prof"])
                                if r_all else None),
        "down_GBps": (r_all["bytes_dn"] / r_all["steps"] / (r_all["prof"]["down_ms"] * 1e-3) / 1e9
                      if r_all and r_all["prof"]["down_ms"] > 0 else None),
        "mean_active_experts": r["mean_active"],
        "max_tokens_per_expert": r["max_tokens_per_expert"],
        "roofline": roof,
    }
    if not args.no_sweep and sweep_T:
        sw = {}
        for t in sweep_T:
            rs = b.run(t, args.steps, args.warmup, profile=0 if args.no_profile else 2, sample=sample)
            g = rs["prof"]["gate_up_ms"]
            sw[f"T={t}"] = {"tokens_per_s": t * rs["steps"] / rs["elapsed"],
                            "ms_per_step": 1e3 * rs["elapsed"] / rs["steps"],
                            "packed_weight_GBps": (rs["bytes_gu"] + rs["bytes_dn"]) / rs["elapsed"] / 1e9,
                            "gate_up_GBps": (rs["bytes_gu_timed"] / rs["timed_forwards"] / (g * 1e-3) / 1e9
                                             if g and rs["timed_forwards"] else None),
                            "mean_active_experts": rs["mean_active"]}
            if sw[f"T={t}"]["gate_up_GBps"]:
                sw[f"T={t}"]["gate_up_frac"] = sw[f"T={t}"]["gate_up_GBps"] / HBM_PEAK_GBPS
        out["sweep"] = sw
    if not args.no_cpu_baseline:
        sample_T = T if args.workload != "prefill" else 64
        cb, y_ref = cpu_baseline(b, sample_T, log)
        if args.workload == "prefill":
            cb["sample"] += " (64 of the 4096 tokens)"
        out["cpu_baseline"] = cb
        out["parity"] = parity_line(b, sample_T, y_ref)
        log(f"parity on the oracle's first batch: {out['parity']}")
    b.release()
    if default_run and not args.no_workloads:
        # the other configurations, each on its own layer (one at a time on
        # the device)
        wls = {}
        for key, w, bias, layout, prof in (
                ("decode_fine_T64", synth.WORKLOADS["decode_fine"], None, "eq2", "decode_fine"),
                ("decode_fine_skewed_T64", synth.WORKLOADS["decode_fine"], "skew", "eq2", "skewed"),
                ("decode_fine_bitplane_T64", synth.WORKLOADS["decode_fine"], None, "bitplane", "bitplane"),
                ("prefill_T4096", synth.WORKLOADS["prefill"], None, "eq2", "prefill")):
            t0 = time.time()
            res, _, _, gu_bytes = measure(w, w.T, args, log, 2 if w.name == "prefill" else args.pools,
                                          skew_bias(w) if bias else None, layout=layout)
            if bias:
                res["routing"] = "logits + log p_e (Zipf 1.1 importance)"
            # HBM bytes per gate/up launch from the committed counter summary
            # (null once the kernel sources changed), and its ratio to the
            # packed code bytes of the routed experts (decode)
            traffic = traffic_from_profiles(prof, w.T) if prof else None
            res["gate_up_traffic_bytes"] = traffic
            if traffic and w.name != "prefill":
                res["gate_up_traffic_over_code_bytes"] = traffic / gu_bytes
            wls[key] = res
            log(f"{key}: {res['tokens_per_s']:.0f} tokens/s ({time.time() - t0:.1f}s)")
        t0 = time.time()
        dyn = bench_dynamic(args, synth.WORKLOADS["dynamic"], log, cpu=False)
        wls["dynamic"] = {k: dyn[k] for k in ("value", "ms_per_step", "requant_GBps", "requant_s_total")}
        wls["dynamic"]["tokens_per_s"] = wls["dynamic"].pop("value")
        log(f"dynamic: {wls['dynamic']['tokens_per_s']:.0f} tokens/s ({time.time() - t0:.1f}s)")
        out["workloads"] = wls
    print(json.dumps(out), flush=True)


def cpu_requant_baseline(masters, wl, p, L, log, min_seconds=10.0):
    """The plain C++ oracle's re-precision on the host, one thread: Eq. 1
    solved for the first budget of the schedule (the library's measured loss
    table as input), then experts re-quantized from the fp16 masters into
    pages (max |w|, scale, codes, packed page), alternating 8/4/3 bits,
    until min_seconds; GB/s counts master bytes read plus page bytes
    written, as requant_GBps does."""
    from oracle import c_oracle
    W = [wl.W_e] * wl.E
    t0 = time.time()
    c_oracle.allocate(list(p), L, W, wl.budget_bits(wl.schedule[0]))
    t_solve = time.time() - t0
    total, nbytes, done = 0.0, 0.0, 0
    for e in range(wl.E):
        w = [m[e].cpu().float().numpy() for m in masters]   # fp16 -> fp32 exactly, not timed
        b = (8, 4, 3)[e % 3]
        t0 = time.time()
        c_oracle.quantize_expert(w[0], w[1], w[2], b)
        total += time.time() - t0
        nbytes += wl.W_e * (2 + b / 8)
        done += 1
        if total >= min_seconds:
            break
    log(f"oracle re-precision: solve {t_solve:.3f}s, {done} experts in {total:.1f}s")
    return {"value": nbytes / total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the plain C++ oracle, one thread: Eq. 1 for {wl.E} experts in {t_solve * 1e3:.1f} ms, then "
                      f"{done} experts re-quantized from fp16 masters into pages at 8/4/3 bits (master bytes read + "
                      f"page bytes written per second, as requant_GBps); {cpu_model()}"}


def bench_dynamic(args, wl, log, cpu=True):
    """40 decode steps of 64 tokens; the budget moves every 8 steps through
    avg 8, 6, 4, 3.5, 5 bits (re-quantization from the fp16 masters between
    steps). Reports end-to-end tokens/s and the requantize rate."""
    import torch

    import synth
    from mixed_precision_weight_page_amd import PagedMoELayer
    masters = synth.expert_weights(wl, device="cuda")
    layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=wl.T, master_dtype=wl.master)
    layer.bind_masters(*masters)
    layer.alloc_pool(layer.pool_bytes_for_bits([8] * wl.E))
    layer.alloc_workspace()
    p = synth.importance(wl)
    layer.set_budget(wl.budget_bits(wl.schedule[-1]), p)   # losses measured, warm
    steps = len(wl.schedule) * wl.steps_per_phase
    batches = [synth.tokens(wl, device="cuda", step=i) for i in range(steps)]
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        layer.moe_forward(*batches[0], y)
    torch.cuda.synchronize()
    prev = None
    req_bytes = 0
    # each budget change bracketed by events on the stream the library uses
    # (torch's current stream), so its time is the GPU's re-precision work
    # and not the forwards still queued before it
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(len(wl.schedule))]
    t0 = time.perf_counter()
    for i in range(steps):
        if i % wl.steps_per_phase == 0:
            e0, e1 = ev[i // wl.steps_per_phase]
            e0.record()
            bits = layer.set_budget(wl.budget_bits(wl.schedule[i // wl.steps_per_phase]), p)
            e1.record()
            changed = [e for e in range(wl.E) if prev is None or bits[e] != prev[e]]
            req_bytes += sum(wl.W_e * (2 + bits[e] / 8) for e in changed)
            prev = bits
        layer.moe_forward(*batches[i], y)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    t_req = sum(a.elapsed_time(b) for a, b in ev) / 1e3
    out = {"metric": METRIC, "value": wl.T * steps / el, "unit": "tokens/s", "n_gpus": 1,
           "steps": steps, "warmup": args.warmup, "ms_per_step": 1e3 * el / steps,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic",
           "config": {"workload": "dynamic: E=128, d_model=2048, d_ff=768, top-8, 64 tokens, fp16 "
                                  "masters, budget avg 8->6->4->3.5->5 bits every 8 steps"},
           "requant_GBps": req_bytes / t_req / 1e9 if t_req else None,
           "requant_s_total": t_req}
    if cpu and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_requant_baseline(masters, wl, p, layer.get_loss_table(), log)
    del layer, masters, batches
    torch.cuda.empty_cache()
    return out


def bench_kvtrace(args, wl, log):
    """The dynamic layer (fp16 masters) under the KV-pressure budget
    scheduler: 128 decode steps of 64 tokens (the first, which makes the first
    allocation, untimed); before each forward one
    pw_budget_step with the KV-cache occupancy of a synthetic trace (peaking
    near the all-8-bit pool size; memory = the all-8-bit pool plus 1/8,
    reserve 1/16, headroom 5%, at least 4 steps between a change and a grow).
    Reports end-to-end tokens/s including the re-quantizations."""
    import torch

    import synth
    from mixed_precision_weight_page_amd import BUDGET_KEEP, PagedMoELayer
    masters = synth.expert_weights(wl, device="cuda")
    layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=wl.T, master_dtype=wl.master)
    layer.bind_masters(*masters)
    pool8 = layer.pool_bytes_for_bits([8] * wl.E)
    layer.alloc_pool(pool8)
    layer.alloc_workspace()
    p = synth.importance(wl)
    layer.get_loss_table()            # statistics measured once, outside the timed steps
    memory, reserve, h, n = pool8 + pool8 // 8, pool8 // 16, 0.05, 4
    steps = 128
    trace = synth.kv_trace(steps, pool8)
    batches = [synth.tokens(wl, device="cuda", step=i) for i in range(8)]
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device="cuda")
    layer.budget_step(memory, reserve, h, n, trace[0], p)      # first allocation (INIT), untimed
    for _ in range(args.warmup):
        layer.moe_forward(*batches[0], y)
    torch.cuda.synchronize()
    actions, bits_sum = [], 0.0
    t0 = time.perf_counter()
    for i in range(1, steps):
        act, B, pressure = layer.budget_step(memory, reserve, h, n, trace[i], p)
        actions.append(act)
        bits_sum += B / (wl.E * wl.W_e)
        layer.moe_forward(*batches[i % 8], y)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    changes = sum(1 for a in actions if a != BUDGET_KEEP)
    timed = steps - 1
    out = {"metric": METRIC, "value": wl.T * timed / el, "unit": "tokens/s", "n_gpus": 1,
           "steps": timed, "warmup": args.warmup, "ms_per_step": 1e3 * el / timed,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic",
           "config": {"workload": "kvtrace: dynamic layer (E=128, d_model=2048, d_ff=768, top-8, 64 tokens, "
                                  "fp16 masters) under the KV-pressure budget scheduler over a synthetic "
                                  "KV-cache trace"},
           "budget_changes": changes, "shrinks": actions.count(1), "grows": actions.count(2),
           "mean_budget_bits_per_weight": bits_sum / timed}
    print(json.dumps(out), flush=True)


def bench_swap(args, wl, log, T=8, slots=32):
    """The decode_fine layer with its pages in a pinned host tier and 32
    device slots for its 128 experts: T = 8 tokens per step, logits N(0, 1)
    plus log p_e (routing in proportion to importance), 5 warm-up and
    `steps` timed forwards (at least 200). Reports tokens/s with the hits,
    copies and host reads the timed steps made, and the same steps with
    every page in the device pool for comparison."""
    import numpy as np
    import torch

    import synth
    from mixed_precision_weight_page_amd import PagedMoELayer
    masters = synth.expert_weights(wl, device="cuda")
    p = np.asarray(synth.importance(wl), dtype=np.float64)
    bias = torch.tensor(np.log(p), dtype=torch.float32, device="cuda")
    steps = max(200, args.steps)
    batches = []
    for i in range(64):
        x, lg = synth.tokens(wl, T=T, device="cuda", step=i)
        batches.append((x, (lg + bias).contiguous()))
    y = torch.empty((T, wl.d), dtype=torch.float32, device="cuda")

    def layer_with(host_tier):
        layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=T, master_dtype=wl.master)
        layer.bind_masters(*masters)
        layer.alloc_workspace()
        if host_tier:
            layer.alloc_host_tier(layer.pool_bytes_for_bits([8] * wl.E))
            layer.alloc_pool(slots * layer.slot_bytes())
        else:
            layer.alloc_pool(layer.pool_bytes_for_bits([8] * wl.E))
        layer.set_budget(wl.budget_bits(), p)
        torch.cuda.synchronize()
        return layer

    def timed(layer):
        for i in range(args.warmup):
            layer.moe_forward(*batches[i % 64], y)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            layer.moe_forward(*batches[i % 64], y)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    tiered = layer_with(True)
    _, st0 = tiered.residency()
    el = timed(tiered)
    _, st1 = tiered.residency()
    table = tiered.get_page_table()
    mean_page = float(np.mean([t["nbytes"] for t in table]))
    d = {k: st1[k] - st0[k] for k in st1}
    routed = d["hits"] + d["copies"] + d["host_reads"]
    del tiered
    resident = layer_with(False)
    el_res = timed(resident)
    log(f"swap: {d} over {steps + args.warmup} forwards")
    out = {"metric": METRIC, "value": T * steps / el, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
           "warmup": args.warmup, "ms_per_step": 1e3 * el / steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": {"workload": f"swap: decode_fine layer (E=128, d_model=2048, d_ff=768, top-8, avg 4 bits) "
                                  f"with its pages in pinned host memory and {slots} device page slots, "
                                  f"{T} tokens per step routed in proportion to importance",
                      "slots": slots, "tokens": T},
           "hit_rate": d["hits"] / routed if routed else None,
           "pages_copied_per_step": d["copies"] / (steps + args.warmup),
           "host_reads_per_step": d["host_reads"] / (steps + args.warmup),
           "host_link_GBps": (d["copies"] + d["host_reads"]) * mean_page / (el * (steps + args.warmup) / steps) / 1e9,
           "all_resident_tokens_per_s": T * steps / el_res}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
