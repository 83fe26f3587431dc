#!/usr/bin/env python3
"""Benchmark of the MiLo W3A16 + low-rank MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C2|C3|C4|C5|C1] [--batch T]

A step is one pass of the whole hot path over one batch of synthetic tokens:
route (softmax top-k + expert sort) -> low-rank pre-pass + fused gate/up
W3A16 GEMM with SwiGLU -> low-rank pre-pass + fused down W3A16 GEMM with
route scaling -> slot combine.  C5 steps through 32 layers.  Weights are
seeded random (RTN int3 g64 on the GPU); inputs are resident in HBM before the
timed region; single-layer workloads rotate through --copies independent
weight sets so that the 256 MB last-level cache cannot serve the weights.

Prints ONE JSON line.  The default workload is C2 (Mixtral-8x7B-shaped MoE FFN
at decode, 16 tokens), the configuration the metric is quoted on.
"""
import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
REL_FRO_TOL, MAX_ABS_TOL = 1e-3, 2e-2   # fp16 outputs vs the float64 oracle
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores
METRIC = "MoE-layer tokens/s + achieved HBM TB/s (decode) / MFMA % (prefill)"

WORKLOAD_TEXT = {
    "C1": "single expert linear, X 16x512 fp16, W 1024x512 int3 g64, rank 16 compensator",
    "C2": "Mixtral-8x7B-shaped MoE FFN decode: 16 tokens, H=4096, F=14336, 8 experts top-2 "
          "(renormalised softmax), SwiGLU, int3 g64 weights, per-expert ranks from {16,32,64}",
    "C3": "Mixtral-8x7B-shaped MoE FFN prefill: 4096 tokens, H=4096, F=14336, 8 experts top-2, "
          "int3 g64, ranks from {16,32,64}",
    "C4": "DeepSeekMoE-16B-shaped layer: 256 tokens, H=2048, 64 routed experts (F=1408) top-6 "
          "+ 2 shared (rank 32), Zipf(1.2) router skew, int3 g64, ranks from {8,16,32}",
    "C5": "32 Mixtral-8x7B-shaped MoE blocks (int3 g64 + rank {16,32,64} compensators resident), decode",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C2", choices=["C1", "C2", "C3", "C4", "C5"])
    ap.add_argument("--batch", type=int, default=None, help="tokens (C5 sweep: 1/8/32/64)")
    ap.add_argument("--copies", type=int, default=8,
                    help="weight sets rotated per step (8 x 650 MB at C2: neither the codes nor "
                         "the compensator factors of all sets fit the 256 MB last-level cache)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-prefill", action="store_true",
                    help="C2 only: skip the prefill (C3) sub-record measured in the same run")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-check-tokens", type=int, default=2)
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="run the workload's steps for this long before the warm-up, so the card "
                         "is at its sustained clock when the timed steps start")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per step in the timed region instead of "
                         "launching every call from Python (measured slower on this stack: C2 "
                         "0.174 vs 0.153 ms per step)")
    ap.add_argument("--lr", default="fp16", choices=["fp16", "int3"],
                    help="storage of the compensator factors U, V")
    ap.add_argument("--build", action="store_true",
                    help="time the offline compensator construction (quantize <-> rank-64 SVD refinement) of "
                         "one Mixtral-shaped 14336x4096 weight matrix instead of the MoE layer")
    ap.add_argument("--ranks", action="store_true",
                    help="time the adaptive-rank inputs (kurtosis of all 24 expert matrices of a "
                         "Mixtral-shaped layer, routed pairs per expert) and run the rank policy")
    ap.add_argument("--quantizer", default="rtn", choices=["rtn", "hqq"],
                    help="--build: quantizer of the refinement rounds")
    ap.add_argument("--hqq", action="store_true",
                    help="time the HQQ-style int3 quantizer on one Mixtral-shaped 14336x4096 matrix")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only measure plain device read (sum) and copy bandwidth on 4 GiB")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times "
                         "(calibrates HBM byte counters against a known size)")
    return ap.parse_args()


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def src_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
class Layer:
    """One MoE layer's device weights, buffers and prebuilt call descriptors."""

    def __init__(self, m, cfg, layer_idx, X, logits, path, lr_format="fp16"):
        import synth
        import torch
        L = m._lib
        self.m, self.cfg = m, cfg
        self.layer_idx = layer_idx
        self.lr_format = lr_format
        self.ranks = synth.gen_ranks(cfg, layer_idx)
        ET = cfg.E + cfg.S
        fam = {}
        for n, a, b in (("W1", "A1", "B1"), ("W3", "A3", "B3"), ("W2", "A2", "B2")):
            Ws, As, Bs = [], [], []
            for e in range(ET):
                d = synth.gen_expert(cfg, layer_idx, e, self.ranks[e], device="cuda", which=(n,))
                Ws.append(d[n])
                As.append(d[a])
                Bs.append(d[b])
            fam[n] = m.Family.from_dense(Ws, As, Bs, max_rank=max(self.ranks), lr_format=lr_format)
            del Ws
        self.fam = fam
        T, slots = cfg.T, cfg.slots
        P = T * slots
        dev = "cuda"
        self.X, self.logits = X, logits
        self.route = {
            "ids": torch.empty((T, cfg.k), dtype=torch.int32, device=dev),
            "w": torch.empty((T, cfg.k), dtype=torch.float32, device=dev),
            "slot_w": torch.empty(P, dtype=torch.float32, device=dev),
            "sorted_pairs": torch.empty(P, dtype=torch.int32, device=dev),
            "pair_pos": torch.empty(P, dtype=torch.int32, device=dev),
            "offsets": torch.empty(ET + 1, dtype=torch.int32, device=dev),
        }
        self.route_wsb = int(L.lib().milo_route_workspace_bytes(T, cfg.E, cfg.k, cfg.S))
        self.route_ws = torch.empty(max(self.route_wsb, 256), dtype=torch.uint8, device=dev)
        self.G = torch.empty((P, cfg.F), dtype=torch.float16, device=dev)
        self.Y = torch.empty((P, cfg.H), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, cfg.H), dtype=torch.float16, device=dev)
        r = self.route
        self.d13 = m.ops.make_gemm_desc((fam["W1"], fam["W3"]), X, r["offsets"], P, L.EPI_SWIGLU,
                                        self.G, sorted_pairs=r["sorted_pairs"], gather_div=slots,
                                        max_rows_per_expert=T, path=path)
        self.d2 = m.ops.make_gemm_desc((fam["W2"],), self.G, r["offsets"], P, L.EPI_ROUTE_SCALE,
                                       self.Y, sorted_pairs=r["sorted_pairs"], gather_div=0,
                                       slot_w=r["slot_w"], y_rows=P, max_rows_per_expert=T, path=path)
        self.d13.flags = L.GEMM_PREPASS_DONE
        self.d2.flags = L.GEMM_PREPASS_DONE
        lib = L.lib()
        need = max(lib.milo_moe_gemm_workspace_bytes(C.byref(self.d13)),
                   lib.milo_moe_gemm_workspace_bytes(C.byref(self.d2)))
        assert need > 0, need
        self.ws_need = need
        self.ws = None            # shared workspace, attached once all layers exist
        self.P, self.T, self.slots = P, T, slots

    def step(self, stream, ev13=None):
        L = self.m._lib
        lib = L.lib()
        r = self.route
        p = lambda t: C.c_void_p(t.data_ptr())
        cfg = self.cfg
        chk = L.check
        chk("route", lib.milo_route_sort(p(self.logits), cfg.T, cfg.E, cfg.k, cfg.S,
                                         1 if cfg.renormalize else 0, p(r["ids"]), p(r["w"]),
                                         p(r["slot_w"]), p(r["sorted_pairs"]), p(r["pair_pos"]),
                                         p(r["offsets"]), p(self.route_ws), self.route_wsb, stream))
        wsp, wsb = p(self.ws), self.ws.numel()
        chk("prepass13", lib.milo_moe_lowrank_prepass(C.byref(self.d13), wsp, wsb, stream))
        if ev13 is not None:
            TIMER.record(ev13[0], stream)
        chk("gemm13", lib.milo_moe_w3a16_lowrank_gemm(C.byref(self.d13), wsp, wsb, stream))
        if ev13 is not None:
            TIMER.record(ev13[1], stream)
        chk("prepass2", lib.milo_moe_lowrank_prepass(C.byref(self.d2), wsp, wsb, stream))
        chk("gemm2", lib.milo_moe_w3a16_lowrank_gemm(C.byref(self.d2), wsp, wsb, stream))
        chk("combine", lib.milo_moe_combine(p(self.Y), cfg.T, self.slots, cfg.H, p(self.out), stream))

    # algorithmic bytes / flops from the routed row counts (host copies)
    def work(self, offsets):
        """Kernel- and step-level work of one layer step.  Step bytes count
        what the layer must move: the touched experts' packed codes,
        scale/zero and compensator factors, the activations read and the
        output written; the intermediates (G, per-slot Y, low-rank products,
        gathered rows) are reported separately.  The gate/up kernel's own
        bytes (the roofline line) are its weights, factors U, gathered rows,
        low-rank products and its output G."""
        cfg = self.cfg
        H, F = cfg.H, cfg.F
        rows = [int(offsets[e + 1] - offsets[e]) for e in range(cfg.E + cfg.S)]
        b13 = b2 = 0
        f13 = f2 = 0
        touched = 0
        q3 = self.lr_format == "int3"
        # compensator factor bytes: fp16, or int3 codes + fp16 scale/zero words
        # (U: one group per output row; V: groups of 64 along the input)
        u_bytes = (lambda n, r: n * r * 3 // 8 + (4 * n if r else 0)) if q3 else (lambda n, r: n * r * 2)
        v_bytes = (lambda r, k: r * k * 3 // 8 + r * (k // 64) * 4) if q3 else (lambda r, k: r * k * 2)
        w_bytes = lambda n, k: 3 * n * k // 8 + n * k // 16      # packed int3 + scale/zero
        wt = lr = 0
        inter = 0
        for e, M in enumerate(rows):
            if M == 0:
                continue
            touched += 1
            r = self.ranks[e]
            wt += 2 * w_bytes(F, H) + w_bytes(H, F)
            lr += 2 * (u_bytes(F, r) + v_bytes(r, H)) + u_bytes(H, r) + v_bytes(r, F)
            # gate/up kernel: W1, W3 + U1, U3, gathered X rows, T rows, G written
            b13 += 2 * (w_bytes(F, H) + u_bytes(F, r)) + M * H * 2 + M * 2 * r * 2 + M * F * 2
            b2 += w_bytes(H, F) + u_bytes(H, r) + M * F * 2 + M * r * 2 + M * H * 4
            f13 += 2 * M * 2 * F * H + 2 * M * 2 * r * (H + F)
            f2 += 2 * M * H * F + 2 * M * r * (H + F)
            # intermediates: G written and read, Y written and read, T13 / T2
            # written and read, gathered activation rows
            inter += 2 * M * F * 2 + 2 * M * H * 4 + 2 * (M * 2 * r * 2 + M * r * 2) + M * H * 2
        io = cfg.T * H * 2 * 2                                  # X read + out written
        return {"rows": rows, "touched": touched, "bytes13": b13, "bytes2": b2, "flops13": f13,
                "flops2": f2, "layer_bytes": wt + lr + io, "layer_flops": f13 + f2,
                "weight_bytes": wt, "compensator_bytes": lr, "io_bytes": io, "intermediate_bytes": inter}


def cpu_baseline(cfg, layer, budget_s):
    """The CPU oracle (float64 NumPy, as it stands) on a bounded sample of the
    same layer: routing of all tokens plus the expert FFNs of as many touched
    experts as fit the time budget, scaled to the whole layer.  Its results
    are kept: the per-slot outputs Y of the sampled experts and the outputs
    of the tokens whose every slot was sampled are compared with the GPU's
    (layer.Y / layer.out from the last timed step on this weight set)."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    X = layer.X.cpu().numpy()
    logits = layer.logits.cpu().numpy()
    t0 = time.perf_counter()
    rt = oracle.route_ref(logits, cfg.k, cfg.S, cfg.renormalize)
    t_route = time.perf_counter() - t0
    sp, off = rt["sorted_pairs"], rt["offsets"]
    slot_w = rt["slot_w"].reshape(-1)
    touched = [e for e in range(cfg.E + cfg.S) if off[e + 1] > off[e]]
    done, t_exp, pairs_done = [], 0.0, 0
    y_ref = {}
    for e in touched:
        exp = synth.gen_expert(cfg, layer.layer_idx, e, layer.ranks[e], device="cuda")
        qe = oracle.quantize_expert({k: v.cpu() for k, v in exp.items()},
                                    lr_format=layer.lr_format)              # offline, untimed
        seg = sp[off[e]:off[e + 1]]
        rows = X[seg // cfg.slots]
        t1 = time.perf_counter()
        _, y = oracle.expert_ffn_ref(rows, qe)
        t_exp += time.perf_counter() - t1
        for i, s in enumerate(seg):
            y_ref[int(s)] = y[i] * slot_w[s]
        done.append(e)
        pairs_done += seg.size
        del qe
        if t_exp > budget_s:
            break
    scale = cfg.P / max(pairs_done, 1)
    layer_s = t_route + t_exp * scale
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    # the check of the timed output
    slots = sorted(y_ref)
    Yg = layer.Y.cpu().numpy().astype(np.float64)
    check = {"what": f"per-slot route-weighted expert outputs Y of {len(slots)} of {cfg.P} slots"}
    rf_y = oracle.rel_fro(Yg[slots], np.stack([y_ref[s] for s in slots]))
    ma_y = oracle.max_abs(Yg[slots], np.stack([y_ref[s] for s in slots]))
    full = [t for t in range(cfg.T) if all((t * cfg.slots + j) in y_ref for j in range(cfg.slots))]
    check.update({"Y_rel_fro": rf_y, "Y_max_abs": ma_y, "tokens_checked": len(full)})
    if full:
        out_ref = np.stack([sum(y_ref[t * cfg.slots + j] for j in range(cfg.slots)) for t in full])
        og = layer.out.cpu().numpy().astype(np.float64)[full]
        check["out_rel_fro"] = oracle.rel_fro(og, out_ref)
        check["out_max_abs"] = oracle.max_abs(og, out_ref)
    check["pass"] = bool(max(rf_y, check.get("out_rel_fro", 0.0)) <= REL_FRO_TOL and
                         max(ma_y, check.get("out_max_abs", 0.0)) <= MAX_ABS_TOL)
    return {
        "value": cfg.T / layer_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": f"oracle.route_ref on all {cfg.T} tokens + oracle.expert_ffn_ref (float64 dequant + "
                  f"matmul) for {len(done)} of {len(touched)} touched experts ({pairs_done} of {cfg.P} "
                  f"pairs) in {t_route + t_exp:.1f} s, scaled x{scale:.2f} by pairs to the whole layer",
        "layer_seconds": layer_s,
        "cpu_model": cpu_model(),
        "host_cpus_available": len(os.sched_getaffinity(0)),
    }, check


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def device_info(timer):
    """GPU name, compute units and clocks: the runtime's figures, and the
    shader clock the driver reports after the timed region (best effort)."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    arch = getattr(pr, "gcnArchName", None)
    # some driver installs report no marketing name (their device id table
    # is missing); the architecture then names the part
    name = pr.name or f"unnamed by the driver ({(arch or '?').split(':')[0]})"
    info = {"gpu": name, "arch": arch, "compute_units": pr.multi_processor_count}
    v = C.c_int()
    h = timer.h
    h.hipDeviceGetAttribute.argtypes = [C.POINTER(C.c_int), C.c_int, C.c_int]
    HIP_ATTR_CLOCK_RATE = 5            # kHz, peak
    if h.hipDeviceGetAttribute(C.byref(v), HIP_ATTR_CLOCK_RATE, 0) == 0:
        info["peak_clock_mhz"] = v.value // 1000
    # the current shader clock level from the driver's sysfs table (the line
    # marked '*'); a file read, so no helper program is started
    try:
        import glob
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        info["sclk_after_run"] = line.split(":", 1)[1].replace("*", "").strip()
                        break
            if "sclk_after_run" in info:
                break
    except Exception:
        pass
    return info


class HipTimer:
    """HIP timing events on the library's stream.  They are created with
    hipEventDisableSystemFence: a default event ends with a system-scope
    release (an L2 writeback) that costs several microseconds between the
    kernels it brackets; a timing-only event needs no such fence, and the
    device-wide synchronize before the read-out orders everything."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.h = C.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
        self.h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]

    def event(self):
        e = C.c_void_p()
        rc = self.h.hipEventCreateWithFlags(C.byref(e), self.DISABLE_SYSTEM_FENCE)
        assert rc == 0, f"hipEventCreateWithFlags: {rc}"
        return e

    def record(self, e, stream):
        rc = self.h.hipEventRecord(e, C.c_void_p(stream))
        assert rc == 0, f"hipEventRecord: {rc}"

    def ms(self, a, b):
        f = C.c_float()
        rc = self.h.hipEventElapsedTime(C.byref(f), a, b)
        assert rc == 0, f"hipEventElapsedTime: {rc}"
        return f.value


TIMER = None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): there is no "
              "multi-GPU path; the MoE layer is measured on one MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    import extreme_quantized_moe_amd as m
    import synth
    from synth import configs as SC

    torch.cuda.set_device(0)
    if args.hbm_probe:
        n = 4 << 30
        x = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        y = torch.empty_like(x)
        out = {}
        for name, fn, nbytes in (("read_sum", lambda: x.sum(), n), ("copy", lambda: y.copy_(x), 2 * n)):
            fn()
            torch.cuda.synchronize()
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record()
            for _ in range(10):
                fn()
            e_.record()
            torch.cuda.synchronize()
            out[name + "_GBps"] = round(10 * nbytes / (s_.elapsed_time(e_) * 1e-3) / 1e9, 1)
        print(json.dumps({"hbm_probe_bytes": n, **out}))
        return
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": n, "copies": 5}))
        return
    if args.build:
        return bench_build(args, m)
    if args.ranks:
        return bench_ranks(args, m)
    if args.hqq:
        return bench_hqq(args, m)
    cfg = SC.get_config(args.config)
    if args.config == "C1":
        return bench_c1(args, m, cfg)
    if args.batch:
        cfg = cfg.with_(T=args.batch)
    path = {"auto": 0, "decode": 1, "prefill": 2}[args.path]
    global TIMER
    TIMER = HipTimer()
    GRAPH[0] = args.graph
    SETTLE_S[0] = args.settle_ms / 1000.0
    run = run_workload(m, cfg, args.config, cfg.layers if cfg.layers > 1 else args.copies, path, args.lr,
                       args.steps, args.warmup)
    ms_step = run["ms_step"]
    tokens_per_s = cfg.T / (ms_step / 1000.0)
    roof = run["roofline"]
    comp = run["work"]
    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}",
            "tokens": cfg.T, "layers": cfg.layers, "experts": cfg.E, "shared": cfg.S, "top_k": cfg.k,
            "hidden": cfg.H, "ffn": cfg.F, "weight_sets_rotated": run["nsets"],
            "touched_experts": run["touched"],
            "step_alg_bytes": int(comp["layer_bytes"]), "step_alg_flops": int(comp["layer_flops"]),
            "step_intermediate_bytes": int(comp["intermediate_bytes"]),
            "achieved_TBps_step": round(comp["layer_bytes"] / (ms_step * 1e-3) / 1e12, 3),
            "achieved_TFLOPs_step": round(comp["layer_flops"] / (ms_step * 1e-3) / 1e12, 2),
            "compensator_share": {
                "of_step_bytes": round(comp["compensator_bytes"] / comp["layer_bytes"], 4),
                "of_resident_weights": run["resident_comp_share"]},
            "host_seconds_timed": run["host_s"],
            "settle": {"ms": args.settle_ms, "steps": run["settle_steps"]},
            "launch": run["launch"],
            "step_ms_p10_p50_p90_event_pass": run["pcts"],
            "path": args.path,
            "compensator_factors": args.lr,
        },
        "roofline": roof,
    }
    res["device"] = device_info(TIMER)
    if args.config == "C2" and not args.no_prefill and args.path == "auto" and not args.batch:
        # the prefill half of the metric, measured in the same run: the same
        # Mixtral-shaped layer at 4096 tokens (matrix-core path)
        c3 = SC.get_config("C3")
        log("prefill sub-record: C3")
        pr = run_workload(m, c3, "C3", 1, 0, args.lr, args.prefill_steps, 2)
        pc = pr["work"]
        res["prefill"] = {
            "workload": f"C3: {WORKLOAD_TEXT['C3']}",
            "ms_per_step": round(pr["ms_step"], 4),
            "tokens_per_s": round(c3.T / (pr["ms_step"] * 1e-3), 1),
            "steps": args.prefill_steps,
            "step_alg_flops": int(pc["layer_flops"]),
            "achieved_TFLOPs_step": round(pc["layer_flops"] / (pr["ms_step"] * 1e-3) / 1e12, 2),
            "mfma_frac_step": round(pc["layer_flops"] / (pr["ms_step"] * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "roofline": pr["roofline"],
        }
        if not args.no_cpu:
            res["prefill"]["check"] = prefill_check(c3, pr["layers"][0], args.prefill_check_tokens)
            del pr
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"], res["check"] = cpu_baseline(cfg, run["layers"][0], args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))
    ok = res.get("check", {}).get("pass", True) and res.get("prefill", {}).get("check", {}).get("pass", True)
    if not ok:
        log("the timed output does not match the oracle (see check)")
        sys.exit(3)


GRAPH = [False]   # --graph: replay one captured HIP graph per step in the timed region
SETTLE_S = [0.25]  # --settle-ms: wall time of steps run before the warm-up


def run_workload(m, cfg, name, nsets, path, lr, steps, warmup):
    """Build nsets weight sets of a workload (one per layer for a stack),
    warm up, time `steps` steps with HIP events on the library's stream (only
    the two bracketing the steps), run them once more with per-step and
    per-kernel events, and account the work."""
    import torch
    import synth
    stack = cfg.layers > 1
    log(f"building {nsets} weight set(s) of {name} (T={cfg.T}) on the GPU")
    X = synth.gen_tokens(cfg, 0, device="cuda")
    t0 = time.time()
    layers = []
    for i in range(nsets):
        logits = synth.gen_logits(cfg, i if stack else 0, device="cuda")
        layers.append(Layer(m, cfg, i if stack else 0, X, logits, path, lr) if (stack or i == 0)
                      else Layer(m, cfg, 100 + i, X, logits, path, lr))
    ws = torch.zeros(max(lay.ws_need for lay in layers), dtype=torch.uint8, device="cuda")
    for lay in layers:
        lay.ws = ws
    torch.cuda.synchronize()
    log(f"weights ready in {time.time() - t0:.1f} s")
    stream = torch.cuda.current_stream().cuda_stream

    def run_step(i, ev=None):
        if stack:
            for li, lay in enumerate(layers):
                lay.step(stream, ev if li == 0 else None)
        else:
            layers[i % nsets].step(stream, ev)

    # Settle: run the workload's own steps for SETTLE_S seconds of wall time
    # before the warm-up.  The card raises its clocks only under sustained
    # load: measured on C2, the first 50 steps after 10 warm-up steps ran at
    # 0.158 ms, after 0.2 s idle at 0.173 ms, and from about 60 ms of load on
    # at 0.143 ms; timing a cold card would report its power ramp, not the
    # kernels.  Not part of the K timed steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S[0]:
        for _ in range(8):
            run_step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    # With --graph: one HIP graph per distinct step (per weight set; the whole
    # stack for a multi-layer workload), captured from the same library calls,
    # so a replay enqueues the step's kernels in one host call.  The library
    # allocates, synchronizes and clears nothing, so its calls capture as they
    # are; the outputs checked after the timed region come from the replays.
    # (Measured: the replays run slower than the eager launches here.)
    graphs = []
    if GRAPH[0]:
        for i in range(1 if stack else nsets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cap = torch.cuda.current_stream().cuda_stream
                if stack:
                    for lay in layers:
                        lay.step(cap)
                else:
                    layers[i].step(cap)
            graphs.append(g)
        for i in range(max(2, warmup)):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
    # the timed region: the K steps and nothing else on the stream between its
    # two events (an event between kernels costs about 2.5 us of its own)
    start, stop = TIMER.event(), TIMER.event()
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    TIMER.record(start, stream)
    for i in range(steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            run_step(i)
    TIMER.record(stop, stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    ms_step = TIMER.ms(start, stop) / steps
    # kernel pass, after the timed region: the same K steps again with events
    # at the step boundaries and around the gate/up GEMM call, for the
    # per-launch duration of the roofline line and the spread of step times
    evs = [(TIMER.event(), TIMER.event()) for _ in range(steps)]
    marks = [TIMER.event() for _ in range(steps + 1)]
    TIMER.record(marks[0], stream)
    for i in range(steps):
        run_step(i, evs[i])
        TIMER.record(marks[i + 1], stream)
    torch.cuda.synchronize()
    step_ms = sorted(TIMER.ms(marks[i], marks[i + 1]) for i in range(steps))
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(q * (len(step_ms) - 1) + 0.5))]
    k13_us = sum(TIMER.ms(a, b) for a, b in evs) / len(evs) * 1000.0

    # work accounting (after the timed region)
    works = [lay.work(lay.route["offsets"].cpu().numpy()) for lay in layers]
    keys = ("layer_bytes", "layer_flops", "bytes13", "flops13", "weight_bytes", "compensator_bytes",
            "io_bytes", "intermediate_bytes")
    if stack:
        comp = {k: sum(w[k] for w in works) for k in keys}
        comp["bytes13"], comp["flops13"] = works[0]["bytes13"], works[0]["flops13"]
    else:
        used = [works[i % nsets] for i in range(steps)]
        comp = {k: sum(w[k] for w in used) / len(used) for k in keys}
    # share of the compensator factors in the resident expert weights (layer 0)
    fams = layers[0].fam.values()
    nb = [f.nbytes() for f in fams]
    comp_b = sum(v for d in nb for k, v in d.items() if k not in ("packed", "sz"))
    resident_comp = round(comp_b / sum(sum(d.values()) for d in nb), 4)
    prefill = cfg.T * cfg.k / cfg.E > 64
    pairs = cfg.T * (cfg.k + cfg.S)
    ET = cfg.E + cfg.S
    # the kernels the library's automatic path launches for the gate/up call
    # (the host plan's rules, with the row bound the bench passes: T)
    small = cfg.F * cfg.H <= (1 << 22)
    if path == 1 or (path == 0 and (cfg.T <= 16 or (cfg.T <= 32 and not small))):
        kname = "gemm_decode_kernel<MT,2> (gate/up + SwiGLU)"
    elif path == 0 and cfg.T <= 32:
        kname = "gemm_decode_kernel<2,2> (gate/up + SwiGLU, two m-tiles)"
    elif path == 0 and not small and cfg.T <= 128 and pairs < 32 * ET:
        kname = "gemm_decode_kernel<1,2> (gate/up + SwiGLU, experts above 16 rows in chunks)"
    elif prefill and (path == 2 or pairs >= 256 * ET):
        kname = "gemm_prefill_kernel<2,...,128> (gate/up + SwiGLU)"
    elif path == 2 or (small and pairs >= 16 * ET) or pairs >= 64 * ET:
        kname = "gate/up call: 64-row tile kernel for every expert (gemm_prefill_persistent<2,...>)"
    else:
        kname = "gate/up call: gemm_decode_kernel<MT,2> + gemm_prefill_persistent<2,...> (both paths)"
    k_bytes, k_flops = comp["bytes13"], comp["flops13"]
    if prefill:
        achieved = k_flops / (k13_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        achieved = k_bytes / (k13_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(name, cfg.T, lr)}
    roof.update({"kernel": kname, "alg_bytes_per_launch": int(k_bytes), "alg_flops_per_launch": int(k_flops),
                 "avg_launch_us": round(k13_us, 2)})
    return {"ms_step": ms_step, "pcts": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
            "host_s": round(t_host, 3), "roofline": roof, "settle_steps": settle_steps,
            "launch": ("one captured HIP graph per step, replayed" if graphs else "eager calls from Python"), "work": comp, "touched": works[0]["touched"],
            "nsets": nsets, "layers": layers, "resident_comp_share": resident_comp}


def prefill_check(cfg, layer, ntok):
    """Sampled oracle check of the prefill layer: every output column of
    ntok tokens (their expert FFNs recomputed in full width in float64)."""
    import numpy as np
    import oracle
    import synth
    toks = [0, cfg.T - 1, cfg.T // 2, cfg.T // 3][:max(1, ntok)]
    X = layer.X.cpu().numpy()[toks]
    logits = layer.logits.cpu().numpy()[toks]

    def get_expert(e):
        d = synth.gen_expert(cfg, layer.layer_idx, e, layer.ranks[e], device="cuda")
        return oracle.quantize_expert({k: v.cpu() for k, v in d.items()}, lr_format=layer.lr_format)

    ref = oracle.moe_layer_ref(X, logits, get_expert, cfg.k, cfg.S, cfg.renormalize)["out"]
    got = layer.out.cpu().numpy().astype(np.float64)[toks]
    rf, ma = oracle.rel_fro(got, ref), oracle.max_abs(got, ref)
    return {"what": f"layer output of tokens {toks}, all {cfg.H} columns", "out_rel_fro": rf, "out_max_abs": ma,
            "pass": bool(rf <= REL_FRO_TOL and ma <= MAX_ABS_TOL)}


def traffic_for(config, T, lr="fp16"):
    """Measured HBM traffic of the dominant kernel from a committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    f = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(f):
        return None
    try:
        d = json.load(open(f))
        ent = d.get(f"{config}_T{T}" + ("" if lr == "fp16" else f"_{lr}"))
        if not ent or ent.get("src_hash") != src_hash(ent.get("src_files", [])):
            return None
        return ent.get("bytes_per_launch")
    except Exception:
        return None


def bench_build(args, m):
    """Offline compensator construction of one Mixtral-shaped gate matrix:
    iters rounds of (RTN int3 of W - L, residual, rank-r randomized SVD with q
    power iterations).  Reported per matrix; the roofline line is the whole
    call's algorithmic fp32 flops against the fp32 vector peak (its big
    products are fp32 FMA on the vector units)."""
    import torch
    import synth
    from synth import configs as SC
    N, K, r, p, q, iters = 14336, 4096, 64, 16, 2, 2
    l = r + p
    cfg = SC.get_config("C2")
    W = synth.gen_expert(cfg, 0, 0, r, device="cuda", which=("W1",))["W1"].contiguous()
    g = torch.Generator(device="cuda")
    g.manual_seed(2504)
    omega = torch.randn((iters, l, K), generator=g, device="cuda")
    steps = max(1, min(args.steps, 5))
    warm = max(1, min(args.warmup, 2))
    for _ in range(warm):
        m.build_compensator(W, r, iters, omega, power_iters=q, quantizer=args.quantizer)
    torch.cuda.synchronize()
    global TIMER
    TIMER = HipTimer()
    a, b = TIMER.event(), TIMER.event()
    stream = torch.cuda.current_stream().cuda_stream
    TIMER.record(a, stream)
    for _ in range(steps):
        out = m.build_compensator(W, r, iters, omega, power_iters=q, quantizer=args.quantizer)
    TIMER.record(b, stream)
    torch.cuda.synchronize()
    ms = TIMER.ms(a, b) / steps
    per_iter = (2 * N * K * l * (2 + 2 * q) + 8 * l * l * (N * (q + 1) + K * q) + 2 * K * l * l
                + 2 * N * l * r + 2 * l * r * K)
    flops = iters * per_iter + (iters - 1) * 2 * N * K * r
    tfl = flops / (ms * 1e-3) / 1e12
    peak = 157.3
    res = {
        "metric": "offline compensator construction time per weight matrix", "value": round(ms, 3),
        "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": round(ms, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"compensator build: W {N}x{K} ~N(0,0.02), rank {r}, oversampling {p}, "
                               f"{q} power iterations, {iters} quantize/compensate rounds, "
                               f"{args.quantizer} quantizer",
                   "alg_flops": int(flops)},
        "roofline": {"bound": "alu", "achieved": round(tfl, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tfl / peak, 4), "traffic": None,
                     "kernel": "whole milo_build_compensator call (single-block l x l factorizations take most of it, "
                               "then the skinny fp32 products)"},
    }
    if not args.no_cpu:
        import numpy as np
        import oracle
        from threadpoolctl import threadpool_info
        Wh = W.cpu().numpy()
        om = omega.cpu().numpy()
        t0 = time.perf_counter()
        oracle.build_ref(Wh, r, iters, om, q, quantizer=args.quantizer)
        cpu_s = time.perf_counter() - t0
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        res["cpu_baseline"] = {"value": round(cpu_s * 1000, 1), "unit": "ms", "cores": int(threads),
                               "kind": "oracle", "sample": "oracle.build_ref on the same full matrix, "
                               "test matrices and settings (float64 NumPy, Householder QR and SVD)"}
    else:
        res["cpu_baseline"] = None
    del out
    print(json.dumps(res))


def bench_ranks(args, m):
    """Adaptive rank policy on a Mixtral-shaped layer: per-matrix weight
    kurtosis of the 8 experts' W1, W3, W2 (24 x 58.7 M fp32 weights, two
    streaming passes: the HBM-bound part), pairs per expert from routing
    4096 tokens, then the host apportionment of an average rank of 32."""
    import torch
    import synth
    from synth import configs as SC
    cfg = SC.get_config("C2")
    mats = []
    for e in range(cfg.E):
        d = synth.gen_expert(cfg, 0, e, 8, device="cuda", which=("W1", "W3", "W2"))
        mats += [d["W1"].reshape(-1), d["W3"].reshape(-1), d["W2"].reshape(-1)]
    W = torch.stack(mats)
    del mats
    count, elems = W.shape
    steps = max(1, min(args.steps, 20))
    for _ in range(max(1, args.warmup)):
        kurt, _ = m.weight_kurtosis(W, count=count)
    torch.cuda.synchronize()
    global TIMER
    TIMER = HipTimer()
    a, b = TIMER.event(), TIMER.event()
    stream = torch.cuda.current_stream().cuda_stream
    TIMER.record(a, stream)
    for _ in range(steps):
        kurt, _ = m.weight_kurtosis(W, count=count)
    TIMER.record(b, stream)
    torch.cuda.synchronize()
    ms = TIMER.ms(a, b) / steps
    nbytes = 2 * count * elems * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    big = cfg.with_(T=4096)
    counts = torch.zeros(cfg.E, dtype=torch.int64, device="cuda")
    r = m.route_sort(synth.gen_logits(big, 0, device="cuda"), cfg.k, 0, True)
    m.expert_counts(r["offsets"], counts)
    freq = (counts.double() / big.T).cpu().tolist()
    kh = kurt.cpu().tolist()
    ranks = m.rank_policy(kh, [freq[i // 3] for i in range(count)], [False] * count, 32 * count, 8, 64, 8)
    res = {
        "metric": "adaptive-rank inputs: weight kurtosis of one Mixtral-shaped MoE layer", "value": round(ms, 3),
        "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": max(1, args.warmup), "ms_per_step": round(ms, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"kurtosis of {count} fp32 matrices of {elems} weights (8 experts x W1, W3, W2, "
                               "N(0,0.02)); pairs per expert of 4096 routed tokens; rank budget 32 per matrix",
                   "ranks": ranks, "kurtosis_range": [round(min(kh), 4), round(max(kh), 4)]},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "moments_kernel (two passes; algorithmic bytes = 2 x 4 B per weight)"},
    }
    if not args.no_cpu:
        import oracle
        from threadpoolctl import threadpool_info
        Wh = W[:2].cpu().numpy()
        t0 = time.perf_counter()
        for i in range(2):
            oracle.kurtosis_ref(Wh[i])
        cpu_s = (time.perf_counter() - t0) * count / 2
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        res["cpu_baseline"] = {"value": round(cpu_s * 1000, 1), "unit": "ms", "cores": int(threads),
                               "kind": "oracle", "sample": f"oracle.kurtosis_ref on 2 of the {count} matrices, "
                               f"scaled x{count / 2:.0f}"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


def bench_hqq(args, m):
    """HQQ-style quantization (RTN scale, 20 half-quadratic zero-point
    iterations, float64) of one Mixtral-shaped gate matrix.  The roofline line
    counts 16 float64 operations per weight and iteration (codes at z, the
    error, the threshold test, the update term and its sum, codes and error
    at the fp16 candidate and that sum; the threshold's power is not counted:
    it is needed only where the threshold can fire, which on weights of this
    magnitude is nowhere) against the fp64 vector peak."""
    import torch
    import numpy as np
    import synth
    from synth import configs as SC
    cfg = SC.get_config("C2")
    W = synth.gen_expert(cfg, 0, 0, 8, device="cuda", which=("W1",))["W1"].contiguous()
    rows, K = W.shape
    iters = 20
    steps = max(1, min(args.steps, 10))
    for _ in range(max(1, args.warmup)):
        m.quantize_hqq_int3(W, iters=iters)
    torch.cuda.synchronize()
    global TIMER
    TIMER = HipTimer()
    a, b = TIMER.event(), TIMER.event()
    stream = torch.cuda.current_stream().cuda_stream
    TIMER.record(a, stream)
    for _ in range(steps):
        c, s, z = m.quantize_hqq_int3(W, iters=iters)
    TIMER.record(b, stream)
    torch.cuda.synchronize()
    ms = TIMER.ms(a, b) / steps
    ops = 16.0 * rows * K * iters
    tfl = ops / (ms * 1e-3) / 1e12
    peak = 78.6
    # quality against RTN on the same matrix (sampled rows, float64 on the host)
    rows_s = np.random.default_rng(0).choice(rows, 512, replace=False)
    import oracle
    Wh = W[torch.from_numpy(rows_s).cuda()].cpu().numpy().astype(np.float64)
    q0, s0, z0 = m.quantize_rtn_int3(W)
    dh = oracle.dequant_int3(c.cpu().numpy()[rows_s], s.cpu().numpy()[rows_s], z.cpu().numpy()[rows_s])
    dr = oracle.dequant_int3(q0.cpu().numpy()[rows_s], s0.cpu().numpy()[rows_s], z0.cpu().numpy()[rows_s])
    res = {
        "metric": "HQQ-style int3 quantization time per weight matrix", "value": round(ms, 3), "unit": "ms",
        "n_gpus": 1, "steps": steps, "warmup": max(1, args.warmup), "ms_per_step": round(ms, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"HQQ-style quantization of W {rows}x{K} ~N(0,0.02), groups of 64, p 0.7, "
                               f"beta 10, kappa 1.01, {iters} iterations",
                   "mae_vs_rtn": round(float(np.abs(Wh - dh).mean() / np.abs(Wh - dr).mean()), 4),
                   "mse_vs_rtn": round(float(((Wh - dh) ** 2).mean() / ((Wh - dr) ** 2).mean()), 4)},
        "roofline": {"bound": "alu", "achieved": round(tfl, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tfl / peak, 4), "traffic": None,
                     "kernel": "hqq_kernel (16 fp64 operations per weight and iteration counted)"},
    }
    if not args.no_cpu:
        from oracle import hqq as HQ
        from threadpoolctl import threadpool_info
        n = 512
        t0 = time.perf_counter()
        HQ.quantize_hqq_int3(W[:n].cpu().numpy(), iters=iters)
        cpu_s = (time.perf_counter() - t0) * rows / n
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        res["cpu_baseline"] = {"value": round(cpu_s * 1000, 1), "unit": "ms", "cores": int(threads),
                               "kind": "oracle", "sample": f"oracle.hqq.quantize_hqq_int3 on {n} of the {rows} rows, "
                               f"scaled x{rows / n:.0f}"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


def bench_c1(args, m, cfg):
    import torch
    import synth
    d = synth.gen_linear(cfg, device="cuda")
    fam = m.Family.from_dense([d["W"]], [d["A"]], [d["B"]])
    x = d["X"]
    offsets = torch.tensor([0, cfg.M], dtype=torch.int32, device="cuda")
    y = torch.empty((cfg.M, cfg.N), dtype=torch.float16, device="cuda")
    for _ in range(args.warmup):
        m.moe_w3a16_lowrank_gemm((fam,), x, offsets, cfg.M, m.EPI_NONE, y)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        m.moe_w3a16_lowrank_gemm((fam,), x, offsets, cfg.M, m.EPI_NONE, y)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"metric": "single linear latency", "value": round(ms * 1000, 2), "unit": "us",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
                      "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                      "data": "synthetic", "config": {"workload": "C1: " + WORKLOAD_TEXT["C1"]},
                      "roofline": None, "cpu_baseline": None}))


if __name__ == "__main__":
    main()
