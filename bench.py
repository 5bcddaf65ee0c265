"""Benchmark of the quantized MoE layer on one MI355X.

One step = one pass of the whole layer (router + top-k/softmax, permutation,
expert-input gather (+ per-token int8 quantisation), gate/up + SwiGLU, down
projection, weighted combine) over one batch of synthetic tokens already
resident in HBM.

Headline: the large-expert W4A8 layer (hidden 8192, 64 experts, top-2,
intermediate 16384, 4-bit group-128 weights, per-token int8 x and h) at
prefill, 8192 tokens: the largest of the synthetic workloads, timed for
exactly --steps steps after --warmup untimed ones. Every other workload is
measured the same way and reported in `workloads`: the tiny layer, the
Mixtral-8x7B-shaped layer (prefill 2048 and decode 1/8/32 tokens), the
fine-grained 256-expert e2m1 layer (1/64/4096 tokens), the hot/cold mixed
4/2-bit layer (4096 tokens) and the W4A8 decode batch (16 tokens). Decode
repetitions are each preceded by a 1 GiB buffer write, so the 256 MB
last-level cache holds no weights.

Each entry carries tokens/s, its roofline fraction (MFMA for prefill, HBM on
packed weight bytes for decode) and parity against the CPU oracle on a stated
sample. The oracle is also timed on the host cores: a bounded sample of the
headline layer (every assignment of 8 of its 64 experts, scaled to tokens/s)
and the whole Mixtral-shaped prefill layer.

Prints one JSON line. `--gpus N` with N > 1 exits: the layer runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "MoE-layer tokens/s; decode weight GB/s and prefill TFLOP/s vs MI355X peak"
PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16/bf16 MFMA
PEAK_INT8_TOPS = 5033.2     # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["quantized_mixture_experts_router_amd/csrc/gemm_impl.h",
                  "quantized_mixture_experts_router_amd/csrc/deq.h",
                  "quantized_mixture_experts_router_amd/csrc/common.h"]
FMT_NAMES = {1: "asym", 2: "e2m1"}
ALL_WORKLOADS = ["w4a8", "mixtral", "fine_e2m1", "hotcold", "tiny"]
HEADLINE = "w4a8"
# experts of the headline layer the CPU baseline runs in full (of 64)
CPU_SAMPLE_EXPERTS = 8


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(name):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def payload_bytes(cfg, e):
    """Algorithmic weight bytes of expert e (codes + scales (+ mins)):
    (all three matrices, gate+up only)."""
    import synth
    fmt, bits, group = synth.expert_format(cfg, e)
    psz = 4 if fmt == synth.FMT_ASYM else 2
    w3, w2 = 3 * cfg.H * cfg.I, 2 * cfg.H * cfg.I
    return w3 * bits // 8 + (w3 // group) * psz, w2 * bits // 8 + (w2 // group) * psz


def kernel_names(cfg, gu=True):
    import synth
    fmts = sorted({synth.expert_format(cfg, e) for e in range(cfg.E)})
    # template arguments: block format, role (0 fused gate/up, 1 down), four-class order
    return [f"ffn_prefill_kernel<moeq::Fmt<{f}, {b}, {g}>, {0 if gu else 1}, *>"
            for f, b, g in fmts]


def weights_desc(cfg):
    f, b, g = cfg.fmt
    s = f"{FMT_NAMES[f]} {b}-bit, group {g}, fp16 scale" + ("+min" if f == 1 else "")
    if cfg.cold_fmt is not None:
        f2, b2, g2 = cfg.cold_fmt
        s = (f"{cfg.n_hot} hot experts {s}; the others {FMT_NAMES[f2]} {b2}-bit, group {g2}, "
             f"fp16 scale+min; Zipf-skewed router bias")
    return s


def workload_desc(cfg, T, phase):
    return {"workload": f"{cfg.name} quantized MoE layer, {phase}", "tokens": T, "hidden": cfg.H,
            "intermediate": cfg.I, "experts": cfg.E, "top_k": cfg.k, "weights": weights_desc(cfg),
            "activations": cfg.x_dtype,
            "expert_inputs": "per-token int8 (x and h)" if cfg.act == 2 else
                             ("per-token int8 (x)" if cfg.act == 1 else "fp16"),
            "router": "fp32 weights, fp64 accumulation", "parallelism": "single GPU"}


def host_cores():
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    return {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "blas_threads": blas}


class Bench:
    def __init__(self, args):
        import torch
        self.args = args
        self.torch = torch
        self.dev = torch.device("cuda:0")

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    # ------------------------------------------------------------------ prefill
    def prefill(self, wl, T):
        """Times exactly args.steps whole-layer steps on T tokens (after
        args.warmup untimed ones); per-step events around gate/up and down,
        recorded on the stream the kernels run on."""
        import numpy as np
        import quantized_mixture_experts_router_amd as moeq
        torch, args, cfg = self.torch, self.args, wl.cfg
        H, I, E, k, act = cfg.H, cfg.I, cfg.E, cfg.k, cfg.act
        x = wl.x[:T].contiguous()
        ws = moeq.workspace(T, H, I, E, k, act, self.dev)
        Y = torch.empty((T * k, H), dtype=torch.float32, device=self.dev)

        def step(evs=None):
            ids_, w_ = moeq.route(x, wl.Wr, wl.b, k)
            counts, offsets, perm, inv, _ = moeq.permute(ids_, E, ws)
            moeq.ffn_gather(x, perm, k, wl.packed, act, ws)
            if evs is not None:
                evs[0].record()
            moeq.ffn_gate_up(T, wl.packed, offsets, k, act, ws)
            if evs is not None:
                evs[1].record()
            moeq.ffn_down(T, wl.packed, offsets, k, act, Y, ws)
            if evs is not None:
                evs[2].record()
            return moeq.combine(Y, w_, inv, T, k), ids_, counts

        for _ in range(args.warmup):
            step()
        evs = [[self.event() for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            o, ids_, counts = step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / args.steps
        gu_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        dn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        # the one-shot entry point on the same batch must agree bit for bit
        out1, _, _ = moeq.layer_forward(x, wl.Wr, wl.b, wl.packed, k, act=act, ws=ws)
        torch.cuda.synchronize()
        same = bool(torch.equal(out1, o))
        flags = moeq.read_flags(ws)
        flop_gu = 2.0 * T * k * H * 2 * I
        flop_dn = 2.0 * T * k * I * H
        flop = flop_gu + flop_dn + 2.0 * T * H * E
        touched = np.nonzero(counts.cpu().numpy())[0]
        wbytes = sum(payload_bytes(cfg, int(e))[0] for e in touched)
        gu_bytes = sum(payload_bytes(cfg, int(e))[1] for e in touched)
        gu_tf = flop_gu / (gu_ms * 1e-3) / 1e12
        d = {"tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
             "layer_tflops": flop / (ms * 1e-3) / 1e12,
             "layer_frac_mfma": flop / (ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
             "gate_up_ms": gu_ms, "gate_up_tflops": gu_tf,
             "gate_up_frac_mfma": gu_tf / PEAK_FP16_TFLOPS,
             "gate_up_weight_GBps": gu_bytes / (gu_ms * 1e-3) / 1e9,
             "down_ms": dn_ms, "down_tflops": flop_dn / (dn_ms * 1e-3) / 1e12,
             "down_frac_mfma": flop_dn / (dn_ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
             "weight_bytes_touched": wbytes,
             "layer_weight_GBps": wbytes / (ms * 1e-3) / 1e9,
             "flop_per_step": flop, "gate_up_flop": flop_gu,
             "split_api_equals_layer_forward": same, "flags": flags}
        log(f"[bench] {cfg.name} prefill T={T}: {ms:.3f} ms/step ({d['tokens_per_s']:.0f} tok/s), "
            f"gate_up {gu_ms:.3f} ms ({gu_tf:.0f} TFLOP/s, {d['gate_up_frac_mfma']:.3f}), "
            f"down {dn_ms:.3f} ms ({d['down_tflops']:.0f} TFLOP/s)")
        return d, o, ids_

    # ------------------------------------------------------------------ decode
    def decode(self, wl, Td, flush, extras):
        """Median over args.decode_reps layer calls on Td tokens, each after a
        1 GiB buffer write (cold last-level cache); phase times from a second
        pass through the split entry points; HIP-graph replay and warm (no
        flush) variants when extras."""
        import numpy as np
        import quantized_mixture_experts_router_amd as moeq
        torch, args, cfg = self.torch, self.args, wl.cfg
        H, I, E, k, act = cfg.H, cfg.I, cfg.E, cfg.k, cfg.act
        x_d = wl.x[:Td].contiguous()
        ws_d = moeq.workspace(Td, H, I, E, k, act, self.dev)
        Yd = torch.empty((Td * k, H), dtype=torch.float32, device=self.dev)
        lay, gu, dn = [], [], []
        out_d = None
        for r in range(args.decode_warmup + args.decode_reps):
            flush.zero_()
            e0, e1 = self.event(), self.event()
            e0.record()
            out_d, ids_d, w_d = moeq.layer_forward(x_d, wl.Wr, wl.b, wl.packed, k, act=act, ws=ws_d)
            e1.record()
            flush.zero_()
            ids2, w2 = moeq.route(x_d, wl.Wr, wl.b, k)
            counts_d, off_d, perm_d, inv_d, _ = moeq.permute(ids2, E, ws_d)
            moeq.ffn_gather(x_d, perm_d, k, wl.packed, act, ws_d)
            g0, g1, g2 = self.event(), self.event(), self.event()
            g0.record()
            moeq.ffn_gate_up(Td, wl.packed, off_d, k, act, ws_d)
            g1.record()
            moeq.ffn_down(Td, wl.packed, off_d, k, act, Yd, ws_d)
            g2.record()
            torch.cuda.synchronize()
            if r >= args.decode_warmup:
                lay.append(e0.elapsed_time(e1))
                gu.append(g0.elapsed_time(g1))
                dn.append(g1.elapsed_time(g2))
        out_d = out_d.clone()
        touched = np.nonzero(counts_d.cpu().numpy())[0]
        tot_b = sum(payload_bytes(cfg, int(e))[0] for e in touched)
        gu_b = sum(payload_bytes(cfg, int(e))[1] for e in touched)
        lay_ms, gu_ms, dn_ms = (float(np.median(v)) for v in (lay, gu, dn))
        ffn_ms = gu_ms + dn_ms
        d = {"tokens": Td, "experts_touched": int(len(touched)),
             "layer_ms": lay_ms,
             "layer_ms_p10_p90": [float(np.percentile(lay, 10)), float(np.percentile(lay, 90))],
             "tokens_per_s": Td / (lay_ms * 1e-3),
             "layer_weight_GBps": tot_b / (lay_ms * 1e-3) / 1e9,
             "layer_frac_hbm": tot_b / (lay_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
             "ffn_ms": ffn_ms, "ffn_weight_GBps": tot_b / (ffn_ms * 1e-3) / 1e9,
             "ffn_frac_hbm": tot_b / (ffn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
             "gate_up_ms": gu_ms, "gate_up_weight_GBps": gu_b / (gu_ms * 1e-3) / 1e9,
             "gate_up_frac_hbm": gu_b / (gu_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
             "down_ms": dn_ms, "weight_bytes_touched": tot_b,
             "flags": moeq.read_flags(ws_d)}
        if extras:
            out_g = torch.empty((Td, H), dtype=torch.float32, device=self.dev)
            ids_g = torch.empty((Td, k), dtype=torch.int32, device=self.dev)
            w_g = torch.empty((Td, k), dtype=torch.float32, device=self.dev)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                moeq.layer_forward(x_d, wl.Wr, wl.b, wl.packed, k, act=act, ws=ws_d, out=out_g,
                                   ids=ids_g, w=w_g)
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                moeq.layer_forward(x_d, wl.Wr, wl.b, wl.packed, k, act=act, ws=ws_d, out=out_g,
                                   ids=ids_g, w=w_g)
            lay_g, lay_w = [], []
            for r in range(args.decode_warmup + args.decode_reps):
                flush.zero_()
                e0, e1 = self.event(), self.event()
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                if r >= args.decode_warmup:
                    lay_g.append(e0.elapsed_time(e1))
            del graph
            for r in range(args.decode_warmup + args.decode_reps):
                # warm: no flush; a spin kernel that touches no memory keeps
                # the device busy while the host queues the layer
                torch.cuda._sleep(300000)
                e0, e1 = self.event(), self.event()
                e0.record()
                moeq.layer_forward(x_d, wl.Wr, wl.b, wl.packed, k, act=act, ws=ws_d)
                e1.record()
                torch.cuda.synchronize()
                if r >= args.decode_warmup:
                    lay_w.append(e0.elapsed_time(e1))
            d["layer_ms_graph"] = float(np.median(lay_g))
            d["layer_ms_warm"] = float(np.median(lay_w))
        log(f"[bench] {cfg.name} decode T={Td}: layer {lay_ms * 1e3:.1f} us "
            f"({d['layer_weight_GBps']:.0f} GB/s), gate_up {gu_ms * 1e3:.1f} us "
            f"({d['gate_up_weight_GBps']:.0f} GB/s), down {dn_ms * 1e3:.1f} us, "
            f"ffn {d['ffn_weight_GBps']:.0f} GB/s ({d['ffn_frac_hbm']:.3f})")
        return d, out_d, ids_d

    # ------------------------------------------------------------------ extras
    def router_i8(self, wl, T, ids_exact):
        """The int8-logit router variant, calibrated on T held-out tokens (the
        rows after the batch's own), against the exact routing."""
        import numpy as np
        import synth
        import quantized_mixture_experts_router_amd as moeq
        from layer_cases import x_to_torch
        cfg, torch = wl.cfg, self.torch
        k = cfg.k
        x = wl.x[:T].contiguous()
        x_cal = x_to_torch(synth.gen_x(cfg, 2 * T)[T:], cfg.x_dtype, self.dev)
        lo, hi = moeq.router_logit_range(x_cal, wl.Wr, wl.b)
        del x_cal
        ids_ex = ids_exact.cpu().numpy()
        r8 = {"calibration_tokens": T}
        for shared in (False, True):
            sc, zp = moeq.router_i8_params(lo, hi, shared)
            sc_d, zp_d = torch.from_numpy(sc).to(self.dev), torch.from_numpy(zp).to(self.dev)
            ids8, _ = moeq.route_i8(x, wl.Wr, wl.b, k, sc_d, zp_d)
            i8 = ids8.cpu().numpy()
            r8["per_expert" if not shared else "shared"] = {
                "same_expert_set": float(np.mean([set(a) == set(c) for a, c in zip(i8, ids_ex)])),
                "assignments_kept": float(np.mean([len(set(a) & set(c)) / k
                                                   for a, c in zip(i8, ids_ex)]))}
        for name, fn in (("route_ms", lambda: moeq.route(x, wl.Wr, wl.b, k)),
                         ("route_i8_ms", lambda: moeq.route_i8(x, wl.Wr, wl.b, k, sc_d, zp_d))):
            fn()
            torch.cuda._sleep(300000)
            a0, a1 = self.event(), self.event()
            a0.record()
            for _ in range(10):
                fn()
            a1.record()
            torch.cuda.synchronize()
            r8[name] = a0.elapsed_time(a1) / 10
        log(f"[bench] {cfg.name} int8 router logits: same expert set "
            f"{r8['per_expert']['same_expert_set']:.3f} (per-expert scales), "
            f"{r8['shared']['same_expert_set']:.3f} (shared); route {r8['route_ms'] * 1e3:.1f} us, "
            f"route_i8 {r8['route_i8_ms'] * 1e3:.1f} us")
        return r8

    def outliers(self, wl, T, flush):
        """Cost of fp16 outlier side lists (0.05% of each expert matrix, the
        field notes' share): the same layer packed with them, prefill and
        decode times against the plain layer's."""
        from dataclasses import replace
        from layer_cases import Workload
        cfg = wl.cfg
        frac = 0.0005
        wl2 = Workload(replace(cfg, weight_outlier_frac=frac), device=self.dev)
        d, _, _ = self.prefill(wl2, T)
        res = {"share": frac, "outliers_per_expert": int(round(frac * 3 * cfg.H * cfg.I)),
               "prefill_ms": d["ms_per_step"], "prefill_gate_up_ms": d["gate_up_ms"],
               "prefill_down_ms": d["down_ms"]}
        if cfg.decode_T:
            dd = []
            for Td in cfg.decode_T:
                r, _, _ = self.decode(wl2, Td, flush, False)
                dd.append({"tokens": Td, "layer_ms": r["layer_ms"], "gate_up_ms": r["gate_up_ms"],
                           "down_ms": r["down_ms"]})
            res["decode"] = dd
        del wl2
        log(f"[bench] {cfg.name} with 0.05% outliers: prefill {res['prefill_ms']:.3f} ms")
        return res

    def int8_gemm(self, wl, T):
        """The opt-in int8 MFMA GEMMs (MOE_MASK_INT8_GEMM) against the default
        fp16 kernels on the same W4A8 batch: whole-layer calls
        (moe_layer_forward), args.steps timed after args.warmup."""
        import numpy as np
        import quantized_mixture_experts_router_amd as moeq
        torch, args, cfg = self.torch, self.args, wl.cfg
        x = wl.x[:T].contiguous()
        ws = moeq.workspace(T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.act, self.dev)
        full = wl.packed.fmt_mask
        res = {}
        try:
            outs = {}
            for label, mask in (("fp16_kernels", full), ("int8_kernels", full | moeq.MASK_INT8_GEMM)):
                wl.packed.fmt_mask = mask
                for _ in range(args.warmup):
                    moeq.layer_forward(x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act, ws=ws)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(args.steps):
                    o, _, _ = moeq.layer_forward(x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act, ws=ws)
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) * 1e3 / args.steps
                outs[label] = o.float().cpu().numpy()
                res[label] = {"layer_ms": ms, "tokens_per_s": T / (ms * 1e-3),
                              "flags": moeq.read_flags(ws)}
        finally:
            wl.packed.fmt_mask = full
        a, b = outs["int8_kernels"], outs["fp16_kernels"]
        res["max_row_rel_l2_between"] = float(np.max(np.linalg.norm(a - b, axis=1) /
                                                     np.maximum(np.linalg.norm(b, axis=1), 1e-30)))
        log(f"[bench] {cfg.name} T={T} whole layer: fp16 kernels {res['fp16_kernels']['layer_ms']:.3f} ms, "
            f"int8 kernels {res['int8_kernels']['layer_ms']:.3f} ms "
            f"(outputs differ by {res['max_row_rel_l2_between']:.2e})")
        return res

    def tiers(self, wl, T, ids_own):
        """Expert-aware precision from a routing profile of T held-out tokens:
        the tier plan within the byte budget of the workload's bias-ranked hot
        set, the layer repacked by it and timed; then three tiers (adding
        1-bit) under the same budget."""
        from dataclasses import replace
        import numpy as np
        import synth
        import quantized_mixture_experts_router_amd as moeq
        from layer_cases import Workload, x_to_torch
        cfg, torch, args = wl.cfg, self.torch, self.args
        E, k, dev = cfg.E, cfg.k, self.dev
        x_cal = x_to_torch(synth.gen_x(cfg, 2 * T)[T:], cfg.x_dtype, dev)
        ids_c, _ = moeq.route(x_cal, wl.Wr, wl.b, k)
        hist = torch.zeros(E, dtype=torch.int64, device=dev)
        moeq.expert_histogram(ids_c, E)  # first launch loads the kernel: not timed
        torch.cuda._sleep(300000)
        h0, h1 = self.event(), self.event()
        h0.record()
        moeq.expert_histogram(ids_c, E, hist)
        h1.record()
        torch.cuda.synchronize()
        counts_cal = hist.cpu().numpy()

        def expert_bytes(fmt):
            ex = synth.gen_expert(replace(cfg, expert_fmts=(fmt,) * E), 0)
            return moeq.packed_expert_bytes(
                *[moeq.DeviceQMat.from_host(ex[r], dev) for r in ("gate", "up", "down")])

        sizes = [expert_bytes(cfg.fmt), expert_bytes(cfg.cold_fmt)]
        budget = cfg.n_hot * sizes[0] + (E - cfg.n_hot) * sizes[1]
        tp0 = time.perf_counter()
        tiers, used = moeq.plan_tiers(counts_cal, sizes, budget)
        plan_us = (time.perf_counter() - tp0) * 1e6
        own = moeq.expert_histogram(ids_own, E).cpu().numpy()
        prior = np.array([synth.expert_format(cfg, e) == cfg.fmt for e in range(E)])
        hot = tiers == 0

        def timed(fmts):
            wl2 = Workload(replace(cfg, expert_fmts=tuple(fmts)), device=dev)
            d, _, _ = self.prefill(wl2, T)
            del wl2
            return d["ms_per_step"]

        ms_p = timed(cfg.fmt if t == 0 else cfg.cold_fmt for t in tiers)
        one = (1, 1, 16)
        sizes3 = sizes + [expert_bytes(one)]
        tiers3, used3 = moeq.plan_tiers(counts_cal, sizes3, budget)
        fm3 = (cfg.fmt, cfg.cold_fmt, one)
        ms_3 = timed(fm3[t] for t in tiers3)
        # four tiers, a bit apart each (4-, 3-, 2-, 1-bit, group 32)
        fm4 = ((1, 4, 32), (1, 3, 32), (1, 2, 32), (1, 1, 32))
        sizes4 = [expert_bytes(f) for f in fm4]
        tiers4, used4 = moeq.plan_tiers(counts_cal, sizes4, budget)
        ms_4 = timed(fm4[t] for t in tiers4)
        res = {"calibration_tokens": T, "hot_experts": int(hot.sum()),
               "tier_bytes": sizes, "budget_bytes": int(budget), "used_bytes": int(used),
               "histogram_ms": h0.elapsed_time(h1), "plan_us": plan_us,
               "hot_set_overlap": int((hot & prior).sum()),
               "hot_share_profiled": float(own[hot].sum() / own.sum()),
               "hot_share_bias_ranked": float(own[prior].sum() / own.sum()),
               "prefill_ms_profiled": ms_p,
               "three_tier": {"tier_bytes": sizes3, "used_bytes": int(used3),
                              "experts_per_tier": [int((tiers3 == t).sum()) for t in range(3)],
                              "slot_share_per_tier": [float(own[tiers3 == t].sum() / own.sum())
                                                      for t in range(3)],
                              "prefill_ms": ms_3},
               "four_tier": {"formats": ["asym 4-bit g32", "asym 3-bit g32", "asym 2-bit g32",
                                         "asym 1-bit g32"],
                             "tier_bytes": sizes4, "used_bytes": int(used4),
                             "experts_per_tier": [int((tiers4 == t).sum()) for t in range(4)],
                             "slot_share_per_tier": [float(own[tiers4 == t].sum() / own.sum())
                                                     for t in range(4)],
                             "prefill_ms": ms_4}}
        log(f"[bench] {cfg.name} tiers: profiled hot set shares {res['hot_share_profiled']:.3f} "
            f"of the slots (bias-ranked {res['hot_share_bias_ranked']:.3f}), prefill {ms_p:.3f} ms; "
            f"three tiers {res['three_tier']['experts_per_tier']}, prefill {ms_3:.3f} ms; "
            f"four tiers {res['four_tier']['experts_per_tier']}, prefill {ms_4:.3f} ms")
        return res


def oracle_parity(cfg, wl, outs, full_ref=None):
    """Max row rel-L2 of GPU outputs {T: (out numpy, ids numpy)} against the
    oracle rows of the same tokens (the batches are prefixes of one seeded
    token stream, and a token's output depends on that token alone)."""
    import numpy as np
    from layer_cases import rel_l2_rows, tolerance
    res = {}
    for T, (out, ids) in outs.items():
        ok = ~full_ref["flagged"][:T]
        ids_ok = bool(np.array_equal(ids[ok], full_ref["ids"][:T][ok]))
        err = rel_l2_rows(out[ok], full_ref["out"][:T][ok])
        res[str(T)] = {"tokens_checked": int(ok.sum()), "ids_bit_exact": ids_ok,
                       "max_row_rel_l2": float(err.max()), "tolerance": tolerance(cfg),
                       "pass": ids_ok and float(err.max()) <= tolerance(cfg)}
    return res


def headline_oracle_sample(cfg, wl, outs):
    """The oracle on a bounded sample of the W4A8 layer: routing of every
    token, then every assignment of CPU_SAMPLE_EXPERTS experts (decode of
    their blocks, their int8-mirrored SwiGLU FFN in fp64), timed and scaled to
    tokens/s of the whole layer (assignments done / k per second). The same
    rows give parity of the GPU's per-assignment outputs, and tokens routed
    only to sampled experts give parity of the combined output."""
    import numpy as np
    import oracle
    from layer_cases import rel_l2_rows, tolerance
    T = cfg.T
    t0 = time.perf_counter()
    X = oracle.x_to_f64(wl.x_np, cfg.x_dtype)
    L = oracle.router_logits(X, wl.Wr_np, None)
    ids, w, gap, flagged = oracle.topk_softmax(L, cfg.k)
    counts, offsets, perm, inv = oracle.canonical_permute(ids, cfg.E)
    A = oracle.dq8(X.astype(np.float32))
    # the sampled experts: those of the first tokens, evenly spread
    S = []
    for e in list(ids[:2].reshape(-1)) + list(range(0, cfg.E, cfg.E // CPU_SAMPLE_EXPERTS)):
        if int(e) not in S and len(S) < CPU_SAMPLE_EXPERTS:
            S.append(int(e))
    Yref, rows_done = {}, 0
    for e in S:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        ex = wl.expert_uncached(e)
        Wg, Wu, Wd = (oracle.decode_qmat(ex["gate"]), oracle.decode_qmat(ex["up"]),
                      oracle.decode_qmat(ex["down"]))
        Ye = oracle.expert_ffn(A[perm[r0:r1]], Wg, Wu, Wd, cfg.act)
        for i, r in enumerate(range(r0, r1)):
            Yref[r] = Ye[i]
        rows_done += r1 - r0
        del Wg, Wu, Wd
    dt = time.perf_counter() - t0
    value = rows_done / cfg.k / dt
    # parity: tokens whose k assignments were all computed
    par = {}
    for Tb, (out, ids_g) in outs.items():
        ok = ~flagged[:Tb]
        ids_ok = bool(np.array_equal(ids_g[ok], ids[:Tb][ok]))
        toks = [t for t in range(Tb) if ok[t] and all(int(inv[t * cfg.k + j]) in Yref
                                                        for j in range(cfg.k))]
        ent = {"tokens_checked": len(toks), "ids_bit_exact": ids_ok, "tolerance": tolerance(cfg),
               "sample": f"tokens routed only to experts {S}"}
        if toks:
            ref = np.stack([sum(w[t, j] * Yref[int(inv[t * cfg.k + j])] for j in range(cfg.k))
                            for t in toks])
            err = rel_l2_rows(out[toks], ref)
            ent["max_row_rel_l2"] = float(err.max())
            ent["pass"] = ids_ok and float(err.max()) <= tolerance(cfg)
        else:
            ent["pass"] = ids_ok
        par[str(Tb)] = ent
    cpu = {"value": value, "unit": "tokens/s", "kind": "oracle",
           "sample": f"{cfg.name} layer, T={T}: routing of every token, then every assignment "
                     f"of {len(S)} of its {cfg.E} experts ({rows_done} rows: block decode and "
                     f"fp64 SwiGLU FFN with the int8 mirror), {dt:.1f} s; tokens/s = rows / k / s",
           "seconds": dt}
    return cpu, par


def hbm_sweep(torch, moeq, dev):
    """Read rate of a 4 GiB buffer (16 x the last-level cache) over launch
    shapes of the shaped streaming read: blocks per CU, block size, 16-byte
    loads in flight per thread, the interleaved and the contiguous layout,
    cached and non-temporal loads. Each shape: one untimed launch, then the
    median of 5 launches timed by HIP events on the launch stream. Prints one
    JSON line per shape and a final line with the fastest shape."""
    import numpy as np
    n = 4 << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    rows = []
    for nt in (True, False):
        for layout in (0, 1):
            for waves in (4, 8, 16):
                for inflight in (4, 8, 16):
                    for per_cu in (1, 2, 4, 8, 16, 32):
                        blocks = cus * per_cu
                        if waves * per_cu > 64 or blocks > (1 << 16):
                            continue
                        moeq.stream_read_shaped(buf, blocks, waves, inflight, layout, nt, sink)
                        st = []
                        for _ in range(5):
                            e0 = torch.cuda.Event(enable_timing=True)
                            e1 = torch.cuda.Event(enable_timing=True)
                            e0.record()
                            moeq.stream_read_shaped(buf, blocks, waves, inflight, layout, nt, sink)
                            e1.record()
                            torch.cuda.synchronize()
                            st.append(e0.elapsed_time(e1))
                        ms = float(np.median(st))
                        row = {"nontemporal": nt, "layout": ["interleaved", "contiguous"][layout],
                               "waves": waves, "inflight": inflight, "blocks_per_cu": per_cu,
                               "blocks": blocks, "ms": ms, "GBps": n / (ms * 1e-3) / 1e9}
                        rows.append(row)
                        print(json.dumps(row), flush=True)
    best = max(rows, key=lambda r: r["GBps"])
    print(json.dumps({"hbm_sweep_bytes": n, "cus": cus, "shapes": len(rows), "best": best,
                      "default_shape_GBps": {
                          "nontemporal": next(r["GBps"] for r in rows if r["nontemporal"] and
                                              r["layout"] == "interleaved" and r["waves"] == 4 and
                                              r["inflight"] == 8 and r["blocks_per_cu"] == 16),
                          "cached": next(r["GBps"] for r in rows if not r["nontemporal"] and
                                         r["layout"] == "interleaved" and r["waves"] == 4 and
                                         r["inflight"] == 8 and r["blocks_per_cu"] == 16)}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default=",".join(ALL_WORKLOADS),
                    help="comma-separated subset of " + ",".join(ALL_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle runs (timing and parity)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="profiling aid: decode batches only")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip graph replay / warm decode, int8 router and tier plans")
    ap.add_argument("--decode-reps", type=int, default=50)
    ap.add_argument("--decode-warmup", type=int, default=10)
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--hbm-sweep", action="store_true",
                    help="only sweep the launch shapes of the streaming read over a 4 GiB buffer")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is designed, not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import quantized_mixture_experts_router_amd as moeq  # noqa: F401
    from layer_cases import Workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.copy_calib:
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": 5}))
        return

    if args.hbm_sweep:
        hbm_sweep(torch, moeq, dev)
        return

    names = [n for n in args.workloads.split(",") if n]
    for n in names:
        if n not in ALL_WORKLOADS:
            raise SystemExit(f"unknown workload {n}")
    bench = Bench(args)
    entries = {}
    cpu_headline = None
    cpu_full = None
    cores = host_cores()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if not args.no_decode else None
    for name in names:
        cfg = synth.get_config(name)
        log(f"[bench] building {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} act={cfg.act}")
        t0 = time.time()
        wl = Workload(cfg, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] packed {wl.packed.nbytes() / 1e6:.1f} MB of experts in {time.time() - t0:.1f}s")
        ent = {"config": workload_desc(cfg, cfg.T, "prefill")}
        outs = {}
        extras = not args.no_extras
        if not args.no_prefill:
            d, o, ids_p = bench.prefill(wl, cfg.T)
            ent["prefill"] = d
            outs[cfg.T] = (o.cpu().numpy(), ids_p.cpu().numpy())
            if extras and name in ("mixtral", "fine_e2m1", "hotcold", "w4a8"):
                ent["router_i8"] = bench.router_i8(wl, cfg.T, ids_p)
            if extras and cfg.cold_fmt is not None and cfg.n_hot > 0:
                ent["tiers"] = bench.tiers(wl, cfg.T, ids_p)
            del o
        if not args.no_decode and cfg.decode_T:
            ent["decode"] = []
            for Td in cfg.decode_T:
                d, od, idd = bench.decode(wl, Td, flush, extras and name == "mixtral")
                ent["decode"].append(d)
                outs[Td] = (od.cpu().numpy(), idd.cpu().numpy())
        if extras and name == "mixtral" and not args.no_prefill and flush is not None:
            ent["outliers"] = bench.outliers(wl, cfg.T, flush)
        if extras and name == "w4a8" and not args.no_prefill:
            ent["int8_gemm"] = bench.int8_gemm(wl, cfg.T)
        if not args.no_cpu_baseline and outs:
            if name == HEADLINE:
                cpu_headline, par = headline_oracle_sample(cfg, wl, outs)
                log(f"[bench] oracle sample of {name}: {cpu_headline['value']:.2f} tokens/s "
                    f"({cpu_headline['seconds']:.1f} s)")
            else:
                b = wl.b_np if cfg.zipf_alpha > 0 else None
                import oracle
                tc0 = time.perf_counter()
                ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, b, wl.expert_uncached,
                                       cfg.E, cfg.k, act=cfg.act)
                tc = time.perf_counter() - tc0
                ent["oracle_full_layer"] = {"tokens": cfg.T, "seconds": tc,
                                            "tokens_per_s": cfg.T / tc}
                log(f"[bench] oracle over all {cfg.T} tokens of {name}: {tc:.1f} s")
                if name == "mixtral":
                    cpu_full = {"value": cfg.T / tc, "unit": "tokens/s", "kind": "oracle",
                                "sample": f"the whole {name} prefill layer, T={cfg.T}: every "
                                          f"expert decoded, fp64 NumPy/BLAS, {tc:.1f} s",
                                **{"cores": cores["affinity"], "host": cores}}
                par = oracle_parity(cfg, wl, outs, ref)
                del ref
            ent["parity"] = par
            log(f"[bench] parity {name}: " + ", ".join(
                f"T={t}: {p.get('max_row_rel_l2', float('nan')):.2e} over {p['tokens_checked']} tokens"
                f"{'' if p['pass'] else ' FAIL'}" for t, p in par.items()))
        entries[name] = ent
        del wl
        torch.cuda.empty_cache()

    # context: what a plain streaming read of the 1 GiB flush buffer reaches
    ctx = {}
    if flush is not None:
        ctx["buffer_bytes"] = flush.numel()
        for nt in (False, True):
            moeq.stream_read(flush, nontemporal=nt)
            st = []
            for _ in range(5):
                e0, e1 = bench.event(), bench.event()
                e0.record()
                moeq.stream_read(flush, nontemporal=nt)
                e1.record()
                torch.cuda.synchronize()
                st.append(e0.elapsed_time(e1))
            ctx["hbm_read_GBps_" + ("nontemporal" if nt else "cached")] = \
                flush.numel() / (float(np.median(st)) * 1e-3) / 1e9
        # the fastest shape of the launch-shape sweep (--hbm-sweep): one block of
        # 4 wavefronts per CU, each block a contiguous run, 16 non-temporal
        # 16-byte loads in flight per thread
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        sink = torch.empty(cus, dtype=torch.int32, device=dev)
        moeq.stream_read_shaped(flush, cus, 4, 16, 1, True, sink)
        st = []
        for _ in range(5):
            e0, e1 = bench.event(), bench.event()
            e0.record()
            moeq.stream_read_shaped(flush, cus, 4, 16, 1, True, sink)
            e1.record()
            torch.cuda.synchronize()
            st.append(e0.elapsed_time(e1))
        ctx["hbm_read_GBps_best_shape"] = flush.numel() / (float(np.median(st)) * 1e-3) / 1e9
        ctx["best_shape"] = "contiguous run per block, 1 block of 4 wavefronts per CU, 16 non-temporal 16-B loads in flight per thread"
        log(f"[bench] streaming read of 1 GiB: {ctx['hbm_read_GBps_cached']:.0f} GB/s cached, "
            f"{ctx['hbm_read_GBps_nontemporal']:.0f} GB/s non-temporal, "
            f"{ctx['hbm_read_GBps_best_shape']:.0f} GB/s in the sweep's fastest shape")
        del flush

    head = HEADLINE if HEADLINE in entries and "prefill" in entries[HEADLINE] else \
        next((n for n in names if "prefill" in entries[n]), None)
    result = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "fp16", "data": "synthetic"}
    if head is not None:
        hcfg = synth.get_config(head)
        p = entries[head]["prefill"]
        result.update({"value": p["tokens_per_s"], "ms_per_step": p["ms_per_step"],
                       "config": entries[head]["config"]})
        result["roofline"] = {
            "bound": "mfma", "kernel": " + ".join(kernel_names(hcfg)) + " (gate/up + SwiGLU)",
            "achieved": p["gate_up_tflops"], "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": p["gate_up_frac_mfma"],
            "traffic": read_traffic(f"ffn_prefill_gate_up_{head}_T{hcfg.T}_traffic.txt"),
            "avg_launch_ms": p["gate_up_ms"], "flop_per_launch": p["gate_up_flop"],
            "note": ("the int8 codes of x and h enter the fp16 matrix cores exactly; against the "
                     f"int8 peak ({PEAK_INT8_TOPS} TOP/s) the fraction is "
                     f"{p['gate_up_tflops'] / PEAK_INT8_TOPS:.3f}") if hcfg.act else None}
    if cpu_headline is not None:
        cpu_headline["cores"] = cores["affinity"]
        cpu_headline["host"] = cores
        result["cpu_baseline"] = cpu_headline
    if cpu_full is not None:
        result["cpu_baseline_full_layer"] = cpu_full
    result["workloads"] = entries
    if ctx:
        result["context"] = ctx
        # decode weight streams against the read rate the same run measured in
        # the sweep's fastest shape (a plain read of the 1 GiB buffer)
        best = ctx.get("hbm_read_GBps_best_shape")
        if best:
            for ent in entries.values():
                for d in ent.get("decode", []):
                    d["ffn_frac_of_best_read"] = d["ffn_weight_GBps"] / best
                    d["layer_frac_of_best_read"] = d["layer_weight_GBps"] / best
    print(json.dumps(result))


if __name__ == "__main__":
    main()
