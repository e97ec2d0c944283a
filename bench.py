#!/usr/bin/env python3
"""Benchmark of the W4A16 NVFP4 routed-expert MLP on one MI355X.

One step = one routed-expert MLP of the decode-shaped MoE layer (288 experts,
top-8, hidden 4096, intermediate 1536, 64 tokens): route, grouped gate/up with
SiLU(gate)*up, grouped down, routing-weighted combine, through the C ABI.
Consecutive steps cycle through 32 independently seeded routings and inputs,
so the 256 MB Infinity Cache cannot keep serving the same experts.

value = algorithmic bytes / time, where algorithmic bytes per call = touched
experts x 10,616,832 B (gate, up, down: 0.5625 B per weight, codes plus e4m3
scales) + their scale_2 + x + y + ids + routing weights. Inputs are resident in
HBM before the timed region starts.

Also reported in the same line: the T = 1 and 16 decode batches, the
prefill-shaped layer (4096 tokens, Zipf(1.1) routing) in TFLOP/s, the dense
Fp4Linear MLP (2048 x 4096 -> 12288 -> 4096) in TFLOP/s, and the load-time
pack of the 288 experts x 3 projections in GB/s; the roofline of the dominant
kernel (from HIP events recorded between the library's stages on the stream
it runs on); and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 W4A16 grouped-expert GB/s (decode) & TFLOP/s (prefill), % roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
E, K_TOP, H, I = 288, 8, 4096, 1536
W_BYTES = 9 / 16                 # bytes per weight: 4-bit code + one e4m3 byte per 16
EXPERT_BYTES = int(3 * I * H * W_BYTES)          # 10,616,832
GATEUP_BYTES = int(2 * I * H * W_BYTES)          # 7,077,888
DOWN_BYTES = int(I * H * W_BYTES)                # 3,538,944
ROTATE = 32
SETTLE_S = 0.25                  # untimed run of the decode step before its warm-up steps


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--tokens", type=int, default=64, help="decode batch of the headline step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="only the headline decode step")
    p.add_argument("--only", choices=["decode", "prefill", "dense", "pack", "w4a4", "block", "bf16", "shards"], default=None,
                   help="run one workload only (profiling runs); prints its figures")
    p.add_argument("--layout", choices=["tiled", "rows"], default="tiled",
                   help="weight layout in HBM: blocks of 32 rows (tiled) or row-major")
    p.add_argument("--calibrate-copy-mib", default="64,256",
                   help="comma-separated sizes of plain device copies run once each after the "
                        "workload, then one elementwise negation of the largest (counter "
                        "calibration); 0 for none")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the library has no multi-GPU "
                                   "(expert- or tensor-parallel) path; run it with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import nvfp4_moe_expert_amd as nv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nv.load_library()
    lay = nv.LAYOUT_TILED32 if args.layout == "tiled" else nv.LAYOUT_ROWS

    # ---------------------------------------------------------------- weights
    raw, layer = {}, {}
    if args.only != "dense":
        log("drawing the 288-expert layer (bf16 ~ N(0, 0.02)) and packing it on the device")
        raw.update({
            "gate": synth.torch_bf16_normal((E, I, H), 0.02, 51, dev),
            "up": synth.torch_bf16_normal((E, I, H), 0.02, 52, dev),
            "down": synth.torch_bf16_normal((E, H, I), 0.02, 53, dev),
        })
        layer.update({k: nv.pack(v, layout=lay) for k, v in raw.items()})
        torch.cuda.synchronize()

    def decode_inputs(T, seed):
        xs, ids, ws = [], [], []
        for r in range(ROTATE):
            xs.append(synth.bf16_normal((T, H), 1.0, seed, synth.S_X, T, r))
            i_, w_ = synth.topk_softmax_routing(T, E, K_TOP, seed, synth.S_ROUTE, T, r)
            ids.append(i_)
            ws.append(w_)
        x = torch.from_numpy(np.stack(xs).view(np.int16)).view(torch.bfloat16).to(dev)
        idt = torch.from_numpy(np.stack(ids)).to(dev)
        wt = torch.from_numpy(np.stack(ws)).to(dev)
        touched = [len(np.unique(i_)) for i_ in ids]
        return x, idt, wt, touched

    def alg_bytes(T, U):
        return U * (EXPERT_BYTES + 3 * 4) + 2 * T * H * 2 + 2 * T * K_TOP * 4

    def run_decode(T, steps, warmup, seed=3):
        x, ids, w, touched = decode_inputs(T, seed)
        ws = torch.empty((nv.moe_workspace_size(T, K_TOP, E, H, I),), dtype=torch.uint8, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        nev = 5
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
        # untimed settle before the warm-up steps: the same call for at least SETTLE_S seconds, so that the
        # timed steps run at the clocks of sustained work whatever the warm-up count (with 5 warm-up steps
        # and 20 timed ones the step measured 1.5-3% slower than after 10 and 50 without it)
        t_end, i = time.perf_counter() + SETTLE_S, 0
        while time.perf_counter() < t_end:
            for _ in range(16):
                r = i % ROTATE
                nv.moe_grouped(x[r], ids[r], w[r], layer["gate"], layer["up"], layer["down"], workspace=ws, out=out)
                i += 1
            torch.cuda.synchronize()
        for i in range(warmup):
            r = i % ROTATE
            nv.moe_grouped(x[r], ids[r], w[r], layer["gate"], layer["up"], layer["down"], workspace=ws, out=out)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        # timed region: the plain calls (value, ms_per_step)
        t0.record()
        for i in range(steps):
            r = (warmup + i) % ROTATE
            nv.moe_grouped(x[r], ids[r], w[r], layer["gate"], layer["up"], layer["down"], workspace=ws, out=out)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        # the same steps again with HIP events recorded between the library's stages on
        # its stream (per-kernel durations for the roofline); not part of `value`
        for i in range(steps):
            r = (warmup + i) % ROTATE
            nv.moe_grouped(x[r], ids[r], w[r], layer["gate"], layer["up"], layer["down"], workspace=ws, out=out,
                           events=evs[i])
        torch.cuda.synchronize()
        us = [touched[(warmup + i) % ROTATE] for i in range(steps)]
        stage = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(nev - 1)] for i in range(steps)])
        total_bytes = sum(alg_bytes(T, u) for u in us)
        gateup_bytes = sum(u * (GATEUP_BYTES + 2 * 4) + T * H * 2 for u in us)
        down_bytes = sum(u * (DOWN_BYTES + 4) for u in us)
        return {
            "T": T, "ms_total": ms, "ms_per_step": ms / steps, "gbs": total_bytes / (ms * 1e-3) / 1e9,
            "experts_touched_mean": float(np.mean(us)),
            "stage_ms_mean": {n: float(stage[:, j].mean()) for j, n in enumerate(["route", "gate_up", "down", "combine"])},
            "gateup_gbs": gateup_bytes / (stage[:, 1].sum() * 1e-3) / 1e9,
            "down_gbs": down_bytes / (stage[:, 2].sum() * 1e-3) / 1e9,
            "gateup_bytes_per_launch": gateup_bytes / steps,
            # per-step times of the event pass (first to last event of each call)
            "step_ms_event": {q: float(np.percentile(stage.sum(axis=1), p))
                              for q, p in (("min", 0), ("p50", 50), ("p90", 90))},
        }

    def w4a4_scales():
        """Synthetic calibration following the model card's policy (per expert the
        amax of each projection's input, the 99th percentile across experts, a 5%
        margin, / 2688) on 18 of the 288 experts and 256 N(0, 1) calibration rows,
        in fp32 on the dequantized weights. The scales decide how often a block
        saturates, not how much work a call does."""
        gen = torch.Generator(device=dev)
        gen.manual_seed(77)
        xf = torch.randn((256, H), generator=gen, device=dev).to(torch.bfloat16).float()
        ax, ah = [], []
        for e in range(0, E, 16):
            _, gs = nv.dequant(layer["gate"].expert(e), unscaled=False)
            _, us = nv.dequant(layer["up"].expert(e), unscaled=False)
            hh = torch.nn.functional.silu(xf @ gs[0].T) * (xf @ us[0].T)
            ax.append(xf.abs().max().item())
            ah.append(hh.abs().max().item())
        f = lambda a: float(np.float32(1.05 * np.percentile(a, 99) / 2688.0))
        return torch.tensor([f(ax), f(ah)], dtype=torch.float32, device=dev)

    def run_w4a4(T_dec, steps, warmup):
        """W4A4 activations (nvfp4_moe_grouped_w4a4): the decode step at T_dec and
        the prefill layer, plain timed loops."""
        log(f"W4A4: decode T={T_dec}, prefill T=4096")
        sc = w4a4_scales()
        x, ids, w, touched = decode_inputs(T_dec, 3)
        ws = torch.empty((nv.moe_workspace_size(T_dec, K_TOP, E, H, I),), dtype=torch.uint8, device=dev)
        out = torch.empty((T_dec, H), dtype=torch.bfloat16, device=dev)
        call = lambda r: nv.moe_grouped(x[r], ids[r], w[r], layer["gate"], layer["up"], layer["down"], workspace=ws,
                                        out=out, input_scales=sc)
        for i in range(warmup):
            call(i % ROTATE)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            call((warmup + i) % ROTATE)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        dec_bytes = sum(alg_bytes(T_dec, touched[(warmup + i) % ROTATE]) for i in range(steps))
        Tp = 4096
        ids_np, w_np = synth.zipf_routing(Tp, E, K_TOP, 1.1, 4, synth.S_ROUTE)
        xp = torch.from_numpy(synth.bf16_normal((Tp, H), 1.0, 4, synth.S_X).view(np.int16)).view(torch.bfloat16).to(dev)
        idp, wp = torch.from_numpy(ids_np).to(dev), torch.from_numpy(w_np).to(dev)
        wsp = torch.empty((nv.moe_workspace_size(Tp, K_TOP, E, H, I),), dtype=torch.uint8, device=dev)
        outp = torch.empty((Tp, H), dtype=torch.bfloat16, device=dev)
        pcall = lambda: nv.moe_grouped(xp, idp, wp, layer["gate"], layer["up"], layer["down"], workspace=wsp,
                                       out=outp, input_scales=sc)
        for _ in range(3):
            pcall()
        torch.cuda.synchronize()
        psteps = max(3, min(steps, 20))
        t0.record()
        for _ in range(psteps):
            pcall()
        t1.record()
        torch.cuda.synchronize()
        pms = t0.elapsed_time(t1) / psteps
        flops = 6.0 * Tp * K_TOP * H * I
        return {"input_scales": [round(v, 9) for v in sc.tolist()],
                f"decode_T{T_dec}": {"GB/s": round(dec_bytes / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms / steps, 5),
                                     "frac_hbm": round(dec_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                "prefill_T4096_zipf": {"TFLOP/s": round(flops / pms / 1e9, 2), "ms_per_call": round(pms, 4),
                                       "frac_mfma_bf16": round(flops / pms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}}

    def run_block(T_dec, steps, warmup):
        """The whole MoE block (nvfp4_moe_block): BF16 router over the 288 experts
        (top-8 softmax), routed NVFP4 experts, BF16 shared expert (intermediate 1536,
        a reading: the pages do not size it), at the decode batch and at 4096 tokens."""
        log(f"MoE block: T={T_dec} and T=4096")
        Is = I
        wr = synth.torch_bf16_normal((E, H), 0.02, 71, dev)
        sg = synth.torch_bf16_normal((Is, H), 0.02, 72, dev)
        su = synth.torch_bf16_normal((Is, H), 0.02, 73, dev)
        sd = synth.torch_bf16_normal((H, Is), 0.02, 74, dev)
        out = {}
        for T in (T_dec, 4096):
            xs = [torch.from_numpy(synth.bf16_normal((T, H), 1.0, 6, synth.S_X, T, r).view(np.int16))
                  .view(torch.bfloat16).to(dev) for r in range(ROTATE if T <= 64 else 1)]
            ws = torch.empty((nv.moe_block_workspace_size(T, K_TOP, E, H, I, Is),), dtype=torch.uint8, device=dev)
            y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            call = lambda r: nv.moe_block(xs[r % len(xs)], wr, K_TOP, layer["gate"], layer["up"], layer["down"],
                                          sg, su, sd, workspace=ws, out=y)
            n = steps if T <= 64 else max(3, min(steps, 20))
            for i in range(warmup if T <= 64 else 3):
                call(i)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for i in range(n):
                call(i)
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / n
            out[f"T{T}_ms_per_call"] = round(ms, 4)
        return {"workload": "MoE block: router 288 x 4096 + routed NVFP4 experts + shared BF16 expert 4096 -> 1536",
                **out}

    def run_bf16_experts(T_dec, steps, warmup):
        """The routed experts on their BF16 weights (nvfp4_moe_grouped_bf16, the MTP
        draft experts' alternative to packing), on the same bf16 draws the pack
        reads: decode at T_dec (HBM: 2 B per weight) and the prefill layer."""
        log(f"BF16 routed experts: decode T={T_dec}, prefill T=4096")
        x, ids, w, touched = decode_inputs(T_dec, 3)
        ws = torch.empty((nv.moe_grouped_bf16_workspace_size(T_dec, K_TOP, E, H, I),), dtype=torch.uint8, device=dev)
        out = torch.empty((T_dec, H), dtype=torch.bfloat16, device=dev)
        call = lambda r: nv.moe_grouped_bf16(x[r], ids[r], w[r], raw["gate"], raw["up"], raw["down"], workspace=ws,
                                             out=out)
        for i in range(warmup):
            call(i % ROTATE)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            call((warmup + i) % ROTATE)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        bpe = 3 * I * H * 2
        dec_bytes = sum(touched[(warmup + i) % ROTATE] * bpe + 2 * T_dec * H * 2 + 2 * T_dec * K_TOP * 4
                        for i in range(steps))
        Tp = 4096
        ids_np, w_np = synth.zipf_routing(Tp, E, K_TOP, 1.1, 4, synth.S_ROUTE)
        xp = torch.from_numpy(synth.bf16_normal((Tp, H), 1.0, 4, synth.S_X).view(np.int16)).view(torch.bfloat16).to(dev)
        idp, wp = torch.from_numpy(ids_np).to(dev), torch.from_numpy(w_np).to(dev)
        wsp = torch.empty((nv.moe_grouped_bf16_workspace_size(Tp, K_TOP, E, H, I),), dtype=torch.uint8, device=dev)
        outp = torch.empty((Tp, H), dtype=torch.bfloat16, device=dev)
        pcall = lambda: nv.moe_grouped_bf16(xp, idp, wp, raw["gate"], raw["up"], raw["down"], workspace=wsp, out=outp)
        for _ in range(2):
            pcall()
        torch.cuda.synchronize()
        psteps = max(3, min(steps, 10))
        t0.record()
        for _ in range(psteps):
            pcall()
        t1.record()
        torch.cuda.synchronize()
        pms = t0.elapsed_time(t1) / psteps
        flops = 6.0 * Tp * K_TOP * H * I
        return {f"decode_T{T_dec}": {"GB/s": round(dec_bytes / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms / steps, 5),
                                     "frac_hbm": round(dec_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                "prefill_T4096_zipf": {"TFLOP/s": round(flops / pms / 1e9, 2), "ms_per_call": round(pms, 4),
                                       "frac_mfma_bf16": round(flops / pms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}}

    def run_shards(steps, warmup):
        """One GPU's share of the sharded layer at its real shape: expert parallel
        over 8 GPUs (36 local experts of the 288 ids, expert_begin = 36, so the
        other ids are skipped) and tensor parallel over I (I/4 = 384 and I/8 = 192,
        gate/up rows and down columns split, whole 16-input groups kept), each at
        the 64-token decode batch (rotating routings) and the 4096-token Zipf
        layer. Expert-parallel calls run with the class picked automatically and
        pinned; tensor-parallel down weights stay row-major (the tiled layout needs
        inputs in multiples of 256)."""
        out = {}
        Tp = 4096
        ids_p, w_p = synth.zipf_routing(Tp, E, K_TOP, 1.1, 4, synth.S_ROUTE)
        xp = torch.from_numpy(synth.bf16_normal((Tp, H), 1.0, 4, synth.S_X).view(np.int16)).view(torch.bfloat16).to(dev)
        idp, wpt = torch.from_numpy(ids_p).to(dev), torch.from_numpy(w_p).to(dev)

        def timed(call, n):
            for i in range(warmup):
                call(i)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for i in range(n):
                call(warmup + i)
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / n

        def leg(name, gate, up, down, Esh, Ish, eb, cls):
            x, ids, w, _ = decode_inputs(64, 3)
            ws = torch.empty((nv.moe_workspace_size(64, K_TOP, Esh, H, Ish),), dtype=torch.uint8, device=dev)
            y = torch.empty((64, H), dtype=torch.bfloat16, device=dev)
            call = lambda i: nv.moe_grouped(x[i % ROTATE], ids[i % ROTATE], w[i % ROTATE], gate, up, down,
                                            expert_begin=eb, workspace=ws, out=y, kernel_class=cls)
            ms = timed(call, steps)
            ids_h = [ids[(warmup + i) % ROTATE].cpu().numpy() for i in range(steps)]
            touched = np.mean([len(np.unique(a[(a >= eb) & (a < eb + Esh)])) for a in ids_h])
            bpe = 3 * Ish * H * W_BYTES
            dec = {"GB/s": round(touched * bpe / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms, 5),
                   "local_experts_touched_mean": round(float(touched), 2)}
            dec["frac_hbm"] = round(dec["GB/s"] / HBM_PEAK_GBS, 4)
            wsp = torch.empty((nv.moe_workspace_size(Tp, K_TOP, Esh, H, Ish),), dtype=torch.uint8, device=dev)
            yp = torch.empty((Tp, H), dtype=torch.bfloat16, device=dev)
            pms = timed(lambda i: nv.moe_grouped(xp, idp, wpt, gate, up, down, expert_begin=eb, workspace=wsp,
                                                 out=yp, kernel_class=cls), max(3, min(steps, 10)))
            local = int(((ids_p >= eb) & (ids_p < eb + Esh)).sum())
            fl = 6.0 * local * H * Ish
            pre = {"TFLOP/s": round(fl / pms / 1e9, 2), "ms_per_call": round(pms, 4), "local_rows": local,
                   "frac_mfma_bf16": round(fl / pms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
            plans = {T: nv.moe_plan(T, K_TOP, Esh, H, Ish, gate.layout, down.layout,
                                    nv.CLASS_AUTO if cls is None else cls) for T in (64, Tp)}
            out[name] = {"decode_T64": dec, "prefill_T4096_zipf": pre,
                         "kernels": {str(T): f"{p['gate_up']} + {p['down']}" for T, p in plans.items()}}

        # expert parallel: GPU 1 of 8 holds experts 36..71 (its slice of the packed layer)
        ep = {k_: nv.NVFP4Weight(v.codes[36:72], v.scales[36:72], v.scale_2[36:72], v.layout) for k_, v in layer.items()}
        log("shards: expert parallel 36 of 288 experts")
        leg("ep8_36_experts_auto", ep["gate"], ep["up"], ep["down"], 36, I, 36, None)
        leg("ep8_36_experts_decode_class", ep["gate"], ep["up"], ep["down"], 36, I, 36, nv.CLASS_DECODE)
        del ep
        for G in (4, 8):
            Ish = I // G
            log(f"shards: tensor parallel I/{G} = {Ish}")
            tg = nv.pack(raw["gate"][:, :Ish, :].contiguous(), layout=lay)
            tu = nv.pack(raw["up"][:, :Ish, :].contiguous(), layout=lay)
            td = nv.pack(raw["down"][:, :, :Ish].contiguous(), layout=nv.LAYOUT_ROWS)
            leg(f"tp{G}_I{Ish}", tg, tu, td, E, Ish, 0, None)
            del tg, tu, td
        return out

    def run_prefill():
        log("prefill T=4096 Zipf(1.1)")
        Tp = 4096
        ids_np, w_np = synth.zipf_routing(Tp, E, K_TOP, 1.1, 4, synth.S_ROUTE)
        xp = torch.from_numpy(synth.bf16_normal((Tp, H), 1.0, 4, synth.S_X).view(np.int16)).view(torch.bfloat16).to(dev)
        idp, wp = torch.from_numpy(ids_np).to(dev), torch.from_numpy(w_np).to(dev)
        wsp = torch.empty((nv.moe_workspace_size(Tp, K_TOP, E, H, I),), dtype=torch.uint8, device=dev)
        outp = torch.empty((Tp, H), dtype=torch.bfloat16, device=dev)
        psteps = max(3, min(args.steps, 20))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(psteps)]
        for _ in range(3):
            nv.moe_grouped(xp, idp, wp, layer["gate"], layer["up"], layer["down"], workspace=wsp, out=outp)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(psteps):
            nv.moe_grouped(xp, idp, wp, layer["gate"], layer["up"], layer["down"], workspace=wsp, out=outp,
                           events=evs[i])
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / psteps
        flops = 6.0 * Tp * K_TOP * H * I
        st = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)] for i in range(psteps)]).mean(0)
        return {
            "workload": "prefill-shaped MoE layer, 4096 tokens, Zipf(1.1) routing", "TFLOP/s": round(flops / ms / 1e9, 2),
            "ms_per_call": round(ms, 4), "frac_mfma_bf16": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "stages_ms": dict(zip(["route", "gate_up", "down", "combine"], [round(v, 4) for v in st])),
            "rows_max_expert": int(np.bincount(ids_np.ravel(), minlength=E).max())}

    def run_dense():
        log("dense MLP 2048 x 4096 -> 12288 -> 4096")
        M, F = 2048, 12288
        dg = nv.pack(synth.torch_bf16_normal((F, H), 0.02, 61, dev), layout=lay)
        du = nv.pack(synth.torch_bf16_normal((F, H), 0.025, 62, dev), layout=lay)
        dd = nv.pack(synth.torch_bf16_normal((H, F), 0.02, 63, dev), layout=lay)
        xm = torch.from_numpy(synth.bf16_normal((M, H), 1.0, 5, synth.S_X).view(np.int16)).view(torch.bfloat16).to(dev)
        hm = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        ym = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        for _ in range(2):
            nv.linear_gated(xm, dg, du, out=hm)
            nv.linear(hm, dd, out=ym)
        torch.cuda.synchronize()
        dsteps = max(3, min(args.steps, 10))
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        tg = td = 0.0
        for _ in range(dsteps):
            e0.record()
            nv.linear_gated(xm, dg, du, out=hm)
            e1.record()
            nv.linear(hm, dd, out=ym)
            e2.record()
            torch.cuda.synchronize()
            tg += e0.elapsed_time(e1)
            td += e1.elapsed_time(e2)
        tg, td = tg / dsteps, td / dsteps
        fg, fd = 2.0 * M * H * F * 2, 2.0 * M * F * H
        return {
            "workload": "dense Fp4Linear MLP 2048 x 4096 -> 12288 -> 4096", "TFLOP/s": round((fg + fd) / (tg + td) / 1e9, 2),
            "ms_per_call": round(tg + td, 4), "frac_mfma_bf16": round((fg + fd) / (tg + td) / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "gated_ms": round(tg, 4), "down_ms": round(td, 4),
            "gated_tflops": round(fg / tg / 1e9, 2), "down_tflops": round(fd / td / 1e9, 2)}

    def run_pack():
        log("pack of 288 experts x 3 projections")
        pk_steps = 3
        for k_ in raw:
            nv.pack(raw[k_], layout=lay)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(pk_steps):
            for k_ in raw:
                nv.pack(raw[k_], layout=lay)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / pk_steps
        nw = 3 * E * I * H
        pbytes = nw * 2 + nw * W_BYTES + 3 * E * 4
        return {"workload": "pack of 288 experts x 3 projections (4096 x 1536 each)",
                "GB/s": round(pbytes / (ms * 1e-3) / 1e9, 1), "ms_per_call": round(ms, 3),
                "frac_hbm": round(pbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    def calibrate():
        """Kernels of known traffic, in dispatch order, for scaling the FETCH_SIZE and
        WRITE_SIZE counters: per size a fill (writes n x 4 bytes) and a blit copy
        (reads and writes n x 4), then a torch elementwise negation of the largest
        (reads and writes n x 4)."""
        sizes = [int(v) for v in str(args.calibrate_copy_mib).split(",") if v.strip()]
        sizes = [v for v in sizes if v > 0]
        out = []
        a = b = None
        for mib in sizes:
            del a, b
            n = mib * (1 << 20) // 4
            a = torch.ones(n, dtype=torch.float32, device=dev)
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
            out.append({"kind": "fill", "read": 0, "write": n * 4})
            out.append({"kind": "copy", "read": n * 4, "write": n * 4})
        if sizes:
            torch.neg(a, out=b)
            torch.cuda.synchronize()
            out.append({"kind": "neg", "read": a.numel() * 4, "write": a.numel() * 4})
        del a, b
        return out

    if args.only is not None:
        # one workload alone (profiling runs): its figures only, no headline line
        fig = {"decode": lambda: run_decode(args.tokens, args.steps, args.warmup), "prefill": run_prefill,
               "dense": run_dense, "pack": run_pack,
               "w4a4": lambda: run_w4a4(args.tokens, args.steps, args.warmup),
               "block": lambda: run_block(args.tokens, args.steps, args.warmup),
               "bf16": lambda: run_bf16_experts(args.tokens, args.steps, args.warmup),
               "shards": lambda: run_shards(args.steps, args.warmup)}[args.only]()
        cal = calibrate()
        if cal:
            fig["calibration"] = cal
        print(json.dumps({"only": args.only, **fig}), flush=True)
        return

    # ------------------------------------------------------- headline: decode
    log(f"decode T={args.tokens}: warmup {args.warmup}, timed {args.steps}")
    head = run_decode(args.tokens, args.steps, args.warmup)
    traffic = measured_traffic(args.tokens, args.layout)
    result = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "dtype_note": ("matrix-core operands of the routed GEMMs: NVFP4 weights dequantized exactly into fp16, the "
                       "bf16 activations scaled per row by a power of two into fp16 (exact down to 2^-28 of the row "
                       "maximum); fp32 accumulation; bf16 in and out"),
        "data": "synthetic",
        "config": {"workload": f"decode-shaped MoE layer, {args.tokens} tokens", "experts": E, "top_k": K_TOP,
                   "hidden": H, "intermediate": I, "tokens": args.tokens, "weights": "NVFP4 (e2m1, e4m3/16, fp32 scale_2)",
                   "weight_layout": args.layout,
                   "activations": "bf16", "routing": "top-8 softmax over N(0,1) logits, 32 rotating draws"},
        "roofline": {"bound": "hbm", "kernel": "gemm_decode_kernel<gate_up, fp16 dequant>",
                     "achieved": round(head["gateup_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["gateup_gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     # frac is the gate/up kernel's; the whole step (route, gate/up, down, combine):
                     "step_frac": round(head["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic_over_algorithmic": (round(traffic / head["gateup_bytes_per_launch"], 3)
                                                  if traffic else None),
                     "algorithmic_bytes_per_launch": round(head["gateup_bytes_per_launch"]),
                     "avg_launch_ms": round(head["stage_ms_mean"]["gate_up"], 5)},
        "stages_ms": {k: round(v, 5) for k, v in head["stage_ms_mean"].items()},
        "step_ms_event_pass": {k: round(v, 5) for k, v in head["step_ms_event"].items()},
        "experts_touched_mean": head["experts_touched_mean"],
        "down_kernel_gbs": round(head["down_gbs"], 1),
    }

    if not args.no_extras:
        sweep = {}
        for T in (1, 2, 3, 4, 8, 16, 64):
            if T == args.tokens:
                continue
            log(f"decode T={T}")
            r = run_decode(T, args.steps, args.warmup)
            sweep[str(T)] = {"GB/s": round(r["gbs"], 1), "ms_per_step": round(r["ms_per_step"], 5),
                             "frac_hbm": round(r["gbs"] / HBM_PEAK_GBS, 4),
                             "experts_touched_mean": r["experts_touched_mean"],
                             "stages_ms": {k: round(v, 5) for k, v in r["stage_ms_mean"].items()}}
        result["decode_sweep"] = sweep

        result["prefill"] = run_prefill()
        result["dense_mlp"] = run_dense()
        result["pack"] = run_pack()
        result["w4a4"] = run_w4a4(args.tokens, args.steps, args.warmup)
        result["moe_block"] = run_block(args.tokens, args.steps, args.warmup)
        result["bf16_experts"] = run_bf16_experts(args.tokens, args.steps, args.warmup)

        # the same headline step on the other weight layout (same values, other byte order)
        other = "rows" if args.layout == "tiled" else "tiled"
        log(f"decode T={args.tokens}, {other} weight layout")
        kept = dict(layer)
        to = nv.LAYOUT_ROWS if other == "rows" else nv.LAYOUT_TILED32
        layer.update({k: nv.relayout(v, to) for k, v in kept.items()})
        r = run_decode(args.tokens, args.steps, args.warmup)
        result[f"decode_T{args.tokens}_{other}_layout"] = {
            "GB/s": round(r["gbs"], 1), "ms_per_step": round(r["ms_per_step"], 5),
            "gateup_kernel_gbs": round(r["gateup_gbs"], 1), "down_kernel_gbs": round(r["down_gbs"], 1)}
        layer.update(kept)
        del kept

    # --------------------------------------------- counter calibration copies
    cal = calibrate()
    if cal:
        result["calibration"] = cal

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(raw, torch, synth)
        if not args.no_extras:
            result["cpu_baseline_configs"] = cpu_baseline_configs(raw, torch, synth)

    print(json.dumps(result), flush=True)


def measured_traffic(tokens, layout):
    """HBM bytes per gate/up launch from the committed counter summary
    (profiles/traffic_gemm_decode_T64.md: FETCH_SIZE + WRITE_SIZE, copy-calibrated),
    or None when it does not apply: another batch or weight layout, or kernel
    sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_gemm_decode_T64.md")
    if tokens != 64 or not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        fp = os.path.join(ROOT, f)
        if not os.path.exists(fp):
            return None
        h.update(open(fp, "rb").read())
    if h.hexdigest() != rec.get("sources_sha256") or rec.get("layout") != layout:
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def cpu_baseline(raw, torch, synth):
    """The CPU oracle (float64 numpy) on a bounded sample of the same workload: one
    decode token, its 8 experts. The oracle packs those experts first (not timed),
    then its routed MLP is timed; GB/s uses the same algorithmic bytes."""
    from oracle import mlp as OM
    from oracle import nvfp4 as ONV
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    T = 1
    x = synth.bf16_normal((T, H), 1.0, 3, synth.S_X, T, 0)
    ids, w = synth.topk_softmax_routing(T, E, K_TOP, 3, synth.S_ROUTE, T, 0)
    experts = sorted(set(ids.ravel().tolist()))
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    packs = {p: [ONV.pack(host(raw[p][e])) for e in experts] for p in raw}
    stack = lambda p: (np.stack([c for c, _, _ in packs[p]]), np.stack([s for _, s, _ in packs[p]]),
                       np.array([s2 for _, _, s2 in packs[p]], np.float32))
    loc = {e: i for i, e in enumerate(experts)}
    lids = np.vectorize(lambda v: loc[int(v)])(ids).astype(np.int32)
    g, u, d = stack("gate"), stack("up"), stack("down")
    t0 = time.perf_counter()
    reps = 0
    while True:
        OM.moe(x, lids, w, g, u, d)
        reps += 1
        if time.perf_counter() - t0 > 10.0:
            break
    sec = (time.perf_counter() - t0) / reps
    nbytes = len(experts) * (EXPERT_BYTES + 12) + 2 * T * H * 2 + 2 * T * K_TOP * 4
    return {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"1 token of the decode-shaped layer ({len(experts)} experts x 3 projections), "
                      f"float64 numpy routed MLP, {reps} repetitions, {sec:.2f} s each",
            "host_cpus": len(os.sched_getaffinity(0))}


def _blas():
    """(library, threads) of numpy's BLAS as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if info:
            return info[0].get("internal_api", "?"), int(info[0].get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return "unknown", 1


def _timed(fn, min_s):
    """Seconds per call of fn(), repeated until min_s seconds have passed (at least once)."""
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return el / reps, reps


def cpu_baseline_configs(raw, torch, synth):
    """The CPU oracle timed on a bounded sample of each workload (float64 numpy
    contractions, float32 pack), with the BLAS thread count set to the host's CPUs
    for the run and restored afterwards. Figures use the same algorithmic bytes and
    flops as the GPU lines; each entry says what its sample was."""
    from oracle import mlp as OM
    from oracle import nvfp4 as ONV
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    out = {}
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        lib, nthreads = _blas()
        out["host"] = {"cores": cores, "blas": lib, "blas_threads": nthreads}
        log("CPU oracle per workload")
        # single NVFP4 linear X[4,512] . W[256,512]^T: pack then linear
        w1 = synth.bf16_normal((256, 512), 0.02, 1, synth.S_W)
        x1 = synth.bf16_normal((4, 512), 1.0, 1, synth.S_X)
        sp, rp = _timed(lambda: ONV.pack(w1), 0.5)
        p1 = ONV.pack(w1)
        sl, rl = _timed(lambda: OM.linear(x1, p1), 0.5)
        out["single_linear_4x512x256"] = {
            "pack_ms": round(sp * 1e3, 3), "pack_GB/s": round((256 * 512 * (2 + W_BYTES)) / sp / 1e9, 4),
            "linear_ms": round(sl * 1e3, 3), "linear_GFLOP/s": round(2 * 4 * 512 * 256 / sl / 1e9, 4),
            "sample": "the whole workload"}
        # grouped decode MoE: 16 experts, top-4, 8 tokens, 2048 -> 512
        E2, k2, T2, H2, I2 = 16, 4, 8, 2048, 512
        x2 = synth.bf16_normal((T2, H2), 1.0, 2, synth.S_X)
        ids2, w2 = synth.topk_softmax_routing(T2, E2, k2, 2, synth.S_ROUTE)
        wg = synth.expert_weights(E2, I2, H2, 0.02, 2, synth.S_GATE)
        t0 = time.perf_counter()
        packs2 = [ONV.pack_batch(wg), ONV.pack_batch(synth.expert_weights(E2, I2, H2, 0.02, 2, synth.S_UP)),
                  ONV.pack_batch(synth.expert_weights(E2, H2, I2, 0.02, 2, synth.S_DOWN))]
        sp2 = time.perf_counter() - t0
        sm2, _ = _timed(lambda: OM.moe(x2, ids2, w2, *packs2), 2.0)
        U2 = len(np.unique(ids2))
        b2 = U2 * 3 * I2 * H2 * W_BYTES + 2 * T2 * H2 * 2
        out["grouped_decode_moe_E16_T8"] = {
            "pack_s": round(sp2, 3), "pack_GB/s": round(3 * E2 * I2 * H2 * (2 + W_BYTES) / sp2 / 1e9, 4),
            "moe_ms": round(sm2 * 1e3, 2), "moe_GB/s": round(b2 / sm2 / 1e9, 4), "experts_touched": U2,
            "sample": "the whole workload (16 experts packed, all 8 tokens)"}
        # the 288-expert layer: oracle packs of the experts a sample touches
        packs = {}

        def layer_packs(experts):
            # the oracle packs the touched experts (not timed; threads: numpy releases the GIL)
            todo = [(e, p) for e in experts if e not in packs for p in ("gate", "up", "down")]
            with cf.ThreadPoolExecutor(max_workers=cores) as ex:
                res = list(ex.map(lambda j: ONV.pack(host(raw[j[1]][j[0]])), todo))
            for i in range(0, len(todo), 3):
                packs[todo[i][0]] = res[i:i + 3]
            st = lambda j: (np.stack([packs[e][j][0] for e in experts]), np.stack([packs[e][j][1] for e in experts]),
                            np.array([packs[e][j][2] for e in experts], np.float32))
            return st(0), st(1), st(2)

        def sample_moe(x, ids, w):
            experts = sorted(set(ids.ravel().tolist()))
            loc = {e: i for i, e in enumerate(experts)}
            lids = np.vectorize(lambda v: loc[int(v)])(ids).astype(np.int32)
            g, u, d = layer_packs(experts)
            sec, reps = _timed(lambda: OM.moe(x, lids, w, g, u, d), 2.0)
            return sec, reps, len(experts)

        for T in (1, 16, 64):
            x3 = synth.bf16_normal((T, H), 1.0, 3, synth.S_X, T)
            ids3, w3 = synth.topk_softmax_routing(T, E, K_TOP, 3, synth.S_ROUTE, T)
            sec, reps, U = sample_moe(x3[:1], ids3[:1], w3[:1])
            out[f"decode_layer_T{T}"] = {
                "ms_per_token": round(sec * 1e3, 1), "GB/s": round((U * EXPERT_BYTES + 2 * H * 2) / sec / 1e9, 4),
                "sample": f"token 0 of the {T}-token batch ({U} experts), {reps} repetitions"}
        xp = synth.bf16_normal((4096, H), 1.0, 4, synth.S_X)
        idp, wp = synth.zipf_routing(4096, E, K_TOP, 1.1, 4, synth.S_ROUTE)
        sel = np.arange(0, 4096, 1024)
        sec, reps, U = sample_moe(xp[sel], idp[sel], wp[sel])
        fl = 6.0 * len(sel) * K_TOP * H * I
        out["prefill_layer_T4096_zipf"] = {
            "s_per_sample": round(sec, 3), "TFLOP/s": round(fl / sec / 1e12, 6),
            "sample": f"{len(sel)} of the 4096 tokens (every 1024th, {U} experts), {reps} repetitions; "
                      f"the whole layer would take about {round(sec * 4096 / len(sel))} s"}
        # dense MLP rows and one projection's pack
        g5 = host(raw["gate"][0])
        sp5, _ = _timed(lambda: ONV.pack(g5), 2.0)
        out["pack_one_projection_1536x4096"] = {
            "s": round(sp5, 3), "GB/s": round(I * H * (2 + W_BYTES) / sp5 / 1e9, 4),
            "sample": "expert 0's gate projection; 288 x 3 would take about " + f"{round(sp5 * 864)} s"}
        M5, F5 = 2048, 12288
        wd5 = {k_: ONV.pack(synth.bf16_normal(shp, sig, 5, synth.S_W, j)) for j, (k_, shp, sig) in
               enumerate((("gate", (F5, H), 0.02), ("up", (F5, H), 0.025), ("down", (H, F5), 0.02)))}
        x5 = synth.bf16_normal((8, H), 1.0, 5, synth.S_X)
        sm5, reps5 = _timed(lambda: OM.dense_mlp(x5, wd5["gate"], wd5["up"], wd5["down"]), 3.0)
        out["dense_mlp_2048x4096x12288"] = {
            "s_per_sample": round(sm5, 3), "TFLOP/s": round(6.0 * 8 * H * F5 / sm5 / 1e12, 6),
            "sample": f"8 of the {M5} rows, {reps5} repetitions (weights dequantized per call, as the oracle does)"}
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    return out


if __name__ == "__main__":
    main()
