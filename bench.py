"""Benchmark of the DeepSeekMoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--decode-steps D] [--skewed-steps S] [--no-backward]

One step is one pass of the whole hot path over one batch of T=16384 tokens
at V3 shapes (hidden 7168, 256 routed experts in 8 groups keeping 4, top-8,
one shared expert, intermediate 2048): route -> quantise x -> permute ->
gate+up GEMM with fused SwiGLU requantisation -> down GEMM -> combine ->
bias update.  Inputs are seeded synthetic tensors already resident in HBM.
Prints one JSON line (rank 0).  On the same weights it also reports: the
decode batch (T=128, under "decode"), the standalone grouped GEMM over 256
groups with Multinomial(65536) rows ("grouped_gemm") and the skewed-load
layer (T=8192, Zipf(1.1) expert popularity, 100 steps of the bias update,
"skewed"), the backward pieces of the two expert GEMMs at T=16384 (input
and weight gradients: "backward") and the whole
expert-path backward step ("backward_step").
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s @T=16384 (TFLOPS, % FP8 MFMA peak); decode HBM GB/s"
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(cfg):
    import torch
    import synth
    import fp8_block_scaled_bias_amd as M
    shape = M.LayerShape(cfg.H, cfg.E, cfg.n_group, cfg.topk_group, cfg.k, cfg.I, cfg.n_shared)
    C = torch.from_numpy(synth.gen_centroids(cfg)).cuda()
    b = torch.from_numpy(synth.gen_bias(cfg)).cuda()
    t0 = time.time()
    layer = M.MoELayer.from_fp32_experts(shape, C, b, synth.gen_all_expert_weights(cfg, "gu"),
                                         synth.gen_all_expert_weights(cfg, "dn"))
    log(f"[bench] weights for {cfg.G} experts generated and quantised in {time.time() - t0:.1f}s")
    return layer


def x_device(cfg):
    import numpy as np
    import torch
    import synth
    return torch.from_numpy(synth.gen_x(cfg).view(np.int16)).cuda().view(torch.bfloat16)


def run_steps(layer, x, steps, warmup, update_bias):
    """Wall time of `steps` layer steps after `warmup` untimed ones, with HIP
    events around the gate+up launch only (the roofline's kernel, measured
    in the timed region); then, outside it, the same number of steps with
    events around every launch for the per-kernel breakdown (every event
    pair lengthens a step by a few microseconds, 14 of them by ~1 %)."""
    import torch
    for _ in range(warmup):
        layer.forward(x, update_bias=update_bias)
    torch.cuda.synchronize()
    live = {"gate_up": []}
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, update_bias=update_bias, events=live)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    events = {}
    for _ in range(steps):
        layer.forward(x, update_bias=update_bias, events=events)
    torch.cuda.synchronize()
    per_kernel = {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in events.items()}
    gu_live = sum(a.elapsed_time(b) for a, b in live["gate_up"]) / len(live["gate_up"])
    return wall, per_kernel, gu_live


def touched_experts(layer, T):
    import torch
    cnt = layer.buffers(T).counts
    torch.cuda.synchronize()
    return int((cnt > 0).sum().item())


def copy_probe(gib=1, reps=5):
    """A plain device-to-device copy of `gib` GiB (torch's copy kernel):
    the practical HBM ceiling, and the reference dispatch that scales the
    FETCH_SIZE / WRITE_SIZE counters of a profiled run to bytes."""
    import torch
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    out = {"bytes_per_copy": 2 * n, "ms": ms, "GB_s": 2 * n / (ms * 1e-3) / 1e9}
    # the read and write ceilings on their own: torch's int64 sum (reads
    # only) and zero_ (writes only) over 4 GiB, the practical bounds for the
    # weight-streaming decode GEMMs and for the stores of the weight gradient
    del src, dst
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    for name, fn in (("read", lambda: big.view(torch.int64).sum()), ("write", lambda: big.zero_())):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms_ = e0.elapsed_time(e1) / reps
        out[name + "_GB_s"] = big.numel() / (ms_ * 1e-3) / 1e9
    del big
    return out


def gemm_source_digest():
    """Digest of the grouped-GEMM kernel sources (both tile shapes)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("gemm_common.h", "gemm.hip", "gemm_wide.hip"):
        with open(os.path.join(ROOT, "fp8_block_scaled_bias_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bench_grouped_gemm(layer, reps=20, warmup=5):
    """Standalone block-scaled FP8 grouped GEMM: 256 groups (the layer's routed
    experts' weights), rows per group Multinomial(65536, uniform) at seed 0,
    A = N(0,1) activations quantised 1x128 on the GPU, bf16 output, no row
    gather.  Fused gate+up (K=7168, N=4096) and down (K=2048, N=7168), each
    timed alone (median of `reps` after `warmup`).  Roofline: the larger of
    the FP8 MFMA time and the HBM time of the algorithmic bytes (A + scales
    + all 256 groups' B + scales + C)."""
    import numpy as np
    import torch
    import synth
    import fp8_block_scaled_bias_amd as M
    s = layer.shape
    G, rows = s.E, s.E * 256
    counts = synth.gen_group_counts(rows, G, seed=0)
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    out = {"workload": "standalone grouped GEMM, 256 groups, Multinomial(65536) rows",
           "groups": G, "rows": rows, "rows_min": int(counts.min()), "rows_max": int(counts.max())}
    st = torch.cuda.current_stream()
    for name, K, N, B, Bs, seed in (("gate_up", s.H, 2 * s.I, layer.w_gu, layer.w_gu_s, 1),
                                    ("down", s.I, s.H, layer.w_dn, layer.w_dn_s, 2)):
        a = torch.from_numpy(synth.gen_gemm_activations(rows, K, seed).view(np.int16)).cuda()
        a = a.view(torch.bfloat16)
        aq = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
        asc = torch.empty((rows, K // 128), dtype=torch.float32, device="cuda")
        M.fp8_quant_1x128(a, rows, K, K, 0, aq, asc)
        del a
        c = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda")
        run = lambda: M.grouped_fp8_gemm(aq, asc, None, B, Bs, offs, G, rows, N, K, c)
        for _ in range(warmup):
            run()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            run()
            e1.record(st)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ts]))
        flop = 2.0 * rows * N * K
        nbytes = (rows * K + rows * (K // 128) * 4 + G * N * K + G * (N // 128) * (K // 128) * 4
                  + rows * N * 2)
        t_mfma, t_hbm = flop / (FP8_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)
        out[name] = {"K": K, "N": N, "ms": ms, "TFLOPS": flop / (ms * 1e-3) / 1e12,
                     "GB_s": nbytes / (ms * 1e-3) / 1e9, "algorithmic_bytes": nbytes,
                     "bound": "hbm" if t_hbm > t_mfma else "mfma",
                     "frac_of_bound": max(t_mfma, t_hbm) / (ms * 1e-3)}
        log(f"[bench] grouped GEMM {name}: {ms:.3f} ms, {out[name]['TFLOPS']:.0f} TFLOP/s, "
            f"{out[name]['GB_s']:.0f} GB/s, {out[name]['frac_of_bound']:.2f} of the "
            f"{out[name]['bound']} roof")
        del aq, asc, c
    out["dense_reference"] = dense_reference(s)
    return out


def dense_reference(s, reps=5, warmup=2):
    """Context for the GEMM rows: the 256x256 kernel on ONE dense group of the
    gate+up size (R = 9T rows x N = 2I x K = H, no ragged tiles, no gather,
    bf16 out; random E4M3 codes, scales in [0.5, 1.5)), and torch._scaled_mm
    (hipBLASLt) on the same codes with per-tensor scales - a plain FP8 GEMM
    without the 128-element block scales, so not the same arithmetic."""
    import numpy as np
    import torch
    import fp8_block_scaled_bias_amd as M
    R, N, K = 9 * 16384, 2 * s.I, s.H
    gen = torch.Generator(device="cuda").manual_seed(7)
    A = torch.randint(0, 256, (R, K), dtype=torch.uint8, device="cuda", generator=gen) & 0x77
    As = torch.rand((R, K // 128), device="cuda", generator=gen) + 0.5
    B = torch.randint(0, 256, (1, N, K), dtype=torch.uint8, device="cuda", generator=gen) & 0x77
    Bs = torch.rand((1, N // 128, K // 128), device="cuda", generator=gen) + 0.5
    C = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    o1 = torch.tensor([0, R], dtype=torch.int32, device="cuda")
    flop = 2.0 * R * N * K
    ms = _median_ms(lambda: M.grouped_fp8_gemm(A, As, None, B, Bs, o1, 1, R, N, K, C), reps, warmup)
    out = {"R": R, "N": N, "K": K, "block_scaled_one_group_ms": ms,
           "block_scaled_one_group_TFLOPS": flop / (ms * 1e-3) / 1e12}
    try:
        one = torch.tensor(1.0, device="cuda")
        a8, b8 = A.view(torch.float8_e4m3fn), B[0].view(torch.float8_e4m3fn).t()
        hb = _median_ms(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                 out_dtype=torch.bfloat16), reps, warmup)
        out["hipblaslt_per_tensor_ms"] = hb
        out["hipblaslt_per_tensor_TFLOPS"] = flop / (hb * 1e-3) / 1e12
    except Exception as e:  # the vendor library is context only
        out["hipblaslt_per_tensor_error"] = f"{type(e).__name__}: {str(e)[:120]}"
    log(f"[bench] dense reference {R}x{N}x{K}: block-scaled, one group {ms:.3f} ms; "
        f"hipBLASLt per-tensor {out.get('hipblaslt_per_tensor_ms', float('nan')):.3f} ms")
    del A, As, B, Bs, C
    torch.cuda.empty_cache()
    return out


def _median_ms(run, reps, warmup):
    import numpy as np
    import torch
    st = torch.cuda.current_stream()
    for _ in range(warmup):
        run()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        run()
        e1.record(st)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ts]))


def bench_backward(layer, T, reps=10, warmup=3):
    """Backward of the two expert GEMMs at T=16384.  Input gradients (backward for input):
    grouped_fp8_gemm_dgrad on the 257 experts' weights as stored for the
    forward.  Rows per group: Multinomial(T*k, uniform over E) at seed 0 plus the
    T-row shared group (R = 147,456); output gradients N(0,1) from a seeded
    device generator, quantised 1x128 along their contraction axis (untimed).
    down: dH [R, I] = dD [R, H] W_dn; gate+up: dX [R, H] = dGU [R, 2I] W_gu.
    Weight gradients (backward for weights): dW_g = dY_g^T A_g per expert with
    dY and A (N(0,1) bf16 from the same generator) quantised 128x1 along the
    tokens by fp8_quant_128x1_grouped (timed: both operands), then
    grouped_fp8_wgrad (fp32 dW, 15 / 30 GB: HBM-bound on its output)."""
    import numpy as np
    import torch
    import synth
    import fp8_block_scaled_bias_amd as M
    s = layer.shape
    G = s.E + s.n_shared
    counts = np.concatenate([synth.gen_group_counts(T * s.k, s.E, seed=0), [T] * s.n_shared])
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    R = int(counts.sum())
    gen = torch.Generator(device="cuda").manual_seed(2024)
    out = {"workload": "backward of the expert GEMMs, T=16384 (257 groups, R=%d rows)" % R}
    for name, W, Ws, N, K in (("down", layer.w_dn, layer.w_dn_s, s.H, s.I),
                              ("gate_up", layer.w_gu, layer.w_gu_s, 2 * s.I, s.H)):
        # forward C = A W^T with W [G, N, K]; dA = dY W contracts over N
        dy = torch.randn((R, N), dtype=torch.float32, device="cuda", generator=gen).to(torch.bfloat16)
        dyq = torch.empty((R, N), dtype=torch.uint8, device="cuda")
        dys = torch.empty((R, N // 128), dtype=torch.float32, device="cuda")
        M.fp8_quant_1x128(dy, R, N, N, 0, dyq, dys)
        del dy
        da = torch.empty((R, K), dtype=torch.bfloat16, device="cuda")
        g_ms = _median_ms(lambda: M.grouped_fp8_gemm_dgrad(dyq, dys, W, Ws, offs, G, R, N, K, da),
                          reps, warmup)
        flop = 2.0 * R * N * K
        tf = flop / (g_ms * 1e-3) / 1e12
        out[name] = {"dgrad_ms": g_ms, "dgrad_TFLOPS": tf, "dgrad_frac_fp8_peak": tf / FP8_PEAK_TFLOPS,
                     "contraction": N, "out_cols": K}
        log(f"[bench] backward {name}: dgrad {g_ms:.3f} ms ({tf:.0f} TFLOP/s), weights read as "
            f"stored for the forward")
        del dyq, dys, da
        # weight gradient dW_g = dY_g^T A_g: both operands quantised 128x1 along the
        # tokens (transposed, chunk-padded), fp32 output [G, N, K]
        cap = M.wgrad_chunks(R, G)
        dy = torch.randn((R, N), dtype=torch.float32, device="cuda", generator=gen).to(torch.bfloat16)
        a = torch.randn((R, K), dtype=torch.float32, device="cuda", generator=gen).to(torch.bfloat16)
        yq = torch.empty((cap, N, 128), dtype=torch.uint8, device="cuda")
        ys = torch.empty((cap, N), dtype=torch.float32, device="cuda")
        aq = torch.empty((cap, K, 128), dtype=torch.uint8, device="cuda")
        asc = torch.empty((cap, K), dtype=torch.float32, device="cuda")
        q_ms = _median_ms(lambda: (M.fp8_quant_128x1_grouped(dy, N, None, offs, G, R, N, yq, ys, cap),
                                   M.fp8_quant_128x1_grouped(a, K, None, offs, G, R, K, aq, asc, cap)),
                          5, 2)
        q_bytes = 3 * R * (N + K) + 4 * (N + K) * (R // 128)
        del dy, a
        dw = torch.empty((G, N, K), dtype=torch.float32, device="cuda")
        w_ms = _median_ms(lambda: M.grouped_fp8_wgrad(yq, ys, aq, asc, cap, offs, G, R, N, K, dw), 5, 2)
        nch = int(((counts + 127) // 128).sum())          # chunks the groups use
        w_bytes = (N + K) * 128 * nch + 4 * (N + K) * nch + 4 * G * N * K
        t_mfma, t_hbm = flop / (FP8_PEAK_TFLOPS * 1e12), w_bytes / (HBM_PEAK_GBS * 1e9)
        out[name].update({
            "quant_128x1_ms": q_ms, "quant_128x1_GB_s": q_bytes / (q_ms * 1e-3) / 1e9,
            "wgrad_ms": w_ms, "wgrad_TFLOPS": flop / (w_ms * 1e-3) / 1e12,
            "wgrad_GB_s": w_bytes / (w_ms * 1e-3) / 1e9, "wgrad_algorithmic_bytes": w_bytes,
            "wgrad_bound": "hbm" if t_hbm > t_mfma else "mfma",
            "wgrad_frac_of_bound": max(t_mfma, t_hbm) / (w_ms * 1e-3)})
        log(f"[bench] backward {name}: quant 128x1 {q_ms:.3f} ms, wgrad {w_ms:.3f} ms "
            f"({out[name]['wgrad_TFLOPS']:.0f} TFLOP/s, {out[name]['wgrad_GB_s']:.0f} GB/s, "
            f"{out[name]['wgrad_frac_of_bound']:.2f} of the {out[name]['wgrad_bound']} roof)")
        del yq, ys, aq, asc, dw
    return out


def bench_backward_step(layer, x, cfg, steps=3, warmup=1):
    """The layer's backward (MoELayer.backward) at T=16384 after a forward of
    the same batch that kept its bf16 gate/up outputs (the pages recompute
    only RMSNorm and MLA's up-projection in the backward and store the other
    activations in FP8/BF16): combine backward, dgrad of down, SwiGLU
    backward from the stored gate/up, dgrad of gate+up, unpermute, both
    weight gradients and the router's backward (dx and the centroids'
    gradient); dy N(0,1) bf16 (synth.gen_dy).  The input gradients read the
    weights as stored for the forward, so the backward depends on nothing
    made from the weights beforehand.  Flops counted: the GEMMs only, 2RHI
    for each of dgrad-down and wgrad-down, 4RHI for each of dgrad-gate+up
    and wgrad-gate+up (26.0 TFLOP).  The same backward is also timed after a
    forward that kept nothing (ms_per_step_recompute_gu: the gate+up GEMM
    runs again in the backward, 34.6 TFLOP).  Then a training step
    (forward + backward, wall clock) both ways; and the 128x128
    requantisation of fp32 master weights (fp8_quant_128x128 over both
    weight sets, the per-update cast after an optimizer step), timed on its
    own."""
    import time
    import numpy as np
    import torch
    import synth
    dy = torch.from_numpy(synth.gen_dy(cfg).view(np.int16)).cuda().view(torch.bfloat16)
    R = cfg.R
    unit = 2.0 * R * cfg.H * cfg.I

    def timed(keep):
        layer.forward(x, keep_gu=keep)
        for _ in range(warmup):
            layer.backward(dy, x)
        torch.cuda.synchronize()
        events = {}
        t0 = time.perf_counter()
        for _ in range(steps):
            layer.backward(dy, x, events=events)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        per = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in events.items()}
        return ms, per

    ms, per = timed(True)
    flop = unit * (1 + 1 + 2 + 2)
    out = {"workload": "layer backward (experts + router), T=16384, V3 shapes, after a forward "
                       "that stored its bf16 gate/up outputs", "ms_per_step": ms,
           "tokens_per_s": cfg.T / (ms * 1e-3), "TFLOPS": flop / (ms * 1e-3) / 1e12,
           "flop_per_step": flop, "per_stage_ms": per}
    log(f"[bench] backward step (gate/up stored by the forward): {ms:.3f} ms "
        f"({out['TFLOPS']:.0f} TFLOP/s); " + ", ".join(f"{k} {v:.3f}" for k, v in per.items()))
    ms_r, per_r = timed(False)
    out["ms_per_step_recompute_gu"] = ms_r
    out["per_stage_ms_recompute_gu"] = per_r
    log(f"[bench] backward step rerunning the gate+up GEMM: {ms_r:.3f} ms; " +
        ", ".join(f"{k} {v:.3f}" for k, v in per_r.items()))
    # a training step (forward + backward) both ways: the fused forward with
    # the gate+up GEMM run again in the backward, or the fused forward that
    # also keeps its bf16 gate/up outputs (1.2 GB) for the backward to read
    for name, keep in (("train_step_recompute", False), ("train_step_keep_gu", True)):
        layer.forward(x, keep_gu=keep)
        layer.backward(dy, x)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            layer.forward(x, keep_gu=keep)
            layer.backward(dy, x)
        torch.cuda.synchronize()
        out[name + "_ms"] = (time.perf_counter() - t0) / steps * 1e3
    log(f"[bench] training step: {out['train_step_recompute_ms']:.3f} ms recomputing gate+up, "
        f"{out['train_step_keep_gu_ms']:.3f} ms keeping it")
    # the per-update requantisation of fp32 master weights (expert by expert,
    # from one fp32 buffer per weight set: the timing covers the quantiser)
    s_ = layer.shape
    gu32 = torch.randn((s_.G, 2 * s_.I, s_.H), dtype=torch.float32, device="cuda").mul_(0.006)
    dn32 = torch.randn((s_.G, s_.H, s_.I), dtype=torch.float32, device="cuda").mul_(0.006)
    wq = [t.clone() for t in (layer.w_gu, layer.w_gu_s, layer.w_dn, layer.w_dn_s)]
    from fp8_block_scaled_bias_amd import _lib as L_
    def requant():
        L_.fp8_quant_128x128(gu32, s_.G, 2 * s_.I, s_.H, wq[0], wq[1])
        L_.fp8_quant_128x128(dn32, s_.G, s_.H, s_.I, wq[2], wq[3])
    q_ms = _median_ms(requant, 5, 1)
    q_bytes = 4.0 * (gu32.numel() + dn32.numel()) + (gu32.numel() + dn32.numel()) * 1.0
    out["requantize_weights_ms"] = q_ms
    out["requantize_weights_GB_s"] = q_bytes / (q_ms * 1e-3) / 1e9
    log(f"[bench] 128x128 requantisation of both fp32 weight sets: {q_ms:.3f} ms "
        f"({out['requantize_weights_GB_s']:.0f} GB/s)")
    del gu32, dn32, wq
    del dy
    return out


# HBM traffic of the gate+up kernel at T=16384, from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE) of this script, each scaled by the same counter on
# the 1 GiB copy probe.  Valid only for the kernel source with this digest.
GATE_UP_TRAFFIC = {"gemm_src": "7f1794fed54dc23c",
                   # FETCH_SIZE 9,126,703 KiB x 2.000 + WRITE_SIZE 311,385 KiB x 1.000
                   "bytes": 9126703 * 1024 * 2 + 311385 * 1024}


def bench_seq_balance(layer, x, cfg, seq_len=4096, steps=10, warmup=2, backward=True):
    """The layer forward with the sequence-wise balance statistic (sequences
    of seq_len tokens): per-step time, the router with its score output and
    the statistic itself (HIP events on the launch stream, mean over steps).
    The statistic reads T*E fp32 scores, T sums and T*k choices."""
    import time
    import numpy as np
    import torch
    for _ in range(warmup):
        layer.forward(x, seq_len=seq_len, update_bias=True)
    torch.cuda.synchronize()
    events = {}
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, seq_len=seq_len, update_bias=True, events=events)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    per = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in events.items()}
    nbytes = cfg.T * cfg.E * 4 + cfg.T * 4 + cfg.T * cfg.k * 4
    out = {"workload": f"layer forward with the sequence-wise balance statistic, T={cfg.T}, "
                       f"sequences of {seq_len}", "ms_per_step": ms,
           "route_with_scores_ms": per["route"], "seq_balance_ms": per["seq_balance"],
           "seq_balance_bytes": nbytes,
           "seq_balance_GB_s": nbytes / (per["seq_balance"] * 1e-3) / 1e9,
           "loss": layer.buffers(cfg.T).seq_loss.cpu().tolist()}
    log(f"[bench] seq balance: step {ms:.3f} ms, route+scores {per['route']:.3f} ms, "
        f"statistic {per['seq_balance']:.4f} ms, loss {out['loss']}")
    if not backward:
        return out
    # the layer's backward with the balance term: the router's dense backward
    # (fp32 GEMMs dlogit C and dlogit^T x: 2 * 2 T E H flop)
    import synth
    dy = torch.from_numpy(synth.gen_dy(cfg).view(np.int16)).cuda().view(torch.bfloat16)
    layer.forward(x, seq_len=seq_len)
    layer.backward(dy, x, seq_len=seq_len)
    torch.cuda.synchronize()
    bev = {}
    for _ in range(3):
        layer.backward(dy, x, seq_len=seq_len, events=bev)
    torch.cuda.synchronize()
    rb = float(np.mean([a.elapsed_time(b) for a, b in bev["router_bwd"]]))
    flop = 4.0 * cfg.T * cfg.E * cfg.H
    out.update({"router_bwd_dense_ms": rb, "router_bwd_dense_flop": flop,
                "router_bwd_dense_TFLOPS": flop / (rb * 1e-3) / 1e12})
    log(f"[bench] dense router backward: {rb:.3f} ms ({out['router_bwd_dense_TFLOPS']:.0f} TFLOP/s fp32)")
    del dy
    return out


def bench_skewed(layer, steps=100):
    """Skewed-load layer: T=8192 at V3 shapes, router centroids with
    Zipf(1.1)-scaled expert rows (stored fit), bias starting at 0, `steps`
    forward steps each on a fresh batch (seed 1000 + step) followed by the
    bias update (gamma = 0.001).  Per step: max/mean expert load of that
    step's routing and the forward time (HIP events on the launch stream).
    Batches are drawn on host threads ahead of use (not timed)."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import torch
    import synth
    import fp8_block_scaled_bias_amd as M
    cfg = synth.SKEWED
    C = torch.from_numpy(synth.gen_zipf_centroids(cfg)).cuda()
    b = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
    sk = M.MoELayer(layer.shape, C, b, layer.w_gu, layer.w_gu_s, layer.w_dn, layer.w_dn_s)
    st = torch.cuda.current_stream()
    loads, times = [], []
    mean = cfg.T * cfg.k / cfg.E
    with ThreadPoolExecutor(8) as ex:
        futs = [ex.submit(synth.gen_x, cfg, synth.ZIPF_STEP_SEED0 + i) for i in range(steps)]
        for i in range(steps):
            xb = torch.from_numpy(futs[i].result().view(np.int16)).cuda().view(torch.bfloat16)
            futs[i] = None
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            sk.forward(xb, update_bias=True)
            e1.record(st)
            cnt = sk.buffers(cfg.T).counts.cpu().numpy()
            times.append(e0.elapsed_time(e1))
            loads.append(float(cnt.max()) / mean)
    ms = float(np.median(times))
    flop = 2.0 * cfg.R * 3 * cfg.I * cfg.H
    log(f"[bench] skewed T={cfg.T}: max/mean load step 0 {loads[0]:.2f} -> step {steps - 1} "
        f"{loads[-1]:.2f}; median {ms:.3f} ms/step")
    return {"workload": "skewed-load layer, Zipf(1.1) centroids, bias update each step",
            "T": cfg.T, "steps": steps, "gamma": 0.001, "max_over_mean_load": loads,
            "ms_per_step": times, "median_ms": ms, "tokens_per_s": cfg.T / (ms * 1e-3),
            "TFLOPS": flop / (ms * 1e-3) / 1e12}


def cpu_baseline(cfg, dcfg, n_tokens=32, n_decode=8, decode_runs=3):
    """The FP64 oracle on bounded samples, with the BLAS threads set to the
    host cores this process may use (its CPU affinity, at most the
    OMP_NUM_THREADS share when that is set).  Prefill: the layer output of
    the first n_tokens tokens of the T=16384 batch, one run.  Decode: the
    layer output of the first n_decode tokens of the T=128 batch, the median
    of decode_runs runs.  Each sample covers the tokens' routes, the weights
    of every expert they touch and the shared expert; the weights' 128x128
    quantisation is setup, not timed (both workloads share the weights)."""
    import numpy as np
    import synth
    from threadpoolctl import threadpool_limits
    from oracle import layer as OL
    from oracle import route as OR
    wts = OL.ExpertWeights(lambda e: synth.gen_expert_weight(cfg, "gu", e),
                           lambda e: synth.gen_expert_weight(cfg, "dn", e))
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))

    def sample(c, n, runs):
        x = synth.gen_x(c)
        C = synth.gen_centroids(c)
        b = synth.gen_bias(c)
        toks = np.arange(n)
        r = OR.route(x[toks], C, b, c.n_group, c.topk_group, c.k)
        experts = set(r["idx"].ravel().tolist()) | {c.E}
        t0 = time.time()
        wts.prefetch(experts, threads=cores)
        log(f"[bench] cpu baseline {c.name}: {len(experts)} experts quantised in "
            f"{time.time() - t0:.1f}s (setup)")
        times = []
        with threadpool_limits(limits=cores):
            for _ in range(runs):
                t0 = time.perf_counter()
                OL.layer_tokens(x, C, b, wts, c.n_group, c.topk_group, c.k, c.I, toks)
                times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(experts), times

    dt, ne, _ = sample(cfg, n_tokens, 1)
    ddt, dne, dtimes = sample(dcfg, n_decode, decode_runs)
    log(f"[bench] cpu baseline: prefill {n_tokens / dt:.2f} tokens/s, decode "
        f"{n_decode / ddt:.2f} tokens/s ({cores} cores)")
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"FP64 oracle layer output for {n_tokens} of the {cfg.T} tokens "
                      f"({ne} experts incl. shared), one run, {dt:.1f}s",
            "decode": {"value": n_decode / ddt, "unit": "tokens/s", "cores": cores,
                       "kind": "oracle",
                       "sample": f"FP64 oracle layer output for {n_decode} of the {dcfg.T} "
                                 f"decode tokens ({dne} experts incl. shared), median of "
                                 f"{decode_runs} runs: " + ", ".join(f"{t:.1f}s" for t in dtimes)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--skewed-steps", type=int, default=100)
    ap.add_argument("--no-backward", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the layer holds all 256 experts on one "
              "MI355X and has no multi-GPU path (got --gpus %d, WORLD_SIZE %d)"
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    cfg = synth.PREFILL
    torch.cuda.set_device(0)
    layer = build_layer(cfg)
    x = x_device(cfg)

    cp = copy_probe()
    log(f"[bench] copy probe: {cp['GB_s']:.0f} GB/s; read alone {cp['read_GB_s']:.0f} GB/s, "
        f"write alone {cp['write_GB_s']:.0f} GB/s")
    log(f"[bench] prefill T={cfg.T}: warmup {args.warmup}, steps {args.steps}")
    wall, per, gu_live = run_steps(layer, x, args.steps, args.warmup, update_bias=True)
    ms = wall / args.steps * 1e3
    R = cfg.R
    flops_gu = 2.0 * R * (2 * cfg.I) * cfg.H
    flops_dn = 2.0 * R * cfg.H * cfg.I
    flops = flops_gu + flops_dn
    tflops = flops / (ms * 1e-3) / 1e12
    gu_ms = gu_live
    achieved_gu = flops_gu / (gu_ms * 1e-3) / 1e12
    log(f"[bench] per-kernel ms: " + ", ".join(f"{k} {v:.3f}" for k, v in per.items()))

    # decode batch on the same weights (HBM-bound weight streaming)
    dcfg = synth.DECODE
    xd = x_device(dcfg)
    dwall, dper, _ = run_steps(layer, xd, args.decode_steps, 5, update_bias=False)
    dms = dwall / args.decode_steps * 1e3
    touched = touched_experts(layer, dcfg.T)
    w_expert = 2 * dcfg.I * dcfg.H + dcfg.H * dcfg.I      # e4m3 bytes per expert
    sc_bytes = 4 * ((2 * dcfg.I // 128) * (dcfg.H // 128) + (dcfg.H // 128) * (dcfg.I // 128))
    dbytes = (touched + 1) * (w_expert + sc_bytes) + 4 * dcfg.E * dcfg.H + 2 * 2 * dcfg.T * dcfg.H
    dgbs = dbytes / (dms * 1e-3) / 1e9
    log(f"[bench] decode per-kernel ms: " + ", ".join(f"{k} {v:.3f}" for k, v in dper.items()))
    # the same decode step captured as one HIP graph and replayed
    gdec = layer.capture(xd)
    for _ in range(5):
        gdec.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.decode_steps):
        gdec.replay()
    torch.cuda.synchronize()
    gms = (time.perf_counter() - t0) / args.decode_steps * 1e3
    del gdec
    log(f"[bench] decode as a HIP graph: {gms:.3f} ms/step (eager {dms:.3f})")

    gg = bench_grouped_gemm(layer)
    bwd = bench_backward(layer, cfg.T) if not args.no_backward else None
    bstep = bench_backward_step(layer, x, cfg) if not args.no_backward else None
    skew = bench_skewed(layer, args.skewed_steps) if args.skewed_steps > 0 else None
    seqb = bench_seq_balance(layer, x, cfg, backward=not args.no_backward)

    traffic = None
    if GATE_UP_TRAFFIC and GATE_UP_TRAFFIC["gemm_src"] == gemm_source_digest():
        traffic = GATE_UP_TRAFFIC["bytes"]
    out = {
        "metric": METRIC,
        "value": cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulation)",
        "data": "synthetic (seeded; x N(0,1) bf16, centroids N(0,0.02), weights N(0,0.006) "
                "quantised 128x128 on the GPU)",
        "config": {"workload": "DeepSeekMoE layer forward, V3 shapes, prefill batch",
                   "T": cfg.T, "H": cfg.H, "E": cfg.E, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "k": cfg.k, "I": cfg.I,
                   "n_shared": cfg.n_shared, "global_batch": cfg.T, "parallelism": "none"},
        "tflops": tflops,
        "frac_fp8_peak": tflops / FP8_PEAK_TFLOPS,
        "per_kernel_ms": per,
        "roofline": {"bound": "mfma", "kernel": "grouped_fp8_gemm_swiglu (gate+up)",
                     "achieved": achieved_gu, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved_gu / FP8_PEAK_TFLOPS, "traffic": traffic,
                     "algorithmic_flop_per_launch": flops_gu, "avg_launch_ms": gu_ms},
        "decode": {"T": dcfg.T, "ms_per_step": dms, "graph_ms_per_step": gms,
                   "touched_experts": touched,
                   "algorithmic_bytes": dbytes, "GB_s": dgbs, "frac_hbm_peak": dgbs / HBM_PEAK_GBS,
                   "per_kernel_ms": dper},
        "grouped_gemm": gg,
        "backward": bwd,
        "backward_step": bstep,
        "skewed": skew,
        "seq_balance": seqb,
        "copy_probe": cp,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, dcfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
