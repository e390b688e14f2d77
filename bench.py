"""Throughput of the gen-tower denoise step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--variant V]

Workload: the 36-layer Qwen3-8B-shaped gen tower at 2048x2048 (4096 image tokens per
branch), CFG batch 2 (cond + uncond, each with its own 400-token prefix-KV cache per layer),
cfg 4.0, shifted flow Euler update (shift 3.0, t_eps 0.02), step 0 of the 50-step schedule.
One timed step = one gen_tower_step call: patch embed + 36 gen blocks over both branches +
final norm + out head + CFG/Euler.  Inputs are synthetic (seeded device RNG, the weight and
activation distributions of the test workloads) and resident in HBM before timing starts.

Prints ONE JSON line with image tokens/s (both branches), the fraction of the bf16 MFMA peak,
the median / min / max of the per-step times, a roofline entry for the dominant kernel (the
fused gate/up + SwiGLU GEMM; its launches are timed with HIP events on the library's stream in a
separate pass after the timed region, so the headline steps carry no per-launch events), the
whole step's own fraction of the peak, and the CPU oracle's rate on a bounded sample (one
full-size gen block, scaled to the 36-layer step).

Other report lines (--variant): block (one 8B gen block, 2 x 1024 tokens, prefix 400), moe (one
A3B MoE block, 2 x 4096 tokens), lora-tower (the 36-layer tower forward with an unmerged rank-32
LoRA, 4 x 1024 tokens, x0 out), lora-merged-cfg1, dual-cfg, prefix, lora-train.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_2048px_tower.traffic.json")
GEMM_SOURCES = ("pixel_space_flow_amd/csrc/gemm.hip", "pixel_space_flow_amd/csrc/gemm.h",
                "pixel_space_flow_amd/csrc/common.h")


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM-side bytes per launch of the gate/up GEMM from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (each scaled by the same counter's reading for a copy of known size), or
    None when the GEMM sources changed after the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != gemm_source_hash():
        return None
    return int((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024)


def step_flops(w) -> dict:
    """Algorithmic FLOPs of one gen_tower_step (2 per multiply-add), by component."""
    d = w.dims
    B, N, D = w.batch, w.n_tokens, d.hidden
    M = B * N
    QD, KV = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    f = {}
    f["qkv"] = 2 * M * D * (QD + 2 * KV)
    f["attention"] = sum(4 * d.n_q_heads * N * (w.prefix_len_of(b) + N) * d.head_dim for b in range(B))
    f["o"] = 2 * M * QD * D
    if d.is_moe:
        f["router"] = 2 * M * D * d.n_experts
        f["experts"] = 2 * M * d.top_k * 3 * D * d.expert_intermediate
    else:
        f["gate_up"] = 2 * M * D * 2 * d.mlp_intermediate
        f["down"] = 2 * M * d.mlp_intermediate * D
    if d.lora_rank:
        ins = (D, D, D, QD, D, D, d.mlp_intermediate)
        outs = (QD, KV, KV, D, d.mlp_intermediate, d.mlp_intermediate, D)
        f["lora"] = sum(2 * M * d.lora_rank * (i + o) for i, o in zip(ins, outs))
    per_layer = sum(f.values())
    out = {k: v * w.n_layers for k, v in f.items()}
    out["embed"] = 2 * w.n_img * N * 3072 * D
    out["head"] = 2 * M * D * 3072
    out["total"] = per_layer * w.n_layers + out["embed"] + out["head"]
    return out


def down_pitch(I: int) -> int:
    """Row pitch (elements) the benches give w_down: dense unless a dense bf16 row is a multiple of
    8 KiB (I = 12288), then I + 64, the layout the library streams fastest (gen_block_weights
    ld_down)."""
    return I + 64 if (2 * I) % 8192 == 0 else I


def down_weight(randn, D: int, I: int, std: float):
    """w_down [D, I] as a view of a [D, down_pitch(I)] allocation, and its pitch."""
    ld = down_pitch(I)
    return randn(D, ld, std=std)[:, :I], ld


def make_device_tower(psf, w, seed=0):
    """Random-init tower weights and prefixes on the GPU (torch's seeded device RNG)."""
    import torch
    d = w.dims
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = torch.bfloat16

    def randn(*shape, std=1.0, mean=0.0):
        t = torch.empty(*shape, device="cuda", dtype=torch.float32)
        t.normal_(mean, std, generator=g)
        return t.to(bf)

    D, I = d.hidden, d.mlp_intermediate
    QKV = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim
    layers_dev = []
    for _ in range(w.n_layers):
        lw = {"g_in": randn(D, std=0.1, mean=1.0), "w_qkv": randn(QKV, D, std=0.02),
              "g_q": randn(d.head_dim, std=0.1, mean=1.0), "g_k": randn(d.head_dim, std=0.1, mean=1.0),
              "w_o": randn(D, d.n_q_heads * d.head_dim, std=0.02), "g_post": randn(D, std=0.1, mean=1.0),
              "w_gate_up": randn(2 * I, D, std=0.02)}
        lw["w_down"], lw["ld_down"] = down_weight(randn, D, I, 0.02)
        layers_dev.append(lw)
    glob = {"w_in": randn(D, 3072, std=0.02), "temb_w1": randn(D, 256, std=0.02), "temb_w2": randn(D, D, std=0.02),
            "g_final": randn(D, std=0.1, mean=1.0), "w_out": randn(3072, D, std=0.02)}
    shp = [(w.prefix_len_of(s), d.n_kv_heads, d.head_dim) for s in range(w.batch)]
    pk = [randn(*shp[i % w.batch]) for i in range(w.n_layers * w.batch)]
    pv = [randn(*shp[i % w.batch]) for i in range(w.n_layers * w.batch)]
    x = torch.empty(w.n_img, 3, w.height, w.width, device="cuda")
    x.normal_(0.0, 1.0, generator=g)
    return layers_dev, glob, pk, pv, x


def merge_lora_at_load(psf, lw, layers_dev, seed=1):
    """Draw a rank-r LoRA per layer (A ~ N(0, 0.02), B ~ N(0, 1e-3), seeded device RNG) and fold
    it into each layer's weights in place with gen_block_lora_merge; returns the merge time (ms)."""
    import torch
    d = lw.dims
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    D, I, r = d.hidden, d.mlp_intermediate, d.lora_rank
    qd, kd = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    ins = {"q": D, "k": D, "v": D, "o": qd, "gate": D, "up": D, "down": I}
    outs = {"q": qd, "k": kd, "v": kd, "o": D, "gate": I, "up": I, "down": D}
    dims = psf.make_dims(d, psf.GEN_BF16)

    def randn(*shape, std):
        t = torch.empty(*shape, device="cuda", dtype=torch.float32)
        t.normal_(0.0, std, generator=g)
        return t.to(torch.bfloat16)
    loras = []
    for lwd in layers_dev:
        full = dict(lwd)
        for s in ("q", "k", "v", "o", "gate", "up", "down"):
            full[f"lora_a_{s}"] = randn(r, ins[s], std=0.02)
            full[f"lora_b_{s}"] = randn(outs[s], r, std=1e-3)
        loras.append(full)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for lwd, full in zip(layers_dev, loras):
        psf.block_lora_merge(dims, psf.make_weights(full), lwd["w_qkv"], lwd["w_o"], lwd["w_gate_up"], lwd["w_down"])
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop)


def prefix_flops(w) -> int:
    """Algorithmic FLOPs of the prompt pass over w.batch prompts of w.prefix_len tokens through
    w.n_layers blocks; causal attention counts only the visible (query, key) pairs."""
    d = w.dims
    B, P, D = w.batch, w.prefix_len, d.hidden
    M = B * P
    QD, KV = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    per = 2 * M * D * (QD + 2 * KV) + 4 * B * d.n_q_heads * d.head_dim * (P * (P + 1) // 2) + 2 * M * QD * D
    per += 2 * M * D * 2 * d.mlp_intermediate + 2 * M * d.mlp_intermediate * D
    return per * w.n_layers


def run_prefix_bench(psf, w, args):
    """gen_prefix_forward over the cond and uncond prompts (400 tokens each) through the 36-layer
    prompt tower, writing the per-layer prefix-KV cache: the pass that runs once per request
    before the denoise loop."""
    import torch
    import workloads as W
    d = W.prefix_dims(w)
    dims = psf.make_dims(d, psf.GEN_BF16)
    layers_dev, _, _, _, _ = make_device_tower(psf, W.scaled(w, dims=d), seed=2)
    layers = [psf.make_weights(l) for l in layers_dev]
    B, P = w.batch, w.prefix_len
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    h0 = torch.randn(B, P, d.hidden, device="cuda", generator=g)
    h = torch.empty_like(h0)
    shp = (P, d.n_kv_heads, d.head_dim)
    kc = [torch.empty(shp, device="cuda", dtype=torch.bfloat16) for _ in range(w.n_layers * B)]
    vc = [torch.empty(shp, device="cuda", dtype=torch.bfloat16) for _ in range(w.n_layers * B)]
    ws = psf.alloc_workspace(psf.workspace_size(dims, 1, B, P, 0))

    def step():
        h.copy_(h0)
        psf.prefix_forward(dims, layers, h, kc, vc, ws)

    ms, per = time_steps(step, args.steps, args.warmup)
    gu_avg, gu_n = kernel_pass(psf, "gate_up", w.n_layers, step, max(2, min(args.steps, 5)))
    M = B * P
    gu_tf = 2 * M * d.hidden * 2 * d.mlp_intermediate / (gu_avg * 1e-3) / 1e12
    tflops = prefix_flops(w) / (ms * 1e-3) / 1e12
    out = {
        "metric": "prompt tokens/s through the 36-layer prompt tower writing the prefix-KV cache; % bf16 MFMA peak",
        "value": round(M / (ms * 1e-3), 1), "unit": "prompt tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        **step_stats(per),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"qwen3-8b-prompt-tower{w.n_layers}-2x{P}tok", "layers": w.n_layers,
                   "prompts": B, "prompt_tokens": P, "hidden": d.hidden,
                   "heads": [d.n_q_heads, d.n_kv_heads, d.head_dim], "mlp_intermediate": d.mlp_intermediate,
                   "cache_bytes": 2 * w.n_layers * B * P * d.n_kv_heads * d.head_dim * 2},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "tflops": round(tflops, 1),
        "roofline": {"kernel": f"gate_up SwiGLU GEMM (M={M}, N=2x{d.mlp_intermediate}, K={d.hidden})",
                     "bound": "mfma", "achieved": round(gu_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": round(gu_avg, 4), "launches_timed": gu_n},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle as O
        wts = W.prefix_layer_weights(w, 0, 0, "bf16")
        hp = W.prompt_hidden(w, 0, "bf16")
        t0 = time.perf_counter()
        O.prefix_block(hp, wts, d)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(M / (dt * w.n_layers), 2), "unit": "prompt tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"one prompt-tower block ({B} x {P} tokens) in numpy fp32 took "
                                         f"{dt:.2f} s; scaled x{w.n_layers} layers",
                               **host_info()}
    print(json.dumps(out), flush=True)


def train_flops(w) -> dict:
    """Algorithmic FLOPs of one LoRA training step (x0 loss, one branch per sample): the forward
    tower, the backward's data gradients (one product per forward GEMM; four attention products:
    dV, dP, dQ, dK) and the LoRA weight gradients.  The forward that the backward recomputes per
    block is not counted."""
    d = w.dims
    M, N, D, I, r = w.batch * w.n_tokens, w.n_tokens, d.hidden, d.mlp_intermediate, d.lora_rank
    QD, KV = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    gemm = 2 * M * D * (QD + 2 * KV) + 2 * M * QD * D + 2 * M * D * 2 * I + 2 * M * I * D
    attn = sum(4 * d.n_q_heads * N * (w.prefix_len_of(b) + N) * d.head_dim for b in range(w.batch))
    ins = (D, D, D, QD, D, D, I)
    outs = (QD, KV, KV, D, I, I, D)
    lora = sum(2 * M * r * (i + o) for i, o in zip(ins, outs))
    per_layer_fwd = gemm + attn + lora
    per_layer_bwd = gemm + 2 * attn + 2 * lora
    head = 2 * M * D * 3072
    f = {"forward": per_layer_fwd * w.n_layers + 2 * w.n_img * N * 3072 * D + head,
         "backward": per_layer_bwd * w.n_layers + head}
    f["total"] = f["forward"] + f["backward"]
    return f


def run_train_bench(psf, w, args):
    """One LoRA training step of the 36-layer tower (x0 loss, 4 samples x 1024^2, rank 32 on all
    seven sites): forward, loss, backward to every layer's LoRA gradients.  Gradients are cleared
    at the start of each step; no optimizer update."""
    import torch
    import workloads as W
    d = w.dims
    dims = psf.make_dims(d, psf.GEN_BF16)
    base = W.scaled(w, dims=W.BlockDims(**{**W.dataclasses.asdict(d), "lora_rank": 0, "lora_alpha": 0.0}))
    layers_dev, glob, pk, pv, x0 = make_device_tower(psf, base, seed=4)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)

    def randn(*shape, std):
        t = torch.empty(*shape, device="cuda", dtype=torch.float32)
        t.normal_(0.0, std, generator=g)
        return t.to(torch.bfloat16)
    D, I, r = d.hidden, d.mlp_intermediate, d.lora_rank
    qd, kd = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    ins = {"q": D, "k": D, "v": D, "o": qd, "gate": D, "up": D, "down": I}
    outs = {"q": qd, "k": kd, "v": kd, "o": D, "gate": I, "up": I, "down": D}
    grads, gstructs = [], []
    for lwd in layers_dev:
        for s_ in ("q", "k", "v", "o", "gate", "up", "down"):
            lwd[f"lora_a_{s_}"] = randn(r, ins[s_], std=0.02)
            lwd[f"lora_b_{s_}"] = randn(outs[s_], r, std=0.02)
    # every layer's LoRA gradients as views of one flat buffer, cleared by one fill per step
    shapes = [[(k, v.shape) for k, v in lwd.items() if k.startswith("lora_")] for lwd in layers_dev]
    flat = torch.zeros(sum(sh.numel() for layer in shapes for _, sh in layer), device="cuda")
    off = 0
    for layer in shapes:
        gb = {}
        for k, sh in layer:
            gb[k] = flat[off:off + sh.numel()].view(sh)
            off += sh.numel()
        grads.append(gb)
        gstructs.append(psf.make_lora_grads(gb))
    layers = [psf.make_weights(l) for l in layers_dev]
    noise = torch.randn(x0.shape, device="cuda", generator=g)
    t = torch.rand(w.n_img, generator=torch.Generator().manual_seed(6))
    x_t = (1 - t.view(-1, 1, 1, 1).cuda()) * x0 + t.view(-1, 1, 1, 1).cuda() * noise
    sig = [float(v) for v in t]
    plen = [w.prefix_len] * w.batch
    loss = torch.zeros(1, device="cuda")
    ws = psf.alloc_workspace(psf.train_workspace_size(dims, w.n_layers, w.n_img, w.n_tokens, w.prefix_len))
    # the frozen base weights' transposes for the backward, made once for the run (like loading)
    ft = psf.alloc_workspace(psf.train_frozen_t_size(dims, w.n_layers))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    psf.train_frozen_t(dims, layers, ft)
    e1.record()
    torch.cuda.synchronize()
    frozen_t_ms = e0.elapsed_time(e1)

    def step():
        flat.zero_()
        psf.tower_lora_train_step(dims, layers, glob, x_t, x0, sig, pk, pv, plen, gstructs, loss, ws, frozen_t=ft)

    ms, per = time_steps(step, args.steps, args.warmup)
    gu_avg, gu_n = kernel_pass(psf, "gate_up", w.n_layers, step, max(2, min(args.steps, 5)))
    M_ = w.batch * w.n_tokens
    gu_tf = 2 * M_ * d.hidden * 2 * d.mlp_intermediate / (gu_avg * 1e-3) / 1e12
    fl = train_flops(w)
    tokens = w.batch * w.n_tokens
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    out = {
        "metric": "LoRA training step of the 36-layer gen tower (x0 loss, forward + backward to the LoRA "
                  "gradients): image tokens/s; % bf16 MFMA peak",
        "value": round(tokens / (ms * 1e-3), 1), "unit": "image tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), **step_stats(per),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "samples": w.n_img, "image_px": [w.height, w.width],
                   "image_tokens_per_sample": w.n_tokens, "prefix_tokens": w.prefix_len,
                   "lora": {"rank": r, "alpha": d.lora_alpha, "sites": "q,k,v,o,gate,up,down"},
                   "loss": float(loss.item()),
                   "frozen_transposes": {"bytes": ft.numel(), "once_ms": round(frozen_t_ms, 2)}},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "tflops": round(tflops, 1),
        "step_tflop": round(fl["total"] / 1e12, 3),
        "roofline": {"kernel": f"forward gate_up GEMM with its LoRA terms, gate and up kept for the backward "
                               f"(M={M_}, N=2x{d.mlp_intermediate}, "
                               f"K={d.hidden})",
                     "bound": "mfma", "achieved": round(gu_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": round(gu_avg, 4), "launches_timed": gu_n},
    }
    print(json.dumps(out), flush=True)


def blas_info() -> dict:
    """numpy's BLAS (vendor, version, threads) as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        b = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if b:
            p = max(b, key=lambda x: x.get("num_threads", 1))
            return {"vendor": p.get("internal_api"), "version": p.get("version"), "threads": int(p.get("num_threads", 1)),
                    "architecture": p.get("architecture")}
    except Exception:
        pass
    return {"vendor": None, "version": None, "threads": os.cpu_count() or 1}


def blas_threads() -> int:
    """Threads numpy's BLAS runs the oracle's products on."""
    return int(blas_info()["threads"])


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_info() -> dict:
    import numpy as np
    return {"cpu_model": cpu_model(), "cores_available": len(os.sched_getaffinity(0)), "numpy": np.__version__,
            "blas": blas_info()}


def time_steps(step, steps: int, warmup: int):
    """W untimed steps, then K steps between device synchronisations with one event after each
    (on the stream the library launches on): (ms per step over the whole timed region, the K
    per-step times)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, per


def step_stats(per) -> dict:
    import statistics
    return {"median_ms": round(statistics.median(per), 3), "min_ms": round(min(per), 3), "max_ms": round(max(per), 3)}


def kernel_pass(psf, family: str, launches_per_step: int, step, steps: int):
    """Average launch duration (ms) of one kernel family over `steps` more steps, each launch
    bracketed by HIP events on its stream (run after the headline timing)."""
    import torch
    psf.timing_begin(family, launches_per_step * steps)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms, n = psf.timing_end()
    return ms / max(n, 1), n


def mfma_roofline(kernel: str, flops_per_launch: float, avg_ms: float, n: int, traffic=None, alg_bytes=None) -> dict:
    tf = flops_per_launch / (avg_ms * 1e-3) / 1e12
    out = {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
           "flop_per_launch": int(flops_per_launch), "avg_launch_ms": round(avg_ms, 4), "launches_timed": n}
    if alg_bytes is not None:
        out["algorithmic_bytes"] = int(alg_bytes)
    return out


def step_roofline(flops: float, ms: float) -> dict:
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def cpu_baseline(w, seed=0):
    """The oracle (numpy fp32, as it stands) on one full-size gen block of the workload (both
    branches, all tokens), scaled to the 36-layer step; the patch embed and head are < 0.3 %
    of the work and are not in the sample."""
    import numpy as np
    import oracle as O
    import workloads as W
    threads = blas_threads()
    wts = W.layer_weights(w, 0, seed, "bf16")
    h = W.block_hidden(w, seed, "bf16")
    pk, pv = zip(*[W.prefix_kv(w, 0, s, seed, "bf16") for s in range(w.batch)])
    t0 = time.perf_counter()
    O.gen_block(h, wts, w.dims, list(pk), list(pv))
    dt = time.perf_counter() - t0
    step_s = dt * w.n_layers
    return {"value": w.batch * w.n_tokens / step_s, "unit": "image tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"one gen block of the workload ({w.batch} x {w.n_tokens} tokens, prefix "
                       f"{list(w.branch_prefix) if w.branch_prefix else w.prefix_len}) "
                       f"in numpy fp32 took {dt:.2f} s; scaled x{w.n_layers} layers"),
            **host_info()}


def run_kernel_only(psf, w, which: str, reps: int):
    """One kernel family of the step at the workload's shapes, `reps` launches (rocprofv3 counter
    runs): the gate/up + SwiGLU GEMM, the down (rows at the tower's w_down pitch) and O
    projections onto an fp32 residual, the QKV
    GEMM, the attention; "copy" is a plain 256 MiB device copy used to calibrate the byte
    counters."""
    import torch
    d = w.dims
    M, D, I = w.batch * w.n_tokens, d.hidden, d.mlp_intermediate
    bf = torch.bfloat16
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    if which in ("gate_up", "down", "o", "qkv"):
        QD = d.n_q_heads * d.head_dim
        K, N, epi, ydt = {"gate_up": (D, I, 2, bf), "down": (I, D, 3, torch.float32), "o": (QD, D, 3, torch.float32),
                          "qkv": (D, d.qkv_out, 0, bf)}[which]
        # the down projection with both operands' rows at the tower's padded pitch: the op takes
        # dense rows, so the pad columns are computed as zeros (0.5 % more FLOPs at I = 12288)
        Kp = down_pitch(K) if which == "down" else K
        x = torch.zeros(M, Kp, device="cuda", dtype=bf)
        x[:, :K] = torch.randn(M, K, device="cuda", generator=g).to(bf)
        wt = torch.zeros(2 * N if epi == 2 else N, Kp, device="cuda", dtype=bf)
        wt[:, :K] = (0.02 * torch.randn(wt.shape[0], K, device="cuda", generator=g)).to(bf)
        y = torch.zeros(M, N, device="cuda", dtype=ydt)
        for _ in range(reps):
            psf.op_linear(x, wt, y, None, epi)
    elif which == "attention":
        Hq, Hkv, hd, P, N = d.n_q_heads, d.n_kv_heads, d.head_dim, w.prefix_len, w.n_tokens
        qkv = torch.randn(M, (Hq + 2 * Hkv) * hd, device="cuda", generator=g).to(bf)
        pk = [torch.randn(P, Hkv, hd, device="cuda", generator=g).to(bf) for _ in range(w.batch)]
        pv = [torch.randn(P, Hkv, hd, device="cuda", generator=g).to(bf) for _ in range(w.batch)]
        out = torch.empty(M, Hq * hd, device="cuda", dtype=bf)
        ws = torch.empty(psf.op_workspace_size(w.batch, N, Hkv, hd, P, psf.GEN_BF16), dtype=torch.uint8, device="cuda")
        for _ in range(reps):
            psf.op_attention(qkv, w.batch, N, Hq, Hkv, hd, pk, pv, [P] * w.batch, out, ws)
    else:
        a = torch.randn(64 * 1024 * 1024, device="cuda", generator=g)    # 256 MiB
        b = torch.empty_like(a)
        for _ in range(reps):
            b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": which, "launches": reps, "workload": w.name}), flush=True)


def make_device_block(psf, w, seed=0):
    """Random-init weights, hidden state and prefixes of one gen block (dense or MoE) on the GPU."""
    import torch
    d = w.dims
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)

    def randn(*shape, std=1.0, mean=0.0):
        t = torch.empty(*shape, device="cuda", dtype=torch.float32)
        t.normal_(mean, std, generator=g)
        return t.to(torch.bfloat16)
    D = d.hidden
    QKV = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim
    lw = {"g_in": randn(D, std=0.1, mean=1.0), "w_qkv": randn(QKV, D, std=0.02),
          "g_q": randn(d.head_dim, std=0.1, mean=1.0), "g_k": randn(d.head_dim, std=0.1, mean=1.0),
          "w_o": randn(D, d.n_q_heads * d.head_dim, std=0.02), "g_post": randn(D, std=0.1, mean=1.0)}
    if d.is_moe:
        E, Ie = d.n_experts, d.expert_intermediate
        lw.update(w_router=randn(E, D, std=D ** -0.5), w_exp_gate_up=randn(E, 2 * Ie, D, std=0.02),
                  w_exp_down=randn(E, D, Ie, std=0.02))
    else:
        lw.update(w_gate_up=randn(2 * d.mlp_intermediate, D, std=0.02))
        lw["w_down"], lw["ld_down"] = down_weight(randn, D, d.mlp_intermediate, 0.02)
    shp = (w.prefix_len, d.n_kv_heads, d.head_dim)
    pk = [randn(*shp) for _ in range(w.batch)]
    pv = [randn(*shp) for _ in range(w.batch)]
    h = torch.empty(w.batch, w.n_tokens, D, device="cuda")
    h.normal_(0.0, 1.0, generator=g)
    return lw, pk, pv, h


def run_block_bench(psf, w, args):
    """gen_block_forward on one block of the workload (config 1: the Qwen3-8B block over 2 x 1024
    tokens; config 4: the A3B MoE block over 2 x 4096 tokens), in place on an fp32 residual."""
    import torch
    d = w.dims
    dims = psf.make_dims(d, psf.GEN_BF16)
    lw, pk, pv, h = make_device_block(psf, w)
    cw = psf.make_weights(lw)
    plen = [w.prefix_len] * w.batch
    ws = psf.alloc_workspace(psf.workspace_size(dims, 1, w.batch, w.n_tokens, w.prefix_len))

    def step():
        psf.block_forward(dims, cw, h, pk, pv, plen, ws)

    ms, per = time_steps(step, args.steps, args.warmup)
    fl = step_flops(W_scaled(w, n_layers=1))
    block_flop = fl["total"] - fl["embed"] - fl["head"]
    tokens = w.batch * w.n_tokens
    M = tokens
    if d.is_moe:
        fam, per_step = "expert", 2
        kflop = 2 * M * d.top_k * d.hidden * 3 * d.expert_intermediate / 2     # per launch (two launches per block)
        kname = (f"grouped expert GEMMs (gate/up + SwiGLU and down; {M} x top-{d.top_k} rows over {d.n_experts} "
                 f"experts of width {d.expert_intermediate}, D={d.hidden})")
    else:
        fam, per_step = "gate_up", 1
        kflop = 2 * M * d.hidden * 2 * d.mlp_intermediate
        kname = f"gate_up SwiGLU GEMM (M={M}, N=2x{d.mlp_intermediate}, K={d.hidden})"
    k_ms, k_n = kernel_pass(psf, fam, per_step, step, max(3, min(args.steps, 10)))
    what = ("one A3B-shaped MoE gen block (32 experts, top-8, width 768) at 2048^2 CFG"
            if d.is_moe else "one Qwen3-8B-shaped gen block at 1024^2 CFG")
    out = {
        "metric": f"image tokens/s through {what}; % bf16 MFMA peak",
        "value": round(tokens / (ms * 1e-3), 1), "unit": "image tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), **step_stats(per),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": 1, "image_px": [w.height, w.width], "image_tokens_per_branch": w.n_tokens,
                   "cfg_branches": w.n_br, "prefix_tokens": w.prefix_len, "hidden": d.hidden,
                   "heads": [d.n_q_heads, d.n_kv_heads, d.head_dim],
                   **({"experts": d.n_experts, "top_k": d.top_k, "expert_intermediate": d.expert_intermediate}
                      if d.is_moe else {"mlp_intermediate": d.mlp_intermediate})},
        "pct_bf16_peak": round(100 * block_flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "tflops": round(block_flop / (ms * 1e-3) / 1e12, 1), "block_tflop": round(block_flop / 1e12, 4),
        "roofline": mfma_roofline(kname, kflop, k_ms, k_n),
        "step_roofline": step_roofline(block_flop, ms),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W_scaled(w, n_layers=1))
    print(json.dumps(out), flush=True)


def W_scaled(w, **kw):
    import workloads as W
    return W.scaled(w, **kw)


def run_lora_tower_bench(psf, w, args):
    """The 36-layer tower forward with an unmerged rank-32 LoRA on all seven sites: 4 samples x
    1024^2 at their own timesteps, each with its own 400-token prefix taken from a 56-sample
    prefix-KV cache, no CFG, x0 out (gen_tower_step with sigma_next NULL)."""
    import torch
    d = w.dims
    dims = psf.make_dims(d, psf.GEN_BF16)
    base = W_scaled(w, dims=type(d)(**{**__import__("dataclasses").asdict(d), "lora_rank": 0, "lora_alpha": 0.0}),
                    prefix_cache_samples=0)
    layers_dev, glob, _, _, x = make_device_tower(psf, base, seed=7)
    g = torch.Generator(device="cuda")
    g.manual_seed(8)

    def randn(*shape, std):
        t = torch.empty(*shape, device="cuda", dtype=torch.float32)
        t.normal_(0.0, std, generator=g)
        return t.to(torch.bfloat16)
    D, I, r = d.hidden, d.mlp_intermediate, d.lora_rank
    qd, kd = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    ins = {"q": D, "k": D, "v": D, "o": qd, "gate": D, "up": D, "down": I}
    outs = {"q": qd, "k": kd, "v": kd, "o": D, "gate": I, "up": I, "down": D}
    for lwd in layers_dev:
        for s_ in ("q", "k", "v", "o", "gate", "up", "down"):
            lwd[f"lora_a_{s_}"] = randn(r, ins[s_], std=0.02)
            lwd[f"lora_b_{s_}"] = randn(outs[s_], r, std=1e-3)
    layers = [psf.make_weights(l) for l in layers_dev]
    # the prefix-KV cache of 56 samples (every layer), 4 distinct slots drawn for this batch
    shp = (w.prefix_len, d.n_kv_heads, d.head_dim)
    cache_k = [[randn(*shp, std=1.0) for _ in range(w.n_layers)] for _ in range(w.prefix_cache_samples)]
    cache_v = [[randn(*shp, std=1.0) for _ in range(w.n_layers)] for _ in range(w.prefix_cache_samples)]
    slots = torch.randperm(w.prefix_cache_samples, generator=torch.Generator().manual_seed(9))[:w.n_img].tolist()
    pk = [cache_k[s_][l] for l in range(w.n_layers) for s_ in slots]
    pv = [cache_v[s_][l] for l in range(w.n_layers) for s_ in slots]
    plen = [w.prefix_len] * w.batch
    sig = [float(v) for v in torch.rand(w.n_img, generator=torch.Generator().manual_seed(10))]
    ws = psf.alloc_workspace(psf.workspace_size(dims, w.n_img, 1, w.n_tokens, w.prefix_len))
    xo = torch.empty_like(x)

    def step():
        psf.tower_step(dims, layers, glob, x, 1, sig, None, 1.0, w.t_eps, pk, pv, plen, xo, ws)

    ms, per = time_steps(step, args.steps, args.warmup)
    fl = step_flops(w)
    tokens = w.batch * w.n_tokens
    kflop = 2 * tokens * 2 * I * (D + r)
    k_ms, k_n = kernel_pass(psf, "gate_up", w.n_layers, step, max(2, min(args.steps, 5)))
    cache_bytes = 2 * w.prefix_cache_samples * w.n_layers * w.prefix_len * kd * 2
    out = {
        "metric": "gen-tower image tokens/s, 36-layer forward with unmerged rank-32 LoRA at 4 x 1024^2 (x0 out, "
                  "per-sample prefixes from a 56-sample cache); % bf16 MFMA peak",
        "value": round(tokens / (ms * 1e-3), 1), "unit": "image tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), **step_stats(per),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "samples": w.n_img, "image_px": [w.height, w.width],
                   "image_tokens_per_sample": w.n_tokens, "prefix_tokens": w.prefix_len,
                   "prefix_cache": {"samples": w.prefix_cache_samples, "bytes": cache_bytes},
                   "lora": {"rank": r, "alpha": d.lora_alpha, "sites": "q,k,v,o,gate,up,down", "merged": False}},
        "pct_bf16_peak": round(100 * fl["total"] / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "tflops": round(fl["total"] / (ms * 1e-3) / 1e12, 1), "step_tflop": round(fl["total"] / 1e12, 3),
        "roofline": mfma_roofline(f"gate_up SwiGLU GEMM with the gate/up LoRA terms as its K extension "
                                  f"(M={tokens}, N=2x{I}, K={D}+{r})", kflop, k_ms, k_n),
        "step_roofline": step_roofline(fl["total"], ms),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", choices=("cfg", "block", "moe", "lora-tower", "lora-merged-cfg1", "prefix", "dual-cfg",
                                          "lora-train"), default="cfg",
                    help="cfg: the 2048^2 two-branch CFG step (default); block: one 8B gen block at 2 x 1024 "
                         "tokens; moe: one A3B MoE block at 2 x 4096 tokens; lora-tower: the 36-layer forward "
                         "with an unmerged rank-32 LoRA, 4 x 1024^2, x0 out; lora-merged-cfg1: one branch at "
                         "1024^2 with cfg 1 and a rank-32 LoRA folded into the weights at load; prefix: the "
                         "prompt pass that writes the prefix-KV cache (2 prompts x 400 tokens, 36 layers); "
                         "dual-cfg: the 2048^2 image-edit step with three branches (cfg 4, image cfg 2); "
                         "lora-train: one LoRA training step (4 x 1024^2, rank 32, x0 loss)")
    ap.add_argument("--kernel", choices=("gate_up", "down", "o", "qkv", "attention", "copy"),
                    help="run only this kernel at the workload's shapes, --steps times (for counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the denoise step here runs on a single GPU and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import pixel_space_flow_amd as psf
    import workloads as W

    torch.cuda.set_device(0)
    if args.variant == "block":
        run_block_bench(psf, W.CONFIGS[1], args)
        return
    if args.variant == "moe":
        run_block_bench(psf, W.CONFIGS[4], args)
        return
    if args.variant == "lora-tower":
        run_lora_tower_bench(psf, W.CONFIGS[3], args)
        return
    w = W.CONFIGS[args.config] if args.variant != "dual-cfg" else W.VARIANTS["dual_cfg"]
    lora_w = None
    if args.variant == "lora-merged-cfg1":
        # the 8-step distilled-LoRA fast path: one image, one branch, cfg 1, LoRA fused at load
        lora_w = W.scaled(W.CONFIGS[3], name="qwen3-8b-tower36-1024px-cfg1-lora-merged", n_img=1, n_br=1,
                          cfg_scale=1.0, n_steps=8, prefix_cache_samples=0)
        w = W.scaled(lora_w, dims=W.BlockDims(**{**W.dataclasses.asdict(lora_w.dims), "lora_rank": 0,
                                                    "lora_alpha": 0.0}))
    assert w.unit == "tower" and not w.dims.is_moe and not w.dims.lora_rank, "bench times the dense tower step"
    if args.variant == "prefix":
        run_prefix_bench(psf, w, args)
        return
    if args.variant == "lora-train":
        run_train_bench(psf, W.scaled(W.CONFIGS[3], prefix_cache_samples=0), args)
        return
    if args.kernel:
        run_kernel_only(psf, w, args.kernel, args.steps)
        return
    dims = psf.make_dims(w.dims, psf.GEN_BF16)
    layers_dev, glob, pk, pv, x = make_device_tower(psf, w)
    merge_ms = None
    if lora_w is not None:
        merge_ms = merge_lora_at_load(psf, lora_w, layers_dev)
    layers = [psf.make_weights(l) for l in layers_dev]
    ws = psf.alloc_workspace(psf.workspace_size(dims, w.n_img, w.n_br, w.n_tokens, w.max_prefix))
    xo = torch.empty_like(x)
    sched = psf.sigma_schedule(w.n_steps, w.shift)
    plen = [w.prefix_len_of(s) for s in range(w.batch)]

    def step():
        psf.tower_step(dims, layers, glob, x, w.n_br, [sched[0]], [sched[1]], w.cfg_scale, w.t_eps, pk, pv, plen,
                       xo, ws, img_cfg_scale=w.img_cfg_scale)

    # headline: K whole steps, no per-launch events inside
    ms, per = time_steps(step, args.steps, args.warmup)
    # then the dominant kernel's launches timed in a pass of their own
    gu_avg_ms, gu_n = kernel_pass(psf, "gate_up", w.n_layers, step, max(2, min(args.steps, 5)))
    fl = step_flops(w)
    tokens = w.batch * w.n_tokens
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    d = w.dims
    gu_flops = 2 * tokens * d.hidden * 2 * d.mlp_intermediate
    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": {"cfg": "gen-tower image tokens/s per denoise step at 2048^2 CFG; % bf16 MFMA peak",
                   "lora-merged-cfg1": "gen-tower image tokens/s per denoise step at 1024^2, one branch (cfg 1), "
                                       "LoRA merged at load; % bf16 MFMA peak",
                   "dual-cfg": "gen-tower image tokens/s per denoise step at 2048^2, image edit with dual guidance "
                               "(three branches); % bf16 MFMA peak"}[args.variant],
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "image tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), **step_stats(per),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "image_px": [w.height, w.width],
                   "image_tokens_per_branch": w.n_tokens, "cfg_branches": w.n_br,
                   "prefix_tokens": w.prefix_len if not w.branch_prefix else list(w.branch_prefix),
                   "hidden": d.hidden, "heads": [d.n_q_heads, d.n_kv_heads, d.head_dim],
                   "mlp_intermediate": d.mlp_intermediate, "cfg_scale": w.cfg_scale, "shift": w.shift,
                   "t_eps": w.t_eps, "schedule_step": f"0 of {w.n_steps}", "global_batch": w.batch, "seq_len": w.n_tokens,
                   **({"img_cfg_scale": w.img_cfg_scale} if w.n_br == 3 else {})},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "tflops": round(tflops, 1),
        "step_tflop": round(fl["total"] / 1e12, 3),
        "image_tokens_per_s_per_output_image": round(w.n_tokens / (ms * 1e-3), 1),
        "roofline": mfma_roofline(f"gate_up SwiGLU GEMM (M={tokens}, N=2x{d.mlp_intermediate}, K={d.hidden})",
                                  gu_flops, gu_avg_ms, gu_n,
                                  traffic=measured_traffic() if lora_w is None else None,
                                  alg_bytes=2 * (tokens * d.hidden + 2 * d.mlp_intermediate * d.hidden
                                                 + tokens * d.mlp_intermediate)),
        "step_roofline": step_roofline(fl["total"], ms),
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    if lora_w is not None:
        out["config"]["lora"] = {"rank": lora_w.dims.lora_rank, "alpha": lora_w.dims.lora_alpha,
                                 "sites": "q,k,v,o,gate,up,down", "merge_ms_all_layers": round(merge_ms, 3)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W.scaled(w, n_layers=w.n_layers))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
