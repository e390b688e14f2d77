"""Row pitch of w_down (gen_block_weights.ld_down).  A padded pitch moves the rows in memory and
changes which GEMM kernel runs the down projection (the 64-deep one instead of the 32-deep ring),
not what is computed: both issue the same v_mfma_f32_16x16x32_bf16 sequence over k.  The block
(dense and LoRA), the tower step, the LoRA merge and the training backward with w_down rows at a
pitch of I + 64 are checked bitwise against the same weights in dense rows.  The padding holds
NaN, so a read past column I would show."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import dev, host, log, weights_to_dev
from test_gpu_block import lora_case
from test_gpu_tower import GpuTower
from test_gpu_train import grad_buffers, strong_lora

pytestmark = pytest.mark.gpu


def padded_down(wd: dict, I: int) -> dict:
    """A copy of device weights whose w_down is a [D, I] view of a NaN-filled [D, I + 64] buffer."""
    import torch
    out = dict(wd)
    w = wd["w_down"]
    buf = torch.full((w.shape[0], I + 64), float("nan"), dtype=w.dtype, device=w.device)
    buf[:, :I] = w
    out["w_down"], out["ld_down"] = buf[:, :I], I + 64
    return out


def run_block(lib, w, wd, h, pk, pv):
    import torch
    dims = lib.make_dims(w.dims, lib.GEN_BF16)
    hd = dev(h, "f32")
    plen = [p.shape[0] for p in pk]
    ws = lib.alloc_workspace(lib.workspace_size(dims, 1, h.shape[0], h.shape[1], max(plen)))
    lib.block_forward(dims, lib.make_weights(wd), hd, [dev(p, "bf16") for p in pk], [dev(p, "bf16") for p in pv],
                      plen, ws)
    torch.cuda.synchronize()
    return host(hd)


def test_padded_down_pitch_block(lib):
    """The 8B block over 2 x 1024 tokens, prefix 400 (I = 12288)."""
    w = W.CONFIGS[1]
    wts = W.layer_weights(w, 0, 0, "bf16")
    h = W.block_hidden(w, 0, "bf16")
    pk, pv = zip(*[W.prefix_kv(w, 0, s, 0, "bf16") for s in range(w.batch)])
    wd = weights_to_dev(wts, "bf16")
    a = run_block(lib, w, wd, h, pk, pv)
    b = run_block(lib, w, padded_down(wd, w.dims.mlp_intermediate), h, pk, pv)
    log(f"  dense vs padded w_down rows: max|diff| {np.max(np.abs(a - b))}")
    assert np.isfinite(b).all() and np.array_equal(a, b)


def test_padded_down_pitch_lora_block(lib):
    """The rank-32 LoRA block over 4 x 1024 tokens: the down site's up-projection rides on the
    down GEMM as its K extension."""
    w, wts, h, pk, pv = lora_case()
    wd = weights_to_dev(wts, "bf16")
    a = run_block(lib, w, wd, h, pk, pv)
    b = run_block(lib, w, padded_down(wd, w.dims.mlp_intermediate), h, pk, pv)
    log(f"  LoRA block, dense vs padded w_down rows: max|diff| {np.max(np.abs(a - b))}")
    assert np.isfinite(b).all() and np.array_equal(a, b)


def test_padded_down_pitch_tower_step(lib):
    """The 2048^2 CFG tower step at depth 1."""
    w = W.scaled(W.CONFIGS[2], n_layers=1)
    import oracle as O
    sched = O.sigma_schedule(w.n_steps, w.shift)
    x = W.noise_image(w)
    t = GpuTower(lib, w, "bf16")
    xa, x0a = t.step(x, [sched[0]], [sched[1]], w.cfg_scale)
    padded = [padded_down(dv, w.dims.mlp_intermediate) for dv in t.layers_dev]   # keeps the buffers alive
    t.layers = [lib.make_weights(dv) for dv in padded]
    xb, x0b = t.step(x, [sched[0]], [sched[1]], w.cfg_scale)
    assert np.isfinite(xb).all() and np.array_equal(xa, xb) and np.array_equal(x0a, x0b)


def test_padded_down_pitch_lora_merge(lib):
    """The merged w_down is written at the input's pitch, the padding left alone."""
    import torch
    w, wts, _, _, _ = lora_case()
    I = w.dims.mlp_intermediate
    dims = lib.make_dims(w.dims, lib.GEN_BF16)
    outs = {}
    for name, wd in (("dense", weights_to_dev(wts, "bf16")), ("padded", padded_down(weights_to_dev(wts, "bf16"), I))):
        o = {k: torch.empty_like(wd[k]) for k in ("w_qkv", "w_o", "w_gate_up")}
        if name == "padded":
            buf = torch.full((wd["w_down"].shape[0], I + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
            buf[:, I:] = 7.0
            o["w_down"], pad = buf[:, :I], buf[:, I:]
        else:
            o["w_down"] = torch.empty_like(wd["w_down"])
        lib.block_lora_merge(dims, lib.make_weights(wd), o["w_qkv"], o["w_o"], o["w_gate_up"], o["w_down"])
        torch.cuda.synchronize()
        outs[name] = {k: host(v) for k, v in o.items()}
    for k in outs["dense"]:
        assert np.array_equal(outs["dense"][k], outs["padded"][k]), k
    assert bool((pad == 7.0).all())


def test_padded_down_pitch_backward(lib):
    """The 8B LoRA training block's backward (1 x 1024 tokens, prefix from the cache): dL/dh and
    every LoRA gradient."""
    import torch
    w = W.scaled(W.CONFIGS[3], n_layers=1, n_img=1)
    d = w.dims
    wts = strong_lora(W.layer_weights(w, 0, 0, "bf16"))
    h = W.maybe_bf16(W.normal(3, 0, "train_hidden", (w.n_img, w.n_tokens, d.hidden)), "bf16")
    pk, pv = zip(*[W.prefix_kv(w, 0, s, 0, "bf16") for s in W.cache_slots(w, 0)])
    dy = W.normal(3, 0, "train_dy", h.shape, 1e-3)
    dims = lib.make_dims(d, lib.GEN_BF16)
    plen = [p.shape[0] for p in pk]
    res = []
    for pad in (False, True):
        wd = weights_to_dev(wts, "bf16")
        if pad:
            wd = padded_down(wd, d.mlp_intermediate)
        hd, dyd = dev(h, "f32"), dev(dy, "f32")
        ws = lib.alloc_workspace(lib.backward_workspace_size(dims, h.shape[0], h.shape[1], max(plen)))
        gt, gc = grad_buffers(lib, wts)
        lib.block_backward(dims, lib.make_weights(wd), hd, dyd, [dev(p, "bf16") for p in pk],
                           [dev(p, "bf16") for p in pv], plen, gc, ws)
        torch.cuda.synchronize()
        res.append((host(dyd), {k: host(v) for k, v in gt.items()}))
    (da, ga), (db, gb) = res
    assert np.isfinite(db).all() and np.array_equal(da, db)
    for k in ga:
        assert np.array_equal(ga[k], gb[k]), k
