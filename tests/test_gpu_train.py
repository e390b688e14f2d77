"""LoRA training backward on the GPU against the oracle's gradients (``oracle/backward.py``):
gen_block_backward per block (dh and the LoRA gradients of all seven sites, with and without
LoRA, ragged token counts and prefixes of different lengths, and at the 8B LoRA block shape),
and gen_tower_lora_train_step end to end (loss and every layer's LoRA gradients)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import DH_TOL, cosine, dev, host, log, rel_max_err, rms, weights_to_dev

pytestmark = pytest.mark.gpu

# Gradients through a bf16 block: the oracle runs in fp32 on the same bf16-rounded inputs.  The
# backward rounds about twice as many operands to bf16 as the forward (the saved activations, then
# dy, dz, dgate/dup, du2, the residual gradient, dO, P and dS in the attention products, dqkv,
# du).  The bar for dh is DH_TOL = 4e-2 RMS; the rounding model of tests/precision_model.py at the
# 8B LoRA block shape gives the error a correct bf16 backward shows, and
# test_tolerance_derivations.py::test_backward_dh_tolerance checks that DH_TOL sits above it with a
# margin.  A LoRA weight gradient is a sum over every token, so it is checked by cosine >= 0.999
# and max |err| <= 3e-2 max |ref|.
G_COS = 0.999
G_TOL = 3e-2


def small_dims(rank=8):
    return W.small_dims(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128, mlp_intermediate=512,
                        lora_rank=rank, lora_alpha=2.0 * rank if rank else 0.0)


def strong_lora(wts, factor=100.0):
    """LoRA up-projections of the size training reaches (the seeded ones start near zero)."""
    out = dict(wts)
    for s in W.LORA_SITES:
        if f"lora_b_{s}" in out:
            out[f"lora_b_{s}"] = W.round_bf16(out[f"lora_b_{s}"] * factor)
    return out


def grad_buffers(lib, wts):
    import torch
    g = {k: torch.zeros(v.shape, dtype=torch.float32, device="cuda") for k, v in wts.items() if k.startswith("lora_")}
    return g, lib.make_lora_grads(g)


def check_grads(got: dict, ref: dict, what: str):
    assert set(ref) <= set(got)
    for k in sorted(ref):
        g, r = host(got[k]), ref[k]
        c = cosine(g, r)
        e = float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-30))
        log(f"    {what} {k}: cos {c:.6f}, max|err|/max|ref| {e:.3e}")
        assert c >= G_COS and e <= G_TOL, (what, k)


def run_block_bwd(lib, d, wts, h, pk, pv, dy):
    import torch
    dims = lib.make_dims(d, lib.GEN_BF16)
    wd = weights_to_dev(wts, "bf16")
    cw = lib.make_weights(wd)
    plen = [p.shape[0] for p in pk]
    pkd = [dev(p, "bf16") if p.size else None for p in pk]
    pvd = [dev(p, "bf16") if p.size else None for p in pv]
    hd = dev(h, "f32")
    dyd = dev(dy, "f32")
    ws = lib.alloc_workspace(lib.backward_workspace_size(dims, h.shape[0], h.shape[1], max(plen)))
    gt, gc = grad_buffers(lib, wts) if d.lora_rank else ({}, None)
    lib.block_backward(dims, cw, hd, dyd, pkd, pvd, plen, gc, ws)
    torch.cuda.synchronize()
    return host(dyd), gt


@pytest.mark.parametrize("rank", [8, 0])
def test_block_backward_small_ragged(lib, rank):
    d = small_dims(rank)
    w = W.scaled(W.CONFIGS[3], dims=d, height=32 * 7, width=32 * 11, prefix_len=40, n_img=2, n_br=1,
                 prefix_cache_samples=0)
    wts = strong_lora(W.layer_weights(w, 0, 1, "bf16")) if rank else W.layer_weights(w, 0, 1, "bf16")
    h = W.block_hidden(w, 1, "bf16")
    pk, pv = zip(*[W.prefix_kv(w, 0, b, 1, "bf16") for b in range(2)])
    pk, pv = [pk[0], pk[1][:0]], [pv[0], pv[1][:0]]            # prefixes of 40 and 0 tokens
    dy = W.normal(3, 1, "dy", h.shape)
    log(f"block backward rank {rank}: B=2 N={w.n_tokens} prefixes 40/0")
    got, gt = run_block_bwd(lib, d, wts, h, pk, pv, dy)
    ref, rg = O.gen_block_bwd(h, wts, d, pk, pv, dy)
    e, c = rel_max_err(got, ref), cosine(got, ref)
    log(f"  dh: max|err|/RMS {e:.3e}, cos {c:.6f}")
    assert e <= DH_TOL
    if rank:
        check_grads(gt, rg, "small")


@pytest.mark.parametrize("heads", [(4, 4), (8, 1), (6, 2)])
def test_block_backward_group_sizes(lib, heads):
    """GQA group sizes 1, 8 and 3 (the attention backward puts 1, 4 or 1 query heads of a kv head
    in one workgroup), ragged token count, prefixes of 40 and 0 tokens."""
    hq, hkv = heads
    d = W.small_dims(hidden=256, n_q_heads=hq, n_kv_heads=hkv, head_dim=128, mlp_intermediate=512,
                     lora_rank=8, lora_alpha=16.0)
    w = W.scaled(W.CONFIGS[3], dims=d, height=32 * 7, width=32 * 11, prefix_len=40, n_img=2, n_br=1,
                 prefix_cache_samples=0)
    wts = strong_lora(W.layer_weights(w, 0, 2, "bf16"))
    h = W.block_hidden(w, 2, "bf16")
    pk, pv = zip(*[W.prefix_kv(w, 0, b, 2, "bf16") for b in range(2)])
    pk, pv = [pk[0], pk[1][:0]], [pv[0], pv[1][:0]]
    dy = W.normal(3, 2, "dy", h.shape)
    log(f"block backward Hq={hq} Hkv={hkv}: B=2 N={w.n_tokens} prefixes 40/0")
    got, gt = run_block_bwd(lib, d, wts, h, pk, pv, dy)
    ref, rg = O.gen_block_bwd(h, wts, d, pk, pv, dy)
    e, c = rel_max_err(got, ref), cosine(got, ref)
    log(f"  dh: max|err|/RMS {e:.3e}, cos {c:.6f}")
    assert e <= DH_TOL
    check_grads(gt, rg, f"Hq {hq} Hkv {hkv}")


def test_block_backward_rank32_partial_sites(lib):
    """Rank 32 (the base GEMMs take the LoRA terms as their K extension) with adapters on q, v, o
    and up only: dh and the gradients of the four adapters."""
    d = small_dims(32)
    w = W.scaled(W.CONFIGS[3], dims=d, height=32 * 7, width=32 * 11, prefix_len=40, n_img=2, n_br=1,
                 prefix_cache_samples=0)
    full = strong_lora(W.layer_weights(w, 0, 4, "bf16"))
    wts = {k: v for k, v in full.items() if not (k.startswith("lora_") and k.split("_")[-1] in ("k", "gate", "down"))}
    h = W.block_hidden(w, 4, "bf16")
    pk, pv = zip(*[W.prefix_kv(w, 0, b, 4, "bf16") for b in range(2)])
    pk, pv = [pk[0], pk[1][:17]], [pv[0], pv[1][:17]]
    dy = W.normal(3, 4, "dy", h.shape)
    log(f"block backward rank 32, sites q v o up: B=2 N={w.n_tokens} prefixes 40/17")
    got, gt = run_block_bwd(lib, d, wts, h, pk, pv, dy)
    ref, rg = O.gen_block_bwd(h, wts, d, pk, pv, dy)
    assert sorted(rg) == sorted(k for k in wts if k.startswith("lora_"))
    e, c = rel_max_err(got, ref), cosine(got, ref)
    log(f"  dh: max|err|/RMS {e:.3e}, cos {c:.6f}")
    assert e <= DH_TOL
    check_grads(gt, rg, "rank 32 partial")


def test_block_backward_8b_lora_block(lib):
    """The 8B LoRA training block: 4 samples x 1024 tokens, 400-token prefixes, rank 32."""
    w = W.scaled(W.CONFIGS[3], n_layers=1)
    d = w.dims
    wts = strong_lora(W.layer_weights(w, 0, 0, "bf16"))
    h = W.maybe_bf16(W.normal(3, 0, "train_hidden", (w.n_img, w.n_tokens, d.hidden)), "bf16")
    slots = W.cache_slots(w, 0)
    pk, pv = zip(*[W.prefix_kv(w, 0, s, 0, "bf16") for s in slots])
    dy = W.normal(3, 0, "train_dy", h.shape, 1e-3)
    log("block backward at the 8B LoRA shape (oracle ~10 s)")
    got, gt = run_block_bwd(lib, d, wts, h, list(pk), list(pv), dy)
    ref, rg = O.gen_block_bwd(h, wts, d, list(pk), list(pv), dy)
    e, c = rel_max_err(got, ref), cosine(got, ref)
    log(f"  dh: max|err|/RMS {e:.3e}, cos {c:.6f}")
    assert e <= DH_TOL
    check_grads(gt, rg, "8B")


def test_tower_train_step(lib):
    """Two layers, two samples at 256^2 with their own prefixes and timesteps: loss and the LoRA
    gradients of both layers."""
    import torch
    d = small_dims(8)
    w = W.scaled(W.CONFIGS[3], dims=d, height=256, width=256, prefix_len=32, n_layers=2, n_img=2,
                 prefix_cache_samples=0)
    glob = W.tower_globals(w, 0, "bf16")
    lw = [strong_lora(W.layer_weights(w, l, 0, "bf16")) for l in range(2)]
    pk = [[W.prefix_kv(w, l, s, 0, "bf16")[0] for s in range(2)] for l in range(2)]
    pv = [[W.prefix_kv(w, l, s, 0, "bf16")[1] for s in range(2)] for l in range(2)]
    t = W.train_timesteps(w)
    x0 = W.clean_image(w)
    x = O.noisy_sample(x0, W.noise_image(w), t).astype(np.float32)
    sig = [float(v) for v in t]
    dims = lib.make_dims(d, lib.GEN_BF16)
    gd = weights_to_dev(glob, "bf16")
    lwd = [weights_to_dev(x_, "bf16") for x_ in lw]
    layers = [lib.make_weights(x_) for x_ in lwd]
    grads = [grad_buffers(lib, x_) for x_ in lw]
    pkd = [dev(p, "bf16") for layer in pk for p in layer]
    pvd = [dev(p, "bf16") for layer in pv for p in layer]
    loss = torch.zeros(1, device="cuda")
    pred = torch.empty(2, 3, 256, 256, device="cuda")
    ws = lib.alloc_workspace(lib.train_workspace_size(dims, 2, 2, w.n_tokens, 32))
    lib.tower_lora_train_step(dims, layers, gd, torch.from_numpy(x).cuda(), torch.from_numpy(x0).cuda(), sig, pkd, pvd,
                              [32, 32], [g[1] for g in grads], loss, ws, x0_pred_out=pred)
    torch.cuda.synchronize()
    rloss, rgrads = O.tower_lora_grads(x, sig, x0, glob, lambda l: lw[l], d, 2, pk, pv, np.float32)
    rpred = O.tower_x0(x, sig, glob, lambda l: lw[l], d, 2, 1, pk, pv, np.float32)
    log(f"  loss {loss.item():.6f} vs {rloss:.6f}; x0 cos {cosine(host(pred), rpred):.6f}")
    assert abs(loss.item() - rloss) <= 1e-3 * rloss
    for l in range(2):
        check_grads(grads[l][0], rgrads[l], f"layer {l}")


@pytest.mark.parametrize("hidden,inter", [(256, 512), (2048, 4096)])
def test_tower_train_step_frozen_t(lib, hidden, inter):
    """The frozen weights' transposes made once (gen_train_frozen_t) give the same loss and LoRA
    gradients, bit for bit, as the step that transposes them itself; at hidden 2048 / intermediate
    4096 the z and gate/up-gradient rows are padded (multiples of 8 KiB otherwise)."""
    import torch
    d = W.small_dims(hidden=hidden, n_q_heads=hidden // 128, n_kv_heads=max(1, hidden // 512), head_dim=128,
                     mlp_intermediate=inter, lora_rank=32, lora_alpha=32.0)
    w = W.scaled(W.CONFIGS[3], dims=d, height=256, width=256, prefix_len=32, n_layers=2, n_img=2,
                 prefix_cache_samples=0)
    log(f"frozen transposes: hidden {hidden}, intermediate {inter}")
    glob = W.tower_globals(w, 0, "bf16")
    lw = [strong_lora(W.layer_weights(w, l, 0, "bf16")) for l in range(2)]
    pk = [[W.prefix_kv(w, l, s, 0, "bf16")[0] for s in range(2)] for l in range(2)]
    pv = [[W.prefix_kv(w, l, s, 0, "bf16")[1] for s in range(2)] for l in range(2)]
    t = W.train_timesteps(w)
    x0 = W.clean_image(w)
    x = O.noisy_sample(x0, W.noise_image(w), t).astype(np.float32)
    sig = [float(v) for v in t]
    dims = lib.make_dims(d, lib.GEN_BF16)
    gd = weights_to_dev(glob, "bf16")
    lwd = [weights_to_dev(x_, "bf16") for x_ in lw]
    layers = [lib.make_weights(x_) for x_ in lwd]
    pkd = [dev(p, "bf16") for layer in pk for p in layer]
    pvd = [dev(p, "bf16") for layer in pv for p in layer]
    ws = lib.alloc_workspace(lib.train_workspace_size(dims, 2, 2, w.n_tokens, 32))
    ft = lib.alloc_workspace(lib.train_frozen_t_size(dims, 2))
    lib.train_frozen_t(dims, layers, ft)
    xt, x0d = torch.from_numpy(x).cuda(), torch.from_numpy(x0).cuda()
    runs = []
    for frozen in (None, ft):
        grads = [grad_buffers(lib, x_) for x_ in lw]
        loss = torch.zeros(1, device="cuda")
        lib.tower_lora_train_step(dims, layers, gd, xt, x0d, sig, pkd, pvd, [32, 32], [g[1] for g in grads], loss, ws,
                                  frozen_t=frozen)
        torch.cuda.synchronize()
        runs.append((loss.clone(), [{k: v.clone() for k, v in g[0].items()} for g in grads]))
    (l0, g0), (l1, g1) = runs
    log(f"  loss {l0.item():.6f} / {l1.item():.6f}")
    assert torch.equal(l0, l1)
    for l in range(2):
        for k in g0[l]:
            assert torch.equal(g0[l][k], g1[l][k]), (l, k)
