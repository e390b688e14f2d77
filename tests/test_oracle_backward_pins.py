"""Pins of the oracle's training gradients (``oracle/backward.py``) on the CPU: each step's
derivative against torch autograd in float64, and the block and tower gradients against
central finite differences of the forward oracle (which involve no derivative code at all)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W

RNG = np.random.default_rng(4321)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def t64(x, grad=False):
    return torch.tensor(x, dtype=torch.float64, requires_grad=grad)


def test_rms_norm_bwd_matches_autograd():
    x, g, dy = rnd(5, 3, 16), 1 + 0.1 * rnd(16), rnd(5, 3, 16)
    tx = t64(x, True)
    F.rms_norm(tx, (16,), t64(g), eps=1e-6).backward(t64(dy))
    np.testing.assert_allclose(O.rms_norm_bwd(x, g, 1e-6, dy), tx.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_rope_bwd_matches_autograd():
    x, dy = rnd(6, 2, 16), rnd(6, 2, 16)
    c, s = O.rope_cos_sin(np.arange(3, 9), 16, 1e6, np.float64)
    tx = t64(x, True)
    half = 8
    tc, ts = t64(c)[:, None, :], t64(s)[:, None, :]
    y = torch.cat([tx[..., :half] * tc - tx[..., half:] * ts, tx[..., half:] * tc + tx[..., :half] * ts], -1)
    y.backward(t64(dy))
    np.testing.assert_allclose(O.rope_bwd(dy, c, s), tx.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_attention_bwd_matches_autograd_gqa():
    q, k, v, do = rnd(9, 8, 16), rnd(13, 2, 16), rnd(13, 2, 16), rnd(9, 8, 16)
    tq, tk, tv = t64(q, True), t64(k, True), t64(v, True)
    o = F.scaled_dot_product_attention(tq.permute(1, 0, 2)[None], tk.permute(1, 0, 2).repeat_interleave(4, 0)[None],
                                       tv.permute(1, 0, 2).repeat_interleave(4, 0)[None])
    o[0].permute(1, 0, 2).backward(t64(do))
    dq, dk, dv = O.attention_bwd(q, k, v, do)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_swiglu_bwd_matches_autograd():
    g, u, dz = rnd(7, 12), rnd(7, 12), rnd(7, 12)
    tg, tu = t64(g, True), t64(u, True)
    (F.silu(tg) * tu).backward(t64(dz))
    dg, du = O.swiglu_bwd(g, u, dz)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(du, tu.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_lora_linear_bwd_matches_autograd():
    x, w, a, b, dy = rnd(6, 10), rnd(7, 10), rnd(3, 10), rnd(7, 3), rnd(6, 7)
    tx, ta, tb = t64(x, True), t64(a, True), t64(b, True)
    (tx @ t64(w).T + 0.75 * (tx @ ta.T) @ tb.T).backward(t64(dy))
    dx, da, db = O.lora_linear_bwd(x, w, a, b, 0.75, dy)
    for got, ref in ((dx, tx.grad), (da, ta.grad), (db, tb.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def lora_block_case(seed=0):
    d = W.small_dims(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, mlp_intermediate=40,
                     lora_rank=4, lora_alpha=8.0)
    w = W.scaled(W.CONFIGS[3], dims=d, height=96, width=64, prefix_len=5, n_img=2, n_br=1,
                 prefix_cache_samples=0)
    wts = {k: v.astype(np.float64) for k, v in W.layer_weights(w, 0, seed, "f32").items()}
    # LoRA up-projections of the size training reaches, so their gradients are not negligible
    for s in W.LORA_SITES:
        wts[f"lora_b_{s}"] = wts[f"lora_b_{s}"] * 100.0
    h = W.block_hidden(w, seed, "f32").astype(np.float64)
    pk, pv = zip(*[W.prefix_kv(w, 0, b, seed, "f32") for b in range(w.batch)])
    pk = [x.astype(np.float64) for x in pk]
    pv = [x.astype(np.float64) for x in pv]
    pv[1] = pv[1][:3]          # prefixes of different lengths
    pk[1] = pk[1][:3]
    return d, wts, h, pk, pv


def fd(f, x0, e, step=1e-5):
    return (f(x0 + step * e) - f(x0 - step * e)) / (2 * step)


def test_block_bwd_finite_differences():
    d, wts, h, pk, pv = lora_block_case()
    dy = rnd(*h.shape)
    dh, grads = O.gen_block_bwd(h, wts, d, pk, pv, dy)

    def loss_h(hh):
        return float(np.sum(dy * O.gen_block(hh, wts, d, pk, pv)))
    for _ in range(3):
        e = rnd(*h.shape)
        np.testing.assert_allclose(fd(loss_h, h, e), np.sum(dh * e), rtol=1e-7)
    assert set(grads) == {f"lora_{ab}_{s}" for s in W.LORA_SITES for ab in "ab"}
    for name, g in grads.items():
        def loss_p(p, name=name):
            ww = dict(wts)
            ww[name] = p
            return float(np.sum(dy * O.gen_block(h, ww, d, pk, pv)))
        e = rnd(*g.shape)
        np.testing.assert_allclose(fd(loss_p, wts[name], e), np.sum(g * e), rtol=1e-6, err_msg=name)


def test_block_bwd_without_lora_is_the_frozen_block():
    d, wts, h, pk, pv = lora_block_case()
    d0 = W.small_dims(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, mlp_intermediate=40)
    dy = rnd(*h.shape)
    dh, grads = O.gen_block_bwd(h, wts, d0, pk, pv, dy)
    assert grads == {}
    e = rnd(*h.shape)
    np.testing.assert_allclose(fd(lambda hh: float(np.sum(dy * O.gen_block(hh, wts, d0, pk, pv))), h, e),
                               np.sum(dh * e), rtol=1e-7)


def test_tower_lora_grads_finite_differences():
    d = W.small_dims(hidden=32, n_q_heads=2, n_kv_heads=1, head_dim=16, mlp_intermediate=48,
                     lora_rank=4, lora_alpha=4.0)
    w = W.scaled(W.CONFIGS[3], dims=d, height=64, width=64, prefix_len=3, n_layers=2, n_img=2,
                 prefix_cache_samples=0)
    glob = {k: v.astype(np.float64) for k, v in W.tower_globals(w, 0, "f32").items()}
    lw = [{k: v.astype(np.float64) for k, v in W.layer_weights(w, l, 0, "f32").items()} for l in range(2)]
    for l in range(2):
        for s in W.LORA_SITES:
            lw[l][f"lora_b_{s}"] *= 100.0
    pk = [[W.prefix_kv(w, l, s, 0, "f32")[0].astype(np.float64) for s in range(2)] for l in range(2)]
    pv = [[W.prefix_kv(w, l, s, 0, "f32")[1].astype(np.float64) for s in range(2)] for l in range(2)]
    t = np.array([0.3, 0.8])
    x0 = W.clean_image(w).astype(np.float64)
    x = O.noisy_sample(x0, W.noise_image(w).astype(np.float64), t)
    loss, grads = O.tower_lora_grads(x, t, x0, glob, lambda l: lw[l], d, 2, pk, pv, np.float64)
    pred = O.tower_x0(x, t, glob, lambda l: lw[l], d, 2, 1, pk, pv, np.float64)
    assert loss == pytest.approx(float(np.mean((pred - x0) ** 2)), rel=1e-12)
    for l, name in [(0, "lora_a_q"), (0, "lora_b_down"), (1, "lora_b_v"), (1, "lora_a_gate"), (0, "lora_b_o")]:
        def loss_p(p, l=l, name=name):
            ww = [dict(x) for x in lw]
            ww[l][name] = p
            return O.x0_loss(O.tower_x0(x, t, glob, lambda j: ww[j], d, 2, 1, pk, pv, np.float64), x0)
        e = rnd(*lw[l][name].shape)
        np.testing.assert_allclose(fd(loss_p, lw[l][name], e), np.sum(grads[l][name] * e), rtol=1e-5,
                                   err_msg=f"layer {l} {name}")
