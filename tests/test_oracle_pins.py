"""Pins of the CPU oracle against things other than itself: brute force on tiny
inputs, torch-CPU library routines, closed forms and invariants.  Each test
names the mistake it would catch."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W

RNG = np.random.default_rng(1234)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ----------------------------------------------------------------------------- schedule
def test_shift_fixes_endpoints_and_is_monotone():
    for shift in (0.5, 1.0, 3.0, 7.0):
        assert O.shift_sigma(0.0, shift) == 0.0
        assert O.shift_sigma(1.0, shift) == 1.0
        s = np.linspace(0, 1, 1001)
        sig = O.shift_sigma(s, shift)
        assert np.all(np.diff(sig) > 0)


def test_shift_one_is_identity():
    s = np.linspace(0, 1, 77)
    np.testing.assert_array_equal(O.shift_sigma(s, 1.0), s)


def test_shift_scales_noise_odds():
    # Independent characterisation: the shifted sigma multiplies the noise odds
    # sigma/(1-sigma) by exactly `shift`.  Catches a swapped (shift-1) term.
    s = np.linspace(0.01, 0.99, 99)
    for shift in (2.0, 3.0, 5.5):
        sig = O.shift_sigma(s, shift)
        np.testing.assert_allclose(sig / (1 - sig), shift * s / (1 - s), rtol=1e-12)


def test_shift_inverse():
    s = np.linspace(0, 1, 101)
    sig = O.shift_sigma(s, 3.0)
    np.testing.assert_allclose(sig / (3.0 - 2.0 * sig), s, atol=1e-15)


def test_schedule_grid():
    sched = O.sigma_schedule(50, 3.0)
    assert sched.shape == (51,) and sched[0] == 1.0 and sched[-1] == 0.0
    # hand-derived: s = 0.98 -> 2.94/2.96; s = 0.02 -> 0.06/1.04
    assert abs(sched[1] - 2.94 / 2.96) < 1e-15 and abs(sched[49] - 0.06 / 1.04) < 1e-15
    np.testing.assert_allclose(O.sigma_schedule(2, 3.0), [1.0, 0.75, 0.0], atol=0)
    # with shift 3 every interior sigma sits above the unshifted grid
    s = 1 - np.arange(51) / 50
    assert np.all(sched[1:-1] > s[1:-1])


# ----------------------------------------------------------------------------- rms norm
def test_rms_norm_matches_torch():
    x = rnd(5, 7, 64)
    g = 1 + rnd(64, scale=0.1)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-12)


def test_rms_norm_unit_gain_rms_and_scale_invariance():
    x = rnd(9, 128)
    eps = 1e-3
    y = O.rms_norm(x, np.ones(128), eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), (1 + eps / ms) ** -0.5, rtol=1e-12)
    np.testing.assert_allclose(O.rms_norm(1e3 * x, np.ones(128), 1e-12), O.rms_norm(x, np.ones(128), 1e-18),
                               rtol=1e-9)


# ----------------------------------------------------------------------------- rope
def test_rope_position_zero_is_identity():
    x = rnd(1, 3, 64)
    c, s = O.rope_cos_sin(np.array([0]), 64, 1e6, np.float64)
    np.testing.assert_array_equal(O.apply_rope(x, c, s), x)


def test_rope_matches_complex_rotation():
    # Independent formulation: pair (x_j, x_{j+d/2}) as the complex number
    # x_j + i x_{j+d/2}, multiplied by exp(i m omega_j), omega_j = theta^(-2j/d).
    d, theta = 16, 1e4
    pos = np.array([0, 1, 5, 400, 4495])
    x = rnd(len(pos), 2, d)
    c, s = O.rope_cos_sin(pos, d, theta, np.float64)
    y = O.apply_rope(x, c, s)
    for t, m in enumerate(pos):
        for h in range(2):
            for j in range(d // 2):
                w = theta ** (-2.0 * j / d)
                z = complex(x[t, h, j], x[t, h, j + d // 2]) * complex(math.cos(m * w), math.sin(m * w))
                assert abs(y[t, h, j] - z.real) < 1e-12 and abs(y[t, h, j + d // 2] - z.imag) < 1e-12


def test_rope_relative_position_property():
    d = 64
    q, k = rnd(1, 1, d), rnd(1, 1, d)
    def dot(m, n):
        cq, sq = O.rope_cos_sin(np.array([m]), d, 1e6, np.float64)
        ck, sk = O.rope_cos_sin(np.array([n]), d, 1e6, np.float64)
        return float(np.sum(O.apply_rope(q, cq, sq) * O.apply_rope(k, ck, sk)))
    assert abs(dot(10, 3) - dot(407, 400)) < 1e-9
    assert abs(dot(3, 10) - dot(400, 407)) < 1e-9
    # norm preservation of each rotated pair
    c, s = O.rope_cos_sin(np.array([123]), d, 1e6, np.float64)
    y = O.apply_rope(q, c, s)
    np.testing.assert_allclose(y[..., :32] ** 2 + y[..., 32:] ** 2, q[..., :32] ** 2 + q[..., 32:] ** 2, rtol=1e-12)


def test_rope_frequencies():
    # omega_0 = 1 (angle = position), ratio between neighbours theta^(-2/d)
    c, s = O.rope_cos_sin(np.array([7]), 128, 1e6, np.float64)
    assert abs(c[0, 0] - math.cos(7)) < 1e-15 and abs(s[0, 0] - math.sin(7)) < 1e-15
    ang = np.arctan2(s[0], c[0])
    c1, s1 = O.rope_cos_sin(np.array([1]), 128, 1e6, np.float64)
    w = np.arctan2(s1[0], c1[0])
    np.testing.assert_allclose(w[1:] / w[:-1], 1e6 ** (-2 / 128), rtol=1e-12)
    assert ang.shape == (64,)


# ----------------------------------------------------------------------------- attention
def brute_attention(q, k, v):
    """Per-element loops: explicit softmax weights for each (query, key)."""
    T, Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros_like(q)
    for t in range(T):
        for h in range(Hq):
            g = h // G
            sc = [sum(q[t, h, i] * k[j, g, i] for i in range(d)) / math.sqrt(d) for j in range(L)]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            for i in range(d):
                out[t, h, i] = sum(e[j] * v[j, g, i] for j in range(L)) / z
    return out


def test_attention_brute_force():
    q, k, v = rnd(3, 4, 8), rnd(5, 2, 8), rnd(5, 2, 8)
    np.testing.assert_allclose(O.attention(q, k, v), brute_attention(q, k, v), rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_gqa():
    q, k, v = rnd(17, 8, 16), rnd(23, 2, 16), rnd(23, 2, 16)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(4, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(4, dim=0)[None]
    ref = F.scaled_dot_product_attention(tq, tk, tv)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(O.attention(q, k, v), ref, rtol=1e-10, atol=1e-12)


def test_attention_invariants():
    q, k, v = rnd(4, 2, 8), rnd(6, 1, 8), rnd(6, 1, 8)
    perm = RNG.permutation(6)
    np.testing.assert_allclose(O.attention(q, k[perm], v[perm]), O.attention(q, k, v), rtol=1e-12)
    one = O.attention(q, k[:1], v[:1])
    np.testing.assert_allclose(one, np.broadcast_to(v[:1, 0][None], one.shape), rtol=1e-14)
    zero = O.attention(np.zeros_like(q), k, v)
    np.testing.assert_allclose(zero, np.broadcast_to(v[:, 0].mean(0), zero.shape), rtol=1e-12)
    # prefix/gen order: splitting the key set differently changes nothing
    np.testing.assert_allclose(O.attention(q, np.concatenate([k[3:], k[:3]]), np.concatenate([v[3:], v[:3]])),
                               O.attention(q, k, v), rtol=1e-12)


def test_attention_gqa_mapping_contiguous_groups():
    # head h must read kv head h // G: give kv heads wildly different values
    q = rnd(2, 4, 8)
    k = rnd(3, 2, 8)
    v = np.stack([np.full((3, 8), 1.0), np.full((3, 8), -5.0)], axis=1)
    o = O.attention(q, k, v)
    np.testing.assert_allclose(o[:, :2], 1.0, rtol=1e-14)
    np.testing.assert_allclose(o[:, 2:], -5.0, rtol=1e-14)


# ----------------------------------------------------------------------------- mlp / lora
def test_silu_swiglu_closed_form():
    x, y = rnd(50), rnd(50)
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14)
    np.testing.assert_allclose(O.swiglu(x, y), x / (1 + np.exp(-x)) * y, rtol=1e-14)
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_lora_zero_b_is_exact_base_and_merge_equivalence():
    x, w = rnd(7, 16), rnd(12, 16)
    a, b = rnd(4, 16), np.zeros((12, 4))
    base = O.linear(x, w)
    assert np.array_equal(base + O.lora_delta(x, a, b, 8.0, 4), base)
    b = rnd(12, 4)
    merged = O.linear(x, w + (8.0 / 4) * (b @ a))
    np.testing.assert_allclose(base + O.lora_delta(x, a, b, 8.0, 4), merged, rtol=1e-11, atol=1e-12)
    # scale is alpha / rank, not alpha or 1/rank
    np.testing.assert_allclose(O.lora_delta(x, a, b, 8.0, 4), 2.0 * (x @ a.T) @ b.T, rtol=1e-13)


# ----------------------------------------------------------------------------- router / moe
def test_router_brute_force_topk_and_weights():
    u, wr = rnd(40, 16), rnd(32, 16)
    idx, w, p = O.route_topk(u, wr, 8)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    for t in range(40):
        logits = [float(np.dot(u[t], wr[e])) for e in range(32)]
        mx = max(logits)
        ex = [math.exp(l - mx) for l in logits]
        z = sum(ex)
        pr = [e_ / z for e_ in ex]
        order = sorted(range(32), key=lambda e: (-pr[e], e))[:8]
        assert list(idx[t]) == order
        s8 = sum(pr[e] for e in order)
        np.testing.assert_allclose(w[t], [pr[e] / s8 for e in order], rtol=1e-12)
    ti = torch.topk(torch.from_numpy(p), 8, dim=1).indices.numpy()
    assert np.array_equal(np.sort(ti, 1), np.sort(idx, 1))


def test_router_ties_go_to_lower_index():
    u = np.ones((1, 4))
    wr = np.zeros((6, 4))
    wr[[1, 4]] = 1.0   # experts 1 and 4 tie on top, the other four tie below
    idx, w, _ = O.route_topk(u, wr, 3)
    assert list(idx[0]) == [1, 4, 0]


def test_moe_special_cases():
    D, E, Ie = 8, 4, 6
    u = rnd(10, D)
    wr, wgu, wd = rnd(E, D), rnd(E, 2 * Ie, D), rnd(E, D, Ie)
    # k = E: dense softmax-weighted mixture of all experts
    p = np.exp(u @ wr.T)
    p /= p.sum(1, keepdims=True)
    dense = sum(p[:, [e]] * (O.swiglu(u @ wgu[e, :Ie].T, u @ wgu[e, Ie:].T) @ wd[e].T) for e in range(E))
    np.testing.assert_allclose(O.moe_mlp(u, wr, wgu, wd, E), dense, rtol=1e-11, atol=1e-12)
    # identical experts: any top-k equals one SwiGLU
    wgu1 = np.repeat(wgu[:1], E, 0)
    wd1 = np.repeat(wd[:1], E, 0)
    one = O.swiglu(u @ wgu[0, :Ie].T, u @ wgu[0, Ie:].T) @ wd[0].T
    np.testing.assert_allclose(O.moe_mlp(u, wr, wgu1, wd1, 2), one, rtol=1e-11, atol=1e-12)


def test_moe_brute_force_per_token():
    D, E, Ie, k = 8, 6, 5, 2
    u = rnd(7, D)
    wr, wgu, wd = rnd(E, D), rnd(E, 2 * Ie, D), rnd(E, D, Ie)
    out = O.moe_mlp(u, wr, wgu, wd, k)
    idx, w, _ = O.route_topk(u, wr, k)
    for t in range(7):
        acc = np.zeros(D)
        for j in range(k):
            e = idx[t, j]
            g = wgu[e, :Ie] @ u[t]
            up = wgu[e, Ie:] @ u[t]
            acc += w[t, j] * (wd[e] @ (g / (1 + np.exp(-g)) * up))
        np.testing.assert_allclose(out[t], acc, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------- block
def torch_block(h, wts, d, pk, pv):
    """Library cross-check: the same block from torch-CPU primitives
    (rms_norm, scaled_dot_product_attention with GQA, silu)."""
    Hq, Hkv, hd = d.n_q_heads, d.n_kv_heads, d.head_dim
    t = {k: torch.from_numpy(v) for k, v in wts.items()}
    outs = []
    for b in range(h.shape[0]):
        x = torch.from_numpy(h[b])
        N = x.shape[0]
        P = pk[b].shape[0]
        u = F.rms_norm(x, (d.hidden,), t["g_in"], eps=d.rms_eps)
        qkv = u @ t["w_qkv"].T
        q, k, v = qkv.split([Hq * hd, Hkv * hd, Hkv * hd], dim=1)
        q = F.rms_norm(q.view(N, Hq, hd), (hd,), t["g_q"], eps=d.rms_eps)
        k = F.rms_norm(k.view(N, Hkv, hd), (hd,), t["g_k"], eps=d.rms_eps)
        pos = torch.arange(P, P + N, dtype=torch.float64)
        inv = d.rope_theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
        ang = torch.outer(pos, inv)
        rot = torch.polar(torch.ones_like(ang), ang)
        def rope(z):
            zc = torch.complex(z[..., :hd // 2], z[..., hd // 2:]) * rot[:, None, :]
            return torch.cat([zc.real, zc.imag], dim=-1)
        q, k = rope(q), rope(k)
        K = torch.cat([torch.from_numpy(pk[b]), k]).permute(1, 0, 2)[None]
        V = torch.cat([torch.from_numpy(pv[b]), v.view(N, Hkv, hd)]).permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], K, V, enable_gqa=True)
        o = o[0].permute(1, 0, 2).reshape(N, Hq * hd)
        x = x + o @ t["w_o"].T
        u = F.rms_norm(x, (d.hidden,), t["g_post"], eps=d.rms_eps)
        I = d.mlp_intermediate
        gu = u @ t["w_gate_up"].T
        x = x + (F.silu(gu[:, :I]) * gu[:, I:]) @ t["w_down"].T
        outs.append(x.numpy())
    return np.stack(outs)


def small_block_case(lora=False, seed=0):
    d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=96,
                     lora_rank=4 if lora else 0, lora_alpha=8.0 if lora else 0.0)
    w = W.scaled(W.CONFIGS[0], dims=d, height=96, width=64, prefix_len=5)
    wts = {k: v.astype(np.float64) for k, v in W.layer_weights(w, 0, seed, "f32").items()}
    h = W.block_hidden(w, seed, "f32").astype(np.float64)
    pk, pv = zip(*[W.prefix_kv(w, 0, b, seed, "f32") for b in range(w.batch)])
    return d, wts, h, [x.astype(np.float64) for x in pk], [x.astype(np.float64) for x in pv]


def test_block_matches_torch_composition():
    d, wts, h, pk, pv = small_block_case()
    np.testing.assert_allclose(O.gen_block(h, wts, d, pk, pv), torch_block(h, wts, d, pk, pv),
                               rtol=1e-9, atol=1e-9)


def test_block_rows_subset_matches_full():
    d, wts, h, pk, pv = small_block_case()
    full = O.gen_block(h, wts, d, pk, pv)
    rows = np.array([0, 2, 5])
    np.testing.assert_allclose(O.gen_block(h, wts, d, pk, pv, rows=rows), full[:, rows], rtol=1e-12)


def test_block_lora_zero_up_is_base_and_nonzero_changes_output():
    d, wts, h, pk, pv = small_block_case(lora=True)
    base_d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=96)
    zero = dict(wts)
    for s in W.LORA_SITES:
        zero[f"lora_b_{s}"] = np.zeros_like(wts[f"lora_b_{s}"])
    assert np.array_equal(O.gen_block(h, zero, d, pk, pv), O.gen_block(h, wts, base_d, pk, pv))
    assert not np.allclose(O.gen_block(h, wts, d, pk, pv), O.gen_block(h, wts, base_d, pk, pv), atol=1e-9)


def test_block_lora_equals_merged_weights():
    d, wts, h, pk, pv = small_block_case(lora=True)
    base_d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=96)
    s = d.lora_alpha / d.lora_rank
    m = dict(wts)
    dq = {site: s * wts[f"lora_b_{site}"] @ wts[f"lora_a_{site}"] for site in W.LORA_SITES}
    m["w_qkv"] = wts["w_qkv"] + np.concatenate([dq["q"], dq["k"], dq["v"]])
    m["w_o"] = wts["w_o"] + dq["o"]
    m["w_gate_up"] = wts["w_gate_up"] + np.concatenate([dq["gate"], dq["up"]])
    m["w_down"] = wts["w_down"] + dq["down"]
    np.testing.assert_allclose(O.gen_block(h, wts, d, pk, pv), O.gen_block(h, m, base_d, pk, pv),
                               rtol=1e-10, atol=1e-10)


def test_merge_lora_reproduces_the_unmerged_block():
    # the oracle's merge, run with LoRA off, against the unmerged LoRA block (itself pinned
    # above by the hand-written merge and by B = 0)
    d, wts, h, pk, pv = small_block_case(lora=True)
    base_d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=96)
    m = O.merge_lora(wts, d)
    assert not any(k.startswith("lora_") for k in m)
    np.testing.assert_allclose(O.gen_block(h, m, base_d, pk, pv), O.gen_block(h, wts, d, pk, pv),
                               rtol=1e-10, atol=1e-10)


def test_block_moe_all_experts_equals_dense_mixture_of_identical_experts():
    d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=0,
                     n_experts=4, top_k=2, expert_intermediate=48)
    w = W.scaled(W.CONFIGS[4], dims=d, height=64, width=64, prefix_len=3)
    wts = {k: v.astype(np.float64) for k, v in W.layer_weights(w, 0, 0, "f32").items()}
    h = W.block_hidden(w, 0, "f32").astype(np.float64)
    pk, pv = zip(*[W.prefix_kv(w, 0, b, 0, "f32") for b in range(w.batch)])
    pk, pv = [x.astype(np.float64) for x in pk], [x.astype(np.float64) for x in pv]
    same = dict(wts)
    same["w_exp_gate_up"] = np.repeat(wts["w_exp_gate_up"][:1], 4, 0)
    same["w_exp_down"] = np.repeat(wts["w_exp_down"][:1], 4, 0)
    dense_d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=48)
    dense = dict(wts)
    dense["w_gate_up"] = wts["w_exp_gate_up"][0]
    dense["w_down"] = wts["w_exp_down"][0]
    np.testing.assert_allclose(O.gen_block(h, same, d, pk, pv), O.gen_block(h, dense, dense_d, pk, pv),
                               rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------------------- prefix forward
def sdpa_gqa(q, k, v, causal):
    G = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    return F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)[0].permute(1, 0, 2).numpy()


def test_causal_attention_brute_force_and_sdpa():
    # query t is the unmasked brute force over keys 0..t
    q, k, v = rnd(6, 4, 8), rnd(6, 2, 8), rnd(6, 2, 8)
    got = O.causal_attention(q, k, v)
    for t in range(6):
        np.testing.assert_allclose(got[t:t + 1], brute_attention(q[t:t + 1], k[:t + 1], v[:t + 1]),
                                   rtol=1e-12, atol=1e-12)
    q, k, v = rnd(19, 8, 16), rnd(19, 2, 16), rnd(19, 2, 16)
    np.testing.assert_allclose(O.causal_attention(q, k, v), sdpa_gqa(q, k, v, True), rtol=1e-10, atol=1e-12)


def test_causal_attention_invariants():
    q, k, v = rnd(7, 2, 8), rnd(7, 1, 8), rnd(7, 1, 8)
    o = O.causal_attention(q, k, v)
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0, 0], o[0].shape), rtol=1e-14)   # one key seen
    np.testing.assert_allclose(o[-1:], O.attention(q[-1:], k, v), rtol=1e-12)           # all keys seen
    k2, v2 = k.copy(), v.copy()
    k2[4:], v2[4:] = 5 * rnd(3, 1, 8), 5 * rnd(3, 1, 8)
    o2 = O.causal_attention(q, k2, v2)
    assert np.array_equal(o2[:4], o[:4])          # later keys never reach earlier queries
    assert not np.allclose(o2[4:], o[4:])


def small_prefix_case(moe=False, seed=0, n_layers=1):
    if moe:
        d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=0,
                         n_experts=4, top_k=2, expert_intermediate=48)
        base = W.CONFIGS[4]
    else:
        d = W.small_dims(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_intermediate=96)
        base = W.CONFIGS[0]
    w = W.scaled(base, dims=d, prefix_len=9, n_layers=n_layers)
    lw = [{k: v.astype(np.float64) for k, v in W.prefix_layer_weights(w, l, seed, "f32").items()}
          for l in range(n_layers)]
    return d, lw, W.prompt_hidden(w, seed, "f32").astype(np.float64)


@pytest.mark.parametrize("moe", [False, True])
def test_prefix_block_token_t_is_a_gen_block_over_the_earlier_cache(moe):
    # Token t of the prompt pass sees tokens 0..t: it is the (pinned) gen block run on token t
    # alone, at position t, with the cache of tokens 0..t-1 as its prefix.  This ties the
    # causal mask, the positions and the cached K (normed, rotated) to the gen block's reading.
    d, lw, h = small_prefix_case(moe)
    out, K, V = O.prefix_block(h, lw[0], d)
    B, P = h.shape[:2]
    assert K.shape == V.shape == (B, P, d.n_kv_heads, d.head_dim)
    for t in range(P):
        g = O.gen_block(h[:, t:t + 1], lw[0], d, [K[b, :t] for b in range(B)], [V[b, :t] for b in range(B)])
        np.testing.assert_allclose(g[:, 0], out[:, t], rtol=1e-10, atol=1e-10)


def test_prefix_tower_last_token_runs_the_gen_blocks_over_its_caches():
    d, lw, h = small_prefix_case(n_layers=3)
    out, Ks, Vs = O.prefix_tower(h, lambda l: lw[l], d, 3)
    B, P = h.shape[:2]
    for t in (0, P - 1):
        x = h[:, t:t + 1]
        for l in range(3):
            x = O.gen_block(x, lw[l], d, [Ks[l][b, :t] for b in range(B)], [Vs[l][b, :t] for b in range(B)])
        np.testing.assert_allclose(x[:, 0], out[:, t], rtol=1e-10, atol=1e-10)
    assert not np.allclose(Ks[1], Ks[0])


# ----------------------------------------------------------------------------- patchify / temb
def test_patchify_bijection_and_conv2d():
    x = rnd(2, 3, 64, 96)
    tok = O.patchify(x)
    assert tok.shape == (2, 6, 3072)
    np.testing.assert_array_equal(O.unpatchify(tok, 64, 96), x)
    w = rnd(8, 3072, scale=0.02)
    conv = F.conv2d(torch.from_numpy(x), torch.from_numpy(w).view(8, 3, 32, 32), stride=32)
    ref = conv.flatten(2).transpose(1, 2).numpy()       # [n, tokens (raster), 8]
    np.testing.assert_allclose(O.linear(tok, w), ref, rtol=1e-10, atol=1e-12)


def test_timestep_features():
    f0 = O.timestep_features(0.0, 256, np.float64)
    np.testing.assert_array_equal(f0[:128], 1.0)
    np.testing.assert_array_equal(f0[128:], 0.0)
    f = O.timestep_features(0.5, 256, np.float64)
    # first frequency is 1, so the angle is 1000*sigma
    assert abs(f[0] - math.cos(500.0)) < 1e-12 and abs(f[128] - math.sin(500.0)) < 1e-12
    ang1 = np.arctan2(O.timestep_features(1e-3, 256, np.float64)[128:], O.timestep_features(1e-3, 256, np.float64)[:128])
    np.testing.assert_allclose(ang1[1:] / ang1[:-1], math.exp(-math.log(1e4) / 128), rtol=1e-9)


def _torch_temb(sigma: float, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """The timestep embedder built from torch-CPU modules in fp64: sinusoidal features of
    1000 sigma (cos half, then sin half), Linear(256 -> D, no bias), SiLU, Linear(D -> D, no bias)."""
    D, F_ = w1.shape
    half = F_ // 2
    freqs = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=torch.float64) / half)
    a = 1000.0 * sigma * freqs
    feat = torch.cat([torch.cos(a), torch.sin(a)])[None]
    l1 = torch.nn.Linear(F_, D, bias=False).double()
    l2 = torch.nn.Linear(D, D, bias=False).double()
    with torch.no_grad():
        l1.weight.copy_(torch.from_numpy(w1))
        l2.weight.copy_(torch.from_numpy(w2))
        return l2(F.silu(l1(feat)))[0].numpy()


@pytest.mark.parametrize("D", [256, 384])
def test_timestep_embed_matches_torch_modules(D):
    # catches W1 and W2 swapped, SiLU moved after W2 (or dropped), a transposed weight, a bias
    w1, w2 = rnd(D, 256, scale=0.5), rnd(D, D, scale=0.5)
    for sigma in (0.0, 0.25, 0.993243, 1.0):
        np.testing.assert_allclose(O.timestep_embed(sigma, w1, w2), _torch_temb(sigma, w1, w2), rtol=1e-10, atol=1e-12)


def test_timestep_embed_pin_catches_planted_mistakes():
    # mistakes planted in copies of the oracle's composition must fail the torch pin at D = 256,
    # where W1 [D, 256] and W2 [D, D] have the same shape and a swap would run without error
    D = 256
    w1, w2 = rnd(D, 256, scale=0.5), rnd(D, D, scale=0.5)
    feat = lambda s: O.timestep_features(s, 256, np.float64)[None]   # noqa: E731
    planted = {
        "W1/W2 swapped": lambda s: O.linear(O.silu(O.linear(feat(s), w2)), w1)[0],
        "SiLU after W2": lambda s: O.silu(O.linear(O.linear(feat(s), w1), w2))[0],
        "SiLU dropped": lambda s: O.linear(O.linear(feat(s), w1), w2)[0],
        "W1 transposed": lambda s: O.linear(O.silu(O.linear(feat(s), w1.T)), w2)[0],
    }
    for name, fn in planted.items():
        got, ref = fn(0.5), _torch_temb(0.5, w1, w2)
        assert not np.allclose(got, ref, rtol=1e-6, atol=1e-8), f"planted mistake not caught: {name}"
    np.testing.assert_allclose(O.timestep_embed(0.5, w1, w2), _torch_temb(0.5, w1, w2), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------- cfg / euler
def test_cfg_special_cases_and_linearity():
    c, u = rnd(3, 8, 8), rnd(3, 8, 8)
    assert O.cfg_mix(c, u, 1.0) is c
    assert O.cfg_mix(c, None, 4.0) is c
    np.testing.assert_array_equal(O.cfg_mix(c, u, 0.0), u)
    m2, m4 = O.cfg_mix(c, u, 2.0), O.cfg_mix(c, u, 4.0)
    np.testing.assert_allclose(m4 - m2, 2.0 * (c - u), rtol=1e-12, atol=1e-12)


def test_cfg_on_x0_equals_cfg_on_velocity():
    x, c, u = rnd(16), rnd(16), rnd(16)
    sig = 0.7
    vc, vu = (x - c) / sig, (x - u) / sig
    vg = vu + 4.0 * (vc - vu)
    np.testing.assert_allclose((x - O.cfg_mix(c, u, 4.0)) / sig, vg, rtol=1e-12, atol=1e-12)


def test_dual_cfg_reductions():
    c, i, u = rnd(3, 8, 8), rnd(3, 8, 8), rnd(3, 8, 8)
    # image guidance off: the uncond branch drops out, two-branch guidance of cond against img_cond
    np.testing.assert_allclose(O.dual_cfg_mix(c, i, u, 4.0, 1.0), i + 4.0 * (c - i), rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(O.dual_cfg_mix(c, i, u, 4.0, 1.0), O.dual_cfg_mix(c, i, None, 4.0, 2.0))
    np.testing.assert_allclose(O.dual_cfg_mix(c, i, u, 1.0, 1.0), c, rtol=1e-14, atol=1e-14)   # no guidance
    np.testing.assert_allclose(O.dual_cfg_mix(c, i, u, 0.0, 0.0), u, rtol=1e-14, atol=1e-14)
    # when cond and img_cond agree the text scale has no effect, and the result is image CFG
    np.testing.assert_allclose(O.dual_cfg_mix(i, i, u, 7.0, 2.5), u + 2.5 * (i - u), rtol=1e-13, atol=1e-13)
    # the weights on (c, i, u) sum to 1: a common shift of all branches shifts the result
    np.testing.assert_allclose(O.dual_cfg_mix(c + 2.0, i + 2.0, u + 2.0, 4.0, 2.0),
                               O.dual_cfg_mix(c, i, u, 4.0, 2.0) + 2.0, rtol=1e-12, atol=1e-12)


def test_dual_cfg_on_x0_equals_dual_cfg_on_velocity():
    x, c, i, u = rnd(3, 8, 8), rnd(3, 8, 8), rnd(3, 8, 8), rnd(3, 8, 8)
    sig = 0.6
    vc, vi, vu = ((x - z) / sig for z in (c, i, u))
    vg = vu + 2.0 * (vi - vu) + 4.0 * (vc - vi)
    np.testing.assert_allclose((x - O.dual_cfg_mix(c, i, u, 4.0, 2.0)) / sig, vg, rtol=1e-12, atol=1e-12)


def test_euler_closed_form_and_perfect_denoiser():
    x0, eps = rnd(50), rnd(50)
    for s, sn in [(1.0, 0.993243), (0.75, 0.0), (0.4, 0.1)]:
        x = (1 - s) * x0 + s * eps
        out = O.euler_step(x, x0, s, sn, 0.02)
        np.testing.assert_allclose(out, (1 - sn) * x0 + sn * eps, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out, x0 + (sn / s) * (x - x0), rtol=1e-12, atol=1e-12)
    # last step to sigma = 0 returns the prediction
    x = rnd(50)
    np.testing.assert_allclose(O.euler_step(x, x0, 0.3, 0.0, 0.02), x0, atol=1e-15)
    # t_eps clamps the denominator only below t_eps
    xs = O.euler_step(x, x0, 0.01, 0.0, 0.02)
    np.testing.assert_allclose(xs, x + (-0.01) * (x - x0) / 0.02, rtol=1e-12)


def test_noisy_sample():
    x0, eps = rnd(2, 3, 4, 4), rnd(2, 3, 4, 4)
    xt = O.noisy_sample(x0, eps, [0.0, 1.0])
    np.testing.assert_array_equal(xt[0], x0[0])
    np.testing.assert_array_equal(xt[1], eps[1])


# ----------------------------------------------------------------------------- tower
def tiny_tower(n_layers=1):
    d = W.small_dims(hidden=32, n_q_heads=2, n_kv_heads=1, head_dim=16, mlp_intermediate=48)
    w = W.scaled(W.CONFIGS[0], dims=d, height=64, width=64, prefix_len=3, n_layers=n_layers)
    glob = {k: v.astype(np.float64) for k, v in W.tower_globals(w, 0, "f32").items()}
    lw = [{k: v.astype(np.float64) for k, v in W.layer_weights(w, l, 0, "f32").items()} for l in range(n_layers)]
    pk = [[W.prefix_kv(w, l, s, 0, "f32")[0].astype(np.float64) for s in range(w.batch)] for l in range(n_layers)]
    pv = [[W.prefix_kv(w, l, s, 0, "f32")[1].astype(np.float64) for s in range(w.batch)] for l in range(n_layers)]
    x = W.noise_image(w).astype(np.float64)
    return w, d, glob, lw, pk, pv, x


def test_tower_step_composition_and_branches():
    w, d, glob, lw, pk, pv, x = tiny_tower(2)
    sched = O.sigma_schedule(2, 3.0)
    xn, x0 = O.tower_step(x, 0, sched, glob, lambda l: lw[l], d, 2, 2, pk, pv, 4.0, 0.02, np.float64)
    # recompute by hand from the parts
    tok = O.patchify(x)
    h = O.linear(tok[0], glob["w_in"]) + O.timestep_embed(1.0, glob["temb_w1"], glob["temb_w2"])
    hh = np.stack([h, h])
    for l in range(2):
        hh = O.gen_block(hh, lw[l], d, pk[l], pv[l])
    y = O.unpatchify(O.linear(O.rms_norm(hh, glob["g_final"], d.rms_eps), glob["w_out"]), 64, 64)
    np.testing.assert_allclose(x0, y, rtol=1e-12, atol=1e-12)
    g = y[1] + 4.0 * (y[0] - y[1])
    np.testing.assert_allclose(xn[0], x[0] + (0.75 - 1.0) * (x[0] - g) / 1.0, rtol=1e-12, atol=1e-12)
    # branches differ only through their prefixes
    assert not np.allclose(x0[0], x0[1])
    pk2 = [[p[0], p[0]] for p in pk]
    pv2 = [[p[0], p[0]] for p in pv]
    _, x0s = O.tower_step(x, 0, sched, glob, lambda l: lw[l], d, 2, 2, pk2, pv2, 4.0, 0.02, np.float64)
    np.testing.assert_array_equal(x0s[0], x0s[1])


def test_tower_step_three_branches_dual_cfg():
    # each branch is the one-branch tower over its own prefix (lengths differ), in the order
    # cond, img_cond, uncond, and the update is the Euler step on the dual-guided prediction
    w, d, glob, lw, _, _, x = tiny_tower(2)
    lens = (7, 5, 3)
    pk = [[W.normal(0, 0, f"dual_pk{l}{b}", (lens[b], 1, 16)) for b in range(3)] for l in range(2)]
    pv = [[W.normal(0, 0, f"dual_pv{l}{b}", (lens[b], 1, 16)) for b in range(3)] for l in range(2)]
    sched = O.sigma_schedule(2, 3.0)
    xn, x0 = O.tower_step(x, 0, sched, glob, lambda l: lw[l], d, 2, 3, pk, pv, 4.0, 0.02, np.float64,
                          img_cfg_scale=2.0)
    assert x0.shape[0] == 3
    for b in range(3):
        one = O.tower_x0(x, [1.0], glob, lambda l: lw[l], d, 2, 1, [[pk[l][b]] for l in range(2)],
                         [[pv[l][b]] for l in range(2)], np.float64)
        np.testing.assert_allclose(x0[b], one[0], rtol=1e-12, atol=1e-12)
    g = O.dual_cfg_mix(x0[0], x0[1], x0[2], 4.0, 2.0)
    np.testing.assert_allclose(xn[0], O.euler_step(x[0], g, sched[0], sched[1], 0.02), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- shapes pinned by the pages
def test_a3b_parameter_table_reproduced_by_config4_dims():
    """tests/golden/a3b_params.txt holds the A3B memory table of the
    vllm-omni recipe "SenseNova-U1" (section Memory); config 4's gen-block
    dims must reproduce its generation-path expert and attention counts."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "a3b_params.txt")
    vals = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    d = W.CONFIGS[4].dims
    layers = int(vals["layers"])
    gen_exp = d.n_experts * 3 * d.hidden * d.expert_intermediate * layers
    assert abs(gen_exp / 1e9 - vals["gen_experts_B"]) < 0.005
    attn = 2 * layers * (d.hidden * d.n_q_heads * d.head_dim + 2 * d.hidden * d.n_kv_heads * d.head_dim
                         + d.n_q_heads * d.head_dim * d.hidden)
    assert abs(attn / 1e9 - vals["attention_dual_tower_B"]) < 0.005


def test_prefix_cache_bytes_match_400_tokens_at_36_layers():
    """Setup notes: 56 samples x ~59 MB prefix-KV cache.  400 tokens x 36 layers
    x 8 KV heads x 128 x (K, V) x 2 bytes is 59.0 MB."""
    d, w = W.CONFIGS[2].dims, W.CONFIGS[2]
    b = w.prefix_len * w.n_layers * d.n_kv_heads * d.head_dim * 2 * 2
    assert abs(b / 1e6 - 59.0) < 0.05


def test_tower_tokens_rows_match_full():
    w, d, glob, lw, pk, pv, x = tiny_tower(2)
    full = O.tower_tokens(x, [0.7], glob, lambda l: lw[l], d, 2, 2, pk, pv, np.float64)
    rows = np.array([1, 3])
    sub = O.tower_tokens(x, [0.7], glob, lambda l: lw[l], d, 2, 2, pk, pv, np.float64, rows=rows)
    np.testing.assert_allclose(sub, full[:, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O.unpatchify(full, 64, 64),
                               O.tower_x0(x, [0.7], glob, lambda l: lw[l], d, 2, 2, pk, pv, np.float64), rtol=0)
