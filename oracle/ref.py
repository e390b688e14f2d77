"""Definitions of the gen-tower denoise step, one function per step of the method.

TEST INFRASTRUCTURE ONLY (see the package docstring).  All arrays are numpy;
arithmetic follows the input dtype.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "shift_sigma", "sigma_schedule", "rms_norm", "rope_cos_sin", "apply_rope", "attention",
    "silu", "swiglu", "lora_delta", "merge_lora", "linear", "route_topk", "moe_mlp", "gen_block",
    "causal_attention", "prefix_block", "prefix_tower",
    "patchify", "unpatchify", "timestep_features", "timestep_embed", "tower_tokens", "tower_x0",
    "cfg_mix", "dual_cfg_mix", "euler_step", "tower_step", "noisy_sample",
]


# ----------------------------------------------------------------------------- schedule
def shift_sigma(s, shift: float):
    """Timestep shift: sigma = shift*s / (1 + (shift-1)*s).

    [DiffSynth] 模型推理 lists ``shift`` (default 3.0) as the timestep offset
    that changes how sigma is computed; [U1.5-recipe] Text-to-Image passes it
    as ``timestep_shift``.  The map is the standard shifted rectified-flow
    schedule: it fixes 0 and 1 and, for shift > 1, moves every interior point
    towards 1 (more of the schedule is spent at high noise)."""
    s = np.asarray(s, dtype=np.float64)
    return shift * s / (1.0 + (shift - 1.0) * s)


def sigma_schedule(n_steps: int, shift: float) -> np.ndarray:
    """n_steps+1 sigmas, float64.  Reading: a uniform grid s_k = 1 - k/n_steps on
    [1, 0], then shifted.  Step k evaluates the model at sigma_k and moves to
    sigma_{k+1}; the last step lands on sigma = 0.
    [DiffSynth] 模型推理 (num_inference_steps, default 50; shift)."""
    s = 1.0 - np.arange(n_steps + 1, dtype=np.float64) / n_steps
    return shift_sigma(s, shift)


# ----------------------------------------------------------------------------- norms / rope
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g (eps inside the
    root, Qwen3 convention).  Used before attention and MLP and, per head, as
    QK-norm ([U1-recipe] kernel table: fused RMSNorm + RoPE on q and k)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * g


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float, dtype=np.float32):
    """cos/sin tables [len(positions), head_dim/2] of 1D RoPE.

    omega_j = theta^(-2j/head_dim) for j < head_dim/2; the angle of position m
    is m*omega_j.  Both are computed in float64 and rounded to ``dtype``.
    Reading: image positions continue after the prefix (m = P + n)."""
    half = head_dim // 2
    j = np.arange(half, dtype=np.float64)
    omega = theta ** (-2.0 * j / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE (Qwen3/HF convention): element j pairs with j + d/2.
    x: [..., T, H, d]; cos, sin: [T, d/2]."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c = cos[:, None, :].astype(x.dtype)
    s = sin[:, None, :].astype(x.dtype)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ----------------------------------------------------------------------------- attention
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Grouped-query attention with a naive (two-pass) softmax and no mask.

    q [T, Hq, d]; k, v [L, Hkv, d] -> [T, Hq, d].  Query head h reads KV head
    floor(h / (Hq/Hkv)) (contiguous groups).  Scores are scaled by 1/sqrt(d).
    The keys are the static prefix cache followed by the image tokens' own
    keys ([DiffSynth] 架构说明: image tokens attend to the prefix
    past_key_values; [SETUP] static prefix-KV cache); every image token sees
    every key."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = q.dtype.type(1.0 / math.sqrt(d))
    out = np.empty_like(q)
    for h in range(Hq):
        g = h // G
        s = (q[:, h, :] @ k[:, g, :].T) * scale              # [T, L]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


# ----------------------------------------------------------------------------- MLPs
def silu(x: np.ndarray) -> np.ndarray:
    return x / (x.dtype.type(1.0) + np.exp(-x))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up ([U1-recipe] kernel table: act_and_mul)."""
    return silu(gate) * up


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T with W stored [out, in] (no bias in any projection)."""
    return x @ w.T


def lora_delta(x: np.ndarray, a: np.ndarray, b: np.ndarray, alpha: float, rank: int) -> np.ndarray:
    """Unmerged LoRA: (alpha/rank) * (x A^T) B^T, A = lora_down [r, in],
    B = lora_up [out, r] ([lilting] lora_down / lora_up / .alpha naming;
    [DiffSynth] 模型训练: targets q/k/v/o/gate/up/down of the gen tower)."""
    return x.dtype.type(alpha / rank) * ((x @ a.T) @ b.T)


def merge_lora(wts: Dict[str, np.ndarray], dims) -> Dict[str, np.ndarray]:
    """Base weights with every LoRA site folded in: W_s + (alpha/rank) B_s A_s on the site's
    rows (q, k, v rows of w_qkv; w_o; gate, up rows of w_gate_up; w_down).  The fast path of
    the 8-step distilled LoRA fuses it at load ([U1.5-recipe] 8-step distilled LoRA;
    [DiffSynth] 快速推理).  Returns a new dict without the lora_* entries."""
    s = wts["w_qkv"].dtype.type(dims.lora_alpha / dims.lora_rank)
    delta = {site: s * (wts[f"lora_b_{site}"] @ wts[f"lora_a_{site}"]) for site in ("q", "k", "v", "o", "gate", "up", "down")}
    out = {k: v for k, v in wts.items() if not k.startswith("lora_")}
    out["w_qkv"] = wts["w_qkv"] + np.concatenate([delta["q"], delta["k"], delta["v"]])
    out["w_o"] = wts["w_o"] + delta["o"]
    out["w_gate_up"] = wts["w_gate_up"] + np.concatenate([delta["gate"], delta["up"]])
    out["w_down"] = wts["w_down"] + delta["down"]
    return out


def route_topk(u: np.ndarray, w_router: np.ndarray, k: int):
    """Softmax router with top-k and renormalised weights ([U1-recipe] A3B (MoE)
    variant: gen MLP routes over 32 experts, top-8).

    logits = u W_r^T; p = softmax(logits); the top-k set is the k largest p
    with ties broken towards the lower expert index; w_j = p_j / sum_{top-k} p.
    Returns (idx [T, k] int64 in descending-p order, weights [T, k], p [T, E])."""
    logits = u @ w_router.T
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    # stable sort on -p keeps lower indices first among equal probabilities
    order = np.argsort(-p, axis=1, kind="stable")
    idx = order[:, :k]
    sel = np.take_along_axis(p, idx, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    return idx, w, p


def moe_mlp(u: np.ndarray, w_router, w_exp_gate_up, w_exp_down, k: int,
            idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Top-k expert SwiGLU mixture: sum_j w_j * SwiGLU_{e_j}(u).  Each expert's
    gate/up weight stacks gate rows above up rows ([E, 2*Ie, D]); down is
    [E, D, Ie].  ``idx`` optionally forces the expert sets (weights are still
    the renormalised router probabilities of those experts)."""
    ridx, w, p = route_topk(u, w_router, k)
    if idx is not None:
        sel = np.take_along_axis(p, idx, axis=1)
        w = sel / sel.sum(axis=1, keepdims=True)
        ridx = idx
    Ie = w_exp_down.shape[2]
    out = np.zeros_like(u)
    for e in range(w_exp_gate_up.shape[0]):
        tok, slot = np.nonzero(ridx == e)
        if tok.size == 0:
            continue
        gu = u[tok] @ w_exp_gate_up[e].T
        z = swiglu(gu[:, :Ie], gu[:, Ie:])
        y = z @ w_exp_down[e].T
        out[tok] += w[tok, slot][:, None] * y
    return out


# ----------------------------------------------------------------------------- block
def gen_block(h: np.ndarray, wts: Dict[str, np.ndarray], dims, prefix_k: Sequence[np.ndarray],
              prefix_v: Sequence[np.ndarray], rows: Optional[np.ndarray] = None,
              moe_idx: Optional[np.ndarray] = None, return_parts: bool = False):
    """One Qwen3-style gen block over a batch of image-token sequences.

    h [B, N, D]; prefix_k[b], prefix_v[b] [P_b, Hkv, d] (already normed and
    rotated, used as given).  Order ([U1-recipe] kernel table and TP=2 notes;
    [DiffSynth] 架构说明):
      u = RMSNorm(h; g_in)
      q, k, v = u W_qkv^T (+ LoRA on q, k, v before the norm)
      q, k <- RoPE(RMSNorm_head(q; g_q)), RoPE(RMSNorm_head(k; g_k)), m = P_b + n
      o = attention(q, [K_pre; k], [V_pre; v])
      h = h + o W_o^T (+ LoRA)
      u = RMSNorm(h; g_post)
      h = h + SwiGLU MLP(u) (dense, + LoRA on gate/up/down) or top-k expert MLP.
    ``rows`` restricts the outputs to those token indices (keys and values are
    still computed for every token).  Returns the new h [B, len(rows) or N, D]."""
    B, N, D = h.shape
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    eps = dims.rms_eps
    lora = dims.lora_rank > 0
    r, alpha = dims.lora_rank, dims.lora_alpha
    sel = np.arange(N) if rows is None else np.asarray(rows)
    qd, kvd = Hq * hd, Hkv * hd

    def proj(x, wname, site, lo=None, hi=None):
        w = wts[wname] if lo is None else wts[wname][lo:hi]
        y = linear(x, w)
        if lora and f"lora_a_{site}" in wts:
            y = y + lora_delta(x, wts[f"lora_a_{site}"], wts[f"lora_b_{site}"], alpha, r)
        return y

    outs, parts = [], []
    for b in range(B):
        hb = h[b]
        u = rms_norm(hb, wts["g_in"], eps)
        P = prefix_k[b].shape[0]
        q = proj(u[sel], "w_qkv", "q", 0, qd).reshape(len(sel), Hq, hd)
        k = proj(u, "w_qkv", "k", qd, qd + kvd).reshape(N, Hkv, hd)
        v = proj(u, "w_qkv", "v", qd + kvd, qd + 2 * kvd).reshape(N, Hkv, hd)
        q = rms_norm(q, wts["g_q"], eps)
        k = rms_norm(k, wts["g_k"], eps)
        cq, sq = rope_cos_sin(P + sel, hd, dims.rope_theta, h.dtype)
        ck, sk = rope_cos_sin(P + np.arange(N), hd, dims.rope_theta, h.dtype)
        q = apply_rope(q, cq, sq)
        k = apply_rope(k, ck, sk)
        K = np.concatenate([prefix_k[b].astype(h.dtype), k], axis=0)
        V = np.concatenate([prefix_v[b].astype(h.dtype), v], axis=0)
        o = attention(q, K, V).reshape(len(sel), qd)
        x = hb[sel] + proj(o, "w_o", "o")
        u2 = rms_norm(x, wts["g_post"], eps)
        if dims.is_moe:
            mi = None if moe_idx is None else moe_idx[b][sel]
            x = x + moe_mlp(u2, wts["w_router"], wts["w_exp_gate_up"], wts["w_exp_down"], dims.top_k, mi)
        else:
            I = dims.mlp_intermediate
            g = proj(u2, "w_gate_up", "gate", 0, I)
            up = proj(u2, "w_gate_up", "up", I, 2 * I)
            z = swiglu(g, up)
            x = x + proj(z, "w_down", "down")
        outs.append(x)
        if return_parts:
            parts.append({"u_post": u2})
    out = np.stack(outs)
    return (out, parts) if return_parts else out


# ----------------------------------------------------------------------------- prefix forward
def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Decoder self-attention of the prompt pass: query t sees keys 0..t only.

    q [T, Hq, d]; k, v [T, Hkv, d] -> [T, Hq, d]; GQA grouping and 1/sqrt(d) as in
    ``attention``.  The prompt is read by the understanding tower as an ordinary
    autoregressive decoder ([DiffSynth] 架构说明: the prefix pass yields the
    past_key_values the image tokens then read)."""
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    scale = q.dtype.type(1.0 / math.sqrt(d))
    seen = np.tril(np.ones((T, T), dtype=bool))             # [query, key]
    out = np.empty_like(q)
    for h in range(Hq):
        s = (q[:, h, :] @ k[:, h // G, :].T) * scale
        s = np.where(seen, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (p / p.sum(axis=1, keepdims=True)) @ v[:, h // G, :]
    return out


def prefix_block(h: np.ndarray, wts: Dict[str, np.ndarray], dims, moe_idx: Optional[np.ndarray] = None,
                 return_parts: bool = False):
    """One block of the prompt pass over h [B, P, D]: the gen block's sequence of steps
    with positions 0..P-1, no earlier cache and causal attention.  Returns
    (h_out [B, P, D], K [B, P, Hkv, d], V [B, P, Hkv, d]) where K holds the keys after
    QK-norm and RoPE: the static prefix-KV cache the gen blocks take as given
    ([SETUP] static prefix-KV cache; [DiffSynth] 架构说明).  ``moe_idx`` [B, P, k] and
    ``return_parts`` (the MLP input u_post per sequence, appended to the tuple) as in
    ``gen_block``."""
    B, P, D = h.shape
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    eps, qd, kvd = dims.rms_eps, Hq * hd, Hkv * hd
    lora, r, alpha = dims.lora_rank > 0, dims.lora_rank, dims.lora_alpha

    def proj(x, wname, site, lo=None, hi=None):
        w = wts[wname] if lo is None else wts[wname][lo:hi]
        y = linear(x, w)
        if lora and f"lora_a_{site}" in wts:
            y = y + lora_delta(x, wts[f"lora_a_{site}"], wts[f"lora_b_{site}"], alpha, r)
        return y

    c, s = rope_cos_sin(np.arange(P), hd, dims.rope_theta, h.dtype)
    outs, Ks, Vs, parts = [], [], [], []
    for b in range(B):
        u = rms_norm(h[b], wts["g_in"], eps)
        q = apply_rope(rms_norm(proj(u, "w_qkv", "q", 0, qd).reshape(P, Hq, hd), wts["g_q"], eps), c, s)
        k = apply_rope(rms_norm(proj(u, "w_qkv", "k", qd, qd + kvd).reshape(P, Hkv, hd), wts["g_k"], eps), c, s)
        v = proj(u, "w_qkv", "v", qd + kvd, qd + 2 * kvd).reshape(P, Hkv, hd)
        x = h[b] + proj(causal_attention(q, k, v).reshape(P, qd), "w_o", "o")
        u2 = rms_norm(x, wts["g_post"], eps)
        if dims.is_moe:
            mi = None if moe_idx is None else moe_idx[b]
            x = x + moe_mlp(u2, wts["w_router"], wts["w_exp_gate_up"], wts["w_exp_down"], dims.top_k, mi)
        else:
            I = dims.mlp_intermediate
            x = x + proj(swiglu(proj(u2, "w_gate_up", "gate", 0, I), proj(u2, "w_gate_up", "up", I, 2 * I)),
                         "w_down", "down")
        outs.append(x)
        Ks.append(k)
        Vs.append(v)
        parts.append({"u_post": u2})
    res = (np.stack(outs), np.stack(Ks), np.stack(Vs))
    return res + (parts,) if return_parts else res


def prefix_tower(h: np.ndarray, layer_weights, dims, n_layers: int):
    """The prompt pass through n_layers blocks: (h_out, [K_l], [V_l]) with one
    [B, P, Hkv, d] key and value cache per block ([U1-recipe] t2i pipeline: one
    prefix forward ahead of the denoise loop)."""
    Ks, Vs = [], []
    for l in range(n_layers):
        h, K, V = prefix_block(h, layer_weights(l), dims)
        Ks.append(K)
        Vs.append(V)
    return h, Ks, Vs


# ----------------------------------------------------------------------------- tower
PATCH = 32


def patchify(x: np.ndarray, patch: int = PATCH) -> np.ndarray:
    """[n, 3, H, W] -> [n, (H/p)(W/p), 3*p*p].  Tokens in raster order of patches;
    features ordered (channel, row-in-patch, column-in-patch), the flattening of
    a stride-p convolution kernel.  ([DiffSynth] 模型推理: H and W are
    multiples of 32; 架构说明: pixel-space latents (1, 3, H, W), no VAE.)"""
    n, c, H, W = x.shape
    t = x.reshape(n, c, H // patch, patch, W // patch, patch)
    t = t.transpose(0, 2, 4, 1, 3, 5)
    return t.reshape(n, (H // patch) * (W // patch), c * patch * patch)


def unpatchify(tok: np.ndarray, H: int, W: int, patch: int = PATCH) -> np.ndarray:
    """Inverse of ``patchify``: [n, N, 3*p*p] -> [n, 3, H, W]."""
    n = tok.shape[0]
    c = tok.shape[2] // (patch * patch)
    t = tok.reshape(n, H // patch, W // patch, c, patch, patch)
    t = t.transpose(0, 3, 1, 4, 2, 5)
    return t.reshape(n, c, H, W)


def timestep_features(sigma: float, dim: int = 256, dtype=np.float32) -> np.ndarray:
    """Sinusoidal timestep features of 1000*sigma: [cos(a f_j), sin(a f_j)],
    f_j = exp(-ln(1e4) j / (dim/2)), computed in float64.  Reading of the
    timestep embedder that conditions the gen tower ([lilting] default.yaml
    trains the ts/ns embedders; their form is not on the pages)."""
    half = dim // 2
    f = np.exp(-math.log(10000.0) * np.arange(half, dtype=np.float64) / half)
    a = 1000.0 * float(sigma) * f
    return np.concatenate([np.cos(a), np.sin(a)]).astype(dtype)


def timestep_embed(sigma: float, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """temb = W2 silu(W1 feat(sigma)), no biases; [D]."""
    feat = timestep_features(sigma, w1.shape[1], w1.dtype)
    return linear(silu(linear(feat[None], w1)), w2)[0]


def tower_tokens(x_t: np.ndarray, sigma: Sequence[float], glob: Dict[str, np.ndarray], layer_weights,
                 dims, n_layers: int, n_br: int, prefix_k, prefix_v, dtype=np.float32,
                 rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Gen tower forward: x0 prediction of every (image, branch) as patch tokens.

    x_t [n_img, 3, H, W]; sigma[i] per image; ``layer_weights(l)`` returns layer
    l's tensors; prefix_k[l][s], prefix_v[l][s] for sample s = i*n_br + br.
      h0 = patchify(x_t) W_in^T + temb(sigma)   (shared by both branches)
      h  = gen_block^L(h0 per branch)
      y  = RMSNorm(h; g_final) W_out^T           (x0 = unpatchify(y))
    Reading: the tower predicts clean pixels x0 ([lilting] default.yaml: x0
    loss), also at inference.  ``rows`` restricts the last block and the head
    to those token indices.  Returns [n_img*n_br, len(rows) or N, 3*32*32]."""
    n_img = x_t.shape[0]
    tok = patchify(x_t.astype(dtype))
    h0 = np.stack([linear(tok[i], glob["w_in"]) + timestep_embed(sigma[i], glob["temb_w1"], glob["temb_w2"])
                   for i in range(n_img)])
    h = np.repeat(h0, n_br, axis=0)
    if n_layers == 0 and rows is not None:
        h = h[:, rows]
    for l in range(n_layers):
        last = l == n_layers - 1
        h = gen_block(h, layer_weights(l), dims, prefix_k[l], prefix_v[l], rows=rows if last else None)
    return linear(rms_norm(h, glob["g_final"], dims.rms_eps), glob["w_out"])


def tower_x0(x_t: np.ndarray, sigma: Sequence[float], glob: Dict[str, np.ndarray], layer_weights,
             dims, n_layers: int, n_br: int, prefix_k, prefix_v, dtype=np.float32) -> np.ndarray:
    """x0 prediction in pixels: unpatchify of ``tower_tokens``; [n_img*n_br, 3, H, W]."""
    H, W = x_t.shape[2], x_t.shape[3]
    y = tower_tokens(x_t, sigma, glob, layer_weights, dims, n_layers, n_br, prefix_k, prefix_v, dtype)
    return unpatchify(y, H, W)


def cfg_mix(x0_cond: np.ndarray, x0_uncond: Optional[np.ndarray], scale: float) -> np.ndarray:
    """Classifier-free guidance on the x0 prediction, cfg_norm "none":
    x0_u + s (x0_c - x0_u); s = 1 (or no uncond branch) returns x0_c unchanged
    ([DiffSynth] 模型推理: cfg_scale default 4.0, fixed uncond text;
    快速推理: cfg 1.0 skips the negative branch).  Guiding x0 equals guiding the
    velocity, which is affine in x0 with the same x_t and sigma."""
    if x0_uncond is None or scale == 1.0:
        return x0_cond
    return x0_uncond + x0_cond.dtype.type(scale) * (x0_cond - x0_uncond)


def dual_cfg_mix(x0_cond: np.ndarray, x0_img: np.ndarray, x0_uncond: Optional[np.ndarray], cfg_scale: float,
                 img_cfg_scale: float) -> np.ndarray:
    """Image-edit guidance over three branches ([U1.5-recipe] img2img: cfg_scale steers
    toward the instruction, img_cfg_scale toward the input image, 1.0 switching image
    guidance off; the 3-way run uses cond + img_cond + uncond; [DiffSynth] 图像编辑: the
    negative branch keeps the input image and drops the instruction).  Reading: the
    pages give no formula, so the nested form is taken
        x0_u + s_img (x0_i - x0_u) + s_txt (x0_c - x0_i)
    with cond = prompt + image, img_cond = image without the instruction, uncond =
    neither.  At s_img = 1 the uncond branch drops out and this is the two-branch
    guidance of cond against img_cond, the pages' 2-way run."""
    if x0_uncond is None or img_cfg_scale == 1.0:
        return cfg_mix(x0_cond, x0_img, cfg_scale)
    t = x0_cond.dtype.type
    return x0_uncond + t(img_cfg_scale) * (x0_img - x0_uncond) + t(cfg_scale) * (x0_cond - x0_img)


def euler_step(x: np.ndarray, x0: np.ndarray, sigma: float, sigma_next: float, t_eps: float) -> np.ndarray:
    """Flow-matching Euler step from sigma to sigma_next with an x0 prediction.
    Convention x_sigma = (1 - sigma) x0 + sigma eps (sigma = 1 is pure noise), so
    the velocity is v = (x - x0)/sigma; reading: t_eps clamps its denominator,
    v = (x - x0)/max(sigma, t_eps).  x' = x + (sigma_next - sigma) v.
    ([U1-recipe] Measured: 50 Euler steps, shift 3.0, t_eps 0.02.)"""
    dt = x.dtype.type(sigma_next - sigma)
    v = (x - x0) / x.dtype.type(max(sigma, t_eps))
    return x + dt * v


def tower_step(x_t, k: int, sched: np.ndarray, glob, layer_weights, dims, n_layers, n_br,
               prefix_k, prefix_v, cfg_scale: float, t_eps: float, dtype=np.float32, img_cfg_scale: float = 1.0):
    """One denoise step k: predict x0 at sigma_k for every branch, mix with CFG (two
    branches: cond, uncond; three: cond, img_cond, uncond with ``dual_cfg_mix``), Euler to
    sigma_{k+1}.  Returns (x_next [n_img,3,H,W], x0 [n_img*n_br,3,H,W])."""
    n_img = x_t.shape[0]
    sig = [float(sched[k])] * n_img
    x0 = tower_x0(x_t, sig, glob, layer_weights, dims, n_layers, n_br, prefix_k, prefix_v, dtype)
    x0 = x0.reshape(n_img, n_br, *x0.shape[1:])
    xs = x_t.astype(dtype)
    outs = []
    for i in range(n_img):
        if n_br == 3:
            g = dual_cfg_mix(x0[i, 0], x0[i, 1], x0[i, 2], cfg_scale, img_cfg_scale)
        else:
            g = cfg_mix(x0[i, 0], x0[i, 1] if n_br == 2 else None, cfg_scale)
        outs.append(euler_step(xs[i], g, float(sched[k]), float(sched[k + 1]), t_eps))
    return np.stack(outs), x0.reshape(n_img * n_br, *x0.shape[2:])


def noisy_sample(x0: np.ndarray, eps: np.ndarray, t) -> np.ndarray:
    """Training input x_t = (1 - t) x0 + t eps per sample (uniform timestep,
    [lilting] default.yaml)."""
    t = np.asarray(t, dtype=np.float64).reshape(-1, *([1] * (x0.ndim - 1)))
    return ((1.0 - t) * x0 + t * eps).astype(x0.dtype)
