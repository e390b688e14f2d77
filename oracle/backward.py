"""Gradients for LoRA training of the gen tower with the x0 loss.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Each function is the
derivative of one forward step of ``ref.py``, written out from its definition in
plain numpy; the block and tower functions run the forward again and walk the
steps in reverse.

Reading ([lilting] default.yaml: x0 loss, uniform timestep, LoRA on attention and
MLP; [SETUP] LoRA training of the gen tower; [DiffSynth] 模型训练: LoRA targets
q/k/v/o/gate/up/down): the loss of a batch is the mean over every pixel of every
sample of (x0_pred - x0)^2; only the LoRA matrices A (lora_down) and B (lora_up)
receive gradients (the base weights, norm gains and embedders are frozen), so
the backward pass carries the gradient of the residual stream down the tower
and forms weight gradients for A and B alone.  Dense gen blocks only, one
branch per sample (no CFG in training).
"""
from __future__ import annotations

import math
from typing import Dict, Sequence

import numpy as np

from .ref import (apply_rope, attention, gen_block, linear, patchify, rms_norm, rope_cos_sin, silu, swiglu,
                  timestep_embed, unpatchify)

__all__ = ["rms_norm_bwd", "rope_bwd", "attention_bwd", "swiglu_bwd", "lora_linear_bwd", "gen_block_bwd",
           "x0_loss", "tower_lora_grads"]

SITES = ("q", "k", "v", "o", "gate", "up", "down")


def rms_norm_bwd(x: np.ndarray, g: np.ndarray, eps: float, dy: np.ndarray) -> np.ndarray:
    """d/dx of y = x r g with r = (mean(x^2) + eps)^(-1/2) over the last axis of length D:
    dx = r (g dy) - x r^3 sum(g dy x) / D."""
    D = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + x.dtype.type(eps))
    gd = g * dy
    return r * gd - x * (r ** 3) * np.sum(gd * x, axis=-1, keepdims=True) / x.dtype.type(D)


def rope_bwd(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """The rotation is orthogonal: its transpose rotates by the opposite angle."""
    return apply_rope(dy, cos, -sin)


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray):
    """Gradients of ``attention`` (no mask, scale 1/sqrt(d), GQA groups h // G):
    P = softmax(q k^T / sqrt(d)), o = P v;
    dv = P^T do, dP = do v^T, dS = P (dP - rowsum(P dP)), dq = dS k / sqrt(d),
    dk = dS^T q / sqrt(d); a kv head sums the contributions of its group's heads."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = q.dtype.type(1.0 / math.sqrt(d))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(Hq):
        g = h // G
        s = (q[:, h] @ k[:, g].T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        dv[:, g] += p.T @ do[:, h]
        dp = do[:, h] @ v[:, g].T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dq[:, h] = (ds @ k[:, g]) * scale
        dk[:, g] += (ds.T @ q[:, h]) * scale
    return dq, dk, dv


def swiglu_bwd(gate: np.ndarray, up: np.ndarray, dz: np.ndarray):
    """z = silu(gate) up: d up = dz silu(gate); d gate = dz up silu'(gate) with
    silu'(x) = s + x s (1 - s), s = sigmoid(x)."""
    one = gate.dtype.type(1.0)
    s = one / (one + np.exp(-gate))
    return dz * up * (s + gate * s * (one - s)), dz * silu(gate)


def lora_linear_bwd(x, w, a, b, scale, dy):
    """y = x W^T + scale (x A^T) B^T.  Returns (dx, dA, dB):
    dx = dy W + scale (dy B) A, dA = scale (dy B)^T x, dB = scale dy^T (x A^T).
    a, b may be None (no LoRA on this site): then only dx = dy W."""
    dx = dy @ w
    if a is None:
        return dx, None, None
    t = dy @ b
    dx = dx + scale * (t @ a)
    return dx, scale * (t.T @ x), scale * (dy.T @ (x @ a.T))


def gen_block_bwd(h: np.ndarray, wts: Dict[str, np.ndarray], dims, prefix_k: Sequence[np.ndarray],
                  prefix_v: Sequence[np.ndarray], dy: np.ndarray):
    """Backward of ``ref.gen_block`` (dense) for B sequences: h [B, N, D] the block input,
    dy [B, N, D] the gradient of the loss with respect to the block output.  The prefix cache is
    a constant.  Returns (dh [B, N, D], grads) with grads["lora_a_<site>"], ["lora_b_<site>"]
    summed over the sequences (empty when the block has no LoRA)."""
    B, N, D = h.shape
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    eps, I = dims.rms_eps, dims.mlp_intermediate
    qd, kvd = Hq * hd, Hkv * hd
    lora = dims.lora_rank > 0
    sc = dims.lora_alpha / dims.lora_rank if lora else 0.0
    rows = {"q": (0, qd), "k": (qd, qd + kvd), "v": (qd + kvd, qd + 2 * kvd)}
    grads = {}

    def lw(site):
        if lora and f"lora_a_{site}" in wts:
            return wts[f"lora_a_{site}"], wts[f"lora_b_{site}"]
        return None, None

    def proj(x, w, site):
        a, b = lw(site)
        y = linear(x, w)
        return y if a is None else y + h.dtype.type(sc) * ((x @ a.T) @ b.T)

    def back(x, w, site, g):
        a, b = lw(site)
        dx, da, db = lora_linear_bwd(x, w, a, b, h.dtype.type(sc), g)
        if da is not None:
            grads[f"lora_a_{site}"] = grads.get(f"lora_a_{site}", 0) + da
            grads[f"lora_b_{site}"] = grads.get(f"lora_b_{site}", 0) + db
        return dx

    wq = {s: wts["w_qkv"][lo:hi] for s, (lo, hi) in rows.items()}
    out = []
    for bi in range(B):
        hb = h[bi]
        P = prefix_k[bi].shape[0]
        # forward, keeping what the backward reads
        u = rms_norm(hb, wts["g_in"], eps)
        q_raw = proj(u, wq["q"], "q").reshape(N, Hq, hd)
        k_raw = proj(u, wq["k"], "k").reshape(N, Hkv, hd)
        v = proj(u, wq["v"], "v").reshape(N, Hkv, hd)
        c, s = rope_cos_sin(P + np.arange(N), hd, dims.rope_theta, h.dtype)
        q = apply_rope(rms_norm(q_raw, wts["g_q"], eps), c, s)
        k = apply_rope(rms_norm(k_raw, wts["g_k"], eps), c, s)
        K = np.concatenate([prefix_k[bi].astype(h.dtype), k])
        V = np.concatenate([prefix_v[bi].astype(h.dtype), v])
        o = attention(q, K, V).reshape(N, qd)
        x = hb + proj(o, wts["w_o"], "o")
        u2 = rms_norm(x, wts["g_post"], eps)
        gate = proj(u2, wts["w_gate_up"][:I], "gate")
        up = proj(u2, wts["w_gate_up"][I:], "up")
        z = swiglu(gate, up)
        # backward
        dx = dy[bi].copy()
        dz = back(z, wts["w_down"], "down", dx)
        dgate, dup = swiglu_bwd(gate, up, dz)
        du2 = back(u2, wts["w_gate_up"][:I], "gate", dgate) + back(u2, wts["w_gate_up"][I:], "up", dup)
        dx = dx + rms_norm_bwd(x, wts["g_post"], eps, du2)
        do = back(o, wts["w_o"], "o", dx).reshape(N, Hq, hd)
        dq, dK, dV = attention_bwd(q, K, V, do)
        dk, dv = dK[P:], dV[P:]
        dq_raw = rms_norm_bwd(q_raw, wts["g_q"], eps, rope_bwd(dq, c, s))
        dk_raw = rms_norm_bwd(k_raw, wts["g_k"], eps, rope_bwd(dk, c, s))
        du = (back(u, wq["q"], "q", dq_raw.reshape(N, qd)) + back(u, wq["k"], "k", dk_raw.reshape(N, kvd))
              + back(u, wq["v"], "v", dv.reshape(N, kvd)))
        out.append(dx + rms_norm_bwd(hb, wts["g_in"], eps, du))
    return np.stack(out), grads


def x0_loss(x0_pred: np.ndarray, x0: np.ndarray) -> float:
    """Mean over every pixel of every sample of (x0_pred - x0)^2 ([lilting] x0 loss)."""
    d = x0_pred.astype(np.float64) - x0.astype(np.float64)
    return float(np.mean(d * d))


def tower_lora_grads(x_t: np.ndarray, sigma: Sequence[float], x0: np.ndarray, glob: Dict[str, np.ndarray],
                     layer_weights, dims, n_layers: int, prefix_k, prefix_v, dtype=np.float32):
    """One training step's loss and LoRA gradients: the gen tower (one branch per sample,
    ``ref.tower_x0``) predicts x0 from x_t at sigma; loss = ``x0_loss``; the gradient runs back
    through the out head and final RMSNorm into every block.  prefix_k[l][s] as in the forward.
    Returns (loss, [grads of layer l]) with grads as ``gen_block_bwd``."""
    n, _, H, W = x_t.shape
    tok = patchify(x_t.astype(dtype))
    h = np.stack([linear(tok[i], glob["w_in"]) + timestep_embed(sigma[i], glob["temb_w1"], glob["temb_w2"])
                  for i in range(n)])
    inputs = []
    for l in range(n_layers):
        inputs.append(h)
        h = gen_block(h, layer_weights(l), dims, prefix_k[l], prefix_v[l])
    hn = rms_norm(h, glob["g_final"], dims.rms_eps)
    pred = unpatchify(linear(hn, glob["w_out"]), H, W)
    loss = x0_loss(pred, x0)
    dpred = (dtype(2.0 / pred.size) * (pred - x0.astype(dtype))).astype(dtype)
    dy = patchify(dpred) @ glob["w_out"]
    dh = rms_norm_bwd(h, glob["g_final"], dims.rms_eps, dy)
    grads = [None] * n_layers
    for l in reversed(range(n_layers)):
        dh, grads[l] = gen_block_bwd(inputs[l], layer_weights(l), dims, prefix_k[l], prefix_v[l], dh)
    return loss, grads
