"""A numpy model of where the bf16 GPU path rounds, used to derive the parity tolerances.

Test infrastructure: each function follows one of the oracle's block functions (``oracle/``)
step for step, in fp32, and rounds to bf16 (round to nearest even) exactly where the HIP kernels
hold a bf16 value: GEMM outputs and operands, the normed q/k, the softmax probabilities fed to
the P.V product, the attention output, the SwiGLU product, the LoRA down-projections, and in
the backward the bf16 copies of every gradient a GEMM reads.  Everything else (accumulation,
norms, softmax statistics, the fp32 residual stream) stays fp32.  Comparing such a model with the
fp32 oracle on the same inputs gives the error a correct bf16 implementation is expected to
show, which is what the GPU tolerances are set against.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence

import numpy as np

import oracle as O
import workloads as W


def bf(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even), kept as fp32."""
    return W.round_bf16(np.asarray(x, np.float32))


POINTS = ("u", "qkv", "qk", "p", "o", "u2", "z")   # the forward's bf16 rounding points


def _attention_bf16(q, K, V, causal_offset=None, round_p=True, round_o=True):
    """Attention as the MFMA kernel computes it: q, K, V bf16; scores accumulated in fp32; the
    probabilities exp(s - rowmax) rounded to bf16 before the P.V product; the row sum taken over
    the rounded probabilities; output rounded to bf16.  causal_offset: query t sees keys
    0 .. causal_offset + t."""
    T, Hq, d = q.shape
    G = Hq // K.shape[1]
    sc = np.float32(1.0 / math.sqrt(d))
    out = np.empty((T, Hq, d), np.float32)
    mask = None
    if causal_offset is not None:
        mask = np.arange(K.shape[0])[None, :] <= (causal_offset + np.arange(T))[:, None]
    for h in range(Hq):
        s = (q[:, h] @ K[:, h // G].T) * sc
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        if round_p:
            p = bf(p)
        out[:, h] = (p @ V[:, h // G]) / p.sum(axis=1, keepdims=True)
    return bf(out) if round_o else out


def _proj(x, w, wts, site, scale, round_t=True):
    """bf16 GEMM with the LoRA up-projection joined to its fp32 accumulators: the down-projection
    t = bf16(scale x A^T) is rounded once (the skinny kernel's bf16 output); returns fp32."""
    y = x @ w.T
    if f"lora_a_{site}" in wts:
        t = np.float32(scale) * (x @ wts[f"lora_a_{site}"].T)
        t = bf(t) if round_t else t
        y = y + t @ wts[f"lora_b_{site}"].T
    return y


def gen_block_bf16(h: np.ndarray, wts: Dict[str, np.ndarray], dims, prefix_k: Sequence[np.ndarray],
                   prefix_v: Sequence[np.ndarray], residual: str = "f32", causal: bool = False,
                   exact=()):
    """Model of the bf16 block (dense), in the order of ``oracle.gen_block``.

    residual: "f32" (the residual stream kept in fp32), "bf16_out" (the block output rounded
    once, the mid-block residual fp32), "bf16_both" (mid-block residual and output rounded).
    causal: the prompt pass (no prefix, query t sees keys 0..t, positions from 0).
    exact: rounding points of POINTS left out (kept fp32), to measure what each one costs."""
    r = {pt: (lambda x: x) if pt in exact else bf for pt in POINTS}
    B, N, D = h.shape
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    eps, I = dims.rms_eps, dims.mlp_intermediate
    qd, kvd = Hq * hd, Hkv * hd
    sc = dims.lora_alpha / dims.lora_rank if dims.lora_rank else 0.0
    wq, wk, wv = wts["w_qkv"][:qd], wts["w_qkv"][qd:qd + kvd], wts["w_qkv"][qd + kvd:]
    outs = []
    for b in range(B):
        hb = h[b].astype(np.float32)
        P = 0 if causal else prefix_k[b].shape[0]
        u = r["u"](O.rms_norm(hb, wts["g_in"], eps))
        q_raw = r["qkv"](_proj(u, wq, wts, "q", sc)).reshape(N, Hq, hd)
        k_raw = r["qkv"](_proj(u, wk, wts, "k", sc)).reshape(N, Hkv, hd)
        v = r["qkv"](_proj(u, wv, wts, "v", sc)).reshape(N, Hkv, hd)
        c, s = O.rope_cos_sin(P + np.arange(N), hd, dims.rope_theta, np.float32)
        q = r["qk"](O.apply_rope(O.rms_norm(q_raw, wts["g_q"], eps), c, s))
        k = r["qk"](O.apply_rope(O.rms_norm(k_raw, wts["g_k"], eps), c, s))
        rp, ro = "p" not in exact, "o" not in exact
        if causal:
            o = _attention_bf16(q, k, v, causal_offset=0, round_p=rp, round_o=ro)
        else:
            K = np.concatenate([prefix_k[b].astype(np.float32), k])
            V = np.concatenate([prefix_v[b].astype(np.float32), v])
            o = _attention_bf16(q, K, V, round_p=rp, round_o=ro)
        x = hb + _proj(o.reshape(N, qd), wts["w_o"], wts, "o", sc)
        if residual == "bf16_both":
            x = bf(x)
        u2 = r["u2"](O.rms_norm(x, wts["g_post"], eps))
        gate = _proj(u2, wts["w_gate_up"][:I], wts, "gate", sc)
        up = _proj(u2, wts["w_gate_up"][I:], wts, "up", sc)
        z = r["z"](O.swiglu(gate, up))
        y = x + _proj(z, wts["w_down"], wts, "down", sc)
        outs.append(bf(y) if residual != "f32" else y)
    return np.stack(outs)


def gen_block_bwd_bf16(h: np.ndarray, wts: Dict[str, np.ndarray], dims, prefix_k, prefix_v, dy: np.ndarray):
    """Model of the bf16 training block's backward (dense, fp32 residual): its training forward
    keeps u, the raw and the normed q/k/v, the attention output, the mid-block residual (fp32),
    u2, gate/up and z (bf16); the backward rounds the bf16 copies of dy and of the residual
    gradient, dz, dgate/dup, du2, dO, the recomputed P and dS of the attention products, dqkv and
    du, and the LoRA dY.B products.  Returns dL/dh (fp32); the LoRA weight gradients are not
    modelled (they do not feed dh)."""
    B, N, D = h.shape
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    eps, I = dims.rms_eps, dims.mlp_intermediate
    qd, kvd = Hq * hd, Hkv * hd
    G = Hq // Hkv
    sc = np.float32(dims.lora_alpha / dims.lora_rank) if dims.lora_rank else np.float32(0)
    ws = {"q": wts["w_qkv"][:qd], "k": wts["w_qkv"][qd:qd + kvd], "v": wts["w_qkv"][qd + kvd:], "o": wts["w_o"],
          "gate": wts["w_gate_up"][:I], "up": wts["w_gate_up"][I:], "down": wts["w_down"]}

    def dgrad(dyb_cols, sites):
        """sum over the sites of dY_site W_site + bf16(scale dY_site B_site) A_site, rounded once."""
        acc = 0
        for site, g in zip(sites, dyb_cols):
            acc = acc + g @ ws[site]
            if f"lora_a_{site}" in wts:
                tp = bf(sc * (g @ wts[f"lora_b_{site}"]))
                acc = acc + tp @ wts[f"lora_a_{site}"]
        return bf(acc)

    def fwd_proj(x, site):
        return _proj(x, ws[site], wts, site, float(sc))

    out = []
    dsc = np.float32(1.0 / math.sqrt(hd))
    for b in range(B):
        hb = h[b].astype(np.float32)
        P = prefix_k[b].shape[0]
        u = bf(O.rms_norm(hb, wts["g_in"], eps))
        q_raw = bf(fwd_proj(u, "q")).reshape(N, Hq, hd)
        k_raw = bf(fwd_proj(u, "k")).reshape(N, Hkv, hd)
        v = bf(fwd_proj(u, "v")).reshape(N, Hkv, hd)
        c, s = O.rope_cos_sin(P + np.arange(N), hd, dims.rope_theta, np.float32)
        q = bf(O.apply_rope(O.rms_norm(q_raw, wts["g_q"], eps), c, s))
        k = bf(O.apply_rope(O.rms_norm(k_raw, wts["g_k"], eps), c, s))
        K = np.concatenate([prefix_k[b].astype(np.float32), k])
        V = np.concatenate([prefix_v[b].astype(np.float32), v])
        o = _attention_bf16(q, K, V)
        x = hb + fwd_proj(o.reshape(N, qd), "o")
        u2 = bf(O.rms_norm(x, wts["g_post"], eps))
        gate, up = bf(fwd_proj(u2, "gate")), bf(fwd_proj(u2, "up"))
        # backward
        dyb = bf(dy[b])
        dz = dgrad([dyb], ["down"])
        dgate, dup = O.swiglu_bwd(gate, up, dz)
        du2 = dgrad([bf(dgate), bf(dup)], ["gate", "up"])
        dxf = dy[b].astype(np.float32) + O.rms_norm_bwd(x, wts["g_post"], eps, du2)
        dO = dgrad([bf(dxf)], ["o"]).reshape(N, Hq, hd)
        Dq = np.sum(dO * o, axis=-1)                                   # [N, Hq] row dots of dO and O
        dq = np.zeros((N, Hq, hd), np.float32)
        dK = np.zeros((P + N, Hkv, hd), np.float32)
        dV = np.zeros((P + N, Hkv, hd), np.float32)
        for hh in range(Hq):
            g = hh // G
            sco = (q[:, hh] @ K[:, g].T) * dsc
            p = np.exp(sco - sco.max(axis=1, keepdims=True))
            p = p / p.sum(axis=1, keepdims=True)
            dV[:, g] += bf(p).T @ dO[:, hh]
            dp = dO[:, hh] @ V[:, g].T
            ds = bf(p * (dp - Dq[:, hh:hh + 1]))
            dq[:, hh] = (ds @ K[:, g]) * dsc
            dK[:, g] += (ds.T @ q[:, hh]) * dsc
        dq_raw = O.rms_norm_bwd(q_raw, wts["g_q"], eps, O.rope_bwd(dq, c, s))
        dk_raw = O.rms_norm_bwd(k_raw, wts["g_k"], eps, O.rope_bwd(dK[P:], c, s))
        du = dgrad([bf(dq_raw.reshape(N, qd)), bf(dk_raw.reshape(N, kvd)), bf(dV[P:].reshape(N, kvd))],
                   ["q", "k", "v"])
        out.append(dxf + O.rms_norm_bwd(hb, wts["g_in"], eps, du))
    return np.stack(out)


def rel_max_err(got, ref) -> float:
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.sqrt(np.mean(ref ** 2)))
