"""gen_prefix_forward on the GPU against the oracle's prefix_block / prefix_tower: the causal
prompt pass that writes the static prefix-KV cache.  Each block is checked on the GPU's own
input (chained one-layer calls), the multi-layer call must reproduce that chain bit for bit,
and the caches it writes must drive gen_block_forward to the oracle's result."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import BLOCK_TOL, BLOCK_TOL_F32, PREFIX_TOL, dev, host, log, rel_max_err, rms, weights_to_dev

pytestmark = pytest.mark.gpu

# Block tolerance of the prompt pass (bf16): max |err| <= PREFIX_TOL = 2.5e-2 RMS(y).  The block
# has the gen block's bf16 rounding points (the normed input, q/k/v, the rotated q/k, the
# probabilities, the attention output, the normed MLP input, the SwiGLU product), but its first
# tokens attend to a handful of keys, so the rounding of v and of the attention output reaches the
# output undiluted instead of being averaged over ~1400 keys.  The rounding model of
# tests/precision_model.py at the 8B shape with 400 tokens, compared with the oracle, gives the
# error a correct bf16 pass shows; test_tolerance_derivations.py::test_prefix_tolerance checks
# that PREFIX_TOL sits above it with a margin.


def cache_err(got, ref, rotated):
    """Worst |got - ref| over its bound, for a bf16 cache.  Each stored value is rounded once
    (2^-8 |ref|); the projection output it comes from was rounded to bf16 before the QK-norm,
    which a rotation mixes over the pair (j, j + d/2): at most 2^-8 (|a| + |c|) <= 2^-8 sqrt(2) rho
    with rho the pair's norm (kept by the rotation).  The projection's bf16 input adds an error
    of standard deviation 2^-8/sqrt(3) RMS per output; 6 sigma of it is 0.014 RMS."""
    ref = np.asarray(ref, np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 0.014 * rms(ref)
    if rotated:
        half = ref.shape[-1] // 2
        rho = np.sqrt(ref ** 2 + np.roll(ref, half, axis=-1) ** 2)
        bound += 2.0 ** -8 * 1.42 * rho
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref) / bound))


def run_prefix(lib, d, layer_wts, h, dtype):
    """One gen_prefix_forward call over len(layer_wts) blocks; fp32 residual stream.
    Returns (hidden out, K[l][b], V[l][b]) as numpy.  Each cache buffer has one guard row
    past its end, filled with NaN, which must survive."""
    import torch
    B, P = h.shape[:2]
    L = len(layer_wts)
    gdt = lib.GEN_BF16 if dtype == "bf16" else lib.GEN_F32
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dims = lib.make_dims(d, gdt, lib.GEN_F32)
    wd = [weights_to_dev(w, dtype) for w in layer_wts]
    cw = [lib.make_weights(x) for x in wd]
    hd = dev(h, "f32")
    row = d.n_kv_heads * d.head_dim
    kbuf = [torch.full(((P + 1) * row,), float("nan"), dtype=tdt, device="cuda") for _ in range(L * B)]
    vbuf = [torch.full(((P + 1) * row,), float("nan"), dtype=tdt, device="cuda") for _ in range(L * B)]
    ws = lib.alloc_workspace(lib.workspace_size(dims, 1, B, P, 0))
    idx = torch.full((L, B * P, d.top_k), -1, dtype=torch.int32, device="cuda") if d.is_moe else None
    lib.prefix_forward(dims, cw, hd, kbuf, vbuf, ws, topk_out=idx)
    torch.cuda.synchronize()
    for t in kbuf + vbuf:
        assert torch.isnan(t[P * row:]).all(), "cache written past its P rows"
    shp = (P, d.n_kv_heads, d.head_dim)
    K = [[host(kbuf[l * B + b][:P * row]).reshape(shp) for b in range(B)] for l in range(L)]
    V = [[host(vbuf[l * B + b][:P * row]).reshape(shp) for b in range(B)] for l in range(L)]
    topk = None if idx is None else idx.cpu().numpy().reshape(L, B, P, d.top_k).astype(np.int64)
    return host(hd), K, V, topk


def check_routing(gidx, parts, wts, d, what, tie_tol=1e-2):
    """The GPU's expert sets equal the oracle's on every token except at near-ties of the 8th/9th
    router logit (gap below 1e-2, where both sets are correct)."""
    mism = near = 0
    worst = 0.0
    for b in range(gidx.shape[0]):
        logits = parts[b]["u_post"].astype(np.float64) @ wts["w_router"].T.astype(np.float64)
        srt = np.sort(logits, axis=1)[:, ::-1]
        gap = srt[:, d.top_k - 1] - srt[:, d.top_k]
        oidx = np.argsort(-logits, axis=1, kind="stable")[:, :d.top_k]
        for t in range(gidx.shape[1]):
            if set(gidx[b, t]) != set(oidx[t]):
                mism += 1
                worst = max(worst, float(gap[t]))
                assert gap[t] < tie_tol, f"{what}: token {t} routed differently with gap {gap[t]}"
        near += int((gap < tie_tol).sum())
    log(f"  {what}: routing {mism} tokens differ (largest oracle gap among them {worst:.2e}), "
        f"{near} near-ties (gap < {tie_tol})")


def check_layer(got, ref, h_in, dtype, what):
    out, K, V = got
    ro, rK, rV = ref
    err = rel_max_err(out, ro)
    log(f"  {what}: hidden max|err|/RMS = {err:.3e} (delta {rel_max_err(out - h_in, ro - h_in):.3e})")
    assert err <= (PREFIX_TOL if dtype == "bf16" else BLOCK_TOL_F32), what
    for b in range(len(K)):
        if dtype == "bf16":
            ek, ev = cache_err(K[b], rK[b], True), cache_err(V[b], rV[b], False)
            log(f"    b={b}: K worst/bound {ek:.3f}  V worst/bound {ev:.3f}")
            assert ek <= 1.0 and ev <= 1.0, what
        else:
            ek, ev = rel_max_err(K[b], rK[b]), rel_max_err(V[b], rV[b])
            log(f"    b={b}: K err {ek:.3e}  V err {ev:.3e}")
            assert ek <= BLOCK_TOL_F32 and ev <= BLOCK_TOL_F32, what


def chained_check(lib, d, lw, h, dtype, tag):
    """Per-block parity on the GPU's own inputs, then the whole call against the chain."""
    x = h
    chain = []
    for l, wts in enumerate(lw):
        got = run_prefix(lib, d, [wts], x, dtype)
        if d.is_moe:
            # route the oracle through the GPU's expert sets once those are shown valid
            parts = O.prefix_block(x, wts, d, return_parts=True)[3]
            check_routing(got[3][0], parts, wts, d, f"{tag} layer {l}")
            ref = O.prefix_block(x, wts, d, moe_idx=got[3][0])
        else:
            ref = O.prefix_block(x, wts, d)
        check_layer((got[0], got[1][0], got[2][0]), ref, x, dtype, f"{tag} layer {l}")
        chain.append(got)
        x = got[0]
    if len(lw) > 1:
        out, K, V, _ = run_prefix(lib, d, lw, h, dtype)
        assert np.array_equal(out, x), "multi-layer call differs from chained one-layer calls"
        for l in range(len(lw)):
            for b in range(h.shape[0]):
                assert np.array_equal(K[l][b], chain[l][1][0][b]) and np.array_equal(V[l][b], chain[l][2][0][b])
        log(f"  {tag}: {len(lw)}-layer call == chain (bitwise)")
    return chain


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("P", [32, 77])
def test_prefix_tiny_two_layers(lib, dtype, P):
    w = W.scaled(W.CONFIGS[0], prefix_len=P)
    d = W.prefix_dims(w)
    log(f"prefix tiny {dtype} P={P} B={w.batch} layers=2")
    lw = [W.prefix_layer_weights(w, l, 0, dtype) for l in range(2)]
    h = W.prompt_hidden(w, 0, dtype)
    chained_check(lib, d, lw, h, dtype, f"tiny P={P}")


def test_prefix_cache_feeds_the_gen_block(lib):
    """The cache the prompt pass writes, handed to gen_block_forward, gives the oracle's gen
    block over the oracle's cache (config 0, both CFG branches with their own prompts)."""
    import torch
    w = W.CONFIGS[0]
    d = W.prefix_dims(w)
    lw = [W.prefix_layer_weights(w, 0, 0, "bf16")]
    h = W.prompt_hidden(w, 0, "bf16")
    _, K, V, _ = run_prefix(lib, d, lw, h, "bf16")
    _, rK, rV = O.prefix_block(h, lw[0], d)
    gw = W.layer_weights(w, 0, 0, "bf16")
    gh = W.block_hidden(w, 0, "bf16")
    ref = O.gen_block(gh, gw, w.dims, list(rK), list(rV))
    dims = lib.make_dims(w.dims, lib.GEN_BF16)
    wd = weights_to_dev(gw, "bf16")
    hd = dev(gh, "f32")
    pk = [dev(k, "bf16") for k in K[0]]
    pv = [dev(v, "bf16") for v in V[0]]
    ws = lib.alloc_workspace(lib.workspace_size(dims, 1, w.batch, w.n_tokens, w.prefix_len))
    lib.block_forward(dims, lib.make_weights(wd), hd, pk, pv, [w.prefix_len] * w.batch, ws)
    torch.cuda.synchronize()
    err = rel_max_err(host(hd), ref)
    log(f"  gen block over the GPU-written cache: max|err|/RMS = {err:.3e}")
    assert err <= BLOCK_TOL


def test_prefix_qwen3_8b_block_400_tokens(lib):
    """The 8B block shape at the prompt length the cache is sized for (400 tokens, 2 prompts)."""
    w = W.CONFIGS[1]
    d = W.prefix_dims(w)
    log(f"prefix 8B block P={w.prefix_len} B={w.batch}")
    chained_check(lib, d, [W.prefix_layer_weights(w, 0, 0, "bf16")], W.prompt_hidden(w, 0, "bf16"), "bf16",
                  "8B")


def test_prefix_a3b_moe_block_400_tokens(lib):
    w = W.CONFIGS[4]
    d = W.prefix_dims(w)
    log(f"prefix A3B MoE block P={w.prefix_len} B={w.batch}")
    chained_check(lib, d, [W.prefix_layer_weights(w, 0, 0, "bf16")], W.prompt_hidden(w, 0, "bf16"), "bf16",
                  "A3B")


@pytest.mark.parametrize("P,B,Hq", [(1, 1, 8), (2, 2, 8), (129, 3, 8), (200, 2, 16), (64, 1, 4)])
def test_prefix_ragged(lib, P, B, Hq):
    """Prompt lengths around the 64-key tile and the 128/256-query workgroup tiles, a single
    token (its attention is its own value), and group sizes 2, 4 and 8."""
    d = W.small_dims(hidden=512, n_q_heads=Hq, n_kv_heads=2, head_dim=128, mlp_intermediate=704)
    w = W.scaled(W.CONFIGS[1], dims=d, prefix_len=P, n_img=B, n_br=1)
    log(f"prefix ragged P={P} B={B} Hq={Hq}")
    lw = [W.prefix_layer_weights(w, l, 5, "bf16") for l in range(2)]
    chained_check(lib, d, lw, W.prompt_hidden(w, 5, "bf16"), "bf16", f"ragged P={P}")
