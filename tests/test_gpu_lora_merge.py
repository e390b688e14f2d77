"""Merged-LoRA fast path (an adapter such as the 8-step distilled LoRA folded into the base
weights at load): gen_block_lora_merge on the GPU against the oracle's merge at the 8B shapes
with the rank-32 adapter of the LoRA workload, the merged block (LoRA off) against the oracle
block on the merged weights, and the single-branch cfg 1 tower step with merged weights against
the oracle's unmerged LoRA tower."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import BLOCK_TOL, TOWER_COS, bf16_faithful, cosine, dev, host, log, weights_to_dev
from test_gpu_block import check, lora_case, run_gpu_block

pytestmark = pytest.mark.gpu

MATS = ("w_qkv", "w_o", "w_gate_up", "w_down")


def gpu_merge(lib, w, wts, in_place=False):
    import torch
    dims = lib.make_dims(w.dims, lib.GEN_BF16)
    wd = weights_to_dev(wts, "bf16")
    cw = lib.make_weights(wd)
    outs = {k: (wd[k] if in_place else torch.empty_like(wd[k])) for k in MATS}
    lib.block_lora_merge(dims, cw, *[outs[k] for k in MATS])
    torch.cuda.synchronize()
    return {k: host(v) for k, v in outs.items()}


def test_merged_matrices_match_the_oracle_merge(lib):
    w, wts, _, _, _ = lora_case()
    log(f"merge rank {w.dims.lora_rank}, alpha {w.dims.lora_alpha}, hidden {w.dims.hidden}")
    got = gpu_merge(lib, w, wts)
    ref = O.merge_lora({k: v.astype(np.float64) for k, v in wts.items()}, w.dims)
    for k in MATS:
        e = bf16_faithful(got[k], ref[k])
        moved = np.mean(got[k] != wts[k])
        log(f"  {k}: {e:.3f} of one bf16 rounding; {100 * moved:.1f} % of entries changed")
        assert e <= 1.0
    inplace = gpu_merge(lib, w, wts, in_place=True)
    for k in MATS:
        np.testing.assert_array_equal(inplace[k], got[k])


def test_merge_of_a_strong_adapter_moves_every_site(lib):
    # B ~ N(0, 0.05): the delta is well above the base weights' bf16 spacing at every site
    w, wts, _, _, _ = lora_case()
    strong = dict(wts)
    for s in W.LORA_SITES:
        strong[f"lora_b_{s}"] = W.maybe_bf16(W.normal(3, 0, f"strong_b_{s}", wts[f"lora_b_{s}"].shape, 0.05), "bf16")
    got = gpu_merge(lib, w, strong)
    ref = O.merge_lora({k: v.astype(np.float64) for k, v in strong.items()}, w.dims)
    for k in MATS:
        assert bf16_faithful(got[k], ref[k]) <= 1.0
        assert np.mean(got[k] != wts[k]) > 0.9


def merged_case():
    w, wts, h, pk, pv = lora_case()
    base_d = W.BlockDims(**{**W.dataclasses.asdict(w.dims), "lora_rank": 0, "lora_alpha": 0.0})
    return w, wts, h, pk, pv, base_d


def test_merged_block_matches_the_oracle_block_on_merged_weights(lib):
    """A merged model holds its weights in bf16, the base weights' type: W + (alpha/r) B A rounded
    to bf16.  The block bar therefore applies against the oracle block on the oracle's merge rounded
    to bf16; the merge's own rounding is pinned by test_merged_matrices_match_the_oracle_merge.
    The distance to the unmerged oracle block (both roundings together) is logged."""
    w, wts, h, pk, pv, base_d = merged_case()
    merged = gpu_merge(lib, w, wts)
    mw = {k: v for k, v in wts.items() if not k.startswith("lora_")}
    mw.update(merged)
    got = run_gpu_block(lib, W.scaled(w, dims=base_d), mw, h, pk, pv, "bf16")
    rows = np.sort(W.rng(3, 0, "rows").choice(w.n_tokens, 256, replace=False))
    om = O.merge_lora({k: v.astype(np.float64) for k, v in wts.items()}, w.dims)
    ow = {k: v for k, v in wts.items() if not k.startswith("lora_")}
    ow.update({k: W.round_bf16(np.asarray(om[k], np.float32)) for k in MATS})
    ref = O.gen_block(h, ow, base_d, pk, pv, rows=rows)
    unmerged = O.gen_block(h, wts, w.dims, pk, pv, rows=rows)
    e_un = float(np.max(np.abs(got[:, rows] - unmerged)) / np.sqrt(np.mean(unmerged ** 2)))
    log(f"  merged block vs the unmerged oracle block: max|err|/RMS(y) = {e_un:.3e} (logged)")
    check(got[:, rows], ref, h[:, rows], BLOCK_TOL, "merged-LoRA block vs oracle block on bf16 merged weights")


def test_merged_tower_single_branch_cfg1(lib):
    """One image at 1024^2, one branch (cfg 1: the uncond branch is skipped), 8-step schedule,
    step 0, LoRA folded in: the tower's x0 against the oracle's unmerged-LoRA tower (depth 1)."""
    import torch
    w3 = W.CONFIGS[3]
    w = W.scaled(w3, n_layers=1, n_img=1)
    base_d = W.BlockDims(**{**W.dataclasses.asdict(w.dims), "lora_rank": 0, "lora_alpha": 0.0})
    dims = lib.make_dims(base_d, lib.GEN_BF16)
    wts = W.layer_weights(w, 0, 0, "bf16")
    glob = W.tower_globals(w, 0, "bf16")
    merged = gpu_merge(lib, w, wts)
    mw = {k: v for k, v in wts.items() if not k.startswith("lora_")}
    mw.update(merged)
    wd = weights_to_dev(mw, "bf16")
    gd = weights_to_dev(glob, "bf16")
    slots = W.cache_slots(w, 0)
    pk_np, pv_np = zip(*[W.prefix_kv(w, 0, s, 0, "bf16") for s in slots])
    pk, pv = [dev(p, "bf16") for p in pk_np], [dev(p, "bf16") for p in pv_np]
    sched = O.sigma_schedule(8, w.shift)
    x = W.noise_image(w)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    xo = torch.empty_like(xd)
    x0 = torch.empty_like(xd)
    ws = lib.alloc_workspace(lib.workspace_size(dims, 1, 1, w.n_tokens, w.prefix_len))
    lib.tower_step(dims, [lib.make_weights(wd)], gd, xd, 1, [sched[0]], [sched[1]], 1.0, w.t_eps, pk, pv,
                   [w.prefix_len], xo, ws, x0_out=x0)
    torch.cuda.synchronize()
    rows = np.sort(W.rng(3, 0, "rows").choice(w.n_tokens, 256, replace=False))
    ref = O.tower_tokens(x, [sched[0]], glob, lambda l: wts, w.dims, 1, 1, [list(pk_np)], [list(pv_np)],
                         np.float32, rows=rows)
    got = O.patchify(host(x0))[:, rows]
    c = cosine(got[0], ref[0])
    log(f"  merged-LoRA cfg-1 tower x0 cosine {c:.6f}")
    assert c >= TOWER_COS
    # one branch, cfg 1: the Euler update uses this x0 alone
    np.testing.assert_allclose(host(xo)[0], O.euler_step(x[0], host(x0)[0], sched[0], sched[1], w.t_eps),
                               rtol=1e-5, atol=1e-5)
