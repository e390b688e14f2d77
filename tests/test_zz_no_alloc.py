"""gen_block_forward_noalloc (the entry point for callers that cannot allocate) against
gen_block_forward on the same inputs: two calls in a row, the second smaller, each bitwise equal
to the workspace entry point (same kernels, same arithmetic), and a call whose workspace exceeds
the library's scratch rejected before anything runs."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import block_inputs, dev, host, log, weights_to_dev

pytestmark = pytest.mark.gpu


def run_both(lib, w, wts, h, pk, pv):
    import torch
    d = w.dims
    dims = lib.make_dims(d, lib.GEN_BF16)
    cw = lib.make_weights(wd := weights_to_dev(wts, "bf16"))
    plen = [p.shape[0] for p in pk]
    pkd = [dev(p, "bf16") for p in pk]
    pvd = [dev(p, "bf16") for p in pv]
    need = lib.workspace_size(dims, 1, h.shape[0], h.shape[1], max(plen))
    assert need <= lib.NOALLOC_SCRATCH_BYTES
    ha, hb = dev(h, "f32"), dev(h, "f32")
    ws = lib.alloc_workspace(need)
    lib.block_forward(dims, cw, ha, pkd, pvd, plen, ws)
    lib.block_forward_noalloc(dims, cw, hb, pkd, pvd, plen)
    torch.cuda.synchronize()
    del wd
    return host(ha), host(hb), need


def test_noalloc_matches_workspace_entry_point_two_calls(lib):
    # first call: the 8B block over 2 x 256 tokens with 400-token prefixes
    w1 = W.scaled(W.CONFIGS[1], height=512, width=512)
    wts, h, pk, pv = block_inputs(w1, 0, 0, "bf16")
    a, b, need = run_both(lib, w1, wts, h, pk, pv)
    log(f"  8B block 2 x 256 tokens: scratch {need / 2**20:.1f} MiB, max|diff| {np.max(np.abs(a - b))}")
    assert np.array_equal(a, b)
    # second call, smaller: config 0's block over one sequence of 40 tokens with a 17-token prefix
    w0 = W.CONFIGS[0]
    wts0, h0, pk0, pv0 = block_inputs(w0, 1, 0, "bf16")
    h0, pk0, pv0 = h0[:1, :40], [pk0[0][:17]], [pv0[0][:17]]
    a, b, need = run_both(lib, w0, wts0, h0, pk0, pv0)
    log(f"  config 0 block 1 x 40 tokens: scratch {need / 2**20:.2f} MiB, max|diff| {np.max(np.abs(a - b))}")
    assert np.array_equal(a, b)


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    import torch
    w = W.CONFIGS[1]                       # 2 x 1024 tokens: about 400 MiB of workspace
    d = w.dims
    dims = lib.make_dims(d, lib.GEN_BF16)
    assert lib.workspace_size(dims, 1, w.batch, w.n_tokens, w.prefix_len) > lib.NOALLOC_SCRATCH_BYTES
    wd = {k: torch.zeros(s, dtype=torch.bfloat16, device="cuda") for k, s in
          [("g_in", (d.hidden,)), ("w_qkv", (d.qkv_out, d.hidden)), ("g_q", (d.head_dim,)), ("g_k", (d.head_dim,)),
           ("w_o", (d.hidden, d.n_q_heads * d.head_dim)), ("g_post", (d.hidden,)),
           ("w_gate_up", (2 * d.mlp_intermediate, d.hidden)), ("w_down", (d.hidden, d.mlp_intermediate))]}
    h = torch.full((w.batch, w.n_tokens, d.hidden), 1.5, device="cuda")
    pk = [torch.zeros(w.prefix_len, d.n_kv_heads, d.head_dim, dtype=torch.bfloat16, device="cuda")] * w.batch
    with pytest.raises(lib.GenError) as e:
        lib.block_forward_noalloc(dims, lib.make_weights(wd), h, pk, pk, [w.prefix_len] * w.batch)
    assert e.value.code == lib.GEN_EWORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((h == 1.5).all()), "a rejected call must leave hidden untouched"
