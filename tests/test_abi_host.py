"""Host-side checks of the C ABI that run without a GPU: the library loads (every kernel
handle resolves), exports every function the headers declare, and rejects bad arguments on
the host before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("psf_gen.h", "psf_gen_ops.h")]


def declared_functions():
    names = []
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\**\s*((?:gen|flow)_\w+)\s*\(", src, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def psf():
    import pixel_space_flow_amd
    return pixel_space_flow_amd


def test_library_loads_and_exports_every_declared_symbol(psf):
    names = declared_functions()
    assert "gen_tower_step" in names and "gen_block_forward" in names and "flow_euler_cfg" in names
    for n in names:
        assert hasattr(psf.lib, n), n
    assert set(names) <= set(psf.EXPORTS)


def test_library_has_no_unresolved_kernel_handles():
    # dlopen with RTLD_NOW resolves every symbol; a kernel whose host stub was not emitted
    # shows up here as an undefined symbol
    import torch  # noqa: F401  (same runtime binding order as the package)
    ctypes.CDLL(os.path.join(ROOT, "pixel_space_flow_amd", "libpsf_gen.so"), mode=os.RTLD_NOW)


def test_sigma_schedule_host(psf):
    import oracle
    s = psf.sigma_schedule(50, 3.0)
    np.testing.assert_allclose(s, oracle.sigma_schedule(50, 3.0), rtol=0, atol=1e-15)
    with pytest.raises(psf.GenError):
        psf.sigma_schedule(0, 3.0)


def dims(psf, **kw):
    import workloads as W
    return psf.make_dims(W.CONFIGS[2].dims, psf.GEN_BF16) if not kw else psf.make_dims(W.small_dims(**kw), psf.GEN_BF16)


def test_workspace_size(psf):
    d = dims(psf)
    n = psf.workspace_size(d, 1, 2, 4096, 400)
    assert 0.5e9 < n < 2e9
    bad = psf.BlockDimsC(**{f: getattr(d, f) for f, _ in d._fields_})
    bad.head_dim = 96
    with pytest.raises(psf.GenError):
        psf.workspace_size(bad, 1, 2, 4096, 400)


def call_block(psf, d, w, hidden=16, B=2, N=16, plen=None, ws_bytes=1 << 20):
    arr = (ctypes.c_void_p * B)()
    pl = (ctypes.c_int * B)(*(plen or [0] * B))
    return psf.lib.gen_block_forward(ctypes.byref(d), ctypes.byref(w), hidden, B, N, arr, arr, pl, None,
                                     4096 if ws_bytes else None, ws_bytes, None)


def fake_weights(psf):
    w = psf.BlockWeightsC()
    for f in ("g_in", "w_qkv", "g_q", "g_k", "w_o", "g_post", "w_gate_up", "w_down"):
        setattr(w, f, 4096)      # non-null, aligned; never dereferenced: validation fails first
    return w


def test_block_forward_rejects_bad_arguments_on_host(psf):
    d = dims(psf)
    w = psf.BlockWeightsC()
    assert call_block(psf, d, w) == psf.GEN_EINVAL and "g_in" in psf.last_error()
    w = fake_weights(psf)
    assert call_block(psf, d, w, hidden=None) == psf.GEN_EINVAL
    assert call_block(psf, d, w, hidden=4097) == psf.GEN_EINVAL            # unaligned
    assert call_block(psf, d, w, B=0) == psf.GEN_EINVAL
    assert call_block(psf, d, w, B=64) == psf.GEN_EUNSUPPORTED
    assert call_block(psf, d, w, plen=[-1, 0]) == psf.GEN_EINVAL
    assert call_block(psf, d, w, plen=[5, 0]) == psf.GEN_EINVAL            # prefix length without pointers
    assert call_block(psf, d, w, ws_bytes=16) == psf.GEN_EWORKSPACE
    d2 = dims(psf)
    d2.n_q_heads = 30
    assert call_block(psf, d2, w) == psf.GEN_EINVAL                        # Hq % Hkv != 0
    d3 = dims(psf)
    d3.dtype = psf.GEN_F32
    d3.hidden_dtype = psf.GEN_BF16
    assert call_block(psf, d3, w) == psf.GEN_EUNSUPPORTED
    d4 = dims(psf)
    d4.lora_rank = 12
    assert call_block(psf, d4, w) == psf.GEN_EUNSUPPORTED                  # rank not a multiple of 8
    d5 = dims(psf)
    d5.n_experts = 32
    assert call_block(psf, d5, w) == psf.GEN_EINVAL                        # dense and MoE at once
    w6 = fake_weights(psf)
    for ld in (d.mlp_intermediate - 8, d.mlp_intermediate + 4, -64):
        w6.ld_down = ld
        assert call_block(psf, d, w6) == psf.GEN_EINVAL and "ld_down" in psf.last_error()   # bad w_down pitch


def test_tower_step_rejects_bad_arguments_on_host(psf):
    d = dims(psf)
    lw = (psf.BlockWeightsC * 1)(fake_weights(psf))
    one = (ctypes.c_float * 1)(1.0)
    nxt = (ctypes.c_float * 1)(0.9)
    arr = (ctypes.c_void_p * 2)(4096, 4096)
    pl = (ctypes.c_int * 2)(4, 4)

    def call(H=64, W=64, n_br=2, cfg_norm=0, sigma_next=nxt, x=4096, ws=1 << 30, img_cfg=1.0):
        return psf.lib.gen_tower_step(ctypes.byref(d), 1, lw, 4096, 4096, 4096, 4096, 4096, x, 1, n_br, H, W,
                                      one, sigma_next, 4.0, img_cfg, cfg_norm, 0.02, arr3, arr3, pl3, 4096, None,
                                      4096, ws, None)
    arr3 = (ctypes.c_void_p * 3)(4096, 4096, 4096)
    pl3 = (ctypes.c_int * 3)(4, 4, 4)
    assert call(H=48) == psf.GEN_EINVAL            # not a multiple of 32
    assert call(n_br=4) == psf.GEN_EINVAL
    assert call(n_br=0) == psf.GEN_EINVAL
    assert call(n_br=3, img_cfg=float("nan")) == psf.GEN_EINVAL
    assert call(cfg_norm=1) == psf.GEN_EUNSUPPORTED
    assert call(sigma_next=None) == psf.GEN_EINVAL  # x0-only output needs one branch
    assert call(x=None) == psf.GEN_EINVAL
    assert call(ws=8) == psf.GEN_EWORKSPACE


def test_flow_euler_cfg_rejects_bad_arguments_on_host(psf):
    f = psf.lib.flow_euler_cfg
    assert f(None, 4096, 4096, 16, 4.0, 1.0, 0.9, 0.02, None) == psf.GEN_EINVAL
    assert f(4096, 4096, None, 16, 4.0, 1.0, 0.9, 0.02, None) == psf.GEN_EINVAL   # uncond needed for cfg != 1
    assert f(4100, 4096, 4096, 16, 4.0, 1.0, 0.9, 0.02, None) == psf.GEN_EINVAL   # unaligned
    assert f(4096, 4096, 4096, 16, 4.0, 0.0, 0.0, 0.0, None) == psf.GEN_EINVAL    # zero denominator


def test_flow_euler_dual_cfg_rejects_bad_arguments_on_host(psf):
    f = psf.lib.flow_euler_dual_cfg
    assert f(4096, 4096, None, 4096, 16, 4.0, 2.0, 1.0, 0.9, 0.02, None) == psf.GEN_EINVAL   # img branch needed
    assert f(4096, 4096, 4096, None, 16, 4.0, 2.0, 1.0, 0.9, 0.02, None) == psf.GEN_EINVAL   # uncond for img cfg != 1
    assert f(4096, 4096, 4100, 4096, 16, 4.0, 2.0, 1.0, 0.9, 0.02, None) == psf.GEN_EINVAL   # unaligned
    assert f(4096, 4096, 4096, 4096, 16, float("inf"), 2.0, 1.0, 0.9, 0.02, None) == psf.GEN_EINVAL
    assert f(4096, 4096, 4096, 4096, 16, 4.0, 2.0, 0.0, 0.0, 0.0, None) == psf.GEN_EINVAL    # zero denominator


def test_block_lora_merge_rejects_bad_arguments_on_host(psf):
    f = psf.lib.gen_block_lora_merge
    d = dims(psf)                                    # lora_rank 0
    w = fake_weights(psf)
    assert f(ctypes.byref(d), ctypes.byref(w), 4096, 4096, 4096, 4096, None) == psf.GEN_EINVAL
    assert "nothing to merge" in psf.last_error()
    d.lora_rank, d.lora_alpha = 32, 32.0
    assert f(ctypes.byref(d), ctypes.byref(w), None, 4096, 4096, 4096, None) == psf.GEN_EINVAL
    assert f(ctypes.byref(d), ctypes.byref(w), 4096, 4100, 4096, 4096, None) == psf.GEN_EINVAL   # unaligned
    d.lora_rank = 12
    assert f(ctypes.byref(d), ctypes.byref(w), 4096, 4096, 4096, 4096, None) == psf.GEN_EUNSUPPORTED


def test_prefix_forward_rejects_bad_arguments_on_host(psf):
    f = psf.lib.gen_prefix_forward
    d = dims(psf)
    lw = (psf.BlockWeightsC * 2)(fake_weights(psf), fake_weights(psf))
    good = (ctypes.c_void_p * 4)(4096, 4096, 4096, 4096)
    hole = (ctypes.c_void_p * 4)(4096, 4096, None, 4096)

    def call(n_layers=2, layers=lw, hidden=4096, B=2, P=400, kc=good, vc=good, ws=1 << 30):
        return f(ctypes.byref(d), n_layers, layers, hidden, B, P, kc, vc, None, 4096, ws, None)
    assert call(n_layers=0) == psf.GEN_EINVAL
    assert call(layers=(psf.BlockWeightsC * 2)(fake_weights(psf), psf.BlockWeightsC())) == psf.GEN_EINVAL
    assert "layer 1" in psf.last_error() or "g_in" in psf.last_error()
    assert call(hidden=None) == psf.GEN_EINVAL
    assert call(hidden=4100) == psf.GEN_EINVAL                    # unaligned
    assert call(P=0) == psf.GEN_EINVAL
    assert call(B=64) == psf.GEN_EUNSUPPORTED
    assert call(kc=hole) == psf.GEN_EINVAL                        # every (layer, sequence) slot needed
    assert call(vc=None) == psf.GEN_EINVAL
    assert call(ws=64) == psf.GEN_EWORKSPACE


def test_training_entry_points_reject_bad_arguments_on_host(psf):
    d = dims(psf)                     # 8B-shaped dense bf16 block, head_dim 128
    d.lora_rank, d.lora_alpha = 32, 32.0
    w = fake_weights(psf)
    for s in range(7):
        w.lora_a[s] = 4096
        w.lora_b[s] = 4096
    g = psf.LoraGradsC()
    arr = (ctypes.c_void_p * 2)(4096, 4096)
    pl = (ctypes.c_int * 2)(4, 4)
    f = psf.lib.gen_block_backward

    def call(dd=d, ww=w, gg=g, h=4096, dh=4096, B=2, N=64, ws=1 << 34):
        return f(ctypes.byref(dd), ctypes.byref(ww), h, dh, B, N, arr, arr, pl,
                 ctypes.byref(gg) if gg is not None else None, 4096, ws, None)
    assert call() == psf.GEN_EINVAL and "gradient" in psf.last_error()      # LoRA sites without buffers
    for s in range(7):
        g.lora_a[s] = 4096
        g.lora_b[s] = 4096
    assert call(h=None) == psf.GEN_EINVAL
    assert call(dh=4100) == psf.GEN_EINVAL                                    # unaligned
    assert call(B=64) == psf.GEN_EUNSUPPORTED
    assert call(ws=64) == psf.GEN_EWORKSPACE
    d64 = dims(psf)
    d64.head_dim = 64
    assert call(dd=d64, gg=None) == psf.GEN_EUNSUPPORTED                     # attention backward needs d = 128
    dm = dims(psf)
    dm.mlp_intermediate, dm.n_experts, dm.top_k, dm.expert_intermediate = 0, 8, 2, 256
    assert call(dd=dm, gg=None) == psf.GEN_EUNSUPPORTED                      # dense blocks only
    assert psf.lib.gen_backward_workspace_size(ctypes.byref(d), 2, 64, 0) > 0
    assert psf.lib.gen_train_workspace_size(ctypes.byref(d), 0, 1, 64, 0) == 0


def test_frozen_transposes_entry_points_reject_bad_arguments_on_host(psf):
    d = dims(psf)                     # 8B-shaped dense bf16 block: w_down^T, w_gate_up^T (rows padded), w_o^T, w_qkv^T
    w = fake_weights(psf)
    lw = (psf.BlockWeightsC * 2)(w, w)
    per_layer = psf.lib.gen_train_frozen_t_size(ctypes.byref(d), 1)
    assert per_layer >= 2 * (12288 * 4096 + 4096 * 24640 + 4096 * 4096 + 4096 * 6144)
    assert psf.lib.gen_train_frozen_t_size(ctypes.byref(d), 2) == 2 * per_layer
    assert psf.lib.gen_train_frozen_t_size(ctypes.byref(d), 0) == 0
    d64 = dims(psf)
    d64.head_dim = 64
    assert psf.lib.gen_train_frozen_t_size(ctypes.byref(d64), 1) == 0      # the training step's dims rules
    f = psf.lib.gen_train_frozen_t

    def call(n_layers=2, layers=lw, buf=4096, nbytes=1 << 40):
        return f(ctypes.byref(d), n_layers, layers, buf, nbytes, None)
    assert call(n_layers=0) == psf.GEN_EINVAL
    assert call(layers=None) == psf.GEN_EINVAL
    assert call(layers=(psf.BlockWeightsC * 2)(w, psf.BlockWeightsC())) == psf.GEN_EINVAL
    assert call(buf=None) == psf.GEN_EINVAL
    assert call(buf=4100) == psf.GEN_EINVAL                                   # unaligned
    assert call(nbytes=2 * per_layer - 1) == psf.GEN_EWORKSPACE
