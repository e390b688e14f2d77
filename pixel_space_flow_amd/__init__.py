"""Python binding of libpsf_gen.so, the MI355X gen-tower denoise step.

Argument marshalling only: every step of the computation runs in the HIP library.
torch is used for device memory (``tensor.data_ptr()``) and the current stream.
Importing this package fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# PSF_GEN_LIB names another build of the same library (the host-only sanitizer build that the
# CPU tests of the argument checks load); by default the in-tree HIP build
LIB_PATH = os.environ.get("PSF_GEN_LIB") or os.path.join(HERE, "libpsf_gen.so")

GEN_OK, GEN_EINVAL, GEN_EUNSUPPORTED, GEN_EWORKSPACE, GEN_EHIP = 0, -1, -2, -3, -4
GEN_F32, GEN_BF16 = 0, 1
LORA_SITES = ("q", "k", "v", "o", "gate", "up", "down")

# every symbol declared in include/psf_gen.h
EXPORTS = ("gen_block_forward", "gen_block_forward_noalloc", "gen_tower_step", "flow_euler_cfg", "flow_euler_dual_cfg", "gen_moe_route",
           "gen_workspace_size",
           "gen_sigma_schedule", "gen_last_error", "gen_block_lora_merge", "gen_prefix_forward",
           "gen_backward_workspace_size", "gen_block_backward", "gen_train_workspace_size", "gen_tower_lora_train_step",
           "gen_train_frozen_t_size", "gen_train_frozen_t",
           # include/psf_gen_ops.h
           "gen_op_rmsnorm", "gen_op_linear", "gen_op_qknorm_rope", "gen_op_attention", "gen_op_workspace_size",
           "gen_timing_begin", "gen_timing_end")
TIMING_FAMILIES = {"gate_up": 0, "attention": 1, "qkv": 2, "down": 3, "o": 4, "expert": 5}


class GenError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class BlockDimsC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("mlp_intermediate", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("top_k", ctypes.c_int), ("expert_intermediate", ctypes.c_int), ("lora_rank", ctypes.c_int),
                ("lora_alpha", ctypes.c_float), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", ctypes.c_int), ("hidden_dtype", ctypes.c_int)]


class BlockWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("g_in", "w_qkv", "g_q", "g_k", "w_o", "g_post", "w_gate_up",
                                                "w_down", "w_router", "w_exp_gate_up", "w_exp_down")] + \
               [("lora_a", ctypes.c_void_p * 7), ("lora_b", ctypes.c_void_p * 7), ("ld_down", ctypes.c_int)]


class LoraGradsC(ctypes.Structure):
    _fields_ = [("lora_a", ctypes.c_void_p * 7), ("lora_b", ctypes.c_void_p * 7)]


def _load():
    # torch bundles its own HIP runtime with the same soname (libamdhip64.so.7) as /opt/rocm's.
    # Mapping torch's first makes the library bind to that one runtime, so device pointers and
    # streams from torch are valid in our calls (two runtimes in one process see no device).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python pixel_space_flow_amd/build.py` "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    P = ctypes.POINTER
    lib.gen_block_forward.argtypes = [P(BlockDimsC), P(BlockWeightsC), vp, i, i, P(vp), P(vp), P(i), vp, vp, sz, vp]
    lib.gen_block_forward_noalloc.argtypes = [P(BlockDimsC), P(BlockWeightsC), vp, i, i, P(vp), P(vp), P(i), vp, vp]
    lib.gen_tower_step.argtypes = [P(BlockDimsC), i, P(BlockWeightsC), vp, vp, vp, vp, vp, vp, i, i, i, i,
                                   P(f), P(f), f, f, i, f, P(vp), P(vp), P(i), vp, vp, vp, sz, vp]
    lib.flow_euler_cfg.argtypes = [vp, vp, vp, sz, f, f, f, f, vp]
    lib.flow_euler_dual_cfg.argtypes = [vp, vp, vp, vp, sz, f, f, f, f, f, vp]
    lib.gen_block_lora_merge.argtypes = [P(BlockDimsC), P(BlockWeightsC), vp, vp, vp, vp, vp]
    lib.gen_backward_workspace_size.argtypes = [P(BlockDimsC), i, i, i]
    lib.gen_backward_workspace_size.restype = sz
    lib.gen_block_backward.argtypes = [P(BlockDimsC), P(BlockWeightsC), vp, vp, i, i, P(vp), P(vp), P(i),
                                       P(LoraGradsC), vp, sz, vp]
    lib.gen_train_workspace_size.argtypes = [P(BlockDimsC), i, i, i, i]
    lib.gen_train_workspace_size.restype = sz
    lib.gen_tower_lora_train_step.argtypes = [P(BlockDimsC), i, P(BlockWeightsC), vp, vp, vp, vp, vp, vp, vp, i, i, i,
                                              P(f), P(vp), P(vp), P(i), P(LoraGradsC), vp, vp, vp, vp, sz, vp]
    lib.gen_train_frozen_t_size.argtypes = [P(BlockDimsC), i]
    lib.gen_train_frozen_t_size.restype = sz
    lib.gen_train_frozen_t.argtypes = [P(BlockDimsC), i, P(BlockWeightsC), vp, sz, vp]
    lib.gen_prefix_forward.argtypes = [P(BlockDimsC), i, P(BlockWeightsC), vp, i, i, P(vp), P(vp), vp, vp, sz, vp]
    lib.gen_moe_route.argtypes = [vp, vp, i, i, i, i, i, vp, vp, vp]
    lib.gen_workspace_size.argtypes = [P(BlockDimsC), i, i, i, i]
    lib.gen_workspace_size.restype = sz
    lib.gen_sigma_schedule.argtypes = [i, ctypes.c_double, P(ctypes.c_double)]
    lib.gen_last_error.restype = ctypes.c_char_p
    lib.gen_op_rmsnorm.argtypes = [vp, vp, vp, i, i, f, i, vp]
    lib.gen_op_linear.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.gen_op_qknorm_rope.argtypes = [vp, i, i, i, i, i, P(i), vp, vp, f, f, vp, sz, i, vp]
    lib.gen_op_attention.argtypes = [vp, i, i, i, i, i, P(vp), P(vp), P(i), vp, vp, sz, i, vp]
    lib.gen_op_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.gen_op_workspace_size.restype = sz
    lib.gen_timing_begin.argtypes = [i, i]
    lib.gen_timing_end.argtypes = [P(ctypes.c_double), P(i)]
    for n in ("gen_block_forward", "gen_block_forward_noalloc", "gen_tower_step", "flow_euler_cfg", "gen_moe_route", "gen_sigma_schedule",
              "gen_op_rmsnorm", "gen_op_linear", "gen_op_qknorm_rope", "gen_op_attention",
              "gen_timing_begin", "gen_timing_end"):
        getattr(lib, n).restype = i
    return lib


lib = _load()


def _check(rc: int):
    if rc != GEN_OK:
        raise GenError(rc, lib.gen_last_error().decode())


def last_error() -> str:
    return lib.gen_last_error().decode()


# ----------------------------------------------------------------------------- marshalling
def make_dims(d, dtype: int, hidden_dtype: int = GEN_F32) -> BlockDimsC:
    """ctypes dims from any object with the gen_block_dims field names.  The residual stream
    defaults to fp32."""
    return BlockDimsC(d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.mlp_intermediate, d.n_experts, d.top_k,
                      d.expert_intermediate, d.lora_rank, float(d.lora_alpha), float(d.rms_eps),
                      float(d.rope_theta), dtype, hidden_dtype)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_weights(w: dict) -> BlockWeightsC:
    """ctypes weights from a dict of device tensors keyed by gen_block_weights field names
    (LoRA: ``lora_a_<site>`` / ``lora_b_<site>``; ``ld_down``: the row pitch of w_down in
    elements, an int, absent or 0 for dense rows)."""
    c = BlockWeightsC()
    for n, _ in BlockWeightsC._fields_[:11]:
        setattr(c, n, _ptr(w.get(n)))
    for k, s in enumerate(LORA_SITES):
        c.lora_a[k] = _ptr(w.get(f"lora_a_{s}"))
        c.lora_b[k] = _ptr(w.get(f"lora_b_{s}"))
    c.ld_down = int(w.get("ld_down", 0) or 0)
    return c


def _stream(stream) -> int:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr_array(ts: Sequence):
    arr = (ctypes.c_void_p * max(1, len(ts)))()
    for k, t in enumerate(ts):
        arr[k] = _ptr(t)
    return arr


def workspace_size(dims: BlockDimsC, n_img: int, n_br: int, n_tokens: int, max_prefix: int) -> int:
    n = lib.gen_workspace_size(ctypes.byref(dims), n_img, n_br, n_tokens, max_prefix)
    if n == 0:
        raise GenError(GEN_EINVAL, last_error())
    return n


def alloc_workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def sigma_schedule(steps: int, shift: float):
    out = (ctypes.c_double * (steps + 1))()
    _check(lib.gen_sigma_schedule(steps, float(shift), out))
    return list(out)


def block_forward(dims: BlockDimsC, weights: BlockWeightsC, hidden, prefix_k, prefix_v, prefix_len, workspace,
                  topk_out=None, stream=None):
    B, N = hidden.shape[0], hidden.shape[1]
    plen = (ctypes.c_int * B)(*prefix_len)
    _check(lib.gen_block_forward(ctypes.byref(dims), ctypes.byref(weights), hidden.data_ptr(), B, N,
                                 _ptr_array(prefix_k), _ptr_array(prefix_v), plen, _ptr(topk_out),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))


def block_forward_noalloc(dims: BlockDimsC, weights: BlockWeightsC, hidden, prefix_k, prefix_v, prefix_len,
                          topk_out=None, stream=None):
    """gen_block_forward without a workspace argument: the library's own per-GPU scratch array
    (NOALLOC_SCRATCH_BYTES) serves instead; nothing is allocated."""
    B, N = hidden.shape[0], hidden.shape[1]
    plen = (ctypes.c_int * B)(*prefix_len)
    _check(lib.gen_block_forward_noalloc(ctypes.byref(dims), ctypes.byref(weights), hidden.data_ptr(), B, N,
                                         _ptr_array(prefix_k), _ptr_array(prefix_v), plen, _ptr(topk_out),
                                         _stream(stream)))


NOALLOC_SCRATCH_BYTES = 128 << 20


def prefix_forward(dims: BlockDimsC, layers: Sequence[BlockWeightsC], hidden, k_cache, v_cache, workspace,
                   topk_out=None, stream=None):
    """Causal prompt pass over hidden [B, P, D] (in place).  k_cache/v_cache: flat lists of
    [P, Hkv, d] device tensors indexed l*B + b, filled with each block's keys (normed and
    rotated) and values.  topk_out: optional int32 [n_layers, B*P, top_k] (MoE)."""
    B, P = hidden.shape[0], hidden.shape[1]
    L = len(layers)
    arr = (BlockWeightsC * max(1, L))(*layers)
    _check(lib.gen_prefix_forward(ctypes.byref(dims), L, arr, hidden.data_ptr(), B, P, _ptr_array(k_cache),
                                  _ptr_array(v_cache), _ptr(topk_out), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def make_lora_grads(g: dict) -> LoraGradsC:
    """ctypes gradient buffers from a dict of float32 device tensors keyed ``lora_a_<site>`` /
    ``lora_b_<site>`` (missing sites: NULL)."""
    c = LoraGradsC()
    for k, s in enumerate(LORA_SITES):
        c.lora_a[k] = _ptr(g.get(f"lora_a_{s}"))
        c.lora_b[k] = _ptr(g.get(f"lora_b_{s}"))
    return c


def backward_workspace_size(dims: BlockDimsC, B: int, N: int, max_prefix: int) -> int:
    n = lib.gen_backward_workspace_size(ctypes.byref(dims), B, N, max_prefix)
    if n == 0:
        raise GenError(GEN_EINVAL, last_error())
    return n


def train_workspace_size(dims: BlockDimsC, n_layers: int, n_img: int, n_tokens: int, max_prefix: int) -> int:
    n = lib.gen_train_workspace_size(ctypes.byref(dims), n_layers, n_img, n_tokens, max_prefix)
    if n == 0:
        raise GenError(GEN_EINVAL, last_error())
    return n


def block_backward(dims: BlockDimsC, weights: BlockWeightsC, hidden_in, d_hidden, prefix_k, prefix_v, prefix_len,
                   grads: Optional[LoraGradsC], workspace, stream=None):
    """d_hidden [B, N, D] fp32: in dL/d(out), out dL/d(in); LoRA gradients accumulate into grads."""
    B, N = hidden_in.shape[0], hidden_in.shape[1]
    plen = (ctypes.c_int * B)(*prefix_len)
    _check(lib.gen_block_backward(ctypes.byref(dims), ctypes.byref(weights), hidden_in.data_ptr(), d_hidden.data_ptr(),
                                  B, N, _ptr_array(prefix_k), _ptr_array(prefix_v), plen,
                                  ctypes.byref(grads) if grads is not None else None, workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def train_frozen_t_size(dims: BlockDimsC, n_layers: int) -> int:
    return lib.gen_train_frozen_t_size(ctypes.byref(dims), n_layers)


def train_frozen_t(dims: BlockDimsC, layers: Sequence[BlockWeightsC], frozen_t, stream=None):
    """The frozen base weights' transposes for the training backward, made once (frozen_t: uint8 device
    buffer of at least train_frozen_t_size bytes)."""
    L = len(layers)
    arr = (BlockWeightsC * L)(*layers)
    _check(lib.gen_train_frozen_t(ctypes.byref(dims), L, arr, frozen_t.data_ptr(),
                                  frozen_t.numel() * frozen_t.element_size(), _stream(stream)))


def tower_lora_train_step(dims: BlockDimsC, layers: Sequence[BlockWeightsC], glob: dict, x_t, x0, sigma, prefix_k,
                          prefix_v, prefix_len, grads: Sequence[LoraGradsC], loss, workspace, x0_pred_out=None,
                          stream=None, frozen_t=None):
    """One LoRA training step (x0 loss): loss (device fp32 scalar) is written, grads[l] accumulate.
    frozen_t: optional buffer filled by train_frozen_t for the same layers."""
    n_img, _, H, W = x_t.shape
    L = len(layers)
    arr = (BlockWeightsC * L)(*layers)
    garr = (LoraGradsC * L)(*grads)
    sig = (ctypes.c_float * n_img)(*sigma)
    plen = (ctypes.c_int * n_img)(*prefix_len)
    _check(lib.gen_tower_lora_train_step(ctypes.byref(dims), L, arr, _ptr(glob["w_in"]), _ptr(glob["temb_w1"]),
                                         _ptr(glob["temb_w2"]), _ptr(glob["g_final"]), _ptr(glob["w_out"]),
                                         x_t.data_ptr(), x0.data_ptr(), n_img, H, W, sig, _ptr_array(prefix_k),
                                         _ptr_array(prefix_v), plen, garr, loss.data_ptr(), _ptr(x0_pred_out),
                                         _ptr(frozen_t), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                         _stream(stream)))


def block_lora_merge(dims: BlockDimsC, weights: BlockWeightsC, w_qkv_out, w_o_out, w_gate_up_out, w_down_out,
                     stream=None):
    """Fold each LoRA site of `weights` into the base matrices (outputs may be the inputs)."""
    _check(lib.gen_block_lora_merge(ctypes.byref(dims), ctypes.byref(weights), w_qkv_out.data_ptr(),
                                    w_o_out.data_ptr(), w_gate_up_out.data_ptr(), w_down_out.data_ptr(),
                                    _stream(stream)))


def tower_step(dims: BlockDimsC, layers: Sequence[BlockWeightsC], glob: dict, x_t, n_br: int, sigma, sigma_next,
               cfg_scale: float, t_eps: float, prefix_k, prefix_v, prefix_len, x_out, workspace, x0_out=None,
               cfg_norm: int = 0, stream=None, img_cfg_scale: float = 1.0):
    """glob: w_in, temb_w1, temb_w2, g_final, w_out.  prefix_k/v: flat lists indexed
    (l*n_img + i)*n_br + br.  sigma/sigma_next: per-image host floats (sigma_next None:
    x_out receives x0)."""
    n_img, _, H, W = x_t.shape
    L = len(layers)
    arr = (BlockWeightsC * max(1, L))(*layers)
    sig = (ctypes.c_float * n_img)(*sigma)
    sn = None if sigma_next is None else (ctypes.c_float * n_img)(*sigma_next)
    plen = (ctypes.c_int * (n_img * n_br))(*prefix_len)
    _check(lib.gen_tower_step(ctypes.byref(dims), L, arr, _ptr(glob["w_in"]), _ptr(glob["temb_w1"]),
                              _ptr(glob["temb_w2"]), _ptr(glob["g_final"]), _ptr(glob["w_out"]), x_t.data_ptr(),
                              n_img, n_br, H, W, sig, sn, float(cfg_scale), float(img_cfg_scale), cfg_norm,
                              float(t_eps),
                              _ptr_array(prefix_k), _ptr_array(prefix_v), plen, x_out.data_ptr(), _ptr(x0_out),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))


def flow_euler_cfg(x, x0_cond, x0_uncond, cfg_scale: float, sigma: float, sigma_next: float, t_eps: float,
                   stream=None):
    _check(lib.flow_euler_cfg(x.data_ptr(), x0_cond.data_ptr(), _ptr(x0_uncond), x.numel(), float(cfg_scale),
                              float(sigma), float(sigma_next), float(t_eps), _stream(stream)))


def flow_euler_dual_cfg(x, x0_cond, x0_img, x0_uncond, cfg_scale: float, img_cfg_scale: float, sigma: float,
                        sigma_next: float, t_eps: float, stream=None):
    _check(lib.flow_euler_dual_cfg(x.data_ptr(), x0_cond.data_ptr(), x0_img.data_ptr(), _ptr(x0_uncond), x.numel(),
                                   float(cfg_scale), float(img_cfg_scale), float(sigma), float(sigma_next),
                                   float(t_eps), _stream(stream)))


def moe_route(u, w_router, top_k: int, idx_out, w_out, dtype: int, stream=None):
    T, D = u.shape
    E = w_router.shape[0]
    _check(lib.gen_moe_route(u.data_ptr(), w_router.data_ptr(), T, D, E, top_k, dtype, idx_out.data_ptr(),
                             w_out.data_ptr(), _stream(stream)))


# ----------------------------------------------------------------------------- step-level ops
def _dt(t) -> int:
    import torch
    return GEN_BF16 if t.dtype == torch.bfloat16 else GEN_F32


def op_rmsnorm(x, g, y, eps: float, stream=None):
    D = x.shape[-1]
    _check(lib.gen_op_rmsnorm(x.data_ptr(), g.data_ptr(), y.data_ptr(), x.numel() // D, D, float(eps), _dt(x),
                              _stream(stream)))


def op_linear(x, w, y, resid=None, epi: int = 0, stream=None):
    M, K = x.shape
    N = y.shape[1]
    _check(lib.gen_op_linear(x.data_ptr(), w.data_ptr(), y.data_ptr(), _ptr(resid), M, N, K, epi, _dt(x),
                             _stream(stream)))


def op_workspace_size(B, N, Hkv, d, max_prefix, dtype) -> int:
    return lib.gen_op_workspace_size(B, N, Hkv, d, max_prefix, dtype)


def op_qknorm_rope(qkv, B, N, Hq, Hkv, d, prefix_len, g_q, g_k, eps, theta, workspace, stream=None):
    plen = (ctypes.c_int * B)(*prefix_len)
    _check(lib.gen_op_qknorm_rope(qkv.data_ptr(), B, N, Hq, Hkv, d, plen, g_q.data_ptr(), g_k.data_ptr(),
                                  float(eps), float(theta), workspace.data_ptr(), workspace.numel(), _dt(qkv),
                                  _stream(stream)))


def op_attention(qkv, B, N, Hq, Hkv, d, prefix_k, prefix_v, prefix_len, out, workspace, stream=None):
    plen = (ctypes.c_int * B)(*prefix_len)
    _check(lib.gen_op_attention(qkv.data_ptr(), B, N, Hq, Hkv, d, _ptr_array(prefix_k), _ptr_array(prefix_v), plen,
                                out.data_ptr(), workspace.data_ptr(), workspace.numel(), _dt(qkv), _stream(stream)))


def timing_begin(family: str, capacity: int):
    _check(lib.gen_timing_begin(TIMING_FAMILIES[family], capacity))


def timing_end():
    """(total milliseconds, number of timed launches) since timing_begin."""
    ms, n = ctypes.c_double(), ctypes.c_int()
    _check(lib.gen_timing_end(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
