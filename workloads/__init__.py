"""Seeded synthetic workloads for the SenseNova-U1 gen-tower denoise step.

This module only defines shapes and draws random tensors.  It holds none of
the method's arithmetic (no norms, projections, attention, schedules or
updates): both the CPU oracle (``oracle/``) and the GPU path read their inputs
from here, and nothing else is shared between them.

Every tensor comes from its own stream,
``Generator(PCG64(SeedSequence([config_id, seed, tag_hash])))``, where
``tag_hash`` is a stable 32-bit hash of a tensor name such as ``"L3.w_qkv"``.
Streams therefore do not depend on generation order, and any single tensor
(one layer's weights, one prefix sample) can be regenerated on its own.

Distributions (the same in every workload): linear weights N(0, 0.02);
norm gains 1 + N(0, 0.1); prefix K and V N(0, 1); noise N(0, 1); LoRA down
(A) N(0, 0.02) and LoRA up (B) N(0, 1e-3); router weights N(0, 1/sqrt(D)) so
that router logits of unit-RMS activations are about N(0, 1).  "N(0, s)"
means standard deviation s.  For bf16 runs every tensor is rounded to bf16
(round to nearest even) once, and both sides see the rounded values.
"""
from __future__ import annotations

import dataclasses
import hashlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

PATCH = 32            # pixels per patch side; images must be multiples of 32
PIX_CH = 3            # RGB pixel latents, no VAE
PATCH_DIM = PIX_CH * PATCH * PATCH   # 3072 features per patch
TEMB_FREQ_DIM = 256   # sinusoidal timestep features fed to the ts embedder

# Indices of the seven LoRA sites of a gen block, in this order.
LORA_SITES = ("q", "k", "v", "o", "gate", "up", "down")


@dataclasses.dataclass(frozen=True)
class BlockDims:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp_intermediate: int = 0          # dense SwiGLU width; 0 for MoE
    n_experts: int = 0                 # MoE; 0 for dense
    top_k: int = 0
    expert_intermediate: int = 0
    lora_rank: int = 0                 # 0 = no LoRA
    lora_alpha: float = 0.0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark configuration of the gen tower."""
    config_id: int
    name: str
    dims: BlockDims
    n_layers: int
    n_img: int               # images (or training samples) per call
    n_br: int                # CFG branches per image: 2 = [cond, uncond], 1 = no CFG
    height: int              # pixels
    width: int
    prefix_len: int          # prefix-KV tokens per sample and layer
    cfg_scale: float = 4.0
    shift: float = 3.0
    n_steps: int = 50
    t_eps: float = 0.02
    unit: str = "tower"      # "tower" (gen_tower_step) or "block" (gen_block_forward)
    prefix_cache_samples: int = 0   # >0: prefixes are drawn from a cache of this many samples
    dtypes: tuple = ("bf16",)
    img_cfg_scale: float = 1.0       # image guidance of the three-branch (image edit) step
    branch_prefix: tuple = ()        # per-branch prefix lengths (else prefix_len for every branch)

    @property
    def n_tokens(self) -> int:
        return (self.height // PATCH) * (self.width // PATCH)

    @property
    def batch(self) -> int:
        return self.n_img * self.n_br

    def prefix_len_of(self, sample: int) -> int:
        """Prefix length of sample = image * n_br + branch."""
        return self.branch_prefix[sample % self.n_br] if self.branch_prefix else self.prefix_len

    @property
    def max_prefix(self) -> int:
        return max(self.branch_prefix) if self.branch_prefix else self.prefix_len


QWEN3_8B = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, mlp_intermediate=12288)

CONFIGS: Dict[int, Workload] = {
    0: Workload(0, "tiny-2layer-256px", BlockDims(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                                    mlp_intermediate=768),
                n_layers=2, n_img=1, n_br=2, height=256, width=256, prefix_len=32,
                cfg_scale=4.0, shift=3.0, n_steps=2, dtypes=("f32", "bf16")),
    1: Workload(1, "qwen3-8b-block-1024px", BlockDims(**QWEN3_8B), n_layers=1, n_img=1, n_br=2,
                height=1024, width=1024, prefix_len=400, unit="block"),
    2: Workload(2, "qwen3-8b-tower36-2048px-cfg", BlockDims(**QWEN3_8B), n_layers=36, n_img=1, n_br=2,
                height=2048, width=2048, prefix_len=400, cfg_scale=4.0, shift=3.0, n_steps=50,
                t_eps=0.02),
    3: Workload(3, "qwen3-8b-tower36-lora-r32-4x1024px",
                BlockDims(**QWEN3_8B, lora_rank=32, lora_alpha=32.0), n_layers=36, n_img=4, n_br=1,
                height=1024, width=1024, prefix_len=400, cfg_scale=1.0, prefix_cache_samples=56),
    4: Workload(4, "a3b-moe-block-2048px", BlockDims(hidden=2048, n_q_heads=32, n_kv_heads=4,
                                                       head_dim=128, n_experts=32, top_k=8,
                                                       expert_intermediate=768),
                n_layers=1, n_img=1, n_br=2, height=2048, width=2048, prefix_len=400, unit="block"),
}


# Workloads beyond the benchmark configurations above.
# Image edit with dual guidance: three branches per image in the order cond (edit image +
# instruction), img_cond (edit image, no instruction), uncond (neither), cfg 4 and image cfg 2
# as in the pages' 3-way run.  Reading for the prefix lengths (the pages give none): the edit
# image adds 1024 tokens (a 1024^2 input in 32-pixel patches) to a 400-token text part, so
# cond and img_cond carry 1424 prefix tokens and uncond the 400-token fixed text.
VARIANTS: Dict[str, Workload] = {
    "dual_cfg": Workload(5, "qwen3-8b-tower36-2048px-dual-cfg-edit", BlockDims(**QWEN3_8B), n_layers=36,
                         n_img=1, n_br=3, height=2048, width=2048, prefix_len=1424, cfg_scale=4.0,
                         img_cfg_scale=2.0, shift=3.0, n_steps=50, t_eps=0.02, branch_prefix=(1424, 1424, 400)),
}


# ----------------------------------------------------------------------------- RNG

def tag_hash(tag: str) -> int:
    return int.from_bytes(hashlib.sha256(tag.encode()).digest()[:4], "little")


def rng(config_id: int, seed: int, tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, seed, tag_hash(tag)])))


def normal(config_id: int, seed: int, tag: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    x = rng(config_id, seed, tag).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def uniform(config_id: int, seed: int, tag: str, shape, lo: float, hi: float) -> np.ndarray:
    return rng(config_id, seed, tag).uniform(lo, hi, size=shape).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32.

    Input preparation only: bf16 runs draw fp32 values and round them once, so
    that both sides start from identical numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint32).view(np.float32)
    if nan.any():
        out = np.where(nan, x, out)
    return out.reshape(x.shape)


def maybe_bf16(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else x


# ----------------------------------------------------------------------------- tensors

WEIGHT_STD = 0.02
GAIN_STD = 0.1
LORA_A_STD = 0.02
LORA_B_STD = 1e-3


def layer_tensor_specs(d: BlockDims, layer: int, tower: str = "L"):
    """(name, shape, kind) of every tensor of one gen block.  Linear weights are
    [out, in]; the fused gate/up weight stacks gate rows above up rows.  ``tower``
    prefixes the names: "L" for the gen tower, "U" for the prompt (prefix) tower."""
    D = d.hidden
    qd, kvd = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    specs = [("g_in", (D,), "gain"), ("w_qkv", (d.qkv_out, D), "w"),
             ("g_q", (d.head_dim,), "gain"), ("g_k", (d.head_dim,), "gain"),
             ("w_o", (D, qd), "w"), ("g_post", (D,), "gain")]
    if d.is_moe:
        E, Ie = d.n_experts, d.expert_intermediate
        specs += [("w_router", (E, D), "router"), ("w_exp_gate_up", (E, 2 * Ie, D), "w"),
                  ("w_exp_down", (E, D, Ie), "w")]
    else:
        I = d.mlp_intermediate
        specs += [("w_gate_up", (2 * I, D), "w"), ("w_down", (D, I), "w")]
    if d.lora_rank:
        r = d.lora_rank
        ins = {"q": D, "k": D, "v": D, "o": qd, "gate": D, "up": D, "down": d.mlp_intermediate}
        outs = {"q": qd, "k": kvd, "v": kvd, "o": D, "gate": d.mlp_intermediate,
                "up": d.mlp_intermediate, "down": D}
        for s in LORA_SITES:
            specs += [(f"lora_a_{s}", (r, ins[s]), "lora_a"), (f"lora_b_{s}", (outs[s], r), "lora_b")]
    return [(f"{tower}{layer}.{n}", shp, kind) for n, shp, kind in specs]


def _draw(config_id, seed, name, shape, kind, D):
    if kind == "w":
        return normal(config_id, seed, name, shape, WEIGHT_STD)
    if kind == "gain":
        return normal(config_id, seed, name, shape, GAIN_STD, 1.0)
    if kind == "router":
        return normal(config_id, seed, name, shape, 1.0 / np.sqrt(D))
    if kind == "lora_a":
        return normal(config_id, seed, name, shape, LORA_A_STD)
    if kind == "lora_b":
        return normal(config_id, seed, name, shape, LORA_B_STD)
    raise ValueError(kind)


def layer_weights(w: Workload, layer: int, seed: int = 0, dtype: str = "bf16",
                  threads: int = 8, tower: str = "L") -> Dict[str, np.ndarray]:
    """All tensors of gen block ``layer`` as fp32 arrays (bf16-rounded for bf16 runs).
    Keys drop the ``L<layer>.`` prefix."""
    specs = layer_tensor_specs(w.dims, layer, tower)

    def one(spec):
        name, shape, kind = spec
        return name.split(".", 1)[1], maybe_bf16(_draw(w.config_id, seed, name, shape, kind, w.dims.hidden), dtype)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        return dict(ex.map(one, specs))


def prefix_dims(w: Workload) -> BlockDims:
    """Block shape of the prompt tower: the gen block's, without LoRA (adapters train the
    gen tower only)."""
    return dataclasses.replace(w.dims, lora_rank=0, lora_alpha=0.0)


def prefix_layer_weights(w: Workload, layer: int, seed: int = 0, dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """Weights of prompt-tower block ``layer`` (names ``U<layer>.*``, same distributions)."""
    return layer_weights(dataclasses.replace(w, dims=prefix_dims(w)), layer, seed, dtype, tower="U")


def prompt_hidden(w: Workload, seed: int = 0, dtype: str = "f32") -> np.ndarray:
    """Embedded prompt [batch, prefix_len, D] ~ N(0, 1): the prompt tower's input, standing in
    for token embeddings of an encoded prompt (one per sample and CFG branch)."""
    shp = (w.batch, w.prefix_len, w.dims.hidden)
    return maybe_bf16(normal(w.config_id, seed, "prompt_hidden", shp), dtype)


def prefix_kv(w: Workload, layer: int, sample: int, seed: int = 0, dtype: str = "bf16"):
    """Static prefix K and V of one (layer, sample): two [P, Hkv, d] arrays, N(0, 1).
    For CFG workloads sample = image * n_br + branch (branch 0 cond, 1 uncond);
    for cache workloads it is the cache slot."""
    shp = (w.prefix_len_of(sample), w.dims.n_kv_heads, w.dims.head_dim)
    k = normal(w.config_id, seed, f"L{layer}.prefix_k.s{sample}", shp)
    v = normal(w.config_id, seed, f"L{layer}.prefix_v.s{sample}", shp)
    return maybe_bf16(k, dtype), maybe_bf16(v, dtype)


def cache_slots(w: Workload, seed: int = 0) -> List[int]:
    """Distinct prefix-cache slots used by the n_img samples of a cache workload."""
    if not w.prefix_cache_samples:
        return list(range(w.batch))
    g = rng(w.config_id, seed, "prefix_cache_slots")
    return [int(i) for i in g.choice(w.prefix_cache_samples, size=w.n_img, replace=False)]


def tower_globals(w: Workload, seed: int = 0, dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """Patch embed, timestep embedder and out head of the tower."""
    D = w.dims.hidden
    specs = {"w_in": (D, PATCH_DIM), "temb_w1": (D, TEMB_FREQ_DIM), "temb_w2": (D, D),
             "w_out": (PATCH_DIM, D)}
    out = {k: maybe_bf16(normal(w.config_id, seed, k, s, WEIGHT_STD), dtype) for k, s in specs.items()}
    out["g_final"] = maybe_bf16(normal(w.config_id, seed, "g_final", (D,), GAIN_STD, 1.0), dtype)
    return out


def noise_image(w: Workload, seed: int = 0) -> np.ndarray:
    """Pixel noise [n_img, 3, H, W] ~ N(0, 1), fp32 (the latent stays fp32)."""
    return normal(w.config_id, seed, "noise", (w.n_img, PIX_CH, w.height, w.width))


def clean_image(w: Workload, seed: int = 0) -> np.ndarray:
    """Clean training pixels [n_img, 3, H, W] ~ U(-1, 1), fp32."""
    return uniform(w.config_id, seed, "x0", (w.n_img, PIX_CH, w.height, w.width), -1.0, 1.0)


def train_timesteps(w: Workload, seed: int = 0) -> np.ndarray:
    """Per-sample training timestep t ~ U(0, 1), float64."""
    return rng(w.config_id, seed, "t").uniform(0.0, 1.0, size=w.n_img)


def block_hidden(w: Workload, seed: int = 0, dtype: str = "bf16") -> np.ndarray:
    """Block-level input hidden state [B, N, D] ~ N(0, 1)."""
    return maybe_bf16(normal(w.config_id, seed, "hidden", (w.batch, w.n_tokens, w.dims.hidden)), dtype)


def small_dims(**kw) -> BlockDims:
    """Reduced block dims for quick tests; keyword overrides on top of config 0's block."""
    base = dataclasses.asdict(CONFIGS[0].dims)
    base.update(kw)
    return BlockDims(**base)


def scaled(w: Workload, **kw) -> Workload:
    """Copy of a workload with some fields replaced (used to shrink depth/size in tests)."""
    return dataclasses.replace(w, **kw)
