/*
 * psf_gen.h -- C ABI of the SenseNova-U1 gen-tower denoise step on MI355X (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *   - vllm-omni recipe "SenseNova-U1", "A3B (MoE) variant" and the kernel table of
 *     "Measured (1x H20 96GB, BF16)": each denoise step runs the generation tower of a
 *     Qwen3 (dense) or Qwen3-MoE (A3B: 32 experts, top-8, width 768) decoder over the
 *     image tokens; a block is QKV projection, fused RMSNorm + RoPE on q and k,
 *     attention, O projection, then SwiGLU (act_and_mul) or the routed expert MLP.
 *   - DiffSynth-Studio "SenseNova-U1", 架构说明 (architecture notes): latents are
 *     (1, 3, H, W) pixels with no VAE; the prompt is encoded once into past_key_values
 *     and every denoise step lets the image tokens attend to that static prefix cache.
 *     模型推理 (inference parameters): H and W are multiples of 32, cfg_scale defaults
 *     to 4.0 with a fixed unconditional branch, shift 3.0 moves sigma.
 *     快速推理 (8-step LoRA): cfg_scale 1.0 skips the negative branch; the LoRA sits on
 *     q/k/v/o/gate/up/down of the generation tower.
 *   - vllm-omni recipe "SenseNova-U1.5", Text-to-Image command: cfg_norm "none",
 *     timestep_shift 3.0, t_eps 0.02.
 *   - sensenova-u1-lora-trainer "Setup notes", "Why bf16 base on CPU + tower offload?":
 *     the prefix-KV cache is precomputed per sample and reused every step.
 *
 * Conventions (all entry points):
 *   - Tensor pointers are DEVICE pointers owned by the caller unless marked "host".
 *     The library never allocates, frees, or keeps any pointer after returning; all
 *     scratch memory is the caller's workspace (size from gen_workspace_size).
 *   - Row-major.  Linear weights are [out, in].  bf16 tensors are IEEE bfloat16;
 *     the pixel latents x_t / x_out / x0 are always float32.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on it and
 *     the call returns without synchronising; success means "enqueued".  Errors during
 *     execution surface at the caller's synchronisation, per HIP semantics.
 *   - Arguments are validated on the host before any HIP call: a call that returns an
 *     error has launched nothing and changed nothing.
 *   - Return value: GEN_OK (0) or a negative gen_status; gen_last_error() then returns
 *     a message (thread-local, valid until the next call on that thread).
 *   - Thread-safe and re-entrant; calls that share a workspace must be ordered by the
 *     caller (same stream or explicit synchronisation).
 */
#ifndef PSF_GEN_H
#define PSF_GEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEN_OK = 0,
  GEN_EINVAL = -1,        /* bad argument: null pointer, bad size, inconsistent dims */
  GEN_EUNSUPPORTED = -2,  /* valid but not implemented: cfg_norm != none, dtype/shape combination */
  GEN_EWORKSPACE = -3,    /* workspace_bytes < gen_workspace_size(...) */
  GEN_EHIP = -4           /* a HIP launch failed; gen_last_error() has hipGetErrorString */
} gen_status;

typedef enum { GEN_F32 = 0, GEN_BF16 = 1 } gen_dtype;

/* Shape of one gen block.  Dense blocks set mlp_intermediate > 0 and n_experts = 0;
 * MoE blocks set n_experts, top_k and expert_intermediate and mlp_intermediate = 0.
 * head_dim must be 64 or 128; hidden a multiple of 64; n_q_heads a multiple of n_kv_heads.
 * lora_rank 0 disables LoRA; otherwise a multiple of 8 (<= 128) with scale lora_alpha/lora_rank. */
typedef struct {
  int hidden, n_q_heads, n_kv_heads, head_dim;
  int mlp_intermediate;
  int n_experts, top_k, expert_intermediate;
  int lora_rank;
  float lora_alpha;
  float rms_eps, rope_theta;
  int dtype;        /* gen_dtype of weights, prefix K/V and every GEMM/attention operand */
  int hidden_dtype; /* gen_dtype of the residual stream `hidden` of gen_block_forward: GEN_F32 keeps
                       the residual in fp32 between and inside blocks (only GEMM operands are
                       rounded to dtype); GEN_BF16 stores it in bf16 (dtype must be GEN_BF16).
                       gen_tower_step always keeps its internal residual stream in fp32. */
} gen_block_dims;

/* Weights of one gen block, all in dims.dtype.  Unused pointers may be NULL.
 *   g_in, g_post [D]         RMSNorm gains before attention / before the MLP
 *   w_qkv  [(Hq+2Hkv)*d, D]  rows: q heads, then k heads, then v heads
 *   g_q, g_k [d]             per-head QK-norm gains shared by all heads
 *   w_o    [D, Hq*d]
 *   dense: w_gate_up [2I, D] (gate rows, then up rows), w_down [D, I]
 *   MoE:   w_router [E, D], w_exp_gate_up [E, 2Ie, D], w_exp_down [E, D, Ie]
 *   LoRA (site order q, k, v, o, gate, up, down): lora_a[s] = lora_down [r, in_s],
 *          lora_b[s] = lora_up [out_s, r]; either both NULL (site off) or both set.
 *          Only dense blocks take LoRA.
 *   ld_down  row pitch of w_down in elements: 0 means I (dense rows); otherwise >= I and a
 *          multiple of 8 (dense blocks; ignored for MoE).  With I = 12288 bf16 a dense row is
 *          24 KiB, a multiple of 8 KiB, and the down projection streams its 256 weight rows per
 *          tile from few memory channels; a pitch of I + 64 spreads them and the projection
 *          runs on the 64-deep GEMM (about 15 % faster at the 8B shapes).  Set it once, when the
 *          weights are laid out. */
typedef struct {
  const void *g_in, *w_qkv, *g_q, *g_k, *w_o, *g_post;
  const void *w_gate_up, *w_down;
  const void *w_router, *w_exp_gate_up, *w_exp_down;
  const void *lora_a[7], *lora_b[7];
  int ld_down;
} gen_block_weights;

/* One gen block in place over B image-token sequences of N tokens each.
 *   hidden       [B, N, D] in/out, dims.hidden_dtype
 *   prefix_k/v   HOST arrays of B device pointers; prefix_k[b] is [prefix_len[b], Hkv, d]
 *                (already normed and rotated: used as given).  Token n of sequence b
 *                sits at RoPE position prefix_len[b] + n.  prefix_len[b] may be 0.
 *   prefix_len   HOST [B]
 *   topk_idx_out nullable [B*N, top_k] int32: the routed experts of every token (MoE only),
 *                in descending router-probability order.
 *   workspace    >= gen_workspace_size(dims, 1, B, N, max_b prefix_len[b]) bytes. */
int gen_block_forward(const gen_block_dims* dims, const gen_block_weights* w, void* hidden, int B, int N,
                      const void* const* prefix_k, const void* const* prefix_v, const int* prefix_len,
                      int32_t* topk_idx_out, void* workspace, size_t workspace_bytes, void* stream);

/* gen_block_forward for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, with the workspace taken from a
 * device array inside the library instead of an argument.  The array holds
 * PSF_GEN_NOALLOC_SCRATCH_BYTES (128 MiB) on every GPU the library runs on, until the process
 * ends; a call whose workspace (gen_workspace_size(dims, 1, B, N, max prefix_len)) exceeds it
 * returns GEN_EWORKSPACE with nothing launched.  The call allocates nothing.  Every call on one GPU
 * uses that GPU's single array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.  Arguments and errors otherwise as
 * gen_block_forward. */
#define PSF_GEN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gen_block_forward_noalloc(const gen_block_dims* dims, const gen_block_weights* w, void* hidden, int B, int N,
                              const void* const* prefix_k, const void* const* prefix_v, const int* prefix_len,
                              int32_t* topk_idx_out, void* stream);

/* One denoise step of the gen tower for n_img images and n_br CFG branches
 * (two: 0 = cond, 1 = uncond; three, for image edits: 0 = cond, 1 = img_cond, 2 = uncond):
 *   h0  = patchify(x_t) W_in^T + temb(sigma)      (tokens in raster order of 32x32 patches,
 *                                                  features ordered channel, row, column)
 *   h   = n_layers gen blocks, per branch with its own prefix
 *   x0  = unpatchify(RMSNorm(h; g_final) W_out^T) (float32)
 *   x0g = x0_u + cfg_scale (x0_c - x0_u)          (x0_c when n_br == 1 or cfg_scale == 1)
 *   three branches (dual guidance, as flow_euler_dual_cfg):
 *   x0g = x0_u + img_cfg_scale (x0_i - x0_u) + cfg_scale (x0_c - x0_i)
 *   x_out = x_t + (sigma_next - sigma) (x_t - x0g) / max(sigma, t_eps)
 * temb = temb_w2 silu(temb_w1 [cos(1000 sigma f), sin(1000 sigma f)]), f_j = 1e4^(-j/128).
 *   layers       HOST [n_layers] weight structs
 *   w_in [D, 3072], temb_w1 [D, 256], temb_w2 [D, D], g_final [D], w_out [3072, D]  (dims.dtype)
 *   x_t          [n_img, 3, H, W] float32; H, W multiples of 32
 *   sigma        HOST [n_img]; sigma_next HOST [n_img] or NULL: then x_out receives x0
 *                (n_br must be 1) and no Euler update is made
 *   img_cfg_scale  image guidance, read only when n_br == 3 (1 switches it off)
 *   cfg_norm     0 ("none"); anything else returns GEN_EUNSUPPORTED
 *   prefix_k/v   HOST [n_layers * n_img * n_br] device pointers, index (l*n_img + i)*n_br + br
 *   prefix_len   HOST [n_img * n_br]
 *   x_out        [n_img, 3, H, W] float32 (may alias x_t)
 *   x0_out       nullable [n_img * n_br, 3, H, W] float32: every branch's x0 prediction
 *   workspace    >= gen_workspace_size(dims, n_img, n_br, (H/32)*(W/32), max prefix_len) */
int gen_tower_step(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers,
                   const void* w_in, const void* temb_w1, const void* temb_w2, const void* g_final,
                   const void* w_out, const float* x_t, int n_img, int n_br, int H, int W,
                   const float* sigma, const float* sigma_next, float cfg_scale, float img_cfg_scale,
                   int cfg_norm, float t_eps, const void* const* prefix_k, const void* const* prefix_v,
                   const int* prefix_len, float* x_out, float* x0_out, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Prefix forward: the prompt pass that writes the static prefix-KV cache the gen tower reads
 * (DiffSynth-Studio "SenseNova-U1", 架构说明: image tokens attend to the prompt's past key/values;
 * sensenova-u1-lora-trainer "Setup notes": the prefix cache is computed once and reused).  B prompt
 * sequences of P tokens each run through n_layers blocks of the same structure as the gen block
 * (RMSNorm, QKV, per-head RMSNorm + RoPE at positions 0..P-1, attention, O-proj, RMSNorm, MLP)
 * with CAUSAL attention (token t sees tokens 0..t); the weights are the prompt tower's own.
 *   hidden     [B, P, D] in dims.hidden_dtype: the embedded prompt in, the last block's output out
 *   k_cache    HOST [n_layers * B] device pointers, index l*B + b, each [P, Hkv, d] in dims.dtype:
 *              receives block l's keys after QK-norm and RoPE (the form gen_block_forward takes)
 *   v_cache    HOST [n_layers * B] device pointers [P, Hkv, d]: block l's values
 *   topk_idx_out  nullable int32 [n_layers, B*P, top_k] (MoE blocks): the experts each token was
 *              routed to, as gen_block_forward reports them
 *   workspace  >= gen_workspace_size(dims, 1, B, P, 0) bytes
 * Token embedding (the vocabulary lookup) is not part of this call. */
int gen_prefix_forward(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers,
                       void* hidden, int B, int P, void* const* k_cache, void* const* v_cache,
                       int32_t* topk_idx_out, void* workspace, size_t workspace_bytes, void* stream);

/* Merged-LoRA weights for the fast path in which a LoRA (such as the 8-step distilled one) is
 * fused into the base weights at load (vllm-omni recipe "SenseNova-U1.5", 8-step distilled LoRA;
 * DiffSynth-Studio "SenseNova-U1", 快速推理).  For every site s (q, k, v, o, gate, up, down) whose
 * lora_a/lora_b are set, the site's rows of the base matrix become
 *   W_s' = W_s + (lora_alpha / lora_rank) lora_b[s] lora_a[s]
 * summed in float32 and rounded once to dims.dtype; sites without LoRA are copied.  The merged
 * block then runs with lora_rank = 0 and the four output matrices in place of w_qkv, w_o,
 * w_gate_up, w_down.  dims.lora_rank must be > 0 (dense block); outputs are device buffers of the
 * base matrices' shapes, 16-byte aligned, and may equal the inputs (merge in place). */
int gen_block_lora_merge(const gen_block_dims* dims, const gen_block_weights* w, void* w_qkv_out,
                         void* w_o_out, void* w_gate_up_out, void* w_down_out, void* stream);

/* CFG mix and shifted-flow Euler update, in place, float32, n elements:
 *   x0g = cfg_scale == 1 ? x0_cond : x0_uncond + cfg_scale (x0_cond - x0_uncond)
 *   x  <- x + (sigma_next - sigma) (x - x0g) / max(sigma, t_eps)
 * x0_uncond may be NULL only when cfg_scale == 1.  x must not alias x0_cond/x0_uncond. */
int flow_euler_cfg(float* x, const float* x0_cond, const float* x0_uncond, size_t n, float cfg_scale,
                   float sigma, float sigma_next, float t_eps, void* stream);

/* ---- LoRA training (the trainer's step; sensenova-u1-lora-trainer "Setup notes";
 * lilting.ch "SenseNova U1 8BのLoRA trainer…", default.yaml: x0 loss, uniform timestep, LoRA on
 * attention and MLP; DiffSynth-Studio "SenseNova-U1", 模型训练: sites q, k, v, o, gate, up, down).
 * Only the LoRA matrices receive gradients: base weights, norm gains and embedders are frozen.
 * Dense blocks, bf16 weights, fp32 residual stream (dims.hidden_dtype = GEN_F32), head_dim 128.
 * Gradient buffers are float32, laid out as the matrices (lora_a [rank, in], lora_b [out, rank]),
 * and ACCUMULATE (+=): clear them before a step.  Sites without LoRA need no buffers. */
typedef struct {
  float* lora_a[7];
  float* lora_b[7];
} gen_lora_grads;

/* Workspace bytes for gen_block_backward (0 on invalid arguments). */
size_t gen_backward_workspace_size(const gen_block_dims* dims, int B, int N, int max_prefix);

/* Backward of one gen block over B sequences of N tokens (their prefixes as in gen_block_forward):
 *   hidden_in  [B, N, D] float32: the block's input
 *   d_hidden   [B, N, D] float32: in, dL/d(block output); out, dL/d(block input)
 *   grads      LoRA gradient buffers (may be NULL when dims.lora_rank == 0)
 * The block's forward is recomputed inside the call (activations are not kept between calls). */
int gen_block_backward(const gen_block_dims* dims, const gen_block_weights* w, const float* hidden_in,
                       float* d_hidden, int B, int N, const void* const* prefix_k, const void* const* prefix_v,
                       const int* prefix_len, const gen_lora_grads* grads, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Workspace bytes for gen_tower_lora_train_step: every block's input (fp32) and the activations
 * its backward reads (normed inputs, raw and normed qkv, attention output and log-sum-exp, mid-block
 * residual, gate/up, SwiGLU output, LoRA down-projections), kept from the forward so that no block
 * forward is recomputed (about 0.55 GB per layer at 4 x 1024 tokens of the 8B tower), plus one
 * shared backward scratch. */
size_t gen_train_workspace_size(const gen_block_dims* dims, int n_layers, int n_img, int n_tokens, int max_prefix);

/* One LoRA training step of the gen tower with the x0 loss, one branch per sample:
 *   x0_pred = gen_tower_step's x0 at sigma[i] from x_t (no CFG), loss = mean over all pixels of
 *   (x0_pred - x0)^2, and the gradient of the loss is carried back through the out head, the
 *   final RMSNorm and every block, accumulating each layer's LoRA gradients into grads[l].
 *   x_t, x0      [n_img, 3, H, W] float32 (x_t = (1 - t) x0 + t eps is the caller's sample)
 *   sigma        HOST [n_img]
 *   prefix_k/v   HOST [n_layers * n_img] device pointers, index l*n_img + i; prefix_len HOST [n_img]
 *   grads        HOST [n_layers]
 *   loss         device float32 scalar (written)
 *   x0_pred_out  nullable [n_img, 3, H, W] float32
 *   frozen_t     nullable: the layers' frozen base weights as the backward's operands, filled by
 *                gen_train_frozen_t for these same layers (16-byte aligned); with NULL every step
 *                transposes them again
 * The forward keeps each block's activations in the workspace; the backward reads them.
 * No optimizer update is applied.  Results are the same with and without frozen_t. */
int gen_tower_lora_train_step(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers,
                              const void* w_in, const void* temb_w1, const void* temb_w2, const void* g_final,
                              const void* w_out, const float* x_t, const float* x0, int n_img, int H, int W,
                              const float* sigma, const void* const* prefix_k, const void* const* prefix_v,
                              const int* prefix_len, const gen_lora_grads* grads, float* loss, float* x0_pred_out,
                              const void* frozen_t, void* workspace, size_t workspace_bytes, void* stream);

/* The base weights stay frozen through LoRA training (sensenova-u1-lora-trainer "Setup notes":
 * only the adapters train), so the transposed copies the backward's data gradients multiply by can
 * be made once per training run instead of once per step.  gen_train_frozen_t_size gives the bytes
 * for n_layers layers of these dims (0 on invalid arguments: the training step's dims rules);
 * gen_train_frozen_t writes them (bf16, per layer: w_down^T, w_gate_up^T, w_o^T, w_qkv^T) into
 * frozen_t (caller-owned device memory, 16-byte aligned, >= that size; errors GEN_EINVAL /
 * GEN_EWORKSPACE).  The copies are valid while the base weights do not change. */
size_t gen_train_frozen_t_size(const gen_block_dims* dims, int n_layers);
int gen_train_frozen_t(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers, void* frozen_t,
                       size_t bytes, void* stream);

/* Dual guidance of an image edit and the Euler update, in place, float32, n elements
 * (vllm-omni recipe "SenseNova-U1.5", img2img: cfg_scale guides toward the instruction,
 * img_cfg_scale toward the input image, 1.0 switching image guidance off, the 3-way run using
 * cond + img_cond + uncond; DiffSynth-Studio "SenseNova-U1", 图像编辑: the negative branch keeps
 * the image and drops the instruction).  The pages print no formula; the nested form is taken:
 *   x0g = x0_uncond + img_cfg_scale (x0_img - x0_uncond) + cfg_scale (x0_cond - x0_img)
 *   x  <- x + (sigma_next - sigma) (x - x0g) / max(sigma, t_eps)
 * With img_cfg_scale == 1 the uncond branch drops out (x0_img + cfg_scale (x0_cond - x0_img)) and
 * x0_uncond may be NULL.  x must not alias the predictions. */
int flow_euler_dual_cfg(float* x, const float* x0_cond, const float* x0_img, const float* x0_uncond, size_t n,
                        float cfg_scale, float img_cfg_scale, float sigma, float sigma_next, float t_eps,
                        void* stream);

/* Router of an MoE gen block on its own, for checking routing decisions:
 *   logits = u w_router^T (float32 accumulate), p = softmax(logits), the top_k largest p
 *   (ties to the lower expert index), weights p / sum over the top_k.
 *   u [T, D] and w_router [E, D] in `dtype`; idx_out [T, top_k] int32 and w_out [T, top_k]
 *   float32, both in descending-probability order.  D a positive multiple of 64, E <= 64,
 *   top_k <= E; otherwise GEN_EINVAL.  (Inside gen_block_forward the router reads the fp32
 *   mid-block residual and applies the post-attention RMSNorm itself, all in float32.) */
int gen_moe_route(const void* u, const void* w_router, int T, int D, int E, int top_k, int dtype,
                  int32_t* idx_out, float* w_out, void* stream);

/* Workspace bytes for gen_tower_step with these sizes (n_tokens = (H/32)*(W/32));
 * the same value covers gen_block_forward with B = n_img*n_br.  0 on invalid dims. */
size_t gen_workspace_size(const gen_block_dims* dims, int n_img, int n_br, int n_tokens, int max_prefix);

/* HOST helper: the shifted sigma schedule, sigmas[k] = shift s_k / (1 + (shift-1) s_k) with
 * s_k = 1 - k/steps, k = 0..steps (float64; sigmas[0] = 1, sigmas[steps] = 0). */
int gen_sigma_schedule(int steps, double shift, double* sigmas);

/* Message of the last failing call on this thread ("" after a success). */
const char* gen_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PSF_GEN_H */
