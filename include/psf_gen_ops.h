/*
 * psf_gen_ops.h -- the individual steps of a gen block as separate entry points, for
 * step-level parity tests and per-kernel timing.  They launch exactly the kernels that
 * gen_block_forward launches for the same step.  Conventions (device pointers, caller-owned
 * memory, host-side validation first, stream semantics, error reporting through
 * gen_last_error) are those of psf_gen.h.  `dtype` is a gen_dtype.
 *
 * Steps and their sources (page title, section):
 *   gen_op_rmsnorm      RMSNorm before attention / MLP and of the tower output (vllm-omni
 *                       recipe "SenseNova-U1", kernel table: RMSNorm + RoPE).
 *   gen_op_linear       the block's projections (QKV, O, gate/up with SwiGLU, down), kernel
 *                       table rows "nvjet GEMMs" and "act_and_mul".
 *   gen_op_qknorm_rope  fused per-head RMSNorm + RoPE on q and k (kernel table:
 *                       qk_norm_rope_kernel).
 *   gen_op_attention    image tokens attending to [prefix cache ; own keys] (DiffSynth-Studio
 *                       "SenseNova-U1", 架构说明).
 */
#ifndef PSF_GEN_OPS_H
#define PSF_GEN_OPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* y[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * g.  x, y [rows, D]; g [D]; D % 64 == 0. */
int gen_op_rmsnorm(const void* x, const void* g, void* y, int rows, int D, float eps, int dtype, void* stream);

/* Linear layer y = x w^T with an epilogue, x [M, K], K % 64 == 0:
 *   epi 0: y [M, N] = x w^T,               w [N, K]
 *   epi 1: y [M, N] = resid + x w^T,       w [N, K], resid [M, N] (may equal y)
 *   epi 2: y [M, N] = silu(x wg^T) * (x wu^T), w [2N, K] = gate rows then up rows
 *   epi 3: y [M, N] float32 += x w^T (dtype GEN_BF16 only; resid ignored): the O and down
 *          projections onto the block's fp32 residual stream */
int gen_op_linear(const void* x, const void* w, void* y, const void* resid, int M, int N, int K, int epi, int dtype,
                  void* stream);

/* In place on qkv [B*N, (Hq+2Hkv)*d]: per-head RMSNorm of the q and k heads (gains g_q, g_k [d])
 * then rotate-half RoPE (theta) at position prefix_len[b] + n.  prefix_len HOST [B].
 * workspace >= gen_op_workspace_size(...) bytes (RoPE table). */
int gen_op_qknorm_rope(void* qkv, int B, int N, int Hq, int Hkv, int d, const int* prefix_len, const void* g_q,
                       const void* g_k, float eps, float theta, void* workspace, size_t workspace_bytes, int dtype,
                       void* stream);

/* out [B*N, Hq*d] = softmax(q K^T / sqrt(d)) V per query head, K/V = [prefix ; the k/v heads of qkv],
 * query head h reading kv head h / (Hq/Hkv).  qkv [B*N, (Hq+2Hkv)*d]; prefix_k/v HOST arrays of B
 * device pointers [prefix_len[b], Hkv, d]; prefix_len HOST [B]. */
int gen_op_attention(const void* qkv, int B, int N, int Hq, int Hkv, int d, const void* const* prefix_k,
                     const void* const* prefix_v, const int* prefix_len, void* out, void* workspace,
                     size_t workspace_bytes, int dtype, void* stream);

/* Workspace bytes for gen_op_qknorm_rope / gen_op_attention. */
size_t gen_op_workspace_size(int B, int N, int Hkv, int d, int max_prefix, int dtype);

#ifdef __cplusplus
}
#endif
#endif /* PSF_GEN_OPS_H */

#ifndef PSF_GEN_TIMING_H
#define PSF_GEN_TIMING_H
#ifdef __cplusplus
extern "C" {
#endif
/* Launch timing of one kernel family inside later gen_* calls, for roofline reports.
 * gen_timing_begin(family, capacity) creates 2*capacity HIP events (host-side objects, no device
 * memory) and from then on brackets every launch of that family with event records on the
 * launch's stream, up to `capacity` launches.  gen_timing_end synchronises on the last event,
 * returns the summed elapsed milliseconds and the number of timed launches, and destroys the
 * events.  Families: 0 gate/up (SwiGLU) GEMM, 1 attention, 2 QKV GEMM, 3 down GEMM, 4 O GEMM,
 * 5 expert GEMMs.  Process-global and not thread-safe: for measurement runs only. */
int gen_timing_begin(int family, int capacity);
int gen_timing_end(double* total_ms, int* n_launches);
#ifdef __cplusplus
}
#endif
#endif
