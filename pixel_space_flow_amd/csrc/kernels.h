// Host launchers of the gen-tower kernels (everything except the GEMMs).
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>
#include "common.h"
#include "gemm.h"

namespace psf {

constexpr int MAXB = 32;  // sequences per block call (prefix pointers travel in kernel arguments)

struct SeqInfo {
  int B, N;                 // sequences, image tokens per sequence
  int plen[MAXB];           // prefix tokens of each sequence
  const void* pk[MAXB];     // prefix K [plen, Hkv, d]
  const void* pv[MAXB];     // prefix V [plen, Hkv, d]
};

// y[r, :] = x[r, :] / sqrt(mean(x^2) + eps) * g   (x: Tin, g/y: T; D % (16/sizeof(Tin)) == 0)
template <typename Tin, typename T>
hipError_t rmsnorm(const Tin* x, const T* g, T* y, int rows, int D, float eps, hipStream_t s);

// table[pos][j] = (cos(pos w_j), sin(pos w_j)), w_j = theta^(-2j/d), pos < n_pos (fp64 math, fp32 out)
hipError_t rope_table(float2* table, int n_pos, int head_dim, float theta, hipStream_t s);

// In place on the q and k heads of qkv [B*N, ld]: per-head RMSNorm (gain g_q / g_k) then
// rotate-half RoPE at position plen[b] + n.
template <typename T>
// raw_out (nullable, pitch ld): receives the q and k heads as they were before the norm.
hipError_t qknorm_rope(T* qkv, int64_t ld, const SeqInfo& si, int Hq, int Hkv, int d, const T* gq, const T* gk,
                       const float2* table, float eps, hipStream_t s, T* raw_out = nullptr);

// Pack keys and transposed values of every (sequence, kv head) contiguously:
//   Kc[b][g][j][:] = j < P_b ? prefix K : (j < P_b + N ? k of token j - P_b : 0)     [B, Hkv, Lpad, d]
//   Vt[b][g][:][j] = same for V, transposed                                          [B, Hkv, d, Lpad]
// The prompt pass's hand-off to the caller's cache: for every sequence b, the rows of qkv hold
// q (QD columns), then k and v (row_elems = Hkv d columns each); k goes to kcache[b] and v to
// vcache[b], each [N, Hkv, d] dense.  One launch, 16 bytes per thread; every pointer must be
// 16-byte aligned.
template <typename T>
hipError_t kv_cache_write(const T* qkv, int64_t ld, int QD, int N, int row_elems, int B, void* const* kcache,
                          void* const* vcache, hipStream_t s);

template <typename T>
hipError_t pack_kv(const T* qkv, int64_t ld, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad, T* Kc, T* Vt,
                   hipStream_t s);

// pack_kv with the image keys put through per-head RMSNorm (gain gk) and RoPE (position = their
// index j in the packed sequence, P_b + n) on the way; prefix keys are copied as they are.
hipError_t pack_kv_knorm(const bf16* qkv, int64_t ld, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad,
                         const bf16* gk, const float2* table, float eps, bf16* Kc, bf16* Vt, hipStream_t s);

// O[b*N + n, h*d:(h+1)*d] = softmax(q k^T / sqrt(d)) v over the L_b = P_b + N keys of Kc/Vt
// (causal: over keys j <= P_b + n only).  With gq non-null the q heads of qkv are raw: per-head
// RMSNorm (gain gq) and RoPE at position P_b + n are applied to each query as it is loaded.
hipError_t attention_bf16(const bf16* qkv, int64_t ldq, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad,
                          const bf16* Kc, const bf16* Vt, bf16* O, int64_t ldo, const bf16* gq,
                          const float2* table, float eps, bool causal, hipStream_t s, float* lse = nullptr);
hipError_t attention_f32(const float* qkv, int64_t ldq, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad,
                         const float* Kc, const float* Vt, float* O, int64_t ldo, bool causal, hipStream_t s);

// Wo [out, in] = W + scale B A with A [rank, in], B [out, rank] (rank a multiple of 8, <= 128;
// fp32 sums, one rounding); A == nullptr copies W.  Wo may equal W.
template <typename T>
hipError_t lora_merge(const T* W, const T* A, const T* B, T* Wo, int out, int in, int64_t ldw, int rank, float scale,
                      hipStream_t s);

// patches[(i*N + t), f] from x [n_img, 3, H, W] (32x32 patches, raster tokens, (c, iy, ix) features)
template <typename T>
hipError_t patchify(const float* x, T* patches, int n_img, int H, int W, hipStream_t s);

// temb[i, :] = w2 silu(w1 feat(sigma_i)); feat = [cos(1000 sigma f_j), sin(1000 sigma f_j)], j < 128
template <typename T>
hipError_t timestep_embed(const float* sigma_dev, const T* w1, const T* w2, float* h1, float* temb, int n_img, int D,
                          hipStream_t s);

// xo = x + (sn - s) (x - x0g) / max(s, t_eps) with x0g the guided prediction: xc alone (no
// other branch, or unit scales), xu + scale (xc - xu) (two branches), or with xm (img_cond, three
// branches) xu + img_scale (xm - xu) + scale (xc - xm); img_scale 1 or xu null gives
// xm + scale (xc - xm).  xo may equal x.
hipError_t cfg_euler(float* xo, const float* x, const float* xc, const float* xm, const float* xu, size_t n,
                     float scale, float img_scale, float sigma, float sigma_next, float t_eps, hipStream_t s);

// ---- training backward (backward.hip)
hipError_t transpose_bf16(const bf16* in, int64_t ldi, bf16* out, int64_t ldo, int R, int C, hipStream_t s);
// out [C, R] (row pitch ldo) = in [R, C]^T (row pitch ldi) for up to TRANSPOSE_MAX_JOBS matrices in
// one launch
constexpr int TRANSPOSE_MAX_JOBS = 16;
struct TransposeJob {
  const bf16* in; int64_t ldi; bf16* out; int64_t ldo; int R, C;
};
hipError_t transpose_many(const TransposeJob* jobs, int n, hipStream_t s);
hipError_t cast_f32_bf16(const float* x, bf16* y, int64_t n, hipStream_t s);
// out = base + (dRMSNorm(x; g))^T dy per row of D (base may alias out or be null); outb, when set,
// also receives bf16(out)
hipError_t rmsnorm_bwd(const float* x, const bf16* g, const bf16* dy, const float* base, float* out, int rows, int D,
                       float eps, hipStream_t s, bf16* outb = nullptr);
// z = silu(gate) up over gu = [gate | up] (rows 2 I); z rows ldz apart
hipError_t swiglu_fwd(const bf16* gu, bf16* z, int64_t ldz, int M, int I, hipStream_t s);
// dgu = [dgate | dup] of z = silu(gate) up (dz rows I, dgu rows ldg apart)
hipError_t swiglu_bwd(const bf16* gu, const bf16* dz, bf16* dgu, int64_t ldg, int M, int I, hipStream_t s);
// dqkv = gradient with respect to the raw q, k heads (through RoPE and the per-head norm) and v
hipError_t qknorm_rope_bwd(const bf16* raw, int64_t ldr, const float* dq, const float* dk, const float* dv,
                           const SeqInfo& si, int Hq, int Hkv, int d, const bf16* gq, const bf16* gk,
                           const float2* table, float eps, bf16* dqkv, int64_t ldo, hipStream_t s);
// qkv: normed, rotated q/k and v of the image tokens; O, dO [M, Hq d]; lse [B, Hq, N] (log2 units);
// Dq scratch [B, Hq, N]; dq [M, Hq d], dk, dv [M, Hkv d] fp32 (image keys only)
hipError_t attention_bwd(const bf16* qkv, int64_t ldq, const SeqInfo& si, int Hq, int Hkv, int d, const bf16* O,
                         const bf16* dO, const float* lse, float* Dq, float* dq, float* dk, float* dv, hipStream_t s);
// C[n1, n2] += sum_m X[m, n1] Y[m, n2]; part: scratch of at least WGRAD_PART_FLOATS floats
constexpr int64_t WGRAD_PART_FLOATS = (int64_t)4 << 20;
int wgrad_splits(int M, int N1, int N2);
hipError_t wgrad(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, int N1, int N2, float* C, float* part,
                 hipStream_t s);
// As wgrad with N1 <= 128 split into up to three blocks of seg_rows rows, block k added into C[k]
// ([seg_rows, N2] each)
hipError_t wgrad_seg(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, int N1, int N2, int seg_rows,
                     float* const* C, float* part, hipStream_t s);
// Block-diagonal B gradients of up to three sites side by side: C[i] [outs[i], r] += sum_m
// X[m, site i's columns]^T Y[m, r i .. r i + r - 1] in one pass (X's sites from column 0, outs[i]
// multiples of 128, Y the sites' down-projections side by side).
hipError_t wgrad_diag(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, const int* outs, int ns, int r,
                      float* const* C, float* part, hipStream_t s);
hipError_t x0_loss(const float* pred, const float* tgt, float* grad, float* part, int nparts, float* loss, int64_t n,
                   hipStream_t s);

// Skinny GEMM (N <= 128, K a multiple of 64; bmode 0 or 2, EPI_SCALED into bf16 C): split over K,
// partial sums in part (skinny_part_floats(M, N) floats), reduced in a fixed order.
constexpr int SKINNY_MAX_SPLITS = 16;
inline size_t skinny_part_floats(int M, int N) { return (size_t)SKINNY_MAX_SPLITS * M * N; }
int skinny_splits(int M, int K);
hipError_t gemm_skinny(const GemmParams& p, float* part, hipStream_t s);
// C [M, 32 ns] (pitch ldc) = scale A B^T with a block-diagonal B: output columns 32 i .. 32 i + 31
// take B[i] [32, outs[i]] (pitch outs[i]) against A's columns of site i (sites side by side from
// column 0, outs[i] multiples of 64); A read once.  part: skinny_part_floats(M, 32 ns) floats.
hipError_t gemm_skinny_diag(const bf16* A, int64_t lda, int M, const bf16* const* B, const int* outs, int ns, float scale,
                           bf16* C, int64_t ldc, float* part, hipStream_t s);
// Low-rank product C (op)= X Y^T, K a multiple of 8 (LoRA up-projection): mode 0 C bf16 = acc,
// 1 C bf16 = bf16(C + acc), 2 C fp32 += acc, 3 C fp32 = acc.
hipError_t gemm_lowrank(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, int N, int K, void* C,
                        int64_t ldc, int mode, hipStream_t s);

// Router over x [T, D] (D a multiple of 64), wr [E, D] (E <= 64): logits of rmsnorm(x; g, eps)
// when g is non-null (x the fp32 residual, everything in fp32), of x itself otherwise; softmax,
// top-k (ties to the lower index), weights renormalised over the k -> idx/w [T, k].  With lrank
// (and blkcnt, moe_route_blocks(T) x E ints) it also writes each assignment's stable rank among
// its router workgroup's assignments of the same expert, and those per-expert counts.
template <typename Tx, typename Tw>
hipError_t moe_route(const Tx* x, const Tw* g, float eps, const Tw* wr, int T_, int D, int E, int k, int* idx, float* w,
                     int* lrank, int* blkcnt, hipStream_t s);
int moe_route_blocks(int T_);

// Counting sort of the T*k assignments by expert (stable in token order) from the router's
// ranks and counts (blkoff: scratch of moe_route_blocks(T) x E ints), tile table for the grouped
// GEMM (bm-row tiles), and each assignment's position in the sorted order.
hipError_t moe_sort(const int* idx, const int* lrank, const int* blkcnt, int* blkoff, int T_, int k, int E,
                    int* counts, int* offsets, int* perm_tok, int* pos_of, int* tiles, int max_tiles, int bm,
                    hipStream_t s);

// h[t, :] = bf16(r[t, :] + sum_j w[t, j] y[pos_of[t*k + j], :])   (fp32 residual r, fixed j order)
template <typename TH>
hipError_t moe_combine(TH* h, const float* r, const bf16* y, const float* w, const int* pos_of, int T_, int k, int D,
                       hipStream_t s);

}  // namespace psf
