// Skinny and low-rank GEMMs of the LoRA projections.
//
// Skinny GEMM (the down-projections): C[m, n] = scale sum_k A[m, k] B[n, k] with N <= 128 output
// columns (rank r, or up to three sites of rank r side by side).  A 256 x 256 tile GEMM gives such
// a product only M/256 workgroups; here one wave owns 32 rows x N columns over one k-range (four
// waves of consecutive row blocks per workgroup share the k-range, so their B loads meet in the
// L1 cache), the k-ranges split K so that about 2048 waves run, and a second pass adds the
// partial sums in a fixed order (no atomics), scales and rounds once to bf16.
//
// Per 64-deep step a wave loads its 32 A rows as whole 128-byte rows (8 rows per instruction),
// passes them through LDS into the v_mfma_f32_32x32x16_bf16 fragment layout (lane l: row l % 32,
// k offset 8 (l / 32)), and takes its B fragments straight from global memory in that layout; the
// next step's loads are issued before this one's MFMAs.
#include "common.h"
#include "gemm.h"
#include "kernels.h"

namespace psf {
namespace {

// DIAG: block-diagonal B, one 32-column block per site: block nb takes B_nb (pitch ldb, ldb1,
// ldb2) over the k-range of its site only ([0, kb1), [kb1, kb2), [kb2, K)), so one pass over A's
// rows serves sites that read different column ranges of A.
template <int NB, bool DIAG = false>
__global__ __launch_bounds__(256) void skinny_kernel(const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ B0,
                                                     const bf16* __restrict__ B1, const bf16* __restrict__ B2,
                                                     int64_t ldb, int seg_rows, int M, int N, int K, int kchunk,
                                                     float* __restrict__ part, int64_t ldb1 = 0, int64_t ldb2 = 0,
                                                     int kb1 = 0, int kb2 = 0) {
  __shared__ __attribute__((aligned(16))) char sa[4][32 * 128];   // one 32-row x 64-deep A step per wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 31, lh = lane >> 5;
  const int m0 = blockIdx.x * 128 + w * 32, z = blockIdx.y;
  if (m0 >= M) return;                          // no workgroup barrier below
  const int k_lo = z * kchunk, k_hi = min(K, k_lo + kchunk);
  char* my = sa[w];
  // A: load i brings rows 8i .. 8i + 7, lane l the 16-byte chunk l % 8 of row 8i + l / 8
  const bf16* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ap[i] = A + (int64_t)min(m0 + i * 8 + (lane >> 3), M - 1) * lda + (lane & 7) * 8;
  const bf16* bp[NB];
  bool bok[NB];
  int klo[NB], khi[NB];                         // DIAG: k-range of block nb's site
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 32 + lr;
    bok[nb] = n < N;
    const int nc = bok[nb] ? n : 0;
    if (DIAG) {
      klo[nb] = nb == 0 ? 0 : (nb == 1 ? kb1 : kb2);
      khi[nb] = nb == 0 ? (NB > 1 ? kb1 : K) : (nb == 1 ? (NB > 2 ? kb2 : K) : K);
      const bf16* base = nb == 0 ? B0 : (nb == 1 ? B1 : B2);
      const int64_t pitch = nb == 0 ? ldb : (nb == 1 ? ldb1 : ldb2);
      bp[nb] = base + (int64_t)(nc - nb * 32) * pitch + lh * 8;   // row of the site's B, k from klo
    } else {
      const int seg = nc / seg_rows;
      const bf16* base = seg == 0 ? B0 : (seg == 1 ? B1 : B2);
      bp[nb] = base + (int64_t)(nc - seg * seg_rows) * ldb + lh * 8;
    }
  }
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[nb][e] = 0.f;
  bf16x8 a[4], b[NB][4], an[4], bn[NB][4];
  const bf16x8 zero = {};
  auto load = [&](int k, bf16x8 (&ao)[4], bf16x8 (&bo)[NB][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ao[i] = *(const bf16x8*)(ap[i] + k);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (DIAG)
          bo[nb][i] = (bok[nb] && k >= klo[nb] && k < khi[nb]) ? *(const bf16x8*)(bp[nb] + (k - klo[nb]) + 16 * i) : zero;
        else
          bo[nb][i] = bok[nb] ? *(const bf16x8*)(bp[nb] + k + 16 * i) : zero;
      }
    }
  };
  if (k_lo < k_hi) load(k_lo, a, b);
  for (int k = k_lo; k < k_hi; k += 64) {
    const bool more = k + 64 < k_hi;
    // the wave's A rows through LDS (chunk c of row r stored at c ^ (r & 7)), read back as
    // fragments: lane l takes row l % 32 at k offset 16 i + 8 (l / 32)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 8 + (lane >> 3);
      *(bf16x8*)(my + r * 128 + (((lane & 7) ^ (r & 7)) << 4)) = a[i];
    }
    __builtin_amdgcn_wave_barrier();
    bf16x8 fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8*)(my + lr * 128 + (((2 * i + lh) ^ (lr & 7)) << 4));
    __builtin_amdgcn_wave_barrier();
    if (more) load(k + 64, an, bn);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], b[nb][i], acc[nb], 0, 0, 0);
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = an[i];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) b[nb][i] = bn[nb][i];
      }
    }
  }
  float* out = part + (int64_t)z * M * N;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + (e >> 2) * 8 + lh * 4 + (e & 3), n = nb * 32 + lr;
      if (m < M && n < N) out[(int64_t)m * N + n] = acc[nb][e];
    }
}

// C[m * ldc + n] = bf16(scale * sum_z part[z][m][n])
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                            float scale, bf16* __restrict__ C, int64_t ldc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n_all = (int64_t)M * N;
  if (i >= n_all) return;
  float s = 0.f;
  for (int z = 0; z < splits; ++z) s += part[(int64_t)z * n_all + i];
  const int64_t m = i / N;
  C[m * ldc + (i - m * N)] = static_cast<bf16>(scale * s);
}

// Low-rank product C (op)= X Y^T with a short k (the LoRA up-projection, k = rank or a few ranks):
// X [M, K], Y [N, K] row-major, K a multiple of 8.  Workgroup tile 128 x 128, four waves of
// 64 x 64 (2 x 2 blocks of 32 x 32); fragments straight from global memory.
//   MODE 0: C bf16 = acc;   MODE 1: C bf16 = bf16(C + acc);   MODE 2: C fp32 += acc;   MODE 3: C fp32 = acc
template <int MODE>
__global__ __launch_bounds__(256) void lowrank_kernel(const bf16* __restrict__ X, int64_t ldx,
                                                      const bf16* __restrict__ Y, int64_t ldy, int M, int N, int K,
                                                      void* C, int64_t ldc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 31, lh = lane >> 5;
  const int m0 = blockIdx.y * 128 + (wave >> 1) * 64, n0 = blockIdx.x * 128 + (wave & 1) * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const bf16* xp[2];
  const bf16* yp[2];
  bool yok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xp[i] = X + (int64_t)min(m0 + 32 * i + lr, M - 1) * ldx + lh * 8;
    const int n = n0 + 32 * i + lr;
    yok[i] = n < N;
    yp[i] = Y + (int64_t)(yok[i] ? n : 0) * ldy + lh * 8;
  }
  const bf16x8 zero = {};
  for (int k = 0; k < K; k += 16) {
    const bool kok = k + lh * 8 < K;              // K a multiple of 8: the last half k-step may be empty
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = kok ? *(const bf16x8*)(xp[i] + k) : zero;
      b[i] = (kok && yok[i]) ? *(const bf16x8*)(yp[i] + k) : zero;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * i + (e >> 2) * 8 + lh * 4 + (e & 3);
        if (m >= M) continue;
        if (MODE == 2) {
          float* c = (float*)C + (int64_t)m * ldc + n;
          *c += acc[i][j][e];
        } else if (MODE == 3) {
          ((float*)C)[(int64_t)m * ldc + n] = acc[i][j][e];
        } else {
          bf16* c = (bf16*)C + (int64_t)m * ldc + n;
          *c = static_cast<bf16>(MODE == 1 ? static_cast<float>(*c) + acc[i][j][e] : acc[i][j][e]);
        }
      }
    }
}

}  // namespace

hipError_t gemm_lowrank(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, int N, int K, void* C,
                        int64_t ldc, int mode, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % 8 || ldx % 8 || ldy % 8) return hipErrorInvalidValue;
  const dim3 grid((N + 127) / 128, (M + 127) / 128);
  if (mode == 0) hipLaunchKernelGGL(lowrank_kernel<0>, grid, dim3(256), 0, s, X, ldx, Y, ldy, M, N, K, C, ldc);
  else if (mode == 1) hipLaunchKernelGGL(lowrank_kernel<1>, grid, dim3(256), 0, s, X, ldx, Y, ldy, M, N, K, C, ldc);
  else if (mode == 2) hipLaunchKernelGGL(lowrank_kernel<2>, grid, dim3(256), 0, s, X, ldx, Y, ldy, M, N, K, C, ldc);
  else if (mode == 3) hipLaunchKernelGGL(lowrank_kernel<3>, grid, dim3(256), 0, s, X, ldx, Y, ldy, M, N, K, C, ldc);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

int skinny_splits(int M, int K) {
  const int groups_m = (M + 31) / 32;
  int splits = (2048 + groups_m - 1) / groups_m;
  splits = std::min(splits, std::max(1, K / 256));
  return std::min(std::max(splits, 1), SKINNY_MAX_SPLITS);
}

hipError_t gemm_skinny(const GemmParams& p, float* part, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.N > 128 || p.K % 64 || p.K <= 0) return hipErrorInvalidValue;
  const bool seg = p.bmode == 2;
  const bf16* B0 = (const bf16*)(seg ? p.Bs[0] : p.B);
  const bf16* B1 = seg ? (const bf16*)p.Bs[1] : B0;
  const bf16* B2 = seg ? (const bf16*)p.Bs[2] : B0;
  const int seg_rows = seg ? p.seg_rows : 128;
  const int splits = skinny_splits(p.M, p.K);
  const int kchunk = (p.K / 64 + splits - 1) / splits * 64;
  const int nz = (p.K + kchunk - 1) / kchunk;
  const dim3 grid((p.M + 127) / 128, nz);
  const int nb = (p.N + 31) / 32;
#define PSF_SK(NBV)                                                                                      \
  hipLaunchKernelGGL(skinny_kernel<NBV>, grid, dim3(256), 0, s, (const bf16*)p.A, p.lda, B0, B1, B2, p.ldb, \
                     seg_rows, p.M, p.N, p.K, kchunk, part)
  if (nb == 1) PSF_SK(1);
  else if (nb == 2) PSF_SK(2);
  else if (nb == 3) PSF_SK(3);
  else PSF_SK(4);
#undef PSF_SK
  const int64_t n = (int64_t)p.M * p.N;
  hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)part, nz,
                     p.M, p.N, p.scale, (bf16*)p.C, p.ldc);
  return hipGetLastError();
}

hipError_t gemm_skinny_diag(const bf16* A, int64_t lda, int M, const bf16* const* B, const int* outs, int ns, float scale,
                           bf16* C, int64_t ldc, float* part, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (ns < 1 || ns > 3) return hipErrorInvalidValue;
  int K = 0;
  for (int i = 0; i < ns; ++i) {
    if (outs[i] <= 0 || outs[i] % 64) return hipErrorInvalidValue;
    K += outs[i];
  }
  const int kb1 = outs[0], kb2 = ns > 2 ? outs[0] + outs[1] : K;
  const int N = 32 * ns;
  const int splits = skinny_splits(M, K);
  const int kchunk = (K / 64 + splits - 1) / splits * 64;
  const int nz = (K + kchunk - 1) / kchunk;
  const dim3 grid((M + 127) / 128, nz);
  const bf16* B1 = ns > 1 ? B[1] : B[0];
  const bf16* B2 = ns > 2 ? B[2] : B[0];
  const int64_t l1 = ns > 1 ? outs[1] : outs[0], l2 = ns > 2 ? outs[2] : outs[0];
  if (ns == 1)
    hipLaunchKernelGGL((skinny_kernel<1, true>), grid, dim3(256), 0, s, A, lda, B[0], B1, B2, (int64_t)outs[0], 32, M, N, K,
                       kchunk, part, l1, l2, kb1, kb2);
  else if (ns == 2)
    hipLaunchKernelGGL((skinny_kernel<2, true>), grid, dim3(256), 0, s, A, lda, B[0], B1, B2, (int64_t)outs[0], 32, M, N, K,
                       kchunk, part, l1, l2, kb1, kb2);
  else
    hipLaunchKernelGGL((skinny_kernel<3, true>), grid, dim3(256), 0, s, A, lda, B[0], B1, B2, (int64_t)outs[0], 32, M, N, K,
                       kchunk, part, l1, l2, kb1, kb2);
  const int64_t n = (int64_t)M * N;
  hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)part, nz, M, N,
                     scale, C, ldc);
  return hipGetLastError();
}

}  // namespace psf
