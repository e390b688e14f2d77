// Host-visible description of one GEMM launch: C = epilogue(A B^T).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace psf {

enum GemmEpi {
  EPI_STORE = 0,       // C[m,n] = acc
  EPI_RESID = 1,       // C[m,n] = R[m,n] + acc          (R may alias C)
  EPI_SWIGLU = 2,      // C[m,j] = silu(gate_j) * up_j   (B rows interleaved gate/up by 32)
  EPI_F32_IMG = 3,     // fp32 unpatchify store: token m, feature n -> image pixel
  EPI_BIAS_BCAST = 4,  // C[(i*n_bcast+br)*rows_per + r, n] = acc + bias[i, n]
  EPI_SCALED = 5,      // C[m,n] = scale * acc
  EPI_RESID_TO_F32 = 6,    // C (fp32) = R (bf16) + acc     mid-block residual kept in fp32
  EPI_RESID_FROM_F32 = 7,  // C (bf16) = R (fp32) + acc     block output
  EPI_RESID_F32 = 8,       // C (fp32) = R (fp32) + acc     fp32 residual stream (may alias)
  EPI_BIAS_BCAST_F32 = 9,  // as EPI_BIAS_BCAST with an fp32 C
  EPI_PARTIAL_F32 = 10,    // C (fp32) = acc over one k-range of a split-K launch (C + split * M * ldc)
};

struct GemmParams {
  const void* A; int64_t lda;        // [M, K] row-major (K contiguous)
  const int* a_rows;                 // optional row gather (logical row -> physical row), or null
  const void* B; int64_t ldb;        // [N, K] row-major: C = A B^T
  int M, N, K;                       // N = B rows consumed (for SWIGLU: 2 x output columns)
  int bmode;                         // 0 plain, 1 swiglu interleave, 2 segmented (Bs[])
  int swiglu_I;                      // bmode 1: row offset of the up half in B
  const void* Bs[3]; int seg_rows;   // bmode 2: B = concat(Bs[0], Bs[1], Bs[2]), each seg_rows rows
  // K extension (unmerged LoRA up-projection folded into the same accumulators):
  // acc += X[m, :xk] . XB_site(n)[n - site_start, :] over the site's xr-wide k range.
  const void* X; int64_t ldx; int xk;
  const void* XB[3]; int xr; int xsite_end[3]; int xoff[3];  // site s: columns [xoff[s], xoff[s]+xr) of X
  // epilogue
  void* C; int64_t ldc;
  const void* R; int64_t ldr;
  float scale;
  const float* bias; int rows_per; int n_bcast;
  int img_H, img_W;                  // EPI_F32_IMG: images of img_H x img_W pixels, rows_per tokens each
  // grouped GEMM (MoE experts): tiles[3*t] = expert, first row, rows
  const int* tiles; int max_tiles; int64_t b_expert_stride;
  // split-K for grids that leave CUs idle (few row tiles): scratch for ksplit fp32 partial
  // products; without it (part == nullptr) the GEMM runs unsplit
  int ksplit; float* part; size_t part_floats;
};

// Launchers (return hipError_t of the launch).
hipError_t gemm_bf16(const GemmParams& p, int epi, hipStream_t s);
hipError_t gemm_bf16_grouped(const GemmParams& p, int epi, int n_col_tiles, hipStream_t s);
hipError_t gemm_f32(const GemmParams& p, int epi, hipStream_t s);
// True when gemm_bf16 runs a K-extended launch (p.X set) on the 32-deep ring kernel: extension
// width, rank and site column offsets multiples of 32, site boundaries multiples of 16, a plain B
// (or the interleaved gate/up B with the SwiGLU epilogue).
bool k32_ext_ok(const GemmParams& p, int epi);

}  // namespace psf
