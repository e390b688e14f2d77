// bf16 MFMA GEMM family for the gen block's projections (QKV, O, gate/up, down, patch
// embed, out head, LoRA, expert GEMMs) on gfx950, plus a plain fp32 GEMM for fp32 runs.
//
// C = epilogue(A B^T), A [M, K] and B [N, K] both K-contiguous (Linear weights are
// [out, in]), fp32 accumulation.  Tile 256 x 256 x 64, 4 waves in a 2 x 2 grid, each
// wave owning 128 x 128 outputs as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16.  Global
// tiles are staged through registers into LDS (double buffered); LDS rows are 64 bf16
// (128 B) with 16-byte chunks XOR-swizzled by (row & 7) so that MFMA fragment reads
// (8 rows per LDS cycle) and chunk writes are bank-conflict free.
#include "common.h"
#include "gemm.h"
#include <cstdlib>

namespace psf {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int STAGE_BYTES = (BM + BN) * BK * 2;  // 64 KiB per stage
// The 64-deep kernel keeps its operands apart in LDS: two A stages, then three B stages (the
// weights, whose loads come from HBM and have the longer latency, run two k-tiles ahead).
constexpr int FAST_ASZ = BM * BK * 2;             // 32 KiB
constexpr int FAST_BSZ = BN * BK * 2;             // 32 KiB
constexpr int FAST_LDS = 2 * FAST_ASZ + 3 * FAST_BSZ;   // 160 KiB

DEVI int swz(int row, int chunk) { return row * (BK * 2) + ((chunk ^ (row & 7)) << 4); }

// Row pointer of B-tile row r (tile column base n0) for the three B modes.
DEVI const bf16* b_row_ptr(const GemmParams& p, const bf16* Bbase, int tn, int r, int& valid) {
  if (p.bmode == 1) {
    // 32-column blocks alternate gate / up: block nb covers output columns
    // tn*128 + (nb/2)*32 + [0, 32).
    const int nb = r >> 5;
    const int j = tn * (BN / 2) + (nb >> 1) * 32 + (r & 31);
    valid = j < p.swiglu_I;
    const int jj = valid ? j : 0;
    return Bbase + (int64_t)((nb & 1) ? p.swiglu_I + jj : jj) * p.ldb;
  }
  int n = tn * BN + r;
  valid = n < p.N;
  if (!valid) n = 0;
  if (p.bmode == 2) {
    const int s = n / p.seg_rows;
    return (const bf16*)p.Bs[s] + (int64_t)(n - s * p.seg_rows) * p.ldb;
  }
  return Bbase + (int64_t)n * p.ldb;
}

// B-row -> output column used by the K extension's site lookup.
DEVI int b_row_outcol(const GemmParams& p, int tn, int r) {
  if (p.bmode == 1) {
    const int nb = r >> 5;
    const int j = tn * (BN / 2) + (nb >> 1) * 32 + (r & 31);
    return (nb & 1) ? p.swiglu_I + j : j;   // gate columns first, then up columns
  }
  return tn * BN + r;
}

template <int EPI>
DEVI void store_one(const GemmParams& p, int row, int col, float v) {
  if (EPI == EPI_STORE) {
    ((bf16*)p.C)[(int64_t)row * p.ldc + col] = from_f<bf16>(v);
  } else if (EPI == EPI_SCALED) {
    ((bf16*)p.C)[(int64_t)row * p.ldc + col] = from_f<bf16>(v * p.scale);
  } else if (EPI == EPI_RESID) {
    const float r = to_f(((const bf16*)p.R)[(int64_t)row * p.ldr + col]);
    ((bf16*)p.C)[(int64_t)row * p.ldc + col] = from_f<bf16>(r + v);
  } else if (EPI == EPI_RESID_TO_F32) {
    const float r = to_f(((const bf16*)p.R)[(int64_t)row * p.ldr + col]);
    ((float*)p.C)[(int64_t)row * p.ldc + col] = r + v;
  } else if (EPI == EPI_RESID_FROM_F32) {
    const float r = ((const float*)p.R)[(int64_t)row * p.ldr + col];
    ((bf16*)p.C)[(int64_t)row * p.ldc + col] = from_f<bf16>(r + v);
  } else if (EPI == EPI_RESID_F32) {
    const float r = ((const float*)p.R)[(int64_t)row * p.ldr + col];
    ((float*)p.C)[(int64_t)row * p.ldc + col] = r + v;
  } else if (EPI == EPI_BIAS_BCAST_F32) {
    const int img = row / p.rows_per, t = row - img * p.rows_per;
    const float x = v + p.bias[(int64_t)img * p.N + col];
    for (int br = 0; br < p.n_bcast; ++br)
      ((float*)p.C)[((int64_t)(img * p.n_bcast + br) * p.rows_per + t) * p.ldc + col] = x;
  } else if (EPI == EPI_F32_IMG) {
    // token row -> (image, patch row, patch col); feature col -> (channel, iy, ix)
    const int img = row / p.rows_per, t = row - img * p.rows_per;
    const int pw = p.img_W >> 5;
    const int py = t / pw, px = t - py * pw;
    const int c = col >> 10, iy = (col >> 5) & 31, ix = col & 31;
    float* out = (float*)p.C;
    out[(((int64_t)img * 3 + c) * p.img_H + py * 32 + iy) * p.img_W + px * 32 + ix] = v;
  } else if (EPI == EPI_BIAS_BCAST) {
    const int img = row / p.rows_per, t = row - img * p.rows_per;
    const float x = v + p.bias[(int64_t)img * p.N + col];
    const bf16 xb = from_f<bf16>(x);
    for (int br = 0; br < p.n_bcast; ++br)
      ((bf16*)p.C)[((int64_t)(img * p.n_bcast + br) * p.rows_per + t) * p.ldc + col] = xb;
  }
}

template <int EPI, bool GROUPED, bool EXT>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(GemmParams p, int n_col_tiles) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile coordinates
  int tm, tn, row0, rows, expert = 0;
  if (GROUPED) {
    const int t = blockIdx.x / n_col_tiles;
    tn = blockIdx.x - t * n_col_tiles;
    expert = p.tiles[3 * t];
    if (expert < 0) return;                      // unused slot of the tile table
    row0 = p.tiles[3 * t + 1];
    rows = p.tiles[3 * t + 2];
    tm = 0;
  } else {
    const int n_m = (p.M + BM - 1) / BM;
    const int n_t = n_m * n_col_tiles;
    const int id = xcd_remap(blockIdx.x, n_t);
    // grouped ordering: 8 m-tiles walk together so concurrently running tiles share A and B panels
    const int GROUP = 8;
    const int per_group = GROUP * n_col_tiles;
    const int g = id / per_group;
    const int first_m = g * GROUP;
    const int gsz = min(n_m - first_m, GROUP);
    const int r_in = id - g * per_group;
    tm = first_m + r_in % gsz;
    tn = r_in / gsz;
    row0 = tm * BM;
    rows = min(BM, p.M - row0);
  }
  const bf16* Bbase = (const bf16*)p.B + (GROUPED ? (int64_t)expert * p.b_expert_stride : 0);

  // ---- per-thread load rows: chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int chunk = tid & 7;
  const bf16* arow[8];
  const bf16* brow[8];
  int bvalid_mask = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int rr = min(r, rows - 1);
    int prow = row0 + rr;
    if (p.a_rows) prow = p.a_rows[prow];
    arow[i] = (const bf16*)p.A + (int64_t)prow * p.lda + chunk * 8;
    int v;
    brow[i] = b_row_ptr(p, Bbase, tn, r, v) + chunk * 8;
    bvalid_mask |= v << i;
  }
  const int KT0 = p.K / BK;
  const int KT = KT0 + (EXT ? (p.xk + BK - 1) / BK : 0);

  u32x4 ra[8], rb[8];
  auto load = [&](int kt) {
    if (!EXT || kt < KT0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ra[i] = *(const u32x4*)(arow[i] + kt * BK);
        rb[i] = *(const u32x4*)(brow[i] + kt * BK);
      }
    } else {
      // LoRA extension: k in [0, xk) of X and of the site's up-projection rows
      const int k = (kt - KT0) * BK + chunk * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int rr = min(r, rows - 1);
        int prow = row0 + rr;
        ra[i] = (k < p.xk) ? *(const u32x4*)((const bf16*)p.X + (int64_t)prow * p.ldx + k) : u32x4{0, 0, 0, 0};
        const int col = b_row_outcol(p, tn, r);
        const int s = col < p.xsite_end[0] ? 0 : (col < p.xsite_end[1] ? 1 : 2);
        const int start = s == 0 ? 0 : p.xsite_end[s - 1];
        const int kk = k - p.xoff[s];
        const bool ok = ((bvalid_mask >> i) & 1) && p.XB[s] != nullptr && kk >= 0 && kk < p.xr;
        rb[i] = ok ? *(const u32x4*)((const bf16*)p.XB[s] + (int64_t)(col - start) * p.xr + kk) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store = [&](int stage) {
    char* As = smem + stage * STAGE_BYTES;
    char* Bs = As + BM * BK * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *(u32x4*)(As + swz(r, chunk)) = ra[i];
      *(u32x4*)(Bs + swz(r, chunk)) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  const int lr = lane & 31, lh = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load(kt + 1);
    const char* As = smem + cur * STAGE_BYTES;
    const char* Bs = As + BM * BK * 2;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) af[mb] = *(const bf16x8*)(As + swz(wm * 128 + mb * 32 + lr, ks * 2 + lh));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bfr[nb] = *(const bf16x8*)(Bs + swz(wn * 128 + nb * 32 + lr, ks * 2 + lh));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (kt + 1 < KT) store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Lane holds column (lane & 31) and rows (e/4)*8 + (lane/32)*4 + e%4 of each block.
  const int orow0 = (GROUPED ? 0 : 0);
  (void)orow0;
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int j = tn * (BN / 2) + (wn * 2 + pr) * 32 + lr;
        if (j >= p.swiglu_I) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = wm * 128 + mb * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
          if (r >= rows) continue;
          const float g = acc[mb][2 * pr][e], u = acc[mb][2 * pr + 1][e];
          ((bf16*)p.C)[(int64_t)(row0 + r) * p.ldc + j] = from_f<bf16>(silu_f(g) * u);
        }
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = tn * BN + wn * 128 + nb * 32 + lr;
        if (col >= p.N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = wm * 128 + mb * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
          if (r >= rows) continue;
          store_one<EPI>(p, row0 + r, col, acc[mb][nb][e]);
        }
      }
  }
}

// ------------------------------------------------------------------ fast path
// Same 256 x 256 x 64 tile and epilogues as gemm_bf16_kernel, but the global->LDS copy uses
// gfx950's buffer loads straight into LDS (16 bytes per lane): no staging VGPRs and no ds_write
// instructions, which leaves registers for the MFMA fragments; the products are
// v_mfma_f32_16x16x32_bf16 blocks (one instruction per 32-deep half of the tile).  One load
// instruction of a wave fills 8 consecutive LDS rows (1 KiB); lane l lands at base + 16 l,
// i.e. row l/8, physical chunk l%8, so it fetches logical chunk (l%8) ^ (l/8) of its row and
// the XOR swizzle comes out of the address arithmetic.  Buffer resources cover only the
// tile's valid rows, so rows past M (or past N) read as zero.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

DEVI __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS at lds + 16*lane (kept out of the kernel
// body: the builtin inside a kernel-local lambda stops clang from emitting the host stub).
DEVI void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// Epilogue of 16 consecutive columns [col0, col0+16) of one output row.  Vector path when
// all 16 columns are valid (col0 is a multiple of 16; leading dimensions are multiples of 8).
template <int EPI>
DEVI void epi_row16(const GemmParams& p, int row, int col0, int ncols, float* v) {
  const bool full = col0 + 16 <= ncols;
  if (EPI == EPI_F32_IMG) {
    const int img = row / p.rows_per, t = row - img * p.rows_per;
    const int pw = p.img_W >> 5;
    const int py = t / pw, px = t - py * pw;
    const int c = col0 >> 10, iy = (col0 >> 5) & 31, ix = col0 & 31;
    float* out = (float*)p.C + (((int64_t)img * 3 + c) * p.img_H + py * 32 + iy) * p.img_W + px * 32 + ix;
    if (full) {
#pragma unroll
      for (int q = 0; q < 4; ++q) *(float4*)(out + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
      for (int j = 0; j < 16 && col0 + j < ncols; ++j) out[j] = v[j];
    }
    return;
  }
  if (EPI == EPI_BIAS_BCAST || EPI == EPI_BIAS_BCAST_F32) {
    const int img = row / p.rows_per, t = row - img * p.rows_per;
    const float* bias = p.bias + (int64_t)img * p.N + col0;
    for (int j = 0; j < 16; ++j) v[j] += (col0 + j < ncols) ? bias[j] : 0.f;
    for (int br = 0; br < p.n_bcast; ++br) {
      const int64_t o = ((int64_t)(img * p.n_bcast + br) * p.rows_per + t) * p.ldc + col0;
      if (EPI == EPI_BIAS_BCAST_F32) {
        float* C = (float*)p.C + o;
        if (full) {
#pragma unroll
          for (int q = 0; q < 4; ++q) *(float4*)(C + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        } else {
          for (int j = 0; j < 16 && col0 + j < ncols; ++j) C[j] = v[j];
        }
      } else {
        bf16* C = (bf16*)p.C + o;
        if (full) {
          bf16x8 a, b;
#pragma unroll
          for (int j = 0; j < 8; ++j) { a[j] = from_f<bf16>(v[j]); b[j] = from_f<bf16>(v[8 + j]); }
          *(bf16x8*)C = a;
          *(bf16x8*)(C + 8) = b;
        } else {
          for (int j = 0; j < 16 && col0 + j < ncols; ++j) C[j] = from_f<bf16>(v[j]);
        }
      }
    }
    return;
  }
  // residual input
  if (EPI == EPI_RESID || EPI == EPI_RESID_TO_F32) {
    const bf16* R = (const bf16*)p.R + (int64_t)row * p.ldr + col0;
    if (full) {
      const bf16x8 a = *(const bf16x8*)R, b = *(const bf16x8*)(R + 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) { v[j] += static_cast<float>(a[j]); v[8 + j] += static_cast<float>(b[j]); }
    } else {
      for (int j = 0; j < 16 && col0 + j < ncols; ++j) v[j] += to_f(R[j]);
    }
  } else if (EPI == EPI_RESID_FROM_F32 || EPI == EPI_RESID_F32) {
    const float* R = (const float*)p.R + (int64_t)row * p.ldr + col0;
    if (full) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *(const float4*)(R + 4 * q);
        v[4 * q] += f.x; v[4 * q + 1] += f.y; v[4 * q + 2] += f.z; v[4 * q + 3] += f.w;
      }
    } else {
      for (int j = 0; j < 16 && col0 + j < ncols; ++j) v[j] += R[j];
    }
  } else if (EPI == EPI_SCALED) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= p.scale;
  }
  // output
  if (EPI == EPI_RESID_TO_F32 || EPI == EPI_RESID_F32 || EPI == EPI_PARTIAL_F32) {
    float* C = (float*)p.C + (int64_t)row * p.ldc + col0;
    if (full) {
#pragma unroll
      for (int q = 0; q < 4; ++q) *(float4*)(C + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
      for (int j = 0; j < 16 && col0 + j < ncols; ++j) C[j] = v[j];
    }
  } else {
    bf16* C = (bf16*)p.C + (int64_t)row * p.ldc + col0;
    if (full) {
      bf16x8 a, b;
#pragma unroll
      for (int j = 0; j < 8; ++j) { a[j] = from_f<bf16>(v[j]); b[j] = from_f<bf16>(v[8 + j]); }
      *(bf16x8*)C = a;
      *(bf16x8*)(C + 8) = b;
    } else {
      for (int j = 0; j < 16 && col0 + j < ncols; ++j) C[j] = from_f<bf16>(v[j]);
    }
  }
}

// Epilogue of 4 consecutive columns [col0, col0+4) of one output row, straight from the
// accumulators (col0 is a multiple of 4; leading dimensions are multiples of 8, so the vector
// accesses are aligned).  Residual inputs come in through rin, loaded by the caller ahead of time.
template <int EPI>
DEVI void epi_row4_store(const GemmParams& p, int row, int col0, int ncols, const float* v) {
  const bool full = col0 + 4 <= ncols;
  if (EPI == EPI_F32_IMG) {
    const int img = row / p.rows_per, t = row - img * p.rows_per;
    const int pw = p.img_W >> 5;
    const int py = t / pw, px = t - py * pw;
    const int c = col0 >> 10, iy = (col0 >> 5) & 31, ix = col0 & 31;
    float* out = (float*)p.C + (((int64_t)img * 3 + c) * p.img_H + py * 32 + iy) * p.img_W + px * 32 + ix;
    if (full) *(float4*)out = make_float4(v[0], v[1], v[2], v[3]);
    else for (int j = 0; j < 4 && col0 + j < ncols; ++j) out[j] = v[j];
    return;
  }
  if (EPI == EPI_BIAS_BCAST || EPI == EPI_BIAS_BCAST_F32) {
    const int img = row / p.rows_per, t = row - img * p.rows_per;
    const float* bias = p.bias + (int64_t)img * p.N + col0;
    float x[4];
    for (int j = 0; j < 4; ++j) x[j] = v[j] + ((col0 + j < ncols) ? bias[j] : 0.f);
    for (int br = 0; br < p.n_bcast; ++br) {
      const int64_t o = ((int64_t)(img * p.n_bcast + br) * p.rows_per + t) * p.ldc + col0;
      if (EPI == EPI_BIAS_BCAST_F32) {
        float* C = (float*)p.C + o;
        if (full) *(float4*)C = make_float4(x[0], x[1], x[2], x[3]);
        else for (int j = 0; j < 4 && col0 + j < ncols; ++j) C[j] = x[j];
      } else {
        bf16* C = (bf16*)p.C + o;
        if (full) {
          bf16x4 a;
#pragma unroll
          for (int j = 0; j < 4; ++j) a[j] = from_f<bf16>(x[j]);
          *(bf16x4*)C = a;
        } else {
          for (int j = 0; j < 4 && col0 + j < ncols; ++j) C[j] = from_f<bf16>(x[j]);
        }
      }
    }
    return;
  }
  if (EPI == EPI_RESID_TO_F32 || EPI == EPI_RESID_F32 || EPI == EPI_PARTIAL_F32) {
    float* C = (float*)p.C + (int64_t)row * p.ldc + col0;
    if (full) *(float4*)C = make_float4(v[0], v[1], v[2], v[3]);
    else for (int j = 0; j < 4 && col0 + j < ncols; ++j) C[j] = v[j];
  } else {
    bf16* C = (bf16*)p.C + (int64_t)row * p.ldc + col0;
    if (full) {
      bf16x4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = from_f<bf16>(v[j]);
      *(bf16x4*)C = a;
    } else {
      for (int j = 0; j < 4 && col0 + j < ncols; ++j) C[j] = from_f<bf16>(v[j]);
    }
  }
}

// The residual term of 4 consecutive columns as fp32 (zero for epilogues without one).
template <int EPI>
DEVI f32x4 epi_row4_resid(const GemmParams& p, int row, int col0, int ncols) {
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  const bool full = col0 + 4 <= ncols;
  if (EPI == EPI_RESID || EPI == EPI_RESID_TO_F32) {
    const bf16* R = (const bf16*)p.R + (int64_t)row * p.ldr + col0;
    if (full) {
      const bf16x4 a = *(const bf16x4*)R;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = static_cast<float>(a[j]);
    } else {
      for (int j = 0; j < 4 && col0 + j < ncols; ++j) r[j] = to_f(R[j]);
    }
  } else if (EPI == EPI_RESID_FROM_F32 || EPI == EPI_RESID_F32) {
    const float* R = (const float*)p.R + (int64_t)row * p.ldr + col0;
    if (full) {
      const float4 f = *(const float4*)R;
      r[0] = f.x; r[1] = f.y; r[2] = f.z; r[3] = f.w;
    } else {
      for (int j = 0; j < 4 && col0 + j < ncols; ++j) r[j] = R[j];
    }
  }
  return r;
}

// Two 16-column blocks b, b+1 of one 16-row group, 4 columns of each per lane (lane l: columns
// 4 (l/16) .. +3 of both blocks), rounded to bf16.  Lanes of the 16-lane rows 1 and 3 hand their
// block-b columns to rows 0 and 2 and take those rows' block-(b+1) columns (v_permlane16_swap), so
// lane l ends with 8 consecutive columns: those of block b + (l/16) % 2 from column 8 ((l/16) / 2),
// i.e. at offset coff from block b's first column.  Every lane of the wave must execute it.
DEVI bf16x8 pair_to_8(const float* v0, const float* v1, int c16, int& coff) {
  bf16x4 a0, a1;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a0[e] = from_f<bf16>(v0[e]); a1[e] = from_f<bf16>(v1[e]); }
  u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(w0[i], w1[i], false, false);
    w0[i] = r[0];
    w1[i] = r[1];
  }
  coff = (c16 & 1) * 16 + (c16 >> 1) * 8;
  const u32x4 o = {w0[0], w0[1], w1[0], w1[1]};
  return __builtin_bit_cast(bf16x8, o);
}

// 8 consecutive bf16 columns [col, col+8) of row pointer C (at col), the valid ones below ncols.
DEVI void store8_bf16(bf16* C, int col, int ncols, bf16x8 o) {
  if (col + 8 <= ncols) {
    *(bf16x8*)C = o;
  } else {
    for (int j = 0; j < 8 && col + j < ncols; ++j) C[j] = o[j];
  }
}

template <int EPI, bool GROUPED, bool GATHER, int NW, bool EXT = false>
__global__ __launch_bounds__(64 * NW, 1) void gemm_fast_kernel(GemmParams p, int n_col_tiles) {
  // NW = 4: 2 x 2 waves of 128 x 128 (one wave per SIMD); NW = 8: 2 x 4 waves of 128 x 64 (two
  // waves per SIMD, so one wave's DMA issue or barrier wait is covered by the other's MFMAs).
  // Each wave tile is a grid of 16 x 16 blocks of v_mfma_f32_16x16x32_bf16.
  // EXT: the LoRA up-projection as ceil(xk / 64) more k-tiles after the K / 64 of A and B: A rows
  // from X, B rows from the up-projection of the site that owns each 8-row group of B; a 16-byte
  // chunk outside X's xk columns or outside the site's xr-wide slice of them loads as zeros.
  constexpr int WN = NW / 2;                 // waves along n
  constexpr int NBW = (BN / WN) / 32;        // 32-column MFMA blocks per wave (4 or 2)
  constexpr int GPW = 32 / NW;               // 8-row load groups per wave per operand
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  int tn, row0, rows, expert = 0, split = 0;
  if (GROUPED) {
    const int t = blockIdx.x / n_col_tiles;
    tn = blockIdx.x - t * n_col_tiles;
    expert = p.tiles[3 * t];
    if (expert < 0) return;
    row0 = p.tiles[3 * t + 1];
    rows = p.tiles[3 * t + 2];
  } else {
    const int n_m = (p.M + BM - 1) / BM;
    const int n_t = n_m * n_col_tiles;
    const int idall = xcd_remap(blockIdx.x, n_t * max(p.ksplit, 1));
    split = idall / n_t;                               // k-range of a split-K launch (else 0)
    const int id = idall - split * n_t;
    const int GROUP = 8;
    const int per_group = GROUP * n_col_tiles;
    const int g = id / per_group;
    const int first_m = g * GROUP;
    const int gsz = min(n_m - first_m, GROUP);
    const int r_in = id - g * per_group;
    tn = r_in / gsz;
    row0 = (first_m + r_in % gsz) * BM;
    rows = min(BM, p.M - row0);
  }
  // LDS rows are 128 B; ds_read_b128 serves 16 lanes per cycle over a 256 B (64-bank) window, so a
  // row pair shares a window and chunk c of row r sits at c ^ ((r >> 1) & 7): the 16 rows read
  // together land on 16 distinct (half, chunk) slots.  A group of 8 rows starting at a multiple of
  // 8 has ((r >> 1) & 7) = 4 (g & 1) + (lrow >> 1) for group index g.
  const int lrow = lane >> 3;                       // row within a group of 8
  const int lch0 = (lane & 7) ^ (lrow >> 1);        // logical chunk fetched, even groups
  const int lch1 = (lane & 7) ^ (4 + (lrow >> 1));  // odd groups
  const uint32_t lda2 = (uint32_t)p.lda * 2, ldb2 = (uint32_t)p.ldb * 2;

  // A operand
  __amdgpu_buffer_rsrc_t ra;
  uint32_t avoff[GATHER ? GPW : 2];
  if (GATHER) {
    ra = make_rsrc(p.A, 0x7fffffff);
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int r = (wave * GPW + i) * 8 + lrow;
      avoff[i] = (uint32_t)p.a_rows[row0 + min(r, rows - 1)] * lda2 + (((wave * GPW + i) & 1) ? lch1 : lch0) * 16;
    }
  } else {
    ra = make_rsrc((const bf16*)p.A + (int64_t)row0 * p.lda, (uint32_t)rows * lda2);
    avoff[0] = lrow * lda2 + lch0 * 16;
    avoff[1] = lrow * lda2 + lch1 * 16;
  }
  // B operand
  const bf16* Bexp = (const bf16*)p.B + (GROUPED ? (int64_t)expert * p.b_expert_stride : 0);
  __amdgpu_buffer_rsrc_t rb;
  uint32_t bsoff[GPW];
  if (p.bmode == 1) {
    rb = make_rsrc(Bexp, (uint32_t)(2 * p.swiglu_I) * ldb2);
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int r0 = (wave * GPW + i) * 8;
      const int nb = r0 >> 5;
      const int brow = ((nb & 1) ? p.swiglu_I : 0) + tn * (BN / 2) + (nb >> 1) * 32 + (r0 & 31);
      bsoff[i] = (uint32_t)brow * ldb2;
    }
  } else {
    const int nvalid = min(BN, p.N - tn * BN);
    rb = make_rsrc(Bexp + (int64_t)tn * BN * p.ldb, (uint32_t)nvalid * ldb2);
#pragma unroll
    for (int i = 0; i < GPW; ++i) bsoff[i] = (uint32_t)((wave * GPW + i) * 8) * ldb2;
  }
  const uint32_t bvoff0 = lrow * ldb2 + lch0 * 16, bvoff1 = lrow * ldb2 + lch1 * 16;

  const int KTM = p.K / BK / max(p.ksplit, 1);  // k-tiles of A B^T in this launch's k-range
  const int KT = KTM + (EXT ? (p.xk + BK - 1) / BK : 0);
  const uint32_t kofs = (uint32_t)(split * KTM) * (BK * 2);   // byte offset of the k-range
  if (EPI == EPI_PARTIAL_F32) p.C = (float*)p.C + (int64_t)split * p.M * p.ldc;
  // K extension: X rows of the tile, and per 8-row group of B its site's up-projection rows
  __amdgpu_buffer_rsrc_t rx, rbx[EXT ? GPW : 1];
  uint32_t ldx2 = 0;
  int bx_lo[EXT ? GPW : 1], bx_hi[EXT ? GPW : 1];
  if (EXT) {
    ldx2 = (uint32_t)p.ldx * 2;
    rx = make_rsrc((const bf16*)p.X + (int64_t)row0 * p.ldx, (uint32_t)rows * ldx2);
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int col = b_row_outcol(p, tn, (wave * GPW + i) * 8);
      const int site = col < p.xsite_end[0] ? 0 : (col < p.xsite_end[1] ? 1 : 2);
      const int start = site == 0 ? 0 : p.xsite_end[site - 1];
      const int nrow = min(8, min(p.xsite_end[site], (p.bmode == 1 ? 2 * p.swiglu_I : p.N)) - col);
      const bf16* xb = (const bf16*)p.XB[site];
      rbx[i] = make_rsrc(xb ? xb + (int64_t)(col - start) * p.xr : p.X, (xb && nrow > 0) ? (uint32_t)nrow * p.xr * 2 : 0u);
      bx_lo[i] = p.xoff[site];                     // X columns [lo, hi) belong to this site
      bx_hi[i] = p.xoff[site] + p.xr;
    }
  }

  // DMA of k-tile kt: A into A stage sa, B into B stage sb (each GPW loads per wave)
  auto issue_a = [&](int kt, int sa) {
    char* As = smem + sa * FAST_ASZ;
    if (EXT && kt >= KTM) {
      const int k0 = (kt - KTM) * BK;              // X column of this extension k-tile
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int grp = wave * GPW + i;
        const int c = k0 + ((i & 1) ? lch1 : lch0) * 8;   // X column of this lane's chunk
        dma16(rx, As + grp * 1024, c < p.xk ? lrow * ldx2 + (uint32_t)c * 2 : 0x40000000u, grp * 8 * ldx2);
      }
      return;
    }
    const uint32_t kb = (uint32_t)kt * (BK * 2) + kofs;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int grp = wave * GPW + i;
      if (GATHER)
        dma16(ra, As + grp * 1024, avoff[i], kb);
      else
        dma16(ra, As + grp * 1024, avoff[i & 1], grp * 8 * lda2 + kb);
    }
  };
  auto issue_b = [&](int kt, int sb) {
    char* Bs = smem + 2 * FAST_ASZ + sb * FAST_BSZ;
    if (EXT && kt >= KTM) {
      const int k0 = (kt - KTM) * BK;
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int grp = wave * GPW + i;
        const int c = k0 + ((i & 1) ? lch1 : lch0) * 8;
        const bool in = c >= bx_lo[i] && c < bx_hi[i];
        dma16(rbx[i], Bs + grp * 1024, in ? (uint32_t)(lrow * p.xr + c - bx_lo[i]) * 2 : 0x40000000u, 0);
      }
      return;
    }
    const uint32_t kb = (uint32_t)kt * (BK * 2) + kofs;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int grp = wave * GPW + i;
      dma16(rb, Bs + grp * 1024, (i & 1) ? bvoff1 : bvoff0, bsoff[i] + kb);
    }
  };

  constexpr int NB16 = 2 * NBW;               // 16-column MFMA blocks per wave (8 or 4)
  f32x4 acc[8][NB16];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < NB16; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[a][b][e] = 0.f;

  // 16x16x32 fragments (v_mfma_f32_16x16x32_bf16): lane l holds row l % 16 of a 16-row block and
  // logical chunk 4 ks + l / 16 of the 32-deep half ks of the 64-deep tile.  The B fragment goes
  // in as the instruction's first operand, so the product block comes out transposed: lane l
  // holds output row l % 16, columns 4 (l / 16) .. 4 (l / 16) + 3, which the epilogue stores
  // straight from the accumulators.
  const int r16 = lane & 15, c16 = lane >> 4;
  const int sw = (r16 >> 1) & 7;              // the same for all blocks: their rows differ by 16
  const int arow0 = (wm * 128 + r16) * (BK * 2), brow0 = (wn * (BN / WN) + r16) * (BK * 2);
  bf16x8 fal[4], fah[4], fb0[NB16], fb1[NB16];   // B fragments of the two 32-deep halves
  auto rd_a = [&](bf16x8 (&f)[4], int stage, int ks, int half) {
    const char* As = smem + stage * FAST_ASZ;
    const int ch = ((4 * ks + c16) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = *(const bf16x8*)(As + arow0 + (half * 4 + i) * 16 * (BK * 2) + ch);
  };
  auto rd_b = [&](bf16x8 (&f)[NB16], int stage, int ks) {   // stage: B stage 0-2
    const char* Bs = smem + 2 * FAST_ASZ + stage * FAST_BSZ;
    const int ch = ((4 * ks + c16) ^ sw) << 4;
#pragma unroll
    for (int nb = 0; nb < NB16; ++nb) f[nb] = *(const bf16x8*)(Bs + brow0 + nb * 16 * (BK * 2) + ch);
  };
  auto mma = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[NB16], int half) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb)
        acc[half * 4 + i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[nb], fa[i], acc[half * 4 + i][nb], 0, 0, 0);
  };
  // MFMAs in pairs, an LDS read after each of the first nds pairs
  auto interleave = [&](int nds) {
#pragma unroll
    for (int i = 0; i < 2 * NB16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      if (i < nds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
  };

  // Software pipeline over the four half-steps of a tile (32-deep half ks, wave-tile rows
  // 0-63 or 64-127): the A fragments of the next half-step are read while this one's MFMAs run;
  // the B fragments of the tile's second half (fb1) at its first half-step, those of the next
  // tile's first half (fb0) right after the last half-step's barrier, so no half-step starts by
  // waiting for LDS.  In the last half-step every wave waits for the loads of tile kt+1 and meets
  // the others, so tile kt+1 is complete and tile kt's A stage and B stage are free: the DMA of
  // A(kt+2) and of B(kt+3) goes into them.  A runs one tile ahead of its use, B (the weights, whose
  // loads carry most of the latency) two; the wait leaves the newest GPW loads, B(kt+2), in flight.
  constexpr int VM_N = GPW;
  constexpr int VM_B_IN_FLIGHT = (VM_N & 15) | ((VM_N >> 4) << 14) | (7 << 4) | (15 << 8);
  issue_a(0, 0);
  issue_b(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // tiles past the end reload the last tile into a stage nobody reads again, so every issue sends
  // the same number of loads and the vmcnt arithmetic holds throughout
  issue_a(min(1, KT - 1), 1);
  issue_b(min(1, KT - 1), 1);
  issue_b(min(2, KT - 1), 2);
  rd_a(fal, 0, 0, 0);
  rd_b(fb0, 0, 0);
  // every k-tile but the last: the body has no branches
  int kt = 0, sb = 0;                           // sb: B stage of tile kt (kt mod 3)
  for (; kt + 1 < KT; ++kt) {
    const int st = kt & 1;
    const int sb1 = sb == 2 ? 0 : sb + 1;
    // half-step 0: rows 0-63 of k 0-31
    __builtin_amdgcn_s_setprio(2);
    rd_a(fah, st, 0, 1);
    rd_b(fb1, sb, 1);
    mma(fal, fb0, 0);
    interleave(8);
    __builtin_amdgcn_sched_barrier(0);
    // half-step 1: rows 64-127 of k 0-31
    __builtin_amdgcn_s_setprio(1);
    rd_a(fal, st, 1, 0);
    mma(fah, fb0, 1);
    interleave(4);
    __builtin_amdgcn_sched_barrier(0);
    // half-step 2: rows 0-63 of k 32-63
    __builtin_amdgcn_s_setprio(0);
    rd_a(fah, st, 1, 1);
    mma(fal, fb1, 0);
    interleave(4);
    __builtin_amdgcn_sched_barrier(0);
    // half-step 3: rows 64-127 of k 32-63
    __builtin_amdgcn_s_setprio(3);
    __builtin_amdgcn_s_waitcnt(VM_B_IN_FLIGHT);
    __builtin_amdgcn_s_waitcnt(0xc07f);          // and this wave's LDS reads of tile kt
    __builtin_amdgcn_s_barrier();
    issue_a(min(kt + 2, KT - 1), st);
    issue_b(min(kt + 3, KT - 1), sb);
    rd_a(fal, st ^ 1, 0, 0);
    rd_b(fb0, sb1, 0);
    mma(fah, fb1, 1);
    interleave(8);
    __builtin_amdgcn_sched_barrier(0);
    sb = sb1;
  }
  {
    const int st = kt & 1;
    rd_a(fah, st, 0, 1);
    rd_b(fb1, sb, 1);
    mma(fal, fb0, 0);
    rd_a(fal, st, 1, 0);
    mma(fah, fb0, 1);
    rd_a(fah, st, 1, 1);
    mma(fal, fb1, 0);
    mma(fah, fb1, 1);
  }
  __builtin_amdgcn_s_setprio(0);

  // ---- epilogue straight from the accumulators: block (a, b) of lane l is output row
  // wm*128 + 16a + l%16, columns 16b + 4(l/16) .. +3 of the wave's slice.  bf16 outputs of block
  // pairs (b, b+1) are exchanged between lanes into 8 consecutive columns and stored as 16 bytes
  // per lane; fp32 outputs as 16 bytes per lane straight away.  The residual rows of block row a+1
  // are loaded before block row a is stored (R may alias C: the two never touch the same element);
  // rows past the tile's end read the last valid row and store nothing.
  __builtin_amdgcn_s_waitcnt(0);   // the trailing reloads of the last tile have landed in LDS
  if (EPI == EPI_SWIGLU) {
    // gate block b (b/2 even) and its up block b+2 hold the same output columns; gate blocks come
    // in pairs b, b+1 (b even)
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int r = wm * 128 + a * 16 + r16;
      const bool rok = r < rows;
      const int row = row0 + r;
#pragma unroll
      for (int b = 0; b < NB16; b += 2) {
        if ((b >> 1) & 1) continue;
        const int colp = tn * (BN / 2) + ((wn * NBW + (b >> 1)) >> 1) * 32;   // first column of the pair
        float v[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = colp + h * 16 + 4 * c16;
          float u[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[h][e] = acc[a][b + h][e]; u[e] = acc[a][b + h + 2][e]; }
          // optional bf16 terms added before the activation (the LoRA up-projection): R holds the
          // gate term at column j and the up term at column swiglu_I + j
          if (p.R && rok) {
            const bf16* rg = (const bf16*)p.R + (int64_t)row * p.ldr + col;
            const bf16* ru = rg + p.swiglu_I;
            if (col + 4 <= p.swiglu_I) {
              const bf16x4 ga = *(const bf16x4*)rg, ua = *(const bf16x4*)ru;
#pragma unroll
              for (int e = 0; e < 4; ++e) { v[h][e] += static_cast<float>(ga[e]); u[e] += static_cast<float>(ua[e]); }
            } else {
              for (int e = 0; e < 4 && col + e < p.swiglu_I; ++e) {
                v[h][e] += static_cast<float>(rg[e]);
                u[e] += static_cast<float>(ru[e]);
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) v[h][e] = silu_f(v[h][e]) * u[e];
        }
        int coff;
        const bf16x8 o = pair_to_8(v[0], v[1], c16, coff);
        if (rok) store8_bf16((bf16*)p.C + (int64_t)row * p.ldc + colp + coff, colp + coff, p.swiglu_I, o);
      }
    }
  } else {
    constexpr bool HAS_R = EPI == EPI_RESID || EPI == EPI_RESID_TO_F32 || EPI == EPI_RESID_FROM_F32 ||
                           EPI == EPI_RESID_F32;
    constexpr bool PAIR = EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_SCALED || EPI == EPI_RESID_FROM_F32;
    const int colw = tn * BN + wn * (BN / WN) + 4 * c16;
    f32x4 rn[NB16];
    auto load_r = [&](int a) {
      const int row = row0 + min(wm * 128 + a * 16 + r16, rows - 1);
#pragma unroll
      for (int b = 0; b < NB16; ++b) rn[b] = epi_row4_resid<EPI>(p, row, colw + 16 * b, p.N);
    };
    load_r(0);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      f32x4 rc[NB16];
#pragma unroll
      for (int b = 0; b < NB16; ++b) rc[b] = rn[b];
      if (a + 1 < 8) load_r(a + 1);
      const int r = wm * 128 + a * 16 + r16;
      const bool rok = r < rows;
      float v[NB16][4];
#pragma unroll
      for (int b = 0; b < NB16; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[b][e] = EPI == EPI_SCALED ? acc[a][b][e] * p.scale : HAS_R ? acc[a][b][e] + rc[b][e] : acc[a][b][e];
      if (PAIR) {
#pragma unroll
        for (int b = 0; b < NB16; b += 2) {
          const int colp = tn * BN + wn * (BN / WN) + 16 * b;
          int coff;
          const bf16x8 o = pair_to_8(v[b], v[b + 1], c16, coff);
          if (rok) store8_bf16((bf16*)p.C + (int64_t)(row0 + r) * p.ldc + colp + coff, colp + coff, p.N, o);
        }
      } else if (rok) {
#pragma unroll
        for (int b = 0; b < NB16; ++b) epi_row4_store<EPI>(p, row0 + r, colw + 16 * b, p.N, v[b]);
      }
    }
  }
}

// bf16 GEMM for the residual and QKV projections: 256 x 256 output tiles, k consumed 32 at a time
// through a ring of four LDS
// stages (32 KB each: 256 rows x 64 B of A, the same of B).  8 waves in a 2 x 4 grid, each
// 128 x 64 (8 x 4 MFMA blocks of 16 x 16, v_mfma_f32_16x16x32_bf16: one instruction takes the
// whole 32-deep k-tile), two waves per SIMD.
// Operands go global -> LDS by buffer loads that write LDS directly (16 B per lane).  The DMA
// of each k-tile is split in two halves sent in consecutive k-steps, interleaved with MFMAs, so
// the vector-memory path sees a steady stream; three k-tiles are in flight while one is read.
// EXT: the LoRA up-projection as xk / 32 more k-tiles after the K / 32 of A and B: A rows from X,
// B rows from the up-projection of the site that owns the 16 output columns of each row group,
// zero (out-of-range loads) outside that site's xr-wide slice of X's columns.
template <int EPI, bool GROUPED, bool GATHER, bool EXT = false>
__global__ __launch_bounds__(512, 1) void gemm_k32_kernel(GemmParams p, int n_col_tiles) {
  constexpr int NBW = 2;                     // 32-column MFMA blocks per wave
  constexpr int KB = 32;                     // k per stage
  constexpr int ROWB = KB * 2;               // bytes of one LDS row (64)
  constexpr int STG = (BM + BN) * ROWB;      // 32 KB
  constexpr int NST = 4;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  int tn, row0, rows, expert = 0, split = 0;
  if (GROUPED) {
    const int t = blockIdx.x / n_col_tiles;
    tn = blockIdx.x - t * n_col_tiles;
    expert = p.tiles[3 * t];
    if (expert < 0) return;
    row0 = p.tiles[3 * t + 1];
    rows = p.tiles[3 * t + 2];
  } else {
    const int n_m = (p.M + BM - 1) / BM;
    const int n_t = n_m * n_col_tiles;
    const int idall = xcd_remap(blockIdx.x, n_t * max(p.ksplit, 1));
    split = idall / n_t;                               // k-range of a split-K launch (else 0)
    const int id = idall - split * n_t;
    const int GROUP = 8;
    const int per_group = GROUP * n_col_tiles;
    const int g = id / per_group;
    const int first_m = g * GROUP;
    const int gsz = min(n_m - first_m, GROUP);
    const int r_in = id - g * per_group;
    tn = r_in / gsz;
    row0 = (first_m + r_in % gsz) * BM;
    rows = min(BM, p.M - row0);
  }
  if (EPI == EPI_PARTIAL_F32) p.C = (float*)p.C + (int64_t)split * p.M * p.ldc;
  // LDS rows are 64 B (4 chunks of 16 B).  ds_read_b128 serves 16 lanes per cycle over a 256 B
  // (64-bank) window, i.e. four rows; chunk c of row r is stored at c ^ ((r >> 2) & 3), so the 16
  // rows read together at one logical chunk occupy 16 distinct slots.  One DMA instruction fills
  // 1 KB = 16 rows: lane l writes row l >> 2, stored chunk l & 3, which holds logical chunk
  // (l & 3) ^ ((l >> 4) & 3) (the groups start at multiples of 16 rows).
  const int lrow = lane >> 2;
  const int lch = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t lda2 = (uint32_t)p.lda * 2, ldb2 = (uint32_t)p.ldb * 2;
  // wave w sends row groups 2w and 2w + 1 (16 rows each) of both operands

  __amdgpu_buffer_rsrc_t ra;
  uint32_t avoff[2];
  if (GATHER) {
    ra = make_rsrc(p.A, 0x7fffffff);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = (2 * wave + h) * 16 + lrow;
      avoff[h] = (uint32_t)p.a_rows[row0 + min(r, rows - 1)] * lda2 + lch * 16;
    }
  } else {
    ra = make_rsrc((const bf16*)p.A + (int64_t)row0 * p.lda, (uint32_t)rows * lda2);
    avoff[0] = avoff[1] = lrow * lda2 + lch * 16;
  }
  const bf16* Bexp = (const bf16*)p.B + (GROUPED ? (int64_t)expert * p.b_expert_stride : 0);
  __amdgpu_buffer_rsrc_t rb;
  uint32_t bsoff[2];
  if (p.bmode == 1) {
    rb = make_rsrc(Bexp, (uint32_t)(2 * p.swiglu_I) * ldb2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r0 = (2 * wave + h) * 16;
      const int nb = r0 >> 5;
      bsoff[h] = (uint32_t)(((nb & 1) ? p.swiglu_I : 0) + tn * (BN / 2) + (nb >> 1) * 32 + (r0 & 31)) * ldb2;
    }
  } else {
    const int nvalid = min(BN, p.N - tn * BN);
    rb = make_rsrc(Bexp + (int64_t)tn * BN * p.ldb, (uint32_t)nvalid * ldb2);
#pragma unroll
    for (int h = 0; h < 2; ++h) bsoff[h] = (uint32_t)((2 * wave + h) * 16) * ldb2;
  }
  const uint32_t bvoff = lrow * ldb2 + lch * 16;

  const int KTM = p.K / KB / max(p.ksplit, 1);            // k-tiles of A B^T in this launch
  const int KT = KTM + (EXT ? p.xk / KB : 0);
  const uint32_t kofs = (uint32_t)(split * KTM) * ROWB;  // byte offset of this launch's k-range
  // K extension: X rows of the tile, and per row group of this wave its site's up-projection rows
  __amdgpu_buffer_rsrc_t rx, rbx[2];
  uint32_t xvoff = 0, bxvoff = 0, ldx2 = 0;
  int bx_lo[2] = {0, 0}, bx_hi[2] = {0, 0};
  if (EXT) {
    ldx2 = (uint32_t)p.ldx * 2;
    rx = make_rsrc((const bf16*)p.X + (int64_t)row0 * p.ldx, (uint32_t)rows * ldx2);
    xvoff = lrow * ldx2 + lch * 16;
    bxvoff = lrow * (uint32_t)p.xr * 2 + lch * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = b_row_outcol(p, tn, (2 * wave + h) * 16);
      const int site = col < p.xsite_end[0] ? 0 : (col < p.xsite_end[1] ? 1 : 2);
      const int start = site == 0 ? 0 : p.xsite_end[site - 1];
      const int nrow = min(16, min(p.xsite_end[site], (p.bmode == 1 ? 2 * p.swiglu_I : p.N)) - col);
      const bf16* xb = (const bf16*)p.XB[site];
      rbx[h] = make_rsrc(xb ? xb + (int64_t)(col - start) * p.xr : p.X, (xb && nrow > 0) ? (uint32_t)nrow * p.xr * 2 : 0u);
      bx_lo[h] = p.xoff[site];                        // X columns [lo, hi) belong to this site
      bx_hi[h] = p.xoff[site] + p.xr;
    }
  }
  // Half h of the DMA of k-tile t (row groups 2w + h of A and of B) into stage t % 4.  Tiles past
  // the end reload the last one into a stage nobody reads again, so every k-step sends the same
  // number of loads and the vmcnt arithmetic below holds throughout.
  auto dma_half = [&](int t, int h) {
    char* As = smem + (t & (NST - 1)) * STG;
    char* Bs = As + BM * ROWB;
    const int tt = min(t, KT - 1);
    const int g = 2 * wave + h;
    if (EXT && tt >= KTM) {
      const int k0 = (tt - KTM) * KB;                 // X column of this extension k-tile
      dma16(rx, As + g * 1024, xvoff, g * 16 * ldx2 + k0 * 2);
      const bool in = k0 >= bx_lo[h] && k0 < bx_hi[h];
      dma16(rbx[h], Bs + g * 1024, bxvoff, in ? (uint32_t)(k0 - bx_lo[h]) * 2 : 0x40000000u);
      return;
    }
    const uint32_t kb = (uint32_t)tt * ROWB + kofs;
    if (GATHER)
      dma16(ra, As + g * 1024, avoff[h], kb);
    else
      dma16(ra, As + g * 1024, avoff[h], g * 16 * lda2 + kb);
    dma16(rb, Bs + g * 1024, bvoff, bsoff[h] + kb);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[a][b][e] = 0.f;

  // 16x16x32 fragments: lane l holds row (l % 16) of a 16-row block, logical chunk l / 16
  const int r16 = lane & 15, c16 = lane >> 4;
  const int sw = (r16 >> 2) & 3;                  // rows of all blocks differ by multiples of 16
  const int aoff = (wm * 128 + r16) * ROWB + ((c16 ^ sw) << 4);
  const int boff = (wn * 64 + r16) * ROWB + ((c16 ^ sw) << 4);
  bf16x8 fal[4], fah[4], fb[4];
  auto rd_a = [&](bf16x8 (&f)[4], int stage, int half) {
    const char* As = smem + stage * STG;
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = *(const bf16x8*)(As + aoff + (half * 4 + i) * 16 * ROWB);
  };
  auto rd_b = [&](bf16x8 (&f)[4], int stage) {
    const char* Bs = smem + stage * STG + BM * ROWB;
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = *(const bf16x8*)(Bs + boff + i * 16 * ROWB);
  };
  auto mma = [&](const bf16x8 (&fa)[4], const bf16x8 (&fbb)[4], int half) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[half * 4 + i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fbb[nb], acc[half * 4 + i][nb], 0, 0, 0);
  };
  // 16 MFMAs in pairs, an LDS read after each of the first nds pairs, a DMA after the first two
  auto interleave = [&](int nds) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      if (i < nds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      if (i < 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM (LDS-DMA)
    }
  };
  constexpr int WAIT_TILE = 8 | (7 << 4);

  dma_half(0, 0); dma_half(0, 1);
  dma_half(1, 0); dma_half(1, 1);
  dma_half(2, 0); dma_half(2, 1);
  dma_half(3, 0);
  __builtin_amdgcn_s_waitcnt(10 | (7 << 4));
  __builtin_amdgcn_s_barrier();
  rd_a(fal, 0, 0);
  rd_b(fb, 0);
  // k-tile kt: the MFMAs of rows 0-63 of the wave tile while the fragments of rows 64-127 are
  // read; past the barrier, rows 64-127 while tile kt+1's rows 0-63 are read; tile kt+1's B
  // fragments are read once the last MFMA on tile kt's B has been issued.
  for (int kt = 0; kt + 1 < KT; ++kt) {
    const int st = kt & (NST - 1);
    __builtin_amdgcn_s_setprio(0);
    rd_a(fah, st, 1);
    dma_half(kt + 3, 1);
    mma(fal, fb, 0);
    interleave(4);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(WAIT_TILE);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(1);
    rd_a(fal, (kt + 1) & (NST - 1), 0);
    dma_half(kt + 4, 0);
    mma(fah, fb, 1);
    interleave(4);
    __builtin_amdgcn_sched_barrier(0);
    rd_b(fb, (kt + 1) & (NST - 1));
  }
  __builtin_amdgcn_s_setprio(0);
  rd_a(fah, (KT - 1) & (NST - 1), 1);
  mma(fal, fb, 0);
  mma(fah, fb, 1);

  // ---- epilogue through LDS: each wave stages one 32x32 fp32 block at a time, then every lane
  // owns 16 consecutive columns of one row (lanes 2r, 2r+1 cover row r), so global accesses are
  // 16-byte vectors and the per-row index math runs once per block.
  __builtin_amdgcn_s_waitcnt(0);   // the trailing reloads have landed
  __syncthreads();   // every wave is done with the LDS stages
  constexpr int TS = 36;                                   // padded fp32 row stride of a staged block
  float* T0 = (float*)smem + wave * (2 * 32 * TS);
  float* T1 = T0 + 32 * TS;
  const int rr = lane >> 1, cc = (lane & 1) * 16;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (EPI == EPI_SWIGLU && (nb & 1)) continue;       // consumed together with its gate block
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          T0[((q >> 1) * 16 + 4 * c16 + e) * TS + (q & 1) * 16 + r16] = acc[2 * mb + (q >> 1)][2 * nb + (q & 1)][e];
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            T1[((q >> 1) * 16 + 4 * c16 + e) * TS + (q & 1) * 16 + r16] = acc[2 * mb + (q >> 1)][2 * (nb + 1) + (q & 1)][e];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);                   // lgkmcnt(0): staged values written
      __builtin_amdgcn_wave_barrier();
      float v[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *(const float4*)(T0 + rr * TS + cc + 4 * q);
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
      if (EPI == EPI_SWIGLU) {
        float u[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *(const float4*)(T1 + rr * TS + cc + 4 * q);
          u[4 * q] = f.x; u[4 * q + 1] = f.y; u[4 * q + 2] = f.z; u[4 * q + 3] = f.w;
        }
        // optional bf16 terms added before the activation (the LoRA up-projection): R holds the
        // gate term at column j and the up term at column swiglu_I + j
        const int rsw = wm * 128 + mb * 32 + rr;
        const int csw = tn * (BN / 2) + (wn * (NBW / 2) + (nb >> 1)) * 32 + cc;
        if (p.R && rsw < rows) {
          const bf16* rg = (const bf16*)p.R + (int64_t)(row0 + rsw) * p.ldr + csw;
          const bf16* ru = rg + p.swiglu_I;
          if (csw + 16 <= p.swiglu_I) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const bf16x8 a = *(const bf16x8*)(rg + 8 * h2), b = *(const bf16x8*)(ru + 8 * h2);
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                v[8 * h2 + j] += static_cast<float>(a[j]);
                u[8 * h2 + j] += static_cast<float>(b[j]);
              }
            }
          } else {
            for (int j = 0; j < 16 && csw + j < p.swiglu_I; ++j) {
              v[j] += static_cast<float>(rg[j]);
              u[j] += static_cast<float>(ru[j]);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = silu_f(v[j]) * u[j];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);                   // reads done before the next block overwrites
      __builtin_amdgcn_wave_barrier();
      const int r = wm * 128 + mb * 32 + rr;
      if (r < rows) {
        const int row = row0 + r;
        const int col0 = (EPI == EPI_SWIGLU) ? tn * (BN / 2) + (wn * (NBW / 2) + (nb >> 1)) * 32 + cc
                                             : tn * BN + wn * 64 + nb * 32 + cc;
        const int ncols = (EPI == EPI_SWIGLU) ? p.swiglu_I : p.N;
        epi_row16<EPI>(p, row, col0, ncols, v);
      }
    }
  }
}

// ------------------------------------------------------------------ plain fp32 GEMM
// 64 x 64 tiles, 256 threads, 4 x 4 outputs per thread.  Used by fp32 runs only.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[2][16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64;
  const int nout = (EPI == EPI_SWIGLU) ? p.swiglu_I : p.N;
  const int n0 = blockIdx.x * 64;
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
  float acc[2][4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      const int kk = i & 15, r = i >> 4;
      const int m = m0 + r, k = k0 + kk;
      int pm = m < p.M ? m : p.M - 1;
      if (p.a_rows) pm = p.a_rows[pm];
      As[kk][r] = (k < p.K) ? A[(int64_t)pm * p.lda + k] : 0.f;
      const int n = n0 + r;
      const bool nv = n < nout;
      float b0 = 0.f, b1 = 0.f;
      if (nv && k < p.K) {
        if (EPI == EPI_SWIGLU) {
          b0 = B[(int64_t)n * p.ldb + k];
          b1 = B[(int64_t)(p.swiglu_I + n) * p.ldb + k];
        } else if (p.bmode == 2) {
          const int s = n / p.seg_rows;
          b0 = ((const float*)p.Bs[s])[(int64_t)(n - s * p.seg_rows) * p.ldb + k];
        } else {
          b0 = B[(int64_t)n * p.ldb + k];
        }
      }
      Bs[0][kk][r] = b0;
      Bs[1][kk][r] = b1;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) { b[j] = Bs[0][kk][tx * 4 + j]; b2[j] = Bs[1][kk][tx * 4 + j]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[0][i][j] += a[i] * b[j];
          if (EPI == EPI_SWIGLU) acc[1][i][j] += a[i] * b2[j];
        }
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m >= p.M || n >= nout) continue;
      const float v = acc[0][i][j];
      float* C = (float*)p.C;
      if (EPI == EPI_STORE) C[(int64_t)m * p.ldc + n] = v;
      else if (EPI == EPI_SCALED) C[(int64_t)m * p.ldc + n] = v * p.scale;
      else if (EPI == EPI_RESID || EPI == EPI_RESID_TO_F32 || EPI == EPI_RESID_FROM_F32 || EPI == EPI_RESID_F32)
        C[(int64_t)m * p.ldc + n] = ((const float*)p.R)[(int64_t)m * p.ldr + n] + v;
      else if (EPI == EPI_SWIGLU) C[(int64_t)m * p.ldc + n] = silu_f(v) * acc[1][i][j];
      else if (EPI == EPI_F32_IMG) {
        const int img = m / p.rows_per, t = m - img * p.rows_per;
        const int pw = p.img_W >> 5;
        const int py = t / pw, px = t - py * pw;
        const int c = n >> 10, iy = (n >> 5) & 31, ix = n & 31;
        C[(((int64_t)img * 3 + c) * p.img_H + py * 32 + iy) * p.img_W + px * 32 + ix] = v;
      } else if (EPI == EPI_BIAS_BCAST || EPI == EPI_BIAS_BCAST_F32) {
        const int img = m / p.rows_per, t = m - img * p.rows_per;
        const float x = v + p.bias[(int64_t)img * p.N + n];
        for (int br = 0; br < p.n_bcast; ++br)
          C[((int64_t)(img * p.n_bcast + br) * p.rows_per + t) * p.ldc + n] = x;
      }
    }
}

// 8 waves (two per SIMD) by default; PSF_GEMM_WAVES=4 selects one wave per SIMD with 128 x 128
// wave tiles (kept for comparison runs).
int fast_waves() {
  static const int w = [] {
    const char* e = getenv("PSF_GEMM_WAVES");
    return (e && atoi(e) == 4) ? 4 : 8;
  }();
  return w;
}

// Long-k launches (8192 deep or more) whose A or B rows sit at a multiple of 8 KiB apart (a
// dense bf16 row of 12288) fetch the 256 rows of a tile from few memory channels; the ring
// kernel's 64-byte row slices tolerate that better than the 64-deep kernel's 128-byte ones.  With
// both pitches off such multiples (rows padded by 128 B) the 64-deep kernel is the faster.
bool long_k_ring(const GemmParams& p) {
  const auto aliased = [](int64_t ld) { return ((ld * 2) & 8191) == 0; };
  return p.K >= 8192 && (aliased(p.lda) || aliased(p.ldb));
}

// The 64-deep kernel for SwiGLU, for the grouped expert GEMMs, for split-K partial products whose
// k-ranges are whole 64-deep tiles and for plain launches but long-k ones with aliased row pitches;
// the 32-deep ring kernel for those, the other split-K products and row-gathered launches outside
// the expert groups.
template <bool GROUPED, bool GATHER>
hipError_t launch_fast(const GemmParams& p, int epi, int grid, int n_col_tiles, hipStream_t s) {
  const size_t lds = 2 * STAGE_BYTES;
  const bool ring = (GATHER && !GROUPED) || long_k_ring(p);
#define PSF_L(E)                                                                                  \
  case E: {                                                                                        \
    if (E != EPI_SWIGLU && (ring || (E == EPI_PARTIAL_F32 && (p.K / max(p.ksplit, 1)) % BK))) {   \
      auto k = gemm_k32_kernel<E, GROUPED, GATHER>;                                                \
      hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                         (int)lds);                                                \
      if (e != hipSuccess) return e;                                                               \
      hipLaunchKernelGGL(k, dim3(grid), dim3(512), lds, s, p, n_col_tiles);                        \
      return hipGetLastError();                                                                    \
    }                                                                                              \
    auto k = fast_waves() == 4 ? gemm_fast_kernel<E, GROUPED, GATHER, 4> : gemm_fast_kernel<E, GROUPED, GATHER, 8>; \
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                       FAST_LDS);                                                  \
    if (e != hipSuccess) return e;                                                                 \
    hipLaunchKernelGGL(k, dim3(grid), dim3(64 * fast_waves()), FAST_LDS, s, p, n_col_tiles);       \
    return hipGetLastError();                                                                      \
  }
  switch (epi) {
    PSF_L(EPI_STORE)
    PSF_L(EPI_RESID)
    PSF_L(EPI_SWIGLU)
    PSF_L(EPI_F32_IMG)
    PSF_L(EPI_BIAS_BCAST)
    PSF_L(EPI_SCALED)
    PSF_L(EPI_RESID_TO_F32)
    PSF_L(EPI_RESID_FROM_F32)
    PSF_L(EPI_RESID_F32)
    PSF_L(EPI_BIAS_BCAST_F32)
    PSF_L(EPI_PARTIAL_F32)
  }
#undef PSF_L
  return hipErrorInvalidValue;
}

// The 32-deep ring kernel with the K extension (no row gather): residual and store epilogues on a
// plain B, the SwiGLU epilogue on the interleaved gate/up B.
hipError_t launch_k32_ext(const GemmParams& p, int epi, int grid, int n_col_tiles, hipStream_t s) {
  const size_t lds = 2 * STAGE_BYTES;
#define PSF_L(E)                                                                                  \
  case E: {                                                                                        \
    auto k = gemm_k32_kernel<E, false, false, true>;                                               \
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                       (int)lds);                                                  \
    if (e != hipSuccess) return e;                                                                 \
    hipLaunchKernelGGL(k, dim3(grid), dim3(512), lds, s, p, n_col_tiles);                          \
    return hipGetLastError();                                                                      \
  }
  switch (epi) {
    PSF_L(EPI_STORE)
    PSF_L(EPI_RESID)
    PSF_L(EPI_SWIGLU)
    PSF_L(EPI_RESID_TO_F32)
    PSF_L(EPI_RESID_FROM_F32)
    PSF_L(EPI_RESID_F32)
  }
#undef PSF_L
  return hipErrorInvalidValue;
}

// The 64-deep kernel with the K extension (no row gather), where long_k_ring does not apply.
hipError_t launch_fast_ext(const GemmParams& p, int epi, int grid, int n_col_tiles, hipStream_t s) {
  const size_t lds = FAST_LDS;
#define PSF_L(E)                                                                                  \
  case E: {                                                                                        \
    auto k = gemm_fast_kernel<E, false, false, 8, true>;                                           \
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                       (int)lds);                                                  \
    if (e != hipSuccess) return e;                                                                 \
    hipLaunchKernelGGL(k, dim3(grid), dim3(512), lds, s, p, n_col_tiles);                          \
    return hipGetLastError();                                                                      \
  }
  switch (epi) {
    PSF_L(EPI_STORE)
    PSF_L(EPI_RESID)
    PSF_L(EPI_SWIGLU)
    PSF_L(EPI_RESID_TO_F32)
    PSF_L(EPI_RESID_FROM_F32)
    PSF_L(EPI_RESID_F32)
  }
#undef PSF_L
  return hipErrorInvalidValue;
}

template <bool GROUPED, bool EXT>
hipError_t launch_bf16(const GemmParams& p, int epi, int grid, int n_col_tiles, hipStream_t s) {
  const size_t lds = 2 * STAGE_BYTES;
#define PSF_L(E)                                                                                  \
  case E: {                                                                                        \
    auto k = gemm_bf16_kernel<E, GROUPED, EXT>;                                                    \
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                       (int)lds);                                                  \
    if (e != hipSuccess) return e;                                                                 \
    hipLaunchKernelGGL(k, dim3(grid), dim3(NT), lds, s, p, n_col_tiles);                           \
    return hipGetLastError();                                                                      \
  }
  // this kernel serves the LoRA products (the down projection, and block GEMMs with the up
  // projection as a K extension): block epilogues only, never the embed or head ones
  switch (epi) {
    PSF_L(EPI_STORE)
    PSF_L(EPI_RESID)
    PSF_L(EPI_SWIGLU)
    PSF_L(EPI_SCALED)
    PSF_L(EPI_RESID_TO_F32)
    PSF_L(EPI_RESID_FROM_F32)
    PSF_L(EPI_RESID_F32)
  }
#undef PSF_L
  return hipErrorInvalidValue;
}

}  // namespace

// Split-K: the sum of the ksplit fp32 partial products goes through the requested epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p, int ks) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t total = (int64_t)p.M * p.N;
  if (i >= total) return;
  const int64_t m = i / p.N;
  const int n = (int)(i - m * p.N);                  // N is a multiple of 4: a float4 stays in one row
  float4 a = *(const float4*)(p.part + i);
  for (int z = 1; z < ks; ++z) {
    const float4 b = *(const float4*)(p.part + (int64_t)z * total + i);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  float v[4] = {a.x, a.y, a.z, a.w};
  if (EPI == EPI_SCALED)
    for (int j = 0; j < 4; ++j) v[j] *= p.scale;
  if (EPI == EPI_RESID || EPI == EPI_RESID_TO_F32)
    for (int j = 0; j < 4; ++j) v[j] += static_cast<float>(((const bf16*)p.R)[m * p.ldr + n + j]);
  if (EPI == EPI_RESID_F32 || EPI == EPI_RESID_FROM_F32)
    for (int j = 0; j < 4; ++j) v[j] += ((const float*)p.R)[m * p.ldr + n + j];
  if (EPI == EPI_RESID_F32 || EPI == EPI_RESID_TO_F32) {
    for (int j = 0; j < 4; ++j) ((float*)p.C)[m * p.ldc + n + j] = v[j];
  } else {
    for (int j = 0; j < 4; ++j) ((bf16*)p.C)[m * p.ldc + n + j] = static_cast<bf16>(v[j]);
  }
}

bool k32_ext_ok(const GemmParams& p, int epi) {
  if (!p.X || p.xk <= 0 || p.xk % 32 || p.xr <= 0 || p.xr % 32 || p.ldx % 8 || p.a_rows) return false;
  if (epi == EPI_SWIGLU) {
    if (p.bmode != 1 || p.swiglu_I % 16) return false;
  } else if (p.bmode != 0 || (epi != EPI_STORE && epi != EPI_RESID && epi != EPI_RESID_TO_F32 &&
                              epi != EPI_RESID_FROM_F32 && epi != EPI_RESID_F32)) {
    return false;
  }
  for (int i = 0; i < 3; ++i)
    if (p.xoff[i] % 32 || p.xoff[i] < 0 || (p.XB[i] && p.xoff[i] + p.xr > p.xk)) return false;
  for (int i = 0; i < 2; ++i)
    if (p.xsite_end[i] % 16) return false;       // every 16-row group of B lies in one site
  return true;
}

// Compute units of the current device (one workgroup of the fast GEMMs per CU).
int device_cus() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return v > 0 ? v : 256;
  }();
  return n;
}

// Number of k-ranges for a plain GEMM whose row x column tiles leave CUs idle (0 = unsplit): the
// split (1, 2 or 4) with the least estimated time, counted in k-columns that one round of tiles
// streams: rounds x K / ks for the products, plus, for a split, the fp32 partials written and read
// back (8 ks M N bytes) at the same rate (a 64-deep k-tile takes ~1.5 us, HBM moves ~5 TB/s, so
// ~117 KB of partials cost as much as one k-column).  A split that adds a round of tiles never
// pays; one that fills idle CUs does unless its partials outweigh the depth it saves.
int splitk_choice(const GemmParams& p, int epi, int tiles) {
  if (!p.part || p.X || p.bmode != 0 || p.a_rows || p.N % 4) return 0;
  if (epi != EPI_STORE && epi != EPI_RESID && epi != EPI_SCALED && epi != EPI_RESID_F32 && epi != EPI_RESID_TO_F32 &&
      epi != EPI_RESID_FROM_F32)
    return 0;
  const int n_cu = device_cus();
  if (tiles >= n_cu) return 0;
  double best = (double)p.K;                       // unsplit: one round
  int best_ks = 0;
  for (int ks = 2; ks <= 4; ks *= 2) {
    if (p.K % (32 * ks) || p.K / ks < 512) continue;
    if ((size_t)ks * p.M * p.N > p.part_floats) continue;
    const double rounds = (double)((tiles * ks + n_cu - 1) / n_cu);
    const double cost = rounds * (p.K / ks) + 8.0 * ks * (double)p.M * p.N / 117000.0;
    if (cost < best) {
      best = cost;
      best_ks = ks;
    }
  }
  return best_ks;
}

hipError_t gemm_bf16(const GemmParams& p, int epi, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  const int n_cols = (epi == EPI_SWIGLU) ? (p.swiglu_I + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  const int n_m = (p.M + BM - 1) / BM;
  if (const int ks = splitk_choice(p, epi, n_m * n_cols)) {
    GemmParams q = p;
    q.ksplit = ks; q.C = p.part; q.ldc = p.N;
    hipError_t e = launch_fast<false, false>(q, EPI_PARTIAL_F32, n_m * n_cols * ks, n_cols, s);
    if (e != hipSuccess) return e;
    const int64_t n4 = ((int64_t)p.M * p.N + 3) / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    switch (epi) {
      case EPI_STORE: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_STORE>, grid, dim3(256), 0, s, p, ks); break;
      case EPI_RESID: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_RESID>, grid, dim3(256), 0, s, p, ks); break;
      case EPI_SCALED: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_SCALED>, grid, dim3(256), 0, s, p, ks); break;
      case EPI_RESID_F32: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_RESID_F32>, grid, dim3(256), 0, s, p, ks); break;
      case EPI_RESID_TO_F32: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_RESID_TO_F32>, grid, dim3(256), 0, s, p, ks); break;
      default: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_RESID_FROM_F32>, grid, dim3(256), 0, s, p, ks); break;
    }
    return hipGetLastError();
  }
  if (p.X && p.xk > 0) {
    if (k32_ext_ok(p, epi)) {
      if (!long_k_ring(p) && p.K % BK == 0) return launch_fast_ext(p, epi, n_m * n_cols, n_cols, s);
      return launch_k32_ext(p, epi, n_m * n_cols, n_cols, s);
    }
    return launch_bf16<false, true>(p, epi, n_m * n_cols, n_cols, s);
  }
  if (p.bmode == 2) return launch_bf16<false, false>(p, epi, n_m * n_cols, n_cols, s);
  if (p.a_rows) return launch_fast<false, true>(p, epi, n_m * n_cols, n_cols, s);
  return launch_fast<false, false>(p, epi, n_m * n_cols, n_cols, s);
}

hipError_t gemm_bf16_grouped(const GemmParams& p, int epi, int n_col_tiles, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (p.a_rows) return launch_fast<true, true>(p, epi, p.max_tiles * n_col_tiles, n_col_tiles, s);
  return launch_fast<true, false>(p, epi, p.max_tiles * n_col_tiles, n_col_tiles, s);
}

hipError_t gemm_f32(const GemmParams& p, int epi, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  const int nout = (epi == EPI_SWIGLU) ? p.swiglu_I : p.N;
  dim3 grid((nout + 63) / 64, (p.M + 63) / 64);
#define PSF_F(E) \
  case E: hipLaunchKernelGGL(gemm_f32_kernel<E>, grid, dim3(256), 0, s, p); return hipGetLastError();
  switch (epi) {
    PSF_F(EPI_STORE)
    PSF_F(EPI_RESID)
    PSF_F(EPI_SWIGLU)
    PSF_F(EPI_F32_IMG)
    PSF_F(EPI_BIAS_BCAST)
    PSF_F(EPI_SCALED)
    PSF_F(EPI_RESID_TO_F32)
    PSF_F(EPI_RESID_FROM_F32)
    PSF_F(EPI_RESID_F32)
    PSF_F(EPI_BIAS_BCAST_F32)
  }
#undef PSF_F
  return hipErrorInvalidValue;
}

}  // namespace psf
