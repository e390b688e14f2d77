// Backward kernels of LoRA training with the x0 loss: the residual-stream gradient goes down the
// tower through every step of the gen block, and weight gradients are formed for the LoRA
// matrices only (base weights frozen).  bf16 operands, fp32 accumulation and fp32 gradients of
// the residual stream.
//
//   transpose_kernel       out[c][r] = in[r][c] (frozen weights as GEMM operands); transpose_many_kernel
//                          the same for up to 16 small matrices in one launch (the LoRA matrices)
//   cast_kernel            fp32 -> bf16 (GEMM operands)
//   rmsnorm_bwd_kernel     out = base + r g dy - x r^3 sum(g dy x) / D, one row per workgroup
//                          (rmsnorm_bwd4_kernel: 16-byte accesses, optionally a bf16 copy of out)
//   swiglu_kernel          z = silu(gate) up, and its backward (swiglu8_*: eight columns per thread)
//   qknorm_rope_bwd_kernel gradient through RoPE (the inverse rotation) and the per-head RMSNorm
//                          (qknorm_rope_bwd128_kernel: head_dim 128, 16 lanes per head)
//   attn_bwd_dot_kernel    D[q] = sum_i dO[q, i] O[q, i] (attn_bwd_dot128_kernel: 16 lanes per head)
//   attn_bwd_dkdv_kernel   dK, dV of the image keys: four waves of 32 keys share each staged Q/dO
//                          block (double buffered), over every query of the group's heads; P
//                          recomputed from the forward's log-sum-exp
//   attn_bwd_dq_kernel     dQ: four waves (query heads of one kv head) share each staged K/V tile
//                          (double buffered), over every key (prefix and image)
//   wgrad_kernel           C[n1, n2] += sum_m X[m, n1] Y[m, n2] (LoRA weight gradients), split over m;
//                          wgrad_lr_kernel when one side is the rank; wgrad_reduce(_seg)_kernel add
//                          the split partial sums in a fixed order
//   x0_loss_kernel         squared error partial sums and dL/dx0
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace psf {
namespace {

// ---------------------------------------------------------------- layout helpers
// 64 x 64 tiles: rows come in as 16-byte pieces (8 columns), go out as 16-byte pieces of the
// transposed rows; LDS rows padded by 8 elements keep the 16-byte writes aligned.  C and ldi,
// ldo must be multiples of 8 for the vector path; other shapes use element accesses.
DEVI void transpose_tile(const bf16* __restrict__ in, int64_t ldi, bf16* __restrict__ out, int64_t ldo, int R, int C,
                         int r0, int c0, uint16_t (&tile)[64][72]) {
  const int tid = threadIdx.x;
  const uint16_t* src = (const uint16_t*)in;
  uint16_t* dst = (uint16_t*)out;
  const bool vec = (C % 8 == 0) && (R % 8 == 0) && (ldi % 8 == 0) && (ldo % 8 == 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = tid / 8 + 32 * i, cc = (tid % 8) * 8;
    const int r = r0 + rr, c = c0 + cc;
    if (vec) {
      u32x4 v = {0, 0, 0, 0};
      if (r < R && c < C) v = *(const u32x4*)(src + (int64_t)r * ldi + c);
      *(u32x4*)&tile[rr][cc] = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rr][cc + e] = (r < R && c + e < C) ? src[(int64_t)r * ldi + c + e] : 0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int oc = tid / 8 + 32 * i, orr = (tid % 8) * 8;   // output row = input column c0 + oc
    const int c = c0 + oc, r = r0 + orr;
    if (c >= C) continue;
    if (vec) {
      if (r < R) {
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[orr + e][oc];
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
        *(u32x4*)(dst + (int64_t)c * ldo + r) = w;
      }
    } else {
      for (int e = 0; e < 8 && r + e < R; ++e) dst[(int64_t)c * ldo + r + e] = tile[orr + e][oc];
    }
  }
}

__global__ __launch_bounds__(256) void transpose_kernel(const bf16* __restrict__ in, int64_t ldi, bf16* __restrict__ out,
                                                        int64_t ldo, int R, int C) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  transpose_tile(in, ldi, out, ldo, R, C, blockIdx.y * 64, blockIdx.x * 64, tile);
}

// Several small transposes in one launch: workgroup b takes tile b - start[j] of job j
// (start[j] <= b < start[j + 1]), tiles of a job in row-major order over its 64 x 64 grid.
struct TransposeJobs {
  const bf16* in[TRANSPOSE_MAX_JOBS];
  bf16* out[TRANSPOSE_MAX_JOBS];
  int64_t ldi[TRANSPOSE_MAX_JOBS], ldo[TRANSPOSE_MAX_JOBS];
  int R[TRANSPOSE_MAX_JOBS], C[TRANSPOSE_MAX_JOBS];
  int start[TRANSPOSE_MAX_JOBS + 1];
  int n;
};
__global__ __launch_bounds__(256) void transpose_many_kernel(TransposeJobs jb) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int b = blockIdx.x;
  int j = 0;
  while (j + 1 < jb.n && b >= jb.start[j + 1]) ++j;
  const int t = b - jb.start[j], ct = (jb.C[j] + 63) / 64;
  transpose_tile(jb.in[j], jb.ldi[j], jb.out[j], jb.ldo[j], jb.R[j], jb.C[j], (t / ct) * 64, (t % ct) * 64, tile);
}

__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ x, bf16* __restrict__ y, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 v = *(const float4*)(x + i);
    bf16x4 o = {static_cast<bf16>(v.x), static_cast<bf16>(v.y), static_cast<bf16>(v.z), static_cast<bf16>(v.w)};
    *(bf16x4*)(y + i) = o;
  } else {
    for (int64_t k = i; k < n; ++k) y[k] = static_cast<bf16>(x[k]);
  }
}

DEVI float block_sum256(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// out[m, :] = base[m, :] + dRMSNorm(x[m, :]; g)^T dy[m, :]   (base may alias out, or be null)
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float* __restrict__ x, const bf16* __restrict__ g,
                                                          const bf16* __restrict__ dy, const float* base,
                                                          float* out, int D, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * D;
  const bf16* dr = dy + row * D;
  float ss = 0.f, sgx = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) {
    const float xv = xr[i], gd = static_cast<float>(g[i]) * static_cast<float>(dr[i]);
    ss += xv * xv;
    sgx += gd * xv;
  }
  ss = block_sum256(ss, red);
  sgx = block_sum256(sgx, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  const float c = r * r * r * sgx / (float)D;
  for (int i = threadIdx.x; i < D; i += 256) {
    const float gd = static_cast<float>(g[i]) * static_cast<float>(dr[i]);
    const float v = r * gd - xr[i] * c;
    out[row * D + i] = (base ? base[row * D + i] : 0.f) + v;
  }
}

// The same for D a multiple of 4: four columns per thread (16-byte x, base and out, 8-byte g and
// dy); outb, when set, receives bf16(out) as well.
__global__ __launch_bounds__(256) void rmsnorm_bwd4_kernel(const float* __restrict__ x, const bf16* __restrict__ g,
                                                           const bf16* __restrict__ dy, const float* base, float* out,
                                                           bf16* __restrict__ outb, int D, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * D;
  const bf16* dr = dy + row * D;
  float ss = 0.f, sgx = 0.f;
  for (int i = threadIdx.x * 4; i < D; i += 1024) {
    const f32x4 xv = *(const f32x4*)(xr + i);
    const bf16x4 gv = *(const bf16x4*)(g + i), dv = *(const bf16x4*)(dr + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gd = static_cast<float>(gv[e]) * static_cast<float>(dv[e]);
      ss += xv[e] * xv[e];
      sgx += gd * xv[e];
    }
  }
  ss = block_sum256(ss, red);
  sgx = block_sum256(sgx, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  const float c = r * r * r * sgx / (float)D;
  for (int i = threadIdx.x * 4; i < D; i += 1024) {
    const f32x4 xv = *(const f32x4*)(xr + i);
    const bf16x4 gv = *(const bf16x4*)(g + i), dv = *(const bf16x4*)(dr + i);
    f32x4 b = {0.f, 0.f, 0.f, 0.f};
    if (base) b = *(const f32x4*)(base + row * D + i);
    f32x4 o;
    bf16x4 ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gd = static_cast<float>(gv[e]) * static_cast<float>(dv[e]);
      o[e] = b[e] + (r * gd - xv[e] * c);
      ob[e] = static_cast<bf16>(o[e]);
    }
    *(f32x4*)(out + row * D + i) = o;
    if (outb) *(bf16x4*)(outb + row * D + i) = ob;
  }
}

// z[m, j] = silu(gu[m, j]) gu[m, I + j]  (z rows ldz apart)
__global__ __launch_bounds__(256) void swiglu_kernel(const bf16* __restrict__ gu, bf16* __restrict__ z, int64_t ldz, int I,
                                                     int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int64_t m = t / I;
  const int j = (int)(t - m * I);
  const float gt = static_cast<float>(gu[m * 2 * I + j]), up = static_cast<float>(gu[m * 2 * I + I + j]);
  z[m * ldz + j] = static_cast<bf16>(silu_f(gt) * up);
}

// The same for I a multiple of 8: eight columns per thread, 16-byte loads and stores.
__global__ __launch_bounds__(256) void swiglu8_kernel(const bf16* __restrict__ gu, bf16* __restrict__ z, int64_t ldz, int I,
                                                      int64_t n8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const int I8 = I >> 3;
  const int64_t m = t / I8;
  const int j = (int)(t - m * I8) * 8;
  const bf16x8 g = *(const bf16x8*)(gu + m * 2 * I + j), u = *(const bf16x8*)(gu + m * 2 * I + I + j);
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gt = static_cast<float>(g[e]), up = static_cast<float>(u[e]);
    o[e] = static_cast<bf16>(silu_f(gt) * up);
  }
  *(bf16x8*)(z + m * ldz + j) = o;
}

// dgu[m, j] = dz up silu'(gate), dgu[m, I + j] = dz silu(gate)  (dgu rows ldg apart)
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const bf16* __restrict__ gu, const bf16* __restrict__ dz,
                                                         bf16* __restrict__ dgu, int64_t ldg, int I, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int64_t m = t / I;
  const int j = (int)(t - m * I);
  const float gt = static_cast<float>(gu[m * 2 * I + j]), up = static_cast<float>(gu[m * 2 * I + I + j]);
  const float d = static_cast<float>(dz[t]);
  const float s = 1.0f / (1.0f + __expf(-gt));
  dgu[m * ldg + j] = static_cast<bf16>(d * up * (s + gt * s * (1.0f - s)));
  dgu[m * ldg + I + j] = static_cast<bf16>(d * gt * s);
}

// The same for I a multiple of 8: eight columns per thread, 16-byte loads and stores.
__global__ __launch_bounds__(256) void swiglu8_bwd_kernel(const bf16* __restrict__ gu, const bf16* __restrict__ dz,
                                                          bf16* __restrict__ dgu, int64_t ldg, int I, int64_t n8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const int I8 = I >> 3;
  const int64_t m = t / I8;
  const int j = (int)(t - m * I8) * 8;
  const bf16x8 g = *(const bf16x8*)(gu + m * 2 * I + j), u = *(const bf16x8*)(gu + m * 2 * I + I + j);
  const bf16x8 dd = *(const bf16x8*)(dz + t * 8);
  bf16x8 og, ou;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gt = static_cast<float>(g[e]), up = static_cast<float>(u[e]), d = static_cast<float>(dd[e]);
    const float sg = 1.0f / (1.0f + __expf(-gt));
    og[e] = static_cast<bf16>(d * up * (sg + gt * sg * (1.0f - sg)));
    ou[e] = static_cast<bf16>(d * gt * sg);
  }
  *(bf16x8*)(dgu + m * ldg + j) = og;
  *(bf16x8*)(dgu + m * ldg + I + j) = ou;
}

// One wave per (token, head) of the q and k heads: lane p < d/2 holds the rotate-half pair
// (p, p + d/2).  grad (fp32, row stride ldg) is the gradient with respect to the normed and
// rotated head; raw the head before the norm.  Writes the gradient with respect to raw (bf16)
// into dqkv; v heads copy their gradient (dv) as it is.
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(const bf16* __restrict__ raw, int64_t ldr,
                                                              const float* __restrict__ dq, const float* __restrict__ dk,
                                                              const float* __restrict__ dv, SeqInfo si, int Hq, int Hkv,
                                                              int d, const bf16* __restrict__ gq,
                                                              const bf16* __restrict__ gk,
                                                              const float2* __restrict__ table, float eps,
                                                              bf16* __restrict__ dqkv, int64_t ldo, int64_t total) {
  const int lane = threadIdx.x & 63;
  const int64_t hv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (hv >= total) return;
  const int H = Hq + 2 * Hkv;
  const int64_t tok = hv / H;
  const int head = (int)(hv - tok * H);
  const int b = (int)(tok / si.N), n = (int)(tok - (int64_t)b * si.N);
  const int half = d / 2;
  bf16* op = dqkv + tok * ldo + (int64_t)head * d;
  if (head >= Hq + Hkv) {                       // v: the gradient passes through
    const float* gp = dv + tok * (int64_t)Hkv * d + (int64_t)(head - Hq - Hkv) * d;
    for (int i = lane; i < d; i += 64) op[i] = static_cast<bf16>(gp[i]);
    return;
  }
  const bool isq = head < Hq;
  const float* gp = isq ? dq + tok * (int64_t)Hq * d + (int64_t)head * d : dk + tok * (int64_t)Hkv * d + (int64_t)(head - Hq) * d;
  const bf16* rp = raw + tok * ldr + (int64_t)head * d;
  const bf16* g = isq ? gq : gk;
  const bool act = lane < half;
  const int p = act ? lane : 0;
  // inverse rotation of the incoming gradient
  const float2 cs = table[(int64_t)(si.plen[b] + n) * half + p];
  const float ga = gp[p], gb = gp[p + half];
  const float ta = ga * cs.x + gb * cs.y, tb = -ga * cs.y + gb * cs.x;
  // RMSNorm backward over the head vector
  const float xa = static_cast<float>(rp[p]), xb = static_cast<float>(rp[p + half]);
  const float wa = static_cast<float>(g[p]), wb = static_cast<float>(g[p + half]);
  float ss = act ? xa * xa + xb * xb : 0.f;
  float sgx = act ? wa * ta * xa + wb * tb * xb : 0.f;
  ss = warp_sum(ss);
  sgx = warp_sum(sgx);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  const float c = r * r * r * sgx / (float)d;
  if (act) {
    op[p] = static_cast<bf16>(r * wa * ta - xa * c);
    op[p + half] = static_cast<bf16>(r * wb * tb - xb * c);
  }
}

// The same for d = 128: 16 lanes per (token, head), four heads per wave; lane j holds the rotation
// pairs 4j .. 4j + 3 (elements 4j .. 4j + 3 and 64 + 4j .. 64 + 4j + 3), 16-byte gradient loads.
__global__ __launch_bounds__(256) void qknorm_rope_bwd128_kernel(const bf16* __restrict__ raw, int64_t ldr,
                                                                 const float* __restrict__ dq, const float* __restrict__ dk,
                                                                 const float* __restrict__ dv, SeqInfo si, int Hq, int Hkv,
                                                                 const bf16* __restrict__ gq, const bf16* __restrict__ gk,
                                                                 const float2* __restrict__ table, float eps,
                                                                 bf16* __restrict__ dqkv, int64_t ldo, int64_t total) {
  constexpr int d = 128, half = 64;
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int64_t hv = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = hv < total;                 // no early return: the reductions use all 64 lanes
  const int H = Hq + 2 * Hkv;
  const int64_t hvc = valid ? hv : 0;
  const int64_t tok = hvc / H;
  const int head = (int)(hvc - tok * H);
  const int b = (int)(tok / si.N), n = (int)(tok - (int64_t)b * si.N);
  bf16* op = dqkv + tok * ldo + (int64_t)head * d;
  const int p0 = 4 * j;
  if (head >= Hq + Hkv) {                        // v: the gradient passes through (uniform per 16 lanes)
    const float* gp = dv + tok * (int64_t)Hkv * d + (int64_t)(head - Hq - Hkv) * d + 8 * j;
    const f32x4 a = *(const f32x4*)gp, c = *(const f32x4*)(gp + 4);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) { o[e] = static_cast<bf16>(a[e]); o[4 + e] = static_cast<bf16>(c[e]); }
    if (valid) *(bf16x8*)(op + 8 * j) = o;
  }
  const bool isq = head < Hq, isk = !isq && head < Hq + Hkv;
  float ss = 0.f, sgx = 0.f;
  f32x4 ta, tb, xa, xb, wa, wb;
  if (isq || isk) {
    const float* gp = isq ? dq + tok * (int64_t)Hq * d + (int64_t)head * d : dk + tok * (int64_t)Hkv * d + (int64_t)(head - Hq) * d;
    const bf16* rp = raw + tok * ldr + (int64_t)head * d;
    const bf16* g = isq ? gq : gk;
    const f32x4 ga = *(const f32x4*)(gp + p0), gb = *(const f32x4*)(gp + half + p0);
    const bf16x4 ra = *(const bf16x4*)(rp + p0), rb = *(const bf16x4*)(rp + half + p0);
    const bf16x4 va = *(const bf16x4*)(g + p0), vb = *(const bf16x4*)(g + half + p0);
    const float2* cs = table + (int64_t)(si.plen[b] + n) * half + p0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 c = cs[e];
      // inverse rotation of the incoming gradient
      ta[e] = ga[e] * c.x + gb[e] * c.y;
      tb[e] = -ga[e] * c.y + gb[e] * c.x;
      xa[e] = static_cast<float>(ra[e]);
      xb[e] = static_cast<float>(rb[e]);
      wa[e] = static_cast<float>(va[e]);
      wb[e] = static_cast<float>(vb[e]);
      ss += xa[e] * xa[e] + xb[e] * xb[e];
      sgx += wa[e] * ta[e] * xa[e] + wb[e] * tb[e] * xb[e];
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {              // sums over the 16 lanes of this head
    ss += __shfl_xor(ss, o, 64);
    sgx += __shfl_xor(sgx, o, 64);
  }
  if (valid && (isq || isk)) {
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    const float c = r * r * r * sgx / (float)d;
    bf16x4 oa, ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      oa[e] = static_cast<bf16>(r * wa[e] * ta[e] - xa[e] * c);
      ob[e] = static_cast<bf16>(r * wb[e] * tb[e] - xb[e] * c);
    }
    *(bf16x4*)(op + p0) = oa;
    *(bf16x4*)(op + half + p0) = ob;
  }
}

// D[(b*Hq + h)*N + n] = sum_i dO[tok, h*d + i] O[tok, h*d + i]: one wave per (token, head)
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(const bf16* __restrict__ dO, const bf16* __restrict__ O,
                                                           int64_t ld, int Hq, int d, int N, float* __restrict__ Dq,
                                                           int64_t total) {
  const int lane = threadIdx.x & 63;
  const int64_t hv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (hv >= total) return;
  const int64_t tok = hv / Hq;
  const int h = (int)(hv - tok * Hq);
  float acc = 0.f;
  for (int i = lane; i < d; i += 64)
    acc += static_cast<float>(dO[tok * ld + (int64_t)h * d + i]) * static_cast<float>(O[tok * ld + (int64_t)h * d + i]);
  acc = warp_sum(acc);
  if (lane == 0) {
    const int64_t b = tok / N, n = tok - b * N;
    Dq[(b * Hq + h) * N + n] = acc;
  }
}

// ---------------------------------------------------------------- attention backward
// Both kernels use v_mfma_f32_32x32x16_bf16.  Operand fragments: lane l holds A[l%32][8(l/32) .. +8]
// and B[8(l/32) .. +8][l%32] of one 16-deep k-step; the accumulator gives lane l the 16 values
// C[(e/4)*8 + (l/32)*4 + e%4][l%32].  A product whose k index is the accumulator's row index
// (P or dS as the B operand) takes the accumulator values e = 8t .. 8t+7 as k-step t, which
// visits k in the order 16t + (i/4)*8 + (l/32)*4 + i%4; its A operand is read from LDS in that
// same order.
//
// Staged [32][128] bf16 tiles (Q and dO, or K) keep rows of 16 chunks of 16 bytes; logical chunk c
// of row r sits at c ^ f(r), f(r) = 4 (r & 3) + ((r >> 2) & 3).  A row read (16 lanes, 16
// consecutive rows, one chunk each) then meets 16 distinct chunks, and a transposed read (16
// lanes, 4 consecutive rows, 32 bytes of each) meets 4 disjoint chunk pairs: no bank conflicts.
DEVI int tile_off(int r, int c) { return r * 128 + ((((c >> 3) ^ ((r & 3) << 2) ^ ((r >> 2) & 3))) << 3) + (c & 7); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

// A lane's element offsets into a staged tile, fixed for the whole kernel.  Row r adds r * 128 and
// the swizzle only flips bits 3-6 (the chunk), so the offsets of other k-steps and column blocks
// are these with constant bits XOR-ed in or 2048 (16 rows) added:
//   rd:       row l%32, logical chunk l/32; chunk 2 ks + l/32 is at rd ^ (ks << 4)
//   tr0, tr1: the transposed reads below for t = 0, column block 0; for (t, db) they are at
//             (tr ^ (db << 5)) + 2048 t
struct TileLane { int rd, tr0, tr1; };
DEVI TileLane tile_lane(int lane) {
  const int lr = lane & 31, lh = lane >> 5, j = lane & 15;
  const int c = ((lane >> 4) & 1) * 16 + 4 * (j & 3), r0 = 4 * lh + (j >> 2);
  return {tile_off(lr, lh * 8), tile_off(r0, c), tile_off(r0 + 8, c)};
}

// A or B operand of k-step ks from a staged tile's rows: lane l gets tile[l%32][16 ks + 8 (l/32) .. +8].
DEVI bf16x8 tile_row(const bf16* tile, const TileLane& tl, int ks) {
  return *(const bf16x8*)(tile + (tl.rd ^ (ks << 4)));
}

// A operand of k-step t, column block db (32 columns), from a staged tile read transposed:
// lane l gets tile[16t + (i/4)*8 + (l/32)*4 + i%4][32 db + l%32] for i = 0..7.  ds_read_tr16_b64 hands
// lane j of each 16-lane group element j%4 of the 8-byte pieces addressed by lanes 4k + j/4,
// k = 0..3; so lane j addresses row 16t + 8h + 4(l/32) + j/4, columns 32 db + 16 ((l/16) & 1) +
// 4 (j%4) .. +3, and the two reads (h = 0, 1) give slots 0-3 and 4-7.
DEVI bf16x8 tile_tr(const bf16* tile, const TileLane& tl, int t, int db) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(tile + ((tl.tr0 ^ (db << 5)) + 2048 * t)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(tile + ((tl.tr1 ^ (db << 5)) + 2048 * t)));
  const s16x4 x[2] = {lo, hi};
  bf16x8 f;
  __builtin_memcpy(&f, x, 16);
  return f;
}

template <int V> using Int = std::integral_constant<int, V>;

// Row pointer of key j (sequence b, kv head g) in the K or V source: the prefix cache for j < P,
// the normed (K) or raw (V) image projections in qkv otherwise.
DEVI const bf16* kv_row(const SeqInfo& si, int b, int g, int j, int Hkv, int d, const bf16* qkv, int64_t ldq,
                        int col0, bool isv) {
  const int P = si.plen[b];
  if (j < P) return (const bf16*)(isv ? si.pv[b] : si.pk[b]) + ((int64_t)j * Hkv + g) * d;
  return qkv + ((int64_t)b * si.N + (j - P)) * ldq + col0 + (int64_t)g * d;
}

// dK, dV of the image keys of (sequence b, kv head g): a workgroup of four waves covers 128 keys,
// wave w the 32 keys [128 kb + 32 w, +32).  The workgroup walks the 32-query blocks of every head
// of the group; each block's Q (normed, rotated), dO, log-sum-exp and D are staged once in LDS for
// the four waves (two stages: the next block is loaded into registers while this one is used).
// S = Q K^T takes A = Q rows from LDS and B = the wave's K rows (registers); dV^T += dO^T P and
// dK^T += Q^T dS read their A operands transposed from LDS.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const bf16* __restrict__ qkv, int64_t ldq, SeqInfo si,
                                                            int Hq, int Hkv, const bf16* __restrict__ dO, int64_t ldo,
                                                            const float* __restrict__ lse, const float* __restrict__ Dq,
                                                            float scale_log2, float scale, float* __restrict__ dk,
                                                            float* __restrict__ dv, int n_kb) {
  static_assert(D == 128, "staged tiles are 32 x 128");
  constexpr int KS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sq[2][32 * D];
  __shared__ __attribute__((aligned(16))) bf16 sdo[2][32 * D];
  __shared__ float slse[2][32], sD[2][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int kb = blockIdx.x % n_kb;
  const int g = (blockIdx.x / n_kb) % Hkv;
  const int b = blockIdx.x / (n_kb * Hkv);
  const int N = si.N, G = Hq / Hkv;
  const int QD = Hq * D;
  const int mykey = 128 * kb + 32 * wave + lr;        // image key index (token) of this lane's column
  const bool keyok = mykey < N;
  const int kc = keyok ? mykey : N - 1;
  bf16x8 kf[KS], vf[KS];
  {
    const bf16* kp = qkv + ((int64_t)b * N + kc) * ldq + QD + (int64_t)g * D + lh * 8;
    const bf16* vp = qkv + ((int64_t)b * N + kc) * ldq + QD + (int64_t)Hkv * D + (int64_t)g * D + lh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *(const bf16x8*)(kp + ks * 16);
      vf[ks] = *(const bf16x8*)(vp + ks * 16);
    }
  }
  f32x16 dkT[NDB], dvT[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dkT[i][e] = 0.f; dvT[i][e] = 0.f; }
  const int nqb = (N + 31) / 32, nblk = G * nqb;

  // staging of block it = (head g G + it / nqb, queries 32 (it % nqb) ..): thread tid moves chunks
  // tid and tid + 256 of Q and of dO (row = chunk / 16); threads 0-31 the lse, 32-63 the D values
  bf16x8 rq[2], rd[2];
  float rs = 0.f;
  auto fetch = [&](int it) {
    const int h = g * G + it / nqb, q0 = (it % nqb) * 32;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * 256 + tid, row = idx >> 4, ch = idx & 15;
      const int64_t tok = (int64_t)b * N + min(q0 + row, N - 1);
      rq[c] = *(const bf16x8*)(qkv + tok * ldq + (int64_t)h * D + ch * 8);
      rd[c] = *(const bf16x8*)(dO + tok * ldo + (int64_t)h * D + ch * 8);
    }
    if (tid < 64) {
      const int64_t o = ((int64_t)b * Hq + h) * N + min(q0 + (tid & 31), N - 1);
      rs = tid < 32 ? lse[o] : Dq[o];
    }
  };
  auto stage = [&](int st) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * 256 + tid, row = idx >> 4, ch = idx & 15;
      *(bf16x8*)&sq[st][tile_off(row, ch * 8)] = rq[c];
      *(bf16x8*)&sdo[st][tile_off(row, ch * 8)] = rd[c];
    }
    if (tid < 32) slse[st][tid] = rs;
    else if (tid < 64) sD[st][tid - 32] = rs;
  };
  const TileLane tl = tile_lane(lane);
  // block it in stage ST (a constant, so the stage's LDS address folds into the instructions)
  auto body = [&](int it, auto stc) {
    constexpr int st = decltype(stc)::value;
    const int q0 = (it % nqb) * 32;
    if (it + 1 < nblk) {
      stage(st ^ 1);                     // every wave left stage st ^ 1 at the last barrier
      if (it + 2 < nblk) fetch(it + 2);
    }
    const bf16* Qs = sq[st];
    const bf16* Ds = sdo[st];
    f32x16 sv, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) { sv[e] = 0.f; dp[e] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row(Qs, tl, ks), kf[ks], sv, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row(Ds, tl, ks), vf[ks], dp, 0, 0, 0);
    }
    // P and dS (rows = queries q0 + (e/4)*8 + lh*4 + e%4, column = this lane's key).  Lanes of
    // keys past N produce columns that are never stored; rows past N (a ragged last block) are
    // zeroed so that they add nothing to the valid keys.
    float4 ls[4], dd[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      ls[a] = *(const float4*)&slse[st][a * 8 + lh * 4];
      dd[a] = *(const float4*)&sD[st][a * 8 + lh * 4];
    }
    const bool full = q0 + 32 <= N;
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float lv = ls[e >> 2][e & 3], dv_ = dd[e >> 2][e & 3];
      float pr = __builtin_amdgcn_exp2f(sv[e] * scale_log2 - lv);
      if (!full && q0 + (e >> 2) * 8 + lh * 4 + (e & 3) >= N) pr = 0.f;
      pf[e >> 3][e & 7] = static_cast<bf16>(pr);
      dsf[e >> 3][e & 7] = static_cast<bf16>(pr * (dp[e] - dv_));
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr(Ds, tl, t, db), pf[t], dvT[db], 0, 0, 0);
        dkT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr(Qs, tl, t, db), dsf[t], dkT[db], 0, 0, 0);
      }
    __syncthreads();
  };
  fetch(0);
  stage(0);
  if (nblk > 1) fetch(1);
  __syncthreads();
  for (int it = 0; it < nblk; it += 2) {
    body(it, Int<0>{});
    if (it + 1 < nblk) body(it + 1, Int<1>{});
  }
  if (keyok) {
    const int64_t tok = (int64_t)b * N + mykey;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int dd = db * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
        dk[tok * Hkv * D + (int64_t)g * D + dd] = dkT[db][e] * scale;
        dv[tok * Hkv * D + (int64_t)g * D + dd] = dvT[db][e];
      }
  }
}

// dQ over every key (prefix and image).  A workgroup of four waves shares one (sequence b, kv head
// g): wave w takes head g G + hg hpw + w % hpw and the 32 queries of block qg (4 / hpw) + w / hpw,
// hpw = the heads per workgroup (4, 2 or 1 as the group size allows).  Tiles of 32 keys of K and V
// are staged once in LDS for the four waves (two stages: the next tile is loaded into registers
// while this one is used).  S^T = K Q^T and dP^T = V dO^T take A = K or V rows from LDS and B = the
// wave's Q or dO rows (registers); dQ^T += K^T dS^T reads K^T transposed from LDS.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(const bf16* __restrict__ qkv, int64_t ldq, SeqInfo si, int Hq,
                                                          int Hkv, const bf16* __restrict__ dO, int64_t ldo,
                                                          const float* __restrict__ lse, const float* __restrict__ Dq,
                                                          float scale_log2, float scale, float* __restrict__ dq,
                                                          int hpw, int n_qg) {
  static_assert(D == 128, "staged tiles are 32 x 128");
  constexpr int KS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sk[2][32 * D];
  __shared__ __attribute__((aligned(16))) bf16 sv[2][32 * D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int G = Hq / Hkv, n_hg = G / hpw;
  const int qg = blockIdx.x % n_qg;
  const int hg = (blockIdx.x / n_qg) % n_hg;
  const int g = (blockIdx.x / (n_qg * n_hg)) % Hkv;
  const int b = blockIdx.x / (n_qg * n_hg * Hkv);
  const int N = si.N, P = si.plen[b], L = P + N;
  const int h = g * G + hg * hpw + wave % hpw;
  const int QD = Hq * D;
  const int myq = (qg * (4 / hpw) + wave / hpw) * 32 + lr;
  const bool qok = myq < N;
  const int64_t tok = (int64_t)b * N + min(myq, N - 1);
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = *(const bf16x8*)(qkv + tok * ldq + (int64_t)h * D + ks * 16 + lh * 8);
    df[ks] = *(const bf16x8*)(dO + tok * ldo + (int64_t)h * D + ks * 16 + lh * 8);
  }
  const float my_lse = lse[((int64_t)b * Hq + h) * N + min(myq, N - 1)];
  const float my_D = Dq[((int64_t)b * Hq + h) * N + min(myq, N - 1)];
  f32x16 dqT[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqT[i][e] = 0.f;

  // staging of key tile t (keys 32 t ..): thread tid moves chunks tid and tid + 256 of K and of V
  const int ntile = (L + 31) / 32;
  bf16x8 rk[2], rv[2];
  auto fetch = [&](int t) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * 256 + tid, row = idx >> 4, ch = idx & 15;
      const int j = min(32 * t + row, L - 1);
      rk[c] = *(const bf16x8*)(kv_row(si, b, g, j, Hkv, D, qkv, ldq, QD, false) + ch * 8);
      rv[c] = *(const bf16x8*)(kv_row(si, b, g, j, Hkv, D, qkv, ldq, QD + Hkv * D, true) + ch * 8);
    }
  };
  auto stage = [&](int st) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * 256 + tid, row = idx >> 4, ch = idx & 15;
      *(bf16x8*)&sk[st][tile_off(row, ch * 8)] = rk[c];
      *(bf16x8*)&sv[st][tile_off(row, ch * 8)] = rv[c];
    }
  };
  const TileLane tl = tile_lane(lane);
  // key tile t in stage ST (a constant, so the stage's LDS address folds into the instructions)
  auto body = [&](int t, auto stc) {
    constexpr int st = decltype(stc)::value;
    const int j0 = 32 * t;
    if (t + 1 < ntile) {
      stage(st ^ 1);                     // every wave left stage st ^ 1 at the last barrier
      if (t + 2 < ntile) fetch(t + 2);
    }
    const bf16* Ks = sk[st];
    const bf16* Vs = sv[st];
    f32x16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s[e] = 0.f; dp[e] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row(Ks, tl, ks), qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row(Vs, tl, ks), df[ks], dp, 0, 0, 0);
    }
    // lanes of queries past N produce columns that are never stored; keys past L (a ragged last
    // tile) are zeroed
    const bool full = j0 + 32 <= L;
    bf16x8 dsf[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float p = __builtin_amdgcn_exp2f(s[e] * scale_log2 - my_lse);
      if (!full && j0 + (e >> 2) * 8 + lh * 4 + (e & 3) >= L) p = 0.f;
      dsf[e >> 3][e & 7] = static_cast<bf16>(p * (dp[e] - my_D));
    }
#pragma unroll
    for (int tk = 0; tk < 2; ++tk)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dqT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr(Ks, tl, tk, db), dsf[tk], dqT[db], 0, 0, 0);
    __syncthreads();
  };
  fetch(0);
  stage(0);
  if (ntile > 1) fetch(1);
  __syncthreads();
  for (int t = 0; t < ntile; t += 2) {
    body(t, Int<0>{});
    if (t + 1 < ntile) body(t + 1, Int<1>{});
  }
  if (qok) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int dd = db * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
        dq[tok * QD + (int64_t)h * D + dd] = dqT[db][e] * scale;
      }
  }
}

// ---------------------------------------------------------------- LoRA weight gradients
// Partial[z][n1][n2] = sum over m in split z of X[m, n1] Y[m, n2].  Workgroup tile 64 x 64 of
// (n1, n2), four waves of 32 x 32; chunks of 64 m are staged in LDS transposed ([n][m], rows
// padded to 72 so the 16-byte fragment reads stay aligned and spread over banks).
__global__ __launch_bounds__(256) void wgrad_kernel(const bf16* __restrict__ X, int64_t ldx, const bf16* __restrict__ Y,
                                                    int64_t ldy, int M, int N1, int N2, int m_per_split,
                                                    float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) bf16 sx[64][72];
  __shared__ __attribute__((aligned(16))) bf16 sy[64][72];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int n1b = blockIdx.x * 64, n2b = blockIdx.y * 64, z = blockIdx.z;
  const int m_lo = z * m_per_split, m_hi = min(M, m_lo + m_per_split);
  const int w1 = (wave >> 1) * 32, w2 = (wave & 1) * 32;
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  for (int m0 = m_lo; m0 < m_hi; m0 += 64) {
    __syncthreads();
    // 64 m x 8 chunks of 8 columns, two per thread, for each of X and Y
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = it * 256 + tid;
      const int mm = idx >> 3, ch = idx & 7;
      const int m = m0 + mm;
      const int c1 = n1b + ch * 8, c2 = n2b + ch * 8;
      bf16x8 vx, vy;
#pragma unroll
      for (int e = 0; e < 8; ++e) { vx[e] = static_cast<bf16>(0.f); vy[e] = static_cast<bf16>(0.f); }
      if (m < m_hi && c1 < N1) vx = *(const bf16x8*)(X + (int64_t)m * ldx + c1);
      if (m < m_hi && c2 < N2) vy = *(const bf16x8*)(Y + (int64_t)m * ldy + c2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sx[ch * 8 + e][mm] = vx[e];
        sy[ch * 8 + e][mm] = vy[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = *(const bf16x8*)&sx[w1 + lr][ks * 16 + lh * 8];
      const bf16x8 bb = *(const bf16x8*)&sy[w2 + lr][ks * 16 + lh * 8];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
    }
  }
  float* out = part + (int64_t)z * N1 * N2;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int r = n1b + w1 + (e >> 2) * 8 + lh * 4 + (e & 3);
    const int c = n2b + w2 + lr;
    if (r < N1 && c < N2) out[(int64_t)r * N2 + c] = acc[e];
  }
}

// Partial sums of a LoRA weight gradient whose one side is the rank (R <= 128 columns, "Small")
// and whose other side is a projection width ("Big", NB columns): over the m-range of split z,
//   BIGX:  part[z][c][j] = sum_m Big[m][c] Small[m][j]   (C = X^T Y with X = Big, N1 = NB, N2 = R)
//   !BIGX: part[z][j][c] = sum_m Small[m][j] Big[m][c]   (X = Small, Y = Big, N1 = R, N2 = NB)
// A workgroup streams 128 Big columns (32 per wave) over its m-range in 32-row tiles staged in LDS
// (two stages, the next tile loaded into registers under this one's MFMAs); both operands are
// read transposed (k = m) from the staged tiles, and the MFMA operand order puts the Big column
// on the accumulator's lane axis so the partial stores are 128-byte rows.
template <bool BIGX>
__global__ __launch_bounds__(256) void wgrad_lr_kernel(const bf16* __restrict__ Big, int64_t ldb,
                                                       const bf16* __restrict__ Small, int64_t lds, int M, int NB,
                                                       int R, int m_per_split, float* __restrict__ part, int bseg1,
                                                       int bseg2, int sm_step) {
  __shared__ __attribute__((aligned(16))) bf16 sb[2][32 * 128];
  __shared__ __attribute__((aligned(16))) bf16 ss[2][32 * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int c0 = blockIdx.x * 128, z = blockIdx.y;
  // block-diagonal use: Big columns from bseg1 (bseg2) on pair with the next sm_step Small columns
  Small += (c0 >= bseg2 ? 2 : (c0 >= bseg1 ? 1 : 0)) * sm_step;
  const int m_lo = z * m_per_split, m_hi = min(M, m_lo + m_per_split);
  const int nchunk = (m_hi - m_lo + 31) / 32;
  const int NJ = (R + 31) / 32;
  const TileLane tl = tile_lane(lane);
  f32x16 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[jb][e] = 0.f;
  // thread tid moves 16-byte chunks tid and tid + 256 of each tile (row = chunk / 16)
  bf16x8 rb[2], rs[2];
  const bf16x8 zero = {};
  auto fetch = [&](int ch) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * 256 + tid, row = idx >> 4, col = (idx & 15) * 8;
      const int m = m_lo + ch * 32 + row;
      rb[c] = (m < m_hi && c0 + col < NB) ? *(const bf16x8*)(Big + (int64_t)m * ldb + c0 + col) : zero;
      rs[c] = (m < m_hi && col < R) ? *(const bf16x8*)(Small + (int64_t)m * lds + col) : zero;
    }
  };
  auto stage = [&](int st) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * 256 + tid, row = idx >> 4, col = (idx & 15) * 8;
      *(bf16x8*)&sb[st][tile_off(row, col)] = rb[c];
      *(bf16x8*)&ss[st][tile_off(row, col)] = rs[c];
    }
  };
  auto body = [&](int ch, auto stc) {
    constexpr int st = decltype(stc)::value;
    if (ch + 1 < nchunk) {
      stage(st ^ 1);                     // every wave left stage st ^ 1 at the last barrier
      if (ch + 2 < nchunk) fetch(ch + 2);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 bigf = tile_tr(sb[st], tl, t, wave);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (jb >= NJ) continue;
        const bf16x8 smf = tile_tr(ss[st], tl, t, jb);
        acc[jb] = BIGX ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bigf, smf, acc[jb], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_bf16(smf, bigf, acc[jb], 0, 0, 0);
      }
    }
    __syncthreads();
  };
  if (nchunk > 0) {
    fetch(0);
    stage(0);
    if (nchunk > 1) fetch(1);
    __syncthreads();
    for (int ch = 0; ch < nchunk; ch += 2) {
      body(ch, Int<0>{});
      if (ch + 1 < nchunk) body(ch + 1, Int<1>{});
    }
  }
  // accumulator of block jb: BIGX rows c = c0 + 32 wave + (e/4)*8 + lh*4 + e%4, lanes j = 32 jb + lr;
  // otherwise rows j = 32 jb + (e/4)*8 + lh*4 + e%4, lanes c = c0 + 32 wave + lr
  float* out = part + (int64_t)z * NB * R;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    if (jb >= NJ) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = (e >> 2) * 8 + lh * 4 + (e & 3);
      const int c = c0 + 32 * wave + (BIGX ? row : lr), j = 32 * jb + (BIGX ? lr : row);
      if (j < R && c < NB) {
        if (BIGX) out[(int64_t)c * R + j] = acc[jb][e];
        else out[(int64_t)j * NB + c] = acc[jb][e];
      }
    }
  }
}

// C[i] += sum_z part[z][i]
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                           float* __restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < splits; ++z) s += part[(int64_t)z * n + i];
  C[i] += s;
}

// The same with C in three pieces: elements [0, e1) added into C0, [e1, e2) into C1, the rest
// into C2 (each piece from its own start).
__global__ __launch_bounds__(256) void wgrad_reduce_seg_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                               int64_t e1, int64_t e2, float* C0, float* C1, float* C2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < splits; ++z) s += part[(int64_t)z * n + i];
  if (i < e1) C0[i] += s;
  else if (i < e2) C1[i - e1] += s;
  else C2[i - e2] += s;
}

// The same for d = 128: 16 lanes per (token, head) with 16-byte loads, four heads per wave.
__global__ __launch_bounds__(256) void attn_bwd_dot128_kernel(const bf16* __restrict__ dO, const bf16* __restrict__ O,
                                                              int64_t ld, int Hq, int N, float* __restrict__ Dq,
                                                              int64_t total) {
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int64_t hv = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = hv < total;
  const int64_t hvc = valid ? hv : 0;
  const int64_t tok = hvc / Hq;
  const int h = (int)(hvc - tok * Hq);
  const bf16x8 a = *(const bf16x8*)(dO + tok * ld + (int64_t)h * 128 + 8 * j);
  const bf16x8 c = *(const bf16x8*)(O + tok * ld + (int64_t)h * 128 + 8 * j);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc += static_cast<float>(a[e]) * static_cast<float>(c[e]);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (valid && j == 0) {
    const int64_t b = tok / N, n = tok - b * N;
    Dq[(b * Hq + h) * N + n] = acc;
  }
}

// ---------------------------------------------------------------- x0 loss
// part[block] = sum of (pred - tgt)^2 over the block's elements; grad = 2 (pred - tgt) / n
__global__ __launch_bounds__(256) void x0_loss_kernel(const float* __restrict__ pred, const float* __restrict__ tgt,
                                                      float* __restrict__ grad, float* __restrict__ part, int64_t n) {
  __shared__ float red[4];
  float acc = 0.f;
  const float two_n = 2.0f / (float)n;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float dlt = pred[i] - tgt[i];
    acc += dlt * dlt;
    grad[i] = two_n * dlt;
  }
  acc = block_sum256(acc, red);
  if (threadIdx.x == 0) part[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void loss_reduce_kernel(const float* __restrict__ part, int nb, int64_t n,
                                                          float* __restrict__ loss) {
  __shared__ float red[4];
  float acc = 0.f;
  for (int i = threadIdx.x; i < nb; i += 256) acc += part[i];
  acc = block_sum256(acc, red);
  if (threadIdx.x == 0) *loss = acc / (float)n;
}

}  // namespace

// ==================================================================== launchers
hipError_t transpose_bf16(const bf16* in, int64_t ldi, bf16* out, int64_t ldo, int R, int C, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3((C + 63) / 64, (R + 63) / 64), dim3(256), 0, s, in, ldi, out, ldo, R, C);
  return hipGetLastError();
}

hipError_t transpose_many(const TransposeJob* jobs, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n > TRANSPOSE_MAX_JOBS) return hipErrorInvalidValue;
  TransposeJobs jb{};
  int tiles = 0;
  for (int i = 0; i < n; ++i) {
    jb.in[i] = jobs[i].in; jb.out[i] = jobs[i].out; jb.ldi[i] = jobs[i].ldi; jb.ldo[i] = jobs[i].ldo;
    jb.R[i] = jobs[i].R; jb.C[i] = jobs[i].C;
    jb.start[i] = tiles;
    tiles += ((jobs[i].R + 63) / 64) * ((jobs[i].C + 63) / 64);
  }
  jb.start[n] = tiles;
  jb.n = n;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_many_kernel, dim3(tiles), dim3(256), 0, s, jb);
  return hipGetLastError();
}

hipError_t cast_f32_bf16(const float* x, bf16* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_kernel, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

hipError_t rmsnorm_bwd(const float* x, const bf16* g, const bf16* dy, const float* base, float* out, int rows, int D,
                       float eps, hipStream_t s, bf16* outb) {
  if (rows <= 0) return hipSuccess;
  if (D % 4 == 0 && aligned16(x) && aligned16(out) && (!base || aligned16(base)) && ((uintptr_t)g & 7) == 0 &&
      ((uintptr_t)dy & 7) == 0 && ((uintptr_t)outb & 7) == 0) {
    hipLaunchKernelGGL(rmsnorm_bwd4_kernel, dim3(rows), dim3(256), 0, s, x, g, dy, base, out, outb, D, eps);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3(rows), dim3(256), 0, s, x, g, dy, base, out, D, eps);
  if (outb) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return cast_f32_bf16(out, outb, (int64_t)rows * D, s);
  }
  return hipGetLastError();
}

hipError_t swiglu_fwd(const bf16* gu, bf16* z, int64_t ldz, int M, int I, hipStream_t s) {
  const int64_t n = (int64_t)M * I;
  if (n <= 0) return hipSuccess;
  if (ldz < I) return hipErrorInvalidValue;
  if (I % 8 == 0 && ldz % 8 == 0 && aligned16(gu) && aligned16(z)) {
    const int64_t n8 = n / 8;
    hipLaunchKernelGGL(swiglu8_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, gu, z, ldz, I, n8);
  } else {
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gu, z, ldz, I, n);
  }
  return hipGetLastError();
}

hipError_t swiglu_bwd(const bf16* gu, const bf16* dz, bf16* dgu, int64_t ldg, int M, int I, hipStream_t s) {
  const int64_t n = (int64_t)M * I;
  if (n <= 0) return hipSuccess;
  if (ldg < 2 * (int64_t)I) return hipErrorInvalidValue;
  if (I % 8 == 0 && ldg % 8 == 0 && aligned16(gu) && aligned16(dz) && aligned16(dgu)) {
    const int64_t n8 = n / 8;
    hipLaunchKernelGGL(swiglu8_bwd_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, gu, dz, dgu, ldg, I, n8);
  } else {
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gu, dz, dgu, ldg, I, n);
  }
  return hipGetLastError();
}

hipError_t qknorm_rope_bwd(const bf16* raw, int64_t ldr, const float* dq, const float* dk, const float* dv,
                           const SeqInfo& si, int Hq, int Hkv, int d, const bf16* gq, const bf16* gk,
                           const float2* table, float eps, bf16* dqkv, int64_t ldo, hipStream_t s) {
  const int64_t total = (int64_t)si.B * si.N * (Hq + 2 * Hkv);
  if (total == 0) return hipSuccess;
  if (d > 128 || d % 2) return hipErrorInvalidValue;
  const bool vec = d == 128 && ldr % 8 == 0 && ldo % 8 == 0 && ((uintptr_t)raw & 15) == 0 && ((uintptr_t)dqkv & 15) == 0 &&
                   ((uintptr_t)dq & 15) == 0 && ((uintptr_t)dk & 15) == 0 && ((uintptr_t)dv & 15) == 0 &&
                   ((uintptr_t)gq & 7) == 0 && ((uintptr_t)gk & 7) == 0;
  if (vec)
    hipLaunchKernelGGL(qknorm_rope_bwd128_kernel, dim3((unsigned)((total + 15) / 16)), dim3(256), 0, s, raw, ldr, dq, dk,
                       dv, si, Hq, Hkv, gq, gk, table, eps, dqkv, ldo, total);
  else
    hipLaunchKernelGGL(qknorm_rope_bwd_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, raw, ldr, dq, dk, dv,
                       si, Hq, Hkv, d, gq, gk, table, eps, dqkv, ldo, total);
  return hipGetLastError();
}

hipError_t attention_bwd(const bf16* qkv, int64_t ldq, const SeqInfo& si, int Hq, int Hkv, int d, const bf16* O,
                         const bf16* dO, const float* lse, float* Dq, float* dq, float* dk, float* dv, hipStream_t s) {
  const int N = si.N, B = si.B;
  if (N == 0) return hipSuccess;
  if (d != 128) return hipErrorInvalidValue;
  const int64_t QD = (int64_t)Hq * d;
  const int64_t tot = (int64_t)B * N * Hq;
  if (QD % 8 == 0 && ((uintptr_t)dO & 15) == 0 && ((uintptr_t)O & 15) == 0)
    hipLaunchKernelGGL(attn_bwd_dot128_kernel, dim3((unsigned)((tot + 15) / 16)), dim3(256), 0, s, dO, O, QD, Hq, N, Dq, tot);
  else
    hipLaunchKernelGGL(attn_bwd_dot_kernel, dim3((unsigned)((tot + 3) / 4)), dim3(256), 0, s, dO, O, QD, Hq, d, N, Dq, tot);
  const float scale = 1.0f / sqrtf((float)d);
  const float scale_log2 = 1.4426950408889634f * scale;
  const int nkb = (N + 127) / 128, nqb = (N + 31) / 32;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, dim3(B * Hkv * nkb), dim3(256), 0, s, qkv, ldq, si, Hq, Hkv, dO, QD,
                     lse, (const float*)Dq, scale_log2, scale, dk, dv, nkb);
  const int G = Hq / Hkv, hpw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1);
  const int nqg = (nqb + 4 / hpw - 1) / (4 / hpw);
  hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, dim3(B * Hkv * (G / hpw) * nqg), dim3(256), 0, s, qkv, ldq, si, Hq, Hkv,
                     dO, QD, lse, (const float*)Dq, scale_log2, scale, dq, hpw, nqg);
  return hipGetLastError();
}

int wgrad_splits(int M, int N1, int N2) {
  const int tiles = ((N1 + 63) / 64) * ((N2 + 63) / 64);
  int splits = std::max(1, 1024 / std::max(tiles, 1));
  splits = std::min(splits, std::max(1, (M + 255) / 256));
  return splits;
}

// One side is the rank: stream the other side in 128-column blocks, about 512 workgroups, the
// partial products [nz, N1, N2] within WGRAD_PART_FLOATS.  Returns nz.
static int wgrad_lr_launch(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, int N1, int N2, float* part,
                           hipStream_t s, int bseg1 = 1 << 30, int bseg2 = 1 << 30, int sm_step = 0) {
  const int64_t n = (int64_t)N1 * N2;
  const int R = std::min(N1, N2), NB = std::max(N1, N2);
  const int nblk = (NB + 127) / 128;
  int splits = std::max(1, 512 / nblk);
  splits = std::min(splits, std::max(1, (M + 127) / 128));
  splits = (int)std::min<int64_t>(splits, std::max<int64_t>(1, WGRAD_PART_FLOATS / n));
  const int per = ((M + splits - 1) / splits + 31) / 32 * 32;
  const int nz = (M + per - 1) / per;
  if (N1 >= N2)
    hipLaunchKernelGGL(wgrad_lr_kernel<true>, dim3(nblk, nz), dim3(256), 0, s, X, ldx, Y, ldy, M, NB, R, per, part, bseg1,
                       bseg2, sm_step);
  else
    hipLaunchKernelGGL(wgrad_lr_kernel<false>, dim3(nblk, nz), dim3(256), 0, s, Y, ldy, X, ldx, M, NB, R, per, part, bseg1,
                       bseg2, sm_step);
  return nz;
}

hipError_t wgrad_seg(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, int N1, int N2, int seg_rows,
                     float* const* C, float* part, hipStream_t s) {
  if (M <= 0 || N1 <= 0 || N2 <= 0) return hipSuccess;
  if (N1 % 8 || N2 % 8 || ldx % 8 || ldy % 8 || N1 > 128 || seg_rows <= 0 || N1 % seg_rows || N1 / seg_rows > 3)
    return hipErrorInvalidValue;
  const int64_t n = (int64_t)N1 * N2;
  const int nz = wgrad_lr_launch(X, ldx, Y, ldy, M, N1, N2, part, s);
  const int ns = N1 / seg_rows;
  const int64_t seg = (int64_t)seg_rows * N2;
  hipLaunchKernelGGL(wgrad_reduce_seg_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)part, nz,
                     n, seg, ns > 2 ? 2 * seg : n, C[0], ns > 1 ? C[1] : C[0], ns > 2 ? C[2] : C[0]);
  return hipGetLastError();
}

hipError_t wgrad_diag(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, const int* outs, int ns, int r,
                      float* const* C, float* part, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (ns < 1 || ns > 3 || r <= 0 || r > 128 || r % 8 || ldx % 8 || ldy % 8) return hipErrorInvalidValue;
  int N1 = 0;
  for (int i = 0; i < ns; ++i) {
    if (outs[i] <= 0 || outs[i] % 128) return hipErrorInvalidValue;
    N1 += outs[i];
  }
  if (N1 < r) return hipErrorInvalidValue;
  const int b1 = outs[0], b2 = ns > 2 ? outs[0] + outs[1] : (1 << 30);
  const int64_t n = (int64_t)N1 * r;
  const int nz = wgrad_lr_launch(X, ldx, Y, ldy, M, N1, r, part, s, ns > 1 ? b1 : (1 << 30), b2, r);
  const int64_t e1 = ns > 1 ? (int64_t)b1 * r : n, e2 = ns > 2 ? (int64_t)b2 * r : n;
  hipLaunchKernelGGL(wgrad_reduce_seg_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)part, nz,
                     n, e1, e2, C[0], ns > 1 ? C[1] : C[0], ns > 2 ? C[2] : C[0]);
  return hipGetLastError();
}

hipError_t wgrad(const bf16* X, int64_t ldx, const bf16* Y, int64_t ldy, int M, int N1, int N2, float* C, float* part,
                 hipStream_t s) {
  if (M <= 0 || N1 <= 0 || N2 <= 0) return hipSuccess;
  if (N1 % 8 || N2 % 8 || ldx % 8 || ldy % 8) return hipErrorInvalidValue;
  const int64_t n = (int64_t)N1 * N2;
  if (std::min(N1, N2) <= 128) {
    const int nz = wgrad_lr_launch(X, ldx, Y, ldy, M, N1, N2, part, s);
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)part, nz, n,
                       C);
    return hipGetLastError();
  }
  const int splits = wgrad_splits(M, N1, N2);
  const int per = ((M + splits - 1) / splits + 63) / 64 * 64;
  const int nz = (M + per - 1) / per;
  hipLaunchKernelGGL(wgrad_kernel, dim3((N1 + 63) / 64, (N2 + 63) / 64, nz), dim3(256), 0, s, X, ldx, Y, ldy, M, N1, N2,
                     per, part);
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)part, nz, n, C);
  return hipGetLastError();
}

hipError_t x0_loss(const float* pred, const float* tgt, float* grad, float* part, int nparts, float* loss, int64_t n,
                   hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(x0_loss_kernel, dim3(nparts), dim3(256), 0, s, pred, tgt, grad, part, n);
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(256), 0, s, (const float*)part, nparts, n, loss);
  return hipGetLastError();
}

}  // namespace psf
