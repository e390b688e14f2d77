// Memory-bound kernels of the gen-tower step: RMSNorm, fused QK-norm + RoPE, RoPE table,
// K/V packing for attention, patchify, timestep embedding and the CFG + Euler update.
// All use 16-byte vector accesses along the contiguous axis; arithmetic is fp32.
#include "common.h"
#include "kernels.h"

namespace psf {
namespace {

// ---- 16-byte vectors of T: 8 bf16 or 4 float
template <typename T> struct V16;
template <> struct V16<bf16> {
  static constexpr int N = 8;
  static DEVI void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  static DEVI u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<bf16>(f[2 * i]));
      const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<bf16>(f[2 * i + 1]));
      v[i] = lo | (hi << 16);
    }
    return v;
  }
};
template <> struct V16<float> {
  static constexpr int N = 4;
  static DEVI void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  static DEVI u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};

// ---------------------------------------------------------------- RMSNorm
// One 256-thread workgroup per row; the row stays in registers between the two passes.
// Input chunks are 16 bytes of Tin; when Tin is wider than T (fp32 residual in, bf16 out)
// a chunk covers 4 elements and is written as 8 bytes.
template <typename Tin, typename T, int CH>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const Tin* __restrict__ x, const T* __restrict__ g,
                                                      T* __restrict__ y, int D, float eps) {
  using V = V16<Tin>;
  const int nch = D / V::N;
  const int64_t base = (int64_t)blockIdx.x * D;
  u32x4 buf[CH];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = threadIdx.x + c * 256;
    if (i < nch) {
      buf[c] = *(const u32x4*)(x + base + i * V::N);
      float f[V::N];
      V::unpack(buf[c], f);
#pragma unroll
      for (int e = 0; e < V::N; ++e) ss += f[e] * f[e];
    }
  }
  __shared__ float red[4];
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(tot / (float)D + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = threadIdx.x + c * 256;
    if (i < nch) {
      float f[V::N];
      V::unpack(buf[c], f);
#pragma unroll
      for (int e = 0; e < V::N; ++e) f[e] = f[e] * r * to_f(g[i * V::N + e]);
      if constexpr (sizeof(Tin) == sizeof(T)) {
        *(u32x4*)(y + base + i * V::N) = V::pack(f);
      } else {
#pragma unroll
        for (int e = 0; e < V::N; ++e) y[base + i * V::N + e] = from_f<T>(f[e]);
      }
    }
  }
}

// ---------------------------------------------------------------- RoPE table
__global__ void rope_table_kernel(float2* table, int n_pos, int half, double theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_pos * half) return;
  const int pos = i / half, j = i - pos * half;
  const double w = pow(theta, -2.0 * (double)j / (double)(2 * half));
  double sn, cs;
  sincos((double)pos * w, &sn, &cs);
  table[i] = make_float2((float)cs, (float)sn);
}

// ---------------------------------------------------------------- QK-norm + RoPE
// A head vector of d elements is spread over L = d / V::N lanes (16-byte chunks); a wave
// covers 64 / L head vectors.  Rotate-half pairs element j with j + d/2, which lives in
// lane ^ (L/2).
template <typename T, int D>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(T* __restrict__ qkv, int64_t ld, SeqInfo si, int Hq, int Hkv,
                                                          const T* __restrict__ gq, const T* __restrict__ gk,
                                                          const float2* __restrict__ table, float eps, int64_t total,
                                                          T* __restrict__ raw_out) {
  using V = V16<T>;
  constexpr int L = D / V::N;
  constexpr int HPW = 64 / L;
  const int lane = threadIdx.x & 63;
  const int64_t hv = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * HPW + lane / L;
  const int sub = lane % L;
  const bool active = hv < total;
  const int64_t hvc = active ? hv : 0;
  const int H = Hq + Hkv;
  const int64_t tok = hvc / H;
  const int head = (int)(hvc - tok * H);
  const int b = (int)(tok / si.N), n = (int)(tok - (int64_t)b * si.N);
  const int pos = si.plen[b] + n;
  T* p = qkv + tok * ld + (int64_t)head * D + sub * V::N;
  const T* g = (head < Hq ? gq : gk) + sub * V::N;
  float x[V::N], gg[V::N];
  const u32x4 raw = *(const u32x4*)p;
  if (raw_out && active) *(u32x4*)(raw_out + tok * ld + (int64_t)head * D + sub * V::N) = raw;   // pre-norm copy
  V::unpack(raw, x);
  V::unpack(*(const u32x4*)g, gg);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < V::N; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int e = 0; e < V::N; ++e) x[e] = x[e] * r * gg[e];
  float pr[V::N];
#pragma unroll
  for (int e = 0; e < V::N; ++e) pr[e] = __shfl_xor(x[e], L / 2, 64);
  const bool first = sub < L / 2;
  const int j0 = (sub % (L / 2)) * V::N;
  const float2* tb = table + (int64_t)pos * (D / 2) + j0;
  float out[V::N];
#pragma unroll
  for (int e = 0; e < V::N; ++e) {
    const float2 cs = tb[e];
    out[e] = first ? (x[e] * cs.x - pr[e] * cs.y) : (x[e] * cs.x + pr[e] * cs.y);
  }
  if (active && head < H) *(u32x4*)p = V::pack(out);
}

// ---------------------------------------------------------------- K/V packing
template <typename T>
__global__ __launch_bounds__(256) void pack_k_kernel(const T* __restrict__ qkv, int64_t ld, SeqInfo si, int Hq,
                                                     int Hkv, int d, int Lpad, T* __restrict__ Kc) {
  using V = V16<T>;
  const int cpr = d / V::N;                        // chunks per row
  const int b = blockIdx.z, g = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int j = t / cpr, c = t - j * cpr;
  if (j >= Lpad) return;
  const int P = si.plen[b];
  u32x4 v = {0, 0, 0, 0};
  if (j < P) v = *(const u32x4*)((const T*)si.pk[b] + ((int64_t)j * Hkv + g) * d + c * V::N);
  else if (j < P + si.N) v = *(const u32x4*)(qkv + ((int64_t)b * si.N + j - P) * ld + (int64_t)(Hq + g) * d + c * V::N);
  *(u32x4*)(Kc + (((int64_t)b * Hkv + g) * Lpad + j) * d + c * V::N) = v;
}

// Vt[b][g][dd][j0..j0+8): each lane gathers 8 keys of one head-dim column; a wave's loads
// of one key row are 64 consecutive elements.
template <typename T>
__global__ __launch_bounds__(256) void pack_vt_kernel(const T* __restrict__ qkv, int64_t ld, SeqInfo si, int Hq,
                                                      int Hkv, int d, int Lpad, T* __restrict__ Vt) {
  using V = V16<T>;
  const int b = blockIdx.z, g = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int dd = t % d, jc = t / d;
  const int j0 = jc * V::N;
  if (j0 >= Lpad) return;
  const int P = si.plen[b];
  float f[V::N];
#pragma unroll
  for (int e = 0; e < V::N; ++e) {
    // bf16 V^T stores each 16-key group as keys [0-3, 8-11, 4-7, 12-15]: the order in which the
    // attention kernel's P^T fragments arrive.  fp32 V^T keeps the natural order.
    const int pos = j0 + e;
    const int j = sizeof(T) == 2 ? (pos & ~15) | (((pos >> 2) & 1) << 3) | (((pos >> 3) & 1) << 2) | (pos & 3) : pos;
    float v = 0.f;
    if (j < P) v = to_f(((const T*)si.pv[b])[((int64_t)j * Hkv + g) * d + dd]);
    else if (j < P + si.N) v = to_f(qkv[((int64_t)b * si.N + j - P) * ld + (int64_t)(Hq + Hkv + g) * d + dd]);
    f[e] = v;
  }
  *(u32x4*)(Vt + (((int64_t)b * Hkv + g) * d + dd) * Lpad + j0) = V::pack(f);
}

// bf16 V^T of one (sequence, kv head, 64-key tile) through LDS: the tile's key rows come in as
// 16-byte vectors (prefix rows from the cache, image rows from qkv, zeros past the end), the V^T
// rows go out as 16-byte vectors, each 16-key group in the order [0-3, 8-11, 4-7, 12-15] as in
// pack_vt_kernel.  Lpad is a multiple of 64.
template <int D>
__global__ __launch_bounds__(256) void pack_vt_tile_kernel(const bf16* __restrict__ qkv, int64_t ld, SeqInfo si,
                                                           int Hq, int Hkv, int Lpad, bf16* __restrict__ Vt) {
  constexpr int CPR = D / 8;                // 16-byte chunks per key row
  constexpr int RS = D + 8;                 // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) bf16 tile[64 * RS];
  const int b = blockIdx.z, g = blockIdx.y, j0 = blockIdx.x * 64;
  const int P = si.plen[b], N = si.N;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, c = i - r * CPR;
    const int j = j0 + r;
    u32x4 v = {0, 0, 0, 0};
    if (j < P) v = *(const u32x4*)((const bf16*)si.pv[b] + ((int64_t)j * Hkv + g) * D + c * 8);
    else if (j < P + N) v = *(const u32x4*)(qkv + ((int64_t)b * N + j - P) * ld + (int64_t)(Hq + Hkv + g) * D + c * 8);
    *(u32x4*)(tile + r * RS + c * 8) = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int dd = i >> 3, kc = i & 7;
    bf16x8 e;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int pos = kc * 8 + q;
      const int j = (pos & ~15) | (((pos >> 2) & 1) << 3) | (((pos >> 3) & 1) << 2) | (pos & 3);
      e[q] = tile[j * RS + dd];
    }
    *(bf16x8*)(Vt + (((int64_t)b * Hkv + g) * D + dd) * Lpad + j0 + kc * 8) = e;
  }
}

// K and V^T of one (sequence, kv head, 64-key tile) in one workgroup.  K as pack_k_kernel, with each
// image key RMS-normalised (gain gk) and rotated (RoPE at its packed index j): one key row per L =
// d / 8 lanes (16-byte chunks), as in qknorm_rope_kernel, every lane running the arithmetic and the
// row kind picking the stored value; then V^T as pack_vt_tile_kernel.
template <int D>
__global__ __launch_bounds__(256) void pack_kv_knorm_tile_kernel(const bf16* __restrict__ qkv, int64_t ld, SeqInfo si,
                                                                 int Hq, int Hkv, int Lpad, const bf16* __restrict__ gk,
                                                                 const float2* __restrict__ table, float eps,
                                                                 bf16* __restrict__ Kc, bf16* __restrict__ Vt) {
  using V = V16<bf16>;
  constexpr int L = D / V::N;               // lanes per key row
  constexpr int RPP = 256 / L;              // key rows per pass
  constexpr int CPR = D / 8;
  constexpr int RS = D + 8;
  __shared__ __attribute__((aligned(16))) bf16 tile[64 * RS];
  const int b = blockIdx.z, g = blockIdx.y, j0 = blockIdx.x * 64;
  const int P = si.plen[b], N = si.N;
  const int lane = threadIdx.x & 63, sub = lane % L;
  float gg[V::N];
  V::unpack(*(const u32x4*)(gk + sub * V::N), gg);
  for (int r0 = 0; r0 < 64; r0 += RPP) {
    const int j = j0 + r0 + threadIdx.x / L;
    const int kind = j < P ? 0 : (j < P + N ? 1 : 2);      // prefix, image, padding
    u32x4 raw = {0, 0, 0, 0};
    if (kind == 0) raw = *(const u32x4*)((const bf16*)si.pk[b] + ((int64_t)j * Hkv + g) * D + sub * V::N);
    else if (kind == 1) raw = *(const u32x4*)(qkv + ((int64_t)b * N + j - P) * ld + (int64_t)(Hq + g) * D + sub * V::N);
    float x[V::N];
    V::unpack(raw, x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < V::N; ++e) ss += x[e] * x[e];
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int e = 0; e < V::N; ++e) x[e] = x[e] * r * gg[e];
    float pr[V::N];
#pragma unroll
    for (int e = 0; e < V::N; ++e) pr[e] = __shfl_xor(x[e], L / 2, 64);
    const bool first = sub < L / 2;
    const int jj = (sub % (L / 2)) * V::N;
    const float2* tb = table + (int64_t)(kind == 1 ? j : 0) * (D / 2) + jj;
    float out[V::N];
#pragma unroll
    for (int e = 0; e < V::N; ++e) {
      const float2 cs = tb[e];
      out[e] = first ? (x[e] * cs.x - pr[e] * cs.y) : (x[e] * cs.x + pr[e] * cs.y);
    }
    *(u32x4*)(Kc + (((int64_t)b * Hkv + g) * Lpad + j) * D + sub * V::N) = kind == 1 ? V::pack(out) : raw;
  }
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, c = i - r * CPR;
    const int j = j0 + r;
    u32x4 v = {0, 0, 0, 0};
    if (j < P) v = *(const u32x4*)((const bf16*)si.pv[b] + ((int64_t)j * Hkv + g) * D + c * 8);
    else if (j < P + N) v = *(const u32x4*)(qkv + ((int64_t)b * N + j - P) * ld + (int64_t)(Hq + Hkv + g) * D + c * 8);
    *(u32x4*)(tile + r * RS + c * 8) = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int dd = i >> 3, kc = i & 7;
    bf16x8 e;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int pos = kc * 8 + q;
      const int j = (pos & ~15) | (((pos >> 2) & 1) << 3) | (((pos >> 3) & 1) << 2) | (pos & 3);
      e[q] = tile[j * RS + dd];
    }
    *(bf16x8*)(Vt + (((int64_t)b * Hkv + g) * D + dd) * Lpad + j0 + kc * 8) = e;
  }
}

hipError_t pack_vt_bf16(const bf16* qkv, int64_t ld, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad, bf16* Vt,
                        hipStream_t s) {
  const dim3 grid(Lpad / 64, Hkv, si.B);
  if (d == 128) hipLaunchKernelGGL((pack_vt_tile_kernel<128>), grid, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, Lpad, Vt);
  else if (d == 64) hipLaunchKernelGGL((pack_vt_tile_kernel<64>), grid, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, Lpad, Vt);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------- LoRA merge
// Wo[o, i] = W[o, i] + scale * sum_r B[o, r] A[r, i] for a [64 x 256] tile per workgroup: the
// 64 rows of B sit in LDS (every lane reads the same entry), each lane owns one column i and
// keeps 64 fp32 sums; the sum is added to W in fp32 and rounded once.  A == nullptr copies W.
// W and Wo have row pitch ldw (>= in).
template <typename T>
__global__ __launch_bounds__(256) void lora_merge_kernel(const T* __restrict__ W, const T* __restrict__ A,
                                                         const T* __restrict__ B, T* __restrict__ Wo, int out, int in,
                                                         int64_t ldw, int rank, float scale) {
  __shared__ float Bs[64][129];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int o0 = blockIdx.y * 64;
  const int nrow = min(64, out - o0);
  if (A) {
    for (int t = threadIdx.x; t < 64 * rank; t += 256) {
      const int o = t / rank, r = t - o * rank;
      Bs[o][r] = o < nrow ? to_f(B[(int64_t)(o0 + o) * rank + r]) : 0.f;
    }
  }
  __syncthreads();
  if (i >= in) return;
  float acc[64];
#pragma unroll
  for (int o = 0; o < 64; ++o) acc[o] = 0.f;
  if (A) {
    for (int rc = 0; rc < rank; rc += 8) {
      float a[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) a[k] = to_f(A[(int64_t)(rc + k) * in + i]);
#pragma unroll
      for (int o = 0; o < 64; ++o)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[o] = fmaf(Bs[o][rc + k], a[k], acc[o]);
    }
  }
#pragma unroll
  for (int o = 0; o < 64; ++o)
    if (o < nrow) {
      const int64_t at = (int64_t)(o0 + o) * ldw + i;
      Wo[at] = from_f<T>(fmaf(scale, acc[o], to_f(W[at])));
    }
}

// ---------------------------------------------------------------- patchify
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(const float* __restrict__ x, T* __restrict__ out, int n_img,
                                                       int H, int W, int64_t total) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t tok = t / 384;
  const int f0 = (int)(t - tok * 384) * 8;
  const int pw = W >> 5, N = (H >> 5) * pw;
  const int i = (int)(tok / N), n = (int)(tok - (int64_t)i * N);
  const int py = n / pw, px = n - py * pw;
  const int c = f0 >> 10, iy = (f0 >> 5) & 31, ix = f0 & 31;
  const float* src = x + (((int64_t)i * 3 + c) * H + py * 32 + iy) * W + px * 32 + ix;
  const float4 a = *(const float4*)src, bq = *(const float4*)(src + 4);
  T* dst = out + tok * 3072 + f0;
  const float v[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = from_f<T>(v[e]);
}

// ---------------------------------------------------------------- timestep embedding
struct Sigmas { float s[MAXB]; };

template <typename T>
__global__ __launch_bounds__(256) void temb1_kernel(Sigmas sg, const T* __restrict__ w1, float* __restrict__ h1, int D) {
  __shared__ float feat[256];
  const int i = blockIdx.y;
  {
    const int k = threadIdx.x;
    const int j = k & 127;
    const double f = exp(-log(10000.0) * (double)j / 128.0);
    const double a = 1000.0 * (double)sg.s[i] * f;
    feat[k] = (float)(k < 128 ? cos(a) : sin(a));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= D) return;
  float acc = 0.f;
  for (int k = lane; k < 256; k += 64) acc += to_f(w1[(int64_t)row * 256 + k]) * feat[k];
  acc = warp_sum(acc);
  if (lane == 0) h1[(int64_t)i * D + row] = acc / (1.0f + expf(-acc));
}

template <typename T>
__global__ __launch_bounds__(256) void temb2_kernel(const T* __restrict__ w2, const float* __restrict__ h1,
                                                    float* __restrict__ temb, int D) {
  const int i = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= D) return;
  float acc = 0.f;
  for (int k = lane; k < D; k += 64) acc += to_f(w2[(int64_t)row * D + k]) * h1[(int64_t)i * D + k];
  acc = warp_sum(acc);
  if (lane == 0) temb[(int64_t)i * D + row] = acc;
}

// ---------------------------------------------------------------- CFG + Euler
// Guided prediction g per pixel, then x' = x + dt (x - g) / den.
//   MIX 0: g = c;   MIX 1: g = u + s (c - u);   MIX 2 (three branches, c / i / u = cond /
//   img_cond / uncond): g = u + s_img (i - u) + s (c - i).
DEVI float guide(int mix, float c, float i, float u, float s, float si) {
  return mix == 0 ? c : (mix == 1 ? u + s * (c - u) : u + si * (i - u) + s * (c - i));
}
template <int MIX>
__global__ __launch_bounds__(256) void cfg_euler_kernel(float* xo, const float* xi, const float* __restrict__ xc,
                                                        const float* __restrict__ xm, const float* __restrict__ xu,
                                                        size_t n, float scale, float iscale, float dt, float den) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    float4 a = *(const float4*)(xi + i);
    const float4 c = *(const float4*)(xc + i);
    float4 m = c, u = c;
    if (MIX == 2) m = *(const float4*)(xm + i);
    if (MIX >= 1) u = *(const float4*)(xu + i);
    const float4 g = make_float4(guide(MIX, c.x, m.x, u.x, scale, iscale), guide(MIX, c.y, m.y, u.y, scale, iscale),
                                 guide(MIX, c.z, m.z, u.z, scale, iscale), guide(MIX, c.w, m.w, u.w, scale, iscale));
    a.x = a.x + dt * ((a.x - g.x) / den);
    a.y = a.y + dt * ((a.y - g.y) / den);
    a.z = a.z + dt * ((a.z - g.z) / den);
    a.w = a.w + dt * ((a.w - g.w) / den);
    *(float4*)(xo + i) = a;
  } else {
    for (size_t k = i; k < n; ++k) {
      const float g = guide(MIX, xc[k], MIX == 2 ? xm[k] : 0.f, MIX >= 1 ? xu[k] : 0.f, scale, iscale);
      xo[k] = xi[k] + dt * ((xi[k] - g) / den);
    }
  }
}

struct KVCacheOut {
  void* k[MAXB];
  void* v[MAXB];
};

// grid (chunk blocks, B, 2): z = 0 copies the keys, z = 1 the values of sequence y
template <typename T>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(const T* __restrict__ qkv, int64_t ld, int QD, int N,
                                                             int row_elems, KVCacheOut out) {
  constexpr int V = 16 / sizeof(T);
  const int cpr = row_elems / V;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)N * cpr) return;
  const int b = blockIdx.y, which = blockIdx.z;
  const int n = (int)(c / cpr), ch = (int)(c - (int64_t)n * cpr);
  const T* src = qkv + ((int64_t)b * N + n) * ld + QD + which * row_elems + ch * V;
  T* dst = (T*)(which ? out.v[b] : out.k[b]) + (int64_t)n * row_elems + ch * V;
  *(u32x4*)dst = *(const u32x4*)src;
}

}  // namespace

// ================================================================== launchers
template <typename Tin, typename T>
hipError_t rmsnorm(const Tin* x, const T* g, T* y, int rows, int D, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int nch = D / V16<Tin>::N;
  if (nch <= 256) hipLaunchKernelGGL((rmsnorm_kernel<Tin, T, 1>), dim3(rows), dim3(256), 0, s, x, g, y, D, eps);
  else if (nch <= 512) hipLaunchKernelGGL((rmsnorm_kernel<Tin, T, 2>), dim3(rows), dim3(256), 0, s, x, g, y, D, eps);
  else if (nch <= 1024) hipLaunchKernelGGL((rmsnorm_kernel<Tin, T, 4>), dim3(rows), dim3(256), 0, s, x, g, y, D, eps);
  else if (nch <= 2048) hipLaunchKernelGGL((rmsnorm_kernel<Tin, T, 8>), dim3(rows), dim3(256), 0, s, x, g, y, D, eps);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
template hipError_t rmsnorm<bf16, bf16>(const bf16*, const bf16*, bf16*, int, int, float, hipStream_t);
template hipError_t rmsnorm<float, float>(const float*, const float*, float*, int, int, float, hipStream_t);
template hipError_t rmsnorm<float, bf16>(const float*, const bf16*, bf16*, int, int, float, hipStream_t);

hipError_t rope_table(float2* table, int n_pos, int head_dim, float theta, hipStream_t s) {
  const int half = head_dim / 2;
  const int total = n_pos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, s, table, n_pos, half, (double)theta);
  return hipGetLastError();
}

template <typename T>
hipError_t qknorm_rope(T* qkv, int64_t ld, const SeqInfo& si, int Hq, int Hkv, int d, const T* gq, const T* gk,
                       const float2* table, float eps, hipStream_t s, T* raw_out) {
  const int64_t total = (int64_t)si.B * si.N * (Hq + Hkv);
  if (total == 0) return hipSuccess;
  const int L = d / V16<T>::N;
  const int64_t per_block = 4 * (64 / L);
  const dim3 grid((unsigned)((total + per_block - 1) / per_block));
  if (d == 128) hipLaunchKernelGGL((qknorm_rope_kernel<T, 128>), grid, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, gq, gk, table, eps, total, raw_out);
  else if (d == 64) hipLaunchKernelGGL((qknorm_rope_kernel<T, 64>), grid, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, gq, gk, table, eps, total, raw_out);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
template hipError_t qknorm_rope<bf16>(bf16*, int64_t, const SeqInfo&, int, int, int, const bf16*, const bf16*, const float2*, float, hipStream_t, bf16*);
template hipError_t qknorm_rope<float>(float*, int64_t, const SeqInfo&, int, int, int, const float*, const float*, const float2*, float, hipStream_t, float*);

template <typename T>
hipError_t kv_cache_write(const T* qkv, int64_t ld, int QD, int N, int row_elems, int B, void* const* kcache,
                          void* const* vcache, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  if (B <= 0 || N <= 0) return hipSuccess;
  if (B > MAXB || row_elems % V || QD % V || ld % V) return hipErrorInvalidValue;
  KVCacheOut out;
  for (int b = 0; b < B; ++b) {
    out.k[b] = kcache[b];
    out.v[b] = vcache[b];
  }
  const int64_t chunks = (int64_t)N * (row_elems / V);
  hipLaunchKernelGGL(kv_cache_write_kernel<T>, dim3((unsigned)((chunks + 255) / 256), B, 2), dim3(256), 0, s, qkv, ld,
                     QD, N, row_elems, out);
  return hipGetLastError();
}
template hipError_t kv_cache_write<bf16>(const bf16*, int64_t, int, int, int, int, void* const*, void* const*, hipStream_t);
template hipError_t kv_cache_write<float>(const float*, int64_t, int, int, int, int, void* const*, void* const*, hipStream_t);

template <typename T>
hipError_t pack_kv(const T* qkv, int64_t ld, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad, T* Kc, T* Vt,
                   hipStream_t s) {
  const int cpr = d / V16<T>::N;
  dim3 gk((Lpad * cpr + 255) / 256, Hkv, si.B);
  hipLaunchKernelGGL(pack_k_kernel<T>, gk, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, d, Lpad, Kc);
  if (sizeof(T) == 2) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return pack_vt_bf16((const bf16*)qkv, ld, si, Hq, Hkv, d, Lpad, (bf16*)Vt, s);
  }
  dim3 gv((d * (Lpad / V16<T>::N) + 255) / 256, Hkv, si.B);
  hipLaunchKernelGGL(pack_vt_kernel<T>, gv, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, d, Lpad, Vt);
  return hipGetLastError();
}
hipError_t pack_kv_knorm(const bf16* qkv, int64_t ld, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad,
                         const bf16* gk, const float2* table, float eps, bf16* Kc, bf16* Vt, hipStream_t s) {
  if ((int64_t)si.B * Hkv * Lpad == 0) return hipSuccess;
  const dim3 g2(Lpad / 64, Hkv, si.B);
  if (d == 128)
    hipLaunchKernelGGL((pack_kv_knorm_tile_kernel<128>), g2, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, Lpad, gk, table, eps, Kc, Vt);
  else if (d == 64)
    hipLaunchKernelGGL((pack_kv_knorm_tile_kernel<64>), g2, dim3(256), 0, s, qkv, ld, si, Hq, Hkv, Lpad, gk, table, eps, Kc, Vt);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
template <typename T>
hipError_t lora_merge(const T* W, const T* A, const T* B, T* Wo, int out, int in, int64_t ldw, int rank, float scale,
                      hipStream_t s) {
  if (out <= 0 || in <= 0) return hipSuccess;
  dim3 grid((in + 255) / 256, (out + 63) / 64);
  hipLaunchKernelGGL(lora_merge_kernel<T>, grid, dim3(256), 0, s, W, A, B, Wo, out, in, ldw, rank, scale);
  return hipGetLastError();
}
template hipError_t lora_merge<bf16>(const bf16*, const bf16*, const bf16*, bf16*, int, int, int64_t, int, float, hipStream_t);
template hipError_t lora_merge<float>(const float*, const float*, const float*, float*, int, int, int64_t, int, float, hipStream_t);

template hipError_t pack_kv<bf16>(const bf16*, int64_t, const SeqInfo&, int, int, int, int, bf16*, bf16*, hipStream_t);
template hipError_t pack_kv<float>(const float*, int64_t, const SeqInfo&, int, int, int, int, float*, float*, hipStream_t);

template <typename T>
hipError_t patchify(const float* x, T* patches, int n_img, int H, int W, hipStream_t s) {
  const int64_t total = (int64_t)n_img * (H / 32) * (W / 32) * 384;
  hipLaunchKernelGGL(patchify_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, x, patches, n_img, H, W, total);
  return hipGetLastError();
}
template hipError_t patchify<bf16>(const float*, bf16*, int, int, int, hipStream_t);
template hipError_t patchify<float>(const float*, float*, int, int, int, hipStream_t);

template <typename T>
hipError_t timestep_embed(const float* sigma_host, const T* w1, const T* w2, float* h1, float* temb, int n_img, int D,
                          hipStream_t s) {
  Sigmas sg;
  for (int i = 0; i < MAXB; ++i) sg.s[i] = i < n_img ? sigma_host[i] : 0.f;
  dim3 grid((D + 3) / 4, n_img);
  hipLaunchKernelGGL(temb1_kernel<T>, grid, dim3(256), 0, s, sg, w1, h1, D);
  hipLaunchKernelGGL(temb2_kernel<T>, grid, dim3(256), 0, s, w2, h1, temb, D);
  return hipGetLastError();
}
template hipError_t timestep_embed<bf16>(const float*, const bf16*, const bf16*, float*, float*, int, int, hipStream_t);
template hipError_t timestep_embed<float>(const float*, const float*, const float*, float*, float*, int, int, hipStream_t);

hipError_t cfg_euler(float* xo, const float* x, const float* xc, const float* xm, const float* xu, size_t n,
                     float scale, float img_scale, float sigma, float sigma_next, float t_eps, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const float dt = sigma_next - sigma;
  const float den = sigma > t_eps ? sigma : t_eps;
  const unsigned grid = (unsigned)((n + 1023) / 1024);
  if (xm && xu && img_scale != 1.0f)
    hipLaunchKernelGGL(cfg_euler_kernel<2>, dim3(grid), dim3(256), 0, s, xo, x, xc, xm, xu, n, scale, img_scale, dt, den);
  else if (xm && scale != 1.0f)   // image guidance off: two-branch guidance of cond against img_cond
    hipLaunchKernelGGL(cfg_euler_kernel<1>, dim3(grid), dim3(256), 0, s, xo, x, xc, xm, xm, n, scale, 1.0f, dt, den);
  else if (!xm && xu && scale != 1.0f)
    hipLaunchKernelGGL(cfg_euler_kernel<1>, dim3(grid), dim3(256), 0, s, xo, x, xc, xu, xu, n, scale, 1.0f, dt, den);
  else
    hipLaunchKernelGGL(cfg_euler_kernel<0>, dim3(grid), dim3(256), 0, s, xo, x, xc, xc, xc, n, 1.0f, 1.0f, dt, den);
  return hipGetLastError();
}

}  // namespace psf

