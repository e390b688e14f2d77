// Routed expert MLP support for the A3B gen block: softmax router (fp32, from the fp32 residual
// through the post-attention RMSNorm) with top-k and renormalised weights, a deterministic
// counting sort of (token, slot) assignments by expert with the grouped-GEMM tile table, and the
// fixed-order weighted combine.
// No floating-point atomics anywhere: results are bitwise reproducible.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace psf {
namespace {

// Router over a tile of RT tokens per workgroup.  With a gain g the logits are those of the
// RMS-normalised row, computed in one pass over x in fp32:
//   logit[t, e] = rs_t sum_c x[t, c] (g[c] w[e, c]),  rs_t = 1 / sqrt(mean_c x[t, c]^2 + eps)
// (g == nullptr: logit = sum_c x[t, c] w[e, c], x already normalised).  256-column chunks of x
// and of g w are staged in LDS as fp32, the next chunk's values loaded into registers while the
// current one is consumed; thread (t, eq) accumulates token t = tid % 16 against experts
// eq + 16 j (eq = tid / 16, j < EJ).  Then one wave per token: softmax, top-k by repeated wave
// argmax of the logit (the softmax is monotone; ties to the lower expert index), weights
// renormalised over the k, and each assignment's stable rank among the workgroup's assignments
// of the same expert (assignment order t k + slot) with the workgroup's per-expert counts, so
// that the sort needs no second pass over the assignments.
constexpr int RT = 16;          // tokens per router workgroup
constexpr int RCH = 256;        // columns per staged chunk
constexpr int RST = RCH + 4;    // padded fp32 row stride (1040 B: 16 consecutive rows hit 16 distinct 16-byte slots)

// 16 consecutive elements (16-byte aligned) as floats
DEVI void load16(const float* p, float* f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *(const float4*)(p + 4 * q);
    f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
  }
}
DEVI void load16(const bf16* p, float* f) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const bf16x8 v = *(const bf16x8*)(p + 8 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[8 * q + e] = static_cast<float>(v[e]);
  }
}

template <typename Tx, typename Tw, int EJ>
__global__ __launch_bounds__(256) void route_kernel(const Tx* __restrict__ x, const Tw* __restrict__ g, float eps,
                                                    const Tw* __restrict__ wr, int T_, int D, int E, int k,
                                                    int* __restrict__ idx, float* __restrict__ w,
                                                    int* __restrict__ lrank, int* __restrict__ blkcnt) {
  __shared__ __attribute__((aligned(16))) float xs[RT * RST];
  __shared__ __attribute__((aligned(16))) float gw[16 * EJ * RST];
  __shared__ float lg[RT * 65];
  __shared__ float rs[RT];
  __shared__ int sel[RT * 64];
  __shared__ int cnt[64], wtot[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tq = tid & 15, eq = tid >> 4;
  const int t0 = blockIdx.x * RT;
  float acc[EJ];
#pragma unroll
  for (int j = 0; j < EJ; ++j) acc[j] = 0.f;
  float ss = 0.f;
  // staging roles: x row eq and g w rows eq + 16 j, columns 16 tq .. 16 tq + 15 of each chunk
  const Tx* xrow = x + (int64_t)min(t0 + eq, T_ - 1) * D + 16 * tq;
  float xn[16], wn[EJ][16], gn[16];
  // a thread's 16 columns lie wholly inside or wholly past D (D is a multiple of 16); past it
  // they stage as zeros
  auto fetch = [&](int c0) {
    const bool in = c0 + 16 * tq < D;
    if (in) load16(xrow + c0, xn);
    else
#pragma unroll
      for (int q = 0; q < 16; ++q) xn[q] = 0.f;
    if (g && in) load16(g + c0 + 16 * tq, gn);
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
      const int e = eq + 16 * j;
      if (e < E && in) load16(wr + (int64_t)e * D + c0 + 16 * tq, wn[j]);
      else
#pragma unroll
        for (int q = 0; q < 16; ++q) wn[j][q] = 0.f;
    }
  };
  fetch(0);
  for (int c0 = 0; c0 < D; c0 += RCH) {
#pragma unroll
    for (int q = 0; q < 16; ++q) ss += xn[q] * xn[q];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(xs + eq * RST + 16 * tq + 4 * q) = make_float4(xn[4 * q], xn[4 * q + 1], xn[4 * q + 2], xn[4 * q + 3]);
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
      float f[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) f[q] = g ? gn[q] * wn[j][q] : wn[j][q];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4*)(gw + (eq + 16 * j) * RST + 16 * tq + 4 * q) = make_float4(f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]);
    }
    __syncthreads();
    if (c0 + RCH < D) fetch(c0 + RCH);      // the next chunk's loads run under this chunk's FMAs
#pragma unroll 8
    for (int c = 0; c < RCH; c += 4) {
      const float4 xv = *(const float4*)(xs + tq * RST + c);
#pragma unroll
      for (int j = 0; j < EJ; ++j) {
        const float4 wv = *(const float4*)(gw + (eq + 16 * j) * RST + c);
        float a = acc[j];
        a = fmaf(xv.x, wv.x, a);
        a = fmaf(xv.y, wv.y, a);
        a = fmaf(xv.z, wv.z, a);
        a = fmaf(xv.w, wv.w, a);
        acc[j] = a;
      }
    }
    __syncthreads();
  }
  // row sums of squares of row eq: its 16 staging lanes are consecutive
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (tq == 0) rs[eq] = g ? 1.0f / sqrtf(ss / (float)D + eps) : 1.0f;
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EJ; ++j)
    if (eq + 16 * j < E) lg[tq * 65 + eq + 16 * j] = acc[j] * rs[tq];
  __syncthreads();
  // one wave per token: softmax, top-k, renormalised weights
  for (int r = wave; r < RT; r += 4) {
    const int t = t0 + r;
    const float logit = lane < E ? lg[r * 65 + lane] : -INFINITY;
    const float mx = warp_max(logit);
    const float ex = lane < E ? expf(logit - mx) : 0.f;
    const float p = ex / warp_sum(ex);
    // selection key: the logit's order as a signed integer (NaN lowest among the experts, an
    // expert already taken and the lanes past E below every expert), so that the k rounds always
    // pick k distinct experts
    int key = INT_MIN;
    if (lane < E) {
      const int b = __float_as_int(logit);
      key = __builtin_isnan(logit) ? INT_MIN + 1 : max(b >= 0 ? b : b ^ 0x7fffffff, INT_MIN + 1);
    }
    float selsum = 0.f;
    int my_rank = -1;
    for (int j = 0; j < k; ++j) {
      int bv = key, bi = lane;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (lane == bi) { my_rank = j; key = INT_MIN; }
      selsum += __shfl(p, bi, 64);
    }
    if (my_rank >= 0) sel[r * k + my_rank] = t < T_ ? lane : -1;
    if (t < T_ && my_rank >= 0) {
      idx[(int64_t)t * k + my_rank] = lane;
      w[(int64_t)t * k + my_rank] = p / selsum;
    }
  }
  if (!lrank) return;
  __syncthreads();
  // stable rank of each assignment among this workgroup's assignments of its expert, in chunks of
  // 256 assignments: per-expert ballots inside each wave, prefix over the 4 waves, running counts
  const int n = RT * k;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int a0 = 0; a0 < n; a0 += 256) {
    const int a = a0 + tid;
    const int e = a < n ? sel[a] : -1;
    int rank = 0;
    for (int xe = 0; xe < E; ++xe) {
      const uint64_t bal = __ballot(e == xe);
      if (e == xe) rank = __popcll(bal & lt_mask);
      if (lane == 0) wtot[wave][xe] = __popcll(bal);
    }
    __syncthreads();
    if (e >= 0) {
      int before = cnt[e];
      for (int w2 = 0; w2 < wave; ++w2) before += wtot[w2][e];
      lrank[(int64_t)t0 * k + a] = before + rank;
    }
    __syncthreads();
    if (tid < E) cnt[tid] += wtot[0][tid] + wtot[1][tid] + wtot[2][tid] + wtot[3][tid];
    __syncthreads();
  }
  if (tid < E) blkcnt[(int64_t)blockIdx.x * E + tid] = cnt[tid];
}

// One workgroup: per-expert totals and, for every router workgroup b, the first sorted position of
// its assignments of expert e: off[b][e] = offsets[e] + sum_{b' < b} blkcnt[b'][e].  16 threads per
// expert, each over a contiguous range of workgroups; then the grouped-GEMM tile table, each
// expert's tiles written by its own thread.
__global__ __launch_bounds__(1024) void moe_scan_kernel(const int* __restrict__ blkcnt, int nblk, int E, int bm,
                                                        int max_tiles, int* __restrict__ blkoff,
                                                        int* __restrict__ counts, int* __restrict__ offsets,
                                                        int* __restrict__ tiles) {
  __shared__ int part[16][64], base[65], tbase[65];
  const int tid = threadIdx.x, e = tid & 63, q = tid >> 6;
  const int per = (nblk + 15) / 16, b0 = min(nblk, q * per), b1 = min(nblk, b0 + per);
  int s = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) s += blkcnt[(int64_t)b * E + e];
  }
  part[q][e] = s;
  __syncthreads();
  if (tid == 0) {
    int o = 0, ts = 0;
    for (int x = 0; x < E; ++x) {
      int c = 0;
      for (int qq = 0; qq < 16; ++qq) c += part[qq][x];
      base[x] = o;
      tbase[x] = ts;
      o += c;
      ts += (c + bm - 1) / bm;
    }
    base[E] = o;
    tbase[E] = ts;
  }
  __syncthreads();
  if (e < E && q == 0) {
    const int c = base[e + 1] - base[e];
    counts[e] = c;
    offsets[e] = base[e];
    if (e == E - 1) offsets[E] = base[E];
    for (int r = 0, ts = tbase[e]; r < c; r += bm, ++ts)
      if (ts < max_tiles) {
        tiles[3 * ts] = e;
        tiles[3 * ts + 1] = base[e] + r;
        tiles[3 * ts + 2] = min(bm, c - r);
      }
  }
  for (int i = tbase[E] + tid; i < max_tiles; i += 1024) tiles[3 * i] = -1;
  if (e < E) {
    int run = base[e];
    for (int qq = 0; qq < q; ++qq) run += part[qq][e];
    for (int b = b0; b < b1; ++b) {
      blkoff[(int64_t)b * E + e] = run;
      run += blkcnt[(int64_t)b * E + e];
    }
  }
}

// Sorted position of every assignment a = t k + slot: its router workgroup's first position for
// the expert plus its stable rank there; perm_tok lists the tokens in sorted order.
__global__ __launch_bounds__(256) void moe_scatter_kernel(const int* __restrict__ idx, const int* __restrict__ lrank,
                                                          const int* __restrict__ blkoff, int n, int k, int E,
                                                          int* __restrict__ perm_tok, int* __restrict__ pos_of) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a >= n) return;
  const int t = a / k;
  const int pos = blkoff[(int64_t)(t / RT) * E + idx[a]] + lrank[a];
  pos_of[a] = pos;
  perm_tok[pos] = t;
}

template <typename TH>
__global__ __launch_bounds__(256) void combine_kernel(TH* __restrict__ h, const float* __restrict__ r,
                                                      const bf16* __restrict__ y, const float* __restrict__ w,
                                                      const int* __restrict__ pos_of, int T_, int k, int D) {
  const int cpr = D / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)T_ * cpr) return;
  const int t = (int)(c / cpr), ch = (int)(c - (int64_t)t * cpr);
  const float4 r0 = *(const float4*)(r + (int64_t)t * D + ch * 8);
  const float4 r1 = *(const float4*)(r + (int64_t)t * D + ch * 8 + 4);
  float acc[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  for (int j = 0; j < k; ++j) {
    const float wj = w[(int64_t)t * k + j];
    const bf16x8 yv = *(const bf16x8*)(y + (int64_t)pos_of[(int64_t)t * k + j] * D + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += wj * static_cast<float>(yv[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) h[(int64_t)t * D + ch * 8 + e] = from_f<TH>(acc[e]);
}

}  // namespace

template <typename Tx, typename Tw>
hipError_t moe_route(const Tx* x, const Tw* g, float eps, const Tw* wr, int T_, int D, int E, int k, int* idx, float* w,
                     int* lrank, int* blkcnt, hipStream_t s) {
  if (T_ <= 0) return hipSuccess;
  const dim3 grid((T_ + RT - 1) / RT);
  if (E <= 32)
    hipLaunchKernelGGL((route_kernel<Tx, Tw, 2>), grid, dim3(256), 0, s, x, g, eps, wr, T_, D, E, k, idx, w, lrank, blkcnt);
  else
    hipLaunchKernelGGL((route_kernel<Tx, Tw, 4>), grid, dim3(256), 0, s, x, g, eps, wr, T_, D, E, k, idx, w, lrank, blkcnt);
  return hipGetLastError();
}
template hipError_t moe_route<float, bf16>(const float*, const bf16*, float, const bf16*, int, int, int, int, int*,
                                           float*, int*, int*, hipStream_t);
template hipError_t moe_route<bf16, bf16>(const bf16*, const bf16*, float, const bf16*, int, int, int, int, int*,
                                          float*, int*, int*, hipStream_t);
template hipError_t moe_route<float, float>(const float*, const float*, float, const float*, int, int, int, int, int*,
                                            float*, int*, int*, hipStream_t);

int moe_route_blocks(int T_) { return (T_ + RT - 1) / RT; }

hipError_t moe_sort(const int* idx, const int* lrank, const int* blkcnt, int* blkoff, int T_, int k, int E,
                    int* counts, int* offsets, int* perm_tok, int* pos_of, int* tiles, int max_tiles, int bm,
                    hipStream_t s) {
  const int nblk = moe_route_blocks(T_);
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), 0, s, blkcnt, nblk, E, bm, max_tiles, blkoff, counts,
                     offsets, tiles);
  const int n = T_ * k;
  if (n > 0)
    hipLaunchKernelGGL(moe_scatter_kernel, dim3((n + 255) / 256), dim3(256), 0, s, idx, lrank, blkoff, n, k, E,
                       perm_tok, pos_of);
  return hipGetLastError();
}

template <typename TH>
hipError_t moe_combine(TH* h, const float* r, const bf16* y, const float* w, const int* pos_of, int T_, int k, int D,
                       hipStream_t s) {
  const int64_t total = (int64_t)T_ * (D / 8);
  hipLaunchKernelGGL(combine_kernel<TH>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, h, r, y, w, pos_of, T_, k, D);
  return hipGetLastError();
}
template hipError_t moe_combine<bf16>(bf16*, const float*, const bf16*, const float*, const int*, int, int, int, hipStream_t);
template hipError_t moe_combine<float>(float*, const float*, const bf16*, const float*, const int*, int, int, int, hipStream_t);

}  // namespace psf
