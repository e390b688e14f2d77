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
// (g == nullptr: logit = sum_c x[t, c] w[e, c], x already normalised).  The contraction runs on
// the fp32 matrix instruction v_mfma_f32_16x16x4_f32 (fp32 products and sums): the four waves
// take contiguous quarters of the D columns, each wave a 16-token x 16-expert block per expert
// block j (EJ blocks), with lane l holding token l % 16 of A and expert 16 j + l % 16 of B for the
// columns 4 (l / 16) + q of each 16-column group (the same column order on both operands, so the
// sum is the plain dot product in another order); x, g and w come in by batches of column
// groups.  The four quarters' partial sums meet in LDS and are added in a fixed order.  Then one
// wave per token: softmax, the top-k by rank (ties to the lower expert index; the softmax is
// monotone, so the order of the logits is that of the probabilities), weights renormalised over
// the k, and each assignment's stable rank among the workgroup's assignments of the same expert
// (assignment order t k + slot) with the workgroup's per-expert counts, so that the sort needs no
// second pass over the assignments.
constexpr int RT = 16;          // tokens per router workgroup

// 4 consecutive elements (aligned to their size) as floats
DEVI void load4(const float* p, float* f) {
  const float4 v = *(const float4*)p;
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
DEVI void load4(const bf16* p, float* f) {
  const bf16x4 v = *(const bf16x4*)p;
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = static_cast<float>(v[e]);
}

template <typename Tx, typename Tw, int EJ>
__global__ __launch_bounds__(256) void route_kernel(const Tx* __restrict__ x, const Tw* __restrict__ g, float eps,
                                                    const Tw* __restrict__ wr, int T_, int D, int E, int k,
                                                    int* __restrict__ idx, float* __restrict__ w,
                                                    int* __restrict__ lrank, int* __restrict__ blkcnt) {
  __shared__ float part[4][RT][65];
  __shared__ float ssw[4][RT];
  __shared__ float lg[RT * 65];
  __shared__ float rs[RT];
  __shared__ int sel[RT * 64];
  __shared__ float psel[RT * 64];
  __shared__ int cnt[64], wtot[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * RT;
  // D is a multiple of 64: each wave owns D / 64 groups of 16 columns, from column c_begin
  const int ng = D / 64;
  const int c_begin = wave * ng * 16 + 4 * kq;
  const Tx* xrow = x + (int64_t)min(t0 + li, T_ - 1) * D + c_begin;   // rows past T_ read row T_ - 1
  const Tw* grow = g ? g + c_begin : nullptr;
  const Tw* wrow[EJ];
  bool wok[EJ];
#pragma unroll
  for (int j = 0; j < EJ; ++j) {
    const int e = 16 * j + li;
    wok[j] = e < E;
    wrow[j] = wr + (int64_t)(wok[j] ? e : 0) * D + c_begin;           // experts past E contribute zero
  }
  auto fetch = [&](int off, float (&xo)[4], float (&go)[4], float (&wo)[EJ][4]) {
    load4(xrow + off, xo);
    if (g) load4(grow + off, go);
#pragma unroll
    for (int j = 0; j < EJ; ++j) load4(wrow[j] + off, wo[j]);
  };
  f32x4 acc[EJ];
#pragma unroll
  for (int j = 0; j < EJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  // batches of NB column groups: all of a batch's loads are issued before its first product, so
  // one memory latency is paid per batch rather than per group
  constexpr int NB = EJ <= 2 ? 8 : 4;
  for (int i0 = 0; i0 < ng; i0 += NB) {
    float xb[NB][4], gb[NB][4], wb[NB][EJ][4];
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (i0 + u < ng) fetch(16 * (i0 + u), xb[u], gb[u], wb[u]);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (i0 + u < ng) {
#pragma unroll
        for (int q = 0; q < 4; ++q) ss += xb[u][q] * xb[u][q];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < EJ; ++j) {
            const float bw = wok[j] ? (g ? gb[u][q] * wb[u][j][q] : wb[u][j][q]) : 0.f;
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xb[u][q], bw, acc[j], 0, 0, 0);
          }
      }
  }
  // lanes li + 16 kq (kq = 0..3) hold partial sums of squares of token li
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (kq == 0) ssw[wave][li] = ss;
  // block j of lane l: tokens 4 (l / 16) + r, expert 16 j + l % 16
#pragma unroll
  for (int j = 0; j < EJ; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][4 * kq + r][16 * j + li] = acc[j][r];
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  if (tid < RT) {
    const float tot = ssw[0][tid] + ssw[1][tid] + ssw[2][tid] + ssw[3][tid];
    rs[tid] = g ? 1.0f / sqrtf(tot / (float)D + eps) : 1.0f;
  }
  __syncthreads();
  for (int i = tid; i < RT * 64; i += 256) {
    const int tk = i >> 6, e = i & 63;
    if (e < E) lg[tk * 65 + e] = (((part[0][tk][e] + part[1][tk][e]) + part[2][tk][e]) + part[3][tk][e]) * rs[tk];
  }
  __syncthreads();
  // one wave per token, lane e for expert e: every lane reads the token's E logits from LDS (the
  // same address across the wave, a broadcast) and finds in-lane the max, the softmax denominator
  // and its own expert's rank: the number of experts before it in the order "larger logit first,
  // ties to the lower index" (NaN below every number).  The top-k are the ranks below k; the
  // weights are renormalised by the sum of the k probabilities taken in rank order.
  auto order_key = [](float v) {
    const int b = __float_as_int(v);
    return __builtin_isnan(v) ? INT_MIN + 1 : max(b >= 0 ? b : b ^ 0x7fffffff, INT_MIN + 1);
  };
  for (int r = wave; r < RT; r += 4) {
    const int t = t0 + r;
    const float* lr = lg + r * 65;
    const float logit = lane < E ? lr[lane] : 0.f;
    const int key = order_key(logit);
    float mx = -INFINITY;
    int rank = 0;
    for (int e = 0; e < E; ++e) {
      const float v = lr[e];
      mx = fmaxf(mx, v);
      const int ke = order_key(v);
      rank += (ke > key || (ke == key && e < lane)) ? 1 : 0;
    }
    float den = 0.f;
    for (int e = 0; e < E; ++e) den += expf(lr[e] - mx);
    const float p = expf(logit - mx) / den;
    const bool chosen = lane < E && rank < k;
    if (chosen) psel[r * 64 + rank] = p;
    __builtin_amdgcn_s_waitcnt(0xc07f);       // this wave's LDS writes, read back below by other lanes
    __builtin_amdgcn_wave_barrier();
    float selsum = 0.f;
    for (int j = 0; j < k; ++j) selsum += psel[r * 64 + j];
    if (chosen) sel[r * k + rank] = t < T_ ? lane : -1;
    if (t < T_ && chosen) {
      idx[(int64_t)t * k + rank] = lane;
      w[(int64_t)t * k + rank] = p / selsum;
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
