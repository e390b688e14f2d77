// Routed expert MLP support for the A3B gen block: softmax router with top-k and
// renormalised weights, a deterministic counting sort of (token, slot) assignments by
// expert with the grouped-GEMM tile table, and the fixed-order weighted combine.
// No floating-point atomics anywhere: results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace psf {
namespace {

// One wave per token; lane e computes expert e's logit from the token row staged in LDS.
// Selection is by logit (the softmax is monotone), ties to the lower expert index.
template <typename T>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ u, const T* __restrict__ wr, int T_, int D,
                                                    int E, int k, int* __restrict__ idx, float* __restrict__ w) {
  extern __shared__ float urow_all[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  float* urow = urow_all + wave * D;
  const int tc = min(t, T_ - 1);
  for (int i = lane; i < D; i += 64) urow[i] = to_f(u[(int64_t)tc * D + i]);
  __syncthreads();
  float logit = -INFINITY;
  if (lane < E) {
    float acc = 0.f;
    const T* wrow = wr + (int64_t)lane * D;
    for (int i = 0; i < D; ++i) acc += to_f(wrow[i]) * urow[i];
    logit = acc;
  }
  const float mx = warp_max(logit);
  const float ex = lane < E ? expf(logit - mx) : 0.f;
  const float z = warp_sum(ex);
  const float p = ex / z;
  // top-k by repeated wave argmax of the logit (lower index wins ties)
  float key = lane < E ? logit : -INFINITY;
  float selsum = 0.f;
  int my_rank = -1;
  for (int j = 0; j < k; ++j) {
    float bv = key;
    int bi = lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == bi) { my_rank = j; key = -INFINITY; }
    selsum += __shfl(p, bi, 64);
  }
  if (t < T_ && my_rank >= 0) {
    idx[(int64_t)t * k + my_rank] = lane;
    w[(int64_t)t * k + my_rank] = p / selsum;
  }
}

// Single workgroup: integer histogram, exclusive scan + tile table, then a stable rank
// pass over chunks of 1024 assignments (per-expert ballots inside each wave, exclusive
// scan over the 16 waves, running per-expert base across chunks).
__global__ __launch_bounds__(1024) void sort_kernel(const int* __restrict__ idx, int n, int E, int k, int bm,
                                                    int max_tiles, int* __restrict__ counts,
                                                    int* __restrict__ offsets, int* __restrict__ perm_tok,
                                                    int* __restrict__ pos_of, int* __restrict__ tiles) {
  __shared__ int cnt[64], base[64], tot[64], wcnt[16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  for (int a = tid; a < n; a += 1024) atomicAdd(&cnt[idx[a]], 1);
  __syncthreads();
  if (tid == 0) {
    int s = 0, ts = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = s;
      offsets[e] = s;
      counts[e] = cnt[e];
      for (int r = 0; r < cnt[e]; r += bm) {
        if (ts < max_tiles) {
          tiles[3 * ts] = e;
          tiles[3 * ts + 1] = s + r;
          tiles[3 * ts + 2] = min(bm, cnt[e] - r);
        }
        ++ts;
      }
      s += cnt[e];
    }
    offsets[E] = s;
    for (int i = ts; i < max_tiles; ++i) tiles[3 * i] = -1;
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < n; c0 += 1024) {
    const int a = c0 + tid;
    const int e = a < n ? idx[a] : -1;
    int rank = 0;
    for (int x = 0; x < E; ++x) {
      const uint64_t bal = __ballot(e == x);
      if (e == x) rank = __popcll(bal & lt_mask);
      if (lane == 0) wcnt[wave][x] = __popcll(bal);
    }
    __syncthreads();
    if (tid < E) {
      int s = 0;
      for (int w2 = 0; w2 < 16; ++w2) { const int c = wcnt[w2][tid]; wcnt[w2][tid] = s; s += c; }
      tot[tid] = s;
    }
    __syncthreads();
    if (e >= 0) {
      const int pos = base[e] + wcnt[wave][e] + rank;
      perm_tok[pos] = a / k;
      pos_of[a] = pos;
    }
    __syncthreads();
    if (tid < E) base[tid] += tot[tid];
    __syncthreads();
  }
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

template <typename T>
hipError_t moe_route(const T* u, const T* wr, int T_, int D, int E, int k, int* idx, float* w, hipStream_t s) {
  if (T_ <= 0) return hipSuccess;
  const size_t lds = 4 * (size_t)D * sizeof(float);
  hipLaunchKernelGGL(route_kernel<T>, dim3((T_ + 3) / 4), dim3(256), lds, s, u, wr, T_, D, E, k, idx, w);
  return hipGetLastError();
}
template hipError_t moe_route<bf16>(const bf16*, const bf16*, int, int, int, int, int*, float*, hipStream_t);
template hipError_t moe_route<float>(const float*, const float*, int, int, int, int, int*, float*, hipStream_t);

hipError_t moe_sort(const int* idx, int T_, int k, int E, int* counts, int* offsets, int* perm_tok, int* pos_of,
                    int* tiles, int max_tiles, int bm, hipStream_t s) {
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(1024), 0, s, idx, T_ * k, E, k, bm, max_tiles, counts, offsets,
                     perm_tok, pos_of, tiles);
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
