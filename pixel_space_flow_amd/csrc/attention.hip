// Prefix + image-token attention of the gen block (grouped-query, no mask, scale 1/sqrt(d)).
//
// Keys/values of one (sequence, kv head) are the static prefix cache followed by the image
// tokens' own k/v, packed contiguously (K [Lpad, d] and V transposed [d, Lpad]).
//
// bf16 path, one workgroup = 4 waves = 128 queries of one q head; each wave owns 32 queries.
// Per 64-key tile (K and V^T staged in LDS, shared by the 4 waves):
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q^T held in registers.
//                   A lane then holds 16 scores of ONE query (column lane&31) for keys
//                   (e/4)*8 + (lane/32)*4 + e%4 of each 32-key block, so the softmax row max
//                   needs only an in-lane reduction plus one exchange with lane^32.
//   online softmax  exp2 with log2(e)/sqrt(d) folded into one multiply, fp32 statistics; each
//                   half-wave keeps a partial row sum, the two are added at the end.
//   O^T += V^T P^T  B = the bf16-rounded P^T values exactly as the first MFMA left them in the
//                   lane; A = V^T rows read from LDS at the matching key order.
// LDS rows are XOR-swizzled (16-byte chunks for K, 8-byte units for V^T) so fragment reads
// are bank-conflict free.
#include "common.h"
#include "kernels.h"

namespace psf {
namespace {

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const bf16* __restrict__ qkv, int64_t ldq, SeqInfo si,
                                                           int Hq, int Hkv, int Lpad, const bf16* __restrict__ Kc,
                                                           const bf16* __restrict__ Vt, bf16* __restrict__ O,
                                                           int64_t ldo, float scale_log2, int n_qb) {
  constexpr int KT = 64;                 // keys per tile
  constexpr int KROW = D * 2;            // bytes per K row in LDS
  constexpr int KCH = D / 8;             // 16-byte chunks per K row
  constexpr int NDB = D / 32;            // 32-row blocks of the head dim
  __shared__ __attribute__((aligned(16))) char Ks[KT * KROW];
  __shared__ __attribute__((aligned(16))) char Vs[D * KT * 2];

  const int G = Hq / Hkv;
  const int total = si.B * Hkv * n_qb * G;
  const int id = xcd_remap(blockIdx.x, total);
  const int hh = id % G;
  int rest = id / G;
  const int qb = rest % n_qb;
  rest /= n_qb;
  const int g = rest % Hkv;
  const int b = rest / Hkv;
  const int h = g * G + hh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int N = si.N;
  const int L = si.plen[b] + N;
  const int query = qb * 128 + wave * 32 + lr;
  const int64_t tok = (int64_t)b * N + min(query, N - 1);

  // Q^T fragments: lane holds q[query][ks*16 + lh*8 .. +8) for every 16-wide slice of d
  bf16x8 qf[D / 16];
  {
    const bf16* qp = qkv + tok * ldq + (int64_t)h * D + lh * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);
  }

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const bf16* Kbase = Kc + ((int64_t)b * Hkv + g) * Lpad * D;
  const bf16* Vbase = Vt + ((int64_t)b * Hkv + g) * D * Lpad;
  const int ntiles = (L + KT - 1) / KT;

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * KT;
    __syncthreads();
    // K tile: 64 rows x KCH chunks
#pragma unroll
    for (int i = 0; i < (KT * KCH) / 256; ++i) {
      const int c = tid + i * 256;
      const int r = c / KCH, ch = c % KCH;
      const u32x4 v = *(const u32x4*)(Kbase + (int64_t)(j0 + r) * D + ch * 8);
      *(u32x4*)(Ks + r * KROW + ((ch ^ (r & 7)) << 4)) = v;
    }
    // V^T tile: D rows x 64 keys (8 chunks of 8 keys per row), stored as swizzled 8-byte units
#pragma unroll
    for (int i = 0; i < (D * 8) / 256; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 3, ch = c & 7;
      const u32x4 v = *(const u32x4*)(Vbase + (int64_t)r * Lpad + j0 + ch * 8);
      const int u0 = (2 * ch) ^ (r & 15), u1 = (2 * ch + 1) ^ (r & 15);
      *(u32x2*)(Vs + r * 128 + u0 * 8) = u32x2{v[0], v[1]};
      *(u32x2*)(Vs + r * 128 + u1 * 8) = u32x2{v[2], v[3]};
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
      const int r = kb * 32 + lr;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(Ks + r * KROW + (((ks * 2 + lh) ^ (r & 7)) << 4));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // scale, mask keys beyond L, tile max
    float mx = -INFINITY;
    const bool tail = j0 + KT > L;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[kb][e] * scale_log2;
        if (tail) {
          const int key = j0 + kb * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
          if (key >= L) x = -INFINITY;
        }
        s[kb][e] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    m = mn;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(s[kb][e] - mn);
        s[kb][e] = p;
        rs += p;
      }
    l = l * alpha + rs;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] *= alpha;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<bf16>(s[kb][st * 8 + e]);
        const int u0 = kb * 8 + st * 4 + lh;   // 8-byte unit of keys kb*32 + st*16 + lh*4 .. +4
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int r = db * 32 + lr;
          const u32x2 lo = *(const u32x2*)(Vs + r * 128 + ((u0 ^ (r & 15)) << 3));
          const u32x2 hi = *(const u32x2*)(Vs + r * 128 + (((u0 + 2) ^ (r & 15)) << 3));
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb, o[db], 0, 0, 0);
        }
      }
  }

  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = 1.0f / lt;
  if (query < N) {
    bf16* op = O + tok * ldo + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d0 = db * 32 + e4 * 8 + lh * 4;
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = static_cast<bf16>(o[db][e4 * 4 + i] * inv);
        *(bf16x4*)(op + d0) = v;
      }
  }
}

// fp32 path (small problems): one thread per (query, head), online softmax over all keys.
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(const float* __restrict__ qkv, int64_t ldq, SeqInfo si, int Hq,
                                                       int Hkv, int Lpad, const float* __restrict__ Kc,
                                                       const float* __restrict__ Vt, float* __restrict__ O,
                                                       int64_t ldo, float scale) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int n = blockIdx.x * 128 + threadIdx.x;
  if (n >= si.N) return;
  const int g = h / (Hq / Hkv);
  const int L = si.plen[b] + si.N;
  const int64_t tok = (int64_t)b * si.N + n;
  float q[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) { q[i] = qkv[tok * ldq + (int64_t)h * D + i]; o[i] = 0.f; }
  const float* K = Kc + ((int64_t)b * Hkv + g) * Lpad * D;
  const float* V = Vt + ((int64_t)b * Hkv + g) * D * Lpad;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < L; ++j) {
    float sc = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) sc += q[i] * K[(int64_t)j * D + i];
    sc *= scale;
    const float mn = fmaxf(m, sc);
    const float a = expf(m - mn), p = expf(sc - mn);
    l = l * a + p;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = o[i] * a + p * V[(int64_t)i * Lpad + j];
    m = mn;
  }
#pragma unroll
  for (int i = 0; i < D; ++i) O[tok * ldo + (int64_t)h * D + i] = o[i] / l;
}

}  // namespace

hipError_t attention_bf16(const bf16* qkv, int64_t ldq, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad,
                          const bf16* Kc, const bf16* Vt, bf16* O, int64_t ldo, hipStream_t s) {
  const int n_qb = (si.N + 127) / 128;
  const int total = si.B * Hkv * n_qb * (Hq / Hkv);
  if (total == 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  if (d == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(total), dim3(256), 0, s, qkv, ldq, si, Hq, Hkv, Lpad, Kc, Vt, O, ldo, scale_log2, n_qb);
  else if (d == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(total), dim3(256), 0, s, qkv, ldq, si, Hq, Hkv, Lpad, Kc, Vt, O, ldo, scale_log2, n_qb);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t attention_f32(const float* qkv, int64_t ldq, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad,
                         const float* Kc, const float* Vt, float* O, int64_t ldo, hipStream_t s) {
  dim3 grid((si.N + 127) / 128, Hq, si.B);
  const float scale = 1.0f / sqrtf((float)d);
  if (d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(128), 0, s, qkv, ldq, si, Hq, Hkv, Lpad, Kc, Vt, O, ldo, scale);
  else if (d == 64) hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(128), 0, s, qkv, ldq, si, Hq, Hkv, Lpad, Kc, Vt, O, ldo, scale);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace psf
