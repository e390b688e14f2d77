// Prefix + image-token attention of the gen block (grouped-query, scale 1/sqrt(d); no mask, or a
// causal mask for the prefix forward that builds the prompt cache).
//
// Keys/values of one (sequence, kv head) are the static prefix cache followed by the image
// tokens' own k/v, packed contiguously (K [Lpad, d] and V transposed [d, Lpad]).
//
// bf16 path, one workgroup = 4 waves of 32 queries that share one kv head (up to 4 of its query
// heads).  Per 64-key tile (K and V^T staged in LDS, shared by the 4 waves):
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

#ifndef ATTN_QB
#define ATTN_QB 1
#endif

namespace psf {
namespace {

// ------------------------------------------------------------------ bf16 kernel
// One workgroup = 4 waves x QB 32-query blocks.  K/V tiles of 64 keys come in by
// LDS-DMA (buffer loads straight into LDS, double buffered, one barrier per tile).  Every K
// fragment and V^T fragment read from LDS feeds QB MFMAs.  V^T is packed with the keys of each
// 16-key group stored in the order [0-3, 8-11, 4-7, 12-15], which is exactly the order in which
// the S^T accumulators hand P^T to the second MFMA, so each P.V fragment is one 16-byte read.
// The running max is only moved when a tile's max exceeds it by more than 2^8 (in exp2 units):
// probabilities stay below 256 and the final normalisation uses the same reference, so the
// result is the plain softmax; most tiles skip the O rescale entirely.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

DEVI __amdgpu_buffer_rsrc_t make_rsrc_a(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
DEVI void dma16_a(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// Query heads per attention workgroup: 4 when the GQA group size allows, else 2 or 1.
__host__ __device__ inline int attn_heads_per_wg(int G) { return (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1); }

// QKN: the q heads in qkv are raw projections; each wave applies the per-head RMSNorm (gain gq)
// and the rotate-half RoPE (cos/sin table [pos][d/2]) to its queries while loading them.
template <int D, int QB, bool QKN>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void attn_v2_kernel(const bf16* __restrict__ qkv, int64_t ldq,
                                                                     SeqInfo si, int Hq, int Hkv, int Lpad,
                                                                     const bf16* __restrict__ Kc,
                                                                     const bf16* __restrict__ Vt, bf16* __restrict__ O,
                                                                     int64_t ldo, float scale_log2, int n_qb,
                                                                     const bf16* __restrict__ gq,
                                                                     const float2* __restrict__ table, float eps,
                                                                     int causal, float* __restrict__ lse) {
  constexpr int KT = 64;                  // keys per tile
  constexpr int KROW = D * 2;             // bytes per K row
  constexpr int KCH = D / 8;              // 16-byte chunks per K row
  constexpr int NDB = D / 32;
  constexpr int STAGE = KT * KROW + D * KT * 2;
  constexpr int QW = 32 * QB;             // queries per wave
  constexpr float RESCALE_TH = 8.0f;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  // ds_read_b128 serves 16 lanes per cycle over a 256 B window: 256 B K rows (d = 128) swizzle
  // chunks by (r & 15); 128 B rows (K at d = 64, V^T) pair up in a window and use ((r >> 1) & 7).
  auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };

  // The four waves share one kv head: they cover HPW query heads of its group times 4 / HPW
  // query blocks, so each K/V tile brought into LDS serves HPW heads.
  const int G = Hq / Hkv;
  const int HPW = attn_heads_per_wg(G);
  const int n_hg = G / HPW;
  const int total = si.B * Hkv * n_qb * n_hg;
  const int id = xcd_remap(blockIdx.x, total);
  const int hg = id % n_hg;
  int rest = id / n_hg;
  const int qbk = rest % n_qb;
  rest /= n_qb;
  const int g = rest % Hkv;
  const int b = rest / Hkv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int h = g * G + hg * HPW + wave % HPW;
  const int N = si.N;
  const int L = si.plen[b] + N;
  const int qbase = qbk * ((4 / HPW) * QW) + (wave / HPW) * QW;

  bf16x8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qn = min(qbase + qb * 32 + lr, N - 1);
    const int64_t tok = (int64_t)b * N + qn;
    const bf16* qp = qkv + tok * ldq + (int64_t)h * D + lh * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[qb][ks] = *(const bf16x8*)(qp + ks * 16);
    if (QKN) {
      // This lane holds elements ks * 16 + lh * 8 + e of its query's head vector (the other half
      // sits in lane ^ 32); the rotate-half partner of element j < d/2 is j + d/2, i.e. k-step
      // ks + d/32 of the same lane.
      float x[D / 16][8];
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[ks][e] = static_cast<float>(qf[qb][ks][e]);
          ss += x[ks][e] * x[ks][e];
        }
      ss += __shfl_xor(ss, 32, 64);
      const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 gg = *(const bf16x8*)(gq + ks * 16 + lh * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[ks][e] = x[ks][e] * r * static_cast<float>(gg[e]);
      }
      const float2* tb = table + (int64_t)(si.plen[b] + qn) * (D / 2) + lh * 8;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = tb[ks * 16 + e];
          const float a = x[ks][e], c = x[ks + D / 32][e];
          x[ks][e] = a * cs.x - c * cs.y;
          x[ks + D / 32][e] = c * cs.x + a * cs.y;
        }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][ks][e] = static_cast<bf16>(x[ks][e]);
    }
  }
  f32x16 o[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[qb][i][e] = 0.f;
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m[qb] = -INFINITY; l[qb] = 0.f; }

  // DMA sources: K rows of this (b, g) and V^T rows, both with Lpad keys
  const __amdgpu_buffer_rsrc_t rk = make_rsrc_a(Kc + ((int64_t)b * Hkv + g) * Lpad * D, (uint32_t)Lpad * KROW);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc_a(Vt + ((int64_t)b * Hkv + g) * D * Lpad, (uint32_t)D * Lpad * 2);
  // K: one wave-load = 64 lanes x 16 B = (1024 / KROW) rows; lane -> row lane / KCH, chunk lane % KCH
  constexpr int KRPL = 1024 / KROW;                 // K rows per wave-load
  constexpr int KLOADS = KT / KRPL / 4;             // wave-loads per wave per tile (K)
  const int krow_l = lane / KCH, kch_p = lane % KCH;
  // V^T: rows of 128 B (64 keys); one wave-load = 8 rows; lane -> row lane/8, chunk lane%8
  constexpr int VLOADS = D / 8 / 4;                 // wave-loads per wave per tile (V)
  const int vrow_l = lane >> 3, vch_p = lane & 7;

  // K tile t into the K half of a stage, V^T tile t into the V half
  auto issue_k = [&](int t, int stage) {
    char* Ks = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int r0 = (wave * KLOADS + i) * KRPL;
      const int row = r0 + krow_l;
      const int lch = kch_p ^ kswz(row);
      dma16_a(rk, Ks + r0 * KROW, (uint32_t)(row * KROW + lch * 16), (uint32_t)t * KT * KROW);
    }
  };
  auto issue_v = [&](int t, int stage) {
    char* Vs = smem + stage * STAGE + KT * KROW;
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int r0 = (wave * VLOADS + i) * 8;
      const int row = r0 + vrow_l;
      const int lch = vch_p ^ ((row >> 1) & 7);
      dma16_a(rv, Vs + r0 * 128, (uint32_t)(row * Lpad * 2 + lch * 16), (uint32_t)t * KT * 2);
    }
  };

  // Per-lane LDS byte offsets of the fragment reads; the stage and the 32-row block offsets are
  // immediates.  K row r = kb * 32 + lr has kswz(r) = kswz(lr); V^T row r = db * 32 + lr has
  // ((r >> 1) & 7) = ((lr >> 1) & 7).
  int koff[D / 16], voff[4];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = lr * KROW + (((ks * 2 + lh) ^ kswz(lr)) << 4);
#pragma unroll
  for (int c = 0; c < 4; ++c) voff[c] = KT * KROW + lr * 128 + (((c * 2 + lh) ^ ((lr >> 1) & 7)) << 4);
  const bf16x2 ones = {static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)};

  // causal: query n sees keys j <= P_b + n, so this workgroup needs keys up to its last query
  const int qwg = (4 / HPW) * QW;
  const int Lc = causal ? min(L, si.plen[b] + min(N - 1, qbk * qwg + qwg - 1) + 1) : L;
  const int ntiles = (Lc + KT - 1) / KT;
  const int myq = si.plen[b] + qbase + lr;               // last key this lane's query may see (causal)
  // tiles below nfull are seen whole by every query of the workgroup: no masking
  const int nfull = causal ? min(ntiles, (si.plen[b] + qbk * qwg + 1) / KT) : L / KT;

  // Software pipeline across k-tiles: the scores of tile t+1 (K . Q^T MFMAs) are computed while
  // the softmax of tile t runs on the VALU, then P(t) . V(t) follows.  K therefore runs one tile
  // ahead of V: K tile t and V tile t both live in stage t & 1, K(t+1) is loaded during tile t-1
  // and V(t) during tile t-1.
  f32x16 sc[QB][2], sn[QB][2];
  auto scores = [&](f32x16 (&dst)[QB][2], const int stage) {
    const char* K0 = smem + stage * STAGE;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[qb][kb][e] = 0.f;
    // K fragments (ks, kb) in order f = 2 ks + kb through a ring of FR registers: FR reads are in
    // flight ahead of each MFMA, so the LDS latency hides under the MFMAs before it
    constexpr int NF = D / 8, FR = 4;
    auto rd = [&](const int f) { return *(const bf16x8*)(K0 + (f & 1) * 32 * KROW + koff[f >> 1]); };
    bf16x8 a[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) a[f] = rd(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        dst[qb][f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f % FR], qf[qb][f >> 1], dst[qb][f & 1], 0, 0, 0);
      if (f + FR < NF) a[f % FR] = rd(f + FR);
    }
    // keep that order: the scheduler would otherwise sink each read next to its MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, FR, 1);                  // DS reads
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 1);                // MFMA
      if (f + FR < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
  };
  // Online softmax of the scores in sc (tile t, keys from j0) and P . V from stage `stage`.
  // masked (a literal at every call): the tile may hold keys past the sequence end or, for causal
  // rows, past the query; those get probability 0.
  auto softmax_pv = [&](const int t, const int stage, const bool masked) {
    const int j0 = t * KT;
    const bool tail = masked && (j0 + KT > L || (causal && j0 + KT - 1 > si.plen[b] + qbase));
    bf16x8 pb[QB][2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (tail) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = j0 + kb * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
            if (key >= L || (causal && key > myq + qb * 32)) sc[qb][kb][e] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[qb][kb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
      const bool move = mx > m[qb] + RESCALE_TH;
      if (__builtin_amdgcn_ballot_w64(move)) {          // wave-uniform: some query moves its max
        const float mn = move ? mx : m[qb];
        const float alpha = exp2f(m[qb] - mn);
        m[qb] = mn;
        l[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[qb][i][e] *= alpha;
      }
      // p = 2^(s log2(e)/sqrt(d) - m): the hardware exp2 (results below 2^-126 flush to zero,
      // far under the bf16 rounding p gets next).  The row sum accumulates the bf16 p that the
      // P.V product uses, two at a time with a bf16 dot product against (1, 1).
      const float nm = -m[qb];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pb[qb][kb][st][e] = static_cast<bf16>(__builtin_amdgcn_exp2f(fmaf(sc[qb][kb][st * 8 + e], scale_log2, nm)));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 pr = {pb[qb][kb][st][2 * e], pb[qb][kb][st][2 * e + 1]};
            rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
          }
        }
      l[qb] += rs;
    }
    const char* S0 = smem + stage * STAGE;
    // V^T fragments (kb, st, db) in order f = (2 kb + st) NDB + db through a ring of FR registers
    constexpr int NF = 4 * NDB, FR = 4;
    auto rd = [&](const int f) { return *(const bf16x8*)(S0 + (f % NDB) * 32 * 128 + voff[f / NDB]); };
    bf16x8 av[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) av[f] = rd(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int ks = f / NDB, db = f % NDB;       // ks = 2 kb + st
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[f % FR], pb[qb][ks >> 1][ks & 1], o[qb][db], 0, 0, 0);
      if (f + FR < NF) av[f % FR] = rd(f + FR);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, FR, 2);                  // DS reads
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 2);                // MFMA
      if (f + FR < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
    }
  };
  // iteration t (every tile but the last): after the barrier K(t+1) and V(t) have landed and no
  // wave reads K(t) or V(t-1) any more, so K(t+2) and V(t+1) go into those halves.
  auto step = [&](const int t, const int stage, const bool masked) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue_k(min(t + 2, ntiles - 1), stage);   // past the end: a reload into a half nobody reads
    issue_v(t + 1, stage ^ 1);
    scores(sn, stage ^ 1);
    softmax_pv(t, stage, masked);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { sc[qb][0] = sn[qb][0]; sc[qb][1] = sn[qb][1]; }
  };

  issue_k(0, 0);
  issue_v(0, 0);
  if (ntiles > 1) issue_k(1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  scores(sc, 0);
  int t = 0;
  for (; t + 2 < ntiles && t + 2 <= nfull; t += 2) {
    step(t, 0, false);
    step(t + 1, 1, false);
  }
  // The rest but the last: the causal diagonal, or one unpaired full tile.  t is even here and
  // at most ceil((qwg - 1) / KT) + 1 tiles remain before the last, qwg <= 4 QW queries.
  constexpr int MAXTAIL = (4 * QW - 1 + KT - 1) / KT + 1;
#pragma unroll
  for (int i = 0; i < MAXTAIL; ++i)
    if (t + 1 < ntiles) {
      step(t, i & 1, true);
      ++t;
    }
  // last tile
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  softmax_pv(t, t & 1, true);

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32, 64);
    const float inv = 1.0f / lt;
    const int query = qbase + qb * 32 + lr;
    // log2-sum-exp of the scaled scores, for the backward pass: p = 2^(s log2(e)/sqrt(d) - lse)
    if (lse && lh == 0 && query < N) lse[((int64_t)b * Hq + h) * N + query] = m[qb] + __log2f(lt);
    if (query < N) {
      bf16* op = O + ((int64_t)b * N + query) * ldo + (int64_t)h * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = static_cast<bf16>(o[qb][db][e4 * 4 + i] * inv);
          *(bf16x4*)(op + db * 32 + e4 * 8 + lh * 4) = v;
        }
    }
  }
}

// fp32 path (small problems): one thread per (query, head), online softmax over all keys.
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(const float* __restrict__ qkv, int64_t ldq, SeqInfo si, int Hq,
                                                       int Hkv, int Lpad, const float* __restrict__ Kc,
                                                       const float* __restrict__ Vt, float* __restrict__ O,
                                                       int64_t ldo, float scale, int causal) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int n = blockIdx.x * 128 + threadIdx.x;
  if (n >= si.N) return;
  const int g = h / (Hq / Hkv);
  const int L = causal ? si.plen[b] + n + 1 : si.plen[b] + si.N;
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
                          const bf16* Kc, const bf16* Vt, bf16* O, int64_t ldo, const bf16* gq,
                          const float2* table, float eps, bool causal, hipStream_t s, float* lse) {
  const int n_qb = (si.N + 127) / 128;
  const int total = si.B * Hkv * n_qb * (Hq / Hkv);
  if (total == 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  // 4 waves x ATTN_QB*32 queries per workgroup
  constexpr int QB = ATTN_QB;
  const int hpw = attn_heads_per_wg(Hq / Hkv);
  const int qpw = (4 / hpw) * 32 * QB;                  // queries of one head per workgroup
  const int n_qb2 = (si.N + qpw - 1) / qpw;
  const int total2 = si.B * Hkv * n_qb2 * (Hq / Hkv / hpw);
#define PSF_ATTN(DD, QKN)                                                                              \
  hipLaunchKernelGGL((attn_v2_kernel<DD, QB, QKN>), dim3(total2), dim3(256), 0, s, qkv, ldq, si, Hq, Hkv, Lpad, Kc, \
                     Vt, O, ldo, scale_log2, n_qb2, gq, table, eps, causal ? 1 : 0, lse)
  if (d == 128) {
    if (gq) PSF_ATTN(128, true); else PSF_ATTN(128, false);
  } else if (d == 64) {
    if (gq) PSF_ATTN(64, true); else PSF_ATTN(64, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef PSF_ATTN
  (void)total;
  return hipGetLastError();
}

hipError_t attention_f32(const float* qkv, int64_t ldq, const SeqInfo& si, int Hq, int Hkv, int d, int Lpad,
                         const float* Kc, const float* Vt, float* O, int64_t ldo, bool causal, hipStream_t s) {
  dim3 grid((si.N + 127) / 128, Hq, si.B);
  const float scale = 1.0f / sqrtf((float)d);
  const int c = causal ? 1 : 0;
  if (d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(128), 0, s, qkv, ldq, si, Hq, Hkv, Lpad, Kc, Vt, O, ldo, scale, c);
  else if (d == 64) hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(128), 0, s, qkv, ldq, si, Hq, Hkv, Lpad, Kc, Vt, O, ldo, scale, c);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace psf
