// C ABI of the gen-tower denoise step: argument validation (host only, before any HIP
// call), workspace layout, and the launch sequence of a gen block and a tower step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/psf_gen.h"
#include "gemm.h"
#include "kernels.h"

#include <mutex>

// Scratch of gen_block_forward_noalloc (for callers that cannot allocate): a file-scope device
// array, one copy on every GPU the library runs on, held until the process ends.  Host code
// never passes its name to a kernel or a copy: the array's device address is looked up once per
// device (hipGetSymbolAddress, that device current) and only that address is used.
static __device__ __align__(256) char scratch[PSF_GEN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

// The current device's address of `scratch` (looked up on the first call on that device).
static int noalloc_scratch(void** out);

using namespace psf;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int ok() {
  g_err.clear();
  return GEN_OK;
}

#define HIP_TRY(expr)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(GEN_EHIP, "%s: %s", #expr, hipGetErrorString(e_));   \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ------------------------------------------------------------------ launch timing (measurement only)
enum { FAM_GATE_UP = 0, FAM_ATTN = 1, FAM_QKV = 2, FAM_DOWN = 3, FAM_O = 4, FAM_EXPERT = 5 };
struct Timing {
  int family = -1, cap = 0, used = 0;
  hipEvent_t* ev = nullptr;
} g_timing;

// Runs `launch` bracketed by event records when its family is being timed.
template <typename F>
hipError_t timed(int family, hipStream_t s, F&& launch) {
  const bool on = g_timing.family == family && g_timing.used < g_timing.cap;
  if (on) {
    hipError_t e = hipEventRecord(g_timing.ev[2 * g_timing.used], s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (on) {
    e = hipEventRecord(g_timing.ev[2 * g_timing.used + 1], s);
    ++g_timing.used;
  }
  return e;
}

// ------------------------------------------------------------------ validation
int check_dims(const gen_block_dims* d) {
  if (!d) return fail(GEN_EINVAL, "dims is NULL");
  if (d->dtype != GEN_F32 && d->dtype != GEN_BF16) return fail(GEN_EINVAL, "dtype %d is not GEN_F32/GEN_BF16", d->dtype);
  if (d->hidden_dtype != GEN_F32 && d->hidden_dtype != GEN_BF16)
    return fail(GEN_EINVAL, "hidden_dtype %d is not GEN_F32/GEN_BF16", d->hidden_dtype);
  if (d->dtype == GEN_F32 && d->hidden_dtype != GEN_F32) return fail(GEN_EUNSUPPORTED, "fp32 weights need an fp32 hidden_dtype");
  if (d->hidden <= 0 || d->hidden % 64) return fail(GEN_EINVAL, "hidden %d must be a positive multiple of 64", d->hidden);
  if (d->hidden > 8192) return fail(GEN_EUNSUPPORTED, "hidden %d > 8192", d->hidden);
  if (d->head_dim != 64 && d->head_dim != 128) return fail(GEN_EINVAL, "head_dim %d must be 64 or 128", d->head_dim);
  if (d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->n_q_heads % d->n_kv_heads)
    return fail(GEN_EINVAL, "n_q_heads %d must be a positive multiple of n_kv_heads %d", d->n_q_heads, d->n_kv_heads);
  if (!(d->rms_eps >= 0.f) || !std::isfinite(d->rms_eps)) return fail(GEN_EINVAL, "rms_eps must be finite and >= 0");
  if (!(d->rope_theta > 0.f) || !std::isfinite(d->rope_theta)) return fail(GEN_EINVAL, "rope_theta must be finite and > 0");
  const bool dense = d->mlp_intermediate > 0, moe = d->n_experts > 0;
  if (dense == moe) return fail(GEN_EINVAL, "exactly one of mlp_intermediate and n_experts must be > 0");
  if (dense && d->mlp_intermediate % 64) return fail(GEN_EINVAL, "mlp_intermediate %d must be a multiple of 64", d->mlp_intermediate);
  if (moe) {
    if (d->n_experts > 64) return fail(GEN_EUNSUPPORTED, "n_experts %d > 64", d->n_experts);
    if (d->top_k < 1 || d->top_k > d->n_experts) return fail(GEN_EINVAL, "top_k %d not in [1, n_experts]", d->top_k);
    if (d->expert_intermediate <= 0 || d->expert_intermediate % 64)
      return fail(GEN_EINVAL, "expert_intermediate %d must be a positive multiple of 64", d->expert_intermediate);
    if (d->dtype != GEN_BF16) return fail(GEN_EUNSUPPORTED, "expert MLP runs in bf16 only");
  }
  if (d->lora_rank < 0) return fail(GEN_EINVAL, "lora_rank %d < 0", d->lora_rank);
  if (d->lora_rank > 0) {
    if (d->lora_rank % 8 || d->lora_rank > 128) return fail(GEN_EUNSUPPORTED, "lora_rank %d must be a multiple of 8, <= 128", d->lora_rank);
    if (moe) return fail(GEN_EUNSUPPORTED, "LoRA is supported on dense blocks only");
    if (d->dtype != GEN_BF16) return fail(GEN_EUNSUPPORTED, "LoRA runs in bf16 only");
    if (!std::isfinite(d->lora_alpha)) return fail(GEN_EINVAL, "lora_alpha must be finite");
  }
  return GEN_OK;
}

int check_weights(const gen_block_dims* d, const gen_block_weights* w, int layer) {
  if (!w) return fail(GEN_EINVAL, "weights of layer %d are NULL", layer);
  const void* req[] = {w->g_in, w->w_qkv, w->g_q, w->g_k, w->w_o, w->g_post};
  const char* names[] = {"g_in", "w_qkv", "g_q", "g_k", "w_o", "g_post"};
  for (int i = 0; i < 6; ++i) {
    if (!req[i]) return fail(GEN_EINVAL, "layer %d: %s is NULL", layer, names[i]);
    if (!aligned16(req[i])) return fail(GEN_EINVAL, "layer %d: %s is not 16-byte aligned", layer, names[i]);
  }
  if (d->mlp_intermediate > 0) {
    if (!w->w_gate_up || !w->w_down) return fail(GEN_EINVAL, "layer %d: w_gate_up/w_down is NULL", layer);
    if (!aligned16(w->w_gate_up) || !aligned16(w->w_down)) return fail(GEN_EINVAL, "layer %d: MLP weights not 16-byte aligned", layer);
    if (w->ld_down != 0 && (w->ld_down < d->mlp_intermediate || w->ld_down % 8))
      return fail(GEN_EINVAL, "layer %d: ld_down %d must be 0 or a multiple of 8 >= mlp_intermediate %d", layer,
                  w->ld_down, d->mlp_intermediate);
  } else {
    if (!w->w_router || !w->w_exp_gate_up || !w->w_exp_down) return fail(GEN_EINVAL, "layer %d: expert weights are NULL", layer);
    if (!aligned16(w->w_exp_gate_up) || !aligned16(w->w_exp_down)) return fail(GEN_EINVAL, "layer %d: expert weights not 16-byte aligned", layer);
  }
  if (d->lora_rank > 0) {
    for (int s = 0; s < 7; ++s) {
      if ((w->lora_a[s] == nullptr) != (w->lora_b[s] == nullptr))
        return fail(GEN_EINVAL, "layer %d: LoRA site %d has only one of lora_a/lora_b", layer, s);
      if ((w->lora_a[s] && !aligned16(w->lora_a[s])) || (w->lora_b[s] && !aligned16(w->lora_b[s])))
        return fail(GEN_EINVAL, "layer %d: LoRA site %d not 16-byte aligned", layer, s);
    }
  }
  return GEN_OK;
}

int check_prefix(const gen_block_dims* d, int B, const void* const* pk, const void* const* pv, const int* plen,
                 int* max_prefix) {
  if (!plen) return fail(GEN_EINVAL, "prefix_len is NULL");
  int mx = 0;
  for (int b = 0; b < B; ++b) {
    if (plen[b] < 0) return fail(GEN_EINVAL, "prefix_len[%d] = %d < 0", b, plen[b]);
    mx = std::max(mx, plen[b]);
  }
  if (mx > 0 && (!pk || !pv)) return fail(GEN_EINVAL, "prefix_k/prefix_v arrays are NULL");
  (void)d;
  *max_prefix = mx;
  return GEN_OK;
}

// ------------------------------------------------------------------ workspace
constexpr size_t ALIGN = 256;
size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Row pitch (elements) of the SwiGLU output z, the down projection's A operand.  GEMM operand rows
// whose pitch is an odd multiple of 8 KiB above 8 KiB (24 KiB at I = 12288 in bf16) load measurably
// slower than rows 128 bytes longer, so such rows get 64 elements of padding.
int z_pitch(int I, size_t es) {
  const size_t b = (size_t)I * es;
  return (b > 8192 && b % 8192 == 0 && (b / 8192) % 2 == 1) ? I + (int)(128 / es) : I;
}

// Row pitch (bf16 elements) of the training path's long-k GEMM operands (the SwiGLU output z and
// the gate/up gradient with the transposed gate/up weight): rows a multiple of 8 KiB apart get 64
// elements of padding, so those products run on the 64-deep kernel at a pitch that loads at full
// speed.
int train_pitch(int n) { return ((size_t)n * 2) % 8192 == 0 ? n + 64 : n; }

struct Ws {
  size_t hidden, patches, u, qkv, attn, kc, vt, z, rope, temb, h1, x0, lora_t, hmid, skinny, lora_gu, lora_f32;
  size_t splitk, splitk_floats;
  size_t m_idx, m_w, m_counts, m_offsets, m_perm, m_pos, m_tiles, m_z, m_y, m_lrank, m_blkcnt, m_blkoff;
  size_t total;
  int Lpad, max_tiles, n_pos;
};

Ws layout(const gen_block_dims& d, int n_img, int n_br, int N, int max_prefix) {
  Ws w{};
  const size_t es = d.dtype == GEN_BF16 ? 2 : 4;
  const size_t B = (size_t)n_img * n_br, M = B * N, D = d.hidden;
  const size_t qkv = (size_t)(d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  w.Lpad = (int)((max_prefix + N + 63) / 64 * 64);
  w.n_pos = max_prefix + N;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
  w.hidden = take(M * D * 4);   // tower residual stream (fp32)
  w.patches = take((size_t)n_img * N * 3072 * es);
  w.u = take(M * D * es);
  w.hmid = take(M * D * 4);   // fp32 residual between attention and MLP
  w.qkv = take(M * qkv * es);
  w.attn = take(M * d.n_q_heads * d.head_dim * es);
  w.kc = take(B * d.n_kv_heads * w.Lpad * d.head_dim * es);
  w.vt = take(B * d.n_kv_heads * w.Lpad * d.head_dim * es);
  w.z = take(d.mlp_intermediate > 0 ? M * (size_t)z_pitch(d.mlp_intermediate, es) * es : 0);
  w.rope = take((size_t)w.n_pos * (d.head_dim / 2) * sizeof(float) * 2);
  w.temb = take((size_t)n_img * D * 4);
  w.h1 = take((size_t)n_img * D * 4);
  w.x0 = take(B * 3 * (size_t)N * 1024 * 4);
  w.lora_t = take(d.lora_rank > 0 ? M * 3 * d.lora_rank * es : 0);
  w.skinny = take(d.lora_rank > 0 ? skinny_part_floats((int)M, std::min(3 * d.lora_rank, 128)) * 4 : 0);
  w.lora_gu = take(d.lora_rank > 0 && d.mlp_intermediate > 0 ? M * 2 * d.mlp_intermediate * es : 0);
  w.lora_f32 = take(d.lora_rank > 0 ? M * qkv * 4 : 0);
  // split-K partial products for small token counts (few row tiles leave CUs idle)
  w.splitk_floats = M <= 2048 ? 4 * M * std::max(qkv, D) : 0;
  w.splitk = take(w.splitk_floats * 4);
  if (d.n_experts > 0) {
    const size_t A = M * d.top_k;
    w.max_tiles = (int)(A / 256 + d.n_experts + 1);
    w.m_idx = take(A * 4);
    w.m_w = take(A * 4);
    w.m_counts = take(d.n_experts * 4);
    w.m_offsets = take((d.n_experts + 1) * 4);
    w.m_perm = take(A * 4);
    w.m_pos = take(A * 4);
    w.m_tiles = take((size_t)w.max_tiles * 3 * 4);
    w.m_z = take(A * d.expert_intermediate * es);
    w.m_y = take(A * D * es);
    w.m_lrank = take(A * 4);
    w.m_blkcnt = take((size_t)moe_route_blocks((int)M) * d.n_experts * 4);
    w.m_blkoff = take((size_t)moe_route_blocks((int)M) * d.n_experts * 4);
  }
  w.total = o;
  return w;
}

template <typename T> T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

GemmParams gp() {
  GemmParams p;
  std::memset(&p, 0, sizeof p);
  p.scale = 1.f;
  return p;
}

// Row pitch of w_down in elements (dense rows unless the caller set one).
int ld_down_of(const gen_block_dims& d, const gen_block_weights& w) {
  return w.ld_down > 0 ? w.ld_down : d.mlp_intermediate;
}

// ------------------------------------------------------------------ one gen block
template <typename T>
hipError_t gemm_any(const GemmParams& p, int epi, hipStream_t s) {
  if (sizeof(T) == 2) return gemm_bf16(p, epi, s);
  return gemm_f32(p, epi, s);
}

// LoRA down-projection of the sites listed: t[:, slot*r:(slot+1)*r] = (alpha/r) x A_site^T.
// Returns the number of sites present; fills per-site column offsets (-1 if absent).
template <typename T>
hipError_t lora_down(const gen_block_dims& d, const gen_block_weights& w, const int* sites, int ns, const T* x, int K,
                     int M, T* t, int* off, int& ldt, hipStream_t s, float* part = nullptr, int ldx = 0) {
  GemmParams p = gp();
  int n = 0;
  for (int i = 0; i < ns; ++i) {
    off[i] = -1;
    if (w.lora_a[sites[i]]) { p.Bs[n] = w.lora_a[sites[i]]; off[i] = n * d.lora_rank; ++n; }
  }
  ldt = std::max(n, 1) * d.lora_rank;
  if (n == 0) return hipSuccess;
  p.A = x; p.lda = ldx ? ldx : K; p.B = p.Bs[0]; p.ldb = K;
  p.M = M; p.N = n * d.lora_rank; p.K = K;
  p.bmode = 2; p.seg_rows = d.lora_rank;
  p.C = t; p.ldc = ldt; p.scale = d.lora_alpha / (float)d.lora_rank;
  if (part && p.N <= 128 && K % 64 == 0) return gemm_skinny(p, part, s);
  return gemm_bf16(p, EPI_SCALED, s);
}

// The column offsets (and row pitch) that lora_down gives the sites listed, without computing t.
void lora_offsets(const gen_block_dims& d, const gen_block_weights& w, const int* sites, int ns, int* off, int& ldt) {
  int n = 0;
  for (int i = 0; i < ns; ++i) off[i] = w.lora_a[sites[i]] ? (n++) * d.lora_rank : -1;
  ldt = std::max(n, 1) * d.lora_rank;
}

// Attach the LoRA up-projection of the given sites as a K extension of p.
void lora_ext(GemmParams& p, const gen_block_dims& d, const gen_block_weights& w, const int* sites, int ns,
              const int* site_end, const void* t, int ldt, const int* off) {
  p.X = t; p.ldx = ldt; p.xk = ldt; p.xr = d.lora_rank;
  for (int i = 0; i < 3; ++i) {
    const int si = std::min(i, ns - 1);
    p.XB[i] = (i < ns && off[i] >= 0) ? w.lora_b[sites[i]] : nullptr;
    p.xsite_end[i] = site_end[si];
    p.xoff[i] = (i < ns && off[i] >= 0) ? off[i] : 0;
  }
}

bool lora_all(const gen_block_weights& w, const int* sites, int ns) {
  for (int i = 0; i < ns; ++i)
    if (!w.lora_b[sites[i]]) return false;
  return true;
}

// The LoRA up-projection as the K extension of the 32-deep ring GEMM when its shape allows (the
// low-rank term then joins the base product's fp32 accumulators, with no scratch round trip);
// false leaves p unchanged.
bool try_k32_ext(GemmParams& p, int epi, const gen_block_dims& d, const gen_block_weights& w, const int* sites,
                 int ns, const int* ends, const void* t, int ldt, const int* off) {
  bool any = false;
  for (int i = 0; i < ns; ++i) any = any || off[i] >= 0;
  if (!any) return false;
  GemmParams q = p;
  lora_ext(q, d, w, sites, ns, ends, t, ldt, off);
  if (!k32_ext_ok(q, epi)) return false;
  p = q;
  return true;
}

// LoRA up-projection as low-rank products: columns [ends[i-1], ends[i]) of C (op)= t_i B_i^T with
// t_i = columns off[i] .. off[i] + r of t.  mode 3 writes fp32 (the base GEMM then adds onto it
// with the fp32-residual epilogue and rounds the sum once), mode 2 adds into fp32, mode 0 writes
// bf16 (the SwiGLU epilogue's additive terms).
hipError_t lora_up(const gen_block_dims& d, const gen_block_weights& w, const int* sites, int ns, const int* ends,
                   const bf16* t, int ldt, const int* off, void* C, int64_t ldc, int M, int mode, hipStream_t s) {
  const int r = d.lora_rank;
  int start = 0;
  for (int i = 0; i < ns; ++i) {
    if (off[i] >= 0) {
      void* c = mode >= 2 ? (void*)((float*)C + start) : (void*)((bf16*)C + start);
      hipError_t e = gemm_lowrank(t + off[i], ldt, (const bf16*)w.lora_b[sites[i]], r, M, ends[i] - start, r, c, ldc,
                                  mode, s);
      if (e != hipSuccess) return e;
    }
    start = ends[i];
  }
  return hipSuccess;
}

// T: operand dtype (weights, GEMM/attention inputs); TH: residual-stream dtype of `hidden`.
// With an fp32 residual the O and down projections accumulate into `hidden` in place; with a
// bf16 residual the mid-block residual lives in the fp32 buffer hmid and `hidden` is rounded
// once, at the block output.
// kcache/vcache (prefix forward): per-sequence outputs [N, Hkv, d] receiving this block's normed,
// rotated keys and its values; attention is then causal.
template <typename T, typename TH>
int run_block(const gen_block_dims& d, const gen_block_weights& w, TH* hidden, const SeqInfo& si, void* ws,
              const Ws& L, int32_t* topk_out, hipStream_t s, void* const* kcache = nullptr,
              void* const* vcache = nullptr) {
  constexpr bool f32res = sizeof(TH) == 4;
  const int B = si.B, N = si.N, M = B * N, D = d.hidden;
  const int Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  const int QKV = (Hq + 2 * Hkv) * hd, QD = Hq * hd;
  const bool lora = d.lora_rank > 0;
  T* u = at<T>(ws, L.u);
  T* qkv = at<T>(ws, L.qkv);
  T* attn = at<T>(ws, L.attn);
  T* Kc = at<T>(ws, L.kc);
  T* Vt = at<T>(ws, L.vt);
  T* lt = at<T>(ws, L.lora_t);
  const float2* rope = at<float2>(ws, L.rope);

  float* hmid = f32res ? (float*)hidden : at<float>(ws, L.hmid);
  HIP_TRY((rmsnorm<TH, T>(hidden, (const T*)w.g_in, u, M, D, d.rms_eps, s)));
  {
    GemmParams p = gp();
    p.A = u; p.lda = D; p.B = w.w_qkv; p.ldb = D; p.M = M; p.N = QKV; p.K = D;
    p.C = qkv; p.ldc = QKV;
    p.part = L.splitk_floats ? at<float>(ws, L.splitk) : nullptr; p.part_floats = L.splitk_floats;
    int epi = EPI_STORE;
    if (lora) {
      const int sites[3] = {0, 1, 2}, ends[3] = {QD, QD + Hkv * hd, QKV};
      int off[3], ldt;
      HIP_TRY(lora_down<T>(d, w, sites, 3, u, D, M, lt, off, ldt, s, at<float>(ws, L.skinny)));
      if (sizeof(T) == 2 && try_k32_ext(p, EPI_STORE, d, w, sites, 3, ends, lt, ldt, off)) {
      } else if (lora_all(w, sites, 3)) {
        float* lf = at<float>(ws, L.lora_f32);
        HIP_TRY(lora_up(d, w, sites, 3, ends, (const bf16*)lt, ldt, off, lf, QKV, M, 3, s));
        epi = EPI_RESID_FROM_F32; p.R = lf; p.ldr = QKV;
      } else if (off[0] >= 0 || off[1] >= 0 || off[2] >= 0) {
        lora_ext(p, d, w, sites, 3, ends, lt, ldt, off);
      }
    }
    HIP_TRY(timed(FAM_QKV, s, [&] { return gemm_any<T>(p, epi, s); }));
  }
  if (kcache) {
    // prefix forward: normalise and rotate q, k in place, hand k and v to the cache, causal attention
    HIP_TRY(qknorm_rope<T>(qkv, QKV, si, Hq, Hkv, hd, (const T*)w.g_q, (const T*)w.g_k, rope, d.rms_eps, s));
    // the cache pointers are 16-byte aligned (checked at the boundary)
    HIP_TRY(kv_cache_write<T>(qkv, QKV, QD, N, Hkv * hd, B, kcache, vcache, s));
    HIP_TRY(pack_kv<T>(qkv, QKV, si, Hq, Hkv, hd, L.Lpad, Kc, Vt, s));
    if (sizeof(T) == 2)
      HIP_TRY(attention_bf16((const bf16*)qkv, QKV, si, Hq, Hkv, hd, L.Lpad, (const bf16*)Kc, (const bf16*)Vt,
                             (bf16*)attn, QD, nullptr, nullptr, 0.f, true, s));
    else
      HIP_TRY(attention_f32((const float*)qkv, QKV, si, Hq, Hkv, hd, L.Lpad, (const float*)Kc, (const float*)Vt,
                            (float*)attn, QD, true, s));
  } else if (sizeof(T) == 2) {
    // bf16: the QK-norm and RoPE ride along with the K packing and the attention's Q loads
    HIP_TRY(pack_kv_knorm((const bf16*)qkv, QKV, si, Hq, Hkv, hd, L.Lpad, (const bf16*)w.g_k, rope, d.rms_eps,
                          (bf16*)Kc, (bf16*)Vt, s));
    HIP_TRY(timed(FAM_ATTN, s, [&] {
      return attention_bf16((const bf16*)qkv, QKV, si, Hq, Hkv, hd, L.Lpad, (const bf16*)Kc, (const bf16*)Vt,
                            (bf16*)attn, QD, (const bf16*)w.g_q, rope, d.rms_eps, false, s);
    }));
  } else {
    HIP_TRY(qknorm_rope<T>(qkv, QKV, si, Hq, Hkv, hd, (const T*)w.g_q, (const T*)w.g_k, rope, d.rms_eps, s));
    HIP_TRY(pack_kv<T>(qkv, QKV, si, Hq, Hkv, hd, L.Lpad, Kc, Vt, s));
    HIP_TRY(timed(FAM_ATTN, s, [&] {
      return attention_f32((const float*)qkv, QKV, si, Hq, Hkv, hd, L.Lpad, (const float*)Kc, (const float*)Vt,
                           (float*)attn, QD, false, s);
    }));
  }
  {
    GemmParams p = gp();
    p.A = attn; p.lda = QD; p.B = w.w_o; p.ldb = QD; p.M = M; p.N = D; p.K = QD;
    p.C = hmid; p.ldc = D; p.R = hidden; p.ldr = D;
    p.part = L.splitk_floats ? at<float>(ws, L.splitk) : nullptr; p.part_floats = L.splitk_floats;
    const int sites[1] = {3}, ends[1] = {D};
    int off[1] = {-1}, ldt = 0;
    const int epi = f32res ? EPI_RESID_F32 : EPI_RESID_TO_F32;
    bool ext = false;
    if (lora) {
      HIP_TRY(lora_down<T>(d, w, sites, 1, attn, QD, M, lt, off, ldt, s, at<float>(ws, L.skinny)));
      ext = sizeof(T) == 2 && try_k32_ext(p, epi, d, w, sites, 1, ends, lt, ldt, off);
    }
    HIP_TRY(timed(FAM_O, s, [&] { return gemm_any<T>(p, epi, s); }));
    // otherwise the LoRA term accumulates into the fp32 mid-block residual
    if (off[0] >= 0 && !ext) HIP_TRY(lora_up(d, w, sites, 1, ends, (const bf16*)lt, ldt, off, hmid, D, M, 2, s));
  }
  HIP_TRY((rmsnorm<float, T>(hmid, (const T*)w.g_post, u, M, D, d.rms_eps, s)));
  if (d.mlp_intermediate > 0) {
    const int I = d.mlp_intermediate;
    const int LZ = z_pitch(I, sizeof(T));
    T* z = at<T>(ws, L.z);
    {
      GemmParams p = gp();
      p.A = u; p.lda = D; p.B = w.w_gate_up; p.ldb = D; p.M = M; p.N = 2 * I; p.K = D;
      p.bmode = 1; p.swiglu_I = I; p.C = z; p.ldc = LZ;
      if (lora) {
        const int sites[2] = {4, 5}, ends[2] = {I, 2 * I};
        int off[2], ldt;
        HIP_TRY(lora_down<T>(d, w, sites, 2, u, D, M, lt, off, ldt, s, at<float>(ws, L.skinny)));
        if (sizeof(T) == 2 && try_k32_ext(p, EPI_SWIGLU, d, w, sites, 2, ends, lt, ldt, off)) {
        } else if (lora_all(w, sites, 2)) {
          // gate and up LoRA terms, added by the SwiGLU epilogue before the activation
          T* lg = at<T>(ws, L.lora_gu);
          HIP_TRY(lora_up(d, w, sites, 2, ends, (const bf16*)lt, ldt, off, lg, 2 * I, M, 0, s));
          p.R = lg; p.ldr = 2 * I;
        } else if (off[0] >= 0 || off[1] >= 0) {
          lora_ext(p, d, w, sites, 2, ends, lt, ldt, off);
        }
      }
      HIP_TRY(timed(FAM_GATE_UP, s, [&] { return gemm_any<T>(p, EPI_SWIGLU, s); }));
    }
    {
      GemmParams p = gp();
      p.A = z; p.lda = LZ; p.B = w.w_down; p.ldb = ld_down_of(d, w); p.M = M; p.N = D; p.K = I;
      p.C = hidden; p.ldc = D; p.R = hmid; p.ldr = D;
      p.part = L.splitk_floats ? at<float>(ws, L.splitk) : nullptr; p.part_floats = L.splitk_floats;
      const int sites[1] = {6}, ends[1] = {D};
      int off[1] = {-1}, ldt = 0;
      bool post = false;
      const int epi = f32res ? EPI_RESID_F32 : EPI_RESID_FROM_F32;
      if (lora) {
        HIP_TRY(lora_down<T>(d, w, sites, 1, z, I, M, lt, off, ldt, s, at<float>(ws, L.skinny), LZ));
        // the K extension of the ring kernel where it applies; otherwise with an fp32 residual the
        // LoRA term is added after the base GEMM, and a bf16 residual keeps the K extension of the
        // register-staged kernel so that the block output is rounded once
        if (off[0] >= 0 && sizeof(T) == 2 && try_k32_ext(p, epi, d, w, sites, 1, ends, lt, ldt, off)) {
        } else if (off[0] >= 0 && f32res) {
          post = true;
        } else if (off[0] >= 0) {
          lora_ext(p, d, w, sites, 1, ends, lt, ldt, off);
        }
      }
      HIP_TRY(timed(FAM_DOWN, s, [&] { return gemm_any<T>(p, epi, s); }));
      if (post) HIP_TRY(lora_up(d, w, sites, 1, ends, (const bf16*)lt, ldt, off, hidden, D, M, 2, s));
    }
  } else {
    const int E = d.n_experts, k = d.top_k, Ie = d.expert_intermediate;
    int* idx = at<int>(ws, L.m_idx);
    float* wt = at<float>(ws, L.m_w);
    int* perm = at<int>(ws, L.m_perm);
    int* pos = at<int>(ws, L.m_pos);
    int* tiles = at<int>(ws, L.m_tiles);
    bf16* zp = at<bf16>(ws, L.m_z);
    bf16* yp = at<bf16>(ws, L.m_y);
    // routed from the fp32 mid-block residual through the post-attention norm, in fp32 (the
    // expert GEMMs take the bf16 copy u)
    int* lrank = at<int>(ws, L.m_lrank);
    int* blkcnt = at<int>(ws, L.m_blkcnt);
    HIP_TRY((moe_route<float, bf16>(hmid, (const bf16*)w.g_post, d.rms_eps, (const bf16*)w.w_router, M, D, E, k, idx,
                                    wt, lrank, blkcnt, s)));
    HIP_TRY(moe_sort(idx, lrank, blkcnt, at<int>(ws, L.m_blkoff), M, k, E, at<int>(ws, L.m_counts),
                     at<int>(ws, L.m_offsets), perm, pos, tiles, L.max_tiles, 256, s));
    {
      GemmParams p = gp();
      p.A = u; p.lda = D; p.a_rows = perm; p.B = w.w_exp_gate_up; p.ldb = D; p.N = 2 * Ie; p.K = D; p.M = M * k;
      p.bmode = 1; p.swiglu_I = Ie; p.C = zp; p.ldc = Ie;
      p.tiles = tiles; p.max_tiles = L.max_tiles; p.b_expert_stride = (int64_t)2 * Ie * D;
      HIP_TRY(timed(FAM_EXPERT, s, [&] { return gemm_bf16_grouped(p, EPI_SWIGLU, (Ie + 127) / 128, s); }));
    }
    {
      GemmParams p = gp();
      p.A = zp; p.lda = Ie; p.B = w.w_exp_down; p.ldb = Ie; p.N = D; p.K = Ie; p.M = M * k;
      p.C = yp; p.ldc = D;
      p.tiles = tiles; p.max_tiles = L.max_tiles; p.b_expert_stride = (int64_t)D * Ie;
      HIP_TRY(timed(FAM_EXPERT, s, [&] { return gemm_bf16_grouped(p, EPI_STORE, (D + 255) / 256, s); }));
    }
    HIP_TRY(moe_combine(hidden, hmid, yp, wt, pos, M, k, D, s));
    if (topk_out) HIP_TRY(hipMemcpyAsync(topk_out, idx, (size_t)M * k * 4, hipMemcpyDeviceToDevice, s));
  }
  return GEN_OK;
}

SeqInfo make_seq(int B, int N, const void* const* pk, const void* const* pv, const int* plen) {
  SeqInfo si;
  std::memset(&si, 0, sizeof si);
  si.B = B; si.N = N;
  for (int b = 0; b < B; ++b) {
    si.plen[b] = plen[b];
    si.pk[b] = plen[b] > 0 ? pk[b] : nullptr;
    si.pv[b] = plen[b] > 0 ? pv[b] : nullptr;
  }
  return si;
}

int check_prefix_ptrs(const SeqInfo& si, int layer) {
  for (int b = 0; b < si.B; ++b)
    if (si.plen[b] > 0) {
      if (!si.pk[b] || !si.pv[b]) return fail(GEN_EINVAL, "layer %d: prefix pointer of sequence %d is NULL", layer, b);
      if (!aligned16(si.pk[b]) || !aligned16(si.pv[b]))
        return fail(GEN_EINVAL, "layer %d: prefix pointer of sequence %d not 16-byte aligned", layer, b);
    }
  return GEN_OK;
}

// ------------------------------------------------------------------ training backward (one block)
// LoRA sites: 0 q, 1 k, 2 v, 3 o, 4 gate, 5 up, 6 down.
// What the backward of one block reads from its forward (one slot per block).
struct Wact {
  size_t u, qkv_raw, qkv_n, attn, lse, xmid, u2, gu, z, t_qkv, t_o, t_gu, t_down, total;
};

Wact layout_act(const gen_block_dims& d, int B, int N) {
  Wact w{};
  const size_t M = (size_t)B * N, D = d.hidden, I = d.mlp_intermediate, r = d.lora_rank;
  const size_t QD = (size_t)d.n_q_heads * d.head_dim, QKV = QD + 2 * (size_t)d.n_kv_heads * d.head_dim;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t a = o; o += up(bytes); return a; };
  w.u = take(M * D * 2);
  w.qkv_raw = take(M * QKV * 2);
  w.qkv_n = take(M * QKV * 2);
  w.attn = take(M * QD * 2);
  w.lse = take((size_t)B * d.n_q_heads * N * 4);
  w.xmid = take(M * D * 4);
  w.u2 = take(M * D * 2);
  w.gu = take(M * 2 * I * 2);
  w.z = take(M * (size_t)train_pitch((int)I) * 2);
  w.t_qkv = take(M * 3 * r * 2);
  w.t_o = take(M * r * 2);
  w.t_gu = take(M * 2 * r * 2);
  w.t_down = take(M * r * 2);
  w.total = o;
  return w;
}

// Scratch of the block backward; with_act: also one activation slot (gen_block_backward).
struct Wb {
  size_t act, kc, vt, rope, dot, tp, dyb, dz, dgu, du, dxf, dO, dq, dk, dv, dqkv, wt, xb, bt, part, lf, total;
  Wact A;
  int Lpad, n_pos;
};

Wb layout_bwd(const gen_block_dims& d, int B, int N, int max_prefix, bool with_act = true) {
  Wb w{};
  const size_t M = (size_t)B * N, D = d.hidden, I = d.mlp_intermediate, r = d.lora_rank;
  const size_t Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  const size_t QD = Hq * hd, KVD = Hkv * hd, QKV = QD + 2 * KVD;
  w.Lpad = (int)((max_prefix + N + 63) / 64 * 64);
  w.n_pos = max_prefix + N;
  w.A = layout_act(d, B, N);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t a = o; o += up(bytes); return a; };
  w.act = take(with_act ? w.A.total : 0);
  w.kc = take((size_t)B * Hkv * w.Lpad * hd * 2);
  w.vt = take((size_t)B * Hkv * w.Lpad * hd * 2);
  w.rope = take((size_t)w.n_pos * (hd / 2) * 8);
  w.dot = take((size_t)B * Hq * N * 4);
  w.tp = take(M * 3 * r * 2);
  w.dyb = take(M * D * 2);
  w.dz = take(M * I * 2);
  w.dgu = take(M * (size_t)train_pitch((int)(2 * I)) * 2);
  w.du = take(M * D * 2);
  w.dxf = take(M * D * 4);
  w.dO = take(M * QD * 2);
  w.dq = take(M * QD * 4);
  w.dk = take(M * KVD * 4);
  w.dv = take(M * KVD * 4);
  w.dqkv = take(M * QKV * 2);
  w.wt = take(std::max(std::max(QKV * D, QD * D), std::max((size_t)train_pitch((int)(2 * I)) * D, I * D)) * 2);
  w.xb = take(((size_t)D * 3 + QD + (size_t)D * 2 + I) * r * 2);   // A^T of the qkv, o, gate/up, down groups
  w.bt = take((size_t)r * (QKV + D + 2 * I + D) * 2);               // B^T of every site
  w.lf = take(r ? M * std::max(std::max(QKV, 2 * I), std::max(D, QD)) * 4 : 0);
  w.part = take(std::max(std::max((size_t)WGRAD_PART_FLOATS, r * std::max(std::max(QD, D), I)),
                         r ? skinny_part_floats((int)M, (int)std::min<size_t>(3 * r, 128)) : 0) * 4);
  w.total = o;
  return w;
}

struct BackSite {
  int site;     // LoRA site index
  int col;      // first column of the site in the gradient dY
  int out;      // its width (rows of lora_b)
};

// For the LoRA sites of one base GEMM whose output gradient is dY [M, lddy]:
//   tp[:, slot r:(slot+1) r] = (alpha/r) dY_site B_site   (dL/d(x A^T), scaled as the forward's t)
//   xb[:, slot r:(slot+1) r] = A_site^T
// and the fp32 scratch lf receives sum_site tp_site A_site, with p.R = lf: the base dgrad GEMM, run
// with the fp32-residual epilogue, adds dY W onto it and rounds once.  Returns the number of sites present (slot order =
// list order); with none, p is untouched and the GEMM runs with a plain store.
int lora_back(const gen_block_dims& d, const gen_block_weights& w, const BackSite* sites, int ns, const bf16* dY,
              int lddy, int in, int M, bf16* tp, bf16* xb, bf16* bt, GemmParams& p, int* slot, float* part,
              float* lf, hipStream_t s, const bf16* const* bts = nullptr) {
  const int r = d.lora_rank;
  int n = 0;
  for (int i = 0; i < ns; ++i) slot[i] = (r > 0 && w.lora_a[sites[i].site]) ? n++ : -1;
  if (n == 0) return 0;
  // every site of a group present at rank 32, side by side from column 0 of dY: one block-diagonal
  // skinny product reads dY once for all of them
  bool diag = bts && r == 32 && n == ns && ns >= 2;
  int outs[3] = {0, 0, 0}, col = 0;
  for (int i = 0; i < ns && diag; ++i) {
    diag = sites[i].col == col && sites[i].out % 64 == 0;
    outs[i] = sites[i].out;
    col += sites[i].out;
  }
  if (diag) HIP_TRY(gemm_skinny_diag(dY, lddy, M, bts, outs, ns, d.lora_alpha / (float)r, tp, n * r, part, s));
  for (int i = 0; i < ns; ++i) {
    if (slot[i] < 0) continue;
    const BackSite& st = sites[i];
    if (!bts) HIP_TRY(transpose_bf16((const bf16*)w.lora_b[st.site], r, bt, st.out, st.out, r, s));
    GemmParams q = gp();
    q.A = dY + st.col; q.lda = lddy; q.B = bts ? bts[i] : bt; q.ldb = st.out; q.M = M; q.N = r; q.K = st.out;
    q.C = tp + slot[i] * r; q.ldc = n * r; q.scale = d.lora_alpha / (float)r;
    if (diag) {
    } else if (r <= 128 && st.out % 64 == 0) HIP_TRY(gemm_skinny(q, part, s));
    else HIP_TRY(gemm_bf16(q, EPI_SCALED, s));
    if (!bts) HIP_TRY(transpose_bf16((const bf16*)w.lora_a[st.site], in, xb + slot[i] * r, n * r, r, in, s));
  }
  // sum_site tp_site A_site: as the K extension of the base dgrad GEMM ([tp | ...] against
  // [A_site^T | ...]), or into the fp32 scratch that the base GEMM adds onto; either way the sum is
  // rounded once
  GemmParams q = p;
  q.X = tp; q.ldx = n * r; q.xk = n * r; q.xr = n * r;
  for (int i = 0; i < 3; ++i) {
    q.XB[i] = i == 0 ? xb : nullptr;
    q.xoff[i] = 0;
    q.xsite_end[i] = p.N;
  }
  if (k32_ext_ok(q, EPI_STORE)) {
    p = q;
    return n;
  }
  HIP_TRY(gemm_lowrank(tp, n * r, xb, n * r, M, p.N, n * r, lf, p.N, 3, s));
  p.R = lf; p.ldr = p.N;
  return n;
}

// Weight gradients of the sites: dB_site += dY_site^T t_site (the forward's scaled x A^T, columns
// toff[i] of t), dA_site += tp_slot^T x.
int lora_wgrad(const gen_block_dims& d, const gen_lora_grads& g, const BackSite* sites, int ns, const int* slot, int n,
               const bf16* dY, int lddy, const bf16* t, int ldt, const int* toff, const bf16* tp, const bf16* x, int in,
               int M, float* part, hipStream_t s, int ldx = 0) {
  const int r = d.lora_rank;
  if (ldx == 0) ldx = in;                        // row pitch of x (in columns are used)
  // B gradients: a complete group whose sites sit side by side in dY and in t as one block-diagonal
  // pass, else site by site
  bool diag = n == ns && ns >= 2;
  int outs[3] = {0, 0, 0}, col = 0;
  float* dstb[3] = {nullptr, nullptr, nullptr};
  for (int i = 0; i < ns && diag; ++i) {
    diag = sites[i].col == col && sites[i].out % 128 == 0 && toff[i] == i * r;
    outs[i] = sites[i].out;
    dstb[i] = g.lora_b[sites[i].site];
    col += sites[i].out;
  }
  if (diag) {
    HIP_TRY(wgrad_diag(dY, lddy, t, ldt, M, outs, ns, r, dstb, part, s));
  } else {
    for (int i = 0; i < ns; ++i) {
      if (slot[i] < 0) continue;
      const int st = sites[i].site;
      HIP_TRY(wgrad(dY + sites[i].col, lddy, t + toff[i], ldt, M, sites[i].out, r, g.lora_b[st], part, s));
    }
  }
  // the A gradients of the sites sharing the input x: one pass over x with their dT side by side
  // (slot order), the row blocks of the product going to the sites' gradients
  if (n >= 2 && n * r <= 128) {
    float* dst[3] = {nullptr, nullptr, nullptr};
    for (int i = 0; i < ns; ++i)
      if (slot[i] >= 0) dst[slot[i]] = g.lora_a[sites[i].site];
    HIP_TRY(wgrad_seg(tp, n * r, x, ldx, M, n * r, in, r, dst, part, s));
    return GEN_OK;
  }
  for (int i = 0; i < ns; ++i)
    if (slot[i] >= 0) HIP_TRY(wgrad(tp + slot[i] * r, n * r, x, ldx, M, r, in, g.lora_a[sites[i].site], part, s));
  return GEN_OK;
}

// Forward of one dense gen block for training (bf16 operands, fp32 residual): keeps in the
// activation slot `act` what block_train_bwd reads; with h_out, also writes the block output
// h_out = h + attention + MLP (fp32).  Scratch in ws (layout L).
int block_train_fwd(const gen_block_dims& d, const gen_block_weights& w, const float* h, float* h_out,
                    const SeqInfo& si, void* act, void* ws, const Wb& L, hipStream_t s, bool rope_ready = false) {
  const int B = si.B, N = si.N, M = B * N, D = d.hidden, I = d.mlp_intermediate, r = d.lora_rank;
  const int Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  const int QD = Hq * hd, KVD = Hkv * hd, QKV = QD + 2 * KVD;
  const bool lora = r > 0;
  const float eps = d.rms_eps;
  bf16* u = at<bf16>(act, L.A.u);
  bf16* qkv_raw = at<bf16>(act, L.A.qkv_raw);
  bf16* qkv_n = at<bf16>(act, L.A.qkv_n);
  bf16* attn = at<bf16>(act, L.A.attn);
  float* lse = at<float>(act, L.A.lse);
  float* xmid = at<float>(act, L.A.xmid);
  bf16* u2 = at<bf16>(act, L.A.u2);
  bf16* gu = at<bf16>(act, L.A.gu);
  bf16* z = at<bf16>(act, L.A.z);
  bf16* t_qkv = at<bf16>(act, L.A.t_qkv);
  bf16* t_o = at<bf16>(act, L.A.t_o);
  bf16* t_gu = at<bf16>(act, L.A.t_gu);
  bf16* t_down = at<bf16>(act, L.A.t_down);
  float* part = at<float>(ws, L.part);
  float* lf = at<float>(ws, L.lf);
  const float2* rope = at<float2>(ws, L.rope);
  if (!rope_ready) HIP_TRY(rope_table(at<float2>(ws, L.rope), L.n_pos, hd, d.rope_theta, s));

  const int qkv_sites[3] = {0, 1, 2}, qkv_ends[3] = {QD, QD + KVD, QKV};
  const int o_site[1] = {3}, gu_sites[2] = {4, 5}, gu_ends[2] = {I, 2 * I}, down_site[1] = {6};
  int off_qkv[3] = {-1, -1, -1}, off_o[1] = {-1}, off_gu[2] = {-1, -1}, off_down[1] = {-1};
  int ld_qkv = r, ld_o = r, ld_gu = r, ld_down = r;
  HIP_TRY((rmsnorm<float, bf16>(h, (const bf16*)w.g_in, u, M, D, eps, s)));
  {
    GemmParams p = gp();
    p.A = u; p.lda = D; p.B = w.w_qkv; p.ldb = D; p.M = M; p.N = QKV; p.K = D; p.C = qkv_n; p.ldc = QKV;
    int epi = EPI_STORE;
    if (lora) {
      HIP_TRY(lora_down<bf16>(d, w, qkv_sites, 3, u, D, M, t_qkv, off_qkv, ld_qkv, s, part));
      if (try_k32_ext(p, EPI_STORE, d, w, qkv_sites, 3, qkv_ends, t_qkv, ld_qkv, off_qkv)) {
      } else if (lora_all(w, qkv_sites, 3)) {
        HIP_TRY(lora_up(d, w, qkv_sites, 3, qkv_ends, t_qkv, ld_qkv, off_qkv, lf, QKV, M, 3, s));
        epi = EPI_RESID_FROM_F32; p.R = lf; p.ldr = QKV;
      } else if (off_qkv[0] >= 0 || off_qkv[1] >= 0 || off_qkv[2] >= 0) {
        lora_ext(p, d, w, qkv_sites, 3, qkv_ends, t_qkv, ld_qkv, off_qkv);
      }
    }
    HIP_TRY(gemm_bf16(p, epi, s));
  }
  // q and k normed and rotated in place; their raw values (all the backward needs of them) to qkv_raw
  HIP_TRY(qknorm_rope<bf16>(qkv_n, QKV, si, Hq, Hkv, hd, (const bf16*)w.g_q, (const bf16*)w.g_k, rope, eps, s, qkv_raw));
  HIP_TRY(pack_kv<bf16>(qkv_n, QKV, si, Hq, Hkv, hd, L.Lpad, at<bf16>(ws, L.kc), at<bf16>(ws, L.vt), s));
  HIP_TRY(attention_bf16(qkv_n, QKV, si, Hq, Hkv, hd, L.Lpad, at<bf16>(ws, L.kc), at<bf16>(ws, L.vt), attn, QD,
                         nullptr, nullptr, 0.f, false, s, lse));
  {
    GemmParams p = gp();
    p.A = attn; p.lda = QD; p.B = w.w_o; p.ldb = QD; p.M = M; p.N = D; p.K = QD;
    p.C = xmid; p.ldc = D; p.R = h; p.ldr = D;
    bool ext = false;
    if (lora) {
      HIP_TRY(lora_down<bf16>(d, w, o_site, 1, attn, QD, M, t_o, off_o, ld_o, s, part));
      ext = try_k32_ext(p, EPI_RESID_F32, d, w, o_site, 1, &D, t_o, ld_o, off_o);
    }
    HIP_TRY(gemm_bf16(p, EPI_RESID_F32, s));
    if (off_o[0] >= 0 && !ext) HIP_TRY(lora_up(d, w, o_site, 1, &D, t_o, ld_o, off_o, xmid, D, M, 2, s));
  }
  HIP_TRY((rmsnorm<float, bf16>(xmid, (const bf16*)w.g_post, u2, M, D, eps, s)));
  {
    GemmParams p = gp();
    p.A = u2; p.lda = D; p.B = w.w_gate_up; p.ldb = D; p.M = M; p.N = 2 * I; p.K = D; p.C = gu; p.ldc = 2 * I;
    int epi = EPI_STORE;
    if (lora) {
      HIP_TRY(lora_down<bf16>(d, w, gu_sites, 2, u2, D, M, t_gu, off_gu, ld_gu, s, part));
      if (try_k32_ext(p, EPI_STORE, d, w, gu_sites, 2, gu_ends, t_gu, ld_gu, off_gu)) {
      } else if (lora_all(w, gu_sites, 2)) {
        HIP_TRY(lora_up(d, w, gu_sites, 2, gu_ends, t_gu, ld_gu, off_gu, lf, 2 * I, M, 3, s));
        epi = EPI_RESID_FROM_F32; p.R = lf; p.ldr = 2 * I;
      } else if (off_gu[0] >= 0 || off_gu[1] >= 0) {
        lora_ext(p, d, w, gu_sites, 2, gu_ends, t_gu, ld_gu, off_gu);
      }
    }
    HIP_TRY(timed(FAM_GATE_UP, s, [&] { return gemm_bf16(p, epi, s); }));
  }
  const int LZ = train_pitch(I);
  HIP_TRY(swiglu_fwd(gu, z, LZ, M, I, s));
  if (lora) HIP_TRY(lora_down<bf16>(d, w, down_site, 1, z, I, M, t_down, off_down, ld_down, s, part, LZ));

  if (h_out) {  // down projection onto the mid-block residual: the block output
    GemmParams p = gp();
    p.A = z; p.lda = LZ; p.B = w.w_down; p.ldb = ld_down_of(d, w); p.M = M; p.N = D; p.K = I;
    p.C = h_out; p.ldc = D; p.R = xmid; p.ldr = D;
    bool ext = false;
    if (off_down[0] >= 0) ext = try_k32_ext(p, EPI_RESID_F32, d, w, down_site, 1, &D, t_down, ld_down, off_down);
    HIP_TRY(gemm_bf16(p, EPI_RESID_F32, s));
    if (off_down[0] >= 0 && !ext) HIP_TRY(lora_up(d, w, down_site, 1, &D, t_down, ld_down, off_down, h_out, D, M, 2, s));
  }
  return GEN_OK;
}

// Gradient of one dense gen block from the activations block_train_fwd kept in `act`.  h: the
// block input [M, D] fp32; dh: in, dL/d(block output); out, dL/d(block input).  LoRA gradients
// accumulate into g.
// The frozen base weights as the backward's data-gradient operands, per layer: W_down^T [I, D],
// W_gate_up^T [D, train_pitch(2 I)], W_o^T [QD, D], W_qkv^T [D, QKV] (bf16).
struct FrozenT {
  size_t down, gu, o, qkv, stride;
};
FrozenT frozen_t_layout(const gen_block_dims& d) {
  FrozenT f{};
  const size_t D = d.hidden, I = d.mlp_intermediate, QD = (size_t)d.n_q_heads * d.head_dim;
  const size_t QKV = QD + 2 * (size_t)d.n_kv_heads * d.head_dim;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t a = o; o += up(bytes); return a; };
  f.down = take(I * D * 2);
  f.gu = take(D * (size_t)train_pitch((int)(2 * I)) * 2);
  f.o = take(QD * D * 2);
  f.qkv = take(D * QKV * 2);
  f.stride = o;
  return f;
}

// ft: nullable, this layer's cached transposes (frozen_t_layout); without them each data-gradient
// operand is transposed into the scratch wt on the call.
int block_train_bwd(const gen_block_dims& d, const gen_block_weights& w, const float* h, float* dh,
                    const SeqInfo& si, const gen_lora_grads& g, void* act, void* ws, const Wb& L, hipStream_t s,
                    bool dyb_ready, const char* ft = nullptr) {
  const FrozenT FT = frozen_t_layout(d);
  const int B = si.B, N = si.N, M = B * N, D = d.hidden, I = d.mlp_intermediate, r = d.lora_rank;
  const int Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  const int QD = Hq * hd, KVD = Hkv * hd, QKV = QD + 2 * KVD;
  const bool lora = r > 0;
  const float eps = d.rms_eps;
  bf16* u = at<bf16>(act, L.A.u);
  bf16* qkv_raw = at<bf16>(act, L.A.qkv_raw);
  bf16* qkv_n = at<bf16>(act, L.A.qkv_n);
  bf16* attn = at<bf16>(act, L.A.attn);
  float* lse = at<float>(act, L.A.lse);
  float* xmid = at<float>(act, L.A.xmid);
  bf16* u2 = at<bf16>(act, L.A.u2);
  bf16* gu = at<bf16>(act, L.A.gu);
  bf16* z = at<bf16>(act, L.A.z);
  bf16* t_qkv = at<bf16>(act, L.A.t_qkv);
  bf16* t_o = at<bf16>(act, L.A.t_o);
  bf16* t_gu = at<bf16>(act, L.A.t_gu);
  bf16* t_down = at<bf16>(act, L.A.t_down);
  float* part = at<float>(ws, L.part);
  float* lf = at<float>(ws, L.lf);
  const float2* rope = at<float2>(ws, L.rope);
  bf16* tp = at<bf16>(ws, L.tp);
  bf16* dyb = at<bf16>(ws, L.dyb);
  bf16* dz = at<bf16>(ws, L.dz);
  bf16* dgu = at<bf16>(ws, L.dgu);
  bf16* du = at<bf16>(ws, L.du);
  float* dxf = at<float>(ws, L.dxf);
  bf16* dO = at<bf16>(ws, L.dO);
  bf16* dqkv = at<bf16>(ws, L.dqkv);
  bf16* wt = at<bf16>(ws, L.wt);
  bf16* xb = at<bf16>(ws, L.xb);
  bf16* bt = at<bf16>(ws, L.bt);
  const int qkv_sites[3] = {0, 1, 2};
  const int o_site[1] = {3}, gu_sites[2] = {4, 5}, down_site[1] = {6};
  int off_qkv[3], off_o[1], off_gu[2], off_down[1];
  int ld_qkv, ld_o, ld_gu, ld_down;
  lora_offsets(d, w, qkv_sites, 3, off_qkv, ld_qkv);
  lora_offsets(d, w, o_site, 1, off_o, ld_o);
  lora_offsets(d, w, gu_sites, 2, off_gu, ld_gu);
  lora_offsets(d, w, down_site, 1, off_down, ld_down);
  (void)lse; (void)xmid; (void)eps; (void)lora;

  // ---- backward
  // every site's B^T and each site group's A^T block in one launch: B^T [r, out] per site, A^T of
  // a group [in, sites x r] with the present sites side by side (lora_back's slot order)
  const bf16* bts_down[1] = {nullptr};
  const bf16* bts_gu[2] = {nullptr, nullptr};
  const bf16* bts_o[1] = {nullptr};
  const bf16* bts_qkv[3] = {nullptr, nullptr, nullptr};
  bf16* xb_qkv = xb;
  bf16* xb_o = xb_qkv + (size_t)D * 3 * r;
  bf16* xb_gu = xb_o + (size_t)QD * r;
  bf16* xb_down = xb_gu + (size_t)D * 2 * r;
  if (lora) {
    TransposeJob jobs[TRANSPOSE_MAX_JOBS];
    int nj = 0;
    bf16* btp = bt;
    auto group = [&](const int* sites, const int* outs, int ns, int in, bf16* xbg, const bf16** bts) {
      int present = 0;
      for (int i = 0; i < ns; ++i) present += w.lora_a[sites[i]] ? 1 : 0;
      int slotn = 0;
      for (int i = 0; i < ns; ++i) {
        if (!w.lora_a[sites[i]]) continue;
        jobs[nj++] = {(const bf16*)w.lora_b[sites[i]], r, btp, outs[i], outs[i], r};
        bts[i] = btp;
        btp += (size_t)r * outs[i];
        jobs[nj++] = {(const bf16*)w.lora_a[sites[i]], in, xbg + slotn * r, present * r, r, in};
        ++slotn;
      }
    };
    const int s_down[1] = {6}, o_down[1] = {D}, s_gu[2] = {4, 5}, o_gu[2] = {I, I}, s_o[1] = {3}, o_o[1] = {D};
    const int s_qkv[3] = {0, 1, 2}, o_qkv[3] = {QD, KVD, KVD};
    group(s_down, o_down, 1, I, xb_down, bts_down);
    group(s_gu, o_gu, 2, D, xb_gu, bts_gu);
    group(s_o, o_o, 1, QD, xb_o, bts_o);
    group(s_qkv, o_qkv, 3, D, xb_qkv, bts_qkv);
    HIP_TRY(transpose_many(jobs, nj, s));
  }
  int slot[3], n;
  if (!dyb_ready) HIP_TRY(cast_f32_bf16(dh, dyb, (int64_t)M * D, s));
  {  // down projection: dz = dy W_down (+ LoRA)
    const BackSite bs[1] = {{6, 0, D}};
    GemmParams p = gp();
    const bf16* wdt = ft ? (const bf16*)(ft + FT.down) : wt;
    if (!ft) HIP_TRY(transpose_bf16((const bf16*)w.w_down, ld_down_of(d, w), wt, D, D, I, s));
    p.A = dyb; p.lda = D; p.B = wdt; p.ldb = D; p.M = M; p.N = I; p.K = D; p.C = dz; p.ldc = I;
    n = lora_back(d, w, bs, 1, dyb, D, I, M, tp, xb_down, bt, p, slot, part, lf, s, bts_down);
    if (n < 0) return n;
    HIP_TRY(gemm_bf16(p, p.R ? EPI_RESID_FROM_F32 : EPI_STORE, s));
    if (n > 0) {
      int rc = lora_wgrad(d, g, bs, 1, slot, n, dyb, D, t_down, ld_down, off_down, tp, z, I, M, part, s,
                          train_pitch(I));
      if (rc) return rc;
    }
  }
  const int LG = train_pitch(2 * I);
  HIP_TRY(swiglu_bwd(gu, dz, dgu, LG, M, I, s));
  {  // gate/up: du2 = dgate W_gate + dup W_up (+ LoRA)
    const BackSite bs[2] = {{4, 0, I}, {5, I, I}};
    GemmParams p = gp();
    const bf16* wgt = ft ? (const bf16*)(ft + FT.gu) : wt;
    if (!ft) HIP_TRY(transpose_bf16((const bf16*)w.w_gate_up, D, wt, LG, 2 * I, D, s));
    p.A = dgu; p.lda = LG; p.B = wgt; p.ldb = LG; p.M = M; p.N = D; p.K = 2 * I; p.C = du; p.ldc = D;
    n = lora_back(d, w, bs, 2, dgu, LG, D, M, tp, xb_gu, bt, p, slot, part, lf, s, bts_gu);
    if (n < 0) return n;
    HIP_TRY(gemm_bf16(p, p.R ? EPI_RESID_FROM_F32 : EPI_STORE, s));
    if (n > 0) {
      int rc = lora_wgrad(d, g, bs, 2, slot, n, dgu, LG, t_gu, ld_gu, off_gu, tp, u2, D, M, part, s);
      if (rc) return rc;
    }
  }
  HIP_TRY(rmsnorm_bwd(xmid, (const bf16*)w.g_post, du, dh, dxf, M, D, eps, s, dyb));
  {  // O projection: dO = dx W_o (+ LoRA)
    const BackSite bs[1] = {{3, 0, D}};
    GemmParams p = gp();
    const bf16* wot = ft ? (const bf16*)(ft + FT.o) : wt;
    if (!ft) HIP_TRY(transpose_bf16((const bf16*)w.w_o, QD, wt, D, D, QD, s));
    p.A = dyb; p.lda = D; p.B = wot; p.ldb = D; p.M = M; p.N = QD; p.K = D; p.C = dO; p.ldc = QD;
    n = lora_back(d, w, bs, 1, dyb, D, QD, M, tp, xb_o, bt, p, slot, part, lf, s, bts_o);
    if (n < 0) return n;
    HIP_TRY(gemm_bf16(p, p.R ? EPI_RESID_FROM_F32 : EPI_STORE, s));
    if (n > 0) {
      int rc = lora_wgrad(d, g, bs, 1, slot, n, dyb, D, t_o, ld_o, off_o, tp, attn, QD, M, part, s);
      if (rc) return rc;
    }
  }
  HIP_TRY(attention_bwd(qkv_n, QKV, si, Hq, Hkv, hd, attn, dO, lse, at<float>(ws, L.dot), at<float>(ws, L.dq),
                        at<float>(ws, L.dk), at<float>(ws, L.dv), s));
  HIP_TRY(qknorm_rope_bwd(qkv_raw, QKV, at<float>(ws, L.dq), at<float>(ws, L.dk), at<float>(ws, L.dv), si, Hq, Hkv, hd,
                          (const bf16*)w.g_q, (const bf16*)w.g_k, rope, eps, dqkv, QKV, s));
  {  // QKV projection: du = dqkv W_qkv (+ LoRA on q, k, v)
    const BackSite bs[3] = {{0, 0, QD}, {1, QD, KVD}, {2, QD + KVD, KVD}};
    GemmParams p = gp();
    const bf16* wqt = ft ? (const bf16*)(ft + FT.qkv) : wt;
    if (!ft) HIP_TRY(transpose_bf16((const bf16*)w.w_qkv, D, wt, QKV, QKV, D, s));
    p.A = dqkv; p.lda = QKV; p.B = wqt; p.ldb = QKV; p.M = M; p.N = D; p.K = QKV; p.C = du; p.ldc = D;
    n = lora_back(d, w, bs, 3, dqkv, QKV, D, M, tp, xb_qkv, bt, p, slot, part, lf, s, bts_qkv);
    if (n < 0) return n;
    HIP_TRY(gemm_bf16(p, p.R ? EPI_RESID_FROM_F32 : EPI_STORE, s));
    if (n > 0) {
      int rc = lora_wgrad(d, g, bs, 3, slot, n, dqkv, QKV, t_qkv, ld_qkv, off_qkv, tp, u, D, M, part, s);
      if (rc) return rc;
    }
  }
  // dL/d(block input), and its bf16 copy in dyb for the next block down the tower
  HIP_TRY(rmsnorm_bwd(h, (const bf16*)w.g_in, du, dxf, dh, M, D, eps, s, dyb));
  return GEN_OK;
}

// Gradient of one dense gen block: its training forward into the workspace's activation slot,
// then the backward from there.
int run_block_bwd(const gen_block_dims& d, const gen_block_weights& w, const float* h, float* dh, const SeqInfo& si,
                  const gen_lora_grads& g, void* ws, const Wb& L, hipStream_t s) {
  void* act = at<char>(ws, L.act);
  const int rc = block_train_fwd(d, w, h, nullptr, si, act, ws, L, s);
  if (rc) return rc;
  return block_train_bwd(d, w, h, dh, si, g, act, ws, L, s, false);
}

int check_train_dims(const gen_block_dims* d) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (d->dtype != GEN_BF16 || d->hidden_dtype != GEN_F32)
    return fail(GEN_EUNSUPPORTED, "the backward pass runs with bf16 weights and an fp32 residual stream");
  if (d->mlp_intermediate <= 0) return fail(GEN_EUNSUPPORTED, "the backward pass covers dense blocks only");
  if (d->head_dim != 128) return fail(GEN_EUNSUPPORTED, "the attention backward needs head_dim 128");
  return GEN_OK;
}

int check_grads(const gen_block_dims* d, const gen_block_weights* w, const gen_lora_grads* g, int layer) {
  if (d->lora_rank == 0) return GEN_OK;
  if (!g) return fail(GEN_EINVAL, "layer %d: grads is NULL", layer);
  for (int s = 0; s < 7; ++s)
    if (w->lora_a[s] && (!g->lora_a[s] || !g->lora_b[s]))
      return fail(GEN_EINVAL, "layer %d: LoRA site %d has no gradient buffers", layer, s);
  return GEN_OK;
}

}  // namespace

int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GEN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(GEN_EUNSUPPORTED, "device %d >= %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(GEN_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GEN_OK;
}

namespace {

// gen_block_forward over a caller workspace, or (noalloc) over this GPU's copy of `scratch`.
int block_forward_ws(const gen_block_dims* dims, const gen_block_weights* w, void* hidden, int B, int N,
                     const void* const* prefix_k, const void* const* prefix_v, const int* prefix_len,
                     int32_t* topk_idx_out, void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_weights(dims, w, 0))) return rc;
  if (!hidden || !aligned16(hidden)) return fail(GEN_EINVAL, "hidden is NULL or not 16-byte aligned");
  if (B < 1 || N < 1) return fail(GEN_EINVAL, "B=%d and N=%d must be >= 1", B, N);
  if (B > MAXB) return fail(GEN_EUNSUPPORTED, "B=%d > %d sequences per call", B, MAXB);
  int maxp = 0;
  if ((rc = check_prefix(dims, B, prefix_k, prefix_v, prefix_len, &maxp))) return rc;
  const SeqInfo si = make_seq(B, N, prefix_k, prefix_v, prefix_len);
  if ((rc = check_prefix_ptrs(si, 0))) return rc;
  if (!workspace || !aligned16(workspace)) return fail(GEN_EINVAL, "workspace is NULL or not 16-byte aligned");
  const Ws L = layout(*dims, 1, B, N, maxp);
  if (workspace_bytes < L.total) {
    if (noalloc)
      return fail(GEN_EWORKSPACE, "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                  "(use gen_block_forward with a workspace)", L.total, workspace_bytes);
    return fail(GEN_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, L.total);
  }
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(rope_table(at<float2>(workspace, L.rope), L.n_pos, dims->head_dim, dims->rope_theta, s));
  if (dims->dtype == GEN_BF16 && dims->hidden_dtype == GEN_F32)
    rc = run_block<bf16, float>(*dims, *w, (float*)hidden, si, workspace, L, topk_idx_out, s);
  else if (dims->dtype == GEN_BF16)
    rc = run_block<bf16, bf16>(*dims, *w, (bf16*)hidden, si, workspace, L, topk_idx_out, s);
  else
    rc = run_block<float, float>(*dims, *w, (float*)hidden, si, workspace, L, topk_idx_out, s);
  return rc ? rc : ok();
}

}  // namespace

// ==================================================================== exported
extern "C" {

const char* gen_last_error(void) { return g_err.c_str(); }

int gen_sigma_schedule(int steps, double shift, double* sigmas) {
  if (steps < 1) return fail(GEN_EINVAL, "steps %d < 1", steps);
  if (!sigmas) return fail(GEN_EINVAL, "sigmas is NULL");
  if (!(shift > 0.0) || !std::isfinite(shift)) return fail(GEN_EINVAL, "shift must be finite and > 0");
  for (int k = 0; k <= steps; ++k) {
    const double sgrid = 1.0 - (double)k / (double)steps;
    sigmas[k] = shift * sgrid / (1.0 + (shift - 1.0) * sgrid);
  }
  return ok();
}

size_t gen_workspace_size(const gen_block_dims* dims, int n_img, int n_br, int n_tokens, int max_prefix) {
  if (check_dims(dims) != GEN_OK) return 0;
  if (n_img < 1 || n_br < 1 || n_tokens < 1 || max_prefix < 0) {
    fail(GEN_EINVAL, "sizes must be positive");
    return 0;
  }
  g_err.clear();
  return layout(*dims, n_img, n_br, n_tokens, max_prefix).total;
}

int flow_euler_cfg(float* x, const float* x0_cond, const float* x0_uncond, size_t n, float cfg_scale, float sigma,
                   float sigma_next, float t_eps, void* stream) {
  if (!x || !x0_cond) return fail(GEN_EINVAL, "x and x0_cond must be non-NULL");
  if (!x0_uncond && cfg_scale != 1.0f) return fail(GEN_EINVAL, "x0_uncond is NULL but cfg_scale != 1");
  if (!aligned16(x) || !aligned16(x0_cond) || (x0_uncond && !aligned16(x0_uncond)))
    return fail(GEN_EINVAL, "pointers must be 16-byte aligned");
  if (!std::isfinite(cfg_scale) || !std::isfinite(sigma) || !std::isfinite(sigma_next) || !std::isfinite(t_eps))
    return fail(GEN_EINVAL, "scalars must be finite");
  if (!(std::max(sigma, t_eps) > 0.f)) return fail(GEN_EINVAL, "max(sigma, t_eps) must be > 0");
  HIP_TRY(cfg_euler(x, x, x0_cond, nullptr, x0_uncond, n, cfg_scale, 1.0f, sigma, sigma_next, t_eps,
                    (hipStream_t)stream));
  return ok();
}

int flow_euler_dual_cfg(float* x, const float* x0_cond, const float* x0_img, const float* x0_uncond, size_t n,
                        float cfg_scale, float img_cfg_scale, float sigma, float sigma_next, float t_eps,
                        void* stream) {
  if (!x || !x0_cond || !x0_img) return fail(GEN_EINVAL, "x, x0_cond and x0_img must be non-NULL");
  if (!x0_uncond && img_cfg_scale != 1.0f) return fail(GEN_EINVAL, "x0_uncond is NULL but img_cfg_scale != 1");
  if (!aligned16(x) || !aligned16(x0_cond) || !aligned16(x0_img) || (x0_uncond && !aligned16(x0_uncond)))
    return fail(GEN_EINVAL, "pointers must be 16-byte aligned");
  if (!std::isfinite(cfg_scale) || !std::isfinite(img_cfg_scale) || !std::isfinite(sigma) ||
      !std::isfinite(sigma_next) || !std::isfinite(t_eps))
    return fail(GEN_EINVAL, "scalars must be finite");
  if (!(std::max(sigma, t_eps) > 0.f)) return fail(GEN_EINVAL, "max(sigma, t_eps) must be > 0");
  HIP_TRY(cfg_euler(x, x, x0_cond, x0_img, x0_uncond, n, cfg_scale, img_cfg_scale, sigma, sigma_next, t_eps,
                    (hipStream_t)stream));
  return ok();
}

int gen_moe_route(const void* u, const void* w_router, int T, int D, int E, int top_k, int dtype, int32_t* idx_out,
                  float* w_out, void* stream) {
  if (!u || !w_router || !idx_out || !w_out) return fail(GEN_EINVAL, "NULL pointer argument");
  if (T < 0 || D <= 0 || D % 64 || E < 1 || E > 64 || top_k < 1 || top_k > E)
    return fail(GEN_EINVAL, "bad sizes T=%d D=%d (a positive multiple of 64) E=%d top_k=%d", T, D, E, top_k);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GEN_BF16)
    HIP_TRY((moe_route<bf16, bf16>((const bf16*)u, nullptr, 0.f, (const bf16*)w_router, T, D, E, top_k, idx_out, w_out,
                                   nullptr, nullptr, s)));
  else if (dtype == GEN_F32)
    HIP_TRY((moe_route<float, float>((const float*)u, nullptr, 0.f, (const float*)w_router, T, D, E, top_k, idx_out,
                                     w_out, nullptr, nullptr, s)));
  else return fail(GEN_EINVAL, "bad dtype %d", dtype);
  return ok();
}

int gen_block_forward(const gen_block_dims* dims, const gen_block_weights* w, void* hidden, int B, int N,
                      const void* const* prefix_k, const void* const* prefix_v, const int* prefix_len,
                      int32_t* topk_idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  return block_forward_ws(dims, w, hidden, B, N, prefix_k, prefix_v, prefix_len, topk_idx_out, workspace,
                          workspace_bytes, stream, false);
}

int gen_block_forward_noalloc(const gen_block_dims* dims, const gen_block_weights* w, void* hidden, int B, int N,
                              const void* const* prefix_k, const void* const* prefix_v, const int* prefix_len,
                              int32_t* topk_idx_out, void* stream) {
  void* ptr = nullptr;
  const int rc = noalloc_scratch(&ptr);
  if (rc) return rc;
  return block_forward_ws(dims, w, hidden, B, N, prefix_k, prefix_v, prefix_len, topk_idx_out, ptr,
                          PSF_GEN_NOALLOC_SCRATCH_BYTES, stream, true);
}

int gen_prefix_forward(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers, void* hidden,
                       int B, int P, void* const* k_cache, void* const* v_cache, int32_t* topk_idx_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_layers < 1) return fail(GEN_EINVAL, "n_layers %d < 1", n_layers);
  if (!layers) return fail(GEN_EINVAL, "layers is NULL");
  for (int l = 0; l < n_layers; ++l)
    if ((rc = check_weights(dims, &layers[l], l))) return rc;
  if (!hidden || !aligned16(hidden)) return fail(GEN_EINVAL, "hidden is NULL or not 16-byte aligned");
  if (B < 1 || P < 1) return fail(GEN_EINVAL, "B=%d and P=%d must be >= 1", B, P);
  if (B > MAXB) return fail(GEN_EUNSUPPORTED, "B=%d > %d sequences per call", B, MAXB);
  if (!k_cache || !v_cache) return fail(GEN_EINVAL, "k_cache/v_cache arrays are NULL");
  for (int i = 0; i < n_layers * B; ++i)
    if (!k_cache[i] || !v_cache[i] || !aligned16(k_cache[i]) || !aligned16(v_cache[i]))
      return fail(GEN_EINVAL, "cache pointer %d is NULL or not 16-byte aligned", i);
  if (!workspace || !aligned16(workspace)) return fail(GEN_EINVAL, "workspace is NULL or not 16-byte aligned");
  const Ws L = layout(*dims, 1, B, P, 0);
  if (workspace_bytes < L.total)
    return fail(GEN_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, L.total);
  SeqInfo si{};
  si.B = B;
  si.N = P;   // the prompt tokens play the role of the block's own tokens; no earlier cache
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(rope_table(at<float2>(workspace, L.rope), L.n_pos, dims->head_dim, dims->rope_theta, s));
  for (int l = 0; l < n_layers; ++l) {
    void* const* kc = k_cache + (size_t)l * B;
    void* const* vc = v_cache + (size_t)l * B;
    int32_t* tk = topk_idx_out && dims->n_experts > 0 ? topk_idx_out + (size_t)l * B * P * dims->top_k : nullptr;
    if (dims->dtype == GEN_BF16 && dims->hidden_dtype == GEN_F32)
      rc = run_block<bf16, float>(*dims, layers[l], (float*)hidden, si, workspace, L, tk, s, kc, vc);
    else if (dims->dtype == GEN_BF16)
      rc = run_block<bf16, bf16>(*dims, layers[l], (bf16*)hidden, si, workspace, L, tk, s, kc, vc);
    else
      rc = run_block<float, float>(*dims, layers[l], (float*)hidden, si, workspace, L, tk, s, kc, vc);
    if (rc) return rc;
  }
  return ok();
}

int gen_block_lora_merge(const gen_block_dims* dims, const gen_block_weights* w, void* w_qkv_out, void* w_o_out,
                         void* w_gate_up_out, void* w_down_out, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (dims->lora_rank == 0) return fail(GEN_EINVAL, "dims.lora_rank is 0: nothing to merge");
  if ((rc = check_weights(dims, w, 0))) return rc;
  void* outs[4] = {w_qkv_out, w_o_out, w_gate_up_out, w_down_out};
  for (void* o : outs)
    if (!o || !aligned16(o)) return fail(GEN_EINVAL, "merged weight outputs must be non-NULL and 16-byte aligned");
  const int D = dims->hidden, hd = dims->head_dim, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads;
  const int I = dims->mlp_intermediate, r = dims->lora_rank;
  const float scale = dims->lora_alpha / (float)r;
  // site s: (matrix, first row, rows, in)
  const void* mats[4] = {w->w_qkv, w->w_o, w->w_gate_up, w->w_down};
  const int mat[7] = {0, 0, 0, 1, 2, 2, 3};
  const int row0[7] = {0, Hq * hd, (Hq + Hkv) * hd, 0, 0, I, 0};
  const int rows[7] = {Hq * hd, Hkv * hd, Hkv * hd, D, I, I, D};
  const int ins[7] = {D, D, D, Hq * hd, D, D, I};
  hipStream_t s = (hipStream_t)stream;
  for (int site = 0; site < 7; ++site) {
    const int m = mat[site];
    const int64_t ld = m == 3 ? ld_down_of(*dims, *w) : ins[site];   // w_down_out keeps w_down's pitch
    const size_t off = (size_t)row0[site] * ld;
    if (dims->dtype == GEN_BF16) {
      HIP_TRY(lora_merge<bf16>((const bf16*)mats[m] + off, (const bf16*)w->lora_a[site], (const bf16*)w->lora_b[site],
                               (bf16*)outs[m] + off, rows[site], ins[site], ld, r, scale, s));
    } else {
      HIP_TRY(lora_merge<float>((const float*)mats[m] + off, (const float*)w->lora_a[site], (const float*)w->lora_b[site],
                                (float*)outs[m] + off, rows[site], ins[site], ld, r, scale, s));
    }
  }
  return ok();
}

int gen_tower_step(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers, const void* w_in,
                   const void* temb_w1, const void* temb_w2, const void* g_final, const void* w_out, const float* x_t,
                   int n_img, int n_br, int H, int W, const float* sigma, const float* sigma_next, float cfg_scale,
                   float img_cfg_scale, int cfg_norm, float t_eps, const void* const* prefix_k,
                   const void* const* prefix_v,
                   const int* prefix_len, float* x_out, float* x0_out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (n_layers < 0) return fail(GEN_EINVAL, "n_layers %d < 0", n_layers);
  if (n_layers > 0 && !layers) return fail(GEN_EINVAL, "layers is NULL");
  for (int l = 0; l < n_layers; ++l)
    if ((rc = check_weights(dims, &layers[l], l))) return rc;
  const void* glob[] = {w_in, temb_w1, temb_w2, g_final, w_out, x_t, x_out};
  const char* gname[] = {"w_in", "temb_w1", "temb_w2", "g_final", "w_out", "x_t", "x_out"};
  for (int i = 0; i < 7; ++i) {
    if (!glob[i]) return fail(GEN_EINVAL, "%s is NULL", gname[i]);
    if (!aligned16(glob[i])) return fail(GEN_EINVAL, "%s is not 16-byte aligned", gname[i]);
  }
  if (x0_out && !aligned16(x0_out)) return fail(GEN_EINVAL, "x0_out is not 16-byte aligned");
  if (n_img < 1) return fail(GEN_EINVAL, "n_img %d < 1", n_img);
  if (n_br < 1 || n_br > 3) return fail(GEN_EINVAL, "n_br %d must be 1, 2 or 3", n_br);
  if (n_img * n_br > MAXB) return fail(GEN_EUNSUPPORTED, "n_img*n_br = %d > %d", n_img * n_br, MAXB);
  if (H <= 0 || W <= 0 || H % 32 || W % 32) return fail(GEN_EINVAL, "H=%d and W=%d must be positive multiples of 32", H, W);
  if (!sigma) return fail(GEN_EINVAL, "sigma is NULL");
  if (cfg_norm != 0) return fail(GEN_EUNSUPPORTED, "cfg_norm %d: only 0 (\"none\") is supported", cfg_norm);
  if (!sigma_next && n_br != 1) return fail(GEN_EINVAL, "x0-only output (sigma_next NULL) needs n_br == 1");
  if (!std::isfinite(cfg_scale) || !std::isfinite(img_cfg_scale) || !std::isfinite(t_eps))
    return fail(GEN_EINVAL, "cfg_scale, img_cfg_scale and t_eps must be finite");
  for (int i = 0; i < n_img; ++i) {
    if (!std::isfinite(sigma[i])) return fail(GEN_EINVAL, "sigma[%d] is not finite", i);
    if (sigma_next) {
      if (!std::isfinite(sigma_next[i])) return fail(GEN_EINVAL, "sigma_next[%d] is not finite", i);
      if (!(std::max(sigma[i], t_eps) > 0.f)) return fail(GEN_EINVAL, "max(sigma[%d], t_eps) must be > 0", i);
    }
  }
  const int B = n_img * n_br, N = (H / 32) * (W / 32);
  int maxp = 0;
  if ((rc = check_prefix(dims, B, prefix_k ? prefix_k : nullptr, prefix_v, prefix_len, &maxp))) return rc;
  if (n_layers > 0 && maxp > 0 && (!prefix_k || !prefix_v)) return fail(GEN_EINVAL, "prefix arrays are NULL");
  for (int l = 0; l < n_layers; ++l) {
    const SeqInfo si = make_seq(B, N, prefix_k + (size_t)l * B, prefix_v + (size_t)l * B, prefix_len);
    if ((rc = check_prefix_ptrs(si, l))) return rc;
  }
  if (!workspace || !aligned16(workspace)) return fail(GEN_EINVAL, "workspace is NULL or not 16-byte aligned");
  const Ws L = layout(*dims, n_img, n_br, N, maxp);
  if (workspace_bytes < L.total)
    return fail(GEN_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, L.total);

  hipStream_t s = (hipStream_t)stream;
  const bool bf = dims->dtype == GEN_BF16;
  const int D = dims->hidden;
  const int M = B * N;
  void* hidden = at<char>(workspace, L.hidden);
  void* patches = at<char>(workspace, L.patches);
  float* temb = at<float>(workspace, L.temb);
  // timestep embedding, patch embedding (+ temb, copied to every branch)
  if (bf) HIP_TRY(timestep_embed<bf16>(sigma, (const bf16*)temb_w1, (const bf16*)temb_w2, at<float>(workspace, L.h1), temb, n_img, D, s));
  else HIP_TRY(timestep_embed<float>(sigma, (const float*)temb_w1, (const float*)temb_w2, at<float>(workspace, L.h1), temb, n_img, D, s));
  if (bf) HIP_TRY(patchify<bf16>(x_t, (bf16*)patches, n_img, H, W, s));
  else HIP_TRY(patchify<float>(x_t, (float*)patches, n_img, H, W, s));
  {
    GemmParams p = gp();
    p.A = patches; p.lda = 3072; p.B = w_in; p.ldb = 3072; p.M = n_img * N; p.N = D; p.K = 3072;
    p.C = hidden; p.ldc = D; p.bias = temb; p.rows_per = N; p.n_bcast = n_br;
    if (bf) HIP_TRY(gemm_bf16(p, EPI_BIAS_BCAST_F32, s));
    else HIP_TRY(gemm_f32(p, EPI_BIAS_BCAST_F32, s));
  }
  HIP_TRY(rope_table(at<float2>(workspace, L.rope), L.n_pos, dims->head_dim, dims->rope_theta, s));
  for (int l = 0; l < n_layers; ++l) {
    const SeqInfo si = make_seq(B, N, prefix_k + (size_t)l * B, prefix_v + (size_t)l * B, prefix_len);
    if (bf) rc = run_block<bf16, float>(*dims, layers[l], (float*)hidden, si, workspace, L, nullptr, s);
    else rc = run_block<float, float>(*dims, layers[l], (float*)hidden, si, workspace, L, nullptr, s);
    if (rc) return rc;
  }
  // final norm + out head (fp32, unpatchified)
  void* u = at<char>(workspace, L.u);
  if (bf) HIP_TRY((rmsnorm<float, bf16>((const float*)hidden, (const bf16*)g_final, (bf16*)u, M, D, dims->rms_eps, s)));
  else HIP_TRY((rmsnorm<float, float>((const float*)hidden, (const float*)g_final, (float*)u, M, D, dims->rms_eps, s)));
  float* x0 = x0_out ? x0_out : (sigma_next ? at<float>(workspace, L.x0) : x_out);
  {
    GemmParams p = gp();
    p.A = u; p.lda = D; p.B = w_out; p.ldb = D; p.M = M; p.N = 3072; p.K = D;
    p.C = x0; p.rows_per = N; p.img_H = H; p.img_W = W;
    if (bf) HIP_TRY(gemm_bf16(p, EPI_F32_IMG, s));
    else HIP_TRY(gemm_f32(p, EPI_F32_IMG, s));
  }
  const size_t img = (size_t)3 * H * W;
  if (!sigma_next) {
    if (x0 != x_out) HIP_TRY(hipMemcpyAsync(x_out, x0, (size_t)n_img * img * 4, hipMemcpyDeviceToDevice, s));
    return ok();
  }
  for (int i = 0; i < n_img; ++i) {
    // branches of image i: cond, then uncond (two) or img_cond, uncond (three)
    const float* xc = x0 + (size_t)i * n_br * img;
    const float* xm = n_br == 3 ? xc + img : nullptr;
    const float* xu = n_br >= 2 ? xc + (size_t)(n_br - 1) * img : nullptr;
    HIP_TRY(cfg_euler(x_out + i * img, x_t + i * img, xc, xm, xu, img, n_br >= 2 ? cfg_scale : 1.0f,
                      n_br == 3 ? img_cfg_scale : 1.0f, sigma[i], sigma_next[i], t_eps, s));
  }
  return ok();
}


// ------------------------------------------------------------------ training backward
size_t gen_backward_workspace_size(const gen_block_dims* dims, int B, int N, int max_prefix) {
  if (check_train_dims(dims) != GEN_OK) return 0;
  if (B < 1 || N < 1 || max_prefix < 0) {
    fail(GEN_EINVAL, "sizes must be positive");
    return 0;
  }
  g_err.clear();
  return layout_bwd(*dims, B, N, max_prefix).total;
}

int gen_block_backward(const gen_block_dims* dims, const gen_block_weights* w, const float* hidden_in, float* d_hidden,
                       int B, int N, const void* const* prefix_k, const void* const* prefix_v, const int* prefix_len,
                       const gen_lora_grads* grads, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_train_dims(dims);
  if (rc) return rc;
  if ((rc = check_weights(dims, w, 0))) return rc;
  if ((rc = check_grads(dims, w, grads, 0))) return rc;
  if (!hidden_in || !d_hidden || !aligned16(hidden_in) || !aligned16(d_hidden))
    return fail(GEN_EINVAL, "hidden_in/d_hidden NULL or not 16-byte aligned");
  if (B < 1 || N < 1) return fail(GEN_EINVAL, "B=%d and N=%d must be >= 1", B, N);
  if (B > MAXB) return fail(GEN_EUNSUPPORTED, "B=%d > %d sequences per call", B, MAXB);
  int maxp = 0;
  if ((rc = check_prefix(dims, B, prefix_k, prefix_v, prefix_len, &maxp))) return rc;
  const SeqInfo si = make_seq(B, N, prefix_k, prefix_v, prefix_len);
  if ((rc = check_prefix_ptrs(si, 0))) return rc;
  if (!workspace || !aligned16(workspace)) return fail(GEN_EINVAL, "workspace is NULL or not 16-byte aligned");
  const Wb L = layout_bwd(*dims, B, N, maxp);
  if (workspace_bytes < L.total) return fail(GEN_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, L.total);
  gen_lora_grads none{};
  rc = run_block_bwd(*dims, *w, hidden_in, d_hidden, si, grads ? *grads : none, workspace, L, (hipStream_t)stream);
  return rc ? rc : ok();
}

namespace {
constexpr int LOSS_PARTS = 1024;
struct Wt {
  size_t fwd, bwd, saved, acts, act_stride, dh, pred, dpred, dtok, dhn, parts, woutT, total;
};
Wt layout_train(const gen_block_dims& d, int n_layers, int n_img, int N, int maxp) {
  Wt w{};
  const size_t M = (size_t)n_img * N, D = d.hidden;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t a = o; o += up(bytes); return a; };
  w.fwd = take(layout(d, n_img, 1, N, maxp).total);
  w.bwd = take(layout_bwd(d, n_img, N, maxp, false).total);
  w.saved = take((size_t)n_layers * M * D * 4);
  w.act_stride = up(layout_act(d, n_img, N).total);
  w.acts = take((size_t)n_layers * w.act_stride);
  w.dh = take(M * D * 4);
  w.pred = take(M * 3072 * 4);
  w.dpred = take(M * 3072 * 4);
  w.dtok = take(M * 3072 * 2);
  w.dhn = take(M * D * 2);
  w.parts = take(LOSS_PARTS * 4);
  w.woutT = take(3072 * D * 2);
  w.total = o;
  return w;
}
}  // namespace

size_t gen_train_workspace_size(const gen_block_dims* dims, int n_layers, int n_img, int n_tokens, int max_prefix) {
  if (check_train_dims(dims) != GEN_OK) return 0;
  if (n_layers < 1 || n_img < 1 || n_tokens < 1 || max_prefix < 0) {
    fail(GEN_EINVAL, "sizes must be positive");
    return 0;
  }
  g_err.clear();
  return layout_train(*dims, n_layers, n_img, n_tokens, max_prefix).total;
}

int gen_tower_lora_train_step(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers,
                              const void* w_in, const void* temb_w1, const void* temb_w2, const void* g_final,
                              const void* w_out, const float* x_t, const float* x0, int n_img, int H, int W,
                              const float* sigma, const void* const* prefix_k, const void* const* prefix_v,
                              const int* prefix_len, const gen_lora_grads* grads, float* loss, float* x0_pred_out,
                              const void* frozen_t, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_train_dims(dims);
  if (rc) return rc;
  if (n_layers < 1) return fail(GEN_EINVAL, "n_layers %d < 1", n_layers);
  if (!layers) return fail(GEN_EINVAL, "layers is NULL");
  for (int l = 0; l < n_layers; ++l) {
    if ((rc = check_weights(dims, &layers[l], l))) return rc;
    if ((rc = check_grads(dims, &layers[l], grads ? &grads[l] : nullptr, l))) return rc;
  }
  const void* glob[] = {w_in, temb_w1, temb_w2, g_final, w_out, x_t, x0, loss};
  const char* gname[] = {"w_in", "temb_w1", "temb_w2", "g_final", "w_out", "x_t", "x0", "loss"};
  for (int i = 0; i < 8; ++i) {
    if (!glob[i]) return fail(GEN_EINVAL, "%s is NULL", gname[i]);
    if (i < 7 && !aligned16(glob[i])) return fail(GEN_EINVAL, "%s is not 16-byte aligned", gname[i]);
  }
  if (x0_pred_out && !aligned16(x0_pred_out)) return fail(GEN_EINVAL, "x0_pred_out is not 16-byte aligned");
  if (frozen_t && !aligned16(frozen_t)) return fail(GEN_EINVAL, "frozen_t is not 16-byte aligned");
  if (n_img < 1) return fail(GEN_EINVAL, "n_img %d < 1", n_img);
  if (n_img > MAXB) return fail(GEN_EUNSUPPORTED, "n_img = %d > %d", n_img, MAXB);
  if (H <= 0 || W <= 0 || H % 32 || W % 32) return fail(GEN_EINVAL, "H=%d and W=%d must be positive multiples of 32", H, W);
  if (!sigma) return fail(GEN_EINVAL, "sigma is NULL");
  for (int i = 0; i < n_img; ++i)
    if (!std::isfinite(sigma[i])) return fail(GEN_EINVAL, "sigma[%d] is not finite", i);
  const int B = n_img, N = (H / 32) * (W / 32), M = B * N, D = dims->hidden;
  int maxp = 0;
  if ((rc = check_prefix(dims, B, prefix_k, prefix_v, prefix_len, &maxp))) return rc;
  for (int l = 0; l < n_layers; ++l) {
    const SeqInfo si = make_seq(B, N, prefix_k + (size_t)l * B, prefix_v + (size_t)l * B, prefix_len);
    if ((rc = check_prefix_ptrs(si, l))) return rc;
  }
  if (!workspace || !aligned16(workspace)) return fail(GEN_EINVAL, "workspace is NULL or not 16-byte aligned");
  const Wt T = layout_train(*dims, n_layers, n_img, N, maxp);
  if (workspace_bytes < T.total) return fail(GEN_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, T.total);

  hipStream_t s = (hipStream_t)stream;
  void* fws = at<char>(workspace, T.fwd);
  const Ws F = layout(*dims, n_img, 1, N, maxp);
  float* hidden = at<float>(fws, F.hidden);
  // forward, saving each block's input
  HIP_TRY(timestep_embed<bf16>(sigma, (const bf16*)temb_w1, (const bf16*)temb_w2, at<float>(fws, F.h1),
                               at<float>(fws, F.temb), n_img, D, s));
  HIP_TRY(patchify<bf16>(x_t, at<bf16>(fws, F.patches), n_img, H, W, s));
  {
    GemmParams p = gp();
    p.A = at<bf16>(fws, F.patches); p.lda = 3072; p.B = w_in; p.ldb = 3072; p.M = M; p.N = D; p.K = 3072;
    p.C = hidden; p.ldc = D; p.bias = at<float>(fws, F.temb); p.rows_per = N; p.n_bcast = 1;
    HIP_TRY(gemm_bf16(p, EPI_BIAS_BCAST_F32, s));
  }
  // the blocks' training forwards: block l reads its input from saved[l], keeps its activations
  // in slot l and writes its output into saved[l + 1] (the last one into hidden)
  void* bws = at<char>(workspace, T.bwd);
  const Wb L = layout_bwd(*dims, n_img, N, maxp, false);
  float* saved = at<float>(workspace, T.saved);
  HIP_TRY(hipMemcpyAsync(saved, hidden, (size_t)M * D * 4, hipMemcpyDeviceToDevice, s));
  for (int l = 0; l < n_layers; ++l) {
    const SeqInfo si = make_seq(B, N, prefix_k + (size_t)l * B, prefix_v + (size_t)l * B, prefix_len);
    float* out = l + 1 < n_layers ? saved + (size_t)(l + 1) * M * D : hidden;
    void* act = at<char>(workspace, T.acts + (size_t)l * T.act_stride);
    if ((rc = block_train_fwd(*dims, layers[l], saved + (size_t)l * M * D, out, si, act, bws, L, s, l > 0))) return rc;
  }
  bf16* u = at<bf16>(fws, F.u);
  HIP_TRY((rmsnorm<float, bf16>(hidden, (const bf16*)g_final, u, M, D, dims->rms_eps, s)));
  float* pred = x0_pred_out ? x0_pred_out : at<float>(workspace, T.pred);
  {
    GemmParams p = gp();
    p.A = u; p.lda = D; p.B = w_out; p.ldb = D; p.M = M; p.N = 3072; p.K = D;
    p.C = pred; p.rows_per = N; p.img_H = H; p.img_W = W;
    HIP_TRY(gemm_bf16(p, EPI_F32_IMG, s));
  }
  // loss and its gradient with respect to the prediction, back through the head and final norm
  float* dpred = at<float>(workspace, T.dpred);
  HIP_TRY(x0_loss(pred, x0, dpred, at<float>(workspace, T.parts), LOSS_PARTS, loss, (int64_t)M * 3072, s));
  bf16* dtok = at<bf16>(workspace, T.dtok);
  HIP_TRY(patchify<bf16>(dpred, dtok, n_img, H, W, s));
  bf16* woutT = at<bf16>(workspace, T.woutT);
  HIP_TRY(transpose_bf16((const bf16*)w_out, D, woutT, 3072, 3072, D, s));
  bf16* dhn = at<bf16>(workspace, T.dhn);
  {
    GemmParams p = gp();
    p.A = dtok; p.lda = 3072; p.B = woutT; p.ldb = 3072; p.M = M; p.N = D; p.K = 3072; p.C = dhn; p.ldc = D;
    HIP_TRY(gemm_bf16(p, EPI_STORE, s));
  }
  float* dh = at<float>(workspace, T.dh);
  HIP_TRY(rmsnorm_bwd(hidden, (const bf16*)g_final, dhn, nullptr, dh, M, D, dims->rms_eps, s, at<bf16>(bws, L.dyb)));
  gen_lora_grads none{};
  for (int l = n_layers - 1; l >= 0; --l) {
    const SeqInfo si = make_seq(B, N, prefix_k + (size_t)l * B, prefix_v + (size_t)l * B, prefix_len);
    void* act = at<char>(workspace, T.acts + (size_t)l * T.act_stride);
    const char* ft = frozen_t ? (const char*)frozen_t + (size_t)l * frozen_t_layout(*dims).stride : nullptr;
    rc = block_train_bwd(*dims, layers[l], saved + (size_t)l * M * D, dh, si, grads ? grads[l] : none, act, bws, L, s,
                         true, ft);
    if (rc) return rc;
  }
  return ok();
}

size_t gen_train_frozen_t_size(const gen_block_dims* dims, int n_layers) {
  if (check_train_dims(dims) || n_layers < 1) return 0;
  return (size_t)n_layers * frozen_t_layout(*dims).stride;
}

int gen_train_frozen_t(const gen_block_dims* dims, int n_layers, const gen_block_weights* layers, void* frozen_t,
                       size_t bytes, void* stream) {
  int rc = check_train_dims(dims);
  if (rc) return rc;
  if (n_layers < 1) return fail(GEN_EINVAL, "n_layers %d < 1", n_layers);
  if (!layers) return fail(GEN_EINVAL, "layers is NULL");
  for (int l = 0; l < n_layers; ++l)
    if ((rc = check_weights(dims, &layers[l], l))) return rc;
  if (!frozen_t || !aligned16(frozen_t)) return fail(GEN_EINVAL, "frozen_t is NULL or not 16-byte aligned");
  const FrozenT F = frozen_t_layout(*dims);
  if (bytes < (size_t)n_layers * F.stride)
    return fail(GEN_EWORKSPACE, "frozen_t %zu bytes < %zu required", bytes, (size_t)n_layers * F.stride);
  hipStream_t s = (hipStream_t)stream;
  const int D = dims->hidden, I = dims->mlp_intermediate, QD = dims->n_q_heads * dims->head_dim;
  const int QKV = QD + 2 * dims->n_kv_heads * dims->head_dim, LG = train_pitch(2 * I);
  for (int l = 0; l < n_layers; ++l) {
    const gen_block_weights& w = layers[l];
    char* ft = (char*)frozen_t + (size_t)l * F.stride;
    HIP_TRY(transpose_bf16((const bf16*)w.w_down, ld_down_of(*dims, w), (bf16*)(ft + F.down), D, D, I, s));
    HIP_TRY(transpose_bf16((const bf16*)w.w_gate_up, D, (bf16*)(ft + F.gu), LG, 2 * I, D, s));
    HIP_TRY(transpose_bf16((const bf16*)w.w_o, QD, (bf16*)(ft + F.o), D, D, QD, s));
    HIP_TRY(transpose_bf16((const bf16*)w.w_qkv, D, (bf16*)(ft + F.qkv), QKV, QKV, D, s));
  }
  return ok();
}

}  // extern "C"

// ==================================================================== step-level entry points
#include "../../include/psf_gen_ops.h"

namespace {
int check_dtype(int dtype) {
  if (dtype != GEN_F32 && dtype != GEN_BF16) return fail(GEN_EINVAL, "bad dtype %d", dtype);
  return GEN_OK;
}
size_t op_ws(int B, int N, int Hkv, int d, int maxp, int dtype, size_t* kc, size_t* vt, size_t* rope) {
  const size_t es = dtype == GEN_BF16 ? 2 : 4;
  const size_t Lpad = (size_t)(maxp + N + 63) / 64 * 64;
  size_t o = 0;
  *kc = o; o += up((size_t)B * Hkv * Lpad * d * es);
  *vt = o; o += up((size_t)B * Hkv * Lpad * d * es);
  *rope = o; o += up((size_t)(maxp + N) * (d / 2) * 8);
  return o;
}
}  // namespace

extern "C" {

size_t gen_op_workspace_size(int B, int N, int Hkv, int d, int max_prefix, int dtype) {
  size_t a, b, c;
  if (B < 1 || N < 1 || Hkv < 1 || d < 1 || max_prefix < 0 || check_dtype(dtype)) return 0;
  return op_ws(B, N, Hkv, d, max_prefix, dtype, &a, &b, &c);
}

int gen_op_rmsnorm(const void* x, const void* g, void* y, int rows, int D, float eps, int dtype, void* stream) {
  if (check_dtype(dtype)) return GEN_EINVAL;
  if (!x || !g || !y || !aligned16(x) || !aligned16(g) || !aligned16(y)) return fail(GEN_EINVAL, "NULL or unaligned pointer");
  if (rows < 0 || D <= 0 || D % 64) return fail(GEN_EINVAL, "rows %d, D %d (D must be a positive multiple of 64)", rows, D);
  if (D > 8192) return fail(GEN_EUNSUPPORTED, "D %d > 8192", D);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GEN_BF16) HIP_TRY((rmsnorm<bf16, bf16>((const bf16*)x, (const bf16*)g, (bf16*)y, rows, D, eps, s)));
  else HIP_TRY((rmsnorm<float, float>((const float*)x, (const float*)g, (float*)y, rows, D, eps, s)));
  return ok();
}

int gen_op_linear(const void* x, const void* w, void* y, const void* resid, int M, int N, int K, int epi, int dtype,
                  void* stream) {
  if (check_dtype(dtype)) return GEN_EINVAL;
  if (!x || !w || !y || !aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(GEN_EINVAL, "NULL or unaligned pointer");
  if (M < 0 || N <= 0 || K <= 0 || K % 64) return fail(GEN_EINVAL, "M %d N %d K %d (K must be a positive multiple of 64)", M, N, K);
  if (epi < 0 || epi > 3) return fail(GEN_EINVAL, "epi %d not in 0..3", epi);
  if (epi == 3 && dtype != GEN_BF16) return fail(GEN_EUNSUPPORTED, "epi 3 needs dtype GEN_BF16");
  if (epi == 1 && !resid) return fail(GEN_EINVAL, "epi 1 needs resid");
  if (epi == 2 && N % 8) return fail(GEN_EINVAL, "epi 2 needs N %% 8 == 0");
  GemmParams p = gp();
  p.A = x; p.lda = K; p.B = w; p.ldb = K; p.M = M; p.K = K; p.C = y;
  int e = EPI_STORE;
  if (epi == 0) { p.N = N; p.ldc = N; }
  if (epi == 1) { p.N = N; p.ldc = N; p.R = resid; p.ldr = N; e = EPI_RESID; }
  if (epi == 2) { p.N = 2 * N; p.ldc = N; p.bmode = 1; p.swiglu_I = N; e = EPI_SWIGLU; }
  if (epi == 3) { p.N = N; p.ldc = N; p.R = y; p.ldr = N; e = EPI_RESID_F32; }
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GEN_BF16) HIP_TRY(gemm_bf16(p, e, s));
  else HIP_TRY(gemm_f32(p, e, s));
  return ok();
}

int gen_op_qknorm_rope(void* qkv, int B, int N, int Hq, int Hkv, int d, const int* prefix_len, const void* g_q,
                       const void* g_k, float eps, float theta, void* workspace, size_t workspace_bytes, int dtype,
                       void* stream) {
  if (check_dtype(dtype)) return GEN_EINVAL;
  if (!qkv || !g_q || !g_k || !prefix_len || !workspace) return fail(GEN_EINVAL, "NULL pointer argument");
  if (B < 1 || B > MAXB || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || (d != 64 && d != 128))
    return fail(GEN_EINVAL, "bad sizes B=%d N=%d Hq=%d Hkv=%d d=%d", B, N, Hq, Hkv, d);
  int maxp = 0;
  for (int b = 0; b < B; ++b) {
    if (prefix_len[b] < 0) return fail(GEN_EINVAL, "prefix_len[%d] < 0", b);
    maxp = std::max(maxp, prefix_len[b]);
  }
  size_t kc, vt, ro;
  const size_t need = op_ws(B, N, Hkv, d, maxp, dtype, &kc, &vt, &ro);
  if (workspace_bytes < need) return fail(GEN_EWORKSPACE, "workspace %zu < %zu", workspace_bytes, need);
  SeqInfo si;
  std::memset(&si, 0, sizeof si);
  si.B = B; si.N = N;
  for (int b = 0; b < B; ++b) si.plen[b] = prefix_len[b];
  hipStream_t s = (hipStream_t)stream;
  float2* table = at<float2>(workspace, ro);
  HIP_TRY(rope_table(table, maxp + N, d, theta, s));
  const int64_t ld = (int64_t)(Hq + 2 * Hkv) * d;
  if (dtype == GEN_BF16) HIP_TRY(qknorm_rope<bf16>((bf16*)qkv, ld, si, Hq, Hkv, d, (const bf16*)g_q, (const bf16*)g_k, table, eps, s));
  else HIP_TRY(qknorm_rope<float>((float*)qkv, ld, si, Hq, Hkv, d, (const float*)g_q, (const float*)g_k, table, eps, s));
  return ok();
}

int gen_op_attention(const void* qkv, int B, int N, int Hq, int Hkv, int d, const void* const* prefix_k,
                     const void* const* prefix_v, const int* prefix_len, void* out, void* workspace,
                     size_t workspace_bytes, int dtype, void* stream) {
  if (check_dtype(dtype)) return GEN_EINVAL;
  if (!qkv || !out || !prefix_len || !workspace) return fail(GEN_EINVAL, "NULL pointer argument");
  if (B < 1 || B > MAXB || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || (d != 64 && d != 128))
    return fail(GEN_EINVAL, "bad sizes B=%d N=%d Hq=%d Hkv=%d d=%d", B, N, Hq, Hkv, d);
  int maxp = 0, rc;
  if ((rc = check_prefix(nullptr, B, prefix_k, prefix_v, prefix_len, &maxp))) return rc;
  const SeqInfo si = make_seq(B, N, prefix_k, prefix_v, prefix_len);
  if ((rc = check_prefix_ptrs(si, 0))) return rc;
  size_t kc, vt, ro;
  const size_t need = op_ws(B, N, Hkv, d, maxp, dtype, &kc, &vt, &ro);
  if (workspace_bytes < need) return fail(GEN_EWORKSPACE, "workspace %zu < %zu", workspace_bytes, need);
  const int Lpad = (maxp + N + 63) / 64 * 64;
  const int64_t ld = (int64_t)(Hq + 2 * Hkv) * d;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GEN_BF16) {
    HIP_TRY(pack_kv<bf16>((const bf16*)qkv, ld, si, Hq, Hkv, d, Lpad, at<bf16>(workspace, kc), at<bf16>(workspace, vt), s));
    HIP_TRY(attention_bf16((const bf16*)qkv, ld, si, Hq, Hkv, d, Lpad, at<bf16>(workspace, kc), at<bf16>(workspace, vt),
                           (bf16*)out, (int64_t)Hq * d, nullptr, nullptr, 0.f, false, s));
  } else {
    HIP_TRY(pack_kv<float>((const float*)qkv, ld, si, Hq, Hkv, d, Lpad, at<float>(workspace, kc), at<float>(workspace, vt), s));
    HIP_TRY(attention_f32((const float*)qkv, ld, si, Hq, Hkv, d, Lpad, at<float>(workspace, kc), at<float>(workspace, vt), (float*)out, (int64_t)Hq * d, false, s));
  }
  return ok();
}

}  // extern "C"

extern "C" {

int gen_timing_begin(int family, int capacity) {
  if (family < 0 || family > 5 || capacity < 1) return fail(GEN_EINVAL, "bad family %d or capacity %d", family, capacity);
  if (g_timing.ev) return fail(GEN_EINVAL, "timing already active");
  g_timing.ev = new hipEvent_t[2 * capacity];
  for (int i = 0; i < 2 * capacity; ++i) {
    hipError_t e = hipEventCreate(&g_timing.ev[i]);
    if (e != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(g_timing.ev[j]);
      delete[] g_timing.ev;
      g_timing.ev = nullptr;
      return fail(GEN_EHIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  g_timing.family = family;
  g_timing.cap = capacity;
  g_timing.used = 0;
  return ok();
}

int gen_timing_end(double* total_ms, int* n_launches) {
  if (!g_timing.ev) return fail(GEN_EINVAL, "timing not active");
  double tot = 0.0;
  hipError_t err = hipSuccess;
  if (g_timing.used > 0) err = hipEventSynchronize(g_timing.ev[2 * g_timing.used - 1]);
  for (int i = 0; i < g_timing.used && err == hipSuccess; ++i) {
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]);
    tot += ms;
  }
  const int n = g_timing.used;
  for (int i = 0; i < 2 * g_timing.cap; ++i) (void)hipEventDestroy(g_timing.ev[i]);
  delete[] g_timing.ev;
  g_timing = Timing();
  if (err != hipSuccess) return fail(GEN_EHIP, "event timing: %s", hipGetErrorString(err));
  if (total_ms) *total_ms = tot;
  if (n_launches) *n_launches = n;
  return ok();
}

}  // extern "C"
