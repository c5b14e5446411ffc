// A pre-norm decoder layer on the packed layout, forward and backward:
//
//   h1 = RMSNorm(x; n1)            q, k, v = h1 Wq, h1 Wk, h1 Wv
//   q, k = RoPE(q, k) at the packed rows' logical positions
//   o = shared-prompt attention(q, k, v)          x1 = x + o Wo
//   h2 = RMSNorm(x1; n2)           u, g = h2 W1, h2 W3
//   m = silu(u) * g                y = x1 + m W2
//
// "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
// the packed P+NR layout reduces the tokens of the whole model, not only
// of attention; every token-wise step here runs once per packed row, and
// the packed layer equals the replicated one on every sequence.  The
// projections are the bf16 MFMA GEMM of gemm.hip (fp32 accumulation), the
// attention the DualKV kernels of this library; activations are kept in
// bf16 between steps.  Weight gradients are sums over the packed rows in
// the GEMM's fixed order, so the backward is bitwise reproducible.
#include <math.h>

#include <algorithm>

#include "common.h"

namespace dualkv {

hipError_t launch_gemm(bool ta, bool tb, int M, int N, int K, const void* A, int64_t lda, const void* B,
                       int64_t ldb, void* C, int64_t ldc, const void* R, int64_t ldr, hipStream_t stream);
int gemm_shape_ok(bool ta, bool tb, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc);
hipError_t launch_gemm_parts(bool ta, bool tb, int M, int N, int K, const GemmParts& P, hipStream_t stream);
hipError_t launch_rmsnorm_fwd(int T, int H, float eps, const void* x, const void* w, void* y, float* rstd,
                              hipStream_t s);
hipError_t launch_rmsnorm_bwd(int T, int H, const void* x, const void* w, const float* rstd, const void* dy,
                              const void* dres, void* dx, void* dw, float* part, hipStream_t s);
int norm_wgrad_chunks(int T);
hipError_t launch_rope(int T, int H, int D, const Groups& G, float base, int inverse, void* x, hipStream_t s);
hipError_t launch_swiglu_fwd(int64_t n, const void* u, const void* g, void* m, hipStream_t s);
hipError_t launch_swiglu_bwd(int64_t n, const void* u, const void* g, const void* dm, void* du, void* dg,
                             hipStream_t s);

namespace {

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// op(A) Ba -> Ca and op(A) Bb -> Cb (same A, B row-major [K][N*], C [M][N*]):
// one launch with two column parts when both widths are whole 256-column
// tiles, else two launches.
hipError_t gemm_cols2(bool ta, int M, int Na, int Nb, int K, const void* A, int64_t lda, const void* Ba,
                      const void* Bb, void* Ca, void* Cb, hipStream_t s) {
  if (Na % 256 != 0 || Nb % 256 != 0) {
    hipError_t e = launch_gemm(ta, false, M, Na, K, A, lda, Ba, Na, Ca, Na, nullptr, 0, s);
    if (e != hipSuccess) return e;
    return launch_gemm(ta, false, M, Nb, K, A, lda, Bb, Nb, Cb, Nb, nullptr, 0, s);
  }
  GemmParts P{};
  P.n = 2;
  P.ksplit = 0;
  P.lo[0] = 0;
  P.lo[1] = Na;
  P.lo[2] = Na + Nb;
  P.A[0] = P.A[1] = static_cast<const uint16_t*>(A);
  P.lda[0] = P.lda[1] = lda;
  P.B[0] = static_cast<const uint16_t*>(Ba);
  P.B[1] = static_cast<const uint16_t*>(Bb);
  P.ldb[0] = Na;
  P.ldb[1] = Nb;
  P.C[0] = static_cast<uint16_t*>(Ca);
  P.C[1] = static_cast<uint16_t*>(Cb);
  P.ldc[0] = Na;
  P.ldc[1] = Nb;
  return launch_gemm_parts(ta, false, M, Na + Nb, K, P, s);
}

// C [M][N] = sum_j A_j B_j^T with A_j [M][K_j] and B_j [N][K_j] (the input
// gradient of several projections of one input): one launch over k parts
// when every K_j is whole 64-k tiles, else one launch per part, each adding
// the previous result as its residual.
hipError_t gemm_ksum(int M, int N, int np, const int* Ks, const void* const* As, const void* const* Bs, void* C,
                     hipStream_t s) {
  bool whole = np <= kMaxGemmParts;
  for (int j = 0; j < np; ++j) whole = whole && Ks[j] % 64 == 0;
  if (!whole) {
    for (int j = 0; j < np; ++j) {
      hipError_t e = launch_gemm(false, true, M, N, Ks[j], As[j], Ks[j], Bs[j], Ks[j], C, N, j ? C : nullptr,
                                 j ? N : 0, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  GemmParts P{};
  P.n = np;
  P.ksplit = 1;
  P.lo[0] = 0;
  for (int j = 0; j < np; ++j) {
    P.lo[j + 1] = P.lo[j] + Ks[j];
    P.A[j] = static_cast<const uint16_t*>(As[j]);
    P.lda[j] = Ks[j];
    P.B[j] = static_cast<const uint16_t*>(Bs[j]);
    P.ldb[j] = Ks[j];
  }
  P.C[0] = static_cast<uint16_t*>(C);
  P.ldc[0] = N;
  return launch_gemm_parts(false, true, M, N, P.lo[np], P, s);
}

struct LayerShape {
  int T, Hm, Hq, Hkv, D, F;
  int QD() const { return Hq * D; }
  int KD() const { return Hkv * D; }
};

// Sub-buffers of a caller buffer, each 256-byte aligned.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += al256(bytes);
    return p;
  }
};

// Activations kept from the forward for the backward.
struct Saved {
  uint16_t *h1, *q, *k, *v, *o, *x1, *h2, *u, *g, *m;
  float *lse, *rstd1, *rstd2;
};
Saved carve_saved(void* buf, const LayerShape& s, size_t* bytes) {
  Carver c(buf);
  const size_t T = s.T, b2 = 2;
  Saved v;
  v.h1 = c.take<uint16_t>(T * s.Hm * b2);
  v.q = c.take<uint16_t>(T * s.QD() * b2);
  v.k = c.take<uint16_t>(T * s.KD() * b2);
  v.v = c.take<uint16_t>(T * s.KD() * b2);
  v.o = c.take<uint16_t>(T * s.QD() * b2);
  v.x1 = c.take<uint16_t>(T * s.Hm * b2);
  v.h2 = c.take<uint16_t>(T * s.Hm * b2);
  v.u = c.take<uint16_t>(T * s.F * b2);
  v.g = c.take<uint16_t>(T * s.F * b2);
  v.m = c.take<uint16_t>(T * s.F * b2);
  v.lse = c.take<float>(T * s.Hq * 4);
  v.rstd1 = c.take<float>(T * 4);
  v.rstd2 = c.take<float>(T * 4);
  *bytes = c.off;
  return v;
}

// Backward temporaries.
struct Scratch {
  uint16_t *dm, *du, *dg, *dh2, *dx1, *dO, *dq, *dk, *dv, *dh1;
  float* part;
  void* att;
  size_t att_bytes;
};
Scratch carve_scratch(void* buf, const LayerShape& s, size_t att_bytes, size_t* bytes) {
  Carver c(buf);
  const size_t T = s.T, b2 = 2;
  Scratch w;
  w.dm = c.take<uint16_t>(T * s.F * b2);
  w.du = c.take<uint16_t>(T * s.F * b2);
  w.dg = c.take<uint16_t>(T * s.F * b2);
  w.dh2 = c.take<uint16_t>(T * s.Hm * b2);
  w.dx1 = c.take<uint16_t>(T * s.Hm * b2);
  w.dO = c.take<uint16_t>(T * s.QD() * b2);
  w.dq = c.take<uint16_t>(T * s.QD() * b2);
  w.dk = c.take<uint16_t>(T * s.KD() * b2);
  w.dv = c.take<uint16_t>(T * s.KD() * b2);
  w.dh1 = c.take<uint16_t>(T * s.Hm * b2);
  w.part = c.take<float>((size_t)std::max(1, norm_wgrad_chunks(s.T)) * s.Hm * 4);
  w.att = c.take<char>(att_bytes);
  w.att_bytes = att_bytes;
  *bytes = c.off;
  return w;
}

int status_of(hipError_t e) { return e == hipSuccess ? DUALKV_OK : DUALKV_ERR_HIP; }

// Validate the layer description; fill the attention parameters and the shape.
int layer_setup(const dualkv_layer_params* lp, const dualkv_group* groups, int32_t n_groups,
                dualkv_params* ap, LayerShape* s) {
  if (lp == nullptr || groups == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  if (lp->hidden < 1 || lp->ffn < 1 || lp->n_q_heads < 1 || lp->n_kv_heads < 1 || lp->head_dim < 1)
    return DUALKV_ERR_INVALID_ARGUMENT;
  if (!(lp->rope_base > 1.f) || !isfinite(lp->rope_base) || !(lp->norm_eps > 0.f) || !isfinite(lp->norm_eps))
    return DUALKV_ERR_INVALID_ARGUMENT;
  if (lp->head_dim % 2 != 0 || lp->n_q_heads % lp->n_kv_heads != 0) return DUALKV_ERR_INVALID_ARGUMENT;
  // GEMM tiles: every feature width a whole number of 128-wide blocks
  if (lp->hidden % 128 || lp->ffn % 128 || (lp->n_q_heads * lp->head_dim) % 128 ||
      (lp->n_kv_heads * lp->head_dim) % 128)
    return DUALKV_ERR_UNSUPPORTED;
  if (lp->ffn > (1 << 24) || lp->hidden > (1 << 20)) return DUALKV_ERR_UNSUPPORTED;
  *ap = dualkv_params{};
  ap->n_q_heads = lp->n_q_heads;
  ap->n_kv_heads = lp->n_kv_heads;
  ap->head_dim = lp->head_dim;
  ap->window = lp->window;
  ap->softmax_scale = 0.f;
  ap->dtype = DUALKV_BF16;
  ap->impl = DUALKV_IMPL_AUTO;
  ap->resp_valid_len = lp->resp_valid_len;
  int64_t T = 0;
  const int st = check_groups(groups, n_groups, &T);
  if (st != DUALKV_OK) return st;
  // the attention's own checks (heads, head dim) on a non-empty batch
  if (T > 0 && dualkv_bwd_groups_workspace_bytes(ap, groups, n_groups) == 0) return DUALKV_ERR_INVALID_ARGUMENT;
  if (T * std::max(lp->ffn, lp->hidden) >= ((int64_t)1 << 40)) return DUALKV_ERR_UNSUPPORTED;
  s->T = (int)T;
  s->Hm = lp->hidden;
  s->Hq = lp->n_q_heads;
  s->Hkv = lp->n_kv_heads;
  s->D = lp->head_dim;
  s->F = lp->ffn;
  return DUALKV_OK;
}

Groups groups_of(const dualkv_group* groups, int32_t n) {
  Groups G{};
  G.n = n;
  int row = 0;
  for (int i = 0; i < n; ++i) {
    G.N[i] = groups[i].n_resp;
    G.P[i] = groups[i].prompt_len;
    G.R[i] = groups[i].resp_len;
    G.row0[i] = row;
    row += groups[i].prompt_len + groups[i].n_resp * groups[i].resp_len;
  }
  return G;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace dualkv

using namespace dualkv;

extern "C" {

int dualkv_gemm_bf16(int32_t trans_a, int32_t trans_b, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                     const void* B, int64_t ldb, void* C, int64_t ldc, const void* R, int64_t ldr, void* stream) {
  if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return DUALKV_ERR_INVALID_ARGUMENT;
  if (M < 0 || N < 0 || K < 0 || lda < 0 || ldb < 0 || ldc < 0) return DUALKV_ERR_INVALID_ARGUMENT;
  if (R != nullptr && ldr < N) return DUALKV_ERR_INVALID_ARGUMENT;
  if (!gemm_shape_ok(trans_a, trans_b, M, N, K, lda, ldb, ldc)) return DUALKV_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return DUALKV_OK;
  if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return DUALKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(A) || !aligned16(B)) return DUALKV_ERR_INVALID_ARGUMENT;
  return status_of(launch_gemm(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, R, ldr,
                               static_cast<hipStream_t>(stream)));
}

int dualkv_rmsnorm_fwd(int32_t T, int32_t H, float eps, const void* x, const void* w, void* y, float* rstd,
                       void* stream) {
  if (T < 0 || H < 8 || H % 8 != 0 || !(eps > 0.f)) return DUALKV_ERR_INVALID_ARGUMENT;
  if (T == 0) return DUALKV_OK;
  if (!x || !w || !y || !rstd || !aligned16(x) || !aligned16(w) || !aligned16(y)) return DUALKV_ERR_INVALID_ARGUMENT;
  return status_of(launch_rmsnorm_fwd(T, H, eps, x, w, y, rstd, static_cast<hipStream_t>(stream)));
}

size_t dualkv_rmsnorm_bwd_workspace_bytes(int32_t T, int32_t H) {
  if (T < 0 || H < 8) return 0;
  return al256((size_t)std::max(1, norm_wgrad_chunks(T)) * H * 4);
}

int dualkv_rmsnorm_bwd(int32_t T, int32_t H, const void* x, const void* w, const float* rstd, const void* dy,
                       const void* dres, void* dx, void* dw, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (T < 0 || H < 8 || H % 8 != 0) return DUALKV_ERR_INVALID_ARGUMENT;
  if (T == 0) return DUALKV_OK;
  if (workspace_bytes < dualkv_rmsnorm_bwd_workspace_bytes(T, H)) return DUALKV_ERR_WORKSPACE_TOO_SMALL;
  if (!x || !w || !rstd || !dy || !dx || !dw || !workspace) return DUALKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w) || !aligned16(dy) || !aligned16(dx) || (dres && !aligned16(dres)))
    return DUALKV_ERR_INVALID_ARGUMENT;
  return status_of(launch_rmsnorm_bwd(T, H, x, w, rstd, dy, dres, dx, dw, static_cast<float*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

int dualkv_rope(const dualkv_group* groups, int32_t n_groups, int32_t n_heads, int32_t head_dim, float base,
                int32_t inverse, void* x, void* stream) {
  if (n_heads < 1 || head_dim < 2 || head_dim % 2 != 0 || !(base > 1.f) || !isfinite(base))
    return DUALKV_ERR_INVALID_ARGUMENT;
  if (inverse != 0 && inverse != 1) return DUALKV_ERR_INVALID_ARGUMENT;
  int64_t rows = 0;
  const int st = check_groups(groups, n_groups, &rows);
  if (st != DUALKV_OK) return st;
  if (rows * n_heads * head_dim >= ((int64_t)1 << 40)) return DUALKV_ERR_UNSUPPORTED;
  const Groups G = groups_of(groups, n_groups);
  const int T = (int)rows;
  if (T == 0) return DUALKV_OK;
  if (x == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  return status_of(launch_rope(T, n_heads, head_dim, G, base, inverse, x, static_cast<hipStream_t>(stream)));
}

int dualkv_swiglu_fwd(int64_t n, const void* u, const void* g, void* m, void* stream) {
  if (n < 0 || n % 8 != 0) return DUALKV_ERR_INVALID_ARGUMENT;
  if (n == 0) return DUALKV_OK;
  if (!aligned16(u) || !aligned16(g) || !aligned16(m) || !u || !g || !m) return DUALKV_ERR_INVALID_ARGUMENT;
  return status_of(launch_swiglu_fwd(n, u, g, m, static_cast<hipStream_t>(stream)));
}

int dualkv_swiglu_bwd(int64_t n, const void* u, const void* g, const void* dm, void* du, void* dg, void* stream) {
  if (n < 0 || n % 8 != 0) return DUALKV_ERR_INVALID_ARGUMENT;
  if (n == 0) return DUALKV_OK;
  if (!u || !g || !dm || !du || !dg) return DUALKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(u) || !aligned16(g) || !aligned16(dm) || !aligned16(du) || !aligned16(dg))
    return DUALKV_ERR_INVALID_ARGUMENT;
  return status_of(launch_swiglu_bwd(n, u, g, dm, du, dg, static_cast<hipStream_t>(stream)));
}

size_t dualkv_layer_saved_bytes(const dualkv_layer_params* lp, const dualkv_group* groups, int32_t n_groups) {
  dualkv_params ap;
  LayerShape s;
  if (layer_setup(lp, groups, n_groups, &ap, &s) != DUALKV_OK) return 0;
  size_t b;
  carve_saved(nullptr, s, &b);
  return b;
}

size_t dualkv_layer_workspace_bytes(const dualkv_layer_params* lp, const dualkv_group* groups, int32_t n_groups) {
  dualkv_params ap;
  LayerShape s;
  if (layer_setup(lp, groups, n_groups, &ap, &s) != DUALKV_OK) return 0;
  size_t b;
  carve_scratch(nullptr, s, dualkv_bwd_groups_workspace_bytes(&ap, groups, n_groups), &b);
  return b;
}

int dualkv_layer_fwd(const dualkv_layer_params* lp, const dualkv_group* groups, int32_t n_groups,
                     const dualkv_layer_weights* wt, const void* x, void* y, void* saved, size_t saved_bytes,
                     void* stream) {
  dualkv_params ap;
  LayerShape s;
  int st = layer_setup(lp, groups, n_groups, &ap, &s);
  if (st != DUALKV_OK) return st;
  if (wt == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  size_t need;
  Saved v = carve_saved(saved, s, &need);
  if (saved_bytes < need) return DUALKV_ERR_WORKSPACE_TOO_SMALL;
  if (s.T == 0) return DUALKV_OK;
  const void* ptrs[] = {x, y, saved, wt->norm1, wt->wq, wt->wk, wt->wv, wt->wo, wt->norm2, wt->w1, wt->w3, wt->w2};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return DUALKV_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(saved) % 256 != 0) return DUALKV_ERR_INVALID_ARGUMENT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const Groups G = groups_of(groups, n_groups);
  const int T = s.T, Hm = s.Hm, QD = s.QD(), KD = s.KD(), F = s.F;
  hipError_t e;
#define DKV_TRY(call) \
  if ((e = (call)) != hipSuccess) return status_of(e)
  DKV_TRY(launch_rmsnorm_fwd(T, Hm, lp->norm_eps, x, wt->norm1, v.h1, v.rstd1, hs));
  DKV_TRY(launch_gemm(false, false, T, QD, Hm, v.h1, Hm, wt->wq, QD, v.q, QD, nullptr, 0, hs));
  DKV_TRY(gemm_cols2(false, T, KD, KD, Hm, v.h1, Hm, wt->wk, wt->wv, v.k, v.v, hs));
  DKV_TRY(launch_rope(T, s.Hq, s.D, G, lp->rope_base, 0, v.q, hs));
  DKV_TRY(launch_rope(T, s.Hkv, s.D, G, lp->rope_base, 0, v.k, hs));
  st = dualkv_fwd_groups(&ap, groups, n_groups, v.q, v.k, v.v, v.o, v.lse, stream);
  if (st != DUALKV_OK) return st;
  DKV_TRY(launch_gemm(false, false, T, Hm, QD, v.o, QD, wt->wo, Hm, v.x1, Hm, x, Hm, hs));
  DKV_TRY(launch_rmsnorm_fwd(T, Hm, lp->norm_eps, v.x1, wt->norm2, v.h2, v.rstd2, hs));
  DKV_TRY(launch_gemm(false, false, T, F, Hm, v.h2, Hm, wt->w1, F, v.u, F, nullptr, 0, hs));
  DKV_TRY(launch_gemm(false, false, T, F, Hm, v.h2, Hm, wt->w3, F, v.g, F, nullptr, 0, hs));
  DKV_TRY(launch_swiglu_fwd((int64_t)T * F, v.u, v.g, v.m, hs));
  DKV_TRY(launch_gemm(false, false, T, Hm, F, v.m, F, wt->w2, Hm, y, Hm, v.x1, Hm, hs));
  return DUALKV_OK;
}

int dualkv_layer_bwd(const dualkv_layer_params* lp, const dualkv_group* groups, int32_t n_groups,
                     const dualkv_layer_weights* wt, const void* x, const void* saved, size_t saved_bytes,
                     const void* dy, void* dx, const dualkv_layer_grads* gr, void* workspace,
                     size_t workspace_bytes, void* stream) {
  dualkv_params ap;
  LayerShape s;
  int st = layer_setup(lp, groups, n_groups, &ap, &s);
  if (st != DUALKV_OK) return st;
  if (wt == nullptr || gr == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  size_t need_saved, need_ws;
  Saved v = carve_saved(const_cast<void*>(saved), s, &need_saved);
  const size_t att_bytes = dualkv_bwd_groups_workspace_bytes(&ap, groups, n_groups);
  Scratch w = carve_scratch(workspace, s, att_bytes, &need_ws);
  if (saved_bytes < need_saved || workspace_bytes < need_ws) return DUALKV_ERR_WORKSPACE_TOO_SMALL;
  if (s.T == 0) return DUALKV_OK;
  const void* ptrs[] = {x, saved, dy, dx, workspace, wt->norm1, wt->wq, wt->wk, wt->wv, wt->wo, wt->norm2, wt->w1,
                        wt->w3, wt->w2, gr->norm1, gr->wq, gr->wk, gr->wv, gr->wo, gr->norm2, gr->w1, gr->w3,
                        gr->w2};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return DUALKV_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(saved) % 256 != 0 || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return DUALKV_ERR_INVALID_ARGUMENT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const Groups G = groups_of(groups, n_groups);
  const int T = s.T, Hm = s.Hm, QD = s.QD(), KD = s.KD(), F = s.F;
  hipError_t e;
  // MLP: y = x1 + m W2, m = silu(u) * g, u = h2 W1, g = h2 W3
  DKV_TRY(launch_gemm(false, true, T, F, Hm, dy, Hm, wt->w2, Hm, w.dm, F, nullptr, 0, hs));
  DKV_TRY(launch_gemm(true, false, F, Hm, T, v.m, F, dy, Hm, gr->w2, Hm, nullptr, 0, hs));
  DKV_TRY(launch_swiglu_bwd((int64_t)T * F, v.u, v.g, w.dm, w.du, w.dg, hs));
  {
    const int Ks[] = {F, F};
    const void* As[] = {w.du, w.dg};
    const void* Bs[] = {wt->w1, wt->w3};
    DKV_TRY(gemm_ksum(T, Hm, 2, Ks, As, Bs, w.dh2, hs));
  }
  DKV_TRY(launch_gemm(true, false, Hm, F, T, v.h2, Hm, w.du, F, gr->w1, F, nullptr, 0, hs));
  DKV_TRY(launch_gemm(true, false, Hm, F, T, v.h2, Hm, w.dg, F, gr->w3, F, nullptr, 0, hs));
  // h2 = RMSNorm(x1); the residual passes dy on to x1
  DKV_TRY(launch_rmsnorm_bwd(T, Hm, v.x1, wt->norm2, v.rstd2, w.dh2, dy, w.dx1, gr->norm2, w.part, hs));
  // attention block: x1 = x + o Wo
  DKV_TRY(launch_gemm(false, true, T, QD, Hm, w.dx1, Hm, wt->wo, Hm, w.dO, QD, nullptr, 0, hs));
  DKV_TRY(launch_gemm(true, false, QD, Hm, T, v.o, QD, w.dx1, Hm, gr->wo, Hm, nullptr, 0, hs));
  st = dualkv_bwd_groups(&ap, groups, n_groups, v.q, v.k, v.v, v.o, v.lse, w.dO, w.dq, w.dk, w.dv, w.att,
                         w.att_bytes, stream);
  if (st != DUALKV_OK) return st;
  DKV_TRY(launch_rope(T, s.Hq, s.D, G, lp->rope_base, 1, w.dq, hs));
  DKV_TRY(launch_rope(T, s.Hkv, s.D, G, lp->rope_base, 1, w.dk, hs));
  {
    const int Ks[] = {QD, KD, KD};
    const void* As[] = {w.dq, w.dk, w.dv};
    const void* Bs[] = {wt->wq, wt->wk, wt->wv};
    DKV_TRY(gemm_ksum(T, Hm, 3, Ks, As, Bs, w.dh1, hs));
  }
  DKV_TRY(launch_gemm(true, false, Hm, QD, T, v.h1, Hm, w.dq, QD, gr->wq, QD, nullptr, 0, hs));
  DKV_TRY(gemm_cols2(true, Hm, KD, KD, T, v.h1, Hm, w.dk, w.dv, gr->wk, gr->wv, hs));
  DKV_TRY(launch_rmsnorm_bwd(T, Hm, x, wt->norm1, v.rstd1, w.dh1, w.dx1, dx, gr->norm1, w.part, hs));
#undef DKV_TRY
  return DUALKV_OK;
}

}  // extern "C"
