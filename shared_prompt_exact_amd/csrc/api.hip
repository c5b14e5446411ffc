// C ABI of the shared-prompt attention library: argument validation,
// workspace sizing and dispatch to the MFMA or scalar kernels.  See
// include/dualkv.h for the contract of every entry point.
#include <math.h>

#include <mutex>

#include "common.h"

using namespace dualkv;

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 30;

// Validate the launch-wide fields of `p` (everything but N, P, R) and fill
// them into `pr`.  Touches no HIP state.
int validate_params(const dualkv_params* p, Problem* pr) {
  if (p == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->n_q_heads < 1 || p->n_kv_heads < 1 || p->n_q_heads % p->n_kv_heads != 0)
    return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->dtype != DUALKV_F32 && p->dtype != DUALKV_BF16) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->impl < DUALKV_IMPL_AUTO || p->impl > DUALKV_IMPL_MFMA) return DUALKV_ERR_INVALID_ARGUMENT;
  if (!(p->softmax_scale >= 0.f) || !isfinite(p->softmax_scale)) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->head_dim < 1) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->head_dim > 512) return DUALKV_ERR_UNSUPPORTED;
  pr->Hq = p->n_q_heads;
  pr->Hkv = p->n_kv_heads;
  pr->D = p->head_dim;
  pr->g = p->n_q_heads / p->n_kv_heads;
  pr->W = p->window > 0 ? p->window : 0;
  pr->scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf((float)p->head_dim);
  pr->valid_len = p->resp_valid_len;
  return DUALKV_OK;
}

}  // namespace

int dualkv::check_groups(const dualkv_group* groups, int32_t n, int64_t* rows) {
  if (groups == nullptr || n < 1) return DUALKV_ERR_INVALID_ARGUMENT;
  if (n > kMaxGroups) return DUALKV_ERR_UNSUPPORTED;
  int64_t r = 0;
  for (int i = 0; i < n; ++i) {
    const dualkv_group& g = groups[i];
    if (g.n_resp < 1 || g.prompt_len < 0 || g.resp_len < 0) return DUALKV_ERR_INVALID_ARGUMENT;
    const int64_t T = (int64_t)g.prompt_len + (int64_t)g.n_resp * g.resp_len;
    if (T > kMaxRows || r + T > kMaxRows) return DUALKV_ERR_UNSUPPORTED;
    r += T;
  }
  *rows = r;
  return DUALKV_OK;
}

namespace {

// Validate the groups and fill `G` and the row counts of `pr` (N, P, R, T
// of group 0; Tld of the whole launch).
int validate_groups(const dualkv_group* groups, int32_t n, Problem* pr, Groups* G) {
  int64_t total;
  const int st = check_groups(groups, n, &total);
  if (st != DUALKV_OK) return st;
  int64_t rows = 0, vl = 0;
  G->n = n;
  for (int i = 0; i < n; ++i) {
    const dualkv_group& g = groups[i];
    const int64_t T = (int64_t)g.prompt_len + (int64_t)g.n_resp * g.resp_len;
    G->N[i] = g.n_resp;
    G->P[i] = g.prompt_len;
    G->R[i] = g.resp_len;
    G->row0[i] = (int)rows;
    G->vl0[i] = (int)vl;
    rows += T;
    vl += g.n_resp;
  }
  if (rows * pr->Hq * pr->D > ((int64_t)1 << 40)) return DUALKV_ERR_UNSUPPORTED;
  if (vl > INT32_MAX) return DUALKV_ERR_UNSUPPORTED;
  pr->N = G->N[0];
  pr->P = G->P[0];
  pr->R = G->R[0];
  pr->T = G->P[0] + G->N[0] * G->R[0];
  pr->Tld = (int)rows;
  return DUALKV_OK;
}

int validate(const dualkv_params* p, const dualkv_group* groups, int32_t n, Problem* pr, Groups* G) {
  const int st = validate_params(p, pr);
  return st != DUALKV_OK ? st : validate_groups(groups, n, pr, G);
}

// The one group that the single-group entry points describe in `p`.
dualkv_group group_of_params(const dualkv_params* p) {
  dualkv_group g = {0, 0, 0};
  if (p) g = {p->n_resp, p->prompt_len, p->resp_len};
  return g;
}

// Which kernels serve these parameters (1 = MFMA, 0 = scalar, -1 = none).
int choose_fwd(const dualkv_params* p, const Problem& pr, const Groups& G) {
  const bool mfma = p->dtype == DUALKV_BF16 && fwd_mfma_supported(pr, G);
  if (p->impl == DUALKV_IMPL_MFMA) return mfma ? 1 : -1;
  if (p->impl == DUALKV_IMPL_SCALAR) return 0;
  return mfma ? 1 : 0;
}
int choose_bwd(const dualkv_params* p, const Problem& pr, const Groups& G) {
  const bool mfma = p->dtype == DUALKV_BF16 && bwd_mfma_supported(pr, G);
  if (p->impl == DUALKV_IMPL_MFMA) return mfma ? 1 : -1;
  if (p->impl == DUALKV_IMPL_SCALAR) return 0;
  return mfma ? 1 : 0;
}

size_t scalar_workspace(const Problem& pr) {
  size_t b = (size_t)pr.Hq * (size_t)pr.Tld * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

int status_of(hipError_t e) { return e == hipSuccess ? DUALKV_OK : DUALKV_ERR_HIP; }

}  // namespace

extern "C" {

const char* dualkv_strerror(int status) {
  switch (status) {
    case DUALKV_OK: return "success";
    case DUALKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DUALKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case DUALKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DUALKV_ERR_HIP: return "HIP runtime error";
    case DUALKV_ERR_SCRATCH_LIMIT:
      return "problem needs more backward workspace than the static scratch buffer of dualkv_bwd_noalloc holds";
    default: return "unknown status";
  }
}

int dualkv_repack_groups(const void* src, void* dst, int64_t row_bytes, const dualkv_group* groups,
                         int32_t n_groups, int32_t direction, void* stream) {
  if (row_bytes < 1 || groups == nullptr || n_groups < 1) return DUALKV_ERR_INVALID_ARGUMENT;
  if (n_groups > kMaxGroups) return DUALKV_ERR_UNSUPPORTED;
  if (direction != DUALKV_GATHER && direction != DUALKV_SCATTER) return DUALKV_ERR_INVALID_ARGUMENT;
  int64_t rows = 0;
  for (int i = 0; i < n_groups; ++i) {
    const dualkv_group& g = groups[i];
    if (g.n_resp < 1 || g.prompt_len < 0 || g.resp_len < 0) return DUALKV_ERR_INVALID_ARGUMENT;
    rows += (int64_t)g.n_resp * ((int64_t)g.prompt_len + g.resp_len);
    if (rows > kMaxRows * 64) return DUALKV_ERR_UNSUPPORTED;
  }
  if (rows == 0) return DUALKV_OK;
  if (src == nullptr || dst == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  // group after group: replicated rows rep0, packed rows pk0
  int64_t rep0 = 0, pk0 = 0;
  for (int i = 0; i < n_groups; ++i) {
    const dualkv_group& g = groups[i];
    const int64_t rep = (int64_t)g.n_resp * ((int64_t)g.prompt_len + g.resp_len);
    const int64_t pk = (int64_t)g.prompt_len + (int64_t)g.n_resp * g.resp_len;
    const int64_t s0 = direction == DUALKV_GATHER ? rep0 : pk0, d0 = direction == DUALKV_GATHER ? pk0 : rep0;
    if (rep > 0) {
      const hipError_t e = launch_repack(static_cast<const char*>(src) + s0 * row_bytes,
                                         static_cast<char*>(dst) + d0 * row_bytes, row_bytes, g.n_resp,
                                         g.prompt_len, g.resp_len, direction, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return status_of(e);
    }
    rep0 += rep;
    pk0 += pk;
  }
  return DUALKV_OK;
}

int dualkv_repack(const void* src, void* dst, int64_t row_bytes, int32_t n_resp, int32_t prompt_len,
                  int32_t resp_len, int32_t direction, void* stream) {
  const dualkv_group g = {n_resp, prompt_len, resp_len};
  return dualkv_repack_groups(src, dst, row_bytes, &g, 1, direction, stream);
}

int dualkv_fwd_groups(const dualkv_params* p, const dualkv_group* groups, int32_t n_groups, const void* q,
                      const void* k, const void* v, void* o, float* lse, void* stream) {
  Problem pr;
  Groups G;
  int st = validate(p, groups, n_groups, &pr, &G);
  if (st != DUALKV_OK) return st;
  const int which = choose_fwd(p, pr, G);
  if (which < 0) return DUALKV_ERR_UNSUPPORTED;
  if (pr.Tld == 0) return DUALKV_OK;
  if (!q || !k || !v || !o || !lse) return DUALKV_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (which == 1) return status_of(launch_fwd_mfma(pr, G, q, k, v, o, lse, s));
  return status_of(launch_fwd_scalar(pr, G, p->dtype, q, k, v, o, lse, s));
}

int dualkv_fwd(const dualkv_params* p, const void* q, const void* k, const void* v, void* o,
               float* lse, void* stream) {
  const dualkv_group g = group_of_params(p);
  return dualkv_fwd_groups(p, &g, 1, q, k, v, o, lse, stream);
}

size_t dualkv_bwd_groups_workspace_bytes(const dualkv_params* p, const dualkv_group* groups,
                                         int32_t n_groups) {
  Problem pr;
  Groups G;
  if (validate(p, groups, n_groups, &pr, &G) != DUALKV_OK) return 0;
  const int which = choose_bwd(p, pr, G);
  if (which < 0) return 0;
  if (which == 1) return bwd_mfma_workspace_bytes(pr, G);
  return scalar_workspace(pr);
}

size_t dualkv_bwd_workspace_bytes(const dualkv_params* p) {
  const dualkv_group g = group_of_params(p);
  return dualkv_bwd_groups_workspace_bytes(p, &g, 1);
}

int dualkv_bwd_groups(const dualkv_params* p, const dualkv_group* groups, int32_t n_groups, const void* q,
                      const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  Problem pr;
  Groups G;
  int st = validate(p, groups, n_groups, &pr, &G);
  if (st != DUALKV_OK) return st;
  const int which = choose_bwd(p, pr, G);
  if (which < 0) return DUALKV_ERR_UNSUPPORTED;
  if (pr.Tld == 0) return DUALKV_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return DUALKV_ERR_INVALID_ARGUMENT;
  const size_t need = which == 1 ? bwd_mfma_workspace_bytes(pr, G) : scalar_workspace(pr);
  if (workspace_bytes < need) return DUALKV_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return DUALKV_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (which == 1)
    return status_of(launch_bwd_mfma(pr, G, q, k, v, o, lse, dout, dq, dk, dv, workspace, s));
  return status_of(launch_bwd_scalar(pr, G, p->dtype, q, k, v, o, lse, dout, dq, dk, dv,
                                     static_cast<float*>(workspace), s));
}

int dualkv_bwd(const dualkv_params* p, const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, void* stream) {
  const dualkv_group g = group_of_params(p);
  return dualkv_bwd_groups(p, &g, 1, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- backward without a caller workspace ---------------------------------
//
// The workspace of dualkv_bwd_noalloc is one static device array per GPU
// (this file's code object is loaded once per device, each with its own
// copy at its own address).  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is passed to
// kernels.  Every call on a device shares the device's array and leaves its
// contents behind; the backward writes every workspace element it reads
// before reading it, so nothing has to start at zero.  Calls that overlap
// on one device (different streams or threads) race on the array.

namespace {

static __device__ __align__(256) unsigned char scratch[DUALKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DUALKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DUALKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return DUALKV_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DUALKV_OK;
}

}  // namespace

extern "C" int dualkv_bwd_noalloc(const dualkv_params* p, const void* q, const void* k, const void* v,
                                  const void* o, const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, void* stream) {
  const dualkv_group g = group_of_params(p);
  Problem pr;
  Groups G;
  int st = validate(p, &g, 1, &pr, &G);
  if (st != DUALKV_OK) return st;
  const int which = choose_bwd(p, pr, G);
  if (which < 0) return DUALKV_ERR_UNSUPPORTED;
  if (pr.Tld == 0) return DUALKV_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return DUALKV_ERR_INVALID_ARGUMENT;
  const size_t need = which == 1 ? bwd_mfma_workspace_bytes(pr, G) : scalar_workspace(pr);
  if (need > DUALKV_NOALLOC_SCRATCH_BYTES) return DUALKV_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != DUALKV_OK) return st;
  return dualkv_bwd(p, q, k, v, o, lse, dout, dq, dk, dv, ws, DUALKV_NOALLOC_SCRATCH_BYTES, stream);
}
