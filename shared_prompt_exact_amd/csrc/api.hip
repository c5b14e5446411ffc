// C ABI of the shared-prompt attention library: argument validation,
// workspace sizing and dispatch to the MFMA or scalar kernels.  See
// include/dualkv.h for the contract of every entry point.
#include <math.h>

#include "common.h"

using namespace dualkv;

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 30;

// Validate `p` and fill `pr`.  Touches no HIP state.
int validate(const dualkv_params* p, Problem* pr) {
  if (p == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->n_resp < 1 || p->prompt_len < 0 || p->resp_len < 0) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->n_q_heads < 1 || p->n_kv_heads < 1 || p->n_q_heads % p->n_kv_heads != 0)
    return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->dtype != DUALKV_F32 && p->dtype != DUALKV_BF16) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->impl < DUALKV_IMPL_AUTO || p->impl > DUALKV_IMPL_MFMA) return DUALKV_ERR_INVALID_ARGUMENT;
  if (!(p->softmax_scale >= 0.f) || !isfinite(p->softmax_scale)) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->head_dim < 1) return DUALKV_ERR_INVALID_ARGUMENT;
  if (p->head_dim > 512) return DUALKV_ERR_UNSUPPORTED;
  const int64_t T = (int64_t)p->prompt_len + (int64_t)p->n_resp * p->resp_len;
  if (T > kMaxRows) return DUALKV_ERR_UNSUPPORTED;
  if (T * p->n_q_heads * p->head_dim > ((int64_t)1 << 40)) return DUALKV_ERR_UNSUPPORTED;
  pr->N = p->n_resp;
  pr->P = p->prompt_len;
  pr->R = p->resp_len;
  pr->Hq = p->n_q_heads;
  pr->Hkv = p->n_kv_heads;
  pr->D = p->head_dim;
  pr->g = p->n_q_heads / p->n_kv_heads;
  pr->W = p->window > 0 ? p->window : 0;
  pr->T = (int)T;
  pr->scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf((float)p->head_dim);
  pr->valid_len = p->resp_valid_len;
  return DUALKV_OK;
}

// Which kernels serve these parameters (1 = MFMA, 0 = scalar, -1 = none).
int choose_fwd(const dualkv_params* p, const Problem& pr) {
  const bool mfma = p->dtype == DUALKV_BF16 && fwd_mfma_supported(pr);
  if (p->impl == DUALKV_IMPL_MFMA) return mfma ? 1 : -1;
  if (p->impl == DUALKV_IMPL_SCALAR) return 0;
  return mfma ? 1 : 0;
}
int choose_bwd(const dualkv_params* p, const Problem& pr) {
  const bool mfma = p->dtype == DUALKV_BF16 && bwd_mfma_supported(pr);
  if (p->impl == DUALKV_IMPL_MFMA) return mfma ? 1 : -1;
  if (p->impl == DUALKV_IMPL_SCALAR) return 0;
  return mfma ? 1 : 0;
}

size_t scalar_workspace(const Problem& pr) {
  size_t b = (size_t)pr.Hq * (size_t)pr.T * sizeof(float);
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
    default: return "unknown status";
  }
}

int dualkv_repack(const void* src, void* dst, int64_t row_bytes, int32_t n_resp,
                  int32_t prompt_len, int32_t resp_len, int32_t direction, void* stream) {
  if (row_bytes < 1 || n_resp < 1 || prompt_len < 0 || resp_len < 0) return DUALKV_ERR_INVALID_ARGUMENT;
  if (direction != DUALKV_GATHER && direction != DUALKV_SCATTER) return DUALKV_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)n_resp * ((int64_t)prompt_len + resp_len);
  if (rows > kMaxRows * 64) return DUALKV_ERR_UNSUPPORTED;
  if (rows == 0) return DUALKV_OK;
  if (src == nullptr || dst == nullptr) return DUALKV_ERR_INVALID_ARGUMENT;
  return status_of(launch_repack(src, dst, row_bytes, n_resp, prompt_len, resp_len, direction,
                                 static_cast<hipStream_t>(stream)));
}

int dualkv_fwd(const dualkv_params* p, const void* q, const void* k, const void* v, void* o,
               float* lse, void* stream) {
  Problem pr;
  int st = validate(p, &pr);
  if (st != DUALKV_OK) return st;
  const int which = choose_fwd(p, pr);
  if (which < 0) return DUALKV_ERR_UNSUPPORTED;
  if (pr.T == 0) return DUALKV_OK;
  if (!q || !k || !v || !o || !lse) return DUALKV_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (which == 1) return status_of(launch_fwd_mfma(pr, q, k, v, o, lse, s));
  return status_of(launch_fwd_scalar(pr, p->dtype, q, k, v, o, lse, s));
}

size_t dualkv_bwd_workspace_bytes(const dualkv_params* p) {
  Problem pr;
  if (validate(p, &pr) != DUALKV_OK) return 0;
  const int which = choose_bwd(p, pr);
  if (which < 0) return 0;
  if (which == 1) return bwd_mfma_workspace_bytes(pr);
  return scalar_workspace(pr);
}

int dualkv_bwd(const dualkv_params* p, const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, void* stream) {
  Problem pr;
  int st = validate(p, &pr);
  if (st != DUALKV_OK) return st;
  const int which = choose_bwd(p, pr);
  if (which < 0) return DUALKV_ERR_UNSUPPORTED;
  if (pr.T == 0) return DUALKV_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return DUALKV_ERR_INVALID_ARGUMENT;
  const size_t need = which == 1 ? bwd_mfma_workspace_bytes(pr) : scalar_workspace(pr);
  if (workspace_bytes < need) return DUALKV_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return DUALKV_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (which == 1)
    return status_of(launch_bwd_mfma(pr, q, k, v, o, lse, dout, dq, dk, dv, workspace, s));
  return status_of(launch_bwd_scalar(pr, p->dtype, q, k, v, o, lse, dout, dq, dk, dv,
                                     static_cast<float*>(workspace), s));
}

}  // extern "C"
