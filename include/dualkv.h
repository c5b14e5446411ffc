/*
 * dualkv.h -- C ABI of the shared-prompt (DualKV) attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is defined in "DualKV: Shared-Prompt Flash Attention for
 * Efficient RL Training with Large Rollouts and Long Contexts" (arXiv
 * 2605.15422), Abstract: N response sequences of R tokens share one prompt
 * of P tokens.  The N(P+R) tokens of such a micro-batch are repacked into
 * P+NR tokens; prompt queries attend causally within the prompt, and each
 * response query attends to the whole prompt plus its own response
 * (causally) under one softmax spanning both key regions.  The result is
 * exactly standard causal attention on the N replicated sequences.
 *
 * Layouts (all row-major, contiguous, no padding between rows):
 *   packed rows   t = 0 .. T-1, T = P + N*R:
 *                 rows 0..P-1 are the prompt; rows P+n*R .. P+n*R+R-1 are
 *                 response n (n = 0..N-1).
 *   replicated    N sequences of P+R rows: sequence n = [prompt; response n].
 *   Q, O, dO, dQ  [T, Hq, D]   (element type: dualkv_params.dtype)
 *   K, V, dK, dV  [T, Hkv, D]
 *   LSE           [Hq, T]      fp32, natural log of sum_j exp(scale*q.k_j)
 *
 * Positions: response token r has logical position P+r; causality and the
 * sliding window use logical positions.  Causal is inclusive (a token sees
 * itself).  A window W > 0 keeps keys with 0 <= pos_q - pos_k < W.
 * GQA: query head h reads KV head h / (Hq/Hkv).
 * Response rows r >= valid_len[n] are padding: masked as queries (O = 0,
 * LSE = -inf, dQ = 0) and as keys (dK = dV = 0 on those rows).
 *
 * Ownership: every pointer is caller-owned device memory (except `p`, a
 * host pointer).  The library never allocates or frees memory, keeps no
 * pointer after a call returns, and holds no mutable global state apart
 * from the opt-in launch profiler declared at the end of this header.
 * Streams: `stream` is a hipStream_t (NULL = default stream); all work is
 * enqueued on it and the call returns after enqueueing.
 * Errors: arguments are validated on the host before anything is
 * launched; on a non-zero return nothing was launched and no output was
 * written.  DUALKV_ERR_HIP reports a failure of the HIP runtime at launch.
 * Outputs must not alias inputs.
 */
#ifndef DUALKV_H
#define DUALKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DUALKV_OK = 0,
  DUALKV_ERR_INVALID_ARGUMENT = 1,
  DUALKV_ERR_UNSUPPORTED = 2,
  DUALKV_ERR_WORKSPACE_TOO_SMALL = 3,
  DUALKV_ERR_HIP = 4,
  DUALKV_ERR_SCRATCH_LIMIT = 5   /* dualkv_bwd_noalloc: workspace need above its static buffer */
};

enum { DUALKV_F32 = 0, DUALKV_BF16 = 1 };        /* dualkv_params.dtype */
enum { DUALKV_GATHER = 0, DUALKV_SCATTER = 1 };  /* dualkv_repack direction */
enum {                                            /* dualkv_params.impl */
  DUALKV_IMPL_AUTO = 0,     /* MFMA tiles when supported, else scalar */
  DUALKV_IMPL_SCALAR = 1,   /* one wavefront per row, fp32 arithmetic */
  DUALKV_IMPL_MFMA = 2      /* bf16 MFMA tiles; UNSUPPORTED if not possible */
};

typedef struct dualkv_params {
  int32_t n_resp;        /* N >= 1 */
  int32_t prompt_len;    /* P >= 0 (P = 0: N independent causal sequences) */
  int32_t resp_len;      /* R >= 0, padded response length */
  int32_t n_q_heads;     /* Hq >= 1 */
  int32_t n_kv_heads;    /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;      /* D: 1..512 (scalar); 64, 128, 256, 512 (MFMA) */
  int32_t window;        /* <= 0: none; else keys with pos_q - pos_k < window */
  float softmax_scale;   /* > 0, or 0 for 1/sqrt(D); negative is invalid */
  int32_t dtype;         /* DUALKV_F32 or DUALKV_BF16, shared by every tensor
                            argument except LSE (always fp32) */
  int32_t impl;          /* DUALKV_IMPL_* */
  const int32_t* resp_valid_len;  /* device int32 [N] or NULL (= all R);
                                     values are clamped to [0, R] */
} dualkv_params;

/*
 * Repack rows between the replicated N(P+R) layout and the packed P+NR
 * layout (arXiv 2605.15422, Abstract: the data-pipeline repack).
 *   DUALKV_GATHER : src replicated [N(P+R) rows] -> dst packed [P+NR rows];
 *                   the prompt is taken from copy 0.
 *   DUALKV_SCATTER: src packed -> dst replicated; the prompt is copied into
 *                   every sequence.
 * Rows are opaque: row_bytes >= 1 bytes each (any element type, any head
 * count).  The copy is bit exact.  src and dst must not overlap.
 * Returns DUALKV_ERR_INVALID_ARGUMENT for null pointers (with a non-empty
 * copy), row_bytes < 1, N < 1, P < 0, R < 0 or an unknown direction.
 */
int dualkv_repack(const void* src, void* dst, int64_t row_bytes,
                  int32_t n_resp, int32_t prompt_len, int32_t resp_len,
                  int32_t direction, void* stream);

/*
 * Forward pass over the packed layout (arXiv 2605.15422, Abstract: one
 * kernel launch iterates over the two disjoint key regions, shared prompt
 * and own response).  Reads q, k, v; writes o [T, Hq, D] (dtype) and
 * lse [Hq, T] (fp32).  Rows with no visible key get O = 0, LSE = -inf.
 */
int dualkv_fwd(const dualkv_params* p, const void* q, const void* k,
               const void* v, void* o, float* lse, void* stream);

/*
 * Bytes of device workspace dualkv_bwd needs for these parameters
 * (per-row softmax statistics and the split partial sums of the prompt
 * dK/dV).  Returns 0 when the parameters are invalid.
 */
size_t dualkv_bwd_workspace_bytes(const dualkv_params* p);

/*
 * Backward pass (arXiv 2605.15422, Abstract: fused backward over the two
 * key regions).  Given q, k, v, the forward's o and lse, and dout (dO),
 * overwrites dq [T, Hq, D], dk and dv [T, Hkv, D].  The prompt rows of
 * dk/dv hold the sum over the prompt's own queries and all N responses;
 * that sum is accumulated in a fixed order, so results are bitwise
 * reproducible run to run.  `workspace` must hold at least
 * dualkv_bwd_workspace_bytes(p) bytes (DUALKV_ERR_WORKSPACE_TOO_SMALL
 * otherwise) and be 256-byte aligned; its contents on entry are ignored.
 */
int dualkv_bwd(const dualkv_params* p, const void* q, const void* k,
               const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * dualkv_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, contract and results as dualkv_bwd, with the
 * workspace taken from a static device buffer of
 * DUALKV_NOALLOC_SCRATCH_BYTES (256 MiB) that the library holds on every
 * GPU it runs on until the process ends.  The call allocates nothing.
 * It runs on the current device (the device of `stream`).  Returns
 * DUALKV_ERR_SCRATCH_LIMIT, launching nothing, when
 * dualkv_bwd_workspace_bytes(p) exceeds the buffer (the Qwen3-8B-shaped
 * layer, N=32, P=8192, R=1024, 32/8 heads, D=128, needs about 179 MB).
 * All calls on one GPU share its buffer: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialised by the caller.
 */
#define DUALKV_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

int dualkv_bwd_noalloc(const dualkv_params* p, const void* q, const void* k,
                       const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv,
                       void* stream);

/*
 * Several prompt groups in one call ("DualKV: Shared-Prompt Flash
 * Attention ..." (arXiv 2605.15422), Abstract: a micro-batch is packed per
 * prompt; a micro-batch that holds several prompts packs each of them and
 * lays the packed groups one after the other, as variable-length attention
 * does with cumulative sequence offsets).
 *
 * Group i has its own N_i >= 1 responses of padded length R_i >= 0 sharing
 * a prompt of P_i >= 0 tokens.  Its T_i = P_i + N_i*R_i packed rows start at
 * row0_i = T_0 + ... + T_{i-1}; the whole call has Tld = sum_i T_i rows:
 *   Q, O, dO, dQ  [Tld, Hq, D],  K, V, dK, dV  [Tld, Hkv, D],  LSE [Hq, Tld].
 * Attention never crosses groups: the rows of group i follow the rules above
 * with (N_i, P_i, R_i), at positions counted from the group's own row 0.
 * In dualkv_params, n_resp, prompt_len and resp_len are ignored;
 * resp_valid_len (device int32, or NULL) holds sum_i N_i entries, group 0's
 * first.  `groups` is a host array of n_groups entries, 1 <= n_groups <=
 * DUALKV_MAX_GROUPS (DUALKV_ERR_UNSUPPORTED above, INVALID_ARGUMENT below
 * or for a malformed entry).  With n_groups = 1 each call is the same as
 * its single-group counterpart, which is defined as exactly that.
 * On the MFMA path every kernel of a call covers all groups in one launch
 * (the launches are those of a single-group call); the scalar path
 * launches its kernels once per group.  Results per group are bit for bit
 * those of the single-group call on that group's rows.
 */
#define DUALKV_MAX_GROUPS 32

typedef struct dualkv_group {
  int32_t n_resp;        /* N_i >= 1 */
  int32_t prompt_len;    /* P_i >= 0 */
  int32_t resp_len;      /* R_i >= 0 */
} dualkv_group;

/* dualkv_fwd over groups: o [Tld, Hq, D], lse [Hq, Tld]. */
int dualkv_fwd_groups(const dualkv_params* p, const dualkv_group* groups,
                      int32_t n_groups, const void* q, const void* k,
                      const void* v, void* o, float* lse, void* stream);

/* Workspace of dualkv_bwd_groups for these parameters (0 if invalid). */
size_t dualkv_bwd_groups_workspace_bytes(const dualkv_params* p,
                                         const dualkv_group* groups,
                                         int32_t n_groups);

/* dualkv_bwd over groups, same contract per group (each prompt's dK/dV is
 * summed over its own queries and its own N_i responses only). */
int dualkv_bwd_groups(const dualkv_params* p, const dualkv_group* groups,
                      int32_t n_groups, const void* q, const void* k,
                      const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, void* stream);

/* dualkv_repack over groups: the replicated layout holds group after group
 * (N_i(P_i+R_i) rows each), the packed layout group after group (T_i rows
 * each); every group is repacked as by dualkv_repack.  Same errors, plus
 * those of `groups` above. */
int dualkv_repack_groups(const void* src, void* dst, int64_t row_bytes,
                         const dualkv_group* groups, int32_t n_groups,
                         int32_t direction, void* stream);

/* ------------------------------------------------------------------------
 * A packed transformer layer (arXiv 2605.15422, Abstract: the packed layout
 * reduces the tokens of the whole model, so every token-wise step runs on
 * P+NR rows).  All tensors bf16, row-major, 16-byte aligned; fp32
 * arithmetic inside every kernel.  Each entry point validates on the host
 * and launches nothing on error.
 * ------------------------------------------------------------------------ */

/*
 * C[M][N] = A B (+ R), fp32 accumulation, bf16 result.  A is stored [M][K]
 * (lda >= K), or with trans_a as [K][M] (lda >= M); B is [K][N] (ldb >= N),
 * or with trans_b as [N][K] (ldb >= K); C and R are [M][N] (ldc, ldr >= N);
 * R may be NULL or equal to C.  trans_a and trans_b are not both set.
 * DUALKV_ERR_UNSUPPORTED for shapes the 128x128x64 tiles do not take: with
 * trans_a M % 128 == 0; without trans_b N % 128 == 0; K % 64 == 0 unless
 * trans_a is set and trans_b is not (K free there); lda, ldb multiples
 * of 8.
 */
int dualkv_gemm_bf16(int32_t trans_a, int32_t trans_b, int32_t M, int32_t N,
                     int32_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, void* C, int64_t ldc, const void* R,
                     int64_t ldr, void* stream);

/*
 * RMSNorm of T rows of H (H % 8 == 0): rstd[t] = 1/sqrt(mean_i x[t][i]^2 +
 * eps) (fp32 [T]), y = x * rstd * w.  The backward writes
 * dx = rstd * (w*dy - xh * mean_i(w*dy*xh)) + dres (xh = x*rstd; dres may be
 * NULL) and dw[i] = sum_t dy[t][i] * xh[t][i] (rows summed in a fixed
 * order), using a workspace of dualkv_rmsnorm_bwd_workspace_bytes(T, H).
 */
int dualkv_rmsnorm_fwd(int32_t T, int32_t H, float eps, const void* x,
                       const void* w, void* y, float* rstd, void* stream);
size_t dualkv_rmsnorm_bwd_workspace_bytes(int32_t T, int32_t H);
int dualkv_rmsnorm_bwd(int32_t T, int32_t H, const void* x, const void* w,
                       const float* rstd, const void* dy, const void* dres,
                       void* dx, void* dw, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Rotary position embedding, in place, on x [rows][n_heads][head_dim] of
 * the packed groups: row t of a group has logical position t (prompt) or
 * P + r (response row r), and the pair (i, i + head_dim/2) of every head is
 * rotated by the angle pos * base^(-2i/head_dim) (by its negative with
 * inverse = 1, which undoes the rotation).
 */
int dualkv_rope(const dualkv_group* groups, int32_t n_groups, int32_t n_heads,
                int32_t head_dim, float base, int32_t inverse, void* x,
                void* stream);

/* SwiGLU over n elements (n % 8 == 0): m = silu(u) * g; backward
 * du = dm * g * silu'(u), dg = dm * silu(u). */
int dualkv_swiglu_fwd(int64_t n, const void* u, const void* g, void* m,
                      void* stream);
int dualkv_swiglu_bwd(int64_t n, const void* u, const void* g, const void* dm,
                      void* du, void* dg, void* stream);

/*
 * Pre-norm decoder layer on the packed groups (Tld rows of `hidden`):
 *   h1 = RMSNorm(x; norm1); q, k, v = h1 wq, h1 wk, h1 wv;
 *   q, k = RoPE at the rows' logical positions;
 *   o = shared-prompt attention (dualkv_fwd_groups, window, valid lengths);
 *   x1 = x + o wo; h2 = RMSNorm(x1; norm2); m = silu(h2 w1) * (h2 w3);
 *   y = x1 + m w2.
 * Weights are [in][out]: wq [hidden][Hq*D], wk, wv [hidden][Hkv*D],
 * wo [Hq*D][hidden], w1, w3 [hidden][ffn], w2 [ffn][hidden], norms [hidden].
 * hidden, ffn, Hq*D and Hkv*D must be multiples of 128
 * (DUALKV_ERR_UNSUPPORTED otherwise).  The forward keeps its activations in
 * `saved` (dualkv_layer_saved_bytes, 256-byte aligned) for the backward,
 * which writes dx and the weight gradients `grads` (same shapes as the
 * weights, overwritten) using `workspace` (dualkv_layer_workspace_bytes,
 * 256-byte aligned).  Each prompt's rows appear once, so the weight
 * gradients sum each prompt token once, with the gradient it receives from
 * all responses of its group.
 */
typedef struct dualkv_layer_params {
  int32_t hidden;
  int32_t n_q_heads, n_kv_heads, head_dim;
  int32_t ffn;
  int32_t window;                 /* attention window, <= 0: none */
  float rope_base;                /* > 1 */
  float norm_eps;                 /* > 0 */
  const int32_t* resp_valid_len;  /* device int32 [sum N_i] or NULL */
} dualkv_layer_params;

typedef struct dualkv_layer_weights {
  const void *norm1, *wq, *wk, *wv, *wo, *norm2, *w1, *w3, *w2;
} dualkv_layer_weights;

typedef struct dualkv_layer_grads {
  void *norm1, *wq, *wk, *wv, *wo, *norm2, *w1, *w3, *w2;
} dualkv_layer_grads;

size_t dualkv_layer_saved_bytes(const dualkv_layer_params* p,
                                const dualkv_group* groups, int32_t n_groups);
size_t dualkv_layer_workspace_bytes(const dualkv_layer_params* p,
                                    const dualkv_group* groups,
                                    int32_t n_groups);
int dualkv_layer_fwd(const dualkv_layer_params* p, const dualkv_group* groups,
                     int32_t n_groups, const dualkv_layer_weights* w,
                     const void* x, void* y, void* saved, size_t saved_bytes,
                     void* stream);
int dualkv_layer_bwd(const dualkv_layer_params* p, const dualkv_group* groups,
                     int32_t n_groups, const dualkv_layer_weights* w,
                     const void* x, const void* saved, size_t saved_bytes,
                     const void* dy, void* dx, const dualkv_layer_grads* grads,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable text for a status code. */
const char* dualkv_strerror(int status);

/*
 * Launch profiler for measurement tools (results are unaffected).
 * dualkv_profile_start() clears earlier records and starts bracketing
 * every kernel the library launches with two HIP events on the launch
 * stream.  dualkv_profile_stop() stops recording, waits for the recorded
 * events and aggregates elapsed time per kernel name; it returns
 * DUALKV_ERR_HIP if an event could not be read.  dualkv_profile_count()
 * then gives the number of kernel names and dualkv_profile_kernel(i, ...)
 * the name (static storage, valid until the next start), launch count and
 * total milliseconds of entry i (DUALKV_ERR_INVALID_ARGUMENT for a bad i or
 * null output).  The profiler is process-wide state guarded by a mutex;
 * it is the only mutable state of the library and is off by default.
 */
int dualkv_profile_start(void);
int dualkv_profile_stop(void);
int dualkv_profile_count(void);
int dualkv_profile_kernel(int index, const char** name, int64_t* launches, double* total_ms);

/*
 * Matrix-core rate probe for measurement tools: enqueues one kernel of
 * `workgroups` x 512 threads in which every wave issues `iters` x 4
 * independent bf16 32x32x16 MFMAs (no memory traffic) and returns the
 * number of floating-point operations it performs (-1 on a bad argument
 * or launch error).  Timing it with events on `stream` gives the dense
 * bf16 rate the device sustains.  It writes no memory.
 */
int64_t dualkv_mfma_probe(int32_t workgroups, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DUALKV_H */
