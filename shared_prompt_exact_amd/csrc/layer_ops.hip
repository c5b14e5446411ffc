// Token-wise operations of a packed transformer layer: RMSNorm, rotary
// position embedding at the packed rows' logical positions, SwiGLU.
//
// "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
// the token reduction of the packed P+NR layout carries over from
// attention to the rest of the model, whose token-wise work then runs once
// per prompt token instead of N times.  The only token-wise operation that
// depends on where a row sits is the rotary embedding: packed response row
// r has logical position P + r (the position it has in its replicated
// sequence), prompt row t position t.
//
// All tensors are bf16 in memory, arithmetic is fp32, results are rounded
// to bf16 once (round to nearest even).  These kernels are bound by HBM
// traffic: rows are read with 16-byte loads, one wave per row (RMSNorm) or
// eight elements per thread (SwiGLU).
#include <math.h>

#include "common.h"

namespace dualkv {
namespace {

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  const unsigned u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(u[j] << 16);
    f[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  unsigned u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    u[j] = (unsigned)f32_to_bf16(f[2 * j]) | ((unsigned)f32_to_bf16(f[2 * j + 1]) << 16);
  return uint4{u[0], u[1], u[2], u[3]};
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// y = x * rstd * w, rstd = 1 / sqrt(mean(x^2) + eps); one wave per row.
__global__ void __launch_bounds__(256)
    rmsnorm_fwd_kernel(int T, int H, float eps, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                       uint16_t* __restrict__ y, float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * H);
  const int nc = H / 8;
  float ss = 0.f;
  for (int c = lane; c < nc; c += 64) {
    float f[8];
    unpack8(xr[c], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(f[j], f[j], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)H + eps);
  const uint4* wr = reinterpret_cast<const uint4*>(w);
  uint4* yr = reinterpret_cast<uint4*>(y + row * H);
  for (int c = lane; c < nc; c += 64) {
    float f[8], g[8];
    unpack8(xr[c], f);
    unpack8(wr[c], g);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = f[j] * r * g[j];
    yr[c] = pack8(f);
  }
  if (lane == 0) rstd[row] = r;
}

// dx = rstd * (w*dy - xh * mean(w*dy*xh)) (+ dres), xh = x * rstd.
__global__ void __launch_bounds__(256)
    rmsnorm_bwd_kernel(int T, int H, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                       const float* __restrict__ rstd, const uint16_t* __restrict__ dy,
                       const uint16_t* __restrict__ dres, uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int nc = H / 8;
  const float r = rstd[row];
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * H);
  const uint4* dr = reinterpret_cast<const uint4*>(dy + row * H);
  const uint4* wr = reinterpret_cast<const uint4*>(w);
  float dot = 0.f;
  for (int c = lane; c < nc; c += 64) {
    float a[8], b[8], g[8];
    unpack8(xr[c], a);
    unpack8(dr[c], b);
    unpack8(wr[c], g);
#pragma unroll
    for (int j = 0; j < 8; ++j) dot = fmaf(g[j] * b[j], a[j] * r, dot);
  }
  const float mdot = wave_sum(dot) / (float)H;
  uint4* out = reinterpret_cast<uint4*>(dx + row * H);
  const uint4* rr = reinterpret_cast<const uint4*>(dres + (dres ? row * H : 0));
  for (int c = lane; c < nc; c += 64) {
    float a[8], b[8], g[8], e[8];
    unpack8(xr[c], a);
    unpack8(dr[c], b);
    unpack8(wr[c], g);
    if (dres) unpack8(rr[c], e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = r * (g[j] * b[j] - a[j] * r * mdot);
      a[j] = dres ? e[j] + v : v;
    }
    out[c] = pack8(a);
  }
}

// Column sums for the norm weight gradient: part[chunk][i] = sum over rows
// t of the chunk of dy[t][i] * x[t][i] * rstd[t] (rows in ascending order).
__global__ void __launch_bounds__(256)
    norm_wgrad_partial_kernel(int T, int H, int rows_per_chunk, const uint16_t* __restrict__ x,
                              const uint16_t* __restrict__ dy, const float* __restrict__ rstd,
                              float* __restrict__ part) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= H) return;
  const int t0 = blockIdx.y * rows_per_chunk, t1 = min(T, t0 + rows_per_chunk);
  float s = 0.f;
  for (int t = t0; t < t1; ++t)
    s = fmaf(bf16_to_f32(dy[(int64_t)t * H + i]), bf16_to_f32(x[(int64_t)t * H + i]) * rstd[t], s);
  part[(int64_t)blockIdx.y * H + i] = s;
}

// out[i] = sum over chunks c (ascending) of part[c][i], rounded to bf16.
__global__ void __launch_bounds__(256)
    sum_chunks_kernel(int n, int H, const float* __restrict__ part, uint16_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= H) return;
  float s = 0.f;
  for (int c = 0; c < n; ++c) s += part[(int64_t)c * H + i];
  out[i] = f32_to_bf16(s);
}

// Logical position of packed row t (rows of all groups, group after group).
__device__ __forceinline__ int packed_position(const Groups& G, int t) {
  int gi = 0;
  while (gi + 1 < G.n && t >= G.row0[gi + 1]) ++gi;
  const int local = t - G.row0[gi], P = G.P[gi], R = G.R[gi];
  return local < P ? local : P + (local - P) % R;
}

// Rotary embedding, rotate-half pairs (i, i + D/2), angle pos * base^(-2i/D)
// (negated for `inverse`, which undoes the rotation, as the backward
// needs).  x is [T][H][D] and is rewritten in place.  The angle is formed
// and reduced modulo 2*pi in fp64 (positions reach 10^5), then sin/cos in
// fp32.
__global__ void __launch_bounds__(256)
    rope_kernel(int64_t n_pairs, int H, int D, Groups G, double log2_base, int inverse,
                uint16_t* __restrict__ x) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_pairs) return;
  const int half = D / 2;
  const int i = (int)(idx % half);
  const int64_t th = idx / half;                 // t * H + h
  const int t = (int)(th / H);
  const int pos = packed_position(G, t);
  const double inv_freq = exp2(-(2.0 * i / D) * log2_base);
  double ang = (double)pos * inv_freq;
  ang -= 6.283185307179586 * rint(ang / 6.283185307179586);
  float s, c;
  sincosf((float)ang, &s, &c);
  if (inverse) s = -s;
  uint16_t* p = x + th * D;
  const float a = bf16_to_f32(p[i]), b = bf16_to_f32(p[i + half]);
  p[i] = f32_to_bf16(a * c - b * s);
  p[i + half] = f32_to_bf16(a * s + b * c);
}

// The same rotation with the angle work shared by the heads: a thread takes
// token t and the eight pairs (8j + e, 8j + e + D/2), forms their eight
// angles and sin/cos once (as above), then rotates them in every head with
// 16-byte loads and stores.  Needs D % 16 == 0 and a 16-byte aligned x.
__global__ void __launch_bounds__(256)
    rope_kernel_x8(int64_t n_threads, int H, int D, Groups G, double log2_base, int inverse,
                 uint16_t* __restrict__ x) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_threads) return;
  const int half = D / 2, g8 = half / 8;
  const int j = (int)(idx % g8);
  const int t = (int)(idx / g8);
  const int pos = packed_position(G, t);
  float c[8], s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = 8 * j + e;
    const double inv_freq = exp2(-(2.0 * i / D) * log2_base);
    double ang = (double)pos * inv_freq;
    ang -= 6.283185307179586 * rint(ang / 6.283185307179586);
    sincosf((float)ang, &s[e], &c[e]);
    if (inverse) s[e] = -s[e];
  }
  uint16_t* row = x + (int64_t)t * H * D + 8 * j;
  for (int h = 0; h < H; ++h) {
    uint4* pa = reinterpret_cast<uint4*>(row + (int64_t)h * D);
    uint4* pb = reinterpret_cast<uint4*>(row + (int64_t)h * D + half);
    float a[8], b[8], ra[8], rb[8];
    unpack8(*pa, a);
    unpack8(*pb, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ra[e] = a[e] * c[e] - b[e] * s[e];
      rb[e] = a[e] * s[e] + b[e] * c[e];
    }
    *pa = pack8(ra);
    *pb = pack8(rb);
  }
}

__device__ __forceinline__ float sigmoid(float u) { return 1.f / (1.f + __expf(-u)); }

// m = silu(u) * g, eight elements per thread.
__global__ void __launch_bounds__(256)
    swiglu_fwd_kernel(int64_t n8, const uint16_t* __restrict__ u, const uint16_t* __restrict__ g,
                      uint16_t* __restrict__ m) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float a[8], b[8];
  unpack8(reinterpret_cast<const uint4*>(u)[i], a);
  unpack8(reinterpret_cast<const uint4*>(g)[i], b);
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = a[j] * sigmoid(a[j]) * b[j];
  reinterpret_cast<uint4*>(m)[i] = pack8(a);
}

// du = dm * g * silu'(u), dg = dm * silu(u); silu'(u) = s (1 + u (1 - s)).
__global__ void __launch_bounds__(256)
    swiglu_bwd_kernel(int64_t n8, const uint16_t* __restrict__ u, const uint16_t* __restrict__ g,
                      const uint16_t* __restrict__ dm, uint16_t* __restrict__ du, uint16_t* __restrict__ dg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float a[8], b[8], d[8], ra[8], rb[8];
  unpack8(reinterpret_cast<const uint4*>(u)[i], a);
  unpack8(reinterpret_cast<const uint4*>(g)[i], b);
  unpack8(reinterpret_cast<const uint4*>(dm)[i], d);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float s = sigmoid(a[j]);
    ra[j] = d[j] * b[j] * s * (1.f + a[j] * (1.f - s));
    rb[j] = d[j] * a[j] * s;
  }
  reinterpret_cast<uint4*>(du)[i] = pack8(ra);
  reinterpret_cast<uint4*>(dg)[i] = pack8(rb);
}

unsigned blocks256(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_rmsnorm_fwd(int T, int H, float eps, const void* x, const void* w, void* y, float* rstd,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  return launch("rmsnorm_fwd", rmsnorm_fwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, H, eps,
                static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), static_cast<uint16_t*>(y),
                rstd);
}

int norm_wgrad_chunks(int T) { return T == 0 ? 0 : (T + 255) / 256; }

hipError_t launch_rmsnorm_bwd(int T, int H, const void* x, const void* w, const float* rstd, const void* dy,
                              const void* dres, void* dx, void* dw, float* part, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipError_t e = launch("rmsnorm_bwd", rmsnorm_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, H,
                        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), rstd,
                        static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(dres),
                        static_cast<uint16_t*>(dx));
  if (e != hipSuccess) return e;
  const int nch = norm_wgrad_chunks(T);
  e = launch("norm_wgrad", norm_wgrad_partial_kernel, dim3(blocks256(H), (unsigned)nch), dim3(256), 0, s, T, H,
             256, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dy), rstd, part);
  if (e != hipSuccess) return e;
  return launch("norm_wgrad", sum_chunks_kernel, dim3(blocks256(H)), dim3(256), 0, s, nch, H,
                static_cast<const float*>(part), static_cast<uint16_t*>(dw));
}

hipError_t launch_rope(int T, int H, int D, const Groups& G, float base, int inverse, void* x, hipStream_t s) {
  const int64_t n = (int64_t)T * H * (D / 2);
  if (n == 0) return hipSuccess;
  if (D % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0) {
    const int64_t n8 = (int64_t)T * (D / 16);
    return launch("rope", rope_kernel_x8, dim3(blocks256(n8)), dim3(256), 0, s, n8, H, D, G, log2((double)base),
                  inverse, static_cast<uint16_t*>(x));
  }
  return launch("rope", rope_kernel, dim3(blocks256(n)), dim3(256), 0, s, n, H, D, G, log2((double)base), inverse,
                static_cast<uint16_t*>(x));
}

hipError_t launch_swiglu_fwd(int64_t n, const void* u, const void* g, void* m, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return launch("swiglu_fwd", swiglu_fwd_kernel, dim3(blocks256(n / 8)), dim3(256), 0, s, n / 8,
                static_cast<const uint16_t*>(u), static_cast<const uint16_t*>(g), static_cast<uint16_t*>(m));
}

hipError_t launch_swiglu_bwd(int64_t n, const void* u, const void* g, const void* dm, void* du, void* dg,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  return launch("swiglu_bwd", swiglu_bwd_kernel, dim3(blocks256(n / 8)), dim3(256), 0, s, n / 8,
                static_cast<const uint16_t*>(u), static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(dm),
                static_cast<uint16_t*>(du), static_cast<uint16_t*>(dg));
}

}  // namespace dualkv
