// Backward of the GroupQueryAttention forward without past (onnx-light-cpu C++
// API page "Custom operators", RegisterCustomOperatorGradients,
// GroupQueryAttention gradient: the probabilities are recomputed from Q, K,
// V, then the softmax backward, the score gradient scaled by the forward's
// scale, dQ = dS K, dK = dS^T Q, dV = P^T dY with the grouped K/V head
// gradients summed back to their KV head, and a cast to the input type).
//
// These kernels take every shape in scope that the matrix-core kernels of
// olk_backward_mfma.hip do not (fp32, other head sizes, Dv != D, head groups
// that are not a power of two up to 32).
// Three kernels, fp32 VALU arithmetic, one 64-lane wavefront per work item:
//   bwd_stats_kernel  per query row: lse_i = log sum_j exp(s_ij) over the
//                     allowed keys (s = scaled score) and
//                     delta_i = sum_j P_ij (dY_i . V_j)
//   bwd_dq_kernel     per query row: dQ_i = sum_j dS_ij K_j
//   bwd_dkv_kernel    per (b, KV head g, key j): dK_j = sum dS_ij Q_i and
//                     dV_j = sum P_ij dY_i over the rows (i, h) of the heads
//                     sharing g
// with P_ij = exp(s_ij - lse_i) and dS_ij = P_ij (dY_i . V_j - delta_i) scale.
// Without past, query i sits at position i; the causal mask allows j <= i and
// a local window W allows j >= i - W + 1.
#include "olk_internal.h"

namespace olk {
namespace {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float wmax(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ float wsum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Row (b, token i, head h) of a (B, S, H*W) tensor.
template <typename T>
__device__ __forceinline__ const T *row_of(const void *base, const Params &p, int b, int i,
                                           int h, int heads, int width) {
  return (const T *)base + (((int64_t)b * p.S + i) * heads + h) * width;
}

__device__ __forceinline__ bool allowed(const Params &p, int i, int j) {
  if (p.causal && j > i) return false;
  if (p.window > 0 && j < i - p.window + 1) return false;
  return true;
}

__device__ __forceinline__ void key_span(const Params &p, int i, int &lo, int &hi) {
  hi = p.causal ? i + 1 : p.S;
  lo = p.window > 0 ? max(0, i - p.window + 1) : 0;
}

// s_ij and dY_i . V_j for key j of the lane (q and dy of row i in LDS)
template <typename T>
__device__ __forceinline__ void score_dp(const Params &p, int b, int g, int j, const float *qs,
                                         const float *dys, float &s, float &dp) {
  const T *kr = row_of<T>(p.k, p, b, j, g, p.Hkv, p.D);
  const T *vr = row_of<T>(p.v, p, b, j, g, p.Hkv, p.Dv);
  float dot = 0.f, d2 = 0.f;
  for (int c = 0; c < p.D; ++c) dot = fmaf(qs[c], (float)kr[c], dot);
  for (int c = 0; c < p.Dv; ++c) d2 = fmaf(dys[c], (float)vr[c], d2);
  s = dot * p.scale;
  dp = d2;
}

template <typename T>
__device__ __forceinline__ void load_row(const T *src, float *dst, int n) {
  for (int c = threadIdx.x; c < n; c += kWave) dst[c] = (float)src[c];
}

template <typename T>
__global__ __launch_bounds__(kWave) void bwd_stats_kernel(Params p, const T *dy, float *lse,
                                                          float *delta) {
  __shared__ float qs[256], dys[256];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / p.G;
  load_row(row_of<T>(p.q, p, b, i, h, p.Hq, p.D), qs, p.D);
  load_row(dy + (((int64_t)b * p.S + i) * p.Hq + h) * p.Dv, dys, p.Dv);
  __syncthreads();
  int lo, hi;
  key_span(p, i, lo, hi);
  float m = kNegInf, l = 0.f, acc = 0.f;
  for (int j0 = lo; j0 < hi; j0 += kWave) {
    const int j = j0 + threadIdx.x;
    float s = kNegInf, dp = 0.f;
    if (j < hi) score_dp<T>(p, b, g, j, qs, dys, s, dp);
    const float cm = wmax(s);
    const float mn = fmaxf(m, cm);
    const float a = m == kNegInf ? 0.f : expf(m - mn);
    const float e = s == kNegInf ? 0.f : expf(s - mn);
    l = l * a + wsum(e);
    acc = acc * a + wsum(e * dp);
    m = mn;
  }
  if (threadIdx.x == 0) {
    const int64_t r = ((int64_t)b * p.Hq + h) * p.S + i;
    lse[r] = m == kNegInf ? kNegInf : m + logf(l);
    delta[r] = m == kNegInf ? 0.f : acc / l;
  }
}

template <typename T>
__global__ __launch_bounds__(kWave) void bwd_dq_kernel(Params p, const T *dy, const float *lse,
                                                       const float *delta, T *dq) {
  __shared__ float qs[256], dys[256], ds[kWave];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / p.G;
  load_row(row_of<T>(p.q, p, b, i, h, p.Hq, p.D), qs, p.D);
  load_row(dy + (((int64_t)b * p.S + i) * p.Hq + h) * p.Dv, dys, p.Dv);
  __syncthreads();
  const int64_t r = ((int64_t)b * p.Hq + h) * p.S + i;
  const float L = lse[r], Dl = delta[r];
  int lo, hi;
  key_span(p, i, lo, hi);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // dims lane + 64 k
  for (int j0 = lo; j0 < hi && L != kNegInf; j0 += kWave) {
    const int j = j0 + threadIdx.x;
    float dsj = 0.f;
    if (j < hi) {
      float s, dp;
      score_dp<T>(p, b, g, j, qs, dys, s, dp);
      dsj = expf(s - L) * (dp - Dl) * p.scale;
    }
    ds[threadIdx.x] = dsj;
    __syncthreads();
    const int nj = min(kWave, hi - j0);
    for (int jj = 0; jj < nj; ++jj) {
      const float w = ds[jj];
      const T *kr = row_of<T>(p.k, p, b, j0 + jj, g, p.Hkv, p.D);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d = threadIdx.x + k * kWave;
        if (d < p.D) acc[k] = fmaf(w, (float)kr[d], acc[k]);
      }
    }
    __syncthreads();
  }
  T *out = dq + (((int64_t)b * p.S + i) * p.Hq + h) * p.D;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = threadIdx.x + k * kWave;
    if (d < p.D) out[d] = (T)acc[k];
  }
}

template <typename T>
__global__ __launch_bounds__(kWave) void bwd_dkv_kernel(Params p, const T *dy, const float *lse,
                                                        const float *delta, T *dk, T *dv) {
  __shared__ float ks[256], vs[256], pw[kWave], dsw[kWave];
  __shared__ int rows[kWave];
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  load_row(row_of<T>(p.k, p, b, j, g, p.Hkv, p.D), ks, p.D);
  load_row(row_of<T>(p.v, p, b, j, g, p.Hkv, p.Dv), vs, p.Dv);
  __syncthreads();
  // query rows that see key j: i in [j, S) causal (else [0, S)), cut by the window
  const int i_lo = p.causal ? j : 0;
  const int i_hi = p.window > 0 ? min(p.S, j + p.window) : p.S;
  const int n_i = max(0, i_hi - i_lo);
  const int n_rows = n_i * p.G;  // rows (i, h) for the G heads of g
  float ak[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < n_rows; r0 += kWave) {
    const int r = r0 + threadIdx.x;
    float pj = 0.f, dsj = 0.f;
    int row = -1;
    if (r < n_rows) {
      const int i = i_lo + r / p.G, h = g * p.G + r % p.G;
      row = i * p.Hq + h;
      const int64_t sr = ((int64_t)b * p.Hq + h) * p.S + i;
      const float L = lse[sr];
      if (L != kNegInf && allowed(p, i, j)) {
        const T *qr = row_of<T>(p.q, p, b, i, h, p.Hq, p.D);
        const T *dr = dy + (((int64_t)b * p.S + i) * p.Hq + h) * p.Dv;
        float dot = 0.f, dp = 0.f;
        for (int c = 0; c < p.D; ++c) dot = fmaf((float)qr[c], ks[c], dot);
        for (int c = 0; c < p.Dv; ++c) dp = fmaf((float)dr[c], vs[c], dp);
        pj = expf(dot * p.scale - L);
        dsj = pj * (dp - delta[sr]) * p.scale;
      }
    }
    pw[threadIdx.x] = pj;
    dsw[threadIdx.x] = dsj;
    rows[threadIdx.x] = row;
    __syncthreads();
    const int nr = min(kWave, n_rows - r0);
    for (int rr = 0; rr < nr; ++rr) {
      const float wp = pw[rr], wd = dsw[rr];
      if (wp == 0.f && wd == 0.f) continue;
      const int rw = rows[rr];
      const int i = rw / p.Hq, h = rw % p.Hq;
      const T *qr = row_of<T>(p.q, p, b, i, h, p.Hq, p.D);
      const T *dr = dy + (((int64_t)b * p.S + i) * p.Hq + h) * p.Dv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d = threadIdx.x + k * kWave;
        if (d < p.D) ak[k] = fmaf(wd, (float)qr[d], ak[k]);
        if (d < p.Dv) av[k] = fmaf(wp, (float)dr[d], av[k]);
      }
    }
    __syncthreads();
  }
  T *ko = dk + (((int64_t)b * p.S + j) * p.Hkv + g) * p.D;
  T *vo = dv + (((int64_t)b * p.S + j) * p.Hkv + g) * p.Dv;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = threadIdx.x + k * kWave;
    if (d < p.D) ko[d] = (T)ak[k];
    if (d < p.Dv) vo[d] = (T)av[k];
  }
}

template <typename T>
hipError_t launch_bwd_t(const Params &p, const void *dy, void *dq, void *dk, void *dv,
                        float *ws, hipStream_t st) {
  float *lse = ws, *delta = ws + (int64_t)p.B * p.Hq * p.S;
  const dim3 rows(p.S, p.Hq, p.B), keys(p.S, p.Hkv, p.B), blk(kWave);
  hipLaunchKernelGGL(bwd_stats_kernel<T>, rows, blk, 0, st, p, (const T *)dy, lse, delta);
  hipLaunchKernelGGL(bwd_dq_kernel<T>, rows, blk, 0, st, p, (const T *)dy, lse, delta, (T *)dq);
  hipLaunchKernelGGL(bwd_dkv_kernel<T>, keys, blk, 0, st, p, (const T *)dy, lse, delta,
                     (T *)dk, (T *)dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Params &p, int dtype, const void *dy, void *dq, void *dk,
                           void *dv, float *ws, hipStream_t st) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  if (backward_mfma_supports(p, dtype, dy, dq, dk, dv))
    return launch_backward_mfma(p, dtype, dy, dq, dk, dv, ws, st);
  if (dtype == DT_BF16) return launch_bwd_t<bf16>(p, dy, dq, dk, dv, ws, st);
  if (dtype == DT_F16) return launch_bwd_t<f16>(p, dy, dq, dk, dv, ws, st);
  return launch_bwd_t<float>(p, dy, dq, dk, dv, ws, st);
}

}  // namespace olk
