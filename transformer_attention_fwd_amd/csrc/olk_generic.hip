// Generic attention kernels: one 64-lane wavefront per query row, fp32 VALU
// arithmetic, every dtype and head size up to 256.  They cover every feature of
// the contract and serve the shapes the MFMA kernels do not (fp32, odd head
// sizes), plus the split-KV partial/combine pair behind olk_attention_decode.
//
// Score pipeline order (onnx-light reference kernels header page, "class
// Attention", qk_matmul_output_mode stages): (Q.K) * scale, + bias, softcap,
// then the masks.  The softmax runs online over 64-key chunks: running max m,
// running sum l, output rescaled by exp(m_old - m_new).  A head_sink (onnx-light-cpu
// Python API, "Microsoft GroupQueryAttention") joins only the denominator.
#include "olk_internal.h"

namespace olk {
namespace {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Row of key (value=false) or value (value=true) j of KV head g in batch b.
template <typename T>
__device__ __forceinline__ const T *kv_row(const Params &p, const Seq &s, int b, int g, int j,
                                           bool value) {
  const int width = value ? p.Dv : p.D;
  if (j < s.src) {
    const T *past = (const T *)(value ? p.past_v : p.past_k);
    return past + (((int64_t)b * p.Hkv + g) * p.past_rows + j) * width;
  }
  const T *cur = (const T *)(value ? p.v : p.k);
  const int64_t sb = value ? p.v_sb : p.k_sb, ss = value ? p.v_ss : p.k_ss,
                sh = value ? p.v_sh : p.k_sh;
  return cur + b * sb + (int64_t)(j - s.src) * ss + g * sh;
}

struct RowState {
  float m, l;
  float o[4];
};

// Online softmax over keys [j_lo, j_hi) of row (b, h, i); keys outside the
// row's allowed set are skipped by the caller's range and the per-key masks.
template <typename T>
__device__ void row_range(const Params &p, const Seq &s, int b, int h, int i, int j_lo,
                          int j_hi, const float *qs, float *ps, RowState &st) {
  const int lane = threadIdx.x;
  const int g = h / p.G;
  const int pos = s.qoff + i;
  for (int j0 = j_lo; j0 < j_hi; j0 += kWave) {
    const int j = j0 + lane;
    float sc = kNegInf;
    if (j < j_hi) {
      const T *kr = kv_row<T>(p, s, b, g, j, false);
      float dot = 0.f;
      // unrolled so that several of the row's loads are in flight at once
      // (the sum keeps its order)
#pragma unroll 8
      for (int c = 0; c < p.D; ++c) dot = fmaf(qs[c], to_f32(kr[c]), dot);
      sc = dot * p.scale;
      if (p.bias) {  // j < bias_cols: the caller's range stops there
        const T *br = (const T *)p.bias + b * p.bias_sb + h * p.bias_sh + (int64_t)i * p.bias_si;
        sc += to_f32(br[j]);
      }
      if (p.softcap > 0.f) sc = p.softcap * tanhf(sc / p.softcap);
      if (p.op == OP_MHA && j >= s.pad) sc += p.mfv;
      // MultiHeadAttention binary mask: a zero marks key padding (+mfv)
      if (p.mask_kind == 2 && !mask_at(p, b, h, i, j)) sc += p.mfv;
      // masks (exclusion) after the score pipeline
      bool ok = j < s.valid;
      if (p.causal && j > pos) ok = false;
      if (p.window > 0 && j < pos - p.window + 1) ok = false;
      if (p.mask_kind == 1 && !mask_at(p, b, h, i, j)) ok = false;  // BOOL false: -inf
      if (!ok) sc = kNegInf;
    }
    const float cmax = wave_max(sc);
    if (cmax == kNegInf) continue;  // whole chunk masked
    const float m_new = fmaxf(st.m, cmax);
    const float alpha = st.m == kNegInf ? 0.f : expf(st.m - m_new);
    const float pj = sc == kNegInf ? 0.f : expf(sc - m_new);
    st.l = st.l * alpha + wave_sum(pj);
    st.m = m_new;
    ps[lane] = pj;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) st.o[k] *= alpha;
    const int nj = min(kWave, j_hi - j0);
    // four keys at a time, their V loads issued together; a zero weight (a
    // masked key) leaves the sums as they are, whatever its V row holds
    int jj = 0;
    for (; jj + 4 <= nj; jj += 4) {
      float w[4], x[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[u] = ps[jj + u];
        const T *vr = kv_row<T>(p, s, b, g, j0 + jj + u, true);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int d = lane + k * kWave;
          x[u][k] = d < p.Dv ? to_f32(vr[d]) : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          st.o[k] = w[u] != 0.f ? fmaf(w[u], x[u][k], st.o[k]) : st.o[k];
    }
    for (; jj < nj; ++jj) {
      const float w = ps[jj];
      if (w == 0.f) continue;
      const T *vr = kv_row<T>(p, s, b, g, j0 + jj, true);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d = lane + k * kWave;
        if (d < p.Dv) st.o[k] = fmaf(w, to_f32(vr[d]), st.o[k]);
      }
    }
    __syncthreads();
  }
}

template <typename T>
__device__ void load_q(const Params &p, int b, int h, int i, float *qs) {
  const T *qr = (const T *)p.q + b * p.q_sb + (int64_t)i * p.q_ss + h * p.q_sh;
  for (int c = threadIdx.x; c < p.D; c += kWave) {
    float x = to_f32(qr[c]);
    if (p.op == OP_MHA && p.proj_bias) x += to_f32(((const T *)p.proj_bias)[h * p.D + c]);
    qs[c] = x;
  }
  __syncthreads();
}

// Allowed key range of query row i: [lo, hi).
__device__ __forceinline__ void key_range(const Params &p, const Seq &s, int i, int &lo,
                                          int &hi) {
  const int pos = s.qoff + i;
  hi = s.valid;
  if (p.causal) hi = min(hi, pos + 1);
  if (p.bias) hi = min(hi, p.bias_cols);  // a short mask excludes the keys beyond it
  lo = 0;
  if (p.window > 0) lo = max(0, pos - p.window + 1);
}

template <typename T>
__global__ __launch_bounds__(kWave) void generic_kernel(Params p) {
  __shared__ float qs[256];
  __shared__ float ps[kWave];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const Seq s = seq_info(p, b);
  load_q<T>(p, b, h, i, qs);
  int lo, hi;
  key_range(p, s, i, lo, hi);
  RowState st{kNegInf, 0.f, {0.f, 0.f, 0.f, 0.f}};
  row_range<T>(p, s, b, h, i, lo, hi, qs, ps, st);
  float inv = 0.f;
  if (st.m != kNegInf) {
    if (p.sink) {
      const float z = to_f32(((const T *)p.sink)[h]);
      const float mf = fmaxf(st.m, z);
      const float a = expf(st.m - mf);
      st.l = st.l * a + expf(z - mf);
#pragma unroll
      for (int k = 0; k < 4; ++k) st.o[k] *= a;
    }
    inv = 1.f / st.l;
  }
  T *yr = (T *)p.y + b * p.y_sb + (int64_t)i * p.y_ss + h * p.y_sh;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = threadIdx.x + k * kWave;
    if (d < p.Dv) yr[d] = from_f32<T>(st.o[k] * inv);
  }
  // present rows of the new keys (the present writer copied only the past):
  // the workgroup of the first query head of each KV group writes new rows
  // i, i + S, ... of that group, bits copied (positions past_b + j)
  if (p.present_past_only && p.present_k && p.present_v && h % p.G == 0) {
    const int g = h / p.G;
    for (int j = i; j < p.L; j += p.S) {
      const int64_t pos = ((int64_t)b * p.Hkv + g) * p.T + s.past + j;
      const T *kr = (const T *)p.k + b * p.k_sb + (int64_t)j * p.k_ss + g * p.k_sh;
      const T *vr = (const T *)p.v + b * p.v_sb + (int64_t)j * p.v_ss + g * p.v_sh;
      for (int c = threadIdx.x; c < p.D; c += kWave) ((T *)p.present_k)[pos * p.D + c] = kr[c];
      for (int c = threadIdx.x; c < p.Dv; c += kWave) ((T *)p.present_v)[pos * p.Dv + c] = vr[c];
    }
  }
}

// Split-KV partial: block (h, b*S + i, split) handles keys
// [split*chunk, (split+1)*chunk) of the row and stores the record
// [m, l, -, -, o[Dv]] (natural-log units, unnormalised; stride Dv + 4 floats).
template <typename T>
__global__ __launch_bounds__(kWave) void generic_split_kernel(Params p, int chunk, int n_split,
                                                              float *ws) {
  __shared__ float qs[256];
  __shared__ float ps[kWave];
  const int split = blockIdx.z, h = blockIdx.x;  // split-major (slowest)
  const int b = blockIdx.y / p.S, i = blockIdx.y % p.S;
  const Seq s = seq_info(p, b);
  load_q<T>(p, b, h, i, qs);
  int lo, hi;
  key_range(p, s, i, lo, hi);
  const int c_lo = max(lo, split * chunk), c_hi = min(hi, (split + 1) * chunk);
  RowState st{kNegInf, 0.f, {0.f, 0.f, 0.f, 0.f}};
  if (c_lo < c_hi) row_range<T>(p, s, b, h, i, c_lo, c_hi, qs, ps, st);
  const int64_t row = ((int64_t)b * p.S + i) * p.Hq + h;
  float *out = ws + (row * n_split + split) * (int64_t)(p.Dv + 4);
  if (threadIdx.x == 0) {
    out[0] = st.m;
    out[1] = st.l;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = threadIdx.x + k * kWave;
    if (d < p.Dv) out[4 + d] = st.o[k];
  }
}

// Merge of the split partials of one row, with the sink in the denominator:
// M = max(max_s m_s, z); Y = sum_s e^{m_s-M} o_s / (sum_s e^{m_s-M} l_s + e^{z-M}).
// Lanes first take one split each (max, then one exponential per split into
// LDS), then one dimension each, summing the weighted records.
constexpr int kMaxSplits = 4096;

template <typename T>
__global__ __launch_bounds__(kWave) void combine_kernel(Params p, int n_split, int split_keys,
                                                        const float *ws) {
  __shared__ float wgt[kMaxSplits];
  const int h = blockIdx.x;
  const int b = blockIdx.y / p.S, i = blockIdx.y % p.S;
  const int lane = threadIdx.x;
  const int64_t row = ((int64_t)b * p.S + i) * p.Hq + h;
  const int64_t rec = p.Dv + 4;
  const float *part = ws + row * n_split * rec;
  // The first record maxima are loaded before the lengths, so the two loads'
  // latencies overlap (records of splits the decode kernels skipped hold
  // stale values, read but never used).
  const float m_first = lane < n_split ? part[lane * rec] : kNegInf;
  // Few splits of short records: every load the merge needs (this lane's
  // split length, its two dimensions of every split's record) goes out now,
  // beside the maxima, so the merge waits for memory once; the sums below
  // keep the order of the general path.
  constexpr int kFewSplits = 16;
  const bool few = n_split <= kFewSplits && p.Dv <= 2 * kWave;
  float l_first = 0.f, ov[kFewSplits][2];
  if (few) {
    l_first = lane < n_split ? part[lane * rec + 1] : 0.f;
#pragma unroll
    for (int sp = 0; sp < kFewSplits; ++sp)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int d = lane + k * kWave;
        ov[sp][k] = sp < n_split && d < p.Dv ? part[sp * rec + 4 + d] : 0.f;
      }
  }
  // Only the splits that hold keys of this row's range [lo, hi) are used:
  // every partial kernel writes the records of those (a split outside the
  // range contributes nothing, and the decode kernels write no record there).
  const Seq s = seq_info(p, b);
  const int pos = s.qoff + i;
  int hi = p.pad_add ? s.total : s.valid;
  if (p.causal) hi = min(hi, pos + 1);
  const int lo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
  const int sp0 = lo / split_keys;
  const int sp1 = hi > lo ? min(n_split, (hi + split_keys - 1) / split_keys) : sp0;
  float M = lane >= sp0 && lane < sp1 ? m_first : kNegInf;
  for (int sp = kWave + lane; sp < sp1; sp += kWave)
    if (sp >= sp0) M = fmaxf(M, part[sp * rec]);
  M = wave_max(M);
  T *yr = (T *)p.y + b * p.y_sb + (int64_t)i * p.y_ss + h * p.y_sh;
  if (M == kNegInf) {  // no allowed key: zeros
    for (int d = lane; d < p.Dv; d += kWave) yr[d] = from_f32<T>(0.f);
    return;
  }
  float z = kNegInf;
  if (p.sink) z = to_f32(((const T *)p.sink)[h]);
  const float Mf = fmaxf(M, z);
  if (few) {
    const bool use = lane >= sp0 && lane < sp1;
    const float w = use && m_first != kNegInf ? expf(m_first - Mf) : 0.f;
    // (the general path's lane sp - sp0 holds split sp's term: the same
    // lanes here, so the wave sum adds in the same order)
    float l = wave_sum(__shfl(use ? w * l_first : 0.f, (lane + sp0) & (kWave - 1), kWave));
    if (p.sink) l += expf(z - Mf);
    const float inv = 1.f / l;
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < kFewSplits; ++sp) {
      if (sp < sp0 || sp >= sp1) continue;
      const float ws_ = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sp));
#pragma unroll
      for (int k = 0; k < 2; ++k) acc[k] += ws_ * ov[sp][k];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int d = lane + k * kWave;
      if (d < p.Dv) yr[d] = from_f32<T>(acc[k] * inv);
    }
    return;
  }
  float l = 0.f;
  for (int sp = sp0 + lane; sp < sp1; sp += kWave) {
    const float m = part[sp * rec];
    const float w = m == kNegInf ? 0.f : expf(m - Mf);
    wgt[sp] = w;
    l += w * part[sp * rec + 1];
  }
  l = wave_sum(l);
  if (p.sink) l += expf(z - Mf);
  __syncthreads();
  const float inv = 1.f / l;
  for (int d = lane; d < p.Dv; d += kWave) {
    float acc = 0.f;
#pragma unroll 8
    for (int sp = sp0; sp < sp1; ++sp) acc += wgt[sp] * part[sp * rec + 4 + d];
    yr[d] = from_f32<T>(acc * inv);
  }
}

// qk_matmul_output of ai.onnx Attention (onnx-light reference kernels header
// page, "class Attention": qk_matmul_output_mode 0 raw (Q K^T) * scale, 1 with
// the bias, 2 after softcap, 3 after softmax; Result: rank-4 FLOAT
// (B, Hq, S, T)).  One wavefront per (b, h, i) row, lanes over keys.  The bias
// of modes 1-3 is attn_bias plus the masks derived from is_causal, BOOL
// attn_mask, nonpad_kv_seqlen and short-mask padding: excluded keys read -inf
// in modes 1 and 2 and 0 in mode 3; mode 0 covers every key.
template <typename T>
__global__ __launch_bounds__(kWave) void qk_kernel(Params p) {
  __shared__ float qs[256];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const Seq s = seq_info(p, b);
  load_q<T>(p, b, h, i, qs);
  const int g = h / p.G, pos = s.qoff + i;
  int lo, hi;
  key_range(p, s, i, lo, hi);
  // score of key j at the output stage (modes 0-2; mode 3 uses stage 2)
  auto score = [&](int j, bool &ok) {
    const T *kr = kv_row<T>(p, s, b, g, j, false);
    float dot = 0.f;
    for (int c = 0; c < p.D; ++c) dot = fmaf(qs[c], to_f32(kr[c]), dot);
    float sc = dot * p.scale;
    ok = j >= lo && j < hi;
    if (p.causal && j > pos) ok = false;
    if (p.mask_kind == 1 && !mask_at(p, b, h, i, j)) ok = false;
    if (p.qk_mode == 0) return sc;
    if (!ok) return kNegInf;
    if (p.bias)
      sc += to_f32(((const T *)p.bias)[b * p.bias_sb + h * p.bias_sh + (int64_t)i * p.bias_si + j]);
    if (p.qk_mode >= 2 && p.softcap > 0.f) sc = p.softcap * tanhf(sc / p.softcap);
    return sc;
  };
  float *out = p.qk_out + (((int64_t)b * p.Hq + h) * p.S + i) * p.T;
  if (p.qk_mode < 3) {
    for (int j = lane; j < p.T; j += kWave) {
      bool ok;
      out[j] = score(j, ok);
    }
    return;
  }
  float m = kNegInf;
  for (int j = lane; j < p.T; j += kWave) {
    bool ok;
    const float v = score(j, ok);
    if (ok) m = fmaxf(m, v);
  }
  m = wave_max(m);
  float l = 0.f;
  for (int j = lane; j < p.T; j += kWave) {
    bool ok;
    const float v = score(j, ok);
    if (ok) l += expf(v - m);
  }
  l = wave_sum(l);
  for (int j = lane; j < p.T; j += kWave) {
    bool ok;
    const float v = score(j, ok);
    out[j] = (ok && m != kNegInf) ? expf(v - m) / l : 0.f;
  }
}

}  // namespace

hipError_t launch_qk(const Params &p, int dtype, hipStream_t st) {
  if (p.B == 0 || p.S == 0 || p.Hq == 0 || p.T == 0) return hipSuccess;
  dim3 grid(p.S, p.Hq, p.B);
  if (dtype == DT_F32) hipLaunchKernelGGL(qk_kernel<float>, grid, dim3(kWave), 0, st, p);
  else if (dtype == DT_F16) hipLaunchKernelGGL(qk_kernel<f16>, grid, dim3(kWave), 0, st, p);
  else hipLaunchKernelGGL(qk_kernel<bf16>, grid, dim3(kWave), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_generic(const Params &p, int dtype, hipStream_t st) {
  if (p.B == 0 || p.S == 0 || p.Hq == 0) return hipSuccess;
  dim3 grid(p.S, p.Hq, p.B);
  if (dtype == DT_F32) hipLaunchKernelGGL(generic_kernel<float>, grid, dim3(kWave), 0, st, p);
  else if (dtype == DT_F16) hipLaunchKernelGGL(generic_kernel<f16>, grid, dim3(kWave), 0, st, p);
  else hipLaunchKernelGGL(generic_kernel<bf16>, grid, dim3(kWave), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_generic_split(const Params &p, int dtype, int chunk, int n_split, float *ws,
                                hipStream_t st) {
  if (p.B == 0 || p.S == 0 || p.Hq == 0) return hipSuccess;
  dim3 grid(p.Hq, p.B * p.S, n_split);
  if (dtype == DT_F32)
    hipLaunchKernelGGL(generic_split_kernel<float>, grid, dim3(kWave), 0, st, p, chunk, n_split, ws);
  else if (dtype == DT_F16)
    hipLaunchKernelGGL(generic_split_kernel<f16>, grid, dim3(kWave), 0, st, p, chunk, n_split, ws);
  else
    hipLaunchKernelGGL(generic_split_kernel<bf16>, grid, dim3(kWave), 0, st, p, chunk, n_split, ws);
  return hipGetLastError();
}

hipError_t launch_combine(const Params &p, int dtype, int n_split, int split_keys,
                          const float *ws, hipStream_t st) {
  if (p.B == 0 || p.S == 0 || p.Hq == 0) return hipSuccess;
  if (split_keys <= 0 || n_split > kMaxSplits) return hipErrorInvalidValue;
  dim3 grid(p.Hq, p.B * p.S);
  if (dtype == DT_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(kWave), 0, st, p, n_split, split_keys, ws);
  else if (dtype == DT_F16)
    hipLaunchKernelGGL(combine_kernel<f16>, grid, dim3(kWave), 0, st, p, n_split, split_keys, ws);
  else
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, dim3(kWave), 0, st, p, n_split, split_keys, ws);
  return hipGetLastError();
}

}  // namespace olk
