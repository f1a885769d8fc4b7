// present_key / present_value writer (onnx-light-cpu Python API page "Custom
// operators": GroupQueryAttention present outputs hold the entire past cache
// followed by the current step; MultiHeadAttention present has P+L positions;
// onnx-light reference kernels header page, "class Attention" Result: present
// equals K/V or their concatenation with the past).
//
// Pure copies: position j < total_b of (b, g) takes row j of the past buffer
// when j < past_b, else row j - past_b of the new K/V.  Bits are copied, never
// converted.  Positions at or beyond total_b are not touched.  In kv_inplace
// mode the past rows are already in place and only the new rows are written.
#include "olk_internal.h"

namespace olk {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 16;

// Copies rows of (g = blockIdx.y, b = blockIdx.z) for both K (which = 0) and
// V (which = 1) in units of U (4 or 2 bytes).  Row r of the launch is key
// position j = first + r, where `first` is 0, or past_b when only the new
// rows are written (kv_inplace); the launch covers no more rows than the mode
// can write, so a KV-cache append costs one row per (b, g), not a cache scan.
template <typename U>
__global__ __launch_bounds__(kThreads) void present_kernel(Params p, int esize, int new_only) {
  const int g = blockIdx.y, b = blockIdx.z;
  const Seq s = seq_info(p, b);
  const int first = new_only ? s.past : 0;
  const int j0 = first + blockIdx.x * kRowsPerBlock;
  for (int which = 0; which < 2; ++which) {
    char *dst_base = (char *)(which ? p.present_v : p.present_k);
    if (!dst_base) continue;
    const int width = which ? p.Dv : p.D;
    const int row_words = width * esize / (int)sizeof(U);
    const char *past = (const char *)(which ? p.past_v : p.past_k);
    const char *cur = (const char *)(which ? p.v : p.k);
    const int64_t sb = which ? p.v_sb : p.k_sb, ss = which ? p.v_ss : p.k_ss,
                  sh = which ? p.v_sh : p.k_sh;
    const int n = kRowsPerBlock * row_words;
    for (int t = threadIdx.x; t < n; t += kThreads) {
      const int j = j0 + t / row_words, w = t % row_words;
      if (j >= s.total || j >= p.T) continue;
      if (p.kv_inplace && j < s.past) continue;
      if (p.present_past_only && j >= s.past) continue;
      const char *src;
      if (j < s.past) src = past + ((((int64_t)b * p.Hkv + g) * p.past_rows + j) * width) * esize;
      else src = cur + (b * sb + (int64_t)(j - s.past) * ss + g * sh) * esize;
      char *dst = dst_base + ((((int64_t)b * p.Hkv + g) * p.T + j) * width) * esize;
      ((U *)dst)[w] = ((const U *)src)[w];
    }
  }
}

// MultiHeadAttention with rank-3 K/V and a projection bias: new row i of
// (b = blockIdx.z, g = blockIdx.y) gets its k / v bias segment added (float32
// add, rounded once to the element type) and lands in present at P + i; the
// attention kernels then read every key from present.
template <typename T>
__global__ __launch_bounds__(kThreads) void kv_bias_kernel(Params p) {
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int j = p.P + i;
  const T *bias = (const T *)p.proj_bias;
  for (int t = threadIdx.x; t < p.D + p.Dv; t += kThreads) {
    const bool value = t >= p.D;
    const int c = value ? t - p.D : t;
    const int width = value ? p.Dv : p.D;
    const T *src = (const T *)(value ? p.v : p.k) + b * (value ? p.v_sb : p.k_sb) +
                   (int64_t)i * (value ? p.v_ss : p.k_ss) + (int64_t)g * (value ? p.v_sh : p.k_sh);
    const int64_t seg = value ? (int64_t)2 * p.Hq * p.D + (int64_t)g * p.Dv
                              : (int64_t)p.Hq * p.D + (int64_t)g * p.D;
    T *dst = (T *)(value ? p.present_v : p.present_k) + (((int64_t)b * p.Hkv + g) * p.T + j) * width;
    dst[c] = (T)((float)src[c] + (float)bias[seg + c]);
  }
}

}  // namespace

hipError_t launch_kv_bias(const Params &p, int dtype, hipStream_t st) {
  if (p.B == 0 || p.L == 0 || p.Hkv == 0) return hipSuccess;
  const dim3 grid(p.L, p.Hkv, p.B);
  if (dtype == DT_BF16) hipLaunchKernelGGL(kv_bias_kernel<bf16>, grid, dim3(kThreads), 0, st, p);
  else if (dtype == DT_F16) hipLaunchKernelGGL(kv_bias_kernel<f16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(kv_bias_kernel<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_present(const Params &p, int dtype, hipStream_t st) {
  if ((!p.present_k && !p.present_v) || p.B == 0 || p.T == 0) return hipSuccess;
  // nothing left to copy: the past is already in place and the new rows are
  // written by the attention kernel
  if (p.present_past_only && (p.kv_inplace || p.P == 0)) return hipSuccess;
  const int esize = dtype == DT_F32 ? 4 : 2;
  // rows the launch must cover: the new keys only when the past is in place
  const int new_only = p.kv_inplace ? 1 : 0;
  const int rows = new_only ? p.L : (p.present_past_only ? p.P : p.T);
  if (rows == 0) return hipSuccess;
  dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock, p.Hkv, p.B);
  if ((p.D * esize) % 4 == 0 && (p.Dv * esize) % 4 == 0)
    hipLaunchKernelGGL(present_kernel<uint32_t>, grid, dim3(kThreads), 0, st, p, esize, new_only);
  else
    hipLaunchKernelGGL(present_kernel<uint16_t>, grid, dim3(kThreads), 0, st, p, esize, new_only);
  return hipGetLastError();
}

}  // namespace olk
