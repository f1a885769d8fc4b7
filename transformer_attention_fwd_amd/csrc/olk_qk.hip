// qk_matmul_output of ai.onnx Attention on the matrix cores (gfx950): f16/bf16
// inputs, head size 64, 128 or 256, float32 output (B, Hq, S, T).
//
// What is written follows the onnx-light reference kernels header page,
// "class Attention" (qk_matmul_output_mode 0: (Q K^T) * scale for every key;
// 1: with the bias; 2: after softcap; 3: after softmax).  The bias of modes
// 1-3 is attn_bias plus the masks that is_causal, a BOOL attn_mask,
// nonpad_kv_seqlen and short-mask padding stand for: excluded keys read -inf
// in modes 1 and 2 and 0 in mode 3.  The decomposition is ours:
//
// * A workgroup is 4 wavefronts x 32 query rows of one head; the key axis is
//   walked in tiles of 64.  S^T = K Q^T on v_mfma_f32_32x32x16 with Q^T held
//   in VGPRs (B operand) and each wavefront reading its K operand (A: key row
//   l % 32, 8 dims at 8 (l / 32)) straight from memory, 16 bytes per lane;
//   the four wavefronts of a workgroup read the same rows, so all but the
//   first read hit the caches.
// * In the S^T accumulator a lane holds one query row and 4 consecutive keys
//   per register quad, which it stores as one 16-byte write (rows of T floats,
//   T a multiple of 4; single floats otherwise and at the row's end).
// * Mode 3 walks the keys twice: the first pass keeps the row's running max
//   and sum (exp2 domain, rescaled as the max grows), the second writes
//   2^(s - m) / l.
#include "olk_internal.h"

namespace olk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct QV;
template <> struct QV<bf16> { typedef bf16x8 v8; };
template <> struct QV<f16> { typedef f16x8 v8; };

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kThreads = 256;
constexpr int kRows = 128;  // query rows per workgroup (4 wavefronts x 32)
constexpr int kBN = 64;     // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void qk_mfma_kernel(Params p, int n_qt) {
  typedef typename QV<T>::v8 vec8;
  constexpr int NKS = D / 16;  // k-steps of the contraction
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int qt = blockIdx.x % n_qt;
  const int h = (blockIdx.x / n_qt) % p.Hq;
  const int b = blockIdx.x / (n_qt * p.Hq);
  const int g = h / p.G;
  const Seq s = seq_info(p, b);
  const int i = qt * kRows + wave * 32 + col;  // this lane's query row
  const bool row_ok = i < p.S;
  const int ic = row_ok ? i : 0;
  if (qt * kRows + wave * 32 >= p.S) return;  // no row of this wavefront (no barriers below)

  // Q^T operand: row i, dims 16 ks + 8 half + e
  vec8 qreg[NKS];
  {
    const T *qr = (const T *)p.q + b * p.q_sb + (int64_t)ic * p.q_ss + h * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[ks] = *(const vec8 *)(qr + ks * 16 + half * 8);
  }
  // allowed keys of row i: [0, hi) cut by causal, the nonpad length and the
  // short-bias / BOOL-mask columns, then the BOOL mask itself per key
  const int pos = s.qoff + ic;
  int hi = s.valid;
  if (p.causal) hi = min(hi, pos + 1);
  if (p.bias) hi = min(hi, p.bias_cols);
  const T *bias_row = p.bias ? (const T *)p.bias + b * p.bias_sb + h * p.bias_sh + (int64_t)ic * p.bias_si
                             : nullptr;
  const float cap_in = p.softcap > 0.f ? 2.0f * kLog2e / p.softcap : 0.f;
  const T *kpast = (const T *)p.past_k + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *knew = (const T *)p.k + b * p.k_sb + g * p.k_sh;
  float *out = p.qk_out + (((int64_t)b * p.Hq + h) * p.S + ic) * p.T;
  const bool vec_store = (p.T & 3) == 0;

  // S^T of tile kt for this wavefront's rows: key j0 + 32 kb + 8 (r / 4) + 4 half + r % 4
  auto scores = [&](int kt, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // A operand row: key j (clamped into [0, T): rows past T are not stored)
      const int j = min(kt * kBN + kb * 32 + col, p.T - 1);
      const T *kr = j < s.src ? kpast + (int64_t)j * D : knew + (int64_t)(j - s.src) * p.k_ss;
      vec8 a[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) a[ks] = *(const vec8 *)(kr + ks * 16 + half * 8);
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) sacc[kb] = mma(a[ks], qreg[ks], sacc[kb]);
    }
  };
  // the output stage of one score (modes 1-3: log2 units for mode 3), ok
  // cleared for an excluded key
  auto stage = [&](float dot, int j, bool &ok) __attribute__((always_inline)) {
    float sc = dot * p.scale;
    ok = j < hi;
    if (ok && p.mask_kind == 1 && !mask_at(p, b, h, ic, j)) ok = false;
    if (p.qk_mode == 0) return sc;
    if (!ok) return kNegInf;
    if (p.bias) sc += (float)bias_row[j];
    if (p.qk_mode >= 2 && p.softcap > 0.f)
      sc = p.softcap - 2.0f * p.softcap * __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sc * cap_in) + 1.0f);
    return p.qk_mode == 3 ? sc * kLog2e : sc;
  };
  auto store4 = [&](int j, const float (&v)[4]) __attribute__((always_inline)) {
    if (!row_ok) return;
    if (vec_store && j + 4 <= p.T) {
      *(float4 *)(out + j) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < p.T) out[j + e] = v[e];
    }
  };
  const int n_kt = (p.T + kBN - 1) / kBN;

  // mode 3, first pass: running max and sum of the allowed keys
  float m = kNegInf, l = 0.f;
  if (p.qk_mode == 3) {
    for (int kt = 0; kt < n_kt; ++kt) {
      f32x16 sacc[2];
      scores(kt, sacc);
      float t[32], mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kt * kBN + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          bool ok;
          const float v = j < p.T ? stage(sacc[kb][r], j, ok) : kNegInf;
          t[kb * 16 + r] = (j < p.T && ok) ? v : kNegInf;
          mx = fmaxf(mx, t[kb * 16 + r]);
        }
      const float m_new = fmaxf(m, mx);
      if (m_new != kNegInf) {
        float add = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) add += __builtin_amdgcn_exp2f(t[e] - m_new);
        l = l * (m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - m_new)) + add;
        m = m_new;
      }
    }
    // the row's two lane halves hold different keys: combine them
    const float m_o = __shfl_xor(m, 32, 64), l_o = __shfl_xor(l, 32, 64);
    const float M = fmaxf(m, m_o);
    if (M != kNegInf) {
      l = (m == kNegInf ? 0.f : l * __builtin_amdgcn_exp2f(m - M)) +
          (m_o == kNegInf ? 0.f : l_o * __builtin_amdgcn_exp2f(m_o - M));
    }
    m = M;
  }
  const float inv_l = (p.qk_mode == 3 && l > 0.f) ? 1.0f / l : 0.f;

  // every mode: write the row's output over all T keys
  for (int kt = 0; kt < n_kt; ++kt) {
    f32x16 sacc[2];
    scores(kt, sacc);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j4 = kt * kBN + kb * 32 + 8 * q4 + 4 * half;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j4 + e;
          bool ok = false;
          const float x = j < p.T ? stage(sacc[kb][4 * q4 + e], j, ok) : 0.f;
          if (p.qk_mode == 3)
            v[e] = (ok && m != kNegInf) ? __builtin_amdgcn_exp2f(x - m) * inv_l : 0.f;
          else
            v[e] = x;
        }
        store4(j4, v);
      }
  }
}

}  // namespace

// The matrix-core qk output: f16/bf16, head size 64, 128 or 256 (D == Dv not
// needed: V is not read), 16-byte aligned Q and key rows.
bool qk_mfma_supports(const Params &p, int dtype) {
  if (dtype != DT_F16 && dtype != DT_BF16) return false;
  if (p.D != 64 && p.D != 128 && p.D != 256) return false;
  auto al = [](const void *x) { return ((uintptr_t)x & 15) == 0; };
  if (!al(p.q) || !al(p.k) || (p.past_k && !al(p.past_k))) return false;
  const int es = 2;
  if ((p.q_sb * es) % 16 || (p.q_ss * es) % 16 || (p.q_sh * es) % 16) return false;
  if ((p.k_sb * es) % 16 || (p.k_ss * es) % 16 || (p.k_sh * es) % 16) return false;
  return true;
}

hipError_t launch_qk_mfma(const Params &p, int dtype, hipStream_t st) {
  if (p.B == 0 || p.S == 0 || p.Hq == 0 || p.T == 0) return hipSuccess;
  const int n_qt = (p.S + kRows - 1) / kRows;
  const dim3 grid((unsigned)((int64_t)p.B * p.Hq * n_qt)), block(kThreads);
  if (dtype == DT_BF16) {
    if (p.D == 64) hipLaunchKernelGGL((qk_mfma_kernel<bf16, 64>), grid, block, 0, st, p, n_qt);
    else if (p.D == 128) hipLaunchKernelGGL((qk_mfma_kernel<bf16, 128>), grid, block, 0, st, p, n_qt);
    else hipLaunchKernelGGL((qk_mfma_kernel<bf16, 256>), grid, block, 0, st, p, n_qt);
  } else {
    if (p.D == 64) hipLaunchKernelGGL((qk_mfma_kernel<f16, 64>), grid, block, 0, st, p, n_qt);
    else if (p.D == 128) hipLaunchKernelGGL((qk_mfma_kernel<f16, 128>), grid, block, 0, st, p, n_qt);
    else hipLaunchKernelGGL((qk_mfma_kernel<f16, 256>), grid, block, 0, st, p, n_qt);
  }
  return hipGetLastError();
}

}  // namespace olk
