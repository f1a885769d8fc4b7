// MFMA tiled attention forward for gfx950 (CDNA4): f16/bf16 inputs, head size
// 64 or 128, fp32 accumulation.
//
// What is computed is Y = Softmax((Q K^T) * scale + bias) V with the grouped
// KV heads, causal / local-window / length masks, softcap and head_sink of the
// GroupQueryAttention, MultiHeadAttention and ai.onnx Attention contracts
// (onnx-light-cpu Python API "Custom operators"; onnx-light reference kernels
// header page, "class Attention").  The decomposition below is ours.
//
// Work split.  A workgroup = 4 wavefronts = 128 "row slots".  Row slots pack
// the GH query heads of one KV head with consecutive queries:
// slot r -> (query i0 + r / GH, head g*G + hg*GH + r % GH).  Every K/V tile
// staged in LDS therefore serves all heads of the group.  Keys advance in
// tiles of 64.
//
// Per tile and wavefront (32 row slots):
//   S^T (64 keys x 32 slots) = K Q^T   v_mfma_f32_32x32x16: A = K rows from LDS,
//                                       B = Q^T held in VGPRs for the whole loop.
//   In the S^T accumulator layout each lane owns one row slot (lane % 32) and
//   32 of its 64 keys, so max/sum are in-lane plus one exchange with lane^32.
//   Online softmax in the exp2 domain, rescaling O only when the running max
//   grows by more than 2^8 (the final division uses the same stale max, so the
//   result is unchanged).
//   O^T (D x 32 slots) += V^T P^T        A = V^T read from the row-major V tile
//   with ds_read_b64_tr_b16 (4 consecutive keys of one column per lane),
//   B = P^T straight from the S^T registers (rounded to the input type).
// K/V tiles are double-buffered in LDS (one barrier per tile); the next tile's
// global loads are issued before the current tile's MFMAs.
#include "olk_internal.h"

namespace olk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct V8;
template <> struct V8<bf16> { typedef bf16x8 t; typedef bf16x4 h; };
template <> struct V8<f16> { typedef f16x8 t; typedef f16x4 h; };

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kThreads = 256;
constexpr int kRows = 128;  // row slots per workgroup
constexpr int kBN = 64;     // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescale = 8.0f;  // lazy-rescale threshold (log2 units)

struct Plan {
  int GH;        // query heads per workgroup (divides G)
  int n_hg;      // head groups per KV head = G / GH
  int QW;        // queries per workgroup = kRows / GH
  int n_qt;      // query tiles = ceil(S / QW)
  int n_split;   // key splits
  int split_tiles;  // key tiles per split
  int xcd_remap;    // 1: place the workgroups of one (b, g) on one XCD
  int bias_vec;     // 1: bias rows are 8-byte aligned (T % 4 == 0)
  float *ws;        // split partials [m, l, -, -, O[Dv]] per (row, split)
};

// 4-byte element pair helpers
template <typename T> __device__ __forceinline__ float lo_f(uint32_t w);
template <> __device__ __forceinline__ float lo_f<bf16>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float lo_f<f16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffff));
}
template <typename T> __device__ __forceinline__ float hi_f(uint32_t w);
template <> __device__ __forceinline__ float hi_f<bf16>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <> __device__ __forceinline__ float hi_f<f16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its exponential form, tanh x = 1 - 2 / (e^{2x} + 1): saturates
// cleanly at both ends; absolute error is a few fp32 ulps of 1.
__device__ __forceinline__ float tanh_fast(float x) {
  const float e = fast_exp2(x * (2.0f * kLog2e));
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

template <typename T, int D, bool BIAS, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void tiled_kernel(Params p, Plan pl) {
  typedef typename V8<T>::t vec8;
  constexpr int KST = D + 8;      // LDS row stride (elements): 16-byte pad
  constexpr int NKS = D / 16;     // k-steps of the QK^T contraction
  constexpr int NDB = D / 32;     // 32-wide output blocks
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int LPT = kBN * CH / kThreads;  // 16-byte loads per thread per tile (K or V)
  __shared__ __attribute__((aligned(16))) T lds[2][2][kBN * KST];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  // ---- workgroup -> (split, q tile, b, g, hg) ----
  const int n_bg = p.B * p.Hkv * pl.n_hg;
  // split-major: the split is the slowest index, so the ids within one split
  // keep the XCD round-robin that the remap below assumes
  const int per_split = n_bg * pl.n_qt;
  const int split = blockIdx.x / per_split;
  int wid = blockIdx.x % per_split;
  int bg, qrank;
  if (pl.xcd_remap) {  // consecutive ids go round-robin over the 8 XCDs
    const int per = n_bg / 8;
    const int xcd = wid & 7, k = wid >> 3;
    qrank = k / per;
    bg = (k % per) * 8 + xcd;
  } else {
    qrank = wid / n_bg;
    bg = wid % n_bg;
  }
  const int qt = pl.n_qt - 1 - qrank;  // heaviest (latest) query tiles first
  const int hg = bg % pl.n_hg;
  const int g = (bg / pl.n_hg) % p.Hkv;
  const int b = bg / (pl.n_hg * p.Hkv);
  const Seq s = seq_info(p, b);
  const int i0 = qt * pl.QW;
  const int i_last = min(i0 + pl.QW, p.S) - 1;

  // ---- key range of the workgroup ----
  const int pos_min = s.qoff + i0, pos_max = s.qoff + i_last;
  int hi = p.pad_add ? s.total : s.valid;
  if (p.causal) hi = min(hi, pos_max + 1);
  if (BIAS) hi = min(hi, p.bias_cols);  // a short mask excludes the keys beyond it
  int lo = 0;
  if (p.window > 0) lo = max(0, pos_min - p.window + 1);
  int kt0 = lo / kBN, kt1 = (hi + kBN - 1) / kBN;
  kt0 = max(kt0, split * pl.split_tiles);
  kt1 = min(kt1, (split + 1) * pl.split_tiles);

  // ---- this lane's row slot ----
  const int slot = wave * 32 + col;
  const int iq = slot / pl.GH;
  const int i = i0 + iq;
  const int h = g * p.G + hg * pl.GH + slot % pl.GH;
  const bool row_ok = i < p.S;
  const int pos = s.qoff + i;
  // waves whose 32 slots all lie beyond the last query only help with loads
  const bool wave_active = i0 + (wave * 32) / pl.GH < p.S;

  // ---- Q^T operand (B of S^T = K Q^T): lane holds slot `col`, d = 16ks + 8half + e ----
  vec8 qreg[NKS];
  {
    const T *qr = (const T *)p.q + b * p.q_sb + (int64_t)(row_ok ? i : 0) * p.q_ss + h * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int d0 = ks * 16 + half * 8;
      if (row_ok) {
        uint4 raw = *(const uint4 *)(qr + d0);
        if (p.proj_bias) {
          const uint4 braw = *(const uint4 *)((const T *)p.proj_bias + h * D + d0);
          const uint32_t *w = (const uint32_t *)&raw;
          const uint32_t *bw = (const uint32_t *)&braw;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qreg[ks][2 * e] = (T)(lo_f<T>(w[e]) + lo_f<T>(bw[e]));
            qreg[ks][2 * e + 1] = (T)(hi_f<T>(w[e]) + hi_f<T>(bw[e]));
          }
        } else {
          qreg[ks] = __builtin_bit_cast(vec8, raw);
        }
      } else {
        qreg[ks] = __builtin_bit_cast(vec8, make_uint4(0, 0, 0, 0));
      }
    }
  }

  // ---- K/V tile loader: thread covers rows (tid / CH) + u * (256 / CH), chunk tid % CH ----
  const int ld_row = tid / CH, ld_chunk = tid % CH;
  constexpr int ROW_STEP = kThreads / CH;
  const T *kpast = (const T *)p.past_k + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *vpast = (const T *)p.past_v + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *knew = (const T *)p.k + b * p.k_sb + g * p.k_sh;
  const T *vnew = (const T *)p.v + b * p.v_sb + g * p.v_sh;
  uint4 kbuf[LPT], vbuf[LPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int j = kt * kBN + ld_row + u * ROW_STEP;
      const int c = ld_chunk * 8;
      if (j >= lo && j < hi) {
        if (j < s.src) {
          kbuf[u] = *(const uint4 *)(kpast + (int64_t)j * D + c);
          vbuf[u] = *(const uint4 *)(vpast + (int64_t)j * D + c);
        } else {
          kbuf[u] = *(const uint4 *)(knew + (int64_t)(j - s.src) * p.k_ss + c);
          vbuf[u] = *(const uint4 *)(vnew + (int64_t)(j - s.src) * p.v_ss + c);
        }
      } else {  // outside the workgroup's key range: zeros (never NaN garbage)
        kbuf[u] = make_uint4(0, 0, 0, 0);
        vbuf[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int r = ld_row + u * ROW_STEP;
      *(uint4 *)&lds[buf][0][r * KST + ld_chunk * 8] = kbuf[u];
      *(uint4 *)&lds[buf][1][r * KST + ld_chunk * 8] = vbuf[u];
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = kNegInf, l = 0.f;

  const float scale_log2 = p.scale * kLog2e;
  const float inv_cap = SOFTCAP ? 1.0f / p.softcap : 0.f;
  const float cap_log2 = p.softcap * kLog2e;
  const float mfv_log2 = p.mfv * kLog2e;
  const T *bias_row = nullptr;
  if (BIAS) bias_row = (const T *)p.bias + b * p.bias_sb + h * p.bias_sh + (int64_t)(row_ok ? i : 0) * p.bias_si;

  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) load_tile(kt + 1);
    const T *Kl = lds[buf][0];
    const T *Vl = lds[buf][1];
    const int j0 = kt * kBN;
    if (!wave_active) {
      if (more) store_tile(buf ^ 1);
      __syncthreads();
      continue;
    }

    // S^T = K Q^T: two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const vec8 a = *(const vec8 *)&Kl[(kb * 32 + col) * KST + ks * 16 + half * 8];
        sacc[kb] = mfma32(a, qreg[ks], sacc[kb]);
      }
    }

    // score epilogue: scale, bias, softcap, masks (log2 domain)
    const bool need_mask = (p.causal && j0 + kBN - 1 > pos_min) ||
                           (p.window > 0 && j0 < pos_max - p.window + 1) ||
                           (j0 + kBN > hi) || (p.pad_add && j0 + kBN > s.pad) || (j0 < lo);
    if (!SOFTCAP && !BIAS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] *= scale_log2;
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int jb = j0 + kb * 32 + 8 * q4 + 4 * half;  // 4 consecutive keys
          float bv[4] = {0.f, 0.f, 0.f, 0.f};
          if (BIAS) {
            if (pl.bias_vec && jb + 3 < p.bias_cols) {
              const uint2 raw = *(const uint2 *)(bias_row + jb);
              bv[0] = lo_f<T>(raw.x); bv[1] = hi_f<T>(raw.x);
              bv[2] = lo_f<T>(raw.y); bv[3] = hi_f<T>(raw.y);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                bv[e] = jb + e < p.bias_cols ? (float)bias_row[jb + e] : 0.f;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float u = sacc[kb][4 * q4 + e] * p.scale + bv[e];
            sacc[kb][4 * q4 + e] = SOFTCAP ? cap_log2 * tanh_fast(u * inv_cap) : u * kLog2e;
          }
        }
      }
    }
    float mx = kNegInf;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          float t = sacc[kb][r];
          if (p.pad_add && j >= s.pad) t += mfv_log2;
          bool ok = j >= lo && j < hi;
          if (p.causal && j > pos) ok = false;
          if (p.window > 0 && j < pos - p.window + 1) ok = false;
          sacc[kb][r] = ok ? t : kNegInf;
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

    // lazy online-softmax rescale
    const float m_new = fmaxf(m, mx);
    const bool grow = m_new > m + kRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(m - m_new) : 1.0f;
      m = grow ? m_new : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    const float m_use = m == kNegInf ? 0.f : m;

    // P = exp2(t - m), row sums, pack P^T operands (16 keys per MFMA step)
    vec8 pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = fast_exp2(sacc[st >> 1][8 * (st & 1) + e] - m_use);
        lsum += pv;
        pb[st][e] = (T)pv;
      }
    }
    l += lsum;

    // O^T += V^T P^T; V^T operand via transposed LDS reads
    const int grp = lane >> 4, tl = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int row = st * 16 + 4 * (grp >> 1) + (tl >> 2);
        const int cc = db * 32 + 16 * (grp & 1) + 4 * (tl & 3);
        typedef s16x4 __attribute__((address_space(3))) * lds4;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4)(&Vl[row * KST + cc]));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4)(&Vl[(row + 8) * KST + cc]));
        const s16x8 a8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = mfma32(__builtin_bit_cast(vec8, a8), pb[st], o[db]);
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = l + __shfl_xor(l, 32, 64);
  if (!row_ok) return;
  const int64_t yrow_idx = ((int64_t)b * p.S + i) * p.Hq + h;
  // unnormalised partial in natural-log units: (m, l, O), combined later
  float *out = pl.ws + (yrow_idx * pl.n_split + split) * (int64_t)(D + 4);
  if (half == 0) {
    out[0] = m == kNegInf ? kNegInf : m * kLn2;
    out[1] = m == kNegInf ? 0.f : l_tot;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = db * 32 + 8 * q4 + 4 * half;
      float4 v4 = make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      if (m == kNegInf) v4 = make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4 *)&out[4 + d] = v4;
    }
}

int heads_per_wg(int G) {
  for (int gh = 32; gh >= 1; gh >>= 1)
    if (G % gh == 0) return gh;
  return 1;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15) == 0; }

Plan make_plan(const Params &p, int n_split, int split_tiles, float *ws) {
  Plan pl;
  pl.GH = heads_per_wg(p.G);
  pl.n_hg = p.G / pl.GH;
  pl.QW = kRows / pl.GH;
  pl.n_qt = (p.S + pl.QW - 1) / pl.QW;
  pl.n_split = n_split;
  pl.split_tiles = split_tiles;
  const int n_bg = p.B * p.Hkv * pl.n_hg;
  pl.xcd_remap = (n_bg % 8 == 0) ? 1 : 0;
  pl.bias_vec = (p.bias_si % 4 == 0 && p.bias_sh % 4 == 0 && p.bias_sb % 4 == 0 &&
                 ((uintptr_t)p.bias & 7) == 0) ? 1 : 0;
  pl.ws = ws;
  return pl;
}

template <typename T, int D>
hipError_t launch_typed(const Params &p, const Plan &pl, hipStream_t st) {
  const int64_t n = (int64_t)p.B * p.Hkv * pl.n_hg * pl.n_qt * pl.n_split;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(kThreads);
  const bool bias = p.bias != nullptr, cap = p.softcap > 0.f;
  if (bias && cap) hipLaunchKernelGGL((tiled_kernel<T, D, true, true>), grid, block, 0, st, p, pl);
  else if (bias) hipLaunchKernelGGL((tiled_kernel<T, D, true, false>), grid, block, 0, st, p, pl);
  else if (cap) hipLaunchKernelGGL((tiled_kernel<T, D, false, true>), grid, block, 0, st, p, pl);
  else hipLaunchKernelGGL((tiled_kernel<T, D, false, false>), grid, block, 0, st, p, pl);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const Params &p, const Plan &pl, hipStream_t st) {
  return p.D == 64 ? launch_typed<T, 64>(p, pl, st) : launch_typed<T, 128>(p, pl, st);
}

hipError_t launch_plan(const Params &p, int dtype, const Plan &pl, hipStream_t st) {
  return dtype == DT_BF16 ? launch_dtype<bf16>(p, pl, st) : launch_dtype<f16>(p, pl, st);
}

}  // namespace

// The matrix-core prefill kernel (head size 64, 128 or 256) and, at head size
// 64 or 128, the tiled split partials (launch_tiled_split refuses 256).
bool tiled_supports(const Params &p, int dtype) {
  if (dtype != DT_F16 && dtype != DT_BF16) return false;
  if (p.D != p.Dv || (p.D != 64 && p.D != 128 && p.D != 256)) return false;
  // attn_mask (BOOL, and MultiHeadAttention's int32 binary mask) runs in the
  // prefill kernel's mask path and the decode kernels (not in the tiled split
  // partials); the qk output is a separate launch after the attention
  if (!aligned16(p.q) || !aligned16(p.k) || !aligned16(p.v) || !aligned16(p.y)) return false;
  if (p.P > 0 && (!aligned16(p.past_k) || !aligned16(p.past_v))) return false;
  if (p.proj_bias && !aligned16(p.proj_bias)) return false;
  // without bias or softcap the prefill kernel folds a positive scale into exp2
  if (!(p.scale > 0.f) && !p.bias && !p.mask && !(p.softcap > 0.f)) return false;
  return true;
}

int tiled_split_count(const Params &p, int split_tiles) {
  const int tiles = (p.T + kBN - 1) / kBN;
  return max(1, (tiles + split_tiles - 1) / split_tiles);
}

hipError_t launch_tiled_split(const Params &p, int dtype, int split_tiles, float *ws,
                              hipStream_t st) {
  if (p.D != 64 && p.D != 128) return hipErrorInvalidValue;
  const int n_split = tiled_split_count(p, split_tiles);
  return launch_plan(p, dtype, make_plan(p, n_split, split_tiles, ws), st);
}

}  // namespace olk
