// Backward of the GroupQueryAttention forward without past on the matrix
// cores (gfx950, f16/bf16, head size 64 or 128 for both Q/K and V).  Same
// result as the VALU kernels of olk_backward.hip (onnx-light-cpu C++ API page
// "Custom operators", RegisterCustomOperatorGradients, GroupQueryAttention
// gradient: P recomputed from Q, K, V; dP = dY V^T; delta_i = sum_j P_ij dP_ij;
// dS = P (dP - delta) scale; dQ = dS K, dK = dS^T Q, dV = P^T dY with the
// query heads of one KV head summed into it), fp32 accumulation, one rounding
// of each output to the element type.
//
// Row slots: the G query heads that share KV head g are packed with the
// queries, slot sigma -> (query sigma / G, head g G + sigma % G), so every K/V
// (or Q/dY) tile in LDS serves the whole group.
//
// bwd_dq_mfma: a workgroup is 4 wavefronts x 32 row slots; keys advance in
//   tiles of 32.  In the S^T = K Q^T and dP^T = V dY^T accumulator layout a
//   lane owns one row slot (Q and dY of that slot sit in registers as the B
//   operands).  Pass 1 runs the online log-sum-exp and delta_i = sum_j P dP
//   in the exp2 domain and stores lse2_i = log2 sum_j 2^(s_ij log2 e) and
//   delta_i for the second kernel; pass 2 recomputes P and dS and accumulates
//   dQ^T += K^T dS^T with dS^T as the B operand, one tile behind the scores,
//   with K^T transposed in LDS from the row-major K tile.
// bwd_dkv_mfma: a workgroup owns 128 keys and is 8 wavefronts, two per SIMD.
//   Producers hold K and V of 32 keys in registers as the B operands of
//   S = Q K^T and dP = dY V^T (a lane owns one key), make P and dS for a tile
//   of 32 row slots and hand them over through LDS; consumers (same keys, one
//   tile behind) accumulate dV^T += dY^T P and dK^T += Q^T dS with P and dS as
//   the B operands and dY^T, Q^T transposed in LDS from the row-major tiles.
// Transposed tiles put each 16-row group in the order {0-3, 8-11, 4-7, 12-15},
// the k order in which a lane half supplies an accumulator column as a B
// operand, pad rows by 16 bytes and XOR-swizzle 16-byte chunks by (row / 32);
// row-major tiles pad rows by 16 bytes.  Tiles are double-buffered in LDS with
// one barrier per step; global loads are in flight while earlier tiles compute.
#include "olk_internal.h"

#include <type_traits>

namespace olk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct BV;
template <> struct BV<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct BV<f16> { typedef f16x8 v8; typedef f16x4 v4; };

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kThreads = 256;
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0) (expcnt 7, lgkmcnt 15)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// (value of lane l & 31, value of lane l | 32): the two halves of a column
__device__ __forceinline__ void halves(float x, float &h0, float &h1) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  h0 = __uint_as_float(r[0]);
  h1 = __uint_as_float(r[1]);
}

struct BwdPlan {
  int log2g;    // query heads per KV head = 2^log2g
  int n_qtile;  // 128-slot tiles per (b, g) of the dQ kernel
};

__device__ __forceinline__ int quad_slot(int qq) { return ((qq & 1) << 1) | (qq >> 1); }

__device__ __forceinline__ uint4 sel4(bool keep, uint4 x) {
  return keep ? x : make_uint4(0, 0, 0, 0);
}

// Raw buffer over `bytes` bytes from `base` (word 3 of the gfx9 descriptor:
// 32-bit raw accesses).  Loads at offsets at or beyond `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)(bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, n, 0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Column offset (elements) inside a transposed row of R columns for the
// quad of 4 rows 4 qq .. 4 qq + 3 of a tile, on transposed row d.
template <int R>
__device__ __forceinline__ int tr_col(int qq, int d) {
  constexpr int NCH = R / 8;
  const int slot = 16 * (qq >> 2) + 4 * quad_slot(qq & 3);
  return (((slot >> 3) ^ (2 * ((d >> 5) & (NCH / 2 - 1)))) * 8) + (slot & 7);
}

// Writes 4 rows x 8 columns (r[u] = row u, 8 elements) transposed: 8 rows of 4.
template <typename T, int R>
__device__ __forceinline__ void store_tr(T *lds, const uint4 (&r)[4], int qq, int chunk) {
  constexpr int ST = R + 8;
  const int off = tr_col<R>(qq, chunk * 8);  // d >> 5 is the same for the 8 rows
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t r0 = ((const uint32_t *)&r[0])[w], r1 = ((const uint32_t *)&r[1])[w];
    const uint32_t r2 = ((const uint32_t *)&r[2])[w], r3 = ((const uint32_t *)&r[3])[w];
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      const uint32_t s = hl ? 0x07060302u : 0x05040100u;
      const uint2 kk = make_uint2(__builtin_amdgcn_perm(r1, r0, s), __builtin_amdgcn_perm(r3, r2, s));
      *(uint2 *)&lds[(chunk * 8 + 2 * w + hl) * ST + off] = kk;
    }
  }
}

// A operand of a transposed tile: row d = 32 db + col, 16-row step st, lane half
template <typename T, int R>
__device__ __forceinline__ typename BV<T>::v8 read_tr(const T *lds, int db, int col, int st,
                                                      int half) {
  constexpr int ST = R + 8, NCH = R / 8;
  const int swz = 2 * (db & (NCH / 2 - 1));
  return *(const typename BV<T>::v8 *)&lds[(db * 32 + col) * ST + (((2 * st + half) ^ swz) * 8)];
}

// ---------------------------------------------------------------------------
// dQ (and the row statistics)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_mfma(Params p, BwdPlan pl,
                                                           const T *__restrict__ dy,
                                                           float *__restrict__ lse2,
                                                           float *__restrict__ delta,
                                                           T *__restrict__ dq) {
  typedef typename BV<T>::v8 vec8;
  constexpr int BN = 32;          // keys per tile
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int NKS = D / 16;     // k-steps of the score MFMAs
  constexpr int NDB = D / 32;     // 32-wide dQ^T blocks
  constexpr int KST = D + 8;      // row-major stride (elements)
  constexpr int TST = BN + 8;     // transposed stride
  constexpr int RPP = kThreads / CH;    // row-major rows per pass
  constexpr int NU = BN / RPP;          // row-major passes per tile
  constexpr int NTT = (BN / 4) * CH;    // transposed tasks (quad x chunk)
  __shared__ __attribute__((aligned(16))) T klds[2][BN * KST];
  __shared__ __attribute__((aligned(16))) T vlds[2][BN * KST];
  __shared__ __attribute__((aligned(16))) T ktlds[2][D * TST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int n_bg = p.B * p.Hkv;
  const int bg = blockIdx.x % n_bg;
  const int tile = pl.n_qtile - 1 - blockIdx.x / n_bg;  // late (heavy) slot tiles first
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int lg = pl.log2g, G = 1 << lg, nslots = p.S << lg;
  const int s0 = tile * 128;
  const int slot = s0 + wave * 32 + col;
  const bool row_ok = slot < nslots;
  const int row_i = row_ok ? slot >> lg : 0;
  const int row_h = g * G + (slot & (G - 1));
  const bool wave_active = s0 + wave * 32 < nslots;
  const int i_first = s0 >> lg, i_last = (min(nslots, s0 + 128) - 1) >> lg;
  const int hi = p.causal ? i_last + 1 : p.S;
  const int lo = p.window > 0 ? max(0, i_first - p.window + 1) : 0;
  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;

  // Q and dY of the slot: B operands (slot column, dims 16 ks + 8 half + e)
  vec8 qreg[NKS], dyreg[NKS];
  {
    const T *qr = (const T *)p.q + b * p.q_sb + (int64_t)row_i * p.q_ss + (int64_t)row_h * p.q_sh;
    const T *dr = dy + (((int64_t)b * p.S + row_i) * p.Hq + row_h) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int d0 = ks * 16 + half * 8;
      qreg[ks] = __builtin_bit_cast(vec8, sel4(row_ok, *(const uint4 *)(qr + d0)));
      dyreg[ks] = __builtin_bit_cast(vec8, sel4(row_ok, *(const uint4 *)(dr + d0)));
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // staging maps: row-major rows tid / CH (+ RPP u), chunk tid % CH; the
  // transposed K^T tile (built from the row-major K tile in LDS) takes quad
  // tid % 8 (keys 4q..4q+3) x chunk tid / 8.  Loads go through buffers that
  // start at the tile's first key and end at key S, so keys past the sequence
  // read as zeros; offsets are per thread.
  const int rrow = tid / CH, rch = tid % CH;
  const int tq = tid % (BN / 4), tc = tid / (BN / 4);
  const bool tstager = tid < NTT;
  const T *kb = (const T *)p.k + b * p.k_sb + (int64_t)g * p.k_sh;
  const T *vb = (const T *)p.v + b * p.v_sb + (int64_t)g * p.v_sh;
  uint32_t ko[NU], vo[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    ko[u] = (uint32_t)(((rrow + u * RPP) * p.k_ss + rch * 8) * (int64_t)sizeof(T));
    vo[u] = (uint32_t)(((rrow + u * RPP) * p.v_ss + rch * 8) * (int64_t)sizeof(T));
  }
  uint4 rk[NU], rv[NU], rt[4];
  auto load = [&](int kt) __attribute__((always_inline)) {
    const int j0 = kt * BN;
    const auto kr = rsrc(kb + (int64_t)j0 * p.k_ss,
                         ((int64_t)(p.S - j0) * p.k_ss - g * p.k_sh) * (int64_t)sizeof(T));
    const auto vr = rsrc(vb + (int64_t)j0 * p.v_ss,
                         ((int64_t)(p.S - j0) * p.v_ss - g * p.v_sh) * (int64_t)sizeof(T));
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      rk[u] = bload(kr, ko[u]);
      rv[u] = bload(vr, vo[u]);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      *(uint4 *)&klds[buf][(rrow + u * RPP) * KST + rch * 8] = rk[u];
      *(uint4 *)&vlds[buf][(rrow + u * RPP) * KST + rch * 8] = rv[u];
    }
  };
  // S^T and dP^T of one tile (key rows, slot columns)
  auto scores = [&](int buf, f32x16 &sacc, f32x16 &dpacc) __attribute__((always_inline)) {
    const T *kl = klds[buf], *vl = vlds[buf];
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const vec8 a = *(const vec8 *)&kl[col * KST + ks * 16 + half * 8];
      const vec8 c = *(const vec8 *)&vl[col * KST + ks * 16 + half * 8];
      sacc = mma(a, qreg[ks], ks == 0 ? zero : sacc);
      dpacc = mma(c, dyreg[ks], ks == 0 ? zero : dpacc);
    }
  };
  auto allowed = [&](int j) __attribute__((always_inline)) {
    return (j < p.S) & (!p.causal | (j <= row_i)) & ((p.window <= 0) | (j >= row_i - p.window + 1));
  };
  auto need_mask = [&](int kt) __attribute__((always_inline)) {
    const int j0 = kt * BN;
    return (p.causal && j0 + BN - 1 > i_first) ||
           (p.window > 0 && j0 < i_last - p.window + 1) || j0 + BN > p.S;
  };
  const float sl = p.scale * kLog2e;

  // ---- pass 1: lse2 and delta of the slot (each lane half over its keys) ----
  float m = kNegInf, l = 0.f, a = 0.f;
  load(kt0);
  store(0);
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) load(kt + 1);
    if (__builtin_amdgcn_readfirstlane((int)wave_active)) {
      f32x16 sacc, dpacc;
      scores(buf, sacc, dpacc);
      // the mask test is one scalar branch per tile
      auto scale_mask = [&](auto MASKED) __attribute__((always_inline)) {
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = sacc[r] * sl;
          if (MASKED) t = allowed(kt * BN + 8 * (r >> 2) + 4 * half + (r & 3)) ? t : kNegInf;
          sacc[r] = t;
          mx = fmaxf(mx, t);
        }
        return mx;
      };
      const float mx = __builtin_amdgcn_readfirstlane((int)need_mask(kt))
                           ? scale_mask(std::true_type()) : scale_mask(std::false_type());
      const float mn = fmaxf(m, mx);
      const float mu = mn == kNegInf ? 0.f : mn;
      const float alpha = ex2(m - mu);
      float ls = 0.f, as = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = ex2(sacc[r] - mu);
        ls += e;
        as = __builtin_fmaf(e, dpacc[r], as);
      }
      l = __builtin_fmaf(l, alpha, ls);
      a = __builtin_fmaf(a, alpha, as);
      m = mn;
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }
  float L2 = kPosInf, Dl = 0.f;  // no allowed key: P = 0 everywhere
  {
    float m0, m1, l0, l1, a0, a1;
    halves(m, m0, m1);
    halves(l, l0, l1);
    halves(a, a0, a1);
    const float mm = fmaxf(m0, m1);
    if (mm != kNegInf) {
      const float e0 = ex2(m0 - mm), e1 = ex2(m1 - mm);
      const float lt = l0 * e0 + l1 * e1, at = a0 * e0 + a1 * e1;
      L2 = mm + log2f(lt);
      Dl = at / lt;
    }
  }
  if (row_ok && half == 0) {
    const int64_t r = ((int64_t)b * p.Hq + row_h) * p.S + row_i;
    lse2[r] = L2;
    delta[r] = Dl;
  }

  // ---- pass 2: dQ^T += K^T dS^T ----
  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;
  // K^T of tile kt is built in LDS from the row-major K tile during step kt
  // and used by the dQ MFMAs of step kt + 1, together with dS of tile kt kept
  // in registers; the last step only finishes dQ.
  vec8 dsh[BN / 16];
  load(kt0);
  store(0);
  __syncthreads();
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool cur = kt < kt1, more = kt + 1 < kt1;
    if (more) load(kt + 1);
    if (cur && tstager) {
#pragma unroll
      for (int u = 0; u < 4; ++u) rt[u] = *(const uint4 *)&klds[buf][(4 * tq + u) * KST + tc * 8];
      store_tr<T, BN>(ktlds[buf], rt, tq, tc);
    }
    if (__builtin_amdgcn_readfirstlane((int)wave_active)) {
      if (kt > kt0) {
        // lane half h supplies keys 16 st + {4h..4h+3, 8+4h..8+4h+3}
#pragma unroll
        for (int st = 0; st < BN / 16; ++st)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            dqacc[db] = mma(read_tr<T, BN>(ktlds[buf ^ 1], db, col, st, half), dsh[st], dqacc[db]);
      }
      if (cur) {
        f32x16 sacc, dpacc;
        scores(buf, sacc, dpacc);
        auto dscore = [&](auto MASKED) __attribute__((always_inline)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float t = __builtin_fmaf(sacc[r], sl, -L2);
            if (MASKED) t = allowed(kt * BN + 8 * (r >> 2) + 4 * half + (r & 3)) ? t : kNegInf;
            const float pr = ex2(t);
            sacc[r] = pr * (dpacc[r] - Dl);  // dS / scale
          }
        };
        if (__builtin_amdgcn_readfirstlane((int)need_mask(kt))) dscore(std::true_type());
        else dscore(std::false_type());
#pragma unroll
        for (int st = 0; st < BN / 16; ++st)
#pragma unroll
          for (int e = 0; e < 8; ++e) dsh[st][e] = (T)sacc[8 * st + e];
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }
  if (!row_ok) return;
  T *out = dq + (((int64_t)b * p.S + row_i) * p.Hq + row_h) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      typename BV<T>::v4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (T)(dqacc[db][4 * q4 + e] * p.scale);
      *(typename BV<T>::v4 *)&out[db * 32 + 8 * q4 + 4 * half] = v4;
    }
}

// ---------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------
constexpr int kDkvThreads = 512;

template <typename T, int D>
__global__ __launch_bounds__(kDkvThreads, 1) void bwd_dkv_mfma(Params p, BwdPlan pl,
                                                               const T *__restrict__ dy,
                                                               const float *__restrict__ lse2,
                                                               const float *__restrict__ delta,
                                                               T *__restrict__ dk,
                                                               T *__restrict__ dv) {
  typedef typename BV<T>::v8 vec8;
  constexpr int QT = 32;          // row slots per tile (a whole number of queries)
  constexpr int CH = D / 8;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int KST = D + 8;
  constexpr int TST = QT + 8;
  constexpr int RPP = 256 / CH;   // row-major rows per pass of the producer threads
  constexpr int NU = QT / RPP;
  constexpr int NTT = (QT / 4) * CH;  // transposed tasks per operand
  static_assert(NTT <= 128, "each half of the consumer threads stages one transposed tile");
  // Producer wavefronts 0-3 (one per SIMD) own keys 32 w .. 32 w + 31 of the
  // block: S = Q K^T and dP = dY V^T of tile t on the matrix core, then P and
  // dS / scale on the VALU, handed over through LDS in the B-operand layout.
  // Consumer wavefronts 4-7 (one per SIMD, same keys) accumulate
  // dV^T += dY^T P and dK^T += Q^T dS of tile t - 1 meanwhile, so one SIMD
  // overlaps a producer's exponentials with a consumer's MFMAs.  Producers
  // load the row-major Q / dY tiles and the row statistics, consumers build
  // the transposed Q^T / dY^T tiles from them in LDS; one barrier per step.
  __shared__ __attribute__((aligned(16))) T qlds[2][QT * KST];
  __shared__ __attribute__((aligned(16))) T dylds[2][QT * KST];
  __shared__ __attribute__((aligned(16))) T qtlds[2][D * TST];
  __shared__ __attribute__((aligned(16))) T dytlds[2][D * TST];
  __shared__ __attribute__((aligned(16))) float lse_s[2][QT];
  __shared__ __attribute__((aligned(16))) float dl_s[2][QT];
  __shared__ __attribute__((aligned(16))) int qi_s[2][QT];
  __shared__ __attribute__((aligned(16))) uint4 xch[2][4][QT / 16][2][64];  // P, dS per lane

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const bool consumer = __builtin_amdgcn_readfirstlane(wave) >= 4;
  const int kw = wave & 3;  // key group of the wavefront
  const int n_bg = p.B * p.Hkv;
  const int bg = blockIdx.x % n_bg;
  const int kblk = blockIdx.x / n_bg;  // early (heavy under causal) key blocks first
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int lg = pl.log2g, G = 1 << lg, nslots = p.S << lg;
  const int j0 = kblk * 128, j_last = min(p.S, j0 + 128) - 1;
  const int jw = j0 + kw * 32, jw_last = min(p.S - 1, jw + 31);
  const int key = jw + col;
  const bool key_ok = key < p.S;
  const bool wave_keys = jw < p.S;
  // queries that see some key of the block
  const int i_lo = p.causal ? j0 : 0;
  const int i_hi = p.window > 0 ? min(p.S, j_last + p.window) : p.S;
  const int s_lo = i_lo << lg, s_hi = i_hi << lg;
  const int n_t = (s_hi - s_lo + QT - 1) / QT;

  // Tile t is QT consecutive slots = QT / G whole queries from query i0; row r
  // is (query i0 + r / G, head g G + r % G).  Q and dY go through buffers from
  // row i0 to the end of the batch, so rows past the sequence read as zeros.
  const int64_t dy_ss = (int64_t)p.Hq * D;
  auto q_off = [&](int r, int c) {
    return (uint32_t)(((r >> lg) * p.q_ss + (int64_t)(g * G + (r & (G - 1))) * p.q_sh + c * 8) *
                      (int64_t)sizeof(T));
  };
  auto dy_off = [&](int r, int c) {
    return (uint32_t)(((r >> lg) * dy_ss + (int64_t)(g * G + (r & (G - 1))) * D + c * 8) *
                      (int64_t)sizeof(T));
  };
  const T *qb = (const T *)p.q + b * p.q_sb;
  const T *dyb = dy + (int64_t)b * p.S * dy_ss;
  auto q_rsrc = [&](int i0) {
    return rsrc(qb + (int64_t)i0 * p.q_ss, (int64_t)(p.S - i0) * p.q_ss * (int64_t)sizeof(T));
  };
  auto dy_rsrc = [&](int i0) {
    return rsrc(dyb + (int64_t)i0 * dy_ss, (int64_t)(p.S - i0) * dy_ss * (int64_t)sizeof(T));
  };
  auto tile_i0 = [&](int t) { return (s_lo + t * QT) >> lg; };

  if (!consumer) {
    // ---------------- producer ----------------
    vec8 kreg[NKS], vreg[NKS];
    {
      const int kk = min(key, p.S - 1);
      const T *kr = (const T *)p.k + b * p.k_sb + (int64_t)kk * p.k_ss + (int64_t)g * p.k_sh;
      const T *vr = (const T *)p.v + b * p.v_sb + (int64_t)kk * p.v_ss + (int64_t)g * p.v_sh;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int d0 = ks * 16 + half * 8;
        kreg[ks] = __builtin_bit_cast(vec8, sel4(key_ok, *(const uint4 *)(kr + d0)));
        vreg[ks] = __builtin_bit_cast(vec8, sel4(key_ok, *(const uint4 *)(vr + d0)));
      }
    }
    // row-major staging: rows tid / CH (+ RPP u), chunk tid % CH, Q and dY
    const int rrow = tid / CH, rch = tid % CH;
    uint32_t qo[NU], dyo[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      qo[u] = q_off(rrow + u * RPP, rch);
      dyo[u] = dy_off(rrow + u * RPP, rch);
    }
    // Loads run two steps ahead of the compute: tile t + 2 is loaded into one
    // register set during step t and stored to LDS at the end of step t + 1.
    struct Stage {
      uint4 q[NU], dy[NU];
      float lse, dl;
      int qi;
    };
    auto load = [&](int t, Stage &sg) __attribute__((always_inline)) {
      const int i0 = tile_i0(t);
      const auto qr = q_rsrc(i0), dr = dy_rsrc(i0);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        sg.q[u] = bload(qr, qo[u]);
        sg.dy[u] = bload(dr, dyo[u]);
      }
      if (tid < QT) {
        const int i = i0 + (tid >> lg);
        const int64_t r = ((int64_t)b * p.Hq + g * G + (tid & (G - 1))) * p.S + min(i, p.S - 1);
        const float lv = lse2[r], dv_ = delta[r];
        sg.lse = i < p.S ? lv : kPosInf;  // rows past the sequence: P = 0
        sg.dl = i < p.S ? dv_ : 0.f;
        sg.qi = i;
      }
    };
    auto store = [&](int buf, const Stage &sg) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        *(uint4 *)&qlds[buf][(rrow + u * RPP) * KST + rch * 8] = sg.q[u];
        *(uint4 *)&dylds[buf][(rrow + u * RPP) * KST + rch * 8] = sg.dy[u];
      }
      if (tid < QT) {
        lse_s[buf][tid] = sg.lse;
        dl_s[buf][tid] = sg.dl;
        qi_s[buf][tid] = sg.qi;
      }
    };
    const float sl = p.scale * kLog2e;
    // P and dS / scale of tile t into the hand-over buffer; rows of the S / dP
    // accumulators are slots 8 q4 + 4 half + e
    auto produce = [&](auto MASKED, int t, bool dead) __attribute__((always_inline)) {
      const int buf = t & 1;
      const T *ql = qlds[buf], *dyl = dylds[buf];
      f32x16 sacc, dpacc;
      const f32x16 zero = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const vec8 aq = *(const vec8 *)&ql[col * KST + ks * 16 + half * 8];
        const vec8 ad = *(const vec8 *)&dyl[col * KST + ks * 16 + half * 8];
        sacc = mma(aq, kreg[ks], ks == 0 ? zero : sacc);
        dpacc = mma(ad, vreg[ks], ks == 0 ? zero : dpacc);
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int s4 = 8 * q4 + 4 * half;
        const float4 lv = *(const float4 *)&lse_s[buf][s4];
        const float4 dl = *(const float4 *)&dl_s[buf][s4];
        int4 qi = make_int4(0, 0, 0, 0);
        if (MASKED) qi = *(const int4 *)&qi_s[buf][s4];
        const float lva[4] = {lv.x, lv.y, lv.z, lv.w}, dla[4] = {dl.x, dl.y, dl.z, dl.w};
        const int qia[4] = {qi.x, qi.y, qi.z, qi.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          float x = __builtin_fmaf(sacc[r], sl, -lva[e]);
          if (MASKED) {
            const int i = qia[e];
            const bool ok = !dead & (!p.causal | (key <= i)) &
                            ((p.window <= 0) | (key >= i - p.window + 1));
            x = ok ? x : kNegInf;
          }
          const float pr = ex2(x);
          sacc[r] = pr;
          dpacc[r] = pr * (dpacc[r] - dla[e]);
        }
      }
      // lane half h supplies slots 16 st + {4h..4h+3, 8+4h..8+4h+3}
#pragma unroll
      for (int st = 0; st < QT / 16; ++st) {
        vec8 pb, dsb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = (T)sacc[8 * st + e];
          dsb[e] = (T)dpacc[8 * st + e];
        }
        xch[buf][kw][st][0][lane] = __builtin_bit_cast(uint4, pb);
        xch[buf][kw][st][1][lane] = __builtin_bit_cast(uint4, dsb);
      }
    };
    auto compute = [&](int t) __attribute__((always_inline)) {
      // A tile that no key of the wave sees is computed too, fully masked.
      const int st0 = s_lo + t * QT;
      const int ia = st0 >> lg, ib = (min(nslots, st0 + QT) - 1) >> lg;
      const bool dead = !wave_keys || (p.causal && ib < jw) ||
                        (p.window > 0 && ia - p.window + 1 > jw_last);
      const bool msk = dead || (p.causal && ia < jw_last) ||
                       (p.window > 0 && ib - p.window + 1 > jw);
      if (__builtin_amdgcn_readfirstlane((int)msk)) produce(std::true_type(), t, dead);
      else produce(std::false_type(), t, dead);
    };
    Stage sa, sb;
    sa.lse = sb.lse = kPosInf;
    sa.dl = sb.dl = 0.f;
    sa.qi = sb.qi = 0;
    if (n_t > 0) {
      load(0, sa);
      store(0, sa);
    }
    __syncthreads();
    if (n_t > 1) load(1, sb);
    for (int t = 0; t < n_t; t += 2) {
      if (t + 2 < n_t) load(t + 2, sa);
      compute(t);
      if (t + 1 < n_t) store((t + 1) & 1, sb);
      __syncthreads();
      if (t + 1 < n_t) {
        if (t + 3 < n_t) load(t + 3, sb);
        compute(t + 1);
        if (t + 2 < n_t) store(t & 1, sa);
        __syncthreads();
      }
    }
    __syncthreads();  // the consumer's last step
    return;
  }

  // ---------------- consumer ----------------
  // The transposed tiles are built from the row-major tiles the producers
  // staged (4 rows x one 16-byte chunk per task): threads 256..383 Q^T,
  // 384..511 dY^T; task t = tid % 128 -> quad t % (QT/4) (rows 4q..4q+3) x
  // chunk t / (QT/4).
  const int tt = tid & 127;
  const bool t_dy = __builtin_amdgcn_readfirstlane(wave) >= 6;  // uniform
  const int tq = tt % (QT / 4), tc = tt / (QT / 4);
  const bool tstager = tt < NTT;
  uint4 rt[4];
  auto load = [&](int t) __attribute__((always_inline)) {
    if (tstager) {
      const T *src = t_dy ? dylds[t & 1] : qlds[t & 1];
#pragma unroll
      for (int u = 0; u < 4; ++u) rt[u] = *(const uint4 *)&src[(4 * tq + u) * KST + tc * 8];
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    if (tstager) store_tr<T, QT>(t_dy ? dytlds[buf] : qtlds[buf], rt, tq, tc);
  };
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[db][r] = 0.f;
      dvacc[db][r] = 0.f;
    }
  __syncthreads();
  for (int t = 0; t <= n_t; ++t) {
    if (t < n_t) load(t);
    if (t > 0) {
      const int buf = (t - 1) & 1;
      const T *qtl = qtlds[buf], *dytl = dytlds[buf];
#pragma unroll
      for (int st = 0; st < QT / 16; ++st) {
        const vec8 pb = __builtin_bit_cast(vec8, xch[buf][kw][st][0][lane]);
        const vec8 dsb = __builtin_bit_cast(vec8, xch[buf][kw][st][1][lane]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dvacc[db] = mma(read_tr<T, QT>(dytl, db, col, st, half), pb, dvacc[db]);
          dkacc[db] = mma(read_tr<T, QT>(qtl, db, col, st, half), dsb, dkacc[db]);
        }
      }
    }
    if (t < n_t) store(t & 1);
    __syncthreads();
  }
  if (!key_ok) return;
  T *ko = dk + (((int64_t)b * p.S + key) * p.Hkv + g) * D;
  T *vo = dv + (((int64_t)b * p.S + key) * p.Hkv + g) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      typename BV<T>::v4 k4, v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = (T)(dkacc[db][4 * q4 + e] * p.scale);
        v4[e] = (T)dvacc[db][4 * q4 + e];
      }
      *(typename BV<T>::v4 *)&ko[db * 32 + 8 * q4 + 4 * half] = k4;
      *(typename BV<T>::v4 *)&vo[db * 32 + 8 * q4 + 4 * half] = v4;
    }
}

template <typename T, int D>
hipError_t launch_t(const Params &p, const void *dy, void *dq, void *dk, void *dv, float *ws,
                    hipStream_t st) {
  BwdPlan pl;
  pl.log2g = __builtin_ctz((unsigned)p.G);
  const int64_t nslots = (int64_t)p.S * p.G;
  pl.n_qtile = (int)((nslots + 127) / 128);
  const int n_bg = p.B * p.Hkv;
  float *lse = ws, *delta = ws + (int64_t)p.B * p.Hq * p.S;
  hipLaunchKernelGGL((bwd_dq_mfma<T, D>), dim3(pl.n_qtile * n_bg), dim3(kThreads), 0, st, p, pl,
                     (const T *)dy, lse, delta, (T *)dq);
  const int n_kb = (p.S + 127) / 128;
  hipLaunchKernelGGL((bwd_dkv_mfma<T, D>), dim3(n_kb * n_bg), dim3(kDkvThreads), 0, st, p, pl,
                     (const T *)dy, lse, delta, (T *)dk, (T *)dv);
  return hipGetLastError();
}

}  // namespace

bool backward_mfma_supports(const Params &p, int dtype, const void *dy, const void *dq,
                            const void *dk, const void *dv) {
  if (dtype != DT_BF16 && dtype != DT_F16) return false;
  if (p.D != p.Dv || (p.D != 64 && p.D != 128)) return false;
  // slot -> (query, head) by shifts; a 32-slot tile holds whole queries
  if (p.G <= 0 || p.G > 32 || (p.G & (p.G - 1)) != 0) return false;
  if ((int64_t)p.S * p.G > (1ll << 30)) return false;
  // buffer loads address one batch of Q, K, V or dY with 32-bit byte offsets
  const int64_t es = 2;
  if ((int64_t)p.S * p.q_ss * es > 0x7fffffff || (int64_t)p.S * p.k_ss * es > 0x7fffffff ||
      (int64_t)p.S * p.v_ss * es > 0x7fffffff || (int64_t)p.S * p.Hq * p.D * es > 0x7fffffff)
    return false;
  auto al16 = [](const void *x) { return ((uintptr_t)x & 15) == 0; };
  auto al8 = [](const void *x) { return ((uintptr_t)x & 7) == 0; };
  // 16-byte operand loads of Q, K, V, dY rows; 8-byte output stores
  if (!al16(p.q) || !al16(p.k) || !al16(p.v) || !al16(dy)) return false;
  if (!al8(dq) || !al8(dk) || !al8(dv)) return false;
  const int64_t strides[] = {p.q_sb, p.q_ss, p.q_sh, p.k_sb, p.k_ss, p.k_sh,
                             p.v_sb, p.v_ss, p.v_sh};
  for (int64_t s : strides)
    if (s % 8 != 0) return false;
  return true;
}

hipError_t launch_backward_mfma(const Params &p, int dtype, const void *dy, void *dq, void *dk,
                                void *dv, float *ws, hipStream_t st) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  if (dtype == DT_BF16)
    return p.D == 128 ? launch_t<bf16, 128>(p, dy, dq, dk, dv, ws, st)
                      : launch_t<bf16, 64>(p, dy, dq, dk, dv, ws, st);
  return p.D == 128 ? launch_t<f16, 128>(p, dy, dq, dk, dv, ws, st)
                    : launch_t<f16, 64>(p, dy, dq, dk, dv, ws, st);
}

}  // namespace olk
