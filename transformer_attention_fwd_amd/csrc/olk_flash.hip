// Prefill attention forward for gfx950 (CDNA4): f16/bf16 inputs, head size 64
// or 128, fp32 accumulation.
//
// Computes Y = Softmax((Q K^T) * scale + bias) V with grouped KV heads, causal /
// local-window / length masks, softcap, head_sink and the present outputs of
// the GroupQueryAttention, MultiHeadAttention and ai.onnx Attention contracts
// (onnx-light-cpu Python API "Custom operators"; onnx-light reference kernels
// header page, "class Attention").  The decomposition is ours:
//
// * A workgroup is 4 wavefronts x 32 row slots; two workgroups share a CU
//   (two wavefronts per SIMD, so one wave's MFMAs overlap the other's softmax;
//   three at head size 64).
//   Slots pack the GH query heads sharing one KV head with consecutive queries
//   (slot -> (query, head)): every K/V tile in LDS serves the whole head group.
// * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16.  In the S^T
//   accumulator layout a lane owns one row slot and half of a tile's keys, so
//   the softmax max/sum are in-lane plus one exchange with lane ^ 32, and P^T
//   is already the B operand of the PV MFMA.
// * K is staged row-major; V is staged transposed (V^T, key-major rows per head
//   dimension) by a 4x4 register transpose, so every MFMA operand is one
//   ds_read_b128.  The key order inside each 16-key group of V^T follows the
//   MFMA's k order of P^T.  Rows are padded by 16 bytes so the operand reads
//   are conflict-free, and 16-byte chunks are XOR-swizzled by (row / 32) to
//   spread the transposing writes; that key is uniform across each read
//   instruction, so reads keep immediate offsets.
// * Keys advance in tiles of 64.
// * K/V tiles are double-buffered in LDS, one barrier per tile; the next
//   tile's global loads are in flight while the current tile computes.
// * Online softmax in the exp2 domain, the scale folded into the exponent's
//   FMA; per-key masks only on boundary tiles, written as -inf in place.  O is rescaled only when a row's running max grows by more
//   than 2^8 (the final division uses the same max, so the result is unchanged).
// * GroupQueryAttention present rows of the new keys are stored by the
//   workgroup whose queries sit at those positions: with causal masking from
//   its last two LDS tiles after the loop, otherwise while the rows pass
//   through registers.
#include "olk_internal.h"

namespace olk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct FV;
template <> struct FV<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct FV<f16> { typedef f16x8 v8; typedef f16x4 v4; };

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// s_waitcnt immediate for vmcnt(0) only (gfx9 encoding: expcnt 7, lgkmcnt 15)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kThreads = 256;
constexpr int kSlots = 128;  // row slots per workgroup (4 wavefronts x 32)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescale = 8.0f;

template <typename T> __device__ __forceinline__ float lo16(uint32_t w);
template <> __device__ __forceinline__ float lo16<bf16>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float lo16<f16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffff));
}
template <typename T> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float hi16<bf16>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <> __device__ __forceinline__ float hi16<f16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// two floats rounded (RNE) to the element type, packed low / high
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const T l = (T)lo, h = (T)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// Value of lane ^ 32 combined with this lane's, via v_permlane32_swap (with
// both operands x, the two results hold x of lane l and of lane l ^ 32).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key k (0 <= k < 16) inside its 16-key group of a V^T row: the
// group stores keys {0-3, 8-11, 4-7, 12-15}, so the 8 keys that lane half h
// supplies to one 16-key MFMA step (4h..4h+3 and 8+4h..8+4h+3) are contiguous.
__device__ __forceinline__ int quad_slot(int qq) { return ((qq & 1) << 1) | (qq >> 1); }

struct FPlan {
  int GH, n_hg, QW, n_qt;
  int xcd_remap;
  int bias_vec;
  int mask_vec;      // BOOL mask rows are 4-byte aligned
  int fuse_present;
};

// Wavefronts per SIMD the register budget is sized for: three at head size 64
// (more workgroups resident when a grid holds few query tiles; the BOOL-mask
// form needs more registers and keeps two), two at head size 128.
template <int D, int BM> constexpr int kOcc = (D == 64 && BM != 2) ? 3 : 2;

// BM: 0 no bias, 1 attn_bias, 2 BOOL attn_mask (with or without attn_bias)
template <typename T, int D, int BM, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, (kOcc<D, BM>)) void flash_fwd_kernel(Params p, FPlan pl) {
  typedef typename FV<T>::v8 vec8;
  constexpr bool BIAS = BM != 0;   // the score epilogue reads a bias row
  constexpr bool MASK = BM == 2;
  constexpr int CH = D / 8;             // 16-byte chunks per K/V row
  constexpr int BN = 64;                // keys per tile
  constexpr int KB = BN / 32;           // 32-key blocks per tile
  constexpr int NST = BN / 16;          // 16-key PV steps per tile
  constexpr int NKS = D / 16;           // QK^T k-steps
  constexpr int NDB = D / 32;           // 32-wide output blocks
  constexpr int KST = D + 8;            // K row stride (elements)
  constexpr int VST = BN + 8;           // V^T row stride (elements)
  constexpr int NCH_V = BN / 8;         // 16-byte chunks per V^T row
  __shared__ __attribute__((aligned(16))) T klds[2][BN * KST];
  __shared__ __attribute__((aligned(16))) T vlds[2][D * VST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  // ---- workgroup -> (q tile, b, g, hg); late (heavy) query tiles first ----
  const int n_bg = p.B * p.Hkv * pl.n_hg;
  const int wid = blockIdx.x;
  int bg, qrank;
  if (pl.xcd_remap) {  // ids go round-robin over 8 XCDs: keep one (b, g) on one XCD
    const int per = n_bg / 8, xcd = wid & 7, k = wid >> 3;
    qrank = k / per;
    bg = (k % per) * 8 + xcd;
  } else {
    qrank = wid / n_bg;
    bg = wid % n_bg;
  }
  const int qt = pl.n_qt - 1 - qrank;
  const int hg = bg % pl.n_hg;
  const int g = (bg / pl.n_hg) % p.Hkv;
  const int b = bg / (pl.n_hg * p.Hkv);
  const Seq s = seq_info(p, b);
  const int i0 = qt * pl.QW;
  const int i_last = min(i0 + pl.QW, p.S) - 1;
  const int pos_min = s.qoff + i0, pos_max = s.qoff + i_last;
  int hi = p.pad_add ? s.total : s.valid;
  if (p.causal) hi = min(hi, pos_max + 1);
  // short masks exclude the keys beyond their columns (BIAS instantiations
  // also serve BOOL attn_mask, with or without a bias)
  if (BM == 1 || (MASK && p.bias)) hi = min(hi, p.bias_cols);
  if (MASK) hi = min(hi, p.mask_cols);
  const int lo = p.window > 0 ? max(0, pos_min - p.window + 1) : 0;
  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;

  // ---- this lane's row slot ----
  const int slot = wave * 32 + col;
  const int row_i = i0 + slot / pl.GH;
  const int row_h = g * p.G + hg * pl.GH + slot % pl.GH;
  const bool row_ok = row_i < p.S;
  const int row_pos = s.qoff + row_i;
  const bool wave_active = i0 + (wave * 32) / pl.GH < p.S;

  // ---- Q^T operand (B of S^T = K Q^T): slot col, d = 16 ks + 8 half + e ----
  vec8 qreg[NKS];
  {
    const T *qr = (const T *)p.q + b * p.q_sb + (int64_t)(row_ok ? row_i : 0) * p.q_ss +
                  row_h * p.q_sh;
    uint4 raw[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      raw[ks] = make_uint4(0, 0, 0, 0);
      if (row_ok) raw[ks] = *(const uint4 *)(qr + ks * 16 + half * 8);
    }
    if (p.rot_q) {
      // Rotary embedding of Q at position past_b + i, the same float32
      // arithmetic and single rounding as the rotary pre-pass (pair (x1, x2)
      // -> (fma(x1, c, -(x2 s)), fma(x2, c, x1 s))).  Split halves over the
      // whole head: dims d and d + D/2 sit in chunks ks and ks + NKS/2 of the
      // same lane; interleaved pairs (2k, 2k+1) sit inside one chunk.
      const int pos = min(s.past + row_i, p.rot_max - 1);
      const T *cs = (const T *)p.cos_cache + (int64_t)pos * (p.rot_dim / 2);
      const T *sn = (const T *)p.sin_cache + (int64_t)pos * (p.rot_dim / 2);
      auto rot1 = [](float x1, float x2, float c, float sv) { return __builtin_fmaf(x1, c, -__fmul_rn(x2, sv)); };
      auto rot2 = [](float x1, float x2, float c, float sv) { return __builtin_fmaf(x2, c, __fmul_rn(x1, sv)); };
      if (!p.rot_inter) {
#pragma unroll
        for (int ks = 0; ks < NKS / 2; ++ks) {
          const int k0 = ks * 16 + half * 8;
          const uint4 c8 = *(const uint4 *)(cs + k0), s8 = *(const uint4 *)(sn + k0);
          const uint32_t *a = (const uint32_t *)&raw[ks], *bb = (const uint32_t *)&raw[ks + NKS / 2];
          const uint32_t *cw = (const uint32_t *)&c8, *sw = (const uint32_t *)&s8;
          uint4 oa, ob;
          uint32_t *oaw = (uint32_t *)&oa, *obw = (uint32_t *)&ob;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float x1l = lo16<T>(a[w]), x1h = hi16<T>(a[w]);
            const float x2l = lo16<T>(bb[w]), x2h = hi16<T>(bb[w]);
            const float cl = lo16<T>(cw[w]), ch = hi16<T>(cw[w]);
            const float sl_ = lo16<T>(sw[w]), sh_ = hi16<T>(sw[w]);
            oaw[w] = pack2<T>(rot1(x1l, x2l, cl, sl_), rot1(x1h, x2h, ch, sh_));
            obw[w] = pack2<T>(rot2(x1l, x2l, cl, sl_), rot2(x1h, x2h, ch, sh_));
          }
          raw[ks] = oa;
          raw[ks + NKS / 2] = ob;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int d0 = ks * 16 + half * 8;
          if (d0 < p.rot_dim) {
            const uint2 c4 = *(const uint2 *)(cs + d0 / 2), s4 = *(const uint2 *)(sn + d0 / 2);
            const uint32_t *a = (const uint32_t *)&raw[ks];
            const float cv[4] = {lo16<T>(c4.x), hi16<T>(c4.x), lo16<T>(c4.y), hi16<T>(c4.y)};
            const float sv[4] = {lo16<T>(s4.x), hi16<T>(s4.x), lo16<T>(s4.y), hi16<T>(s4.y)};
            uint4 o;
            uint32_t *ow = (uint32_t *)&o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float x1 = lo16<T>(a[w]), x2 = hi16<T>(a[w]);
              ow[w] = pack2<T>(rot1(x1, x2, cv[w], sv[w]), rot2(x1, x2, cv[w], sv[w]));
            }
            raw[ks] = o;
          }
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int d0 = ks * 16 + half * 8;
      if (p.proj_bias && row_ok) {
        const uint4 braw = *(const uint4 *)((const T *)p.proj_bias + row_h * D + d0);
        const uint32_t *w = (const uint32_t *)&raw[ks], *bw = (const uint32_t *)&braw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qreg[ks][2 * e] = (T)(lo16<T>(w[e]) + lo16<T>(bw[e]));
          qreg[ks][2 * e + 1] = (T)(hi16<T>(w[e]) + hi16<T>(bw[e]));
        }
      } else {
        qreg[ks] = __builtin_bit_cast(vec8, raw[ks]);
      }
    }
  }
  // Q is in registers from here on.  Waiting for its loads now, on every path,
  // keeps the wait-count analysis from assuming they may still be in flight
  // inside the loop, where it would otherwise hold the first MFMA of every
  // tile until the next tile's prefetch loads have landed as well.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---- staging: thread owns key quad q (4 keys) x 16-byte chunk c; at head
  // size 64 the upper half of the workgroup has no quad to stage ----
  // ---- staging.  LDS writes are bank-conflict free on gfx950 when 16 lanes
  // cover one contiguous row, so K and V use different lane maps:
  //  K: lane -> 16-byte chunk lane % CH of row lane / CH; the workgroup covers
  //     4 * RPI rows per pass, NUK passes per tile.
  //  V: lane -> key quad vq = lane % 16 (4 keys) x chunk vc = 4 * wave + lane / 16;
  //     after the 4x4 register transpose, 16 lanes write one full V^T row.
  //     At head size 64 only waves 0-1 stage V. ----
  constexpr int RPI = 64 / CH;              // K rows per wavefront pass
  constexpr int NUK = BN / (4 * RPI);       // K passes per tile
  const int kchunk = lane % CH;
  const int krow0 = wave * RPI + lane / CH;  // row of pass 0; pass u adds 4 * RPI * u
  const int vq = lane & 15, vc = 4 * wave + (lane >> 4);
  const bool vstager = vc < CH;
  const int vslot = 16 * (vq >> 2) + 4 * quad_slot(vq & 3);  // V^T slot of the quad's key 0
  // V^T column offset of the quad: chunk XOR-swizzled by (row / 32) = vc / 4,
  // which is the same for all 8 rows a thread writes
  const int vchunk_off = (((vslot >> 3) ^ (2 * ((vc >> 2) & (NCH_V / 2 - 1)))) * 8) + (vslot & 7);
  const T *kpast = (const T *)p.past_k + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *vpast = (const T *)p.past_v + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *knew = (const T *)p.k + b * p.k_sb + g * p.k_sh;
  const T *vnew = (const T *)p.v + b * p.v_sb + g * p.v_sh;
  const bool fuse = pl.fuse_present && hg == 0;
  const int own_lo = s.past + i0, own_hi = s.past + i_last + 1;
  // Causal: the owned rows are the last keys the loop stages (at most BN of
  // them), so both LDS buffers still hold them afterwards and present is
  // written once the loop is done; stores inside the loop would make every
  // later wait for tile loads also wait for the store acknowledgements.
  const bool fuse_end = fuse && p.causal && pl.QW <= BN;
  const bool fuse_loop = fuse && !fuse_end;
  T *pres_k = (T *)p.present_k + ((int64_t)b * p.Hkv + g) * p.T * D;
  T *pres_v = (T *)p.present_v + ((int64_t)b * p.Hkv + g) * p.T * D;

  uint4 rk[NUK], rv[4];  // staging registers: K of tile t+2, V of tile t+1

  // Row j of K or V: the past buffer below past_b, the new input above; keys
  // outside [lo, hi) read as zeros, never NaN.
  auto load_row = [&](int j, const T *pastp, const T *newp, int64_t new_ss, int chunk) __attribute__((always_inline)) {
    const T *src = j >= s.src ? newp + (int64_t)(j - s.src) * new_ss : pastp + (int64_t)j * D;
    return j >= lo && j < hi ? *(const uint4 *)(src + chunk * 8) : make_uint4(0, 0, 0, 0);
  };
  // Whole tiles inside one source use a uniform base plus 32-bit lane offsets.
  // first row r0 and row step of the NU rows a thread loads
  auto load_rows = [&](int kt, const T *pastp, const T *newp, int64_t new_ss, int r0, int rstep,
                       int chunk, auto &buf) __attribute__((always_inline)) {
    constexpr int NU = sizeof(buf) / sizeof(buf[0]);
    const int j0 = kt * BN;
    const bool full = j0 >= lo && j0 + BN <= hi;
    if (full && j0 >= s.src) {
      const char *base = (const char *)(newp + (int64_t)(j0 - s.src) * new_ss);
      const uint32_t rs = (uint32_t)new_ss * (uint32_t)sizeof(T);
      const uint32_t off = (uint32_t)r0 * rs + (uint32_t)chunk * 16u;
#pragma unroll
      for (int u = 0; u < NU; ++u) buf[u] = *(const uint4 *)(base + off + u * rstep * rs);
    } else if (full && j0 + BN <= s.src) {
      const char *base = (const char *)(pastp + (int64_t)j0 * D);
      const uint32_t rs = D * (uint32_t)sizeof(T);
      const uint32_t off = (uint32_t)r0 * rs + (uint32_t)chunk * 16u;
#pragma unroll
      for (int u = 0; u < NU; ++u) buf[u] = *(const uint4 *)(base + off + u * rstep * rs);
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) buf[u] = load_row(j0 + r0 + u * rstep, pastp, newp, new_ss, chunk);
    }
  };
  auto load_k = [&](int kt) __attribute__((always_inline)) {
    load_rows(kt, kpast, knew, p.k_ss, krow0, 4 * RPI, kchunk, rk);
  };
  auto load_v = [&](int kt) __attribute__((always_inline)) {
    if (vstager) load_rows(kt, vpast, vnew, p.v_ss, 4 * vq, 1, vc, rv);
  };
  auto store_k = [&](int kt, int buf) __attribute__((always_inline)) {
    T *kl = klds[buf];
#pragma unroll
    for (int u = 0; u < NUK; ++u) *(uint4 *)&kl[(krow0 + 4 * RPI * u) * KST + kchunk * 8] = rk[u];
    if (fuse_loop && kt * BN < own_hi && kt * BN + BN > own_lo) {
#pragma unroll
      for (int u = 0; u < NUK; ++u) {
        const int j = kt * BN + krow0 + 4 * RPI * u;
        if (j >= own_lo && j < own_hi)
          *(uint4 *)((char *)pres_k + ((uint32_t)j * D + (uint32_t)kchunk * 8u) * sizeof(T)) = rk[u];
      }
    }
  };
  // 4 keys x 8 dims -> 8 dims x 4 keys (V^T), 8 bytes per dim row
  auto store_v = [&](int kt, int buf) __attribute__((always_inline)) {
    if (!vstager) return;
    T *vl = vlds[buf];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t r0 = ((const uint32_t *)&rv[0])[w], r1 = ((const uint32_t *)&rv[1])[w];
      const uint32_t r2 = ((const uint32_t *)&rv[2])[w], r3 = ((const uint32_t *)&rv[3])[w];
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) {
        const uint32_t sel = hl ? 0x07060302u : 0x05040100u;
        const uint2 kk = make_uint2(__builtin_amdgcn_perm(r1, r0, sel), __builtin_amdgcn_perm(r3, r2, sel));
        const int d = vc * 8 + 2 * w + hl;
        *(uint2 *)&vl[d * VST + vchunk_off] = kk;
      }
    }
    if (fuse_loop && kt * BN < own_hi && kt * BN + BN > own_lo) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = kt * BN + 4 * vq + u;
        if (j >= own_lo && j < own_hi)
          *(uint4 *)((char *)pres_v + ((uint32_t)j * D + (uint32_t)vc * 8u) * sizeof(T)) = rv[u];
      }
    }
  };

  const float sl = p.scale * kLog2e;
  const bool scale_pos = p.scale > 0.f;
  // softcap in the log2 domain: c tanh(u) = c - 2c / (e^{2u} + 1) with
  // u = (s scale + bias) / c; e^{2u} = 2^(s cap_a + bias cap_b)
  const float inv_cap = SOFTCAP ? 1.0f / p.softcap : 0.f;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_b = 2.0f * kLog2e * inv_cap, cap_a = p.scale * cap_b;
  const float mfv_l2 = p.mfv * kLog2e;
  const float mfv_raw = p.mfv / p.scale;  // the same offset before the scale (scale > 0)
  const T *bias_row = BIAS ? (const T *)p.bias + b * p.bias_sb + row_h * p.bias_sh +
                                 (int64_t)(row_ok ? row_i : 0) * p.bias_si
                           : nullptr;

  // 4 bias values of keys jb..jb+3 as raw 16-bit pairs (zeros past the bias columns)
  auto bias4 = [&](int jb) {
    if (MASK && !p.bias) return make_uint2(0, 0);
    if (pl.bias_vec && jb + 3 < p.bias_cols) return *(const uint2 *)(bias_row + jb);
    uint16_t e4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      e4[e] = jb + e < p.bias_cols ? __builtin_bit_cast(uint16_t, bias_row[jb + e]) : (uint16_t)0;
    return make_uint2(e4[0] | ((uint32_t)e4[1] << 16), e4[2] | ((uint32_t)e4[3] << 16));
  };
  // BOOL attn_mask: bytes of keys jb..jb+3 of this row slot (0 past the mask's columns)
  const uint8_t *mask_row = MASK ? (const uint8_t *)p.mask + b * p.mask_sb +
                                                 row_h * p.mask_sh +
                                                 (int64_t)(row_ok ? row_i : 0) * p.mask_si
                                           : nullptr;
  auto mask4 = [&](int jb) {
    if (pl.mask_vec && jb + 3 < p.mask_cols) return *(const uint32_t *)(mask_row + jb);
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (jb + e < p.mask_cols) w |= (uint32_t)mask_row[jb + e] << (8 * e);
    return w;
  };
  // At head size 64 with two wavefronts per SIMD the bias of the next tile is
  // prefetched with its K/V (with three, its registers are not available).
  constexpr bool BPRE = BIAS && D == 64 && kOcc<D, BM> == 2;
  uint2 bcur[BPRE ? KB : 1][4], bnext[BPRE ? KB : 1][4];
  auto load_bias = [&](int kt, uint2 (&bb)[BPRE ? KB : 1][4]) {
#pragma unroll
    for (int kb = 0; kb < (BPRE ? KB : 1); ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) bb[kb][q4] = bias4(kt * BN + kb * 32 + 8 * q4 + 4 * half);
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = kNegInf, l = 0.f;

  // S^T of one tile: KB blocks of 32 keys
  auto qk = [&](int buf, f32x16 (&sacc)[KB]) {
    const T *kl = klds[buf];
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const vec8 a = *(const vec8 *)&kl[(kb * 32 + col) * KST + ks * 16 + half * 8];
        sacc[kb] = mma(a, qreg[ks], ks == 0 ? zero : sacc[kb]);
      }
    }
    // schedule: four operand reads in flight ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 0x100: LDS reads
#pragma unroll
    for (int i = 0; i < NKS * KB - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };

  // Softmax and PV of one tile.  With bias or softcap (GENERAL) the scores
  // are rewritten into the log2 domain; otherwise they stay raw (scale > 0,
  // folded into the exponent's FMA) and masking only writes -inf in place, so
  // masked and unmasked tiles share one body.
  auto softmax_pv = [&](int kt, int buf, f32x16 (&sacc)[KB], bool masked) {
    constexpr bool GENERAL = BIAS || SOFTCAP;
    const T *vl = vlds[buf];
    const int j0 = kt * BN;
    auto allowed = [&](int j) {
      bool ok = j >= lo && j < hi;
      if (p.causal && j > row_pos) ok = false;
      if (p.window > 0 && j < row_pos - p.window + 1) ok = false;
      return ok;
    };
    if (GENERAL) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int jb = j0 + kb * 32 + 8 * q4 + 4 * half;  // 4 consecutive keys
          float bv[4] = {0.f, 0.f, 0.f, 0.f};
          if (BIAS) {
            const uint2 raw = BPRE ? bcur[BPRE ? kb : 0][q4] : bias4(jb);
            bv[0] = lo16<T>(raw.x); bv[1] = hi16<T>(raw.x);
            bv[2] = lo16<T>(raw.y); bv[3] = hi16<T>(raw.y);
          }
          uint32_t mw = 0x01010101u;  // BOOL attn_mask bytes of the 4 keys
          if (MASK) mw = mask4(jb);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float t;
            if (SOFTCAP) {
              const float x2 = BIAS ? __builtin_fmaf(sacc[kb][4 * q4 + e], cap_a, bv[e] * cap_b)
                                    : sacc[kb][4 * q4 + e] * cap_a;
              // saturates to +-c without NaN (rcp of +inf is 0)
              t = __builtin_fmaf(__builtin_amdgcn_rcpf(ex2(x2) + 1.0f), -2.0f * cap_l2, cap_l2);
            }
            else t = (sacc[kb][4 * q4 + e] * p.scale + bv[e]) * kLog2e;
            // a false mask element excludes the key after the score pipeline
            sacc[kb][4 * q4 + e] = ((mw >> (8 * e)) & 0xffu) ? t : kNegInf;
          }
        }
    }
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          float t = sacc[kb][r];
          if (p.pad_add && j >= s.pad) t += GENERAL ? mfv_l2 : mfv_raw;
          sacc[kb][r] = allowed(j) ? t : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_halves(mx);
    if (!GENERAL) mx *= sl;
    const float m_new = fmaxf(m, mx);
    const bool grow = m_new > m + kRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? ex2(m - m_new) : 1.0f;
      m = grow ? m_new : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    const float mu = m == kNegInf ? 0.f : m;
    // P in 16-key steps, each feeding its PV MFMAs at once, so the matrix
    // core starts while the VALU computes the next step's exponentials.
    // Lane half h supplies keys 16st + {4h..4h+3, 8+4h..8+4h+3}.
    float lsum = 0.f;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      vec8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = sacc[st >> 1][8 * (st & 1) + e];
        const float pv = GENERAL ? ex2(x - mu) : ex2(__builtin_fmaf(x, sl, -mu));
        lsum += pv;
        pb[e] = (T)pv;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 32 + col;
        const int swz = 2 * (db & (NCH_V / 2 - 1));  // uniform across the instruction
        const vec8 a = *(const vec8 *)&vl[d * VST + (((2 * st + half) ^ swz) * 8)];
        o[db] = mma(a, pb, o[db]);
      }
    }
    l += lsum;
  };

  if (kt0 < kt1) {
    load_k(kt0);
    load_v(kt0);
    if (BPRE) load_bias(kt0, bcur);
    store_k(kt0, 0);
    store_v(kt0, 0);
  }
  __syncthreads();
  // The next tile's loads go out first and land in the other LDS buffer
  // after this tile's compute, so a full tile (and the other workgroup on the
  // CU) covers their latency.
  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) {
      load_k(kt + 1);
      load_v(kt + 1);
      if (BPRE) load_bias(kt + 1, bnext);
    }
    if (wave_active) {
      f32x16 sacc[KB];
      qk(buf, sacc);
      const int j0 = kt * BN;
      const bool need_mask = (p.causal && j0 + BN - 1 > pos_min) ||
                             (p.window > 0 && j0 < pos_max - p.window + 1) || j0 + BN > hi ||
                             j0 < lo || (p.pad_add && j0 + BN > s.pad);
      softmax_pv(kt, buf, sacc, need_mask);
    }
    if (more) {
      store_k(kt + 1, buf ^ 1);
      store_v(kt + 1, buf ^ 1);
      if (BPRE) {
#pragma unroll
        for (int kb = 0; kb < (BPRE ? KB : 1); ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) bcur[kb][q4] = bnext[kb][q4];
      }
    }
    __syncthreads();
  }

  // ---- present rows of the owned keys, from the last two LDS tiles ----
  if (fuse_end && kt0 < kt1) {
    const int n_own = own_hi - own_lo;
    for (int t = tid; t < n_own * CH; t += kThreads) {
      const int j = own_lo + t / CH, cc = t % CH;
      const int kt = j / BN, bi = (kt - kt0) & 1, r = j - kt * BN;
      *(uint4 *)((char *)pres_k + ((uint32_t)j * D + cc * 8u) * sizeof(T)) =
          *(const uint4 *)&klds[bi][r * KST + cc * 8];
      // V row r from V^T: element d sits at its row's swizzled key slot
      const int slot = 16 * (r >> 4) + 4 * quad_slot((r >> 2) & 3) + (r & 3);
      uint16_t e8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = cc * 8 + e;
        const int chunk = (slot >> 3) ^ (2 * ((d >> 5) & (NCH_V / 2 - 1)));
        e8[e] = __builtin_bit_cast(uint16_t, vlds[bi][d * VST + chunk * 8 + (slot & 7)]);
      }
      uint4 row;
      row.x = e8[0] | ((uint32_t)e8[1] << 16);
      row.y = e8[2] | ((uint32_t)e8[3] << 16);
      row.z = e8[4] | ((uint32_t)e8[5] << 16);
      row.w = e8[6] | ((uint32_t)e8[7] << 16);
      *(uint4 *)((char *)pres_v + ((uint32_t)j * D + cc * 8u) * sizeof(T)) = row;
    }
  }

  // ---- epilogue: combine halves, sink, normalise, store ----
  const float l_tot = sum_halves(l);
  if (!row_ok) return;
  float inv = 0.f;
  if (m != kNegInf) {
    float lt = l_tot;
    if (p.sink) {
      const float z = (float)((const T *)p.sink)[row_h] * kLog2e;
      if (z > m) {
        const float a = ex2(m - z);
        lt = lt * a + 1.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= a;
      } else {
        lt += ex2(z - m);
      }
    }
    inv = 1.0f / lt;
  }
  T *yr = (T *)p.y + b * p.y_sb + (int64_t)row_i * p.y_ss + row_h * p.y_sh;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = db * 32 + 8 * q4 + 4 * half;
      typename FV<T>::v4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (T)(o[db][4 * q4 + e] * inv);
      *(typename FV<T>::v4 *)&yr[d] = v4;
    }
}

int gh_for(int G) {
  for (int gh = 32; gh >= 1; gh >>= 1)
    if (G % gh == 0) return gh;
  return 1;
}

template <typename T, int D>
hipError_t launch_td(const Params &p, const FPlan &pl, hipStream_t st) {
  const int64_t n = (int64_t)p.B * p.Hkv * pl.n_hg * pl.n_qt;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(kThreads);
  const int bm = p.mask ? 2 : (p.bias ? 1 : 0);
  const bool cap = p.softcap > 0.f;
#define OLK_FLASH(BMV, CAPV) hipLaunchKernelGGL((flash_fwd_kernel<T, D, BMV, CAPV>), grid, block, 0, st, p, pl)
  if (bm == 2) { if (cap) OLK_FLASH(2, true); else OLK_FLASH(2, false); }
  else if (bm == 1) { if (cap) OLK_FLASH(1, true); else OLK_FLASH(1, false); }
  else { if (cap) OLK_FLASH(0, true); else OLK_FLASH(0, false); }
#undef OLK_FLASH
  return hipGetLastError();
}

}  // namespace

// Whether the prefill kernel can rotate Q itself (do_rotary): split halves
// over the whole head, or interleaved pairs over a multiple of 8 dims, with
// cos/sin rows aligned for 16-byte (8-byte) loads.
bool flash_rotates_q(const Params &p) {
  if (p.op != OP_GQA || !p.cos_cache || !p.sin_cache || p.rot_dim <= 0) return false;
  const uintptr_t al = p.rot_inter ? 7 : 15;
  if ((((uintptr_t)p.cos_cache | (uintptr_t)p.sin_cache) & al) != 0) return false;
  if (p.rot_inter) return p.rot_dim % 8 == 0 && (p.rot_dim / 2) % 4 == 0;
  return p.rot_dim == p.D && (p.rot_dim / 2) % 8 == 0;
}

// Whether the prefill kernel writes the present rows of the new keys itself.
bool flash_fuses_present(const Params &p) {
  return p.op == OP_GQA && p.present_k != nullptr && p.present_v != nullptr;
}

hipError_t launch_flash(const Params &p, int dtype, hipStream_t st) {
  FPlan pl;
  pl.GH = gh_for(p.G);
  pl.n_hg = p.G / pl.GH;
  pl.QW = kSlots / pl.GH;
  pl.n_qt = (p.S + pl.QW - 1) / pl.QW;
  const int n_bg = p.B * p.Hkv * pl.n_hg;
  pl.xcd_remap = n_bg % 8 == 0 ? 1 : 0;
  pl.bias_vec = (p.bias_si % 4 == 0 && p.bias_sh % 4 == 0 && p.bias_sb % 4 == 0 &&
                 ((uintptr_t)p.bias & 7) == 0) ? 1 : 0;
  pl.mask_vec = (p.mask_si % 4 == 0 && p.mask_sh % 4 == 0 && p.mask_sb % 4 == 0 &&
                 ((uintptr_t)p.mask & 3) == 0) ? 1 : 0;
  pl.fuse_present = flash_fuses_present(p) ? 1 : 0;
  if (dtype == DT_BF16)
    return p.D == 64 ? launch_td<bf16, 64>(p, pl, st) : launch_td<bf16, 128>(p, pl, st);
  return p.D == 64 ? launch_td<f16, 64>(p, pl, st) : launch_td<f16, 128>(p, pl, st);
}

}  // namespace olk
