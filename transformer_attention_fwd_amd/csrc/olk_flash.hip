// Prefill attention forward for gfx950 (CDNA4): f16/bf16 inputs, head size 64,
// 128 or 256, fp32 accumulation.
//
// Computes Y = Softmax((Q K^T) * scale + bias) V with grouped KV heads, causal /
// local-window / length masks, softcap, head_sink and the present outputs of
// the GroupQueryAttention, MultiHeadAttention and ai.onnx Attention contracts
// (onnx-light-cpu Python API "Custom operators"; onnx-light reference kernels
// header page, "class Attention").  The decomposition is ours:
//
// * A workgroup is 4 wavefronts x 32 row slots; two workgroups share a CU
//   (two wavefronts per SIMD, so one wave's MFMAs overlap the other's softmax;
//   three at head size 64, and for the plain form at head size 128).
//   Slots pack the GH query heads sharing one KV head with consecutive queries
//   (slot -> (query, head)): every K/V tile in LDS serves the whole head group.
// * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16.  In the S^T
//   accumulator layout a lane owns one row slot and half of a tile's keys, so
//   the softmax max/sum are in-lane plus one exchange with lane ^ 32, and P^T
//   is already the B operand of the PV MFMA.
// * K and V tiles go from memory straight into LDS (buffer_load_dwordx4 ...
//   lds for tiles from one source, else global_load_lds_dwordx4: 16 bytes per
//   lane, no staging registers), unpadded rows with the 16-byte
//   chunks of each row XOR-swizzled by a function of the row, one function
//   for K (the QK^T operand reads 16 rows at one chunk per 16 lanes) and one
//   for V.  The V^T operand of PV is read with ds_read_b64_tr_b16 from the
//   row-major V tile: each transposed read hands a lane 4 consecutive keys of
//   its head dimension, in the k order in which the accumulator supplies P^T.
// * Keys advance in tiles of 64 (32 for the plain form at head size 128, so
//   that three workgroups fit a CU's LDS), double-buffered in LDS with one barrier per
//   tile; the next tile's loads are in flight while the current tile
//   computes.  The buffers are separate LDS variables and the key loop is
//   unrolled by two, so the compiler can tell the loads landing in one
//   buffer from the reads of the other.  A tile's bias / BOOL-mask words are
//   loaded before the next tile's K/V (the memory counter is in order).
// * S^T is accumulated block-major (32 keys at a time), so the first block's
//   row max can start beside the second block's MFMAs.
// * Online softmax in the exp2 domain, the scale folded into the exponent's
//   FMA; per-key masks only on boundary tiles, written as -inf in place.  O
//   is rescaled only when a row's running max grows by more than 2^8 (the
//   final division uses the same max, so the result is unchanged).  The row
//   sum adds the P values as rounded for the PV product (packed dot
//   products), so Y is an exactly normalised mean of V rows.
// * GroupQueryAttention present rows of the new keys are stored by the
//   workgroup whose queries sit at those positions, copied from LDS: with
//   causal masking from its last two tiles after the loop, otherwise while
//   the owning tile is resident.
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
// s_waitcnt immediate for lgkmcnt(0) only (vmcnt 63, expcnt 7)
constexpr int kWaitLgkmcnt0 = 0xC07F;
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

// acc + the sum of the 8 elements of p, as packed 2-element dot products with
// ones (v_dot2c_f32_{bf16,f16}: four instructions instead of eight adds)
__device__ __forceinline__ float add8(const bf16x8 &p, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[2 * w], p[2 * w + 1]}, one, acc, false);
  return acc;
}
__device__ __forceinline__ float add8(const f16x8 &p, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2(f16x2{p[2 * w], p[2 * w + 1]}, one, acc, false);
  return acc;
}

// 16 bytes from global memory straight into LDS: lane l's bytes land at
// lds + 16 l (the LDS address is the same for every lane of the instruction)
__device__ __forceinline__ void load_lds16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// The same through a buffer descriptor (buffer_load_dwordx4 ... lds): lane
// l's 16 bytes from byte off (per lane) of the descriptor's range land at
// lds + 16 l.  Unlike global_load_lds this form issues without waiting while
// MFMAs stream elsewhere on the CU.  Written as inline asm (the builtin for it
// is taken to alias every LDS access and made the compiler wait for these
// loads ahead of unrelated LDS reads): the compiler does not count these
// loads, so every read of their destination follows the kernel's own
// vmcnt(0) wait and barrier.  M0 holds the LDS base; the ISA asks for one wait
// state between an M0 write and a load into LDS.
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, uint32_t off, const void *lds) {
  const uint32_t la = (uint32_t)(size_t)(__attribute__((address_space(3))) const void *)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(off), "s"(r), "s"(la) : "memory", "m0");
}
// raw buffer descriptor at base: no stride, 2^31 - 1 bytes, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}

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

struct FPlan {
  int GH, n_hg, QW, n_qt;
  int ghs;           // log2 GH (GH is a power of two)
  int qs;            // Q pre-scaled, bias in the accumulator (see flash_fwd_kernel)
  int xcd_remap;
  int bias_vec;
  int mask_vec;      // BOOL mask rows are 4-byte aligned
  int fuse_present;
  int fixm;          // softcap with bf16 P: fixed exponent offset 0 instead of a running max
};

// Wavefronts per SIMD the register budget is sized for: three at head size 64
// (more workgroups resident when a grid holds few query tiles; four for the
// softcap form without bias or mask, 128 registers: 5 % faster than three;
// the BOOL-mask form needs more registers and keeps two); at head size 128
// three without bias or mask (at most 168 registers, with 32-key tiles so
// that three workgroups' K/V buffers fit the LDS; measured 1-2 % faster than
// two with 64-key tiles, 8 % with softcap) and two otherwise; one at 256
// (whose K/V double buffers take 128 KB of LDS: one workgroup per CU).
template <int D, int BM, bool CAP>
constexpr int kOcc = D == 256                   ? 1
                     : (D == 64 && BM == 0 && CAP) ? 4
                     : ((D == 64 && BM != 2) || (D == 128 && BM == 0)) ? 3 : 2;

// BM: 0 no bias, 1 attn_bias, 2 attn_mask (BOOL, or MultiHeadAttention's int32
// binary mask) with attn_bias, 3 attn_mask without attn_bias (no bias terms in
// the score pipeline).
// QS (attn_bias without softcap, the scale an exact power of two): Q is
// multiplied by the scale as it is loaded (exact: a change of exponent) and
// the bias seeds the QK^T accumulator, so the matrix cores add it and the
// scores leave the MFMAs as (Q K^T) * scale + bias, in natural-log units.
template <typename T, int D, int BM, bool SOFTCAP, bool QS = false>
__global__ __launch_bounds__(kThreads, (kOcc<D, BM, SOFTCAP>)) void flash_fwd_kernel(Params p, FPlan pl) {
  typedef typename FV<T>::v8 vec8;
  static_assert(!QS || (BM == 1 && !SOFTCAP), "the bias seeds the accumulator only without softcap");
  constexpr bool BIAS = BM == 1 || BM == 2;  // the score epilogue reads a bias row
  constexpr bool MASK = BM >= 2;
  constexpr bool WORDS = BM != 0;            // bias or mask words per tile
  constexpr int CH = D / 8;             // 16-byte chunks per K/V row
  constexpr int BN = (D == 128 && kOcc<D, BM, SOFTCAP> == 3) ? 32 : 64;  // keys per tile
  constexpr int KB = BN / 32;           // 32-key blocks per tile
  constexpr int NST = BN / 16;          // 16-key PV steps per tile
  constexpr int NKS = D / 16;           // QK^T k-steps
  constexpr int NDB = D / 32;           // 32-wide output blocks
  constexpr int RB = D * 2;             // bytes per K / V row in LDS (unpadded)
  // Double buffers as four separate variables.  With the key loop unrolled by
  // two (UNROLL2) each access names one of them, so the wait-count analysis
  // can tell the loads landing in one buffer from the reads of the other and
  // does not wait for the next tile's loads before the first read of this
  // one.  The forms whose registers do not allow the unrolled body (head
  // size 64 at three wavefronts per SIMD, BOOL mask with softcap, bias or
  // mask at head size 256) select the buffers at run time and keep that wait.
  constexpr bool UNROLL2 = !(MASK && SOFTCAP) && !(D == 64 && SOFTCAP) && !(D == 256 && BM != 0);
  __shared__ __attribute__((aligned(16))) T klds0[BN * D];
  __shared__ __attribute__((aligned(16))) T klds1[BN * D];
  __shared__ __attribute__((aligned(16))) T vlds0[BN * D];
  __shared__ __attribute__((aligned(16))) T vlds1[BN * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
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
  // short masks (a bias row, a mask row) exclude the keys beyond their columns
  if (BIAS && p.bias) hi = min(hi, p.bias_cols);
  if (MASK) hi = min(hi, p.mask_cols);
  const int lo = p.window > 0 ? max(0, pos_min - p.window + 1) : 0;
  // no key tile at all when no key is allowed (every row then outputs 0)
  const int kt0 = lo / BN, kt1 = hi > lo ? (hi + BN - 1) / BN : kt0;

  // ---- this lane's row slot ----
  const int slot = wave * 32 + col;
  const int row_i = i0 + (slot >> pl.ghs);
  const int row_h = g * p.G + hg * pl.GH + (slot & (pl.GH - 1));
  const bool row_ok = row_i < p.S;
  const int row_pos = s.qoff + row_i;
  // the keys this row slot may attend form one interval [a_lo, a_lo + a_w):
  // the workgroup's range, cut by the causal and window limits of its position
  const int a_lo = p.window > 0 ? max(lo, row_pos - p.window + 1) : lo;
  const int a_hi = p.causal ? min(hi, row_pos + 1) : hi;
  const uint32_t a_w = a_hi > a_lo ? (uint32_t)(a_hi - a_lo) : 0u;
  const bool wave_active = i0 + ((wave * 32) >> pl.ghs) < p.S;

  // ---- Q^T operand (B of S^T = K Q^T): slot col, d = 16 ks + 8 half + e ----
  vec8 qreg[NKS];  // filled by load_q below, after the first tile's loads are issued
  auto load_q = [&]() __attribute__((always_inline)) {
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
      if constexpr (QS) {
        // q * scale, scale = 2^k: only the exponent changes
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[ks][e] = (T)((float)qreg[ks][e] * p.scale);
      }
    }
  }
  };

  // ---- staging: K and V tiles go from memory straight into LDS ----
  // A direct load writes 16 bytes per lane at consecutive LDS addresses (1 KB
  // per instruction = RPL rows); each lane picks which 16-byte chunk of its
  // row it loads, so a row's chunks are stored XOR-swizzled:
  //  K: slot p of row r holds chunk p ^ fk(r); the QK^T operand reads (16
  //     rows at one chunk per 16 lanes) then hit 16 different bank groups;
  //  V: slot p of row r holds chunk p ^ fv(r); the transposed PV operand reads
  //     (4 rows x 64 bytes per 32 lanes) hit 64 different banks.
  // Keys outside [lo, hi) load the nearest row inside it instead (caller data,
  // finite; their scores are masked, so their P is exactly 0).
  constexpr int RPL = 1024 / RB;        // rows per load instruction
  constexpr int NLD = BN / (4 * RPL);   // load instructions per wavefront per tile and matrix
  auto fk = [](int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); };
  auto fv = [](int r) { return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  // per lane: tile row and byte offsets inside a tile of new K/V rows
  // (strides k_ss / v_ss), fixed for the kernel
  int lrow[NLD];
  uint32_t kcb[NLD], vcb[NLD];        // byte offset of the loaded chunk inside its row
  uint32_t kon[NLD], von[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int r = (wave * NLD + i) * RPL + lane / CH, pch = lane % CH;
    lrow[i] = r;
    kcb[i] = 16u * (uint32_t)(pch ^ fk(r));
    vcb[i] = 16u * (uint32_t)(pch ^ fv(r));
    kon[i] = (uint32_t)r * (uint32_t)p.k_ss * (uint32_t)sizeof(T) + kcb[i];
    von[i] = (uint32_t)r * (uint32_t)p.v_ss * (uint32_t)sizeof(T) + vcb[i];
  }
  const T *kpast = (const T *)p.past_k + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *vpast = (const T *)p.past_v + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *knew = (const T *)p.k + b * p.k_sb + g * p.k_sh;
  const T *vnew = (const T *)p.v + b * p.v_sb + g * p.v_sh;
  const bool fuse = pl.fuse_present && hg == 0;
  const int own_lo = s.past + i0, own_hi = s.past + i_last + 1;
  // Causal: the owned rows are the last keys the loop stages (at most BN of
  // them), so both LDS buffers still hold them afterwards and present is
  // written once the loop is done; otherwise each owned row is copied from
  // LDS while its tile is resident.
  const bool fuse_end = fuse && p.causal && pl.QW <= BN;
  const bool fuse_loop = fuse && !fuse_end;
  T *pres_k = (T *)p.present_k + ((int64_t)b * p.Hkv + g) * p.T * D;
  T *pres_v = (T *)p.present_v + ((int64_t)b * p.Hkv + g) * p.T * D;

  auto issue_loads = [&](int kt, T *kdst, T *vdst) __attribute__((always_inline)) {
    const int j0 = kt * BN;
    char *kl = (char *)kdst + wave * NLD * 1024;
    char *vl = (char *)vdst + wave * NLD * 1024;
    const bool full = j0 >= lo && j0 + BN <= hi;
    if (full && s.vsrc != s.src && (j0 >= s.src || j0 + BN <= s.src) &&
        (j0 >= s.vsrc || j0 + BN <= s.vsrc)) {
      // K and V from different sources (V of the new keys still in V, every
      // K row in the past buffer): each tile from one source per matrix
      const bool kn = j0 >= s.src, vn = j0 >= s.vsrc;
      const __amdgpu_buffer_rsrc_t rk =
          rsrc_of(kn ? knew + (int64_t)(j0 - s.src) * p.k_ss : kpast + (int64_t)j0 * D);
      const __amdgpu_buffer_rsrc_t rv =
          rsrc_of(vn ? vnew + (int64_t)(j0 - s.vsrc) * p.v_ss : vpast + (int64_t)j0 * D);
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint32_t ro = (uint32_t)lrow[i] * (uint32_t)(D * sizeof(T));
        buf_lds16(rk, kn ? kon[i] : ro + kcb[i], kl + i * 1024);
        buf_lds16(rv, vn ? von[i] : ro + vcb[i], vl + i * 1024);
      }
    } else if (full && s.vsrc == s.src && (j0 >= s.src || j0 + BN <= s.src)) {
      // the whole tile from one source: a descriptor based at the tile's
      // first row plus the fixed 32-bit lane offsets of that source
      if (j0 >= s.src) {
        const __amdgpu_buffer_rsrc_t rk = rsrc_of(knew + (int64_t)(j0 - s.src) * p.k_ss);
        const __amdgpu_buffer_rsrc_t rv = rsrc_of(vnew + (int64_t)(j0 - s.src) * p.v_ss);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          buf_lds16(rk, kon[i], kl + i * 1024);
          buf_lds16(rv, von[i], vl + i * 1024);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rk = rsrc_of(kpast + (int64_t)j0 * D);
        const __amdgpu_buffer_rsrc_t rv = rsrc_of(vpast + (int64_t)j0 * D);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const uint32_t ro = (uint32_t)lrow[i] * (uint32_t)(D * sizeof(T));  // past rows are dense
          buf_lds16(rk, ro + kcb[i], kl + i * 1024);
          buf_lds16(rv, ro + vcb[i], vl + i * 1024);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int j = j0 + lrow[i];
        const int jj = j < lo ? lo : (j >= hi ? hi - 1 : j);
        const bool nw = jj >= s.src, nwv = jj >= s.vsrc;
        const char *kr = (const char *)(nw ? knew + (int64_t)(jj - s.src) * p.k_ss : kpast + (int64_t)jj * D);
        const char *vr = (const char *)(nwv ? vnew + (int64_t)(jj - s.vsrc) * p.v_ss : vpast + (int64_t)jj * D);
        load_lds16(kr + kcb[i], kl + i * 1024);
        load_lds16(vr + vcb[i], vl + i * 1024);
      }
    }
  };
  // present rows of the owned keys of tile kt (resident in kbuf / vbuf);
  // only V when K is already there (the rotary pre-pass wrote the rotated K)
  const bool pres_k_on = p.present_k != nullptr;
  auto copy_owned = [&](int kt, const T *kbuf, const T *vbuf) __attribute__((always_inline)) {
    const int j0 = kt * BN;
    const int a = max(own_lo, j0), e = min(own_hi, j0 + BN);
    for (int t = tid; t < (e - a) * CH; t += kThreads) {
      const int j = a + t / CH, cc = t % CH, r = j - j0;
      if (pres_k_on)
        *(uint4 *)((char *)pres_k + ((uint32_t)j * D + cc * 8u) * sizeof(T)) =
            *(const uint4 *)((const char *)kbuf + r * RB + 16 * (cc ^ fk(r)));
      *(uint4 *)((char *)pres_v + ((uint32_t)j * D + cc * 8u) * sizeof(T)) =
          *(const uint4 *)((const char *)vbuf + r * RB + 16 * (cc ^ fv(r)));
    }
  };
  // K operand offsets inside a tile (row kb * 32 + col; fk does not depend on kb).
  // The swizzle XORs the chunk index and the k-step picks chunk 2 ks + half,
  // so koff[ks] = koff[0] ^ 32 ks (the chunk bits lie below the row's byte
  // offset); likewise voff[db] = voff[0] ^ 64 db.  XOFF forms keep only the
  // first offset live and form the others with one XOR per read: fewer
  // registers (the softcap forms at head sizes 128 and 64 then fit three and
  // four wavefronts per SIMD, and the head-size-256 bias / mask forms stop spilling) for a
  // few VALU instructions, which cost 1-3 % where registers were not short.
  constexpr bool XOFF = (D <= 128 && BM == 0 && SOFTCAP) || (D == 256 && BM != 0 && !QS);
  uint32_t koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = (uint32_t)(col * RB + 16 * ((2 * ks + half) ^ fk(col)));
  // V^T operand (transposed reads): lane (group g4 = lane / 16, j = lane % 16)
  // addresses row 4 half + j / 4 (+ 16 st + 8 rd), dims 32 db + 16 (g4 & 1) + 4 (j & 3);
  // the read hands lane l dim 32 db + (l & 31) of 4 consecutive keys
  uint32_t voff[NDB];
  {
    const int j = lane & 15, g4 = lane >> 4, q = j >> 2;
    const int t2 = 2 * (g4 & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      voff[db] = (uint32_t)((4 * half + q) * RB + 16 * ((4 * db + t2) ^ fv(4 * half + q)) + 8 * (j & 1));
  }

  // exponent factor of raw scores (with QS the scale is already in Q)
  const float sl = QS ? kLog2e : p.scale * kLog2e;
  const bool scale_pos = p.scale > 0.f;
  // softcap in the log2 domain: c tanh(u) = c - 2c / (e^{2u} + 1) with
  // u = (s scale + bias) / c; e^{2u} = 2^(s cap_a + bias cap_b)
  const float inv_cap = SOFTCAP ? 1.0f / p.softcap : 0.f;
  const float cap_l2 = p.softcap * kLog2e;
  const float cap_b = 2.0f * kLog2e * inv_cap, cap_a = p.scale * cap_b;
  const float mfv_l2 = p.mfv * kLog2e;
  const float mfv_raw = QS ? p.mfv : p.mfv / p.scale;  // the same offset in raw-score units (scale > 0)
  const T *bias_row = BIAS ? (const T *)p.bias + b * p.bias_sb + row_h * p.bias_sh +
                                 (int64_t)(row_ok ? row_i : 0) * p.bias_si
                           : nullptr;

  // 4 bias values of keys jb..jb+3 as raw 16-bit pairs (zeros past the bias
  // columns); full: the whole tile lies inside the columns and rows are
  // aligned (the same for every lane, so no lane takes the other path)
  auto bias4 = [&](int jb, bool full) {
    if (MASK && !p.bias) return make_uint2(0, 0);
    if (full) return *(const uint2 *)(bias_row + jb);
    uint16_t e4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      e4[e] = jb + e < p.bias_cols ? __builtin_bit_cast(uint16_t, bias_row[jb + e]) : (uint16_t)0;
    return make_uint2(e4[0] | ((uint32_t)e4[1] << 16), e4[2] | ((uint32_t)e4[3] << 16));
  };
  // attn_mask of keys jb..jb+3 of this row slot as 4 flag bytes (nonzero =
  // attend; 0 past the mask's columns): BOOL masks are bytes, MultiHeadAttention
  // binary masks int32 (mask_kind 2)
  const bool mask_i32 = MASK && p.mask_kind == 2;
  const int64_t mask_e = MASK ? b * p.mask_sb + row_h * p.mask_sh +
                                    (int64_t)(row_ok ? row_i : 0) * p.mask_si
                              : 0;
  const uint8_t *mask_row = MASK ? (const uint8_t *)p.mask + mask_e : nullptr;
  const int32_t *mask_row32 = MASK ? (const int32_t *)p.mask + mask_e : nullptr;
  auto mask4 = [&](int jb, bool full) {
    if (mask_i32) {
      if (full) {
        const uint4 v = *(const uint4 *)(mask_row32 + jb);
        return (uint32_t)(v.x != 0) | ((uint32_t)(v.y != 0) << 8) | ((uint32_t)(v.z != 0) << 16) |
               ((uint32_t)(v.w != 0) << 24);
      }
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (jb + e < p.mask_cols) w |= (uint32_t)(mask_row32[jb + e] != 0) << (8 * e);
      return w;
    }
    if (full) return *(const uint32_t *)(mask_row + jb);
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (jb + e < p.mask_cols) w |= (uint32_t)mask_row[jb + e] << (8 * e);
    return w;
  };
  // At head size 64 with two wavefronts per SIMD, or with QS (whose scores
  // need fewer registers), the bias of the next tile is prefetched with its
  // K/V.
  // Otherwise a tile's bias and mask words are loaded at the start of the
  // tile, before the next tile's K/V loads: the memory counter is in order,
  // so waiting for loads issued after those would wait for them too.
  // BLDS (QS at head size 64, one query per row slot): the next tile's bias
  // rows go from memory straight into a per-wavefront LDS tile (8 rows x 128
  // bytes per instruction) and each lane reads its values from there in the
  // accumulator layout; gathered per lane they took 8 bytes from each of 32
  // rows per instruction
  constexpr bool BLDS = QS && D == 64;
  constexpr bool BPRE = BIAS && D == 64 && kOcc<D, BM, SOFTCAP> == 2 && !BLDS;
  typedef uint2 BiasWords[BIAS ? KB : 1][4];
  typedef uint32_t MaskWords[MASK ? KB : 1][4];
  BiasWords bcur, bnext;
  // BLDS: bias of a wavefront's 32 row slots for one tile, 128 bytes per row;
  // the 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 7), so the
  // 8-byte reads below (32 rows at one chunk) spread over the banks
  __shared__ __attribute__((aligned(16))) char blds[BLDS ? 4 * 32 * 128 : 16];
  const T *bias_g = BIAS ? (const T *)p.bias + b * p.bias_sb + (g * p.G + hg * pl.GH) * p.bias_sh
                         : nullptr;
  auto bias_rows_whole = [&](int kt) { return pl.bias_vec && kt * BN + BN <= p.bias_cols; };
  auto load_bias_rows = [&](int kt) __attribute__((always_inline)) {
    if constexpr (BLDS) {
      // lane l of instruction t lands in slot l % 8 of row 8 t + l / 8 (one
      // query per row slot, clamped to the last query)
      char *bl = blds + wave * 32 * 128;
      const __amdgpu_buffer_rsrc_t rb = rsrc_of(bias_g + kt * BN);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 8 * t + (lane >> 3);
        const int ri = min(i0 + wave * 32 + r, p.S - 1);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        buf_lds16(rb, (uint32_t)(((int64_t)ri * p.bias_si + 8 * c) * (int64_t)sizeof(T)), bl + t * 1024);
      }
    }
  };
  auto bias_from_lds = [&]() __attribute__((always_inline)) {
    if constexpr (BLDS) {
      const char *bl = blds + wave * 32 * 128 + col * 128;
      const int f = (col >> 1) & 7;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          bcur[kb][q4] = *(const uint2 *)(bl + 16 * ((4 * kb + q4) ^ f) + 8 * half);
    }
  };
  auto load_bias = [&](int kt, BiasWords &bb) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      // one uniform choice for the tile (per-call choices leave the
      // compiler unable to count the loads still in flight)
      if (pl.bias_vec && kt * BN + BN <= p.bias_cols) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) bb[kb][q4] = bias4(kt * BN + kb * 32 + 8 * q4 + 4 * half, true);
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) bb[kb][q4] = bias4(kt * BN + kb * 32 + 8 * q4 + 4 * half, false);
      }
    }
  };
  auto load_mask = [&](int kt, MaskWords &mw) __attribute__((always_inline)) {
    if constexpr (MASK) {
      if (pl.mask_vec && kt * BN + BN <= p.mask_cols) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) mw[kb][q4] = mask4(kt * BN + kb * 32 + 8 * q4 + 4 * half, true);
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) mw[kb][q4] = mask4(kt * BN + kb * 32 + 8 * q4 + 4 * half, false);
      }
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // With softcap every score lies in [-c, c] (log2 units: +-c log2 e), so for
  // c log2 e <= 100 the exponentials 2^s need no running max: bf16 / fp32
  // hold 2^-100..2^100 and a row sum of them (fixm; the result is the same
  // weighted mean, only the common factor differs).
  const bool fixm = SOFTCAP && pl.fixm;
  float m = fixm ? 0.f : kNegInf, l = 0.f;

  // S^T of one tile: KB blocks of 32 keys; seed: the accumulators' start
  // (zeros, or with QS the tile's bias values)
  auto qk = [&](const T *kbuf, f32x16 (&sacc)[KB], const f32x16 (&seed)[KB]) __attribute__((always_inline)) {
    const char *kl = (const char *)kbuf;
    uint32_t koff0 = koff[0];
    // (an opaque copy per tile, so the XORs are not hoisted out of the loop)
    if constexpr (XOFF) asm volatile("" : "+v"(koff0));
    // block-major: the first 32 keys' scores are final while the second
    // block's MFMAs run, so their row max can start (each chain keeps its
    // k order, so the sums are the same)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const vec8 a = *(const vec8 *)(kl + kb * 32 * RB + (XOFF ? koff0 ^ (32u * ks) : koff[ks]));
        sacc[kb] = mma(a, qreg[ks], ks == 0 ? seed[kb] : sacc[kb]);
      }
    }
    // schedule: six operand reads in flight ahead of the MFMAs (four and
    // eight measured 1-2 % slower at head size 128)
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // 0x100: LDS reads
#pragma unroll
    for (int i = 0; i < NKS * KB - 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };

  // Softmax and PV of one tile.  With bias or softcap (GENERAL) the scores
  // are rewritten into the log2 domain; otherwise they stay raw (scale > 0,
  // folded into the exponent's FMA) and masking only writes -inf in place, so
  // masked and unmasked tiles share one body.
  // With softcap the scores are kept as r = 1 / (e^{2u} + 1) in [0, 1]: the
  // capped score is t = c' - 2 c' r (c' = c log2 e), decreasing in r, so the
  // row max is taken as a min over r (masked keys: r = +inf, t = -inf) and
  // the exponent t - m folds into one FMA, fma(r, -2c', c' - m).  (Softcap
  // never meets MultiHeadAttention's additive filter value: that operator
  // has no softcap.)
  auto softmax_pv = [&](int kt, const T *vbuf, f32x16 (&sacc)[KB], bool masked, const BiasWords &bwt,
                        const MaskWords &mwt) __attribute__((always_inline)) {
    constexpr bool GENERAL = (WORDS && !QS) || SOFTCAP;
    constexpr float kOut = SOFTCAP ? __builtin_huge_valf() : kNegInf;  // an excluded key
    const char *vl = (const char *)vbuf;
    const int j0 = kt * BN;
    uint32_t voff0 = voff[0];
    if constexpr (XOFF) asm volatile("" : "+v"(voff0));
    const auto vo = [&](int db) { return XOFF ? voff0 ^ (64u * db) : voff[db]; };
    if (GENERAL) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int jb = j0 + kb * 32 + 8 * q4 + 4 * half;  // 4 consecutive keys
          float bv[4] = {0.f, 0.f, 0.f, 0.f};
          if (BIAS) {
            const uint2 raw = BPRE ? bcur[kb][q4] : bwt[kb][q4];
            bv[0] = lo16<T>(raw.x); bv[1] = hi16<T>(raw.x);
            bv[2] = lo16<T>(raw.y); bv[3] = hi16<T>(raw.y);
          }
          uint32_t mw = 0x01010101u;  // BOOL attn_mask bytes of the 4 keys
          if constexpr (MASK) mw = mwt[kb][q4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float t;
            if (SOFTCAP) {
              const float x2 = BIAS ? __builtin_fmaf(sacc[kb][4 * q4 + e], cap_a, bv[e] * cap_b)
                                    : sacc[kb][4 * q4 + e] * cap_a;
              // r in [0, 1] without NaN (rcp of +inf is 0)
              t = __builtin_amdgcn_rcpf(ex2(x2) + 1.0f);
            }
            else t = BIAS ? (sacc[kb][4 * q4 + e] * p.scale + bv[e]) * kLog2e : sacc[kb][4 * q4 + e] * sl;
            // a false BOOL element excludes the key after the score pipeline;
            // a zero binary (int32) element adds mask_filter_value to it
            sacc[kb][4 * q4 + e] = ((mw >> (8 * e)) & 0xffu) ? t : (mask_i32 ? t + mfv_l2 : kOut);
          }
        }
    }
    if (masked) {
      // key of element r of block kb: j0 + 4 half + kb 32 + 8 (r / 4) + r % 4
      if (p.pad_add) {
        // keys from s.pad on get the filter value added: a select per score
        const int jp = j0 + 4 * half - s.pad;
        const float add = GENERAL ? mfv_l2 : mfv_raw;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][r] += jp + kb * 32 + 8 * (r >> 2) + (r & 3) >= 0 ? add : 0.f;
      }
      const int jr = j0 + 4 * half - a_lo;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[kb][r] = (uint32_t)(jr + kb * 32 + 8 * (r >> 2) + (r & 3)) < a_w ? sacc[kb][r] : kOut;
    }
    if (!fixm) {
      float mx;
      if (SOFTCAP) {
        float mn = kOut;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mn = fminf(mn, sacc[kb][r]);
        mx = __builtin_fmaf(mn, -2.0f * cap_l2, cap_l2);
      } else {
        mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      }
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
    }
    const float mu = m == kNegInf ? 0.f : m;
    const float cap_off = cap_l2 - mu;  // softcap: exponent fma(r, -2c', c' - m)
    // P in 16-key steps, each feeding its PV MFMAs at once, so the matrix
    // core starts while the VALU computes the next step's exponentials.
    // Lane half h supplies keys 16st + {4h..4h+3, 8+4h..8+4h+3}.  The row
    // sum adds the rounded P the product weighs (two chains, even / odd steps).
    float lsum2[2] = {0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      vec8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = sacc[st >> 1][8 * (st & 1) + e];
        pb[e] = (T)(SOFTCAP ? ex2(__builtin_fmaf(x, -2.0f * cap_l2, cap_off))
                            : GENERAL ? ex2(x - mu) : ex2(__builtin_fmaf(x, sl, -mu)));
      }
      lsum2[st & 1] = add8(pb, lsum2[st & 1]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // keys 16 st + 4 half + {0..3} and 16 st + 8 + 4 half + {0..3} of dim 32 db + col
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 *tr_ptr;
        const uint2 lo = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((tr_ptr)(vl + 16 * st * RB + vo(db))));
        const uint2 hi = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((tr_ptr)(vl + (16 * st + 8) * RB + vo(db))));
        const vec8 a = __builtin_bit_cast(vec8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[db] = mma(a, pb, o[db]);
      }
    }
    l += lsum2[0] + lsum2[1];
  };

  // The first tile's loads go out before the Q loads, so the two latencies
  // overlap.  Waiting for all of them here, on every path, also keeps the
  // wait-count analysis from assuming Q may still be in flight inside the
  // loop (it would then hold the first MFMA of every tile until the next
  // tile's loads had landed as well).  Direct loads write LDS behind the
  // compiler's back: the wait comes before the barrier that publishes them.
  if (kt0 < kt1) {
    issue_loads(kt0, klds0, vlds0);
    if (BPRE) load_bias(kt0, bcur);
    if (BLDS && wave_active && bias_rows_whole(kt0)) load_bias_rows(kt0);
  }
  load_q();
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  // One tile: the next tile's loads go out first and land in the other
  // buffers while this tile computes (a full tile and the other workgroup on
  // the CU cover their latency).
  auto tile = [&](int kt, const T *kc, const T *vc, T *kn, T *vn) __attribute__((always_inline)) {
    const bool more = kt + 1 < kt1;
    // present rows of this tile first: their stores count in the same
    // in-order counter, so after the word loads they would hold up the wait
    // for those words
    if (fuse_loop && kt * BN < own_hi && kt * BN + BN > own_lo) copy_owned(kt, kc, vc);
    BiasWords bwt;
    MaskWords mwt;
    if (wave_active) {
      if constexpr (BLDS) {
        if (!bias_rows_whole(kt)) load_bias(kt, bcur);  // a tile past the bias columns: per key
      } else if (!BPRE) {
        load_bias(kt, bwt);
      }
      load_mask(kt, mwt);
    }
    // (the empty asm keeps the compiler from issuing the word loads after
    // the K/V loads below)
    asm volatile("" ::: "memory");
    // the next tile's K/V; with bias or mask words the last tile reloads the
    // previous one into the buffers that hold it (unread meanwhile), so every
    // tile issues the same loads and the wait for the words below can leave
    // these in flight
    if (more || WORDS) issue_loads(more ? kt + 1 : max(kt - 1, kt0), kn, vn);
    if (more && BPRE) load_bias(kt + 1, bnext);
    if (BLDS && wave_active && bias_rows_whole(kt)) {
      bias_from_lds();
      // the reads are done before the next tile's rows overwrite them
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    }
    if (BLDS && more && wave_active && bias_rows_whole(kt + 1)) load_bias_rows(kt + 1);
    if (wave_active) {
      const int j0 = kt * BN;
      const bool need_mask = (p.causal && j0 + BN - 1 > pos_min) ||
                             (p.window > 0 && j0 < pos_max - p.window + 1) || j0 + BN > hi ||
                             j0 < lo || (p.pad_add && j0 + BN > s.pad);
      // the words have landed once at most the 2 NLD K/V loads issued after
      // them are in flight (the counter is in order)
      if constexpr (WORDS && !BPRE && !BLDS) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | (2 * NLD));
      f32x16 seed[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) seed[kb][r] = 0.f;
        if constexpr (QS) {
          // bias of keys j0 + kb 32 + 8 q4 + 4 half + e, element 4 q4 + e
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const uint2 raw = (BPRE || BLDS) ? bcur[kb][q4] : bwt[kb][q4];
            seed[kb][4 * q4 + 0] = lo16<T>(raw.x);
            seed[kb][4 * q4 + 1] = hi16<T>(raw.x);
            seed[kb][4 * q4 + 2] = lo16<T>(raw.y);
            seed[kb][4 * q4 + 3] = hi16<T>(raw.y);
          }
        }
      }
      f32x16 sacc[KB];
      qk(kc, sacc, seed);
      softmax_pv(kt, vc, sacc, need_mask, bwt, mwt);
    }
    if (more && BPRE) {
#pragma unroll
      for (int kb = 0; kb < (BIAS ? KB : 1); ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) bcur[kb][q4] = bnext[kb][q4];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  if constexpr (UNROLL2) {
    for (int kt = kt0; kt < kt1; kt += 2) {
      tile(kt, klds0, vlds0, klds1, vlds1);
      if (kt + 1 < kt1) tile(kt + 1, klds1, vlds1, klds0, vlds0);
    }
  } else {
    for (int kt = kt0; kt < kt1; ++kt) {
      const bool odd = (kt - kt0) & 1;
      tile(kt, odd ? klds1 : klds0, odd ? vlds1 : vlds0, odd ? klds0 : klds1, odd ? vlds0 : vlds1);
    }
  }

  // ---- present rows of the owned keys, from the last two LDS tiles ----
  if (fuse_end && kt0 < kt1) {
    const int kt_first = max(kt0, own_lo / BN);
    for (int kt = kt_first; kt < kt1; ++kt) {
      const bool odd = (kt - kt0) & 1;
      copy_owned(kt, odd ? klds1 : klds0, odd ? vlds1 : vlds0);
    }
  }

  // ---- epilogue: combine halves, sink, normalise, store ----
  const float l_tot = sum_halves(l);
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
    inv = lt > 0.f ? 1.0f / lt : 0.f;  // (fixm: every key masked leaves lt = 0)
  }
  // Y goes through LDS so that whole rows are stored: each wavefront writes
  // its 32 rows (row-major, 16-byte chunks XOR-swizzled by the row) into its
  // own 32 RB bytes of the K buffers (of the K and V buffers with 32-key
  // tiles, one buffer each), then CH lanes store one row (16 bytes
  // each), 64 / CH rows per instruction (lane-per-row stores of 8 bytes at a
  // time were measured to take ~4k clocks per workgroup).  Rows past S are
  // staged but not stored.
  if (fuse_end && kt0 < kt1) __syncthreads();  // the present copy read the K/V buffers
  char *ys = BN == 32 ? (char *)(wave == 0 ? klds0 : wave == 1 ? klds1 : wave == 2 ? vlds0 : vlds1)
                      : (char *)(wave < 2 ? klds0 : klds1) + (wave & 1) * 32 * RB;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      typename FV<T>::v4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (T)(o[db][4 * q4 + e] * inv);
      const int c = db * 4 + q4;  // 16-byte chunk of dims 8c..8c+7; this lane's half: 4 half..
      *(typename FV<T>::v4 *)(ys + col * RB + 16 * (c ^ (col & (CH - 1))) + 8 * half) = v4;
    }
  constexpr int RPI = 64 / CH;  // rows per store instruction
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int r = k * RPI + lane / CH, c = lane % CH;
    const uint4 v = *(const uint4 *)(ys + r * RB + 16 * (c ^ (r & (CH - 1))));
    const int sl = wave * 32 + r;
    const int ri = i0 + (sl >> pl.ghs), rh = g * p.G + hg * pl.GH + (sl & (pl.GH - 1));
    if (ri < p.S) *(uint4 *)((T *)p.y + b * p.y_sb + (int64_t)ri * p.y_ss + rh * p.y_sh + c * 8) = v;
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
  const int bm = p.mask ? (p.bias ? 2 : 3) : (p.bias ? 1 : 0);
  const bool cap = p.softcap > 0.f;
#define OLK_FLASH(BMV, CAPV) hipLaunchKernelGGL((flash_fwd_kernel<T, D, BMV, CAPV>), grid, block, 0, st, p, pl)
  if (bm == 3) { if (cap) OLK_FLASH(3, true); else OLK_FLASH(3, false); }
  else if (bm == 2) { if (cap) OLK_FLASH(2, true); else OLK_FLASH(2, false); }
  else if (bm == 1 && pl.qs) hipLaunchKernelGGL((flash_fwd_kernel<T, D, 1, false, true>), grid, block, 0, st, p, pl);
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

// Whether the prefill kernel writes the present rows of the new keys itself
// (K and V, or V alone when the rotary pre-pass has written the rotated K).
bool flash_fuses_present(const Params &p) {
  return p.op == OP_GQA && p.present_v != nullptr && (p.present_k != nullptr || p.v_new_rows);
}

hipError_t launch_flash(const Params &p, int dtype, hipStream_t st) {
  FPlan pl;
  pl.GH = gh_for(p.G);
  pl.ghs = __builtin_ctz((unsigned)pl.GH);
  pl.n_hg = p.G / pl.GH;
  pl.QW = kSlots / pl.GH;
  pl.n_qt = (p.S + pl.QW - 1) / pl.QW;
  const int n_bg = p.B * p.Hkv * pl.n_hg;
  pl.xcd_remap = n_bg % 8 == 0 ? 1 : 0;
  pl.bias_vec = (p.bias_si % 4 == 0 && p.bias_sh % 4 == 0 && p.bias_sb % 4 == 0 &&
                 ((uintptr_t)p.bias & 7) == 0) ? 1 : 0;
  // word loads of 4 mask elements: 4-byte (BOOL) or 16-byte (int32) aligned rows
  pl.mask_vec = (p.mask_si % 4 == 0 && p.mask_sh % 4 == 0 && p.mask_sb % 4 == 0 &&
                 ((uintptr_t)p.mask & (p.mask_kind == 2 ? 15 : 3)) == 0) ? 1 : 0;
  pl.fuse_present = flash_fuses_present(p) ? 1 : 0;
  // fixed exponent offset: softcap bounds the scores to +-c; bf16 P (f16 would
  // overflow), and no additive filter value after the cap
  pl.fixm = (dtype == DT_BF16 && p.softcap > 0.f && p.softcap * 1.4426950408889634f <= 100.f &&
             !p.pad_add && p.mask_kind != 2) ? 1 : 0;
  // Q pre-scaled (bias in the accumulator): attn_bias without softcap or BOOL
  // mask, the scale an exact power of two in [2^-8, 1] (1/sqrt(head size) for
  // head sizes 4, 16, 64, 256), so q * scale is exact for normal q
  {
    int ex = 0;
    const float mant = frexpf(p.scale, &ex);
    pl.qs = (p.bias && !p.mask && !(p.softcap > 0.f) && mant == 0.5f && ex >= -7 && ex <= 1) ? 1 : 0;
    // at head size 64 the bias rows go through LDS, which takes one query per
    // row slot (GH = 1), with 32-bit byte offsets inside one (b, head) slab
    if (p.D == 64 && (pl.GH != 1 || (int64_t)p.S * p.bias_si * 2 >= (int64_t)1 << 31)) pl.qs = 0;
  }
  if (dtype == DT_BF16)
    return p.D == 64 ? launch_td<bf16, 64>(p, pl, st)
           : p.D == 128 ? launch_td<bf16, 128>(p, pl, st) : launch_td<bf16, 256>(p, pl, st);
  return p.D == 64 ? launch_td<f16, 64>(p, pl, st)
         : p.D == 128 ? launch_td<f16, 128>(p, pl, st) : launch_td<f16, 256>(p, pl, st);
}

}  // namespace olk
