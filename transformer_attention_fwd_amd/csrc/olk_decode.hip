// Split-KV decode for gfx950 (head size 64, 128 or 256): a few query rows (G
// heads x S queries <= 16 per KV head) against a long key sequence.
// HBM-bound: every cached key row is read once per (batch, KV head) and
// serves all G query heads of the group.
//
// Same result as the prefill path (onnx-light-cpu Python API "Custom
// operators", "Microsoft GroupQueryAttention": grouped heads, causal / local
// window masks, head_sink; onnx-light reference kernels header page, "class
// Attention"); the decomposition is ours:
//
// * A workgroup owns one split (a range of SPLIT keys) of one (batch, KV head);
//   its 4 wavefronts take interleaved 16-key steps of the split.  Workgroup
//   ids are split-major: consecutive ids go round-robin over the 8 XCDs, so
//   with (batch, KV head) fastest every split spreads over all XCDs whatever
//   the split count (split-minor ids put split s on XCD s when the count is a
//   multiple of 8, and the later splits of short sequences are empty), and
//   the always-full first splits are dispatched before the short last ones.
// * QK^T: v_mfma_f32_16x16x32 with Q^T held in VGPRs as the B operand (16
//   columns = the row slots (query, head)).  K is loaded as whole rows (4 rows
//   per instruction) and its A operand (16 keys x 32 dims) read back from a
//   per-wavefront LDS tile at head size 128 / 256; at head size 64 K goes from
//   memory straight into the A operand (16 bytes per lane).
// * The S^T accumulator puts each row slot's 16 scores in 4 lanes; the online
//   softmax (exp2 domain, lazy rescale) reduces across them with lane swaps.
// * PV: at head size 128 / 256 on v_mfma_f32_16x16x16 (decode_mfma_kernel below:
//   P^T straight from the score accumulator, V^T by transposed LDS reads);
//   at head size 64 on the VALU: P goes through a 1 KB LDS buffer per
//   wavefront and is read back as broadcasts; lanes own 4 head dimensions of
//   one key (two keys per instruction), so V rows are read fully coalesced
//   and never transposed.
// * The K and V of the next two steps are in flight while a step computes;
//   the stream is read once, with non-temporal loads.
// * Scores with an additive bias, softcap or attn_mask (EPI instantiations)
//   take the general score pipeline per key, in the order of the contracts:
//   (Q K^T) * scale, + bias, softcap, + mask_filter_value at MultiHeadAttention
//   padded keys and at zeros of its int32 binary mask; a false BOOL element
//   excludes the key.  The MultiHeadAttention Q projection bias is added as Q
//   loads (the K/V segments go through a pre-pass into present).
// * The 4 wavefronts merge (m, l, O) through LDS and write one partial record
//   [m (natural log), l, -, -, O[Dv]] per (row, split); the combine kernel
//   merges the splits and adds the sink.
#include "olk_internal.h"

namespace olk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Streaming (read-once) loads: non-temporal, so the KV stream does not evict
// reusable lines from the caches.
__device__ __forceinline__ uint4 ld_stream16(const char *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4 *)p));
}
__device__ __forceinline__ uint2 ld_stream8(const char *p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load((const u32x2 *)p));
}

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0, 32-bit data
// format word of the gfx9 family): loads at offsets >= bytes return zeros and
// access no memory.
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufWord3);
}
// Streaming buffer loads (cache policy nt: read once).
constexpr int kBufNT = 2;
__device__ __forceinline__ uint4 ld_buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kBufNT));
}
__device__ __forceinline__ uint2 ld_buf8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kBufNT));
}

template <typename T> struct DV;
template <> struct DV<bf16> { typedef bf16x8 v8; };
template <> struct DV<f16> { typedef f16x8 v8; };

__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

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

constexpr int kThreads = 256;
constexpr int kStep = 16;  // keys per wavefront step

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15: no wait on those)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescale = 8.0f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// x of lanes l and l ^ 32 combined (v_permlane32_swap with both operands x).
__device__ __forceinline__ float max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct DPlan {
  int n_split;     // splits per (batch, KV head)
  int split_keys;  // keys per split (multiple of 4 * kStep)
  float *ws;       // records [m, l, -, -, O[Dv]] per (row, split)
  int append;      // in-place cache: the kernel writes the new rows itself
};

// Score of row (row_q, row_h) and key j in the log2 domain through the
// general pipeline (onnx-light reference kernels header page, "class
// Attention": scale, + bias, softcap; Python API "Custom operators",
// "Microsoft MultiHeadAttention": mask_filter_value added at padded keys and
// at zeros of the int32 binary mask); a false BOOL mask element clears ok.
// Called only for keys inside the row's range (below the bias / BOOL-mask
// columns).  cap_in = 2 log2(e) / softcap: c tanh(x / c) = c - 2c / (2^(x cap_in) + 1).
template <typename T>
__device__ __forceinline__ float score_general(const Params &p, const Seq &s, float dot, int b,
                                               int row_q, int row_h, int j, float cap_in,
                                               bool &ok) {
  float sc = dot * p.scale;
  if (p.bias)
    sc += (float)((const T *)p.bias)[b * p.bias_sb + row_h * p.bias_sh + (int64_t)row_q * p.bias_si + j];
  if (p.softcap > 0.f)
    sc = p.softcap - 2.0f * p.softcap * __builtin_amdgcn_rcpf(ex2(sc * cap_in) + 1.0f);
  if (p.pad_add && j >= s.pad) sc += p.mfv;
  if (p.mask_kind == 2 && !mask_at(p, b, row_h, row_q, j)) sc += p.mfv;
  if (p.mask_kind == 1 && !mask_at(p, b, row_h, row_q, j)) ok = false;
  return sc * kLog2e;
}

// Q row chunk (8 elements) plus the MultiHeadAttention Q projection bias,
// each sum rounded once to the element type.
template <typename T, typename V>
__device__ __forceinline__ V add_qbias(uint4 raw, const T *pb) {
  V v = __builtin_bit_cast(V, raw);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (T)((float)v[e] + (float)pb[e]);
  return v;
}

// NR: row slots (G * S) rounded up to a power of two <= 16.
template <typename T, int D, int NR, bool EPI>
__global__ __launch_bounds__(kThreads) void decode_kernel(Params p, DPlan pl) {
  typedef typename DV<T>::v8 vec8;
  constexpr int NKS = D / 32;  // k-steps of QK^T (32 dims each)
  constexpr int DPL = D / 32;  // head dims per lane in PV (lanes 0-31 span D)
  __shared__ __attribute__((aligned(16))) float pbuf[4][16 * kStep];     // P per wave: [slot][parity-major key]
  __shared__ __attribute__((aligned(16))) float mrg_ml[4][2][16];        // per-wave m, l per slot
  __shared__ __attribute__((aligned(16))) float mrg_o[4][NR][D];         // per-wave O

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x / (p.B * p.Hkv);  // split-major workgroup ids
  const int bg = blockIdx.x % (p.B * p.Hkv);
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const Seq s = seq_info(p, b);
  const int nrows = p.G * p.S;

  // key range of the workgroup: union over its rows, cut to the split
  const int pos_min = s.qoff, pos_max = s.qoff + p.S - 1;
  int hi = p.pad_add ? s.total : s.valid;
  if (p.causal) hi = min(hi, pos_max + 1);
  // a short bias or BOOL mask excludes the keys beyond its columns
  if (EPI && p.bias) hi = min(hi, p.bias_cols);
  if (EPI && p.mask_kind == 1) hi = min(hi, p.mask_cols);
  int lo = p.window > 0 ? max(0, pos_min - p.window + 1) : 0;
  const int sp_lo = max(lo, split * pl.split_keys);
  const int sp_hi = min(hi, (split + 1) * pl.split_keys);
  const int base = (sp_lo / kStep) * kStep;
  const int n_steps = sp_lo < sp_hi ? (sp_hi - base + kStep - 1) / kStep : 0;
  // a split with no key of the range: no record (the combine reads only the
  // splits that hold keys of a row's range)
  if (n_steps == 0) return;

  // ---- Q^T operand: column n = lane % 16 is row slot n = (query n / G, head n % G) ----
  const int n = lane & 15, kq = lane >> 4;
  const int row_q = n / p.G, row_h = g * p.G + n % p.G;
  const bool col_ok = n < nrows;
  const int col_pos = s.qoff + row_q;
  vec8 qreg[NKS];
  {
    const T *qr = (const T *)p.q + b * p.q_sb + (int64_t)(col_ok ? row_q : 0) * p.q_ss +
                  (col_ok ? row_h : 0) * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (col_ok) raw = *(const uint4 *)(qr + ks * 32 + kq * 8);
      qreg[ks] = (p.proj_bias && col_ok)
                     ? add_qbias<T, vec8>(raw, (const T *)p.proj_bias + row_h * D + ks * 32 + kq * 8)
                     : __builtin_bit_cast(vec8, raw);
    }
  }
  // Q is in registers from here on: wait for its loads on every path, so the
  // wait-count analysis does not treat them as in flight inside the step loop
  // (vmcnt(0) only; gfx9 encoding: expcnt 7, lgkmcnt 15).
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const T *kpast = (const T *)p.past_k + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *vpast = (const T *)p.past_v + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *knew = (const T *)p.k + b * p.k_sb + g * p.k_sh;
  const T *vnew = (const T *)p.v + b * p.v_sb + g * p.v_sh;

  // per-step registers: K (A operand: key lane % 16, dims 32 ks + 8 kq + e) and
  // V (key 2 t + lane / 32, dims DPL * (lane % 32) + e)
  const int vcol = DPL * (lane & 31), vpar = lane >> 5;
  static_assert(DPL == 4 || DPL == 2, "head size 64 or 128");
  auto load_step = [&](int st, uint4 (&kk)[NKS], uint2 (&vv)[kStep / 2]) {
    const int j0 = base + (wave + 4 * st) * kStep;
    const bool full = j0 >= sp_lo && j0 + kStep <= sp_hi;
    if (full && (j0 >= s.src || j0 + kStep <= s.src)) {
      // the whole step from one source: uniform base + 32-bit lane offsets
      const bool from_new = j0 >= s.src;
      const char *kb = (const char *)(from_new ? knew + (int64_t)(j0 - s.src) * p.k_ss
                                               : kpast + (int64_t)j0 * D);
      const char *vb = (const char *)(from_new ? vnew + (int64_t)(j0 - s.src) * p.v_ss
                                               : vpast + (int64_t)j0 * D);
      const uint32_t krs = (uint32_t)(from_new ? p.k_ss : D) * (uint32_t)sizeof(T);
      const uint32_t vrs = (uint32_t)(from_new ? p.v_ss : D) * (uint32_t)sizeof(T);
      const uint32_t koff = (uint32_t)n * krs + (uint32_t)kq * 16u;
#pragma unroll
      for (int s2 = 0; s2 < NKS; ++s2)
        kk[s2] = ld_stream16(kb + koff + s2 * 64);
      const uint32_t voff = (uint32_t)vpar * vrs + (uint32_t)vcol * (uint32_t)sizeof(T);
#pragma unroll
      for (int t = 0; t < kStep / 2; ++t) {
        if constexpr (DPL == 4) vv[t] = ld_stream8(vb + voff + 2 * t * vrs);
        else vv[t] = make_uint2(__builtin_nontemporal_load((const uint32_t *)(vb + voff + 2 * t * vrs)), 0u);
      }
      return;
    }
    // Steps that straddle the range or the past/new boundary: per-lane rows.
    // Rows outside [sp_lo, sp_hi) load row sp_lo instead (valid memory, finite
    // values; their scores are masked, so their P is exactly 0).  Both source
    // offsets are computed and one selected: no branch, no select on loaded
    // data, so the compiler's count of loads in flight stays exact.
    auto row_ptr = [&](const T *pastp, const T *newp, int64_t new_ss, int j) {
      const int jj = j >= sp_lo && j < sp_hi ? j : sp_lo;
      const bool nw = jj >= s.src;
      const int64_t off_new = (int64_t)(jj - s.src) * new_ss, off_past = (int64_t)jj * D;
      return (nw ? newp : pastp) + (nw ? off_new : off_past);
    };
    const T *ks = row_ptr(kpast, knew, p.k_ss, j0 + n);
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) kk[s2] = *(const uint4 *)(ks + s2 * 32 + kq * 8);
#pragma unroll
    for (int t = 0; t < kStep / 2; ++t) {
      const T *vs = row_ptr(vpast, vnew, p.v_ss, j0 + 2 * t + vpar) + vcol;
      if constexpr (DPL == 4) vv[t] = *(const uint2 *)vs;
      else vv[t] = make_uint2(*(const uint32_t *)vs, 0u);
    }
  };

  float m = kNegInf, l = 0.f;
  float o[NR][DPL];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[r][e] = 0.f;
  const float sl = p.scale * kLog2e;
  const float cap_in = p.softcap > 0.f ? 2.0f * kLog2e / p.softcap : 0.f;

  const int my_steps = n_steps > wave ? (n_steps - wave + 3) / 4 : 0;
  // Three register buffers rotate so the loads of step it + 2 are in flight
  // while step it computes.
  uint4 k0[NKS], k1[NKS], k2[NKS];
  uint2 v0[kStep / 2], v1[kStep / 2], v2[kStep / 2];
  auto body = [&](int it, uint4 (&kr)[NKS], uint2 (&vr)[kStep / 2], uint4 (&kf)[NKS],
                  uint2 (&vf2)[kStep / 2]) {
    if (it + 2 < my_steps) load_step(it + 2, kf, vf2);
    const int j0 = base + (wave + 4 * it) * kStep;
    // S^T (16 keys x 16 slots)
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) sacc = mma16(__builtin_bit_cast(vec8, kr[s2]), qreg[s2], sacc);
    // scores of slot n for keys j0 + 4 kq + r, log2 domain, masked
    float t4[4];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 4 * kq + r;
      bool ok = j >= sp_lo && j < sp_hi;
      if (p.causal && j > col_pos) ok = false;
      if (p.window > 0 && j < col_pos - p.window + 1) ok = false;
      float t;
      if constexpr (EPI) {
        t = (ok && col_ok) ? score_general<T>(p, s, sacc[r], b, row_q, row_h, j, cap_in, ok) : 0.f;
      } else {
        t = sacc[r] * sl;
        if (p.pad_add && j >= s.pad) t += p.mfv * kLog2e;
      }
      t4[r] = ok ? t : kNegInf;
      mx = fmaxf(mx, t4[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = max32(mx);
    const float m_new = fmaxf(m, mx);
    const bool grow = m_new > m + kRescale;
    const float alpha = grow ? ex2(m - m_new) : 1.0f;  // same in the 4 lanes of slot n
    if (grow) m = m_new;
    const float mu = m == kNegInf ? 0.f : m;
    float pv[4], lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = ex2(t4[r] - mu);
      lsum += pv[r];
    }
    l = l * alpha + lsum;  // lane-local partial of slot n
    // P of this step, parity-major (key k at (k & 1) * 8 + k / 2), for the
    // broadcast reads of the PV loop (LDS operations of one wave complete in order)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = 4 * kq + r;
      pbuf[wave][n * kStep + (k & 1) * 8 + (k >> 1)] = pv[r];
    }
    // O rows scale by their slot's factor, which lane r holds
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float ar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r));
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[r][e] *= ar;
    }
    // PV: this lane accumulates keys 2t + vpar for its DPL dims
#pragma unroll
    for (int t = 0; t < kStep / 2; ++t) {
      float vf[DPL];
      vf[0] = lo16<T>(vr[t].x);
      vf[1] = hi16<T>(vr[t].x);
      if constexpr (DPL == 4) {
        vf[2] = lo16<T>(vr[t].y);
        vf[3] = hi16<T>(vr[t].y);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float w = pbuf[wave][r * kStep + vpar * 8 + t];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[r][e] = __builtin_fmaf(w, vf[e], o[r][e]);
      }
    }
  };
  if (my_steps > 0) load_step(0, k0, v0);
  if (my_steps > 1) load_step(1, k1, v1);
  for (int it = 0; it < my_steps; it += 3) {
    body(it, k0, v0, k2, v2);
    if (it + 1 < my_steps) body(it + 1, k1, v1, k0, v0);
    if (it + 2 < my_steps) body(it + 2, k2, v2, k1, v1);
  }

  // ---- wave partials -> LDS: m, l per slot (from the 4 lanes of each slot) ----
  float lsl = l + __shfl_xor(l, 16, 64);
  lsl = sum32(lsl);
  if (lane < 16) {
    mrg_ml[wave][0][lane] = m;
    mrg_ml[wave][1][lane] = lsl;
  }
  // O rows: lanes of parity 0 and 1 hold different keys of the same dims
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float v = sum32(o[r][e]);
      if (lane < 32) mrg_o[wave][r][vcol + e] = v;
    }
  __syncthreads();

  // ---- merge the 4 wavefronts; one record per valid row slot ----
  for (int r = wave; r < NR; r += 4) {
    if (r >= nrows) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_ml[w][0][r]);
    float sc[4], L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mrg_ml[w][0][r];
      sc[w] = mw == kNegInf ? 0.f : ex2(mw - M);
      L += sc[w] * mrg_ml[w][1][r];
    }
    const int rq = r / p.G, rh = g * p.G + r % p.G;
    const int64_t row = ((int64_t)b * p.S + rq) * p.Hq + rh;
    float *out = pl.ws + (row * pl.n_split + split) * (int64_t)(D + 4);
    if (lane == 0) {
      out[0] = M == kNegInf ? kNegInf : M * kLn2;
      out[1] = M == kNegInf ? 0.f : L;
    }
    for (int d = lane; d < D; d += 64) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += sc[w] * mrg_o[w][r][d];
      out[4 + d] = M == kNegInf ? 0.f : acc;
    }
  }
}


// ---- head size 128 and 256: PV on the matrix cores ----
// O^T += V^T P^T runs on v_mfma_f32_16x16x16: P^T (the B operand: lane l
// holds keys 4 (l / 16) + i of slot l % 16) is the S^T accumulator itself,
// and V^T (the A operand: lane l holds keys 4 (l / 16) + i of dim 16 blk +
// l % 16) comes from ds_read_b64_tr_b16 on a per-wavefront LDS copy of the
// step's 16 V rows.  The rows are loaded into registers (two steps ahead, like
// K) and written to LDS just before their transposed reads; 16-byte chunk c of
// row r sits at slot c ^ 2 (r & 7), so the four rows one 16-lane group reads
// hit distinct banks.  A wavefront only reads the rows it wrote, and one
// wavefront's LDS operations run in order, so no barrier or wait is needed
// between the writes and the reads (nor against the previous step's reads).
// (Loading V straight into LDS instead left direct-to-LDS loads and register
// loads in flight together, and the compiler then waits for all loads.)
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <typename T> struct DV4;
template <> struct DV4<bf16> { typedef s16x4 v4; };
template <> struct DV4<f16> { typedef f16x4 v4; };
__device__ __forceinline__ f32x4 mma16k16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// two P values rounded to the element type, as the low / high halves of a word
template <typename T> __device__ __forceinline__ uint32_t pack2p(float a, float b) {
  const T x = (T)a, y = (T)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <typename T, int D, int NR, bool EPI>
__global__ __launch_bounds__(kThreads, (D == 128 ? 2 : 1)) void decode_mfma_kernel(Params p, DPlan pl) {
  static_assert(D == 128 || D == 256, "head size 128 or 256");
  typedef typename DV<T>::v8 vec8;
  typedef typename DV4<T>::v4 vec4;
  constexpr int NKS = D / 32;   // k-steps of QK^T (32 dims each)
  constexpr int NBLK = D / 16;  // 16-dim blocks of O^T
  constexpr int VRB = D * 2;    // bytes per K/V row, in memory and in LDS
  constexpr int CHR = D / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / CHR; // whole rows per load instruction
  constexpr int NV = kStep / RPI;  // V load instructions per step (K: NKS = kStep / RPI too)
  static_assert(NKS * RPI == kStep, "one K load per k-step");
  // K and V rows of the current step, one tile each per wavefront (separate
  // variables: the compiler then orders one's writes freely against the
  // other's reads), and the wavefronts' partials for the merge (128 KB in all
  // at head size 256, where the registers allow one workgroup per CU anyway)
  __shared__ __attribute__((aligned(16))) T vbw[4][kStep * D];
  __shared__ __attribute__((aligned(16))) T kbw[4][kStep * D];
  __shared__ __attribute__((aligned(16))) float mrg_ml[4][2][16];
  __shared__ __attribute__((aligned(16))) float mrg_o[4][NR][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x / (p.B * p.Hkv);  // split-major workgroup ids
  const int bg = blockIdx.x % (p.B * p.Hkv);
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const Seq s = seq_info(p, b);
  const int nrows = p.G * p.S;

  if (pl.append) {
    // In-place cache (present is the past buffer): the new rows [past_b,
    // total_b) that fall in this split's key range are copied from the new
    // K/V here, and the barrier's workgroup fence makes them visible to the
    // loads below; one workgroup per (split, b, KV head) owns each row.
    const int r0 = max(s.past, split * pl.split_keys);
    const int r1 = min(s.total, (split + 1) * pl.split_keys);
    if (r0 < r1) {
      T *kc = (T *)p.past_k + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
      T *vc = (T *)p.past_v + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
      for (int t = tid; t < (r1 - r0) * (D / 8); t += kThreads) {
        const int r = r0 + t / (D / 8), c = 8 * (t % (D / 8));
        const int64_t i = r - s.past;
        *(uint4 *)(kc + (int64_t)r * D + c) =
            *(const uint4 *)((const T *)p.k + b * p.k_sb + i * p.k_ss + g * p.k_sh + c);
        *(uint4 *)(vc + (int64_t)r * D + c) =
            *(const uint4 *)((const T *)p.v + b * p.v_sb + i * p.v_ss + g * p.v_sh + c);
      }
      __syncthreads();
    }
  }

  // key range of the workgroup: union over its rows, cut to the split
  const int pos_min = s.qoff, pos_max = s.qoff + p.S - 1;
  int hi = p.pad_add ? s.total : s.valid;
  if (p.causal) hi = min(hi, pos_max + 1);
  // a short bias or BOOL mask excludes the keys beyond its columns
  if (EPI && p.bias) hi = min(hi, p.bias_cols);
  if (EPI && p.mask_kind == 1) hi = min(hi, p.mask_cols);
  int lo = p.window > 0 ? max(0, pos_min - p.window + 1) : 0;
  const int sp_lo = max(lo, split * pl.split_keys);
  const int sp_hi = min(hi, (split + 1) * pl.split_keys);
  const int base = sp_lo;  // steps start at the first key of the split
  const int n_steps = sp_lo < sp_hi ? (sp_hi - sp_lo + kStep - 1) / kStep : 0;
  // a split with no key of the range: no record (the combine reads only the
  // splits that hold keys of a row's range)
  if (n_steps == 0) return;

  // ---- Q^T operand: column n = lane % 16 is row slot n = (query n / G, head n % G) ----
  const int n = lane & 15, kq = lane >> 4;
  const int row_q = n / p.G, row_h = g * p.G + n % p.G;
  const bool col_ok = n < nrows;
  const int col_pos = s.qoff + row_q;
  vec8 qreg[NKS];
  {
    const T *qr = (const T *)p.q + b * p.q_sb + (int64_t)(col_ok ? row_q : 0) * p.q_ss +
                  (col_ok ? row_h : 0) * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (col_ok) raw = *(const uint4 *)(qr + ks * 32 + kq * 8);
      qreg[ks] = (p.proj_bias && col_ok)
                     ? add_qbias<T, vec8>(raw, (const T *)p.proj_bias + row_h * D + ks * 32 + kq * 8)
                     : __builtin_bit_cast(vec8, raw);
    }
  }

  // Every key is in the past buffer (the present append ran before this
  // kernel, or above for the in-place cache). The
  // split's rows [sp_lo, sp_hi) are read through buffer descriptors based at
  // row sp_lo and sized to the split: rows at or past sp_hi read as zeros
  // without a memory access (range-checked offsets), so a partial last step
  // needs no clamping and no per-lane path, and no row outside the split
  // (unwritten cache slots included) is ever read.
  const T *kpast = (const T *)p.past_k + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const T *vpast = (const T *)p.past_v + ((int64_t)b * p.Hkv + g) * p.past_rows * D;
  const uint32_t nrec = (uint32_t)max(sp_hi - sp_lo, 0) * (uint32_t)VRB;
  const __amdgpu_buffer_rsrc_t krs = row_rsrc(kpast + (int64_t)sp_lo * D, nrec);
  const __amdgpu_buffer_rsrc_t vrs = row_rsrc(vpast + (int64_t)sp_lo * D, nrec);

  // V registers: row RPI t + lane / CHR of the step, 16-byte chunk lane % CHR;
  // written to LDS at that row, slot chunk ^ 2 (row & 7)
  // transposed reads: this lane addresses row 4 (l / 16) + (l % 16) / 4 and
  // dims 16 blk + 4 ((l % 16) & 3), i.e. byte tro + 32 (blk ^ (row & 7))
  const int trr = 4 * kq + ((lane & 15) >> 2);
  const uint32_t tro = (uint32_t)(trr * VRB + 16 * (((lane & 3) >> 1)) + 8 * (lane & 1));
  const int trx = trr & 7;
  // lane byte offset within a step, for K and V alike: row lane / CHR (+ RPI
  // t), 16-byte chunk lane % CHR, so one load instruction reads RPI whole rows
  // (full cache lines).  K loaded in the MFMA operand layout instead (16 rows x
  // 64 bytes per instruction) took twice the address work per byte: 218 vs
  // 202 us on the decode workload.
  const uint32_t voff = (uint32_t)(lane / CHR) * VRB + (uint32_t)(lane % CHR) * 16u;
  const int my_steps = n_steps > wave ? (n_steps - wave + 3) / 4 : 0;

  auto load_step = [&](int st, uint4 (&kk)[NKS], uint4 (&vv)[NV]) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)((wave + 4 * st) * kStep * VRB);
#pragma unroll
    for (int t = 0; t < NKS; ++t) kk[t] = ld_buf16(krs, voff + so + RPI * t * VRB);
#pragma unroll
    for (int t = 0; t < NV; ++t) vv[t] = ld_buf16(vrs, voff + so + RPI * t * VRB);
  };

  float m = kNegInf, l = 0.f;
  f32x4 o[NBLK];
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) o[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl = p.scale * kLog2e;
  const float cap_in = p.softcap > 0.f ? 2.0f * kLog2e / p.softcap : 0.f;

  uint4 k0[NKS], k1[NKS], k2[NKS];
  uint4 v0[NV], v1[NV], v2[NV];
  char *vl = (char *)vbw[wave];
  char *kl = (char *)kbw[wave];
  auto body = [&](int it, uint4 (&kr)[NKS], const uint4 (&vr)[NV], uint4 (&kf)[NKS],
                  uint4 (&vf)[NV]) __attribute__((always_inline)) {
    if (it + 2 < my_steps) load_step(it + 2, kf, vf);
    const int j0 = base + (wave + 4 * it) * kStep;
    // S^T (16 keys x 16 slots)
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NKS; ++t) {
      // the step's K rows into this wavefront's LDS tile: chunk c of row r at
      // slot c ^ (r & 15), so the operand reads below (16 rows at one chunk)
      // hit distinct banks; one wavefront's LDS operations run in order, so
      // no barrier is needed
      const int r = RPI * t + lane / CHR, c = lane % CHR;
      *(uint4 *)(kl + r * VRB + 16 * (c ^ (r & 15))) = kr[t];
    }
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) {
      // A operand: key row n, dims 32 s2 + 8 kq + e (chunk 4 s2 + kq)
      const vec8 a = *(const vec8 *)(kl + n * VRB + 16 * ((4 * s2 + kq) ^ n));
      sacc = mma16(a, qreg[s2], sacc);
    }
    // scores of slot n for keys j0 + 4 kq + r, log2 domain, masked
    float t4[4];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 4 * kq + r;
      bool ok = j >= sp_lo && j < sp_hi;
      if (p.causal && j > col_pos) ok = false;
      if (p.window > 0 && j < col_pos - p.window + 1) ok = false;
      float t;
      if constexpr (EPI) {
        t = (ok && col_ok) ? score_general<T>(p, s, sacc[r], b, row_q, row_h, j, cap_in, ok) : 0.f;
      } else {
        t = sacc[r] * sl;
        if (p.pad_add && j >= s.pad) t += p.mfv * kLog2e;
      }
      t4[r] = ok ? t : kNegInf;
      mx = fmaxf(mx, t4[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = max32(mx);
    const float m_new = fmaxf(m, mx);
    const bool grow = m_new > m + kRescale;
    const float m_prev = m;
    if (grow) m = m_new;
    const float mu = m == kNegInf ? 0.f : m;
    // P^T as the B operand, rounded; the row sum adds the rounded values
    const uint32_t w0 = pack2p<T>(ex2(t4[0] - mu), ex2(t4[1] - mu));
    const uint32_t w1 = pack2p<T>(ex2(t4[2] - mu), ex2(t4[3] - mu));
    const vec4 pb = __builtin_bit_cast(vec4, make_uint2(w0, w1));
    const float lsum = (lo16<T>(w0) + hi16<T>(w0)) + (lo16<T>(w1) + hi16<T>(w1));
    // O^T columns and l follow a grown max (each lane holds its own slot)
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? ex2(m_prev - m) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[blk][r] *= alpha;
    }
    l += lsum;  // lane-local partial of slot n
    // the step's V rows into this wavefront's LDS tile (swizzled chunks)
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int r = RPI * t + lane / CHR;
      const int c = lane % CHR;
      *(uint4 *)(vl + r * VRB + 16 * (c ^ (2 * (r & 7)))) = vr[t];
    }
    // PV on the matrix cores
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      typedef __attribute__((address_space(3))) s16x4 *tr_ptr;
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((tr_ptr)(vl + tro + 32 * (blk ^ trx)));
      o[blk] = mma16k16(__builtin_bit_cast(vec4, a), pb, o[blk]);
    }
  };
  // The first two steps' loads go out behind the Q loads, so the latencies
  // overlap; then wait for Q alone (the 8 K/V loads of each issued step may
  // stay in flight: the counter is in order).  Waiting on every path keeps the
  // wait-count analysis from treating Q as in flight inside the step loop.
  if (my_steps > 0) load_step(0, k0, v0);
  if (my_steps > 1) load_step(1, k1, v1);
  constexpr int kLoadsPerStep = NKS + NV;
  static_assert(2 * kLoadsPerStep < 64, "vmcnt holds 6 bits");
  if (my_steps > 1) __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kLoadsPerStep));
  else if (my_steps == 1) __builtin_amdgcn_s_waitcnt(vmcnt_only(kLoadsPerStep));
  else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  {
    for (int it = 0; it < my_steps; it += 3) {
      body(it, k0, v0, k2, v2);
      if (it + 1 < my_steps) body(it + 1, k1, v1, k0, v0);
      if (it + 2 < my_steps) body(it + 2, k2, v2, k1, v1);
    }
  }

  // ---- wave partials -> LDS: m, l per slot (from the 4 lanes of each slot) ----
  float lsl = l + __shfl_xor(l, 16, 64);
  lsl = sum32(lsl);
  if (lane < 16) {
    mrg_ml[wave][0][lane] = m;
    mrg_ml[wave][1][lane] = lsl;
  }
  // O^T: lane l holds dims 16 blk + 4 (l / 16) + r of slot l % 16
  if (n < NR) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) mrg_o[wave][n][16 * blk + 4 * kq + r] = o[blk][r];
  }
  __syncthreads();

  // ---- merge the 4 wavefronts; one record per valid row slot ----
  for (int r = wave; r < NR; r += 4) {
    if (r >= nrows) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_ml[w][0][r]);
    float sc[4], L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mrg_ml[w][0][r];
      sc[w] = mw == kNegInf ? 0.f : ex2(mw - M);
      L += sc[w] * mrg_ml[w][1][r];
    }
    const int rq = r / p.G, rh = g * p.G + r % p.G;
    const int64_t row = ((int64_t)b * p.S + rq) * p.Hq + rh;
    float *out = pl.ws + (row * pl.n_split + split) * (int64_t)(D + 4);
    if (lane == 0) {
      out[0] = M == kNegInf ? kNegInf : M * kLn2;
      out[1] = M == kNegInf ? 0.f : L;
    }
    for (int d = lane; d < D; d += 64) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += sc[w] * mrg_o[w][r][d];
      out[4 + d] = M == kNegInf ? 0.f : acc;
    }
  }
}

template <typename T, int D, bool EPI>
void launch_nr_epi(const Params &p, const DPlan &pl, int nr, dim3 grid, hipStream_t st) {
  if constexpr (D >= 128) {
    // head size 128 or 256: PV on the matrix cores
    if (nr <= 4) hipLaunchKernelGGL((decode_mfma_kernel<T, D, 4, EPI>), grid, dim3(kThreads), 0, st, p, pl);
    else if (nr <= 8) hipLaunchKernelGGL((decode_mfma_kernel<T, D, 8, EPI>), grid, dim3(kThreads), 0, st, p, pl);
    else hipLaunchKernelGGL((decode_mfma_kernel<T, D, 16, EPI>), grid, dim3(kThreads), 0, st, p, pl);
  } else {
    if (nr <= 4) hipLaunchKernelGGL((decode_kernel<T, D, 4, EPI>), grid, dim3(kThreads), 0, st, p, pl);
    else if (nr <= 8) hipLaunchKernelGGL((decode_kernel<T, D, 8, EPI>), grid, dim3(kThreads), 0, st, p, pl);
    else hipLaunchKernelGGL((decode_kernel<T, D, 16, EPI>), grid, dim3(kThreads), 0, st, p, pl);
  }
}

template <typename T, int D>
hipError_t launch_nr(const Params &p, const DPlan &pl, int nr, dim3 grid, hipStream_t st) {
  // bias, softcap or attn_mask: the general score pipeline
  if (p.bias || p.mask || p.softcap > 0.f) launch_nr_epi<T, D, true>(p, pl, nr, grid, st);
  else launch_nr_epi<T, D, false>(p, pl, nr, grid, st);
  return hipGetLastError();
}

}  // namespace

// The decode kernel takes every (query, head) row of one KV head in 16 slots;
// at head size 128 / 256 it reads every key from the past buffer (keys_in_past).
bool decode_supports(const Params &p, int dtype) {
  return (dtype == DT_F16 || dtype == DT_BF16) && p.D == p.Dv &&
         (p.D == 64 || p.D == 128 || p.D == 256) && p.G * p.S <= 16 && p.scale > 0.f &&
         (p.D == 64 || p.keys_in_past);
}

// Head size 128 or 256 in place (present is the past buffer, every key read
// from it): the decode kernel can append the new rows itself.
bool decode_appends(const Params &p, int dtype) {
  return decode_supports(p, dtype) && p.D >= 128 && p.kv_inplace && p.keys_in_past;
}

hipError_t launch_decode(const Params &p, int dtype, int split_keys, int n_split, float *ws,
                         bool append, hipStream_t st) {
  if (append && !decode_appends(p, dtype)) return hipErrorInvalidValue;
  DPlan pl;
  pl.n_split = n_split;
  pl.split_keys = split_keys;
  pl.ws = ws;
  pl.append = append ? 1 : 0;
  const int64_t n = (int64_t)p.B * p.Hkv * n_split;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n);
  const int nr = p.G * p.S;
  if (dtype == DT_BF16)
    return p.D == 64 ? launch_nr<bf16, 64>(p, pl, nr, grid, st)
           : p.D == 128 ? launch_nr<bf16, 128>(p, pl, nr, grid, st) : launch_nr<bf16, 256>(p, pl, nr, grid, st);
  return p.D == 64 ? launch_nr<f16, 64>(p, pl, nr, grid, st)
         : p.D == 128 ? launch_nr<f16, 128>(p, pl, nr, grid, st) : launch_nr<f16, 256>(p, pl, nr, grid, st);
}

}  // namespace olk
