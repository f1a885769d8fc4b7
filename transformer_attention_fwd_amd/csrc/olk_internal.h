// Internal declarations shared by the HIP sources of libolk (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace olk {

enum { OP_GQA = 0, OP_MHA = 1, OP_ATTENTION = 2 };
enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef _Float16 f16;
typedef __bf16 bf16;

// Everything a kernel needs about one call, resolved on the host.  Strides are
// in elements.  Past and present tensors are (B, Hkv, P|T, D|Dv), dense.
struct Params {
  const void *q, *k, *v, *past_k, *past_v;
  const int32_t *seqlens;
  const void *bias, *sink, *proj_bias;
  void *y, *present_k, *present_v;
  int64_t q_sb, q_ss, q_sh;   // Q: batch, sequence, head strides (last dim dense)
  int64_t k_sb, k_ss, k_sh;   // new K
  int64_t v_sb, v_ss, v_sh;   // new V
  int64_t y_sb, y_ss, y_sh;   // Y
  int64_t bias_sb, bias_sh, bias_si;  // bias batch / head / query-row strides (0 when broadcast)
  int bias_cols;              // keys j >= bias_cols are excluded (short mask padding); T otherwise
  const void *mask;           // attn_mask (mask_kind != 0)
  int mask_kind;              // 1: uint8 bool (exclusion), 2: int32 binary (+mfv on zero)
  int64_t mask_sb, mask_sh, mask_si;  // element strides (0 when broadcast)
  int mask_cols;              // keys j >= mask_cols: false
  int seqlens64;              // seqlens points at int64 values
  float *qk_out;              // (B, Hq, S, T) float32 or null
  int qk_mode;
  int B, S, L, P, T, Hq, Hkv, G, D, Dv;
  int past_rows;   // rows per (b, g) of the past buffer: P, or T when the past lives in present
  int op, causal, window;
  int pad_add;     // MultiHeadAttention lengths: 1 = padded keys get mfv added, 0 = excluded
                   // (the host excludes them when mfv <= -5000: identical after underflow)
  int kv_inplace;  // present already holds the valid past
  int present_past_only;  // present writer copies only rows j < past_b (the
                          // attention kernel writes the new rows itself)
  float scale;     // score multiplier
  float softcap;   // > 0: softcap * tanh(s / softcap)
  float mfv;       // mask_filter_value
  int keys_in_past;  // every key j < total_b is read from past_k/past_v (the rotary
                     // path has already written the rotated new keys into present)
  // rotary embedding (used by the rotary pre-pass only)
  const void *cos_cache, *sin_cache;
  int rot_dim, rot_inter, rot_max;
  int rot_q;  // the prefill kernel rotates Q as it loads it (the pre-pass skips Q)
  int rot_skip_v;  // the pre-pass leaves V alone (the prefill kernel copies the new V rows)
  int v_new_rows;  // with keys_in_past: V rows of the new keys still come from the new V
                   // (keys j >= past_b), only K is read from the past buffer throughout
};

// Per-batch sequence bookkeeping (integer; read once per workgroup).
struct Seq {
  int past;   // keys taken from the past buffer
  int total;  // keys in the concatenated sequence
  int valid;  // keys j < valid may be attended
  int pad;    // keys j >= pad get mfv added (MultiHeadAttention, additive mode)
  int qoff;   // absolute position of query 0: the number of cached keys before the new ones
  int src;    // keys j < src are read from the past buffer, the rest from the new K/V
  int vsrc;   // the same boundary for V (differs from src only with v_new_rows)
};

__device__ __forceinline__ Seq seq_info(const Params &p, int b) {
  Seq s;
  if (p.op == OP_GQA) {
    // seqlens_k = total length - 1; the new keys follow the valid past.
    long long past = (long long)p.seqlens[b] + 1 - p.S;
    past = past < 0 ? 0 : (past > p.P ? p.P : past);
    s.past = (int)past;
    s.total = s.past + p.S;
    s.valid = s.total;
    s.pad = s.total;
    s.qoff = s.past;
  } else {
    s.past = p.P;
    s.total = p.T;
    // causal mask aligned to the upper-left corner of the new keys, shifted by
    // the cached keys (every cached key precedes every query)
    s.qoff = p.P;
    s.valid = p.T;
    s.pad = p.T;
    if (p.seqlens) {
      long long n64 = p.seqlens64 ? ((const long long *)p.seqlens)[b] : (long long)p.seqlens[b];
      int n = (int)(n64 < 0 ? 0 : (n64 > p.T ? p.T : n64));
      if (p.op == OP_ATTENTION) {
        s.valid = n;
      } else if (n > 0) {  // MHA: a fully padded row is a uniform shift = no mask
        if (p.pad_add) s.pad = n;
        else s.valid = n;
      }
    }
  }
  s.src = p.keys_in_past ? s.total : s.past;
  s.vsrc = (p.keys_in_past && !p.v_new_rows) ? s.total : s.past;
  return s;
}

// attn_mask element of (b, h, i, j): true = attend.  BOOL masks are uint8,
// binary masks int32; keys beyond the mask's columns read false.
__device__ __forceinline__ bool mask_at(const Params &p, int b, int h, int i, int j) {
  if (j >= p.mask_cols) return false;
  const int64_t e = b * p.mask_sb + h * p.mask_sh + i * p.mask_si + j;
  return p.mask_kind == 1 ? ((const uint8_t *)p.mask)[e] != 0 : ((const int32_t *)p.mask)[e] != 0;
}

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

// Launchers (defined in the .hip files); return hipSuccess or the launch error.
hipError_t launch_generic(const Params &p, int dtype, hipStream_t st);
hipError_t launch_generic_split(const Params &p, int dtype, int chunk, int n_split,
                                float *ws, hipStream_t st);
hipError_t launch_combine(const Params &p, int dtype, int n_split, int split_keys,
                          const float *ws, hipStream_t st);
hipError_t launch_present(const Params &p, int dtype, hipStream_t st);
hipError_t launch_rope(const Params &p, int dtype, hipStream_t st);
hipError_t launch_qk(const Params &p, int dtype, hipStream_t st);
hipError_t launch_kv_bias(const Params &p, int dtype, hipStream_t st);
hipError_t launch_backward(const Params &p, int dtype, const void *dy, void *dq, void *dk,
                           void *dv, float *ws, hipStream_t st);
// Matrix-core backward: f16/bf16, D == Dv in {64, 128}, power-of-two head
// groups, 16-byte aligned rows.  launch_backward takes it when it applies.
bool backward_mfma_supports(const Params &p, int dtype, const void *dy, const void *dq,
                            const void *dk, const void *dv);
hipError_t launch_backward_mfma(const Params &p, int dtype, const void *dy, void *dq, void *dk,
                                void *dv, float *ws, hipStream_t st);

}  // namespace olk
