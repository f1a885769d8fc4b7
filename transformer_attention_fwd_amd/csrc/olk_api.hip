// Host side of libolk: validation, planning, kernel choice and launches.
//
// Validation follows the operator contracts: local_window_size -1 or positive
// and only with causal=1 (onnx-light-cpu Python API "Custom operators",
// "Microsoft GroupQueryAttention"); q_num_heads a multiple of kv_num_heads
// (onnx-light reference kernels header page, "class Attention"); MultiHeadAttention
// uses one head count, rank-3 or rank-4 K/V, and rejects what it does not
// model ("Microsoft MultiHeadAttention").  Nothing here reads device memory.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/olk.h"
#include "olk_internal.h"

namespace olk {
hipError_t launch_flash(const Params &p, int dtype, hipStream_t st);
bool flash_fuses_present(const Params &p);
bool flash_rotates_q(const Params &p);
hipError_t launch_tiled_split(const Params &p, int dtype, int split_tiles, float *ws,
                              hipStream_t st);
bool tiled_supports(const Params &p, int dtype);
bool decode_supports(const Params &p, int dtype);
bool decode_appends(const Params &p, int dtype);
hipError_t launch_decode(const Params &p, int dtype, int split_keys, int n_split, float *ws,
                         bool append, hipStream_t st);
bool qk_mfma_supports(const Params &p, int dtype);
hipError_t launch_qk_mfma(const Params &p, int dtype, hipStream_t st);
}  // namespace olk

namespace {

thread_local const char *g_last_kernel = "";
thread_local char g_name_buf[96];

// qk_matmul_output after the attention kernels: on the matrix cores where the
// shapes allow (not with the generic kernel forced), else the VALU kernel; the
// last-kernel name gains the qk kernel's.
hipError_t launch_qk_output(const olk::Params &p, const olk_attn_desc *desc, hipStream_t s) {
  const bool mf = desc->kernel != OLK_KERNEL_GENERIC && olk::qk_mfma_supports(p, desc->dtype);
  const hipError_t e = mf ? olk::launch_qk_mfma(p, desc->dtype, s) : olk::launch_qk(p, desc->dtype, s);
  snprintf(g_name_buf, sizeof(g_name_buf), "%s+%s", g_last_kernel, mf ? "olk_qk_mfma" : "olk_qk");
  g_last_kernel = g_name_buf;
  return e;
}

// Keys per split of the decode path (both kernel families; a multiple of the
// tiled kernel's 64-key tile).
constexpr int kSplitKeys = 512;
constexpr int kDecodeSplitKeys = 1024;  // keys per split of the dedicated decode kernel

size_t esize_of(int dtype) { return dtype == OLK_F32 ? 4 : 2; }

struct Range {
  const char *p;
  size_t n;
};

bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  return a.p < b.p + b.n && b.p < a.p + a.n;
}

// Sizes of every tensor in bytes (int64 arithmetic, checked by the caller).
struct Sizes {
  size_t q, k, v, past_k, past_v, bias, sink, proj, y, pres_k, pres_v, rot, mask, qk;
};

// attn_bias / attn_mask extents: rows per (b, h) and columns
int64_t rows_of(int32_t ext_s, int64_t S) { return ext_s == 1 ? 1 : S; }
int64_t cols_of(int32_t ext_t, int64_t T) { return ext_t > 0 ? ext_t : T; }

Sizes sizes_of(const olk_attn_desc *d) {
  const size_t es = esize_of(d->dtype);
  const size_t B = d->batch, S = d->q_seq, L = d->kv_seq, P = d->past_seq;
  const size_t Hq = d->q_num_heads, Hkv = d->kv_num_heads, D = d->head_size,
               Dv = d->v_head_size, T = P + L;
  Sizes s;
  s.q = B * S * Hq * D * es;
  s.k = B * L * Hkv * D * es;
  s.v = B * L * Hkv * Dv * es;
  s.past_k = B * Hkv * P * D * es;
  s.past_v = B * Hkv * P * Dv * es;
  s.bias = (size_t)(d->bias_b > 0 ? d->bias_b : 0) * (size_t)(d->bias_h > 0 ? d->bias_h : 0) *
           (size_t)rows_of(d->bias_s, S) * (size_t)cols_of(d->bias_t, T) * es;
  s.mask = (size_t)(d->mask_b > 0 ? d->mask_b : 0) * (size_t)(d->mask_h > 0 ? d->mask_h : 0) *
           (size_t)rows_of(d->mask_s, S) * (size_t)cols_of(d->mask_t, T) *
           (d->mask_kind == OLK_MASK_BINARY_I32 ? 4 : 1);
  s.qk = B * Hq * S * T * 4;
  s.sink = Hq * es;
  s.proj = (2 * Hq * D + Hq * Dv) * es;
  s.y = B * S * Hq * Dv * es;
  s.pres_k = B * Hkv * T * D * es;
  s.pres_v = B * Hkv * T * Dv * es;
  const size_t R = d->rotary_dim > 0 ? d->rotary_dim : D;
  s.rot = d->do_rotary ? (size_t)(d->rotary_max_pos > 0 ? d->rotary_max_pos : 0) * (R / 2) * es : 0;
  return s;
}

olk_status validate(const olk_attn_desc *d, const olk_attn_io *io) {
  if (!d || !io) return OLK_E_NULL;
  if (d->op < OLK_OP_GQA || d->op > OLK_OP_ATTENTION) return OLK_E_ATTR;
  if (d->dtype < OLK_F32 || d->dtype > OLK_BF16) return OLK_E_ATTR;
  if (d->kernel < OLK_KERNEL_AUTO || d->kernel > OLK_KERNEL_TILED) return OLK_E_ATTR;
  if (d->causal != 0 && d->causal != 1) return OLK_E_ATTR;
  if (d->kv_inplace != 0 && d->kv_inplace != 1) return OLK_E_ATTR;
  if (d->has_scale && !isfinite(d->scale)) return OLK_E_ATTR;
  if (!(d->softcap >= 0.f) || isinf(d->softcap)) return OLK_E_ATTR;
  if (d->op == OLK_OP_MHA && !isfinite(d->mask_filter_value)) return OLK_E_ATTR;
  // local_window_size: -1 (full) or positive; zero and values below -1 are
  // rejected, and so is a local window without causal masking.
  const int w = d->local_window_size;
  if (w == 0 || w < -1) return OLK_E_ATTR;
  if (w > 0 && (d->op != OLK_OP_GQA || !d->causal)) return OLK_E_ATTR;
  if (d->softcap > 0.f && d->op == OLK_OP_MHA) return OLK_E_ATTR;
  // rotary embedding: GroupQueryAttention only; R even, 0 < R <= D
  if (d->do_rotary != 0 && d->do_rotary != 1) return OLK_E_ATTR;
  if (d->rotary_interleaved != 0 && d->rotary_interleaved != 1) return OLK_E_ATTR;
  if (d->do_rotary) {
    const int R = d->rotary_dim > 0 ? d->rotary_dim : d->head_size;
    if (d->op != OLK_OP_GQA || d->rotary_dim < 0 || R % 2 || R > d->head_size) return OLK_E_ATTR;
    if (d->rotary_max_pos <= 0) return OLK_E_SHAPE;
  }

  if (d->batch < 0 || d->q_seq < 0 || d->kv_seq < 0 || d->past_seq < 0) return OLK_E_SHAPE;
  if (d->q_num_heads <= 0 || d->kv_num_heads <= 0) return OLK_E_SHAPE;
  if (d->q_num_heads % d->kv_num_heads) return OLK_E_SHAPE;
  if (d->head_size <= 0 || d->v_head_size <= 0) return OLK_E_SHAPE;
  if (d->q_rank != 3 && d->q_rank != 4) return OLK_E_SHAPE;
  if (d->kv_rank != 3 && d->kv_rank != 4) return OLK_E_SHAPE;
  if ((int64_t)d->past_seq + d->kv_seq > INT32_MAX) return OLK_E_SHAPE;
  const int64_t T_all = (int64_t)d->past_seq + d->kv_seq;
  if (io->attn_bias) {
    if (d->bias_b != 1 && d->bias_b != d->batch) return OLK_E_SHAPE;
    if (d->bias_h != 1 && d->bias_h != d->q_num_heads) return OLK_E_SHAPE;
    if (d->bias_s != 0 && d->bias_s != 1 && d->bias_s != d->q_seq) return OLK_E_SHAPE;
    if (d->bias_t < 0 || d->bias_t > T_all) return OLK_E_SHAPE;
    // a shorter last dimension (padded with -inf) is an ai.onnx Attention mask
    if (d->bias_t > 0 && d->bias_t < T_all && d->op != OLK_OP_ATTENTION) return OLK_E_SHAPE;
  }
  if (d->mask_kind < OLK_MASK_NONE || d->mask_kind > OLK_MASK_BINARY_I32) return OLK_E_ATTR;
  if (d->mask_kind == OLK_MASK_BOOL && d->op != OLK_OP_ATTENTION) return OLK_E_ATTR;
  if (d->mask_kind == OLK_MASK_BINARY_I32) {
    // one key-padding input: lengths or a binary mask
    if (d->op != OLK_OP_MHA || io->seqlens) return OLK_E_ATTR;
    if (d->mask_t != 0 && d->mask_t != T_all) return OLK_E_SHAPE;
  }
  if (d->mask_kind != OLK_MASK_NONE) {
    if (d->mask_b != 1 && d->mask_b != d->batch) return OLK_E_SHAPE;
    if (d->mask_h != 1 && d->mask_h != d->q_num_heads) return OLK_E_SHAPE;
    if (d->mask_s != 0 && d->mask_s != 1 && d->mask_s != d->q_seq) return OLK_E_SHAPE;
    if (d->mask_t < 0 || d->mask_t > T_all) return OLK_E_SHAPE;
  }
  if (d->seqlens_i64 != 0 && d->seqlens_i64 != 1) return OLK_E_ATTR;
  if (d->seqlens_i64 && d->op != OLK_OP_ATTENTION) return OLK_E_ATTR;
  if (io->qk_out && (d->op != OLK_OP_ATTENTION || d->qk_mode < 0 || d->qk_mode > 3))
    return OLK_E_ATTR;

  switch (d->op) {
    case OLK_OP_GQA:
      if (d->q_rank != 3 || d->kv_rank != 3) return OLK_E_SHAPE;
      if (d->kv_seq != d->q_seq) return OLK_E_SHAPE;
      if (io->proj_bias) return OLK_E_ATTR;
      if (!io->seqlens && d->batch > 0) return OLK_E_NULL;
      break;
    case OLK_OP_MHA:
      if (d->q_rank != 3) return OLK_E_SHAPE;
      if (d->kv_num_heads != d->q_num_heads) return OLK_E_SHAPE;
      if (io->head_sink || d->kv_inplace) return OLK_E_ATTR;
      // rank-3 K/V with their projection-bias segments: the biased rows are
      // written to present and read back, so present is required
      if (io->proj_bias && d->kv_rank == 3 && d->batch > 0 && d->kv_seq > 0 &&
          (!io->present_k || !io->present_v))
        return OLK_E_UNSUPPORTED;
      break;
    default:  // ai.onnx::Attention
      if (io->head_sink || io->proj_bias || d->kv_inplace) return OLK_E_ATTR;
      break;
  }

  const Sizes sz = sizes_of(d);
  if (!io->q && sz.q) return OLK_E_NULL;
  if ((!io->k && sz.k) || (!io->v && sz.v)) return OLK_E_NULL;
  if (!io->y && sz.y) return OLK_E_NULL;
  if (d->mask_kind != OLK_MASK_NONE && !io->attn_mask && sz.mask) return OLK_E_NULL;
  if (d->kv_inplace) {
    if ((!io->present_k && sz.pres_k) || (!io->present_v && sz.pres_v)) return OLK_E_NULL;
    if (io->past_k && io->past_k != io->present_k) return OLK_E_SHAPE;
    if (io->past_v && io->past_v != io->present_v) return OLK_E_SHAPE;
  } else if (d->past_seq > 0) {
    if ((!io->past_k && sz.past_k) || (!io->past_v && sz.past_v)) return OLK_E_NULL;
  }
  if (d->head_size > 256 || d->v_head_size > 256) return OLK_E_UNSUPPORTED;
  if (d->do_rotary && sz.q) {
    if (!io->cos_cache || !io->sin_cache) return OLK_E_NULL;
    // the rotated keys are written to present and read back; rotated Q is
    // staged in Y, which needs Y rows of Q's width
    if (!io->present_k || !io->present_v) return OLK_E_UNSUPPORTED;
    if (d->v_head_size != d->head_size) return OLK_E_UNSUPPORTED;
  }
  if (d->q_num_heads > 65535 || d->batch > 65535) return OLK_E_UNSUPPORTED;

  // Outputs must not overlap inputs or each other (kv_inplace: present is the past).
  const Range outs[4] = {{(const char *)io->y, sz.y},
                         {(const char *)io->present_k, sz.pres_k},
                         {(const char *)io->present_v, sz.pres_v},
                         {(const char *)io->qk_out, io->qk_out ? sz.qk : 0}};
  const Range ins[11] = {{(const char *)io->q, sz.q},
                        {(const char *)io->k, sz.k},
                        {(const char *)io->v, sz.v},
                        {d->kv_inplace ? nullptr : (const char *)io->past_k,
                         d->past_seq ? sz.past_k : 0},
                        {d->kv_inplace ? nullptr : (const char *)io->past_v,
                         d->past_seq ? sz.past_v : 0},
                        {(const char *)io->attn_bias, io->attn_bias ? sz.bias : 0},
                        {(const char *)io->head_sink, io->head_sink ? sz.sink : 0},
                        {(const char *)io->proj_bias, io->proj_bias ? sz.proj : 0},
                        {(const char *)io->cos_cache, sz.rot},
                        {(const char *)io->sin_cache, sz.rot},
                        {(const char *)io->attn_mask, d->mask_kind ? sz.mask : 0}};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 11; ++b)
      if (overlaps(outs[a], ins[b])) return OLK_E_SHAPE;
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], outs[b])) return OLK_E_SHAPE;
  }
  return OLK_OK;
}

olk::Params make_params(const olk_attn_desc *d, const olk_attn_io *io) {
  olk::Params p;
  memset(&p, 0, sizeof(p));
  p.q = io->q;
  p.k = io->k;
  p.v = io->v;
  p.past_k = d->kv_inplace ? io->present_k : io->past_k;
  p.past_v = d->kv_inplace ? io->present_v : io->past_v;
  p.seqlens = io->seqlens;
  p.bias = io->attn_bias;
  p.sink = io->head_sink;
  p.proj_bias = d->op == OLK_OP_MHA ? io->proj_bias : nullptr;
  p.y = io->y;
  p.present_k = io->present_k;
  p.present_v = io->present_v;
  const int64_t S = d->q_seq, L = d->kv_seq, Hq = d->q_num_heads, Hkv = d->kv_num_heads,
                D = d->head_size, Dv = d->v_head_size;
  p.B = d->batch;
  p.S = d->q_seq;
  p.L = d->kv_seq;
  p.P = d->past_seq;
  p.T = d->past_seq + d->kv_seq;
  p.past_rows = d->kv_inplace ? p.T : p.P;
  p.Hq = d->q_num_heads;
  p.Hkv = d->kv_num_heads;
  p.G = d->q_num_heads / d->kv_num_heads;
  p.D = d->head_size;
  p.Dv = d->v_head_size;
  if (d->q_rank == 3) {  // (B, S, Hq*D)
    p.q_sb = S * Hq * D; p.q_ss = Hq * D; p.q_sh = D;
    p.y_sb = S * Hq * Dv; p.y_ss = Hq * Dv; p.y_sh = Dv;
  } else {               // (B, Hq, S, D)
    p.q_sb = Hq * S * D; p.q_sh = S * D; p.q_ss = D;
    p.y_sb = Hq * S * Dv; p.y_sh = S * Dv; p.y_ss = Dv;
  }
  if (d->kv_rank == 3) {  // (B, L, Hkv*D)
    p.k_sb = L * Hkv * D; p.k_ss = Hkv * D; p.k_sh = D;
    p.v_sb = L * Hkv * Dv; p.v_ss = Hkv * Dv; p.v_sh = Dv;
  } else {                // (B, Hkv, L, D)
    p.k_sb = Hkv * L * D; p.k_sh = L * D; p.k_ss = D;
    p.v_sb = Hkv * L * Dv; p.v_sh = L * Dv; p.v_ss = Dv;
  }
  const int64_t T = p.T;
  {
    const int64_t rs = rows_of(d->bias_s, S), cs = cols_of(d->bias_t, T);
    p.bias_si = rs > 1 ? cs : 0;
    p.bias_sh = d->bias_h > 1 ? rs * cs : 0;
    p.bias_sb = d->bias_b > 1 ? (int64_t)d->bias_h * rs * cs : 0;
    p.bias_cols = (int)cs;
  }
  if (d->mask_kind != OLK_MASK_NONE) {
    const int64_t rs = rows_of(d->mask_s, S), cs = cols_of(d->mask_t, T);
    p.mask = io->attn_mask;
    p.mask_kind = d->mask_kind;
    p.mask_si = rs > 1 ? cs : 0;
    p.mask_sh = d->mask_h > 1 ? rs * cs : 0;
    p.mask_sb = d->mask_b > 1 ? (int64_t)d->mask_h * rs * cs : 0;
    p.mask_cols = (int)cs;
  }
  p.seqlens64 = d->seqlens_i64;
  p.qk_out = io->qk_out;
  p.qk_mode = d->qk_mode;
  p.op = d->op;
  p.causal = d->causal;
  p.window = d->local_window_size > 0 ? d->local_window_size : -1;
  p.kv_inplace = d->kv_inplace;
  p.scale = d->has_scale ? d->scale : 1.0f / sqrtf((float)d->head_size);
  p.softcap = d->softcap;
  p.mfv = d->mask_filter_value;
  // MultiHeadAttention key padding adds mask_filter_value to the padded keys'
  // scores.  At -5000 or below, exp of such a score relative to the row's
  // maximum underflows to exactly 0 in float32 unless it exceeds the largest
  // real score by thousands, so the padded keys are excluded instead: the
  // kernels stop at the row's length and never read them.
  p.pad_add = (d->op == OLK_OP_MHA && io->seqlens && !(d->mask_filter_value <= -5000.f)) ? 1 : 0;
  p.cos_cache = io->cos_cache;
  p.sin_cache = io->sin_cache;
  p.rot_dim = d->rotary_dim > 0 ? d->rotary_dim : d->head_size;
  p.rot_inter = d->rotary_interleaved;
  p.rot_max = d->rotary_max_pos;
  return p;
}

// MultiHeadAttention rank-3 K/V with a projection bias: the past rows and the
// biased new rows go to present, and the attention reads every key from there
// (Q keeps its bias segment in the kernels).
bool kv_bias_path(const olk_attn_desc *d, const olk_attn_io *io) {
  return d->op == OLK_OP_MHA && d->kv_rank == 3 && io->proj_bias != nullptr;
}

hipError_t kv_bias_prepass(olk::Params &p, int dtype, hipStream_t st) {
  olk::Params pp = p;
  pp.present_past_only = 1;
  hipError_t e = olk::launch_present(pp, dtype, st);
  if (e != hipSuccess) return e;
  e = olk::launch_kv_bias(p, dtype, st);
  if (e != hipSuccess) return e;
  p.past_k = p.present_k;
  p.past_v = p.present_v;
  p.past_rows = p.T;
  p.keys_in_past = 1;
  p.present_k = p.present_v = nullptr;
  return hipSuccess;
}

// do_rotary: copy the past rows into present (out of place), run the rotary
// pre-pass (rotated Q into Y, rotated new K and new V into present), and
// return the parameters of the attention proper: Q read from Y, every key read
// from present, nothing left for the attention kernels to write into present.
// With q_in_kernel the prefill kernel rotates Q as it loads it: the pre-pass
// leaves Q alone and the attention reads Q from Q.
hipError_t rotary_prepass(olk::Params &p, int dtype, hipStream_t st, bool q_in_kernel = false) {
  olk::Params pp = p;
  pp.present_past_only = 1;
  hipError_t e = olk::launch_present(pp, dtype, st);
  if (e != hipSuccess) return e;
  p.rot_q = q_in_kernel ? 1 : 0;
  // with Q rotated in the prefill kernel, that kernel also takes the new V
  // rows from V and writes their present rows (the pre-pass writes only K)
  p.rot_skip_v = q_in_kernel ? 1 : 0;
  e = olk::launch_rope(p, dtype, st);
  if (e != hipSuccess) return e;
  if (!q_in_kernel) {
    p.q = p.y;
    p.q_sb = p.y_sb; p.q_ss = p.y_ss; p.q_sh = p.y_sh;
  }
  p.past_k = p.present_k;
  p.past_v = p.present_v;
  p.past_rows = p.T;
  p.keys_in_past = 1;
  p.present_k = nullptr;
  if (q_in_kernel) {
    p.v_new_rows = 1;  // present_v stays set: the new V rows are written there
  } else {
    p.present_v = nullptr;
  }
  return hipSuccess;
}

// Built-in scratch of olk_attention_decode_noalloc: the split partials that
// olk_attention_decode keeps in the caller's workspace live here instead.
// Each device holds its own copy until the process ends.  In host code the
// name `scratch` is only a host-side handle: kernels get the device address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = OLK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not yet looked up)

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
olk_status scratch_for_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return OLK_E_HIP;
  if (dev >= kMaxDevices) return OLK_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return OLK_E_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return OLK_OK;
}

int n_splits(const olk_attn_desc *d, int split_keys = kSplitKeys) {
  const int64_t T = (int64_t)d->past_seq + d->kv_seq;
  const int64_t n = (T + split_keys - 1) / split_keys;
  return n < 1 ? 1 : (int)n;
}

}  // namespace

extern "C" {

olk_status olk_validate(const olk_attn_desc *desc, const olk_attn_io *io) {
  return validate(desc, io);
}

size_t olk_workspace_bytes(const olk_attn_desc *d) {
  if (!d || d->batch <= 0 || d->q_seq <= 0 || d->q_num_heads <= 0 || d->v_head_size <= 0)
    return 0;
  const size_t rows = (size_t)d->batch * d->q_seq * d->q_num_heads;
  // one record [m, l, -, -, O[Dv]] of floats per (row, split)
  const size_t bytes = rows * (size_t)n_splits(d) * (size_t)(d->v_head_size + 4) * 4;
  return (bytes + 255) & ~(size_t)255;
}

olk_status olk_attention_fwd(const olk_attn_desc *desc, const olk_attn_io *io, void *stream) {
  const olk_status st = validate(desc, io);
  if (st != OLK_OK) return st;
  olk::Params p = make_params(desc, io);
  hipStream_t s = (hipStream_t)stream;
  // the kernel choice is made on the parameters the attention kernel gets (with
  // do_rotary, Q is read from Y); check it before anything is launched
  olk::Params pa = p;
  // do_rotary: the prefill kernel rotates Q itself where it can, otherwise Q is
  // rotated into Y by the pre-pass and read from there
  const bool q_in_kernel = desc->do_rotary && desc->kernel != OLK_KERNEL_GENERIC &&
                           olk::tiled_supports(p, desc->dtype) && olk::flash_rotates_q(p);
  if (desc->do_rotary && !q_in_kernel) {
    pa.q = pa.y; pa.q_sb = pa.y_sb; pa.q_ss = pa.y_ss; pa.q_sh = pa.y_sh;
  }
  const bool tiled_ok = q_in_kernel || olk::tiled_supports(pa, desc->dtype);
  if (desc->kernel == OLK_KERNEL_TILED && !tiled_ok) return OLK_E_UNSUPPORTED;
  const bool use_tiled = desc->kernel != OLK_KERNEL_GENERIC && tiled_ok;
  hipError_t e = hipSuccess;
  if (desc->do_rotary) {
    e = rotary_prepass(p, desc->dtype, s, q_in_kernel);
  } else if (kv_bias_path(desc, io)) {
    e = kv_bias_prepass(p, desc->dtype, s);
  } else {
    // the attention kernel writes the present rows of the new keys itself
    // (the generic kernel always, the prefill kernel for GroupQueryAttention)
    if (!use_tiled || olk::flash_fuses_present(p)) p.present_past_only = 1;
    e = olk::launch_present(p, desc->dtype, s);
  }
  if (e != hipSuccess) return OLK_E_HIP;
  if (use_tiled) {
    e = olk::launch_flash(p, desc->dtype, s);
    g_last_kernel = desc->do_rotary ? "olk_rope+olk_tiled_fwd" : "olk_tiled_fwd";
  } else {
    e = olk::launch_generic(p, desc->dtype, s);
    g_last_kernel = desc->do_rotary ? "olk_rope+olk_generic_fwd" : "olk_generic_fwd";
  }
  if (e == hipSuccess && p.qk_out) e = launch_qk_output(p, desc, s);
  return e == hipSuccess ? OLK_OK : OLK_E_HIP;
}

olk_status olk_attention_decode(const olk_attn_desc *desc, const olk_attn_io *io,
                                void *workspace, size_t workspace_bytes, void *stream) {
  const olk_status st = validate(desc, io);
  if (st != OLK_OK) return st;
  if ((int64_t)desc->batch * desc->q_seq > 65535) return OLK_E_UNSUPPORTED;
  if (n_splits(desc) > 4096) return OLK_E_UNSUPPORTED;  // combine kernel's weight buffer
  const size_t need = olk_workspace_bytes(desc);
  if (need && (!workspace || workspace_bytes < need)) return OLK_E_WORKSPACE;
  if (((uintptr_t)workspace & 15) != 0) return OLK_E_WORKSPACE;
  olk::Params p = make_params(desc, io);
  hipStream_t s = (hipStream_t)stream;
  olk::Params pa = p;
  if (desc->do_rotary) { pa.q = pa.y; pa.q_sb = pa.y_sb; pa.q_ss = pa.y_ss; pa.q_sh = pa.y_sh; }
  // Matrix-core paths: the decode kernel (up to 16 rows per KV head; its key
  // source is the past buffer, or present once the new rows are appended
  // there), else the tiled split partials, which take no attn_mask.
  const bool tiled_ok = olk::tiled_supports(pa, desc->dtype);
  olk::Params pchk = p;
  if (pchk.present_k && pchk.present_v) pchk.keys_in_past = 1;
  const bool decode_ok = tiled_ok && olk::decode_supports(pchk, desc->dtype);
  const bool split_ok = tiled_ok && !pa.mask && pa.D != 256;  // the split partials: 64 or 128
  if (desc->kernel == OLK_KERNEL_TILED && !decode_ok && !split_ok) return OLK_E_UNSUPPORTED;
  // In place at head size 128 the decode kernel appends the new rows itself
  // (no separate copy launch); every other case appends before the split kernels.
  bool append_in_decode = false;
  if (!desc->do_rotary && !kv_bias_path(desc, io) && desc->kernel != OLK_KERNEL_GENERIC &&
      decode_ok && p.kv_inplace) {
    olk::Params pk = p;
    pk.keys_in_past = 1;
    append_in_decode = olk::decode_appends(pk, desc->dtype);
  }
  hipError_t e = desc->do_rotary        ? rotary_prepass(p, desc->dtype, s)
                 : kv_bias_path(desc, io) ? kv_bias_prepass(p, desc->dtype, s)
                 : append_in_decode       ? hipSuccess
                                          : olk::launch_present(p, desc->dtype, s);
  if (e != hipSuccess) return OLK_E_HIP;
  if (!p.keys_in_past && p.present_k && p.present_v) {
    // present now holds the whole key sequence (past rows, then the new ones):
    // the split kernels read every key from it, as from one past buffer
    p.past_k = p.present_k;
    p.past_v = p.present_v;
    p.past_rows = p.T;
    p.keys_in_past = 1;
    p.present_k = p.present_v = nullptr;
  }
  const int n_split = n_splits(desc);
  int n_comb = n_split, comb_keys = kSplitKeys;
  if (desc->kernel != OLK_KERNEL_GENERIC && decode_ok && olk::decode_supports(p, desc->dtype)) {
    n_comb = n_splits(desc, kDecodeSplitKeys);
    comb_keys = kDecodeSplitKeys;
    e = olk::launch_decode(p, desc->dtype, kDecodeSplitKeys, n_comb, (float *)workspace,
                           append_in_decode, s);
    g_last_kernel = "olk_decode_split+combine";
  } else if (desc->kernel != OLK_KERNEL_GENERIC && split_ok) {
    e = olk::launch_tiled_split(p, desc->dtype, kSplitKeys / 64, (float *)workspace, s);
    g_last_kernel = "olk_tiled_split+combine";
  } else {
    e = olk::launch_generic_split(p, desc->dtype, kSplitKeys, n_split, (float *)workspace, s);
    g_last_kernel = "olk_generic_split+combine";
  }
  if (e != hipSuccess) return OLK_E_HIP;
  e = olk::launch_combine(p, desc->dtype, n_comb, comb_keys, (const float *)workspace, s);
  if (e == hipSuccess && p.qk_out) e = launch_qk_output(p, desc, s);
  return e == hipSuccess ? OLK_OK : OLK_E_HIP;
}

olk_status olk_attention_decode_noalloc(const olk_attn_desc *desc, const olk_attn_io *io,
                                        void *stream) {
  const olk_status st = validate(desc, io);
  if (st != OLK_OK) return st;
  const size_t need = olk_workspace_bytes(desc);
  if (need > kScratchBytes) return OLK_E_WORKSPACE;
  void *ws = nullptr;
  if (need) {
    const olk_status e = scratch_for_current_device(&ws);
    if (e != OLK_OK) return e;
  }
  return olk_attention_decode(desc, io, ws, need, stream);
}

size_t olk_bwd_workspace_bytes(const olk_attn_desc *d) {
  if (!d || d->batch <= 0 || d->q_seq <= 0 || d->q_num_heads <= 0) return 0;
  const size_t bytes = (size_t)d->batch * d->q_seq * d->q_num_heads * 2 * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

olk_status olk_attention_bwd(const olk_attn_desc *desc, const olk_attn_bwd_io *io,
                             void *workspace, size_t workspace_bytes, void *stream) {
  if (!desc || !io) return OLK_E_NULL;
  // scope of the backward first, then the forward contract on the same tensors
  if (desc->op != OLK_OP_GQA || desc->past_seq != 0 || desc->softcap > 0.f ||
      desc->do_rotary || desc->mask_kind != OLK_MASK_NONE || desc->kv_inplace)
    return OLK_E_UNSUPPORTED;
  olk_attn_io fio;
  memset(&fio, 0, sizeof(fio));
  fio.q = io->q;
  fio.k = io->k;
  fio.v = io->v;
  fio.seqlens = io->seqlens;
  fio.y = io->dq;  // stands in for a Y-sized output in the null checks only
  olk_status st = validate(desc, &fio);
  if (st != OLK_OK) return st;
  const olk_attn_desc *d = desc;
  const size_t es = esize_of(d->dtype);
  const size_t B = d->batch, S = d->q_seq, Hq = d->q_num_heads, Hkv = d->kv_num_heads,
               D = d->head_size, Dv = d->v_head_size;
  const size_t nq = B * S * Hq * D * es, nk = B * S * Hkv * D * es, nv = B * S * Hkv * Dv * es,
               ndy = B * S * Hq * Dv * es;
  if (ndy && !io->dy) return OLK_E_NULL;
  if ((nq && !io->dq) || (nk && !io->dk) || (nv && !io->dv)) return OLK_E_NULL;
  const Range outs[3] = {{(const char *)io->dq, nq}, {(const char *)io->dk, nk},
                         {(const char *)io->dv, nv}};
  const Range ins[4] = {{(const char *)io->q, nq}, {(const char *)io->k, nk},
                        {(const char *)io->v, nv}, {(const char *)io->dy, ndy}};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 4; ++b)
      if (overlaps(outs[a], ins[b])) return OLK_E_SHAPE;
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], outs[b])) return OLK_E_SHAPE;
  }
  const size_t need = olk_bwd_workspace_bytes(desc);
  if (need && (!workspace || workspace_bytes < need)) return OLK_E_WORKSPACE;
  if (((uintptr_t)workspace & 15) != 0) return OLK_E_WORKSPACE;
  const olk::Params p = make_params(desc, &fio);
  const hipError_t e = olk::launch_backward(p, desc->dtype, io->dy, io->dq, io->dk, io->dv,
                                            (float *)workspace, (hipStream_t)stream);
  g_last_kernel = olk::backward_mfma_supports(p, desc->dtype, io->dy, io->dq, io->dk, io->dv)
                      ? "olk_bwd_dq_mfma+dkv_mfma"
                      : "olk_bwd_stats+dq+dkv";
  return e == hipSuccess ? OLK_OK : OLK_E_HIP;
}

const char *olk_status_str(olk_status s) {
  switch (s) {
    case OLK_OK: return "ok";
    case OLK_E_NULL: return "required pointer is NULL";
    case OLK_E_ATTR: return "attribute value rejected by the operator contract";
    case OLK_E_SHAPE: return "inconsistent sizes, ranks or overlapping buffers";
    case OLK_E_UNSUPPORTED: return "valid but not supported by this library";
    case OLK_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case OLK_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char *olk_last_kernel_name(void) { return g_last_kernel; }

}  // extern "C"
