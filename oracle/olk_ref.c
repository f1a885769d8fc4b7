/*
 * olk_ref — the oracle for the attention forward.  TEST INFRASTRUCTURE ONLY:
 * it is loaded by tests/, by the smoke check and by the benchmark's CPU
 * baseline, never by the product path (transformer_attention_fwd_amd/).
 * It shares no code, header or table with the HIP library.
 *
 * What it computes is the plain definition of scaled dot-product attention,
 * written out row by row in float64 with libm exp/tanh:
 *
 *   Y = Softmax((Q @ K^T) * scale + bias) @ V
 *     (onnx-light reference kernels header page, "class Attention": the
 *      baseline computation, the scale default 1/sqrt(head_size), the
 *      softcap s -> softcap*tanh(s/softcap), GQA head sharing, past/present
 *      concatenation, nonpad_kv_seqlen)
 *
 * with the operator-specific parts of
 *   - onnx-light-cpu Python API "Custom operators", section "Microsoft
 *     GroupQueryAttention": causal local window (a positive window counts the
 *     attended tokens including the current one), present = entire past
 *     followed by the current step, head_sink as a virtual logit that adds to
 *     the denominator only, masks applied to real keys only;
 *   - same page, section "Microsoft MultiHeadAttention": rank-4
 *     cross-attention K/V, projection bias (only its query segment with rank-4
 *     K/V), int32 key-padding lengths, additive bias (1|B, 1|N, S, T),
 *     scale 1/sqrt(H), mask_filter_value -10000;
 *   - onnx-light-cpu C++ API "Custom operators", GroupQueryAttention gradient
 *     (default scale 1/sqrt(Shape(Q)[2]/num_heads), grouped K/V heads) and
 *     GroupQueryAttentionFusionPattern (seqlens_k derived from the key length).
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes with its support):
 *   R1  GroupQueryAttention seqlens_k[b] = total_b - 1, past_b = total_b - S.
 *   R3  causal alignment: query i sits at absolute position past_b + i, where
 *       past_b is the number of cached keys in front of the new ones (GQA:
 *       the valid past of batch b; MHA / Attention: the past buffer length
 *       P).  For Attention the header page aligns the causal mask to the
 *       upper-left corner of the score matrix and shifts it by the cached KV:
 *       query i attends every cached key and the new keys 0..i.
 *   R4  window W > 0 allows keys j with pos_i - W + 1 <= j <= pos_i.
 *   R5  query head h reads KV head h / (Hq / Hkv).
 *   R6  order: scale, + bias, softcap, then masks as exclusion.
 *   R7  the sink logit is used raw (not scaled, not softcapped).
 *   R9  MHA key padding adds mask_filter_value to the padded keys' scores;
 *       they stay in the softmax.
 *   R10 a row with no allowed key outputs 0.
 *   R11 MHA projection bias layout is [q (N*H) | k (N*H) | v (N*Hv)].
 *   R21 with rank-3 K/V (self-attention) the k and v segments are added to
 *       the new K/V rows; the biased rows are element-type tensors (float32
 *       add, rounded once) and present holds them.
 *   R18 rotary embedding (GroupQueryAttention do_rotary): Q and the new K rows
 *       are rotated at their absolute positions (past_b + i), the past is used
 *       as stored, V is not rotated, and present_key holds the rotated keys.
 *       The rotation follows the RotaryEmbedding kernel of the reference
 *       kernels header page ("class RotaryEmbedding": rank-2 cos/sin caches
 *       indexed by position, rotary_embedding_dim, interleaved pairing), i.e.
 *       each pair (x1, x2) becomes (x1 cos - x2 sin, x2 cos + x1 sin) as in
 *       arXiv 2104.09864.  The rotated values are tensors of the element type:
 *       computed in float32 as fmaf(x1, c, -(x2*s)) and fmaf(x2, c, x1*s) and
 *       rounded once (RNE), so present holds exactly these bits.  Positions
 *       beyond the cache use its last row.
 *   R19 masks (reference kernels header page, "class Attention": FLOAT masks
 *       rank 2-4 broadcast to (B, Hq, S, T) and added as a bias, BOOL masks
 *       with false = -inf, a last dimension shorter than T padded with
 *       -inf/false, INT64 nonpad_kv_seqlen; Python API page,
 *       MultiHeadAttention: binary key-padding masks (B,T)/(B,S,T)).  A FLOAT
 *       mask is the additive bias; keys beyond its columns, BOOL-false keys
 *       and keys at or beyond nonpad are excluded after the score pipeline
 *       (R6); a zero in a MultiHeadAttention binary mask adds
 *       mask_filter_value like key padding (R9).
 *   R20 qk_matmul_output (modes 0-3): mode 0 is (Q K^T) * scale for every
 *       (i, j); modes 1 and 2 add the bias and apply the softcap to allowed
 *       keys and hold -inf for excluded ones; mode 3 is the softmax weight
 *       (0 for excluded keys).
 * Intermediate values are not rounded (apart from R18's rotated Q/K); Y is
 * returned in float64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_GQA = 0, REF_MHA = 1, REF_ATTENTION = 2 };
enum { REF_F32 = 0, REF_F16 = 1, REF_BF16 = 2 };

typedef struct {
  int32_t op, dtype;
  int32_t batch, q_seq, kv_seq, past_seq;
  int32_t q_heads, kv_heads, head_size, v_head_size;
  int32_t q_rank, kv_rank;
  int32_t causal, window;
  int32_t has_scale;
  float scale, softcap, mask_filter_value;
  int32_t bias_b, bias_h;
  int32_t do_rotary, rotary_interleaved, rotary_dim, rotary_max_pos;
  int32_t bias_s, bias_t;                      /* bias rows: 1 = broadcast; columns (0 = T) */
  int32_t mask_kind, mask_b, mask_h, mask_s, mask_t;
  int32_t seqlens_i64;
} ref_desc;

typedef struct {
  const void *q, *k, *v, *past_k, *past_v;
  const int32_t *lens;
  const void *bias, *sink, *proj_bias;
  const void *cos_cache, *sin_cache;
  const void *mask;
} ref_inputs;

/* ---- element decoding (format definitions, not attention arithmetic) ---- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float x;
  memcpy(&x, &u, 4);
  return (double)x;
}

static double elem(const void *base, int dtype, size_t idx) {
  if (dtype == REF_F32) return (double)((const float *)base)[idx];
  uint16_t h = ((const uint16_t *)base)[idx];
  return dtype == REF_F16 ? half_to_double(h) : bf16_to_double(h);
}

static size_t esize(int dtype) { return dtype == REF_F32 ? 4 : 2; }

/* float32 -> binary16, round to nearest even (IEEE 754 conversion). */
static uint16_t float_to_half(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t e = (u >> 23) & 0xff, m = u & 0x7fffffu;
  if (e == 0xff) return sign | 0x7c00u | (m ? 0x200u : 0u);   /* inf / NaN */
  int ex = (int)e - 127 + 15;
  if (ex >= 31) return sign | 0x7c00u;                         /* overflow */
  if (ex <= 0) {                                               /* subnormal or zero */
    if (ex < -10) return sign;
    uint32_t mant = m | 0x800000u;
    int shift = 14 - ex;                                       /* 24-bit mantissa -> 10 - ex bits */
    uint32_t q = mant >> shift, rem = mant & ((1u << shift) - 1), halfway = 1u << (shift - 1);
    if (rem > halfway || (rem == halfway && (q & 1))) ++q;
    return sign | (uint16_t)q;
  }
  uint32_t q = ((uint32_t)ex << 10) | (m >> 13), rem = m & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (q & 1))) ++q;     /* may carry into the exponent */
  return sign | (uint16_t)q;
}

/* float32 -> bfloat16 (upper half), round to nearest even. */
static uint16_t float_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* ---- R18: rotary embedding of one channel ---- */

static int rot_dim(const ref_desc *d) { return d->rotary_dim > 0 ? d->rotary_dim : d->head_size; }

/* Channel c of a row (element 0 at index base of src) after the rotation at
 * position pos, as the element type's bits (f32: the float's bits). */
static uint32_t rot_bits(const ref_desc *d, const ref_inputs *in, const void *src, size_t base,
                         int c, long pos) {
  const int R = rot_dim(d), half = R / 2;
  float out;
  if (c >= R) {
    out = (float)elem(src, d->dtype, base + c);
  } else {
    int k, first, partner;
    if (d->rotary_interleaved) { k = c / 2; first = (c % 2) == 0; partner = c ^ 1; }
    else { k = c % half; first = c < half; partner = first ? c + half : c - half; }
    const float x1 = (float)elem(src, d->dtype, base + (first ? c : partner));
    const float x2 = (float)elem(src, d->dtype, base + (first ? partner : c));
    if (pos < 0) pos = 0;
    if (pos >= d->rotary_max_pos) pos = d->rotary_max_pos - 1;
    const float cs = (float)elem(in->cos_cache, d->dtype, (size_t)pos * half + k);
    const float sn = (float)elem(in->sin_cache, d->dtype, (size_t)pos * half + k);
    if (first) {
      const float t = x2 * sn;
      out = fmaf(x1, cs, -t);
    } else {
      const float t = x1 * sn;
      out = fmaf(x2, cs, t);
    }
  }
  if (d->dtype == REF_F32) { uint32_t u; memcpy(&u, &out, 4); return u; }
  return d->dtype == REF_F16 ? float_to_half(out) : float_to_bf16(out);
}

static double rot_elem(const ref_desc *d, const ref_inputs *in, const void *src, size_t base,
                       int c, long pos) {
  const uint32_t bits = rot_bits(d, in, src, base, c, pos);
  if (d->dtype == REF_F32) { float f; memcpy(&f, &bits, 4); return (double)f; }
  return d->dtype == REF_F16 ? half_to_double((uint16_t)bits) : bf16_to_double((uint16_t)bits);
}

/* ---- index helpers ---- */

static size_t q_index(const ref_desc *d, int b, int h, int i, int c) {
  if (d->q_rank == 4)
    return (((size_t)b * d->q_heads + h) * d->q_seq + i) * d->head_size + c;
  return (((size_t)b * d->q_seq + i) * d->q_heads + h) * d->head_size + c;
}

static size_t new_kv_index(const ref_desc *d, int b, int g, int j, int c, int width) {
  if (d->kv_rank == 4)
    return (((size_t)b * d->kv_heads + g) * d->kv_seq + j) * width + c;
  return (((size_t)b * d->kv_seq + j) * d->kv_heads + g) * width + c;
}

static size_t past_index(const ref_desc *d, int b, int g, int j, int c, int width) {
  return (((size_t)b * d->kv_heads + g) * d->past_seq + j) * width + c;
}

/* Per-batch sequence bookkeeping of one (b) row set. */
typedef struct {
  long past_b;   /* keys taken from the past buffer */
  long total_b;  /* keys in the concatenated sequence */
  long valid_b;  /* keys j < valid_b may be attended (exclusion) */
  long pad_b;    /* MHA: keys j >= pad_b get mask_filter_value added */
  long q_off;    /* absolute position of query 0 */
} seqinfo;

static int seq_info(const ref_desc *d, const ref_inputs *in, int b, seqinfo *s) {
  long T = (long)d->past_seq + d->kv_seq;
  if (d->op == REF_GQA) {
    /* R1: seqlens_k = total - 1; the new keys follow the valid past. */
    s->total_b = (long)in->lens[b] + 1;
    s->past_b = s->total_b - d->q_seq;
    if (s->past_b < 0 || s->past_b > d->past_seq) return -1;
    s->valid_b = s->total_b;
    s->pad_b = s->total_b;
    s->q_off = s->past_b;
  } else {
    /* MHA / Attention: literal concatenation of the whole past buffer. */
    s->total_b = T;
    s->past_b = d->past_seq;
    s->q_off = d->past_seq; /* R3: upper-left, shifted by the cache */
    s->valid_b = T;
    s->pad_b = T;
    if (in->lens) {
      long n = d->seqlens_i64 ? (long)((const int64_t *)in->lens)[b] : (long)in->lens[b];
      if (n < 0) n = 0;
      if (n > T) n = T;
      if (d->op == REF_ATTENTION) s->valid_b = n; /* -inf beyond nonpad length */
      else s->pad_b = n;                           /* R9: additive mask */
    }
  }
  return 0;
}

/* R21: new K/V element with its projection-bias segment, as the element type */
static int kv_biased(const ref_desc *d, const ref_inputs *in) {
  return d->op == REF_MHA && d->kv_rank == 3 && in->proj_bias != NULL;
}

static uint32_t biased_bits(const ref_desc *d, const ref_inputs *in, const void *cur, size_t idx,
                            int g, int c, int value) {
  const size_t seg = value ? (size_t)2 * d->q_heads * d->head_size + (size_t)g * d->v_head_size
                           : (size_t)d->q_heads * d->head_size + (size_t)g * d->head_size;
  const float x = (float)elem(cur, d->dtype, idx);
  const float bb = (float)elem(in->proj_bias, d->dtype, seg + c);
  const float r = x + bb;
  if (d->dtype == REF_F32) { uint32_t u; memcpy(&u, &r, 4); return u; }
  return d->dtype == REF_F16 ? float_to_half(r) : float_to_bf16(r);
}

static double bits_to_double(int dtype, uint32_t bits) {
  if (dtype == REF_F32) { float f; memcpy(&f, &bits, 4); return (double)f; }
  return dtype == REF_F16 ? half_to_double((uint16_t)bits) : bf16_to_double((uint16_t)bits);
}

static double key_elem(const ref_desc *d, const ref_inputs *in, const seqinfo *s,
                       int b, int g, long j, int c, int value) {
  int width = value ? d->v_head_size : d->head_size;
  const void *past = value ? in->past_v : in->past_k;
  const void *cur = value ? in->v : in->k;
  if (j < s->past_b) return elem(past, d->dtype, past_index(d, b, g, (int)j, c, width));
  const size_t base = new_kv_index(d, b, g, (int)(j - s->past_b), 0, width);
  if (d->do_rotary && !value) return rot_elem(d, in, cur, base, c, j); /* R18: new key at position j */
  if (kv_biased(d, in)) return bits_to_double(d->dtype, biased_bits(d, in, cur, base + c, g, c, value));
  return elem(cur, d->dtype, base + c);
}

/* R19: bias rows / columns and the attn_mask element of (b, h, i, j) */
static long bias_cols(const ref_desc *d) {
  long T = (long)d->past_seq + d->kv_seq;
  return d->bias_t > 0 ? d->bias_t : T;
}

static double bias_at(const ref_desc *d, const ref_inputs *in, int b, int h, int i, long j) {
  size_t bb = d->bias_b > 1 ? (size_t)b : 0, bh = d->bias_h > 1 ? (size_t)h : 0;
  size_t rows = d->bias_s == 1 ? 1 : (size_t)d->q_seq, bi = d->bias_s == 1 ? 0 : (size_t)i;
  return elem(in->bias, d->dtype, ((bb * d->bias_h + bh) * rows + bi) * (size_t)bias_cols(d) + j);
}

static int mask_at(const ref_desc *d, const ref_inputs *in, int b, int h, int i, long j) {
  long T = (long)d->past_seq + d->kv_seq;
  long cols = d->mask_t > 0 ? d->mask_t : T;
  if (j >= cols) return 0;
  size_t mb = d->mask_b > 1 ? (size_t)b : 0, mh = d->mask_h > 1 ? (size_t)h : 0;
  size_t rows = d->mask_s == 1 ? 1 : (size_t)d->q_seq, mi = d->mask_s == 1 ? 0 : (size_t)i;
  size_t e = ((mb * d->mask_h + mh) * rows + mi) * (size_t)cols + j;
  if (d->mask_kind == 1) return ((const uint8_t *)in->mask)[e] != 0;
  return ((const int32_t *)in->mask)[e] != 0;
}

static double scale_of(const ref_desc *d) {
  /* Explicit scale as its float32 value; default 1/sqrt(head_size). */
  return d->has_scale ? (double)d->scale : 1.0 / sqrt((double)d->head_size);
}

/*
 * Softmax weights of row (b, h, i): w[j] for j < total_b (0 for excluded keys)
 * and the sink's share *sink_w.  Returns the number of allowed keys, or -1 on
 * inconsistent lengths.  Writes q into qbuf (head_size doubles).
 */
static long row_weights(const ref_desc *d, const ref_inputs *in, int b, int h, int i,
                        double *w, double *sink_w, double *qbuf, seqinfo *s_out) {
  seqinfo s;
  if (seq_info(d, in, b, &s) != 0) return -1;
  if (s_out) *s_out = s;
  const int D = d->head_size;
  const int G = d->q_heads / d->kv_heads;
  const int g = h / G; /* R5 */
  for (int c = 0; c < D; ++c) {
    double x = d->do_rotary ? rot_elem(d, in, in->q, q_index(d, b, h, i, 0), c, s.q_off + i) /* R18 */
                            : elem(in->q, d->dtype, q_index(d, b, h, i, c));
    /* MHA projection bias: the query segment is added to q (R11). */
    if (d->op == REF_MHA && in->proj_bias) x += elem(in->proj_bias, d->dtype, (size_t)h * D + c);
    qbuf[c] = x;
  }
  const double scale = scale_of(d);
  const long pos = s.q_off + i;
  const long T = (long)d->past_seq + d->kv_seq;
  long n_allowed = 0;
  double m = -INFINITY;
  unsigned char *ok = (unsigned char *)malloc((size_t)s.total_b + 1);
  (void)T;
  for (long j = 0; j < s.total_b; ++j) {
    int allowed = j < s.valid_b;
    if (d->causal && j > pos) allowed = 0;
    if (d->window > 0 && j < pos - d->window + 1) allowed = 0;
    if (in->bias && j >= bias_cols(d)) allowed = 0;                     /* R19: short mask */
    if (d->mask_kind == 1 && !mask_at(d, in, b, h, i, j)) allowed = 0;  /* R19: BOOL false */
    ok[j] = (unsigned char)allowed;
    if (!allowed) { w[j] = 0.0; continue; }
    double dot = 0.0;
    for (int c = 0; c < D; ++c) dot += qbuf[c] * key_elem(d, in, &s, b, g, j, c, 0);
    double sc = dot * scale;
    if (in->bias) sc += bias_at(d, in, b, h, i, j);
    if (d->softcap > 0.0f) sc = (double)d->softcap * tanh(sc / (double)d->softcap);
    if (d->op == REF_MHA && j >= s.pad_b) sc += (double)d->mask_filter_value;
    if (d->mask_kind == 2 && !mask_at(d, in, b, h, i, j)) sc += (double)d->mask_filter_value; /* R19 */
    w[j] = sc;
    if (sc > m) m = sc;
    ++n_allowed;
  }
  *sink_w = 0.0;
  if (n_allowed == 0) { /* R10 */
    free(ok);
    return 0;
  }
  double z = 0.0;
  int has_sink = in->sink != NULL;
  if (has_sink) {
    z = elem(in->sink, d->dtype, (size_t)h); /* R7: raw logit */
    if (z > m) m = z;
  }
  double den = has_sink ? exp(z - m) : 0.0;
  for (long j = 0; j < s.total_b; ++j) {
    if (!ok[j]) continue;
    w[j] = exp(w[j] - m);
    den += w[j];
  }
  for (long j = 0; j < s.total_b; ++j) w[j] /= den;
  if (has_sink) *sink_w = exp(z - m) / den;
  free(ok);
  return n_allowed;
}

static int check_desc(const ref_desc *d, const ref_inputs *in) {
  if (!d || !in || !in->q || !in->k || !in->v) return -1;
  if (d->q_heads <= 0 || d->kv_heads <= 0 || d->q_heads % d->kv_heads) return -1;
  if (d->head_size <= 0 || d->v_head_size <= 0 || d->batch < 0 || d->q_seq < 0) return -1;
  if (d->op == REF_GQA && (!in->lens || d->kv_seq != d->q_seq)) return -1;
  if (d->past_seq > 0 && (!in->past_k || !in->past_v)) return -1;
  if (d->mask_kind && !in->mask) return -1;
  if (d->do_rotary) {
    const int R = rot_dim(d);
    if (d->op != REF_GQA || !in->cos_cache || !in->sin_cache) return -1;
    if (R <= 0 || R % 2 || R > d->head_size || d->rotary_max_pos <= 0) return -1;
  }
  return 0;
}

static int one_row(const ref_desc *d, const ref_inputs *in, int b, int h, int i,
                   double *out, double *w, double *qbuf) {
  seqinfo s;
  double sink_w;
  long n = row_weights(d, in, b, h, i, w, &sink_w, qbuf, &s);
  if (n < 0) return -1;
  const int G = d->q_heads / d->kv_heads, g = h / G;
  for (int c = 0; c < d->v_head_size; ++c) out[c] = 0.0;
  if (n == 0) return 0;
  for (long j = 0; j < s.total_b; ++j) {
    if (w[j] == 0.0) continue; /* excluded key, or a weight that underflowed */
    for (int c = 0; c < d->v_head_size; ++c)
      out[c] += w[j] * key_elem(d, in, &s, b, g, j, c, 1);
  }
  return 0;
}

static long max_keys(const ref_desc *d) { return (long)d->past_seq + d->kv_seq + 1; }

/* Y for every row, float64, logical order (B, S, Hq, Dv). */
int olk_ref_attention(const ref_desc *d, const ref_inputs *in, double *y, int threads) {
  if (check_desc(d, in) != 0 || !y) return -1;
  const long rows = (long)d->batch * d->q_seq * d->q_heads;
  int err = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#endif
#pragma omp parallel reduction(|| : err)
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)max_keys(d));
    double *qbuf = (double *)malloc(sizeof(double) * (size_t)d->head_size);
#pragma omp for schedule(dynamic, 4)
    for (long r = 0; r < rows; ++r) {
      int h = (int)(r % d->q_heads);
      int i = (int)((r / d->q_heads) % d->q_seq);
      int b = (int)(r / ((long)d->q_heads * d->q_seq));
      if (one_row(d, in, b, h, i, y + (size_t)r * d->v_head_size, w, qbuf)) err = 1;
    }
    free(w);
    free(qbuf);
  }
  return err ? -1 : 0;
}

/* Y for selected rows: rows[3*r .. 3*r+2] = (b, h, i); out is (nrows, Dv). */
int olk_ref_attention_rows(const ref_desc *d, const ref_inputs *in, const int32_t *rows,
                           long nrows, double *out, int threads) {
  if (check_desc(d, in) != 0 || !rows || !out) return -1;
  int err = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#endif
#pragma omp parallel reduction(|| : err)
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)max_keys(d));
    double *qbuf = (double *)malloc(sizeof(double) * (size_t)d->head_size);
#pragma omp for schedule(dynamic, 1)
    for (long r = 0; r < nrows; ++r) {
      int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      if (b < 0 || b >= d->batch || h < 0 || h >= d->q_heads || i < 0 || i >= d->q_seq) { err = 1; continue; }
      if (one_row(d, in, b, h, i, out + (size_t)r * d->v_head_size, w, qbuf)) err = 1;
    }
    free(w);
    free(qbuf);
  }
  return err ? -1 : 0;
}

/* Softmax weights of one row: w has room for P+L+1 doubles.  Returns the
 * number of keys of the row's concatenated sequence (total_b), or -1. */
long olk_ref_row_weights(const ref_desc *d, const ref_inputs *in, int b, int h, int i,
                         double *w, double *sink_w) {
  if (check_desc(d, in) != 0) return -1;
  double *qbuf = (double *)malloc(sizeof(double) * (size_t)d->head_size);
  seqinfo s;
  long n = row_weights(d, in, b, h, i, w, sink_w, qbuf, &s);
  free(qbuf);
  return n < 0 ? -1 : s.total_b;
}

/* present_key / present_value (B, Hkv, P+L, D|Dv): position j < total_b holds
 * the past prefix followed by the current step, copied bit for bit; positions
 * at or beyond total_b are left as they are. */
int olk_ref_present(const ref_desc *d, const ref_inputs *in, void *pk, void *pv) {
  if (check_desc(d, in) != 0) return -1;
  const size_t es = esize(d->dtype);
  const long Tp = (long)d->past_seq + d->kv_seq;
  for (int b = 0; b < d->batch; ++b) {
    seqinfo s;
    if (seq_info(d, in, b, &s) != 0) return -1;
    for (int g = 0; g < d->kv_heads; ++g) {
      for (int which = 0; which < 2; ++which) {
        void *dst = which ? pv : pk;
        if (!dst) continue;
        int width = which ? d->v_head_size : d->head_size;
        const void *past = which ? in->past_v : in->past_k;
        const void *cur = which ? in->v : in->k;
        for (long j = 0; j < s.total_b && j < Tp; ++j) {
          const char *src;
          char *o = (char *)dst + ((((size_t)b * d->kv_heads + g) * Tp + j) * width) * es;
          if (j >= s.past_b && kv_biased(d, in)) { /* R21: biased new K/V */
            const size_t base = new_kv_index(d, b, g, (int)(j - s.past_b), 0, width);
            for (int c = 0; c < width; ++c) {
              const uint32_t bits = biased_bits(d, in, cur, base + c, g, c, which);
              if (es == 4) memcpy(o + 4 * (size_t)c, &bits, 4);
              else { const uint16_t h16 = (uint16_t)bits; memcpy(o + 2 * (size_t)c, &h16, 2); }
            }
            continue;
          }
          if (j >= s.past_b && d->do_rotary && !which) { /* R18: rotated new key */
            const size_t base = new_kv_index(d, b, g, (int)(j - s.past_b), 0, width);
            for (int c = 0; c < width; ++c) {
              const uint32_t bits = rot_bits(d, in, cur, base, c, j);
              if (es == 4) memcpy(o + 4 * (size_t)c, &bits, 4);
              else { const uint16_t h16 = (uint16_t)bits; memcpy(o + 2 * (size_t)c, &h16, 2); }
            }
            continue;
          }
          if (j < s.past_b) src = (const char *)past + past_index(d, b, g, (int)j, 0, width) * es;
          else src = (const char *)cur + new_kv_index(d, b, g, (int)(j - s.past_b), 0, width) * es;
          memcpy(o, src, (size_t)width * es);
        }
      }
    }
  }
  return 0;
}

/* R20: qk_matmul_output of every row, float64 (B, Hq, S, T). */
int olk_ref_qk(const ref_desc *d, const ref_inputs *in, int mode, double *out, int threads) {
  if (check_desc(d, in) != 0 || !out || mode < 0 || mode > 3) return -1;
  const long T = (long)d->past_seq + d->kv_seq;
  const long rows = (long)d->batch * d->q_heads * d->q_seq;
  int err = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#endif
#pragma omp parallel reduction(|| : err)
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)max_keys(d));
    double *qbuf = (double *)malloc(sizeof(double) * (size_t)d->head_size);
#pragma omp for schedule(dynamic, 4)
    for (long r = 0; r < rows; ++r) {
      int i = (int)(r % d->q_seq);
      int h = (int)((r / d->q_seq) % d->q_heads);
      int b = (int)(r / ((long)d->q_heads * d->q_seq));
      double *o = out + (size_t)r * T;
      double sink_w;
      seqinfo s;
      long n = row_weights(d, in, b, h, i, w, &sink_w, qbuf, &s); /* fills qbuf, weights */
      if (n < 0) { err = 1; continue; }
      const int g = h / (d->q_heads / d->kv_heads);
      const long pos = s.q_off + i;
      for (long j = 0; j < T; ++j) {
        if (mode == 3) { o[j] = j < s.total_b ? w[j] : 0.0; continue; }
        double dot = 0.0;
        if (j < s.total_b)
          for (int c = 0; c < d->head_size; ++c) dot += qbuf[c] * key_elem(d, in, &s, b, g, j, c, 0);
        double sc = dot * scale_of(d);
        if (mode == 0) { o[j] = sc; continue; }
        int allowed = j < s.valid_b && j < s.total_b;
        if (d->causal && j > pos) allowed = 0;
        if (d->window > 0 && j < pos - d->window + 1) allowed = 0;
        if (in->bias && j >= bias_cols(d)) allowed = 0;
        if (d->mask_kind == 1 && !mask_at(d, in, b, h, i, j)) allowed = 0;
        if (!allowed) { o[j] = -INFINITY; continue; }
        if (in->bias) sc += bias_at(d, in, b, h, i, j);
        if (mode == 2 && d->softcap > 0.0f) sc = (double)d->softcap * tanh(sc / (double)d->softcap);
        o[j] = sc;
      }
    }
    free(w);
    free(qbuf);
  }
  return err ? -1 : 0;
}

/*
 * R22: backward of the GroupQueryAttention forward without past (onnx-light-cpu
 * C++ API "Custom operators", RegisterCustomOperatorGradients, GroupQueryAttention
 * gradient: probabilities P recomputed by the forward, softmax backward, the
 * score gradient scaled by the forward scale, dQ = dS K, dK = dS^T Q and
 * dV = P^T dY summed over the query heads that share a KV head).  In float64:
 *   dP_ij = dY_i . V_j,  Di = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - Di) * scale,
 *   dQ_i = sum_j dS_ij K_j,  dK_j = sum_(h in group) sum_i dS_ij Q_i,
 *   dV_j = sum_(h in group) sum_i P_ij dY_i.
 * dy is (B, S, Hq*Dv) of the element type; dq (B,S,Hq,D), dk (B,S,Hkv,D) and
 * dv (B,S,Hkv,Dv) are float64 outputs (rounding to the element type is the
 * caller's comparison).
 */
int olk_ref_attention_bwd(const ref_desc *d, const ref_inputs *in, const void *dy, double *dq,
                          double *dk, double *dv) {
  if (check_desc(d, in) != 0 || !dy || !dq || !dk || !dv) return -1;
  if (d->op != REF_GQA || d->past_seq != 0 || in->bias || in->sink || d->softcap > 0.0f ||
      d->do_rotary || d->q_rank != 3 || d->kv_rank != 3)
    return -1;
  const int B = d->batch, S = d->q_seq, Hq = d->q_heads, Hkv = d->kv_heads;
  const int D = d->head_size, Dv = d->v_head_size, G = Hq / Hkv;
  const double scale = scale_of(d);
  memset(dq, 0, sizeof(double) * (size_t)B * S * Hq * D);
  memset(dk, 0, sizeof(double) * (size_t)B * S * Hkv * D);
  memset(dv, 0, sizeof(double) * (size_t)B * S * Hkv * Dv);
  double *w = (double *)malloc(sizeof(double) * (size_t)max_keys(d));
  double *qbuf = (double *)malloc(sizeof(double) * (size_t)D);
  double *dp = (double *)malloc(sizeof(double) * (size_t)max_keys(d));
  int err = 0;
  for (int b = 0; b < B && !err; ++b)
    for (int h = 0; h < Hq && !err; ++h) {
      const int g = h / G;
      for (int i = 0; i < S; ++i) {
        double sink_w;
        seqinfo s;
        long n = row_weights(d, in, b, h, i, w, &sink_w, qbuf, &s);
        if (n < 0) { err = 1; break; }
        double Di = 0.0;
        for (long j = 0; j < s.total_b; ++j) {
          dp[j] = 0.0;
          if (w[j] == 0.0) continue;
          for (int c = 0; c < Dv; ++c)
            dp[j] += elem(dy, d->dtype, (((size_t)b * S + i) * Hq + h) * Dv + c) *
                     key_elem(d, in, &s, b, g, j, c, 1);
          Di += w[j] * dp[j];
        }
        for (long j = 0; j < s.total_b; ++j) {
          if (w[j] == 0.0) continue;
          const double ds = w[j] * (dp[j] - Di) * scale;
          double *dqi = dq + (((size_t)b * S + i) * Hq + h) * D;
          double *dkj = dk + (((size_t)b * S + j) * Hkv + g) * D;
          double *dvj = dv + (((size_t)b * S + j) * Hkv + g) * Dv;
          for (int c = 0; c < D; ++c) {
            dqi[c] += ds * key_elem(d, in, &s, b, g, j, c, 0);
            dkj[c] += ds * qbuf[c];
          }
          for (int c = 0; c < Dv; ++c)
            dvj[c] += w[j] * elem(dy, d->dtype, (((size_t)b * S + i) * Hq + h) * Dv + c);
        }
      }
    }
  free(w);
  free(qbuf);
  free(dp);
  return err ? -1 : 0;
}
