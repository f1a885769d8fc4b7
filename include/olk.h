/*
 * olk.h — C ABI of the MI355X (gfx950) attention-forward library libolk.so.
 *
 * One computation, three operator contracts:
 *
 *   Y = Softmax((Q @ K^T) * scale + bias) @ V
 *
 * - com.microsoft::GroupQueryAttention (onnx-light-cpu Python API page
 *   "Custom operators", section "Microsoft GroupQueryAttention"): grouped KV
 *   heads, causal and local_window_size masking, head_sink virtual logits,
 *   seqlens_k, present = past cache followed by the current step;
 * - com.microsoft::MultiHeadAttention (same page, section "Microsoft
 *   MultiHeadAttention"): rank-3 or rank-4 (cross-attention) K/V, projection
 *   bias, int32 key-padding lengths with mask_filter_value, additive bias;
 * - ai.onnx::Attention (onnx-light reference kernels header page,
 *   "class Attention", its Attributes and Result structs): scale, is_causal,
 *   softcap, grouped heads, past/present concatenation, non-padding lengths.
 *
 * Conventions shared by every entry point
 * - Ownership: the caller owns every buffer (inputs, outputs, workspace).  The
 *   library allocates no device memory and keeps no pointer after a call
 *   returns.  NULL means "absent" for optional tensors (as the comprehensive
 *   Attention overload takes nullptr for absent inputs).
 * - Memory: every tensor pointer is a device pointer on the current HIP
 *   device, row-major and densely packed in the layout stated at its field.
 *   Element type of every floating tensor is desc->dtype; lengths are int32.
 * - Asynchrony: launches go to `stream` (a hipStream_t; NULL = the null
 *   stream).  Outputs are valid after the stream has synchronised.  Lengths
 *   stay on the device: no call synchronises with the host.
 * - Errors: every check happens on the host before any launch and returns a
 *   status; nothing is launched when a check fails.  Unsupported
 *   representations are rejected, not reinterpreted.  Device lengths that are
 *   out of range are clamped (memory-safe; values then unspecified).  There is
 *   no CPU fallback.
 * - Aliasing: outputs must not overlap inputs, except in kv_inplace mode (see
 *   olk_attn_desc.kv_inplace).
 * - Thread safety: reentrant; the only global state is the per-thread name of
 *   the last kernel launched.
 */
#ifndef OLK_H
#define OLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OLK_OK = 0,
  OLK_E_NULL = 1,        /* a required pointer is NULL */
  OLK_E_ATTR = 2,        /* an attribute value the operator contract rejects */
  OLK_E_SHAPE = 3,       /* inconsistent sizes or ranks */
  OLK_E_UNSUPPORTED = 4, /* valid for the operator, not implemented here */
  OLK_E_WORKSPACE = 5,   /* workspace missing or smaller than olk_workspace_bytes */
  OLK_E_HIP = 6          /* a HIP launch failed */
} olk_status;

typedef enum { OLK_F32 = 0, OLK_F16 = 1, OLK_BF16 = 2 } olk_dtype;

typedef enum { OLK_OP_GQA = 0, OLK_OP_MHA = 1, OLK_OP_ATTENTION = 2 } olk_op;

/* Kernel family requested by the caller (diagnostics and tests). */
typedef enum {
  OLK_KERNEL_AUTO = 0,    /* the library picks */
  OLK_KERNEL_GENERIC = 1, /* one-wave-per-row VALU kernel: any dtype, any head size <= 256 */
  OLK_KERNEL_TILED = 2    /* MFMA tiled kernel (f16/bf16, head size 64 or 128) */
} olk_kernel;

typedef enum {
  OLK_MASK_NONE = 0,
  OLK_MASK_BOOL = 1,         /* uint8, nonzero = attend (ai.onnx Attention) */
  OLK_MASK_BINARY_I32 = 2    /* int32, nonzero = attend, zero = key padding: the score gets
                                mask_filter_value added (MultiHeadAttention; excludes the
                                key-padding lengths in seqlens) */
} olk_mask_kind;

/*
 * Attributes and sizes of one call.
 *  B = batch, S = q_seq, L = kv_seq (new keys), P = past_seq (past buffer
 *  length), T = P + L (present length), Hq/Hkv = heads, D/Dv = head sizes.
 */
typedef struct {
  int32_t op;                /* olk_op */
  int32_t dtype;             /* olk_dtype: Q, K, V, past, bias, sink, proj_bias, Y, present */
  int32_t batch;             /* B >= 0 */
  int32_t q_seq;             /* S >= 0 */
  int32_t kv_seq;            /* L >= 0; GroupQueryAttention requires L == S */
  int32_t past_seq;          /* P >= 0; 0 = no past inputs */
  int32_t q_num_heads;       /* Hq > 0 */
  int32_t kv_num_heads;      /* Hkv > 0, Hq % Hkv == 0; MultiHeadAttention: Hkv == Hq */
  int32_t head_size;         /* D */
  int32_t v_head_size;       /* Dv */
  int32_t q_rank;            /* 3: Q (B,S,Hq*D), Y (B,S,Hq*Dv); 4 (Attention only): Q (B,Hq,S,D), Y (B,Hq,S,Dv) */
  int32_t kv_rank;           /* 3: K (B,L,Hkv*D), V (B,L,Hkv*Dv); 4 (MHA/Attention): K (B,Hkv,L,D), V (B,Hkv,L,Dv) */
  int32_t causal;            /* 0/1: GQA causal, MHA unidirectional, Attention is_causal.
                                Query i sits at position past_b + i, past_b = the cached
                                keys in front of the new ones (GQA: seqlens_k + 1 - S;
                                MHA / Attention: P): every cached key is visible and new
                                key j iff j <= i, i.e. the mask is aligned to the
                                upper-left corner of the new keys and shifted by the
                                cache (reference kernels header page, "class Attention",
                                is_causal) */
  int32_t local_window_size; /* GroupQueryAttention only: -1 = full; W > 0 attends the
                                current key and up to W-1 preceding; needs causal = 1 */
  int32_t has_scale;         /* 0: scale = 1/sqrt(D) */
  float scale;               /* used when has_scale != 0; must be finite */
  float softcap;             /* > 0: s -> softcap*tanh(s/softcap) after the bias (GQA, Attention) */
  float mask_filter_value;   /* MultiHeadAttention: added to scores of padded keys (default -10000) */
  int32_t bias_b, bias_h;    /* attn_bias broadcast extents: 1 or B, 1 or Hq */
  int32_t kv_inplace;        /* GroupQueryAttention only.  0: present = concat(past, new)
                                written out of place.  1: present_k/v already hold the
                                valid past at [0, past_b) (past_k/v NULL or equal to
                                present_k/v); only the new positions are written. */
  int32_t kernel;            /* olk_kernel */
  /* Rotary position embedding fused into GroupQueryAttention (the operator's
   * do_rotary / rotary_interleaved attributes; the rotation itself is the
   * RotaryEmbedding kernel of the onnx-light reference kernels header page,
   * "class RotaryEmbedding", after arXiv 2104.09864).  Q and the new K rows are
   * rotated at their absolute positions (query i and new key i of batch b at
   * past_b + i); the past is used as stored; V is not rotated.  present_key
   * receives the rotated keys.  Each rotated pair (x1, x2) with cosine c and
   * sine s becomes (x1*c - x2*s, x2*c + x1*s), computed in float32 as
   * fma(x1, c, -(x2*s)) and fma(x2, c, x1*s) and rounded once to the element
   * type.  Requires op = GQA, D == Dv and present_k/present_v (the rotated
   * keys are written there and read back).  Positions at or beyond
   * rotary_max_pos use the last cache row (memory-safe; values unspecified). */
  int32_t do_rotary;         /* 0/1 */
  int32_t rotary_interleaved;/* 1: pairs (2k, 2k+1); 0: pairs (k, k + R/2) */
  int32_t rotary_dim;        /* R: channels rotated, even, 0 < R <= D; 0 = D.  Channels >= R
                                are copied unchanged. */
  int32_t rotary_max_pos;    /* rows of cos_cache / sin_cache (> 0 when do_rotary) */
  /* Further attn_bias extents (the ai.onnx Attention FLOAT attn_mask is an
   * attn_bias: onnx-light reference kernels header page, "class Attention",
   * rank 2-4 masks broadcast to (B, Hq, S, T) and added; a mask whose last
   * dimension is shorter than T is padded with -inf). */
  int32_t bias_s;            /* 0 or S: one bias row per query; 1: broadcast over queries */
  int32_t bias_t;            /* 0 or T: full rows; 0 < bias_t < T (Attention only): keys
                                j >= bias_t are excluded (-inf padding) */
  /* attn_mask (the same page: BOOL rank 2-4, true = attend, false = -inf,
   * short masks padded with false; onnx-light-cpu Python API "Custom
   * operators", MultiHeadAttention: binary key-padding masks (B,T) / (B,S,T)).
   * Broadcast extents as for attn_bias; element (b, h, i, j) at
   * ((b'*mask_h + h')*mask_s' + i')*mask_t + j with b', h', i' = 0 on broadcast
   * dimensions. */
  int32_t mask_kind;         /* olk_mask_kind */
  int32_t mask_b, mask_h;    /* 1 or B, 1 or Hq */
  int32_t mask_s;            /* 0 or S: per query row; 1: broadcast */
  int32_t mask_t;            /* 0 or T: full; BOOL may be shorter (keys beyond are false) */
  int32_t seqlens_i64;       /* ai.onnx Attention: 1 = seqlens points at int64
                                nonpad_kv_seqlen values */
  int32_t qk_mode;           /* ai.onnx Attention qk_matmul_output_mode when qk_out != NULL:
                                0 (Q.K^T)*scale for every (i, j); 1 + attn_bias, excluded
                                keys (causal, masks, nonpad, short padding) -inf; 2 after
                                softcap (excluded -inf); 3 softmax weights (excluded 0) */
} olk_attn_desc;

/* Device pointers (caller-owned); NULL = absent. */
typedef struct {
  const void *q;             /* required; see q_rank */
  const void *k, *v;         /* required; see kv_rank */
  const void *past_k;        /* (B,Hkv,P,D) or NULL */
  const void *past_v;        /* (B,Hkv,P,Dv) or NULL */
  const int32_t *seqlens;    /* (B) int32.  GQA: seqlens_k = total length - 1 (required);
                                MHA: key-padding lengths; Attention: non-padding lengths */
  const void *attn_bias;     /* (bias_b, bias_h, S or 1, T or bias_t) additive, or NULL */
  const void *head_sink;     /* (Hq) GroupQueryAttention virtual logits, or NULL */
  const void *proj_bias;     /* MultiHeadAttention (2*Hq*D + Hq*Dv) = [q | k | v], or NULL;
                                with rank-4 K/V only the q segment applies */
  void *y;                   /* required output; see q_rank */
  void *present_k;           /* (B,Hkv,T,D) output, or NULL = not requested */
  void *present_v;           /* (B,Hkv,T,Dv) output, or NULL = not requested */
  const void *cos_cache;     /* do_rotary: (rotary_max_pos, R/2) element type, row = position */
  const void *sin_cache;     /* do_rotary: (rotary_max_pos, R/2) element type */
  const void *attn_mask;     /* see mask_kind, or NULL */
  float *qk_out;             /* ai.onnx Attention: (B, Hq, S, T) float32 output, or NULL */
} olk_attn_io;

/*
 * Host-only check of desc and io (no GPU is touched).  Returns the status the
 * compute entry points would return before launching.  The rejections follow
 * the operator contracts: local_window_size 0, below -1, or with causal = 0
 * (onnx-light-cpu Python API page "Custom operators", section "Microsoft
 * GroupQueryAttention"); MultiHeadAttention takes one head count, rank-3 or
 * rank-4 K/V and no head_sink, and has no slot for the inputs that section
 * ("Microsoft MultiHeadAttention") lists as explicitly unsupported (packed
 * rank-5 inputs, shared-buffer inputs, the qk output); q_num_heads must be a
 * multiple of kv_num_heads (reference kernels header page, "class
 * Attention").  OLK_E_NULL for a missing required pointer, OLK_E_ATTR for a
 * rejected attribute, OLK_E_SHAPE for inconsistent sizes or overlapping
 * buffers, OLK_E_UNSUPPORTED for valid shapes this library does not take.
 */
olk_status olk_validate(const olk_attn_desc *desc, const olk_attn_io *io);

/*
 * Bytes of workspace olk_attention_decode needs for this desc (0 when the
 * call needs none): one float record (m, l, O[Dv]) per query row and key chunk
 * of its split-KV decomposition.  The decomposition is ours (the pages
 * describe CPU kernels); the size depends only on sizes, never on device data.
 * Returns 0 for a NULL desc.
 */
size_t olk_workspace_bytes(const olk_attn_desc *desc);

/*
 * Attention forward, one pass over every query row (prefill and general
 * shapes).  Computes Y and, when requested, present_key/present_value
 * (onnx-light reference kernels header page, "class Attention", comprehensive
 * overload and Result; GroupQueryAttention and MultiHeadAttention sections of
 * the onnx-light-cpu Python API page).  Takes no workspace: each kernel it
 * launches keeps a row's softmax state in registers over all of the row's
 * keys and writes only Y, present and the qk output, so nothing is left to
 * merge in memory.  `stream` is a hipStream_t.  Errors: as olk_validate, and
 * OLK_E_UNSUPPORTED when OLK_KERNEL_TILED is forced on a shape the matrix-core
 * kernels do not take; OLK_E_HIP reports a failed launch.
 */
olk_status olk_attention_fwd(const olk_attn_desc *desc, const olk_attn_io *io, void *stream);

/*
 * Same result as olk_attention_fwd, computed split-KV for short query
 * sequences against long key sequences (decode against a KV cache: present =
 * the entire past cache followed by the current step, and a head_sink logit
 * adds to the denominator only; onnx-light-cpu Python API page "Custom
 * operators", section "Microsoft GroupQueryAttention").  The keys of each
 * (batch, KV head) are cut into chunks whose partial softmax states are merged
 * by a second kernel, which also adds the sink (the decomposition is ours).  workspace: device memory of at least
 * olk_workspace_bytes(desc) bytes, 16-byte aligned, owned by the caller; its
 * contents on entry do not matter.  `stream` is a hipStream_t.  Errors: as
 * olk_validate; OLK_E_WORKSPACE for a missing, short or misaligned
 * workspace; OLK_E_UNSUPPORTED when batch * q_seq exceeds 65535, the keys
 * need more than 4096 chunks of 512, or OLK_KERNEL_TILED is forced on a
 * shape the tiled kernels do not take.  These are checked before anything is
 * launched; OLK_E_HIP reports a failed launch.
 */
olk_status olk_attention_decode(const olk_attn_desc *desc, const olk_attn_io *io,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the built-in scratch of olk_attention_decode_noalloc (32 MiB). */
#define OLK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * olk_attention_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the split partials go to a scratch array built into the
 * library, one per device, held until the process ends, instead of a caller
 * workspace.  The call allocates nothing (no hipMalloc, no library allocator);
 * the first call on a device looks up that device's scratch address.
 * Arguments, result and errors as olk_attention_decode; OLK_E_WORKSPACE when
 * olk_workspace_bytes(desc) exceeds OLK_NOALLOC_SCRATCH_BYTES (nothing is
 * launched).  The scratch keeps the last call's partials and every call on a
 * device shares it: calls that overlap on one device (on different streams,
 * or from different threads without ordering) race and give wrong results.
 */
olk_status olk_attention_decode_noalloc(const olk_attn_desc *desc, const olk_attn_io *io,
                                        void *stream);

/*
 * Backward of the GroupQueryAttention forward (onnx-light-cpu C++ API page
 * "Custom operators", RegisterCustomOperatorGradients, GroupQueryAttention
 * gradient): the probabilities P are recomputed from Q, K, V; with
 * dP = dY V^T, delta_i = sum_j P_ij dP_ij and dS = P * (dP - delta) * scale,
 *   dQ = dS K,  dK = dS^T Q,  dV = P^T dY,
 * the gradients of the query heads that share a KV head summed into that KV
 * head, each output rounded once to the element type.  Scope: op GQA without
 * past (past_seq 0; query i at position i), causal 0/1, local_window_size,
 * scale; rank-3 tensors.  Attention bias, softcap, head_sink, rotary, masks
 * and the qk output are OLK_E_UNSUPPORTED.  seqlens is required as for the
 * forward (with no past every batch attends over its S keys).
 */
typedef struct {
  const void *q;             /* (B,S,Hq*D) */
  const void *k, *v;         /* (B,S,Hkv*D), (B,S,Hkv*Dv) */
  const int32_t *seqlens;    /* (B) seqlens_k */
  const void *dy;            /* (B,S,Hq*Dv) gradient of Y */
  void *dq;                  /* (B,S,Hq*D) output */
  void *dk, *dv;             /* (B,S,Hkv*D), (B,S,Hkv*Dv) outputs */
} olk_attn_bwd_io;

/* Bytes of workspace olk_attention_bwd needs: two floats per (b, h, i) row. */
size_t olk_bwd_workspace_bytes(const olk_attn_desc *desc);

/* Validates, then launches the backward on `stream`.  Workspace: at least
 * olk_bwd_workspace_bytes(desc) bytes, 16-byte aligned (OLK_E_WORKSPACE).
 * Outputs must not overlap inputs or each other (OLK_E_SHAPE). */
olk_status olk_attention_bwd(const olk_attn_desc *desc, const olk_attn_bwd_io *io,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Static string naming a status (ours); never NULL, "unknown status" for a
 * value outside olk_status. */
const char *olk_status_str(olk_status status);

/* Name of the kernels the last call on this thread launched ("" if none), a
 * static string owned by the library.  It tells which implementation ran, as
 * each onnx-light-cpu kernel carries a unique name it can record when it runs
 * (onnx-light-cpu design page "Registering kernels", section "Checking which
 * kernels are used"); here the record is one per thread, always on. */
const char *olk_last_kernel_name(void);

#ifdef __cplusplus
}
#endif

#endif /* OLK_H */
