// Rotary pre-pass of GroupQueryAttention with do_rotary (onnx-light-cpu
// Python API page "Custom operators", GroupQueryAttention: RoPE at absolute
// positions; the rotation is the RotaryEmbedding kernel of the onnx-light
// reference kernels header page, "class RotaryEmbedding": rank-2 cos/sin
// caches indexed by position, rotary_embedding_dim, interleaved pairing, after
// arXiv 2104.09864).
//
// For every (batch b, new row i) at position past_b + i:
//   * the Hq query heads are rotated into Y (same (B, S, Hq*D) layout as Q);
//     the attention kernels then read Q from Y, and each workgroup reads all
//     of its Q rows before it writes any Y row, or (split paths) Y is written
//     by a later kernel.  With rot_q the prefill kernel rotates Q itself as
//     it loads it, with the same arithmetic, and this pass skips Q;
//   * the Hkv new key heads are rotated into present_k[b, g, past_b + i];
//   * the new value heads are copied (bits) into present_v[b, g, past_b + i],
//     unless rot_skip_v: then the prefill kernel reads them from V and
//     writes those present rows itself.
// The attention kernels then take every key from present.
//
// A pair (x1, x2) with cosine c and sine s becomes (x1*c - x2*s, x2*c + x1*s),
// computed in float32 as fma(x1, c, -(x2*s)) and fma(x2, c, x1*s) with no
// other rounding, then rounded once to the element type (RNE).  Channels at or
// beyond the rotary dimension are copied.  A position beyond the cache uses
// its last row.
#include "olk_internal.h"

namespace olk {
namespace {

constexpr int kThreads = 256;

// Output channel c of a row (src, element type T) rotated at cache row `pos`.
template <typename T>
__device__ __forceinline__ T rotate_channel(const Params &p, const T *src, int c, int pos) {
  const int R = p.rot_dim, half = R / 2;
  if (c >= R) return src[c];
  int k, partner;
  bool first;
  if (p.rot_inter) {
    k = c >> 1;
    first = (c & 1) == 0;
    partner = c ^ 1;
  } else {
    first = c < half;
    k = first ? c : c - half;
    partner = first ? c + half : c - half;
  }
  const float x1 = (float)src[first ? c : partner];
  const float x2 = (float)src[first ? partner : c];
  const float cs = (float)((const T *)p.cos_cache)[(int64_t)pos * half + k];
  const float sn = (float)((const T *)p.sin_cache)[(int64_t)pos * half + k];
  const float r = first ? __builtin_fmaf(x1, cs, -__fmul_rn(x2, sn))
                        : __builtin_fmaf(x2, cs, __fmul_rn(x1, sn));
  return (T)r;
}

// 8 consecutive channels of one row
template <typename T> struct Chunk8 { T e[8]; };

template <typename T>
__device__ __forceinline__ Chunk8<T> ld8(const T *src) {
  Chunk8<T> c;
  if constexpr (sizeof(T) == 2) {
    *(uint4 *)c.e = *(const uint4 *)src;
  } else {
    *(uint4 *)c.e = *(const uint4 *)src;
    *(uint4 *)(c.e + 4) = *(const uint4 *)(src + 4);
  }
  return c;
}

template <typename T>
__device__ __forceinline__ void st8(T *dst, const Chunk8<T> &c) {
  if constexpr (sizeof(T) == 2) {
    *(uint4 *)dst = *(const uint4 *)c.e;
  } else {
    *(uint4 *)dst = *(const uint4 *)c.e;
    *(uint4 *)(dst + 4) = *(const uint4 *)(c.e + 4);
  }
}

__device__ __forceinline__ float rot_first(float x1, float x2, float c, float s) {
  return __builtin_fmaf(x1, c, -__fmul_rn(x2, s));
}
__device__ __forceinline__ float rot_second(float x1, float x2, float c, float s) {
  return __builtin_fmaf(x2, c, __fmul_rn(x1, s));
}

// Rotates (or copies) the head row `src` into `dst` with 16-byte accesses:
// task t of the row is one 8-channel chunk, or with split halves the chunk
// pair (8t, 8t + R/2); R/2 is a multiple of 8 (R a multiple of 16).
template <typename T>
__device__ __forceinline__ int vec_tasks(const Params &p) {
  const int R = p.rot_dim;
  return p.rot_inter ? p.D / 8 : (R / 2) / 8 + (p.D - R) / 8;
}

template <typename T>
__device__ __forceinline__ void rotate_task(const Params &p, const T *src, T *dst, int t,
                                            int pos) {
  const int R = p.rot_dim, half = R / 2;
  const T *cs = (const T *)p.cos_cache + (int64_t)pos * half;
  const T *sn = (const T *)p.sin_cache + (int64_t)pos * half;
  if (p.rot_inter) {
    const int c0 = 8 * t;
    Chunk8<T> x = ld8(src + c0);
    if (c0 < R) {  // 4 pairs (2k, 2k+1), k = c0/2 .. c0/2 + 3
      Chunk8<T> o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = (float)x.e[2 * e], x2 = (float)x.e[2 * e + 1];
        const float c = (float)cs[c0 / 2 + e], s = (float)sn[c0 / 2 + e];
        o.e[2 * e] = (T)rot_first(x1, x2, c, s);
        o.e[2 * e + 1] = (T)rot_second(x1, x2, c, s);
      }
      x = o;
    }
    st8(dst + c0, x);
    return;
  }
  const int npair = half / 8;
  if (t < npair) {  // channels 8t.. and their partners 8t + R/2..
    const int c0 = 8 * t;
    const Chunk8<T> a = ld8(src + c0), bb = ld8(src + c0 + half);
    const Chunk8<T> c8 = ld8(cs + c0), s8 = ld8(sn + c0);
    Chunk8<T> oa, ob;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x1 = (float)a.e[e], x2 = (float)bb.e[e];
      const float c = (float)c8.e[e], s = (float)s8.e[e];
      oa.e[e] = (T)rot_first(x1, x2, c, s);
      ob.e[e] = (T)rot_second(x1, x2, c, s);
    }
    st8(dst + c0, oa);
    st8(dst + c0 + half, ob);
  } else {  // channels beyond R: copy
    const int c0 = R + 8 * (t - npair);
    st8(dst + c0, ld8(src + c0));
  }
}

// Vector form (R a multiple of 16, D a multiple of 8, 16-byte aligned rows),
// float32 elements (16-bit types take the multi-row form below):
// one workgroup per (b, i) row; threads sweep the query-head tasks, the
// key-head tasks and the 8-channel value chunks.
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_vec_kernel(Params p) {
  const int i = blockIdx.x, b = blockIdx.y;
  const Seq s = seq_info(p, b);
  const int j = s.past + i;
  if (j >= p.T) return;
  const int pos = j < p.rot_max ? j : p.rot_max - 1;
  const int nt = vec_tasks<T>(p), vt = p.Dv / 8;
  const int nq = p.rot_q ? 0 : p.Hq * nt, nk = p.Hkv * nt, nv = p.rot_skip_v ? 0 : p.Hkv * vt;
  const T *qrow = (const T *)p.q + b * p.q_sb + (int64_t)i * p.q_ss;
  T *yrow = (T *)p.y + b * p.y_sb + (int64_t)i * p.y_ss;
  for (int t = threadIdx.x; t < nq + nk + nv; t += kThreads) {
    if (t < nq) {
      const int h = t / nt;
      rotate_task(p, qrow + (int64_t)h * p.q_sh, yrow + (int64_t)h * p.y_sh, t % nt, pos);
    } else if (t < nq + nk) {
      const int u = t - nq, g = u / nt;
      const T *krow = (const T *)p.k + b * p.k_sb + (int64_t)i * p.k_ss + (int64_t)g * p.k_sh;
      T *dst = (T *)p.present_k + (((int64_t)b * p.Hkv + g) * p.T + j) * p.D;
      rotate_task(p, krow, dst, u % nt, pos);
    } else {
      const int u = t - nq - nk, g = u / vt, c0 = 8 * (u % vt);
      const T *vrow = (const T *)p.v + b * p.v_sb + (int64_t)i * p.v_ss + (int64_t)g * p.v_sh;
      T *dst = (T *)p.present_v + (((int64_t)b * p.Hkv + g) * p.T + j) * p.Dv;
      st8(dst + c0, ld8(vrow + c0));
    }
  }
}

// Vector form for 16-bit types, several rows per workgroup: a thread takes up
// to TPT tasks (16-byte chunks of any row, head and kind) and issues all their
// loads before it computes and stores any, so each thread keeps several loads
// in flight and the grid is RPW times smaller than one workgroup per row.
constexpr int kRowsPerWg = 8;
template <typename T, int TPT>
__global__ __launch_bounds__(kThreads) void rope_vec2_kernel(Params p) {
  static_assert(sizeof(T) == 2, "16-bit element types");
  const int b = blockIdx.y;
  const Seq s = seq_info(p, b);
  const int nt = vec_tasks<T>(p), vt = p.Dv / 8;
  const int nq = p.rot_q ? 0 : p.Hq * nt, nk = p.Hkv * nt, nv = p.rot_skip_v ? 0 : p.Hkv * vt;
  const int per_row = nq + nk + nv;
  const int i0 = blockIdx.x * kRowsPerWg;
  const int total = min(kRowsPerWg, p.S - i0) * per_row;
  const int R = p.rot_dim, half = R / 2, npair = half / 8;
  for (int base = 0; base < total; base += kThreads * TPT) {
    // phase 1: addresses and loads of every task of this thread
    uint4 xa[TPT], xb[TPT], xc[TPT], xs[TPT];
    T *dst[TPT];
    int kind[TPT];  // 0: none, 1: rotate split pair, 2: rotate interleaved, 3: copy
    int c0s[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      kind[u] = 0;
      const int t = base + u * kThreads + threadIdx.x;
      if (t >= total) continue;
      const int i = i0 + t / per_row, r = t % per_row;
      const int j = s.past + i;
      if (j >= p.T) continue;
      const int pos = j < p.rot_max ? j : p.rot_max - 1;
      const T *src;
      int task;
      if (r < nq + nk) {
        if (r < nq) {
          const int h = r / nt;
          task = r % nt;
          src = (const T *)p.q + b * p.q_sb + (int64_t)i * p.q_ss + (int64_t)h * p.q_sh;
          dst[u] = (T *)p.y + b * p.y_sb + (int64_t)i * p.y_ss + (int64_t)h * p.y_sh;
        } else {
          const int g = (r - nq) / nt;
          task = (r - nq) % nt;
          src = (const T *)p.k + b * p.k_sb + (int64_t)i * p.k_ss + (int64_t)g * p.k_sh;
          dst[u] = (T *)p.present_k + (((int64_t)b * p.Hkv + g) * p.T + j) * p.D;
        }
        const T *cs = (const T *)p.cos_cache + (int64_t)pos * half;
        const T *sn = (const T *)p.sin_cache + (int64_t)pos * half;
        if (p.rot_inter) {
          const int c0 = 8 * task;
          c0s[u] = c0;
          xa[u] = *(const uint4 *)(src + c0);
          if (c0 < R) {
            kind[u] = 2;
            const uint2 c4 = *(const uint2 *)(cs + c0 / 2), s4 = *(const uint2 *)(sn + c0 / 2);
            xc[u] = make_uint4(c4.x, c4.y, 0, 0);
            xs[u] = make_uint4(s4.x, s4.y, 0, 0);
          } else {
            kind[u] = 3;
          }
        } else if (task < npair) {
          const int c0 = 8 * task;
          c0s[u] = c0;
          kind[u] = 1;
          xa[u] = *(const uint4 *)(src + c0);
          xb[u] = *(const uint4 *)(src + c0 + half);
          xc[u] = *(const uint4 *)(cs + c0);
          xs[u] = *(const uint4 *)(sn + c0);
        } else {
          const int c0 = R + 8 * (task - npair);
          c0s[u] = c0;
          kind[u] = 3;
          xa[u] = *(const uint4 *)(src + c0);
        }
      } else {
        const int g = (r - nq - nk) / vt, c0 = 8 * ((r - nq - nk) % vt);
        c0s[u] = c0;
        kind[u] = 3;
        xa[u] = *(const uint4 *)((const T *)p.v + b * p.v_sb + (int64_t)i * p.v_ss +
                                 (int64_t)g * p.v_sh + c0);
        dst[u] = (T *)p.present_v + (((int64_t)b * p.Hkv + g) * p.T + j) * p.Dv;
      }
    }
    // phase 2: the same float32 arithmetic as rotate_task, one rounding
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      if (kind[u] == 0) continue;
      const int c0 = c0s[u];
      if (kind[u] == 3) {
        *(uint4 *)(dst[u] + c0) = xa[u];
      } else if (kind[u] == 2) {
        const T *x = (const T *)&xa[u], *c = (const T *)&xc[u], *sv = (const T *)&xs[u];
        Chunk8<T> o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x1 = (float)x[2 * e], x2 = (float)x[2 * e + 1];
          o.e[2 * e] = (T)rot_first(x1, x2, (float)c[e], (float)sv[e]);
          o.e[2 * e + 1] = (T)rot_second(x1, x2, (float)c[e], (float)sv[e]);
        }
        st8(dst[u] + c0, o);
      } else {
        const T *a = (const T *)&xa[u], *bb = (const T *)&xb[u];
        const T *c = (const T *)&xc[u], *sv = (const T *)&xs[u];
        Chunk8<T> oa, ob;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x1 = (float)a[e], x2 = (float)bb[e];
          oa.e[e] = (T)rot_first(x1, x2, (float)c[e], (float)sv[e]);
          ob.e[e] = (T)rot_second(x1, x2, (float)c[e], (float)sv[e]);
        }
        st8(dst[u] + c0, oa);
        st8(dst[u] + c0 + half, ob);
      }
    }
  }
}

// Channel form (any even R): one workgroup per (b, i) row: threads sweep the
// Hq*D query channels, then the Hkv*D key channels, then the Hkv*Dv value
// channels.
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(Params p) {
  const int i = blockIdx.x, b = blockIdx.y;
  const Seq s = seq_info(p, b);
  const int j = s.past + i;  // absolute position of query i and of new key i
  if (j >= p.T) return;
  const int pos = j < p.rot_max ? j : p.rot_max - 1;
  const int nq = p.rot_q ? 0 : p.Hq * p.D, nk = p.Hkv * p.D, nv = p.rot_skip_v ? 0 : p.Hkv * p.Dv;
  const T *qrow = (const T *)p.q + b * p.q_sb + (int64_t)i * p.q_ss;
  T *yrow = (T *)p.y + b * p.y_sb + (int64_t)i * p.y_ss;
  for (int t = threadIdx.x; t < nq + nk + nv; t += kThreads) {
    if (t < nq) {
      const int h = t / p.D, c = t % p.D;
      yrow[(int64_t)h * p.y_sh + c] = rotate_channel(p, qrow + (int64_t)h * p.q_sh, c, pos);
    } else if (t < nq + nk) {
      const int u = t - nq, g = u / p.D, c = u % p.D;
      const T *krow = (const T *)p.k + b * p.k_sb + (int64_t)i * p.k_ss + (int64_t)g * p.k_sh;
      T *dst = (T *)p.present_k + (((int64_t)b * p.Hkv + g) * p.T + j) * p.D;
      dst[c] = rotate_channel(p, krow, c, pos);
    } else {
      const int u = t - nq - nk, g = u / p.Dv, c = u % p.Dv;
      const T *vrow = (const T *)p.v + b * p.v_sb + (int64_t)i * p.v_ss + (int64_t)g * p.v_sh;
      T *dst = (T *)p.present_v + (((int64_t)b * p.Hkv + g) * p.T + j) * p.Dv;
      dst[c] = vrow[c];
    }
  }
}

}  // namespace

hipError_t launch_rope(const Params &p, int dtype, hipStream_t st) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  const dim3 grid(p.S, p.B);
  // 16-byte accesses need 8-channel chunks on 16-byte boundaries everywhere
  auto al = [](const void *x) { return ((uintptr_t)x & 15) == 0; };
  const int es = dtype == DT_F32 ? 4 : 2;
  const bool vec = p.rot_dim % 16 == 0 && p.D % 8 == 0 && p.Dv % 8 == 0 && al(p.q) && al(p.k) &&
                   al(p.v) && al(p.y) && al(p.present_k) && al(p.present_v) &&
                   al(p.cos_cache) && al(p.sin_cache) && (p.q_sh * es) % 16 == 0 &&
                   (p.q_ss * es) % 16 == 0 && (p.k_sh * es) % 16 == 0 && (p.k_ss * es) % 16 == 0 &&
                   (p.v_sh * es) % 16 == 0 && (p.v_ss * es) % 16 == 0 &&
                   (p.q_sb * es) % 16 == 0 && (p.k_sb * es) % 16 == 0 && (p.v_sb * es) % 16 == 0;
  if (vec) {
    const dim3 grid2((p.S + kRowsPerWg - 1) / kRowsPerWg, p.B);
    if (dtype == DT_BF16) hipLaunchKernelGGL((rope_vec2_kernel<bf16, 4>), grid2, dim3(kThreads), 0, st, p);
    else if (dtype == DT_F16) hipLaunchKernelGGL((rope_vec2_kernel<f16, 4>), grid2, dim3(kThreads), 0, st, p);
    else hipLaunchKernelGGL(rope_vec_kernel<float>, grid, dim3(kThreads), 0, st, p);
  } else {
    if (dtype == DT_BF16) hipLaunchKernelGGL(rope_kernel<bf16>, grid, dim3(kThreads), 0, st, p);
    else if (dtype == DT_F16) hipLaunchKernelGGL(rope_kernel<f16>, grid, dim3(kThreads), 0, st, p);
    else hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace olk
