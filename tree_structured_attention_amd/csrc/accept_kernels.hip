// Greedy acceptance of verified draft trees on device logits ("HSD:
// Training-Free Acceleration for Document Parsing Vision-Language Models with
// Hierarchical Speculative Decoding" notes, key design 3, the greedy tree
// traversal; "HPD-Parsing" notes, Algorithm 1, the acceptance length n_acc).
//
// Two launches on the caller's stream:
//   1. row_argmax: every logits row (one per tree node plus one root row per
//      tree) is cut into chunks; one workgroup streams one chunk with 16-byte
//      loads and writes its (max, first index of the max).  This is the whole
//      HBM cost: rows x vocab x element size, read once.
//   2. tree_walk: one wave per tree combines the chunk results of the rows it
//      visits and walks from the root: the child with the highest logit
//      (ties: lowest node index) is accepted iff z(u*) - z(u_hat) >= log tau,
//      evaluated in fp64 (only logit differences matter: the log-softmax
//      normaliser cancels); in exact mode the child whose token is u_hat is
//      accepted.  The walk ends at the first rejection or at a leaf; the
//      free token is u_hat of the row it ends on.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <climits>
#include <cstdint>

#include "ta_kernels.h"

namespace ta {

namespace {

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxUnroll = 4;

// (value, index) pairs: a higher value wins, equal values keep the lower
// index; index -1 is "nothing yet" and loses to everything.
__device__ __forceinline__ void take_best(float& bv, int32_t& bi, float ov, int32_t oi) {
  const bool take = oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi));
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

__device__ __forceinline__ void wave_best(float& bv, int32_t& bi) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int32_t oi = __shfl_xor(bi, off, 64);
    take_best(bv, bi, ov, oi);
  }
}

__device__ __forceinline__ float elt_to_f32(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float elt_to_f32(const __hip_bfloat16* p, int64_t i) {
  return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
}

// Elements of one 16-byte vector, as fp32.
template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const v4u32& u, float* x) {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  }
};
template <>
struct Vec<__hip_bfloat16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const v4u32& u, float* x) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <typename T>
__global__ __launch_bounds__(kArgmaxThreads) void row_argmax_kernel(AcceptParams p) {
  constexpr int N = Vec<T>::N;
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / p.chunks;
  const int64_t chunk = bid - row * p.chunks;
  const T* base = static_cast<const T*>(p.logits) + row * p.ld;
  const int64_t lo = chunk * p.chunk_elems;
  const int64_t hi = lo + p.chunk_elems < p.vocab ? lo + p.chunk_elems : p.vocab;
  const int tid = threadIdx.x;

  float bv = -INFINITY;
  int32_t bi = -1;
  // scalar head up to the first 16-byte boundary, vector body, scalar tail
  const uintptr_t addr = reinterpret_cast<uintptr_t>(base + lo);
  int64_t head = int64_t(((16 - (addr & 15)) & 15) / sizeof(T));
  if (head > hi - lo) head = hi - lo;
  const int64_t body = lo + head;
  const int64_t n_vec = (hi - body) / N;
  const int64_t tail = body + n_vec * N;
  for (int64_t i = lo + tid; i < body; i += kArgmaxThreads) take_best(bv, bi, elt_to_f32(base, i), int32_t(i));

  const v4u32* vp = reinterpret_cast<const v4u32*>(base + body);
  int64_t v = tid;
  for (; v + (kArgmaxUnroll - 1) * kArgmaxThreads < n_vec; v += kArgmaxUnroll * kArgmaxThreads) {
    v4u32 u[kArgmaxUnroll];
#pragma unroll
    for (int k = 0; k < kArgmaxUnroll; ++k) u[k] = __builtin_nontemporal_load(vp + v + k * kArgmaxThreads);
#pragma unroll
    for (int k = 0; k < kArgmaxUnroll; ++k) {
      float x[N];
      Vec<T>::unpack(u[k], x);
      const int32_t i0 = int32_t(body + (v + k * kArgmaxThreads) * N);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        // indices rise within a thread, so a strict > keeps the first maximum
        const bool gt = x[e] > bv || bi < 0;
        bv = gt ? x[e] : bv;
        bi = gt ? i0 + e : bi;
      }
    }
  }
  for (; v < n_vec; v += kArgmaxThreads) {
    float x[N];
    Vec<T>::unpack(vp[v], x);
    const int32_t i0 = int32_t(body + v * N);
#pragma unroll
    for (int e = 0; e < N; ++e) take_best(bv, bi, x[e], i0 + e);
  }
  for (int64_t i = tail + tid; i < hi; i += kArgmaxThreads) take_best(bv, bi, elt_to_f32(base, i), int32_t(i));

  wave_best(bv, bi);
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int32_t si[kArgmaxThreads / 64];
  const int wave = tid >> 6;
  if ((tid & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < kArgmaxThreads / 64; ++w) take_best(bv, bi, sv[w], si[w]);
    p.part_max[bid] = bv;
    p.part_idx[bid] = bi;
  }
}

template <typename T>
__global__ __launch_bounds__(64) void tree_walk_kernel(AcceptParams p) {
  const int32_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t off = p.tree_tab[b];
  const int32_t n = p.tree_tab[b + 1] - off;
  const int32_t* parent = p.tree_tab + (p.n_trees + 1) + off;
  const int32_t* tokens = p.tokens + off;
  const T* logits = static_cast<const T*>(p.logits);
  const int64_t row0 = int64_t(off) + b;  // root row of this tree

  int32_t cur = -1, len = 0;
  int64_t row = row0;
  int32_t top;
  for (;;) {
    // u_hat of this row from its chunk results
    float mv = -INFINITY;
    int32_t mi = -1;
    for (int32_t c = lane; c < p.chunks; c += 64)
      take_best(mv, mi, p.part_max[row * p.chunks + c], p.part_idx[row * p.chunks + c]);
    wave_best(mv, mi);
    top = mi;
    // best child of `cur`
    float cv = -INFINITY;
    int32_t ci = -1;
    for (int32_t i = lane; i < n; i += 64) {
      const int32_t t = tokens[i];
      if (parent[i] != cur || t < 0 || int64_t(t) >= p.vocab) continue;
      if (p.exact) {
        if (t == top && ci < 0) ci = i;  // lanes visit rising indices
      } else {
        take_best(cv, ci, elt_to_f32(logits, row * p.ld + t), i);
      }
    }
    if (p.exact) {
      // lowest node index that carries u_hat
      int32_t m = ci < 0 ? INT_MAX : ci;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = min(m, __shfl_xor(m, o, 64));
      ci = m == INT_MAX ? -1 : m;
    } else {
      wave_best(cv, ci);
    }
    if (ci < 0) break;
    if (!p.exact && !(double(cv) - double(mv) >= p.log_tau)) break;
    if (lane == 0) p.path[off + len] = ci;
    ++len;
    cur = ci;
    row = row0 + 1 + ci;
  }
  if (lane == 0) {
    p.n_path[b] = len;
    p.next_token[b] = top;
  }
}

}  // namespace

hipError_t launch_accept(int dtype, const AcceptParams& p, int64_t n_rows, hipStream_t st) {
  const int64_t blocks = n_rows * p.chunks;
  if (blocks > 0) {
    if (dtype == TA_DTYPE_BF16)
      row_argmax_kernel<__hip_bfloat16><<<dim3(uint32_t(blocks)), kArgmaxThreads, 0, st>>>(p);
    else
      row_argmax_kernel<float><<<dim3(uint32_t(blocks)), kArgmaxThreads, 0, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.n_trees > 0) {
    if (dtype == TA_DTYPE_BF16)
      tree_walk_kernel<__hip_bfloat16><<<dim3(uint32_t(p.n_trees)), 64, 0, st>>>(p);
    else
      tree_walk_kernel<float><<<dim3(uint32_t(p.n_trees)), 64, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace ta
