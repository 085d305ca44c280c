// Shared device/host helpers of the gfx950 contextual-sparsity LoRA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparselora.h"

namespace sl {

// bf16 is carried as raw 16-bit patterns; conversions round to nearest even.
struct bf16 {
  uint16_t v;
};

__host__ __device__ inline float bf2f(uint16_t h) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)h << 16;
  return x.f;
}
__host__ __device__ inline uint16_t f2bf(float f) {
  union { uint32_t u; float f; } x;
  x.f = f;
  uint32_t u = x.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static inline float load(const float* p, long long i) { return p[i]; }
  __device__ static inline void store(float* p, long long i, float v) { p[i] = v; }
};
template <> struct Elem<bf16> {
  __device__ static inline float load(const bf16* p, long long i) { return bf2f(p[i].v); }
  __device__ static inline void store(bf16* p, long long i, float v) { p[i].v = f2bf(v); }
};

template <typename T> __device__ inline float ldv(const T* p, long long i) { return Elem<T>::load(p, i); }
template <typename T> __device__ inline void stv(T* p, long long i, float v) { Elem<T>::store(p, i, v); }

// Sequence layout as seen by the kernels (passed by value in kernel arguments).
// Group g < nseq is the context part of sequence g (ctx[g] rows, the sequence's
// selected channels); group nseq is every output row of the batch (all channels).
struct SeqTab {
  int nseq, L, T_ctx, T_out;
  int ctx[SL_MAX_SEQS];
  int ctx_pre[SL_MAX_SEQS + 1];   // exclusive prefix of ctx
  int out_pre[SL_MAX_SEQS + 1];   // exclusive prefix of output-span lengths
};

// Token row of row i of the output group.
__device__ inline int out_token(const SeqTab& st, int i) {
  int lo = 0, hi = st.nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (st.out_pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo * st.L + st.ctx[lo] + (i - st.out_pre[lo]);
}

__device__ inline int group_rows(const SeqTab& st, int g) {
  return g < st.nseq ? st.ctx[g] : st.T_out;
}
// Token row of row i of group g.
__device__ inline int group_token(const SeqTab& st, int g, int i) {
  return g < st.nseq ? g * st.L + i : out_token(st, i);
}
// Row of row i of group g in the compact buffers (context region first).
__device__ inline int group_crow(const SeqTab& st, int g, int i) {
  return g < st.nseq ? st.ctx_pre[g] + i : i;
}

// Map blockIdx to a logical tile so that consecutive logical tiles run on the
// same XCD (blocks are dispatched round-robin over the 8 XCDs, each with its
// own L2): tiles that share an operand then share that XCD's L2.
__device__ inline int xcd_remap(int bid, int nb) {
  int xcd = bid & 7, loc = bid >> 3;
  int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + loc;
}

inline long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

}  // namespace sl
