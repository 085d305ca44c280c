// Bandwidth-bound kernels of the contextual-sparsity LoRA path on gfx950:
// the skinny low-rank products (estimator stage 1, LoRA activations), the
// per-channel criterion over context tokens, the per-sequence top-k, the LoRA
// factor gradients and a few layout helpers.
#pragma once

#include "sl_common.hpp"

#include <type_traits>

namespace sl {

typedef __bf16 bf16x8_t_s __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_s __attribute__((ext_vector_type(16)));

// ===========================================================================
// Skinny product  out[row, c] = sum_k A[row, k] * Bm(c, k),  c < C <= 64
//
// Estimator stage 1 (SparseLoRA article §二: the input is projected onto the
// leading right singular vectors, x V_r Sigma_r) and the LoRA activations
// x A^T, h A_d[:,S]^T, dY B_d, dG B_g[S].  Bandwidth-bound on A, which is
// streamed once.  A workgroup takes SK_RB rows and one K slice; each K chunk
// (256 bytes of a row) of A and of the (tiny, cache-resident) B operand is
// loaded with coalesced 16-byte loads, staged in LDS and consumed by 16x16
// MFMA tiles (one wave per 16 rows).  Rows too long for one workgroup are cut
// into K slices whose partial sums a second, small kernel adds in slice order
// (deterministic).
// ===========================================================================
constexpr int SK_RB = 32;                  // rows per workgroup (two waves of 16)
constexpr int SK_THREADS = 64 * (SK_RB / 16);
constexpr int SK_CB = 256;                 // bytes of a row per K chunk
constexpr int SK_LDB = SK_CB + 16;         // LDS row pitch in bytes (bank spread)
constexpr int SK_SLICE_BYTES = 1024;       // bytes of a row per K slice (4 chunks)
constexpr int SK_MAXSL = 64;               // slices per row block at most
constexpr int SK_PC = 64;                  // partial-sum row pitch at most (pc = NB*16)
constexpr int SK_PF = SK_SLICE_BYTES / SK_CB;   // chunks loaded at once (a whole slice)

struct SkinnyArgs {
  SeqTab st;
  int mode;               // 0: token rows 0..T-1; 1: compact rows of every group; 2: context rows
  int T;
  const void* A; long long lda, lda_out, a_out_off;   // compact geometry when mode 1
  int K;                  // > 0 fixed; <= 0: the group's channel count
  int kidx, n_out;
  // B operand: up to 4 row blocks; block j has nbk[j] rows, row c, column k at
  // Bb[j][c*ldbb[j] + k].  In mode 1, block 0 of context group g is read at
  // Bb[0] + g*b0_gstride and that of the output group at B0o (ld ldb0o).
  int nblk;
  const void* Bb[4]; int nbk[4]; long long ldbb[4];
  long long b0_gstride; const void* B0o; long long ldb0o;
  // Results at token rows; block j lands in columns [col0 + pj, col0 + pj + nbk[j])
  // where pj = sum of the previous blocks' sizes rounded up to 8; padding is 0.
  float* out; long long ldo; int col0; float oscale;
  void* outs; long long ldos; float scale;   // optional copy in the call dtype
  // Workgroups: group g owns [blk_start[g], blk_start[g+1]), row block major,
  // nsl[g] K slices of ksl[g] elements each.
  int blk_start[SL_MAX_SEQS + 2];
  int nsl[SL_MAX_SEQS + 1];
  int ksl[SL_MAX_SEQS + 1];
  int ngroups;
  int mrows;              // rows of the launch row space (see launch_row)
  int pc;                 // partial-sum row pitch: logical columns rounded up to 16
  float* part;            // partial sums [slice][launch row][pc] when a group has nsl > 1
  // Further problems of the same launch (nprob > 1, at most SK_MAXPROB): the
  // same mode, rows, K per group and B block sizes, with their own A operand,
  // block-0 B operand, output column offset and partial sums at part + p *
  // pstride.  Problem 0 is the fields above; the grid is nprob copies of the
  // one-problem layout.
  int nprob;
  long long pstride;
  struct {
    const void* A; long long lda, lda_out, a_out_off;
    const void* B0; long long ldb0, b0_gstride;
    const void* B0o; long long ldb0o;
    int col0;
  } xp[2];
};
constexpr int SK_MAXPROB = 3;

// Operands of problem p of a skinny launch.
struct SkProbView {
  const void* A; long long lda, lda_out, a_out_off;
  const void* B0; long long ldb0, b0_gstride;
  const void* B0o; long long ldb0o;
  int col0;
  float* part;
};
__device__ inline SkProbView skinny_prob(const SkinnyArgs& a, int p) {
  SkProbView v;
  if (p == 0) {
    v.A = a.A; v.lda = a.lda; v.lda_out = a.lda_out; v.a_out_off = a.a_out_off;
    v.B0 = a.Bb[0]; v.ldb0 = a.ldbb[0]; v.b0_gstride = a.b0_gstride;
    v.B0o = a.B0o; v.ldb0o = a.ldb0o; v.col0 = a.col0;
  } else {
    const auto& x = a.xp[p - 1];
    v.A = x.A; v.lda = x.lda; v.lda_out = x.lda_out; v.a_out_off = x.a_out_off;
    v.B0 = x.B0; v.ldb0 = x.ldb0; v.b0_gstride = x.b0_gstride;
    v.B0o = x.B0o; v.ldb0o = x.ldb0o; v.col0 = x.col0;
  }
  v.part = a.part ? a.part + p * a.pstride : nullptr;
  return v;
}

// Row of the launch row space: token order in mode 0, compact order otherwise
// (context rows of every sequence, then, in mode 1, the output rows).
__device__ inline int launch_row(const SkinnyArgs& a, int g, int r) {
  if (a.mode == 0) return r;
  return g < a.st.nseq ? a.st.ctx_pre[g] + r : a.st.T_ctx + r;
}
__device__ inline int skinny_group_of(const SkinnyArgs& a, int lrow, int& r) {
  if (a.mode == 0) { r = lrow; return 0; }
  if (lrow >= a.st.T_ctx) { r = lrow - a.st.T_ctx; return a.st.nseq; }
  int lo = 0, hi = a.st.nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.st.ctx_pre[mid] <= lrow) lo = mid; else hi = mid - 1;
  }
  r = lrow - a.st.ctx_pre[lo];
  return lo;
}
// Padded output column oc -> logical column (-1 for padding).
__device__ inline int skinny_logical_col(const SkinnyArgs& a, int oc) {
  int pc = 0, lc = 0;
  for (int j = 0; j < a.nblk; ++j) {
    const int pj = (a.nbk[j] + 7) / 8 * 8;
    if (oc < pc + pj) return (oc - pc) < a.nbk[j] ? lc + (oc - pc) : -1;
    pc += pj;
    lc += a.nbk[j];
  }
  return -1;
}
__device__ inline int skinny_padded_cols(const SkinnyArgs& a) {
  int p = 0;
  for (int j = 0; j < a.nblk; ++j) p += (a.nbk[j] + 7) / 8 * 8;
  return p;
}

// Keep the first `valid` elements of a 16-byte vector and zero the rest,
// without branches: the selects depend on `valid` only, so a batch of loads
// can all be in flight before the first mask is applied.
template <typename T>
__device__ inline uint4 mask_tail(uint4 v, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t m = valid >= 2 * i + 2 ? 0xFFFFFFFFu : (valid == 2 * i + 1 ? 0x0000FFFFu : 0u);
      w[i] &= m;
    } else {
      w[i] = valid > i ? w[i] : 0u;
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename T, int NB>
__global__ void __launch_bounds__(SK_THREADS)
skinny_kernel(const SkinnyArgs a) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte piece
  constexpr int KC = SK_CB / sizeof(T);      // elements per chunk
  constexpr int PR = SK_CB / 16;             // pieces per row and chunk (16)
  constexpr int AL = SK_RB * PR / SK_THREADS;                      // A pieces per thread
  constexpr int BL = (NB * 16 * PR + SK_THREADS - 1) / SK_THREADS; // B pieces per thread
  constexpr int STAGE_LD = NB * 16 + 1;
  constexpr int LDS_AB = (SK_RB + NB * 16) * SK_LDB;
  constexpr int LDS_ST = SK_RB * STAGE_LD * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_AB > LDS_ST ? LDS_AB : LDS_ST];
  unsigned char* As = smem;
  unsigned char* Bs = smem + SK_RB * SK_LDB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbs = a.blk_start[a.ngroups];              // workgroups per problem
  const int prob = a.nprob > 1 ? (int)blockIdx.x / nbs : 0;
  const int bid = (int)blockIdx.x - prob * nbs;
  const SkProbView pv = skinny_prob(a, prob);
  int g = 0;
  while (g + 1 < a.ngroups && a.blk_start[g + 1] <= bid) ++g;
  g = __builtin_amdgcn_readfirstlane(g);
  const int nsl = a.nsl[g];
  const int local = bid - a.blk_start[g];
  const int rb = local / nsl, sl = local % nsl;
  const bool is_out = (a.mode == 1 && g == a.st.nseq);
  const int m_rows = a.mode == 0 ? a.T : group_rows(a.st, g);
  const int Kfull = a.K > 0 ? a.K : (is_out ? a.n_out : a.kidx);
  const int kbeg = sl * a.ksl[g];
  const int kend = min(Kfull, kbeg + a.ksl[g]);
  const int nch = kend > kbeg ? (kend - kbeg + KC - 1) / KC : 0;

  // this thread's A pieces: row tid/PR + i*(SK_THREADS/PR), piece tid%PR
  const T* A = reinterpret_cast<const T*>(pv.A);
  const int q = tid % PR;
  const T* arow[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    int r = rb * SK_RB + tid / PR + i * (SK_THREADS / PR);
    if (r >= m_rows) r = m_rows - 1;        // loaded and dropped
    long long off;
    if (a.mode == 1)
      off = is_out ? pv.a_out_off + (long long)r * pv.lda_out : (long long)(a.st.ctx_pre[g] + r) * pv.lda;
    else
      off = (long long)(a.mode == 0 ? r : group_token(a.st, g, r)) * pv.lda;
    arow[i] = A + off;
  }
  // B pieces: logical column c = tid/PR + i*(SK_THREADS/PR)
  const T* brow[BL];
  bool bok[BL];
  int C = 0;
  for (int j = 0; j < a.nblk; ++j) C += a.nbk[j];
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    int c = tid / PR + i * (SK_THREADS / PR);
    bok[i] = c < C && c < NB * 16;
    brow[i] = nullptr;
    if (bok[i]) {
      for (int j = 0; j < a.nblk; ++j) {
        if (c < a.nbk[j]) {
          if (j == 0) {
            const T* B0 = reinterpret_cast<const T*>(pv.B0);
            long long ldb0 = pv.ldb0;
            if (a.mode == 1) {
              if (is_out && pv.B0o) { B0 = reinterpret_cast<const T*>(pv.B0o); ldb0 = pv.ldb0o; }
              else if (!is_out) B0 += (long long)g * pv.b0_gstride;
            }
            brow[i] = B0 + (long long)c * ldb0;
          } else {
            brow[i] = reinterpret_cast<const T*>(a.Bb[j]) + (long long)c * a.ldbb[j];
          }
          break;
        }
        c -= a.nbk[j];
      }
    }
    if (!brow[i]) brow[i] = arow[0];   // in range; loaded and zeroed
  }

  // SK_PF chunks are loaded at once, unconditionally (a chunk past the slice
  // reads in-range addresses and is never stored), so all their loads are in
  // flight together; the masks are applied on the way into LDS.
  uint4 ra[SK_PF][AL], rbv[SK_PF][BL];
  auto load = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < SK_PF; ++j) {
      const int k = kbeg + (c0 + j) * KC + q * E;
      const int kc = k < kend ? k : kbeg;
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[j][i] = *reinterpret_cast<const uint4*>(arow[i] + kc);
#pragma unroll
      for (int i = 0; i < BL; ++i) rbv[j][i] = *reinterpret_cast<const uint4*>(brow[i] + kc);
    }
  };
  auto store = [&](int c, int j) __attribute__((always_inline)) {
    const int valid = kend - (kbeg + c * KC + q * E);
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int r = tid / PR + i * (SK_THREADS / PR);
      *reinterpret_cast<uint4*>(As + r * SK_LDB + q * 16) = mask_tail<T>(ra[j][i], valid);
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int r = tid / PR + i * (SK_THREADS / PR);
      if (r < NB * 16)
        *reinterpret_cast<uint4*>(Bs + r * SK_LDB + q * 16) = mask_tail<T>(rbv[j][i], bok[i] ? valid : 0);
    }
  };

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&]() {
    const unsigned char* ap = As + (wave * 16 + (lane & 15)) * SK_LDB;
    if constexpr (sizeof(T) == 2) {
      // 4 k-steps of 32: lane holds 8 consecutive k at 8*(lane>>4)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 av = *reinterpret_cast<const uint4*>(ap + ks * 64 + 16 * (lane >> 4));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint4 bv = *reinterpret_cast<const uint4*>(Bs + (nb * 16 + (lane & 15)) * SK_LDB +
                                                           ks * 64 + 16 * (lane >> 4));
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t_s, av),
                                                            __builtin_bit_cast(bf16x8_t_s, bv), acc[nb],
                                                            0, 0, 0);
        }
      }
    } else {
      // 4 groups of 16 k: lane reads k = 4*(lane>>4) + 0..3 of the group and
      // feeds element j to MFMA j, whose k index p = lane>>4 then stands for
      // k = 4*p + j (the four MFMAs together cover the group)
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const float4 av = *reinterpret_cast<const float4*>(ap + kg * 64 + 16 * (lane >> 4));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float4 bv = *reinterpret_cast<const float4*>(Bs + (nb * 16 + (lane & 15)) * SK_LDB +
                                                             kg * 64 + 16 * (lane >> 4));
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc[nb], 0, 0, 0);
        }
      }
    }
  };

  for (int c0 = 0; c0 < nch; c0 += SK_PF) {
    load(c0);
    __builtin_amdgcn_sched_barrier(0);   // the batch's loads all issue before the first store waits
#pragma unroll
    for (int j = 0; j < SK_PF; ++j) {
      if (c0 + j < nch) {
        store(c0 + j, j);
        __syncthreads();
        compute();
        __syncthreads();
      }
    }
  }

  // accumulator element e: row 4*(lane>>4) + e of the wave's 16, column lane & 15
  if (nsl > 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rb * SK_RB + wave * 16 + 4 * (lane >> 4) + e;
        if (r < m_rows)
          pv.part[((long long)sl * a.mrows + launch_row(a, g, r)) * a.pc + nb * 16 + (lane & 15)] =
              acc[nb][e];
      }
    return;
  }
  float* stage = reinterpret_cast<float*>(smem);   // [SK_RB][STAGE_LD] logical columns
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      stage[(wave * 16 + 4 * (lane >> 4) + e) * STAGE_LD + nb * 16 + (lane & 15)] = acc[nb][e];
  __syncthreads();
  const int ptot = skinny_padded_cols(a);
  for (int i = tid; i < SK_RB * ptot; i += SK_THREADS) {
    const int rr = i / ptot, oc = i % ptot;
    const int row = rb * SK_RB + rr;
    if (row >= m_rows) continue;
    const int c = skinny_logical_col(a, oc);
    const float v = (c >= 0 && c < NB * 16) ? stage[rr * STAGE_LD + c] : 0.f;
    const long long tok = a.mode == 0 ? row : group_token(a.st, g, row);
    a.out[tok * a.ldo + pv.col0 + oc] = v * a.oscale;
    if (a.outs) stv<T>(reinterpret_cast<T*>(a.outs), tok * a.ldos + pv.col0 + oc, v * a.scale);
  }
}

// Adds the K slices of the groups with nsl > 1, in slice order, and writes the
// results (one thread per problem, launch row and padded column).
template <typename T>
__global__ void skinny_finish_kernel(const SkinnyArgs a) {
  const int ptot = skinny_padded_cols(a);
  const long long per = (long long)a.mrows * ptot;
  const long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int np = a.nprob > 1 ? a.nprob : 1;
  if (i0 >= per * np) return;
  const int prob = (int)(i0 / per);
  const long long i = i0 - prob * per;
  const SkProbView pv = skinny_prob(a, prob);
  const int lrow = (int)(i / ptot), oc = (int)(i % ptot);
  int r;
  const int g = skinny_group_of(a, lrow, r);
  const int nsl = a.nsl[g];
  if (nsl <= 1) return;
  const int c = skinny_logical_col(a, oc);
  float v = 0.f;
  if (c >= 0) {
    // slices in order; loads issued in groups of 8 before they are summed
    const float* p = pv.part + (long long)lrow * a.pc + c;
    const long long sstride = (long long)a.mrows * a.pc;
    for (int s0 = 0; s0 < nsl; s0 += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = s0 + j < nsl ? p[(s0 + j) * sstride] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) v += t[j];
    }
  }
  const long long tok = a.mode == 0 ? r : group_token(a.st, g, r);
  a.out[tok * a.ldo + pv.col0 + oc] = v * a.oscale;
  if (a.outs) stv<T>(reinterpret_cast<T*>(a.outs), tok * a.ldos + pv.col0 + oc, v * a.scale);
}

// ===========================================================================
// Channel criterion over context tokens (SparseLoRA article §一, §二).
// The estimate of channel n at context token t is z_t . Q[:, n], where z_t is
// the token's projection onto the estimator's leading directions (rank r).
// Each kernel writes per-sequence partial sums part[b][chunk][n] over chunks of
// context tokens; the select kernel adds a sequence's chunks in chunk order.
// ===========================================================================

// L2 criterion, sum over context rows t of (z_t . q_n)^2.  The identity
//   sum_t (z_t . q_n)^2 = q_n^T G q_n,   G = sum_t z_t z_t^T  (r x r),
// turns the token loop into one Gram matrix per sequence and a quadratic form
// per channel.  G and the form are taken in fp64: every product in G is exact
// (fp32 times fp32), so the fp32 result is at least as accurate as a direct
// fp32 sum of squares.  One partial per sequence.  One launch covers up to four
// projections (the QK-norm criterion's q and k, the L2 criterion's v of the
// same layer input): grid (channel blocks, nseq, projections); every workgroup rebuilds its sequence's G and scores
// GR_THREADS channels.
//
// G = Z^T Z runs on the fp64 matrix cores (16x16x4, K = 4 tokens per step):
// lane l supplies z[t][c], t = 4 g + l / 16, c = 16 blk + l % 16, to both the
// A (= Z^T) and the B (= Z) operand.  Wave w takes token groups w, w + 4, ...,
// loading GR_BATCH groups ahead of the matrix cores; the four waves' partial
// tiles are added in LDS in wave order.
constexpr int GR_THREADS = 256;
constexpr int GR_BATCH = 16;
typedef double f64x4_s __attribute__((ext_vector_type(4)));

struct GramArgs {
  SeqTab st;
  const float* Zh; long long ldz;
  int rank;
  int zc[4]; const void* Q[4]; int N[4]; float* part[4];   // up to 4 projections
};

template <typename T, int RM>
__global__ void __launch_bounds__(GR_THREADS)
score_gram_kernel(const GramArgs a) {
  constexpr int NB = RM <= 16 ? 1 : 2;        // 16-wide blocks per side of G
  constexpr int NW = GR_THREADS / 64;
  __shared__ double gs[NW][NB * NB][256];
  __shared__ double G[RM * RM];
  const int p = blockIdx.z, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N[p];
  const int n = blockIdx.x * GR_THREADS + tid;
  if ((int)blockIdx.x * GR_THREADS >= N) return;   // uniform
  const int ctx = a.st.ctx[b];
  if (ctx == 0) return;                            // no partial: the select reads none
  const T* Q = reinterpret_cast<const T*>(a.Q[p]);
  float qv[RM];
#pragma unroll
  for (int q = 0; q < RM; ++q) qv[q] = (n < N && q < a.rank) ? ldv<T>(Q, (long long)q * N + n) : 0.f;

  const float* zb = a.Zh + (long long)b * a.st.L * a.ldz + a.zc[p];
  const int ngrp = (ctx + 3) / 4;
  const int tl = lane >> 4, cl = lane & 15;
  auto load = [&](int g0, float (&z)[GR_BATCH][NB]) {
#pragma unroll
    for (int i = 0; i < GR_BATCH; ++i) {
      const int t = 4 * (g0 + NW * i) + tl;
#pragma unroll
      for (int bk = 0; bk < NB; ++bk) {
        const int c = 16 * bk + cl;
        z[i][bk] = (t < ctx && c < a.rank) ? zb[(long long)t * a.ldz + c] : 0.f;
      }
    }
  };
  f64x4_s acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f64x4_s{0.0, 0.0, 0.0, 0.0};
  float zcur[GR_BATCH][NB], zn[GR_BATCH][NB];
  load(wave, zcur);
  for (int g0 = wave; g0 < ngrp; g0 += NW * GR_BATCH) {
    if (g0 + NW * GR_BATCH < ngrp) load(g0 + NW * GR_BATCH, zn);
#pragma unroll
    for (int i = 0; i < GR_BATCH; ++i)
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)zcur[i][bi], (double)zcur[i][bj], acc[bi][bj],
                                                             0, 0, 0);
#pragma unroll
    for (int i = 0; i < GR_BATCH; ++i)
#pragma unroll
      for (int bk = 0; bk < NB; ++bk) zcur[i][bk] = zn[i][bk];
  }
  // element r of a lane's 16x16 fp64 tile: row lane / 16 + 4 r, column lane % 16
  // (rows strided by 4, unlike the fp32 16x16 tiles)
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
#pragma unroll
      for (int r = 0; r < 4; ++r) gs[wave][bi * NB + bj][(tl + 4 * r) * 16 + cl] = acc[bi][bj][r];
  __syncthreads();
  for (int e = tid; e < RM * RM; e += GR_THREADS) {
    const int r = e / RM, c = e % RM;
    const int blk = (r / 16) * NB + c / 16, off = (r % 16) * 16 + c % 16;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += gs[w][blk][off];
    G[e] = v;
  }
  __syncthreads();
  if (n >= N) return;
  double sc = 0.0;
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    double row = 0.0;
#pragma unroll
    for (int c = 0; c < RM; ++c) row = fma(G[r * RM + c], (double)qv[c], row);
    sc = fma((double)qv[r], row, sc);
  }
  a.part[p][(long long)b * N + n] = (float)sc;
}

// SwiGLU criterion, sum over context rows t of (SiLU(g) u)^2 with
// g = z_t . Qg[:, n] and u = z'_t . Qu[:, n].  The rank-r products run on the
// fp32 matrix cores (32x32x2): per wave a tile of 32 tokens x 32 channels, A =
// the tokens' projections (from LDS), B = the wave's 32 columns of Qg and Qu
// (registers).  The k order is permuted (lane half h takes k = h r/2 + s at
// step s, on both operands) so each lane reads contiguous LDS and factor rows;
// the sum over k does not depend on it.  Every accumulator element of a lane
// belongs to its column (lane % 32), so SiLU, the square and the sum over
// tokens stay in the lane; the two lane halves are added at the end.  Rows past
// the context are zero in LDS and contribute (SiLU(0) 0)^2 = 0.
// Workgroup: 4 waves = 128 channels over a chunk of SW_CHUNK tokens.
constexpr int SW_CHUNK = 128;        // context tokens per partial sum (fp32 kernel, bf16 default)
constexpr int SW_CHUNK_LONG = 256;   // bf16 kernel when every context fits two such chunks
constexpr int SW_THREADS = 256;

struct SwiArgs {
  SeqTab st;
  const float* Zh; long long ldz; int zc0, zc1;
  const void* Q0; const void* Q1; int rank; int N;
  float* part; int nchunk_max;
};

template <typename T, int RM>
__global__ void __launch_bounds__(SW_THREADS)
score_swiglu_kernel(const SwiArgs a) {
  constexpr int LDZ = 2 * RM + 4;        // padded LDS row: g part, u part
  constexpr int KH = RM / 2;             // k steps per projection
  __shared__ __attribute__((aligned(16))) float zs[SW_CHUNK * LDZ];
  const int b = blockIdx.z, chunk = blockIdx.y;
  const int ctx = a.st.ctx[b];
  const int t0 = chunk * SW_CHUNK;
  if (t0 >= ctx) return;
  const int nt = min(SW_CHUNK, ctx - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int n = blockIdx.x * 128 + wave * 32 + (lane & 31);
  // B operands first (latency overlaps the Z staging)
  float bg[KH], bu[KH];
  const T* Q0 = reinterpret_cast<const T*>(a.Q0);
  const T* Q1 = reinterpret_cast<const T*>(a.Q1);
#pragma unroll
  for (int s = 0; s < KH; ++s) {
    const int k = h * KH + s;
    const bool ok = n < a.N && k < a.rank;
    bg[s] = ok ? ldv<T>(Q0, (long long)k * a.N + n) : 0.f;
    bu[s] = ok ? ldv<T>(Q1, (long long)k * a.N + n) : 0.f;
  }
  const float* zb = a.Zh + (long long)(b * a.st.L + t0) * a.ldz;
  for (int i = tid; i < SW_CHUNK * 2 * RM; i += SW_THREADS) {
    const int t = i / (2 * RM), c = i % (2 * RM);
    const int pj = c / RM, q = c % RM;
    zs[t * LDZ + c] = (t < nt && q < a.rank) ? zb[(long long)t * a.ldz + (pj ? a.zc1 : a.zc0) + q] : 0.f;
  }
  __syncthreads();
  // Software pipeline over the chunk's SW_CHUNK / 32 tiles: tile t+1's
  // products are issued before tile t's SiLU, so the matrix cores work while
  // the VALU evaluates (sched_barrier keeps that order).  Tiles past the
  // context hold zero rows and add exactly 0.
  float acc0 = 0.f, acc1 = 0.f;
  auto mm = [&](int tt, f32x16_s& g, f32x16_s& u) {
    const float* zr = &zs[(tt * 32 + (lane & 31)) * LDZ + h * KH];
    float ag[KH], au[KH];
#pragma unroll
    for (int s = 0; s < KH; s += 4) {
      const float4 x = *reinterpret_cast<const float4*>(zr + s);
      const float4 y = *reinterpret_cast<const float4*>(zr + RM + s);
      ag[s] = x.x; ag[s + 1] = x.y; ag[s + 2] = x.z; ag[s + 3] = x.w;
      au[s] = y.x; au[s + 1] = y.y; au[s + 2] = y.z; au[s + 3] = y.w;
    }
    g = f32x16_s{};
    u = f32x16_s{};
#pragma unroll
    for (int s = 0; s < KH; ++s) {
      g = __builtin_amdgcn_mfma_f32_32x32x2f32(ag[s], bg[s], g, 0, 0, 0);
      u = __builtin_amdgcn_mfma_f32_32x32x2f32(au[s], bu[s], u, 0, 0, 0);
    }
  };
  auto act = [&](const f32x16_s& g, const f32x16_s& u) {
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float h0 = g[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[e])) * u[e];
      const float h1 = g[e + 1] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[e + 1])) * u[e + 1];
      acc0 = fmaf(h0, h0, acc0);
      acc1 = fmaf(h1, h1, acc1);
    }
  };
  static_assert(SW_CHUNK / 32 == 4, "four tiles per chunk");
  f32x16_s g0, u0, g1, u1;
  mm(0, g0, u0);
  mm(1, g1, u1);
  __builtin_amdgcn_sched_barrier(0);
  act(g0, u0);
  __builtin_amdgcn_sched_barrier(0);
  mm(2, g0, u0);
  __builtin_amdgcn_sched_barrier(0);
  act(g1, u1);
  __builtin_amdgcn_sched_barrier(0);
  mm(3, g1, u1);
  __builtin_amdgcn_sched_barrier(0);
  act(g0, u0);
  act(g1, u1);
  float v = acc0 + acc1;
  v += __shfl_xor(v, 32, 64);
  if (h == 0 && n < a.N) a.part[((long long)b * a.nchunk_max + chunk) * a.N + n] = v;
}

// bf16 form of the SwiGLU criterion.  Each context token's fp32 projection z
// is split exactly into three bf16 terms, z = hi + mid + lo (each term takes
// the next 8 significant bits; the bf16 factor Q is exact), so the bf16 matrix
// cores form g = sum_q (hi_q + mid_q + lo_q) Q_q from exact products with fp32
// accumulation, the accuracy of an fp32 dot product, in one 16x16x32 MFMA per
// 16 tokens x 16 channels and 32 k (k = s RM + q for term s, rank index q;
// padding k add zero).  The gate projection is scaled by -log2(e) first, so
// the MFMA yields g' = -g log2(e), exp2(g') = e^{-g}, and
//   (SiLU(g) u)^2 = (g' u / (1 + exp2(g')))^2 ln(2)^2,
// with ln(2)^2 applied once per channel sum.  Per wave 32 channels (two
// 16-column blocks) over the chunk's CH tokens (CH / 16 row blocks, those
// past the context skipped in pairs); a lane's accumulator values all belong
// to its column, so the square and the token sum stay in the lane until the
// four lane groups are added at the end.
template <int RM, int CH>
__global__ void __launch_bounds__(SW_THREADS)
score_swiglu_split_kernel(const SwiArgs a) {
  constexpr int KA = (3 * RM + 31) / 32 * 32;   // k of the split products, whole MFMA steps
  constexpr int NKB = KA / 32;
  constexpr int PITCH = KA * 2 + 16;            // LDS row pitch in bytes (bank spread)
  constexpr int NRB = CH / 16;                  // 16-token row blocks per chunk
  static_assert(CH % 32 == 0 && CH <= SW_CHUNK_LONG, "row blocks in pairs");
  __shared__ __attribute__((aligned(16))) unsigned char zs[2][CH * PITCH];   // [g/u][token][k]
  const int b = blockIdx.z, chunk = blockIdx.y;
  const int ctx = a.st.ctx[b];
  const int t0 = chunk * CH;
  if (t0 >= ctx) return;
  const int nt = min(CH, ctx - t0);
  const int nrb = (nt + 31) / 32 * 2;           // row blocks holding context tokens, rounded to pairs
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;

  // B operands (the factors' columns, k = s RM + q -> Q[q][n]) first, so
  // their latency overlaps the Z staging
  const uint16_t* Qp[2] = {reinterpret_cast<const uint16_t*>(a.Q0), reinterpret_cast<const uint16_t*>(a.Q1)};
  bf16x8_t_s bq[2][2][NKB];   // [g/u][column block][k step]
#pragma unroll
  for (int pj = 0; pj < 2; ++pj)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int n = blockIdx.x * 128 + wave * 32 + cb * 16 + col;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int k0 = kb * 32 + 8 * grp;
        const int s = k0 / RM, q0 = k0 % RM;
        uint16_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = (s < 3 && q0 + j < a.rank && n < a.N) ? Qp[pj][(long long)(q0 + j) * a.N + n] : (uint16_t)0;
        uint4 w = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                             v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
        bq[pj][cb][kb] = __builtin_bit_cast(bf16x8_t_s, w);
      }
    }
  // Z staging: thread (t, pj) splits one token's RM projections into three
  // bf16 rows hi | mid | lo at k = 0, RM, 2 RM; rows past the context are 0
  static_assert(SW_THREADS == 2 * SW_CHUNK, "one thread per token and projection of a 128-token pass");
#pragma unroll
  for (int tp = 0; tp < CH; tp += SW_CHUNK) {
    const int t = tp + (tid >> 1), pj = tid & 1;
    const float sc = pj == 0 ? -1.4426950408889634f : 1.f;   // -log2(e) on the gate
    const float* zr = a.Zh + (long long)(b * a.st.L + t0 + t) * a.ldz + (pj ? a.zc1 : a.zc0);
    unsigned char* row = zs[pj] + t * PITCH;
    static_assert(RM % 8 == 0, "whole 16-byte groups of k");
#pragma unroll
    for (int q0 = 0; q0 < RM; q0 += 8) {
      uint32_t w[3][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < nt && q0 + 4 * h < a.rank) z4 = *reinterpret_cast<const float4*>(zr + q0 + 4 * h);
        const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          uint16_t hi[2], mid[2], lo[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const float z = q0 + 4 * h + j + i < a.rank ? zz[j + i] * sc : 0.f;
            hi[i] = f2bf(z);
            const float r1 = z - bf2f(hi[i]);
            mid[i] = f2bf(r1);
            lo[i] = f2bf(r1 - bf2f(mid[i]));
          }
          w[0][2 * h + j / 2] = hi[0] | (uint32_t)hi[1] << 16;
          w[1][2 * h + j / 2] = mid[0] | (uint32_t)mid[1] << 16;
          w[2][2 * h + j / 2] = lo[0] | (uint32_t)lo[1] << 16;
        }
      }
#pragma unroll
      for (int sgm = 0; sgm < 3; ++sgm)
        *reinterpret_cast<uint4*>(row + 2 * (sgm * RM + q0)) = make_uint4(w[sgm][0], w[sgm][1], w[sgm][2], w[sgm][3]);
    }
#pragma unroll
    for (int k = 3 * RM; k < KA; k += 8) *reinterpret_cast<uint4*>(row + 2 * k) = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  auto mm = [&](int rb, f32x4_t (&g)[2], f32x4_t (&u)[2]) __attribute__((always_inline)) {
    const int off = (rb * 16 + col) * PITCH + 16 * grp;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) { g[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f}; u[cb] = g[cb]; }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8_t_s ag = *reinterpret_cast<const bf16x8_t_s*>(zs[0] + off + 64 * kb);
      const bf16x8_t_s au = *reinterpret_cast<const bf16x8_t_s*>(zs[1] + off + 64 * kb);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        g[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bq[0][cb][kb], g[cb], 0, 0, 0);
        u[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, bq[1][cb][kb], u[cb], 0, 0, 0);
      }
    }
  };
  auto act = [&](const f32x4_t (&g)[2], const f32x4_t (&u)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float h = g[cb][e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g[cb][e])) * u[cb][e];
        acc[cb][e] = fmaf(h, h, acc[cb][e]);
      }
  };
  // two row blocks in flight: block rb + 1's products are issued before
  // block rb's activation (rows past the context are zero and add exactly 0;
  // pairs of blocks wholly past it are skipped)
  f32x4_t g0[2], u0[2], g1[2], u1[2];
  mm(0, g0, u0);
#pragma unroll
  for (int rb = 0; rb < NRB; rb += 2) {
    if (rb >= nrb) break;
    mm(rb + 1, g1, u1);
    __builtin_amdgcn_sched_barrier(0);
    act(g0, u0);
    __builtin_amdgcn_sched_barrier(0);
    if (rb + 2 < NRB && rb + 2 < nrb) mm(rb + 2, g0, u0);
    __builtin_amdgcn_sched_barrier(0);
    act(g1, u1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane sums (4 tokens each) -> column sums over the four lane groups
  constexpr float LN2SQ = 0.480453013918201424667f;   // ln(2)^2
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    float v = (acc[cb][0] + acc[cb][1]) + (acc[cb][2] + acc[cb][3]);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    const int n = blockIdx.x * 128 + wave * 32 + cb * 16 + col;
    if (grp == 0 && n < a.N) a.part[((long long)b * a.nchunk_max + chunk) * a.N + n] = v * LN2SQ;
  }
}

// ===========================================================================
// Per-sequence top-k (SparseLoRA article §一: per input, keep the most active
// channels), in two launches.  score_finish_kernel adds each channel's
// partial sums (many workgroups, chunks in chunk order) and writes the scores
// as keys: scores are >= 0, so the fp32 bit pattern is an order-preserving
// unsigned key.  select_kernel, one 1024-thread workgroup per sequence and
// job, finds the k-th largest key tau with radix passes of up to 8 bits and
// writes every key > tau plus the lowest-index keys == tau, in ascending
// channel order, each thread owning a contiguous range of keys (in registers
// up to SEL_KPT_REG keys per thread; SEL_MAXN channels at most).
// ===========================================================================
constexpr int SEL_THREADS = 1024;
constexpr int SEL_KPT_REG = 32;
constexpr int SEL_MAXN = 65536;

// One selection job: its partial sums, channel count, k and outputs.
struct SelJob {
  int qk;                 // 0: score = sum of part0 chunks; 1: QK combination
  const float* part0; const float* part1;
  int nchunk_max;
  int chunk;              // context tokens per partial (a sequence has ceil(ctx / chunk))
  int N;                  // channels selected over
  int N0;                 // columns of part0 rows (QK: Hq*hd; else N)
  int group, head_dim;    // QK: query heads per kv head, head size
  int k;
  int* idx; float* scores;
  uint32_t* gkeys;        // [batch][N] keys in workspace
};
constexpr int SEL_MAXJOBS = 3;

// grid (sequences, jobs): workgroup (b, j) selects job j's set for sequence b.
struct SelectArgs {
  SeqTab st;
  int njobs;
  SelJob job[SEL_MAXJOBS];
};

// Scores of one sequence and job from the criterion's partial sums: grid
// (channel blocks, sequences, jobs), one channel per thread.  The L2-type
// score of channel n is the sum of its chunk partials in chunk order; the QK
// score is sk_n sq_n with sk_n the key projection's sum and sq_n the sum over
// the kv head's query heads of the query projection's sums.
constexpr int SF_THREADS = 256;
static __global__ void __launch_bounds__(SF_THREADS) score_finish_kernel(const SelectArgs a) {
  const SelJob& J = a.job[blockIdx.z];
  const int b = blockIdx.y;
  const int n = (int)blockIdx.x * SF_THREADS + (int)threadIdx.x;
  if (n >= J.N) return;
  const int ctx = a.st.ctx[b];
  const int nch = (int)(((long long)ctx + J.chunk - 1) / J.chunk);
  const long long pb = (long long)b * J.nchunk_max;
  // chunks added in order, eight loads in flight
  auto colsum = [&](const float* part, int ld, int col) {
    float v = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = c0 + u < nch ? part[(pb + c0 + u) * ld + col] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < nch) v += t[u];
    }
    return v;
  };
  float sc;
  if (!J.qk) {
    sc = colsum(J.part0, J.N0, n);
  } else {
    sc = colsum(J.part1, J.N, n);
    float sq = 0.f;
    for (int h = 0; h < J.group; ++h)
      sq += colsum(J.part0, J.N0, ((n / J.head_dim) * J.group + h) * J.head_dim + n % J.head_dim);
    sc *= sq;
  }
  if (J.scores) J.scores[(long long)b * J.N + n] = sc;
  J.gkeys[(long long)b * J.N + n] = __float_as_uint(sc);
}

__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive prefix of a pair of counts over the workgroup, packed as
// (a << 32) | b in 64 bits (each sum stays below 2^32).
__device__ inline unsigned long long block_excl_scan2(unsigned long long v, unsigned long long* wsum2, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  unsigned long long incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wsum2[wave] = incl;
  __syncthreads();
  unsigned long long base = 0;
#pragma unroll
  for (int w = 0; w < SEL_THREADS / 64; ++w) base += w < wave ? wsum2[w] : 0ull;
  return base + incl - v;
}

template <int KPT, bool FUSED>
__global__ void __launch_bounds__(SEL_THREADS)
select_kernel(const SelectArgs a) {
  // Thread tid owns keys [tid per, tid per + per), per = ceil(N / SEL_THREADS).
  // KPT > 0: they are held in registers (per <= KPT), so the radix passes and
  // the ordered compaction read no memory; KPT == 0: they are re-read from the
  // workspace (L2-resident) in every pass.  FUSED (KPT > 0, few partials per
  // channel): the keys are formed here from the criterion's partial sums, with
  // the arithmetic of score_finish_kernel, and no finish launch precedes.
  extern __shared__ float sdyn[];   // FUSED: the N scores (dynamic, N * 4 bytes)
  __shared__ int hist[16][256];
  __shared__ int cnt_s[4];
  __shared__ unsigned long long wsum2[SEL_THREADS / 64];
  __shared__ uint32_t wmax[SEL_THREADS / 64], wmin[SEL_THREADS / 64];
  __shared__ int s_sel[3];
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const SelJob& J = a.job[blockIdx.y];
  const int N = J.N;
  const int per = (N + SEL_THREADS - 1) / SEL_THREADS;
  const int n0 = min(N, tid * per), n1 = min(N, n0 + per);
  const uint32_t* gk = J.gkeys + (long long)b * N;

  uint32_t key[KPT > 0 ? KPT : 1];
  if constexpr (FUSED) {
    static_assert(KPT > 0, "fused keys live in registers");
    // Scores with coalesced loads (channel n = tid + SEL_THREADS i, up to four
    // chunks' loads in flight at once), staged in LDS, then read back as this
    // thread's contiguous range.  Same arithmetic and order as
    // score_finish_kernel: chunks added in order from 0, QK = sk * sq.
    const int ctx = a.st.ctx[b];
    const int nch = (int)(((long long)ctx + J.chunk - 1) / J.chunk);
    const long long pb = (long long)b * J.nchunk_max;
    // The fused form serves at most two partials per channel (the host's
    // rule), so all KPT channels' loads of two chunks are in flight at once.
    constexpr int CS = 2;                    // chunks per load batch
    auto colsum = [&](const float* part, int ld, auto col, float (&out)[KPT]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) out[i] = 0.f;
      for (int c0 = 0; c0 < nch; c0 += CS) {
        float t[CS][KPT];
#pragma unroll
        for (int u = 0; u < CS; ++u)
#pragma unroll
          for (int i = 0; i < KPT; ++i) {
            const int n = tid + SEL_THREADS * i;
            t[u][i] = (c0 + u < nch && n < N) ? part[(pb + c0 + u) * ld + col(n)] : 0.f;
          }
#pragma unroll
        for (int u = 0; u < CS; ++u)
#pragma unroll
          for (int i = 0; i < KPT; ++i)
            if (c0 + u < nch) out[i] += t[u][i];
      }
    };
    float sc[KPT];
    if (!J.qk) {
      colsum(J.part0, J.N0, [](int n) { return n; }, sc);
    } else {
      colsum(J.part1, J.N, [](int n) { return n; }, sc);
      float sq[KPT], t[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) sq[i] = 0.f;
      for (int h = 0; h < J.group; ++h) {
        colsum(J.part0, J.N0,
               [&](int n) { return ((n / J.head_dim) * J.group + h) * J.head_dim + n % J.head_dim; }, t);
#pragma unroll
        for (int i = 0; i < KPT; ++i) sq[i] += t[i];
      }
#pragma unroll
      for (int i = 0; i < KPT; ++i) sc[i] *= sq[i];
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int n = tid + SEL_THREADS * i;
      if (n < N) {
        sdyn[n] = sc[i];
        if (J.scores) J.scores[(long long)b * N + n] = sc[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = n0 + j < n1 ? __float_as_uint(sdyn[n0 + j]) : 0u;
  } else if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = n0 + j < n1 ? gk[n0 + j] : 0u;
  }
  // f(key, channel) over this thread's keys, in channel order
  auto for_keys = [&](auto&& f) __attribute__((always_inline)) {
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (n0 + j < n1) f(key[j], n0 + j);
    } else {
      for (int n = n0; n < n1; ++n) f(gk[n], n);
    }
  };
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  for_keys([&](uint32_t kv, int) {
    kmax = kv > kmax ? kv : kmax;
    kmin = kv < kmin ? kv : kmin;
  });
  // range of the keys: bits above the highest one in which any two differ are common
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t x = (uint32_t)__shfl_xor((int)kmax, off, 64);
    const uint32_t y = (uint32_t)__shfl_xor((int)kmin, off, 64);
    kmax = x > kmax ? x : kmax;
    kmin = y < kmin ? y : kmin;
  }
  if (lane == 0) { wmax[wave] = kmax; wmin[wave] = kmin; }
  for (int i = tid; i < 16 * 256; i += SEL_THREADS) (&hist[0][0])[i] = 0;   // first pass's histograms
  __syncthreads();
#pragma unroll
  for (int w = 0; w < SEL_THREADS / 64; ++w) {
    kmax = wmax[w] > kmax ? wmax[w] : kmax;
    kmin = wmin[w] < kmin ? wmin[w] : kmin;
  }
  const int hbit = kmax == kmin ? -1 : 31 - __clz(kmax ^ kmin);
  const uint32_t low = hbit >= 31 ? 0xFFFFFFFFu : ((1u << (hbit + 1)) - 1u);
  uint32_t mask = ~low, prefix = kmax & ~low;
  int kr = J.k;   // still to take among keys matching prefix

  // radix passes of up to 8 bits from the highest differing bit down, three
  // barriers per pass: the 256 bins (in descending digit order) are summed
  // over the per-wave copies, which are cleared as they are read, and scanned
  // by four waves.  The passes stop early once the bin that holds the k-th
  // key is taken whole: then no tie inside the set needs breaking.
  int cbin = 0;
  for (int hi = hbit; hi >= 0;) {
    const int w = hi + 1 < 8 ? hi + 1 : 8;
    const int lo = hi - w + 1;
    const int nb = 1 << w;
    for_keys([&](uint32_t kv, int) {
      if ((kv & mask) == prefix) atomicAdd(&hist[wave][(kv >> lo) & (uint32_t)(nb - 1)], 1);
    });
    __syncthreads();
    int c = 0, incl = 0;
    if (tid < 256) {
      if (tid < nb) {
        const int d = nb - 1 - tid;
#pragma unroll
        for (int wv = 0; wv < 16; ++wv) { c += hist[wv][d]; hist[wv][d] = 0; }
      }
      incl = wave_incl_scan(c);
      if (lane == 63) cnt_s[wave] = incl;
    }
    __syncthreads();
    if (tid < nb) {
      int before = incl - c;
      for (int wv = 0; wv < wave; ++wv) before += cnt_s[wv];
      if (before < kr && kr <= before + c) { s_sel[0] = nb - 1 - tid; s_sel[1] = before; s_sel[2] = c; }
    }
    __syncthreads();
    prefix |= (uint32_t)s_sel[0] << lo;
    mask |= (uint32_t)(nb - 1) << lo;
    kr -= s_sel[1];
    cbin = s_sel[2];
    hi = lo - 1;
    if (kr == cbin) break;
  }
  // The set: every key whose masked value exceeds prefix, plus the first kr
  // (in channel order) of those equal to it.

  // ordered compaction over the contiguous per-thread ranges: one scan of the
  // (greater, equal) counts; a thread's first output position is
  // greater-before + min(kr, equal-before)
  int n_gt = 0, n_eq = 0;
  for_keys([&](uint32_t kv, int) {
    const uint32_t m = kv & mask;
    n_gt += m > prefix;
    n_eq += m == prefix;
  });
  const unsigned long long sc2 = block_excl_scan2(((unsigned long long)n_gt << 32) | (unsigned)n_eq, wsum2, tid);
  const int gt_before = (int)(sc2 >> 32), eq_before = (int)(sc2 & 0xFFFFFFFFull);
  int take_eq = kr - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
  int pos = gt_before + (kr < eq_before ? kr : eq_before), eq_seen = 0;
  int* out = J.idx + (long long)b * J.k;
  for_keys([&](uint32_t kv, int n) {
    const uint32_t m = kv & mask;
    bool take = m > prefix;
    if (m == prefix) { take = eq_seen < take_eq; ++eq_seen; }
    if (take) out[pos++] = n;
  });
}

// ===========================================================================
// LoRA factor gradients: column reductions over tokens,
//   part[chunk][n][q] = sum over the chunk's rows t of P[t, n] * Z[tok(t), zc0 + q]
// (dA = dz^T X, dB = s dG^T z, dB_d = s dY^T z_d, dA_d[:,S] = dz_d^T H).  Each
// thread owns two adjacent columns; chunks of 128 rows; the finish kernels add
// the chunks in a fixed order (deterministic, no atomics).
// ===========================================================================
constexpr int CR_CHUNK = 128;
constexpr int CR_THREADS = 256;

struct ColredArgs {
  SeqTab st;
  int mode;                 // 0: token rows 0..T-1; 1: compact rows per group
  int T;
  const void* P; long long ldp, ldp_out, p_out_off;
  int N;                    // mode 0: columns; mode 1: ignored (group channel count)
  int kidx, n_out;
  const float* Z; long long ldz; int zc0; int R;   // R padded to a multiple of 8
  float* part;
  int chunk_start[SL_MAX_SEQS + 2];   // first chunk of each group (mode 1)
  long long part_off[SL_MAX_SEQS + 2];
  int ngroups;
};

template <typename T, int RM>
__global__ void __launch_bounds__(CR_THREADS)
colred_kernel(const ColredArgs a) {
  __shared__ float zsh[CR_CHUNK][RM];
  int g = 0, ch = blockIdx.y;
  if (a.mode == 1) {
    while (g + 1 < a.ngroups && a.chunk_start[g + 1] <= (int)blockIdx.y) ++g;
    ch = blockIdx.y - a.chunk_start[g];
  }
  const bool is_out = a.mode == 1 && g == a.st.nseq;
  const int m_rows = a.mode == 0 ? a.T : group_rows(a.st, g);
  const int N = a.mode == 0 ? a.N : (is_out ? a.n_out : a.kidx);
  const int r0 = ch * CR_CHUNK;
  const int nr = min(CR_CHUNK, m_rows - r0);
  for (int i = threadIdx.x; i < CR_CHUNK * RM; i += CR_THREADS) {
    const int t = i / RM, q = i % RM;
    float v = 0.f;
    if (t < nr && q < a.R) {
      const long long tok = a.mode == 0 ? r0 + t : group_token(a.st, g, r0 + t);
      v = a.Z[tok * a.ldz + a.zc0 + q];
    }
    zsh[t][q] = v;
  }
  __syncthreads();
  const int n = (blockIdx.x * CR_THREADS + threadIdx.x) * 2;
  if (n >= N) return;
  const T* P = reinterpret_cast<const T*>(a.P);
  float acc0[RM], acc1[RM];
#pragma unroll
  for (int q = 0; q < RM; ++q) { acc0[q] = 0.f; acc1[q] = 0.f; }
  const bool two = n + 1 < N;
  for (int t = 0; t < nr; ++t) {
    long long prow;
    if (a.mode == 0) prow = (long long)(r0 + t) * a.ldp;
    else prow = is_out ? a.p_out_off + (long long)(r0 + t) * a.ldp_out
                       : (long long)(a.st.ctx_pre[g] + r0 + t) * a.ldp;
    const float p0 = ldv<T>(P, prow + n);
    const float p1 = two ? ldv<T>(P, prow + n + 1) : 0.f;
#pragma unroll
    for (int q = 0; q < RM; ++q) {
      const float z = zsh[t][q];
      acc0[q] = fmaf(p0, z, acc0[q]);
      acc1[q] = fmaf(p1, z, acc1[q]);
    }
  }
  float* dst = a.part + (a.mode == 1 ? a.part_off[g] : 0) + ((long long)ch * N + n) * RM;
#pragma unroll
  for (int q = 0; q < RM; ++q) dst[q] = acc0[q];
  if (two) {
#pragma unroll
    for (int q = 0; q < RM; ++q) dst[RM + q] = acc1[q];
  }
}

// Geometry of the bf16 (matrix-core) form below: a workgroup owns CRM_COLS
// columns of P and a chunk of CRM_CHUNK rows, taken as CRM_SLICES slices of
// CRM_SLICE rows whose global loads are all issued before the first is
// consumed (the work is latency-bound otherwise).
constexpr int CRM_SLICE = 64;
constexpr int CRM_SLICES = 2;
constexpr int CRM_CHUNK = CRM_SLICE * CRM_SLICES;
constexpr int CRM_COLS = 256;

// ---------------------------------------------------------------------------
// Batched form for bf16: every column reduction of a backward pass in one
// launch, then every finish in one launch.  A job is one reduction
//   part[chunk][n][q] = sum over the chunk's rows t of P[t, n] * Z[tok(t), zc0 + q]
// over token rows (mode 0) or over the compact rows of each group (mode 1,
// context groups on their kidx selected columns, the output group on all
// n_out); q < R, partial rows RM wide (RM a multiple of 16, R <= RM).  Mode-1
// partials of group g start at part + sum over earlier groups of
// chunks x columns x RM, the layout the finish kernels read.  Work item =
// (job, group, chunk of CRM_CHUNK rows, block of CRM_COLS columns).  Each
// slice of P is transposed into LDS as [column][row] (K-contiguous for the
// matrix cores) and Z is converted to bf16 and stored as [q][row]; 16x16x32
// MFMAs accumulate C[column][q], each wave owning 64 columns.  (Chunks of 4
// slices, walked with the next slice's loads in flight, measured slower: half
// the partials, but too few workgroups to hide the latency.)
// ---------------------------------------------------------------------------
constexpr int CB_MAXJOBS = 8;

struct CbJob {
  int mode, N, kidx, n_out, R, RM;
  const void* P; long long ldp, ldp_out, p_out_off;
  const float* Z; long long ldz; int zc0;
  float* part;
  long long item0;
};

struct CbArgs {
  SeqTab st;
  int T, njobs;
  long long nitems;
  CbJob job[CB_MAXJOBS];
};

__device__ inline int cb_group_cols(const CbJob& j, const SeqTab& st, int g) {
  return g == st.nseq ? j.n_out : j.kidx;
}

template <int RMX>
__global__ void __launch_bounds__(256)
colred_batch_kernel(const CbArgs a) {
  constexpr int LD = CRM_SLICE + 8;   // padded LDS row (144 bytes)
  __shared__ __attribute__((aligned(16))) uint16_t Ps[CRM_COLS * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Zs[RMX * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long item = blockIdx.x;
  int jb = 0;
  while (jb + 1 < a.njobs && a.job[jb + 1].item0 <= item) ++jb;
  jb = __builtin_amdgcn_readfirstlane(jb);
  const CbJob& J = a.job[jb];
  long long e = item - J.item0;
  // locate (group, chunk, column block) and the group's partial offset
  int g = 0, ch, cb, N, m_rows;
  long long poff = 0;
  if (J.mode == 0) {
    N = J.N; m_rows = a.T;
    const int ncb = (N + CRM_COLS - 1) / CRM_COLS;
    ch = (int)(e / ncb); cb = (int)(e % ncb);
  } else {
    for (;;) {
      const int rows = group_rows(a.st, g);
      const int cols = cb_group_cols(J, a.st, g);
      const int nch = (rows + CRM_CHUNK - 1) / CRM_CHUNK;
      const int ncb = (cols + CRM_COLS - 1) / CRM_COLS;
      const long long ni = (long long)nch * ncb;
      if (e < ni || g == a.st.nseq) { ch = (int)(e / ncb); cb = (int)(e % ncb); N = cols; m_rows = rows; break; }
      e -= ni;
      poff += (long long)nch * cols * J.RM;
      ++g;
    }
  }
  const bool is_out = J.mode == 1 && g == a.st.nseq;
  const int n0 = cb * CRM_COLS;
  const uint16_t* P = reinterpret_cast<const uint16_t*>(J.P);
  const int ctx_pre_g = (J.mode == 1 && !is_out) ? a.st.ctx_pre[g] : 0;
  const int nq16 = J.RM / 16;
  const int pr0 = (tid & 7) * 8;
  const int pc = (tid >> 3) * 8;
  const bool c_ok = n0 + pc < N;                     // N is a multiple of 8
  const int pcol = c_ok ? n0 + pc : 0;
  f32x4_t acc[4][RMX / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < RMX / 16; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int r_begin = ch * CRM_CHUNK;
  const int r_end = min(m_rows, r_begin + CRM_CHUNK);
  uint4 pv[CRM_SLICES][8];
  float zv[CRM_SLICES][RMX / 4];
  const int zt = tid & 63;
  const int zq0 = (tid >> 6) * (RMX / 4);
#pragma unroll
  for (int sl = 0; sl < CRM_SLICES; ++sl) {
    const int r0 = r_begin + sl * CRM_SLICE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = r0 + pr0 + i;
      if (r >= m_rows) r = m_rows - 1;   // loaded and zeroed below
      long long prow;
      if (J.mode == 0) prow = (long long)r * J.ldp;
      else prow = is_out ? J.p_out_off + (long long)r * J.ldp_out : (long long)(ctx_pre_g + r) * J.ldp;
      pv[sl][i] = *reinterpret_cast<const uint4*>(P + prow + pcol);
    }
    const int r = r0 + zt;
    const bool ok = r < r_end;
    const long long tok = ok ? (J.mode == 0 ? r : group_token(a.st, g, r)) : 0;
#pragma unroll
    for (int q = 0; q < RMX / 4; ++q)
      zv[sl][q] = (ok && zq0 + q < J.R) ? J.Z[tok * J.ldz + J.zc0 + zq0 + q] : 0.f;
  }
#pragma unroll
  for (int sl = 0; sl < CRM_SLICES; ++sl) {
    const int r0 = r_begin + sl * CRM_SLICE;
    if (r0 >= r_end) break;   // uniform
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(r0 + pr0 + i < r_end && c_ok)) pv[sl][i] = make_uint4(0, 0, 0, 0);
    if (sl > 0) __syncthreads();   // previous slice fully consumed
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t* c0 = reinterpret_cast<const uint32_t*>(&pv[sl][2 * p]);
        const uint32_t* c1 = reinterpret_cast<const uint32_t*>(&pv[sl][2 * p + 1]);
        const uint32_t lo = (c0[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        const uint32_t hi = (c1[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        w[p] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(&Ps[(pc + j) * LD + pr0]) = make_uint4(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int q = 0; q < RMX / 4; ++q) Zs[(zq0 + q) * LD + zt] = f2bf(zv[sl][q]);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < CRM_SLICE / 32; ++ks) {
      bf16x8_t_s bfr[RMX / 16];
#pragma unroll
      for (int j = 0; j < RMX / 16; ++j)
        if (j < nq16)
          bfr[j] = *reinterpret_cast<const bf16x8_t_s*>(&Zs[(16 * j + (lane & 15)) * LD + ks * 32 + 8 * (lane >> 4)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t_s af = *reinterpret_cast<const bf16x8_t_s*>(
            &Ps[(64 * wave + 16 * i + (lane & 15)) * LD + ks * 32 + 8 * (lane >> 4)]);
#pragma unroll
        for (int j = 0; j < RMX / 16; ++j)
          if (j < nq16) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  float* dst = J.part + poff + (long long)ch * N * J.RM;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int n = n0 + 64 * wave + 16 * i + 4 * (lane >> 4) + e4;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < RMX / 16; ++j)
        if (j < nq16) dst[(long long)n * J.RM + 16 * j + (lane & 15)] = acc[i][j][e4];
    }
}

// Batched finishes.  A dense job (mode-0 partials, nchunk chunks of N x RM)
// writes out1 from partial columns [0, r1) and, if out2 is set, out2 from
// [off2, off2 + r2); a scatter job (mode-1 partials) writes, for every channel
// c < N and q < r1, the sum over the groups that hold c (context groups
// through the inverse map inv, the output group always) into out1.  Outputs
// are [N, r] or, transposed, [r, N], times scale.  One thread per (job, c, q).
// (Issuing every group's loads in one predicated batch, 8 groups x 8 chunks,
// measured slower: the address arithmetic of the idle slots costs more issue
// time than the saved round trips.)
struct FbJob {
  int kind;                 // 0 dense, 1 scatter
  const float* part; int RM, N, kidx, nchunk;
  const int* inv;
  float* out1; int r1, t1;
  float* out2; int r2, t2, off2;
  float scale;
  long long item0;
};

struct FbArgs {
  SeqTab st;
  int njobs;
  long long nitems;
  FbJob job[CB_MAXJOBS];
};

static __global__ void finish_batch_kernel(const FbArgs a) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.nitems) return;
  int jb = 0;
  while (jb + 1 < a.njobs && a.job[jb + 1].item0 <= i) ++jb;
  const FbJob& J = a.job[jb];
  const long long e = i - J.item0;
  if (J.kind == 0) {
    const int n = (int)(e / J.RM), q = (int)(e % J.RM);
    float* out = nullptr; int oq = 0, tr = 0, rr = 0;
    if (q < J.r1) { out = J.out1; oq = q; tr = J.t1; rr = J.r1; }
    else if (J.out2 && q >= J.off2 && q < J.off2 + J.r2) { out = J.out2; oq = q - J.off2; tr = J.t2; rr = J.r2; }
    if (!out) return;
    // chunk loads issued 8 at a time, added in chunk order
    float s = 0.f;
    for (int c0 = 0; c0 < J.nchunk; c0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < J.nchunk) v[u] = J.part[((long long)(c0 + u) * J.N + n) * J.RM + q];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < J.nchunk) s += v[u];
    }
    s *= J.scale;
    if (tr) out[(long long)oq * J.N + n] = s;
    else out[(long long)n * rr + oq] = s;
  } else {
    const int c = (int)(e / J.r1), q = (int)(e % J.r1);
    float s = 0.f;
    long long off = 0;
    for (int g = 0; g <= a.st.nseq; ++g) {
      const int rows = group_rows(a.st, g);
      const int cols = g < a.st.nseq ? J.kidx : J.N;
      const int nch = (rows + CRM_CHUNK - 1) / CRM_CHUNK;
      const int pos = g < a.st.nseq ? J.inv[(long long)g * J.N + c] : c;
      if (pos >= 0) {
        for (int c0 = 0; c0 < nch; c0 += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (c0 + u < nch) v[u] = J.part[off + ((long long)(c0 + u) * cols + pos) * J.RM + q];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (c0 + u < nch) s += v[u];
        }
      }
      off += (long long)nch * cols * J.RM;
    }
    s *= J.scale;
    if (J.t1) J.out1[(long long)q * J.N + c] = s;
    else J.out1[(long long)c * J.r1 + q] = s;
  }
}

// Dense finish: out[n, q] (or out[q, n] when transposed) = scale * sum_chunks part.
// Two outputs may take column ranges [0, r1) and [off2, off2 + r2) of the part.
struct FinishArgs {
  const float* part; int nchunk; int N; int RM;
  float* out1; int r1; int t1;
  float* out2; int r2; int t2; int off2;
  float scale;
};
static __global__ void finish_dense_kernel(const FinishArgs a) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)a.N * a.RM;
  if (i >= total) return;
  const int n = (int)(i / a.RM), q = (int)(i % a.RM);
  float* out = nullptr; int oq = 0, tr = 0, rr = 0;
  if (q < a.r1) { out = a.out1; oq = q; tr = a.t1; rr = a.r1; }
  else if (a.out2 && q >= a.off2 && q < a.off2 + a.r2) { out = a.out2; oq = q - a.off2; tr = a.t2; rr = a.r2; }
  if (!out) return;
  float s = 0.f;
  for (int c = 0; c < a.nchunk; ++c) s += a.part[((long long)c * a.N + n) * a.RM + q];
  s *= a.scale;
  if (tr) out[(long long)oq * a.N + n] = s;
  else out[(long long)n * rr + oq] = s;
}

// Scatter finish over channel sets: for channel c (of Nfull) and q < r,
//   out = scale * sum over groups g containing c of sum_chunks part_g[pos_g(c)][q]
// with pos from the inverse maps (context groups) or c itself (output group).
struct FinishScatterArgs {
  SeqTab st;
  const float* part; int RM; int Nfull; int kidx;
  const int* inv;                         // [nseq][Nfull], -1 = not selected
  int chunk_count[SL_MAX_SEQS + 1];
  long long part_off[SL_MAX_SEQS + 1];
  float* out; int r; int transposed;      // [Nfull, r] or [r, Nfull]
  float scale;
};
static __global__ void finish_scatter_kernel(const FinishScatterArgs a) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)a.Nfull * a.r) return;
  const int c = (int)(i / a.r), q = (int)(i % a.r);
  float s = 0.f;
  for (int g = 0; g <= a.st.nseq; ++g) {
    int pos, n;
    if (g < a.st.nseq) { pos = a.inv[(long long)g * a.Nfull + c]; n = a.kidx; }
    else { pos = c; n = a.Nfull; }
    if (pos < 0) continue;
    for (int ch = 0; ch < a.chunk_count[g]; ++ch)
      s += a.part[a.part_off[g] + ((long long)ch * n + pos) * a.RM + q];
  }
  s *= a.scale;
  if (a.transposed) a.out[(long long)q * a.Nfull + c] = s;
  else a.out[(long long)c * a.r + q] = s;
}

// ===========================================================================
// Packing of the LoRA operands in one launch.  Each job writes a whole
// destination region (padding included):
//   type 0:  dst[r][c] = src block placed at (row_off, col_off), 0 elsewhere;
//            the block is src[r][c] or, transposed, src[c][r]
//   type 1:  per context group g: dst[g][q][p] = src(q, idx[g][p]) for q < src_rows,
//            p < k, 0 elsewhere; src(q, c) = src[q*lds + c] or, transposed, src[c*lds + q]
//   type 2:  int32 dst[p] = p for p < cols (identity rows)
//   type 3:  int32 inverse map of an ascending channel set, per context group g:
//            dst[g][c] = position of channel c in idx[g][0..k), or -1, c < cols
// ===========================================================================
constexpr int PK_MAXJOBS = 16;

struct PackJob {
  int type;
  void* dst; long long ldd, gstride;
  int rows, cols, row_off, col_off;
  const void* src; long long lds;
  int src_rows, src_cols, tr;
  const int* idx; int k, nseq;
};

struct PackArgs {
  int njobs;
  long long start[PK_MAXJOBS + 1];
  PackJob job[PK_MAXJOBS];
};

// One thread per 8 consecutive destination elements of a row (an item): the
// 8 source loads are independent, and a whole aligned item goes out as one
// 16-byte store (two for fp32).  Inverse maps take one element per item: each
// is a binary search, a chain of dependent loads.
template <typename T>
__global__ void pack_kernel(const PackArgs a) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.start[a.njobs]) return;
  int j = 0;
  while (j + 1 < a.njobs && a.start[j + 1] <= i) ++j;
  const PackJob& b = a.job[j];
  const long long e = i - a.start[j];
  const int per = b.type == 3 ? 1 : 8;         // elements per item
  const int cg = (b.cols + per - 1) / per;     // items per destination row
  const int c0 = (int)(e % cg) * per;
  const long long row = e / cg;                // type 1: g * rows + q; type 3: g
  const int n = b.cols - c0 < per ? b.cols - c0 : per;
  if (b.type == 2) {
    int* d = reinterpret_cast<int*>(b.dst) + c0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < n) d[u] = c0 + u;
    return;
  }
  if (b.type == 3) {
    const int* set = b.idx + row * b.k;
    const int c = c0;
    int lo = 0, hi = b.k;
    while (lo < hi) { const int mid = (lo + hi) >> 1; if (set[mid] < c) lo = mid + 1; else hi = mid; }
    reinterpret_cast<int*>(b.dst)[row * b.cols + c] = (lo < b.k && set[lo] == c) ? lo : -1;
    return;
  }
  const T* src = reinterpret_cast<const T*>(b.src);
  T zero;
  stv<T>(&zero, 0, 0.f);
  alignas(16) T v[8];
  T* d;
  if (b.type == 0) {
    const int sr = (int)row - b.row_off;
    const bool rok = sr >= 0 && sr < b.src_rows;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sc = c0 + u - b.col_off;
      v[u] = (u < n && rok && sc >= 0 && sc < b.src_cols)
                 ? (b.tr ? src[(long long)sc * b.lds + sr] : src[(long long)sr * b.lds + sc])
                 : zero;
    }
    d = reinterpret_cast<T*>(b.dst) + row * b.ldd + c0;
  } else {
    const int q = (int)(row % b.rows);
    const long long g = row / b.rows;
    const int* set = b.idx + g * b.k;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = c0 + u;
      T x = zero;
      if (u < n && q < b.src_rows && p < b.k) {
        const int c = set[p];
        x = b.tr ? src[(long long)c * b.lds + q] : src[(long long)q * b.lds + c];
      }
      v[u] = x;
    }
    d = reinterpret_cast<T*>(b.dst) + g * b.gstride + (long long)q * b.ldd + c0;
  }
  if (n == 8 && (reinterpret_cast<uintptr_t>(d) & 15) == 0) {
#pragma unroll
    for (int h = 0; h < (int)sizeof(T) * 8 / 16; ++h)
      reinterpret_cast<uint4*>(d)[h] = reinterpret_cast<const uint4*>(v)[h];
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < n) d[u] = v[u];
  }
}

// ===========================================================================
// Row layout jobs over the token layout, one launch for several buffers; one
// workgroup per (job, row), 8 consecutive elements per thread and pass.
//   LJ_ZERO:   token-major [T, ld] buffer, context rows, columns [0, n) := 0
//   LJ_GATHER: compact copy of the selected columns of the context rows,
//              dst[ctx_pre[b] + t][p] = src[b*L + t][idx[b][p]] for p < n (= k);
//              the source row (nsrc columns) is first staged in LDS with
//              16-byte loads when it fits (stage = 1)
//   LJ_ROWS:   compact copy of the output rows, dst[i][c] = src[tok(i)][c], c < n
// `vec` (set by the host when row strides are multiples of 8 elements and the
// bases 16-byte aligned) selects 16-byte accesses.
// ===========================================================================
enum { LJ_ZERO = 0, LJ_GATHER = 1, LJ_ROWS = 2 };
constexpr int LJ_MAXJOBS = 12;
constexpr int LJ_THREADS = 256;

struct LayJob {
  int type, n, vec, nsrc, stage;
  void* dst; long long ldd;
  const void* src; long long lds;
  const int* idx;
  int row0;                 // first workgroup of the job
};

struct LayArgs {
  SeqTab st;
  int njobs, nrows;
  LayJob job[LJ_MAXJOBS];
};

// Token row of context row r (rows of all context groups, concatenated).
__device__ inline int ctx_token(const SeqTab& st, int r, int& b) {
  int lo = 0, hi = st.nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (st.ctx_pre[mid] <= r) lo = mid; else hi = mid - 1;
  }
  b = lo;
  return lo * st.L + (r - st.ctx_pre[lo]);
}

template <typename T>
__global__ void __launch_bounds__(LJ_THREADS) layout_kernel(const LayArgs a) {
  using R = typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type;
  constexpr int W = 8 * sizeof(T) / 16;   // 16-byte words per 8 elements
  extern __shared__ __attribute__((aligned(16))) unsigned char lrow[];
  const int tid = threadIdx.x;
  int j = 0;
  while (j + 1 < a.njobs && a.job[j + 1].row0 <= (int)blockIdx.x) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const LayJob& job = a.job[j];
  const int r = blockIdx.x - job.row0;
  union Buf { R v[8]; uint4 w[W]; };
  if (job.type == LJ_ZERO) {
    int b;
    R* dst = reinterpret_cast<R*>(job.dst) + (long long)ctx_token(a.st, r, b) * job.ldd;
    for (int c0 = tid * 8; c0 < job.n; c0 += LJ_THREADS * 8) {
      const int cnt = min(8, job.n - c0);
      if (job.vec && cnt == 8) {
#pragma unroll
        for (int q = 0; q < W; ++q) reinterpret_cast<uint4*>(dst + c0)[q] = make_uint4(0, 0, 0, 0);
      } else {
        for (int q = 0; q < cnt; ++q) dst[c0 + q] = (R)0;
      }
    }
  } else if (job.type == LJ_ROWS) {
    const R* src = reinterpret_cast<const R*>(job.src) + (long long)out_token(a.st, r) * job.lds;
    R* dst = reinterpret_cast<R*>(job.dst) + (long long)r * job.ldd;
    for (int c0 = tid * 8; c0 < job.n; c0 += LJ_THREADS * 8) {
      const int cnt = min(8, job.n - c0);
      if (job.vec && cnt == 8) {
#pragma unroll
        for (int q = 0; q < W; ++q) reinterpret_cast<uint4*>(dst + c0)[q] = reinterpret_cast<const uint4*>(src + c0)[q];
      } else {
        for (int q = 0; q < cnt; ++q) dst[c0 + q] = src[c0 + q];
      }
    }
  } else {
    int b;
    const R* src = reinterpret_cast<const R*>(job.src) + (long long)ctx_token(a.st, r, b) * job.lds;
    const int* sel = job.idx + (long long)b * job.n;
    R* dst = reinterpret_cast<R*>(job.dst) + (long long)r * job.ldd;
    const R* from = src;
    if (job.stage) {   // uniform: the whole source row into LDS (nsrc is a multiple of 8)
      R* rowl = reinterpret_cast<R*>(lrow);
      for (int c0 = tid * 8; c0 < job.nsrc; c0 += LJ_THREADS * 8) {
#pragma unroll
        for (int q = 0; q < W; ++q) reinterpret_cast<uint4*>(rowl + c0)[q] = reinterpret_cast<const uint4*>(src + c0)[q];
      }
      __syncthreads();
      from = rowl;
    }
    // the set row starts 16-byte aligned when b*k is a multiple of 4 (idx itself is aligned)
    const bool sel_vec = ((reinterpret_cast<uintptr_t>(sel) & 15) == 0);
    for (int p0 = tid * 8; p0 < job.n; p0 += LJ_THREADS * 8) {
      const int cnt = min(8, job.n - p0);
      Buf buf;
      int c[8];
      if (sel_vec && cnt == 8) {
        const int4 i0 = reinterpret_cast<const int4*>(sel + p0)[0];
        const int4 i1 = reinterpret_cast<const int4*>(sel + p0)[1];
        c[0] = i0.x; c[1] = i0.y; c[2] = i0.z; c[3] = i0.w;
        c[4] = i1.x; c[5] = i1.y; c[6] = i1.z; c[7] = i1.w;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) c[q] = q < cnt ? sel[p0 + q] : 0;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) buf.v[q] = q < cnt ? from[c[q]] : (R)0;
      if (job.vec && cnt == 8) {
#pragma unroll
        for (int q = 0; q < W; ++q) reinterpret_cast<uint4*>(dst + p0)[q] = buf.w[q];
      } else {
        for (int q = 0; q < cnt; ++q) dst[p0 + q] = buf.v[q];
      }
    }
  }
}

// Output-group split-K reduction: out[tok(i), n] = sum_s part[s][i][n].
template <typename T>
__global__ void splitk_reduce_kernel(const SeqTab st, const float* part, int ks, int N, T* out,
                                     long long ldo) {
  // one thread per 4 consecutive columns (N is a multiple of 8); the pieces'
  // loads are issued 8 at a time and added in piece order
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int N4 = N >> 2;
  if (i >= (long long)st.T_out * N4) return;
  const int row = (int)(i / N4), n = (int)(i % N4) * 4;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < ks; j0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < ks) v[u] = *reinterpret_cast<const float4*>(part + ((long long)(j0 + u) * st.T_out + row) * N + n);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < ks) { s[0] += v[u].x; s[1] += v[u].y; s[2] += v[u].z; s[3] += v[u].w; }
  }
  T* o = out + (long long)out_token(st, row) * ldo + n;
#pragma unroll
  for (int q = 0; q < 4; ++q) stv<T>(o, q, s[q]);
}

// kv-channel set -> query-channel set: every query head of a group keeps the
// kv head's selected dims.  idx_q[b] has k*G entries in ascending order.
// Thread per (sequence, kv position p, head offset j): kv channel c = (gk, d)
// becomes q channel (gk*G + j, d) at position lo*G + j*cnt + (p - lo), where
// [lo, lo+cnt) are the positions of kv head gk's channels in the ascending set.
__device__ inline int lower_bound_i(const int* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) { const int mid = (lo + hi) >> 1; if (a[mid] < v) lo = mid + 1; else hi = mid; }
  return lo;
}
static __global__ void expand_kv_kernel(const int* idx_kv, int k, int nseq, int group, int head_dim,
                                 int* idx_q) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)nseq * k * group) return;
  const int b = (int)(i / ((long long)k * group));
  const int rem = (int)(i % ((long long)k * group));
  const int p = rem / group, j = rem % group;
  const int* in = idx_kv + (long long)b * k;
  const int c = in[p];
  const int gk = c / head_dim, d = c % head_dim;
  const int lo = lower_bound_i(in, k, gk * head_dim);
  const int hi = lower_bound_i(in, k, (gk + 1) * head_dim);
  const int cnt = hi - lo;
  idx_q[(long long)b * k * group + (long long)lo * group + (long long)j * cnt + (p - lo)] =
      (gk * group + j) * head_dim + d;
}

}  // namespace sl
