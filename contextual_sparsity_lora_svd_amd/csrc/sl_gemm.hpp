// Grouped gather-GEMM for gfx950 (CDNA4): the dense contractions of the sparse
// LoRA layers, restricted per sequence to that sequence's selected channels.
//
// SparseLoRA article §六 (structured channel sparsity so that GPUs see real
// speedups) and §七 (careful slicing of the sparse weights and compute order):
// every selected channel is a whole weight row, so a gathered tile is a set of
// contiguous 128-byte row segments, staged through LDS and fed to the matrix
// cores.  Context rows of sequence b form group b (its own channel set); the
// output rows of the whole batch form one dense group (all channels).
//
// C[m, n] = sum over K segments s of  A_s[row(m), k] * B_s(n, k)
//   MODE_NG (gather along N): B_s(n, k) = Bmat_s[ch(n), k]   (rows K-contiguous)
//   MODE_KG (gather along K): B_s(n, k) = Bmat_s[ch(k), n]   (rows N-contiguous;
//           the tile is transposed on its way into LDS)
// A K segment is a main contraction (X·W, H·Wd^T, ...) or a LoRA term whose A
// operand is the low-rank activation z and whose B operand the other factor,
// so LoRA runs inside the same tiles as the frozen weight.
//
// Tile 128 x 256 x BK, 256 threads = 4 waves in a 2 x 2 grid, each wave a
// 64 x 128 block of 32x32 MFMA accumulators.  bf16: v_mfma_f32_32x32x16_bf16,
// BK = 64.  fp32: v_mfma_f32_32x32x2_f32 (true fp32), BK = 32.  Global loads of
// tile k+1 are in flight in registers while tile k is consumed from LDS.
#pragma once

#include "sl_common.hpp"

namespace sl {

enum { MODE_NG = 0, MODE_KG = 1 };
enum { EPI_SWIGLU = 0, EPI_DSWIGLU = 1, EPI_TOKEN = 2, EPI_SCATTER = 3 };

constexpr int G_BM = 128;
constexpr int G_BN = 256;
constexpr int G_THREADS = 256;
constexpr int G_MAXSEG = 4;

struct GSeg {
  const void* A;       // A operand base
  long long lda;       // token mode: row stride; compact mode: context-region row stride
  long long lda_out;   // compact mode: output-region row stride
  long long a_out_off; // compact mode: element offset of the output region
  int a_tok;           // 1: A row = token row; 0: compact row of the group
  const void* B;       // B operand (gate half in dual mode)
  const void* B2;      // dual mode: up half
  long long ldb;
  int b_gather;        // 1: B row = a channel number; 0: its position
  int K;               // > 0 fixed length; <= 0: the segment's channel count
  // KG segments with K <= 0: channel set of the segment (context group g uses
  // idx + g*kidx, kidx channels; the output group uses all n_out channels).
  const int* idx; int kidx; int n_out;
};

struct GemmArgs {
  SeqTab st;
  int ngroups;                          // nseq + 1
  int tile_start[SL_MAX_SEQS + 2];
  // NG: output channel set (context group g: idx + g*kidx; output group: all n_out)
  const int* idx;
  int kidx;
  int n_out;
  int N;                                // KG: output columns
  int nseg;
  GSeg seg[G_MAXSEG];
  int ksplit_out;                       // KG: K splits of the output group
  void* o0; void* o1; void* o2;
  const void* i0; const void* i1;
  long long ldo;                        // TOKEN / SCATTER output row stride
  long long ldc_ctx, ldc_out, c_out_off;  // compact geometry of o*/i* buffers
  float* part;                          // KG split partials [ksplit][T_out][N]
};

template <typename T> struct GTraits;
template <> struct GTraits<bf16> {
  static constexpr int VEC = 8;       // elements per 16-byte chunk
  static constexpr int BK = 64;
  static constexpr int KSTEP = 16;    // K per MFMA
};
template <> struct GTraits<float> {
  static constexpr int VEC = 4;
  static constexpr int BK = 32;
  static constexpr int KSTEP = 2;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct alignas(16) Chunk { uint32_t w[4]; };

__device__ inline Chunk zero_chunk() { Chunk c; c.w[0] = c.w[1] = c.w[2] = c.w[3] = 0u; return c; }

__device__ inline Chunk load_chunk(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  Chunk c; c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  return c;
}

// Zero the elements of a chunk at or beyond `valid` (0..VEC).
template <typename T>
__device__ inline void mask_chunk(Chunk& c, int valid) {
  if (valid >= GTraits<T>::VEC) return;
  if (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= valid) c.w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e >= valid) c.w[e] = 0u;
  }
}

__device__ inline float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ inline float sigmoid_exact(float x) { return 1.0f / (1.0f + expf(-x)); }

template <typename T, int MODE, int EPI, bool DUAL>
__global__ void __launch_bounds__(G_THREADS, 2)
gather_gemm_kernel(const GemmArgs args) {
  constexpr int VEC = GTraits<T>::VEC;
  constexpr int BK = GTraits<T>::BK;
  constexpr int KSTEP = GTraits<T>::KSTEP;
  constexpr int LDS_LD = BK + VEC;          // padded row: 144 bytes
  constexpr int BNC = DUAL ? G_BN / 2 : G_BN; // output columns (channels) per tile
  constexpr int KR = BK / 8;                // KG: k-rows per thread

  __shared__ __attribute__((aligned(16))) T As[G_BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) T Bs[G_BN * LDS_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- locate the tile --------------------------------------------------
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  int g = 0;
  while (g + 1 < args.ngroups && args.tile_start[g + 1] <= tile) ++g;
  g = __builtin_amdgcn_readfirstlane(g);
  const int t_in = tile - args.tile_start[g];
  const bool is_out = (g == args.st.nseq);
  const int m_rows = group_rows(args.st, g);
  const int ctx_pre_g = is_out ? 0 : args.st.ctx_pre[g];
  const int nch = is_out ? args.n_out : args.kidx;
  const int* gidx = is_out ? nullptr : args.idx + (long long)g * args.kidx;
  const int ntm = (m_rows + G_BM - 1) / G_BM;
  int ntn, nks;
  if (MODE == MODE_NG) { ntn = (nch + BNC - 1) / BNC; nks = 1; }
  else { ntn = (args.N + G_BN - 1) / G_BN; nks = is_out ? args.ksplit_out : 1; }
  const int mt = t_in % ntm;
  const int nt = (t_in / ntm) % ntn;
  const int ks = t_in / (ntm * ntn);
  const int m0 = mt * G_BM;
  const int n0 = nt * BNC;

  // ---- K-tile range (all segments, then this split's share) ---------------
  auto seg_len = [&](int s) -> int {
    const GSeg& q = args.seg[s];
    return q.K > 0 ? q.K : (is_out ? q.n_out : q.kidx);
  };
  int total_kt = 0;
  for (int s = 0; s < args.nseg; ++s) total_kt += (seg_len(s) + BK - 1) / BK;
  const int kt_begin = (int)((long long)total_kt * ks / nks);
  const int kt_end = (int)((long long)total_kt * (ks + 1) / nks);
  // ---- per-thread load geometry ------------------------------------------
  // A: 4 chunks per thread, rows (tid>>3) + 32 i, chunk column tid & 7.
  // B (NG): 8 chunks per thread, rows (tid>>3) + 32 i; in dual mode rows
  //         [0, BNC) come from the gate weight and [BNC, 2 BNC) from the up weight.
  // B (KG): k-rows (tid&7)*KR .. +KR, n-columns (tid>>3)*8 .. +8.
  // Loads are unconditional (addresses clamped into the operands); elements
  // past a segment's K or the N edge are zeroed when the tile is stored to LDS,
  // so no wait follows a load inside the prefetch.  Segment-dependent row
  // offsets live in registers and change only at segment boundaries.
  const int a_row0 = tid >> 3;
  const int a_kc = tid & 7;
  int a_r[4], a_t[4];   // group row and token row of each A row this thread loads
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = m0 + a_row0 + 32 * i;
    if (r >= m_rows) r = m_rows - 1;    // rows past the group are computed and dropped
    a_r[i] = r;
    a_t[i] = group_token(args.st, g, r);
  }
  int b_pos[8];         // NG: channel position of each B row this thread loads
  int b_ch[8];          // NG: its channel number
  if (MODE == MODE_NG) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = n0 + a_row0 + ((32 * i) % BNC);
      if (c >= nch) c = nch - 1;
      b_pos[i] = c;
      b_ch[i] = gidx ? gidx[c] : c;
    }
  }
  const int kg_kr0 = (tid & 7) * KR;
  const int kg_n = (tid >> 3) * 8;
  const bool kg_nok = (n0 + kg_n) < args.N;      // N is a multiple of 8
  const int kg_c0 = kg_nok ? n0 + kg_n : 0;

  Chunk ra[4];
  Chunk rb[8];
  int va = VEC;          // valid elements of this thread's A / N-gather B chunks
  int kg_rv = KR;        // K-gather: valid k-rows of this thread's B rows
  int kg_row[KR];        // K-gather: B rows of the tile being loaded
  int kg_row_next[KR] = {};  // ... and of the tile after it (indices fetched a tile ahead)

  // current segment state (uniform scalars + per-thread offsets)
  int cur_s = 0, cur_kk = 0, cur_K = 0, cur_nkt = 0;
  const T* a_base = nullptr;
  const T* b_base = nullptr;
  const T* b2_base = nullptr;
  long long a_off[4];
  long long b_off[8];
  long long cur_ldb = 0;

  auto enter_seg = [&](int s) {
    s = __builtin_amdgcn_readfirstlane(s);
    const GSeg& sg = args.seg[s];
    cur_s = s;
    cur_K = __builtin_amdgcn_readfirstlane(seg_len(s));
    cur_nkt = (cur_K + BK - 1) / BK;
    a_base = reinterpret_cast<const T*>(sg.A);
    b_base = reinterpret_cast<const T*>(sg.B);
    b2_base = reinterpret_cast<const T*>(DUAL ? sg.B2 : sg.B);
    cur_ldb = sg.ldb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (sg.a_tok) a_off[i] = (long long)a_t[i] * sg.lda;
      else a_off[i] = is_out ? sg.a_out_off + (long long)a_r[i] * sg.lda_out
                             : (long long)(ctx_pre_g + a_r[i]) * sg.lda;
    }
    if (MODE == MODE_NG) {
#pragma unroll
      for (int i = 0; i < 8; ++i) b_off[i] = (long long)(sg.b_gather ? b_ch[i] : b_pos[i]) * sg.ldb;
    }
  };

  // KG: B rows of tile (s, kk) of this thread
  auto kg_rows = [&](int s, int kk, int* rows) {
    s = __builtin_amdgcn_readfirstlane(s);
    const GSeg& sg = args.seg[s];
    const int K = seg_len(s);
    const int* sidx = (sg.b_gather && !is_out) ? sg.idx + (long long)g * sg.kidx : nullptr;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const int kpos = kk * BK + kg_kr0 + i;
      rows[i] = kpos < K ? (sidx ? sidx[kpos] : kpos) : 0;
    }
  };

  // position the segment cursor on K-tile kt_begin
  if (kt_begin < kt_end) {
    int s = 0, kk = kt_begin;
    for (;;) {
      const int nkt = (seg_len(s) + BK - 1) / BK;
      if (s + 1 >= args.nseg || kk < nkt) break;
      kk -= nkt;
      ++s;
    }
    enter_seg(s);
    cur_kk = __builtin_amdgcn_readfirstlane(kk);
    if (MODE == MODE_KG) kg_rows(cur_s, cur_kk, kg_row);
  }

  // issue the global loads of the next K-tile into registers and advance the cursor
  auto load_tile = [&](bool more) {
    while (cur_kk >= cur_nkt) {   // segment boundary (segments may be empty)
      enter_seg(cur_s + 1);
      cur_kk = 0;
    }
    const int k0 = cur_kk * BK;
    const int kcol = k0 + a_kc * VEC;
    va = cur_K - kcol < 0 ? 0 : (cur_K - kcol > VEC ? VEC : cur_K - kcol);
    const int kc = kcol < cur_K ? kcol : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = load_chunk(a_base + a_off[i] + kc);
    if (MODE == MODE_NG) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rb[i] = load_chunk(((DUAL && 32 * i >= BNC) ? b2_base : b_base) + b_off[i] + kc);
    } else {
      const int kr = cur_K - (k0 + kg_kr0);
      kg_rv = kr < 0 ? 0 : (kr > KR ? KR : kr);
#pragma unroll
      for (int i = 0; i < KR; ++i)
#pragma unroll
        for (int h = 0; h < 8 / VEC; ++h)
          rb[i * (8 / VEC) + h] = load_chunk(b_base + (long long)kg_row[i] * cur_ldb + kg_c0 + h * VEC);
      if (more) {   // indices of the following tile
        int s = cur_s, kk = cur_kk + 1;
        while (kk >= (seg_len(s) + BK - 1) / BK && s + 1 < args.nseg) { kk = 0; ++s; }
        kg_rows(s, kk, kg_row_next);
      }
    }
    ++cur_kk;
  };

  auto store_tile = [&]() {
    if (va < VEC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mask_chunk<T>(ra[i], va);
      if (MODE == MODE_NG) {
#pragma unroll
        for (int i = 0; i < 8; ++i) mask_chunk<T>(rb[i], va);
      }
    }
    if (MODE == MODE_KG) {
#pragma unroll
      for (int i = 0; i < KR; ++i)
        if (i >= kg_rv || !kg_nok) {
#pragma unroll
          for (int h = 0; h < 8 / VEC; ++h) rb[i * (8 / VEC) + h] = zero_chunk();
        }
#pragma unroll
      for (int i = 0; i < KR; ++i) kg_row[i] = kg_row_next[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&As[(a_row0 + 32 * i) * LDS_LD + a_kc * VEC]) =
          make_uint4(ra[i].w[0], ra[i].w[1], ra[i].w[2], ra[i].w[3]);
    if (MODE == MODE_NG) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint4*>(&Bs[(a_row0 + 32 * i) * LDS_LD + a_kc * VEC]) =
            make_uint4(rb[i].w[0], rb[i].w[1], rb[i].w[2], rb[i].w[3]);
    } else {
      // transpose KR k-rows x 8 n-values into 8 n-rows x KR k-values
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
        if (sizeof(T) == 2) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const Chunk& c0 = rb[2 * p];
            const Chunk& c1 = rb[2 * p + 1];
            const uint32_t lo = (c0.w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            const uint32_t hi = (c1.w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            w[p] = lo | (hi << 16);
          }
        } else {
#pragma unroll
          for (int p = 0; p < 4; ++p) w[p] = rb[p * 2 + (j >> 2)].w[j & 3];
        }
        *reinterpret_cast<uint4*>(&Bs[(kg_n + j) * LDS_LD + kg_kr0]) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // B-tile row of the first column of accumulator block nb of this wave
  auto brow = [&](int nb) -> int {
    if (DUAL) return (nb < 2) ? (64 * wn + 32 * nb) : (BNC + 64 * wn + 32 * (nb - 2));
    return 128 * wn + 32 * nb;
  };

  if (kt_begin < kt_end) {
    load_tile(kt_begin + 1 < kt_end);
    store_tile();
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const bool more = kt + 1 < kt_end;
      if (more) load_tile(kt + 2 < kt_end);
#pragma unroll
      for (int kstep = 0; kstep < BK / KSTEP; ++kstep) {
        if constexpr (sizeof(T) == 2) {
          bf16x8_t af[2], bfr[4];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            af[mb] = *reinterpret_cast<const bf16x8_t*>(
                &As[(64 * wm + 32 * mb + (lane & 31)) * LDS_LD + kstep * 16 + (lane >> 5) * 8]);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            bfr[nb] = *reinterpret_cast<const bf16x8_t*>(
                &Bs[(brow(nb) + (lane & 31)) * LDS_LD + kstep * 16 + (lane >> 5) * 8]);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
        } else {
          float af[2], bfr[4];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            af[mb] = reinterpret_cast<const float*>(As)[(64 * wm + 32 * mb + (lane & 31)) * LDS_LD +
                                                         kstep * 2 + (lane >> 5)];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            bfr[nb] = reinterpret_cast<const float*>(Bs)[(brow(nb) + (lane & 31)) * LDS_LD +
                                                          kstep * 2 + (lane >> 5)];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
        }
      }
      __syncthreads();
      if (more) {
        store_tile();
        __syncthreads();
      }
    }
  }

  // ---- epilogue -----------------------------------------------------------
  // accumulator element e of block (mb, nb): row 8*(e/4) + 4*(lane/32) + e%4,
  // column lane%32 of the block.
  const long long ldc = is_out ? args.ldc_out : args.ldc_ctx;
  const long long cbase = is_out ? args.c_out_off : (long long)args.st.ctx_pre[g] * args.ldc_ctx;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + 64 * wm + 32 * mb + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (r >= m_rows) continue;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int c = n0 + 64 * wn + 32 * nb + (lane & 31);
          if (c >= nch) continue;
          const float gv = acc[mb][nb][e];
          const float uv = acc[mb][nb + 2][e];
          const float sg = (sizeof(T) == 4) ? sigmoid_exact(gv) : sigmoidf_(gv);
          const long long o = cbase + (long long)r * ldc + c;
          stv<T>(reinterpret_cast<T*>(args.o0), o, gv);
          stv<T>(reinterpret_cast<T*>(args.o1), o, uv);
          stv<T>(reinterpret_cast<T*>(args.o2), o, gv * sg * uv);
        }
      } else if constexpr (EPI == EPI_DSWIGLU) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int c = n0 + 128 * wn + 32 * nb + (lane & 31);
          if (c >= nch) continue;
          const long long o = cbase + (long long)r * ldc + c;
          const float dh = acc[mb][nb][e];
          const float gv = ldv<T>(reinterpret_cast<const T*>(args.i0), o);
          const float uv = ldv<T>(reinterpret_cast<const T*>(args.i1), o);
          const float sg = (sizeof(T) == 4) ? sigmoid_exact(gv) : sigmoidf_(gv);
          stv<T>(reinterpret_cast<T*>(args.o0), o, dh * uv * sg * (1.0f + gv * (1.0f - sg)));
          stv<T>(reinterpret_cast<T*>(args.o1), o, dh * gv * sg);
        }
      } else if constexpr (EPI == EPI_TOKEN) {
        const long long tok = group_token(args.st, g, r);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int c = n0 + 128 * wn + 32 * nb + (lane & 31);
          if (c >= args.N) continue;
          if (is_out && nks > 1)
            args.part[((long long)ks * args.st.T_out + r) * args.N + c] = acc[mb][nb][e];
          else
            stv<T>(reinterpret_cast<T*>(args.o0), tok * args.ldo + c, acc[mb][nb][e]);
        }
      } else {  // EPI_SCATTER: column = the channel number
        const long long tok = group_token(args.st, g, r);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int c = n0 + 128 * wn + 32 * nb + (lane & 31);
          if (c >= nch) continue;
          const int col = gidx ? gidx[c] : c;
          stv<T>(reinterpret_cast<T*>(args.o0), tok * args.ldo + col, acc[mb][nb][e]);
        }
      }
    }
  }
}

// Host side: count tiles per group and launch.
bool timer_on();
void timer_begin(int slot, hipStream_t s);
void timer_end(int slot, hipStream_t s);

template <typename T, int MODE, int EPI, bool DUAL>
hipError_t launch_gather_gemm(GemmArgs& a, hipStream_t stream, int timer_slot) {
  constexpr int BNC = DUAL ? G_BN / 2 : G_BN;
  a.ngroups = a.st.nseq + 1;
  int total = 0;
  for (int g = 0; g < a.ngroups; ++g) {
    a.tile_start[g] = total;
    const bool is_out = g == a.st.nseq;
    const int m = is_out ? a.st.T_out : a.st.ctx[g];
    const int nch = is_out ? a.n_out : a.kidx;
    if (m <= 0 || (MODE == MODE_NG && nch <= 0)) continue;
    const int ntm = (m + G_BM - 1) / G_BM;
    int ntn, nks;
    if (MODE == MODE_NG) { ntn = (nch + BNC - 1) / BNC; nks = 1; }
    else { ntn = (a.N + G_BN - 1) / G_BN; nks = is_out ? a.ksplit_out : 1; }
    total += ntm * ntn * nks;
  }
  a.tile_start[a.ngroups] = total;
  if (total == 0) return hipSuccess;
  timer_begin(timer_slot, stream);
  hipLaunchKernelGGL((gather_gemm_kernel<T, MODE, EPI, DUAL>), dim3(total), dim3(G_THREADS), 0,
                     stream, a);
  const hipError_t e = hipGetLastError();
  timer_end(timer_slot, stream);
  return e;
}

}  // namespace sl
