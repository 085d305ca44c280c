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
// Three tile variants, every wave a 64 x 128 block of 32x32 MFMA accumulators
// (bf16: v_mfma_f32_32x32x16_bf16, BK = 64; fp32: v_mfma_f32_32x32x2_f32, true
// fp32, BK = 32):
//   128 x 256, 4 waves, two workgroups per CU, operands staged through
//     registers (the K-gather B operand of bf16 calls by LDS-DMA), the next
//     K-tile's loads in flight while the current one is consumed from LDS;
//   128 x 512 (wide, N-gather) and 256 x 256 (tall, N- or K-gather), 8 waves,
//     one workgroup per CU, bf16 only: both operands go from memory straight
//     into LDS (LDS-DMA) through two stages.
#pragma once

#include <initializer_list>
#include <type_traits>

#include "sl_common.hpp"

namespace sl {

enum { MODE_NG = 0, MODE_KG = 1 };
enum { EPI_SWIGLU = 0, EPI_DSWIGLU = 1, EPI_TOKEN = 2, EPI_SCATTER = 3 };

#ifndef SL_GEMM_BM
#define SL_GEMM_BM 128      // tile rows (128 or 256)
#endif
constexpr int G_BM = SL_GEMM_BM;
constexpr int G_BM_TALL = 256;  // rows of the tall LDS-DMA tile (K-gather)
constexpr int G_BN = 256;
constexpr int G_THREADS = 256;
constexpr int G_MAXSEG = 4;
constexpr int G_MAXPROB = 3;

struct GSeg {
  const void* A;       // A operand base
  long long lda;       // token mode: row stride; compact mode: context-region row stride
  long long lda_out;   // compact mode: output-region row stride
  long long a_out_off; // compact mode: element offset of the output region
  int a_tok;           // 1: A row = token row; 0: compact row of the group
  const void* B;       // B operand (gate half in dual mode)
  const void* B2;      // dual mode: up half
  long long ldb;
  int b_gather;        // KG: 1: B row = a channel number; 0: its position.  NG: always gathered
  int K;               // > 0 fixed length; <= 0: the segment's channel count
  // KG segments with K <= 0: channel set of the segment (context group g uses
  // idx + g*kidx, kidx channels; the output group uses all n_out channels).
  const int* idx; int kidx; int n_out;
  // bq4 = 1: B (and B2) hold 4-bit codes of a quantized frozen weight, row
  // stride ldb/2 bytes, element 2j of a row in the low nibble of byte j (two's
  // complement), and Bs (B2s) one fp32 scale per 64 elements of a row, row
  // stride ldb/64; the element is code * scale (ldb a multiple of 64).  In
  // multi-problem launches each problem's scales are in GProb::Bs.
  const float* Bs; const float* B2s; int bq4;
};

// One problem of a launch: its channel set, the B operand of each segment, a
// column offset into each segment's A, and its output.  Problems share the
// token layout and every other segment field.
struct GProb {
  const int* idx;                       // NG: context group g uses idx + g*kidx
  int kidx, n_out;
  int swidth;                           // NG scatter: columns of the output rows
  const void* B[G_MAXSEG];
  const float* Bs[G_MAXSEG];            // 4-bit segments (bq4): the scales of B[s]
  int a_col[G_MAXSEG];
  void* o0;
  long long ldo;
};

struct GemmArgs {
  SeqTab st;
  // Tiles run problem by problem, and within a problem group by group
  // (context groups 0..nseq-1, then the output group): flat group
  // p*(nseq+1) + g starts at logical tile tile_start[.].
  int ngroups;                          // nprob * (nseq + 1)
  int tile_start[G_MAXPROB * (SL_MAX_SEQS + 1) + 1];
  // N-gather launches may hold up to G_MAXPROB problems (prob[1..]); a launch
  // that leaves nprob at 0 has one, taken from idx/kidx/n_out/seg[].B/o0/ldo.
  int nprob;
  GProb prob[G_MAXPROB];
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
  int swidth;                           // SCATTER: columns of an output row (n of the channel set)
  long long ldc_ctx, ldc_out, c_out_off;  // compact geometry of o*/i* buffers
  float* part;                          // KG split partials [ksplit][T_out][N]
  const int* iota;                      // KG: 0, 1, 2, ... (rows of ungathered segments)
  // NG: logical tiles [0, rem_start) run whole; every later tile runs as
  // rem_split K pieces (the grid's last, partial round) that write fp32
  // partial tiles [piece][G_BM][tile columns] to rpart for ng_fixup_kernel.
  int ntiles, rem_start, rem_split;
  float* rpart;
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

// 8 consecutive 4-bit codes (element j in bits 4j..4j+3, two's complement)
// times a scale, as 8 bf16 (round to nearest even).  Flipping each nibble's
// sign bit gives u = q + 8 in 0..15; the even and odd nibbles, spread into
// bytes, convert to float one instruction each, and fma(u, s, -8 s) is q * s
// rounded once (-8 s is exact); pairs go to bf16 by the packed conversion.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline Chunk deq8(uint32_t code, float scale) {
  const uint32_t u = code ^ 0x88888888u;
  const uint32_t ev = u & 0x0F0F0F0Fu, od = (u >> 4) & 0x0F0F0F0Fu;
  const float bias = -8.0f * scale;
  Chunk c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2_t f = {__builtin_fmaf((float)((ev >> (8 * j)) & 0xFFu), scale, bias),
                       __builtin_fmaf((float)((od >> (8 * j)) & 0xFFu), scale, bias)};
    c.w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  }
  return c;
}

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

// Store / load N consecutive elements (N a multiple of 8) with 16-byte
// accesses; only the first `valid` (clamped to [0, N]) are touched.  The
// address must be 16-byte aligned when all N are valid.
template <typename T, int N>
__device__ inline void store_row(T* p, const float* v, int valid) {
  if (valid >= N) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int q = 0; q < N / 8; ++q) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t] = (uint32_t)f2bf(v[8 * q + 2 * t]) | ((uint32_t)f2bf(v[8 * q + 2 * t + 1]) << 16);
        *reinterpret_cast<uint4*>(p + 8 * q) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < N / 4; ++q)
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + 4 * q) =
            make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (j < valid) stv<T>(p, j, v[j]);
  }
}

template <typename T, int N>
__device__ inline void load_row(const T* p, float* v, int valid) {
  if (valid >= N) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int q = 0; q < N / 8; ++q) {
        const uint4 u = *reinterpret_cast<const uint4*>(p + 8 * q);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[8 * q + 2 * t] = bf2f((uint16_t)(w[t] & 0xFFFFu));
          v[8 * q + 2 * t + 1] = bf2f((uint16_t)(w[t] >> 16));
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + 4 * q);
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = j < valid ? ldv<T>(p, j) : 0.f;
  }
}

__device__ inline float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ inline float sigmoid_exact(float x) { return 1.0f / (1.0f + expf(-x)); }

#ifndef SL_KG_DMA
#define SL_KG_DMA 1
#endif

// 16-byte chunk swizzles of the KGD LDS tiles.  A rows hold 8 chunks: chunk c
// of row r sits at c ^ kgd_aswz(r), so the 32 rows an A-fragment read touches
// spread over all banks.  B rows (one k, 256 n = 32 chunks) XOR chunk bits 2-4
// with kgd_bswz(k): the 8 k-rows a transposing fragment read touches (k0..k0+3,
// k0+8..k0+11, k0 a multiple of 4) then land in 8 different 64-byte windows.
__device__ inline int kgd_aswz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ inline int kgd_bswz(int k) { return ((k & 3) | ((k >> 1) & 4)) << 2; }
// Wide N-gather tiles hold 64-element (128-byte) rows: 16-byte chunk c of row
// r sits at c ^ wng_swz(r % 16).  The 16 rows one 16-lane phase of a fragment
// read touches (same logical chunk) then fill the 16 bank groups of a 256-byte
// window, and any aligned 8 of them the 8 groups of a 128-byte one.
__device__ inline int wng_swz(int r16) { return (r16 ^ (r16 >> 3)) & 7; }

// A pointer that every lane holds alike, in scalar registers (the base
// operand of the LDS-DMA loads must be scalar).
template <typename P>
__device__ inline const P* uniform_ptr(const P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const P*>(((uint64_t)hi << 32) | lo);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (the LDS-DMA loads issued by inline assembly are not tracked by the
// compiler).  The count field is split: bits 3:0 and 15:14 of the immediate.
template <int N>
__device__ inline void wait_vmcnt_le(int n) {
  if constexpr (N == 0) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  } else {
    if (n >= N) __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
    else wait_vmcnt_le<N - 1>(n);
  }
}
__device__ inline void wait_vmcnt(int n) { wait_vmcnt_le<31>(n); }   // n > 31 waits for 31

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Scatter epilogue of one context row: channels c .. c+7 (positions in the
// row's ascending set gidx of nch channels) take the row's columns
// [gidx[c], gidx[c + 8]) -- from column 0 for c = 0 and up to the row width
// for the set's last 8 -- writing each selected column's value and 0 in every
// other column.  The groups of 8 of a set cover the row exactly once, so the
// unselected columns need no separate zeroing; whole aligned 8-column chunks
// go out as 16-byte stores when `vec` (row 16-byte aligned).
template <typename T>
__device__ inline void scatter_row8(T* row, const int* gidx, int c, int nch, int width, const float* v,
                                    bool vec) {
  if (c >= nch) return;
  const int cnt = nch - c < 8 ? nch - c : 8;
  int cols[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cols[j] = j < cnt ? gidx[c + j] : 0x7FFFFFFF;
  const int lo = c == 0 ? 0 : cols[0];
  const int hi = c + 8 >= nch ? width : gidx[c + 8];
  for (int a0 = lo & ~7; a0 < hi; a0 += 8) {
    // the set's columns are distinct: at most one of the 8 lands on a column
    float w8[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      float val = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) val = cols[j] == a0 + x ? v[j] : val;
      w8[x] = val;
    }
    const int s0 = lo - a0 > 0 ? lo - a0 : 0;
    const int s1 = hi - a0 < 8 ? hi - a0 : 8;
    if (vec && s0 == 0 && s1 == 8) {
      store_row<T, 8>(row + a0, w8, 8);
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x)
        if (x >= s0 && x < s1) stv<T>(row, a0 + x, w8[x]);
    }
  }
}

template <typename T, int MODE, int EPI, bool DUAL, int BM, int WN, bool QB>
__global__ void __launch_bounds__((WN == 4 || BM > 128) ? 512 : G_THREADS,
                                  (WN == 4 || BM > 128) ? 1 : 2)
gather_gemm_kernel(const GemmArgs args) {
  // QB: segments with bq4 set read their B operand as 4-bit codes and scales
  // (bf16 only, register-staged tiles), dequantized on the way into LDS.
  // WN = 2, BM = 128: 128 x 256 tile, 4 waves in a 2 x 2 grid of 64 x 128
  //   blocks, two workgroups per CU, operands staged through registers
  //   (K-gather bf16: B by LDS-DMA).
  // WN = 4 (wide N-gather, bf16): 128 x 512 tile, 8 waves in a 2 x 4 grid of
  //   64 x 128 blocks, one workgroup per CU.  Both operands go from memory
  //   straight into LDS (LDS-DMA) through two stages of 64-element K-tiles, so
  //   no register staging or LDS store phase remains, and the tile moves 17 %
  //   fewer operand bytes per MFMA than two 128 x 256 tiles.
  // WN = 2, BM = 256 (tall, bf16, N-gather or K-gather): 256 x 256 tile, 8
  //   waves in a 4 x 2 grid of 64 x 128 blocks, one workgroup per CU, both
  //   operands by LDS-DMA through the wide tile's two-stage loop (2 x 64 KB
  //   stages).  A CU moves 64 KB per K-tile for 256 x 256 outputs, against
  //   80 KB for a 128 x 512 tile and 2 x 48 KB for two 128 x 256 workgroups.
  constexpr bool TALL = BM > 128;           // tall: 8 waves in a 4 x 2 grid
  constexpr bool WIDE = WN == 4 || TALL;
  static_assert(BM == 128 || BM == G_BM_TALL, "tile rows: 128 or 256");
  static_assert(!WIDE || (sizeof(T) == 2 && !QB && (WN == 4 ? MODE == MODE_NG && BM == 128 : WN == 2)),
                "LDS-DMA tiles: bf16, wide N-gather 128 x 512 or tall 256 x 256");
  static_assert(!QB || (!WIDE && sizeof(T) == 2), "quantized B: bf16 register-staged tiles");
  constexpr int NWAVE = (WN == 4 || TALL) ? 8 : 4;   // waves per workgroup
  constexpr int WMROWS = NWAVE / WN;        // wave rows of the wave grid
  constexpr int BN_T = 128 * WN;            // B rows (accumulator columns) per tile
  constexpr int VEC = GTraits<T>::VEC;
  constexpr int BK = GTraits<T>::BK;
  constexpr int KSTEP = GTraits<T>::KSTEP;
  constexpr int LDS_LD = BK + VEC;          // padded row: 144 bytes
  constexpr int BNC = DUAL ? BN_T / 2 : BN_T; // output columns (channels) per tile
  constexpr int W_ROWB = 2 * BK;            // wide: bytes of a staged row (128)
  constexpr int W_STG = (BM + BN_T) * W_ROWB;   // wide: bytes per stage (A rows, then B rows)
  constexpr int KR = BK / 8;                // KG: k-rows per thread
  constexpr int WM = BM / WMROWS;           // wave tile rows
  constexpr int MB = WM / 32;               // 32-row accumulator blocks per wave
  constexpr int ACH = BM / 32;              // A chunks per thread (register staging)

  // K-gather in bf16 (KGD): the gathered B rows go from memory straight into
  // LDS (global_load_lds) as [k row][n] tiles in two stages, and the matrix
  // cores read them with transposing LDS reads; A is staged through registers
  // into an unpadded tile with XOR-swizzled 16-byte chunks.  Two workgroups
  // then fill the CU's 160 KB of LDS exactly.  Otherwise both operands are
  // staged through registers into padded [row][k] tiles.
  // (A 4-bit B takes the register path: its dequantized tile is transposed
  // on the way into LDS.)
  constexpr bool KGD = SL_KG_DMA && MODE == MODE_KG && sizeof(T) == 2 && BM == 128 && !QB && !WIDE;
  constexpr int A_LD = KGD ? BK : LDS_LD;   // A tile row stride (elements)
  constexpr int B_STAGE = BK * G_BN * (int)sizeof(T);   // KGD: bytes per B stage
  constexpr int EP_LD = 64 + 4;             // epilogue staging row (floats)
  constexpr int SMEM_TILES = WIDE ? 2 * W_STG
                             : KGD ? BM * A_LD * (int)sizeof(T) + 2 * B_STAGE
                                   : (BM + G_BN) * LDS_LD * (int)sizeof(T);
  constexpr int SMEM = SMEM_TILES + (KGD || WIDE ? 0 : 64 * (int)sizeof(int));
  static_assert(NWAVE * 32 * EP_LD * 4 <= SMEM_TILES, "epilogue staging must fit in the tile buffers");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  // K-gather (register path): B rows of the next tile, published by wave 0
  int* krow_s = reinterpret_cast<int*>(smem + SMEM_TILES);
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + BM * LDS_LD;
  unsigned char* Bst0 = smem + BM * A_LD * (int)sizeof(T);   // KGD: B stage 0 (stage 1 follows)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = __builtin_amdgcn_readfirstlane(wave / WN);
  const int wn = __builtin_amdgcn_readfirstlane(wave % WN);

  // ---- locate the tile --------------------------------------------------
  const bool split_grid = MODE == MODE_NG && args.rem_split > 1;
  int tile, rks = 0, rnks = 1;
  if (split_grid && (int)blockIdx.x >= args.rem_start) {
    const int p = blockIdx.x - args.rem_start;
    tile = args.rem_start + p / args.rem_split;
    rks = p % args.rem_split;
    rnks = args.rem_split;
  } else {
    tile = xcd_remap(blockIdx.x, split_grid ? args.rem_start : (int)gridDim.x);
  }
  int g, pid, mt, nt, ks;
  {
    // flat group: the last one starting at or before the tile (empty groups
    // start where the next one does)
    int gg = 0;
    {
      int hi = args.ngroups - 1;
      while (gg < hi) {
        const int mid = (gg + hi + 1) >> 1;
        if (args.tile_start[mid] <= tile) gg = mid; else hi = mid - 1;
      }
    }
    gg = __builtin_amdgcn_readfirstlane(gg);
    const int t_in = tile - args.tile_start[gg];
    pid = gg / (args.st.nseq + 1);
    g = gg - pid * (args.st.nseq + 1);
    const int m_g = group_rows(args.st, g);
    const int ntm_g = (m_g + BM - 1) / BM;
    const GProb& q = args.prob[pid];
    const int nch_g = g == args.st.nseq ? q.n_out : q.kidx;
    const int ntn_g = MODE == MODE_NG ? (nch_g + BNC - 1) / BNC : (args.N + G_BN - 1) / G_BN;
    mt = t_in % ntm_g;
    nt = (t_in / ntm_g) % ntn_g;
    ks = MODE == MODE_NG ? rks : t_in / (ntm_g * ntn_g);
  }
  mt = __builtin_amdgcn_readfirstlane(mt);
  nt = __builtin_amdgcn_readfirstlane(nt);
  ks = __builtin_amdgcn_readfirstlane(ks);
  const GProb& pr = args.prob[pid];
  const bool is_out = (g == args.st.nseq);
  const int m_rows = __builtin_amdgcn_readfirstlane(group_rows(args.st, g));
  const int ctx_pre_g = is_out ? 0 : args.st.ctx_pre[g];
  const int nch = is_out ? pr.n_out : pr.kidx;
  const int* gidx = is_out ? nullptr : pr.idx + (long long)g * pr.kidx;
  int nks;
  if (MODE == MODE_NG) nks = rnks;
  else nks = is_out ? args.ksplit_out : 1;
  const int m0 = mt * BM;
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
  const int nkt = kt_end - kt_begin;

  f32x16_t acc[MB][4];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // B-tile row of the first column of accumulator block nb of this wave
  auto brow = [&](int nb) -> int {
    if (DUAL) return (nb < 2) ? (64 * wn + 32 * nb) : (BNC + 64 * wn + 32 * (nb - 2));
    return 128 * wn + 32 * nb;
  };

  if constexpr (!WIDE) {
  // ---- per-thread load geometry ------------------------------------------
  // A: ACH chunks per thread, rows (tid>>3) + 32 i, chunk column tid & 7.
  // B (NG): 8 chunks per thread, rows (tid>>3) + 32 i; in dual mode rows
  //         [0, BNC) come from the gate weight and [BNC, 2 BNC) from the up weight.
  // B (KG): k-rows (tid&7)*KR .. +KR, n-columns (tid>>3)*8 .. +8.
  // Loads are unconditional (addresses clamped into the operands); elements
  // past a segment's K or the N edge are zeroed when the tile is stored to LDS,
  // so no wait follows a load inside the prefetch.  Segment-dependent row
  // offsets live in registers and change only at segment boundaries.
  const int a_row0 = tid >> 3;
  const int a_kc = tid & 7;
  int b_ch[8];          // NG: channel number (B row) of each B row this thread loads
  if (MODE == MODE_NG) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = n0 + a_row0 + ((32 * i) % BNC);
      if (c >= nch) c = nch - 1;
      b_ch[i] = gidx ? gidx[c] : c;
    }
  }
  const int kg_kr0 = (tid & 7) * KR;
  const int kg_n = (tid >> 3) * 8;
  const bool kg_nok = (n0 + kg_n) < args.N;      // N is a multiple of 8
  const int kg_c0 = kg_nok ? n0 + kg_n : 0;

  constexpr int PF = 1;  // register sets
  Chunk ra[PF][ACH];
  Chunk rb[PF][8];
  int va[PF];            // valid elements of the A / N-gather B chunks of each set
  int kg_rv[PF];         // K-gather: valid k-rows of each set
  bool qv[PF];           // QB: the set's B chunks hold (codes, scale) still to dequantize
#pragma unroll
  for (int p = 0; p < PF; ++p) { va[p] = VEC; kg_rv[p] = KR; qv[p] = false; }

  // loader cursor: uniform scalars + per-thread element offsets (32-bit; the
  // host checks that every operand has fewer than 2^31 elements)
  int cur_s = 0, cur_kk = 0, cur_K = 0, cur_nkt = 0;
  const T* a_base = nullptr;
  const T* b_base = nullptr;
  const T* b2_base = nullptr;
  unsigned a_off[ACH];
  unsigned b_off[8];
  int cur_ldb = 0;
  bool cur_q = false;               // QB: the segment's B is 4-bit
  const float* bs_base = nullptr;   // QB: its scales (dual: gate rows)
  const float* bs2_base = nullptr;  //     (dual: up rows)

  auto enter_seg = [&](int s) {
    s = __builtin_amdgcn_readfirstlane(s);
    const GSeg& sg = args.seg[s];
    cur_s = s;
    cur_K = __builtin_amdgcn_readfirstlane(seg_len(s));
    cur_nkt = (cur_K + BK - 1) / BK;
    a_base = reinterpret_cast<const T*>(sg.A) + pr.a_col[s];
    b_base = reinterpret_cast<const T*>(pr.B[s]);
    b2_base = reinterpret_cast<const T*>(DUAL ? sg.B2 : pr.B[s]);
    cur_ldb = (int)sg.ldb;
    if constexpr (QB) {
      cur_q = sg.bq4 != 0;
      bs_base = pr.Bs[s];
      bs2_base = DUAL ? sg.B2s : pr.Bs[s];
    }
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      int r = m0 + a_row0 + 32 * i;
      if (r >= m_rows) r = m_rows - 1;    // rows past the group are computed and dropped
      if (sg.a_tok) a_off[i] = (unsigned)group_token(args.st, g, r) * (unsigned)sg.lda;
      else a_off[i] = is_out ? (unsigned)sg.a_out_off + (unsigned)r * (unsigned)sg.lda_out
                             : (unsigned)(ctx_pre_g + r) * (unsigned)sg.lda;
    }
    if (MODE == MODE_NG) {
#pragma unroll
      for (int i = 0; i < 8; ++i) b_off[i] = (unsigned)b_ch[i] * (unsigned)sg.ldb;
    }
  };

  // KG: the B row of k-position `lane` of tile (s, kk), fetched into a
  // register and handed to all waves through LDS at the next store phase.  Rows always come from memory (ungathered segments read the iota
  // array) and positions past K are clamped (those rows are zeroed at store
  // time), so the loaded index is consumed only at the store phase.
  int krow_reg = 0;
  auto fetch_rows = [&](int s, int kk) {
    s = __builtin_amdgcn_readfirstlane(s);
    const GSeg& sg = args.seg[s];
    const int K = seg_len(s);
    const int* sidx = (sg.b_gather && !is_out) ? sg.idx + (long long)g * sg.kidx : args.iota;
    // every wave loads (no divergent definition of the register; wave 0 publishes)
    krow_reg = sidx[min(kk * BK + min(lane, BK - 1), K - 1)];
  };
  auto publish_rows = [&]() {
    if (!KGD && wave == 0) krow_s[lane] = krow_reg;
  };
  // KGD: B stage the next load_tile fills, and the K-tiles loaded so far
  int b_stage = 0, n_loaded = 0;

  // position the cursor on K-tile kt_begin
  if (nkt > 0) {
    int s = 0, kk = kt_begin;
    for (;;) {
      const int n = (seg_len(s) + BK - 1) / BK;
      if (s + 1 >= args.nseg || kk < n) break;
      kk -= n;
      ++s;
    }
    enter_seg(s);
    cur_kk = __builtin_amdgcn_readfirstlane(kk);
  }

  // Issue the global loads of the next K-tile into register set P; K-gather
  // rows come from krow_s.
  auto load_tile = [&](auto Pc) {
    constexpr int P = decltype(Pc)::value;   // register set
    if (cur_kk >= cur_nkt && cur_s + 1 < args.nseg) {   // segment boundary (segments are never empty)
      enter_seg(cur_s + 1);
      cur_kk = 0;
    }
    const int k0 = cur_kk * BK;
    const int kcol = k0 + a_kc * VEC;
    va[P] = cur_K - kcol < 0 ? 0 : (cur_K - kcol > VEC ? VEC : cur_K - kcol);
    const int kc = kcol < cur_K ? kcol : 0;
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[P][i] = load_chunk(a_base + (a_off[i] + kc));
    if constexpr (QB) qv[P] = cur_q;
    if (MODE == MODE_NG) {
      if (QB && cur_q) {
        // 8 codes (4 bytes) and the scale of their 64-element block per row
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool up = DUAL && 32 * i >= BNC;
          const unsigned e = b_off[i] + (unsigned)kc;
          const unsigned char* cb = reinterpret_cast<const unsigned char*>(up ? b2_base : b_base);
          rb[P][i].w[0] = *reinterpret_cast<const uint32_t*>(cb + e / 2);
          rb[P][i].w[1] = __float_as_uint((up ? bs2_base : bs_base)[e / 64]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          rb[P][i] = load_chunk(((DUAL && 32 * i >= BNC) ? b2_base : b_base) + (b_off[i] + kc));
      }
    } else if constexpr (KGD) {
      // The tile's 64 B rows (krow_reg of lane p = row of k-position p) as 32
      // LDS-DMA blocks of two k-rows; wave w issues blocks 4 j + w.  Lane l
      // fills physical chunk l%32 of k-row 2 (4 j + w) + l/32 with the logical
      // chunk that the swizzle puts there.  Columns past N are clamped (their
      // outputs are dropped); rows past K hold a clamped row whose A columns
      // are zero.  Tiles past the range are not loaded.
      // (The row indices are read on every path, so the index load never
      // stays pending into the next compute phase.)
      unsigned char* st = Bst0 + b_stage * B_STAGE;
      const bool issue = n_loaded < nkt;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kr0 = 8 * j + 2 * wave;
        const int r0 = __builtin_amdgcn_readlane(krow_reg, kr0);
        const int r1 = __builtin_amdgcn_readlane(krow_reg, kr0 + 1);
        const int kr = kr0 + (lane >> 5);
        const int c = (lane & 31) ^ kgd_bswz(kr);
        int col = n0 + 8 * c;
        if (col >= args.N) col = 0;
        const unsigned off = ((unsigned)(lane < 32 ? r0 : r1) * (unsigned)cur_ldb + (unsigned)col) * 2u;
        const unsigned la = __builtin_amdgcn_readfirstlane(
            (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(st + (4 * j + wave) * 1024));
        if (issue)
          asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
                       :: "v"(off), "s"(la), "s"(b_base) : "memory", "m0");
      }
      b_stage ^= 1;
      ++n_loaded;
    } else {
      const int kr = cur_K - (k0 + kg_kr0);
      kg_rv[P] = kr < 0 ? 0 : (kr > KR ? KR : kr);
      int rows[KR];
#pragma unroll
      for (int i = 0; i < KR; i += 4) {
        const int4 q = *reinterpret_cast<const int4*>(&krow_s[kg_kr0 + i]);
        rows[i] = q.x; rows[i + 1] = q.y; rows[i + 2] = q.z; rows[i + 3] = q.w;
      }
      if (QB && cur_q) {
        // 8 codes of n-columns kg_c0.. (one 64-element block) and its scale per k-row
#pragma unroll
        for (int i = 0; i < KR; ++i) {
          const unsigned e = (unsigned)rows[i] * (unsigned)cur_ldb + (unsigned)kg_c0;
          rb[P][i].w[0] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const unsigned char*>(b_base) + e / 2);
          rb[P][i].w[1] = __float_as_uint(bs_base[e / 64]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < KR; ++i)
#pragma unroll
          for (int h = 0; h < 8 / VEC; ++h)
            rb[P][i * (8 / VEC) + h] =
                load_chunk(b_base + ((unsigned)rows[i] * (unsigned)cur_ldb + kg_c0 + h * VEC));
      }
    }
    ++cur_kk;
  };

  // K-gather: fetch the rows of the tile the cursor points at (the next one to
  // load; the cursor advances past each loaded tile).
  auto fetch_rows_next = [&]() {
    int s = cur_s, kk = cur_kk;
    if (kk >= cur_nkt && s + 1 < args.nseg) { kk = 0; ++s; }
    fetch_rows(s, kk);
  };

  auto store_tile = [&](auto Pc) {
    constexpr int P = decltype(Pc)::value;
    if constexpr (KGD) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the tile's B DMA has landed
    if constexpr (QB) {
      if (qv[P]) {   // 8 B chunks of (codes, scale) either way (bf16: KR = 8, 8 / VEC = 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[P][i] = deq8(rb[P][i].w[0], __uint_as_float(rb[P][i].w[1]));
      }
    }
    if (va[P] < VEC) {
#pragma unroll
      for (int i = 0; i < ACH; ++i) mask_chunk<T>(ra[P][i], va[P]);
      if (MODE == MODE_NG) {
#pragma unroll
        for (int i = 0; i < 8; ++i) mask_chunk<T>(rb[P][i], va[P]);
      }
    }
    if (MODE == MODE_KG && !KGD) {
#pragma unroll
      for (int i = 0; i < KR; ++i)
        if (i >= kg_rv[P] || !kg_nok) {
#pragma unroll
          for (int h = 0; h < 8 / VEC; ++h) rb[P][i * (8 / VEC) + h] = zero_chunk();
        }
    }
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int ar = a_row0 + 32 * i;
      T* dst = KGD ? &As[ar * A_LD + (a_kc ^ kgd_aswz(ar)) * VEC] : &As[ar * LDS_LD + a_kc * VEC];
      *reinterpret_cast<uint4*>(dst) = make_uint4(ra[P][i].w[0], ra[P][i].w[1], ra[P][i].w[2], ra[P][i].w[3]);
    }
    if constexpr (KGD) {
      // B arrived by DMA
    } else if (MODE == MODE_NG) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint4*>(&Bs[(a_row0 + 32 * i) * LDS_LD + a_kc * VEC]) =
            make_uint4(rb[P][i].w[0], rb[P][i].w[1], rb[P][i].w[2], rb[P][i].w[3]);
    } else {
      // transpose KR k-rows x 8 n-values into 8 n-rows x KR k-values
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
        if (sizeof(T) == 2) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const Chunk& c0 = rb[P][2 * p];
            const Chunk& c1 = rb[P][2 * p + 1];
            const uint32_t lo = (c0.w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            const uint32_t hi = (c1.w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            w[p] = lo | (hi << 16);
          }
        } else {
#pragma unroll
          for (int p = 0; p < 4; ++p) w[p] = rb[P][p * 2 + (j >> 2)].w[j & 3];
        }
        *reinterpret_cast<uint4*>(&Bs[(kg_n + j) * LDS_LD + kg_kr0]) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };

  // KGD: byte offset from stage 0 of the B words this lane supplies to the
  // transposing reads of block nb (k-row 8 (lane/32) + (lane%16)/4 of K-step 0,
  // first half), in the stage the next compute phase reads (bit 15 = stage).  Other K-steps and the second
  // half are fixed offsets (the swizzle ignores k-row bits 2, 4 and 5); the
  // stage bit flips after every compute phase.
  unsigned boff[4];
  if constexpr (KGD) {
    const int grp = lane >> 4, gi = lane & 15;
    const int kr = 8 * (grp >> 1) + (gi >> 2);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int ncol = brow(nb) + 16 * (grp & 1) + 4 * (gi & 3);
      boff[nb] = (unsigned)(kr * (G_BN * 2)) +
                 ((unsigned)((ncol >> 3) ^ kgd_bswz(kr)) << 4) + (unsigned)(ncol & 7) * 2u;
    }
  }
  auto compute = [&]() {
    if constexpr (!KGD && sizeof(T) == 2) {
      // bf16 from padded tiles, software-pipelined: the A fragments of the
      // next K-step are read while this K-step's MFMAs run, and each B
      // fragment is re-read for the next K-step right after the two MFMAs
      // that use it.  Scheduling barriers keep the reads where they are (left
      // alone, the scheduler moves each read down to its use and exposes the
      // LDS latency twice per K-step).
      constexpr int NKS = BK / KSTEP;
      static_assert(NKS == 4, "the pipelined K-steps assume BK = 4 KSTEP");
      auto lda = [&](int ks, int mb) -> bf16x8_t {
        return *reinterpret_cast<const bf16x8_t*>(
            &As[(WM * wm + 32 * mb + (lane & 31)) * LDS_LD + ks * 16 + (lane >> 5) * 8]);
      };
      auto ldb = [&](int ks, int nb) -> bf16x8_t {
        return *reinterpret_cast<const bf16x8_t*>(
            &Bs[(brow(nb) + (lane & 31)) * LDS_LD + ks * 16 + (lane >> 5) * 8]);
      };
      bf16x8_t a0[MB], a1[MB], b[4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) a0[mb] = lda(0, mb);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) b[nb] = ldb(0, nb);
      auto step = [&](auto KS, bf16x8_t (&ac)[MB], bf16x8_t (&an)[MB]) {
        constexpr int ks = decltype(KS)::value;
        if constexpr (ks + 1 < NKS) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) an[mb] = lda(ks + 1, mb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[mb], b[nb], acc[mb][nb], 0, 0, 0);
          if constexpr (ks + 1 < NKS) {
            __builtin_amdgcn_sched_barrier(0);
            b[nb] = ldb(ks + 1, nb);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      };
      step(std::integral_constant<int, 0>{}, a0, a1);
      step(std::integral_constant<int, 1>{}, a1, a0);
      step(std::integral_constant<int, 2>{}, a0, a1);
      step(std::integral_constant<int, 3>{}, a1, a0);
      return;
    }
#pragma unroll
    for (int kstep = 0; kstep < BK / KSTEP; ++kstep) {
      if constexpr (KGD) {
        bf16x8_t af[MB], bfr[4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int ar = WM * wm + 32 * mb + (lane & 31);
          af[mb] = *reinterpret_cast<const bf16x8_t*>(
              &As[ar * A_LD + ((2 * kstep + (lane >> 5)) ^ kgd_aswz(ar)) * 8]);
        }
        // B operand (k = 16 kstep + 8 (lane/32) + e, n = block column + lane%32)
        // from two transposing reads: in each 16-lane group, lane i supplies
        // the address of 4 consecutive n (4 (i%4) ..) of k-row i/4 and
        // receives element i%4 of the words of lanes 4 e + i/4 (e < 4).
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          v4i16_t h2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const unsigned char* pa = Bst0 + boff[nb] + (16 * kstep + 4 * h) * (G_BN * 2);
            h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16_t*)(
                    (__attribute__((address_space(3))) unsigned char*)(pa)));
          }
          bfr[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
      } else {
        float af[MB], bfr[4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[mb] = reinterpret_cast<const float*>(As)[(WM * wm + 32 * mb + (lane & 31)) * LDS_LD +
                                                       kstep * 2 + (lane >> 5)];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          bfr[nb] = reinterpret_cast<const float*>(Bs)[(brow(nb) + (lane & 31)) * LDS_LD +
                                                        kstep * 2 + (lane >> 5)];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  };

  // One register set: the loads of tile i+1 are in flight while tile i is
  // consumed from LDS; they are issued right after tile i is stored.  K-gather
  // rows of tile i+2 are fetched after the compute phase of iteration i and
  // used at its end, so no loaded index is carried across an iteration.  (A second
  // register set for a deeper prefetch needs an unrolled loop body whose
  // register pressure spills the accumulators.)
  using I0 = std::integral_constant<int, 0>;
  if (nkt > 0) {
    if (MODE == MODE_KG) {
      fetch_rows(cur_s, cur_kk);
      publish_rows();
      __syncthreads();
    }
    load_tile(I0{});
    if (MODE == MODE_KG) {
      __syncthreads();   // everyone has read the rows of tile 0
      fetch_rows_next();
      publish_rows();
    }
    store_tile(I0{});
    __syncthreads();
    if (nkt > 1) load_tile(I0{});
    for (int i = 0; i < nkt; ++i) {
      compute();
      if constexpr (KGD) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) boff[nb] ^= (unsigned)B_STAGE;
      }
      // K-gather rows of tile i+2, fetched after the compute phase: a load in
      // flight across the MFMAs makes the compiler drain every outstanding
      // load (the prefetched tile included) before them.  Unconditional, so
      // every fetched row is consumed (past the range the cursor stays on the
      // last segment and the clamped loads are never stored).
      if (MODE == MODE_KG) fetch_rows_next();
      __syncthreads();
      if (i + 1 >= nkt) break;
      store_tile(I0{});
      if (MODE == MODE_KG) publish_rows();
      __syncthreads();
      load_tile(I0{});
    }
  }
  } else {
  // ---- LDS-DMA main loop (wide N-gather and tall K-gather tiles) -------------
  // Stage layout: A rows [0, BM), 128 bytes each, then the B part (BN_T x 128
  // bytes).  N-gather: B rows [0, BN_T), 128 bytes each; A and B rows have
  // their 16-byte chunks swizzled by wng_swz.  K-gather: 64 k-rows of 256
  // n-values (512 bytes), 16-byte chunk c of k-row k at c ^ kgd_bswz(k), read by
  // the transposing LDS reads.  One LDS-DMA instruction fills one 1 KB block:
  // 8 rows of A or N-gather B (lane l: row l / 8, physical chunk l % 8), or 2
  // k-rows of K-gather B (lane l: k-row l / 32, physical chunk l % 32).  Per
  // K-tile wave w issues A blocks W_AB w .. and B blocks W_BB w .. (dual: the
  // first half of the B blocks hold gate rows, the second up rows).  Rows past
  // the group or channel count, and K-gather columns past N, are clamped
  // (their outputs are dropped).  A K-tile that ends inside its segment
  // (k0 + BK > K) stages A through registers with the columns past K zeroed;
  // its B columns (N-gather) or k-rows (K-gather) past K are clamped and meet
  // those zeros.
  constexpr int W_AB = BM / 8 / NWAVE;       // A blocks per wave
  constexpr int W_BB = BN_T / 8 / NWAVE;     // B blocks per wave
  static_assert(W_AB % 2 == 0 && W_BB % 2 == 0, "a block's parity must follow its index");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int w_r = lane >> 3;
  // element offset of the logical chunk this lane fetches in even / odd blocks
  // (bit 3 of the row, which the swizzle reads, is the block's parity)
  auto kcl = [&](int par) __attribute__((always_inline)) -> int { return 8 * ((lane & 7) ^ wng_swz(8 * par + w_r)); };
  // A row of block j of this wave (rows past the group clamp to its last)
  auto arow = [&](int j) __attribute__((always_inline)) -> int {
    const int r = m0 + 8 * (W_AB * wv + j) + w_r;
    return r < m_rows ? r : m_rows - 1;
  };
  int bch[W_BB];        // N-gather: channel (B row) of each B block row this lane fetches
  if constexpr (MODE == MODE_NG) {
#pragma unroll
    for (int j = 0; j < W_BB; ++j) {
      int c = n0 + (8 * (W_BB * wv + j) + w_r) % BNC;
      if (c >= nch) c = nch - 1;
      bch[j] = gidx ? gidx[c] : c;
    }
  }
  int cur_s = 0, cur_kk = 0, cur_K = 0, cur_nkt = 0;
  const T* a_base = nullptr;
  const T* b_base = nullptr;
  const T* b2_base = nullptr;
  int cur_ldb = 0;
  unsigned a_off[W_AB];   // element offset of each A block row of this lane (current segment)
  auto enter_seg = [&](int s) __attribute__((always_inline)) {
    s = __builtin_amdgcn_readfirstlane(s);
    const GSeg& sg = args.seg[s];
    cur_s = s;
    cur_K = __builtin_amdgcn_readfirstlane(seg_len(s));
    cur_nkt = (cur_K + BK - 1) / BK;
    a_base = reinterpret_cast<const T*>(sg.A) + pr.a_col[s];
    b_base = reinterpret_cast<const T*>(pr.B[s]);
    b2_base = reinterpret_cast<const T*>(DUAL ? sg.B2 : pr.B[s]);
    cur_ldb = __builtin_amdgcn_readfirstlane((int)sg.ldb);
#pragma unroll
    for (int j = 0; j < W_AB; ++j) {
      const int r = arow(j);
      if (sg.a_tok) a_off[j] = (unsigned)group_token(args.st, g, r) * (unsigned)sg.lda;
      else a_off[j] = is_out ? (unsigned)sg.a_out_off + (unsigned)r * (unsigned)sg.lda_out
                             : (unsigned)(ctx_pre_g + r) * (unsigned)sg.lda;
    }
  };
  if (nkt > 0) {
    int s = 0, kk = kt_begin;
    for (;;) {
      const int n = (seg_len(s) + BK - 1) / BK;
      if (s + 1 >= args.nseg || kk < n) break;
      kk -= n;
      ++s;
    }
    enter_seg(s);
    cur_kk = __builtin_amdgcn_readfirstlane(kk);
  }

  // K-gather: the weight rows of a K-tile (lane p: the row of k-position p;
  // positions past K clamp to K-1, whose A columns are zero), fetched one
  // K-tile ahead of its DMA issue by a cursor of their own.
  int f_s = cur_s, f_kk = cur_kk;
  auto fetch_rows = [&]() __attribute__((always_inline)) -> int {
    int r = 0;
    if constexpr (MODE == MODE_KG) {
      const int s = __builtin_amdgcn_readfirstlane(f_s);
      const GSeg& sg = args.seg[s];
      const int K = seg_len(s);
      const int* sidx = (sg.b_gather && !is_out) ? sg.idx + (long long)g * sg.kidx : args.iota;
      r = sidx[min(f_kk * BK + min(lane, BK - 1), K - 1)];
      ++f_kk;
      if (f_kk >= (K + BK - 1) / BK && s + 1 < args.nseg) { f_s = s + 1; f_kk = 0; }
    }
    return r;
  };

  // Issue the loads of the cursor's K-tile into the stage at byte offset st
  // (K-gather: krow = its weight rows); returns the LDS-DMA instructions issued
  // (a register-staged A is waited for before its LDS store, so only DMA
  // instructions stay outstanding).
  auto issue = [&](int st, int krow) __attribute__((always_inline)) -> int {
    if (cur_kk >= cur_nkt && cur_s + 1 < args.nseg) {   // segments are never empty
      enter_seg(cur_s + 1);
      cur_kk = 0;
    }
    const int k0 = cur_kk * BK;
    const bool full = k0 + BK <= cur_K;
    unsigned char* sb = smem + st;
    int n = W_BB;
    if (full) {
#pragma unroll
      for (int j = 0; j < W_AB; ++j) {
        const unsigned la = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(
            __attribute__((address_space(3))) unsigned char*)(sb + 1024 * (W_AB * wv + j)));
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
                     :: "v"((a_off[j] + (unsigned)(k0 + kcl(j & 1))) * 2u), "s"(la), "s"(uniform_ptr(a_base))
                     : "memory", "m0");
      }
      n += W_AB;
    } else {
#pragma unroll
      for (int j = 0; j < W_AB; ++j) {
        const int kc = k0 + kcl(j & 1);
        Chunk v = zero_chunk();
        if (kc < cur_K) {
          // the chunk that straddles K (a K-gather segment's channel count
          // need not be a multiple of 8) keeps only its elements below K
          v = load_chunk(a_base + (a_off[j] + (unsigned)kc));
          mask_chunk<T>(v, cur_K - kc);
        }
        *reinterpret_cast<uint4*>(sb + 1024 * (W_AB * wv + j) + 16 * lane) =
            make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
      }
    }
    if constexpr (MODE == MODE_NG) {
#pragma unroll
      for (int j = 0; j < W_BB; ++j) {
        const int q = W_BB * wv + j;
        const T* base = (DUAL && q >= BN_T / 16) ? b2_base : b_base;
        const int kc = k0 + kcl(j & 1);
        const unsigned kb = kc < cur_K ? (unsigned)kc : 0u;
        const unsigned la = __builtin_amdgcn_readfirstlane(
            (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(sb + BM * W_ROWB + 1024 * q));
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
                     :: "v"(((unsigned)bch[j] * (unsigned)cur_ldb + kb) * 2u), "s"(la), "s"(uniform_ptr(base))
                     : "memory", "m0");
      }
    } else {
      // block q: k-rows 2 q and 2 q + 1 (lanes 0-31 / 32-63)
#pragma unroll
      for (int j = 0; j < W_BB; ++j) {
        const int q = W_BB * wv + j;
        const int r0 = __builtin_amdgcn_readlane(krow, 2 * q);
        const int r1 = __builtin_amdgcn_readlane(krow, 2 * q + 1);
        const int kr = 2 * q + (lane >> 5);
        const int c = (lane & 31) ^ kgd_bswz(kr);
        int col = n0 + 8 * c;
        if (col >= args.N) col = 0;
        const unsigned off = ((unsigned)(lane < 32 ? r0 : r1) * (unsigned)cur_ldb + (unsigned)col) * 2u;
        const unsigned la = __builtin_amdgcn_readfirstlane(
            (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(sb + BM * W_ROWB + 1024 * q));
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
                     :: "v"(off), "s"(la), "s"(uniform_ptr(b_base)) : "memory", "m0");
      }
    }
    ++cur_kk;
    return n;
  };

  // Fragment offsets inside a stage for K-step 0 (K-step s: byte offset ^ 32 s,
  // the logical chunk 2 s + lane / 32 differing from K-step 0's in bits 1..2).
  // Fragment rows start on 32-row boundaries, so a lane's row has
  // row % 16 = lane % 16.
  // Block mb's rows start 32 mb rows (4096 mb bytes) after block 0's, and
  // N-gather B block nb's at a fixed offset from block 0's, so one base per
  // operand plus an immediate offset addresses those fragments (the K-step
  // XOR touches bits 5-6 only, below every block offset).  K-gather B blocks
  // keep an offset each: their k-row swizzle XORs the chunk bits a block
  // offset would add to.
  const int f_ch = (((lane >> 5) ^ wng_swz(lane & 15)) << 4);
  const unsigned fa0 = (unsigned)((WM * wm + (lane & 31)) * W_ROWB + f_ch);
  unsigned fb[MODE == MODE_NG ? 1 : 4];
  if constexpr (MODE == MODE_NG) {
    fb[0] = (unsigned)(BM * W_ROWB + (brow(0) + (lane & 31)) * W_ROWB + f_ch);
  } else {
    // transposing reads: in each 16-lane group lane i supplies the address of
    // 4 consecutive n (4 (i % 4) ..) of k-row i / 4 (+ 8 for the second pair
    // of groups); K-step s adds 16 s k-rows and the second read 4 more (the
    // swizzle ignores k-row bits 2, 4 and 5)
    const int grp = lane >> 4, gi = lane & 15;
    const int kr = 8 * (grp >> 1) + (gi >> 2);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int ncol = brow(nb) + 16 * (grp & 1) + 4 * (gi & 3);
      fb[nb] = (unsigned)(BM * W_ROWB) + (unsigned)(kr * (G_BN * 2)) +
               ((unsigned)((ncol >> 3) ^ kgd_bswz(kr)) << 4) + (unsigned)(ncol & 7) * 2u;
    }
  }
  auto rda = [&](int st, int ks, int mb) __attribute__((always_inline)) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(smem + st + (fa0 ^ (unsigned)(32 * ks)) + 4096u * mb);
  };
  auto rdb = [&](int st, int ks, int nb) __attribute__((always_inline)) -> bf16x8_t {
    if constexpr (MODE == MODE_NG) {
      return *reinterpret_cast<const bf16x8_t*>(smem + st + (fb[0] ^ (unsigned)(32 * ks)) +
                                                 (unsigned)((brow(nb) - brow(0)) * W_ROWB));
    } else {
      v4i16_t h2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned char* pa = smem + st + fb[nb] + (16 * ks + 4 * h) * (G_BN * 2);
        h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(
                (__attribute__((address_space(3))) unsigned char*)(pa)));
      }
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // One K-step: MFMAs on (ac, b); meanwhile the A fragments of the next step
  // go to an and each B fragment is re-read for the next step (stage nst,
  // K-step nks) right after its MFMAs.  nxt = false: no next step.
  auto kstep = [&](bf16x8_t (&ac)[MB], bf16x8_t (&an)[MB], bf16x8_t (&b)[4], bool nxt, int nst, int nks) {
    if (nxt) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) an[mb] = rda(nst, nks, mb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[mb], b[nb], acc[mb][nb], 0, 0, 0);
      if (nxt) {
        __builtin_amdgcn_sched_barrier(0);
        b[nb] = rdb(nst, nks, nb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Two stages: K-tile i is consumed from stage i % 2 while K-tile i+1 lands
  // in the other.  Each K-tile's loads are issued as soon as the stage it
  // fills is free: right after the barrier that follows the last fragment
  // read of the K-tile two before it.  K-gather rows of K-tile i+3 are fetched
  // right after K-tile i+2 is issued; the wait before the next barrier covers
  // them.
  if (nkt > 0) {
    static_assert(BK / KSTEP == 4, "four K-steps per K-tile");
    bf16x8_t a0[MB], a1[MB], b[4];
    const int kr0 = fetch_rows();
    const int kr1 = fetch_rows();
    issue(0, kr0);
    const int n1 = nkt > 1 ? issue(W_STG, kr1) : 0;
    int krow_next = fetch_rows();
    wait_vmcnt(n1);    // K-tile 0 has landed (K-tile 1 may be in flight)
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a0[mb] = rda(0, 0, mb);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) b[nb] = rdb(0, 0, nb);
    int st = 0;
    for (int i = 0; i < nkt; ++i) {
      const int st_next = st ^ W_STG;
      const bool more = i + 1 < nkt;
      auto handover = [&]() __attribute__((always_inline)) {
        if (more) {
          wait_vmcnt(0);       // K-tile i+1 (the only loads in flight) has landed
          __syncthreads();     // ... for every wave; and stage i is read by none
          if (i + 2 < nkt) {
            issue(st, krow_next);
            krow_next = fetch_rows();
          }
        }
      };
      kstep(a0, a1, b, true, st, 1);
      kstep(a1, a0, b, true, st, 2);
      kstep(a0, a1, b, true, st, 3);
      handover();
      kstep(a1, a0, b, more, st_next, 0);
      st = st_next;
    }
  }
  wait_vmcnt(0);   // no LDS-DMA may land in the staging area
  __syncthreads();
  }
  if constexpr (KGD) __builtin_amdgcn_s_waitcnt(0x0F70);   // no LDS-DMA may land in the staging area

  // ---- epilogue -----------------------------------------------------------
  // The accumulators go through LDS: per 32-row block and pair of 32-column
  // blocks, each wave writes a 32 x 64 fp32 tile (accumulator element e of a
  // block sits at row 8*(e/4) + 4*(lane/32) + e%4, column lane%32), then every
  // lane takes 32 consecutive columns of one row (half a row per lane pair
  // in dual mode) and applies the element-wise step with 16-byte accesses.
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * EP_LD;
  const long long ldc = is_out ? args.ldc_out : args.ldc_ctx;
  const long long cbase = is_out ? args.c_out_off : (long long)ctx_pre_g * args.ldc_ctx;
  const int er = lane >> 1;            // row of the 32-row block this lane finishes
  const int ec = (lane & 1) * 32;      // first of its 32 staged columns
  if (!WIDE && nkt <= 0) __syncthreads();   // (the main loop ends with a barrier otherwise)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      // blocks staged in this pass: dual -> gate hp and up hp; else nb = 2 hp, 2 hp + 1
      const int nb0 = DUAL ? hp : 2 * hp;
      const int nb1 = DUAL ? hp + 2 : 2 * hp + 1;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        ep[rr * EP_LD + (lane & 31)] = acc[mb][nb0][e];
        ep[rr * EP_LD + 32 + (lane & 31)] = acc[mb][nb1][e];
      }
      __syncthreads();
      const int r = m0 + WM * wm + 32 * mb + er;
      const float* src = ep + er * EP_LD;
      if (MODE == MODE_NG && nks > 1) {
        // K piece of a split tile: raw accumulators, tile-local [row][accumulator column]
        if (r < m_rows) {
          float* dst = args.rpart +
                       ((long long)(blockIdx.x - args.rem_start) * BM + WM * wm + 32 * mb + er) * BN_T +
                       128 * wn + 32 * (ec ? nb1 : nb0);
#pragma unroll
          for (int q = 0; q < 4; ++q) store_row<float, 8>(dst + 8 * q, src + ec + 8 * q, 8);
        }
      } else if (r < m_rows) {
        // 8 columns at a time keeps the temporaries small while later
        // accumulator blocks are still live
#pragma unroll 1
        for (int q = 0; q < (DUAL ? 2 : 4); ++q) {
          if constexpr (EPI == EPI_SWIGLU) {
            // lane pair: even lane channels 0..15, odd lane 16..31 of the 32-channel block
            const int cl = (lane & 1) * 16 + 8 * q;
            const int c = n0 + 64 * wn + 32 * hp + cl;
            const long long o = cbase + (long long)r * ldc + c;
            float gv[8], uv[8], hv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              gv[j] = src[cl + j];
              uv[j] = src[32 + cl + j];
              const float sg = (sizeof(T) == 4) ? sigmoid_exact(gv[j]) : sigmoidf_(gv[j]);
              hv[j] = gv[j] * sg * uv[j];
            }
            store_row<T, 8>(reinterpret_cast<T*>(args.o0) + o, gv, nch - c);
            store_row<T, 8>(reinterpret_cast<T*>(args.o1) + o, uv, nch - c);
            store_row<T, 8>(reinterpret_cast<T*>(args.o2) + o, hv, nch - c);
          } else {
            const int cl = ec + 8 * q;
            const int c = n0 + 128 * wn + 64 * hp + cl;
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = src[cl + j];
            if constexpr (EPI == EPI_DSWIGLU) {
              const long long o = cbase + (long long)r * ldc + c;
              float gv[8], uv[8], dg[8], du[8];
              load_row<T, 8>(reinterpret_cast<const T*>(args.i0) + o, gv, nch - c);
              load_row<T, 8>(reinterpret_cast<const T*>(args.i1) + o, uv, nch - c);
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float sg = (sizeof(T) == 4) ? sigmoid_exact(gv[j]) : sigmoidf_(gv[j]);
                dg[j] = v[j] * uv[j] * sg * (1.0f + gv[j] * (1.0f - sg));
                du[j] = v[j] * gv[j] * sg;
              }
              store_row<T, 8>(reinterpret_cast<T*>(args.o0) + o, dg, nch - c);
              store_row<T, 8>(reinterpret_cast<T*>(args.o1) + o, du, nch - c);
            } else if constexpr (EPI == EPI_TOKEN) {
              if (is_out && nks > 1)
                store_row<float, 8>(args.part + ((long long)ks * args.st.T_out + r) * args.N + c, v,
                                    args.N - c);
              else
                store_row<T, 8>(reinterpret_cast<T*>(pr.o0) +
                                    (long long)group_token(args.st, g, r) * pr.ldo + c,
                                v, args.N - c);
            } else {  // EPI_SCATTER: column = the channel number
              T* out = reinterpret_cast<T*>(pr.o0) + (long long)group_token(args.st, g, r) * pr.ldo;
              const bool vec = pr.ldo % 8 == 0;
              if (!gidx) {
                if (vec) store_row<T, 8>(out + c, v, nch - c);
                else {
#pragma unroll
                  for (int j = 0; j < 8; ++j)
                    if (c + j < nch) stv<T>(out, c + j, v[j]);
                }
              } else {
                scatter_row8<T>(out, gidx, c, nch, pr.swidth, v, vec);
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

// Adds the K pieces of every split N-gather tile in piece order and applies
// the tile's element-wise epilogue (the same arithmetic as the GEMM's own).
// One thread per (split tile, row, 8 channels).
template <typename T, int EPI, bool DUAL, int WN, int BM>
__global__ void __launch_bounds__(256) ng_fixup_kernel(const GemmArgs args) {
  constexpr int BN_T = 128 * WN;   // partial-tile row: accumulator columns of the GEMM tile
  constexpr int BNC = DUAL ? BN_T / 2 : BN_T;
  constexpr int CG = BNC / 8;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nrem = args.ntiles - args.rem_start;
  if (i >= (long long)nrem * BM * CG) return;
  const int cg = (int)(i % CG);
  const int rloc = (int)((i / CG) % BM);
  const int tr = (int)(i / ((long long)CG * BM));
  const int tile = args.rem_start + tr;
  int g = 0;   // split launches hold one problem: flat group = group
  while (g + 1 < args.ngroups && args.tile_start[g + 1] <= tile) ++g;
  const int t_in = tile - args.tile_start[g];
  const int ntm = (group_rows(args.st, g) + BM - 1) / BM;
  const int mt = t_in % ntm, nt = t_in / ntm;
  const bool is_out = (g == args.st.nseq);
  const int m_rows = group_rows(args.st, g);
  const int nch = is_out ? args.n_out : args.kidx;
  const int r = mt * BM + rloc;
  if (r >= m_rows) return;
  const int cl = cg * 8;
  const int c = nt * BNC + cl;
  if (c >= nch) return;
  // accumulator column of channel cl (8 consecutive channels stay in one 32-block)
  int ag;
  if (DUAL) ag = 128 * (cl / 64) + 32 * ((cl % 64) / 32) + (cl % 32);
  else ag = cl;
  float v0[8], v1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { v0[j] = 0.f; v1[j] = 0.f; }
  // pieces loaded 4 at a time, added in piece order
  for (int sp0 = 0; sp0 < args.rem_split; sp0 += 4) {
    float a0[4][8], a1[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (sp0 + u >= args.rem_split) break;
      const float* src = args.rpart + ((long long)(tr * args.rem_split + sp0 + u) * BM + rloc) * BN_T + ag;
      load_row<float, 8>(src, a0[u], 8);
      if (DUAL) load_row<float, 8>(src + 64, a1[u], 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (sp0 + u >= args.rem_split) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) v0[j] += a0[u][j];
      if (DUAL) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v1[j] += a1[u][j];
      }
    }
  }
  const int ctx_pre_g = is_out ? 0 : args.st.ctx_pre[g];
  const long long ldc = is_out ? args.ldc_out : args.ldc_ctx;
  const long long cbase = is_out ? args.c_out_off : (long long)ctx_pre_g * args.ldc_ctx;
  const long long o = cbase + (long long)r * ldc + c;
  if constexpr (EPI == EPI_SWIGLU) {
    float hv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float sg = (sizeof(T) == 4) ? sigmoid_exact(v0[j]) : sigmoidf_(v0[j]);
      hv[j] = v0[j] * sg * v1[j];
    }
    store_row<T, 8>(reinterpret_cast<T*>(args.o0) + o, v0, nch - c);
    store_row<T, 8>(reinterpret_cast<T*>(args.o1) + o, v1, nch - c);
    store_row<T, 8>(reinterpret_cast<T*>(args.o2) + o, hv, nch - c);
  } else if constexpr (EPI == EPI_SCATTER) {
    // column = the channel number (single-problem launches)
    T* out = reinterpret_cast<T*>(args.o0) + (long long)group_token(args.st, g, r) * args.ldo;
    if (is_out) {
      // dense output rows: 8 consecutive channels (16-byte stores when the row stride allows)
      if (args.ldo % 8 == 0) store_row<T, 8>(out + c, v0, nch - c);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (c + j < nch) stv<T>(out, c + j, v0[j]);
      }
    } else {
      scatter_row8<T>(out, args.idx + (long long)g * args.kidx, c, nch, args.swidth, v0, args.ldo % 8 == 0);
    }
  } else {   // EPI_DSWIGLU
    float gv[8], uv[8], dg[8], du[8];
    load_row<T, 8>(reinterpret_cast<const T*>(args.i0) + o, gv, nch - c);
    load_row<T, 8>(reinterpret_cast<const T*>(args.i1) + o, uv, nch - c);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float sg = (sizeof(T) == 4) ? sigmoid_exact(gv[j]) : sigmoidf_(gv[j]);
      dg[j] = v0[j] * uv[j] * sg * (1.0f + gv[j] * (1.0f - sg));
      du[j] = v0[j] * gv[j] * sg;
    }
    store_row<T, 8>(reinterpret_cast<T*>(args.o0) + o, dg, nch - c);
    store_row<T, 8>(reinterpret_cast<T*>(args.o1) + o, du, nch - c);
  }
}

bool timer_on();
void timer_begin(int slot, hipStream_t s);
void timer_end(int slot, hipStream_t s);
int device_cus();

// N-gather tiles of a launch (all groups) at bm rows and bnc channels per tile.
inline long long ng_tiles(const SeqTab& st, int kidx, int n_out, int bnc, int bm = G_BM) {
  long long total = 0;
  for (int g = 0; g <= st.nseq; ++g) {
    const bool is_out = g == st.nseq;
    const int m = is_out ? st.T_out : st.ctx[g];
    const int nch = is_out ? n_out : kidx;
    if (m <= 0 || nch <= 0) continue;
    total += (long long)((m + bm - 1) / bm) * ((nch + bnc - 1) / bnc);
  }
  return total;
}

// Split of the last, partial round of an N-gather grid: with `slots` resident
// workgroups, the remainder tiles (total mod slots, or every tile when the
// grid is under half a round; if at most half the slots) run as `split` K
// pieces each so that the round is filled.  split = 1: none.
inline void ng_split_plan(long long total, int total_kt, int slots, int& rem_start, int& split) {
  rem_start = (int)total;
  split = 1;
  if (slots <= 0 || total <= 0) return;
  // a grid under half a round splits every tile; otherwise the last round's
  // tiles split when that round is at most half full
  const long long rem = total <= slots ? total : total % slots;
  if (rem == 0 || 2 * rem > slots) return;
  int s = (int)(slots / rem);
  if (s > 8) s = 8;
  if (s > total_kt / 4) s = total_kt / 4;
  if (s < 2) return;
  split = s;
  rem_start = (int)(total - rem);
}

// Workgroup slots of a gather-GEMM variant on the current device: two 128 x 256
// workgroups, or one wide 128 x 512 or tall 256 x 256 workgroup, per CU.
inline int gemm_slots(int wn, int bm = G_BM) { return (wn == 4 || bm > 128 ? 1 : 2) * device_cus(); }

// Rounds of resident workgroups an N-gather grid of `total` tiles takes: its
// whole rounds, plus the last partial round at the length of one K piece when
// ng_split_plan splits it (can_split: the launch may split).
inline double ng_grid_rounds(long long total, int total_kt, int slots, bool can_split) {
  if (total <= 0 || slots <= 0) return 0.0;
  int rs = (int)total, sp = 1;
  if (can_split) ng_split_plan(total, total_kt, slots, rs, sp);
  if (sp > 1) return (double)(rs / slots) + 1.0 / sp;
  return (double)((total + slots - 1) / slots);
}

// Rounds of resident workgroups a grid of `total` tiles takes: a last round at
// most half full runs as K pieces (ng_split_plan) and counts by its fill.
inline double grid_rounds(long long total, int slots) {
  if (slots <= 0 || total <= 0) return 0.0;
  const long long full = total / slots, rem = total % slots;
  if (full == 0) return 1.0;
  return (double)full + (2 * rem <= slots ? (double)rem / slots : 1.0);
}

// GEMM variants the calling thread allows (bit mask): bit 0 = wide 128 x 512
// N-gather tiles, bit 1 = tall 256 x 256 tiles (K-gather and N-gather), bit 2 =
// tall tiles whatever their grid (tests); 0 = 128 x 256 tiles only.  Default: wide and
// tall.  The LDS-DMA variants need 16-byte aligned operands.
enum { GV_WIDE = 1, GV_TALL = 2, GV_TALL_ALWAYS = 4 };
inline thread_local int g_gemm_variants = GV_WIDE | GV_TALL;

// K-tiles of a set of N-gather segments (fixed lengths) at depth bk.
inline int ng_ktiles(std::initializer_list<int> seg_k, int bk) {
  int n = 0;
  for (int k : seg_k) n += (k + bk - 1) / bk;
  return n;
}

// Floats of partial tiles a split N-gather launch needs (0 when it does not
// split): the larger of the two variants, since the variant is chosen per launch.
inline long long ng_rpart_floats(const SeqTab& st, int kidx, int n_out, bool dual, int esz,
                                 std::initializer_list<int> seg_k) {
  long long best = 0;
  // (tile rows, waves in N) of the narrow, wide and tall N-gather variants
  const int vars[3][2] = {{G_BM, 2}, {G_BM, 4}, {G_BM_TALL, 2}};
  for (int v = 0; v < (esz == 2 ? 3 : 1); ++v) {
    const int bm = vars[v][0], wn = vars[v][1];
    const int bn = 128 * wn;
    const int bk = esz == 2 ? 64 : 32;
    int rs, sp;
    const long long total = ng_tiles(st, kidx, n_out, dual ? bn / 2 : bn, bm);
    ng_split_plan(total, ng_ktiles(seg_k, bk), gemm_slots(wn, bm), rs, sp);
    const long long f = sp > 1 ? (total - rs) * sp * (long long)bm * bn : 0;
    if (f > best) best = f;
  }
  return best;
}

// Whether every operand of an N-gather launch suits the wide variant's 16-byte
// LDS-DMA loads: 16-byte aligned bases and row starts, K a multiple of 8.
inline bool wide_ng_ok(const GemmArgs& a, int esz) {
  if (esz != 2) return false;
  auto al = [](const void* p, long long off_el) {
    return ((uintptr_t)p + (uintptr_t)(off_el * 2)) % 16 == 0;
  };
  for (int s = 0; s < a.nseg; ++s) {
    const GSeg& g = a.seg[s];
    if (g.K <= 0 || g.K % 8 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0) return false;
    if (!g.a_tok && (g.lda_out % 8 != 0 || g.a_out_off % 8 != 0)) return false;
    for (int p = 0; p < a.nprob; ++p) {
      if (!al(g.A, a.prob[p].a_col[s]) || !al(a.prob[p].B[s], 0)) return false;
    }
    if (g.B2 && !al(g.B2, 0)) return false;
  }
  return true;
}

// Whether a bf16 N-gather launch whose operands suit the LDS-DMA loads
// (wide_ng_ok) takes the tall 256 x 256 tiles: its grid, priced as rounds of
// resident workgroups times the operand bytes a CU moves per K-tile (tall: one
// 64 KB workgroup; wide: one of 80 KB; 128 x 256: two of 48 KB), costs less
// than that of the other variant allowed.  The 256-row tiles leave rows idle
// in a group whose row count is not a multiple of 256 (a 384-row context
// group fills 3 of its 4 row halves), which the price counts in full.
inline bool tall_ng_ok(const GemmArgs& a, bool dual, bool can_split, bool wide, bool always) {
  if (always) return true;
  int total_kt = 0;
  for (int s = 0; s < a.nseg; ++s) total_kt += (a.seg[s].K + 63) / 64;
  auto tiles = [&](int bnc, int bm) {
    long long t = 0;
    for (int p = 0; p < a.nprob; ++p) t += ng_tiles(a.st, a.prob[p].kidx, a.prob[p].n_out, bnc, bm);
    return t;
  };
  const double rt = ng_grid_rounds(tiles(dual ? 128 : 256, G_BM_TALL), total_kt, gemm_slots(2, G_BM_TALL), can_split);
  const double ro = wide ? ng_grid_rounds(tiles(dual ? 256 : 512, G_BM), total_kt, gemm_slots(4), can_split)
                         : ng_grid_rounds(tiles(dual ? 128 : 256, G_BM), total_kt, gemm_slots(2), can_split);
  return rt > 0 && rt * 64.0 < 0.97 * ro * (wide ? 80.0 : 96.0);
}

// K-gather tiles of a launch at bm rows (256-column tiles, the output group split ksplit_out ways).
inline long long kg_tiles(const GemmArgs& a, int bm) {
  const long long ntn = (a.N + G_BN - 1) / G_BN;
  long long total = 0;
  for (int g = 0; g <= a.st.nseq; ++g) {
    const bool is_out = g == a.st.nseq;
    const int m = is_out ? a.st.T_out : a.st.ctx[g];
    if (m > 0) total += (long long)((m + bm - 1) / bm) * ntn * (is_out ? a.ksplit_out : 1);
  }
  return total;
}

// Whether a bf16 K-gather launch takes the tall 256-row LDS-DMA tiles: its
// operands suit the LDS-DMA loads, and its grid, priced as rounds of resident
// workgroups times the operand bytes a CU moves per K-tile (tall: one 64 KB
// workgroup; narrow: two of 48 KB), costs less.
inline bool tall_kg_ok(const GemmArgs& a, bool always) {
  auto al = [](const void* p, long long off_el) {
    return ((uintptr_t)p + (uintptr_t)(off_el * 2)) % 16 == 0;
  };
  for (int s = 0; s < a.nseg; ++s) {
    const GSeg& g = a.seg[s];
    if (g.lda % 8 != 0 || g.ldb % 8 != 0) return false;
    if (!g.a_tok && (g.lda_out % 8 != 0 || g.a_out_off % 8 != 0)) return false;
    if (!al(g.A, 0) || !al(g.B, 0)) return false;
  }
  if (a.N % 8 != 0 || a.nprob > 1) return false;
  if (always) return true;
  const double rt = grid_rounds(kg_tiles(a, G_BM_TALL), gemm_slots(2, G_BM_TALL));
  const double rn = grid_rounds(kg_tiles(a, G_BM), gemm_slots(2));
  return rt > 0 && rt * 64.0 < 0.97 * rn * 96.0;
}

// Host side: count tiles per group and launch one variant.
template <typename T, int MODE, int EPI, bool DUAL, int BM, int WN, bool QB>
hipError_t launch_gather_gemm_wn(GemmArgs& a, hipStream_t stream, int timer_slot) {
  constexpr int BN_T = 128 * WN;
  constexpr int BNC = DUAL ? BN_T / 2 : BN_T;
  constexpr int BK = GTraits<T>::BK;
  constexpr bool TALL = BM > 128;
  const int gpp = a.st.nseq + 1;
  a.ngroups = a.nprob * gpp;
  int total = 0;
  for (int q = 0; q < a.ngroups; ++q) {
    a.tile_start[q] = total;
    const GProb& pr = a.prob[q / gpp];
    const int g = q % gpp;
    const bool is_out = g == a.st.nseq;
    const int m = is_out ? a.st.T_out : a.st.ctx[g];
    const int nch = is_out ? pr.n_out : pr.kidx;
    if (m <= 0 || (MODE == MODE_NG && nch <= 0)) continue;
    const int ntm = (m + BM - 1) / BM;
    int ntn, nks;
    if (MODE == MODE_NG) { ntn = (nch + BNC - 1) / BNC; nks = 1; }
    else { ntn = (a.N + G_BN - 1) / G_BN; nks = is_out ? a.ksplit_out : 1; }
    total += ntm * ntn * nks;
  }
  a.tile_start[a.ngroups] = total;
  a.ntiles = total;
  a.rem_start = total;
  a.rem_split = 1;
  if (total == 0) return hipSuccess;
  long long grid = total;
  if constexpr (MODE == MODE_NG && (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU || EPI == EPI_SCATTER)) {
    if (a.rpart && a.nprob == 1) {
      int total_kt = 0;
      for (int s = 0; s < a.nseg; ++s) total_kt += (a.seg[s].K + BK - 1) / BK;   // NG segments: fixed K
      ng_split_plan(total, total_kt, gemm_slots(WN, BM), a.rem_start, a.rem_split);
      grid = a.rem_start + (long long)(total - a.rem_start) * a.rem_split;
    }
  }
  timer_begin(timer_slot, stream);
  hipLaunchKernelGGL((gather_gemm_kernel<T, MODE, EPI, DUAL, BM, WN, QB>), dim3((unsigned)grid),
                     dim3((WN == 4 || TALL) ? 512 : G_THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if constexpr (MODE == MODE_NG && (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU || EPI == EPI_SCATTER)) {
    if (e == hipSuccess && a.rem_split > 1) {
      constexpr int CG = BNC / 8;
      const long long n = (long long)(total - a.rem_start) * BM * CG;
      hipLaunchKernelGGL((ng_fixup_kernel<T, EPI, DUAL, WN, BM>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                         0, stream, a);
      e = hipGetLastError();
    }
  }
  timer_end(timer_slot, stream);
  return e;
}

template <typename T, int MODE, int EPI, bool DUAL>
hipError_t launch_gather_gemm(GemmArgs& a, hipStream_t stream, int timer_slot) {
  if (a.nprob <= 0) {
    a.nprob = 1;
    GProb& p0 = a.prob[0];
    p0.idx = a.idx; p0.kidx = a.kidx; p0.n_out = a.n_out;
    for (int s = 0; s < G_MAXSEG; ++s) { p0.B[s] = a.seg[s].B; p0.Bs[s] = a.seg[s].Bs; p0.a_col[s] = 0; }
    p0.o0 = a.o0; p0.ldo = a.ldo; p0.swidth = a.swidth;
  }
  if (a.nprob > G_MAXPROB || (a.nprob > 1 && (MODE != MODE_NG || EPI != EPI_SCATTER)))
    return hipErrorInvalidValue;
  bool quant = false;
  for (int s = 0; s < a.nseg; ++s) quant |= a.seg[s].bq4 != 0;
  if constexpr (sizeof(T) == 2) {
    if (quant) return launch_gather_gemm_wn<T, MODE, EPI, DUAL, G_BM, 2, true>(a, stream, timer_slot);
  } else {
    if (quant) return hipErrorInvalidValue;   // 4-bit weights: bf16 launches only
  }
  if constexpr (sizeof(T) == 2 && MODE == MODE_KG) {
    if ((g_gemm_variants & GV_TALL) && tall_kg_ok(a, (g_gemm_variants & GV_TALL_ALWAYS) != 0))
      return launch_gather_gemm_wn<T, MODE, EPI, DUAL, G_BM_TALL, 2, false>(a, stream, timer_slot);
  }
  if constexpr (MODE == MODE_NG && sizeof(T) == 2) {
    if ((g_gemm_variants & (GV_WIDE | GV_TALL)) && wide_ng_ok(a, 2)) {
      constexpr bool SPLITS = EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU || EPI == EPI_SCATTER;
      const bool wide = (g_gemm_variants & GV_WIDE) != 0;
      if ((g_gemm_variants & GV_TALL) &&
          tall_ng_ok(a, DUAL, SPLITS && a.rpart && a.nprob == 1, wide, (g_gemm_variants & GV_TALL_ALWAYS) != 0))
        return launch_gather_gemm_wn<T, MODE, EPI, DUAL, G_BM_TALL, 2, false>(a, stream, timer_slot);
      if (wide) return launch_gather_gemm_wn<T, MODE, EPI, DUAL, G_BM, 4, false>(a, stream, timer_slot);
    }
  }
  return launch_gather_gemm_wn<T, MODE, EPI, DUAL, G_BM, 2, false>(a, stream, timer_slot);
}

}  // namespace sl
