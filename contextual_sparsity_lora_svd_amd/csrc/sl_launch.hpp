// Launch helpers shared by the entry points.
#pragma once

#include "sl_gemm.hpp"
#include "sl_host.hpp"
#include "sl_small.hpp"

namespace sl {

// Workgroup layout of a skinny product: row blocks of SK_RB rows, each cut
// into K slices of about SK_SLICE_BYTES per row (so long rows spread over more
// workgroups).  Returns the number of workgroups.
inline int skinny_layout(SkinnyArgs& a, int esz) {
  const SeqTab& st = a.st;
  int ng;
  if (a.mode == 0) ng = 1;
  else if (a.mode == 1) ng = st.nseq + 1;
  else ng = st.nseq;
  a.ngroups = ng;
  a.mrows = a.mode == 0 ? a.T : (a.mode == 1 ? st.T_ctx + st.T_out : st.T_ctx);
  const int kc = SK_CB / esz, target = SK_SLICE_BYTES / esz;
  int nb = 0;
  for (int g = 0; g < ng; ++g) {
    a.blk_start[g] = nb;
    int m, K;
    if (a.mode == 0) { m = a.T; K = a.K; }
    else {
      const bool is_out = a.mode == 1 && g == st.nseq;
      m = is_out ? st.T_out : st.ctx[g];
      K = a.K > 0 ? a.K : (is_out ? a.n_out : a.kidx);
    }
    int nsl = K > target ? ceil_div(K, target) : 1;
    if (nsl > SK_MAXSL) nsl = SK_MAXSL;
    const int ksl = (int)round_up(ceil_div(K > 0 ? K : 1, nsl), kc);
    nsl = K > 0 ? ceil_div(K, ksl) : 1;   // no empty slices
    a.nsl[g] = nsl;
    a.ksl[g] = ksl;
    nb += ceil_div(m, SK_RB) * nsl;
  }
  a.blk_start[ng] = nb;
  return nb;
}

// Floats of partial sums a skinny product over at most T rows and K <= Kmax
// may need (any element size up to 4 bytes).
inline long long skinny_part_floats(long long T, long long Kmax) {
  long long nsl = (Kmax * 4 + SK_SLICE_BYTES - 1) / SK_SLICE_BYTES;
  if (nsl < 1) nsl = 1;
  if (nsl > SK_MAXSL) nsl = SK_MAXSL;
  return nsl > 1 ? nsl * T * SK_PC : 0;
}

template <typename T>
inline sl_status launch_skinny_one(SkinnyArgs& a, hipStream_t s) {
  int C = 0;
  for (int j = 0; j < a.nblk; ++j) C += a.nbk[j];
  const int nblocks = skinny_layout(a, (int)sizeof(T));
  if (nblocks <= 0 || C <= 0) return SL_OK;
  if (a.nprob < 1) a.nprob = 1;
  if (a.nprob > SK_MAXPROB) SL_FAIL(SL_ERR_SHAPE, "internal: %d > %d skinny problems", a.nprob, SK_MAXPROB);
  if ((long long)nblocks * a.nprob > 0x7FFFFFFFLL) SL_FAIL(SL_ERR_SHAPE, "skinny grid too large");
  a.pc = (C + 15) / 16 * 16;
  bool sliced = false;
  for (int g = 0; g < a.ngroups; ++g) sliced |= a.nsl[g] > 1;
  if (sliced && !a.part) SL_FAIL(SL_ERR_NULL, "internal: K-sliced skinny product without scratch");
  const dim3 grid(nblocks * a.nprob), block(SK_THREADS);
  if (C <= 16) hipLaunchKernelGGL((skinny_kernel<T, 1>), grid, block, 0, s, a);
  else if (C <= 32) hipLaunchKernelGGL((skinny_kernel<T, 2>), grid, block, 0, s, a);
  else if (C <= 48) hipLaunchKernelGGL((skinny_kernel<T, 3>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((skinny_kernel<T, 4>), grid, block, 0, s, a);
  SL_HIP(hipGetLastError());
  if (sliced) {
    int ptot = 0;
    for (int j = 0; j < a.nblk; ++j) ptot += (a.nbk[j] + 7) / 8 * 8;
    hipLaunchKernelGGL((skinny_finish_kernel<T>), grid1d((long long)a.mrows * ptot * a.nprob), dim3(256), 0,
                       s, a);
    SL_HIP(hipGetLastError());
  }
  return SL_OK;
}

// Skinny product over any number of B blocks: blocks are grouped into launches
// of at most 64 columns; each launch writes its padded column range.
template <typename T>
inline sl_status launch_skinny(SkinnyArgs& a, hipStream_t s) {
  int C = 0;
  for (int j = 0; j < a.nblk; ++j) C += a.nbk[j];
  if (C <= 64) return launch_skinny_one<T>(a, s);
  if (a.mode == 1) SL_FAIL(SL_ERR_SHAPE, "per-group skinny product with %d > 64 columns", C);
  if (a.nprob > 1) SL_FAIL(SL_ERR_SHAPE, "internal: multi-problem skinny product with %d > 64 columns", C);
  int j = 0, col = a.col0;
  while (j < a.nblk) {
    SkinnyArgs b = a;
    b.nblk = 0;
    int c = 0, pc = 0;
    while (j < a.nblk && b.nblk < 4 && c + a.nbk[j] <= 64) {
      b.Bb[b.nblk] = a.Bb[j]; b.nbk[b.nblk] = a.nbk[j]; b.ldbb[b.nblk] = a.ldbb[j];
      c += a.nbk[j];
      pc += (a.nbk[j] + 7) / 8 * 8;
      ++b.nblk;
      ++j;
    }
    if (b.nblk == 0) SL_FAIL(SL_ERR_SHAPE, "skinny block with %d > 64 columns", a.nbk[j]);
    b.col0 = col;
    sl_status rc = launch_skinny_one<T>(b, s);
    if (rc != SL_OK) return rc;
    col += pc;
  }
  return SL_OK;
}

// Split-K of a K-gather launch's output group, whose K (every channel) is much
// longer than a context group's (its selected channels).  Pieces balanced
// against the context tiles: round(K_out / K_ctx).  When the context tiles
// take at most half a round of the machine, the pieces are capped so that the
// whole launch fits one round: past that, more pieces add fp32 partial traffic
// and a second round, not balance (down product at 99 % sparsity, 4 x 512
// tokens: 4 pieces 114 us, 8 pieces 127 us, 16 pieces 132 us).  Tile geometry:
// the tall 256 x 256 tile (one per CU) for bf16, 128 x 256 (two per CU) else.
inline int kg_choose_ksplit(const SeqTab& st, long long K_ctx, long long K_out, long long N, int bk, bool tall) {
  if (st.T_out == 0) return 1;
  const long long kt_out = (K_out + bk - 1) / bk;
  const int bm = tall ? G_BM_TALL : G_BM;
  int cus = device_cus();
  if (cus <= 0) cus = 256;
  const long long slots = (tall ? 1 : 2) * (long long)cus;
  const long long ntn = (N + G_BN - 1) / G_BN;
  long long ctx_tiles = 0;
  for (int b = 0; b < st.nseq; ++b) ctx_tiles += (st.ctx[b] + bm - 1) / bm * ntn;
  const long long out_tiles = (st.T_out + bm - 1) / bm * ntn;
  long long ks;
  if (st.T_ctx > 0 && K_ctx > 0) ks = (K_out + K_ctx / 2) / K_ctx;
  else ks = slots / (out_tiles > 0 ? out_tiles : 1);
  if (2 * ctx_tiles <= slots && out_tiles > 0) {
    long long fill = (slots - ctx_tiles) / out_tiles;
    if (fill < 1) fill = 1;
    if (ks > fill) ks = fill;
  }
  if (ks > kt_out / 8) ks = kt_out / 8;
  if (ks > 16) ks = 16;
  if (ks < 1) ks = 1;
  return (int)ks;
}

// Token rows per column-reduction chunk and the padded width of its partials.
inline int cr_chunk(size_t esz) { return esz == 2 ? CRM_CHUNK : CR_CHUNK; }
inline int cr_rm(size_t esz, int R) {
  const int rm = pow2_rm(R);
  return (esz == 2 && rm < 16) ? 16 : rm;
}

template <typename T>
inline sl_status launch_colred(ColredArgs& a, int nchunks_total, int nmax, int RM, hipStream_t s) {
  if (nchunks_total <= 0 || nmax <= 0) return SL_OK;
  if (sizeof(T) == 2) SL_FAIL(SL_ERR_DTYPE, "internal: bf16 column reductions run batched");
  const dim3 grid(ceil_div(nmax, 2 * CR_THREADS), nchunks_total), block(CR_THREADS);
  switch (RM) {
    case 8: hipLaunchKernelGGL((colred_kernel<T, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((colred_kernel<T, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((colred_kernel<T, 32>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((colred_kernel<T, 64>), grid, block, 0, s, a); break;
  }
  SL_HIP(hipGetLastError());
  return SL_OK;
}

// Builder of one pack launch.
struct Packer {
  PackArgs a;
  PackJob spare;        // target of jobs beyond the limit (reported by launch)
  bool overflow = false;
  Packer() { std::memset(&a, 0, sizeof(a)); }
  PackJob& next() {
    if (a.njobs >= PK_MAXJOBS) { overflow = true; return spare; }
    return a.job[a.njobs++];
  }
  // dst region [rows x cols] (row stride ldd) holding src block at (row_off, col_off)
  void copy(void* dst, long long ldd, int rows, int cols, const void* src, long long lds,
            int src_rows, int src_cols, int tr, int row_off = 0, int col_off = 0) {
    PackJob& j = next();
    j.type = 0; j.dst = dst; j.ldd = ldd; j.rows = rows; j.cols = cols;
    j.row_off = row_off; j.col_off = col_off;
    j.src = src; j.lds = lds; j.src_rows = src_rows; j.src_cols = src_cols; j.tr = tr;
  }
  // per context group g: dst + g*gstride, [rows x cols], src factor gathered by idx
  void gather(void* dst, long long ldd, long long gstride, int rows, int cols, const void* src,
              long long lds, int src_rows, int tr, const int* idx, int k, int nseq) {
    PackJob& j = next();
    j.type = 1; j.dst = dst; j.ldd = ldd; j.gstride = gstride; j.rows = rows; j.cols = cols;
    j.src = src; j.lds = lds; j.src_rows = src_rows; j.tr = tr; j.idx = idx; j.k = k; j.nseq = nseq;
  }
  // int32 identity rows 0 .. n-1
  void iota(int* dst, int n) {
    PackJob& j = next();
    j.type = 2; j.dst = dst; j.rows = 1; j.cols = n;
  }
  // inv [nseq, n] <- positions of channels 0..n-1 in the ascending sets idx [nseq, k]
  void inverse(int* inv, const int* idx, int k, int n, int nseq) {
    PackJob& j = next();
    j.type = 3; j.dst = inv; j.rows = 1; j.cols = n; j.idx = idx; j.k = k; j.nseq = nseq;
  }
  template <typename T>
  sl_status launch(hipStream_t s) {
    if (overflow) SL_FAIL(SL_ERR_SHAPE, "internal: more than %d pack jobs", PK_MAXJOBS);
    long long n = 0;
    for (int i = 0; i < a.njobs; ++i) {
      a.start[i] = n;
      const PackJob& j = a.job[i];
      // items of 8 consecutive destination elements of a row (inverse maps: 1)
      const int per = j.type == 3 ? 1 : 8;
      n += (long long)j.rows * ((j.cols + per - 1) / per) * (j.type == 1 || j.type == 3 ? j.nseq : 1);
    }
    a.start[a.njobs] = n;
    if (n == 0) return SL_OK;
    hipLaunchKernelGGL((pack_kernel<T>), grid1d(n), dim3(256), 0, s, a);
    SL_HIP(hipGetLastError());
    return SL_OK;
  }
};

// Builder of one row-layout launch.
struct Layouter {
  LayArgs a;
  bool overflow = false;
  explicit Layouter(const SeqTab& st) { std::memset(&a, 0, sizeof(a)); a.st = st; }
  LayJob* next() {
    if (a.njobs >= LJ_MAXJOBS) { overflow = true; return nullptr; }
    return &a.job[a.njobs++];
  }
  static int vec_ok(const void* p, long long ld) {
    return ((reinterpret_cast<uintptr_t>(p) & 15) == 0) && (ld % 8 == 0);
  }
  // context rows of token-major out [T, ld], columns [0, n) := 0
  void zero_ctx(void* out, long long ld, int n) {
    if (a.st.T_ctx == 0 || n <= 0) return;
    LayJob* j = next();
    if (!j) return;
    j->type = LJ_ZERO; j->n = n; j->dst = out; j->ldd = ld;
    j->vec = vec_ok(out, ld);
  }
  // compact copy of a [T, lds] buffer whose rows hold n channels: context
  // rows' columns idx[b][0..k) at row stride ldc, then the output rows' n
  // columns at dst + out_off, row stride n
  void compact(const void* src, long long lds, const int* idx, int k, int n, void* dst, long long ldc,
               long long out_off, size_t esz) {
    if (a.st.T_ctx > 0 && k > 0) {
      LayJob* j = next();
      if (!j) return;
      j->type = LJ_GATHER; j->n = k; j->nsrc = n; j->dst = dst; j->ldd = ldc; j->src = src; j->lds = lds;
      j->idx = idx; j->vec = vec_ok(dst, ldc);
      j->stage = vec_ok(src, lds) && n % 8 == 0 && (long long)n * (long long)esz <= LJ_STAGE_BYTES;
    }
    if (a.st.T_out > 0 && n > 0) {
      LayJob* j = next();
      if (!j) return;
      void* d = static_cast<char*>(dst) + out_off * (long long)esz;
      j->type = LJ_ROWS; j->n = n; j->dst = d; j->ldd = n; j->src = src; j->lds = lds;
      j->vec = vec_ok(d, n) && vec_ok(src, lds);
    }
  }
  static constexpr long long LJ_STAGE_BYTES = 64 * 1024;
  template <typename T>
  sl_status launch(hipStream_t s) {
    if (overflow) SL_FAIL(SL_ERR_SHAPE, "internal: more than %d layout jobs", LJ_MAXJOBS);
    long long rows = 0;
    size_t shm = 0;
    for (int i = 0; i < a.njobs; ++i) {
      LayJob& j = a.job[i];
      j.row0 = (int)rows;
      rows += j.type == LJ_ROWS ? a.st.T_out : a.st.T_ctx;
      if (j.type == LJ_GATHER && j.stage) shm = std::max(shm, (size_t)j.nsrc * sizeof(T));
    }
    if (rows == 0) return SL_OK;
    if (rows > 0x7FFFFFFFLL) SL_FAIL(SL_ERR_SHAPE, "layout grid too large");
    a.nrows = (int)rows;
    hipLaunchKernelGGL((layout_kernel<T>), dim3((unsigned)rows), dim3(LJ_THREADS), shm, s, a);
    SL_HIP(hipGetLastError());
    return SL_OK;
  }
};


template <typename T>
inline sl_status splitk_reduce(const SeqTab& st, const float* part, int ks, int N, void* out,
                               long long ldo, hipStream_t s) {
  const long long n = (long long)st.T_out * (N / 4);   // N is a multiple of 8
  if (n <= 0 || ks <= 1) return SL_OK;
  hipLaunchKernelGGL((splitk_reduce_kernel<T>), grid1d(n), dim3(256), 0, s, st, part, ks, N,
                     reinterpret_cast<T*>(out), ldo);
  SL_HIP(hipGetLastError());
  return SL_OK;
}

// Chunks of the column reduction per group (mode 1).
inline int colred_chunks_compact(const SeqTab& st, ColredArgs& a, int kidx, int n_out, int RM,
                                 int chunk) {
  int nc = 0;
  long long off = 0;
  for (int g = 0; g <= st.nseq; ++g) {
    a.chunk_start[g] = nc;
    a.part_off[g] = off;
    const int m = g < st.nseq ? st.ctx[g] : st.T_out;
    const int c = ceil_div(m, chunk);
    nc += c;
    off += (long long)c * (g < st.nseq ? kidx : n_out) * RM;
  }
  a.chunk_start[st.nseq + 1] = nc;
  a.part_off[st.nseq + 1] = off;
  a.ngroups = st.nseq + 1;
  return nc;
}

inline long long colred_part_elems_compact(const SeqTab& st, int kidx, int n_out, int RM,
                                           int chunk) {
  long long off = 0;
  for (int g = 0; g <= st.nseq; ++g) {
    const int m = g < st.nseq ? st.ctx[g] : st.T_out;
    off += (long long)ceil_div(m, chunk) * (g < st.nseq ? kidx : n_out) * RM;
  }
  return off;
}

// Partial-row width of a column-reduction job with R Z columns.
inline int cb_rm(size_t esz, int R) { return esz == 2 ? (int)round_up(R, 16) : pow2_rm(R); }

// Floats of partials of a dense job (token rows) and of a scatter job (compact rows).
inline long long cb_dense_floats(const SeqTab& st, size_t esz, int N, int R) {
  return (long long)ceil_div(st.nseq * st.L, cr_chunk(esz)) * N * cb_rm(esz, R);
}
inline long long cb_scatter_floats(const SeqTab& st, size_t esz, int kidx, int n_out, int R) {
  return colred_part_elems_compact(st, kidx, n_out, cb_rm(esz, R), cr_chunk(esz));
}

// Builder of the LoRA-gradient column reductions of one backward pass: jobs
// take consecutive ranges of the partial buffer; bf16 runs all reductions in
// one launch and all finishes in another, fp32 runs each job's reduction and
// finish in turn.
struct ColredBatch {
  CbArgs c;
  FbArgs f;
  const void* P32[CB_MAXJOBS];
  float* part; long long cap, used = 0;
  size_t esz;
  bool overflow = false;
  ColredBatch(const SeqTab& st, size_t esz_, float* part_, long long cap_) : part(part_), cap(cap_), esz(esz_) {
    std::memset(&c, 0, sizeof(c));
    std::memset(&f, 0, sizeof(f));
    c.st = st; f.st = st;
    c.T = st.nseq * st.L;
  }
  bool take(long long n, float*& p) {
    if (c.njobs >= CB_MAXJOBS || used + n > cap) { overflow = true; return false; }
    p = part + used;
    used += n;
    return true;
  }
  // out1 (r1 columns of Z from zc0) and optionally out2 (columns zc0+off2 ..):
  // out[n, q] (transposed: [q, n]) = scale * sum over all tokens P[t, n] Z[t, zc0 + q]
  void dense(const void* P, long long ldp, int N, const float* Z, long long ldz, int zc0, int R,
             float* out1, int r1, int t1, float* out2, int r2, int t2, int off2, float scale) {
    float* p;
    if (!take(cb_dense_floats(c.st, esz, N, R), p)) return;
    CbJob& j = c.job[c.njobs];
    j.mode = 0; j.N = N; j.R = R; j.RM = cb_rm(esz, R);
    j.P = P; j.ldp = ldp; j.Z = Z; j.ldz = ldz; j.zc0 = zc0; j.part = p;
    FbJob& q = f.job[f.njobs];
    q.kind = 0; q.part = p; q.RM = j.RM; q.N = N; q.nchunk = ceil_div(c.T, cr_chunk(esz));
    q.out1 = out1; q.r1 = r1; q.t1 = t1; q.out2 = out2; q.r2 = r2; q.t2 = t2; q.off2 = off2; q.scale = scale;
    ++c.njobs; ++f.njobs;
  }
  // out[c, q] (transposed: [q, c]) = scale * sum over the rows whose channel
  // set holds c of P[row, pos(c)] Z[tok(row), zc0 + q], P compact
  void scatter(const void* P, long long ldp, long long ldp_out, long long p_out_off, int kidx, int n_out,
               const float* Z, long long ldz, int zc0, int R, const int* inv, float* out, int r,
               int transposed, float scale) {
    float* p;
    if (!take(cb_scatter_floats(c.st, esz, kidx, n_out, R), p)) return;
    CbJob& j = c.job[c.njobs];
    j.mode = 1; j.kidx = kidx; j.n_out = n_out; j.R = R; j.RM = cb_rm(esz, R);
    j.P = P; j.ldp = ldp; j.ldp_out = ldp_out; j.p_out_off = p_out_off;
    j.Z = Z; j.ldz = ldz; j.zc0 = zc0; j.part = p;
    FbJob& q = f.job[f.njobs];
    q.kind = 1; q.part = p; q.RM = j.RM; q.N = n_out; q.kidx = kidx; q.inv = inv;
    q.out1 = out; q.r1 = r; q.t1 = transposed; q.scale = scale;
    ++c.njobs; ++f.njobs;
  }
  template <typename T>
  sl_status launch(hipStream_t s) {
    if (overflow) SL_FAIL(SL_ERR_SHAPE, "internal: gradient reductions exceed %d jobs or the workspace", CB_MAXJOBS);
    if (c.njobs == 0) return SL_OK;
    if (sizeof(T) == 2) {
      long long items = 0, fitems = 0;
      int rmx = 16;
      for (int i = 0; i < c.njobs; ++i) {
        CbJob& j = c.job[i];
        j.item0 = items;
        if (j.mode == 0) {
          items += (long long)ceil_div(c.T, CRM_CHUNK) * ceil_div(j.N, CRM_COLS);
        } else {
          for (int g = 0; g <= c.st.nseq; ++g) {
            const int rows = g < c.st.nseq ? c.st.ctx[g] : c.st.T_out;
            const int cols = g < c.st.nseq ? j.kidx : j.n_out;
            items += (long long)ceil_div(rows, CRM_CHUNK) * ceil_div(cols, CRM_COLS);
          }
        }
        rmx = std::max(rmx, j.RM);
        FbJob& q = f.job[i];
        q.item0 = fitems;
        fitems += q.kind == 0 ? (long long)q.N * q.RM : (long long)q.N * q.r1;
      }
      c.nitems = items;
      f.nitems = fitems;
      if (items > 0) {
        if (items > 0x7FFFFFFFLL) SL_FAIL(SL_ERR_SHAPE, "gradient reduction grid too large");
        const dim3 grid((unsigned)items), block(256);
        if (rmx <= 16) hipLaunchKernelGGL((colred_batch_kernel<16>), grid, block, 0, s, c);
        else if (rmx <= 32) hipLaunchKernelGGL((colred_batch_kernel<32>), grid, block, 0, s, c);
        else if (rmx <= 64) hipLaunchKernelGGL((colred_batch_kernel<64>), grid, block, 0, s, c);
        else SL_FAIL(SL_ERR_SHAPE, "gradient reduction with %d > 64 columns", rmx);
        SL_HIP(hipGetLastError());
      }
      if (fitems > 0) {
        hipLaunchKernelGGL(finish_batch_kernel, grid1d(fitems), dim3(256), 0, s, f);
        SL_HIP(hipGetLastError());
      }
      return SL_OK;
    }
    // fp32: each job's reduction and finish with the scalar kernels
    for (int i = 0; i < c.njobs; ++i) {
      const CbJob& j = c.job[i];
      const FbJob& q = f.job[i];
      ColredArgs a;
      std::memset(&a, 0, sizeof(a));
      a.st = c.st; a.mode = j.mode; a.T = c.T;
      a.P = j.P; a.ldp = j.ldp; a.ldp_out = j.ldp_out; a.p_out_off = j.p_out_off;
      a.N = j.N; a.kidx = j.kidx; a.n_out = j.n_out;
      a.Z = j.Z; a.ldz = j.ldz; a.zc0 = j.zc0; a.R = j.R;
      a.part = j.part;
      sl_status rc;
      if (j.mode == 0) {
        const int nc = ceil_div(c.T, cr_chunk(esz));
        if ((rc = launch_colred<T>(a, nc, j.N, j.RM, s))) return rc;
        FinishArgs fa{j.part, nc, j.N, j.RM, q.out1, q.r1, q.t1, q.out2, q.r2, q.t2, q.off2, q.scale};
        hipLaunchKernelGGL(finish_dense_kernel, grid1d((long long)j.N * j.RM), dim3(256), 0, s, fa);
        SL_HIP(hipGetLastError());
      } else {
        const int nc = colred_chunks_compact(c.st, a, j.kidx, j.n_out, j.RM, cr_chunk(esz));
        if ((rc = launch_colred<T>(a, nc, std::max(j.n_out, j.kidx), j.RM, s))) return rc;
        FinishScatterArgs fs;
        std::memset(&fs, 0, sizeof(fs));
        fs.st = c.st; fs.part = j.part; fs.RM = j.RM; fs.Nfull = j.n_out; fs.kidx = j.kidx; fs.inv = q.inv;
        for (int g = 0; g <= c.st.nseq; ++g) {
          const int m = g < c.st.nseq ? c.st.ctx[g] : c.st.T_out;
          fs.chunk_count[g] = ceil_div(m, cr_chunk(esz));
          fs.part_off[g] = a.part_off[g];
        }
        fs.out = q.out1; fs.r = q.r1; fs.transposed = q.t1; fs.scale = q.scale;
        hipLaunchKernelGGL(finish_scatter_kernel, grid1d((long long)j.n_out * q.r1), dim3(256), 0, s, fs);
        SL_HIP(hipGetLastError());
      }
    }
    return SL_OK;
  }
};

}  // namespace sl
