// a1-a3: low-rank activation estimate, per-channel criterion over each
// sequence's context tokens, per-sequence top-k.
//   SparseLoRA article §一 — L2-norm criterion for the FFN, QK-norm for q/k,
//     per-input channel choice; §二 — activations estimated from the offline
//     truncated SVD of the frozen weight; §三 — only context tokens are sparse,
//     so only they vote.
#include "sl_launch.hpp"

using namespace sl;

namespace {

struct EstGeom {
  int rep, ldz, nchunk_max, chunk, N0, nproj;
  size_t w_zh, w_p0, w_p1, w_skp, total;
};

sl_status est_geom(sl_criterion crit, const SeqTab& st, const sl_heads* heads, long long d_in,
                   int rank, long long N, EstGeom& g) {
  if (crit != SL_CRIT_SWIGLU_L2 && crit != SL_CRIT_L2 && crit != SL_CRIT_QK_NORM)
    SL_FAIL(SL_ERR_DTYPE, "unknown criterion %d", (int)crit);
  if (rank < 1 || rank > 32) SL_FAIL(SL_ERR_RANGE, "estimator rank %d outside [1, 32]", rank);
  if (N < 1 || N > SEL_MAXN) SL_FAIL(SL_ERR_RANGE, "N = %lld outside [1, %d]", N, SEL_MAXN);
  g.rep = (int)round_up(rank, 8);
  g.nproj = crit == SL_CRIT_L2 ? 1 : 2;
  g.ldz = g.nproj * g.rep;
  g.N0 = (int)N;
  if (crit == SL_CRIT_QK_NORM) {
    if (!heads) SL_FAIL(SL_ERR_NULL, "heads is NULL for the QK-norm criterion");
    if (heads->n_q_heads < 1 || heads->n_kv_heads < 1 || heads->head_dim < 1 ||
        heads->n_q_heads % heads->n_kv_heads)
      SL_FAIL(SL_ERR_SHAPE, "bad heads (%d q, %d kv, dim %d)", heads->n_q_heads, heads->n_kv_heads,
              heads->head_dim);
    if ((long long)heads->n_kv_heads * heads->head_dim != N)
      SL_FAIL(SL_ERR_SHAPE, "QK-norm selects over n_kv_heads*head_dim = %d channels, N = %lld",
              heads->n_kv_heads * heads->head_dim, N);
    g.N0 = heads->n_q_heads * heads->head_dim;
  }
  int maxctx = 0;
  for (int b = 0; b < st.nseq; ++b) maxctx = st.ctx[b] > maxctx ? st.ctx[b] : maxctx;
  // SwiGLU partials per SW_CHUNK tokens; the L2 forms (Gram) one per sequence
  g.chunk = crit == SL_CRIT_SWIGLU_L2 ? SW_CHUNK : (1 << 30);
  g.nchunk_max = crit == SL_CRIT_SWIGLU_L2 ? ceil_div(maxctx, SW_CHUNK) : 1;
  if (g.nchunk_max < 1) g.nchunk_max = 1;
  const long long T = (long long)st.nseq * st.L;
  Bump bp;
  g.w_zh = bp.take((size_t)T * g.ldz * 4);
  g.w_p0 = bp.take((size_t)st.nseq * g.nchunk_max * g.N0 * 4);
  g.w_p1 = bp.take(crit == SL_CRIT_QK_NORM ? (size_t)st.nseq * g.nchunk_max * N * 4 : 0);
  g.w_skp = bp.take((size_t)skinny_part_floats(T, d_in) * 4);   // K-sliced stage 1
  g.total = bp.off;
  return SL_OK;
}

template <typename T>
sl_status launch_swiglu(const SwiArgs& a, int nseq, int rank, hipStream_t s) {
  const dim3 grid(ceil_div(a.N, 128), a.nchunk_max, nseq), block(SW_THREADS);
  if (rank <= 8) hipLaunchKernelGGL((score_swiglu_kernel<T, 8>), grid, block, 0, s, a);
  else if (rank <= 16) hipLaunchKernelGGL((score_swiglu_kernel<T, 16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((score_swiglu_kernel<T, 32>), grid, block, 0, s, a);
  SL_HIP(hipGetLastError());
  return SL_OK;
}

template <typename T>
sl_status launch_gram(const GramArgs& a, int nproj, int nseq, int rank, hipStream_t s) {
  const int nmax = nproj > 1 && a.N[1] > a.N[0] ? a.N[1] : a.N[0];
  const dim3 grid(ceil_div(nmax, GR_THREADS), nseq, nproj), block(GR_THREADS);
  if (rank <= 8) hipLaunchKernelGGL((score_gram_kernel<T, 8>), grid, block, 0, s, a);
  else if (rank <= 16) hipLaunchKernelGGL((score_gram_kernel<T, 16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((score_gram_kernel<T, 32>), grid, block, 0, s, a);
  SL_HIP(hipGetLastError());
  return SL_OK;
}

sl_status launch_select(const SelectArgs& a, int nseq, hipStream_t s) {
  const size_t lds = (size_t)a.N * 4;
  static bool attr_set = false;
  if (!attr_set) {
    SL_HIP(hipFuncSetAttribute((const void*)select_kernel,
                               hipFuncAttributeMaxDynamicSharedMemorySize, SEL_MAXN * 4));
    attr_set = true;
  }
  timer_begin(TS_SELECT, s);
  hipLaunchKernelGGL(select_kernel, dim3(nseq), dim3(SEL_THREADS), lds, s, a);
  timer_end(TS_SELECT, s);
  SL_HIP(hipGetLastError());
  return SL_OK;
}

template <typename T>
sl_status estimate_select_impl(sl_criterion crit, const SeqTab& st, const sl_heads* heads,
                               const void* X, long long d_in, int rank, const void* Pt0,
                               const void* Q0, const void* Pt1, const void* Q1, long long N, int k,
                               int32_t* idx, float* scores, char* ws, const EstGeom& g,
                               hipStream_t stream) {
  float* zh = reinterpret_cast<float*>(ws + g.w_zh);
  float* p0 = reinterpret_cast<float*>(ws + g.w_p0);
  float* p1 = reinterpret_cast<float*>(ws + g.w_p1);
  timer_begin(TS_ESTIMATE, stream);
  if (st.T_ctx > 0) {
    // stage 1: Zh = X_ctx [Pt0; Pt1]^T on the context rows
    SkinnyArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.st = st;
    sa.mode = 2;
    sa.T = st.nseq * st.L;
    sa.A = X; sa.lda = d_in;
    sa.K = (int)d_in;
    sa.nblk = g.nproj;
    sa.Bb[0] = Pt0; sa.nbk[0] = rank; sa.ldbb[0] = d_in;
    sa.Bb[1] = Pt1; sa.nbk[1] = g.nproj > 1 ? rank : 0; sa.ldbb[1] = d_in;
    sa.out = zh; sa.ldo = g.ldz; sa.col0 = 0; sa.oscale = 1.f;
    sa.part = reinterpret_cast<float*>(ws + g.w_skp);
    sl_status s = launch_skinny<T>(sa, stream);
    if (s != SL_OK) return s;
    // stage 2 + criterion
    if (crit == SL_CRIT_SWIGLU_L2) {
      SwiArgs sc;
      std::memset(&sc, 0, sizeof(sc));
      sc.st = st;
      sc.Zh = zh; sc.ldz = g.ldz; sc.zc0 = 0; sc.zc1 = g.rep;
      sc.Q0 = Q0; sc.Q1 = Q1; sc.rank = rank; sc.N = (int)N;
      sc.part = p0; sc.nchunk_max = g.nchunk_max;
      if ((s = launch_swiglu<T>(sc, st.nseq, rank, stream)) != SL_OK) return s;
    } else {
      GramArgs ga;
      std::memset(&ga, 0, sizeof(ga));
      ga.st = st;
      ga.Zh = zh; ga.ldz = g.ldz; ga.rank = rank;
      ga.zc[0] = 0; ga.Q[0] = Q0; ga.N[0] = g.N0; ga.part[0] = p0;
      if (crit == SL_CRIT_QK_NORM) { ga.zc[1] = g.rep; ga.Q[1] = Q1; ga.N[1] = (int)N; ga.part[1] = p1; }
      if ((s = launch_gram<T>(ga, crit == SL_CRIT_QK_NORM ? 2 : 1, st.nseq, rank, stream)) != SL_OK) return s;
    }
  }
  timer_end(TS_ESTIMATE, stream);
  SelectArgs se;
  std::memset(&se, 0, sizeof(se));
  se.st = st;
  se.qk = crit == SL_CRIT_QK_NORM;
  se.part0 = p0; se.part1 = p1;
  se.nchunk_max = g.nchunk_max;
  se.chunk = g.chunk;
  se.N = (int)N; se.N0 = g.N0;
  if (se.qk) { se.group = heads->n_q_heads / heads->n_kv_heads; se.head_dim = heads->head_dim; }
  se.k = k; se.idx = idx; se.scores = scores;
  return launch_select(se, st.nseq, stream);
}

}  // namespace

extern "C" {

size_t sl_estimate_select_workspace_bytes(sl_criterion crit, const sl_layout* lay,
                                          const sl_heads* heads, int64_t d_in, int32_t rank,
                                          int64_t N) {
  SeqTab st;
  if (build_seqtab(lay, st) != SL_OK) return 0;
  EstGeom g;
  if (d_in < 8 || d_in % 8) return 0;
  if (est_geom(crit, st, heads, d_in, rank, N, g) != SL_OK) return 0;
  return g.total;
}

sl_status sl_estimate_select(sl_criterion crit, sl_dtype dt, const sl_layout* lay,
                             const sl_heads* heads, const void* X, int64_t d_in, int32_t rank,
                             const void* Pt0, const void* Q0, const void* Pt1, const void* Q1,
                             int64_t N, int32_t k, int32_t* idx, float* scores, void* ws,
                             size_t ws_bytes, void* stream) {
  if (dt != SL_F32 && dt != SL_BF16) SL_FAIL(SL_ERR_DTYPE, "unknown dtype %d", (int)dt);
  SeqTab st;
  sl_status s = build_seqtab(lay, st);
  if (s != SL_OK) return s;
  EstGeom g;
  if (d_in < 8 || d_in % 8)
    SL_FAIL(SL_ERR_SHAPE, "d_in = %lld must be a positive multiple of 8", (long long)d_in);
  if ((s = est_geom(crit, st, heads, d_in, rank, N, g)) != SL_OK) return s;
  if (k < 1 || k > N) SL_FAIL(SL_ERR_RANGE, "k = %d outside [1, %lld]", k, (long long)N);
  if (rank > d_in) SL_FAIL(SL_ERR_RANGE, "rank %d > d_in %lld", rank, (long long)d_in);
  const bool two = crit != SL_CRIT_L2;
  if (!X || !Pt0 || !Q0 || !idx || !ws || (two && (!Pt1 || !Q1)))
    SL_FAIL(SL_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(X) || !aligned16(Pt0) || (two && !aligned16(Pt1)) || !aligned16(ws))
    SL_FAIL(SL_ERR_ALIGN, "X, Pt0, Pt1 and ws must be 16-byte aligned");
  if (ws_bytes < g.total)
    SL_FAIL(SL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, g.total);
  if ((s = check_arch()) != SL_OK) return s;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  if (dt == SL_BF16)
    return estimate_select_impl<bf16>(crit, st, heads, X, d_in, rank, Pt0, Q0, Pt1, Q1, N, k, idx,
                                      scores, reinterpret_cast<char*>(ws), g, strm);
  return estimate_select_impl<float>(crit, st, heads, X, d_in, rank, Pt0, Q0, Pt1, Q1, N, k, idx,
                                     scores, reinterpret_cast<char*>(ws), g, strm);
}

}  // extern "C"
