// a1-a3: low-rank activation estimate, per-channel criterion over each
// sequence's context tokens, per-sequence top-k.
//   SparseLoRA article §一 — L2-norm criterion for the FFN, QK-norm for q/k,
//     per-input channel choice; §二 — activations estimated from the offline
//     truncated SVD of the frozen weight; §三 — only context tokens are sparse,
//     so only they vote.
// A call carries one or more criterion jobs over the same input: the first
// stage projects X once onto the leading directions of every job, the L2-type
// criteria of all jobs share one Gram launch, and the selections share one
// launch.
#include "sl_launch.hpp"

#include <mutex>

using namespace sl;

namespace {

constexpr int EST_MAXPROJ = 4;   // stage-1 projections share one skinny launch of at most 4 blocks
static_assert(SL_EST_MAXJOBS == SEL_MAXJOBS, "select jobs per launch");

// One criterion job and its place in the workspace.
struct EJob {
  sl_criterion crit;
  sl_heads heads;
  const void* Pt[2]; const void* Q[2];
  long long N;
  int k;
  int32_t* idx; float* scores;
  int nproj;        // projections: 1 (L2) or 2
  int N0;           // columns of the first projection's partials (QK: Hq*hd; else N)
  int chunk;        // context tokens per partial
  int nchunk_max;
  int zcol;         // first Zh column of the job's projections (rep columns each)
  size_t w_p0, w_p1;
  size_t w_keys;    // the job's selection keys [nseq][N]
};

struct EstPlan {
  int njobs, nproj, rank, rep, ldz;
  EJob job[SL_EST_MAXJOBS];
  size_t w_zh, w_skp, total;
};

// Shapes, projection columns and workspace of a set of jobs (every job's
// crit, heads and N are read; pointers are not).
sl_status plan_estimate(const SeqTab& st, long long d_in, int rank, int njobs, const sl_est_job* in,
                        EstPlan& P) {
  if (njobs < 1 || njobs > SL_EST_MAXJOBS)
    SL_FAIL(SL_ERR_RANGE, "njobs = %d outside [1, %d]", njobs, SL_EST_MAXJOBS);
  if (rank < 1 || rank > 32) SL_FAIL(SL_ERR_RANGE, "estimator rank %d outside [1, 32]", rank);
  P.njobs = njobs;
  P.rank = rank;
  P.rep = (int)round_up(rank, 8);
  int maxctx = 0;
  for (int b = 0; b < st.nseq; ++b) maxctx = st.ctx[b] > maxctx ? st.ctx[b] : maxctx;
  int zcol = 0, nproj = 0;
  for (int j = 0; j < njobs; ++j) {
    const sl_est_job& s = in[j];
    EJob& e = P.job[j];
    e.crit = s.crit;
    if (s.crit != SL_CRIT_SWIGLU_L2 && s.crit != SL_CRIT_L2 && s.crit != SL_CRIT_QK_NORM)
      SL_FAIL(SL_ERR_DTYPE, "job %d: unknown criterion %d", j, (int)s.crit);
    if (s.N < 1 || s.N > SEL_MAXN)
      SL_FAIL(SL_ERR_RANGE, "job %d: N = %lld outside [1, %d]", j, (long long)s.N, SEL_MAXN);
    e.N = s.N;
    e.heads = s.heads;
    e.nproj = s.crit == SL_CRIT_L2 ? 1 : 2;
    e.N0 = (int)s.N;
    if (s.crit == SL_CRIT_QK_NORM) {
      const sl_heads& h = s.heads;
      if (h.n_q_heads < 1 || h.n_kv_heads < 1 || h.head_dim < 1 || h.n_q_heads % h.n_kv_heads)
        SL_FAIL(SL_ERR_SHAPE, "job %d: bad heads (%d q, %d kv, dim %d)", j, h.n_q_heads, h.n_kv_heads,
                h.head_dim);
      if ((long long)h.n_kv_heads * h.head_dim != s.N)
        SL_FAIL(SL_ERR_SHAPE, "job %d: QK-norm selects over n_kv_heads*head_dim = %d channels, N = %lld", j,
                h.n_kv_heads * h.head_dim, (long long)s.N);
      e.N0 = h.n_q_heads * h.head_dim;
    }
    // SwiGLU partials per SW_CHUNK tokens (the most a call can need: a bf16
    // call may take longer chunks); the L2 forms (Gram) one per sequence
    e.chunk = s.crit == SL_CRIT_SWIGLU_L2 ? SW_CHUNK : (1 << 30);
    e.nchunk_max = s.crit == SL_CRIT_SWIGLU_L2 ? ceil_div(maxctx, SW_CHUNK) : 1;
    if (e.nchunk_max < 1) e.nchunk_max = 1;
    e.zcol = zcol;
    zcol += e.nproj * P.rep;
    nproj += e.nproj;
  }
  if (nproj > EST_MAXPROJ) SL_FAIL(SL_ERR_RANGE, "%d projections in one call; at most %d", nproj, EST_MAXPROJ);
  P.nproj = nproj;
  P.ldz = zcol;
  const long long T = (long long)st.nseq * st.L;
  Bump bp;
  P.w_zh = bp.take((size_t)T * P.ldz * 4);
  for (int j = 0; j < njobs; ++j) {
    EJob& e = P.job[j];
    e.w_p0 = bp.take((size_t)st.nseq * e.nchunk_max * e.N0 * 4);
    e.w_p1 = e.crit == SL_CRIT_QK_NORM ? bp.take((size_t)st.nseq * e.nchunk_max * e.N * 4) : 0;
  }
  long long nmax = 0;
  for (int j = 0; j < njobs; ++j) nmax = P.job[j].N > nmax ? P.job[j].N : nmax;
  for (int j = 0; j < njobs; ++j) P.job[j].w_keys = bp.take((size_t)st.nseq * P.job[j].N * 4);
  P.w_skp = bp.take((size_t)skinny_part_floats(T, d_in) * 4);   // K-sliced stage 1
  P.total = bp.off;
  return SL_OK;
}

// Per-job checks that need the pointers and k.
sl_status check_jobs(int njobs, const sl_est_job* jobs, long long d_in, int rank) {
  if (rank > d_in) SL_FAIL(SL_ERR_RANGE, "rank %d > d_in %lld", rank, (long long)d_in);
  for (int j = 0; j < njobs; ++j) {
    const sl_est_job& s = jobs[j];
    if (s.k < 1 || s.k > s.N) SL_FAIL(SL_ERR_RANGE, "job %d: k = %d outside [1, %lld]", j, s.k, (long long)s.N);
    const bool two = s.crit != SL_CRIT_L2;
    if (!s.Pt0 || !s.Q0 || !s.idx || (two && (!s.Pt1 || !s.Q1)))
      SL_FAIL(SL_ERR_NULL, "job %d: a required pointer is NULL", j);
    if (!aligned16(s.Pt0) || (two && !aligned16(s.Pt1)))
      SL_FAIL(SL_ERR_ALIGN, "job %d: Pt0 and Pt1 must be 16-byte aligned", j);
  }
  return SL_OK;
}

// Context tokens per SwiGLU partial sum: 256 for the bf16 kernel at ranks up
// to 16 when every context fits two such chunks (the select kernel then adds
// the at most two partials of a channel itself, and no sum launch runs), else
// 128.  The workspace is sized for 128-token chunks, which need the most.
template <typename T>
int swiglu_chunk(const SeqTab& st, int rank) {
  int maxctx = 0;
  for (int b = 0; b < st.nseq; ++b) maxctx = st.ctx[b] > maxctx ? st.ctx[b] : maxctx;
  if (std::is_same<T, bf16>::value && rank <= 16 && maxctx > SW_CHUNK && maxctx <= 2 * SW_CHUNK_LONG)
    return SW_CHUNK_LONG;
  return SW_CHUNK;
}

template <typename T>
sl_status launch_swiglu(const SwiArgs& a, int nseq, int rank, int chunk, hipStream_t s) {
  const dim3 grid(ceil_div(a.N, 128), a.nchunk_max, nseq), block(SW_THREADS);
  if constexpr (std::is_same<T, bf16>::value) {
    if (chunk == SW_CHUNK_LONG) {
      if (rank <= 8) hipLaunchKernelGGL((score_swiglu_split_kernel<8, SW_CHUNK_LONG>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((score_swiglu_split_kernel<16, SW_CHUNK_LONG>), grid, block, 0, s, a);
    } else if (rank <= 8) {
      hipLaunchKernelGGL((score_swiglu_split_kernel<8, SW_CHUNK>), grid, block, 0, s, a);
    } else if (rank <= 16) {
      hipLaunchKernelGGL((score_swiglu_split_kernel<16, SW_CHUNK>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((score_swiglu_split_kernel<32, SW_CHUNK>), grid, block, 0, s, a);
    }
  } else {
    if (rank <= 8) hipLaunchKernelGGL((score_swiglu_kernel<T, 8>), grid, block, 0, s, a);
    else if (rank <= 16) hipLaunchKernelGGL((score_swiglu_kernel<T, 16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((score_swiglu_kernel<T, 32>), grid, block, 0, s, a);
  }
  SL_HIP(hipGetLastError());
  return SL_OK;
}

template <typename T>
sl_status launch_gram(const GramArgs& a, int nproj, int nseq, int rank, hipStream_t s) {
  int nmax = 0;
  for (int p = 0; p < nproj; ++p) nmax = a.N[p] > nmax ? a.N[p] : nmax;
  const dim3 grid(ceil_div(nmax, GR_THREADS), nseq, nproj), block(GR_THREADS);
  if (rank <= 8) hipLaunchKernelGGL((score_gram_kernel<T, 8>), grid, block, 0, s, a);
  else if (rank <= 16) hipLaunchKernelGGL((score_gram_kernel<T, 16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((score_gram_kernel<T, 32>), grid, block, 0, s, a);
  SL_HIP(hipGetLastError());
  return SL_OK;
}

// Selection launch(es).  With one or two partial sums per channel (every
// job's chunks x terms <= SEL_FUSE_LOADS, at most 16 keys per thread: the
// L2 and MHA QK-norm criteria) the select kernel forms the keys itself;
// otherwise score_finish_kernel forms them first with one thread per channel
// over many workgroups (one workgroup reading many partials is bound by its
// CU's outstanding loads: 15k cycles against 8k for the two launches at the
// LLaMA2-7B FFN shape).
constexpr int SEL_FUSE_LOADS = 2;

sl_status launch_select(const SelectArgs& a, int nseq, int nmax, bool fuse, hipStream_t s) {
  static std::once_flag attr_once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(attr_once, [] {
    attr_err = hipFuncSetAttribute((const void*)select_kernel<16, true>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 16 * SEL_THREADS * 4);
  });
  SL_HIP(attr_err);
  timer_begin(TS_SELECT, s);
  const dim3 grid(nseq, a.njobs), block(SEL_THREADS);
  if (fuse && nmax <= 4 * SEL_THREADS) {
    hipLaunchKernelGGL((select_kernel<4, true>), grid, block, (size_t)nmax * 4, s, a);
  } else if (fuse && nmax <= 16 * SEL_THREADS) {
    hipLaunchKernelGGL((select_kernel<16, true>), grid, block, (size_t)nmax * 4, s, a);
  } else {
    hipLaunchKernelGGL(score_finish_kernel, dim3(ceil_div(nmax, SF_THREADS), nseq, a.njobs), dim3(SF_THREADS), 0,
                       s, a);
    if (nmax <= 4 * SEL_THREADS) hipLaunchKernelGGL((select_kernel<4, false>), grid, block, 0, s, a);
    else if (nmax <= 16 * SEL_THREADS) hipLaunchKernelGGL((select_kernel<16, false>), grid, block, 0, s, a);
    else if (nmax <= SEL_KPT_REG * SEL_THREADS)
      hipLaunchKernelGGL((select_kernel<SEL_KPT_REG, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((select_kernel<0, false>), grid, block, 0, s, a);
  }
  timer_end(TS_SELECT, s);
  SL_HIP(hipGetLastError());
  return SL_OK;
}

template <typename T>
sl_status estimate_select_impl(const SeqTab& st, const void* X, long long d_in, const EstPlan& P, char* ws,
                               hipStream_t stream) {
  float* zh = reinterpret_cast<float*>(ws + P.w_zh);
  const int sw_chunk = swiglu_chunk<T>(st, P.rank);
  auto chunk_of = [&](const EJob& e) { return e.crit == SL_CRIT_SWIGLU_L2 ? sw_chunk : e.chunk; };
  auto nchunk_of = [&](const EJob& e) {
    if (e.crit != SL_CRIT_SWIGLU_L2) return e.nchunk_max;
    int maxctx = 0;
    for (int b = 0; b < st.nseq; ++b) maxctx = st.ctx[b] > maxctx ? st.ctx[b] : maxctx;
    return std::max(1, ceil_div(maxctx, sw_chunk));
  };
  auto p0 = [&](const EJob& e) { return reinterpret_cast<float*>(ws + e.w_p0); };
  auto p1 = [&](const EJob& e) { return reinterpret_cast<float*>(ws + e.w_p1); };
  timer_begin(TS_ESTIMATE, stream);
  if (st.T_ctx > 0) {
    // stage 1: Zh = X_ctx [Pt of every projection]^T on the context rows;
    // projection i of the call lands in Zh columns [i rep, i rep + rank)
    SkinnyArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.st = st;
    sa.mode = 2;
    sa.T = st.nseq * st.L;
    sa.A = X; sa.lda = d_in;
    sa.K = (int)d_in;
    for (int j = 0; j < P.njobs; ++j)
      for (int p = 0; p < P.job[j].nproj; ++p) {
        sa.Bb[sa.nblk] = P.job[j].Pt[p]; sa.nbk[sa.nblk] = P.rank; sa.ldbb[sa.nblk] = d_in;
        ++sa.nblk;
      }
    sa.out = zh; sa.ldo = P.ldz; sa.col0 = 0; sa.oscale = 1.f;
    sa.part = reinterpret_cast<float*>(ws + P.w_skp);
    sl_status s = launch_skinny<T>(sa, stream);
    if (s != SL_OK) return s;
    // stage 2 + criterion: every L2-type projection in one Gram launch, each
    // SwiGLU job in a launch of its own
    GramArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.st = st;
    ga.Zh = zh; ga.ldz = P.ldz; ga.rank = P.rank;
    int ng = 0;
    for (int j = 0; j < P.njobs; ++j) {
      const EJob& e = P.job[j];
      if (e.crit == SL_CRIT_SWIGLU_L2) {
        SwiArgs sc;
        std::memset(&sc, 0, sizeof(sc));
        sc.st = st;
        sc.Zh = zh; sc.ldz = P.ldz; sc.zc0 = e.zcol; sc.zc1 = e.zcol + P.rep;
        sc.Q0 = e.Q[0]; sc.Q1 = e.Q[1]; sc.rank = P.rank; sc.N = (int)e.N;
        sc.part = p0(e); sc.nchunk_max = nchunk_of(e);
        if ((s = launch_swiglu<T>(sc, st.nseq, P.rank, chunk_of(e), stream)) != SL_OK) return s;
        continue;
      }
      ga.zc[ng] = e.zcol; ga.Q[ng] = e.Q[0]; ga.N[ng] = e.N0; ga.part[ng] = p0(e); ++ng;
      if (e.crit == SL_CRIT_QK_NORM) {
        ga.zc[ng] = e.zcol + P.rep; ga.Q[ng] = e.Q[1]; ga.N[ng] = (int)e.N; ga.part[ng] = p1(e); ++ng;
      }
    }
    if (ng > 0 && (s = launch_gram<T>(ga, ng, st.nseq, P.rank, stream)) != SL_OK) return s;
  }
  timer_end(TS_ESTIMATE, stream);
  SelectArgs se;
  std::memset(&se, 0, sizeof(se));
  se.st = st;
  se.njobs = P.njobs;
  int nmax = 0;
  for (int j = 0; j < P.njobs; ++j) {
    const EJob& e = P.job[j];
    SelJob& q = se.job[j];
    q.qk = e.crit == SL_CRIT_QK_NORM;
    q.part0 = p0(e); q.part1 = p1(e);
    q.nchunk_max = nchunk_of(e);
    q.chunk = chunk_of(e);
    q.N = (int)e.N; q.N0 = e.N0;
    if (q.qk) { q.group = e.heads.n_q_heads / e.heads.n_kv_heads; q.head_dim = e.heads.head_dim; }
    q.k = e.k; q.idx = e.idx; q.scores = e.scores;
    q.gkeys = reinterpret_cast<uint32_t*>(ws + e.w_keys);
    nmax = q.N > nmax ? q.N : nmax;
  }
  bool fuse = true;
  for (int j = 0; j < P.njobs; ++j) {
    const SelJob& q = se.job[j];
    fuse &= (long long)q.nchunk_max * (q.qk ? q.group + 1 : 1) <= SEL_FUSE_LOADS;
  }
  return launch_select(se, st.nseq, nmax, fuse, stream);
}

sl_est_job one_job(sl_criterion crit, const sl_heads* heads, const void* Pt0, const void* Q0, const void* Pt1,
                   const void* Q1, int64_t N, int32_t k, int32_t* idx, float* scores) {
  sl_est_job j;
  std::memset(&j, 0, sizeof(j));
  j.crit = crit;
  if (heads) j.heads = *heads;
  j.Pt0 = Pt0; j.Q0 = Q0; j.Pt1 = Pt1; j.Q1 = Q1;
  j.N = N; j.k = k; j.idx = idx; j.scores = scores;
  return j;
}

// ---- allocation-free variant ------------------------------------------------
// Scratch of sl_estimate_select_noalloc: one array per device, in the code
// object's device memory (each device that loads the library holds its own
// copy until the process ends).  In host code `scratch` names a host-side
// stand-in, never the device array: its device address is resolved once per
// device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) unsigned char scratch[SL_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};

sl_status scratch_address(void** out) {
  int dev = 0;
  SL_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) SL_FAIL(SL_ERR_HIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      SL_FAIL(SL_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SL_OK;
}

sl_status estimate_select_call(sl_dtype dt, const sl_layout* lay, const void* X, int64_t d_in, int32_t rank,
                               int32_t njobs, const sl_est_job* jobs, void* ws, size_t ws_bytes, void* stream,
                               bool use_scratch = false) {
  if (dt != SL_F32 && dt != SL_BF16) SL_FAIL(SL_ERR_DTYPE, "unknown dtype %d", (int)dt);
  if (!jobs) SL_FAIL(SL_ERR_NULL, "jobs is NULL");
  SeqTab st;
  sl_status s = build_seqtab(lay, st);
  if (s != SL_OK) return s;
  if (d_in < 8 || d_in % 8)
    SL_FAIL(SL_ERR_SHAPE, "d_in = %lld must be a positive multiple of 8", (long long)d_in);
  EstPlan P;
  if ((s = plan_estimate(st, d_in, rank, njobs, jobs, P)) != SL_OK) return s;
  if ((s = check_jobs(njobs, jobs, d_in, rank)) != SL_OK) return s;
  for (int j = 0; j < njobs; ++j) {
    EJob& e = P.job[j];
    e.Pt[0] = jobs[j].Pt0; e.Q[0] = jobs[j].Q0; e.Pt[1] = jobs[j].Pt1; e.Q[1] = jobs[j].Q1;
    e.k = jobs[j].k; e.idx = jobs[j].idx; e.scores = jobs[j].scores;
  }
  if (use_scratch) {
    if (!X) SL_FAIL(SL_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(X)) SL_FAIL(SL_ERR_ALIGN, "X must be 16-byte aligned");
    if (P.total > (size_t)SL_NOALLOC_SCRATCH_BYTES)
      SL_FAIL(SL_ERR_WORKSPACE,
              "this call needs %zu bytes of scratch; the allocation-free variant holds %zu "
              "(use sl_estimate_select with a workspace)", P.total, (size_t)SL_NOALLOC_SCRATCH_BYTES);
    if ((s = check_arch()) != SL_OK) return s;
    if ((s = scratch_address(&ws)) != SL_OK) return s;
  } else {
    if (!X || !ws) SL_FAIL(SL_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(X) || !aligned16(ws)) SL_FAIL(SL_ERR_ALIGN, "X and ws must be 16-byte aligned");
    if (ws_bytes < P.total) SL_FAIL(SL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, P.total);
    if ((s = check_arch()) != SL_OK) return s;
  }
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  if (dt == SL_BF16) return estimate_select_impl<bf16>(st, X, d_in, P, reinterpret_cast<char*>(ws), strm);
  return estimate_select_impl<float>(st, X, d_in, P, reinterpret_cast<char*>(ws), strm);
}

size_t workspace_of(const sl_layout* lay, int64_t d_in, int32_t rank, int32_t njobs, const sl_est_job* jobs) {
  SeqTab st;
  if (!jobs || build_seqtab(lay, st) != SL_OK) return 0;
  if (d_in < 8 || d_in % 8) return 0;
  EstPlan P;
  if (plan_estimate(st, d_in, rank, njobs, jobs, P) != SL_OK) return 0;
  return P.total;
}

}  // namespace

extern "C" {

size_t sl_estimate_select_workspace_bytes(sl_criterion crit, const sl_layout* lay,
                                          const sl_heads* heads, int64_t d_in, int32_t rank,
                                          int64_t N) {
  if (crit == SL_CRIT_QK_NORM && !heads) return 0;
  const sl_est_job j = one_job(crit, heads, nullptr, nullptr, nullptr, nullptr, N, 1, nullptr, nullptr);
  return workspace_of(lay, d_in, rank, 1, &j);
}

sl_status sl_estimate_select(sl_criterion crit, sl_dtype dt, const sl_layout* lay,
                             const sl_heads* heads, const void* X, int64_t d_in, int32_t rank,
                             const void* Pt0, const void* Q0, const void* Pt1, const void* Q1,
                             int64_t N, int32_t k, int32_t* idx, float* scores, void* ws,
                             size_t ws_bytes, void* stream) {
  if (crit == SL_CRIT_QK_NORM && !heads) SL_FAIL(SL_ERR_NULL, "heads is NULL for the QK-norm criterion");
  const sl_est_job j = one_job(crit, heads, Pt0, Q0, Pt1, Q1, N, k, idx, scores);
  return estimate_select_call(dt, lay, X, d_in, rank, 1, &j, ws, ws_bytes, stream);
}

sl_status sl_estimate_select_noalloc(sl_criterion crit, sl_dtype dt, const sl_layout* lay,
                                     const sl_heads* heads, const void* X, int64_t d_in, int32_t rank,
                                     const void* Pt0, const void* Q0, const void* Pt1, const void* Q1,
                                     int64_t N, int32_t k, int32_t* idx, float* scores, void* stream) {
  if (crit == SL_CRIT_QK_NORM && !heads) SL_FAIL(SL_ERR_NULL, "heads is NULL for the QK-norm criterion");
  const sl_est_job j = one_job(crit, heads, Pt0, Q0, Pt1, Q1, N, k, idx, scores);
  return estimate_select_call(dt, lay, X, d_in, rank, 1, &j, nullptr, 0, stream, true);
}

size_t sl_estimate_select_multi_workspace_bytes(const sl_layout* lay, int64_t d_in, int32_t rank,
                                                int32_t njobs, const sl_est_job* jobs) {
  return workspace_of(lay, d_in, rank, njobs, jobs);
}

sl_status sl_estimate_select_multi(sl_dtype dt, const sl_layout* lay, const void* X, int64_t d_in,
                                   int32_t rank, int32_t njobs, const sl_est_job* jobs, void* ws,
                                   size_t ws_bytes, void* stream) {
  return estimate_select_call(dt, lay, X, d_in, rank, njobs, jobs, ws, ws_bytes, stream);
}

}  // extern "C"
