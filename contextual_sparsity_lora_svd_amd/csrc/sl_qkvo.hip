// a6/a7: sparse LoRA q/k/v/o projections, forward and backward.
//   SparseLoRA article §一 — QK-norm criterion picks q/k channels (one kv-channel
//   set, shared by every query head of the group); v/o use the L2 set of v;
//   §三 — context rows sparse, output rows dense; §六 — channel sparsity.
//
//   forward  q = X Wq[Sq]^T + s (X Aq^T) Bq[Sq]^T   scattered into the dense
//            layout, unselected context channels written as 0; k, v likewise
//            o = a[:, So] WoT[So] + s (a[:, So] Ao[:, So]^T) Bo^T
//   backward da = (d_out WoT[So]^T + dz_o Ao[:, So]) on So, 0 elsewhere at
//            context rows; dX = dq Wq[Sq] + dk Wk[Sk] + dv Wv[Sv] + LoRA terms;
//            factor gradients by column reductions.
#include "sl_launch.hpp"

using namespace sl;

namespace {

struct Comp {       // compact copy of a projection's selected columns
  int kc, ld, n;    // channels per context group, context row stride, full width
  long long out_off, elems;
};

Comp make_comp(const SeqTab& st, int kc, int n) {
  Comp c;
  c.kc = kc; c.n = n;
  c.ld = (int)round_up(kc, 8);
  c.out_off = (long long)st.T_ctx * c.ld;
  c.elems = c.out_off + (long long)st.T_out * n;
  return c;
}

struct QkvoGeom {
  SeqTab st;
  int T, D, Hq, Hkv, hd, G, nq, nkv, r, rp, kqk, kvo, kq, ko;
  size_t esz;
  Comp cq, ck, cv, co;
  int ks_o, ks_dx, chunk;
  long long cr_floats, skp_floats;
  size_t s_zqkv, s_zo, s_BoT, s_AoT, saved_bytes;
  size_t w_idxq, w_idxo, w_zs_qkv, w_zs_o, w_Bqp, w_Bkp, w_Bvp, w_Aog, w_ac, w_part,
      w_dz_o, w_dzs_o, w_dqc, w_dkc, w_dvc, w_Bqg, w_Bkg, w_Bvg, w_BqTo, w_BkTo, w_BvTo,
      w_dz_qkv, w_dzs_qkv, w_Aqkvp, w_cr, w_inv_o, w_inv_q, w_inv_k, w_inv_v, w_iota, w_rp, w_skp, ws_bytes;
};

sl_status qkvo_geom(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w, int kqk, int kvo,
                    bool check_k, QkvoGeom& g) {
  if (dt != SL_F32 && dt != SL_BF16) SL_FAIL(SL_ERR_DTYPE, "unknown dtype %d", (int)dt);
  if (!w) SL_FAIL(SL_ERR_NULL, "weights is NULL");
  sl_status s = build_seqtab(lay, g.st);
  if (s != SL_OK) return s;
  const SeqTab& st = g.st;
  const sl_heads& h = w->heads;
  if (h.n_q_heads < 1 || h.n_kv_heads < 1 || h.head_dim < 1 || h.n_q_heads % h.n_kv_heads)
    SL_FAIL(SL_ERR_SHAPE, "bad heads (%d q, %d kv, dim %d)", h.n_q_heads, h.n_kv_heads, h.head_dim);
  const long long D = w->d_model;
  const long long nq = (long long)h.n_q_heads * h.head_dim, nkv = (long long)h.n_kv_heads * h.head_dim;
  if (D < 8 || D % 8 || nq % 8 || nkv % 8 || D > (1 << 20) || nq > (1 << 20))
    SL_FAIL(SL_ERR_SHAPE, "d_model, Hq*hd and Hkv*hd must be positive multiples of 8");
  if (w->lora_rank < 1 || w->lora_rank > 32)
    SL_FAIL(SL_ERR_RANGE, "lora_rank %d outside [1, 32]", w->lora_rank);
  if (check_k) {
    if (kqk < 1 || kqk > nkv) SL_FAIL(SL_ERR_RANGE, "k_qk = %d outside [1, %lld]", kqk, nkv);
    if (kvo < 1 || kvo > nkv) SL_FAIL(SL_ERR_RANGE, "k_vo = %d outside [1, %lld]", kvo, nkv);
  } else {
    kqk = kqk < 1 ? 1 : kqk;
    kvo = kvo < 1 ? 1 : kvo;
  }
  g.T = st.nseq * st.L;
  g.D = (int)D; g.Hq = h.n_q_heads; g.Hkv = h.n_kv_heads; g.hd = h.head_dim;
  g.G = g.Hq / g.Hkv;
  g.nq = (int)nq; g.nkv = (int)nkv;
  g.r = w->lora_rank; g.rp = (int)round_up(g.r, 8);
  g.kqk = kqk; g.kvo = kvo; g.kq = kqk * g.G; g.ko = kvo * g.G;
  g.esz = dt == SL_BF16 ? 2 : 4;
  g.cq = make_comp(st, g.kq, g.nq);
  g.ck = make_comp(st, g.kqk, g.nkv);
  g.cv = make_comp(st, g.kvo, g.nkv);
  g.co = make_comp(st, g.ko, g.nq);
  if ((s = check_extent("X / dX / o / d_out", g.T, D)) != SL_OK) return s;
  if ((s = check_extent("q / a / dq / da", g.T, nq)) != SL_OK) return s;
  if ((s = check_extent("Wq / WoT", nq, D)) != SL_OK) return s;
  for (const Comp* c : {&g.cq, &g.ck, &g.cv, &g.co})
    if ((s = check_extent("a compact projection buffer", 1, c->elems)) != SL_OK) return s;
  const int bk = dt == SL_BF16 ? 64 : 32;
  g.ks_o = kg_choose_ksplit(st, g.ko + g.rp, g.nq + g.rp, g.D, bk, dt == SL_BF16);
  g.ks_dx = kg_choose_ksplit(st, (long long)g.kq + g.kqk + g.kvo + 3 * g.rp,
                             (long long)g.nq + 2 * g.nkv + 3 * g.rp, g.D, bk, dt == SL_BF16);
  const size_t T = g.T, e = g.esz, rp = g.rp, B = st.nseq;
  Bump sv;
  g.s_zqkv = sv.take(T * 3 * rp * 4);
  g.s_zo = sv.take(T * rp * 4);
  // Bo^T and Ao^T, packed by the forward: the backward's first products read
  // them while its own packing runs on the side stream
  g.s_BoT = sv.take(rp * D * e);
  g.s_AoT = sv.take((size_t)g.nq * rp * e);
  g.saved_bytes = sv.off;
  Bump b;
  g.w_idxq = b.take(B * g.kq * 4);
  g.w_idxo = b.take(B * g.ko * 4);
  g.w_zs_qkv = b.take(T * 3 * rp * e);
  g.w_zs_o = b.take(T * rp * e);
  g.w_Bqp = b.take((size_t)g.nq * rp * e);
  g.w_Bkp = b.take((size_t)g.nkv * rp * e);
  g.w_Bvp = b.take((size_t)g.nkv * rp * e);
  g.w_Aog = b.take(B * rp * g.co.ld * e);
  g.w_ac = b.take(g.co.elems * e);
  const int ks = std::max(g.ks_o, g.ks_dx);
  g.w_part = b.take(ks > 1 ? (size_t)ks * st.T_out * D * 4 : 0);
  g.w_dz_o = b.take(T * rp * 4);
  g.w_dzs_o = b.take(T * rp * e);
  g.w_dqc = b.take(g.cq.elems * e);
  g.w_dkc = b.take(g.ck.elems * e);
  g.w_dvc = b.take(g.cv.elems * e);
  g.w_Bqg = b.take(B * rp * g.cq.ld * e);
  g.w_Bkg = b.take(B * rp * g.ck.ld * e);
  g.w_Bvg = b.take(B * rp * g.cv.ld * e);
  g.w_BqTo = b.take(rp * g.nq * e);
  g.w_BkTo = b.take(rp * g.nkv * e);
  g.w_BvTo = b.take(rp * g.nkv * e);
  g.w_dz_qkv = b.take(T * 3 * rp * 4);
  g.w_dzs_qkv = b.take(T * 3 * rp * e);
  g.w_Aqkvp = b.take(3 * rp * D * e);
  g.chunk = cr_chunk(g.esz);
  // partials of the seven gradient reductions of the backward
  const size_t es = g.esz;
  const long long cr = cb_scatter_floats(st, es, g.ko, g.nq, g.rp) + 2 * cb_dense_floats(st, es, g.D, g.rp) +
                       cb_dense_floats(st, es, g.D, 2 * g.rp) + cb_scatter_floats(st, es, g.kq, g.nq, g.rp) +
                       cb_scatter_floats(st, es, g.kqk, g.nkv, g.rp) + cb_scatter_floats(st, es, g.kvo, g.nkv, g.rp);
  g.cr_floats = cr;
  g.w_cr = b.take((size_t)cr * 4);
  g.w_inv_o = b.take(B * g.nq * 4);
  g.w_inv_q = b.take(B * g.nq * 4);
  g.w_inv_k = b.take(B * g.nkv * 4);
  g.w_inv_v = b.take(B * g.nkv * 4);
  g.w_iota = b.take((size_t)std::max(g.nq, 3 * g.rp) * 4);
  // skinny partial sums: room for the three problems of the dz_q / dz_k / dz_v launch
  g.skp_floats = skinny_part_floats(g.T, std::max(g.D, g.nq));
  g.w_skp = b.take((size_t)g.skp_floats * 3 * 4);
  // K pieces of the da gather-GEMM when its grid is under half a round
  g.w_rp = b.take((size_t)ng_rpart_floats(st, g.ko, g.nq, false, g.esz, {g.D, g.rp}) * 4);
  g.ws_bytes = b.off;
  return SL_OK;
}

// idx_q (or idx_o) from a kv-channel set
sl_status expand_set(const QkvoGeom& g, const int* idx_kv, int k, int* out, hipStream_t s) {
  const long long n = (long long)g.st.nseq * k * g.G;
  hipLaunchKernelGGL(expand_kv_kernel, grid1d(n), dim3(256), 0, s, idx_kv, k, g.st.nseq, g.G, g.hd,
                     out);
  SL_HIP(hipGetLastError());
  return SL_OK;
}

// compact copy of a projection's buffer (job of a layout launch)
void add_compact(Layouter& L, const Comp& c, const void* src, const int* idx, void* dst, size_t esz) {
  L.compact(src, c.n, idx, c.kc, c.n, dst, c.ld, c.out_off, esz);
}

// Base segment of an o-weight gather-GEMM: WoT, or its 4-bit codes and scales.
inline void set_o_base(GSeg& sg, const sl_qkvo_weights* w) {
  if (w->WoT_q) { sg.B = w->WoT_q; sg.Bs = w->WoT_s; sg.bq4 = 1; }
}

template <typename T>
sl_status qkvo_fwd_impl(const QkvoGeom& g, const sl_qkvo_weights* w, const void* X, const void* a,
                        const int* idx_qk, const int* idx_vo, void* q, void* k, void* v, void* o,
                        char* sv, char* ws, hipStream_t strm) {
  const SeqTab& st = g.st;
  const int D = g.D, r = g.r, rp = g.rp;
  const float s = w->lora_scale;
  sl_status rc;
  float* zqkv = reinterpret_cast<float*>(sv + g.s_zqkv);
  float* zo = reinterpret_cast<float*>(sv + g.s_zo);
  int* idx_q = g.G > 1 ? reinterpret_cast<int*>(ws + g.w_idxq) : const_cast<int*>(idx_qk);
  int* idx_o = g.G > 1 ? reinterpret_cast<int*>(ws + g.w_idxo) : const_cast<int*>(idx_vo);
  T* zs_qkv = reinterpret_cast<T*>(ws + g.w_zs_qkv);
  T* zs_o = reinterpret_cast<T*>(ws + g.w_zs_o);
  float* part = reinterpret_cast<float*>(ws + g.w_part);
  float* skp = reinterpret_cast<float*>(ws + g.w_skp);
  T* ac = reinterpret_cast<T*>(ws + g.w_ac);
  T* Aog = reinterpret_cast<T*>(ws + g.w_Aog);
  T* BoTp = reinterpret_cast<T*>(sv + g.s_BoT);
  T* AoTp = reinterpret_cast<T*>(sv + g.s_AoT);
  const bool qq = w->Wq_q != nullptr;   // 4-bit q/k/v base
  const void* Wm[3] = {qq ? w->Wq_q : w->Wq, qq ? w->Wk_q : w->Wk, qq ? w->Wv_q : w->Wv};
  const float* Ws[3] = {w->Wq_s, w->Wk_s, w->Wv_s};
  const void* Bl[3] = {w->Bq, w->Bk, w->Bv};
  void* outp[3] = {q, k, v};
  const int* sets[3] = {idx_q, idx_qk, idx_vo};
  const int kk[3] = {g.kq, g.kqk, g.kvo};
  const int nn[3] = {g.nq, g.nkv, g.nkv};
  T* Bp[3] = {reinterpret_cast<T*>(ws + g.w_Bqp), reinterpret_cast<T*>(ws + g.w_Bkp),
              reinterpret_cast<T*>(ws + g.w_Bvp)};

  // query-channel sets, then one launch each for operand packing and row layout
  if (g.G > 1 && X && (rc = expand_set(g, idx_qk, g.kqk, idx_q, strm))) return rc;
  if (g.G > 1 && a && (rc = expand_set(g, idx_vo, g.kvo, idx_o, strm))) return rc;
  Packer pk;
  pk.iota(reinterpret_cast<int*>(ws + g.w_iota), std::max(g.nq, 3 * g.rp));
  Layouter L(st);
  if (X) {
    for (int j = 0; j < 3; ++j) {
      pk.copy(Bp[j], rp, nn[j], rp, Bl[j], r, nn[j], r, 0);          // B_j, rank padded to rp
    }
  }
  if (a) {
    pk.copy(BoTp, D, rp, D, w->Bo, r, r, D, 1);                      // Bo^T [rp, D] (saved)
    pk.copy(AoTp, rp, g.nq, rp, w->Ao, g.nq, g.nq, r, 1);            // Ao^T [nq, rp] (saved)
    pk.gather(Aog, g.co.ld, (long long)rp * g.co.ld, rp, g.co.ld, w->Ao, g.nq, r, 0, idx_o, g.ko,
              st.nseq);                                             // Ao[:, So] per sequence
    add_compact(L, g.co, a, idx_o, ac, g.esz);
  }
  // packing and row layout on the side stream: they overlap the z product
  // below, which reads neither
  SideFork fork;
  if ((rc = fork.begin(strm))) return rc;
  rc = pk.launch<T>(fork.side);
  if (rc == SL_OK) rc = L.launch<T>(fork.side);
  if (rc == SL_OK && X) {
    // z = X [Aq; Ak; Av]^T
    SkinnyArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.st = st; sa.mode = 0; sa.T = g.T;
    sa.A = X; sa.lda = D; sa.K = D;
    sa.nblk = 3;
    sa.Bb[0] = w->Aq; sa.nbk[0] = r; sa.ldbb[0] = D;
    sa.Bb[1] = w->Ak; sa.nbk[1] = r; sa.ldbb[1] = D;
    sa.Bb[2] = w->Av; sa.nbk[2] = r; sa.ldbb[2] = D;
    sa.out = zqkv; sa.ldo = 3 * rp; sa.oscale = 1.f;
    sa.outs = zs_qkv; sa.ldos = 3 * rp; sa.scale = s;
    sa.part = skp;
    rc = launch_skinny<T>(sa, strm);
  }
  {
    const sl_status rj = fork.end(strm);   // joined on every path
    if (rc != SL_OK) return rc;
    if (rj != SL_OK) return rj;
  }
  if (X) {
    // the three projections in one launch: y_j = X W_j[S_j]^T + (s z_j) B_j[S_j]^T
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.st = st;
    ga.nseg = 2;
    ga.seg[0] = GSeg{X, D, 0, 0, 1, nullptr, nullptr, D, 1, D, nullptr, 0, 0};
    ga.seg[1] = GSeg{zs_qkv, 3 * rp, 0, 0, 1, nullptr, nullptr, rp, 1, rp, nullptr, 0, 0};
    ga.seg[0].bq4 = qq ? 1 : 0;
    ga.nprob = 3;
    for (int j = 0; j < 3; ++j) {
      GProb& pr = ga.prob[j];
      pr.idx = sets[j]; pr.kidx = kk[j]; pr.n_out = nn[j];
      pr.B[0] = Wm[j]; pr.B[1] = Bp[j];
      pr.Bs[0] = qq ? Ws[j] : nullptr;
      pr.a_col[0] = 0; pr.a_col[1] = j * rp;
      pr.o0 = outp[j]; pr.ldo = nn[j]; pr.swidth = nn[j];
    }
    SL_HIP((launch_gather_gemm<T, MODE_NG, EPI_SCATTER, false>(ga, strm, TS_QKV_FWD)));
  }
  if (a) {
    // z_o = a_m Ao^T
    SkinnyArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.st = st; sa.mode = 1; sa.T = g.T;
    sa.A = ac; sa.lda = g.co.ld; sa.lda_out = g.nq; sa.a_out_off = g.co.out_off;
    sa.K = 0; sa.kidx = g.ko; sa.n_out = g.nq;
    sa.nblk = 1;
    sa.Bb[0] = Aog; sa.nbk[0] = r; sa.ldbb[0] = g.co.ld; sa.b0_gstride = (long long)rp * g.co.ld;
    sa.B0o = w->Ao; sa.ldb0o = g.nq;
    sa.out = zo; sa.ldo = rp; sa.oscale = 1.f;
    sa.outs = zs_o; sa.ldos = rp; sa.scale = s;
    sa.part = skp;
    if ((rc = launch_skinny<T>(sa, strm))) return rc;
    // o = a_m WoT[So] + s z_o Bo^T
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.st = st;
    ga.kidx = 1; ga.n_out = 1;
    ga.N = D;
    ga.nseg = 2;
    ga.seg[0] = GSeg{ac, g.co.ld, g.nq, g.co.out_off, 0, w->WoT, nullptr, D, 1, 0, idx_o, g.ko, g.nq};
    set_o_base(ga.seg[0], w);
    ga.seg[1] = GSeg{zs_o, rp, 0, 0, 1, BoTp, nullptr, D, 0, rp, nullptr, 0, 0};
    ga.ksplit_out = g.ks_o;
    ga.o0 = o; ga.ldo = D;
    ga.part = part;
    ga.iota = reinterpret_cast<const int*>(ws + g.w_iota);
    SL_HIP((launch_gather_gemm<T, MODE_KG, EPI_TOKEN, false>(ga, strm, TS_O_FWD)));
    if ((rc = splitk_reduce<T>(st, part, g.ks_o, D, o, D, strm))) return rc;
  }
  return SL_OK;
}

template <typename T>
sl_status qkvo_bwd_impl(const QkvoGeom& g, const sl_qkvo_weights* w, const void* X, const void* a,
                        const int* idx_qk, const int* idx_vo, const char* sv, const void* dq,
                        const void* dk, const void* dv, const void* d_out, void* dX, void* da,
                        const sl_qkvo_grads* gr, char* ws, hipStream_t strm) {
  const SeqTab& st = g.st;
  const int D = g.D, r = g.r, rp = g.rp;
  const float s = w->lora_scale;
  sl_status rc;
  const float* zqkv = reinterpret_cast<const float*>(sv + g.s_zqkv);
  const float* zo = reinterpret_cast<const float*>(sv + g.s_zo);
  int* idx_q = g.G > 1 ? reinterpret_cast<int*>(ws + g.w_idxq) : const_cast<int*>(idx_qk);
  int* idx_o = g.G > 1 ? reinterpret_cast<int*>(ws + g.w_idxo) : const_cast<int*>(idx_vo);
  float* part = reinterpret_cast<float*>(ws + g.w_part);
  float* crp = reinterpret_cast<float*>(ws + g.w_cr);
  int* inv_o = reinterpret_cast<int*>(ws + g.w_inv_o);
  float* skp = reinterpret_cast<float*>(ws + g.w_skp);
  T* ac = reinterpret_cast<T*>(ws + g.w_ac);
  const T* BoTp = reinterpret_cast<const T*>(sv + g.s_BoT);   // packed by the forward
  const T* AoTp = reinterpret_cast<const T*>(sv + g.s_AoT);
  T* Aqkvp = reinterpret_cast<T*>(ws + g.w_Aqkvp);
  const void* dsrc[3] = {dq, dk, dv};
  T* dcomp[3] = {reinterpret_cast<T*>(ws + g.w_dqc), reinterpret_cast<T*>(ws + g.w_dkc),
                 reinterpret_cast<T*>(ws + g.w_dvc)};
  const Comp* cc[3] = {&g.cq, &g.ck, &g.cv};
  const int* sets[3] = {idx_q, idx_qk, idx_vo};
  int* inv[3] = {reinterpret_cast<int*>(ws + g.w_inv_q), reinterpret_cast<int*>(ws + g.w_inv_k),
                 reinterpret_cast<int*>(ws + g.w_inv_v)};
  const void* Bl[3] = {w->Bq, w->Bk, w->Bv};
  const void* Al[3] = {w->Aq, w->Ak, w->Av};
  const bool qq = w->Wq_q != nullptr;   // 4-bit q/k/v base
  const void* Wm[3] = {qq ? w->Wq_q : w->Wq, qq ? w->Wk_q : w->Wk, qq ? w->Wv_q : w->Wv};
  const float* Ws[3] = {w->Wq_s, w->Wk_s, w->Wv_s};
  T* Bg[3] = {reinterpret_cast<T*>(ws + g.w_Bqg), reinterpret_cast<T*>(ws + g.w_Bkg),
              reinterpret_cast<T*>(ws + g.w_Bvg)};
  T* BTo[3] = {reinterpret_cast<T*>(ws + g.w_BqTo), reinterpret_cast<T*>(ws + g.w_BkTo),
               reinterpret_cast<T*>(ws + g.w_BvTo)};
  float* dB[3] = {gr->dBq, gr->dBk, gr->dBv};

  // query-channel sets; then one launch for operand packing with the inverse
  // maps of the channel sets, and one for the row layout
  if (g.G > 1 && d_out && (rc = expand_set(g, idx_vo, g.kvo, idx_o, strm))) return rc;
  if (g.G > 1 && dq && (rc = expand_set(g, idx_qk, g.kqk, idx_q, strm))) return rc;
  Packer pk;
  pk.iota(reinterpret_cast<int*>(ws + g.w_iota), std::max(g.nq, 3 * g.rp));
  Layouter L(st);
  if (d_out) {
    add_compact(L, g.co, a, idx_o, ac, g.esz);
    pk.inverse(inv_o, idx_o, g.ko, g.nq, st.nseq);
  }
  if (dq) {
    for (int j = 0; j < 3; ++j) {
      const Comp& c = *cc[j];
      pk.copy(Aqkvp + (size_t)j * rp * D, D, rp, D, Al[j], D, r, D, 0);        // A_j, rank padded
      pk.gather(Bg[j], c.ld, (long long)rp * c.ld, rp, c.ld, Bl[j], r, r, 1, sets[j], c.kc,
                st.nseq);                                                    // B_j[S_j]^T per sequence
      pk.copy(BTo[j], c.n, r, c.n, Bl[j], r, r, c.n, 1);                     // B_j^T
      add_compact(L, c, dsrc[j], sets[j], dcomp[j], g.esz);
      pk.inverse(inv[j], sets[j], c.kc, c.n, st.nseq);
    }
  }
  ColredBatch cb(st, g.esz, crp, g.cr_floats);
  float* dz_o = reinterpret_cast<float*>(ws + g.w_dz_o);
  T* dzs_o = reinterpret_cast<T*>(ws + g.w_dzs_o);
  // the o-branch products: dz_o = s d_out Bo, then da on So (dense at output
  // rows, 0 at the other context columns)
  auto o_branch = [&]() -> sl_status {
    SkinnyArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.st = st; sa.mode = 0; sa.T = g.T;
    sa.A = d_out; sa.lda = D; sa.K = D;
    sa.nblk = 1;
    sa.Bb[0] = BoTp; sa.nbk[0] = r; sa.ldbb[0] = D;
    sa.out = dz_o; sa.ldo = rp; sa.oscale = s;
    sa.outs = dzs_o; sa.ldos = rp; sa.scale = s;
    sa.part = skp;
    sl_status st_ = launch_skinny<T>(sa, strm);
    if (st_ != SL_OK) return st_;
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.st = st;
    ga.idx = idx_o; ga.kidx = g.ko; ga.n_out = g.nq;
    ga.nseg = 2;
    ga.seg[0] = GSeg{d_out, D, 0, 0, 1, w->WoT, nullptr, D, 1, D, nullptr, 0, 0};
    set_o_base(ga.seg[0], w);
    ga.seg[1] = GSeg{dzs_o, rp, 0, 0, 1, AoTp, nullptr, rp, 1, rp, nullptr, 0, 0};
    ga.o0 = da; ga.ldo = g.nq; ga.swidth = g.nq;
    ga.rpart = reinterpret_cast<float*>(ws + g.w_rp);
    SL_HIP((launch_gather_gemm<T, MODE_NG, EPI_SCATTER, false>(ga, strm, TS_DA_BWD)));
    return SL_OK;
  };
  // the operand packing and the row layout (compact a and dq / dk / dv) on the
  // side stream: the o-branch reads neither (its Bo^T and Ao^T come from the
  // forward), so they overlap
  {
    SideFork lay;
    if ((rc = lay.begin(strm))) return rc;
    rc = pk.launch<T>(lay.side);
    if (rc == SL_OK) rc = L.launch<T>(lay.side);
    if (rc == SL_OK && d_out) rc = o_branch();
    const sl_status rj = lay.end(strm);   // joined on every path
    if (rc != SL_OK) return rc;
    if (rj != SL_OK) return rj;
  }
  if (d_out) {
    // dAo = dz_o^T a_m (scattered into So), dBo = s d_out^T z_o
    cb.scatter(ac, g.co.ld, g.co.n, g.co.out_off, g.co.kc, g.co.n, dz_o, rp, 0, rp, inv_o, gr->dAo, r, 1, 1.f);
    cb.dense(d_out, D, D, zo, rp, 0, rp, gr->dBo, r, 0, nullptr, 0, 0, 0, s);
  }
  if (dq) {
    float* dz = reinterpret_cast<float*>(ws + g.w_dz_qkv);
    T* dzs = reinterpret_cast<T*>(ws + g.w_dzs_qkv);
    // dz_j = s dj_m B_j[S_j]; products whose channel counts match (all three
    // when the q, k and v sets have equal sizes) share one launch
    for (int j0 = 0; j0 < 3;) {
      const Comp& c = *cc[j0];
      SkinnyArgs sa;
      std::memset(&sa, 0, sizeof(sa));
      sa.st = st; sa.mode = 1; sa.T = g.T;
      sa.A = dcomp[j0]; sa.lda = c.ld; sa.lda_out = c.n; sa.a_out_off = c.out_off;
      sa.K = 0; sa.kidx = c.kc; sa.n_out = c.n;
      sa.nblk = 1;
      sa.Bb[0] = Bg[j0]; sa.nbk[0] = r; sa.ldbb[0] = c.ld; sa.b0_gstride = (long long)rp * c.ld;
      sa.B0o = BTo[j0]; sa.ldb0o = c.n;
      sa.out = dz; sa.ldo = 3 * rp; sa.col0 = j0 * rp; sa.oscale = s;
      sa.outs = dzs; sa.ldos = 3 * rp; sa.scale = s;
      sa.part = skp;
      sa.nprob = 1; sa.pstride = g.skp_floats;
      int j = j0 + 1;
      for (; j < 3 && cc[j]->kc == c.kc && cc[j]->n == c.n; ++j) {
        const Comp& cj = *cc[j];
        auto& x = sa.xp[sa.nprob - 1];
        x.A = dcomp[j]; x.lda = cj.ld; x.lda_out = cj.n; x.a_out_off = cj.out_off;
        x.B0 = Bg[j]; x.ldb0 = cj.ld; x.b0_gstride = (long long)rp * cj.ld;
        x.B0o = BTo[j]; x.ldb0o = cj.n;
        x.col0 = j * rp;
        ++sa.nprob;
      }
      if ((rc = launch_skinny<T>(sa, strm))) return rc;
      j0 = j;
    }
    // dAq, dAk = dz^T X (one pass for q and k), dAv
    cb.dense(X, D, D, dz, 3 * rp, 0, 2 * rp, gr->dAq, r, 1, gr->dAk, r, 1, rp, 1.f);
    cb.dense(X, D, D, dz, 3 * rp, 2 * rp, rp, gr->dAv, r, 1, nullptr, 0, 0, 0, 1.f);
    // dB_j[S_j] = s dj_m^T z_j
    for (int j = 0; j < 3; ++j) {
      const Comp& c = *cc[j];
      cb.scatter(dcomp[j], c.ld, c.n, c.out_off, c.kc, c.n, zqkv, 3 * rp, j * rp, rp, inv[j], dB[j], r, 0, s);
    }
    // the factor gradients (one reduction launch, one finish launch) on the
    // side stream: they read only what is ready now and write their own
    // buffers, so they overlap the dX product below
    // (an optional timing event for the dX product goes before the fork, so
    // that the product and the side work become ready together)
    timer_begin(TS_DXQKV_BWD, strm);
    SideFork fork;
    if ((rc = fork.begin(strm))) return rc;
    if ((rc = cb.launch<T>(fork.side))) { (void)fork.end(strm); return rc; }
    // dX = dq Wq[Sq] + dk Wk[Sk] + dv Wv[Sv] + dz [Aq; Ak; Av]
    auto dxq = [&]() -> sl_status {
      GemmArgs ga;
      std::memset(&ga, 0, sizeof(ga));
      ga.st = st;
      ga.kidx = 1; ga.n_out = 1;
      ga.N = D;
      ga.nseg = 4;
      for (int j = 0; j < 3; ++j) {
        const Comp& c = *cc[j];
        ga.seg[j] = GSeg{dcomp[j], c.ld, c.n, c.out_off, 0, Wm[j], nullptr, D, 1, 0, sets[j], c.kc, c.n};
        if (qq) { ga.seg[j].Bs = Ws[j]; ga.seg[j].bq4 = 1; }
      }
      ga.seg[3] = GSeg{dzs, 3 * rp, 0, 0, 1, Aqkvp, nullptr, D, 0, 3 * rp, nullptr, 0, 0};
      ga.ksplit_out = g.ks_dx;
      ga.o0 = dX; ga.ldo = D;
      ga.part = part;
      ga.iota = reinterpret_cast<const int*>(ws + g.w_iota);
      SL_HIP((launch_gather_gemm<T, MODE_KG, EPI_TOKEN, false>(ga, strm, -1)));
      timer_end(TS_DXQKV_BWD, strm);
      return splitk_reduce<T>(st, part, g.ks_dx, D, dX, D, strm);
    };
    rc = dxq();
    const sl_status rj = fork.end(strm);   // joined on every path
    return rc != SL_OK ? rc : rj;
  }
  // the factor gradients of o alone: one reduction launch and one finish launch
  return cb.launch<T>(strm);
}

// A 4-bit frozen base (SparseLoRA article §六): bf16 calls, d_model % 64 == 0.
sl_status check_q4(sl_dtype dt, const sl_qkvo_weights* w) {
  if (dt != SL_BF16) SL_FAIL(SL_ERR_DTYPE, "a 4-bit frozen base needs bf16 calls");
  if (w->d_model % 64 != 0) SL_FAIL(SL_ERR_SHAPE, "a 4-bit frozen base needs d_model %% 64 == 0");
  return SL_OK;
}

sl_status check_weights(sl_dtype dt, const sl_qkvo_weights* w, bool need_qkv, bool need_o) {
  sl_status s;
  if (need_qkv) {
    if (w->Wq_q) {
      if ((s = check_q4(dt, w)) != SL_OK) return s;
      if (!w->Wk_q || !w->Wv_q || !w->Wq_s || !w->Wk_s || !w->Wv_s)
        SL_FAIL(SL_ERR_NULL, "Wq_q is set: Wk_q, Wv_q, Wq_s, Wk_s, Wv_s must be non-NULL");
      if (!aligned16(w->Wq_q) || !aligned16(w->Wk_q) || !aligned16(w->Wv_q) || !aligned16(w->Wq_s) ||
          !aligned16(w->Wk_s) || !aligned16(w->Wv_s))
        SL_FAIL(SL_ERR_ALIGN, "4-bit codes and scales must be 16-byte aligned");
    } else {
      if (!w->Wq || !w->Wk || !w->Wv) SL_FAIL(SL_ERR_NULL, "a q/k/v weight pointer is NULL");
      if (!aligned16(w->Wq) || !aligned16(w->Wk) || !aligned16(w->Wv))
        SL_FAIL(SL_ERR_ALIGN, "Wq, Wk, Wv, Aq, Ak, Av must be 16-byte aligned");
    }
    if (!w->Aq || !w->Bq || !w->Ak || !w->Bk || !w->Av || !w->Bv)
      SL_FAIL(SL_ERR_NULL, "a q/k/v weight pointer is NULL");
    if (!aligned16(w->Aq) || !aligned16(w->Ak) || !aligned16(w->Av))
      SL_FAIL(SL_ERR_ALIGN, "Wq, Wk, Wv, Aq, Ak, Av must be 16-byte aligned");
  }
  if (need_o) {
    if (w->WoT_q) {
      if ((s = check_q4(dt, w)) != SL_OK) return s;
      if (!w->WoT_s) SL_FAIL(SL_ERR_NULL, "WoT_q is set: WoT_s must be non-NULL");
      if (!aligned16(w->WoT_q) || !aligned16(w->WoT_s))
        SL_FAIL(SL_ERR_ALIGN, "4-bit codes and scales must be 16-byte aligned");
    } else {
      if (!w->WoT) SL_FAIL(SL_ERR_NULL, "an o weight pointer is NULL");
      if (!aligned16(w->WoT)) SL_FAIL(SL_ERR_ALIGN, "WoT, Ao must be 16-byte aligned");
    }
    if (!w->Ao || !w->Bo) SL_FAIL(SL_ERR_NULL, "an o weight pointer is NULL");
    if (!aligned16(w->Ao)) SL_FAIL(SL_ERR_ALIGN, "WoT, Ao must be 16-byte aligned");
  }
  return SL_OK;
}


}  // namespace

extern "C" {

size_t sl_qkvo_saved_bytes(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w) {
  QkvoGeom g;
  if (qkvo_geom(dt, lay, w, 1, 1, false, g) != SL_OK) return 0;
  return g.saved_bytes;
}

size_t sl_qkvo_workspace_bytes(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w,
                               int32_t k_qk, int32_t k_vo) {
  QkvoGeom g;
  if (qkvo_geom(dt, lay, w, k_qk, k_vo, true, g) != SL_OK) return 0;
  return g.ws_bytes;
}

sl_status sl_qkvo_fwd(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w, const void* X,
                      const void* a, int32_t k_qk, const int32_t* idx_qk, int32_t k_vo,
                      const int32_t* idx_vo, void* q, void* k, void* v, void* o, void* saved,
                      size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
  QkvoGeom g;
  sl_status s = qkvo_geom(dt, lay, w, k_qk, k_vo, true, g);
  if (s != SL_OK) return s;
  if (!X && !a) SL_FAIL(SL_ERR_NULL, "both X and a are NULL: nothing to compute");
  if ((s = check_weights(dt, w, X != nullptr, a != nullptr)) != SL_OK) return s;
  if (X && (!q || !k || !v || !idx_qk || !idx_vo))
    SL_FAIL(SL_ERR_NULL, "q, k, v, idx_qk and idx_vo are required with X");
  if (a && (!o || !idx_vo)) SL_FAIL(SL_ERR_NULL, "o and idx_vo are required with a");
  if (!saved || !ws) SL_FAIL(SL_ERR_NULL, "saved and ws must be non-NULL");
  if ((X && (!aligned16(X) || !aligned16(q) || !aligned16(k) || !aligned16(v))) ||
      (a && (!aligned16(a) || !aligned16(o))) || !aligned16(saved) || !aligned16(ws))
    SL_FAIL(SL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (saved_bytes < g.saved_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "saved buffer %zu bytes < %zu needed", saved_bytes, g.saved_bytes);
  if (ws_bytes < g.ws_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, g.ws_bytes);
  if ((s = check_arch()) != SL_OK) return s;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  if (dt == SL_BF16)
    return qkvo_fwd_impl<bf16>(g, w, X, a, idx_qk, idx_vo, q, k, v, o, reinterpret_cast<char*>(saved),
                               reinterpret_cast<char*>(ws), strm);
  return qkvo_fwd_impl<float>(g, w, X, a, idx_qk, idx_vo, q, k, v, o, reinterpret_cast<char*>(saved),
                              reinterpret_cast<char*>(ws), strm);
}

sl_status sl_qkvo_bwd(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w, const void* X,
                      const void* a, int32_t k_qk, const int32_t* idx_qk, int32_t k_vo,
                      const int32_t* idx_vo, const void* saved, size_t saved_bytes, const void* dq,
                      const void* dk, const void* dv, const void* d_out, void* dX, void* da,
                      const sl_qkvo_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  QkvoGeom g;
  sl_status s = qkvo_geom(dt, lay, w, k_qk, k_vo, true, g);
  if (s != SL_OK) return s;
  if (!dq && !d_out) SL_FAIL(SL_ERR_NULL, "both dq and d_out are NULL: nothing to compute");
  if ((s = check_weights(dt, w, dq != nullptr, d_out != nullptr)) != SL_OK) return s;
  if (!gr) SL_FAIL(SL_ERR_NULL, "grads is NULL");
  if (dq && (!dk || !dv || !X || !dX || !idx_qk || !idx_vo || !gr->dAq || !gr->dBq || !gr->dAk ||
             !gr->dBk || !gr->dAv || !gr->dBv))
    SL_FAIL(SL_ERR_NULL, "dk, dv, X, dX, idx_qk, idx_vo and the q/k/v gradients are required with dq");
  if (d_out && (!a || !da || !idx_vo || !gr->dAo || !gr->dBo))
    SL_FAIL(SL_ERR_NULL, "a, da, idx_vo, dAo and dBo are required with d_out");
  if (!saved || !ws) SL_FAIL(SL_ERR_NULL, "saved and ws must be non-NULL");
  if ((dq && (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(X) || !aligned16(dX))) ||
      (d_out && (!aligned16(d_out) || !aligned16(a) || !aligned16(da))) || !aligned16(saved) ||
      !aligned16(ws))
    SL_FAIL(SL_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (saved_bytes < g.saved_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "saved buffer %zu bytes < %zu needed", saved_bytes, g.saved_bytes);
  if (ws_bytes < g.ws_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, g.ws_bytes);
  if ((s = check_arch()) != SL_OK) return s;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  if (dt == SL_BF16)
    return qkvo_bwd_impl<bf16>(g, w, X, a, idx_qk, idx_vo, reinterpret_cast<const char*>(saved), dq,
                               dk, dv, d_out, dX, da, gr, reinterpret_cast<char*>(ws), strm);
  return qkvo_bwd_impl<float>(g, w, X, a, idx_qk, idx_vo, reinterpret_cast<const char*>(saved), dq, dk,
                              dv, d_out, dX, da, gr, reinterpret_cast<char*>(ws), strm);
}

}  // extern "C"
