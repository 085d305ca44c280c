// a4/a5: sparse LoRA SwiGLU FFN, forward and backward.
//   SparseLoRA article §一 — per-input channel choice; §三 — context tokens on
//   the selected channels, output tokens dense; §六/§七 — structured channel
//   sparsity with sliced weights; SparseLoRA abstract — loss and gradients on
//   the selected subset; SALR page §2.1 — LoRA notation.
//
// Per call (T tokens, D = d_model, F = d_ff, r = LoRA rank, rp = r rounded up
// to 8, k channels per context group):
//   forward   z = X [Ag;Au]^T                      (skinny, all tokens)
//             G, U, H = SiLU(G)*U                  (N-gather GEMM, gate+up fused,
//                                                   LoRA as an extra K segment)
//             z_d = H Ad[:,S]^T                    (skinny, per group)
//             Y = H WdT[S] + s z_d Bd^T            (K-gather GEMM)
//   backward  dz_d = s dY Bd                       (skinny)
//             dH = dY WdT[S]^T + dz_d Ad[:,S];  dG, dU from saved G, U (N-gather GEMM)
//             dz_g = s dG Bg[S], dz_u = s dU Bu[S] (skinny, per group)
//             dX = dG Wg[S] + dU Wu[S] + dz_g Ag + dz_u Au   (K-gather GEMM)
//             dA*, dB* by column reductions over tokens.
#include "sl_launch.hpp"

using namespace sl;

namespace {

struct FfnGeom {
  SeqTab st;
  int T, D, F, r, rp, k, ldk, ldF;
  size_t esz;
  long long comp, c_out_off;
  int ks_down, ks_dx, RM1, RM2, chunk;
  long long cr_floats, skp_floats;
  size_t s_zgu, s_zd, s_G, s_U, s_H, s_BdT, s_AdT, s_Agup, s_Bgg, s_Bug, s_BgTo, s_BuTo, s_iota, saved_bytes;
  size_t w_zs_gu, w_zs_d, w_Pg, w_Pu, w_Adg, w_part, w_dz_d, w_dzs_d, w_dG, w_dU,
      w_dz_gu, w_dzs_gu, w_cr, w_inv, w_skp, w_rp, ws_bytes;
};

sl_status ffn_geom(sl_dtype dt, const sl_layout* lay, long long D, long long F, int r, int k,
                   FfnGeom& g) {
  if (dt != SL_F32 && dt != SL_BF16) SL_FAIL(SL_ERR_DTYPE, "unknown dtype %d", (int)dt);
  sl_status s = build_seqtab(lay, g.st);
  if (s != SL_OK) return s;
  if (D < 8 || D % 8 || F < 8 || F % 8 || D > (1 << 20) || F > (1 << 20))
    SL_FAIL(SL_ERR_SHAPE, "d_model = %lld and d_ff = %lld must be positive multiples of 8", D, F);
  if (r < 1 || r > 32) SL_FAIL(SL_ERR_RANGE, "lora_rank %d outside [1, 32]", r);
  if (k < 1 || k > F) SL_FAIL(SL_ERR_RANGE, "k = %d outside [1, %lld]", k, F);
  const SeqTab& st = g.st;
  if ((s = check_extent("X / dY / Y / dX", (long long)st.nseq * st.L, D)) != SL_OK) return s;
  if ((s = check_extent("a frozen weight", F, D)) != SL_OK) return s;
  if ((s = check_extent("the compact G / U / H buffers", 1,
                        (long long)st.T_ctx * round_up(k, 8) + (long long)st.T_out * F)) != SL_OK)
    return s;
  g.T = st.nseq * st.L;
  g.D = (int)D; g.F = (int)F; g.r = r; g.k = k;
  g.rp = (int)round_up(r, 8);
  g.ldk = (int)round_up(k, 8);
  g.ldF = (int)F;
  g.esz = dt == SL_BF16 ? 2 : 4;
  g.comp = (long long)st.T_ctx * g.ldk + (long long)st.T_out * g.ldF;
  g.c_out_off = (long long)st.T_ctx * g.ldk;
  const int bk = dt == SL_BF16 ? 64 : 32;
  g.ks_down = kg_choose_ksplit(st, k + g.rp, F + g.rp, g.D, bk, dt == SL_BF16);
  g.ks_dx = kg_choose_ksplit(st, 2LL * k + 2 * g.rp, 2 * F + 2 * g.rp, g.D, bk, dt == SL_BF16);
  g.RM1 = cr_rm(g.esz, g.rp);
  g.RM2 = cr_rm(g.esz, 2 * g.rp);
  g.chunk = cr_chunk(g.esz);
  const size_t T = g.T, e = g.esz;
  Bump sv;
  g.s_zgu = sv.take(T * 2 * g.rp * 4);
  g.s_zd = sv.take(T * g.rp * 4);
  g.s_G = sv.take(g.comp * e);
  g.s_U = sv.take(g.comp * e);
  g.s_H = sv.take(g.comp * e);
  // the backward's LoRA operands, packed by the forward: Bd^T and Ad^T for its
  // first products, [Ag; Au] (rank padded), B_g[S]^T and B_u[S]^T per context
  // group, B_g^T and B_u^T, and 0, 1, 2, ... for the K-gather products
  g.s_BdT = sv.take((size_t)g.rp * D * e);
  g.s_AdT = sv.take((size_t)F * g.rp * e);
  g.s_Agup = sv.take((size_t)2 * g.rp * D * e);
  g.s_Bgg = sv.take((size_t)st.nseq * g.rp * g.ldk * e);
  g.s_Bug = sv.take((size_t)st.nseq * g.rp * g.ldk * e);
  g.s_BgTo = sv.take((size_t)g.rp * F * e);
  g.s_BuTo = sv.take((size_t)g.rp * F * e);
  g.s_iota = sv.take((size_t)(F > 2 * g.rp ? F : 2 * g.rp) * 4);
  g.saved_bytes = sv.off;
  Bump w;
  g.w_zs_gu = w.take(T * 2 * g.rp * e);
  g.w_zs_d = w.take(T * g.rp * e);
  g.w_Pg = w.take((size_t)F * 2 * g.rp * e);
  g.w_Pu = w.take((size_t)F * 2 * g.rp * e);
  g.w_Adg = w.take((size_t)st.nseq * g.rp * g.ldk * e);
  const int ks = g.ks_down > g.ks_dx ? g.ks_down : g.ks_dx;
  g.w_part = w.take(ks > 1 ? (size_t)ks * st.T_out * D * 4 : 0);
  g.w_dz_d = w.take(T * g.rp * 4);
  g.w_dzs_d = w.take(T * g.rp * e);
  g.w_dG = w.take(g.comp * e);
  g.w_dU = w.take(g.comp * e);
  g.w_dz_gu = w.take(T * 2 * g.rp * 4);
  g.w_dzs_gu = w.take(T * 2 * g.rp * e);
  // partials of the five gradient reductions (dA_g,u; dB_d; dB_g, dB_u, dA_d)
  const long long cr = cb_dense_floats(st, e, D, 2 * g.rp) + cb_dense_floats(st, e, D, g.rp) +
                       3 * cb_scatter_floats(st, e, k, g.F, g.rp);
  g.cr_floats = cr;
  g.w_cr = w.take((size_t)cr * 4);
  g.w_inv = w.take((size_t)st.nseq * F * 4);
  // skinny partial sums: room for the two problems of the dz_g / dz_u launch
  g.skp_floats = skinny_part_floats(g.T, D > F ? D : F);
  g.w_skp = w.take((size_t)g.skp_floats * 2 * 4);
  {
    // split last round of the gate/up (dual) and dH gather-GEMMs
    const long long f1 = ng_rpart_floats(st, g.k, F, true, g.esz, {(int)D, 2 * g.rp});
    const long long f2 = ng_rpart_floats(st, g.k, F, false, g.esz, {(int)D, g.rp});
    g.w_rp = w.take((size_t)(f1 > f2 ? f1 : f2) * 4);
  }
  g.ws_bytes = w.off;
  return SL_OK;
}

sl_status check_ffn_ptrs(sl_dtype dt, const sl_ffn_weights* w, const void* X) {
  if (!w) SL_FAIL(SL_ERR_NULL, "weights is NULL");
  if (w->Wg_q) {
    // 4-bit frozen base (SparseLoRA article §六): codes and block scales
    if (dt != SL_BF16) SL_FAIL(SL_ERR_DTYPE, "a 4-bit frozen base needs bf16 calls");
    if (w->d_model % 64 != 0) SL_FAIL(SL_ERR_SHAPE, "a 4-bit frozen base needs d_model %% 64 == 0");
    if (!w->Wu_q || !w->WdT_q || !w->Wg_s || !w->Wu_s || !w->WdT_s)
      SL_FAIL(SL_ERR_NULL, "Wg_q is set: Wu_q, WdT_q, Wg_s, Wu_s, WdT_s must be non-NULL");
    if (!aligned16(w->Wg_q) || !aligned16(w->Wu_q) || !aligned16(w->WdT_q) || !aligned16(w->Wg_s) ||
        !aligned16(w->Wu_s) || !aligned16(w->WdT_s))
      SL_FAIL(SL_ERR_ALIGN, "4-bit codes and scales must be 16-byte aligned");
  } else {
    if (!w->Wg || !w->Wu || !w->WdT) SL_FAIL(SL_ERR_NULL, "a weight or input pointer is NULL");
    if (!aligned16(w->Wg) || !aligned16(w->Wu) || !aligned16(w->WdT))
      SL_FAIL(SL_ERR_ALIGN, "X, Wg, Wu, WdT, Ag, Au must be 16-byte aligned");
  }
  if (!X || !w->Ag || !w->Bg || !w->Au || !w->Bu || !w->Ad || !w->Bd)
    SL_FAIL(SL_ERR_NULL, "a weight or input pointer is NULL");
  if (!aligned16(X) || !aligned16(w->Ag) || !aligned16(w->Au))
    SL_FAIL(SL_ERR_ALIGN, "X, Wg, Wu, WdT, Ag, Au must be 16-byte aligned");
  return SL_OK;
}

// Base segment of a gather-GEMM over frozen weight W (plain) or its 4-bit
// codes Wq with scales Ws (w->Wg_q set); B2 / B2q / B2s: dual mode's up half.
inline void set_base(GSeg& sg, const sl_ffn_weights* w, const void* W, const void* Wq, const float* Ws,
                     const void* W2 = nullptr, const void* W2q = nullptr, const float* W2s = nullptr) {
  if (w->Wg_q) {
    sg.B = Wq; sg.Bs = Ws; sg.B2 = W2q; sg.B2s = W2s; sg.bq4 = 1;
  } else {
    sg.B = W; sg.B2 = W2;
  }
}

template <typename T>
sl_status ffn_fwd_impl(const FfnGeom& g, const sl_ffn_weights* w, const void* X, const int* idx,
                       void* Y, char* sv, char* ws, hipStream_t strm) {
  const SeqTab& st = g.st;
  const int D = g.D, F = g.F, r = g.r, rp = g.rp;
  const float s = w->lora_scale;
  sl_status rc;
  float* zgu = reinterpret_cast<float*>(sv + g.s_zgu);
  float* zd = reinterpret_cast<float*>(sv + g.s_zd);
  T* Gc = reinterpret_cast<T*>(sv + g.s_G);
  T* Uc = reinterpret_cast<T*>(sv + g.s_U);
  T* Hc = reinterpret_cast<T*>(sv + g.s_H);
  T* zs_gu = reinterpret_cast<T*>(ws + g.w_zs_gu);
  T* zs_d = reinterpret_cast<T*>(ws + g.w_zs_d);
  T* Pg = reinterpret_cast<T*>(ws + g.w_Pg);
  T* Pu = reinterpret_cast<T*>(ws + g.w_Pu);
  T* BdTp = reinterpret_cast<T*>(sv + g.s_BdT);
  T* AdTp = reinterpret_cast<T*>(sv + g.s_AdT);
  T* Adg = reinterpret_cast<T*>(ws + g.w_Adg);
  float* part = reinterpret_cast<float*>(ws + g.w_part);
  float* skp = reinterpret_cast<float*>(ws + g.w_skp);

  // LoRA operands padded to rp columns, one launch: Pg = [Bg | 0], Pu = [0 |
  // Bu] and Adg[g] = Ad[:, S_g] (gathered per context group) for this pass;
  // for the backward, in the saved buffer, Bd^T, Ad^T, [Ag; Au], B_g[S]^T and
  // B_u[S]^T per context group, B_g^T, B_u^T and the index ramp, so that the
  // backward's products never wait for a packing launch (each wait or fork on
  // the caller's stream leaves it idle about 5 us).  It stays on the caller's
  // stream: on a side stream it overlapped the z product below, but the fork
  // and join cost more than the 11 us it hid (FFN step 853 us with the fork,
  // 849 us without, same box).
  {
    Packer pk;
    pk.copy(Pg, 2 * rp, F, 2 * rp, w->Bg, r, F, r, 0);
    pk.copy(Pu, 2 * rp, F, 2 * rp, w->Bu, r, F, r, 0, 0, rp);
    pk.copy(BdTp, D, rp, D, w->Bd, r, r, D, 1);
    pk.copy(AdTp, rp, F, rp, w->Ad, F, F, r, 1);
    pk.gather(Adg, g.ldk, (long long)rp * g.ldk, rp, g.ldk, w->Ad, F, r, 0, idx, g.k, st.nseq);
    T* Agup = reinterpret_cast<T*>(sv + g.s_Agup);
    pk.copy(Agup, D, rp, D, w->Ag, D, r, D, 0);
    pk.copy(Agup + (long long)rp * D, D, rp, D, w->Au, D, r, D, 0);
    pk.gather(reinterpret_cast<T*>(sv + g.s_Bgg), g.ldk, (long long)rp * g.ldk, rp, g.ldk, w->Bg, r, r, 1, idx,
              g.k, st.nseq);
    pk.gather(reinterpret_cast<T*>(sv + g.s_Bug), g.ldk, (long long)rp * g.ldk, rp, g.ldk, w->Bu, r, r, 1, idx,
              g.k, st.nseq);
    pk.copy(reinterpret_cast<T*>(sv + g.s_BgTo), F, r, F, w->Bg, r, r, F, 1);
    pk.copy(reinterpret_cast<T*>(sv + g.s_BuTo), F, r, F, w->Bu, r, r, F, 1);
    pk.iota(reinterpret_cast<int*>(sv + g.s_iota), F > 2 * rp ? F : 2 * rp);
    rc = pk.launch<T>(strm);
  }
  // z = X [Ag; Au]^T  (fp32 saved, s*z in T for the GEMM)
  if (rc == SL_OK) {
    SkinnyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st; a.mode = 0; a.T = g.T;
    a.A = X; a.lda = D; a.K = D;
    a.nblk = 2;
    a.Bb[0] = w->Ag; a.nbk[0] = r; a.ldbb[0] = D;
    a.Bb[1] = w->Au; a.nbk[1] = r; a.ldbb[1] = D;
    a.out = zgu; a.ldo = 2 * rp; a.col0 = 0; a.oscale = 1.f;
    a.outs = zs_gu; a.ldos = 2 * rp; a.scale = s;
    a.part = skp;
    rc = launch_skinny<T>(a, strm);
  }
  if (rc != SL_OK) return rc;
  // G, U, H on the selected channels (context) / all channels (output rows)
  {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st;
    a.idx = idx; a.kidx = g.k; a.n_out = F;
    a.nseg = 2;
    a.seg[0] = GSeg{X, D, 0, 0, 1, w->Wg, w->Wu, D, 1, D, nullptr, 0, 0};
    set_base(a.seg[0], w, w->Wg, w->Wg_q, w->Wg_s, w->Wu, w->Wu_q, w->Wu_s);
    a.seg[1] = GSeg{zs_gu, 2 * rp, 0, 0, 1, Pg, Pu, 2 * rp, 1, 2 * rp, nullptr, 0, 0};
    a.o0 = Gc; a.o1 = Uc; a.o2 = Hc;
    a.rpart = reinterpret_cast<float*>(ws + g.w_rp);
    a.ldc_ctx = g.ldk; a.ldc_out = g.ldF; a.c_out_off = g.c_out_off;
    SL_HIP((launch_gather_gemm<T, MODE_NG, EPI_SWIGLU, true>(a, strm, TS_GU_FWD)));
  }
  // z_d = H Ad[:, S]^T
  {
    SkinnyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st; a.mode = 1; a.T = g.T;
    a.A = Hc; a.lda = g.ldk; a.lda_out = g.ldF; a.a_out_off = g.c_out_off;
    a.K = 0; a.kidx = g.k; a.n_out = F;
    a.nblk = 1;
    a.Bb[0] = Adg; a.nbk[0] = r; a.ldbb[0] = g.ldk; a.b0_gstride = (long long)rp * g.ldk;
    a.B0o = w->Ad; a.ldb0o = F;
    a.out = zd; a.ldo = rp; a.oscale = 1.f;
    a.outs = zs_d; a.ldos = rp; a.scale = s;
    a.part = skp;
    if ((rc = launch_skinny<T>(a, strm))) return rc;
  }
  // Y = H WdT[S] + s z_d Bd^T
  {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st;
    a.kidx = 1; a.n_out = 1;
    a.N = D;
    a.nseg = 2;
    a.seg[0] = GSeg{Hc, g.ldk, g.ldF, g.c_out_off, 0, w->WdT, nullptr, D, 1, 0, idx, g.k, F};
    set_base(a.seg[0], w, w->WdT, w->WdT_q, w->WdT_s);
    a.seg[1] = GSeg{zs_d, rp, 0, 0, 1, BdTp, nullptr, D, 0, rp, nullptr, 0, 0};
    a.ksplit_out = g.ks_down;
    a.o0 = Y; a.ldo = D;
    a.part = part;
    a.iota = reinterpret_cast<const int*>(sv + g.s_iota);
    SL_HIP((launch_gather_gemm<T, MODE_KG, EPI_TOKEN, false>(a, strm, TS_DOWN_FWD)));
    if ((rc = splitk_reduce<T>(st, part, g.ks_down, D, Y, D, strm))) return rc;
  }
  return SL_OK;
}

template <typename T>
sl_status ffn_bwd_impl(const FfnGeom& g, const sl_ffn_weights* w, const void* X, const int* idx,
                       const char* sv, const void* dY, void* dX, const sl_ffn_grads* gr, char* ws,
                       hipStream_t strm) {
  const SeqTab& st = g.st;
  const int D = g.D, F = g.F, r = g.r, rp = g.rp;
  const float s = w->lora_scale;
  sl_status rc;
  const float* zgu = reinterpret_cast<const float*>(sv + g.s_zgu);
  const float* zd = reinterpret_cast<const float*>(sv + g.s_zd);
  const T* Gc = reinterpret_cast<const T*>(sv + g.s_G);
  const T* Uc = reinterpret_cast<const T*>(sv + g.s_U);
  const T* Hc = reinterpret_cast<const T*>(sv + g.s_H);
  float* part = reinterpret_cast<float*>(ws + g.w_part);
  float* dz_d = reinterpret_cast<float*>(ws + g.w_dz_d);
  T* dzs_d = reinterpret_cast<T*>(ws + g.w_dzs_d);
  const T* AdTp = reinterpret_cast<const T*>(sv + g.s_AdT);   // packed by the forward
  T* dGc = reinterpret_cast<T*>(ws + g.w_dG);
  T* dUc = reinterpret_cast<T*>(ws + g.w_dU);
  // packed by the forward
  const T* Bgg = reinterpret_cast<const T*>(sv + g.s_Bgg);
  const T* Bug = reinterpret_cast<const T*>(sv + g.s_Bug);
  const T* BgTo = reinterpret_cast<const T*>(sv + g.s_BgTo);
  const T* BuTo = reinterpret_cast<const T*>(sv + g.s_BuTo);
  float* dz_gu = reinterpret_cast<float*>(ws + g.w_dz_gu);
  T* dzs_gu = reinterpret_cast<T*>(ws + g.w_dzs_gu);
  const T* Agup = reinterpret_cast<const T*>(sv + g.s_Agup);
  const T* BdTp = reinterpret_cast<const T*>(sv + g.s_BdT);
  float* crp = reinterpret_cast<float*>(ws + g.w_cr);
  int* inv = reinterpret_cast<int*>(ws + g.w_inv);
  float* skp = reinterpret_cast<float*>(ws + g.w_skp);

  // dz_d = s dY Bd (Bd^T and every other LoRA operand the backward reads come
  // packed from the forward, so no product here waits for a packing launch)
  {
    SkinnyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st; a.mode = 0; a.T = g.T;
    a.A = dY; a.lda = D; a.K = D;
    a.nblk = 1;
    a.Bb[0] = BdTp; a.nbk[0] = r; a.ldbb[0] = D;
    a.out = dz_d; a.ldo = rp; a.oscale = s;
    a.outs = dzs_d; a.ldos = rp; a.scale = s;
    a.part = skp;
    if ((rc = launch_skinny<T>(a, strm))) return rc;
  }
  // Side stream: the inverse map of the channel sets, then the factor
  // gradients that need neither dG nor dU (dBd = s dY^T z_d, dAd[:, S] =
  // dz_d^T H), beside the dH product, whose grid leaves CUs idle (their own
  // partials: the first part of the reduction workspace).
  SideFork side;
  if ((rc = side.begin(strm))) return rc;
  auto side_fail = [&](sl_status e) { (void)side.end(strm); return e; };
  {
    Packer pk;
    pk.inverse(inv, idx, g.k, F, st.nseq);
    if ((rc = pk.launch<T>(side.side))) return side_fail(rc);
  }
  ColredBatch cb_d(st, g.esz, crp, g.cr_floats);
  cb_d.dense(dY, D, D, zd, rp, 0, rp, gr->dBd, r, 0, nullptr, 0, 0, 0, s);
  cb_d.scatter(Hc, g.ldk, g.ldF, g.c_out_off, g.k, F, dz_d, rp, 0, rp, inv, gr->dAd, r, 1, 1.f);
  if ((rc = cb_d.launch<T>(side.side))) return side_fail(rc);
  // dH = dY WdT[S]^T + dz_d Ad[:, S]  ->  dG, dU
  {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st;
    a.idx = idx; a.kidx = g.k; a.n_out = F;
    a.nseg = 2;
    a.seg[0] = GSeg{dY, D, 0, 0, 1, w->WdT, nullptr, D, 1, D, nullptr, 0, 0};
    set_base(a.seg[0], w, w->WdT, w->WdT_q, w->WdT_s);
    a.seg[1] = GSeg{dzs_d, rp, 0, 0, 1, AdTp, nullptr, rp, 1, rp, nullptr, 0, 0};
    a.o0 = dGc; a.o1 = dUc;
    a.i0 = Gc; a.i1 = Uc;
    a.rpart = reinterpret_cast<float*>(ws + g.w_rp);
    a.ldc_ctx = g.ldk; a.ldc_out = g.ldF; a.c_out_off = g.c_out_off;
    const hipError_t e = launch_gather_gemm<T, MODE_NG, EPI_DSWIGLU, false>(a, strm, TS_DH_BWD);
    if (e != hipSuccess) {
      set_error("dH product launch failed: %s", hipGetErrorString(e));
      return side_fail(SL_ERR_HIP);
    }
  }
  // dBg[S] = s dG^T z_g, dBu[S] = s dU^T z_u on the side stream as soon as dG
  // and dU exist: they run beside the dz_g / dz_u product, whose small grid
  // leaves CUs idle, instead of behind the dX product that fills every CU
  if ((rc = side.refork(strm))) return side_fail(rc);
  ColredBatch cb_gu(st, g.esz, crp + cb_d.used, g.cr_floats - cb_d.used);
  cb_gu.scatter(dGc, g.ldk, g.ldF, g.c_out_off, g.k, F, zgu, 2 * rp, 0, rp, inv, gr->dBg, r, 0, s);
  cb_gu.scatter(dUc, g.ldk, g.ldF, g.c_out_off, g.k, F, zgu, 2 * rp, rp, rp, inv, gr->dBu, r, 0, s);
  if ((rc = cb_gu.launch<T>(side.side))) return side_fail(rc);
  // dz_g = s dG Bg[S], dz_u = s dU Bu[S]: one launch, two problems
  {
    SkinnyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st; a.mode = 1; a.T = g.T;
    a.A = dGc; a.lda = g.ldk; a.lda_out = g.ldF; a.a_out_off = g.c_out_off;
    a.K = 0; a.kidx = g.k; a.n_out = F;
    a.nblk = 1;
    a.Bb[0] = Bgg; a.nbk[0] = r; a.ldbb[0] = g.ldk; a.b0_gstride = (long long)rp * g.ldk;
    a.B0o = BgTo; a.ldb0o = F;
    a.out = dz_gu; a.ldo = 2 * rp; a.col0 = 0; a.oscale = s;
    a.outs = dzs_gu; a.ldos = 2 * rp; a.scale = s;
    a.part = skp;
    a.nprob = 2; a.pstride = g.skp_floats;
    auto& u = a.xp[0];
    u.A = dUc; u.lda = g.ldk; u.lda_out = g.ldF; u.a_out_off = g.c_out_off;
    u.B0 = Bug; u.ldb0 = g.ldk; u.b0_gstride = (long long)rp * g.ldk;
    u.B0o = BuTo; u.ldb0o = F;
    u.col0 = rp;
    if ((rc = launch_skinny<T>(a, strm))) return side_fail(rc);
  }
  // dAg, dAu = dz^T X (one reduction launch, one finish launch) on the side
  // stream, after the other factor gradients: they read only what is ready
  // now and write their own buffers (the rest of the reduction workspace), so
  // they overlap the dX product below.
  // (an optional timing event for the dX product goes before the fork, so that
  // the product and the side work become ready together)
  timer_begin(TS_DX_BWD, strm);
  if ((rc = side.refork(strm))) return side_fail(rc);
  {
    ColredBatch cb(st, g.esz, crp + cb_d.used + cb_gu.used, g.cr_floats - cb_d.used - cb_gu.used);
    cb.dense(X, D, D, dz_gu, 2 * rp, 0, 2 * rp, gr->dAg, r, 1, gr->dAu, r, 1, rp, 1.f);
    if ((rc = cb.launch<T>(side.side))) return side_fail(rc);
  }
  // dX = dG Wg[S] + dU Wu[S] + dz_g Ag + dz_u Au
  auto dx = [&]() -> sl_status {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st = st;
    a.kidx = 1; a.n_out = 1;
    a.N = D;
    a.nseg = 3;
    a.seg[0] = GSeg{dGc, g.ldk, g.ldF, g.c_out_off, 0, w->Wg, nullptr, D, 1, 0, idx, g.k, F};
    a.seg[1] = GSeg{dUc, g.ldk, g.ldF, g.c_out_off, 0, w->Wu, nullptr, D, 1, 0, idx, g.k, F};
    set_base(a.seg[0], w, w->Wg, w->Wg_q, w->Wg_s);
    set_base(a.seg[1], w, w->Wu, w->Wu_q, w->Wu_s);
    a.seg[2] = GSeg{dzs_gu, 2 * rp, 0, 0, 1, Agup, nullptr, D, 0, 2 * rp, nullptr, 0, 0};
    a.ksplit_out = g.ks_dx;
    a.o0 = dX; a.ldo = D;
    a.part = part;
    a.iota = reinterpret_cast<const int*>(sv + g.s_iota);
    SL_HIP((launch_gather_gemm<T, MODE_KG, EPI_TOKEN, false>(a, strm, -1)));
    timer_end(TS_DX_BWD, strm);
    return splitk_reduce<T>(st, part, g.ks_dx, D, dX, D, strm);
  };
  rc = dx();
  const sl_status rj = side.end(strm);   // joined on every path
  return rc != SL_OK ? rc : rj;
}

}  // namespace

extern "C" {

size_t sl_ffn_saved_bytes(sl_dtype dt, const sl_layout* lay, int64_t d_model, int64_t d_ff,
                          int32_t lora_rank, int32_t k) {
  FfnGeom g;
  if (ffn_geom(dt, lay, d_model, d_ff, lora_rank, k, g) != SL_OK) return 0;
  return g.saved_bytes;
}

size_t sl_ffn_workspace_bytes(sl_dtype dt, const sl_layout* lay, int64_t d_model, int64_t d_ff,
                              int32_t lora_rank, int32_t k) {
  FfnGeom g;
  if (ffn_geom(dt, lay, d_model, d_ff, lora_rank, k, g) != SL_OK) return 0;
  return g.ws_bytes;
}

sl_status sl_ffn_fwd(sl_dtype dt, const sl_layout* lay, const sl_ffn_weights* w, const void* X,
                     int32_t k, const int32_t* idx, void* Y, void* saved, size_t saved_bytes,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!w) SL_FAIL(SL_ERR_NULL, "weights is NULL");
  FfnGeom g;
  sl_status s = ffn_geom(dt, lay, w->d_model, w->d_ff, w->lora_rank, k, g);
  if (s != SL_OK) return s;
  if ((s = check_ffn_ptrs(dt, w, X)) != SL_OK) return s;
  if (!idx || !Y || !saved || !ws) SL_FAIL(SL_ERR_NULL, "idx, Y, saved and ws must be non-NULL");
  if (!aligned16(Y) || !aligned16(saved) || !aligned16(ws))
    SL_FAIL(SL_ERR_ALIGN, "Y, saved and ws must be 16-byte aligned");
  if (saved_bytes < g.saved_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "saved buffer %zu bytes < %zu needed", saved_bytes, g.saved_bytes);
  if (ws_bytes < g.ws_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, g.ws_bytes);
  if ((s = check_arch()) != SL_OK) return s;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  if (dt == SL_BF16)
    return ffn_fwd_impl<bf16>(g, w, X, idx, Y, reinterpret_cast<char*>(saved),
                              reinterpret_cast<char*>(ws), strm);
  return ffn_fwd_impl<float>(g, w, X, idx, Y, reinterpret_cast<char*>(saved),
                             reinterpret_cast<char*>(ws), strm);
}

sl_status sl_ffn_bwd(sl_dtype dt, const sl_layout* lay, const sl_ffn_weights* w, const void* X,
                     int32_t k, const int32_t* idx, const void* saved, size_t saved_bytes,
                     const void* dY, void* dX, const sl_ffn_grads* gr, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!w) SL_FAIL(SL_ERR_NULL, "weights is NULL");
  FfnGeom g;
  sl_status s = ffn_geom(dt, lay, w->d_model, w->d_ff, w->lora_rank, k, g);
  if (s != SL_OK) return s;
  if ((s = check_ffn_ptrs(dt, w, X)) != SL_OK) return s;
  if (!gr || !gr->dAg || !gr->dBg || !gr->dAu || !gr->dBu || !gr->dAd || !gr->dBd)
    SL_FAIL(SL_ERR_NULL, "a gradient pointer is NULL");
  if (!idx || !saved || !dY || !dX || !ws)
    SL_FAIL(SL_ERR_NULL, "idx, saved, dY, dX and ws must be non-NULL");
  if (!aligned16(saved) || !aligned16(dY) || !aligned16(dX) || !aligned16(ws))
    SL_FAIL(SL_ERR_ALIGN, "saved, dY, dX and ws must be 16-byte aligned");
  if (saved_bytes < g.saved_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "saved buffer %zu bytes < %zu needed", saved_bytes, g.saved_bytes);
  if (ws_bytes < g.ws_bytes)
    SL_FAIL(SL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, g.ws_bytes);
  if ((s = check_arch()) != SL_OK) return s;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  if (dt == SL_BF16)
    return ffn_bwd_impl<bf16>(g, w, X, idx, reinterpret_cast<const char*>(saved), dY, dX, gr,
                              reinterpret_cast<char*>(ws), strm);
  return ffn_bwd_impl<float>(g, w, X, idx, reinterpret_cast<const char*>(saved), dY, dX, gr,
                             reinterpret_cast<char*>(ws), strm);
}

}  // extern "C"
