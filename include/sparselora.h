/* sparselora.h — C ABI of the contextual-sparsity LoRA hot path on gfx950.
 *
 * What the library computes (sources are the pages the method is described on):
 *   - "SparseLoRA article": the lsdiaocha.cn write-up of SparseLoRA (ICML 2025),
 *     sections 一 (dynamic contextual sparsity; L2-norm criterion for the FFN,
 *     QK-norm criterion for q/k), 二 (training-free SVD sparsity estimator,
 *     computed once offline, low-rank approximation of the activations),
 *     三 (non-uniform per-layer sparsity; context tokens sparse, output tokens
 *     dense), 六 (structured sparsity for real GPU speedups) and 七 (rank-8
 *     estimator; careful slicing of sparse weights and compute order).
 *   - "SparseLoRA abstract": the xinfinite.net page "SparseLoRA：利用上下文稀疏性
 *     高效微调大语言模型" — loss and gradients are computed on a dynamically
 *     selected sparse subset of the weights.
 *   - "SALR page": the lshu.cn article, §2.1 — LoRA notation: frozen W plus a
 *     trained product of two low-rank factors.
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to row-major, contiguous arrays,
 *     16-byte aligned, unless a comment says [host].  Element type is given by
 *     the call's sl_dtype (fp32 or bf16) unless the comment says fp32/int32.
 *   - Tokens are packed as T = batch * seq_len rows; sequence b owns rows
 *     [b*seq_len, (b+1)*seq_len).  Its first ctx_len[b] rows are context tokens
 *     (computed on the selected channels only); the remaining seq_len-ctx_len[b]
 *     rows are output (loss) tokens and are computed dense.
 *   - LoRA: y = x W^T + s (x A^T) B^T with A [r, in], B [out, r] and s = lora_scale.
 *     A dropped channel drops its LoRA part too.
 *   - Channel index sets idx [batch, k] hold, per sequence, k distinct channel
 *     numbers in ascending order (what sl_estimate_select writes).  Callers may
 *     pass their own; they are not re-validated on the device.
 *   - The library never allocates device memory.  Scratch space is the caller's
 *     `ws` buffer (query its size with the *_workspace_bytes function); state the
 *     backward needs is written by the forward into the caller's `saved` buffer.
 *     No pointer is kept after a call returns.
 *   - All work is enqueued on `stream` (a hipStream_t, NULL = default stream).
 *     Calls never synchronise, except sl_build_estimator (documented there).
 *     Calls overlap independent parts of their work on a side stream (default
 *     priority, non-blocking), forked from and joined back to `stream` with
 *     events: the call's work completes in order on `stream` as if it had all
 *     been enqueued there.  Each (device, `stream`) pair gets a side stream of
 *     its own at its first call, kept until the process ends, so calls on
 *     independent streams never wait for each other; past 256 such pairs a
 *     call keeps all of its work on `stream`.  While `stream` is being
 *     captured into a graph, all of the call's work stays on it (the graph
 *     holds no cross-stream events).
 *   - Every argument is validated on the host before anything is launched.  On
 *     error nothing is launched, the status says which class of error, and
 *     sl_last_error() (thread-local) holds a message.  Launch failures map to
 *     SL_ERR_HIP; device faults surface at the caller's next synchronisation.
 *   - Calls that share a `ws` or `saved` buffer must be stream-ordered.
 */
#ifndef SPARSELORA_H
#define SPARSELORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SL_ABI_VERSION 3
#define SL_MAX_SEQS 64  /* sequences per call (batch) */

typedef enum sl_status {
  SL_OK = 0,
  SL_ERR_NULL = 1,              /* a required pointer is NULL */
  SL_ERR_ALIGN = 2,             /* a pointer is not 16-byte aligned */
  SL_ERR_SHAPE = 3,             /* inconsistent or unsupported sizes */
  SL_ERR_DTYPE = 4,             /* unknown sl_dtype / sl_criterion */
  SL_ERR_RANGE = 5,             /* k, rank, ctx_len or batch out of range */
  SL_ERR_WORKSPACE = 6,         /* ws or saved buffer too small */
  SL_ERR_UNSUPPORTED_ARCH = 7,  /* current device is not gfx950 */
  SL_ERR_HIP = 8                /* a HIP runtime call or launch failed */
} sl_status;

typedef enum sl_dtype { SL_F32 = 0, SL_BF16 = 1 } sl_dtype;

/* Channel criteria (SparseLoRA article §一):
 *   SWIGLU_L2 — FFN: sum over context tokens of h^2, h = SiLU(g) * u with g, u
 *               the low-rank estimates of the gate and up projections.
 *   L2        — a plain projection (v; o reuses v's set): sum of v^2.
 *   QK_NORM   — q/k, in kv-channel space: ||k_c||^2 * sum over the query heads
 *               sharing kv head of c of ||q_(h,d)||^2 ((||q_c|| ||k_c||)^2 when
 *               every query head has its own kv head). */
typedef enum sl_criterion { SL_CRIT_SWIGLU_L2 = 0, SL_CRIT_L2 = 1, SL_CRIT_QK_NORM = 2 } sl_criterion;

typedef struct sl_layout {
  int32_t batch;            /* 1..SL_MAX_SEQS sequences */
  int32_t seq_len;          /* rows per sequence */
  const int32_t* ctx_len;   /* [host] batch entries, 0 <= ctx_len[b] <= seq_len */
} sl_layout;

typedef struct sl_heads {
  int32_t n_q_heads, n_kv_heads, head_dim;   /* n_q_heads % n_kv_heads == 0 */
} sl_heads;

/* Frozen weights and LoRA factors of one SwiGLU FFN layer (call dtype).
 *   Wg, Wu  [d_ff, d_model]   gate / up projection weights
 *   WdT     [d_ff, d_model]   TRANSPOSE of the down projection weight [d_model, d_ff]
 *                             (a one-time copy; the weight is frozen)
 *   Ag, Au  [r, d_model]      Bg, Bu [d_ff, r]
 *   Ad      [r, d_ff]         Bd     [d_model, r]                               */
typedef struct sl_ffn_weights {
  int64_t d_model, d_ff;
  int32_t lora_rank;
  float lora_scale;
  const void *Wg, *Wu, *WdT;
  const void *Ag, *Bg, *Au, *Bu, *Ad, *Bd;
  /* Optional 4-bit frozen base (SparseLoRA article §六: SparseLoRA over a
   * QLoRA-style quantized base).  When Wg_q is not NULL the frozen weights are
   * these, and Wg, Wu, WdT are ignored (may be NULL):
   *   Wg_q, Wu_q, WdT_q  uint8 [d_ff, d_model / 2]: element 2j of a row in the
   *                      low nibble of byte j, element 2j+1 in the high nibble,
   *                      signed two's-complement codes
   *   Wg_s, Wu_s, WdT_s  fp32 [d_ff, d_model / 64]: the scale of each block of
   *                      64 consecutive elements of a row
   * The weight element is code * scale.  bf16 calls only; d_model a multiple of
   * 64; all six 16-byte aligned.  Zero-initialised (C) or NULL: plain weights. */
  const void *Wg_q, *Wu_q, *WdT_q;
  const float *Wg_s, *Wu_s, *WdT_s;
} sl_ffn_weights;

/* LoRA gradients of one FFN layer, fp32, shapes of the factors; OVERWRITTEN. */
typedef struct sl_ffn_grads {
  float *dAg, *dBg, *dAu, *dBu, *dAd, *dBd;
} sl_ffn_grads;

/* Frozen weights and LoRA factors of one attention block's projections.
 *   Wq  [Hq*hd, d_model]   Wk, Wv [Hkv*hd, d_model]
 *   WoT [Hq*hd, d_model]   TRANSPOSE of the o projection weight [d_model, Hq*hd]
 *   Aq, Ak, Av [r, d_model]; Bq [Hq*hd, r]; Bk, Bv [Hkv*hd, r]
 *   Ao [r, Hq*hd]; Bo [d_model, r]                                             */
typedef struct sl_qkvo_weights {
  int64_t d_model;
  sl_heads heads;
  int32_t lora_rank;
  float lora_scale;
  const void *Wq, *Wk, *Wv, *WoT;
  const void *Aq, *Bq, *Ak, *Bk, *Av, *Bv, *Ao, *Bo;
  /* Optional 4-bit frozen bases, in the format of sl_ffn_weights (uint8 codes
   * [rows, d_model / 2], fp32 scales [rows, d_model / 64]).  Wq_q set: q, k and
   * v read Wq_q/Wk_q/Wv_q with Wq_s/Wk_s/Wv_s, and Wq, Wk, Wv are ignored.
   * WoT_q set: o reads WoT_q with WoT_s, and WoT is ignored.  bf16 calls
   * only; d_model a multiple of 64; 16-byte aligned.  NULL: plain weights. */
  const void *Wq_q, *Wk_q, *Wv_q, *WoT_q;
  const float *Wq_s, *Wk_s, *Wv_s, *WoT_s;
} sl_qkvo_weights;

typedef struct sl_qkvo_grads {   /* fp32, shapes of the factors; OVERWRITTEN */
  float *dAq, *dBq, *dAk, *dBk, *dAv, *dBv, *dAo, *dBo;
} sl_qkvo_grads;

int sl_abi_version(void);
const char* sl_status_string(sl_status s);
const char* sl_last_error(void);          /* thread-local message of the last error */

/* ---------------------------------------------------------------------------
 * a0 — offline estimator build (SparseLoRA article §二 and §七: truncated SVD of
 * each frozen projection weight, done once before training).
 *   W     [out_f, in_f]  frozen weight (call dtype)
 *   Pt    [rank, in_f]   (V_r diag(sigma_r))^T, call dtype      (output)
 *   Q     [rank, out_f]  U_r^T, call dtype                       (output)
 *   sigma [rank] fp32, optional (NULL = not written)            (output)
 * so that x Pt^T Q approximates x W^T.  Computed by block subspace iteration
 * on the GPU in fp32 with a host fp64 Rayleigh-Ritz step; 1 <= rank <= 64 and
 * rank <= min(out_f, in_f).  SYNCHRONISES `stream` (offline, untimed).
 * ------------------------------------------------------------------------- */
size_t sl_estimator_workspace_bytes(int64_t out_f, int64_t in_f, int32_t rank);
sl_status sl_build_estimator(sl_dtype dt, const void* W, int64_t out_f, int64_t in_f,
                             int32_t rank, int32_t iters, void* Pt, void* Q, float* sigma,
                             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * a1-a3 — estimate, score, select (SparseLoRA article §一, §二, §三).
 *   X   [T, d_in]  layer input (call dtype); only context rows are read.
 *   SWIGLU_L2: (Pt0,Q0) = gate factors, (Pt1,Q1) = up factors, N = d_ff.
 *   L2:        (Pt0,Q0) = the projection's factors, N = its out features.
 *   QK_NORM:   (Pt0,Q0) = q factors (Q0 [rank, Hq*hd]), (Pt1,Q1) = k factors
 *              (Q1 [rank, Hkv*hd]); N = Hkv*hd (selection in kv-channel space).
 *   Pt* [rank, d_in], Q* [rank, N_proj] (call dtype), 1 <= rank <= 32.
 *   idx    [batch, k] int32 out: per sequence the k best channels, ascending;
 *          ties in score go to the lower channel index.
 *   scores [batch, N] fp32 out, optional (NULL = not written): the criterion
 *          (a sum of squares over the sequence's context tokens).
 * 1 <= k <= N <= 65536.  The workspace holds the context tokens' projections,
 * the criterion's partial sums and every sequence's N selection keys.  heads
 * is read for QK_NORM only.  The workspace size query takes the same
 * criterion, layout, heads, d_in, rank and N as the call.
 * ------------------------------------------------------------------------- */
size_t sl_estimate_select_workspace_bytes(sl_criterion crit, const sl_layout* lay,
                                          const sl_heads* heads, int64_t d_in, int32_t rank,
                                          int64_t N);
sl_status sl_estimate_select(sl_criterion crit, sl_dtype dt, const sl_layout* lay,
                             const sl_heads* heads, const void* X, int64_t d_in, int32_t rank,
                             const void* Pt0, const void* Q0, const void* Pt1, const void* Q1,
                             int64_t N, int32_t k, int32_t* idx, float* scores,
                             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sl_estimate_select without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as sl_estimate_select,
 * minus ws / ws_bytes: the scratch is a fixed array of SL_NOALLOC_SCRATCH_BYTES
 * in the library's device memory, one per device, held from the library's
 * load until the process ends.  A call whose sl_estimate_select_workspace_bytes
 * exceeds that size returns SL_ERR_WORKSPACE (nothing launched).  The call
 * allocates nothing.  Every call on one device shares that device's array, so
 * calls that overlap on one device (different streams, or different threads
 * without stream order) race; calls in one stream's order do not.  Nothing in
 * the array needs to start at zero: every call writes what it reads.
 * ------------------------------------------------------------------------- */
#define SL_NOALLOC_SCRATCH_BYTES (32u << 20)
sl_status sl_estimate_select_noalloc(sl_criterion crit, sl_dtype dt, const sl_layout* lay,
                                     const sl_heads* heads, const void* X, int64_t d_in, int32_t rank,
                                     const void* Pt0, const void* Q0, const void* Pt1, const void* Q1,
                                     int64_t N, int32_t k, int32_t* idx, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * a1-a3 for several criteria over one input (SparseLoRA article §一, §二, §三:
 * an attention layer scores q/k by the QK-norm and v/o by the L2 norm of the
 * same layer input).  Same results as one sl_estimate_select call per job, but
 * X is projected once onto every job's leading directions, all L2-type
 * criteria share one launch and all selections share one launch.
 *   jobs[j]: crit, heads (QK_NORM only), Pt0/Q0/Pt1/Q1, N, k, idx, scores as in
 *            sl_estimate_select; every job shares X, the layout, d_in and rank.
 * 1 <= njobs <= SL_EST_MAXJOBS, and the jobs' projections (2 for SWIGLU_L2 and
 * QK_NORM, 1 for L2) number at most 4.  Jobs must write distinct idx / scores
 * buffers.  The workspace query takes the same layout, d_in, rank and jobs
 * (only crit, heads and N are read).
 * ------------------------------------------------------------------------- */
#define SL_EST_MAXJOBS 3
typedef struct sl_est_job {
  sl_criterion crit;
  sl_heads heads;                  /* QK_NORM only */
  const void *Pt0, *Q0, *Pt1, *Q1;  /* Pt1 / Q1 unused for L2 */
  int64_t N;
  int32_t k;
  int32_t* idx;                    /* [batch, k] out */
  float* scores;                   /* [batch, N] out, optional */
} sl_est_job;
size_t sl_estimate_select_multi_workspace_bytes(const sl_layout* lay, int64_t d_in, int32_t rank,
                                                int32_t njobs, const sl_est_job* jobs);
sl_status sl_estimate_select_multi(sl_dtype dt, const sl_layout* lay, const void* X, int64_t d_in,
                                   int32_t rank, int32_t njobs, const sl_est_job* jobs, void* ws,
                                   size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * a4/a5 — sparse SwiGLU FFN forward and backward (SparseLoRA article §一, §三,
 * §六, §七; SparseLoRA abstract).  Context rows of sequence b use channels
 * idx[b, :k]; output rows use all d_ff channels.
 *   fwd:  X [T, d_model] -> Y [T, d_model]; writes `saved` for the backward.
 *   bwd:  dY [T, d_model] + saved -> dX [T, d_model] and the six LoRA gradients.
 *         X, w, k, idx and the layout must be those of the forward call.
 * d_model % 8 == 0, d_ff % 8 == 0, 1 <= lora_rank <= 32, 1 <= k <= d_ff.
 * Every matrix a call reads or writes holds fewer than 2^31 elements:
 * batch*seq_len*d_model, d_ff*d_model and the compact activation buffers
 * (sum of ctx_len * round_up(k, 8) + output rows * d_ff); SL_ERR_RANGE
 * otherwise, before anything is launched.
 * ------------------------------------------------------------------------- */
size_t sl_ffn_saved_bytes(sl_dtype dt, const sl_layout* lay, int64_t d_model, int64_t d_ff,
                          int32_t lora_rank, int32_t k);
size_t sl_ffn_workspace_bytes(sl_dtype dt, const sl_layout* lay, int64_t d_model, int64_t d_ff,
                              int32_t lora_rank, int32_t k);
sl_status sl_ffn_fwd(sl_dtype dt, const sl_layout* lay, const sl_ffn_weights* w, const void* X,
                     int32_t k, const int32_t* idx, void* Y, void* saved, size_t saved_bytes,
                     void* ws, size_t ws_bytes, void* stream);
sl_status sl_ffn_bwd(sl_dtype dt, const sl_layout* lay, const sl_ffn_weights* w, const void* X,
                     int32_t k, const int32_t* idx, const void* saved, size_t saved_bytes,
                     const void* dY, void* dX, const sl_ffn_grads* g,
                     void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * a6/a7 — sparse q/k/v/o projections (SparseLoRA article §一, §三, §六).
 * idx_qk [batch, k_qk] and idx_vo [batch, k_vo] are kv-channel sets (as written
 * by sl_estimate_select with QK_NORM and L2); q and o use them expanded to every
 * query head of the group.  At context rows, unselected channels of q, k, v are
 * written as 0 and unselected columns of the attention output a are ignored.
 *   fwd:  X [T, d_model] -> q [T, Hq*hd], k, v [T, Hkv*hd]   (if X != NULL)
 *         a [T, Hq*hd]   -> o [T, d_model]                  (if a != NULL)
 *         so a caller may run q/k/v, its attention, then o, as two calls
 *         sharing one `saved` buffer.
 *   bwd:  d_out -> da [T, Hq*hd] and dAo, dBo                (if d_out != NULL)
 *         dq, dk, dv -> dX and dAq..dBv                      (if dq != NULL)
 *         X and a (the forward's inputs) are read for the factor gradients.
 *         The d_out part reads what the forward's a part left in `saved`
 *         (z_o and the packed Bo^T, Ao^T); the dq part what its X part left
 *         (z_q, z_k, z_v).
 * d_model, Hq*hd and Hkv*hd multiples of 8; 1 <= lora_rank <= 32;
 * 1 <= k_qk, k_vo <= Hkv*hd.  Every matrix a call reads or writes holds
 * fewer than 2^31 elements (T*d_model, T*Hq*hd, Hq*hd*d_model and the compact
 * projection buffers); SL_ERR_RANGE otherwise, before anything is launched.
 * ------------------------------------------------------------------------- */
size_t sl_qkvo_saved_bytes(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w);
size_t sl_qkvo_workspace_bytes(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w,
                               int32_t k_qk, int32_t k_vo);
sl_status sl_qkvo_fwd(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w,
                      const void* X, const void* a,
                      int32_t k_qk, const int32_t* idx_qk, int32_t k_vo, const int32_t* idx_vo,
                      void* q, void* k, void* v, void* o, void* saved, size_t saved_bytes,
                      void* ws, size_t ws_bytes, void* stream);
sl_status sl_qkvo_bwd(sl_dtype dt, const sl_layout* lay, const sl_qkvo_weights* w,
                      const void* X, const void* a,
                      int32_t k_qk, const int32_t* idx_qk, int32_t k_vo, const int32_t* idx_vo,
                      const void* saved, size_t saved_bytes,
                      const void* dq, const void* dk, const void* dv, const void* d_out,
                      void* dX, void* da, const sl_qkvo_grads* g,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Offline quantization of a frozen weight to the 4-bit base of sl_ffn_weights
 * (SparseLoRA article §六: SparseLoRA over a QLoRA-style quantized base; the
 * pages name no format, this is the plainest 4-bit one).  W [rows, cols] in dt
 * -> codes uint8 [rows, cols/2] and scales fp32 [rows, cols/64]: each block of
 * 64 consecutive row elements gets s = max|w| / 7 (0 for an all-zero block)
 * and codes q = rint(w / s) in [-7, 7] (IEEE fp32 division, ties to even);
 * element 2j of a row sits in the low nibble of byte j, element 2j+1 in the
 * high nibble (two's complement).  cols a positive multiple of 64; all
 * pointers device, 16-byte aligned; the caller owns every buffer.  Stream-
 * ordered, never synchronises.  Errors: SL_ERR_NULL, SL_ERR_DTYPE,
 * SL_ERR_SHAPE, SL_ERR_RANGE, SL_ERR_ALIGN, SL_ERR_UNSUPPORTED_ARCH,
 * SL_ERR_HIP; nothing is launched on error.
 * ------------------------------------------------------------------------- */
sl_status sl_quantize_q4(sl_dtype dt, const void* W, int64_t rows, int64_t cols, void* codes, float* scales,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics (not part of the computation).  When enabled, the library's main
 * launches are bracketed by HIP events on the caller's stream and attributed
 * to the slots below, so a caller can time individual kernels inside a timed
 * region.  The timer state is per calling thread: it covers the calls that
 * thread makes.  sl_timer_enable(n) keeps room for n
 * launches (0 disables and frees the events); sl_timer_read waits for the
 * recorded events and returns the slot's total milliseconds and launch count
 * since the last sl_timer_reset.  sl_timer_select(mask) records only the slots
 * whose bit (1 << slot) is set (all after sl_timer_enable), so that a timed
 * region carries events around the kernels of interest only.
 * ------------------------------------------------------------------------- */
typedef enum sl_timer_slot {
  SL_TS_ESTIMATE = 0,   /* estimator stage 1 + criterion (a1, a2) */
  SL_TS_SELECT = 1,     /* top-k (a3) */
  SL_TS_GU_FWD = 2,     /* gate/up gather-GEMM + SwiGLU (a4) */
  SL_TS_DOWN_FWD = 3,   /* down K-gather GEMM (a4) */
  SL_TS_DH_BWD = 4,     /* dH gather-GEMM + SwiGLU backward (a5) */
  SL_TS_DX_BWD = 5,     /* dX K-gather GEMM (a5) */
  SL_TS_QKV_FWD = 6, SL_TS_O_FWD = 7, SL_TS_DA_BWD = 8, SL_TS_DXQKV_BWD = 9
} sl_timer_slot;
int sl_timer_enable(int max_launches);
void sl_timer_select(uint32_t slot_mask);
void sl_timer_reset(void);
int sl_timer_read(int slot, double* total_ms, int* count);

/* ---------------------------------------------------------------------------
 * GEMM variants (tuning and testing; results agree to the same tolerance).
 * The gather-GEMMs run as 128 x 256 tiles staged through registers, as wide
 * 128 x 512 N-gather tiles fed by LDS-DMA, or as tall 256 x 256 tiles (N- or
 * K-gather) fed by LDS-DMA.  The LDS-DMA tiles need bf16 calls with every
 * operand 16-byte aligned (N-gather: K a multiple of 8); the tall tiles are
 * taken when their grid moves fewer operand bytes per CU than the other
 * variant's.  `variants` is a bit mask of what the calling thread allows: 1 =
 * wide tiles, 2 = tall tiles, 4 = tall tiles whatever their grid (with 2); 0 =
 * 128 x 256 tiles only; a negative value leaves the setting.  Default 3.
 * Returns the previous setting.  The setting is per calling thread and
 * applies to the calls that thread makes.
 * ------------------------------------------------------------------------- */
int sl_gemm_config(int variants);

#ifdef __cplusplus
}
#endif
#endif /* SPARSELORA_H */
