// a0: offline estimator build — leading singular triplets of a frozen weight.
//   SparseLoRA article §二: the pretrained weight is decomposed once, before
//   training, and only the leading singular values and vectors are kept;
//   §七: rank 8 is the chosen trade-off.
//
// Block subspace iteration (a randomized range finder followed by power
// iterations), with the large products on the GPU in fp32 and the small
// l x l eigenproblems on the host in fp64 (cyclic Jacobi):
//   Y = W Omega;  repeat: Z = orth(W^T Y), Y = orth(W Z)
//   Z = W^T Y  (so B = Y^T W = Z^T);  B B^T = Z^T Z = U~ S^2 U~^T
//   Pt = U~_r^T Z^T  (= Sigma_r V_r^T),  Q = U~_r^T Y^T  (= U_r^T)
// Orthonormalisation uses the Gram matrix: G = Y^T Y = V L V^T and
// Y <- Y V L^-1/2 (columns with a negligible eigenvalue are dropped).
#include <cmath>
#include <vector>

#include "sl_host.hpp"

using namespace sl;

namespace {

__device__ inline float ldw(const float* p, long long i) { return p[i]; }
__device__ inline float ldw(const bf16* p, long long i) { return bf2f(p[i].v); }

__global__ void omega_kernel(float* Z, long long n, unsigned long long seed) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  // splitmix64 of the element counter -> uniform in [-1, 1)
  unsigned long long x = seed + 0x9E3779B97F4A7C15ull * (unsigned long long)(i + 1);
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  x ^= x >> 31;
  Z[i] = (float)((double)(x >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0);
}

// Y[i][j] = sum_d W[i][d] X[d][j]    (W [n_out, n_in], X [n_in, l], Y [n_out, l])
template <typename T>
__global__ void wx_kernel(const T* W, const float* X, float* Y, int n_out, int n_in, int l) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)n_out * l) return;
  const int i = (int)(t / l), j = (int)(t % l);
  const T* w = W + (long long)i * n_in;
  float acc = 0.f;
  for (int d = 0; d < n_in; ++d) acc = fmaf(ldw(w, d), X[(long long)d * l + j], acc);
  Y[t] = acc;
}

// Z[d][j] = sum_i W[i][d] Y[i][j]
template <typename T>
__global__ void wtx_kernel(const T* W, const float* Y, float* Z, int n_out, int n_in, int l) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)n_in * l) return;
  const int d = (int)(t / l), j = (int)(t % l);
  float acc = 0.f;
  for (int i = 0; i < n_out; ++i) acc = fmaf(ldw(W, (long long)i * n_in + d), Y[(long long)i * l + j], acc);
  Z[t] = acc;
}

// G[a][b] = sum_i Y[i][a] Y[i][b] in fp64
__global__ void gram_kernel(const float* Y, double* G, int n, int l) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= l * l) return;
  const int a = t / l, b = t % l;
  double acc = 0.0;
  for (int i = 0; i < n; ++i) acc += (double)Y[(long long)i * l + a] * (double)Y[(long long)i * l + b];
  G[t] = acc;
}

// Yo[i][j] = sum_a Y[i][a] M[a][j]
__global__ void apply_kernel(const float* Y, const double* M, float* Yo, int n, int l) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)n * l) return;
  const int i = (int)(t / l), j = (int)(t % l);
  double acc = 0.0;
  for (int a = 0; a < l; ++a) acc += (double)Y[(long long)i * l + a] * M[a * l + j];
  Yo[t] = (float)acc;
}

// out[q][c] = sum_j M[j][q] S[c][j]   (q < rank, c < n), written in the call dtype
template <typename T>
__global__ void project_kernel(const float* S, const double* M, T* out, int n, int l, int rank) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)rank * n) return;
  const int q = (int)(t / n), c = (int)(t % n);
  double acc = 0.0;
  for (int j = 0; j < l; ++j) acc += M[j * l + q] * (double)S[(long long)c * l + j];
  stv<T>(out, t, (float)acc);
}

// cyclic Jacobi: A (symmetric l x l, destroyed) = V diag(w) V^T, sorted descending
void jacobi_eig(std::vector<double>& A, int l, std::vector<double>& w, std::vector<double>& V) {
  V.assign((size_t)l * l, 0.0);
  for (int i = 0; i < l; ++i) V[(size_t)i * l + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int i = 0; i < l; ++i)
      for (int j = 0; j < l; ++j) (i == j ? diag : off) += A[(size_t)i * l + j] * A[(size_t)i * l + j];
    if (off <= 1e-30 * (diag + 1e-300)) break;
    for (int p = 0; p < l - 1; ++p)
      for (int q = p + 1; q < l; ++q) {
        const double apq = A[(size_t)p * l + q];
        if (std::fabs(apq) < 1e-300) continue;
        const double app = A[(size_t)p * l + p], aqq = A[(size_t)q * l + q];
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < l; ++k) {
          const double akp = A[(size_t)k * l + p], akq = A[(size_t)k * l + q];
          A[(size_t)k * l + p] = c * akp - s * akq;
          A[(size_t)k * l + q] = s * akp + c * akq;
        }
        for (int k = 0; k < l; ++k) {
          const double apk = A[(size_t)p * l + k], aqk = A[(size_t)q * l + k];
          A[(size_t)p * l + k] = c * apk - s * aqk;
          A[(size_t)q * l + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < l; ++k) {
          const double vkp = V[(size_t)k * l + p], vkq = V[(size_t)k * l + q];
          V[(size_t)k * l + p] = c * vkp - s * vkq;
          V[(size_t)k * l + q] = s * vkp + c * vkq;
        }
      }
  }
  std::vector<int> ord(l);
  for (int i = 0; i < l; ++i) ord[i] = i;
  for (int i = 0; i < l; ++i)
    for (int j = i + 1; j < l; ++j)
      if (A[(size_t)ord[j] * l + ord[j]] > A[(size_t)ord[i] * l + ord[i]]) std::swap(ord[i], ord[j]);
  std::vector<double> Vs((size_t)l * l);
  w.resize(l);
  for (int j = 0; j < l; ++j) {
    w[j] = A[(size_t)ord[j] * l + ord[j]];
    for (int k = 0; k < l; ++k) Vs[(size_t)k * l + j] = V[(size_t)k * l + ord[j]];
  }
  V.swap(Vs);
}

struct SvdGeom {
  int l;
  size_t w_y, w_y2, w_z, w_z2, w_g, w_m, total;
};

SvdGeom svd_geom(long long out_f, long long in_f, int rank) {
  SvdGeom g;
  const long long mn = std::min(out_f, in_f);
  g.l = (int)std::min<long long>(2LL * rank + 8, mn);
  Bump b;
  g.w_y = b.take((size_t)out_f * g.l * 4);
  g.w_y2 = b.take((size_t)out_f * g.l * 4);
  g.w_z = b.take((size_t)in_f * g.l * 4);
  g.w_z2 = b.take((size_t)in_f * g.l * 4);
  g.w_g = b.take((size_t)g.l * g.l * 8);
  g.w_m = b.take((size_t)g.l * g.l * 8);
  g.total = b.off;
  return g;
}

// S <- S V L^-1/2 using the Gram matrix of S (S [n, l] fp32; tmp same size)
sl_status orthonormalize(float* S, float* tmp, int n, int l, double* dG, double* dM, hipStream_t s) {
  hipLaunchKernelGGL(gram_kernel, grid1d((long long)l * l), dim3(256), 0, s, S, dG, n, l);
  SL_HIP(hipGetLastError());
  std::vector<double> G((size_t)l * l), w, V;
  SL_HIP(hipMemcpyAsync(G.data(), dG, G.size() * 8, hipMemcpyDeviceToHost, s));
  SL_HIP(hipStreamSynchronize(s));
  jacobi_eig(G, l, w, V);
  const double wmax = w.empty() ? 0.0 : std::max(w[0], 0.0);
  std::vector<double> M((size_t)l * l, 0.0);
  for (int j = 0; j < l; ++j) {
    const double sc = (w[j] > 1e-12 * wmax && w[j] > 0) ? 1.0 / std::sqrt(w[j]) : 0.0;
    for (int a = 0; a < l; ++a) M[(size_t)a * l + j] = V[(size_t)a * l + j] * sc;
  }
  SL_HIP(hipMemcpyAsync(dM, M.data(), M.size() * 8, hipMemcpyHostToDevice, s));
  hipLaunchKernelGGL(apply_kernel, grid1d((long long)n * l), dim3(256), 0, s, S, dM, tmp, n, l);
  SL_HIP(hipGetLastError());
  SL_HIP(hipMemcpyAsync(S, tmp, (size_t)n * l * 4, hipMemcpyDeviceToDevice, s));
  SL_HIP(hipStreamSynchronize(s));
  return SL_OK;
}

template <typename T>
sl_status build_impl(const T* W, int out_f, int in_f, int rank, int iters, T* Pt, T* Q, float* sigma,
                     char* ws, const SvdGeom& g, hipStream_t s) {
  const int l = g.l;
  float* Y = reinterpret_cast<float*>(ws + g.w_y);
  float* Y2 = reinterpret_cast<float*>(ws + g.w_y2);
  float* Z = reinterpret_cast<float*>(ws + g.w_z);
  float* Z2 = reinterpret_cast<float*>(ws + g.w_z2);
  double* dG = reinterpret_cast<double*>(ws + g.w_g);
  double* dM = reinterpret_cast<double*>(ws + g.w_m);
  sl_status rc;
  hipLaunchKernelGGL(omega_kernel, grid1d((long long)in_f * l), dim3(256), 0, s, Z,
                     (long long)in_f * l, 0x5EEDull);
  SL_HIP(hipGetLastError());
  hipLaunchKernelGGL((wx_kernel<T>), grid1d((long long)out_f * l), dim3(256), 0, s, W, Z, Y, out_f,
                     in_f, l);
  SL_HIP(hipGetLastError());
  if ((rc = orthonormalize(Y, Y2, out_f, l, dG, dM, s))) return rc;
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL((wtx_kernel<T>), grid1d((long long)in_f * l), dim3(256), 0, s, W, Y, Z, out_f,
                       in_f, l);
    SL_HIP(hipGetLastError());
    if ((rc = orthonormalize(Z, Z2, in_f, l, dG, dM, s))) return rc;
    hipLaunchKernelGGL((wx_kernel<T>), grid1d((long long)out_f * l), dim3(256), 0, s, W, Z, Y, out_f,
                       in_f, l);
    SL_HIP(hipGetLastError());
    if ((rc = orthonormalize(Y, Y2, out_f, l, dG, dM, s))) return rc;
  }
  // Rayleigh-Ritz: Z = W^T Y, B B^T = Z^T Z
  hipLaunchKernelGGL((wtx_kernel<T>), grid1d((long long)in_f * l), dim3(256), 0, s, W, Y, Z, out_f,
                     in_f, l);
  SL_HIP(hipGetLastError());
  hipLaunchKernelGGL(gram_kernel, grid1d((long long)l * l), dim3(256), 0, s, Z, dG, in_f, l);
  SL_HIP(hipGetLastError());
  std::vector<double> G((size_t)l * l), w, V;
  SL_HIP(hipMemcpyAsync(G.data(), dG, G.size() * 8, hipMemcpyDeviceToHost, s));
  SL_HIP(hipStreamSynchronize(s));
  jacobi_eig(G, l, w, V);
  SL_HIP(hipMemcpyAsync(dM, V.data(), V.size() * 8, hipMemcpyHostToDevice, s));
  hipLaunchKernelGGL((project_kernel<T>), grid1d((long long)rank * in_f), dim3(256), 0, s, Z, dM, Pt,
                     in_f, l, rank);
  SL_HIP(hipGetLastError());
  hipLaunchKernelGGL((project_kernel<T>), grid1d((long long)rank * out_f), dim3(256), 0, s, Y, dM, Q,
                     out_f, l, rank);
  SL_HIP(hipGetLastError());
  if (sigma) {
    std::vector<float> sg(rank);
    for (int i = 0; i < rank; ++i) sg[i] = (float)std::sqrt(std::max(w[i], 0.0));
    SL_HIP(hipMemcpyAsync(sigma, sg.data(), rank * 4, hipMemcpyHostToDevice, s));
  }
  SL_HIP(hipStreamSynchronize(s));
  return SL_OK;
}

}  // namespace

extern "C" {

size_t sl_estimator_workspace_bytes(int64_t out_f, int64_t in_f, int32_t rank) {
  if (out_f < 1 || in_f < 1 || rank < 1 || rank > 64 || rank > std::min(out_f, in_f)) return 0;
  return svd_geom(out_f, in_f, rank).total;
}

sl_status sl_build_estimator(sl_dtype dt, const void* W, int64_t out_f, int64_t in_f, int32_t rank,
                             int32_t iters, void* Pt, void* Q, float* sigma, void* ws,
                             size_t ws_bytes, void* stream) {
  if (dt != SL_F32 && dt != SL_BF16) SL_FAIL(SL_ERR_DTYPE, "unknown dtype %d", (int)dt);
  if (out_f < 1 || in_f < 1 || out_f > (1 << 24) || in_f > (1 << 24))
    SL_FAIL(SL_ERR_SHAPE, "bad weight shape %lld x %lld", (long long)out_f, (long long)in_f);
  if (rank < 1 || rank > 64 || rank > std::min(out_f, in_f))
    SL_FAIL(SL_ERR_RANGE, "rank %d outside [1, min(64, out_f, in_f)]", rank);
  if (iters < 0 || iters > 100) SL_FAIL(SL_ERR_RANGE, "iters %d outside [0, 100]", iters);
  if (!W || !Pt || !Q || !ws) SL_FAIL(SL_ERR_NULL, "W, Pt, Q and ws must be non-NULL");
  if (!aligned16(ws)) SL_FAIL(SL_ERR_ALIGN, "ws must be 16-byte aligned");
  const SvdGeom g = svd_geom(out_f, in_f, rank);
  if (ws_bytes < g.total) SL_FAIL(SL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, g.total);
  sl_status s = check_arch();
  if (s != SL_OK) return s;
  const int it = iters == 0 ? 6 : iters;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  if (dt == SL_BF16)
    return build_impl<bf16>(reinterpret_cast<const bf16*>(W), (int)out_f, (int)in_f, rank, it,
                            reinterpret_cast<bf16*>(Pt), reinterpret_cast<bf16*>(Q), sigma,
                            reinterpret_cast<char*>(ws), g, strm);
  return build_impl<float>(reinterpret_cast<const float*>(W), (int)out_f, (int)in_f, rank, it,
                           reinterpret_cast<float*>(Pt), reinterpret_cast<float*>(Q), sigma,
                           reinterpret_cast<char*>(ws), g, strm);
}

}  // extern "C"
