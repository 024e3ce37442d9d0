// Teacher hidden-state recovery from k cached log-probabilities for gfx950
// ("The Gradient That Top-k Distillation Never Computes", abstract and
// Table 1: the retained set determines the teacher's distribution once
// k >= d + 1).  Cached log q_v = U_v g + b_v - c on S (c the teacher's
// logsumexp) is linear in (g, c), so per position the least-squares
// solution of [U_S, -1] (g; c) = log q_S - b_S recovers them; from it the
// full distribution softmax(U g + b) follows.
//
// One workgroup per position, fp64 throughout: the k x (d+1) system sits in
// LDS (column-major, odd column pitch against bank conflicts) and is solved
// by Householder QR and back substitution.  Sized for the identifiability
// study: (d + 2) * k <= 19968.
#include <hip/hip_runtime.h>
#include <math.h>

#include "../../include/kdtopk.h"
#include "kd_common.h"
#include "kd_internal.h"

namespace {

constexpr int RN = 256;          // threads per position
constexpr int RCAP = 19968;      // doubles of the system in LDS (156 KB)

__global__ void k_fill_flags(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__device__ __forceinline__ double block_sum_rn(double v, double* red) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(RN) void k_recover(const int32_t* __restrict__ idx, const float* __restrict__ tlp,
                                                const bf16_t* __restrict__ U, const float* __restrict__ b,
                                                int64_t V, int d, int k, int kp, float* __restrict__ g_hat,
                                                float* __restrict__ c_hat) {
  extern __shared__ double sh[];
  __shared__ int any_bad;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = d + 1;
  double* a = sh;              // column c, row r at a[c * kp + r]; y is column n
  double* rdiag = a + (n + 1) * kp;
  double* x = rdiag + n;
  double* red = x + n;
  if (tid == 0) any_bad = 0;
  __syncthreads();
  bool bad = false;
  for (int i = tid; i < (n + 1) * k; i += RN) {
    const int c = i / k, r = i % k;
    const int v = idx[t * k + r];
    if (v < 0 || v >= V) {
      bad = true;
      a[c * kp + r] = 0.0;
      continue;
    }
    double e;
    if (c < d) e = (double)bf16_to_f32(U[(int64_t)v * d + c]);
    else if (c == d) e = -1.0;
    else e = (double)tlp[t * k + r] - (b != nullptr ? (double)b[v] : 0.0);
    a[c * kp + r] = e;
  }
  if (bad) atomicOr(&any_bad, 1);
  __syncthreads();
  // Householder QR; column j's reflector v overwrites rows j.. of column j
  for (int j = 0; j < n; ++j) {
    double ss = 0.0;
    for (int r = j + tid; r < k; r += RN) ss += a[j * kp + r] * a[j * kp + r];
    ss = block_sum_rn(ss, red);
    const double x0 = a[j * kp + j];
    const double nrm = sqrt(ss);
    const double alpha = x0 >= 0.0 ? -nrm : nrm;
    const double vv = ss - x0 * x0 + (x0 - alpha) * (x0 - alpha);
    __syncthreads();
    if (tid == 0) {
      a[j * kp + j] = x0 - alpha;
      rdiag[j] = alpha;
    }
    __syncthreads();
    if (vv > 0.0) {
      for (int c = j + 1 + tid; c <= n; c += RN) {  // the remaining columns and y
        double s = 0.0;
        for (int r = j; r < k; ++r) s += a[j * kp + r] * a[c * kp + r];
        const double f = 2.0 * s / vv;
        for (int r = j; r < k; ++r) a[c * kp + r] -= f * a[j * kp + r];
      }
    }
    __syncthreads();
  }
  // back substitution: R x = (Q^T y)[0..n)
  for (int i = n - 1; i >= 0; --i) {
    double s = 0.0;
    for (int c = i + 1 + tid; c < n; c += RN) s += a[c * kp + i] * x[c];
    s = block_sum_rn(s, red);
    if (tid == 0) x[i] = (a[n * kp + i] - s) / rdiag[i];
    __syncthreads();
  }
  const float nan = __builtin_nanf("");
  for (int c = tid; c < d; c += RN) g_hat[t * d + c] = any_bad ? nan : (float)x[c];
  if (tid == 0) c_hat[t] = any_bad ? nan : (float)x[d];
}

// ---------------------------------------------------------------------------
// Multi-workgroup solver for wide heads (d in the thousands), fp64, batched
// over positions.  Per position t a column-major matrix M (ld rows) in the
// workspace:
//   k >= d + 1 (least squares): M = [U_S, -1 | y], P = k rows, n = d + 1
//     unknown columns plus the right-hand side y = log q_S - b_S as column n;
//     Householder QR column by column, the reflectors applied to y as well,
//     then R x = (Q^T y)[0..n) by back substitution;
//   k <= d (minimum-norm solution, below the identifiability threshold):
//     M = [U_S, -1]^T, P = d + 1 rows, k columns; its QR gives A = R^T Q^T,
//     so R^T w = y by forward substitution and x = Q [w; 0].
// Reflector j overwrites rows j.. of column j (v, with v_j = x_0 - alpha),
// rdiag[j] = alpha = R_jj and vvs[j] = v^T v.  One launch per column: each
// wavefront updates one trailing column with reflector j; the wavefront that
// updated column j + 1 then forms reflector j + 1 from its registers.
// ---------------------------------------------------------------------------
constexpr int QW = 4;                 // wavefronts (columns) per workgroup
constexpr int QMAXP = 1 << 16;        // rows (max(k, d + 1)) of the stored system

struct QrDims {
  int P, ncols, ld, n;                // rows, stored columns, pitch, unknowns (d + 1)
  int64_t per;                        // doubles per position
  bool lsq;                           // k >= d + 1
};

__device__ __forceinline__ double* qr_mat(double* ws, const QrDims& q, int64_t t) { return ws + t * q.per; }
__device__ __forceinline__ double* qr_vec(double* ws, const QrDims& q, int64_t t, int which) {
  return ws + t * q.per + (int64_t)q.ncols * q.ld + (int64_t)which * (q.ld > q.ncols ? q.ld : q.ncols);
}

// Fill M (and y for the minimum-norm case); a position with an index out of
// range gets flag 1 (its outputs become NaN).
__global__ __launch_bounds__(256) void k_qr_fill(const int32_t* __restrict__ idx, const float* __restrict__ tlp,
                                                 const bf16_t* __restrict__ U, const float* __restrict__ b, int64_t V,
                                                 int d, int k, QrDims q, double* __restrict__ ws,
                                                 int32_t* __restrict__ flag) {
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x;  // stored column
  double* M = qr_mat(ws, q, t) + (int64_t)c * q.ld;
  if (q.lsq) {
    // column c < d: U_S[:, c]; c == d: -1; c == d + 1: y
    for (int r = threadIdx.x; r < q.P; r += 256) {
      const int v = idx[t * k + r];
      double e = 0.0;
      if (v < 0 || v >= V) {
        flag[t] = 1;
      } else if (c < d) {
        e = (double)bf16_to_f32(U[(int64_t)v * d + c]);
      } else if (c == d) {
        e = -1.0;
      } else {
        e = (double)tlp[t * k + r] - (b != nullptr ? (double)b[v] : 0.0);
      }
      M[r] = e;
    }
  } else {
    // column c = entry c: row r < d: U[S_c][r]; row d: -1; y[c] beside
    const int v = idx[t * k + c];
    const bool ok = v >= 0 && v < V;
    if (!ok && threadIdx.x == 0) flag[t] = 1;
    for (int r = threadIdx.x; r < q.P; r += 256)
      M[r] = !ok ? 0.0 : (r < d ? (double)bf16_to_f32(U[(int64_t)v * d + r]) : -1.0);
    if (threadIdx.x == 0)
      qr_vec(ws, q, t, 2)[c] = ok ? (double)tlp[t * k + c] - (b != nullptr ? (double)b[v] : 0.0) : 0.0;
  }
}

// Reflector from the sum of squares ss of a column's rows j.. and its first
// value x0: v = x - alpha e_j overwrites rows j.. (only row j changes),
// R_jj = alpha, v^T v recorded (0: the column is already zero below j).
__device__ __forceinline__ void qr_reflector(double ss, double x0, double* col, int j, double* rdiag, double* vvs) {
  const double nrm = sqrt(ss);
  const double alpha = x0 >= 0.0 ? -nrm : nrm;
  const double vv = ss - x0 * x0 + (x0 - alpha) * (x0 - alpha);
  col[j] = x0 - alpha;
  rdiag[j] = alpha;
  vvs[j] = vv;
}

// Reflector 0 of each position (one wavefront).
__global__ __launch_bounds__(64) void k_qr_first(QrDims q, double* __restrict__ ws) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  double* col = qr_mat(ws, q, t);
  double ss = 0.0;
  for (int r = lane; r < q.P; r += 64) ss += col[r] * col[r];
  ss = wave_sum_f64(ss);
  const double x0 = col[0];
  if (lane == 0) qr_reflector(ss, x0, col, 0, qr_vec(ws, q, t, 0), qr_vec(ws, q, t, 1));
}

// Apply reflector j to columns j+1 .. ncols-1, one wavefront per column
// (dot product, then the update, rows j..P-1); the wavefront on column j+1
// (when it is one of the nfact factored columns) sums the squares of its
// updated rows j+1.. on the way and forms reflector j+1.
__global__ __launch_bounds__(256) void k_qr_step(QrDims q, int j, int nfact, double* __restrict__ ws) {
  const int64_t t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int c = j + 1 + (int)blockIdx.x * QW + (int)(threadIdx.x >> 6);
  if (c >= q.ncols) return;
  double* M = qr_mat(ws, q, t);
  const double* vj = M + (int64_t)j * q.ld;
  double* col = M + (int64_t)c * q.ld;
  double* vvs = qr_vec(ws, q, t, 1);
  const double vv = vvs[j];
  const int nr = q.P - j;  // rows j .. P-1
  double s = 0.0;
  for (int r = lane; r < nr; r += 64) s += vj[j + r] * col[j + r];
  s = wave_sum_f64(s);
  const double f = vv > 0.0 ? 2.0 * s / vv : 0.0;
  const bool next = c == j + 1 && c < nfact;
  double ss = 0.0, x0 = 0.0;
  for (int r = lane; r < nr; r += 64) {
    const double x = col[j + r] - f * vj[j + r];
    if (!(next && r == 1)) col[j + r] = x;  // row j+1 of the next reflector column is written once, below
    if (r >= 1) ss += x * x;
    if (r == 1) x0 = x;
  }
  if (next) {
    ss = wave_sum_f64(ss);
    x0 = __shfl(x0, 1, 64);  // row j+1 is lane 1's first row
    if (lane == 0) qr_reflector(ss, x0, col, j + 1, qr_vec(ws, q, t, 0), vvs);
  }
}

// Least squares: back substitution R x = (Q^T y)[0..n), column-oriented, one
// workgroup per position; y (column n of M) is consumed in place.
__global__ __launch_bounds__(256) void k_qr_backsub(QrDims q, double* __restrict__ ws,
                                                    const int32_t* __restrict__ flag, int d,
                                                    float* __restrict__ g_hat, float* __restrict__ c_hat) {
  const int64_t t = blockIdx.x;
  double* M = qr_mat(ws, q, t);
  double* y = M + (int64_t)q.n * q.ld;
  const double* rdiag = qr_vec(ws, q, t, 0);
  double* x = qr_vec(ws, q, t, 2);
  __shared__ double xi_s;
  for (int i = q.n - 1; i >= 0; --i) {
    if (threadIdx.x == 0) {
      xi_s = y[i] / rdiag[i];
      x[i] = xi_s;
    }
    __syncthreads();
    const double xi = xi_s;
    const double* ci = M + (int64_t)i * q.ld;  // R[r][i], r < i
    for (int r = threadIdx.x; r < i; r += 256) y[r] -= ci[r] * xi;
    __syncthreads();
  }
  const bool bad = flag[t] != 0;
  const float nan = __builtin_nanf("");
  for (int c = threadIdx.x; c < d; c += 256) g_hat[t * d + c] = bad ? nan : (float)x[c];
  if (threadIdx.x == 0) c_hat[t] = bad ? nan : (float)x[d];
}

// Minimum norm: R^T w = y (forward substitution, R = the k x k upper
// triangle), then x = Q [w; 0] = H_0 H_1 .. H_{k-1} [w; 0].
__global__ __launch_bounds__(256) void k_qr_minnorm(QrDims q, double* __restrict__ ws,
                                                    const int32_t* __restrict__ flag, int d,
                                                    float* __restrict__ g_hat, float* __restrict__ c_hat) {
  const int64_t t = blockIdx.x;
  const double* M = qr_mat(ws, q, t);
  const double* rdiag = qr_vec(ws, q, t, 0);
  const double* vvs = qr_vec(ws, q, t, 1);
  double* y = qr_vec(ws, q, t, 2);
  double* x = qr_vec(ws, q, t, 3);
  const int m = q.ncols, n = q.P;
  __shared__ double wi_s;
  __shared__ double red[4];
  for (int i = 0; i < m; ++i) {
    if (threadIdx.x == 0) wi_s = y[i] / rdiag[i];
    __syncthreads();
    const double wi = wi_s;
    // R[i][r] (r > i) is row i of column r
    for (int r = i + 1 + threadIdx.x; r < m; r += 256) y[r] -= M[(int64_t)r * q.ld + i] * wi;
    if (threadIdx.x == 0) y[i] = wi;
    __syncthreads();
  }
  for (int r = threadIdx.x; r < n; r += 256) x[r] = r < m ? y[r] : 0.0;
  __syncthreads();
  for (int j = m - 1; j >= 0; --j) {
    const double* vj = M + (int64_t)j * q.ld;
    double s = 0.0;
    for (int r = j + threadIdx.x; r < n; r += 256) s += vj[r] * x[r];
    s = wave_sum_f64(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    s = red[0] + red[1] + red[2] + red[3];
    const double f = vvs[j] > 0.0 ? 2.0 * s / vvs[j] : 0.0;
    for (int r = j + threadIdx.x; r < n; r += 256) x[r] -= f * vj[r];
    __syncthreads();
  }
  const bool bad = flag[t] != 0;
  const float nan = __builtin_nanf("");
  for (int c = threadIdx.x; c < d; c += 256) g_hat[t * d + c] = bad ? nan : (float)x[c];
  if (threadIdx.x == 0) c_hat[t] = bad ? nan : (float)x[d];
}

static bool qr_plan(int64_t T, int64_t d, int32_t k, QrDims& q, size_t& bytes) {
  if (T < 0 || d <= 0 || k < 1) return false;
  q.n = (int)(d + 1);
  q.lsq = k >= d + 1;
  q.P = q.lsq ? k : (int)(d + 1);
  q.ncols = q.lsq ? (int)(d + 2) : k;
  if (q.P > QMAXP || q.ncols > QMAXP) return false;
  q.ld = (q.P + 1) & ~1;
  const int vlen = q.ld > q.ncols ? q.ld : q.ncols;
  q.per = (int64_t)q.ncols * q.ld + 4 * (int64_t)vlen;
  bytes = (size_t)(T > 0 ? T : 1) * q.per * sizeof(double) + (size_t)kd_round_up((T > 0 ? T : 1) * 4, 256);
  return true;
}

}  // namespace

extern "C" size_t kd_teacher_recover_workspace(int64_t T, int64_t d, int32_t k) {
  QrDims q;
  size_t bytes;
  if (!qr_plan(T, d, k, q, bytes)) return 0;
  return bytes;
}

extern "C" kd_status kd_teacher_recover_ws(const int32_t* idx, const float* teacher_logp, const kd_bf16* U,
                                           const float* b, int64_t T, int64_t d, int64_t V, int32_t k, float* g_hat,
                                           float* c_hat, void* ws, size_t ws_bytes, void* stream) {
  QrDims q;
  size_t bytes;
  if (T < 0 || d <= 0 || V <= 0 || k < 1 || k > V || !qr_plan(T, d, k, q, bytes))
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld d=%lld V=%lld k=%d (need 1 <= k <= V, max(k, d+2) <= %d)",
                   (long long)T, (long long)d, (long long)V, (int)k, QMAXP);
  if (T == 0) return KD_OK;
  if (!idx || !teacher_logp || !U || !g_hat || !c_hat) return kd_fail(KD_EINVAL, "null required pointer");
  if (!ws || ws_bytes < bytes) return kd_fail(KD_ENOWS, "workspace too small: need %zu bytes, got %zu", bytes, ws_bytes);
  if (T > 65535) return kd_fail(KD_EUNSUPPORTED, "at most 65535 positions per call (got %lld)", (long long)T);
  hipStream_t s = (hipStream_t)stream;
  double* w = (double*)ws;
  int32_t* flag = (int32_t*)((char*)ws + (size_t)T * q.per * sizeof(double));
  KD_LAUNCH(k_fill_flags, dim3((unsigned)kd_ceil_div(T, 256)), dim3(256), 0, s, flag, T);
  KD_LAUNCH(k_qr_fill, dim3((unsigned)q.ncols, (unsigned)T), dim3(256), 0, s, idx, teacher_logp, (const bf16_t*)U, b, V,
            (int)d, (int)k, q, w, flag);
  // factored columns: all n unknowns (least squares) or all k (minimum norm)
  const int nfact = q.lsq ? q.n : q.ncols;
  KD_LAUNCH(k_qr_first, dim3((unsigned)T), dim3(64), 0, s, q, w);
  for (int j = 0; j + 1 < q.ncols && j < nfact; ++j) {
    const int ncol = q.ncols - j - 1;
    KD_LAUNCH(k_qr_step, dim3((unsigned)kd_ceil_div(ncol, QW), (unsigned)T), dim3(256), 0, s, q, j, nfact, w);
  }
  if (q.lsq)
    KD_LAUNCH(k_qr_backsub, dim3((unsigned)T), dim3(256), 0, s, q, w, (const int32_t*)flag, (int)d, g_hat, c_hat);
  else
    KD_LAUNCH(k_qr_minnorm, dim3((unsigned)T), dim3(256), 0, s, q, w, (const int32_t*)flag, (int)d, g_hat, c_hat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e));
  return KD_OK;
}

extern "C" kd_status kd_teacher_recover(const int32_t* idx, const float* teacher_logp, const kd_bf16* U,
                                        const float* b, int64_t T, int64_t d, int64_t V, int32_t k, float* g_hat,
                                        float* c_hat, void* stream) {
  if (T < 0 || d <= 0 || V <= 0 || k < d + 1 || k > V)
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld d=%lld V=%lld k=%d (need d+1 <= k <= V)", (long long)T,
                   (long long)d, (long long)V, (int)k);
  const int kp = (k % 2 == 0) ? k + 1 : k;
  if ((int64_t)(d + 2) * kp > RCAP)
    return kd_fail(KD_EUNSUPPORTED, "system too large for one workgroup: (d+2)*k = %lld > %d", (long long)((d + 2) * kp),
                   RCAP);
  if (T == 0) return KD_OK;
  if (!idx || !teacher_logp || !U || !g_hat || !c_hat) return kd_fail(KD_EINVAL, "null required pointer");
  hipStream_t s = (hipStream_t)stream;
  const size_t lds = ((size_t)(d + 2) * kp + 2 * (size_t)(d + 1) + 4) * sizeof(double);
  KD_LAUNCH(k_recover, dim3((unsigned)T), dim3(RN), lds, s, idx, teacher_logp, (const bf16_t*)U, b, V, (int)d, (int)k,
            kp, g_hat, c_hat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e));
  return KD_OK;
}
