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

}  // namespace

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
