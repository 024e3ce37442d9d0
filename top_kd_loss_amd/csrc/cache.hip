// Teacher-cache build for gfx950: z = U g + b per token on the matrix cores
// ("The Gradient That Top-k Distillation Never Computes", Figure 3: a
// hidden-state cache reconstructs the logits at 2dV FLOP per token), then a
// row pass that keeps the top-K logits ("keep the top-k of the teacher's
// logits", same figure; "Efficient Knowledge Distillation for LLMs: Offline
// Top-K Logits and a Fused Chunked KL Loss", section 3.2), the logsumexp,
// the tail mass m_q, and the adaptive support k_rho = min{k : top-k mass
// >= rho} ("Sparse Teacher Support Cuts LLM Distillation Cost Without
// Losing Accuracy").
//
// Row pass, one workgroup per row (HBM bound, the row is streamed a few
// times and stays in the last-level cache between passes):
//   A  row max and an 11-bit radix histogram of order-preserving keys
//   B  sum of exp(z - max); per-bin fixed-point mass; candidates of the
//      top-K (every key in bins above the K-th one plus that bin), refined
//      by further radix digits only when that bin is too large
//   sort the candidates by (key desc, index asc) in LDS: ties go to the
//      lower index, -0.0 ties with +0.0
//   C, D  two more radix digits of the mass histogram, only around the bin
//      where the cumulative mass crosses rho, to get k_rho exactly
#include <hip/hip_runtime.h>
#include <math.h>

#include "../../include/kdtopk.h"
#include "gemm.h"
#include "kd_internal.h"

namespace {

using CC = PipeCfg<256, 256, 2, 2>;
constexpr int RT = 1024;      // threads of the row kernel
constexpr int NB = 2048;      // radix bins per digit (11 bits)
constexpr int CAP = 4096;     // candidate capacity (LDS)
constexpr int KMAX = 1024;
constexpr int RHO_MAX = 8;

__device__ __forceinline__ bool tile_of(int bid, int nblocks, int nM, int nN, int group_m, int& mi, int& ni) {
  const int per = nblocks / 8;
  const int L = (bid % 8) * per + bid / 8;
  if (L >= nM * nN) return false;
  const int width = group_m * nN;
  const int group = L / width;
  const int first_m = group * group_m;
  const int gsz = min(nM - first_m, group_m);
  const int r = L - group * width;
  mi = first_m + r % gsz;
  ni = r / gsz;
  return true;
}

// z[t][v] = sum_j g[t][j] U[v][j] + b[v] for the token block [t0, t0+Tb).
__global__ __launch_bounds__(256, 1) void k_cache_gemm(const bf16_t* __restrict__ g, const bf16_t* __restrict__ U,
                                                       const float* __restrict__ b, int64_t Tb, int64_t d,
                                                       int64_t V, int nTT, int nVT, float* __restrict__ z) {
  extern __shared__ __align__(16) bf16_t lds[];
  int tt, vt;
  if (!tile_of(blockIdx.x, gridDim.x, nTT, nVT, 4, tt, vt)) return;
  const int64_t m0 = (int64_t)tt * CC::BM, n0 = (int64_t)vt * CC::BN;
  Acc<CC> acc;
  gemm_tile_pipe<CC>(g, d, m0, Tb, U, d, n0, V, (int)d, lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / CC::WN, wn = wave % CC::WN;
#pragma unroll
  for (int fn = 0; fn < CC::FN; ++fn) {
    const int64_t v = n0 + acc_col<CC>(wn, fn, lane);
    const float bv = (b != nullptr && v < V) ? b[v] : 0.f;
#pragma unroll
    for (int fm = 0; fm < CC::FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = m0 + acc_row<CC>(wm, fm, e, lane);
        if (t < Tb && v < V) z[t * V + v] = acc.v[fm][fn][e] + bv;
      }
  }
}

// Order-preserving key of a float: larger value -> larger key; -0.0 -> +0.0.
__device__ __forceinline__ uint32_t fkey(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct RowShared {
  unsigned long long cand[CAP];   // ((~key) << 32) | index, sorted ascending
  int hist[NB];
  unsigned long long mass[NB];
  int scan_i[RT / 64];
  float red_f[RT / 64];
  double red_d[RT / 64];
  int ncand;
  int sel_bin;
  int sel_above;
  int sel_eq;
  unsigned long long rho_target, rho_cum;
  int rho_cnt, rho_done, rho_bin;
  uint32_t rho_pre;
};

__device__ __forceinline__ float block_max(float v, RowShared& S) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) S.red_f[w] = v;
  __syncthreads();
  float r = S.red_f[0];
  for (int i = 1; i < RT / 64; ++i) r = fmaxf(r, S.red_f[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ double block_sum_d(double v, RowShared& S) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) S.red_d[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < RT / 64; ++i) r += S.red_d[i];
  __syncthreads();
  return r;
}

// From the histogram of a digit, find the bin holding the `need`-th largest
// element (1-based, counting from the top): returns the bin, the count
// strictly above it, and its own count.  Thread 0 scans; result in S.
__device__ void find_kth_bin(RowShared& S, int need) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int cum = 0, b = NB - 1;
    for (; b > 0; --b) {
      if (cum + S.hist[b] >= need) break;
      cum += S.hist[b];
    }
    S.sel_bin = b;
    S.sel_above = cum;
    S.sel_eq = S.hist[b];
  }
  __syncthreads();
}

__device__ void clear_hist(RowShared& S, bool with_mass) {
  for (int i = threadIdx.x; i < NB; i += RT) {
    S.hist[i] = 0;
    if (with_mass) S.mass[i] = 0ull;
  }
  __syncthreads();
}

// Bitonic sort of S.cand[0..n) ascending, padded to a power of two with ~0.
__device__ void sort_cand(RowShared& S, int n) {
  int np = 1;
  while (np < n) np <<= 1;
  for (int i = n + threadIdx.x; i < np; i += RT) S.cand[i] = ~0ull;
  __syncthreads();
  for (int size = 2; size <= np; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < np / 2; i += RT) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long a = S.cand[lo], c = S.cand[hi];
        if ((a > c) == up) {
          S.cand[lo] = c;
          S.cand[hi] = a;
        }
      }
      __syncthreads();
    }
}

// Block-wide exclusive prefix count of `flag` in thread order; returns this
// thread's rank and writes the total to *total.
__device__ int block_rank(bool flag, RowShared& S, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int before = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) S.scan_i[w] = __popcll(bal);
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < RT / 64; ++i) {
    if (i < w) off += S.scan_i[i];
    tot += S.scan_i[i];
  }
  __syncthreads();
  *total = tot;
  return off + before;
}

__global__ __launch_bounds__(RT) void k_topk_rows(const float* __restrict__ z, int64_t ldz, int64_t V, int K,
                                                  int n_rho, float rho0, float rho1, float rho2, float rho3,
                                                  float rho4, float rho5, float rho6, float rho7,
                                                  int32_t* __restrict__ idx_out, float* __restrict__ val_out,
                                                  float* __restrict__ lse_out, float* __restrict__ mq_out,
                                                  int32_t* __restrict__ krho_out) {
  __shared__ RowShared S;
  const int64_t row = blockIdx.x;
  const float* zr = z + row * ldz;
  const int tid = threadIdx.x;

  // ---- pass A: max and the first-digit histogram
  clear_hist(S, true);
  float mx = -KD_INF;
  for (int64_t i = tid; i < V; i += RT) {
    const float x = zr[i];
    mx = fmaxf(mx, x);
    atomicAdd(&S.hist[fkey(x) >> 21], 1);
  }
  const float M = block_max(mx, S);
  find_kth_bin(S, K);

  // ---- candidate selection, refining the digit while the bin is too big
  uint32_t pre = (uint32_t)S.sel_bin;  // key prefix of the K-th element
  int pbits = 11;                      // bits of the key fixed by `pre`
  int above = S.sel_above;             // elements with key prefix > pre
  int eq = S.sel_eq;
  while (above + eq > CAP && pbits < 32) {
    const int dbits = (pbits == 11) ? 11 : 10;
    const int sh = 32 - pbits - dbits;
    clear_hist(S, false);
    for (int64_t i = tid; i < V; i += RT) {
      const uint32_t k = fkey(zr[i]);
      if ((k >> (32 - pbits)) == pre) atomicAdd(&S.hist[(k >> sh) & ((1u << dbits) - 1u)], 1);
    }
    find_kth_bin(S, K - above);
    pre = (pre << dbits) | (uint32_t)S.sel_bin;
    pbits += dbits;
    above += S.sel_above;
    eq = S.sel_eq;
  }

  // ---- pass B: exp-sum and candidate collection
  if (tid == 0) S.ncand = 0;
  const int vbits = 64 - __clzll((unsigned long long)V);  // V < 2^vbits
  const double fx_scale = ldexp(1.0, 62 - vbits);          // exp(x - M) <= 1 per element
  __syncthreads();
  float se = 0.f;
  const bool exact_tail = (above + eq > CAP);  // only when all 32 key bits tie
  for (int64_t i = tid; i < V; i += RT) {
    const float x = zr[i];
    const float ex = __expf(x - M);
    se += ex;
    const uint32_t k = fkey(x);
    const uint32_t kp = k >> (32 - pbits);
    if (kp > pre || (!exact_tail && kp == pre)) {
      const int slot = atomicAdd(&S.ncand, 1);
      S.cand[slot] = ((unsigned long long)(~k) << 32) | (unsigned long long)i;
    }
  }
  const double sum_e = block_sum_d((double)se, S);
  const double lse = (double)M + log(sum_e);
  __syncthreads();
  int nc = S.ncand;
  if (exact_tail) {
    // all remaining ties share one key: take the lowest indices, in order
    int need = K - nc;
    for (int64_t base = 0; base < V && need > 0; base += RT) {
      const int64_t i = base + tid;
      const bool f = (i < V) && (fkey(zr[i]) == pre);
      int tot;
      const int r = block_rank(f, S, &tot);
      if (f && r < need) S.cand[nc + r] = ((unsigned long long)(~pre) << 32) | (unsigned long long)i;
      const int took = tot < need ? tot : need;
      nc += took;
      need -= took;
      __syncthreads();
    }
  }
  sort_cand(S, nc);

  // ---- outputs of the top-K
  double kept = 0.0;
  for (int k = tid; k < K; k += RT) {
    const int64_t i = (int64_t)(S.cand[k] & 0xffffffffull);
    const float x = zr[i];
    idx_out[row * K + k] = (int32_t)i;
    val_out[row * K + k] = x;
    kept += exp((double)x - lse);
  }
  kept = block_sum_d(kept, S);
  if (tid == 0) {
    lse_out[row] = (float)lse;
    mq_out[row] = (float)(1.0 - kept);
  }
  if (n_rho == 0) return;

  // ---- k_rho: cumulative mass from the top, refined digit by digit around
  // the crossing.  Masses are fixed point (exact integer sums), so the
  // result does not depend on the order of the atomics.
  const float rhos[RHO_MAX] = {rho0, rho1, rho2, rho3, rho4, rho5, rho6, rho7};
  for (int j = 0; j < n_rho; ++j) {
    clear_hist(S, true);
    for (int64_t i = tid; i < V; i += RT) {
      const float x = zr[i];
      const uint32_t k = fkey(x);
      atomicAdd(&S.hist[k >> 21], 1);
      atomicAdd(&S.mass[k >> 21], (unsigned long long)llrint((double)__expf(x - M) * fx_scale));
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long tot = 0;
      for (int bb = 0; bb < NB; ++bb) tot += S.mass[bb];
      unsigned long long target = (unsigned long long)ceil((double)rhos[j] * (double)tot);
      if (target == 0) target = 1;
      unsigned long long cum = 0;
      int cnt = 0, bb = NB - 1;
      for (; bb >= 0; --bb) {
        if (cum + S.mass[bb] >= target) break;
        cum += S.mass[bb];
        cnt += S.hist[bb];
      }
      S.rho_target = target;
      S.rho_cum = cum;
      S.rho_cnt = bb < 0 ? (int)V : cnt;
      S.rho_done = bb < 0 ? 1 : 0;  // rounding kept the total below rho
      S.rho_pre = (uint32_t)(bb < 0 ? 0 : bb);
      S.rho_bin = bb < 0 ? 0 : bb;
    }
    __syncthreads();
    for (int pb = 11; pb < 32 && !S.rho_done;) {
      const int dbits = (pb == 11) ? 11 : 10;
      const int sh = 32 - pb - dbits;
      const uint32_t pfx = S.rho_pre;
      clear_hist(S, true);
      for (int64_t i = tid; i < V; i += RT) {
        const float x = zr[i];
        const uint32_t k = fkey(x);
        if ((k >> (32 - pb)) == pfx) {
          const int dg = (int)((k >> sh) & ((1u << dbits) - 1u));
          atomicAdd(&S.hist[dg], 1);
          atomicAdd(&S.mass[dg], (unsigned long long)llrint((double)__expf(x - M) * fx_scale));
        }
      }
      __syncthreads();
      if (tid == 0) {
        unsigned long long cum = S.rho_cum;
        int cnt = S.rho_cnt, bb = (1 << dbits) - 1;
        for (; bb > 0; --bb) {
          if (cum + S.mass[bb] >= S.rho_target) break;
          cum += S.mass[bb];
          cnt += S.hist[bb];
        }
        S.rho_cum = cum;
        S.rho_cnt = cnt;
        S.rho_pre = (pfx << dbits) | (uint32_t)bb;
        S.rho_bin = bb;
      }
      __syncthreads();
      pb += dbits;
    }
    if (tid == 0) {
      int cnt = S.rho_cnt;
      if (!S.rho_done) {
        // every element of the final bin has one key, hence one mass
        const int nb = S.hist[S.rho_bin];
        const unsigned long long each = nb > 0 ? S.mass[S.rho_bin] / (unsigned long long)nb : 0ull;
        const unsigned long long gap = S.rho_target - S.rho_cum;
        long long jn = each > 0 ? (long long)((gap + each - 1) / each) : (long long)nb;
        if (jn < 1) jn = 1;
        if (jn > nb) jn = nb;
        cnt += (int)jn;
      }
      krho_out[row * n_rho + j] = cnt;
    }
    __syncthreads();
  }
}

struct CachePlan {
  int64_t Tb;
  size_t zbytes, total;
};

static bool plan_cache(int64_t T, int64_t d, int64_t V, int32_t K, int32_t n_rho, CachePlan& p) {
  if (T < 0 || d <= 0 || V <= 0 || K < 1 || K > KMAX || K > V || d % 64 != 0 || d > 16384) return false;
  if (n_rho < 0 || n_rho > RHO_MAX || V >= ((int64_t)1 << 31)) return false;
  // token block: bounded fp32 logit scratch of about 1.25 GB or less
  int64_t tb = (int64_t)((1.25e9 / 4.0) / (double)V);
  tb = (tb / CC::BM) * CC::BM;
  if (tb < CC::BM) tb = CC::BM;
  if (tb > kd_round_up(T > 0 ? T : 1, CC::BM)) tb = kd_round_up(T > 0 ? T : 1, CC::BM);
  p.Tb = tb;
  p.zbytes = (size_t)tb * V * 4;
  p.total = p.zbytes + 256;
  return true;
}

static kd_status check_rho(const float* rho_host, int32_t n_rho) {
  if (n_rho > 0 && !rho_host) return kd_fail(KD_EINVAL, "rho_host is NULL with n_rho=%d", (int)n_rho);
  for (int j = 0; j < n_rho; ++j)
    if (!(rho_host[j] > 0.f && rho_host[j] <= 1.f)) return kd_fail(KD_EINVAL, "rho[%d]=%g outside (0, 1]", j, rho_host[j]);
  return KD_OK;
}

static void launch_rows(const float* z, int64_t ldz, int64_t rows, int64_t V, int K, const float* rho, int n_rho,
                        int32_t* idx, float* val, float* lse, float* m_q, int32_t* k_rho, hipStream_t s) {
  float r[RHO_MAX] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < n_rho; ++j) r[j] = rho[j];
  KD_LAUNCH(k_topk_rows, dim3((unsigned)rows), dim3(RT), 0, s, z, ldz, V, K, n_rho, r[0], r[1], r[2], r[3],
                     r[4], r[5], r[6], r[7], idx, val, lse, m_q, k_rho);
}

}  // namespace

extern "C" size_t kd_topk_cache_build_workspace(int64_t T, int64_t d, int64_t V, int32_t K, int32_t n_rho) {
  CachePlan p;
  if (!plan_cache(T, d, V, K, n_rho, p)) return 0;
  return p.total;
}

extern "C" kd_status kd_topk_cache_build(const kd_bf16* g, const kd_bf16* U, const float* b, int64_t T, int64_t d,
                                         int64_t V, int32_t K, const float* rho_host, int32_t n_rho, int32_t* idx,
                                         float* val, float* lse, float* m_q, int32_t* k_rho, void* ws, size_t ws_bytes,
                                         void* stream) {
  CachePlan p;
  if (!plan_cache(T, d, V, K, n_rho, p))
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld d=%lld V=%lld K=%d n_rho=%d (need 1<=K<=min(V,1024), d%%64==0, 0<=n_rho<=8)",
                   (long long)T, (long long)d, (long long)V, (int)K, (int)n_rho);
  kd_status st = check_rho(rho_host, n_rho);
  if (st != KD_OK) return st;
  if (T == 0) return KD_OK;
  if (!g || !U || !idx || !val || !lse || !m_q || (n_rho > 0 && !k_rho))
    return kd_fail(KD_EINVAL, "null required pointer");
  if (!ws || ws_bytes < p.total) return kd_fail(KD_ENOWS, "workspace too small: need %zu bytes, got %zu", p.total, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  float* z = (float*)ws;
  for (int64_t t0 = 0; t0 < T; t0 += p.Tb) {
    const int64_t tb = (T - t0 < p.Tb) ? T - t0 : p.Tb;
    const int nTT = (int)kd_ceil_div(tb, CC::BM), nVT = (int)kd_ceil_div(V, CC::BN);
    const int grid = (int)kd_round_up((int64_t)nTT * nVT, 8);
    KD_LAUNCH(k_cache_gemm, dim3(grid), dim3(CC::NT), CC::LDS_BYTES, s, (const bf16_t*)g + t0 * d,
                       (const bf16_t*)U, b, tb, d, V, nTT, nVT, z);
    launch_rows(z, V, tb, V, K, rho_host, n_rho, idx + t0 * K, val + t0 * K, lse + t0, m_q + t0,
                n_rho ? k_rho + t0 * n_rho : nullptr, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e));
  }
  return KD_OK;
}

extern "C" size_t kd_topk_rows_workspace(int64_t T, int64_t V, int32_t K, int32_t n_rho) {
  if (T < 0 || V <= 0 || K < 1 || K > KMAX || K > V || n_rho < 0 || n_rho > RHO_MAX) return 0;
  return 256;
}

extern "C" kd_status kd_topk_rows(const float* z, int64_t T, int64_t V, int32_t K, const float* rho_host,
                                  int32_t n_rho, int32_t* idx, float* val, float* lse, float* m_q, int32_t* k_rho,
                                  void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || V <= 0 || K < 1 || K > KMAX || K > V || n_rho < 0 || n_rho > RHO_MAX || V >= ((int64_t)1 << 31))
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld V=%lld K=%d n_rho=%d", (long long)T, (long long)V, (int)K, (int)n_rho);
  kd_status st = check_rho(rho_host, n_rho);
  if (st != KD_OK) return st;
  if (T == 0) return KD_OK;
  if (!z || !idx || !val || !lse || !m_q || (n_rho > 0 && !k_rho)) return kd_fail(KD_EINVAL, "null required pointer");
  (void)ws;
  (void)ws_bytes;
  launch_rows(z, V, T, V, K, rho_host, n_rho, idx, val, lse, m_q, k_rho, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e));
  return KD_OK;
}
