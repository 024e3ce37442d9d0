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
// Row pass, one workgroup per row (HBM bound; the row is streamed two or
// three times and stays in the last-level cache between passes):
//   1  an 11-bit radix histogram of order-preserving keys with, per bin, the
//      count and the sum of exp(z - upper edge of the bin) in 2^-31 fixed
//      point (exact 64-bit integer sums: independent of atomic order);
//      logsumexp follows from the bin masses
//   2  candidates of the top-K (every key in bins above the K-th one plus
//      that bin; extra digit passes only when that bin is too large), and the
//      next 11-bit digit of the bins where the cumulative mass crosses rho
//   3  the last 10-bit digit of those bins: the crossing key is exact
//   sort the candidates by (key desc, index asc) in LDS: ties go to the
//      lower index, -0.0 ties with +0.0
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
// The tile is computed as z^T (rows = vocabulary, columns = tokens), so each
// lane holds 4 consecutive vocabulary entries of one token.  The epilogue
// stages half of the tile's tokens at a time in LDS (fp32, 1 KB token rows,
// 16-byte chunks XOR-swizzled by token) and stores whole token rows with the
// bias added: 1 KB of contiguous z per wavefront store.
constexpr int CG_LDS = (CC::BN / 2) * CC::BM * 4;  // 128 tokens x 256 vocabulary fp32
static_assert(CG_LDS >= CC::LDS_BYTES, "epilogue staging reuses the operand stages");

__device__ __forceinline__ int cg_swz(int tl) { return (tl & 31) << 1; }

__global__ __launch_bounds__(256, 1) void k_cache_gemm(const bf16_t* __restrict__ g, const bf16_t* __restrict__ U,
                                                       const float* __restrict__ b, int64_t Tb, int64_t d,
                                                       int64_t V, int nTT, int nVT, float* __restrict__ z) {
  extern __shared__ __align__(16) bf16_t lds[];
  int vt, tt;
  if (!tile_of(blockIdx.x, gridDim.x, nVT, nTT, 4, vt, tt)) return;
  const int64_t m0 = (int64_t)vt * CC::BM, n0 = (int64_t)tt * CC::BN;
  Acc<CC> acc;
  gemm_tile_pipe<CC>(U, d, m0, V, g, d, n0, Tb, (int)d, lds, acc);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / CC::WN, wn = wave % CC::WN;
  float* E = (float*)lds;
  // readout: thread -> 16-byte chunk c of the token rows wave, wave+4, ...
  const int c = tid & 63;
  const int64_t v = m0 + 4 * c;
  float bv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) bv[e] = (b != nullptr && v + e < V) ? b[v + e] : 0.f;
  const bool vec = ((V & 3) == 0) && (v + 3 < V);
  __syncthreads();  // every wavefront is done with the operand stages
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wn == half) {
#pragma unroll
      for (int fn = 0; fn < CC::FN; ++fn) {
        const int tl = fn * 32 + (lane & 31);
        float* row = E + tl * CC::BM;
#pragma unroll
        for (int fm = 0; fm < CC::FM; ++fm)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cv = (wm * CC::TM + fm * 32 + 8 * q + 4 * (lane >> 5)) >> 2;
            *(f32x4*)(row + ((cv ^ cg_swz(tl)) << 2)) =
                f32x4{acc.v[fm][fn][4 * q], acc.v[fm][fn][4 * q + 1], acc.v[fm][fn][4 * q + 2], acc.v[fm][fn][4 * q + 3]};
          }
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < CC::BN / 2 / 4; ++i) {
      const int tl = wave + 4 * i;
      const int64_t t = n0 + half * (CC::BN / 2) + tl;
      f32x4 x = *(const f32x4*)(E + tl * CC::BM + ((c ^ cg_swz(tl)) << 2));
      x += f32x4{bv[0], bv[1], bv[2], bv[3]};
      if (t < Tb) {
        float* dst = z + t * V + v;
        if (vec) {
          *(f32x4*)dst = x;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < V) dst[e] = x[e];
        }
      }
    }
    __syncthreads();
  }
}

// Order-preserving key of a float: larger value -> larger key; -0.0 -> +0.0.
__device__ __forceinline__ uint32_t fkey(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int RHO_GROUP = 2;  // k_rho targets refined together in one pass

constexpr int NCOPY = 4;       // level-0 histogram copies in pass 1 (by lane % 4): fewer same-address atomics

struct RowShared {
  // Pass 1 uses `copies`; afterwards the same bytes hold the top-K candidates
  // and the refinement histograms.
  union {
    struct {
      int cnt[NCOPY][NB];
      unsigned long long mass[NCOPY][NB];
    } copies;
    struct {
      unsigned long long cand[CAP];             // ((~key) << 32) | index
      int cntR[RHO_GROUP][NB];                  // refinement digits (top-K uses cntR[0])
      unsigned long long massR[RHO_GROUP][NB];
    } late;
  } u;
  float ref0[NB];                               // upper edge of each level-0 bin
  int cnt0[NB];                                 // level-0 counts
  unsigned long long mass0[NB];                 // level-0 fixed-point masses, each vs its bin's upper edge
  int scan_i[RT / 64];
  double red_d[RT / 64];
  int ncand, sel_bin, sel_above, sel_eq;
  double scan_w[RT / 64];
  int scan_wi[RT / 64];
  int f_bin, f_cnt_above;
  double f_above, f_total;
  // k_rho state per target of the current group
  double r_target[RHO_GROUP], r_cum[RHO_GROUP];
  int r_cnt[RHO_GROUP], r_done[RHO_GROUP];
  uint32_t r_pre[RHO_GROUP];
  double lse;
};

// Largest float whose key has prefix `p` in its top `bits` bits: the upper
// edge of a histogram bin.  Clamped to FLT_MAX for bins above the finite range.
__device__ __forceinline__ float bin_upper(uint32_t p, int bits) {
  const uint32_t k = (bits == 32) ? p : ((p << (32 - bits)) | ((1u << (32 - bits)) - 1u));
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  const float f = __uint_as_float(u);
  return (f != f || f > 3.4028234663852886e38f) ? 3.4028234663852886e38f : f;
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

// Block-wide inclusive scan of (double, int) pairs in thread order; also
// returns the exclusive values, taken as the previous thread's inclusive ones
// so that consecutive threads agree exactly.
__device__ __forceinline__ void block_scan2(double v, int c, RowShared& S, double& incl, double& excl, int& cincl,
                                            int& cexcl) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double x = v;
  int y = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double tx = __shfl_up(x, o, 64);
    const int ty = __shfl_up(y, o, 64);
    if (lane >= o) {
      x += tx;
      y += ty;
    }
  }
  if (lane == 63) {
    S.scan_w[w] = x;
    S.scan_wi[w] = y;
  }
  __syncthreads();
  double off = 0.0;
  int offi = 0;
  for (int i = 0; i < w; ++i) {
    off += S.scan_w[i];
    offi += S.scan_wi[i];
  }
  __syncthreads();
  const double px = __shfl_up(x, 1, 64);
  const int py = __shfl_up(y, 1, 64);
  incl = off + x;
  cincl = offi + y;
  excl = lane == 0 ? off : off + px;
  cexcl = lane == 0 ? offi : offi + py;
}

// Walk bins nb-1 .. 0 (descending key) accumulating mass(b) and count(b);
// find the bin where the running mass first reaches `target`.  Returns the
// bin (-1 when the total stays below), the mass and the count strictly above
// it.  Thread t owns the descending positions 2t and 2t+1 (nb <= 2 * RT).
// With mass = count and an integer target this is the K-th element search.
template <class FM, class FC>
__device__ void find_from_top(RowShared& S, int nb, double target, FM&& mass, FC&& count, int* bin,
                              double* above, int* cnt_above) {
  const int t = threadIdx.x;
  const int b0 = nb - 1 - 2 * t, b1 = b0 - 1;
  const double v0 = b0 >= 0 ? mass(b0) : 0.0, v1 = b1 >= 0 ? mass(b1) : 0.0;
  const int c0 = b0 >= 0 ? count(b0) : 0, c1 = b1 >= 0 ? count(b1) : 0;
  double incl, excl;
  int cincl, cexcl;
  if (t == 0) S.f_bin = -1;
  block_scan2(v0 + v1, c0 + c1, S, incl, excl, cincl, cexcl);
  // a target beyond the level's total (rounding of per-bin references) is
  // met at the last non-empty bin
  if (t == RT - 1) S.f_total = incl;
  __syncthreads();
  const double tg = target < S.f_total ? target : S.f_total;
  if (b0 >= 0 && excl < tg && incl >= tg) {
    if (excl + v0 >= tg || b1 < 0) {
      S.f_bin = b0;
      S.f_above = excl;
      S.f_cnt_above = cexcl;
    } else {
      S.f_bin = b1;
      S.f_above = excl + v0;
      S.f_cnt_above = cexcl + c0;
    }
  }
  __syncthreads();
  *bin = S.f_bin;
  *above = S.f_above;
  *cnt_above = S.f_cnt_above;
  __syncthreads();
}

// Bin of a count histogram holding the need-th largest element (1-based):
// the bin, the count strictly above it, its own count (in S.sel_*).
__device__ void find_kth_bin(RowShared& S, const int* hist, int nbins, int need) {
  __syncthreads();
  int bin, ca;
  double ma;
  find_from_top(S, nbins, (double)need, [&](int b) { return (double)hist[b]; }, [&](int b) { return hist[b]; },
                &bin, &ma, &ca);
  if (bin < 0) {  // cannot happen for need <= total; keep the lowest bin
    bin = 0;
  }
  if (threadIdx.x == 0) {
    S.sel_bin = bin;
    S.sel_above = (int)ma;
    S.sel_eq = hist[bin];
  }
  __syncthreads();
}

// Sort S.u.late.cand[0..n) ascending, keeping at least the K smallest at the
// front.  Candidates are distinct 64-bit keys, so each one's rank is the
// number of smaller ones (broadcast LDS reads, no network of barriers); the
// K smallest are written by rank to [CAP-K, CAP) (disjoint from [0, n) since
// n <= 2*RT <= CAP-K) and moved to the front.  Larger n: bitonic network.
__device__ void sort_cand(RowShared& S, int n, int K) {
  constexpr int PER = 2;  // candidates ranked per thread
  static_assert(RT * PER + KMAX <= CAP, "rank-sort staging must not overlap the candidates");
  if (n <= RT * PER) {
    unsigned long long mine[PER];
    int rank[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = threadIdx.x + q * RT;
      mine[q] = i < n ? S.u.late.cand[i] : ~0ull;
      rank[q] = 0;
    }
    for (int j = 0; j < n; ++j) {
      const unsigned long long c = S.u.late.cand[j];
#pragma unroll
      for (int q = 0; q < PER; ++q) rank[q] += (c < mine[q]) ? 1 : 0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = threadIdx.x + q * RT;
      if (i < n && rank[q] < K) S.u.late.cand[CAP - K + rank[q]] = mine[q];
    }
    __syncthreads();
    unsigned long long v = 0ull;
    if ((int)threadIdx.x < K) v = S.u.late.cand[CAP - K + threadIdx.x];  // K <= KMAX <= RT
    __syncthreads();
    if ((int)threadIdx.x < K) S.u.late.cand[threadIdx.x] = v;
    __syncthreads();
    return;
  }
  int np = 1;
  while (np < n) np <<= 1;
  for (int i = n + threadIdx.x; i < np; i += RT) S.u.late.cand[i] = ~0ull;
  __syncthreads();
  for (int size = 2; size <= np; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < np / 2; i += RT) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long a = S.u.late.cand[lo], c = S.u.late.cand[hi];
        if ((a > c) == up) {
          S.u.late.cand[lo] = c;
          S.u.late.cand[hi] = a;
        }
      }
      __syncthreads();
    }
}

// Block-wide exclusive prefix count of `flag` in thread order.
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

// Visit every element of the row: f(index, value).  16-byte loads when the
// row is 16-byte aligned and V is a multiple of 4; each thread keeps ROW_U
// loads in flight before it processes them.
constexpr int ROW_U = 4;
template <class F>
__device__ __forceinline__ void row_loop(const float* zr, int64_t V, bool vec, F&& f) {
  if (vec) {
    const float4* z4 = (const float4*)zr;
    const int64_t n4 = V >> 2;
    for (int64_t base = threadIdx.x; base < n4; base += (int64_t)RT * ROW_U) {
      float4 v[ROW_U];
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * RT;
        v[u] = i < n4 ? z4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * RT;
        if (i < n4) {
          f(4 * i, v[u].x);
          f(4 * i + 1, v[u].y);
          f(4 * i + 2, v[u].z);
          f(4 * i + 3, v[u].w);
        }
      }
    }
  } else {
    for (int64_t base = threadIdx.x; base < V; base += (int64_t)RT * ROW_U) {
      float v[ROW_U];
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * RT;
        v[u] = i < V ? zr[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * RT;
        if (i < V) f(i, v[u]);
      }
    }
  }
}

// Histogram update: one LDS atomic per element and counter (merging runs of
// equal bins per thread cost more in divergent control flow than it saved).
struct HistRun {
  __device__ __forceinline__ void add(int b, unsigned long long m, int* cnt_h, unsigned long long* mass_h) {
    atomicAdd(&cnt_h[b], 1);
    if (mass_h) atomicAdd(&mass_h[b], m);
  }
  __device__ __forceinline__ void flush(int*, unsigned long long*) {}
};

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
  const bool vec = ((V & 3) == 0) && ((((uintptr_t)zr) & 15) == 0);
  // fixed point: a mass term exp(z - edge) <= 1 is stored as round(term * 2^31)
  // (32 bits); sums over a bin are exact 64-bit integers for V < 2^32
  const float fxs = 2147483648.0f;
  const double fxs_inv = 1.0 / 2147483648.0;

  for (int i = tid; i < NB * NCOPY; i += RT) {
    (&S.u.copies.cnt[0][0])[i] = 0;
    (&S.u.copies.mass[0][0])[i] = 0ull;
  }
  for (int i = tid; i < NB; i += RT) S.ref0[i] = bin_upper((uint32_t)i, 11);
  __syncthreads();

  // ---- pass 1: counts and masses of the first 11-bit digit; masses are
  // exp(z - upper edge of the element's bin), so no row maximum is needed.
  {
    const int cp = tid & (NCOPY - 1);
    HistRun run;
    row_loop(zr, V, vec, [&](int64_t, float x) {
      const int b = (int)(fkey(x) >> 21);
      const float ex = __expf(x - S.ref0[b]);
      run.add(b, (unsigned long long)(uint32_t)fmaf(ex, fxs, 0.5f), S.u.copies.cnt[cp], S.u.copies.mass[cp]);
    });
    run.flush(S.u.copies.cnt[cp], S.u.copies.mass[cp]);
  }
  __syncthreads();
  for (int i = tid; i < NB; i += RT) {
    int c = 0;
    unsigned long long m = 0ull;
#pragma unroll
    for (int k = 0; k < NCOPY; ++k) {
      c += S.u.copies.cnt[k][i];
      m += S.u.copies.mass[k][i];
    }
    S.cnt0[i] = c;
    S.mass0[i] = m;
  }
  __syncthreads();
  // logsumexp from the bin masses (fixed reduction order: deterministic)
  {
    float top = -KD_INF;
    for (int bb = tid; bb < NB; bb += RT)
      if (S.mass0[bb] > 0) top = fmaxf(top, S.ref0[bb]);
    top = wave_max(top);
    if ((tid & 63) == 0) S.scan_w[tid >> 6] = (double)top;
    __syncthreads();
    double tmax = S.scan_w[0];
    for (int i = 1; i < RT / 64; ++i) tmax = fmax(tmax, S.scan_w[i]);
    __syncthreads();
    double acc = 0.0;
    for (int bb = tid; bb < NB; bb += RT)
      if (S.mass0[bb] > 0) acc += (double)S.mass0[bb] * fxs_inv * exp((double)S.ref0[bb] - tmax);
    acc = block_sum_d(acc, S);
    if (tid == 0) S.lse = tmax + log(acc);
  }
  find_kth_bin(S, S.cnt0, NB, K);
  const double lse = S.lse;

  // ---- top-K: refine the digit while the K-th element's bin is too big
  uint32_t pre = (uint32_t)S.sel_bin;
  int pbits = 11;
  int above = S.sel_above;
  int eq = S.sel_eq;
  while (above + eq > CAP && pbits < 32) {
    const int dbits = (pbits == 11) ? 11 : 10;
    const int sh = 32 - pbits - dbits;
    for (int i = tid; i < NB; i += RT) S.u.late.cntR[0][i] = 0;
    __syncthreads();
    HistRun run;
    row_loop(zr, V, vec, [&](int64_t, float x) {
      const uint32_t k = fkey(x);
      if ((k >> (32 - pbits)) == pre) run.add((int)((k >> sh) & ((1u << dbits) - 1u)), 0ull, S.u.late.cntR[0], nullptr);
    });
    run.flush(S.u.late.cntR[0], nullptr);
    find_kth_bin(S, S.u.late.cntR[0], 1 << dbits, K - above);
    pre = (pre << dbits) | (uint32_t)S.sel_bin;
    pbits += dbits;
    above += S.sel_above;
    eq = S.sel_eq;
  }
  const bool exact_tail = (above + eq > CAP);  // all 32 key bits tie

  // ---- k_rho: crossing bins of the first digit, from the top
  const float rhos[RHO_MAX] = {rho0, rho1, rho2, rho3, rho4, rho5, rho6, rho7};
  auto mass0_of = [&](int b) {
    return S.mass0[b] > 0 ? (double)S.mass0[b] * fxs_inv * exp((double)S.ref0[b] - lse) : 0.0;
  };
  double total = 0.0;
  if (n_rho > 0) {
    double part = 0.0;
    for (int bb = tid; bb < NB; bb += RT) part += mass0_of(bb);
    total = block_sum_d(part, S);
  }

  for (int g0 = 0; g0 < (n_rho > 0 ? n_rho : 1); g0 += RHO_GROUP) {
    const int ng = (n_rho - g0) < RHO_GROUP ? (n_rho - g0) : RHO_GROUP;
    for (int j = 0; j < ng; ++j) {
      const double target = (double)rhos[g0 + j] * total;
      int bin, ca;
      double ma;
      find_from_top(S, NB, target, mass0_of, [&](int b) { return S.cnt0[b]; }, &bin, &ma, &ca);
      if (tid == 0) {
        S.r_target[j] = target;
        S.r_cum[j] = ma;
        S.r_cnt[j] = bin < 0 ? (int)V : ca;
        S.r_done[j] = bin < 0 ? 1 : 0;
        S.r_pre[j] = (uint32_t)(bin < 0 ? 0 : bin);
      }
      __syncthreads();
    }
    // refinement levels: 11 more bits, then the last 10
    for (int pb = 11; pb < 32;) {
      const int dbits = (pb == 11) ? 11 : 10;
      const int sh = 32 - pb - dbits;
      for (int i = tid; i < NB; i += RT)
        for (int j = 0; j < RHO_GROUP; ++j) {
          S.u.late.cntR[j][i] = 0;
          S.u.late.massR[j][i] = 0ull;
        }
      if (tid == 0 && g0 == 0 && pb == 11) S.ncand = 0;
      __syncthreads();
      uint32_t pj[RHO_GROUP];
      bool act[RHO_GROUP];
      for (int j = 0; j < RHO_GROUP; ++j) {
        act[j] = j < ng && !S.r_done[j];
        pj[j] = S.r_pre[j];
      }
      const bool collect = (g0 == 0 && pb == 11);  // top-K candidates ride on the first refinement pass
      HistRun run[RHO_GROUP];
      row_loop(zr, V, vec, [&](int64_t i, float x) {
        const uint32_t k = fkey(x);
        if (collect) {
          const uint32_t kp = k >> (32 - pbits);
          if (kp > pre || (!exact_tail && kp == pre)) {
            const int slot = atomicAdd(&S.ncand, 1);
            S.u.late.cand[slot] = ((unsigned long long)(~k) << 32) | (unsigned long long)i;
          }
        }
#pragma unroll
        for (int j = 0; j < RHO_GROUP; ++j) {
          if (act[j] && (k >> (32 - pb)) == pj[j]) {
            const int dg = (int)((k >> sh) & ((1u << dbits) - 1u));
            const float ex = __expf(x - bin_upper((pj[j] << dbits) | (uint32_t)dg, pb + dbits));
            run[j].add(dg, (unsigned long long)(uint32_t)fmaf(ex, fxs, 0.5f), S.u.late.cntR[j], S.u.late.massR[j]);
          }
        }
      });
      for (int j = 0; j < RHO_GROUP; ++j) run[j].flush(S.u.late.cntR[j], S.u.late.massR[j]);
      __syncthreads();
      for (int j = 0; j < ng; ++j) {
        if (S.r_done[j]) continue;  // uniform: written by thread 0 before a barrier
        const uint32_t p = S.r_pre[j];
        auto massj = [&](int b) {
          return S.u.late.massR[j][b] > 0 ? (double)S.u.late.massR[j][b] * fxs_inv *
                                         exp((double)bin_upper((p << dbits) | (uint32_t)b, pb + dbits) - lse) : 0.0;
        };
        int bin, ca;
        double ma;
        find_from_top(S, 1 << dbits, S.r_target[j] - S.r_cum[j], massj, [&](int b) { return S.u.late.cntR[j][b]; }, &bin,
                      &ma, &ca);
        if (bin < 0) bin = 0;  // rounding: the crossing is in this bin's lowest digit
        if (tid == 0) {
          const double cum = S.r_cum[j] + ma;
          const int cnt = S.r_cnt[j] + ca;
          if (pb + dbits == 32) {
            // all elements of the final bin share one key, hence one mass
            const int nbin = S.u.late.cntR[j][bin];
            const double each = exp((double)bin_upper((p << dbits) | (uint32_t)bin, 32) - lse);
            long long jn = each > 0.0 ? (long long)ceil((S.r_target[j] - cum) / each) : (long long)nbin;
            if (jn < 1) jn = 1;
            if (jn > nbin) jn = nbin;
            S.r_cnt[j] = cnt + (int)jn;
            S.r_done[j] = 1;
          } else {
            S.r_cum[j] = cum;
            S.r_cnt[j] = cnt;
            S.r_pre[j] = (p << dbits) | (uint32_t)bin;
          }
        }
        __syncthreads();
      }
      pb += dbits;
      if (n_rho == 0) break;  // the pass only collected the top-K candidates
    }
    if (tid == 0)
      for (int j = 0; j < ng; ++j) krho_out[row * n_rho + g0 + j] = S.r_cnt[j];
    __syncthreads();
  }

  int nc = S.ncand;
  if (exact_tail) {
    // all remaining ties share one key: take the lowest indices, in order
    int need = K - nc;
    for (int64_t base = 0; base < V && need > 0; base += RT) {
      const int64_t i = base + tid;
      const bool f = (i < V) && (fkey(zr[i]) == pre);
      int tot;
      const int r = block_rank(f, S, &tot);
      if (f && r < need) S.u.late.cand[nc + r] = ((unsigned long long)(~pre) << 32) | (unsigned long long)i;
      const int took = tot < need ? tot : need;
      nc += took;
      need -= took;
      __syncthreads();
    }
  }
  sort_cand(S, nc, K);

  double kept = 0.0;
  for (int k = tid; k < K; k += RT) {
    const int64_t i = (int64_t)(S.u.late.cand[k] & 0xffffffffull);
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
    KD_LAUNCH(k_cache_gemm, dim3(grid), dim3(CC::NT), CG_LDS, s, (const bf16_t*)g + t0 * d,
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
