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
// Row pass, one workgroup per row, in two kernels:
//   k_topk_rows (fast)  value bins of width 1/512 below the row maximum (the
//      maximum, and a lower bound of the K-th largest value, come from the
//      GEMM epilogue's per-tile maxima, or from a first streaming read); one
//      streaming read builds packed (count, fixed-point mass) bins, whose
//      exact integer prefix sums give logsumexp and each rho's crossing bin,
//      and collects the top-K candidates; a crossing bin whose count and mass
//      do not pin k_rho is collected by a second read and ordered exactly in
//      LDS.  Rows it cannot finish are flagged.
//   k_topk_rows_exact  for the flagged rows (or every row when V >= 2^18):
//      radix digits of order-preserving keys, refined until exact:
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

#include <mutex>

#include "../../include/kdtopk.h"
#include "gemm.h"
#include "kd_internal.h"

// Scratch of kd_topk_rows_noalloc: one fallback flag per row, for callers
// that cannot allocate.  Each device holds its own copy until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// returns for that device.
constexpr int64_t KD_NOALLOC_ROWS = (int64_t)1 << 20;
static __device__ __align__(256) int32_t scratch[KD_NOALLOC_ROWS];

namespace {

using CC = GemmCfg;
constexpr int RT = 1024;      // threads of the row kernel
// Row flags set by the fast kernel: done, for the exact kernel, crossing
// bins deferred (collected by k_rows_cross, ranked by the exact kernel's
// launch).
constexpr int F_DONE = 0, F_EXACT = 1, F_DEFER = 2;
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
// bias added: 1 KB of contiguous z per wavefront store.  The maximum of each
// token row of the tile goes to tmax[t][vt] (the row pass starts from it).
constexpr int CG_LDS = (CC::BN / 2) * CC::BM * 4;  // 128 tokens x 256 vocabulary fp32
static_assert(CG_LDS >= GEMM_LDS, "epilogue staging reuses the operand stages");

__device__ __forceinline__ int cg_swz(int tl) { return (tl & 31) << 1; }

// Maximum over the wavefront without LDS traffic: rotations within each
// 16-lane row (DPP row_ror 1, 2, 4, 8), then the four row results read as
// scalars.  Every lane returns the maximum.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__global__ __launch_bounds__(256, 1) void k_cache_gemm(const bf16_t* __restrict__ g, const bf16_t* __restrict__ U,
                                                       const float* __restrict__ b, int64_t Tb, int64_t d,
                                                       int64_t V, int nTT, int nVT, float* __restrict__ z,
                                                       float* __restrict__ tmax) {
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
      float m = -KD_INF;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v + e < V) m = fmaxf(m, x[e]);
      m = wave_max_dpp(m);  // the wavefront holds the token row's 256 values
      if (t < Tb && lane == 0) tmax[t * nVT + vt] = m;
      if (t < Tb) {
        float* dst = z + t * V + v;
        if (vec) {
          // streamed past the caches: the block (1.2 GB at 2048 tokens) is far
          // larger than them, and the row pass then reads clean memory instead
          // of competing with the write-back of dirty lines
          __builtin_nontemporal_store(x, (f32x4*)dst);
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

constexpr int RF = 512;                        // threads of the fast row kernel

// Deferred crossing bins.  A row whose top-K is settled but whose k_rho for
// some target is not pinned by its crossing bin's count and mass is handed
// to k_rows_cross instead of being read again by its own workgroup (which
// would hold its CU past the other rows): the state below, and up to CAPX
// elements of the crossing bin per (row, target) in the candidate buffer.
constexpr int CAPX = 512;   // crossing-bin elements per (row, target)
constexpr int NSX = 16;     // slices of one deferred row
constexpr int XL = 4096;    // rows per k_rows_cross launch
constexpr int XG = 768;     // workgroups of k_rows_cross (three per CU)
struct CrossRow {
  double lse;
  double base[RHO_MAX];     // mass above the crossing bin / total
  float zmax;
  int pad;
  int b[RHO_MAX];           // crossing bin, -1 when resolved
  int n[RHO_MAX];           // elements in it
  int above[RHO_MAX];       // elements above it
  int fill[RHO_MAX];        // elements collected so far
  float rho[RHO_MAX];
};

// Sort key: ascending order = value descending, then index ascending.
__device__ __forceinline__ unsigned long long cand_key(float x, int64_t i) {
  return ((unsigned long long)(~fkey(x)) << 32) | (unsigned long long)i;
}
__device__ __forceinline__ float cand_value(unsigned long long c) {
  const uint32_t k = ~(uint32_t)(c >> 32);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// k_rho inside a crossing bin: the bin's n candidates (keys, unordered) are
// ranked by (value desc, index asc), their masses exp(z - lse) stored by rank
// in m[], and the first rank r where base0 + the masses of ranks 0..r
// reaches target is returned (n when none).  Thread t of RF adds ranks
// [t*per, t*per + per) (per = ceil(n / RF)), the thread totals combine in
// thread order (a wavefront scan, then the wavefronts in order): the sums,
// hence the result, depend only on the candidates.  Both row kernels use it.
__device__ __forceinline__ int crossing_rank(const unsigned long long* keys, int n, double lse, double base0,
                                             double target, double* m, double* red_d, int* red_i) {
  const int tid = threadIdx.x;
  const bool act = tid < RF;  // a larger block: its threads past RF only pass the barriers
  for (int p = tid; act && p < n; p += RF) {
    const unsigned long long mine = keys[p];
    int r = 0;
#pragma unroll 8
    for (int q = 0; q < n; ++q) r += (keys[q] < mine) ? 1 : 0;
    m[r] = exp((double)cand_value(mine) - lse);
  }
  __syncthreads();
  const int per = (n + RF - 1) / RF;
  const int r0 = act ? tid * per : n, r1 = min(n, r0 + per);
  double own_sum = 0.0;
  for (int r = r0; r < r1; ++r) own_sum += m[r];
  double x = own_sum;
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(x, o, 64);
    if (lane >= o) x += t;
  }
  if (act && lane == 63) red_d[w] = x;
  __syncthreads();
  double base = base0 + (x - own_sum);
  for (int i = 0; act && i < w; ++i) base += red_d[i];
  __syncthreads();
  int hit = n;
  for (int r = r0; r < r1; ++r) {
    base += m[r];
    if (base >= target) {
      hit = r;
      break;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) hit = min(hit, __shfl_xor(hit, o, 64));
  if (act && lane == 0) red_i[w] = hit;
  __syncthreads();
  int h = red_i[0];
  for (int i = 1; i < RF / 64; ++i) h = min(h, red_i[i]);
  __syncthreads();
  return h;
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
  float ref0[NB];                               // reference of each level-0 bin (bin_ref)
  int cnt0[NB];                                 // level-0 counts
  unsigned long long mass0[NB];                 // level-0 fixed-point masses, each vs its bin's reference
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
  float zref;                                   // the row maximum (FLT_MAX when it is not finite)
};

// Largest float whose key has prefix `p` in its top `bits` bits: the upper
// edge of a histogram bin.  Clamped to FLT_MAX for bins above the finite range.
__device__ __forceinline__ float bin_upper(uint32_t p, int bits) {
  const uint32_t k = (bits == 32) ? p : ((p << (32 - bits)) | ((1u << (32 - bits)) - 1u));
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  const float f = __uint_as_float(u);
  return (f != f || f > 3.4028234663852886e38f) ? 3.4028234663852886e38f : f;
}

// Reference of a bin's fixed-point masses: its upper edge, capped at the row
// maximum.  Every element of the bin is <= it, so each mass exp(z - ref) is
// <= 1; and since ref <= zmax, rounding a mass to 2^-F costs at most 2^-F of
// exp(zmax) however wide the bin is (the first digit's bins are 32 wide for
// values in [128, 256): against the bare edge, the row maximum itself could
// sit 32 below it and keep only a few bits).
__device__ __forceinline__ float bin_ref(uint32_t p, int bits, float zref) { return fminf(bin_upper(p, bits), zref); }

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

// Visit every element of the row with NT threads: f(index, value).  16-byte
// loads when the row is 16-byte aligned and V is a multiple of 4; each thread
// keeps ROW_U loads in flight before it processes them.
constexpr int ROW_U = 4;
template <int NT, class F>
__device__ __forceinline__ void row_loop(const float* zr, int64_t V, bool vec, F&& f) {
  if (vec) {
    const float4* z4 = (const float4*)zr;
    const int64_t n4 = V >> 2;
    for (int64_t base = threadIdx.x; base < n4; base += (int64_t)NT * ROW_U) {
      float4 v[ROW_U];
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * NT;
        v[u] = i < n4 ? z4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * NT;
        if (i < n4) {
          f(4 * i, v[u].x);
          f(4 * i + 1, v[u].y);
          f(4 * i + 2, v[u].z);
          f(4 * i + 3, v[u].w);
        }
      }
    }
  } else {
    for (int64_t base = threadIdx.x; base < V; base += (int64_t)NT * ROW_U) {
      float v[ROW_U];
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * NT;
        v[u] = i < V ? zr[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * NT;
        if (i < V) f(i, v[u]);
      }
    }
  }
}

// Software-pipelined variant for the fast row pass: batch b + 1 (ROW_U
// 16-byte loads per thread, indices clamped into the row so every load is
// issued unconditionally) is in flight while batch b is processed.
// f(index, value, e) sees each valid element, e = its slot 0..4*ROW_U-1 in
// the thread's batch; g(base, vec) runs after each batch, where the element
// of slot e has index 4*(base + (e/4)*NT) + e%4 (vec) or base + e*NT.
template <int NT, class F, class G>
__device__ __forceinline__ void row_loop_pipe(const float* zr, int64_t V, bool vec, F&& f, G&& g) {
  if (vec) {
    const float4* z4 = (const float4*)zr;
    const int64_t n4 = V >> 2, last = n4 - 1;
    const int64_t step = (int64_t)NT * ROW_U;
    const int64_t iters = (n4 + step - 1) / step;
    float4 cur[ROW_U];
#pragma unroll
    for (int u = 0; u < ROW_U; ++u) {
      const int64_t i = threadIdx.x + (int64_t)u * NT;
      cur[u] = z4[i < last ? i : last];
    }
    for (int64_t it = 0; it < iters; ++it) {
      const int64_t base = threadIdx.x + it * step;
      float4 nxt[ROW_U];
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + step + (int64_t)u * NT;
        nxt[u] = z4[i < last ? i : last];
      }
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) {
        const int64_t i = base + (int64_t)u * NT;
        if (i < n4) {
          f(4 * i, cur[u].x, 4 * u);
          f(4 * i + 1, cur[u].y, 4 * u + 1);
          f(4 * i + 2, cur[u].z, 4 * u + 2);
          f(4 * i + 3, cur[u].w, 4 * u + 3);
        }
      }
      g(base, true);
#pragma unroll
      for (int u = 0; u < ROW_U; ++u) cur[u] = nxt[u];
    }
  } else {
    constexpr int U = 4 * ROW_U;
    const int64_t last = V - 1;
    const int64_t step = (int64_t)NT * U;
    const int64_t iters = (V + step - 1) / step;
    float cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = threadIdx.x + (int64_t)u * NT;
      cur[u] = zr[i < last ? i : last];
    }
    for (int64_t it = 0; it < iters; ++it) {
      const int64_t base = threadIdx.x + it * step;
      float nxt[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + step + (int64_t)u * NT;
        nxt[u] = zr[i < last ? i : last];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * NT;
        if (i < V) f(i, cur[u], u);
      }
      g(base, false);
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
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

// Exact row pass for the rows the fast pass flagged (F_EXACT, F_DEFER_EXACT), or
// for every row when flags is NULL.
__global__ __launch_bounds__(RT) void k_topk_rows_exact(const float* __restrict__ z, int64_t ldz, int64_t V, int K,
                                                        int n_rho, float rho0, float rho1, float rho2, float rho3,
                                                        float rho4, float rho5, float rho6, float rho7,
                                                        const int32_t* __restrict__ flags,
                                                        int32_t* __restrict__ idx_out, float* __restrict__ val_out,
                                                        float* __restrict__ lse_out, float* __restrict__ mq_out,
                                                        int32_t* __restrict__ krho_out, float* __restrict__ logp_out,
                                                        const CrossRow* __restrict__ cross,
                                                        const unsigned long long* __restrict__ xcand) {
  __shared__ RowShared S;
  const int64_t row = blockIdx.x;
  if (flags != nullptr) {
    const int f = flags[row];
    if (f == F_DEFER && cross != nullptr) {
      // the fast kernel's deferred crossing bins: rank each one's elements
      // (collected by k_rows_cross); a count that does not match the
      // histogram's falls through to the exact pass of the whole row
      const CrossRow& c = cross[row];
      bool ok = true;
      for (int j = 0; j < n_rho; ++j)
        if (c.b[j] >= 0 && (c.fill[j] != c.n[j] || c.n[j] > CAPX || c.n[j] < 1)) ok = false;
      if (ok) {
        unsigned long long* keys = (unsigned long long*)&S.u;
        double* mass = (double*)&S.u + CAPX;
        for (int j = 0; j < n_rho; ++j) {
          if (c.b[j] < 0) continue;
          const int n = c.n[j];
          for (int p = threadIdx.x; p < n; p += RT) keys[p] = xcand[(row * n_rho + j) * CAPX + p];
          __syncthreads();
          const int hit = crossing_rank(keys, n, c.lse, c.base[j], (double)c.rho[j], mass, S.red_d, S.scan_i);
          if (threadIdx.x == 0) krho_out[row * n_rho + j] = c.above[j] + (hit < n ? hit + 1 : n);
        }
        return;
      }
    } else if (f != F_EXACT) {
      return;
    }
  }
  const float* zr = z + row * ldz;
  const int tid = threadIdx.x;
  const bool vec = ((V & 3) == 0) && ((((uintptr_t)zr) & 15) == 0);
  // fixed point: a mass term exp(z - ref) <= 1, ref the bin's reference
  // (bin_ref), is stored as round(term * 2^F) with F = 62 - bits(V), so the
  // sums over a bin stay exact 64-bit integers
  const int fx_bits = 62 - (64 - __clzll((unsigned long long)V));
  const double fxs = ldexp(1.0, fx_bits);
  const double fxs_inv = ldexp(1.0, -fx_bits);

  // ---- pass 0: the row maximum, which caps the bins' references
  {
    float mx = -KD_INF;
    row_loop<RT>(zr, V, vec, [&](int64_t, float x) { mx = fmaxf(mx, x); });
    mx = wave_max(mx);
    if ((tid & 63) == 0) S.scan_w[tid >> 6] = (double)mx;
    __syncthreads();
    if (tid == 0) {
      double m = S.scan_w[0];
      for (int i = 1; i < RT / 64; ++i) m = fmax(m, S.scan_w[i]);
      S.zref = (fabs(m) <= 3.4028234663852886e38) ? (float)m : 3.4028234663852886e38f;
    }
  }
  for (int i = tid; i < NB * NCOPY; i += RT) {
    (&S.u.copies.cnt[0][0])[i] = 0;
    (&S.u.copies.mass[0][0])[i] = 0ull;
  }
  __syncthreads();
  const float zref = S.zref;
  for (int i = tid; i < NB; i += RT) S.ref0[i] = bin_ref((uint32_t)i, 11, zref);
  __syncthreads();

  // ---- pass 1: counts and masses of the first 11-bit digit; masses are
  // exp(z - reference of the element's bin).
  {
    const int cp = tid & (NCOPY - 1);
    HistRun run;
    row_loop<RT>(zr, V, vec, [&](int64_t, float x) {
      const int b = (int)(fkey(x) >> 21);
      const float ex = __expf(x - S.ref0[b]);
      run.add(b, __double2ull_rn((double)ex * fxs), S.u.copies.cnt[cp], S.u.copies.mass[cp]);
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
    row_loop<RT>(zr, V, vec, [&](int64_t, float x) {
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
      row_loop<RT>(zr, V, vec, [&](int64_t i, float x) {
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
            const float ex = __expf(x - bin_ref((pj[j] << dbits) | (uint32_t)dg, pb + dbits, zref));
            run[j].add(dg, __double2ull_rn((double)ex * fxs), S.u.late.cntR[j], S.u.late.massR[j]);
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
                                         exp((double)bin_ref((p << dbits) | (uint32_t)b, pb + dbits, zref) - lse) : 0.0;
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
    if (logp_out != nullptr) logp_out[row * K + k] = (float)((double)x - lse);
    kept += exp((double)x - lse);
  }
  kept = block_sum_d(kept, S);
  if (tid == 0) {
    lse_out[row] = (float)lse;
    mq_out[row] = (float)(1.0 - kept);
  }
}

// ---------------------------------------------------------------------------
// Fast row pass: one workgroup of RF threads per row, up to three streaming
// reads of the row (one when the producer's tile maxima are given and every
// k_rho is pinned by its bin).
//   A  the row maximum zmax and a lower bound tau of the K-th largest value
//      (K distinct elements are >= it): from the producer's per-tile maxima,
//      or from a read of the row and the threads' maxima;
//   B  a histogram over NBL value bins below zmax, bin b holding the values
//      with floor(512 (zmax - z)) = b (the last bin also everything lower),
//      and the elements >= tau (the top-K candidates).  A bin packs its
//      count (bits 46..63) and the sum of round(2^23 exp(z - e_b)),
//      e_b = zmax - b/512 its upper edge, into one 64-bit word: one LDS
//      atomic per element, integer sums independent of the atomic order.
//      The bin masses, rescaled to a common 2^-44 fixed point relative to
//      exp(zmax), give logsumexp, the bin of the K-th largest value and, per
//      rho, the bin where the mass accumulated from the top reaches rho of
//      the total (exact integer prefix sums).  Without k_rho targets no
//      histogram is built: the read sums exp(z - zmax) instead;
//   C  only for what B left open: the elements of a crossing bin whose count
//      and mass do not pin k_rho (and of the bins down to the K-th one when
//      the candidates were not collected), ordered in LDS by
//      (value desc, index asc): the top-K and each k_rho follow exactly.
// The bin of a value is a monotone function of it, so equal values share a
// bin and every bin above another holds only larger values.  Rows this path
// cannot finish (non-finite maximum, too many candidates, a crossing in the
// lowest bin) are flagged for k_topk_rows_exact.
// ---------------------------------------------------------------------------
constexpr int NBL = 8192;                      // value bins
constexpr int BPT = NBL / RF;                  // bins per thread in the scans
constexpr float BIN_INVW = 512.f;              // bins per unit of logit (NBL bins cover 16 below the maximum)
constexpr float BIN_W = 1.f / 512.f;
constexpr int CAPK = 1536;                     // top-K candidates
constexpr int CAPR = 2048;                     // crossing-bin candidates, all targets
constexpr int CNT_SHIFT = 46;
constexpr unsigned long long MASS_MASK = (1ull << CNT_SHIFT) - 1ull;
constexpr int64_t VFAST_MAX = ((int64_t)1 << 18) - 1;  // bin counts fit 18 bits

struct FastShared {
  union {
    unsigned long long hist[NBL];  // pass B and the scans
    struct {
      unsigned long long poolR[CAPR];  // crossing-bin candidates (pass C)
      double m[CAPR];                  // candidate masses by rank
    } c;
  } u;
  unsigned long long poolK[CAPK];  // ((~key) << 32) | index
  unsigned long long scan_m[RF / 64];
  int scan_c[RF / 64];
  double red_d[RF / 64];
  float red_f[RF / 64];
  int red_i[RF / 64];
  unsigned long long total_q;
  float tau;                       // lower bound of the K-th largest value (single-pass collection)
  int tau_ok, tau_b;
  int bK, aboveK, nbK, fillK;
  int bR[RHO_MAX], cntAboveR[RHO_MAX], nR[RHO_MAX], fillR[RHO_MAX], segR[RHO_MAX];
  unsigned long long massAboveR[RHO_MAX], massR[RHO_MAX];
  int kres[RHO_MAX];               // k_rho resolved from the histogram alone (0: not resolved)
  float rho[RHO_MAX];
};
static_assert(sizeof(FastShared) <= 80 * 1024, "two rows per CU");


// Value bin of x below the row maximum: monotone non-increasing in x
// (rounded subtraction, exact scaling by 512); -inf goes to the last bin.
__device__ __forceinline__ int vbin(float x, float zmax) {
  return (int)fminf(fmaxf((zmax - x) * BIN_INVW, 0.f), (float)(NBL - 1));  // in [0, NBL) for any input
}
// Upper edge of bin b, rounded once (b / 512 is exact).
__device__ __forceinline__ float vedge(int b, float zmax) { return fmaf(-(float)b, BIN_W, zmax); }

__device__ __forceinline__ float fast_block_max(float v, FastShared& S) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) S.red_f[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = S.red_f[0];
  for (int i = 1; i < RF / 64; ++i) r = fmaxf(r, S.red_f[i]);
  __syncthreads();
  return r;
}

// Sum in a fixed order (per thread, then the wavefront tree, then the waves
// in order): deterministic for a fixed assignment of terms to threads.
__device__ __forceinline__ double fast_block_sum(double v, FastShared& S) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) S.red_d[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < RF / 64; ++i) r += S.red_d[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int fast_block_min(int v, FastShared& S) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) S.red_i[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = S.red_i[0];
  for (int i = 1; i < RF / 64; ++i) r = min(r, S.red_i[i]);
  __syncthreads();
  return r;
}

// Exclusive prefix over threads (thread order) of (m, c); integer sums, so
// the result does not depend on the order of the additions.
__device__ __forceinline__ void fast_excl_scan(unsigned long long m, int c, FastShared& S, unsigned long long& em,
                                               int& ec, unsigned long long& tm, int& tc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned long long x = m;
  int y = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long tx = __shfl_up(x, o, 64);
    const int ty = __shfl_up(y, o, 64);
    if (lane >= o) {
      x += tx;
      y += ty;
    }
  }
  if (lane == 63) {
    S.scan_m[w] = x;
    S.scan_c[w] = y;
  }
  __syncthreads();
  unsigned long long om = 0ull, all_m = 0ull;
  int oc = 0, all_c = 0;
  for (int i = 0; i < RF / 64; ++i) {
    if (i < w) {
      om += S.scan_m[i];
      oc += S.scan_c[i];
    }
    all_m += S.scan_m[i];
    all_c += S.scan_c[i];
  }
  __syncthreads();
  em = om + x - m;
  ec = oc + y - c;
  tm = all_m;
  tc = all_c;
}



// Top K of the nKc candidates in S.poolK (every element ranked above a
// candidate is a candidate): rank by key, write idx / val, and lse and the
// tail mass 1 - sum over the top K of exp(z - lse).
__device__ __forceinline__ void fast_emit_topk(FastShared& S, int nKc, int K, const float* zr, int64_t row,
                                               double lse, int32_t* idx_out, float* val_out, float* lse_out,
                                               float* mq_out, float* logp_out) {
  const int tid = threadIdx.x;
  for (int p = tid; p < nKc; p += RF) {
    const unsigned long long mine = S.poolK[p];
    int r = 0;
#pragma unroll 8
    for (int q = 0; q < nKc; ++q) r += (S.poolK[q] < mine) ? 1 : 0;
    if (r < K) {
      const int64_t i = (int64_t)(mine & 0xffffffffull);
      const float x = zr[i];  // the stored value keeps its bits (-0.0)
      idx_out[row * K + r] = (int32_t)i;
      val_out[row * K + r] = x;
      if (logp_out != nullptr) logp_out[row * K + r] = (float)((double)x - lse);
      S.u.c.m[r] = exp((double)x - lse);
    }
  }
  __syncthreads();
  double kept = 0.0;
  for (int r = tid; r < K; r += RF) kept += S.u.c.m[r];
  kept = fast_block_sum(kept, S);
  if (tid == 0) {
    lse_out[row] = (float)lse;
    mq_out[row] = (float)(1.0 - kept);
  }
}

// Lower bound tau of the K-th largest value of a row from n partial maxima
// a[] (each the maximum of a disjoint part of the row, so n distinct
// elements): the maxima are counted in TAU_NB bins of width 1/16 below the
// row maximum, b is the bin where the count from the top reaches K, and tau
// is the smallest maximum in bins 0..b.  At least K maxima, hence K distinct
// elements of the row, are >= tau; it lies at most one bin below the maximum
// of rank K.  a[] is in LDS (n <= NBL values, the counts after them);
// S.tau_ok stays 0 when fewer than K of the maxima are numbers.
constexpr int TAU_NB = 512;
__device__ __forceinline__ int tau_bin(float x, float zmax) {
  return (int)fminf(fmaxf((zmax - x) * 16.f, 0.f), (float)(TAU_NB - 1));
}

// S.tau_b = the first of TAU_NB bins where the count from bin 0 reaches K
// (-1 when the counts sum to less): wavefront 0 scans, 8 bins per lane.
__device__ __forceinline__ void tau_crossing(const int* cnt, int K, FastShared& S) {
  const int tid = threadIdx.x;
  if (tid >= 64) return;
  constexpr int PER = TAU_NB / 64;
  int c[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = cnt[tid * PER + i];
    sum += c[i];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (tid >= o) incl += y;
  }
  int run = incl - sum;
  if (run < K && incl >= K) {  // this lane holds the crossing
    int b = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      run += c[i];
      if (b < 0 && run >= K) b = tid * PER + i;
    }
    S.tau_b = b;
  }
}

__device__ __forceinline__ void fast_tau(const float* a, int n, int K, float zmax, FastShared& S) {
  int* cnt = (int*)(S.u.hist + NBL / 2);
  const int tid = threadIdx.x;
  for (int i = tid; i < TAU_NB; i += RF) cnt[i] = 0;
  if (tid == 0) {
    S.tau_ok = 0;
    S.tau_b = -1;
  }
  __syncthreads();
  if (n >= K)
    for (int p = tid; p < n; p += RF) {
      const float x = a[p];
      if (x == x) atomicAdd(&cnt[tau_bin(x, zmax)], 1);
    }
  __syncthreads();
  if (n >= K) tau_crossing(cnt, K, S);
  __syncthreads();
  const int b = S.tau_b;
  float m = KD_INF;
  if (b >= 0)
    for (int p = tid; p < n; p += RF) {
      const float x = a[p];
      if (x == x && tau_bin(x, zmax) <= b) m = fminf(m, x);
    }
  m = -fast_block_max(-m, S);
  if (b >= 0 && tid == 0) {
    S.tau = m;
    S.tau_ok = 1;
  }
  __syncthreads();
}

// Trims the top-K candidate pool (the nKc elements >= tau) to the elements
// in or above the bin of the K-th largest one, TAU_NB bins spanning
// [tau, zmax].  The bin is monotone in the value, so the first bin where the
// count from the top reaches K is that element's bin and the kept ones
// include every element >= it: about K of them are ranked instead of nKc.
// Returns the new count (nKc when there is little to trim).
__device__ __forceinline__ int fast_trim_pool(FastShared& S, int nKc, int K, float zmax, float tau) {
  const float span = zmax - tau;
  if (nKc <= K + 32 || !(span > 0.f) || !(span < KD_INF)) return nKc;
  const float inv = (float)TAU_NB / span;
  int* cnt = (int*)(S.u.hist + NBL / 2);
  const int tid = threadIdx.x;
  for (int i = tid; i < TAU_NB; i += RF) cnt[i] = 0;
  if (tid == 0) S.tau_b = -1;
  __syncthreads();
  constexpr int PT = (CAPK + RF - 1) / RF;
  unsigned long long c[PT];
  int bb[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int p = tid + i * RF;
    c[i] = 0ull;
    bb[i] = TAU_NB;
    if (p < nKc) {
      c[i] = S.poolK[p];
      bb[i] = (int)fminf(fmaxf((zmax - cand_value(c[i])) * inv, 0.f), (float)(TAU_NB - 1));
      atomicAdd(&cnt[bb[i]], 1);
    }
  }
  __syncthreads();
  tau_crossing(cnt, K, S);
  if (tid == 0) S.fillK = 0;
  __syncthreads();
  const int b = S.tau_b;
  if (b < 0) return nKc;  // cannot happen with nKc >= K numbers; the pool is untouched
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if (bb[i] <= b) S.poolK[atomicAdd(&S.fillK, 1)] = c[i];
  __syncthreads();
  return S.fillK;
}

__global__ __launch_bounds__(RF) __attribute__((amdgpu_waves_per_eu(4))) void k_topk_rows(const float* __restrict__ z, int64_t ldz, int64_t V, int K,
                                                  int n_rho, float rho0, float rho1, float rho2, float rho3,
                                                  float rho4, float rho5, float rho6, float rho7,
                                                  const float* __restrict__ tmax, int n_tmax,
                                                  int32_t* __restrict__ flags, int32_t* __restrict__ idx_out,
                                                  float* __restrict__ val_out, float* __restrict__ lse_out,
                                                  float* __restrict__ mq_out, int32_t* __restrict__ krho_out,
                                                  float* __restrict__ logp_out, CrossRow* __restrict__ cross) {
  __shared__ FastShared S;
  const int64_t row = blockIdx.x;
  const float* zr = z + row * ldz;
  const int tid = threadIdx.x;
  const bool vec = ((V & 3) == 0) && ((((uintptr_t)zr) & 15) == 0);
  const float rhos[RHO_MAX] = {rho0, rho1, rho2, rho3, rho4, rho5, rho6, rho7};

  // ---- A: the row maximum (from the producer's per-tile maxima when given)
  float mx = -KD_INF;
  if (tmax != nullptr) {
    for (int p = tid; p < n_tmax; p += RF) mx = fmaxf(mx, tmax[row * n_tmax + p]);
  } else {
    row_loop_pipe<RF>(zr, V, vec, [&](int64_t, float x, int) { mx = fmaxf(mx, x); }, [](int64_t, bool) {});
  }
  const float zmax = fast_block_max(mx, S);
  if (!(fabsf(zmax) <= 3.4028234663852886e38f)) {  // all -inf, +inf present, or NaN only
    if (tid == 0) flags[row] = F_EXACT;
    return;
  }
  // The top-K candidates are collected during pass B already: every element
  // >= tau, a lower bound of the K-th largest value (from the producer's
  // tile maxima or the threads' maxima of pass A).
  float tau = 0.f;
  bool collectK = false;
  {
    float* a = (float*)S.u.hist;
    int n;
    if (tmax != nullptr) {
      n = n_tmax <= NBL ? n_tmax : 0;
      for (int p = tid; p < n; p += RF) a[p] = tmax[row * n_tmax + p];
    } else {
      n = RF;
      a[tid] = mx;
    }
    __syncthreads();
    fast_tau(a, n, K, zmax, S);
    collectK = S.tau_ok != 0;
    tau = S.tau;
    if (tid == 0) S.fillK = 0;
    __syncthreads();  // a[] is overwritten by the histogram below
  }

  if (n_rho == 0 && collectK) {
    // ---- B': one read: the exponential sum (fp64 per thread, then the fixed
    // block order: deterministic) and the elements >= tau.  The top K are
    // among them; more than CAPK of them (a huge tie) sends the row to the
    // exact kernel.
    double acc = 0.0;
    row_loop_pipe<RF>(
        zr, V, vec,
        [&](int64_t i, float x, int) {
          acc += (double)__builtin_amdgcn_exp2f((x - zmax) * KD_LOG2E);
          if (x >= tau) {
            const int slot = atomicAdd(&S.fillK, 1);
            if (slot < CAPK) S.poolK[slot] = cand_key(x, i);
          }
        },
        [](int64_t, bool) {});
    const double total = fast_block_sum(acc, S);  // its barriers also complete the pool
    const int nKc = S.fillK;
    if (nKc < K || nKc > CAPK) {
      if (tid == 0) flags[row] = F_EXACT;
      return;
    }
    if (tid == 0) flags[row] = F_DONE;
    const int nKt = fast_trim_pool(S, nKc, K, zmax, tau);
    fast_emit_topk(S, nKt, K, zr, row, (double)zmax + log(total), idx_out, val_out, lse_out, mq_out, logp_out);
    return;
  }

  // ---- B: packed (count, fixed-point mass) histogram of the value bins,
  // and the elements >= tau
  for (int i = tid; i < NBL; i += RF) S.u.hist[i] = 0ull;
  __syncthreads();
  row_loop_pipe<RF>(
      zr, V, vec,
      [&](int64_t i, float x, int) {
        const int b = vbin(x, zmax);
        const float m = __builtin_amdgcn_exp2f((x - vedge(b, zmax)) * KD_LOG2E);
        const unsigned long long w = (1ull << CNT_SHIFT) | (unsigned long long)(uint32_t)fmaf(m, 8388608.f, 0.5f);
        atomicAdd(&S.u.hist[b], w);
        if (collectK && x >= tau) {
          const int slot = atomicAdd(&S.fillK, 1);
          if (slot < CAPK) S.poolK[slot] = cand_key(x, i);
        }
      },
      [](int64_t, bool) {});
  __syncthreads();

  // bins [tid*BPT, tid*BPT + BPT) per thread: masses in 2^-44 units of exp(zmax)
  unsigned long long bm[BPT];
  int bc[BPT];
  unsigned long long tm = 0ull;
  int tc = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int b = tid * BPT + i;
    const unsigned long long w = S.u.hist[b];
    const unsigned long long fix = w & MASS_MASK;
    bc[i] = (int)(w >> CNT_SHIFT);
    bm[i] = fix ? (unsigned long long)__double2ll_rn((double)fix * 2097152.0 *
                                                      exp((double)vedge(b, zmax) - (double)zmax))
                : 0ull;
    tm += bm[i];
    tc += bc[i];
  }
  unsigned long long em, total;
  int ec, ctot;
  fast_excl_scan(tm, tc, S, em, ec, total, ctot);
  const double lse = (double)zmax + log((double)total * 5.684341886080802e-14);  // 2^-44
  unsigned long long tq[RHO_MAX];
#pragma unroll
  for (int j = 0; j < RHO_MAX; ++j) {
    double t = ceil((double)rhos[j] * (double)total);
    unsigned long long q = (unsigned long long)t;
    tq[j] = (j < n_rho) ? (q < total ? (q > 0ull ? q : 1ull) : total) : ~0ull;
  }
  if (tid == 0) {
    S.bK = -1;
#pragma unroll
    for (int j = 0; j < RHO_MAX; ++j) {
      S.bR[j] = -1;
      S.rho[j] = rhos[j];
    }
  }
  __syncthreads();
  {
    unsigned long long cm = em;
    int cc = ec;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int b = tid * BPT + i;
      const unsigned long long nm = cm + bm[i];
      const int nc = cc + bc[i];
      if (cc < K && nc >= K) {
        S.bK = b;
        S.aboveK = cc;
        S.nbK = bc[i];
      }
#pragma unroll
      for (int j = 0; j < RHO_MAX; ++j)
        if (j < n_rho && cm < tq[j] && nm >= tq[j]) {
          S.bR[j] = b;
          S.cntAboveR[j] = cc;
          S.massAboveR[j] = cm;
          S.massR[j] = bm[i];
          S.nR[j] = bc[i];
        }
      cm = nm;
      cc = nc;
    }
  }
  __syncthreads();
  // k_rho from the crossing bin's (count, mass) when that pins it: with
  // R = rho - (mass above the bin) and the bin's n masses in
  // [m_lo, m_hi] (its edges) summing to M, the top i of them sum to at most
  // min(i m_hi, M - (n - i) m_lo) and at least i M / n, so the first i whose
  // partial sum reaches R lies in [i_lo, i_hi]; equal bounds give it without
  // looking at the bin's elements.  (1e-6 relative margins cover the
  // rounding of the fixed-point masses and of the bin edges.)
  if (tid < n_rho) {
    const int j = tid;
    int kr = 0;
    const int b = S.bR[j], n = S.nR[j];
    if (b >= 0 && b < NBL - 1 && n > 0) {
      const double inv_total = 1.0 / (double)total;
      const double R = (double)rhos[j] - (double)S.massAboveR[j] * inv_total;
      const double M = (double)S.massR[j] * inv_total;
      const double eb = (double)vedge(b, zmax) - lse;
      const double m_hi = exp(eb) * (1.0 + 1e-6), m_lo = exp(eb - (double)BIN_W) * (1.0 - 1e-6);
      if (R > 0.0 && M > 0.0) {
        double ilo = ceil(R / m_hi);
        const double ilo2 = ceil((double)n - (M - R) / m_lo);
        ilo = fmax(ilo, ilo2);
        const double ihi = ceil(R * (double)n / (M * (1.0 - 1e-6)));
        if (ilo == ihi && ilo >= 1.0 && ilo <= (double)n) kr = S.cntAboveR[j] + (int)ilo;
      }
    }
    S.kres[j] = kr;
  }
  __syncthreads();
  // candidate segments of the crossing bins still to rank: one per distinct
  // bin; fall back when the candidates do not fit or a crossing lies in the
  // last (unbounded) bin
  const bool topk_ok = collectK && S.fillK >= K && S.fillK <= CAPK;
  const int bK = topk_ok ? -1 : S.bK;
  const int nKc = topk_ok ? S.fillK : S.aboveK + S.nbK;
  int bR[RHO_MAX], seg[RHO_MAX];
  bool own[RHO_MAX];
  int used = 0;
  bool fail = !topk_ok && (S.bK < 0 || nKc > CAPK);
#pragma unroll
  for (int j = 0; j < RHO_MAX; ++j) {
    bR[j] = -1;
    seg[j] = 0;
    own[j] = false;
    if (j < n_rho && S.kres[j] == 0) {
      bR[j] = S.bR[j];
      if (bR[j] < 0 || bR[j] == NBL - 1) fail = true;
      int first = j;
      for (int q = 0; q < j; ++q)
        if (bR[q] == bR[j] && first == j) first = q;
      own[j] = (first == j);
      seg[j] = own[j] ? used : seg[first];
      if (own[j]) used += S.nR[j];
    }
  }
  // with the top-K settled, unpinned targets go to k_rows_cross when a state
  // array is given (each crossing bin holding at most CAPX elements)
  bool defer = cross != nullptr && topk_ok && used > 0;
#pragma unroll
  for (int j = 0; j < RHO_MAX; ++j)
    if (defer && own[j] && S.nR[j] > CAPX) fail = true;
  if (!defer && used > CAPR) fail = true;
  if (fail) {
    if (tid == 0) flags[row] = F_EXACT;
    return;
  }
  const bool needC = bK >= 0 || (used > 0 && !defer);
  if (tid == 0 && defer) {
    CrossRow& c = cross[row];
    c.lse = lse;
    c.zmax = zmax;
#pragma unroll
    for (int j = 0; j < RHO_MAX; ++j) {
      c.b[j] = bR[j];
      c.n[j] = bR[j] >= 0 ? S.nR[j] : 0;
      c.above[j] = S.cntAboveR[j];
      c.fill[j] = 0;
      c.base[j] = (double)S.massAboveR[j] * (1.0 / (double)total);
      c.rho[j] = rhos[j];
    }
  }
  if (tid == 0) {
    flags[row] = defer ? F_DEFER : F_DONE;
    if (!topk_ok) S.fillK = 0;
#pragma unroll
    for (int j = 0; j < RHO_MAX; ++j) {
      S.fillR[j] = 0;
      S.segR[j] = seg[j];
    }
  }
  __syncthreads();

  if (needC) {
    // ---- C: collect the candidates still needed (rare: the LDS slot
    // atomics run only for the lanes holding one)
    row_loop_pipe<RF>(
        zr, V, vec,
        [&](int64_t i, float x, int) {
          const int b = vbin(x, zmax);
          // the bins are recomputed exactly as in pass B, so the counts match;
          // the bounds tests only keep LDS writes inside the pools regardless
          if (b <= bK) {
            const int slot = atomicAdd(&S.fillK, 1);
            if (slot < CAPK) S.poolK[slot] = cand_key(x, i);
          }
          int jr = -1;  // the first target with this crossing bin owns its segment
#pragma unroll
          for (int j = RHO_MAX - 1; j >= 0; --j) jr = (b == bR[j]) ? j : jr;  // bR[j] = -1: resolved or unused
          if (jr >= 0) {
            const int slot = S.segR[jr] + atomicAdd(&S.fillR[jr], 1);
            if (slot < CAPR) S.u.c.poolR[slot] = cand_key(x, i);
          }
        },
        [](int64_t, bool) {});
    __syncthreads();
  }

  const int nKt = topk_ok ? fast_trim_pool(S, nKc, K, zmax, tau) : nKc;
  fast_emit_topk(S, nKt, K, zr, row, lse, idx_out, val_out, lse_out, mq_out, logp_out);

  // k_rho: resolved from the histogram, or the masses of the crossing bin's
  // elements in rank order, then the first rank where the mass from the top
  // reaches rho
  const double inv_total = 1.0 / (double)total;
  for (int j = 0; j < n_rho; ++j) {
    if (S.kres[j] > 0) {
      if (tid == 0) krho_out[row * n_rho + j] = S.kres[j];
      continue;
    }
    if (defer) continue;  // k_rows_cross writes it
    const int s0 = S.segR[j], n = S.nR[j];
    const int hit = crossing_rank(S.u.c.poolR + s0, n, lse, (double)S.massAboveR[j] * inv_total, (double)S.rho[j],
                                  S.u.c.m, S.red_d, S.red_i);
    if (tid == 0) krho_out[row * n_rho + j] = S.cntAboveR[j] + (hit < n ? hit + 1 : n);
    __syncthreads();
  }
}

// The deferred rows among r0 .. r0 + nr - 1 (nr <= XL) in row order, into
// list[]; returns their number (the same list in every workgroup: the flags
// do not change during k_rows_cross).
__device__ __forceinline__ int deferred_list(const int32_t* flags, int64_t r0, int nr, int* list, int* wcount) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int PT = XL / RF;  // thread t looks at rows PT*t .. PT*t + PT - 1
  bool dfr[PT];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int r = tid * PT + i;
    const int f = r < nr ? flags[r0 + r] : F_DONE;
    dfr[i] = f == F_DEFER;
    cnt += dfr[i] ? 1 : 0;
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wcount[w] = incl;
  __syncthreads();
  int off = incl - cnt, total = 0;
  for (int i = 0; i < RF / 64; ++i) {
    if (i < w) off += wcount[i];
    total += wcount[i];
  }
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if (dfr[i]) list[off++] = tid * PT + i;
  __syncthreads();
  return total;
}

// Deferred crossing bins: the workgroups take (row, slice) items of the
// deferred rows in turn, read the slice and append the elements of the row's
// crossing bins (recomputed exactly as in the histogram read) to its
// buffers.  No workgroup waits for another: the ranking is done by the exact
// kernel's launch, which follows.
__global__ __launch_bounds__(RF) void k_rows_cross(const float* __restrict__ z, int64_t ldz, int64_t V, int64_t r0,
                                                   int nr, int n_rho, const int32_t* __restrict__ flags,
                                                   CrossRow* __restrict__ cross,
                                                   unsigned long long* __restrict__ xcand) {
  __shared__ int list[XL];
  __shared__ int wcount[RF / 64];
  __shared__ unsigned long long lbuf[RHO_MAX][CAPX];  // the slice's elements per target, then one global append
  __shared__ int lfill[RHO_MAX], gbase[RHO_MAX];
  const int tid = threadIdx.x;
  const int total = deferred_list(flags, r0, nr, list, wcount);
  const int64_t per = ((V + NSX - 1) / NSX + 3) & ~(int64_t)3;
  const bool vec = ((V & 3) == 0) && ((((uintptr_t)z) & 15) == 0) && ((ldz & 3) == 0);
  for (int it = blockIdx.x; it < total * NSX; it += gridDim.x) {
    const int rl = list[it / NSX];  // row - r0
    const int slice = it % NSX;
    CrossRow* c = cross + rl;
    const float zmax = c->zmax;
    int bj[RHO_MAX], blo = NBL, bhi = -1;
#pragma unroll
    for (int j = 0; j < RHO_MAX; ++j) {
      bj[j] = j < n_rho ? c->b[j] : -1;
      if (bj[j] >= 0) {
        blo = min(blo, bj[j]);
        bhi = max(bhi, bj[j]);
      }
    }
    const float* zr = z + (r0 + rl) * ldz;
    const int64_t s0 = (int64_t)slice * per, s1 = min(V, s0 + per);
    if (tid < RHO_MAX) lfill[tid] = 0;
    __syncthreads();
    auto take = [&](int64_t i, float x) {
      const int b = vbin(x, zmax);
      if (b < blo || b > bhi) return;  // nearly every element
#pragma unroll
      for (int j = 0; j < RHO_MAX; ++j)
        if (b == bj[j]) {
          const int slot = atomicAdd(&lfill[j], 1);
          if (slot < CAPX) lbuf[j][slot] = cand_key(x, i);
        }
    };
    if (vec) {
      // 8 loads per thread in flight, then their elements
      const float4* z4 = (const float4*)zr;
      const int64_t a4 = s0 / 4, b4 = s1 / 4;
      for (int64_t base = a4 + tid; base < b4; base += (int64_t)RF * 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t i4 = base + (int64_t)u * RF;
          v[u] = z4[i4 < b4 ? i4 : b4 - 1];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t i4 = base + (int64_t)u * RF;
          if (i4 < b4) {
            take(4 * i4, v[u].x);
            take(4 * i4 + 1, v[u].y);
            take(4 * i4 + 2, v[u].z);
            take(4 * i4 + 3, v[u].w);
          }
        }
      }
    } else {
      for (int64_t i = s0 + tid; i < s1; i += RF) take(i, zr[i]);
    }
    __syncthreads();
    // one global append per target: reserve the range, then copy (a count
    // past CAPX is kept so that the ranking launch sees the mismatch)
    if (tid < n_rho && lfill[tid] > 0) gbase[tid] = atomicAdd(&c->fill[tid], lfill[tid]);
    __syncthreads();
    for (int j = 0; j < n_rho; ++j) {
      const int nl = min(lfill[j], CAPX);
      for (int p = tid; p < nl; p += RF)
        if (gbase[j] + p < CAPX) xcand[((int64_t)rl * n_rho + j) * CAPX + gbase[j] + p] = lbuf[j][p];
    }
    __syncthreads();
  }
}

// Workspace of the deferred crossing bins for `rows` rows: the per-row state,
// then CAPX candidates per (row, target).  None without k_rho targets or
// when the fast kernel does not run.
static size_t cross_bytes(int64_t rows, int64_t V, int n_rho) {
  if (n_rho == 0 || V > VFAST_MAX) return 0;
  return (size_t)kd_round_up(rows * (int64_t)sizeof(CrossRow), 256) + (size_t)rows * n_rho * CAPX * 8;
}

struct CachePlan {
  int64_t Tb;
  int nVT;
  size_t zbytes, o_flags, o_tmax, o_cross, total;
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
  p.nVT = (int)kd_ceil_div(V, CC::BM);
  // logit block, per-row fallback flags, per-(row, vocabulary tile) maxima
  p.zbytes = (size_t)tb * V * 4;
  p.o_flags = p.zbytes;
  p.o_tmax = p.o_flags + (size_t)kd_round_up(tb * 4, 256);
  p.o_cross = p.o_tmax + (size_t)kd_round_up(tb * p.nVT * 4, 256);
  p.total = p.o_cross + cross_bytes(tb, V, n_rho);
  return true;
}

static kd_status check_rho(const float* rho_host, int32_t n_rho) {
  if (n_rho > 0 && !rho_host) return kd_fail(KD_EINVAL, "rho_host is NULL with n_rho=%d", (int)n_rho);
  for (int j = 0; j < n_rho; ++j)
    if (!(rho_host[j] > 0.f && rho_host[j] <= 1.f)) return kd_fail(KD_EINVAL, "rho[%d]=%g outside (0, 1]", j, rho_host[j]);
  return KD_OK;
}

// Fast pass over all rows, then the exact pass over the rows it flagged
// (every row when V is beyond the fast pass's packed counts).  `flags` holds
// `rows` int32; tmax (optional) the rows' maxima in n_tmax parts each.
// The row pass: the fast kernel, the deferred crossing bins (when `cross`
// holds cross_bytes(rows, V, n_rho); else the fast kernel reads those rows
// again itself), and the exact kernel for the flagged rows.
static void launch_rows(const float* z, int64_t ldz, int64_t rows, int64_t V, int K, const float* rho, int n_rho,
                        int32_t* idx, float* val, float* lse, float* m_q, int32_t* k_rho, float* logp,
                        int32_t* flags, const float* tmax, int n_tmax, void* cross, hipStream_t s) {
  float r[RHO_MAX] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < n_rho; ++j) r[j] = rho[j];
  const bool fast = V <= VFAST_MAX;
  CrossRow* cr = (fast && n_rho > 0) ? (CrossRow*)cross : nullptr;
  unsigned long long* xc =
      cr ? (unsigned long long*)((char*)cross + kd_round_up(rows * (int64_t)sizeof(CrossRow), 256)) : nullptr;
  if (fast)
    KD_LAUNCH(k_topk_rows, dim3((unsigned)rows), dim3(RF), 0, s, z, ldz, V, K, n_rho, r[0], r[1], r[2], r[3],
                       r[4], r[5], r[6], r[7], tmax, n_tmax, flags, idx, val, lse, m_q, k_rho, logp, cr);
  for (int64_t r0 = 0; cr && r0 < rows; r0 += XL) {
    const int nr = (int)(rows - r0 < XL ? rows - r0 : XL);
    KD_LAUNCH(k_rows_cross, dim3(XG), dim3(RF), 0, s, z, ldz, V, r0, nr, n_rho, flags, cr + r0,
              xc + r0 * n_rho * CAPX);
  }
  KD_LAUNCH(k_topk_rows_exact, dim3((unsigned)rows), dim3(RT), 0, s, z, ldz, V, K, n_rho, r[0], r[1], r[2], r[3],
                     r[4], r[5], r[6], r[7], fast ? (const int32_t*)flags : nullptr, idx, val, lse, m_q, k_rho,
                     logp, (const CrossRow*)cr, (const unsigned long long*)xc);
}

}  // namespace

extern "C" size_t kd_topk_cache_build_workspace(int64_t T, int64_t d, int64_t V, int32_t K, int32_t n_rho) {
  CachePlan p;
  if (!plan_cache(T, d, V, K, n_rho, p)) return 0;
  return p.total;
}

extern "C" kd_status kd_topk_cache_build(const kd_bf16* g, const kd_bf16* U, const float* b, int64_t T, int64_t d,
                                         int64_t V, int32_t K, const float* rho_host, int32_t n_rho, int32_t* idx,
                                         float* val, float* lse, float* m_q, int32_t* k_rho, float* teacher_logp,
                                         void* ws, size_t ws_bytes, void* stream) {
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
  if (!kd_aligned16(g) || !kd_aligned16(U) || !kd_aligned16(ws))
    return kd_fail(KD_EINVAL, "g, U and ws must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  float* z = (float*)ws;
  for (int64_t t0 = 0; t0 < T; t0 += p.Tb) {
    const int64_t tb = (T - t0 < p.Tb) ? T - t0 : p.Tb;
    const int nTT = (int)kd_ceil_div(tb, CC::BN), nVT = p.nVT;
    const int grid = (int)kd_round_up((int64_t)nTT * nVT, 8);
    float* tmax = (float*)((char*)ws + p.o_tmax);
    KD_LAUNCH(k_cache_gemm, dim3(grid), dim3(CC::NT), CG_LDS, s, (const bf16_t*)g + t0 * d,
                       (const bf16_t*)U, b, tb, d, V, nTT, nVT, z, tmax);
    launch_rows(z, V, tb, V, K, rho_host, n_rho, idx + t0 * K, val + t0 * K, lse + t0, m_q + t0,
                n_rho ? k_rho + t0 * n_rho : nullptr, teacher_logp ? teacher_logp + t0 * K : nullptr,
                (int32_t*)((char*)ws + p.o_flags), tmax, nVT, (char*)ws + p.o_cross, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e));
  }
  return KD_OK;
}

// Device address of `scratch` on the current device, taken once per device.
static kd_status noalloc_scratch(int32_t** out) {
  static std::mutex mu;
  static int32_t* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kd_fail(KD_EHIP, "hipGetDevice failed");
  if (dev >= 64) return kd_fail(KD_EUNSUPPORTED, "device %d beyond the 64 this library tracks", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return kd_fail(KD_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = (int32_t*)p;
  }
  *out = addr[dev];
  return KD_OK;
}

extern "C" kd_status kd_topk_rows_noalloc(const float* z, int64_t T, int64_t V, int32_t K, const float* rho_host,
                                          int32_t n_rho, int32_t* idx, float* val, float* lse, float* m_q,
                                          int32_t* k_rho, float* teacher_logp, void* stream) {
  if (T < 0 || V <= 0 || K < 1 || K > KMAX || K > V || n_rho < 0 || n_rho > RHO_MAX || V >= ((int64_t)1 << 31))
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld V=%lld K=%d n_rho=%d", (long long)T, (long long)V, (int)K, (int)n_rho);
  kd_status st = check_rho(rho_host, n_rho);
  if (st != KD_OK) return st;
  if (T > KD_NOALLOC_ROWS)
    return kd_fail(KD_EUNSUPPORTED, "kd_topk_rows_noalloc takes at most %lld rows per call (got %lld)",
                   (long long)KD_NOALLOC_ROWS, (long long)T);
  if (T == 0) return KD_OK;
  if (!z || !idx || !val || !lse || !m_q || (n_rho > 0 && !k_rho)) return kd_fail(KD_EINVAL, "null required pointer");
  int32_t* flags = nullptr;
  st = noalloc_scratch(&flags);
  if (st != KD_OK) return st;
  launch_rows(z, V, T, V, K, rho_host, n_rho, idx, val, lse, m_q, k_rho, teacher_logp, flags, nullptr, 0, nullptr,
              (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e));
  return KD_OK;
}

extern "C" size_t kd_topk_rows_workspace(int64_t T, int64_t V, int32_t K, int32_t n_rho) {
  if (T < 0 || V <= 0 || K < 1 || K > KMAX || K > V || n_rho < 0 || n_rho > RHO_MAX) return 0;
  // per-row fallback flags, then the deferred crossing bins
  return (size_t)kd_round_up((T > 0 ? T : 1) * 4, 256) + cross_bytes(T > 0 ? T : 1, V, n_rho);
}

extern "C" kd_status kd_topk_rows(const float* z, int64_t T, int64_t V, int32_t K, const float* rho_host,
                                  int32_t n_rho, int32_t* idx, float* val, float* lse, float* m_q, int32_t* k_rho,
                                  float* teacher_logp, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || V <= 0 || K < 1 || K > KMAX || K > V || n_rho < 0 || n_rho > RHO_MAX || V >= ((int64_t)1 << 31))
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld V=%lld K=%d n_rho=%d", (long long)T, (long long)V, (int)K, (int)n_rho);
  kd_status st = check_rho(rho_host, n_rho);
  if (st != KD_OK) return st;
  if (T == 0) return KD_OK;
  if (!z || !idx || !val || !lse || !m_q || (n_rho > 0 && !k_rho)) return kd_fail(KD_EINVAL, "null required pointer");
  const size_t o_cross = (size_t)kd_round_up(T * 4, 256);
  const size_t need = o_cross + cross_bytes(T, V, n_rho);
  if (!ws || ws_bytes < need) return kd_fail(KD_ENOWS, "workspace too small: need %zu bytes, got %zu", need, ws_bytes);
  if (!kd_aligned16(ws)) return kd_fail(KD_EINVAL, "ws must be 16-byte aligned");
  launch_rows(z, V, T, V, K, rho_host, n_rho, idx, val, lse, m_q, k_rho, teacher_logp, (int32_t*)ws, nullptr, 0,
              (char*)ws + o_cross, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e));
  return KD_OK;
}
