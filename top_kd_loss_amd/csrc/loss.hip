// Fused chunked LM head + sparse top-K KD loss, forward and backward, for
// gfx950 ("Efficient Knowledge Distillation for LLMs: Offline Top-K Logits
// and a Fused Chunked KL Loss", section 3.2: the output projection is fused
// into the loss and the [T, V] logits are never materialised).
//
// Pipeline of kd_topk_loss_fwd_bwd (one stream, in order):
//   prep     sort each token's (idx, teacher_logp) by index; per-token
//            teacher constants; per-(vocab tile, token) cursor starts.
//   pass 1   z^T tile = W_tile h_tile^T on the matrix cores; epilogue keeps a
//            per-(vocab tile, token) running max / sum of exp and gathers z
//            at the retained indices.  Only log Z spans the vocabulary
//            (identity (2) of the fused-loss paper), so this is all the
//            forward needs from the full vocabulary.
//   combine  per token: logsumexp, student tail mass, the loss of the mode,
//            the dense coefficient alpha and the sparse coefficients r on S,
//            so that dL/dz = alpha * softmax(z) + r [v in S] (Eq. (3) for the
//            partial-mass loss; the other modes by exact differentiation).
//   pass 2   dense modes, one vocabulary chunk at a time: recompute the z
//            tile, write dz = scale * dL/dz as bf16 (two layouts), then
//            dh += dz W_chunk and dW_chunk = dz^T h on the matrix cores.
//            Sparse modes: dh_t = sum_S r W_v and dW_v = sum_t r h_t over a
//            CSR-by-vocabulary list, deterministic without float atomics.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/kdtopk.h"
#include "gemm.h"
#include "kd_internal.h"

namespace {

using TC = GemmCfg;
constexpr int VT = TC::BM;        // vocabulary rows per tile (M of the z^T tile)
constexpr int TT = TC::BN;        // tokens per tile
constexpr int KMAX = 1024;
constexpr int SENT = 0x7fffffff;  // sorted-index sentinel (padding)

// Per-token scalars kept in the workspace (float, stride TOKF).
enum {
  TK_LSE = 0, TK_ALPHA = 1, TK_L = 2, TK_MP = 3, TK_Q = 4, TK_LSEQ = 5, TK_NV = 6,
  TK_ZY = 7,   // logit of the token's label / sampled token
  TK_YR = 8,   // scaled full dz at that token when it lies outside S
  TK_B = 9,    // reference of the off-S dense term A e^(z - B) (A = TK_ALPHA)
  TOKF = 12
};

// ---------------------------------------------------------------------------
// Tile ordering: workgroup id -> (m tile, n tile).  Workgroups are handed to
// the 8 XCDs round robin; this sends consecutive groups of tiles to one XCD
// and orders them GROUP_M m-tiles at a time, so the workgroups resident on
// an XCD share operand tiles in its L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool tile_of(int bid, int nblocks, int nM, int nN, int group_m, int& mi, int& ni) {
  const int per = nblocks / 8;  // nblocks is a multiple of 8
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

static inline int grid_of(int tiles) { return (int)kd_round_up(tiles, 8); }

// ---------------------------------------------------------------------------
// prep: one 64-lane workgroup per token.  Sort (idx, tlp) ascending by idx
// with a bitonic network in LDS; padding slots (idx < 0) and indices >= V
// sort last as SENT (the latter also raise the error flag).
// ---------------------------------------------------------------------------
// zin (optional): the student's logits at idx, already known; they are
// sorted along into zout (0 at padding slots).
__global__ __launch_bounds__(64) void k_prep(const int32_t* __restrict__ idx, const float* __restrict__ tlp,
                                             const float* __restrict__ zin, int64_t T, int64_t V, int K, int Kp2,
                                             int nVT, int64_t Tp, int32_t* __restrict__ sidx,
                                             float* __restrict__ stlp, float* __restrict__ zout,
                                             int2* __restrict__ starts, float* __restrict__ tok,
                                             int32_t* __restrict__ err) {
  __shared__ int key[KMAX];
  __shared__ float val[KMAX];
  __shared__ float zv[KMAX];
  const int lane = threadIdx.x;
  // Consecutive tokens run on one XCD (workgroups are dealt to the 8 XCDs in
  // turn; the grid is a multiple of 8), so the cursor starts of neighbouring
  // tokens, 8 bytes apart in each tile's row, merge into whole lines in that
  // XCD's L2 instead of being written back as partial lines by 8 of them.
  const int64_t per = (int64_t)gridDim.x / 8;
  const int64_t t = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= T) return;
  bool bad = false;
  for (int k = lane; k < Kp2; k += 64) {
    int id = SENT;
    float v = 0.f, zz = 0.f;
    if (k < K) {
      const int raw = idx[t * K + k];
      if (raw >= V) {
        bad = true;
      } else if (raw >= 0) {
        id = raw;
        v = tlp[t * K + k];
        if (zin != nullptr) zz = zin[t * K + k];
      }
    }
    key[k] = id;
    val[k] = v;
    zv[k] = zz;
  }
  __syncthreads();
  for (int size = 2; size <= Kp2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = lane; i < Kp2 / 2; i += 64) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const int a = key[lo], b = key[hi];
        if ((a > b) == up) {
          key[lo] = b;
          key[hi] = a;
          const float x = val[lo];
          val[lo] = val[hi];
          val[hi] = x;
          const float y = zv[lo];
          zv[lo] = zv[hi];
          zv[hi] = y;
        }
      }
      __syncthreads();
    }
  }
  int nv = 0;
  double mx = -INFINITY;
  for (int k = lane; k < K; k += 64) {
    const int id = key[k];
    sidx[t * K + k] = id;
    stlp[t * K + k] = val[k];
    if (zout != nullptr) zout[t * K + k] = zv[k];
    if (id != SENT) {
      ++nv;
      mx = fmax(mx, (double)val[k]);
      if (k + 1 < K && key[k + 1] == id) bad = true;  // duplicate index
    }
  }
  nv = wave_sum_i32(nv);
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  double q = 0.0;
  for (int k = lane; k < nv; k += 64) q += exp((double)val[k] - mx);
  q = wave_sum_f64(q);
  // vocabulary-tile cursor starts: first sorted position with idx >= vt*VT,
  // and the index there (SENT past the last), so that a tile learns from one
  // load whether the token has an entry in it
  for (int vt = lane; vt < nVT; vt += 64) {
    int lo = 0, hi = nv;
    const int target = vt * VT;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (key[mid] < target) lo = mid + 1; else hi = mid;
    }
    starts[(int64_t)vt * Tp + t] = make_int2(lo, lo < nv ? key[lo] : SENT);
  }
  if (lane == 0) {
    tok[t * TOKF + TK_NV] = (float)nv;
    tok[t * TOKF + TK_Q] = nv > 0 ? (float)(exp(mx) * q) : 0.f;    // Q = sum_S exp(tlp)
    tok[t * TOKF + TK_LSEQ] = nv > 0 ? (float)(mx + log(q)) : 0.f;  // logsumexp of tlp over S
  }
  if (bad) atomicOr(err, 1);
}

// ---------------------------------------------------------------------------
// pass 1: z^T tile (vocab x tokens) with the logsumexp / gather epilogue.
// Before the main loop the thread owning token n0 + tid walks the token's
// sorted indices inside the tile and parks a 256-bit row mask (bit r = row
// m0 + r is retained) with the sorted position of the first of them.  After
// the main loop every lane takes, for each of its 4 token columns, the
// retained rows among its own 64 accumulators: it writes their logits to z_S
// and sets them to -inf.  The per-token (max, sum exp(z - max)) partials of
// the tile then cover the vocabulary OUTSIDE S only (in-lane over the 64
// accumulators plus one xor-32 exchange, merged across the WM wavefront
// rows in LDS), so the student's tail mass m_p = sum_{v not in S} p_v comes
// out as a sum of positive terms instead of 1 - sum_S p.
// ---------------------------------------------------------------------------
constexpr int P1_RED = TC::WM * TT * 2 * 4;           // (max, sum) per wavefront row and token
constexpr int P1_MASKW = VT / 32;                     // mask words per token
constexpr int P1_PARK = (P1_MASKW + 1) * TC::NT * 4;  // masks + first positions
constexpr int P1_LDS = GEMM_LDS + P1_PARK;
static_assert(P1_RED <= GEMM_LDS, "pass-1 reduction space");

// Tile rows at or past vlim (the vocabulary's end) are set to -inf in the
// accumulators, so the epilogues below need no per-element row test: they
// drop out of maxima and exp() of them is 0.
__device__ __forceinline__ void mask_rows(Acc<TC>& acc, int vlim, int wm, int lane) {
  const int rbase = wm * TC::TM + 4 * (lane >> 5);
#pragma unroll
  for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TC::FN; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (rbase + fm * 32 + 8 * (e >> 2) + (e & 3) >= vlim) acc.v[fm][fn][e] = -KD_INF;
}

// Row reductions of one wavefront's accumulators per token column, leaving
// out the retained rows: bit 8g + r of sm[fn][fm] set = element 4g + r of
// block (fm, fn) is retained.
__device__ __forceinline__ void pass1_reduce(const Acc<TC>& acc, const uint32_t (&sm)[TC::FN][TC::FM], float* red,
                                             int wm, int wn, int lane) {
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    float mx = -KD_INF;
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool ret = (sm[fn][fm] >> (8 * (e >> 2) + (e & 3))) & 1u;
        mx = fmaxf(mx, ret ? -KD_INF : acc.v[fm][fn][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float nm = (mx == -KD_INF) ? 0.f : -mx * KD_LOG2E;
    float s = 0.f;
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool ret = (sm[fn][fm] >> (8 * (e >> 2) + (e & 3))) & 1u;
        const float x = __builtin_amdgcn_exp2f(fmaf(acc.v[fm][fn][e], KD_LOG2E, nm));
        s += ret ? 0.f : x;
      }
    s += __shfl_xor(s, 32, 64);
    const int col = acc_col<TC>(wn, fn, lane);
    if (lane < 32) {
      red[(wm * TT + col) * 2 + 0] = mx;
      red[(wm * TT + col) * 2 + 1] = s;
    }
    __builtin_amdgcn_sched_barrier(0);  // one token column's values live at a time
  }
}

// Retained-row mask of token ts inside the tile [m0, m0 + VT): bit r of word
// r / 32 is row m0 + r.  kc0 receives the sorted position of the first
// retained index >= m0 (K if none).  Indices are read eight at a time.
__device__ __forceinline__ void tile_row_mask(const int32_t* __restrict__ sidx, const int2* __restrict__ starts,
                                              int64_t ts, int64_t T, int K, int vt, int64_t Tp, int64_t m0,
                                              uint32_t (&mk)[P1_MASKW], int& kc0) {
#pragma unroll
  for (int w = 0; w < P1_MASKW; ++w) mk[w] = 0u;
  kc0 = K;
  if (ts >= T) return;
  const int2 sf = starts[(int64_t)vt * Tp + ts];
  kc0 = sf.x;
  if ((int64_t)sf.y - m0 >= VT) return;  // no entry in this tile (most tiles)
  for (int kc = kc0; kc < K; kc += 8) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (kc + j < K) ? sidx[ts * K + kc + j] : SENT;
    bool done = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t r = (int64_t)v[j] - m0;  // >= 0: sorted from the tile's first entry on
      if (r < VT) {
#pragma unroll
        for (int w = 0; w < P1_MASKW; ++w) mk[w] |= ((int)(r >> 5) == w) ? (1u << (r & 31)) : 0u;
      } else {
        done = true;
      }
    }
    if (done) break;
  }
}

// The retained rows this lane holds in token column fn: their logits go to
// z_S, and sm[fm] receives the lane's bits (bit 8g + r = element 4g + r of
// block fm).  mk: the token's tile mask, kc0 its first sorted position.
__device__ __forceinline__ void pass1_gather(const Acc<TC>& acc, int fn, const uint32_t (&mk)[P1_MASKW], int kc0,
                                             int64_t t, int K, float* __restrict__ zS, int wm, int lane,
                                             uint32_t (&sm)[TC::FM]) {
  const int h4 = 4 * (lane >> 5);  // this lane's rows: h4 + r of each group of 8
  uint32_t any = 0u;
#pragma unroll
  for (int fm = 0; fm < TC::FM; ++fm) {
    sm[fm] = ((wm ? mk[TC::FM + fm] : mk[fm]) >> h4) & 0x0F0F0F0Fu;
    any |= sm[fm];
  }
  if (any == 0u) return;
  int base = kc0;
  if (wm) {
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm) base += __builtin_popcount(mk[fm]);
  }
#pragma unroll
  for (int fm = 0; fm < TC::FM; ++fm) {
    const uint32_t w = wm ? mk[TC::FM + fm] : mk[fm];
    if (sm[fm]) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int bit = 8 * (e >> 2) + h4 + (e & 3);
        if ((w >> bit) & 1u) zS[t * K + base + __builtin_popcount(w & ((1u << bit) - 1u))] = acc.v[fm][fn][e];
      }
    }
    base += __builtin_popcount(w);
  }
}

// Token-block variant (STORE): the tile's logits also leave as
// E = bf16(exp(z - m)) token rows [n][ldE], with m the tile's maximum over
// the token's vocabulary rows outside S; retained rows, rows past the
// vocabulary end and padding tokens give 0.  The tile is transposed through
// LDS (the pass-2 layout) for 16-byte coalesced stores.
constexpr int P1S_LDS = (VT * TT * 2 > P1_LDS) ? VT * TT * 2 : P1_LDS;
__device__ __forceinline__ int zdz_swz(int t);

__device__ __forceinline__ void pass1_store_E(const Acc<TC>& acc, const uint32_t (&sm)[TC::FN][TC::FM],
                                              const float (&mt)[TC::FN], char* Et, int64_t n0, int64_t T, int wm,
                                              int wn, int lane) {
  const int rbase = wm * TC::TM + 4 * (lane >> 5);
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    const int tl = acc_col<TC>(wn, fn, lane);
    const float nl = (n0 + tl < T && mt[fn] != -KD_INF) ? -mt[fn] * KD_LOG2E : -KD_INF;
    char* row = Et + tl * (VT * 2);
    const int sw = zdz_swz(tl);
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ret = (sm[fn][fm] >> (8 * g + r)) & 1u;
          const float e = __builtin_amdgcn_exp2f(fmaf(acc.v[fm][fn][g * 4 + r], KD_LOG2E, nl));
          x[r] = ret ? 0.f : e;
        }
        const int vl = rbase + fm * 32 + 8 * g;
        uint2 pk;
        pk.x = pack_bf16x2(x[0], x[1]);
        pk.y = pack_bf16x2(x[2], x[3]);
        *(uint2*)(row + (((vl >> 3) ^ sw) << 4) + (vl & 7) * 2) = pk;
      }
  }
}

// One pass-1 tile; MASK: the tile runs past the vocabulary end (own code
// path, so the common one carries no masking registers).
template <bool MASK, bool STORE = false>
__device__ __forceinline__ void pass1_tile(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                  int64_t T, int64_t d, int64_t V, int K, int nVT, int nTT,
                                                  int64_t Tp, const int32_t* __restrict__ sidx,
                                                  const int2* __restrict__ starts, float* __restrict__ zS,
                                                  float2* __restrict__ part, int vt, int tt, bf16_t* lds,
                                                  bf16_t* __restrict__ Eg = nullptr, int64_t ldE = 0) {
  const int64_t m0 = (int64_t)vt * VT, n0 = (int64_t)tt * TT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TC::WN, wn = wave % TC::WN;
  const int tid = threadIdx.x;
  uint32_t* park = (uint32_t*)((char*)lds + GEMM_LDS);
  {
    uint32_t mk[P1_MASKW];
    int kc0;
    tile_row_mask(sidx, starts, n0 + tid, T, K, vt, Tp, m0, mk, kc0);
#pragma unroll
    for (int w = 0; w < P1_MASKW; ++w) park[w * TC::NT + tid] = mk[w];
    park[P1_MASKW * TC::NT + tid] = (uint32_t)kc0;
  }

  Acc<TC> acc;
  gemm_tile_pipe<TC>(W, d, m0, V, h, d, n0, T, (int)d, lds, acc);
  __syncthreads();  // every wavefront is done with the operand stages (and the masks are parked)

  if (MASK) mask_rows(acc, (int)(V - m0), wm, lane);
  uint32_t sm[TC::FN][TC::FM];
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    const int col = acc_col<TC>(wn, fn, lane);
    uint32_t mk[P1_MASKW];
#pragma unroll
    for (int w = 0; w < P1_MASKW; ++w) mk[w] = park[w * TC::NT + col];
    const int kc0 = (int)park[P1_MASKW * TC::NT + col];
    pass1_gather(acc, fn, mk, kc0, n0 + col, K, zS, wm, lane, sm[fn]);
  }
  float* red = (float*)lds;
  pass1_reduce(acc, sm, red, wm, wn, lane);
  __syncthreads();
  // merge the WM wavefront rows of the tile and write one partial per token
  for (int col = threadIdx.x; col < TT; col += TC::NT) {
    float m = -KD_INF, s = 0.f;
#pragma unroll
    for (int w = 0; w < TC::WM; ++w) {
      const float mw = red[(w * TT + col) * 2 + 0], sw = red[(w * TT + col) * 2 + 1];
      const float mn = fmaxf(m, mw);
      s = (m == -KD_INF ? 0.f : s * __expf(m - mn)) + (mw == -KD_INF ? 0.f : sw * __expf(mw - mn));
      m = mn;
    }
    const int64_t t = n0 + col;
    if (t < T) part[(int64_t)vt * Tp + t] = make_float2(m, s);
  }
  if constexpr (STORE) {
    float mt[TC::FN];
#pragma unroll
    for (int fn = 0; fn < TC::FN; ++fn) {
      const int col = acc_col<TC>(wn, fn, lane);
      mt[fn] = fmaxf(red[col * 2], red[(TT + col) * 2]);
    }
    __syncthreads();  // red is read before the E tile overwrites it
    char* Et = (char*)lds;
    pass1_store_E(acc, sm, mt, Et, n0, T, wm, wn, lane);
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < TT / 8; ++it) {
      const int tl = it * 8 + (tid >> 5), c = tid & 31;
      const u32x4 q = *(const u32x4*)(Et + tl * (VT * 2) + ((c ^ zdz_swz(tl)) << 4));
      // streamed past the caches: the block of E is far larger than them
      __builtin_nontemporal_store(q, (u32x4*)(Eg + (n0 + tl) * ldE + m0 + c * 8));
    }
  }
}

// Token-block pass 1: as k_pass1, and the tile's E rows go to Eg [nTT*TT][ldE].
__global__ __launch_bounds__(256, 1) void k_pass1_store(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                        int64_t T, int64_t d, int64_t V, int K, int nVT, int nTT,
                                                        int64_t Tp, const int32_t* __restrict__ sidx,
                                                        const int2* __restrict__ starts, float* __restrict__ zS,
                                                        float2* __restrict__ part, bf16_t* __restrict__ Eg,
                                                        int64_t ldE) {
  extern __shared__ __align__(16) bf16_t lds[];
  int vt, tt;
  if (!tile_of(blockIdx.x, gridDim.x, nVT, nTT, 8, vt, tt)) return;
  if ((int64_t)(vt + 1) * VT > V)
    pass1_tile<true, true>(W, h, T, d, V, K, nVT, nTT, Tp, sidx, starts, zS, part, vt, tt, lds, Eg, ldE);
  else
    pass1_tile<false, true>(W, h, T, d, V, K, nVT, nTT, Tp, sidx, starts, zS, part, vt, tt, lds, Eg, ldE);
}

__global__ __launch_bounds__(256, 1) void k_pass1(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                  int64_t T, int64_t d, int64_t V, int K, int nVT, int nTT,
                                                  int64_t Tp, const int32_t* __restrict__ sidx,
                                                  const int2* __restrict__ starts, float* __restrict__ zS,
                                                  float2* __restrict__ part) {
  extern __shared__ __align__(16) bf16_t lds[];
  int vt, tt;
  if (!tile_of(blockIdx.x, gridDim.x, nVT, nTT, 8, vt, tt)) return;
  if ((int64_t)(vt + 1) * VT > V)
    pass1_tile<true>(W, h, T, d, V, K, nVT, nTT, Tp, sidx, starts, zS, part, vt, tt, lds);
  else
    pass1_tile<false>(W, h, T, d, V, K, nVT, nTT, Tp, sidx, starts, zS, part, vt, tt, lds);
}

// ---------------------------------------------------------------------------
// Label logit for the hard-label cross-entropy term: z_y = h_t . W_y in fp32
// (products of bf16 values are exact), one wavefront per token.  Labels >= V
// raise the error flag; y < 0 means no label.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_label_logit(const bf16_t* __restrict__ h, const bf16_t* __restrict__ W,
                                                     const int32_t* __restrict__ labels, int64_t T, int64_t d,
                                                     int64_t V, float* __restrict__ tok, int32_t* __restrict__ err) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int y = labels[t];
  float acc = 0.f;
  if (y >= 0 && y < V) {
    const bf16_t* hr = h + t * d;
    const bf16_t* wr = W + (int64_t)y * d;
    for (int64_t j = (int64_t)lane * 8; j < d; j += 64 * 8) {
      const u32x4 a = *(const u32x4*)(hr + j), b = *(const u32x4*)(wr + j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), acc);
        acc = fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(b[i] & 0xffff0000u), acc);
      }
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    tok[t * TOKF + TK_ZY] = acc;
    if (y >= V) atomicOr(err, 1);
  }
}

// ---------------------------------------------------------------------------
// combine: one wavefront per token.  All per-token math in fp64.
// ---------------------------------------------------------------------------
// Pass 1's partials cover the vocabulary outside S, so per token
//   lse_off = log sum_{v not in S} e^z,  lse_S = log sum_{v in S} e^z,
//   lse = logaddexp(lse_off, lse_S),    m_p = e^(lse_off - lse),
// all sums of positive terms.  With the student's lse given instead (pass 1
// skipped), m_p = -expm1(lse_S - lse) and lse_off = lse + log m_p.
//
// The backward's dz is written as
//   off S:  A e^(z - B)           (dense; A = TK_ALPHA, B = TK_B, scaled)
//   on S:   coef                  (the full dz of the entry, fp64 -> fp32)
//   at y:   TK_YR                 (the full dz of a label / sampled token
//                                  outside S, which pass 2 writes)
// B = lse, A = the mode's dense coefficient alpha, except in KD_TAIL with
// m_q > 0, whose off-S gradient (Q + m_q + lam - m_q / m_p) p equals
// ((Q + m_q + lam) m_p - m_q) e^(z - lse_off): B = lse_off keeps the
// exponent and the amplitude bounded however small m_p is.  On S the
// m_q / m_p terms of the dense coefficient and of the residual cancel
// exactly, so coef takes (Q + m_q + lam) p - q directly.
//
// Tokens y per token (labels; -1 = none):
//  * cross-entropy term (ce_weight != 0): L += ce_weight (lse - z_y),
//    alpha += ce_weight, residual -ce_weight at y;
//  * KD_REVERSE_TT (y = the sampled token, tly its teacher log-prob): when y
//    is outside S, with l = z_y - lse - tly: L += l, alpha -= l, residual +l.
// ylab[t] = y when y carries a residual outside S (pass 2 writes that entry),
// else -1.
__device__ __forceinline__ double logaddexp_d(double a, double b) {
  if (a == -INFINITY) return b;
  if (b == -INFINITY) return a;
  const double m = fmax(a, b);
  return m + log1p(exp(-fabs(a - b)));
}

__global__ __launch_bounds__(256) void k_combine(int64_t T, int K, int nVT, int64_t Tp, int mode, float scale,
                                                 const float2* __restrict__ part, const float* __restrict__ zS,
                                                 const int32_t* __restrict__ sidx, const float* __restrict__ stlp,
                                                 const float* __restrict__ m_q, const int32_t* __restrict__ labels,
                                                 float ce_weight, const float* __restrict__ tly, int64_t V,
                                                 float* __restrict__ tok,
                                                 float* __restrict__ coef, int32_t* __restrict__ ylab,
                                                 float* __restrict__ loss_tok, float* __restrict__ lse_out,
                                                 float* __restrict__ mp_out, const float* __restrict__ lse_in) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;

  const float* tk = tok + t * TOKF;
  const int nv = (int)tk[TK_NV];
  const double Q = tk[TK_Q], lseq = tk[TK_LSEQ];
  // retained-logit logsumexp
  double zmax = -INFINITY;
  for (int k = lane; k < nv; k += 64) zmax = fmax(zmax, (double)zS[t * K + k]);
  for (int o = 32; o > 0; o >>= 1) zmax = fmax(zmax, __shfl_xor(zmax, o, 64));
  double es = 0.0;
  for (int k = lane; k < nv; k += 64) es += exp((double)zS[t * K + k] - zmax);
  es = wave_sum_f64(es);
  const double lseS = (nv > 0) ? zmax + log(es) : -INFINITY;

  double lse, lse_off, mp;
  if (lse_in != nullptr) {
    lse = (double)lse_in[t];
    mp = (nv > 0) ? -expm1(lseS - lse) : 1.0;
    if (mp < 0.0) mp = 0.0;
    lse_off = mp > 0.0 ? lse + log(mp) : -INFINITY;
  } else {
    // logsumexp of the per-tile partials outside S
    double m = -INFINITY, s = 0.0;
    for (int vt = lane; vt < nVT; vt += 64) {
      const float2 p = part[(int64_t)vt * Tp + t];
      if (p.x == -KD_INF) continue;
      const double mn = fmax(m, (double)p.x);
      s = (m == -INFINITY ? 0.0 : s * exp(m - mn)) + (double)p.y * exp((double)p.x - mn);
      m = mn;
    }
    double M = m;
    for (int o = 32; o > 0; o >>= 1) M = fmax(M, __shfl_xor(M, o, 64));
    s = (m == -INFINITY) ? 0.0 : s * exp(m - M);
    s = wave_sum_f64(s);
    lse_off = (s > 0.0) ? M + log(s) : -INFINITY;
    lse = logaddexp_d(lse_off, lseS);
    mp = (lse_off == -INFINITY) ? 0.0 : exp(lse_off - lse);
  }

  const double mq = (mode == KD_TAIL || mode == KD_TAIL_REVERSE) ? (double)m_q[t] : 0.0;
  const double tiny = 1.1754943508222875e-38;
  const double mps = mp > tiny ? mp : tiny;
  const double ratio = (mode == KD_TAIL && mq > 0.0) ? mq / mps : 0.0;

  // per-entry terms; L accumulates in fp64
  double L = 0.0;
  for (int k = lane; k < nv; k += 64) {
    const double z = zS[t * K + k], tl = stlp[t * K + k];
    const double q = exp(tl);
    if (mode == KD_RENORM) {
      const double lqh = tl - lseq, lph = z - lseS;
      L += exp(lqh) * (lqh - lph);
    } else if (mode == KD_TAIL) {
      L += q * (tl - (z - lse));
    } else if (mode == KD_TAIL_REVERSE || mode == KD_REVERSE_TT) {
      L += exp(z - lse) * ((z - lse) - tl);
    } else if (mode == KD_FULL) {
      L += q * (tl - z);
    } else {
      const double lqh = tl - lseq, lph = z - lseS;
      L += exp(lph) * (lph - lqh);
    }
  }
  L = wave_sum_f64(L);
  if (mode == KD_TAIL && mq > 0.0) L += mq * (log(mq) - log(mps));
  // tail-token reverse KL: a_v = log(p_v / q_v) - log(m_p / m_q) on S, alpha = -sum_S p a
  const double tail_log = log(mps) - log(mq > tiny ? mq : tiny);
  double rev_A = 0.0;
  if (mode == KD_TAIL_REVERSE) {
    rev_A = L - tail_log * ((nv > 0) ? exp(lseS - lse) : 0.0);
    L += mp * tail_log;
  }
  if (mode == KD_FULL) L += Q * lse;
  const double Lkd = L;  // the distillation term alone (REVERSE's gradient uses it)

  // dense coefficient alpha_S as it acts on S (TAIL's -m_q/m_p acts off S only)
  double alpha = 0.0;
  if (mode == KD_TAIL) alpha = Q + mq;
  if (mode == KD_TAIL_REVERSE) alpha = -rev_A;
  if (mode == KD_FULL) alpha = Q;
  if (mode == KD_REVERSE_TT) alpha = -L;  // -sum_S p a, a = log p - log q
  const bool tt = mode == KD_REVERSE_TT;
  const int y = (labels != nullptr && (ce_weight != 0.f || tt)) ? labels[t] : -1;
  const bool has_y = y >= 0 && y < V;
  bool y_in_s = false;
  if (has_y)
    for (int k = lane; k < nv; k += 64) y_in_s = y_in_s || sidx[t * K + k] == y;
  y_in_s = __ballot(y_in_s) != 0ull;
  const double lam = (has_y && !tt) ? (double)ce_weight : 0.0;
  double yres = 0.0;  // unscaled residual at y outside S
  if (has_y && !tt) {
    L += lam * (lse - (double)tk[TK_ZY]);
    alpha += lam;
    yres = -lam;
  }
  if (has_y && tt && !y_in_s) {
    const double ell = ((double)tk[TK_ZY] - lse) - (double)tly[t];
    L += ell;
    alpha -= ell;
    yres = ell;
  }
  // off-S dense term A e^(z - B)
  double A = alpha, B = lse;
  if (mode == KD_TAIL && mq > 0.0) {
    if (lse_off == -INFINITY) {
      A = 0.0;  // S covers the vocabulary: nothing lies off S
      B = 0.0;
    } else {
      A = alpha * mp - mq;
      B = lse_off;
    }
  }
  for (int k = lane; k < K; k += 64) {
    double g = 0.0;  // dL/dz at the entry
    if (k < nv) {
      const double z = zS[t * K + k], tl = stlp[t * K + k];
      const double q = exp(tl), p = exp(z - lse);
      double r;
      if (mode == KD_RENORM) {
        r = exp(z - lseS) - exp(tl - lseq);
      } else if (mode == KD_TAIL || mode == KD_FULL) {
        r = -q;
      } else if (mode == KD_TAIL_REVERSE) {
        r = p * ((z - lse - tl) - tail_log);
      } else if (mode == KD_REVERSE_TT) {
        r = p * (z - lse - tl);
      } else {
        const double lph = z - lseS, lqh = tl - lseq;
        r = exp(lph) * (lph - lqh - Lkd);
      }
      if (has_y && !tt && sidx[t * K + k] == y) r -= lam;
      g = alpha * p + r;
    }
    coef[t * K + k] = (float)(scale * g);
  }
  // the full dz at y when it lies outside S
  double gy = 0.0;
  const bool y_out = has_y && !y_in_s && yres != 0.0;
  if (y_out) gy = (A != 0.0 ? A * exp((double)tk[TK_ZY] - B) : 0.0) + yres;
  if (ylab != nullptr && lane == 0) ylab[t] = y_out ? y : -1;
  if (lane == 0) {
    float* tw = tok + t * TOKF;
    tw[TK_LSE] = (float)lse;
    tw[TK_ALPHA] = (float)(scale * A);
    tw[TK_B] = (float)B;
    tw[TK_L] = (float)L;
    tw[TK_MP] = (float)mp;
    tw[TK_YR] = (float)(scale * gy);
    if (loss_tok) loss_tok[t] = (float)L;
    if (lse_out) lse_out[t] = (float)lse;
    if (mp_out) mp_out[t] = (float)mp;
  }
}

// loss = scale * sum_t L_t in a fixed order; NaN when the prep flagged bad
// indices (err may be NULL: no flag).
__global__ __launch_bounds__(1024) void k_loss_sum(int64_t T, float scale, const float* __restrict__ tok,
                                                   const int32_t* __restrict__ err, float* __restrict__ loss) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t t = threadIdx.x; t < T; t += 1024) s += (double)tok[t * TOKF + TK_L];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (err != nullptr && *err) ? __builtin_nanf("") : (float)(scale * red[0]);
}

// ---------------------------------------------------------------------------
// pass 2 (dense modes): recompute the z^T tile of one vocabulary chunk and
// write dz = A * exp(z - B) off S and the combine's full dz on S as bf16
// token rows,
// dz [Tp][Cp].  The tile is staged in LDS as E[t][v] (512-byte token rows,
// 16-byte chunks XOR-swizzled by zdz_swz(t)) and leaves in 16-byte stores,
// 32 threads per row.  Both backward GEMMs read dz in this one layout (the
// dW GEMM as an MN-major operand).
// ---------------------------------------------------------------------------
constexpr int ZDZ_PARK = (2 * TC::FN + 2) * TC::NT * 4;
// the 128 KB bf16 tile, or the operand stages and the parked values
constexpr int ZDZ_LDS = VT * TT * 2 > GEMM_LDS + ZDZ_PARK ? VT * TT * 2 : GEMM_LDS + ZDZ_PARK;

// Bijection on 0..31: 32 consecutive rows hit 32 distinct chunk positions
// (conflict-free stores), 4 consecutive rows fall into different aligned
// groups of 8 chunks (transposing reads).
__device__ __forceinline__ int zdz_swz(int t) { return ((t & 3) << 3) | ((t >> 2) & 7); }


// Dense part of dz for one tile into E: A * exp(z - B) as bf16 (the token's
// off-S term), zero for padding tokens (nl = -inf) and for rows masked to -inf.
__device__ __forceinline__ void zdz_dense(const Acc<TC>& acc, char* E, int64_t n0, int64_t T,
                                          const float (&lse_t)[TC::FN], const float (&al_t)[TC::FN], int wm, int wn,
                                          int lane) {
  const int rbase = wm * TC::TM + 4 * (lane >> 5);
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    const int tl = acc_col<TC>(wn, fn, lane);  // token row of E
    const float nl = (n0 + tl < T) ? -lse_t[fn] * KD_LOG2E : -KD_INF;
    const float a = al_t[fn];
    char* row = E + tl * (VT * 2);
    const int sw = zdz_swz(tl);
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = a * __builtin_amdgcn_exp2f(fmaf(acc.v[fm][fn][g * 4 + r], KD_LOG2E, nl));
        const int vl = rbase + fm * 32 + 8 * g;  // multiple of 4
        uint2 pk;
        pk.x = pack_bf16x2(x[0], x[1]);
        pk.y = pack_bf16x2(x[2], x[3]);
        *(uint2*)(row + (((vl >> 3) ^ sw) << 4) + (vl & 7) * 2) = pk;
      }
  }
}

// One pass-2 tile; MASK: the tile runs past the chunk end.
template <bool MASK>
__device__ __forceinline__ void zdz_tile(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                int64_t T, int64_t d, int64_t V, int K, int64_t Tp, int64_t Cp,
                                                int64_t c0, int64_t c1, int nCT, int nTT,
                                                const int32_t* __restrict__ sidx, const int2* __restrict__ starts,
                                                const float* __restrict__ tok, const float* __restrict__ zS,
                                                const float* __restrict__ coef, const int32_t* __restrict__ ylab,
                                                bf16_t* __restrict__ dz, int ct, int tt, bf16_t* lds) {
  const int64_t m0 = c0 + (int64_t)ct * VT, n0 = (int64_t)tt * TT;
  const int vt = (int)(m0 / VT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TC::WN, wn = wave % TC::WN;

  // per-token values fetched before the main loop and parked in LDS past the
  // operand stages (nothing stays live in registers across the loop): the
  // lanes' (lse, alpha) of their 4 token columns, and for thread tid, owner
  // of token row n0 + tid, its first retained index >= m0
  const int tid = threadIdx.x;
  const int64_t ts = n0 + tid;
  const int64_t vend = (m0 + VT < c1) ? m0 + VT : c1;
  {
    float* park = (float*)((char*)lds + GEMM_LDS);
#pragma unroll
    for (int fn = 0; fn < TC::FN; ++fn) {
      const int64_t t = n0 + acc_col<TC>(wn, fn, lane);
      const bool ok = t < T;
      park[(2 * fn) * TC::NT + tid] = ok ? tok[t * TOKF + TK_B] : 0.f;
      park[(2 * fn + 1) * TC::NT + tid] = ok ? tok[t * TOKF + TK_ALPHA] : 0.f;
    }
    int kc = K, vn = SENT;
    if (ts < T) {
      const int2 sf = starts[(int64_t)vt * Tp + ts];
      kc = sf.x;
      vn = sf.y;
    }
    ((int*)park)[(2 * TC::FN) * TC::NT + tid] = kc;
    ((int*)park)[(2 * TC::FN + 1) * TC::NT + tid] = vn;
  }

  Acc<TC> acc;
  gemm_tile_pipe<TC>(W, d, m0, c1, h, d, n0, T, (int)d, lds, acc);
  __syncthreads();  // every wavefront is done with the operand stages
  float lse_t[TC::FN], al_t[TC::FN];
  int kcur, vnext;
  {
    const float* park = (const float*)((const char*)lds + GEMM_LDS);
#pragma unroll
    for (int fn = 0; fn < TC::FN; ++fn) {
      lse_t[fn] = park[(2 * fn) * TC::NT + tid];
      al_t[fn] = park[(2 * fn + 1) * TC::NT + tid];
    }
    kcur = ((const int*)park)[(2 * TC::FN) * TC::NT + tid];
    vnext = ((const int*)park)[(2 * TC::FN + 1) * TC::NT + tid];
  }
  __syncthreads();  // parked values read before the epilogue reuses that LDS

  char* E = (char*)lds;
  if (MASK) mask_rows(acc, (int)(c1 - m0), wm, lane);  // tile rows inside the chunk
  zdz_dense(acc, E, n0, T, lse_t, al_t, wm, wn, lane);
  __syncthreads();
  // entries on S: their full dz, formed in fp64 by the combine
  if (vnext < vend) {
    char* row = E + tid * (VT * 2);
    const int sw = zdz_swz(tid);
    while (vnext < vend) {
      const int vl = vnext - (int)m0;
      *(bf16_t*)(row + (((vl >> 3) ^ sw) << 4) + (vl & 7) * 2) = f32_to_bf16(coef[ts * K + kcur]);
      ++kcur;
      vnext = kcur < K ? sidx[ts * K + kcur] : SENT;
    }
  }
  // label / sampled token outside S: its full dz, also from the combine
  if (ylab != nullptr && ts < T) {
    const int y = ylab[ts];
    if (y >= m0 && y < vend) {
      const float val = tok[ts * TOKF + TK_YR];
      const int vl = y - (int)m0;
      *(bf16_t*)(E + tid * (VT * 2) + (((vl >> 3) ^ zdz_swz(tid)) << 4) + (vl & 7) * 2) = f32_to_bf16(val);
    }
  }
  __syncthreads();

  // token rows: 32 threads per 512-byte row
  const int64_t vo = m0 - c0;
#pragma unroll 4
  for (int it = 0; it < TT / 8; ++it) {
    const int tl = it * 8 + (tid >> 5), c = tid & 31;
    const u32x4 q = *(const u32x4*)(E + tl * (VT * 2) + ((c ^ zdz_swz(tl)) << 4));
    // streamed past the caches (the chunk's dz, 0.5 GB at T = 32K, is far larger
    // than them): k_dhdw then reads it without competing write-backs
    __builtin_nontemporal_store(q, (u32x4*)(dz + (n0 + tl) * Cp + vo + c * 8));
  }
}

__global__ __launch_bounds__(256, 1) void k_zdz(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                int64_t T, int64_t d, int64_t V, int K, int64_t Tp, int64_t Cp,
                                                int64_t c0, int64_t c1, int nCT, int nTT,
                                                const int32_t* __restrict__ sidx, const int2* __restrict__ starts,
                                                const float* __restrict__ tok, const float* __restrict__ zS,
                                                const float* __restrict__ coef, const int32_t* __restrict__ ylab,
                                                bf16_t* __restrict__ dz) {
  extern __shared__ __align__(16) bf16_t lds[];
  int ct, tt;
  if (!tile_of(blockIdx.x, gridDim.x, nCT, nTT, 4, ct, tt)) return;
  if (c0 + (int64_t)(ct + 1) * VT > c1)
    zdz_tile<true>(W, h, T, d, V, K, Tp, Cp, c0, c1, nCT, nTT, sidx, starts, tok, zS, coef, ylab, dz, ct, tt, lds);
  else
    zdz_tile<false>(W, h, T, d, V, K, Tp, Cp, c0, c1, nCT, nTT, sidx, starts, tok, zS, coef, ylab, dz, ct, tt, lds);
}

// ---------------------------------------------------------------------------
// Token-block backward input: E (from k_pass1_store) becomes dz in place.
// Off S, dz = A e^(z - B) = A e^(m - B) E with m the tile maximum of the
// pass-1 partial; one thread per 8 consecutive vocabulary rows of a token
// row (16-byte loads and stores, RNE to bf16).  Padding token rows stay 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dz_scale(bf16_t* __restrict__ E, int64_t ldE, int64_t T, int64_t Tp,
                                                  const float2* __restrict__ part, const float* __restrict__ tok) {
  const int64_t t = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (t >= T || c >= ldE) return;
  const float A = tok[t * TOKF + TK_ALPHA], B = tok[t * TOKF + TK_B];
  const float m = part[(c / VT) * Tp + t].x;
  const float f = (A == 0.f || m == -KD_INF) ? 0.f : A * expf(m - B);
  u32x4* p = (u32x4*)(E + t * ldE + c);
  u32x4 q = __builtin_nontemporal_load(p);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    q[i] = pack_bf16x2(f * __uint_as_float(q[i] << 16), f * __uint_as_float(q[i] & 0xffff0000u));
  __builtin_nontemporal_store(q, p);
}

// The entries on S (the combine's full dz) and at a label / sampled token
// outside S: thread k < K of token t writes its sorted entry, thread K the
// token's label entry.
__global__ __launch_bounds__(256) void k_dz_entries(bf16_t* __restrict__ E, int64_t ldE, int64_t T, int K,
                                                    const int32_t* __restrict__ sidx, const float* __restrict__ coef,
                                                    const float* __restrict__ tok, const int32_t* __restrict__ ylab) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * (K + 1)) return;
  const int64_t t = i / (K + 1);
  const int k = (int)(i % (K + 1));
  if (k < K) {
    if (k < (int)tok[t * TOKF + TK_NV]) E[t * ldE + sidx[t * K + k]] = f32_to_bf16(coef[t * K + k]);
  } else if (ylab != nullptr) {
    const int y = ylab[t];
    if (y >= 0) E[t * ldE + y] = f32_to_bf16(tok[t * TOKF + TK_YR]);
  }
}

// ---------------------------------------------------------------------------
// dh / dW GEMMs of one chunk in a single launch.  Both are computed as
// transposed tiles (rows = feature j, columns = token t or vocabulary row v)
// so that each lane's accumulator group e = 4g..4g+3 holds four consecutive
// features of one output row: the epilogue moves float4s.
//   dh tiles: dh[t][j] (+)= sum_v W[c0+v][j] * dz[t][v]   (K = chunk rows;
//             W is read as an MN-major operand straight from its rows)
//   dW tiles: dW[c0+v][j] = sum_t h[t][j] * dz[t][v]      (K = Tp; both read
//             as MN-major operands: h's and dz's rows are token rows)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void k_dhdw(const bf16_t* __restrict__ dz, const bf16_t* __restrict__ W,
                                                 const bf16_t* __restrict__ h,
                                                 int64_t T, int64_t d, int64_t Tp, int64_t Cp, int64_t c0,
                                                 int64_t clen, int kdh, int first_chunk, int nTT, int nDT, int nCT,
                                                 int grid_dh, int dw_first, int dw_accum, float* __restrict__ dh,
                                                 float* __restrict__ dW) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TC::WN, wn = wave % TC::WN;
  Acc<TC> acc;
  // the class of tiles with the longer k-loop is dispatched first, so the
  // short ones fill the CUs at the end of the launch
  const int grid_dw = (int)gridDim.x - grid_dh;
  const bool is_dh = dw_first ? (int)blockIdx.x >= grid_dw : (int)blockIdx.x < grid_dh;
  const int bid = dw_first ? (is_dh ? (int)blockIdx.x - grid_dw : (int)blockIdx.x)
                           : (is_dh ? (int)blockIdx.x : (int)blockIdx.x - grid_dh);
  if (is_dh) {
    int dj, ti;
    if (!tile_of(bid, grid_dh, nDT, nTT, 4, dj, ti)) return;
    const int64_t m0 = (int64_t)dj * TC::BM, n0 = (int64_t)ti * TC::BN;
    gemm_tile_pipe<TC, true, false>(W + c0 * d, d, m0, d, dz, Cp, n0, Tp, kdh, lds, acc, (int)clen);
#pragma unroll
    for (int fn = 0; fn < TC::FN; ++fn) {
      const int64_t t = n0 + acc_col<TC>(wn, fn, lane);
      f32x4 x[TC::FM][4];
#pragma unroll
      for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t j = m0 + acc_row<TC>(wm, fm, 4 * g, lane);
          x[fm][g] = f32x4{acc.v[fm][fn][4 * g], acc.v[fm][fn][4 * g + 1], acc.v[fm][fn][4 * g + 2],
                           acc.v[fm][fn][4 * g + 3]};
          if (!first_chunk && t < T && j < d) x[fm][g] += *(const f32x4*)(dh + t * d + j);
        }
#pragma unroll
      for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t j = m0 + acc_row<TC>(wm, fm, 4 * g, lane);
          if (t < T && j < d) *(f32x4*)(dh + t * d + j) = x[fm][g];
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    int dj, ci;
    if (!tile_of(bid, grid_dw, nDT, nCT, 4, dj, ci)) return;
    const int64_t m0 = (int64_t)dj * TC::BM, n0 = (int64_t)ci * TC::BN;
    gemm_tile_pipe<TC, true, true>(h, d, m0, d, dz, Cp, n0, clen, (int)Tp, lds, acc, (int)T, (int)Tp);
#pragma unroll
    for (int fn = 0; fn < TC::FN; ++fn) {
      const int64_t v = n0 + acc_col<TC>(wn, fn, lane);
#pragma unroll
      for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t j = m0 + acc_row<TC>(wm, fm, 4 * g, lane);
          if (v < clen && j < d) {
            f32x4 x = f32x4{acc.v[fm][fn][4 * g], acc.v[fm][fn][4 * g + 1], acc.v[fm][fn][4 * g + 2],
                            acc.v[fm][fn][4 * g + 3]};
            if (dw_accum) x += *(const f32x4*)(dW + (c0 + v) * d + j);
            *(f32x4*)(dW + (c0 + v) * d + j) = x;
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Exact full-vocabulary KL(q || p) with the teacher rebuilt from a cached
// hidden state, q = softmax(U g + b) ("The Gradient That Top-k Distillation
// Never Computes", Figure 3 bottom).  Per token
//   L = sum_v q_v (log q_v - log p_v) = H_t - sum_v q_v z_v + lse,
//   H_t = sum_v q_v log q_v = E_q[zt] - lse_t,    dL/dz = p - q.
// Pass 1: logsumexp partials of the student and the teacher tiles (the
// teacher's also carry sum exp(x - m) (x - m), which gives E_q[zt]); per
// vocabulary chunk: the teacher tiles again -> q (fp32 [Tp, C] workspace),
// the student tiles -> dz = scale (p - q) and per-tile sums of q z, then the
// dh / dW GEMMs of the dense path.
// ---------------------------------------------------------------------------
constexpr int LP_RED = TC::WM * TT * 3 * 4;  // (m, s, u) per wavefront row and token
static_assert(LP_RED + VT * 4 <= GEMM_LDS, "lse-pass reduction space");

// Rows of the tile's accumulators get the bias of their vocabulary row
// (bl: the tile's VT biases in LDS).
__device__ __forceinline__ void add_row_bias(Acc<TC>& acc, const float* bl, int wm, int lane) {
#pragma unroll
  for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float bv = bl[acc_row<TC>(wm, fm, e, lane)];
#pragma unroll
      for (int fn = 0; fn < TC::FN; ++fn) acc.v[fm][fn][e] += bv;
    }
}

// Teacher tiles of an int8 cache (gscale != NULL) scale each token column by
// its position's scale before the bias.
template <bool TEACHER, bool MASK>
__device__ __forceinline__ void lse_tile(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, int64_t K,
                                         int64_t T, int64_t V, const float* __restrict__ bias,
                                         const float* __restrict__ gscale, int vt, int tt, int64_t Tp,
                                         float2* __restrict__ part, float4* __restrict__ partT, bf16_t* lds) {
  const int64_t m0 = (int64_t)vt * VT, n0 = (int64_t)tt * TT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TC::WN, wn = wave % TC::WN;
  Acc<TC> acc;
  gemm_tile_pipe<TC>(A, K, m0, V, B, K, n0, T, (int)K, lds, acc);
  __syncthreads();  // every wavefront is done with the operand stages
  float* red = (float*)lds;
  if (TEACHER) {
    if (gscale != nullptr) {
#pragma unroll
      for (int fn = 0; fn < TC::FN; ++fn) {
        const int64_t t = n0 + acc_col<TC>(wn, fn, lane);
        const float sc = t < T ? gscale[t] : 1.f;
#pragma unroll
        for (int fm = 0; fm < TC::FM; ++fm) acc.v[fm][fn] *= sc;
      }
    }
    float* bl = (float*)((char*)lds + LP_RED);
    for (int i = threadIdx.x; i < VT; i += TC::NT) bl[i] = (bias != nullptr && m0 + i < V) ? bias[m0 + i] : 0.f;
    __syncthreads();
    add_row_bias(acc, bl, wm, lane);
  }
  if (MASK) mask_rows(acc, (int)(V - m0), wm, lane);
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    float mx = -KD_INF;
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc.v[fm][fn][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float nm = (mx == -KD_INF) ? 0.f : -mx * KD_LOG2E;
    float s = 0.f, u = 0.f;
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = acc.v[fm][fn][e];
        const float ex = __builtin_amdgcn_exp2f(fmaf(x, KD_LOG2E, nm));
        s += ex;
        if (TEACHER) u += (ex > 0.f) ? ex * (x - mx) : 0.f;  // masked rows: 0, not 0 * -inf
      }
    s += __shfl_xor(s, 32, 64);
    if (TEACHER) u += __shfl_xor(u, 32, 64);
    const int col = acc_col<TC>(wn, fn, lane);
    if (lane < 32) {
      red[(wm * TT + col) * 3 + 0] = mx;
      red[(wm * TT + col) * 3 + 1] = s;
      red[(wm * TT + col) * 3 + 2] = u;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  for (int col = threadIdx.x; col < TT; col += TC::NT) {
    float M = -KD_INF;
#pragma unroll
    for (int w = 0; w < TC::WM; ++w) M = fmaxf(M, red[(w * TT + col) * 3]);
    float S = 0.f, Uq = 0.f;
#pragma unroll
    for (int w = 0; w < TC::WM; ++w) {
      const float mw = red[(w * TT + col) * 3], sw = red[(w * TT + col) * 3 + 1], uw = red[(w * TT + col) * 3 + 2];
      if (mw == -KD_INF) continue;
      const float f = __expf(mw - M);
      S += sw * f;
      if (TEACHER) Uq += f * (uw + (mw - M) * sw);
    }
    const int64_t t = n0 + col;
    if (t < T) {
      if (TEACHER)
        partT[(int64_t)vt * Tp + t] = make_float4(M, S, Uq, 0.f);
      else
        part[(int64_t)vt * Tp + t] = make_float2(M, S);
    }
  }
}

template <bool TEACHER>
__global__ __launch_bounds__(256, 1) void k_lse_pass(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
                                                     int64_t K, int64_t T, int64_t V, const float* __restrict__ bias,
                                                     const float* __restrict__ gscale, int nVT, int nTT, int64_t Tp,
                                                     float2* __restrict__ part, float4* __restrict__ partT) {
  extern __shared__ __align__(16) bf16_t lds[];
  int vt, tt;
  if (!tile_of(blockIdx.x, gridDim.x, nVT, nTT, 8, vt, tt)) return;
  if ((int64_t)(vt + 1) * VT > V)
    lse_tile<TEACHER, true>(A, B, K, T, V, bias, gscale, vt, tt, Tp, part, partT, lds);
  else
    lse_tile<TEACHER, false>(A, B, K, T, V, bias, gscale, vt, tt, Tp, part, partT, lds);
}

// Per token (one wavefront): student lse; teacher lse_t and H_t = E_q[zt] -
// lse_t from the (m, s, u) partials, merged in fp64.
// partT == nullptr: the teacher's logsumexp comes from lse_t_in, and its
// entropy term from the per-tile sums of k_teacher_q (added in k_kl_finish).
__global__ __launch_bounds__(256) void k_kl_combine(int64_t T, int nVT, int64_t Tp, float scale,
                                                    const float2* __restrict__ part,
                                                    const float4* __restrict__ partT,
                                                    const float* __restrict__ lse_t_in, float* __restrict__ tok) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  double m = -INFINITY, s = 0.0, mt = -INFINITY, st = 0.0, ut = 0.0;
  for (int vt = lane; vt < nVT; vt += 64) {
    const float2 p = part[(int64_t)vt * Tp + t];
    if (p.x != -INFINITY) {
      const double mn = fmax(m, (double)p.x);
      s = (m == -INFINITY ? 0.0 : s * exp(m - mn)) + (double)p.y * exp((double)p.x - mn);
      m = mn;
    }
    const float4 q = partT != nullptr ? partT[(int64_t)vt * Tp + t] : float4{-INFINITY, 0.f, 0.f, 0.f};
    if (q.x != -INFINITY) {
      const double mn = fmax(mt, (double)q.x);
      const double fo = (mt == -INFINITY) ? 0.0 : exp(mt - mn), fp = exp((double)q.x - mn);
      ut = (mt == -INFINITY ? 0.0 : fo * (ut + (mt - mn) * st)) + fp * ((double)q.z + ((double)q.x - mn) * (double)q.y);
      st = (mt == -INFINITY ? 0.0 : st * fo) + (double)q.y * fp;
      mt = mn;
    }
  }
  double M = m, Mt = mt;
  for (int o = 32; o > 0; o >>= 1) {
    M = fmax(M, __shfl_xor(M, o, 64));
    Mt = fmax(Mt, __shfl_xor(Mt, o, 64));
  }
  const double f = (m == -INFINITY) ? 0.0 : exp(m - M);
  const double ft = (mt == -INFINITY) ? 0.0 : exp(mt - Mt);
  s = wave_sum_f64(s * f);
  const double ut_l = (mt == -INFINITY) ? 0.0 : ft * (ut + (mt - Mt) * st);
  st = wave_sum_f64(st * ft);
  ut = wave_sum_f64(ut_l);
  if (lane == 0) {
    float* tk = tok + t * TOKF;
    tk[TK_LSE] = (float)(M + log(s));
    tk[TK_ALPHA] = scale;
    if (partT != nullptr) {
      tk[TK_LSEQ] = (float)(Mt + log(st));
      tk[TK_L] = (float)(ut / st - log(st));  // H_t = E_q[zt] - lse_t
    } else {
      tk[TK_LSEQ] = lse_t_in[t];
      tk[TK_L] = 0.f;
    }
  }
}

// q workspace layout: fragment-major per 256x256 (vocabulary x token) tile of
// a chunk, in the order (tile = tt * nCT + ct, wavefront, fn, fm, g, lane) with
// four fp32 per lane: element r of entry (fm, fn, g) is vocabulary row
// wm*128 + fm*32 + 8g + 4(lane/32) + r and token wn*128 + fn*32 + lane%32 of
// the tile, which is where the matrix-core accumulators of both heads hold
// them.  Each wavefront then writes and reads 1 KB contiguous per access.
__device__ __forceinline__ int64_t qfrag_index(int64_t tile, int wave, int fn, int fm, int g, int lane) {
  return ((((tile * (TC::WM * TC::WN) + wave) * TC::FN + fn) * TC::FM + fm) * 4 + g) * 64 + lane;
}

// Teacher tile of one chunk -> q = exp(U g + b - lse_t) (0 past the chunk end
// and for padding tokens), written straight from the accumulators.
__global__ __launch_bounds__(256, 1) void k_teacher_q(const bf16_t* __restrict__ U, const bf16_t* __restrict__ g,
                                                      const float* __restrict__ bias,
                                                      const float* __restrict__ gscale, int64_t T, int64_t dt,
                                                      int64_t c0, int64_t c1, int nCT, int nTT, int64_t Tp,
                                                      const float* __restrict__ tok, f32x4* __restrict__ qbuf,
                                                      float* __restrict__ partH) {
  extern __shared__ __align__(16) bf16_t lds[];
  int ct, tt;
  if (!tile_of(blockIdx.x, gridDim.x, nCT, nTT, 4, ct, tt)) return;
  const int64_t m0 = c0 + (int64_t)ct * VT, n0 = (int64_t)tt * TT;
  Acc<TC> acc;
  gemm_tile_pipe<TC>(U, dt, m0, c1, g, dt, n0, T, (int)dt, lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TC::WN, wn = wave % TC::WN;
  const int64_t rbase = m0 + wm * TC::TM + 4 * (lane >> 5);
  const int64_t tile = (int64_t)tt * nCT + ct;
  float nl[TC::FN], sc[TC::FN], hq[TC::FN];  // per token column; hq: sum of q log2 q over this lane's rows
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    const int64_t t = n0 + acc_col<TC>(wn, fn, lane);
    const bool tok_ok = t < T;
    nl[fn] = tok_ok ? -tok[t * TOKF + TK_LSEQ] * KD_LOG2E : -KD_INF;
    sc[fn] = (tok_ok && gscale != nullptr) ? gscale[t] : 1.f;
    hq[fn] = 0.f;
  }
#pragma unroll
  for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      float bv[4];  // bias of this lane's 4 rows; -inf past the chunk end
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t v = rbase + fm * 32 + 8 * gi + r;
        bv[r] = v < c1 ? (bias != nullptr ? bias[v] : 0.f) : -KD_INF;
      }
#pragma unroll
      for (int fn = 0; fn < TC::FN; ++fn) {
        f32x4 q;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float y = fmaf(acc.v[fm][fn][gi * 4 + r] * sc[fn] + bv[r], KD_LOG2E, nl[fn]);  // log2 q
          q[r] = __builtin_amdgcn_exp2f(y);
          hq[fn] += (q[r] != 0.f) ? q[r] * y : 0.f;
        }
        qbuf[qfrag_index(tile, wave, fn, fm, gi, lane)] = q;
      }
    }
  if (partH != nullptr) {
    // sum_v q_v log q_v of this tile per token, merged over the wavefront rows
    float* red = (float*)lds;
    __syncthreads();  // every wavefront is done with the operand stages
#pragma unroll
    for (int fn = 0; fn < TC::FN; ++fn) {
      const float hs = hq[fn] + __shfl_xor(hq[fn], 32, 64);
      if (lane < 32) red[wm * TT + acc_col<TC>(wn, fn, lane)] = hs;
    }
    __syncthreads();
    static_assert(TT == TC::NT, "one thread per token column");
    const int col = threadIdx.x;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < TC::WM; ++w) sum += red[w * TT + col];
    if (n0 + col < T) partH[(m0 / VT) * Tp + n0 + col] = sum * KD_LN2;
  }
}

// Student tile of one chunk: dz = scale (exp(z - lse) - q) as bf16 token rows
// (staged in LDS as in k_zdz), and per (vocabulary tile, token) the sum of
// q z, merged over the wavefront rows.
constexpr int ZK_LDS = ZDZ_LDS + TC::WM * TT * 4;

template <bool MASK>
__device__ __forceinline__ void zdz_kl_tile(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h, int64_t T,
                                            int64_t d, int64_t Tp, int64_t Cp, int64_t c0, int64_t c1,
                                            const float* __restrict__ tok, const f32x4* __restrict__ qbuf,
                                            float* __restrict__ partQZ, bf16_t* __restrict__ dz, int nCT, int ct,
                                            int tt, bf16_t* lds) {
  const int64_t m0 = c0 + (int64_t)ct * VT, n0 = (int64_t)tt * TT;
  const int vt = (int)(m0 / VT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TC::WN, wn = wave % TC::WN;
  const int64_t tile = (int64_t)tt * nCT + ct;
  Acc<TC> acc;
  gemm_tile_pipe<TC>(W, d, m0, c1, h, d, n0, T, (int)d, lds, acc);
  if (MASK) mask_rows(acc, (int)(c1 - m0), wm, lane);
  // Per-token constants and the q of the first token column are loaded before
  // the barrier; each column's loop then loads the next column's q.
  float nlv[TC::FN], av[TC::FN];
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    const int64_t t = n0 + acc_col<TC>(wn, fn, lane);
    nlv[fn] = t < T ? -tok[t * TOKF + TK_LSE] * KD_LOG2E : -KD_INF;
    av[fn] = t < T ? tok[t * TOKF + TK_ALPHA] : 0.f;
  }
  f32x4 qv[2][TC::FM][4];
#pragma unroll
  for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
    for (int g = 0; g < 4; ++g) qv[0][fm][g] = qbuf[qfrag_index(tile, wave, 0, fm, g, lane)];  // 0 for padding tokens
  __syncthreads();  // every wavefront is done with the operand stages
  char* E = (char*)lds;
  float* red = (float*)((char*)lds + ZDZ_LDS);
  const int rbase = wm * TC::TM + 4 * (lane >> 5);
#pragma unroll
  for (int fn = 0; fn < TC::FN; ++fn) {
    const int tl = acc_col<TC>(wn, fn, lane);
    const float nl = nlv[fn], a = av[fn];
    char* row = E + tl * (VT * 2);
    const int sw = zdz_swz(tl);
    float qz = 0.f;
    if (fn + 1 < TC::FN) {
#pragma unroll
      for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
        for (int g = 0; g < 4; ++g) qv[(fn + 1) & 1][fm][g] = qbuf[qfrag_index(tile, wave, fn + 1, fm, g, lane)];
    }
#pragma unroll
    for (int fm = 0; fm < TC::FM; ++fm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int vl = rbase + fm * 32 + 8 * g;  // multiple of 4
        const f32x4 q = qv[fn & 1][fm][g];
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = acc.v[fm][fn][g * 4 + r];
          x[r] = a * (__builtin_amdgcn_exp2f(fmaf(z, KD_LOG2E, nl)) - q[r]);
          qz += (q[r] != 0.f) ? q[r] * z : 0.f;  // masked rows: q = 0, z = -inf
        }
        uint2 pk;
        pk.x = pack_bf16x2(x[0], x[1]);
        pk.y = pack_bf16x2(x[2], x[3]);
        *(uint2*)(row + (((vl >> 3) ^ sw) << 4) + (vl & 7) * 2) = pk;
      }
    qz += __shfl_xor(qz, 32, 64);
    if (lane < 32) red[wm * TT + tl] = qz;
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  for (int col = threadIdx.x; col < TT; col += TC::NT) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < TC::WM; ++w) sum += red[w * TT + col];
    if (n0 + col < T) partQZ[(int64_t)vt * Tp + n0 + col] = sum;
  }
  const int tid = threadIdx.x;
  const int64_t vo = m0 - c0;
#pragma unroll 4
  for (int it = 0; it < TT / 8; ++it) {
    const int tl = it * 8 + (tid >> 5), cc = tid & 31;
    const u32x4 q = *(const u32x4*)(E + tl * (VT * 2) + ((cc ^ zdz_swz(tl)) << 4));
    __builtin_nontemporal_store(q, (u32x4*)(dz + (n0 + tl) * Cp + vo + cc * 8));  // as in k_zdz
  }
}

__global__ __launch_bounds__(256, 1) void k_zdz_kl(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                   int64_t T, int64_t d, int64_t Tp, int64_t Cp, int64_t c0,
                                                   int64_t c1, int nCT, int nTT, const float* __restrict__ tok,
                                                   const f32x4* __restrict__ qbuf, float* __restrict__ partQZ,
                                                   bf16_t* __restrict__ dz) {
  extern __shared__ __align__(16) bf16_t lds[];
  int ct, tt;
  if (!tile_of(blockIdx.x, gridDim.x, nCT, nTT, 4, ct, tt)) return;
  if (c0 + (int64_t)(ct + 1) * VT > c1)
    zdz_kl_tile<true>(W, h, T, d, Tp, Cp, c0, c1, tok, qbuf, partQZ, dz, nCT, ct, tt, lds);
  else
    zdz_kl_tile<false>(W, h, T, d, Tp, Cp, c0, c1, tok, qbuf, partQZ, dz, nCT, ct, tt, lds);
}

// L_t = H_t - sum_v q_v z_v + lse, with H_t = sum_v q_v log q_v from the
// teacher partials (k_kl_combine) or, with a cached teacher logsumexp, from
// the per-tile sums partH.  A workgroup covers 32 tokens; its 32
// groups of 32 threads each sum every 32nd vocabulary tile (coalesced across
// tokens), and the group sums are added in group order (deterministic).
__global__ __launch_bounds__(1024) void k_kl_finish(int64_t T, int nVT, int64_t Tp, const float* __restrict__ partQZ,
                                                    const float* __restrict__ partH, float* __restrict__ tok,
                                                    float* __restrict__ loss_tok, float* __restrict__ lse_out,
                                                    float* __restrict__ lset_out) {
  __shared__ double red[32][33];
  const int tl = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int64_t t = (int64_t)blockIdx.x * 32 + tl;
  double part = 0.0;  // sum over tiles of (sum q log q, when given) - sum q z
  if (t < T)
    for (int vt = grp; vt < nVT; vt += 32) {
      part -= (double)partQZ[(int64_t)vt * Tp + t];
      if (partH != nullptr) part += (double)partH[(int64_t)vt * Tp + t];
    }
  red[grp][tl] = part;
  __syncthreads();
  if (grp != 0 || t >= T) return;
  double acc = 0.0;
  for (int g = 0; g < 32; ++g) acc += red[g][tl];
  float* tk = tok + t * TOKF;
  const float L = (float)((double)tk[TK_L] + acc + (double)tk[TK_LSE]);
  tk[TK_L] = L;
  if (loss_tok) loss_tok[t] = L;
  if (lse_out) lse_out[t] = tk[TK_LSE];
  if (lset_out) lset_out[t] = tk[TK_LSEQ];
}

// int8 hidden-state cache: per position s = max|g| / 127 and codes rint(g / s)
// clamped to [-127, 127], in fp32 with IEEE division (a zero row: s = 0, zero
// codes).  One workgroup per position.
__global__ __launch_bounds__(256) void k_quantize_int8(const bf16_t* __restrict__ g, int64_t d,
                                                       int8_t* __restrict__ codes, float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const bf16_t* gr = g + t * d;
  float amax = 0.f;
  for (int64_t j = threadIdx.x; j < d; j += 256) amax = fmaxf(amax, fabsf(bf16_to_f32(gr[j])));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 127.f);
  for (int64_t j = threadIdx.x; j < d; j += 256) {
    float q = 0.f;
    if (s > 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(bf16_to_f32(gr[j]), s)), -127.f), 127.f);
    codes[t * d + j] = (int8_t)q;
  }
  if (threadIdx.x == 0) scale[t] = s;
}

// int8 codes -> bf16 (exact: |code| <= 127 fits bf16's 8 significant bits).
__global__ void k_codes_to_bf16(const int8_t* __restrict__ codes, int64_t n, bf16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (bf16_t)(__float_as_uint((float)codes[i]) >> 16);
}

// ---------------------------------------------------------------------------
// Sparse backward (RENORM, REVERSE): dz is zero off S.
// ---------------------------------------------------------------------------
// dh[t] = sum_k r_tk W[s_tk], k ascending.  One workgroup per token.
__global__ __launch_bounds__(256) void k_sparse_dh(const bf16_t* __restrict__ W, int64_t d, int K,
                                                   const int32_t* __restrict__ sidx, const float* __restrict__ coef,
                                                   const float* __restrict__ tok, float* __restrict__ dh) {
  const int64_t t = blockIdx.x;
  const int nv = (int)tok[t * TOKF + TK_NV];
  for (int64_t j0 = (int64_t)threadIdx.x * 8; j0 < d; j0 += 256 * 8) {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < nv; ++k) {
      const int v = sidx[t * K + k];
      const float r = coef[t * K + k];
      const u32x4 w = *(const u32x4*)(W + (int64_t)v * d + j0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[2 * i] = fmaf(r, __uint_as_float(w[i] << 16), a[2 * i]);
        a[2 * i + 1] = fmaf(r, __uint_as_float(w[i] & 0xffff0000u), a[2 * i + 1]);
      }
    }
    float4* o = (float4*)(dh + t * d + j0);
    o[0] = make_float4(a[0], a[1], a[2], a[3]);
    o[1] = make_float4(a[4], a[5], a[6], a[7]);
  }
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// Count retained entries per vocabulary row (integer atomics: exact).
__global__ void k_csr_count(int64_t T, int K, const int32_t* __restrict__ sidx, const float* __restrict__ tok,
                            int32_t* __restrict__ cnt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * K) return;
  const int64_t t = i / K;
  const int k = (int)(i % K);
  if (k < (int)tok[t * TOKF + TK_NV]) atomicAdd(&cnt[sidx[i]], 1);
}

// Exclusive scan of cnt[0..n) into off[0..n] in segments of SCAN_SEG:
// k_seg_sum sums each segment, k_seg_scan scans it after adding the sums of
// the segments before it (few: n / SCAN_SEG).
constexpr int SCAN_SEG = 4096;  // 256 threads x 16 elements

__global__ __launch_bounds__(256) void k_seg_sum(const int32_t* __restrict__ cnt, int64_t n,
                                                 int32_t* __restrict__ segsum) {
  __shared__ int32_t red[4];
  const int64_t b = (int64_t)blockIdx.x * SCAN_SEG;
  int32_t s = 0;
  for (int i = threadIdx.x; i < SCAN_SEG; i += 256) s += (b + i < n) ? cnt[b + i] : 0;
  s = wave_sum_i32(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) segsum[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void k_seg_scan(const int32_t* __restrict__ cnt, int64_t n,
                                                  const int32_t* __restrict__ segsum, int nseg,
                                                  int32_t* __restrict__ off) {
  __shared__ int32_t wsum[4];
  __shared__ int32_t base_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (w == 0) {
    int32_t p = 0;
    for (int i = lane; i < (int)blockIdx.x; i += 64) p += segsum[i];
    p = wave_sum_i32(p);
    if (lane == 0) base_s = p;
  }
  const int64_t b = (int64_t)blockIdx.x * SCAN_SEG + tid * 16;
  int32_t v[16], t = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = (b + i < n) ? cnt[b + i] : 0;
    t += v[i];
  }
  // inclusive scan of the thread totals: within the wavefront, then across
  int32_t x = t;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int32_t run = base_s + x - t;
  for (int i = 0; i < w; ++i) run += wsum[i];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (b + i < n) off[b + i] = run;
    run += v[i];
  }
  if ((int)blockIdx.x == nseg - 1 && tid == 255) off[n] = run;
}

// Scatter entries (token, coefficient) into their vocabulary row's bucket.
// The order inside a bucket is arbitrary; the consumer is order-independent.
__global__ void k_csr_fill(int64_t T, int K, const int32_t* __restrict__ sidx, const float* __restrict__ coef,
                           const float* __restrict__ tok, const int32_t* __restrict__ off, int32_t* __restrict__ fillc,
                           int32_t* __restrict__ ent_t, float* __restrict__ ent_r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * K) return;
  const int64_t t = i / K;
  const int k = (int)(i % K);
  if (k >= (int)tok[t * TOKF + TK_NV]) return;
  const int v = sidx[i];
  const int pos = off[v] + atomicAdd(&fillc[v], 1);
  ent_t[pos] = (int32_t)t;
  ent_r[pos] = coef[i];
}

// dW rows of the sparse backward, SDW_ROWS vocabulary rows per workgroup and
// four consecutive features per thread (d % 64 == 0).  A row without entries
// is written as zeros, one entry as its product.  A row with 2..SDW_SORT
// entries (the tokens of a row are distinct for valid input) has them ranked by token in LDS
// and summed in fp32 in token order; a longer one (a vocabulary row shared by
// more than SDW_SORT tokens) takes an exact fixed-point sum.  Both orders are
// fixed, so dW does not depend on the order the CSR fill wrote the entries.
constexpr int SDW_ROWS = 4;
constexpr int SDW_SORT = 1024;

__device__ __forceinline__ float sparse_dw_elem(const bf16_t* __restrict__ h, int64_t d, int64_t j,
                                                const int32_t* __restrict__ ent_t, const float* __restrict__ ent_r,
                                                int b, int n) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) {
    const double p = (double)ent_r[b + i] * (double)bf16_to_f32(h[(int64_t)ent_t[b + i] * d + j]);
    amax = fmax(amax, fabs(p));
  }
  if (amax == 0.0) return 0.f;
  int ex;
  frexp(amax * (double)n, &ex);  // amax*n < 2^ex
  const int sh = 61 - ex;
  long long acc = 0;
  for (int i = 0; i < n; ++i) {
    const double p = (double)ent_r[b + i] * (double)bf16_to_f32(h[(int64_t)ent_t[b + i] * d + j]);
    acc += llrint(ldexp(p, sh));
  }
  return (float)ldexp((double)acc, -sh);
}

__device__ __forceinline__ f32x4 bf16x4_scaled(const bf16_t* p, float r) {
  const uint2 hv = *(const uint2*)p;
  return f32x4{r * __uint_as_float(hv.x << 16), r * __uint_as_float(hv.x & 0xffff0000u),
               r * __uint_as_float(hv.y << 16), r * __uint_as_float(hv.y & 0xffff0000u)};
}

__global__ __launch_bounds__(256) void k_sparse_dw(const bf16_t* __restrict__ h, int64_t d, int64_t V,
                                                   const int32_t* __restrict__ off, const int32_t* __restrict__ ent_t,
                                                   const float* __restrict__ ent_r, float* __restrict__ dW) {
  __shared__ int32_t tin[SDW_SORT], ts[SDW_SORT];
  __shared__ float rs[SDW_SORT];
  const int64_t d4 = d >> 2;
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int r = 0; r < SDW_ROWS; ++r) {
    const int64_t v = (int64_t)blockIdx.x * SDW_ROWS + r;
    if (v >= V) return;
    const int b = off[v], n = off[v + 1] - b;
    f32x4* row = (f32x4*)(dW + v * d);
    if (n == 0) {
      for (int64_t j4 = tid; j4 < d4; j4 += 256) row[j4] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (n == 1) {
      const float rr = ent_r[b];
      const bf16_t* hr = h + (int64_t)ent_t[b] * d;
      for (int64_t j4 = tid; j4 < d4; j4 += 256) row[j4] = bf16x4_scaled(hr + 4 * j4, rr);
    } else if (n <= SDW_SORT) {
      for (int i = tid; i < n; i += 256) tin[i] = ent_t[b + i];
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        // equal tokens (only from a duplicated index, an input error) are
        // ranked by position, so the ranks stay a permutation of 0..n-1
        const int ti = tin[i];
        int rank = 0;
        for (int j = 0; j < n; ++j) rank += (tin[j] < ti) || (tin[j] == ti && j < i);
        ts[rank] = ti;
        rs[rank] = ent_r[b + i];
      }
      __syncthreads();
      for (int64_t j4 = tid; j4 < d4; j4 += 256) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < n; ++i) {
          const f32x4 x = bf16x4_scaled(h + (int64_t)ts[i] * d + 4 * j4, 1.f);
          acc[0] = fmaf(rs[i], x[0], acc[0]);
          acc[1] = fmaf(rs[i], x[1], acc[1]);
          acc[2] = fmaf(rs[i], x[2], acc[2]);
          acc[3] = fmaf(rs[i], x[3], acc[3]);
        }
        row[j4] = acc;
      }
      __syncthreads();  // the next row reuses tin, ts, rs
    } else {
      for (int64_t j4 = tid; j4 < d4; j4 += 256) {
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = sparse_dw_elem(h, d, 4 * j4 + e, ent_t, ent_r, b, n);
        row[j4] = out;
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

struct LossPlan {
  int64_t T, d, V, Tp, Cp, C;
  int64_t TB, Vp;                                    // token-block path: tokens per block, E row pitch (0: chunked)
  int K, Kp2, mode, nVT, nTT, nDT, nchunks;
  bool ce, dense;                                    // label term; dense backward
  size_t o_sidx, o_stlp, o_zS, o_coef, o_tok, o_starts, o_part, o_err, o_ylab;
  size_t o_dz;                                       // dense modes
  size_t o_cnt, o_off, o_fill, o_entt, o_entr, o_seg; // sparse modes
  size_t total;
};

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// ce: a hard-label cross-entropy term is present (its dense gradient makes
// every mode take the dense backward).
// tb > 0 (dense modes): the token-block path, tb tokens (rounded up to 256)
// per block with their [tb, V] bf16 logit block kept in the workspace.
static bool plan_loss(int64_t T, int64_t d, int64_t V, int32_t K, int32_t mode, int32_t chunk, bool ce,
                      LossPlan& p, int64_t tb = 0) {
  if (T < 0 || d <= 0 || V <= 0 || K < 1 || K > KMAX || K > V || d % 64 != 0 || d > 16384 || chunk <= 0) return false;
  if (tb < 0) return false;
  if (mode < KD_RENORM || mode > KD_REVERSE_TT) return false;
  if (V > (int64_t)1 << 30 || T > (int64_t)1 << 26) return false;
  p.T = T;
  p.d = d;
  p.V = V;
  p.K = K;
  p.mode = mode;
  p.ce = ce;
  p.dense = (mode == KD_TAIL || mode == KD_FULL || mode == KD_TAIL_REVERSE || mode == KD_REVERSE_TT || ce);
  // the sparse backward's CSR offsets and positions are int32
  if (!p.dense && (uint64_t)T * (uint64_t)K >= ((uint64_t)1 << 31)) return false;
  p.Kp2 = 1;
  while (p.Kp2 < K) p.Kp2 <<= 1;
  p.Tp = kd_round_up(T > 0 ? T : 1, TT);
  p.C = kd_round_up(chunk, VT);
  if (p.C > kd_round_up(V, VT)) p.C = kd_round_up(V, VT);
  p.Cp = p.C;
  // the GEMMs address MN-major operands (a chunk of W, h, dz) with 32-bit byte offsets
  const uint64_t lim = (uint64_t)1 << 32;
  const uint64_t Tp64 = (uint64_t)kd_round_up(T > 0 ? T : 1, TT);
  if ((uint64_t)p.C * (uint64_t)d * 2u >= lim || Tp64 * (uint64_t)d * 2u >= lim || Tp64 * (uint64_t)p.C * 2u >= lim)
    return false;
  p.nVT = (int)kd_ceil_div(V, VT);
  p.nTT = (int)(p.Tp / TT);
  p.nDT = (int)kd_ceil_div(d, TC::BN);
  p.nchunks = (int)kd_ceil_div(V, p.C);
  size_t o = 0;
  const size_t TK = (size_t)(T > 0 ? T : 1) * K;
  p.o_sidx = o; o = align_up(o + TK * 4);
  p.o_stlp = o; o = align_up(o + TK * 4);
  p.o_zS = o; o = align_up(o + TK * 4);
  p.o_coef = o; o = align_up(o + TK * 4);
  p.o_tok = o; o = align_up(o + (size_t)p.Tp * TOKF * 4);
  p.o_starts = o; o = align_up(o + (size_t)p.nVT * p.Tp * 8);
  p.o_part = o; o = align_up(o + (size_t)p.nVT * p.Tp * 8);
  p.o_err = o; o = align_up(o + 4);
  p.o_ylab = 0;
  if (ce || mode == KD_REVERSE_TT) {
    p.o_ylab = o; o = align_up(o + (size_t)(T > 0 ? T : 1) * 4);
  }
  p.o_dz = 0;
  p.o_cnt = p.o_off = p.o_fill = p.o_entt = p.o_entr = p.o_seg = 0;
  p.TB = p.Vp = 0;
  if (p.dense && tb > 0) {
    p.TB = kd_round_up(tb, TT);
    if (p.TB > p.Tp) p.TB = p.Tp;
    p.Vp = kd_round_up(V, VT);
    // the dW GEMM reads the block as an MN-major operand with 32-bit byte offsets
    if ((uint64_t)p.TB * (uint64_t)p.Vp * 2u >= lim || (uint64_t)p.Vp * (uint64_t)d * 2u >= lim) return false;
    p.o_dz = o; o = align_up(o + (size_t)p.TB * p.Vp * 2);
  } else if (p.dense) {
    p.o_dz = o; o = align_up(o + (size_t)p.Tp * p.Cp * 2);
  } else {
    p.o_cnt = o; o = align_up(o + (size_t)(V + 1) * 4);
    p.o_off = o; o = align_up(o + (size_t)(V + 1) * 4);
    p.o_fill = o; o = align_up(o + (size_t)(V + 1) * 4);
    p.o_entt = o; o = align_up(o + TK * 4);
    p.o_entr = o; o = align_up(o + TK * 4);
    p.o_seg = o; o = align_up(o + (size_t)kd_ceil_div(V, SCAN_SEG) * 4);
  }
  p.total = o;
  return true;
}

template <typename T>
static T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

}  // namespace

extern "C" size_t kd_topk_loss_workspace(int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode, int32_t chunk) {
  LossPlan p;
  if (!plan_loss(T, d, V, K, mode, chunk, false, p)) return 0;
  return p.total;
}

extern "C" size_t kd_topk_loss_ce_workspace(int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode, int32_t chunk,
                                            float ce_weight) {
  LossPlan p;
  if (!plan_loss(T, d, V, K, mode, chunk, ce_weight != 0.f, p)) return 0;
  return p.total;
}

extern "C" size_t kd_topk_loss_tokblock_workspace(int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode,
                                                 int32_t token_block) {
  LossPlan p;
  if (token_block <= 0 || !plan_loss(T, d, V, K, mode, 8192, false, p, token_block)) return 0;
  return p.total;
}

#define KD_LAUNCH_CHECK()                                                              \
  do {                                                                                 \
    hipError_t e_ = hipGetLastError();                                                 \
    if (e_ != hipSuccess) return kd_fail(KD_EHIP, "launch failed: %s", hipGetErrorString(e_)); \
  } while (0)

// The loss with optional per-token tokens: labels + ce_weight (cross-entropy
// term) or, for KD_REVERSE_TT, sampled tokens + their teacher log-probs tly.
// st_lse / st_z (optional, together): the student's logsumexp [T] and its
// logits at idx [T, K], already known; the forward GEMM (pass 1) is skipped.
static kd_status loss_impl(const kd_bf16* h, const kd_bf16* W, const int32_t* idx, const float* teacher_logp,
                           const float* m_q, const int32_t* labels, float ce_weight, const float* tly, int64_t T,
                           int64_t d, int64_t V, int32_t K, int32_t mode, int32_t chunk, float scale, float* loss,
                           float* loss_tok, float* lse, float* m_p, float* dh, float* dW, void* ws, size_t ws_bytes,
                           void* stream, const float* st_lse = nullptr, const float* st_z = nullptr,
                           int64_t tb = 0) {
  LossPlan p;
  const bool given = st_lse != nullptr || st_z != nullptr;
  if (given && T > 0 && (st_lse == nullptr || st_z == nullptr))
    return kd_fail(KD_EINVAL, "the student's logsumexp and its logits at idx come together");
  if (mode < KD_RENORM || mode > KD_REVERSE_TT) return kd_fail(KD_EINVAL, "unknown mode %d", (int)mode);
  if (mode == KD_REVERSE_TT && ce_weight != 0.f)
    return kd_fail(KD_EINVAL, "KD_REVERSE_TT takes no cross-entropy term");
  if (mode == KD_REVERSE_TT && labels != nullptr && T > 0 && !tly)
    return kd_fail(KD_EINVAL, "sampled tokens need their teacher log-probabilities");
  if (!(ce_weight == ce_weight) || ce_weight < 0.f || ce_weight > 3.4e38f)
    return kd_fail(KD_EINVAL, "ce_weight must be finite and >= 0 (got %g)", (double)ce_weight);
  const bool ce = ce_weight != 0.f;
  if (ce && T > 0 && !labels) return kd_fail(KD_EINVAL, "ce_weight != 0 needs labels");
  const bool with_y = ce || (mode == KD_REVERSE_TT && labels != nullptr);
  if (!(mode == KD_TAIL || mode == KD_FULL || mode == KD_TAIL_REVERSE || mode == KD_REVERSE_TT || ce) && T > 0 &&
      (uint64_t)T * (uint64_t)K >= ((uint64_t)1 << 31))
    return kd_fail(KD_EUNSUPPORTED, "sparse modes need T*K < 2^31 (got T=%lld K=%d)", (long long)T, (int)K);
  if (tb > 0 && given) return kd_fail(KD_EINVAL, "the token-block path computes the student's logits itself");
  if (!plan_loss(T, d, V, K, mode, chunk, ce, p, tb))
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld d=%lld V=%lld K=%d chunk=%d (need 1<=K<=min(V,1024), d%%64==0, d<=16384, chunk>0, and chunk*d, T*d, T*chunk bf16 each < 4 GiB)",
                   (long long)T, (long long)d, (long long)V, (int)K, (int)chunk);
  if (!loss || !dW || !W) return kd_fail(KD_EINVAL, "null required pointer (loss, W, dW)");
  if (T > 0 && (!h || !idx || !teacher_logp || !dh)) return kd_fail(KD_EINVAL, "null required pointer (h, idx, teacher_logp, dh)");
  if (T > 0 && (mode == KD_TAIL || mode == KD_TAIL_REVERSE) && !m_q)
    return kd_fail(KD_EINVAL, "KD_TAIL and KD_TAIL_REVERSE need m_q");
  if (!ws || ws_bytes < p.total)
    return kd_fail(KD_ENOWS, "workspace too small: need %zu bytes, got %zu", p.total, ws_bytes);
  if (!kd_aligned16(W) || !kd_aligned16(dW) || !kd_aligned16(ws) || (T > 0 && (!kd_aligned16(h) || !kd_aligned16(dh))))
    return kd_fail(KD_EINVAL, "h, W, dh, dW and ws must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;

  int32_t* err = at<int32_t>(ws, p.o_err);
  KD_LAUNCH(k_fill_i32, dim3(1), dim3(64), 0, s, err, (int64_t)1, 0);
  KD_LAUNCH_CHECK();
  if (T == 0) {
    KD_LAUNCH(k_fill_i32, dim3(1024), dim3(256), 0, s, (int32_t*)dW, V * d, 0);
    KD_LAUNCH(k_loss_sum, dim3(1), dim3(1024), 0, s, (int64_t)0, scale, at<float>(ws, p.o_tok), err, loss);
    KD_LAUNCH_CHECK();
    return KD_OK;
  }
  int32_t* sidx = at<int32_t>(ws, p.o_sidx);
  float* stlp = at<float>(ws, p.o_stlp);
  float* zS = at<float>(ws, p.o_zS);
  float* coef = at<float>(ws, p.o_coef);
  float* tok = at<float>(ws, p.o_tok);
  int2* starts = at<int2>(ws, p.o_starts);
  float2* part = at<float2>(ws, p.o_part);

  KD_LAUNCH(k_prep, dim3((unsigned)(8 * kd_ceil_div(T, 8))), dim3(64), 0, s, idx, teacher_logp, given ? st_z : (const float*)nullptr, T, V,
            (int)K, p.Kp2, p.nVT, p.Tp, sidx, stlp, given ? zS : (float*)nullptr, starts, tok, err);
  KD_LAUNCH_CHECK();
  if (p.TB > 0) {
    // Token-block path: per block of TB tokens, pass 1 keeps the block's
    // logits as E (bf16), the combine gives the block's coefficients, E
    // becomes dz in place and one dh / dW launch covers the whole
    // vocabulary (dh written, dW accumulated over the blocks).
    KD_LAUNCH(k_fill_i32, dim3(256), dim3(256), 0, s, (int32_t*)zS, T * K, 0);
    int32_t* ylab = with_y ? at<int32_t>(ws, p.o_ylab) : nullptr;
    if (with_y) {
      KD_LAUNCH(k_label_logit, dim3((unsigned)kd_ceil_div(T, 4)), dim3(256), 0, s, (const bf16_t*)h, (const bf16_t*)W,
                labels, T, d, V, tok, err);
      KD_LAUNCH_CHECK();
    }
    bf16_t* E = at<bf16_t>(ws, p.o_dz);
    const int nDT = p.nDT;
    for (int64_t t0 = 0; t0 < T; t0 += p.TB) {
      const int64_t tb = (T - t0 < p.TB) ? T - t0 : p.TB;
      const int nTTb = (int)kd_ceil_div(tb, TT);
      const int64_t rows = (int64_t)nTTb * TT;
      const int g1 = grid_of(p.nVT * nTTb);
      KD_LAUNCH(k_pass1_store, dim3(g1), dim3(TC::NT), P1S_LDS, s, (const bf16_t*)W, (const bf16_t*)h + t0 * d, tb, d,
                V, (int)K, p.nVT, nTTb, p.Tp, sidx + t0 * K, starts + t0, zS + t0 * K, part + t0, E, p.Vp);
      KD_LAUNCH(k_combine, dim3((unsigned)kd_ceil_div(tb, 4)), dim3(256), 0, s, tb, (int)K, p.nVT, p.Tp, (int)mode,
                scale, part + t0, zS + t0 * K, sidx + t0 * K, stlp + t0 * K, m_q ? m_q + t0 : nullptr,
                with_y ? labels + t0 : nullptr, ce_weight, tly ? tly + t0 : nullptr, V, tok + t0 * TOKF, coef + t0 * K,
                ylab ? ylab + t0 : nullptr, loss_tok ? loss_tok + t0 : nullptr, lse ? lse + t0 : nullptr,
                m_p ? m_p + t0 : nullptr, (const float*)nullptr);
      KD_LAUNCH(k_dz_scale, dim3((unsigned)kd_ceil_div(p.Vp, 2048), (unsigned)tb), dim3(256), 0, s, E, p.Vp, tb, p.Tp,
                (const float2*)part + t0, (const float*)tok + t0 * TOKF);
      KD_LAUNCH(k_dz_entries, dim3((unsigned)kd_ceil_div(tb * (K + 1), 256)), dim3(256), 0, s, E, p.Vp, tb, (int)K,
                (const int32_t*)sidx + t0 * K, (const float*)coef + t0 * K, (const float*)tok + t0 * TOKF,
                (const int32_t*)(ylab ? ylab + t0 : nullptr));
      KD_LAUNCH_CHECK();
      const int kdh = (int)kd_round_up(V, 64);
      const int gdh = grid_of(nTTb * nDT);
      const int nCTw = (int)kd_ceil_div(V, TC::BN);
      const int gdw = grid_of(nCTw * nDT);
      KD_LAUNCH(k_dhdw, dim3(gdh + gdw), dim3(TC::NT), GEMM_LDS, s, (const bf16_t*)E, (const bf16_t*)W,
                (const bf16_t*)h + t0 * d, tb, d, rows, p.Vp, (int64_t)0, V, kdh, 1, nTTb, nDT, nCTw, gdh,
                rows > kdh ? 1 : 0, t0 > 0 ? 1 : 0, dh + t0 * d, dW);
      KD_LAUNCH_CHECK();
    }
    KD_LAUNCH(k_loss_sum, dim3(1), dim3(1024), 0, s, T, scale, tok, err, loss);
    KD_LAUNCH_CHECK();
    return KD_OK;
  }
  if (!given) {
    // zero the gathered logits so padding slots read as finite values
    KD_LAUNCH(k_fill_i32, dim3(256), dim3(256), 0, s, (int32_t*)zS, T * K, 0);
    const int g1 = grid_of(p.nVT * p.nTT);
    KD_LAUNCH(k_pass1, dim3(g1), dim3(TC::NT), P1_LDS, s, (const bf16_t*)W, (const bf16_t*)h, T, d, V, (int)K,
              p.nVT, p.nTT, p.Tp, sidx, starts, zS, part);
    KD_LAUNCH_CHECK();
  }
  int32_t* ylab = with_y ? at<int32_t>(ws, p.o_ylab) : nullptr;
  if (with_y) {
    KD_LAUNCH(k_label_logit, dim3((unsigned)kd_ceil_div(T, 4)), dim3(256), 0, s, (const bf16_t*)h, (const bf16_t*)W,
                       labels, T, d, V, tok, err);
    KD_LAUNCH_CHECK();
  }
  KD_LAUNCH(k_combine, dim3((unsigned)kd_ceil_div(T, 4)), dim3(256), 0, s, T, (int)K, p.nVT, p.Tp, (int)mode,
                     scale, part, zS, sidx, stlp, m_q, with_y ? labels : nullptr, ce_weight, tly, V, tok, coef,
                     ylab, loss_tok, lse, m_p, given ? st_lse : (const float*)nullptr);
  KD_LAUNCH_CHECK();
  KD_LAUNCH(k_loss_sum, dim3(1), dim3(1024), 0, s, T, scale, tok, err, loss);
  KD_LAUNCH_CHECK();

  if (p.dense) {
    bf16_t* dz = at<bf16_t>(ws, p.o_dz);
    for (int c = 0; c < p.nchunks; ++c) {
      const int64_t c0 = (int64_t)c * p.C;
      const int64_t c1 = (c0 + p.C < V) ? c0 + p.C : V;
      const int64_t clen = c1 - c0;
      const int nCT = (int)kd_ceil_div(clen, VT);
      const int gz = grid_of(nCT * p.nTT);
      KD_LAUNCH(k_zdz, dim3(gz), dim3(TC::NT), ZDZ_LDS, s, (const bf16_t*)W, (const bf16_t*)h, T, d, V, (int)K,
                         p.Tp, p.Cp, c0, c1, nCT, p.nTT, sidx, starts, tok, zS, coef, ylab, dz);
      KD_LAUNCH_CHECK();
      const int kdh = (int)kd_round_up(clen, 64);
      const int gdh = grid_of(p.nTT * p.nDT);
      const int nCTw = (int)kd_ceil_div(clen, TC::BN);
      const int gdw = grid_of(nCTw * p.nDT);
      KD_LAUNCH(k_dhdw, dim3(gdh + gdw), dim3(TC::NT), GEMM_LDS, s, dz, (const bf16_t*)W, (const bf16_t*)h, T, d, p.Tp, p.Cp, c0, clen,
                         kdh, c == 0 ? 1 : 0, p.nTT, p.nDT, nCTw, gdh, p.Tp > kdh ? 1 : 0, 0, dh, dW);
      KD_LAUNCH_CHECK();
    }
  } else {
    int32_t* cnt = at<int32_t>(ws, p.o_cnt);
    int32_t* off = at<int32_t>(ws, p.o_off);
    int32_t* fillc = at<int32_t>(ws, p.o_fill);
    int32_t* ent_t = at<int32_t>(ws, p.o_entt);
    float* ent_r = at<float>(ws, p.o_entr);
    KD_LAUNCH(k_sparse_dh, dim3((unsigned)T), dim3(256), 0, s, (const bf16_t*)W, d, (int)K, sidx, coef, tok, dh);
    KD_LAUNCH_CHECK();
    KD_LAUNCH(k_fill_i32, dim3(512), dim3(256), 0, s, cnt, V + 1, 0);
    KD_LAUNCH(k_fill_i32, dim3(512), dim3(256), 0, s, fillc, V + 1, 0);
    const unsigned ge = (unsigned)kd_ceil_div(T * K, 256);
    KD_LAUNCH(k_csr_count, dim3(ge), dim3(256), 0, s, T, (int)K, sidx, tok, cnt);
    const int nseg = (int)kd_ceil_div(V, SCAN_SEG);
    int32_t* segsum = at<int32_t>(ws, p.o_seg);
    KD_LAUNCH(k_seg_sum, dim3(nseg), dim3(256), 0, s, cnt, V, segsum);
    KD_LAUNCH(k_seg_scan, dim3(nseg), dim3(256), 0, s, cnt, V, segsum, nseg, off);
    KD_LAUNCH(k_csr_fill, dim3(ge), dim3(256), 0, s, T, (int)K, sidx, coef, tok, off, fillc, ent_t, ent_r);
    KD_LAUNCH(k_sparse_dw, dim3((unsigned)kd_ceil_div(V, SDW_ROWS)), dim3(256), 0, s, (const bf16_t*)h, d, V, off,
              ent_t, ent_r, dW);
    KD_LAUNCH_CHECK();
  }
  return KD_OK;
}

extern "C" kd_status kd_topk_loss_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                          const float* teacher_logp, const float* m_q, int64_t T, int64_t d,
                                          int64_t V, int32_t K, kd_mode mode, int32_t chunk, float scale,
                                          float* loss, float* loss_tok, float* lse, float* m_p, float* dh,
                                          float* dW, void* ws, size_t ws_bytes, void* stream) {
  return loss_impl(h, W, idx, teacher_logp, m_q, nullptr, 0.f, nullptr, T, d, V, K, mode, chunk, scale, loss, loss_tok,
                   lse, m_p, dh, dW, ws, ws_bytes, stream);
}

extern "C" kd_status kd_topk_loss_fwd_bwd_tokblock(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                                   const float* teacher_logp, const float* m_q, int64_t T, int64_t d,
                                                   int64_t V, int32_t K, kd_mode mode, int32_t token_block,
                                                   float scale, float* loss, float* loss_tok, float* lse, float* m_p,
                                                   float* dh, float* dW, void* ws, size_t ws_bytes, void* stream) {
  if (token_block <= 0) return kd_fail(KD_EINVAL, "token_block must be > 0 (got %d)", (int)token_block);
  const bool dense = mode == KD_TAIL || mode == KD_FULL || mode == KD_TAIL_REVERSE || mode == KD_REVERSE_TT;
  return loss_impl(h, W, idx, teacher_logp, m_q, nullptr, 0.f, nullptr, T, d, V, K, mode, 8192, scale, loss, loss_tok,
                   lse, m_p, dh, dW, ws, ws_bytes, stream, nullptr, nullptr, dense ? token_block : 0);
}

extern "C" kd_status kd_topk_loss_fwd_bwd_selected(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                                   const float* teacher_logp, const float* m_q,
                                                   const float* student_lse, const float* student_logits,
                                                   const int32_t* sampled, const float* teacher_logp_sampled,
                                                   int64_t T, int64_t d, int64_t V, int32_t K, kd_mode mode,
                                                   int32_t chunk, float scale, float* loss, float* loss_tok,
                                                   float* lse, float* m_p, float* dh, float* dW, void* ws,
                                                   size_t ws_bytes, void* stream) {
  if (T > 0 && (student_lse == nullptr || student_logits == nullptr))
    return kd_fail(KD_EINVAL, "null required pointer (student_lse, student_logits)");
  if (sampled != nullptr && mode != KD_REVERSE_TT)
    return kd_fail(KD_EINVAL, "sampled tokens belong to KD_REVERSE_TT");
  return loss_impl(h, W, idx, teacher_logp, m_q, sampled, 0.f, teacher_logp_sampled, T, d, V, K, mode, chunk, scale,
                   loss, loss_tok, lse, m_p, dh, dW, ws, ws_bytes, stream, student_lse, student_logits);
}

extern "C" kd_status kd_topk_loss_fwd_bwd_ce(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                             const float* teacher_logp, const float* m_q, const int32_t* labels,
                                             float ce_weight, int64_t T, int64_t d, int64_t V, int32_t K,
                                             kd_mode mode, int32_t chunk, float scale, float* loss,
                                             float* loss_tok, float* lse, float* m_p, float* dh, float* dW,
                                             void* ws, size_t ws_bytes, void* stream) {
  if (mode == KD_REVERSE_TT) return kd_fail(KD_EINVAL, "KD_REVERSE_TT takes sampled tokens: kd_topk_loss_fwd_bwd_tt");
  return loss_impl(h, W, idx, teacher_logp, m_q, labels, ce_weight, nullptr, T, d, V, K, mode, chunk, scale, loss,
                   loss_tok, lse, m_p, dh, dW, ws, ws_bytes, stream);
}

extern "C" kd_status kd_topk_loss_fwd_bwd_tt(const kd_bf16* h, const kd_bf16* W, const int32_t* idx,
                                             const float* teacher_logp, const int32_t* sampled,
                                             const float* teacher_logp_sampled, int64_t T, int64_t d, int64_t V,
                                             int32_t K, int32_t chunk, float scale, float* loss, float* loss_tok,
                                             float* lse, float* m_p, float* dh, float* dW, void* ws,
                                             size_t ws_bytes, void* stream) {
  return loss_impl(h, W, idx, teacher_logp, nullptr, sampled, 0.f, teacher_logp_sampled, T, d, V, K, KD_REVERSE_TT,
                   chunk, scale, loss, loss_tok, lse, m_p, dh, dW, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Exact full-vocabulary KL from a hidden-state teacher cache: host side
// ---------------------------------------------------------------------------
namespace {

struct KlPlan {
  int64_t Tp, C, Cp;
  int nVT, nTT, nDT, nchunks;
  size_t o_tok, o_part, o_partT, o_partQZ, o_partH, o_q, o_dz, o_g, total;
};

// int8: room for the bf16 copy of the codes.
static bool plan_kl(int64_t T, int64_t d, int64_t dt, int64_t V, int32_t chunk, bool int8, KlPlan& p) {
  if (T < 0 || d <= 0 || dt <= 0 || V <= 0 || d % 64 != 0 || dt % 64 != 0 || d > 16384 || dt > 16384 || chunk <= 0)
    return false;
  if (V > (int64_t)1 << 30 || T > (int64_t)1 << 26) return false;
  p.Tp = kd_round_up(T > 0 ? T : 1, TT);
  p.C = kd_round_up(chunk, VT);
  if (p.C > kd_round_up(V, VT)) p.C = kd_round_up(V, VT);
  p.Cp = p.C;
  const uint64_t lim = (uint64_t)1 << 32;
  const uint64_t dm = (uint64_t)(d > dt ? d : dt);
  if ((uint64_t)p.C * dm * 2u >= lim || (uint64_t)p.Tp * dm * 2u >= lim || (uint64_t)p.Tp * (uint64_t)p.C * 4u >= lim)
    return false;
  p.nVT = (int)kd_ceil_div(V, VT);
  p.nTT = (int)(p.Tp / TT);
  p.nDT = (int)kd_ceil_div(d, TC::BN);
  p.nchunks = (int)kd_ceil_div(V, p.C);
  size_t o = 0;
  p.o_tok = o; o = align_up(o + (size_t)p.Tp * TOKF * 4);
  p.o_part = o; o = align_up(o + (size_t)p.nVT * p.Tp * 8);
  p.o_partT = o; o = align_up(o + (size_t)p.nVT * p.Tp * 16);
  p.o_partQZ = o; o = align_up(o + (size_t)p.nVT * p.Tp * 4);
  p.o_partH = o; o = align_up(o + (size_t)p.nVT * p.Tp * 4);
  p.o_q = o; o = align_up(o + (size_t)p.Tp * p.Cp * 4);
  p.o_dz = o; o = align_up(o + (size_t)p.Tp * p.Cp * 2);
  p.o_g = 0;
  if (int8) {
    p.o_g = o; o = align_up(o + (size_t)(T > 0 ? T : 1) * dt * 2);
  }
  p.total = o;
  return true;
}

}  // namespace

extern "C" size_t kd_kl_hidden_workspace(int64_t T, int64_t d, int64_t dt, int64_t V, int32_t chunk) {
  KlPlan p;
  if (!plan_kl(T, d, dt, V, chunk, false, p)) return 0;
  return p.total;
}

extern "C" size_t kd_kl_hidden_int8_workspace(int64_t T, int64_t d, int64_t dt, int64_t V, int32_t chunk) {
  KlPlan p;
  if (!plan_kl(T, d, dt, V, chunk, true, p)) return 0;
  return p.total;
}

extern "C" kd_status kd_hidden_quantize_int8(const kd_bf16* g, int64_t T, int64_t d, int8_t* codes, float* scale,
                                             void* stream) {
  if (T < 0 || d <= 0) return kd_fail(KD_EINVAL, "invalid sizes T=%lld d=%lld", (long long)T, (long long)d);
  if (T == 0) return KD_OK;
  if (!g || !codes || !scale) return kd_fail(KD_EINVAL, "null required pointer");
  if (T > 0x7fffffffLL) return kd_fail(KD_EINVAL, "T too large");
  hipStream_t s = (hipStream_t)stream;
  KD_LAUNCH(k_quantize_int8, dim3((unsigned)T), dim3(256), 0, s, (const bf16_t*)g, d, codes, scale);
  KD_LAUNCH_CHECK();
  return KD_OK;
}

// The KL with the teacher hidden states as bf16 (g) or as int8 codes with a
// per-position scale (codes8, gscale).
// teacher_lse != nullptr: the teacher's logsumexp is given (cached), and the
// teacher head is evaluated once instead of twice.
static kd_status kl_impl(const kd_bf16* h, const kd_bf16* W, const kd_bf16* g, const int8_t* codes8,
                         const float* gscale, const kd_bf16* U, const float* b, const float* teacher_lse, int64_t T,
                         int64_t d, int64_t dt, int64_t V, int32_t chunk, float scale, float* loss, float* loss_tok,
                         float* lse, float* lse_t, float* dh, float* dW, void* ws, size_t ws_bytes, void* stream) {
  KlPlan p;
  const bool int8 = codes8 != nullptr || gscale != nullptr;
  if (!plan_kl(T, d, dt, V, chunk, int8, p))
    return kd_fail(KD_EINVAL, "invalid sizes T=%lld d=%lld dt=%lld V=%lld chunk=%d (need d%%64==0, dt%%64==0, d,dt<=16384, chunk>0, and chunk*d, T*d bf16 and T*chunk fp32 each < 4 GiB)",
                   (long long)T, (long long)d, (long long)dt, (long long)V, (int)chunk);
  if (!loss || !dW || !W || !U) return kd_fail(KD_EINVAL, "null required pointer (loss, W, U, dW)");
  if (T > 0 && (!h || !dh || (!int8 && !g) || (int8 && (!codes8 || !gscale))))
    return kd_fail(KD_EINVAL, "null required pointer (h, dh and g, or the int8 codes and their scales)");
  if (int8 && g != nullptr) return kd_fail(KD_EINVAL, "give either g or the int8 codes and their scales, not both");
  if (!ws || ws_bytes < p.total)
    return kd_fail(KD_ENOWS, "workspace too small: need %zu bytes, got %zu", p.total, ws_bytes);
  if (!kd_aligned16(W) || !kd_aligned16(U) || !kd_aligned16(dW) || !kd_aligned16(ws) ||
      (T > 0 && (!kd_aligned16(h) || !kd_aligned16(dh) || (!int8 && !kd_aligned16(g)))))
    return kd_fail(KD_EINVAL, "h, W, g, U, dh, dW and ws must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  float* tok = at<float>(ws, p.o_tok);
  if (T == 0) {
    KD_LAUNCH(k_fill_i32, dim3(1024), dim3(256), 0, s, (int32_t*)dW, V * d, 0);
    KD_LAUNCH(k_loss_sum, dim3(1), dim3(1024), 0, s, (int64_t)0, scale, (const float*)tok, (const int32_t*)nullptr, loss);
    KD_LAUNCH_CHECK();
    return KD_OK;
  }
  float2* part = at<float2>(ws, p.o_part);
  float4* partT = at<float4>(ws, p.o_partT);
  float* partQZ = at<float>(ws, p.o_partQZ);
  float* partH = teacher_lse != nullptr ? at<float>(ws, p.o_partH) : nullptr;
  f32x4* qbuf = at<f32x4>(ws, p.o_q);
  bf16_t* dz = at<bf16_t>(ws, p.o_dz);
  if (int8) {
    bf16_t* gb = at<bf16_t>(ws, p.o_g);
    KD_LAUNCH(k_codes_to_bf16, dim3(1024), dim3(256), 0, s, codes8, T * dt, gb);
    g = (const kd_bf16*)gb;
  }
  const int g1 = grid_of(p.nVT * p.nTT);
  KD_LAUNCH(k_lse_pass<false>, dim3(g1), dim3(TC::NT), GEMM_LDS, s, (const bf16_t*)W, (const bf16_t*)h, d, T, V,
                     (const float*)nullptr, (const float*)nullptr, p.nVT, p.nTT, p.Tp, part, (float4*)nullptr);
  if (teacher_lse == nullptr)
    KD_LAUNCH(k_lse_pass<true>, dim3(g1), dim3(TC::NT), GEMM_LDS, s, (const bf16_t*)U, (const bf16_t*)g, dt, T,
              V, b, gscale, p.nVT, p.nTT, p.Tp, (float2*)nullptr, partT);
  KD_LAUNCH_CHECK();
  KD_LAUNCH(k_kl_combine, dim3((unsigned)kd_ceil_div(T, 4)), dim3(256), 0, s, T, p.nVT, p.Tp, scale, part,
            teacher_lse != nullptr ? (const float4*)nullptr : (const float4*)partT, teacher_lse, tok);
  KD_LAUNCH_CHECK();
  for (int c = 0; c < p.nchunks; ++c) {
    const int64_t c0 = (int64_t)c * p.C;
    const int64_t c1 = (c0 + p.C < V) ? c0 + p.C : V;
    const int64_t clen = c1 - c0;
    const int nCT = (int)kd_ceil_div(clen, VT);
    const int gz = grid_of(nCT * p.nTT);
    KD_LAUNCH(k_teacher_q, dim3(gz), dim3(TC::NT), GEMM_LDS, s, (const bf16_t*)U, (const bf16_t*)g, b, gscale, T,
                       dt, c0, c1, nCT, p.nTT, p.Tp, (const float*)tok, qbuf, partH);
    KD_LAUNCH(k_zdz_kl, dim3(gz), dim3(TC::NT), ZK_LDS, s, (const bf16_t*)W, (const bf16_t*)h, T, d, p.Tp, p.Cp, c0,
                       c1, nCT, p.nTT, (const float*)tok, (const f32x4*)qbuf, partQZ, dz);
    KD_LAUNCH_CHECK();
    const int kdh = (int)kd_round_up(clen, 64);
    const int gdh = grid_of(p.nTT * p.nDT);
    const int nCTw = (int)kd_ceil_div(clen, TC::BN);
    const int gdw = grid_of(nCTw * p.nDT);
    KD_LAUNCH(k_dhdw, dim3(gdh + gdw), dim3(TC::NT), GEMM_LDS, s, (const bf16_t*)dz, (const bf16_t*)W,
                       (const bf16_t*)h, T, d, p.Tp, p.Cp, c0, clen, kdh, c == 0 ? 1 : 0, p.nTT, p.nDT, nCTw, gdh,
                       p.Tp > kdh ? 1 : 0, 0, dh, dW);
    KD_LAUNCH_CHECK();
  }
  KD_LAUNCH(k_kl_finish, dim3((unsigned)kd_ceil_div(T, 32)), dim3(1024), 0, s, T, p.nVT, p.Tp, (const float*)partQZ,
                     (const float*)partH, tok, loss_tok, lse, lse_t);
  KD_LAUNCH(k_loss_sum, dim3(1), dim3(1024), 0, s, T, scale, (const float*)tok, (const int32_t*)nullptr, loss);
  KD_LAUNCH_CHECK();
  return KD_OK;
}

extern "C" kd_status kd_kl_hidden_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const kd_bf16* g, const kd_bf16* U,
                                          const float* b, int64_t T, int64_t d, int64_t dt, int64_t V, int32_t chunk,
                                          float scale, float* loss, float* loss_tok, float* lse, float* lse_t,
                                          float* dh, float* dW, void* ws, size_t ws_bytes, void* stream) {
  return kl_impl(h, W, g, nullptr, nullptr, U, b, nullptr, T, d, dt, V, chunk, scale, loss, loss_tok, lse, lse_t, dh,
                 dW, ws, ws_bytes, stream);
}

extern "C" kd_status kd_kl_hidden_int8_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const int8_t* codes,
                                               const float* gscale, const kd_bf16* U, const float* b, int64_t T,
                                               int64_t d, int64_t dt, int64_t V, int32_t chunk, float scale,
                                               float* loss, float* loss_tok, float* lse, float* lse_t, float* dh,
                                               float* dW, void* ws, size_t ws_bytes, void* stream) {
  return kl_impl(h, W, nullptr, codes, gscale, U, b, nullptr, T, d, dt, V, chunk, scale, loss, loss_tok, lse, lse_t,
                 dh, dW, ws, ws_bytes, stream);
}

extern "C" kd_status kd_kl_hidden_cached_lse_fwd_bwd(const kd_bf16* h, const kd_bf16* W, const kd_bf16* g,
                                                     const int8_t* codes, const float* gscale, const kd_bf16* U,
                                                     const float* b, const float* teacher_lse, int64_t T, int64_t d,
                                                     int64_t dt, int64_t V, int32_t chunk, float scale, float* loss,
                                                     float* loss_tok, float* lse, float* lse_t, float* dh, float* dW,
                                                     void* ws, size_t ws_bytes, void* stream) {
  if (T > 0 && teacher_lse == nullptr) return kd_fail(KD_EINVAL, "null required pointer (teacher_lse)");
  return kl_impl(h, W, g, codes, gscale, U, b, teacher_lse, T, d, dt, V, chunk, scale, loss, loss_tok, lse, lse_t, dh,
                 dW, ws, ws_bytes, stream);
}
