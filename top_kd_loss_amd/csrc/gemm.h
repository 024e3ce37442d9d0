// bf16 MFMA GEMM core for gfx950: C[m][n] = sum_k A[m][k] * B[n][k].
//
// Both operands are K-contiguous ("NT"): row m of A and row n of B each hold
// K consecutive bf16 values.  A workgroup of WM x WN wavefronts computes a
// BM x BN tile; each wavefront owns a (BM/WM) x (BN/WN) sub-tile made of
// 32x32 MFMA blocks with fp32 accumulators in registers.  Tiles of A and B
// are staged through LDS in BK-deep slices, double buffered: the global
// loads of slice k+1 are in flight while the matrix cores work on slice k.
//
// K must be a multiple of BK (callers pad K with zeros).  Rows past the end
// of A or B are clamped to the last valid row; the epilogue discards them.
#pragma once
#include "kd_common.h"

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int NWAVE = WM * WN, NT = 64 * NWAVE;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wavefront sub-tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 blocks per wavefront
  static constexpr int LDK = BK + 8;                // LDS row pitch (bf16), +16 B against bank conflicts
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int CPR = BK / 8;                // 16-byte chunks per row slice
  static constexpr int A_LD = BM * CPR / NT;        // chunks per thread per slice
  static constexpr int B_LD = BN * CPR / NT;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile");
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "loader");
  static_assert(BK % 16 == 0, "k slice");
};

template <class C>
struct Acc {
  f32x16 v[C::FM][C::FN];
};

// Position of accumulator element e of block (fm, fn) for lane `lane` of the
// wavefront at (wm, wn): row = m_of(...), column = n_of(...), both within the tile.
template <class C>
__device__ __forceinline__ int acc_row(int wm, int fm, int e, int lane) {
  return wm * C::TM + fm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
template <class C>
__device__ __forceinline__ int acc_col(int wn, int fn, int lane) {
  return wn * C::TN + fn * 32 + (lane & 31);
}

// One BM x BN tile over the full K range.  `lds` must hold C::LDS_BYTES.
// A is read from rows [m0, m_end) (clamped), B from rows [n0, n_end).
template <class C>
__device__ __forceinline__ void gemm_tile(const bf16_t* __restrict__ A, int64_t lda, int64_t m0, int64_t m_end,
                                          const bf16_t* __restrict__ B, int64_t ldb, int64_t n0, int64_t n_end,
                                          int K, bf16_t* lds, Acc<C>& acc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = f32x16{};

  const bf16_t* Ab = A + m0 * lda;
  const bf16_t* Bb = B + n0 * ldb;
  int a_off[C::A_LD], a_lds[C::A_LD];
  int b_off[C::B_LD], b_lds[C::B_LD];
  const int64_t m_rows = m_end - m0, n_rows = n_end - n0;
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    int c = tid + i * C::NT;
    int r = c / C::CPR, k8 = (c % C::CPR) * 8;
    int rr = (int)((r < m_rows) ? r : (m_rows - 1));
    a_off[i] = rr * (int)lda + k8;
    a_lds[i] = r * C::LDK + k8;
  }
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    int c = tid + i * C::NT;
    int r = c / C::CPR, k8 = (c % C::CPR) * 8;
    int rr = (int)((r < n_rows) ? r : (n_rows - 1));
    b_off[i] = rr * (int)ldb + k8;
    b_lds[i] = C::A_ELEMS + r * C::LDK + k8;
  }

  u32x4 ra[C::A_LD], rb[C::B_LD];
  const int nk = K / C::BK;

#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) ra[i] = *(const u32x4*)(Ab + a_off[i]);
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) rb[i] = *(const u32x4*)(Bb + b_off[i]);
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) *(u32x4*)(lds + a_lds[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) *(u32x4*)(lds + b_lds[i]) = rb[i];
  __syncthreads();

  const int l32 = lane & 31, khalf = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = (kt & 1) * C::STAGE;
    const bool more = (kt + 1) < nk;
    if (more) {
      const int k0 = (kt + 1) * C::BK;
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) ra[i] = *(const u32x4*)(Ab + a_off[i] + k0);
#pragma unroll
      for (int i = 0; i < C::B_LD; ++i) rb[i] = *(const u32x4*)(Bb + b_off[i] + k0);
    }
    const bf16_t* sA = lds + cur + (wm * C::TM + l32) * C::LDK + khalf;
    const bf16_t* sB = lds + cur + C::A_ELEMS + (wn * C::TN + l32) * C::LDK + khalf;
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      bf16x8 a[C::FM], b[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) a[i] = *(const bf16x8*)(sA + i * 32 * C::LDK + ks * 16);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) b[j] = *(const bf16x8*)(sB + j * 32 * C::LDK + ks * 16);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32x32x16(a[i], b[j], acc.v[i][j]);
    }
    if (more) {
      const int nxt = ((kt + 1) & 1) * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) *(u32x4*)(lds + nxt + a_lds[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < C::B_LD; ++i) *(u32x4*)(lds + nxt + b_lds[i]) = rb[i];
    }
    __syncthreads();
  }
}
