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

// Instruction order of one BK slice for the scheduler: the fragments of the
// first k-substep; the global prefetch of the next slice issued among the
// first substep's MFMAs (so it has the whole slice to land); the fragment
// reads of each next substep among the current substep's MFMAs; the LDS
// stores of the prefetched slice among the last substep's MFMAs.
template <class C>
__device__ __forceinline__ void gemm_schedule() {
  constexpr int NKS = C::BK / 16;
  constexpr int NMF = C::FM * C::FN;          // MFMAs per substep
  constexpr int NFR = C::FM + C::FN;          // fragment reads per substep
  constexpr int NGL = C::A_LD + C::B_LD;      // global loads (and LDS stores) per slice
#pragma unroll
  for (int r = 0; r < NFR; ++r) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int m = 0; m < NMF; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (ks == 0 && m < NGL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (ks + 1 < NKS && (m % 2) == 1 && m / 2 < NFR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (ks + 1 == NKS && m < NGL) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
  }
}

// One BM x BN tile over the full K range.  `lds` must hold C::LDS_BYTES.
// A is read from rows [m0, m_end) (clamped), B from rows [n0, n_end).
// Global reads use 32-bit byte offsets from a uniform row-block base; the
// MFMA fragments of k-substep s+1 are read from LDS while the matrix cores
// work on substep s.
template <class C>
__device__ __forceinline__ void gemm_tile(const bf16_t* __restrict__ A, int64_t lda, int64_t m0, int64_t m_end,
                                          const bf16_t* __restrict__ B, int64_t ldb, int64_t n0, int64_t n_end,
                                          int K, bf16_t* lds, Acc<C>& acc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  constexpr int RSTEP = C::NT / C::CPR;  // rows between a thread's successive chunks
  constexpr int NKS = C::BK / 16;

#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = f32x16{};

  const char* Ab = (const char*)(A + m0 * lda);
  const char* Bb = (const char*)(B + n0 * ldb);
  const int r0 = tid / C::CPR, k8 = (tid % C::CPR) * 8;
  const int m_rows = (int)(m_end - m0), n_rows = (int)(n_end - n0);
  uint32_t a_off[C::A_LD], b_off[C::B_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int r = r0 + i * RSTEP;
    a_off[i] = (uint32_t)(((r < m_rows ? r : m_rows - 1) * (int)lda + k8) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    const int r = r0 + i * RSTEP;
    b_off[i] = (uint32_t)(((r < n_rows ? r : n_rows - 1) * (int)ldb + k8) * 2);
  }
  bf16_t* sa_st = lds + r0 * C::LDK + k8;
  bf16_t* sb_st = lds + C::A_ELEMS + r0 * C::LDK + k8;

  u32x4 ra[C::A_LD], rb[C::B_LD];
  const int nk = K / C::BK;
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) ra[i] = *(const u32x4*)(Ab + a_off[i]);
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) rb[i] = *(const u32x4*)(Bb + b_off[i]);
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) *(u32x4*)(sa_st + i * RSTEP * C::LDK) = ra[i];
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) *(u32x4*)(sb_st + i * RSTEP * C::LDK) = rb[i];
  __syncthreads();

  const int l32 = lane & 31, khalf = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = (kt & 1) * C::STAGE;
    const int nxt = C::STAGE - cur;
    // prefetch slice kt+1 (the last iteration re-reads the last slice into
    // the idle buffer, so the loop body stays one basic block)
    const uint32_t kb = (uint32_t)(((kt + 1 < nk) ? kt + 1 : kt) * C::BK * 2);
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) ra[i] = *(const u32x4*)(Ab + (a_off[i] + kb));
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) rb[i] = *(const u32x4*)(Bb + (b_off[i] + kb));
    const bf16_t* sA = lds + cur + (wm * C::TM + l32) * C::LDK + khalf;
    const bf16_t* sB = lds + cur + C::A_ELEMS + (wn * C::TN + l32) * C::LDK + khalf;
    bf16x8 fa[2][C::FM], fb[2][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) fa[0][i] = *(const bf16x8*)(sA + i * 32 * C::LDK);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) fb[0][j] = *(const bf16x8*)(sB + j * 32 * C::LDK);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int cb = ks & 1, nb = cb ^ 1;
      if (ks + 1 < NKS) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) fa[nb][i] = *(const bf16x8*)(sA + i * 32 * C::LDK + (ks + 1) * 16);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) fb[nb][j] = *(const bf16x8*)(sB + j * 32 * C::LDK + (ks + 1) * 16);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32x32x16(fa[cb][i], fb[cb][j], acc.v[i][j]);
    }
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) *(u32x4*)(sa_st + nxt + i * RSTEP * C::LDK) = ra[i];
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) *(u32x4*)(sb_st + nxt + i * RSTEP * C::LDK) = rb[i];
    gemm_schedule<C>();
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Pipelined variant: BK = 32 slices in a ring of three LDS stages.
//   iteration kt:  issue global loads of slice kt+3 (register set (kt+1)%2)
//                  MFMAs of slice kt (stage kt%3), reading the fragments of
//                  its second k-substep during the first
//                  store slice kt+2 (register set kt%2) into stage (kt+2)%3
//                  read the first fragments of slice kt+1 (stage (kt+1)%3,
//                  complete since the previous barrier)
//                  barrier
// Global loads have two iterations to land; no MFMA waits on LDS after a
// barrier because the next slice's first fragments are already in registers.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_>
struct PipeCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 32, WM = WM_, WN = WN_, NSTAGE = 3;
  static constexpr int NWAVE = WM * WN, NT = 64 * NWAVE;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int LDK = BK;                    // 64-byte rows, 16-byte chunks XOR-swizzled per row
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = NSTAGE * STAGE * 2;
  static constexpr int CPR = BK / 8;
  static constexpr int A_LD = BM * CPR / NT;
  static constexpr int B_LD = BN * CPR / NT;
  static constexpr int NLD = A_LD + B_LD;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile");
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "loader");
};

// Chunk swizzle of the LDS tiles: 16-byte chunk c of row r is stored at
// chunk position c ^ pipe_swz(r).  Fragment reads (32 consecutive rows, one
// chunk) and the tile stores (4 chunks of a row per 4 lanes) then spread over
// all LDS banks.
__device__ __forceinline__ int pipe_swz(int r) { return (r ^ (r >> 2)) & 3; }

template <class C>
struct PipeState {
  const char* Ab;
  const char* Bb;
  uint32_t a_off[C::A_LD], b_off[C::B_LD];
  bf16_t* sa_st;
  bf16_t* sb_st;
  const bf16_t* sA[2];  // per k-substep (the swizzled chunk differs)
  const bf16_t* sB[2];
  u32x4 r[2][C::NLD];
  bf16x8 fa[2][C::FM], fb[2][C::FN];
};

template <class C>
__device__ __forceinline__ void pipe_gload(PipeState<C>& P, int set, int slice) {
  const uint32_t kb = (uint32_t)(slice * C::BK * 2);
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) P.r[set][i] = *(const u32x4*)(P.Ab + (P.a_off[i] + kb));
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) P.r[set][C::A_LD + i] = *(const u32x4*)(P.Bb + (P.b_off[i] + kb));
}

template <class C>
__device__ __forceinline__ void pipe_lstore(PipeState<C>& P, int set, int stage) {
  constexpr int RSTEP = C::NT / C::CPR;
  const int so = stage * C::STAGE;
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) *(u32x4*)(P.sa_st + so + i * RSTEP * C::LDK) = P.r[set][i];
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) *(u32x4*)(P.sb_st + so + i * RSTEP * C::LDK) = P.r[set][C::A_LD + i];
}

template <class C>
__device__ __forceinline__ void pipe_fread(PipeState<C>& P, int buf, int stage, int ks) {
  const int so = stage * C::STAGE;
  // order of first use by the MFMA loop below: a0, b0..b(FN-1), a1..
  P.fa[buf][0] = *(const bf16x8*)(P.sA[ks] + so);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) P.fb[buf][j] = *(const bf16x8*)(P.sB[ks] + so + j * 32 * C::LDK);
#pragma unroll
  for (int i = 1; i < C::FM; ++i) P.fa[buf][i] = *(const bf16x8*)(P.sA[ks] + so + i * 32 * C::LDK);
}

template <class C>
__device__ __forceinline__ void pipe_mfma(PipeState<C>& P, int buf, Acc<C>& acc) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32x32x16(P.fa[buf][i], P.fb[buf][j], acc.v[i][j]);
}

template <class C>
__device__ __forceinline__ void pipe_schedule() {
  constexpr int NMF = C::FM * C::FN;
  constexpr int NFR = C::FM + C::FN;
  // substep 0: global loads and the second substep's fragments among the MFMAs
#pragma unroll
  for (int m = 0; m < NMF; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m < NFR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (m < C::NLD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  // substep 1: LDS stores of slice kt+2, then the next slice's first fragments
#pragma unroll
  for (int m = 0; m < NMF; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m < C::NLD) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (m >= NMF - NFR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

__device__ __forceinline__ int pipe_slice(int s, int nk, int rot) {
  const int x = s + rot;
  return x >= nk ? x - nk : x;
}

template <class C, int SET>
__device__ __forceinline__ void pipe_iter(PipeState<C>& P, int kt, int nk, int rot, Acc<C>& acc) {
  const int last = nk - 1;
  pipe_gload<C>(P, SET ^ 1, pipe_slice(kt + 3 < nk ? kt + 3 : last, nk, rot));
  pipe_fread<C>(P, 1, kt % 3, 1);
  pipe_mfma<C>(P, 0, acc);
  pipe_mfma<C>(P, 1, acc);
  pipe_lstore<C>(P, SET, (kt + 2) % 3);
  pipe_fread<C>(P, 0, (kt + 1) % 3, 0);
  pipe_schedule<C>();
  __syncthreads();
}

// One BM x BN tile over K (a multiple of 32).  `lds` holds C::LDS_BYTES.
template <class C>
__device__ __forceinline__ void gemm_tile_pipe(const bf16_t* __restrict__ A, int64_t lda, int64_t m0, int64_t m_end,
                                               const bf16_t* __restrict__ B, int64_t ldb, int64_t n0, int64_t n_end,
                                               int K, bf16_t* lds, Acc<C>& acc, int rot = 0) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  constexpr int RSTEP = C::NT / C::CPR;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = f32x16{};
  PipeState<C> P;
  P.Ab = (const char*)(A + m0 * lda);
  P.Bb = (const char*)(B + n0 * ldb);
  const int r0 = tid / C::CPR, k8 = (tid % C::CPR) * 8;
  const int m_rows = (int)(m_end - m0), n_rows = (int)(n_end - n0);
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int r = r0 + i * RSTEP;
    P.a_off[i] = (uint32_t)(((r < m_rows ? r : m_rows - 1) * (int)lda + k8) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    const int r = r0 + i * RSTEP;
    P.b_off[i] = (uint32_t)(((r < n_rows ? r : n_rows - 1) * (int)ldb + k8) * 2);
  }
  // rows r0 + i*RSTEP share r0's swizzle (RSTEP is a multiple of 16)
  const int kst = ((k8 >> 3) ^ pipe_swz(r0)) * 8;
  P.sa_st = lds + r0 * C::LDK + kst;
  P.sb_st = lds + C::A_ELEMS + r0 * C::LDK + kst;
  const int l32 = lane & 31, kh = lane >> 5;
  const int rsw = pipe_swz(l32);  // fragment rows differ from l32 by multiples of 32
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int kc = ((ks * 2 + kh) ^ rsw) * 8;
    P.sA[ks] = lds + (wm * C::TM + l32) * C::LDK + kc;
    P.sB[ks] = lds + C::A_ELEMS + (wn * C::TN + l32) * C::LDK + kc;
  }

  const int nk = K / C::BK;
  const int last = nk - 1;
  rot = rot % nk;
  pipe_gload<C>(P, 0, pipe_slice(0, nk, rot));
  pipe_gload<C>(P, 1, pipe_slice(1 < nk ? 1 : last, nk, rot));
  pipe_lstore<C>(P, 0, 0);
  pipe_lstore<C>(P, 1, 1);
  pipe_gload<C>(P, 0, pipe_slice(2 < nk ? 2 : last, nk, rot));
  __syncthreads();
  pipe_fread<C>(P, 0, 0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    pipe_iter<C, 0>(P, kt, nk, rot, acc);
    pipe_iter<C, 1>(P, kt + 1, nk, rot, acc);
  }
  if (kt < nk) pipe_iter<C, 0>(P, kt, nk, rot, acc);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant: BK = 64 slices (128-byte row segments, one cache
// line per row) loaded straight into LDS with global_load_lds_dwordx4, two
// stages.  Lane l of a wave-load lands at LDS byte 16*l of the wave's 1 KB
// destination, so the 16-byte chunks of a row are XOR-swizzled by choosing
// which global chunk each lane fetches.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_>
struct DtlCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_;
  static constexpr int NWAVE = WM * WN, NT = 64 * NWAVE;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int LDK = BK;                    // 128-byte rows
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int ROWS_PER_LOAD = 8;           // 1 KB wave-load = 8 rows x 128 B
  static constexpr int A_WL = BM / ROWS_PER_LOAD / NWAVE;  // wave-loads per wave per slice
  static constexpr int B_WL = BN / ROWS_PER_LOAD / NWAVE;
  static_assert(BM % (ROWS_PER_LOAD * NWAVE) == 0 && BN % (ROWS_PER_LOAD * NWAVE) == 0, "loader");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "tile");
};

__device__ __forceinline__ int dtl_swz(int r) { return (r >> 1) & 7; }

// Issue order of one slice: the direct-to-LDS loads of the next slice and
// the first substep's fragments, then each substep's MFMAs with the next
// substep's fragment reads among them.
template <class C>
__device__ __forceinline__ void dtl_schedule() {
  constexpr int NKS = C::BK / 16, NMF = C::FM * C::FN, NFR = C::FM + C::FN, NWL = C::A_WL + C::B_WL;
#pragma unroll
  for (int r = 0; r < NWL; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if (r < NFR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int m = 0; m < NMF; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (ks + 1 < NKS && m < NFR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}

template <class C>
__device__ __forceinline__ void gemm_tile_dtl(const bf16_t* __restrict__ A, int64_t lda, int64_t m0, int64_t m_end,
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
  const char* Ab = (const char*)(A + m0 * lda);
  const char* Bb = (const char*)(B + n0 * ldb);
  const int m_rows = (int)(m_end - m0), n_rows = (int)(n_end - n0);
  // this lane's global chunk for each of its wave-loads
  uint32_t a_off[C::A_WL], b_off[C::B_WL];
  const int lrow = lane >> 3, lchunk = lane & 7;
#pragma unroll
  for (int i = 0; i < C::A_WL; ++i) {
    const int r = (wave * C::A_WL + i) * C::ROWS_PER_LOAD + lrow;
    const int c = lchunk ^ dtl_swz(r);
    a_off[i] = (uint32_t)(((r < m_rows ? r : m_rows - 1) * (int)lda + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::B_WL; ++i) {
    const int r = (wave * C::B_WL + i) * C::ROWS_PER_LOAD + lrow;
    const int c = lchunk ^ dtl_swz(r);
    b_off[i] = (uint32_t)(((r < n_rows ? r : n_rows - 1) * (int)ldb + c * 8) * 2);
  }
  // LDS destinations (wave-uniform) of the wave-loads, bf16 elements
  const int a_dst0 = wave * C::A_WL * C::ROWS_PER_LOAD * C::LDK;
  const int b_dst0 = C::A_ELEMS + wave * C::B_WL * C::ROWS_PER_LOAD * C::LDK;
  // fragment rows: R = w*T + f*32 + l32, swizzle depends on l32 only
  const int l32 = lane & 31, kh = lane >> 5;
  const int fsw = dtl_swz(l32);
  const bf16_t* sA = lds + (wm * C::TM + l32) * C::LDK;
  const bf16_t* sB = lds + C::A_ELEMS + (wn * C::TN + l32) * C::LDK;

  auto issue = [&](int slice, int stage) {
    const uint32_t kb = (uint32_t)(slice * C::BK * 2);
    bf16_t* base = lds + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_WL; ++i)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Ab + (a_off[i] + kb)),
                                       (__attribute__((address_space(3))) void*)(base + a_dst0 + i * C::ROWS_PER_LOAD * C::LDK),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_WL; ++i)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Bb + (b_off[i] + kb)),
                                       (__attribute__((address_space(3))) void*)(base + b_dst0 + i * C::ROWS_PER_LOAD * C::LDK),
                                       16, 0, 0);
  };

  const int nk = K / C::BK;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = (kt & 1) * C::STAGE;
    issue(kt + 1 < nk ? kt + 1 : kt, (kt + 1) & 1);
    bf16x8 fa[2][C::FM], fb[2][C::FN];
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      const int b = ks & 1;
      const int ko = (((ks * 2 + kh) ^ fsw) * 8) + cur;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) fa[b][i] = *(const bf16x8*)(sA + ko + i * 32 * C::LDK);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) fb[b][j] = *(const bf16x8*)(sB + ko + j * 32 * C::LDK);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32x32x16(fa[b][i], fb[b][j], acc.v[i][j]);
    }
    dtl_schedule<C>();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}
