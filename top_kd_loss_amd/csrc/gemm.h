// bf16 MFMA GEMM core for gfx950: C[m][n] = sum_k A(m, k) * B(n, k).
//
// A workgroup of 2 x 2 wavefronts computes a 256 x 256 tile; each wavefront
// owns a 128 x 128 sub-tile made of 4 x 4 blocks of 32x32 MFMAs
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulators in registers (AGPRs).
// Operand tiles are staged through LDS in BK = 64 slices in two stages.
//
// Each operand is stored in global memory in one of two layouts:
//   K-major  (MN = false): element (r, k) at P[r * ld + k]; the tile's rows
//            [r0, r_end) are read, clamped to r_end - 1.
//   MN-major (MN = true):  element (r, k) at P[k * ld + r]; the tile's
//            columns [r0, r_end) are read in aligned groups of 8, chunks
//            past the one holding column r_end - 1 clamped to it (each row
//            must hold r_end rounded up to 8 elements), from rows k < k_end
//            (clamped to k_end - 1).
// K-major slices sit in LDS as 128-byte rows (one per M/N index); MN-major
// slices as 512-byte rows (one per k) that reach the matrix cores through
// transposing LDS reads (ds_read_b64_tr_b16), so no operand is ever
// transposed in memory.
//
// K must be a multiple of 64.  Clamped rows or columns feed finite values
// whose results the caller discards (or whose partner operand is zero).
//
// Pipeline.  Each slice feeds four 16-deep substeps of 16 MFMAs; the global
// loads of slice kt+2 and the LDS stores of slice kt+1 hide behind them, so
// the workgroup meets one barrier per 64 of K.
//   iteration kt (stage kt%2 holds slice kt, complete since the last barrier):
//     region 0: MFMAs of substep 3 of slice kt-1 | fragments of substep 0 |
//               A loads of slice kt+2 into register set kt%2
//     region 1: MFMAs of substep 0 | fragments of substep 1 | B loads of
//               slice kt+2 | stores of slice kt+1 (register set (kt+1)%2)
//               into stage (kt+1)%2, first 6 chunks
//     region 2: MFMAs of substep 1 | fragments of substep 2 | 5 more chunks
//     region 3: MFMAs of substep 2 | last 5 chunks | fragments of substep 3
//     s_waitcnt lgkmcnt(0); s_barrier
// Stage (kt+1)%2 held slice kt-1, whose last fragment reads (region 3 of the
// previous iteration) completed before that barrier.  The instruction
// interleave of each region is pinned with sched_group_barrier.
#pragma once
#include "kd_common.h"

struct GemmCfg {
  static constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 2, NSTAGE = 2;
  static constexpr int NWAVE = WM * WN, NT = 64 * NWAVE;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK, STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = NSTAGE * STAGE * 2;
  static constexpr int LDN = BM * BK / 8 / NT;  // 16-byte chunks per thread, operand and slice
  static_assert(BM == BN && TM == TN && BM * BK / 8 % NT == 0, "loader");
};
constexpr int GEMM_LDS = GemmCfg::LDS_BYTES;  // 128 KB

template <class C>
struct Acc {
  f32x16 v[C::FM][C::FN];
};

// Position of accumulator element e of block (fm, fn) for lane `lane` of the
// wavefront at (wm, wn): row and column within the tile.
template <class C>
__device__ __forceinline__ int acc_row(int wm, int fm, int e, int lane) {
  return wm * C::TM + fm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
template <class C>
__device__ __forceinline__ int acc_col(int wn, int fn, int lane) {
  return wn * C::TN + fn * 32 + (lane & 31);
}

// K-major LDS rows of 128 bytes: chunk c of row r at c ^ kswz(r).  Rows 2j
// and 2j+1 share a 256-byte bank span; (r >> 1) & 7 spreads the same chunk
// of 16 consecutive rows over the 16 sixteen-byte bank slots.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
// MN-major LDS rows (one per k): chunk c of row k is stored at c ^ mswz(k).
// A transposing fragment read touches 4 consecutive k-rows x 64 bytes (and
// the same 4 rows + 8); the XOR puts those 4 rows on disjoint bank quarters.
__device__ __forceinline__ int mswz(int k) { return (k & 3) << 2; }

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

template <bool MN>
struct GemmOperand;

// K-major operand: thread tid loads chunk tid % 8 of rows tid / 8 + 32 i.
template <>
struct GemmOperand<false> {
  using C = GemmCfg;
  static constexpr int CPR = C::BK / 8;      // chunks per row slice
  static constexpr int RSTEP = C::NT / CPR;  // rows between a thread's chunks
  static constexpr int LDN = C::LDN;
  static constexpr int NREAD = C::FM;        // LDS read instructions per substep
  static_assert(RSTEP % 16 == 0, "rows rr + i*RSTEP share rr's swizzle");
  const char* base;
  uint32_t off[LDN];
  bf16_t* st;           // this thread's store slot (stage 0)
  const bf16_t* rd[4];  // fragment 0 of each k-substep (stage 0)

  __device__ __forceinline__ void init(const bf16_t* P, int64_t ld, int64_t r0, int64_t r_end, int,
                                       bf16_t* lds_op, int w, int lane) {
    const int tid = threadIdx.x;
    base = (const char*)(P + r0 * ld);
    const int rr = tid / CPR, c = tid % CPR;
    const int nrows = (int)(r_end - r0);
#pragma unroll
    for (int i = 0; i < LDN; ++i) {
      const int r = rr + i * RSTEP;
      off[i] = (uint32_t)(((r < nrows ? r : nrows - 1) * (int)ld + c * 8) * 2);
    }
    st = lds_op + rr * C::BK + ((c ^ kswz(rr)) << 3);
    // fragment rows differ from l32 by multiples of 32: same swizzle
    const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      rd[ks] = lds_op + (w * C::TM + l32) * C::BK + (((ks * 2 + kh) ^ kswz(l32)) << 3);
  }
  __device__ __forceinline__ void gload(u32x4* r, int slice) const {
    const uint32_t kb = (uint32_t)(slice * C::BK * 2);
#pragma unroll
    for (int i = 0; i < LDN; ++i) r[i] = *(const u32x4*)(base + (off[i] + kb));
  }
  template <int I0 = 0, int I1 = LDN>
  __device__ __forceinline__ void lstore(const u32x4* r, int stage) const {
#pragma unroll
    for (int i = I0; i < I1; ++i) *(u32x4*)(st + stage * C::STAGE + i * RSTEP * C::BK) = r[i];
  }
  __device__ __forceinline__ bf16x8 fread(int f, int stage, int ks) const {
    return *(const bf16x8*)(rd[ks] + stage * C::STAGE + f * 32 * C::BK);
  }
};

// MN-major operand: thread tid loads column chunk tid % 32 of k-rows
// tid / 32 + 8 i.
template <>
struct GemmOperand<true> {
  using C = GemmCfg;
  static constexpr int ROWS = C::BM;         // tile extent along M (or N)
  static constexpr int CPK = ROWS / 8;       // chunks per k-row
  static constexpr int KSTEP = C::NT / CPK;  // k-rows between a thread's chunks
  static constexpr int LDN = C::LDN;
  static constexpr int NREAD = 2 * C::FM;    // two transposing reads per fragment
  static_assert(KSTEP * LDN == C::BK && KSTEP % 4 == 0, "MN-major loader");
  static_assert(C::TM % 128 == 0 && C::FM <= 4, "MN-major fragment addressing");
  const char* base;
  uint32_t col;  // byte offset of this thread's column chunk
  uint32_t ld2;  // k-row pitch in bytes
  int kr, kend;
  bf16_t* st;
  const bf16_t* rd;  // substep 0, first half, without the fragment term
  int foff[C::FM];   // fragment terms (swizzled)

  __device__ __forceinline__ void init(const bf16_t* P, int64_t ld, int64_t r0, int64_t r_end, int k_end,
                                       bf16_t* lds_op, int w, int lane) {
    const int tid = threadIdx.x;
    base = (const char*)(P + r0);
    const int mc = tid % CPK;
    kr = tid / CPK;
    kend = k_end;
    ld2 = (uint32_t)(ld * 2);
    const int cmax = (((int)(r_end - r0) - 1) >> 3) << 3;  // chunk holding the last column
    col = (uint32_t)((mc * 8 < cmax ? mc * 8 : cmax) * 2);
    // rows kr + i*KSTEP share kr's swizzle (KSTEP is a multiple of 4)
    st = lds_op + kr * ROWS + ((mc ^ mswz(kr)) << 3);
    // Transposing read (per 16-lane group g, lane j = lane % 16): lane j
    // names 4 consecutive columns 16*(g%2) + 4*(j%4) of k-row 8*(g/2) + j/4;
    // lane j receives column 16*(g%2) + j of k-rows 8*(g/2) .. +3, which is
    // the MFMA operand layout (column lane%32, k = 8*(lane/32) .. +3).
    // Element address of (k, m): k*ROWS + ((m/8) ^ mswz(k))*8 + m%8, with
    // m = w*TM + 32*f + 16*(g%2) + 4*(j%4): the XOR acts on the bits of f.
    const int g = lane >> 4, j = lane & 15;
    const int lowc = 2 * (g & 1) + ((j & 3) >> 1);
    rd = lds_op + (8 * (g >> 1) + (j >> 2)) * ROWS + w * C::TM + 8 * lowc + 4 * (j & 1);
#pragma unroll
    for (int f = 0; f < C::FM; ++f) foff[f] = 32 * (f ^ (j >> 2));
  }
  __device__ __forceinline__ void gload(u32x4* r, int slice) const {
#pragma unroll
    for (int i = 0; i < LDN; ++i) {
      int k = slice * C::BK + kr + i * KSTEP;
      k = k < kend ? k : kend - 1;
      r[i] = *(const u32x4*)(base + ((uint32_t)k * ld2 + col));
    }
  }
  template <int I0 = 0, int I1 = LDN>
  __device__ __forceinline__ void lstore(const u32x4* r, int stage) const {
#pragma unroll
    for (int i = I0; i < I1; ++i) *(u32x4*)(st + stage * C::STAGE + i * KSTEP * ROWS) = r[i];
  }
  __device__ __forceinline__ bf16x8 fread(int f, int stage, int ks) const {
    const bf16_t* p = rd + stage * C::STAGE + ks * 16 * ROWS + foff[f];
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 4 * ROWS));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

template <bool AT, bool BT>
struct GemmState {
  using C = GemmCfg;
  GemmOperand<AT> a;
  GemmOperand<BT> b;
  u32x4 ra[2][C::LDN], rb[2][C::LDN];  // register sets of two slices in flight
  bf16x8 fa[2][C::FM], fb[2][C::FN];   // fragments of two consecutive substeps
};

template <int BUF, bool AT, bool BT>
__device__ __forceinline__ void gemm_fread(GemmState<AT, BT>& P, int stage, int ks) {
  // order of first use by the MFMA loop below: a0, b0..b3, a1..a3
  P.fa[BUF][0] = P.a.fread(0, stage, ks);
#pragma unroll
  for (int j = 0; j < GemmCfg::FN; ++j) P.fb[BUF][j] = P.b.fread(j, stage, ks);
#pragma unroll
  for (int i = 1; i < GemmCfg::FM; ++i) P.fa[BUF][i] = P.a.fread(i, stage, ks);
}

template <class C, int BUF, bool AT, bool BT>
__device__ __forceinline__ void gemm_mfma(GemmState<AT, BT>& P, Acc<C>& acc) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32x32x16(P.fa[BUF][i], P.fb[BUF][j], acc.v[i][j]);
}

// 16 MFMAs with NR fragment reads, NL global loads and NS LDS stores spread
// among them (at most one of each per MFMA).
template <int NR, int NL, int NS>
__device__ __forceinline__ void gemm_schedule() {
  static_assert(NR <= 16 && NL <= 16 && NS <= 16, "one of each per MFMA slot");
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
    if (m < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    if (m < NS) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
    if (m < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
  }
}

template <class C, bool AT, bool BT, int SET, bool FIRST>
__device__ __forceinline__ void gemm_iter(GemmState<AT, BT>& P, int kt, int nk, Acc<C>& acc) {
  constexpr int NR = GemmOperand<AT>::NREAD + GemmOperand<BT>::NREAD;
  constexpr int L = GemmCfg::LDN;
  static_assert(L == 8, "stores of one slice split 6 / 2+3 / 5 over regions 1-3");
  const int s = kt & 1, sn = s ^ 1;
  const int ld = kt + 2 < nk ? kt + 2 : nk - 1;
  // region 0
  if constexpr (!FIRST) gemm_mfma<C, 1>(P, acc);
  gemm_fread<0>(P, s, 0);
  P.a.gload(P.ra[SET], ld);
  if constexpr (!FIRST) gemm_schedule<NR, L, 0>();
  __builtin_amdgcn_sched_barrier(0);
  // region 1
  gemm_mfma<C, 0>(P, acc);
  gemm_fread<1>(P, s, 1);
  P.b.gload(P.rb[SET], ld);
  P.a.template lstore<0, 6>(P.ra[SET ^ 1], sn);
  gemm_schedule<NR, L, 6>();
  __builtin_amdgcn_sched_barrier(0);
  // region 2
  gemm_mfma<C, 1>(P, acc);
  gemm_fread<0>(P, s, 2);
  P.a.template lstore<6, 8>(P.ra[SET ^ 1], sn);
  P.b.template lstore<0, 3>(P.rb[SET ^ 1], sn);
  gemm_schedule<NR, 0, 5>();
  __builtin_amdgcn_sched_barrier(0);
  // region 3
  gemm_mfma<C, 0>(P, acc);
  P.b.template lstore<3, 8>(P.rb[SET ^ 1], sn);
  gemm_fread<1>(P, s, 3);
  gemm_schedule<NR, 0, 5>();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 256 x 256 tile over K (a multiple of 64).  `lds` holds GEMM_LDS bytes.
// AT / BT select the MN-major layout for A / B; a_kend / b_kend bound their
// k-rows (ignored for K-major operands).
template <class C, bool AT = false, bool BT = false>
__device__ __forceinline__ void gemm_tile_pipe(const bf16_t* __restrict__ A, int64_t lda, int64_t m0, int64_t m_end,
                                               const bf16_t* __restrict__ B, int64_t ldb, int64_t n0, int64_t n_end,
                                               int K, bf16_t* lds, Acc<C>& acc, int a_kend = 0, int b_kend = 0) {
  static_assert(C::BM == GemmCfg::BM && C::BN == GemmCfg::BN && C::WM == GemmCfg::WM && C::WN == GemmCfg::WN,
                "the accumulators of the 256 x 256 tile");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = f32x16{};
  GemmState<AT, BT> P;
  P.a.init(A, lda, m0, m_end, a_kend > 0 ? a_kend : K, lds, wm, lane);
  P.b.init(B, ldb, n0, n_end, b_kend > 0 ? b_kend : K, lds + GemmCfg::A_ELEMS, wn, lane);
  const int nk = K / GemmCfg::BK;
  // slice 0 into stage 0, slice 1 into register set 1
  P.a.gload(P.ra[0], 0);
  P.b.gload(P.rb[0], 0);
  P.a.gload(P.ra[1], 1 < nk ? 1 : nk - 1);
  P.b.gload(P.rb[1], 1 < nk ? 1 : nk - 1);
  P.a.lstore(P.ra[0], 0);
  P.b.lstore(P.rb[0], 0);
  __syncthreads();
  gemm_iter<C, AT, BT, 0, true>(P, 0, nk, acc);
  int kt = 1;
  for (; kt + 1 < nk; kt += 2) {
    gemm_iter<C, AT, BT, 1, false>(P, kt, nk, acc);
    gemm_iter<C, AT, BT, 0, false>(P, kt + 1, nk, acc);
  }
  if (kt < nk) gemm_iter<C, AT, BT, 1, false>(P, kt, nk, acc);
  gemm_mfma<C, 1>(P, acc);  // substep 3 of the last slice
}
