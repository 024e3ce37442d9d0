// bf16 MFMA GEMM core for gfx950: C[m][n] = sum_k A(m, k) * B(n, k).
//
// A workgroup of WM x WN wavefronts computes a BM x BN tile; each wavefront
// owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulators in registers.  Operand
// tiles are staged through LDS in BK = 32 slices (gemm_tile_pipe, either
// layout) or, for 256 x 256 tiles with both operands K-major, in BK = 64
// slices (gemm_tile_kpipe, at the end of this file).
//
// Each operand is stored in global memory in one of two layouts:
//   K-major  (MN = false): element (r, k) at P[r * ld + k]; the tile's rows
//            [r0, r_end) are read, clamped to r_end - 1.
//   MN-major (MN = true):  element (r, k) at P[k * ld + r]; the tile's
//            columns [r0, r_end) are read in aligned groups of 8, chunks
//            past the one holding column r_end - 1 clamped to it (each row
//            must hold r_end rounded up to 8 elements), from rows k < k_end
//            (clamped to k_end - 1).
// K-major slices sit in LDS as 64-byte rows (one per M/N index); MN-major
// slices as BM- (or BN-) wide rows (one per k) that reach the matrix cores
// through transposing LDS reads (ds_read_b64_tr_b16), so no operand is ever
// transposed in memory.
//
// K must be a multiple of BK.  Clamped rows or columns feed finite values
// whose results the caller discards (or whose partner operand is zero).
#pragma once
#include "kd_common.h"

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

// ---------------------------------------------------------------------------
// Pipeline: BK = 32 slices in a ring of three LDS stages.
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
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = NSTAGE * STAGE * 2;
  static constexpr int A_LD = BM * BK / 8 / NT;  // 16-byte chunks per thread per slice
  static constexpr int B_LD = BN * BK / 8 / NT;
  static constexpr int NLD = A_LD + B_LD;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile");
  static_assert((BM * BK / 8) % NT == 0 && (BN * BK / 8) % NT == 0, "loader");
};

// K-major LDS rows: 16-byte chunk c of row r is stored at chunk c ^ kswz(r).
// Fragment reads (32 consecutive rows, one chunk) and tile stores (4 chunks
// of a row per 4 lanes) then spread over all LDS banks.
__device__ __forceinline__ int kswz(int r) { return (r ^ (r >> 2)) & 3; }
// MN-major LDS rows (one per k): chunk c of row k is stored at c ^ mswz(k).
// A transposing fragment read touches 4 consecutive k-rows x 64 bytes (and
// the same 4 rows + 8); the XOR puts those 4 rows on disjoint bank quarters.
__device__ __forceinline__ int mswz(int k) { return (k & 3) << 2; }

#ifndef PIPE_BARRIER_LGKM
#define PIPE_BARRIER_LGKM 1
#endif

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// One operand of the pipeline.  ROWS = BM or BN, TW = its wavefront extent,
// NF = fragments per k-substep, LDN = 16-byte chunks per thread per slice.
template <class C, int ROWS, int TW, int NF, int LDN, bool MN>
struct PipeOperand;

template <class C, int ROWS, int TW, int NF, int LDN>
struct PipeOperand<C, ROWS, TW, NF, LDN, false> {
  static constexpr int CPR = C::BK / 8;         // chunks per 64-byte row slice
  static constexpr int RSTEP = C::NT / CPR;     // rows between a thread's chunks
  static constexpr int NREAD = NF;              // LDS read instructions per substep
  static_assert(RSTEP % 16 == 0, "K-major loader");
  const char* base;
  uint32_t off[LDN];
  bf16_t* st;                                   // this thread's store slot (stage 0)
  const bf16_t* rd[2];                          // fragment 0 of each k-substep (stage 0)

  __device__ __forceinline__ void init(const bf16_t* P, int64_t ld, int64_t r0, int64_t r_end, int,
                                       bf16_t* lds_op, int w, int lane) {
    const int tid = threadIdx.x;
    base = (const char*)(P + r0 * ld);
    const int rr = tid / CPR, k8 = (tid % CPR) * 8;
    const int nrows = (int)(r_end - r0);
#pragma unroll
    for (int i = 0; i < LDN; ++i) {
      const int r = rr + i * RSTEP;
      off[i] = (uint32_t)(((r < nrows ? r : nrows - 1) * (int)ld + k8) * 2);
    }
    // rows rr + i*RSTEP share rr's swizzle (RSTEP is a multiple of 16)
    st = lds_op + rr * C::BK + (((k8 >> 3) ^ kswz(rr)) << 3);
    // fragment rows differ from l32 by multiples of 32: same swizzle
    const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) rd[ks] = lds_op + (w * TW + l32) * C::BK + (((ks * 2 + kh) ^ kswz(l32)) << 3);
  }
  __device__ __forceinline__ void gload(u32x4* r, int slice) const {
    const uint32_t kb = (uint32_t)(slice * C::BK * 2);
#pragma unroll
    for (int i = 0; i < LDN; ++i) r[i] = *(const u32x4*)(base + (off[i] + kb));
  }
  __device__ __forceinline__ void lstore(const u32x4* r, int stage) const {
#pragma unroll
    for (int i = 0; i < LDN; ++i) *(u32x4*)(st + stage * C::STAGE + i * RSTEP * C::BK) = r[i];
  }
  __device__ __forceinline__ bf16x8 fread(int f, int stage, int ks) const {
    return *(const bf16x8*)(rd[ks] + stage * C::STAGE + f * 32 * C::BK);
  }
};

template <class C, int ROWS, int TW, int NF, int LDN>
struct PipeOperand<C, ROWS, TW, NF, LDN, true> {
  static constexpr int CPK = ROWS / 8;          // chunks per k-row
  static constexpr int KSTEP = C::NT / CPK;     // k-rows between a thread's chunks
  static constexpr int NREAD = 2 * NF;
  static_assert(KSTEP * LDN == C::BK && KSTEP % 4 == 0, "MN-major loader");
  static_assert(TW % 128 == 0 && NF <= 4, "MN-major fragment addressing");
  const char* base;
  uint32_t col;                                 // byte offset of this thread's column chunk
  uint32_t ld2;                                 // k-row pitch in bytes
  int kr, kend;
  bf16_t* st;
  const bf16_t* rd;                             // substep 0, first half, without the fragment term
  int foff[NF];                                 // fragment terms (swizzled)

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
    // m = w*TW + 32*f + 16*(g%2) + 4*(j%4): the XOR acts on the bits of f.
    const int g = lane >> 4, j = lane & 15;
    const int lowc = 2 * (g & 1) + ((j & 3) >> 1);
    rd = lds_op + (8 * (g >> 1) + (j >> 2)) * ROWS + w * TW + 8 * lowc + 4 * (j & 1);
#pragma unroll
    for (int f = 0; f < NF; ++f) foff[f] = 32 * (f ^ (j >> 2));
  }
  __device__ __forceinline__ void gload(u32x4* r, int slice) const {
#pragma unroll
    for (int i = 0; i < LDN; ++i) {
      int k = slice * C::BK + kr + i * KSTEP;
      k = k < kend ? k : kend - 1;
      r[i] = *(const u32x4*)(base + ((uint32_t)k * ld2 + col));
    }
  }
  __device__ __forceinline__ void lstore(const u32x4* r, int stage) const {
#pragma unroll
    for (int i = 0; i < LDN; ++i) *(u32x4*)(st + stage * C::STAGE + i * KSTEP * ROWS) = r[i];
  }
  __device__ __forceinline__ bf16x8 fread(int f, int stage, int ks) const {
    const bf16_t* p = rd + stage * C::STAGE + ks * 16 * ROWS + foff[f];
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 4 * ROWS));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

template <class C, bool AT, bool BT>
struct PipeState {
  PipeOperand<C, C::BM, C::TM, C::FM, C::A_LD, AT> a;
  PipeOperand<C, C::BN, C::TN, C::FN, C::B_LD, BT> b;
  u32x4 ra[2][C::A_LD], rb[2][C::B_LD];
  bf16x8 fa[2][C::FM], fb[2][C::FN];
};

template <class C, bool AT, bool BT, int SET>
__device__ __forceinline__ void pipe_gload(PipeState<C, AT, BT>& P, int slice) {
  P.a.gload(P.ra[SET], slice);
  P.b.gload(P.rb[SET], slice);
}

template <class C, bool AT, bool BT, int SET>
__device__ __forceinline__ void pipe_lstore(PipeState<C, AT, BT>& P, int stage) {
  P.a.lstore(P.ra[SET], stage);
  P.b.lstore(P.rb[SET], stage);
}

template <class C, bool AT, bool BT, int BUF>
__device__ __forceinline__ void pipe_fread(PipeState<C, AT, BT>& P, int stage, int ks) {
  // order of first use by the MFMA loop below: a0, b0..b(FN-1), a1..
  P.fa[BUF][0] = P.a.fread(0, stage, ks);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) P.fb[BUF][j] = P.b.fread(j, stage, ks);
#pragma unroll
  for (int i = 1; i < C::FM; ++i) P.fa[BUF][i] = P.a.fread(i, stage, ks);
}

template <class C, bool AT, bool BT, int BUF, int I0 = 0, int I1 = C::FM>
__device__ __forceinline__ void pipe_mfma(PipeState<C, AT, BT>& P, Acc<C>& acc) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32x32x16(P.fa[BUF][i], P.fb[BUF][j], acc.v[i][j]);
}

// Interleave of one slice for the scheduler, in two regions separated by a
// scheduling barrier.  Region 1: the first substep's MFMAs with the global
// loads and the second substep's fragment reads among them, then the first
// half of the second substep's MFMAs with the LDS stores.  Region 2: the
// rest of the second substep's MFMAs with the next slice's first fragment
// reads.  Every LDS store thus precedes those reads, which the barrier
// below relies on.
template <class C, int NFR>
__device__ __forceinline__ void pipe_schedule1() {
  constexpr int NMF = C::FM * C::FN;
  static_assert(NFR <= NMF, "fragment reads per substep");
#pragma unroll
  for (int m = 0; m < NMF; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m < NFR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (m < C::NLD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
#pragma unroll
  for (int m = 0; m < NMF / 2; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m < C::NLD) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
  }
  static_assert(C::NLD <= NMF / 2, "LDS stores per half substep");
}
template <class C, int NFR>
__device__ __forceinline__ void pipe_schedule2() {
  constexpr int NMF = C::FM * C::FN;
#pragma unroll
  for (int m = 0; m < NMF / 2; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    // spread NFR reads over NMF/2 slots
    constexpr int H = NMF / 2;
    const int r = ((m + 1) * NFR) / H - (m * NFR) / H;
    if (r == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (r == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  static_assert(NFR <= NMF, "at most two reads per slot");
}

// End-of-slice barrier.  Every LDS store and every read of the slice just
// consumed precede the last N reads (the next slice's first fragments, from a
// stage completed earlier), so waiting until at most N LDS operations are
// outstanding orders all cross-wavefront hazards while those N reads stay in
// flight across the barrier.
template <int N>
__device__ __forceinline__ void pipe_barrier() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt");
  if constexpr (PIPE_BARRIER_LGKM) {
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
  } else {
    __syncthreads();
  }
}

template <class C, bool AT, bool BT, int SET>
__device__ __forceinline__ void pipe_iter(PipeState<C, AT, BT>& P, int kt, int nk, Acc<C>& acc) {
  constexpr int NFR = decltype(P.a)::NREAD + decltype(P.b)::NREAD;
  pipe_gload<C, AT, BT, SET ^ 1>(P, kt + 3 < nk ? kt + 3 : nk - 1);
  pipe_fread<C, AT, BT, 1>(P, kt % 3, 1);
  pipe_mfma<C, AT, BT, 0>(P, acc);
  pipe_mfma<C, AT, BT, 1, 0, C::FM / 2>(P, acc);
  pipe_lstore<C, AT, BT, SET>(P, (kt + 2) % 3);
  pipe_schedule1<C, NFR>();
  __builtin_amdgcn_sched_barrier(0);
  pipe_mfma<C, AT, BT, 1, C::FM / 2, C::FM>(P, acc);
  pipe_fread<C, AT, BT, 0>(P, (kt + 1) % 3, 0);
  pipe_schedule2<C, NFR>();
  pipe_barrier<(NFR < 15 ? NFR : 15)>();
}

// One BM x BN tile over K (a multiple of 32).  `lds` holds C::LDS_BYTES.
// AT / BT select the MN-major layout for A / B; a_kend / b_kend bound their
// k-rows (ignored for K-major operands).
template <class C, bool AT = false, bool BT = false>
__device__ __forceinline__ void gemm_tile_pipe(const bf16_t* __restrict__ A, int64_t lda, int64_t m0, int64_t m_end,
                                               const bf16_t* __restrict__ B, int64_t ldb, int64_t n0, int64_t n_end,
                                               int K, bf16_t* lds, Acc<C>& acc, int a_kend = 0, int b_kend = 0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = f32x16{};
  PipeState<C, AT, BT> P;
  P.a.init(A, lda, m0, m_end, a_kend > 0 ? a_kend : K, lds, wm, lane);
  P.b.init(B, ldb, n0, n_end, b_kend > 0 ? b_kend : K, lds + C::A_ELEMS, wn, lane);

  const int nk = K / C::BK;
  const int last = nk - 1;
  pipe_gload<C, AT, BT, 0>(P, 0);
  pipe_gload<C, AT, BT, 1>(P, 1 < nk ? 1 : last);
  pipe_lstore<C, AT, BT, 0>(P, 0);
  pipe_lstore<C, AT, BT, 1>(P, 1);
  pipe_gload<C, AT, BT, 0>(P, 2 < nk ? 2 : last);
  __syncthreads();
  pipe_fread<C, AT, BT, 0>(P, 0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    pipe_iter<C, AT, BT, 0>(P, kt, nk, acc);
    pipe_iter<C, AT, BT, 1>(P, kt + 1, nk, acc);
  }
  if (kt < nk) pipe_iter<C, AT, BT, 0>(P, kt, nk, acc);
}

// ---------------------------------------------------------------------------
// K-major pipeline: BK = 64 slices in two LDS stages, for 256 x 256 tiles of
// four 128 x 128 wavefronts whose operands are both K-major.  Each slice
// feeds four 16-deep substeps of 16 MFMAs; the global loads of slice kt+2
// and the LDS stores of slice kt+1 hide behind them, so the workgroup meets
// one barrier per 64 of K instead of per 32.  Same MFMA, accumulator layout
// and order of the 16-deep k-chunks as gemm_tile_pipe, so C is bitwise the
// same.
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
// previous iteration) completed before that barrier.
// ---------------------------------------------------------------------------
constexpr int KP_BK = 64;
constexpr int KP_STAGE = 2 * 256 * KP_BK;                    // A and B elements of one slice
constexpr int KPIPE_LDS = 2 * KP_STAGE * (int)sizeof(bf16_t);  // 128 KB

// 128-byte K-major LDS rows: chunk c of row r at c ^ kpswz(r).  Rows 2j and
// 2j+1 share a 256-byte bank span; (r >> 1) & 7 spreads the same chunk of 16
// consecutive rows over the 16 sixteen-byte bank slots.
__device__ __forceinline__ int kpswz(int r) { return (r >> 1) & 7; }

struct KPipeOperand {
  static constexpr int CPR = KP_BK / 8;  // 16-byte chunks per row slice
  static constexpr int RSTEP = 256 / CPR;  // rows between a thread's chunks
  static constexpr int LDN = 256 / RSTEP;  // chunks per thread per slice
  static_assert(RSTEP % 16 == 0, "rows rr + i*RSTEP share rr's swizzle");
  const char* base;
  uint32_t off[LDN];
  bf16_t* st;
  const bf16_t* rd[4];  // fragment 0 of each k-substep (stage 0)

  __device__ __forceinline__ void init(const bf16_t* P, int64_t ld, int64_t r0, int64_t r_end, bf16_t* lds_op,
                                       int w, int lane) {
    const int tid = threadIdx.x;
    base = (const char*)(P + r0 * ld);
    const int rr = tid / CPR, c = tid % CPR;
    const int nrows = (int)(r_end - r0);
#pragma unroll
    for (int i = 0; i < LDN; ++i) {
      const int r = rr + i * RSTEP;
      off[i] = (uint32_t)(((r < nrows ? r : nrows - 1) * (int)ld + c * 8) * 2);
    }
    st = lds_op + rr * KP_BK + ((c ^ kpswz(rr)) << 3);
    // fragment rows differ from l32 by multiples of 32: same swizzle
    const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rd[ks] = lds_op + (w * 128 + l32) * KP_BK + (((ks * 2 + kh) ^ kpswz(l32)) << 3);
  }
  __device__ __forceinline__ void gload(u32x4* r, int slice) const {
    const uint32_t kb = (uint32_t)(slice * KP_BK * 2);
#pragma unroll
    for (int i = 0; i < LDN; ++i) r[i] = *(const u32x4*)(base + (off[i] + kb));
  }
  template <int I0, int I1>
  __device__ __forceinline__ void lstore(const u32x4* r, int stage) const {
#pragma unroll
    for (int i = I0; i < I1; ++i) *(u32x4*)(st + stage * KP_STAGE + i * RSTEP * KP_BK) = r[i];
  }
  __device__ __forceinline__ bf16x8 fread(int f, int stage, int ks) const {
    return *(const bf16x8*)(rd[ks] + stage * KP_STAGE + f * 32 * KP_BK);
  }
};

struct KPipeState {
  KPipeOperand a, b;
  u32x4 ra[2][KPipeOperand::LDN], rb[2][KPipeOperand::LDN];
  bf16x8 fa[2][4], fb[2][4];
};

template <int BUF>
__device__ __forceinline__ void kp_fread(KPipeState& P, int stage, int ks) {
  P.fa[BUF][0] = P.a.fread(0, stage, ks);
#pragma unroll
  for (int j = 0; j < 4; ++j) P.fb[BUF][j] = P.b.fread(j, stage, ks);
#pragma unroll
  for (int i = 1; i < 4; ++i) P.fa[BUF][i] = P.a.fread(i, stage, ks);
}

template <class C, int BUF>
__device__ __forceinline__ void kp_mfma(KPipeState& P, Acc<C>& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[i][j] = mfma32x32x16(P.fa[BUF][i], P.fb[BUF][j], acc.v[i][j]);
}

// 16 MFMAs with NR fragment reads, NL global loads and NS LDS stores spread
// among them.
template <int NR, int NL, int NS>
__device__ __forceinline__ void kp_schedule() {
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (m < NS) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (m < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

template <class C, int SET, bool FIRST>
__device__ __forceinline__ void kp_iter(KPipeState& P, int kt, int nk, Acc<C>& acc) {
  const int s = kt & 1, sn = s ^ 1;
  const int ld = kt + 2 < nk ? kt + 2 : nk - 1;
  // region 0
  if constexpr (!FIRST) kp_mfma<C, 1>(P, acc);
  kp_fread<0>(P, s, 0);
  P.a.gload(P.ra[SET], ld);
  if constexpr (!FIRST) kp_schedule<8, 8, 0>();
  __builtin_amdgcn_sched_barrier(0);
  // region 1
  kp_mfma<C, 0>(P, acc);
  kp_fread<1>(P, s, 1);
  P.b.gload(P.rb[SET], ld);
  P.a.lstore<0, 6>(P.ra[SET ^ 1], sn);
  kp_schedule<8, 8, 6>();
  __builtin_amdgcn_sched_barrier(0);
  // region 2
  kp_mfma<C, 1>(P, acc);
  kp_fread<0>(P, s, 2);
  P.a.lstore<6, 8>(P.ra[SET ^ 1], sn);
  P.b.lstore<0, 3>(P.rb[SET ^ 1], sn);
  kp_schedule<8, 0, 5>();
  __builtin_amdgcn_sched_barrier(0);
  // region 3
  kp_mfma<C, 0>(P, acc);
  P.b.lstore<3, 8>(P.rb[SET ^ 1], sn);
  kp_fread<1>(P, s, 3);
  kp_schedule<8, 0, 5>();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 256 x 256 tile over K (a multiple of 64), both operands K-major, rows
// clamped as in gemm_tile_pipe.  `lds` holds KPIPE_LDS bytes.
template <class C>
__device__ __forceinline__ void gemm_tile_kpipe(const bf16_t* __restrict__ A, int64_t lda, int64_t m0, int64_t m_end,
                                                const bf16_t* __restrict__ B, int64_t ldb, int64_t n0, int64_t n_end,
                                                int K, bf16_t* lds, Acc<C>& acc) {
  static_assert(C::BM == 256 && C::BN == 256 && C::WM == 2 && C::WN == 2, "256 x 256 tile of 128 x 128 wavefronts");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc.v[i][j] = f32x16{};
  KPipeState P;
  P.a.init(A, lda, m0, m_end, lds, wm, lane);
  P.b.init(B, ldb, n0, n_end, lds + 256 * KP_BK, wn, lane);
  const int nk = K / KP_BK;
  // slice 0 into stage 0, slice 1 into register set 1
  P.a.gload(P.ra[0], 0);
  P.b.gload(P.rb[0], 0);
  P.a.gload(P.ra[1], 1 < nk ? 1 : nk - 1);
  P.b.gload(P.rb[1], 1 < nk ? 1 : nk - 1);
  P.a.lstore<0, KPipeOperand::LDN>(P.ra[0], 0);
  P.b.lstore<0, KPipeOperand::LDN>(P.rb[0], 0);
  __syncthreads();
  kp_iter<C, 0, true>(P, 0, nk, acc);
  int kt = 1;
  for (; kt + 1 < nk; kt += 2) {
    kp_iter<C, 1, false>(P, kt, nk, acc);
    kp_iter<C, 0, false>(P, kt + 1, nk, acc);
  }
  if (kt < nk) kp_iter<C, 1, false>(P, kt, nk, acc);
  kp_mfma<C, 1>(P, acc);  // substep 3 of the last slice
}
