// Quintic Newton-Schulz core on gfx950 bf16 matrix cores.
//
// One iteration X <- a X + (b A + c A A) X with A = X X^T (the "new optimizer"
// thread, tweets 5/8 and 6/8: a quintic Newton-Schulz iteration in bfloat16)
// is three batched GEMM launches over every matrix of a call:
//   GRAM    A = bf16(X X^T)              K = n, symmetric: only tiles touching
//                                        the upper triangle, mirrored on store
//   POLY    B = bf16(b A + c (A A^T))    K = m, symmetric (A is exactly
//                                        symmetric, so A A = A A^T)
//   UPDATE  X' = bf16(a X + B X)         K = m, X read k-major
// Products accumulate in fp32 on v_mfma_f32_32x32x16_bf16; the epilogue
// combinations are plain fp32 products and sums (no fused multiply-add) and
// every stored value is rounded to bf16, nearest-even.
//
// Pipeline: WAVES_M x WAVES_N waves over a BM x BN output tile.  K advances in
// slices of 64 through a ring of NSTAGE LDS buffers filled by
// global_load_lds_dwordx4 (global memory straight into LDS, no registers):
// NSTAGE-1 slices are in flight while one is multiplied, and every row
// segment fetched is a whole 128-byte line.  Each lane's 16-byte DMA slot is
// fixed by its lane id, so a tile's XOR swizzle is applied on the global side
// (each lane fetches the chunk that belongs in its slot).  UPDATE blocks are
// persistent, one per CU: while a tile's epilogue stages and stores its
// output, the first K slice of the block's next tile is already on its way
// into the other stage.  k-contiguous tiles
// (X for GRAM, A for POLY, B for UPDATE) feed MFMA fragments with
// ds_read_b128; the k-major X tile of UPDATE is read with ds_read_b64_tr_b16
// (see read_tr_frag).  The swizzles assume gfx950's LDS of 64 four-byte
// banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bf16_util.h"
#include "muon_internal.h"

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt_hi[15:14],
// expcnt[6:4], lgkmcnt[11:8]): wait until at most n vector-memory operations
// are outstanding and every LDS operation has completed.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8); }

template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(n));
}

// Wait until at most `after` K slices of PER transfers each (issued after the
// one needed now) are in flight; `after` is below NSTAGE - 1.
template <int PER, int NSTAGE>
__device__ __forceinline__ void wait_slices(int after) {
  if (NSTAGE > 7 && after >= 6) wait_vm_lgkm0<6 * PER>();
  else if (NSTAGE > 6 && after == 5) wait_vm_lgkm0<5 * PER>();
  else if (NSTAGE > 5 && after == 4) wait_vm_lgkm0<4 * PER>();
  else if (NSTAGE > 4 && after == 3) wait_vm_lgkm0<3 * PER>();
  else if (NSTAGE > 3 && after == 2) wait_vm_lgkm0<2 * PER>();
  else if (NSTAGE > 2 && after == 1) wait_vm_lgkm0<PER>();
  else wait_vm_lgkm0<0>();
}

// k-contiguous tile, K slice of BK elements: rows of 2 BK bytes.  A fragment
// read has 16 lanes on 16 consecutive rows at one 16-byte chunk.  128-byte
// rows (BK 64, 8 chunks): two rows share a 256-byte bank line, so XOR by
// (r/2)%8.  64-byte rows (BK 32, 4 chunks): four rows share one, so XOR by
// (r/4)%4.  Either way the 16 reads land on 16 distinct chunks.
template <int BK>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  static_assert(BK == 64 || BK == 32, "k-contiguous rows of 64 or 128 bytes");
  return BK == 64 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}
// k-major tile: rows of BN*2 bytes.  A transposing read has each 16-lane
// group on 4 consecutive rows, 32 bytes each, and pairs of groups 32 bytes
// apart; XOR by 4(r%4) moves the 4 rows into different 64-byte bank groups.
// The extra XOR by (r/4)%4 stays inside each 64-byte group (so the
// transposing reads keep their banks) and spreads the epilogue's reads of
// one column over 32 consecutive rows across 16 chunks.
__device__ __forceinline__ int swz_n(int row, int chunk) { return chunk ^ (4 * (row & 3)) ^ ((row >> 2) & 3); }

// B fragments of one k-step from a k-major LDS tile: two transposing reads
// per 32-column fragment (ds_read_b64_tr_b16 transposes 16-bit elements
// across each group of 16 lanes: with lane L of a group addressing row
// k0 + L/4, columns j0 + 4(L%4) .. +3, lane i of the group receives column
// j0 + i, rows k0 .. k0+3).  The compiler waits for these reads where their
// results are used and, in this kernel, inserts no wait for the in-flight
// global -> LDS transfers before them (checked in the generated code).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 read_tr_frag(uint32_t lo_addr, uint32_t hi_addr) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(uintptr_t)lo_addr);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(uintptr_t)hi_addr);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace

// State a block carries from one of its tiles to the next.
struct TileCarry {
  bool pre;        // slice 0 of the next tile is already in flight into stage 0
  bool prev_full;  // the previous tile issued all of its copy-out stores
};

// One output tile: work item idx of the list (not a padding item).  PERSIST:
// the blocks of the launch are persistent and each walks several items (only
// for UPDATE, which then prefetches across tiles).
template <int KIND, int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int ROWU, int BK, bool PERSIST>
__device__ __forceinline__ void ns_gemm_tile(const MatDesc* __restrict__ descs, const GemmItem* __restrict__ items,
                                             int n_items, int idx, int src, float ca, float cb, float cc,
                                             float* __restrict__ part, TileCarry& carry) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;   // threads
  constexpr bool NN = (KIND == GEMM_UPDATE);   // B operand stored k-major
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;            // 32x32 MFMA tiles per wave
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / (16 * NT);  // DMA instructions per wave per stage
  constexpr int B_INSTR = B_BYTES / (16 * NT);
  constexpr int LPW = A_INSTR + B_INSTR;
  constexpr int NCHUNK_N = BN / 8;  // chunks per k-major row
  constexpr int RB = BK * 2;        // bytes per k-contiguous row of a slice
  constexpr int CPR = BK / 8;       // 16-byte chunks per k-contiguous row
  constexpr int RPI = 1024 / RB;    // k-contiguous rows per wave DMA instruction
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && A_INSTR * 16 * NT == A_BYTES && B_INSTR * 16 * NT == B_BYTES,
                "tile does not split into whole DMA instructions");
  static_assert(NSTAGE >= 2 && NSTAGE <= 8 && TM >= 1 && TN >= 1, "unsupported tile");
  static_assert((NSTAGE - 2) * (A_INSTR + B_INSTR) <= 63, "in-flight transfers beyond the wait counter");
  static_assert(!PERSIST || KIND == GEMM_UPDATE, "only the update launch is persistent");
  static_assert(!NN || BK == 64, "the k-major X slice is read 64 rows at a time");
  static_assert(!NN || ((TN == 2 || TN == 4) && BM % 32 == 0 && BK % 32 == 0 && ROWU % 32 == 0),
                "UPDATE tiling: 32-row blocks of the tile each inside one K slice");
  static_assert(NN || ROWU == BM, "symmetric tiles are addressed in units of their own size");
  static_assert(!NN || BN >= 128, "k-major swizzle needs 16 chunks per row");
  // Persistent UPDATE blocks (one per CU, each walking its tiles) fetch the
  // next tile's first K slice into stage 0 while the current tile's epilogue
  // runs, so the staged output tile lives past stage 0.
  constexpr bool PF = NN && PERSIST;
  static_assert(!PF || NSTAGE == 2, "cross-tile prefetch: the last slice of a tile sits in stage 1");
  constexpr int E_OFF = PF ? STAGE_BYTES : 0;  // byte offset of the staged output tile
  // Staged output rows: BN bf16 values.  A power-of-two count of 16-byte
  // chunks (at least 16) is laid out with an XOR swizzle; fewer chunks get a
  // row pitch one chunk longer instead, which moves consecutive rows to
  // other banks by itself.
  constexpr int RCH = BN / 8;  // 16-byte chunks per staged row
  constexpr bool E_SWZ = (RCH >= 16) && ((RCH & (RCH - 1)) == 0);
  constexpr int ROWB = E_SWZ ? BN * 2 : BN * 2 + 16;  // staged row pitch in bytes
  constexpr int LDS_BYTES = (E_OFF + BM * ROWB > NSTAGE * STAGE_BYTES) ? E_OFF + BM * ROWB : NSTAGE * STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  // byte offsets of slice s's A and B operand buffers
  auto a_off = [](int s) { return (s % NSTAGE) * STAGE_BYTES; };
  auto b_off = [](int s) { return (s % NSTAGE) * STAGE_BYTES + A_BYTES; };

  const GemmItem it = items[idx];
  const MatDesc& d = descs[it.mat];
  const uint16_t* Aop;
  const uint16_t* Bop;
  MUON_GLOBAL uint16_t* C;
  int lda, ldb, ldc;
  if (KIND == GEMM_GRAM) {
    Aop = d.X[src]; Bop = Aop; lda = ldb = d.ld_x; C = gptr(d.A); ldc = d.ld_a;
  } else if (KIND == GEMM_POLY) {
    Aop = d.A; Bop = Aop; lda = ldb = d.ld_a; C = gptr(d.B); ldc = d.ld_a;
  } else {
    Aop = d.B; lda = d.ld_a; Bop = d.X[src]; ldb = d.ld_x; C = gptr(d.X[src ^ 1]);
    ldc = d.ld_x;
  }
  // Output rows are rows of Aop.  An UPDATE tile starts at a multiple of
  // ROWU = 64 rows and may hang over m_pad: its rows past m_pad fetch rows of
  // the A/B buffers' spare block, compute values that are never stored.
  const int row0 = it.ti * ROWU;
  const int col0 = it.tj * BN;  // output columns: rows of Bop (GRAM/POLY), columns of X (UPDATE)
  const int row_lim = d.m_pad;
  // The item walks K slices k0 .. k0+kn-1 (the host stops at the true n or
  // m, past which the padding is zero; an UPDATE item's count is even).
  const int KT = it.kn;
  // K is walked in order, slice s = k-range (k0+s)*BK .. +BK-1, by every
  // tile: the row tiles of one UPDATE column block fetch the same X slices at
  // about the same time and share them in L2.
  const int k0 = it.k0;
  auto kt_of = [&](int s) { return k0 + s; };

  // In the persistent UPDATE loop an opaque zero makes lane-derived offsets
  // be recomputed per tile instead of hoisted out of the loop, where they
  // would stay live across it.
  int opq0 = 0;
  if constexpr (PF) asm volatile("v_mov_b32 %0, 0" : "=v"(opq0));
  const int tid = threadIdx.x + opq0;
  const int lane = tid & 63;
  // the wave index is uniform: held in a scalar register, so the wave's
  // tile offsets derived from it cost no vector registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave / WAVES_N, wj = wave % WAVES_N;

  // DMA sources.  Instruction q of this wave fills LDS slots
  // g*64 + lane, g = wave*INSTR + q; its rows are a wave-uniform base plus a
  // lane part, and the swizzle depends on g only through g % 2, so each
  // operand needs two per-lane offsets.
  int a_vo[2], b_vo[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    {
      // the swizzle repeats every 16 rows: 2 instructions of 8 rows (BK 64)
      // or 1 of 16 (BK 32), so instruction parity p is all it needs
      const int row = p * RPI + lane / CPR;
      a_vo[p] = (lane / CPR) * lda + swz_k<BK>(row, lane % CPR) * 8;
    }
    if (!NN) {
      const int row = p * RPI + lane / CPR;
      b_vo[p] = (lane / CPR) * ldb + swz_k<BK>(row, lane % CPR) * 8;
    } else {
      b_vo[p] = 0;  // k-major: the swizzle depends on more than g % 2, computed per instruction
    }
  }
  // A diagonal tile of a symmetric product multiplies a row block by itself:
  // its B operand is the A slice already in LDS, fetched once.
  const bool same_rows = !NN && row0 == col0;
  auto issue = [&](int s) {
    const int kt = kt_of(s);
    LDS_AS char* st = (LDS_AS char*)lds + a_off(s);
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) {
      const int g = wave * A_INSTR + q;
      const uint16_t* src_row = Aop + (int64_t)(row0 + g * RPI) * lda + (int64_t)kt * BK;
      __builtin_amdgcn_global_load_lds((const void*)(src_row + a_vo[g & 1]), (LDS_AS void*)(st + g * 1024), 16, 0, 0);
    }
    if (same_rows) return;
#pragma unroll
    for (int q = 0; q < B_INSTR; ++q) {
      const int g = wave * B_INSTR + q;
      const uint16_t* src_row;
      int vo;
      if (NN) {
        const int row = g * (64 / NCHUNK_N) + lane / NCHUNK_N;  // row within the slice
        src_row = Bop + (int64_t)(kt * BK + g * (64 / NCHUNK_N)) * ldb + col0;
        vo = (lane / NCHUNK_N) * ldb + swz_n(row, lane % NCHUNK_N) * 8;
      } else {
        src_row = Bop + (int64_t)(col0 + g * RPI) * ldb + (int64_t)kt * BK;
        vo = b_vo[g & 1];
      }
      __builtin_amdgcn_global_load_lds((const void*)(src_row + vo), (LDS_AS void*)(st + A_BYTES + g * 1024), 16, 0, 0);
    }
  };
  // slice 0 of another UPDATE tile of this call into stage 0
  auto issue_first = [&](const GemmItem& nit) {
    const MatDesc& nd = descs[nit.mat];
    const uint16_t* nA = nd.B;
    const uint16_t* nB = nd.X[src];
    const int nlda = nd.ld_a, nldb = nd.ld_x;
    const int nrow0 = nit.ti * ROWU, ncol0 = nit.tj * BN;
    LDS_AS char* st = (LDS_AS char*)lds;
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) {
      const int g = wave * A_INSTR + q;
      const int row = (g & 1) * RPI + lane / CPR;
      const int vo = (lane / CPR) * nlda + swz_k<BK>(row, lane % CPR) * 8;
      const uint16_t* src_row = nA + (int64_t)(nrow0 + g * RPI) * nlda;
      __builtin_amdgcn_global_load_lds((const void*)(src_row + vo), (LDS_AS void*)(st + g * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < B_INSTR; ++q) {
      const int g = wave * B_INSTR + q;
      const int row = g * (64 / NCHUNK_N) + lane / NCHUNK_N;
      const uint16_t* src_row = nB + (int64_t)(g * (64 / NCHUNK_N)) * nldb + ncol0;
      const int vo = (lane / NCHUNK_N) * nldb + swz_n(row, lane % NCHUNK_N) * 8;
      __builtin_amdgcn_global_load_lds((const void*)(src_row + vo), (LDS_AS void*)(st + A_BYTES + g * 1024), 16, 0, 0);
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int nj = 0; nj < TN; ++nj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][nj][e] = 0.0f;

  // LDS byte offsets (within a stage) of this lane's fragment reads at k-step
  // 0 of a stage: chunk lane/32 of each k-contiguous row.
  int a_rd[TM], b_rd[TN][2];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
    const int r = wi * WTM + mi * 32 + (lane & 31);
    a_rd[mi] = r * RB + swz_k<BK>(r, lane >> 5) * 16;
  }
#pragma unroll
  for (int nj = 0; nj < TN; ++nj) {
    if (!NN) {
      const int r = wj * WTN + nj * 32 + (lane & 31);
      b_rd[nj][0] = (same_rows ? 0 : A_BYTES) + r * RB + swz_k<BK>(r, lane >> 5) * 16;
      b_rd[nj][1] = 0;
    } else {
      const int g = (lane >> 4) & 3, l16 = lane & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 8 * (g >> 1) + 4 * h + (l16 >> 2);
        const int j = wj * WTN + nj * 32 + 16 * (g & 1) + 4 * (l16 & 3);
        b_rd[nj][h] = k * (BN * 2) + swz_n(k, j >> 3) * 16 + (j & 7) * 2;  // within the X slice
      }
    }
  }

  auto read_a_rows = [&](const LDS_AS char* st, int kk, int m0, int m1, bf16x8* af) {
    // k-step kk reads logical chunk 2kk + lane/32; the swizzle is an XOR, so
    // that is the k-step-0 chunk XOR 2kk, i.e. the byte offset XOR 32kk.
#pragma unroll
    for (int mi = m0; mi < m1; ++mi)
      af[mi] = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4*)(st + (a_rd[mi] ^ (32 * kk))));
  };
  auto read_b_tr = [&](uint32_t st_addr, int kk, bf16x8* bfr) {
    // k-step kk is 16 rows further on; (row % 4), hence the swizzle, is unchanged
    const uint32_t dk = st_addr + kk * 16 * (BN * 2);
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) bfr[nj] = read_tr_frag(dk + b_rd[nj][0], dk + b_rd[nj][1]);
  };
  auto mfma_rows = [&](int m0, int m1, const bf16x8* af, const bf16x8* bfr) {
    // operands swapped so each lane ends up with 4 consecutive output columns
#pragma unroll
    for (int mi = m0; mi < m1; ++mi)
#pragma unroll
      for (int nj = 0; nj < TN; ++nj)
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nj], af[mi], acc[mi][nj], 0, 0, 0);
  };

  // A diagonal tile keeps only its values on and above the diagonal (the
  // mirror supplies the rest): a wave whose sub-tile lies strictly below it
  // multiplies nothing.
  // Likewise a wave whose sub-tile lies wholly in the zero padding past the
  // true m rows (or m / n columns) keeps its zero accumulators, which are
  // exactly the padding's values.
  const int out_cols = NN ? d.n : d.m;
  const bool skip_wave = (same_rows && wi * WTM >= wj * WTN + WTN) || row0 + wi * WTM >= d.m ||
                         col0 + wj * WTN >= out_cols;
  auto compute = [&](int s) {
    if (skip_wave) return;
    const LDS_AS char* st = (const LDS_AS char*)lds + a_off(s);
    const uint32_t st_addr = (uint32_t)(uintptr_t)((const LDS_AS char*)lds + b_off(s));
    if constexpr (!NN) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[TM], bfr[TN];
        read_a_rows(st, kk, 0, TM, af);
#pragma unroll
        for (int nj = 0; nj < TN; ++nj)
          bfr[nj] = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4*)(st + (b_rd[nj][0] ^ (32 * kk))));
        mfma_rows(0, TM, af, bfr);
      }
    } else {
      // Operands of k-step kk+1 are read between the two halves of k-step kk's
      // MFMAs, so their latency overlaps queued MFMA work.  A
      // fragments: the first half is refreshed for kk+1 once its MFMAs have
      // issued; the second half is read for kk at the start of the step.
      constexpr int MH = (TM + 1) / 2;
      bf16x8 af[TM], bfr[2][TN];
      read_a_rows(st, 0, 0, MH, af);
      read_b_tr(st_addr, 0, bfr[0]);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cur = kk & 1;
        read_a_rows(st, kk, MH, TM, af);
        mfma_rows(0, MH, af, bfr[cur]);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < BK / 16) {
          read_a_rows(st, kk + 1, 0, MH, af);
          read_b_tr(st_addr, kk + 1, bfr[cur ^ 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(MH, TM, af, bfr[cur]);
      }
    }
  };

  // Epilogue inputs come out of staged K slices that already hold them, so
  // they cost no extra global traffic; both are picked up during the loop.
  // POLY: A[i][j] is column k = j of the A slice.  UPDATE: X[i][j] is row
  // k = i of the k-major X slice.  The epilogue combines them in the fixed
  // order of the storage-point reading.
  u32x2 ein[TM][TN][4];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int nj = 0; nj < TN; ++nj)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) ein[mi][nj][e4] = u32x2{0u, 0u};
  auto capture_poly = [&](int s) {
    const LDS_AS char* st = (const LDS_AS char*)lds + a_off(s);
    const int kt = kt_of(s);
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) {
      const int cbase = col0 + wj * WTN + nj * 32;  // 32 columns inside one K slice
      if (cbase / BK != kt) continue;
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int ar = wi * WTM + mi * 32 + (lane & 31);
          const int kl = cbase % BK + 8 * e4 + 4 * (lane >> 5);
          ein[mi][nj][e4] = *(const LDS_AS u32x2*)(st + ar * RB + swz_k<BK>(ar, kl >> 3) * 16 + (kl & 7) * 2);
        }
    }
  };
  // With the cross-tile prefetch the LDS past the two stages is idle during
  // the K loop; the a.X values of each wave's last 32-row block wait there
  // (in register order, 8 bytes a lane) instead of in registers.
  constexpr int PARK_OFF = NSTAGE * STAGE_BYTES;
  constexpr int PARK_MI = PF ? TM - 1 : TM;  // TM: nothing parked
  static_assert(!PF || PARK_OFF + (NT / 64) * TN * 4 * 512 <= LDS_BYTES, "parking space");
  auto park_addr = [&](int nj, int e4) {
    return (LDS_AS char*)lds + PARK_OFF + ((wave * TN + nj) * 4 + e4) * 512 + lane * 8;
  };
  auto capture_update = [&](int s) {
    // slice s holds X rows s*BK .. s*BK+BK-1; a 32-row block of output rows
    // lies inside one slice (rows past m_pad fall in none and are not stored)
    const LDS_AS char* slice = (const LDS_AS char*)lds + b_off(s);
    const int kt = kt_of(s);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const int grow = row0 + wi * WTM + mi * 32;
      if (grow / BK != kt) continue;
      const int lr = grow % BK + (lane & 31);
#pragma unroll
      for (int nj = 0; nj < TN; ++nj)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int cl = wj * WTN + nj * 32 + 8 * e4 + 4 * (lane >> 5);
          const u32x2 xv = *(const LDS_AS u32x2*)(slice + lr * (BN * 2) + swz_n(lr, cl >> 3) * 16 + (cl & 7) * 2);
          if (mi == PARK_MI)
            *(LDS_AS u32x2*)park_addr(nj, e4) = xv;
          else
            ein[mi][nj][e4] = xv;
        }
    }
  };

  // Main loop over s = 0 .. KT-1 (slice kt_of(s), stage buffer s % NSTAGE).
  // Slice s is complete once this wave has at most (slices issued after it)
  // x LPW DMA operations outstanding and every wave has passed the barrier;
  // the buffer refilled next was last read in step s-1, which every wave
  // finished (its LDS reads included) before the barrier.
  if (!carry.pre) {
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < KT) issue(s);
  }
  constexpr int NSTORE = BM * (BN / 8) / NT;  // copy-out stores per lane
  for (int s = 0; s < KT; ++s) {
    // slices issued after s: min(NSTAGE - 2, KT - 1 - s), each LPW transfers
    // per wave (A_INSTR on a diagonal tile, which fetches one operand)
    const int after = min(NSTAGE - 2, KT - 1 - s);
    if (PF && s == 0 && carry.pre) {
      // slice 0 went out before the previous tile's copy-out stores; vector
      // memory operations complete in order, so it has landed once at most
      // those stores remain
      if (carry.prev_full) wait_vm_lgkm0<NSTORE>(); else wait_vm_lgkm0<0>();
    } else if (same_rows) {
      wait_slices<A_INSTR, NSTAGE>(after);
    } else {
      wait_slices<LPW, NSTAGE>(after);
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + NSTAGE - 1 < KT) issue(s + NSTAGE - 1);
    if constexpr (KIND == GEMM_POLY) capture_poly(s);
    if constexpr (NN) capture_update(s);
    compute(s);
  }

  // Epilogue.  Lane holds, for MFMA tile (mi, nj) and quad e4, output row
  // i = wi*WTM + mi*32 + lane%32 and columns j .. j+3 with
  // j = wj*WTN + nj*32 + 8*e4 + 4*(lane/32) (tile-relative).
  if constexpr (KIND == GEMM_GRAM) {
    if (it.slot >= 0) {
      // K chunk of a split tile: its fp32 partial sums, unrounded, for the
      // reduce pass (BM x BN row-major)
      float* pt = part + (size_t)it.slot * (BM * BN);
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int nj = 0; nj < TN; ++nj)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int r = wi * WTM + mi * 32 + (lane & 31);
            const int c = wj * WTN + nj * 32 + 8 * e4 + 4 * (lane >> 5);
            *reinterpret_cast<float4*>(pt + r * BN + c) = float4{acc[mi][nj][4 * e4], acc[mi][nj][4 * e4 + 1],
                                                                 acc[mi][nj][4 * e4 + 2], acc[mi][nj][4 * e4 + 3]};
          }
      return;
    }
  }
  // Results are rounded to bf16 and staged in LDS (the pipeline buffers are
  // free now), then written out as whole 16-byte row segments.
  bool has_next = false;
  if constexpr (PF) {
    // Every wave released stage 0 (slice KT-2) at the last step's barrier, so
    // the next tile's first slice goes out at once; each wave then collects
    // the a.X values it parked itself.  The barrier below keeps the staged
    // tile from overwriting stage 1 or the parking space while another wave
    // still reads them.
    int nidx = idx + gridDim.x;
    while (nidx < n_items && items[nidx].mat < 0) nidx += gridDim.x;
    has_next = nidx < n_items;  // stage 0 is free: KT is even, the last slice sits in stage 1
    if (has_next) issue_first(items[nidx]);
#pragma unroll
    for (int nj = 0; nj < TN; ++nj)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) ein[PARK_MI][nj][e4] = *(const LDS_AS u32x2*)park_addr(nj, e4);
    wait_vm_lgkm0<63>();  // LDS only: the prefetch stays in flight
  } else {
    wait_vm_lgkm0<0>();
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  LDS_AS char* E = (LDS_AS char*)lds + E_OFF;
  static_assert(KIND == GEMM_UPDATE || BM == BN, "symmetric tiles are square");
  static_assert(BM * ROWB <= LDS_BYTES, "staging does not fit");
  static_assert(E_SWZ || (RCH & (RCH - 1)) == 0, "staged rows of a power-of-two chunk count");
  // Chunk swizzle of a staged row.  Copy-out reads 16 lanes along one row
  // (any XOR keeps them distinct); the transposing reads of the mirror put a
  // 32-lane half on 4 consecutive rows and 4 consecutive chunks, which the
  // XOR by 4 (r % 4) sends to 4 different 64-byte bank groups.
  auto ech = [&](int r, int c) { return E_SWZ ? c ^ (4 * (r & 3)) ^ ((r >> 2) & 3) : c; };
  const bool diag = (KIND != GEMM_UPDATE) && (row0 == col0);
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int r = wi * WTM + mi * 32 + (lane & 31);
        const int c = wj * WTN + nj * 32 + 8 * e4 + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = acc[mi][nj][4 * e4 + k];
        if (KIND != GEMM_GRAM) {
          const u32x2 e2 = ein[mi][nj][e4];
          const float ev[4] = {bf16_lo(e2.x), bf16_hi(e2.x), bf16_lo(e2.y), bf16_hi(e2.y)};
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = (KIND == GEMM_POLY) ? cb * ev[k] + cc * v[k] : ca * ev[k] + v[k];
        }
        *(LDS_AS u32x2*)(E + r * ROWB + ech(r, c >> 3) * 16 + (c & 7) * 2) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
  if constexpr (KIND == GEMM_UPDATE) {
    // Each wave copies out the sub-tile it staged itself (its own LDS
    // writes, complete once its LDS counter is zero), so no block barrier
    // sits between staging and copy-out: WTN/8 16-byte pieces per row, a
    // whole 128-byte line.  The next tile touches the staged region only
    // after its first step's barrier.
    if constexpr (PF) wait_vm_lgkm0<63>(); else wait_vm_lgkm0<0>();  // LDS only: the prefetch stays in flight
    asm volatile("" ::: "memory");
    constexpr int WCH = WTN / 8;  // 16-byte pieces per row of a wave's sub-tile
    static_assert((WTM * WCH) % 64 == 0 && (WTM * WCH) / 64 == NSTORE, "per-wave copy-out split");
#pragma unroll
    for (int s = 0; s < WTM * WCH / 64; ++s) {
      const int k = lane + 64 * s;
      const int r = wi * WTM + k / WCH, c = wj * WCH + k % WCH;
      const u32x4 val = *(const LDS_AS u32x4*)(E + r * ROWB + ech(r, c) * 16);
      if (row0 + r < row_lim)
        *reinterpret_cast<MUON_GLOBAL u32x4*>(C + (int64_t)(row0 + r) * ldc + col0 + c * 8) = val;
    }
    if constexpr (PF) {
      carry.pre = has_next;
      carry.prev_full = row0 + BM <= row_lim;
    }
    return;
  }
  // Symmetric kinds: the block copies out whole staged rows and writes the
  // mirror, both reading other waves' staged values, so a barrier first.
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  constexpr int CHUNKS = BM * RCH;
  static_assert(CHUNKS % NT == 0, "copy-out split");
  if (!diag) {
#pragma unroll
    for (int s = 0; s < CHUNKS / NT; ++s) {
      const int q = tid + s * NT;
      const int r = q / RCH, c = q % RCH;
      const u32x4 val = *(const LDS_AS u32x4*)(E + r * ROWB + ech(r, c) * 16);
      if (row0 + r < row_lim)
        *reinterpret_cast<MUON_GLOBAL u32x4*>(C + (int64_t)(row0 + r) * ldc + col0 + c * 8) = val;
    }
  }
  {
    // Mirror (and the diagonal tile's lower triangle) from transposing reads
    // of the staged tile: in each 16-lane group, lane L reads row k0 + L/4,
    // columns j0 + 4 (L % 4) .. +3, and lane i receives column j0 + i, rows
    // k0 .. k0+3; two reads give 8 rows, one 16-byte piece of a mirrored
    // row.  Group task g covers columns j0 = 16 (g % (BN/16)), rows
    // k0 = 8 (g / (BN/16)); the two groups of a 32-lane half share k0.
    constexpr int NGT = (BN / 16) * (BM / 8);
    static_assert(NGT % (NT / 16) == 0, "mirror split");
    const int i16 = tid & 15;
#pragma unroll
    for (int it = 0; it < NGT / (NT / 16); ++it) {
      const int g = it * (NT / 16) + (tid >> 4);
      const int j0 = 16 * (g % (BN / 16)), k0 = 8 * (g / (BN / 16));
      const int kr = k0 + (i16 >> 2), jc = j0 + 4 * (i16 & 3);
      const LDS_AS char* p0 = E + kr * ROWB + ech(kr, jc >> 3) * 16 + (jc & 7) * 2;
      const LDS_AS char* p1 = E + (kr + 4) * ROWB + ech(kr + 4, jc >> 3) * 16 + (jc & 7) * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p1);
      u32x4 val = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      const int j = j0 + i16;  // mirrored row = staged column
      if (diag) {
        // row j of the diagonal tile: staged row j where it lies on or above
        // the diagonal (column >= j), its mirror below
        const u32x4 rm = *(const LDS_AS u32x4*)(E + j * ROWB + ech(j, k0 >> 3) * 16);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo16 = (j <= k0 + 2 * e) ? (rm[e] & 0xffffu) : (val[e] & 0xffffu);
          const uint32_t hi16 = (j <= k0 + 2 * e + 1) ? (rm[e] >> 16) : (val[e] >> 16);
          w[e] = lo16 | (hi16 << 16);
        }
        val = u32x4{w[0], w[1], w[2], w[3]};
      }
      *reinterpret_cast<MUON_GLOBAL u32x4*>(C + (int64_t)(col0 + j) * ldc + row0 + k0) = val;
    }
  }
}

template <int KIND, int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int ROWU, int BK, bool PERSIST>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void ns_gemm_kernel(const MatDesc* __restrict__ descs,
                                                                        const GemmItem* __restrict__ items,
                                                                        int src, float ca, float cb, float cc, int n_items,
                                                                        float* __restrict__ part) {
  TileCarry carry{false, false};
  if constexpr (PERSIST) {
    // UPD_BLOCKS persistent blocks: block b takes items b, b + gridDim.x, ...,
    // all planned for XCD b % 8 (gridDim.x is a multiple of 8 or n_items)
    for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
      if (items[idx].mat < 0) continue;  // padding item of a shorter per-XCD run
      ns_gemm_tile<KIND, BM, BN, WAVES_M, WAVES_N, NSTAGE, ROWU, BK, PERSIST>(descs, items, n_items, idx, src, ca, cb,
                                                                              cc, part, carry);
    }
  } else {
    if (items[blockIdx.x].mat < 0) return;  // padding item of a shorter per-XCD run
    ns_gemm_tile<KIND, BM, BN, WAVES_M, WAVES_N, NSTAGE, ROWU, BK, PERSIST>(descs, items, n_items, blockIdx.x, src, ca,
                                                                            cb, cc, part, carry);
  }
}

}  // namespace muon
