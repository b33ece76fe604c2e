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
// Pipeline: 256 threads = 4 waves in a 2x2 grid over a BM x BN output tile.
// K advances in slices of 32 through a ring of NSTAGE LDS buffers filled by
// global_load_lds_dwordx4 (global memory straight into LDS, no registers), so
// NSTAGE-1 slices are in flight while one is multiplied.  Each lane's 16-byte
// DMA slot is fixed by its lane id; the XOR swizzle of a tile is therefore
// applied on the global side (each lane fetches the chunk that belongs in its
// slot).  k-contiguous tiles (X for GRAM, A for POLY, B for UPDATE) feed MFMA
// fragments with ds_read_b128; the k-major X tile of UPDATE is read with
// ds_read_b64_tr_b16 (see read_tr_frags), which transposes 16-bit elements across each group of
// 16 lanes: with lane L of a group addressing row k0 + L/4, columns
// j0 + 4(L%4) .. +3, lane i of the group receives column j0 + i, rows
// k0 .. k0+3.
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

constexpr int BK = 32;  // K per pipeline stage: 4 chunks of 16 B per k-contiguous row

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt_hi[15:14],
// expcnt[6:4], lgkmcnt[11:8]): wait until at most n vector-memory operations
// are outstanding and every LDS operation has completed.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8); }

// Swizzled 16-byte chunk of a k-contiguous row (4 chunks per row): rows r and
// r+1 share a 128-byte bank line, so XOR by (r/2)%4 gives eight consecutive
// rows eight distinct bank groups.
__device__ __forceinline__ int swz_k(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }
// Swizzled chunk of a k-major row (BN/8 chunks per row): the transposing
// read touches 4 consecutive rows at the same columns; XOR by 2(r%4) puts
// them in four different 32-byte bank groups.
__device__ __forceinline__ int swz_n(int row, int chunk) { return chunk ^ (2 * (row & 3)); }

template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(n));
}

// B fragments of one k-step from a k-major LDS tile: 2 x TN transposing
// reads.  They are issued from inline assembly because the compiler would
// otherwise wait for every in-flight global->LDS transfer (including later
// pipeline stages) before each such read.  The block ends with its own wait,
// so every output is complete when the block retires; outputs are
// early-clobber so no output register aliases an address input.
template <int TN>
__device__ __forceinline__ void read_tr_frags(bf16x8* bfr, const LDS_AS char* st, const int (*b_rd)[2][2],
                                              int kk) {
  static_assert(TN == 4, "read_tr_frags is written for four 32-column fragments");
  uint64_t r[8];
  const uint32_t base = (uint32_t)(uintptr_t)st;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(base + b_rd[0][kk][0]), "v"(base + b_rd[0][kk][1]), "v"(base + b_rd[1][kk][0]),
        "v"(base + b_rd[1][kk][1]), "v"(base + b_rd[2][kk][0]), "v"(base + b_rd[2][kk][1]),
        "v"(base + b_rd[3][kk][0]), "v"(base + b_rd[3][kk][1])
      : "memory");
#pragma unroll
  for (int nj = 0; nj < 4; ++nj)
    bfr[nj] = __builtin_bit_cast(bf16x8, u32x4{(uint32_t)r[2 * nj], (uint32_t)(r[2 * nj] >> 32),
                                               (uint32_t)r[2 * nj + 1], (uint32_t)(r[2 * nj + 1] >> 32)});
}

}  // namespace

template <int KIND, int BM, int BN, int NSTAGE>
__global__ __launch_bounds__(NS_THREADS, 2) void ns_gemm_kernel(const MatDesc* __restrict__ descs,
                                                               const GemmItem* __restrict__ items,
                                                               int src, float ca, float cb, float cc) {
  constexpr bool NN = (KIND == GEMM_UPDATE);  // B operand stored k-major
  constexpr int TM = BM / 64, TN = BN / 64;   // 32x32 MFMA tiles per wave (2x2 waves)
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / (16 * NS_THREADS);  // DMA instructions per wave per stage
  constexpr int B_INSTR = B_BYTES / (16 * NS_THREADS);
  constexpr int LPW = A_INSTR + B_INSTR;
  constexpr int NCHUNK_N = BN / 8;  // chunks per k-major row
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && NSTAGE >= 2 && NSTAGE <= 4, "unsupported tile");
  static_assert(NS_THREADS == 256, "2x2 waves");
  __shared__ __attribute__((aligned(16))) char lds[NSTAGE * STAGE_BYTES];

  const GemmItem it = items[blockIdx.x];
  if (it.mat < 0) return;  // padding item of a shorter per-XCD run
  const MatDesc& d = descs[it.mat];
  const uint16_t* Aop;
  const uint16_t* Bop;
  MUON_GLOBAL uint16_t* C;
  int lda, ldb, ldc, K;
  if (KIND == GEMM_GRAM) {
    Aop = d.X[src]; Bop = Aop; lda = ldb = d.n_pad; K = d.n_pad; C = gptr(d.A); ldc = d.m_pad;
  } else if (KIND == GEMM_POLY) {
    Aop = d.A; Bop = Aop; lda = ldb = d.m_pad; K = d.m_pad; C = gptr(d.B); ldc = d.m_pad;
  } else {
    Aop = d.B; lda = d.m_pad; Bop = d.X[src]; ldb = d.n_pad; K = d.m_pad; C = gptr(d.X[src ^ 1]);
    ldc = d.n_pad;
  }
  const int row0 = it.ti * BM;  // output rows    (rows of Aop)
  const int col0 = it.tj * BN;  // output columns (rows of Bop for GRAM/POLY, columns of X for UPDATE)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  // Per-lane global source of each DMA instruction at k = 0 (element offsets).
  int64_t a_off[A_INSTR], b_off[B_INSTR];
#pragma unroll
  for (int q = 0; q < A_INSTR; ++q) {
    const int s = (wave * A_INSTR + q) * 64 + lane;
    const int row = s >> 2;
    a_off[q] = (int64_t)(row0 + row) * lda + swz_k(row, s & 3) * 8;
  }
#pragma unroll
  for (int q = 0; q < B_INSTR; ++q) {
    const int s = (wave * B_INSTR + q) * 64 + lane;
    if (!NN) {
      const int row = s >> 2;
      b_off[q] = (int64_t)(col0 + row) * ldb + swz_k(row, s & 3) * 8;
    } else {
      const int row = s / NCHUNK_N;
      b_off[q] = (int64_t)row * ldb + col0 + swz_n(row, s % NCHUNK_N) * 8;
    }
  }
  auto issue = [&](int kt) {
    LDS_AS char* st = (LDS_AS char*)lds + (kt % NSTAGE) * STAGE_BYTES;
    const int64_t ka = (int64_t)kt * BK;
    const int64_t kb = NN ? (int64_t)kt * BK * ldb : (int64_t)kt * BK;
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(Aop + a_off[q] + ka),
                                       (LDS_AS void*)(st + (wave * A_INSTR + q) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < B_INSTR; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(Bop + b_off[q] + kb),
                                       (LDS_AS void*)(st + A_BYTES + (wave * B_INSTR + q) * 1024), 16, 0, 0);
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int nj = 0; nj < TN; ++nj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][nj][e] = 0.0f;

  // LDS byte offsets (within a stage) of this lane's fragment reads.
  int a_rd[TM][2], b_rd[TN][2][2];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r = wi * (BM / 2) + mi * 32 + (lane & 31);
      a_rd[mi][kk] = r * 64 + swz_k(r, 2 * kk + (lane >> 5)) * 16;
    }
#pragma unroll
  for (int nj = 0; nj < TN; ++nj)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (!NN) {
        const int r = wj * (BN / 2) + nj * 32 + (lane & 31);
        b_rd[nj][kk][0] = A_BYTES + r * 64 + swz_k(r, 2 * kk + (lane >> 5)) * 16;
        b_rd[nj][kk][1] = 0;
      } else {
        const int g = (lane >> 4) & 3, l16 = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = 16 * kk + 8 * (g >> 1) + 4 * h + (l16 >> 2);
          const int j = wj * (BN / 2) + nj * 32 + 16 * (g & 1) + 4 * (l16 & 3);
          b_rd[nj][kk][h] = A_BYTES + k * (BN * 2) + swz_n(k, j >> 3) * 16 + (j & 7) * 2;
        }
      }
    }

  auto compute = [&](int kt) {
    const LDS_AS char* st = (const LDS_AS char*)lds + (kt % NSTAGE) * STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
        af[mi] = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4*)(st + a_rd[mi][kk]));
      if constexpr (!NN) {
#pragma unroll
        for (int nj = 0; nj < TN; ++nj)
          bfr[nj] = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4*)(st + b_rd[nj][kk][0]));
      } else {
        read_tr_frags<TN>(bfr, st, b_rd, kk);
      }
      // operands swapped so each lane ends up with 4 consecutive output columns
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int nj = 0; nj < TN; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nj], af[mi], acc[mi][nj], 0, 0, 0);
    }
  };

  // Epilogue inputs (A for POLY, X for UPDATE) at the positions this lane
  // owns; fetched during the last K step so their latency is hidden.
  u32x2 ein[TM][TN][4];
  auto eload = [&]() {
    if (KIND == GEMM_GRAM) return;
    const MUON_GLOBAL uint16_t* E = (KIND == GEMM_POLY) ? gptr(d.A) : gptr(d.X[src]);
    const int lde = (KIND == GEMM_POLY) ? d.m_pad : d.n_pad;
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
      for (int nj = 0; nj < TN; ++nj)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int i = row0 + wi * (BM / 2) + mi * 32 + (lane & 31);
          const int j = col0 + wj * (BN / 2) + nj * 32 + 8 * e4 + 4 * (lane >> 5);
          ein[mi][nj][e4] = *reinterpret_cast<const MUON_GLOBAL u32x2*>(E + (int64_t)i * lde + j);
        }
  };

  // Main loop.  Stage kt is complete once this wave has at most
  // (stages issued after kt) x LPW DMA operations outstanding and every wave
  // has passed the barrier; the buffer refilled next was last read in kt-1,
  // which every wave finished (its LDS reads included) before the barrier.
  const int KT = K / BK;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KT) issue(s);
  for (int kt = 0; kt < KT; ++kt) {
    const int ahead = min(NSTAGE - 2, KT - 1 - kt);
    if (NSTAGE >= 4 && ahead >= 2)
      wait_vm_lgkm0<2 * LPW>();
    else if (ahead >= 1)
      wait_vm_lgkm0<LPW>();
    else
      wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + NSTAGE - 1 < KT)
      issue(kt + NSTAGE - 1);
    else if (kt == KT - 1)
      eload();
    compute(kt);
  }

  // Epilogue.  Lane holds, for MFMA tile (mi, nj) and quad e4, output row
  // i = .. + lane%32 and columns j .. j+3 with j = .. + 8*e4 + 4*(lane/32).
  // A symmetric tile that reaches below the diagonal stores only i <= j and
  // mirrors i < j; other symmetric tiles store both triangles' copies.
  const bool masked = (KIND != GEMM_UPDATE) && (row0 + BM - 1 > col0);
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int i = row0 + wi * (BM / 2) + mi * 32 + (lane & 31);
        const int j = col0 + wj * (BN / 2) + nj * 32 + 8 * e4 + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = acc[mi][nj][4 * e4 + k];
        if (KIND != GEMM_GRAM) {
          const u32x2 e2 = ein[mi][nj][e4];
          const float ev[4] = {bf16_lo(e2.x), bf16_hi(e2.x), bf16_lo(e2.y), bf16_hi(e2.y)};
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = (KIND == GEMM_POLY) ? cb * ev[k] + cc * v[k] : ca * ev[k] + v[k];
        }
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) h[k] = f32_to_bf16_bits(v[k]);
        if (!masked) {
          u32x2 o;
          o.x = h[0] | (h[1] << 16);
          o.y = h[2] | (h[3] << 16);
          *reinterpret_cast<MUON_GLOBAL u32x2*>(C + (int64_t)i * ldc + j) = o;
          if (KIND != GEMM_UPDATE) {
#pragma unroll
            for (int k = 0; k < 4; ++k) C[(int64_t)(j + k) * ldc + i] = (uint16_t)h[k];
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int jj = j + k;
            if (i <= jj) C[(int64_t)i * ldc + jj] = (uint16_t)h[k];
            if (i < jj) C[(int64_t)jj * ldc + i] = (uint16_t)h[k];
          }
        }
      }
    }
  }
}

hipError_t launch_gemm(int kind, const MatDesc* d, const GemmItem* items, int n_items, int src,
                       float ca, float cb, float cc, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  switch (kind) {
    case GEMM_GRAM:
      ns_gemm_kernel<GEMM_GRAM, SYM_BM, SYM_BN, 4><<<n_items, NS_THREADS, 0, s>>>(d, items, src, ca, cb, cc);
      break;
    case GEMM_POLY:
      ns_gemm_kernel<GEMM_POLY, SYM_BM, SYM_BN, 4><<<n_items, NS_THREADS, 0, s>>>(d, items, src, ca, cb, cc);
      break;
    default:
      ns_gemm_kernel<GEMM_UPDATE, UPD_BM, UPD_BN, 3><<<n_items, NS_THREADS, 0, s>>>(d, items, src, ca, cb, cc);
      break;
  }
  return hipGetLastError();
}

}  // namespace muon
