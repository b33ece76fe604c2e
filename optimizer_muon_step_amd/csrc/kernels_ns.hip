// Quintic Newton-Schulz core on gfx950 bf16 matrix cores.
//
// One iteration X <- a X + (b A + c A A) X with A = X X^T (the "new optimizer"
// thread, tweets 5/8 and 6/8: a quintic Newton-Schulz iteration in bfloat16)
// is three batched GEMM launches over every matrix of a call:
//   GRAM    A = bf16(X X^T)              K = n, symmetric: upper tiles only,
//                                        each also written mirrored
//   POLY    B = bf16(b A + c (A A^T))    K = m, symmetric (A is exactly
//                                        symmetric, so A A = A A^T)
//   UPDATE  X' = bf16(a X + B X)         K = m, X read k-major and transposed
//                                        in registers on its way to LDS
// Products accumulate in fp32 on v_mfma_f32_32x32x16_bf16; the epilogue
// combinations are plain fp32 products and sums (no fused multiply-add) and
// every stored value is rounded to bf16, nearest-even.
//
// Tiling: a 256-thread workgroup computes one 128x128 output tile; its four
// waves each own a 64x64 quadrant (2x2 MFMA tiles of 32x32).  K advances in
// slices of 64, double-buffered in LDS (2 x 32 KB).  LDS rows are 128 B with a
// 16-byte-chunk XOR swizzle (chunk ^ row%8 ^ (row/8)%8) so that both the
// MFMA fragment reads and the transposing stores spread over all banks.
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

constexpr int TILE = NS_TILE;                  // 128
constexpr int BK = NS_BK;                      // 64
constexpr int CHUNKS_PER_ROW = BK / 8;         // 8 chunks of 16 B
constexpr int STAGE_CHUNKS = TILE * CHUNKS_PER_ROW;  // 1024 per operand

static_assert(TILE == 128 && BK == 64 && NS_THREADS == 256, "loader index math assumes these");

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * CHUNKS_PER_ROW + (chunk ^ (row & 7) ^ ((row >> 3) & 7));
}

// Interleave the 16-bit halves `h` (0 low, 1 high) of two dwords.
__device__ __forceinline__ uint32_t pick_half(uint32_t r0, uint32_t r1, int h) {
  return h ? ((r0 >> 16) | (r1 & 0xffff0000u)) : ((r0 & 0xffffu) | (r1 << 16));
}

}  // namespace

template <int KIND>
__global__ __launch_bounds__(NS_THREADS, 2) void ns_gemm_kernel(const MatDesc* __restrict__ descs,
                                                               const GemmItem* __restrict__ items,
                                                               int src, float ca, float cb, float cc) {
  __shared__ u32x4 lds[2][2][STAGE_CHUNKS];  // [stage][operand][chunk], 64 KB

  const GemmItem it = items[blockIdx.x];
  if (it.mat < 0) return;  // padding item of a shorter per-XCD run
  const MatDesc& d = descs[it.mat];
  const MUON_GLOBAL uint16_t* Aop;
  const MUON_GLOBAL uint16_t* Bop;
  MUON_GLOBAL uint16_t* C;
  int lda, ldb, ldc, K;
  if (KIND == GEMM_GRAM) {
    Aop = gptr(d.X[src]); Bop = Aop; lda = ldb = d.n_pad; K = d.n_pad; C = gptr(d.A); ldc = d.m_pad;
  } else if (KIND == GEMM_POLY) {
    Aop = gptr(d.A); Bop = Aop; lda = ldb = d.m_pad; K = d.m_pad; C = gptr(d.B); ldc = d.m_pad;
  } else {
    Aop = gptr(d.B); lda = d.m_pad; Bop = gptr(d.X[src]); ldb = d.n_pad; K = d.m_pad; C = gptr(d.X[src ^ 1]);
    ldc = d.n_pad;
  }
  const int row0 = it.ti * TILE;  // output rows   (rows of Aop)
  const int col0 = it.tj * TILE;  // output columns (rows of Bop for GRAM/POLY, columns of X for UPDATE)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + NS_THREADS * q;
      const int row = c >> 3, ch = c & 7;
      ra[q] = *reinterpret_cast<const MUON_GLOBAL u32x4*>(Aop + (int64_t)(row0 + row) * lda + k0 + ch * 8);
    }
    if (KIND != GEMM_UPDATE) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid + NS_THREADS * q;
        const int row = c >> 3, ch = c & 7;
        rb[q] = *reinterpret_cast<const MUON_GLOBAL u32x4*>(Bop + (int64_t)(col0 + row) * ldb + k0 + ch * 8);
      }
    } else {
      // X tile: k rows k0 + 4kq .. +3, columns col0 + 8jb .. +7
      const int jb = tid & 15, kq = tid >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rb[r] = *reinterpret_cast<const MUON_GLOBAL u32x4*>(Bop + (int64_t)(k0 + 4 * kq + r) * ldb + col0 + 8 * jb);
    }
  };
  auto sstore = [&](int stage) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + NS_THREADS * q;
      lds[stage][0][swz(c >> 3, c & 7)] = ra[q];
    }
    if (KIND != GEMM_UPDATE) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid + NS_THREADS * q;
        lds[stage][1][swz(c >> 3, c & 7)] = rb[q];
      }
    } else {
      // 4 k-rows x 8 columns -> 8 column-rows of 4 k each (8 bytes)
      const int jb = tid & 15, kq = tid >> 4;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 8 * jb + 2 * w + h;
          u32x2 v;
          v.x = pick_half(rb[0][w], rb[1][w], h);
          v.y = pick_half(rb[2][w], rb[3][w], h);
          u32x2* p = reinterpret_cast<u32x2*>(&lds[stage][1][swz(j, kq >> 1)]) + (kq & 1);
          *p = v;
        }
      }
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][nj][e] = 0.0f;

  // Fragments for k-step kk+1 are read from LDS while the MFMAs of k-step kk run.
  auto read_frags = [&](int stage, int kk, bf16x8* af, bf16x8* bfr) {
    const int ch = 2 * kk + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      af[mi] = __builtin_bit_cast(bf16x8, lds[stage][0][swz(wi * 64 + mi * 32 + (lane & 31), ch)]);
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
      bfr[nj] = __builtin_bit_cast(bf16x8, lds[stage][1][swz(wj * 64 + nj * 32 + (lane & 31), ch)]);
  };
  auto compute = [&](int stage) {
    bf16x8 af[2][2], bfr[2][2];
    read_frags(stage, 0, af[0], bfr[0]);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) read_frags(stage, kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
      // operands swapped so each lane ends up with 4 consecutive output columns
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][nj], af[kk & 1][mi], acc[mi][nj], 0, 0, 0);
    }
  };

  // Epilogue inputs (A for POLY, X for UPDATE) at the positions this lane
  // owns; fetched during the last K step so their latency is hidden.
  u32x2 ein[2][2][4];
  auto eload = [&]() {
    if (KIND == GEMM_GRAM) return;
    const MUON_GLOBAL uint16_t* E = (KIND == GEMM_POLY) ? gptr(d.A) : gptr(d.X[src]);
    const int lde = (KIND == GEMM_POLY) ? d.m_pad : d.n_pad;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nj = 0; nj < 2; ++nj)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int i = row0 + wi * 64 + mi * 32 + (lane & 31);
          const int j = col0 + wj * 64 + nj * 32 + 8 * e4 + 4 * (lane >> 5);
          ein[mi][nj][e4] = *reinterpret_cast<const MUON_GLOBAL u32x2*>(E + (int64_t)i * lde + j);
        }
  };

  const int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT)
      gload((kt + 1) * BK);
    else
      eload();
    compute(cur);
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Lane holds, for MFMA tile (mi, nj) and quad e4, output row
  // i = .. + lane%32 and columns j .. j+3 with j = .. + 8*e4 + 4*(lane/32).
  const bool diag = (KIND != GEMM_UPDATE) && (it.ti == it.tj);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int i = row0 + wi * 64 + mi * 32 + (lane & 31);
        const int j = col0 + wj * 64 + nj * 32 + 8 * e4 + 4 * (lane >> 5);
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
        if (!diag) {
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
      ns_gemm_kernel<GEMM_GRAM><<<n_items, NS_THREADS, 0, s>>>(d, items, src, ca, cb, cc);
      break;
    case GEMM_POLY:
      ns_gemm_kernel<GEMM_POLY><<<n_items, NS_THREADS, 0, s>>>(d, items, src, ca, cb, cc);
      break;
    default:
      ns_gemm_kernel<GEMM_UPDATE><<<n_items, NS_THREADS, 0, s>>>(d, items, src, ca, cb, cc);
      break;
  }
  return hipGetLastError();
}

}  // namespace muon
