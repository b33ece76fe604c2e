// POLY and UPDATE of one Newton-Schulz iteration in a single launch, for
// small calls whose matrices all have m_pad = 256 (m <= 256; see
// ns_gemm_tile.h for the iteration).  Such calls are bound by the chain of
// dependent launches, not by arithmetic, so each block recomputes the rows
// of B = b A + c A A that its update tile needs instead of waiting for a
// poly launch:
//   phase 1  B[rows, 0:256] for the tile's 64 rows, K = 256, A streamed in
//            K slices of 64 (all 256 rows of A per slice: the tile's own
//            rows are among them), kept in LDS as the update's A operand;
//   phase 2  X' = a X + B X for the tile's 64 x 128 outputs, the X slices
//            fetched during phase 1.
// Every output element of B takes the same MFMA sequence (same operand
// fragments, same K order) as in the 64 x 64 poly tiles, and A is exactly
// symmetric, so an element below the diagonal, which the poly launch mirrors
// from above it, is the same sum of the same products: B, hence X', has the
// same bits as with the two launches.  Walking K to 256 past the true m adds
// only zero products to accumulators that start at +0, which changes no bit.
#include "ns_gemm_tile.h"

namespace muon {

namespace {

constexpr int PU_BM = 64;    // update tile rows
constexpr int PU_BN = 128;   // update tile columns
constexpr int PU_M = 256;    // m_pad of every matrix of the launch
constexpr int PU_BK = 64;    // K slice
constexpr int PU_KT = PU_M / PU_BK;                 // K slices of either phase
constexpr int PU_NT = 256;                          // 4 waves
constexpr int PANEL_BYTES = PU_M * PU_BK * 2;       // one K slice of A: 256 rows x 128 bytes
constexpr int XS_BYTES = PU_BK * PU_BN * 2;         // one K slice of X: 64 rows x 256 bytes
constexpr int NSTAGE = 3;                           // phase-1 ring
constexpr int BP_OFF = NSTAGE * PANEL_BYTES;        // B rows, 4 slices of 64 x 64
constexpr int BP_SLICE = PU_BM * PU_BK * 2;
constexpr int PU_LDS = BP_OFF + PU_KT * BP_SLICE;   // 128 KB
constexpr int P_INSTR = PANEL_BYTES / (16 * PU_NT);  // DMA instructions per wave per A slice (8)
constexpr int X_INSTR = XS_BYTES / (16 * PU_NT);     // per X slice (4)
static_assert(P_INSTR == 8 && X_INSTR == 4, "DMA split");
static_assert(2 * XS_BYTES <= PANEL_BYTES, "two X slices fill a freed ring stage");
static_assert(PU_LDS <= 160 * 1024, "LDS");

}  // namespace

__global__ __launch_bounds__(PU_NT) void poly_update_kernel(const MatDesc* __restrict__ descs,
                                                            const GemmItem* __restrict__ items, int src, float ca,
                                                            float cb, float cc) {
  __shared__ __attribute__((aligned(16))) char lds[PU_LDS];
  const GemmItem it = items[blockIdx.x];
  if (it.mat < 0) return;  // padding item of a shorter per-XCD run
  const MatDesc& d = descs[it.mat];
  const uint16_t* A = d.A;
  const uint16_t* X = d.X[src];
  MUON_GLOBAL uint16_t* Xo = gptr(d.X[src ^ 1]);
  const int lda = d.ld_a, ldx = d.ld_x;
  const int row0 = it.ti * UPD_ROWU;  // tile rows row0 .. row0+63 (of A, B and X)
  const int col0 = it.tj * PU_BN;     // tile columns of X
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: a scalar register

  // ---- DMA ----
  // A slice kt: 256 rows of 128 bytes; instruction g fills rows 8g .. 8g+7,
  // lane l slot (row 8g + l/8, chunk l%8) with global chunk swz_k(row, l%8).
  auto issue_panel = [&](int kt, int stage) {
    LDS_AS char* st = (LDS_AS char*)lds + stage * PANEL_BYTES;
#pragma unroll
    for (int q = 0; q < P_INSTR; ++q) {
      const int g = wave * P_INSTR + q;
      const int row = 8 * g + (lane >> 3);
      const uint16_t* p = A + (int64_t)row * lda + kt * PU_BK + swz_k<PU_BK>(row, lane & 7) * 8;
      __builtin_amdgcn_global_load_lds((const void*)p, (LDS_AS void*)(st + g * 1024), 16, 0, 0);
    }
  };
  // X slice kt (rows k = 64 kt ..), the tile's 128 columns: rows of 256
  // bytes, 4 rows per instruction, lane l slot (row, l%16) with global chunk
  // swz_n(row, l%16).
  auto issue_x = [&](int kt, int byte_off) {
    LDS_AS char* st = (LDS_AS char*)lds + byte_off;
#pragma unroll
    for (int q = 0; q < X_INSTR; ++q) {
      const int g = wave * X_INSTR + q;
      const int row = 4 * g + (lane >> 4);
      const uint16_t* p = X + (int64_t)(kt * PU_BK + row) * ldx + col0 + swz_n(row, lane & 15) * 8;
      __builtin_amdgcn_global_load_lds((const void*)p, (LDS_AS void*)(st + g * 1024), 16, 0, 0);
    }
  };
  // where X slice x lands: two in ring stage 1 (free once A slice 1 is
  // consumed), two in stage 2 (free once A slice 2 is)
  auto x_off = [](int x) { return (1 + x / 2) * PANEL_BYTES + (x & 1) * XS_BYTES; };

  // ---- phase 1: B[row0 .. row0+63, 0 .. 255] ----
  // 2 x 2 waves of 32 rows x 128 columns (4 MFMA tiles each).
  const int wi = wave >> 1, wj = wave & 1;
  floatx16 acc[4];
#pragma unroll
  for (int nj = 0; nj < 4; ++nj)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[nj][e] = 0.0f;
  const int ar = row0 + wi * 32 + (lane & 31);  // panel row of this lane's A fragment
  const int a_rd = ar * 128 + swz_k<PU_BK>(ar, lane >> 5) * 16;
  int b_rd[4];
#pragma unroll
  for (int nj = 0; nj < 4; ++nj) {
    const int r = wj * 128 + nj * 32 + (lane & 31);
    b_rd[nj] = r * 128 + swz_k<PU_BK>(r, lane >> 5) * 16;
  }
  u32x2 ein[4][4];  // A[i][j .. j+3] for the epilogue
#pragma unroll
  for (int nj = 0; nj < 4; ++nj)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) ein[nj][e4] = u32x2{0u, 0u};

  issue_panel(0, 0);
  issue_panel(1, 1);
#pragma unroll
  for (int s = 0; s < PU_KT; ++s) {
    // In flight after A slice s, per wave: slice s+1 (8 transfers) while
    // s < 3; at s = 3 the X slices 0 and 1 (8).
    wait_vm_lgkm0<8>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + 2 < PU_KT) issue_panel(s + 2, (s + 2) % NSTAGE);
    if (s == 2) { issue_x(0, x_off(0)); issue_x(1, x_off(1)); }  // stage 1: A slice 1 consumed
    if (s == 3) { issue_x(2, x_off(2)); issue_x(3, x_off(3)); }  // stage 2: A slice 2 consumed
    const LDS_AS char* st = (const LDS_AS char*)lds + (s % NSTAGE) * PANEL_BYTES;
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
      const int cbase = wj * 128 + nj * 32;  // 32 columns inside one K slice
      if (cbase / PU_BK != s) continue;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int kl = cbase % PU_BK + 8 * e4 + 4 * (lane >> 5);
        ein[nj][e4] = *(const LDS_AS u32x2*)(st + ar * 128 + swz_k<PU_BK>(ar, kl >> 3) * 16 + (kl & 7) * 2);
      }
    }
#pragma unroll
    for (int kk = 0; kk < PU_BK / 16; ++kk) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4*)(st + (a_rd ^ (32 * kk))));
      bf16x8 bfr[4];
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) bfr[nj] = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4*)(st + (b_rd[nj] ^ (32 * kk))));
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) acc[nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nj], af, acc[nj], 0, 0, 0);
    }
  }
  // B = bf16(b A + c A A) into the B panel, laid out as the update's
  // k-contiguous A operand: slice j/64, row i, swizzled chunk.
  {
    LDS_AS char* bp = (LDS_AS char*)lds + BP_OFF;
    const int i = wi * 32 + (lane & 31);
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int j = wj * 128 + nj * 32 + 8 * e4 + 4 * (lane >> 5);
        const u32x2 e2 = ein[nj][e4];
        const float ev[4] = {bf16_lo(e2.x), bf16_hi(e2.x), bf16_lo(e2.y), bf16_hi(e2.y)};
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = cb * ev[k] + cc * acc[nj][4 * e4 + k];
        const int kl = j % PU_BK;
        *(LDS_AS u32x2*)(bp + (j / PU_BK) * BP_SLICE + i * 128 + swz_k<PU_BK>(i, kl >> 3) * 16 + (kl & 7) * 2) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
  wait_vm_lgkm0<0>();  // every X slice has landed, the B panel is written
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // ---- phase 2: X'[row0 .., col0 ..] = a X + B X ----
  // 2 x 2 waves of 32 rows x 64 columns (2 MFMA tiles each).
  floatx16 acc2[2];
#pragma unroll
  for (int nj = 0; nj < 2; ++nj)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc2[nj][e] = 0.0f;
  const int i2 = wi * 32 + (lane & 31);
  const int a2_rd = i2 * 128 + swz_k<PU_BK>(i2, lane >> 5) * 16;
  int x_rd[2][2];
  {
    const int g = (lane >> 4) & 3, l16 = lane & 15;
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 8 * (g >> 1) + 4 * h + (l16 >> 2);
        const int j = wj * 64 + nj * 32 + 16 * (g & 1) + 4 * (l16 & 3);
        x_rd[nj][h] = k * (PU_BN * 2) + swz_n(k, j >> 3) * 16 + (j & 7) * 2;
      }
  }
  u32x2 xin[2][4];  // X[i][j .. j+3] for the epilogue
  const int grow = row0 + wi * 32;  // first output row of this wave: row k = grow of X
#pragma unroll
  for (int s = 0; s < PU_KT; ++s) {
    const LDS_AS char* bs = (const LDS_AS char*)lds + BP_OFF + s * BP_SLICE;
    const LDS_AS char* xs = (const LDS_AS char*)lds + x_off(s);
    if (grow / PU_BK == s) {
      const int lr = grow % PU_BK + (lane & 31);
#pragma unroll
      for (int nj = 0; nj < 2; ++nj)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int cl = wj * 64 + nj * 32 + 8 * e4 + 4 * (lane >> 5);
          xin[nj][e4] = *(const LDS_AS u32x2*)(xs + lr * (PU_BN * 2) + swz_n(lr, cl >> 3) * 16 + (cl & 7) * 2);
        }
    }
    const uint32_t xa = (uint32_t)(uintptr_t)xs;
#pragma unroll
    for (int kk = 0; kk < PU_BK / 16; ++kk) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4*)(bs + (a2_rd ^ (32 * kk))));
      const uint32_t dk = xa + kk * 16 * (PU_BN * 2);
      bf16x8 bfr[2];
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) bfr[nj] = read_tr_frag(dk + x_rd[nj][0], dk + x_rd[nj][1]);
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) acc2[nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nj], af, acc2[nj], 0, 0, 0);
    }
  }
  // rows of the tile lie inside m_pad (m_pad = 256, tiles of 64 rows)
#pragma unroll
  for (int nj = 0; nj < 2; ++nj)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int j = wj * 64 + nj * 32 + 8 * e4 + 4 * (lane >> 5);
      const u32x2 e2 = xin[nj][e4];
      const float ev[4] = {bf16_lo(e2.x), bf16_hi(e2.x), bf16_lo(e2.y), bf16_hi(e2.y)};
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = ca * ev[k] + acc2[nj][4 * e4 + k];
      *reinterpret_cast<MUON_GLOBAL u32x2*>(Xo + (int64_t)(row0 + i2) * ldx + col0 + j) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
}

hipError_t launch_poly_update(const MatDesc* d, const GemmItem* items, int n_items, int src, float ca, float cb,
                              float cc, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  poly_update_kernel<<<n_items, PU_NT, 0, s>>>(d, items, src, ca, cb, cc);
  return hipGetLastError();
}

}  // namespace muon
