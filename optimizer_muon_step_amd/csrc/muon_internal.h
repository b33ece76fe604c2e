// Internal declarations shared by the host plan code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Tile geometry of the Newton-Schulz GEMMs.  Inside the workspace the
// canonical m is padded to NS_PAD_M and n to NS_PAD_N, with the padding held
// at exact zero, so the GEMM kernels never bounds-check.
constexpr int GRAM_BM = 256;               // GRAM output tile (square), 8 waves
constexpr int SYM_BM = 128, SYM_BN = 128;  // POLY output tile
constexpr int SYM_BK = 64, SYM_NSTAGE = 2;  // GRAM / POLY K slice and ring depth (measured best)
constexpr int UPD_BM = 192, UPD_BN = 256;  // UPDATE output tile (rows may overhang m_pad)
constexpr int UPD_ROWU = 64;               // UPDATE tile rows start at multiples of this
// Persistent UPDATE grid: one block per CU of the 256 (8 XCDs x 32); a
// multiple of 8 so that every tile a block takes was planned for its XCD.
constexpr int UPD_BLOCKS = 256;
constexpr int NS_PAD_M = 256;              // multiple of GRAM_BM and SYM_BM
constexpr int NS_PAD_N = 256;              // multiple of UPD_BN
constexpr int NS_THREADS = 256;
// Row strides of X (n_pad + NS_LD_PAD) and of A / B (m_pad + NS_LD_PAD), in
// elements: 128 bytes past a multiple of 512 bytes, so that the rows a tile
// touches spread over the L2 channels instead of repeating a few of them.
constexpr int NS_LD_PAD = 64;

// Elementwise kernels.
constexpr int EW_THREADS = 256;
constexpr int MOM_CHUNK = 16384;  // elements per momentum work item (16 float4 per thread and array)
constexpr int CAST_TILE = 64;     // square tile for the cast / apply kernels

// One matrix of a call, in device memory.
struct MatDesc {
  float* W;               // caller params (rows x cols) or null
  const float* G;         // caller gradient or null
  float* M;               // caller momentum buffer or null
  uint16_t* upd;          // optional bf16 update output (rows x cols) or null
  const uint16_t* xin;    // bf16 input of the NS-only entry (rows x cols) or null
  uint16_t* X[2];         // canonical padded iterate, ping-pong (m_pad x n_pad)
  uint16_t* A;            // X X^T, m_pad x m_pad
  uint16_t* B;            // b A + c A A, m_pad x m_pad
  double* part;           // norm partial sums of this matrix (part_cnt of them)
  float* scale;           // s = 1 / (||U||_F + eps), written by norm_finalize_kernel
  int32_t rows, cols;     // caller orientation
  int32_t m, n;           // canonical, m <= n
  int32_t m_pad, n_pad;   // multiples of NS_PAD_M / NS_PAD_N
  int32_t transposed;     // 1 when rows > cols
  int32_t part_cnt;
  int32_t vec4;           // 1 when every row start allows 4-element vector access
  int32_t ld_x;           // row stride of X[0], X[1] (elements)
  int32_t ld_a;           // row stride of A and B (elements)
  int32_t pad_;
};

// GEMM work item: one output tile of one matrix, or (GRAM only) one K chunk
// of a tile whose chunks are summed by the reduce pass.
struct GemmItem {
  int32_t mat;
  int16_t ti, tj;  // tile row / column in units of the launch's tile shape
  int32_t k0;      // first K slice (units of 64)
  int32_t kn;      // K slices walked: to the true n (GRAM) or m (POLY, UPDATE; even for UPDATE), or a chunk's
  int32_t slot;    // fp32 partial tile this chunk writes, -1 = none
};

// Long-K Gram tiles.  When a tile's K is more than twice the per-CU share of
// a Gram launch (so a few tiles would keep most CUs idle), tiles longer than
// the share are cut into K chunks of about that share, at least
// GRAM_SPLIT_MIN slices; each chunk writes an fp32 partial tile and the
// reduce pass sums a tile's chunks in K order, rounds once to bf16 and
// mirrors.
constexpr int GRAM_SPLIT_MIN = 16;  // slices of 64
constexpr int NS_CUS = 256;         // CUs of the device the split is sized for
constexpr int RED_TILE = 64;        // reduce pass: 64x64 sub-tile per block

// Reduce work item: one 64x64 sub-tile of a split Gram tile.
struct RedItem {
  int32_t mat;
  int16_t ti, tj;    // Gram tile (units of GRAM_BM)
  int32_t slot0;     // first partial tile of its chunks
  int16_t nchunk;    // chunks, summed in order
  int8_t bi, bj;     // sub-tile within the Gram tile (units of RED_TILE)
};

// Elementwise work item: chunk (momentum) or tile (cast / apply) of a matrix.
struct EwItem {
  int32_t mat;
  int32_t idx;
};

enum GemmKind { GEMM_GRAM = 0, GEMM_POLY = 1, GEMM_UPDATE = 2 };

// ---- multi-tensor AdamW ----
constexpr int ADAM_CHUNK = 4096;  // elements per work item (4 float4 per thread per array)

// One tensor of an AdamW call (flat, contiguous fp32).
struct AdamDesc {
  float* p;        // parameters, updated in place
  const float* g;  // gradient
  float* u;        // first moment (exp_avg), updated in place
  float* v;        // second moment (exp_avg_sq), updated in place
  int64_t numel;
  float wd;           // this tensor's weight decay lambda (when not shared)
  int32_t wd_shared;  // 1: the call's shared lambda (AdamConst::wd_shared) applies
  int32_t vec4;       // 1 when all four arrays are 16-byte aligned
  int32_t pad_;
};

// Per-call scalars: the fp32 arguments and the constants derived from them
// on the host (fp64, rounded once to fp32).
struct AdamConst {
  float lr, beta1, beta2, eps;
  float omb1, omb2;  // 1 - beta1, 1 - beta2
  float bc1, bc2;    // 1 - beta1^t, 1 - beta2^t
  float wd_shared;   // the lambda of every tensor flagged wd_shared
};

// ---- host launchers (kernels_*.hip) ----
hipError_t launch_momentum(const MatDesc* d, const EwItem* items, int n_items, int n_mats, float beta,
                           hipStream_t s);
hipError_t launch_cast(const MatDesc* d, const EwItem* items, int n_items, float beta, int from_bf16,
                       hipStream_t s);
hipError_t launch_apply(const MatDesc* d, const EwItem* items, int n_items, float lr, int src,
                        int write_w, hipStream_t s);
hipError_t launch_gemm(int kind, const MatDesc* d, const GemmItem* items, int n_items, int src,
                       float ca, float cb, float cc, float* part, hipStream_t s);
hipError_t launch_gemm_gram(const MatDesc* d, const GemmItem* items, int n_items, int src, float* part,
                            hipStream_t s);
hipError_t launch_gram_reduce(const MatDesc* d, const RedItem* items, int n_items, const float* part,
                              hipStream_t s);
hipError_t launch_adamw(const AdamDesc* d, const EwItem* items, int n_items, const AdamConst& c, hipStream_t s);

// Source and destination of the three arrays (param, exp_avg, exp_avg_sq)
// of a delayed-untying copy.
struct UntieArgs {
  const float* src[3];
  float* dst[3];
};
hipError_t launch_untie_transpose(const UntieArgs& a, int64_t rows, int64_t cols, hipStream_t s);

}  // namespace muon
