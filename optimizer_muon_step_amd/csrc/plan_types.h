// Plain types and constants shared by the host plan code (plain C++, no HIP
// headers: it is also built with the host compiler alone) and the gfx950
// kernels.
#pragma once

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
// Calls of at most SMALL_MAX_UPD_TILES update tiles (above) use small tiles
// with deep rings instead: 64 x 64 Gram and poly tiles and 64 x 128 update
// tiles, four waves each, K slices of 64, most of a tile's slices in flight
// at once (SMALL_*_NSTAGE stages: 128 KB and 144 KB of LDS), one tile per
// block, and no Gram K cut, so a call with a Gram K of more than
// SMALL_MAX_GRAM_SLICES slices of 64 (n > 2048) is not small: the medium
// tiles below cut that K.  Measured per step: small tiles better than medium
// ones on calls of up to 36 update tiles with n <= 1536, worse from n = 2048
// on (256 x 4096 by 20 %) and on every call from 48 update tiles.
constexpr int SMALL_MAX_UPD_TILES = 40;
constexpr int SMALL_MAX_GRAM_SLICES = 32;
constexpr int SMALL_SYM = 64;
constexpr int SMALL_UPD_BM = 64, SMALL_UPD_BN = 128;
constexpr int SMALL_SYM_NSTAGE = 8, SMALL_UPD_NSTAGE = 6;
// Tiles of a call that is not small, chosen per kernel kind from its tile
// counts ("medium" tiles where the large ones would leave CUs idle):
//   Gram    MED_GRAM_BM x MED_GRAM_BM (two blocks per CU) when the call has
//           fewer Gram tiles of GRAM_BM than NS_CUS;
//   poly    MED_POLY_BM x MED_POLY_BM with a MED_POLY_NSTAGE ring (two blocks
//           per CU) when it has at most MED_POLY_MAX_TILES tiles of SYM_BM;
//   update  MED_UPD_BM x MED_UPD_BN (one block per CU, not persistent) when
//           3 x their rounds over NS_CUS CUs is below 4 x the rounds of the
//           UPD_BM x UPD_BN tiles over NS_CUS persistent blocks (a medium
//           tile takes about three quarters of a large one's time).
// Each output element accumulates its K in the same MFMA order whatever the
// tile, so the choices change no bit, except where a Gram tile is cut.
// A call whose medium update would have at most MED_UPD_MIN_TILES - 1 tiles
// (leaving half the CUs or more idle) runs the update on the small tiles
// instead, with a SHALLOW_UPD_NSTAGE ring (48 KB of LDS, several blocks per
// CU): TILE_SHALLOW.
enum TileKind { TILE_LARGE = 0, TILE_SMALL = 1, TILE_MEDIUM = 2, TILE_SHALLOW = 3 };
constexpr int MED_GRAM_BM = 128;
constexpr int MED_POLY_BM = 64, MED_POLY_NSTAGE = 4, MED_POLY_MAX_TILES = 128;
constexpr int MED_UPD_BM = 128, MED_UPD_BN = 256;
constexpr int MED_UPD_MIN_TILES = 129, SHALLOW_UPD_NSTAGE = 2;

// A small call whose matrices all have m_pad = FUSED_M_PAD (m <= 256) runs
// poly and update as one launch per iteration (kernels_ns_fused.hip) over
// the small update tiles.
constexpr int FUSED_M_PAD = 256;
// Row strides of X (n_pad + NS_LD_PAD) and of A / B (m_pad + NS_LD_PAD), in
// elements: 128 bytes past a multiple of 512 bytes, so that the rows a tile
// touches spread over the L2 channels instead of repeating a few of them.
constexpr int NS_LD_PAD = 64;

// Elementwise kernels.
constexpr int EW_THREADS = 256;
constexpr int MOM_CHUNK = 16384;  // elements per momentum work item (16 float4 per thread and array)
// A matrix with at most NORM_FOLD_MAX norm partials has its scale summed by
// every cast block itself, in the same fixed order as the finalisation
// kernel (so to the same bits); only larger matrices take that launch.
constexpr int NORM_FOLD_MAX = 256;
constexpr int CAST_TILE = 64;     // square tile for the cast / apply kernels
// The cast and apply passes cut an untransposed matrix into CAST_WIDE_ROWS x
// CAST_WIDE_COLS tiles instead (1 KB row pieces of the fp32 arrays).  The
// cast's item count is the same for both shapes (m_pad and n_pad are
// multiples of both edges); the apply's follows the caller's rows and cols.
constexpr int CAST_WIDE_ROWS = 16, CAST_WIDE_COLS = 256;
static_assert(CAST_WIDE_ROWS * CAST_WIDE_COLS == CAST_TILE * CAST_TILE, "cast tiles of equal size");
static_assert(NS_PAD_N % CAST_WIDE_COLS == 0 && NS_PAD_M % CAST_WIDE_ROWS == 0, "wide cast tiles cover the padding");
// Workgroups of a launch go to the 8 XCDs round-robin (workgroup b to XCD
// b % 8).  The elementwise passes give each XCD runs of consecutive work
// items in turn instead of every 8th item: XCD x takes items
// 8Rg + xR .. 8Rg + xR + R - 1 of group g (a last, shorter group is split
// into 8 near-equal runs), so fewer XCDs touch each page of the streamed
// arrays while all of them stay inside one compact window of the list.
// Measured per step (MI355X): c3 elementwise 440 -> 434 us, 192 GPT-2-XL
// matrices 8.99 -> 8.46 ms; results do not depend on the map (every norm
// partial is stored at its item's slot).
constexpr int EW_MOM_RUN = 4;    // momentum items (MOM_CHUNK elements each)
constexpr int EW_TILE_RUN = 16;  // cast / apply tiles
constexpr int ew_item_of_block(int b, int nb, int run) {
  const int group = 8 * run;
  const int base = (b / group) * group;
  const int t = (nb - base < group) ? nb - base : group;  // items of this group
  const int w = b - base, x = w & 7, q = w >> 3;
  const int full = t >> 3, rem = t & 7;
  return base + x * full + (x < rem ? x : rem) + q;
}

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
constexpr int GRAM_SPLIT_MIN = 8;  // slices of 64
constexpr int NS_CUS = 256;         // CUs of the device the split is sized for
constexpr int RED_TILE = 64;        // reduce pass: 64x64 sub-tile per block

// Reduce work item: one 64x64 sub-tile of a split Gram tile.
struct RedItem {
  int32_t mat;
  int16_t ti, tj;    // Gram tile (units of the call's Gram tile edge)
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

// Caller pointers of one matrix for one call: written into its descriptor
// (MatDesc W, G, M, upd, xin, vec4) in stream order by the patch kernel, so
// that a plan built for a set of shapes serves any set of pointers.
struct PtrRecord {
  float* W;
  const float* G;
  float* M;
  uint16_t* upd;
  const uint16_t* xin;
  int32_t vec4;
  int32_t mat;  // descriptor index
};

// Kernel-argument payloads (passed by value, so a captured graph holds its
// own copy): up to PATCH_MAX pointer records, or BLOB_WORDS words of a table
// image.  Both stay below 2 KB of kernel arguments.
constexpr int PATCH_MAX = 40;
struct PtrPatch {
  int32_t count;
  int32_t pad_;
  PtrRecord rec[PATCH_MAX];
};
constexpr int BLOB_WORDS = 480;
struct BlobChunk {
  int32_t words;
  int32_t pad_;
  uint32_t w[BLOB_WORDS];
};

}  // namespace muon
