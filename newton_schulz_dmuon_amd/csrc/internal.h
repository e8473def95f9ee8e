// Internal declarations shared by the host planner (host_api.cpp) and the
// gfx950 kernels (elementwise.hip, gemm.hip).  Not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace dmuon {

// Newton-Schulz operands live in the workspace padded to multiples of this
// many rows and columns, zero in the padding.  The padding stays zero through
// every stage (X X^T, b A + c A A and a X + B X all map zero rows/columns to
// zero), so the GEMM kernels never mask.
constexpr int64_t kPad = 256;
// Elements per work-group of the flat elementwise kernels.
constexpr int64_t kEwChunk = 8192;
// Side of the square tiles of the normalise/transpose kernel.
constexpr int64_t kTrTile = 64;
// Square output tile of the Newton-Schulz GEMM kernels.
constexpr int64_t kGemmTile = 256;
// In a bf16 step, matrices with min(rows, cols) below this run their
// Newton-Schulz chain in fp32 (see build_plan).
constexpr int64_t kFp32BelowM = 128;

enum Dtype : int32_t { kBF16 = 0, kF32 = 1 };

// Per-matrix descriptor, uploaded to the workspace on every step call.
struct MatDev {
  // caller memory
  void *param;
  const void *grad;
  float *mom;
  void *orth;
  void *packed;     // nullable: this matrix's slot of the packed param buffer
  // workspace memory (element type bf16, or fp32 in the fp32 mode)
  void *xt[2];      // X^T, n_p x m_p, row-major: the iterate, ping-pong; in
                    // a GEMM launch's table xt[0] is the iterate read and
                    // xt[1] the one Apply writes
  void *a;          // m_p x m_p: A = X X^T (Gram output, Square's L operand)
  void *b;          // m_p x m_p: B = b A + c A A (Square output, Apply's L operand)
  const void *sq_r; // Square's R operand; nullptr: R = a (the product A A)
  // Low halves of bf16 hi + lo pairs (nullable; bf16 chain only).  A pair
  // holds v as hi = RNE(v) and lo = RNE(v - hi), about 16 significant bits.
  // An operand with a low half adds a pass over it to the K loop:
  // L R^T = L R^T + L R_lo^T + L_lo R^T (the lo x lo term is below fp32
  // accumulation noise).  When sq_r is nullptr, R = L and R's low half is
  // l_lo.
  const void *l_lo;  // low half of Square's L (a) or Apply's L (b)
  const void *r_lo;  // low half of Square's sq_r
  void *out_lo;      // Square: also store the low half of the output here
  double *partials; // sum of U^2 per flat chunk (ns_steps = 0) or per
                    // 8192-element momentum-pass group (ns_steps >= 1)
  float *inv_norm;  // one float: 1 / (||U||_F + eps)
  int32_t *nonfinite; // nullable: set to 1 when U holds a NaN or an Inf, else 0
  int64_t rows, cols;   // caller shape r x c
  int64_t m, n;         // wide orientation m = min(r, c), n = max(r, c)
  int64_t mp, np;       // m, n rounded up to kPad
  int64_t ew_first;     // first flat chunk index of this matrix
  int64_t tr_first;     // first normalise-tile index of this matrix
  int32_t ew_count;     // number of flat chunks
  int32_t part_count;   // number of partial sums of U^2
  int32_t param_dt, grad_dt;
  int32_t transposed;   // rows > cols
  float scale;
  int32_t tm, tn;       // mp / kGemmTile, np / kGemmTile
  // Per-launch values of the GEMM stages, set in each launch's table (the
  // parts of one grouped launch may come from different chains):
  float ca;             // Apply / Final: weight of the a X term
  float cb, cc;         // Square: C = cb A + cc L R^T
  float cdiag;          // Square: added on the diagonal (rows < m)
  int32_t first_it;     // X holds U unnormalised: Gram scales by inv_norm^2,
                        // Apply / Final by inv_norm
  int32_t ws_f32;       // X^T, A, B of this matrix are fp32 (the fp32 mode, or
                        // a matrix with min(r, c) < kFp32BelowM in a bf16
                        // step), else bf16
  int32_t gemm_kind;    // in a launch of Gram and Square tiles
                        // (kModeGramSquare): kModeGram or kModeSquare for
                        // this matrix; unused otherwise
};

// One 256 x 256 output tile of a grouped GEMM stage, or a piece of one
// (split K).  In a launch of whole tiles only mat, ti, tj count.  In a
// launch of pieces: steps [k0, k1) of the tile's K loop (counted over all
// of its passes), whose fp32 accumulators go to partial slot `slot`.  In a
// reduce launch (after the pieces' launch): the sum of partial slots
// slot .. slot + k0 - 1, in that order, then the tile's epilogue.
struct TileEntry {
  int32_t mat;
  uint16_t ti, tj;
  int32_t k0, k1;
  int32_t slot;
  int32_t reserved_;
};
// fp32 accumulators of one 256 x 256 tile in a partial slot: 32 fragments
// of 16 x 16 per wave, four floats per lane, laid out [fragment][thread]
// so that every fragment's store is one contiguous 8 KB run.
constexpr int64_t kPartialSlotFloats = int64_t(256) * 256;

// Work-groups are handed to the 8 XCDs (each with its own L2) in turn: group
// w runs on XCD w % 8.  A stage therefore keeps one tile list per XCD, and
// group w computes entry first[w % 8] + w / 8 if w / 8 < count[w % 8].
constexpr int kXcds = 8;
struct StageXcd {
  int32_t first[kXcds];
  int32_t count[kXcds];
};

struct StepScalars {
  float a, b, c;
  float lr, mu, eps;
  int32_t nesterov;
  int32_t pad_;
};

enum GemmMode : int32_t {
  kModeGram = 0,    // C = X X^T (upper tiles, mirrored)        -> A
  kModeSquare = 1,  // C = cb A + cc A R^T + cdiag I (upper tiles, mirrored)
                    // -> B; R = A unless sq_r is set (then cb = 0: a product
                    // of two commuting symmetric matrices, itself symmetric)
  kModeApply = 2,   // C = a X + B X                             -> X', X'^T
  kModeFinal = 3,   // last apply: P -= lr*scale*C, orth <- C
  kModeGramSquare = 4  // Gram or Square tiles of different matrices in one
                       // launch, per MatDev::gemm_kind
};

// ---- launchers (elementwise.hip) ----
hipError_t launch_momentum_sumsq(const MatDev *mats, int32_t nmat,
                                 int64_t total_chunks, StepScalars s,
                                 hipStream_t st);
hipError_t launch_finalize_norm(const MatDev *mats, int32_t nmat, float eps,
                                hipStream_t st);
hipError_t launch_momentum_orient(const MatDev *mats, int32_t nmat,
                                  int64_t total_tiles, StepScalars s,
                                  hipStream_t st);
hipError_t launch_update_direct(const MatDev *mats, int32_t nmat,
                                int64_t total_chunks, StepScalars s,
                                hipStream_t st);

// Pack / unpack: batches of up to kPackBatch byte-copies per launch, passed
// by value in the kernel arguments.
constexpr int kPackBatch = 48;
struct PackBatch {
  int32_t n;
  int32_t pad_;
  int64_t first_block[kPackBatch + 1];  // prefix sum of blocks per copy
  const void *src[kPackBatch];
  void *dst[kPackBatch];
  int64_t bytes[kPackBatch];
};
constexpr int64_t kPackBlockBytes = 4 * 1024;  // one 16-byte vector per thread
hipError_t launch_pack_batch(const PackBatch &b, hipStream_t st);

// AdamW: batches of up to kAdamBatch tensors per launch, by value.
constexpr int kAdamBatch = 32;
constexpr int64_t kAdamChunk = 1024;  // elements per work-group: four per thread
struct AdamBatch {
  int32_t n;
  int32_t pad_;
  int64_t first_block[kAdamBatch + 1];  // prefix sum of kAdamChunk blocks
  void *param[kAdamBatch];
  const void *grad[kAdamBatch];
  float *m[kAdamBatch];
  float *v[kAdamBatch];
  int64_t numel[kAdamBatch];
  int32_t param_dt[kAdamBatch];
  int32_t grad_dt[kAdamBatch];
};
struct AdamScalars {
  float decay;          // 1 - lr * wd
  float beta1, beta2;
  float step_size;      // lr / (1 - beta1^t)
  float inv_sqrt_bc2;   // 1 / sqrt(1 - beta2^t)
  float eps;
};
hipError_t launch_adamw_batch(const AdamBatch &b, AdamScalars s, hipStream_t st);

// ---- static scratch (scratch.hip) ----
// Size of the file-scope device array that dmuon_muon_step_noalloc uses as
// its workspace (DMUON_NOALLOC_SCRATCH_BYTES of the C ABI).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// This device's address of that array (looked up once per device, with the
// device current, then kept).
hipError_t noalloc_scratch(void **ptr);

// ---- launchers (gemm.hip) ----
// mats: the launch's table (per-matrix operands and coefficients).
// role: 0 whole tiles, 1 pieces of split tiles, 2 their reduce entries
// (TileEntry); splitk: the partial slots (nullptr when the launch has none).
hipError_t launch_ns_stage(GemmMode mode, bool fp32, int role, const MatDev *mats,
                           const TileEntry *tiles, const StageXcd &xcd,
                           StepScalars s, float *splitk, hipStream_t st);
// A bf16 Square launch of 128 x 128 tiles (TileEntry ti, tj in 128-tile
// units; whole tiles only).
// The chained mode's one launch of every bf16 stage (gemm.hip): sync holds
// kXcds tickets, a timeout word and the stage counters from kChainCounters,
// all zero at the start (launch_zero_i32).
constexpr int32_t kChainCounters = 16;
hipError_t launch_ns_chain(const MatDev *mats, const TileEntry *tiles, const StageXcd &xcd, StepScalars s,
                           int32_t *sync, hipStream_t st);
hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t st);
hipError_t launch_ns_small_square(const MatDev *mats, const TileEntry *tiles, const StageXcd &xcd,
                                  StepScalars s, hipStream_t st);

}  // namespace dmuon
