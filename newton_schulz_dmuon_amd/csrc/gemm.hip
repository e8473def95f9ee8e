// Newton-Schulz stages of the owner's Muon step on gfx950 matrix cores.
//
// One iteration X <- a X + (b A + c A^2) X, A = X X^T, is three products,
// each a grouped launch over every matrix of the step:
//
//   Gram    A = X X^T        upper-triangle 256x256 tiles only, each tile also
//                            written mirrored (A is symmetric)
//   Square  B = b A + c A A  A A = A A^T is again a Gram product of a
//                            symmetric matrix: upper tiles + mirror, with
//                            b A + c (.) applied in the epilogue
//   Apply   X' = a X + B X   full tiles; the a X term is added in the
//                            epilogue; X' is written twice, row-major and
//                            transposed, because the next Gram reads X' by
//                            rows and the next Apply reads it by columns
//   Final   the last Apply: P -= lr*scale*X' in the caller's orientation,
//           and X' to orth_out; no workspace write
//
// Every product is C[i][j] = sum_k L[i][k] R[j][k] with both operands stored
// k-contiguous (row-major L, row-major R), which is the operand layout the
// MFMA instructions read.  Operands are bf16 (v_mfma_f32_16x16x32_bf16) or
// fp32 in the checking mode (v_mfma_f32_16x16x4_f32); accumulation is fp32.
//
// Tiling: 256x256 output tile per work-group of 8 waves (2 x 4), each wave
// 128x64 = 8x4 MFMA 16x16 blocks.  K advances 128 bytes per step (64 bf16 or
// 32 fp32).  Operand tiles go straight from global memory into LDS with
// global_load_lds_dwordx4 (no register staging): each wave instruction fills
// one contiguous KB of LDS, and every lane picks the global 16-byte chunk that
// belongs at its LDS slot.  Two LDS stages (2 x 64 KB) form a ring: after the
// barrier that opens step k, the loads of step k+1 go into the stage step k-1
// used, and run while step k is on the matrix cores.
//
// LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with
// (row / 2) mod 8.  A fragment read of 16 consecutive rows then touches 16
// distinct 16-byte bank groups of the 256-byte LDS line (two rows per line),
// which the bank-conflict counter confirms at zero.
//
// Operands are zero-padded to multiples of 256 in the workspace, so no
// load or store is masked except the caller-visible writes of Final.

#include "device_common.h"

namespace dmuon {

namespace {

constexpr int kThreads = 512;
constexpr int kTile = static_cast<int>(kGemmTile);  // 256
constexpr int kRowBytes = 128;                      // K bytes per LDS row
constexpr int kOperandBytes = kTile * kRowBytes;    // 32 KB per operand tile
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kWaveM = kTile / kWavesM;             // 128
constexpr int kWaveN = kTile / kWavesN;             // 64
constexpr int kFragM = kWaveM / 16;                 // 8
constexpr int kFragN = kWaveN / 16;                 // 4
constexpr int kStageBytes = 2 * kOperandBytes;     // L and R tiles of one K step
constexpr int kDmaPerWave = kOperandBytes / 1024 / 8;  // 4 KB-sized DMA instructions

typedef __attribute__((address_space(3))) char lds_char;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ int swz(int chunk, int row) { return chunk ^ ((row >> 1) & 7); }

// Waits until this wave's LDS-bound global loads and LDS reads are complete,
// then synchronises the work-group.  The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Synchronises the work-group once this wave's LDS reads are complete (its
// global stores may still be in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename T> struct Mfma;
template <> struct Mfma<uint16_t> {
  // one 16-byte chunk per lane = 8 bf16 along k = one 16x16x32 MFMA
  static __device__ __forceinline__ void run(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // one 16-byte chunk per lane = 4 fp32 along k = four 16x16x4 MFMAs
  static __device__ __forceinline__ void run(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// Four consecutive workspace elements as one vector access (8 bytes for bf16,
// 16 for fp32); the address is a multiple of four elements.
// Accesses go through global (address space 1) pointers, so they count on
// vmcnt only and never wait on LDS traffic.  raw() / cvt() split a load so
// that a batch of loads can be issued before the first use.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x2 g_u32x2;
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
template <typename T> struct Vec4;
template <> struct Vec4<uint16_t> {
  typedef u32x2 Raw;
  static __device__ __forceinline__ Raw raw(const uint16_t *p) { return *(const g_u32x2 *)p; }
  static __device__ __forceinline__ f32x4 cvt(const Raw &v) {
    return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                 __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
  }
  static __device__ __forceinline__ f32x4 ld(const uint16_t *p) { return cvt(raw(p)); }
  static __device__ __forceinline__ void st(uint16_t *p, const f32x4 &v) {
    u32x2 u;
    u.x = static_cast<uint32_t>(f32_to_bf16_bits(v[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
    u.y = static_cast<uint32_t>(f32_to_bf16_bits(v[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
    *(g_u32x2 *)p = u;
  }
};
template <> struct Vec4<float> {
  typedef u32x4 Raw;
  static __device__ __forceinline__ Raw raw(const float *p) { return *(const g_u32x4 *)p; }
  static __device__ __forceinline__ f32x4 cvt(const Raw &v) {
    return f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
  }
  static __device__ __forceinline__ f32x4 ld(const float *p) { return cvt(raw(p)); }
  static __device__ __forceinline__ void st(float *p, const f32x4 &v) {
    *(g_u32x4 *)p = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                          __float_as_uint(v[3])};
  }
};

// Row-major 256 x 256 bf16 tile in LDS (512-byte rows, 32 chunks of 16 B),
// two chunk swizzles, one per way the tile is filled:
//  kSwzRows: stage_tile_put writes four rows of one column (2-byte stores);
//    the chunk is XORed with bits 2-3 of the row (moved to chunk bits 1-2),
//    so the 64 lanes of one put touch 4 rows x 2 chunks in distinct banks.
//  kSwzCols: stage_tile_put_t writes four consecutive elements of a row
//    (one 8-byte store); a put touches 16 consecutive rows x 32 bytes, and
//    the chunk is XORed with (row mod 8) * 2, which keeps the chunk pair of
//    a row together and spreads 8 rows over 256 bytes of banks.
// A flush reads whole rows, so either swizzle is a permutation within a row.
constexpr int kSwzRows = 0, kSwzCols = 1;
template <int SW>
__device__ __forceinline__ int tile_swz(int row, int chunk) {
  return SW == kSwzRows ? chunk ^ (((row >> 2) & 3) << 1) : chunk ^ ((row & 7) << 1);
}

// Puts rows r0 .. r0+3 of column c (one lane's four values) as bf16.
__device__ __forceinline__ void stage_tile_put(lds_char *lds, int r0, int c, const f32x4 &v) {
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = r0 + k;
    const int off = row * 512 + tile_swz<kSwzRows>(row, c >> 3) * 16 + (c & 7) * 2;
    *(lds_u16 *)(lds + off) = f32_to_bf16_bits(v[k]);
  }
}

// Puts elements c0 .. c0+3 of row r (c0 a multiple of four) as bf16: the
// transposed placement of a lane's four values.
__device__ __forceinline__ void stage_tile_put_t(lds_char *lds, int r, int c0, const f32x4 &v) {
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  u32x2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16_bits(v[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16_bits(v[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
  *(lds_u32x2 *)(lds + r * 512 + tile_swz<kSwzCols>(r, c0 >> 3) * 16 + (c0 & 7) * 2) = u;
}

// Writes the staged tile to dst (row-major, leading dimension ld elements)
// with 16-byte stores: thread t moves chunks t, t + 512, ... (row = f / 32).
// Starts with a barrier (the puts are visible); a later put into the same
// LDS needs stage_barrier() first.
template <int SW>
__device__ __forceinline__ void stage_tile_flush(lds_char *lds, uint16_t *dst, int64_t ld, int tid) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int f = q * 512 + tid;
    const int row = f >> 5, chunk = f & 31;
    const u32x4 v = *(const lds_u32x4 *)(lds + row * 512 + tile_swz<SW>(row, chunk) * 16);
    *reinterpret_cast<u32x4 *>(dst + row * ld + chunk * 8) = v;
  }
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(const MatDev *__restrict__ mats,
                                                           const TileEntry *__restrict__ tiles,
                                                           StageXcd xcd, int32_t cur,
                                                           int32_t first, StepScalars s) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kOperandBytes];  // 128 KB
  // C cast: generic -> LDS address space.  [2 stages][L, R][256 rows][128 B]
  lds_char *const lds = (lds_char *)smem;

  // this work-group's tile: entry w / 8 of XCD (w % 8)'s list
  const int32_t w = static_cast<int32_t>(blockIdx.x);
  const int32_t xi = w % kXcds, k = w / kXcds;
  if (k >= xcd.count[xi]) return;  // whole group leaves before any barrier
  const TileEntry e = tiles[xcd.first[xi] + k];
  const MatDev &d = mats[e.mat];
  const int32_t ti = e.ti, tj = e.tj;

  const T *L, *R;
  int64_t ld;  // elements; both operands have the same leading dimension
  if (MODE == kModeGram) {
    L = R = static_cast<const T *>(d.x[cur]);
    ld = d.np;
  } else if (MODE == kModeSquare) {
    L = R = static_cast<const T *>(d.a);
    ld = d.mp;
  } else {
    L = static_cast<const T *>(d.b);
    R = static_cast<const T *>(d.xt[cur]);
    ld = d.mp;
  }
  const int64_t ld_bytes = ld * static_cast<int64_t>(sizeof(T));
  const int nkt = static_cast<int>(ld_bytes / kRowBytes);
  // The last Apply of a wide matrix (P is m x n, not transposed) computes
  // the transposed tile, (B X)^T = X^T B: each lane's four consecutive
  // values then run along a row of P, so the update is a vector access.
  const bool swap = (MODE == kModeFinal) && !d.transposed;
  const char *gl = reinterpret_cast<const char *>(swap ? R : L) +
                   static_cast<int64_t>(swap ? tj : ti) * kTile * ld_bytes;
  const char *gr = reinterpret_cast<const char *>(swap ? L : R) +
                   static_cast<int64_t>(swap ? ti : tj) * kTile * ld_bytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // This wave's share of a stage: kDmaPerWave instructions per operand, each
  // filling LDS rows [8b, 8b + 8) of the operand tile, b = j*8 + wave.  Lane
  // l writes LDS byte 16*l of that KB: row 8b + l/8, physical chunk l%8,
  // which holds logical chunk swz(l%8, row) of the row.
  int64_t goff[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int row = (j * 8 + wave) * 8 + (lane >> 3);
    goff[j] = static_cast<int64_t>(row) * ld_bytes + swz(lane & 7, row) * 16;
  }
  auto issue = [&](int kt) {
    lds_char *st = lds + (kt & 1) * kStageBytes;
    const int64_t kofs = static_cast<int64_t>(kt) * kRowBytes;
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const int lofs = (j * 8 + wave) * 1024;
      __builtin_amdgcn_global_load_lds((const void *)(gl + goff[j] + kofs),
                                       (__attribute__((address_space(3))) void *)(st + lofs), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(gr + goff[j] + kofs),
                                       (__attribute__((address_space(3))) void *)(st + kOperandBytes + lofs),
                                       16, 0, 0);
    }
  };

  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int r16 = lane & 15, g4 = lane >> 4;

  f32x4 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments of one K step: sub-step 0 covers k chunks 0-3, sub-step 1
  // chunks 4-7 of the 128-byte rows.
  struct Frag {
    u32x4 l[kFragM], r[kFragN];
  };
  auto read_frag = [&](const lds_char *st, int sub, Frag &f) {
    const int chunk = sub * 4 + g4;
#pragma unroll
    for (int i = 0; i < kFragM; ++i) {
      const int row = wm * kWaveM + i * 16 + r16;
      f.l[i] = *(const lds_u32x4 *)(st + row * kRowBytes + swz(chunk, row) * 16);
    }
#pragma unroll
    for (int j = 0; j < kFragN; ++j) {
      const int row = wn * kWaveN + j * 16 + r16;
      f.r[j] = *(const lds_u32x4 *)(st + kOperandBytes + row * kRowBytes + swz(chunk, row) * 16);
    }
  };
  auto mfma_frag = [&](const Frag &f) {
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) Mfma<T>::run(acc[i][j], f.l[i], f.r[j]);
  };

  // Software pipeline across the barrier: the products of step k-1's
  // sub-step 1 (already in registers) run right after the barrier of step
  // k, while step k's sub-step 0 fragments come out of LDS.  The loads of
  // step k+1 are issued unconditionally (the last step re-loads its own K
  // range into the free stage), so each iteration is one basic block the
  // compiler can interleave.  nkt >= 4 because operands are padded to 256.
  // The aX term of Apply comes from the R operand, X^T: its rows are the tile's columns and its K range
  // [ti*256, ti*256 + 256) holds the tile's rows.  While the K steps of the
  // wave's 128 rows are in LDS, each lane reads its four values (four
  // consecutive k of one R row) and adds a*X to the accumulators.
  constexpr int kKStep = kRowBytes / static_cast<int>(sizeof(T));  // K elements per step
  constexpr int kCapSteps = kWaveM / kKStep;                         // steps holding the wave's rows
  constexpr int kCapFrags = kKStep / 16;                             // fragment rows per step
  constexpr bool cap_ax = MODE == kModeApply;
  const int cap_kt0 = ti * (kTile / kKStep) + wm * kCapSteps;
  // Step c of the wave's kCapSteps holds fragment rows [c*kCapFrags,
  // (c+1)*kCapFrags).  Every fragment row reads and adds at every capture
  // step, with weight a on its own step and 0 on the others (at an address
  // of the same step), so no accumulator is indexed by a run-time value.
  auto capture_ax = [&](const lds_char *st, int kt) {
    if constexpr (!cap_ax) return;
    const int c = kt - cap_kt0;  // uniform in the wave
    if (c < 0 || c >= kCapSteps) return;
#pragma unroll
    for (int i = 0; i < kFragM; ++i) {
      const float w = (i / kCapFrags == c) ? s.a : 0.f;
      const int kb = ((i % kCapFrags) * 16 + 4 * g4) * static_cast<int>(sizeof(T));  // byte offset in the R row
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int row = wn * kWaveN + j * 16 + r16;
        const lds_char *pr = st + kOperandBytes + row * kRowBytes + swz(kb >> 4, row) * 16 + (kb & 15);
        f32x4 xv;
        if constexpr (sizeof(T) == 2) {
          typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
          const u32x2 raw = *(const lds_u32x2 *)pr;
          xv = Vec4<uint16_t>::cvt(raw);
        } else {
          const u32x4 raw = *(const lds_u32x4 *)pr;
          xv = Vec4<float>::cvt(raw);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(w, xv[v], acc[i][j][v]);
      }
      // one fragment row per group: at most 8 VGPRs of reads in flight
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Frag fa, fb;
  issue(0);
  stage_barrier();
  issue(1);
  capture_ax(lds, 0);
  read_frag(lds, 0, fa);
  read_frag(lds, 1, fb);
  mfma_frag(fa);
  for (int kt = 1; kt < nkt; ++kt) {
    stage_barrier();  // step kt is in LDS; step kt-1's stage is free
    const lds_char *st = lds + (kt & 1) * kStageBytes;
    issue(min(kt + 1, nkt - 1));
    capture_ax(st, kt);
    read_frag(st, 0, fa);
    mfma_frag(fb);    // sub-step 1 of step kt-1
    read_frag(st, 1, fb);
    mfma_frag(fa);
  }
  mfma_frag(fb);
  // no LDS-bound load may still be in flight when the LDS is reused or the
  // work-group ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds C[row0 + 4*g4 + v][col0 + r16], v = 0..3 ----
  // The four values of a lane are four consecutive rows of one column, i.e.
  // four consecutive elements of a row of the transposed matrix: transposed
  // reads and writes move them as one 8-byte (bf16) or 16-byte (fp32) vector.
  // Row-major bf16 outputs are staged through LDS (the 128 KB of the two
  // stages hold one 256 x 256 bf16 tile) and leave as 16-byte row segments.
  // rows of the computed product come from the L panel, columns from R
  const int64_t row_base = static_cast<int64_t>(swap ? tj : ti) * kTile + wm * kWaveM + 4 * g4;
  const int64_t col_base = static_cast<int64_t>(swap ? ti : tj) * kTile + wn * kWaveN + r16;
  constexpr bool kStage = sizeof(T) == 2;
  // fragment rows whose epilogue inputs are read in one batch: all of them
  // for bf16 (2 VGPRs per vector), two at a time for fp32 (4 per vector)
  constexpr int kReadRows = sizeof(T) == 2 ? kFragM : 2;
  if (kStage && MODE != kModeFinal) stage_barrier();  // mainloop LDS reads done

  // The first iteration's X is U unnormalised (X0 = U * inv_norm): A0 picks
  // up inv_norm^2 and the first X' (or O) inv_norm.
  const float inv = first ? *d.inv_norm : 1.f;
  const float gram_scale = inv * inv;
  if (MODE == kModeGram || MODE == kModeSquare) {
    T *out = static_cast<T *>(MODE == kModeGram ? d.a : d.b);
    const T *prev = static_cast<const T *>(d.a);
    const int64_t mp = d.mp;
    // all of a lane's reads first: the compiler cannot prove that the
    // stores below miss them, so interleaving would serialise each one
#pragma unroll
    for (int i0 = 0; i0 < kFragM; i0 += kReadRows) {
    typename Vec4<T>::Raw araw[kReadRows][kFragN];
    if (MODE == kModeSquare)
#pragma unroll
      for (int ii = 0; ii < kReadRows; ++ii)
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
          // A[row + v][col] = A[col][row + v]: A is exactly symmetric
          araw[ii][j] = Vec4<T>::raw(prev + (col_base + j * 16) * mp + row_base + (i0 + ii) * 16);
#pragma unroll
    for (int ii = 0; ii < kReadRows; ++ii)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int i = i0 + ii;
        const int64_t col = col_base + j * 16, row = row_base + i * 16;
        f32x4 val = acc[i][j];
        if (MODE == kModeGram) val *= gram_scale;
        if (MODE == kModeSquare) {
          const f32x4 av = Vec4<T>::cvt(araw[ii][j]);
#pragma unroll
          for (int v = 0; v < 4; ++v) val[v] = fmaf(s.b, av[v], s.c * val[v]);
        }
        if constexpr (kStage) {
          stage_tile_put(lds, wm * kWaveM + i * 16 + 4 * g4, wn * kWaveN + j * 16 + r16, val);
          acc[i][j] = val;  // kept for the mirror tile
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) WsType<T>::st(out, (row + v) * mp + col, val[v]);
          if (ti != tj) Vec4<T>::st(out + col * mp + row, val);
        }
      }
    }
    if constexpr (kStage) {
      uint16_t *const o16 = reinterpret_cast<uint16_t *>(out);
      stage_tile_flush<kSwzRows>(lds, o16 + static_cast<int64_t>(ti) * kTile * mp + static_cast<int64_t>(tj) * kTile,
                                 mp, tid);
      if (ti != tj) {  // the mirror tile (tj, ti), staged the transposed way
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kFragM; ++i)
#pragma unroll
          for (int j = 0; j < kFragN; ++j)
            stage_tile_put_t(lds, wn * kWaveN + j * 16 + r16, wm * kWaveM + i * 16 + 4 * g4, acc[i][j]);
        stage_tile_flush<kSwzCols>(lds, o16 + static_cast<int64_t>(tj) * kTile * mp + static_cast<int64_t>(ti) * kTile,
                                   mp, tid);
      }
    }
  } else if (MODE == kModeApply) {
    T *Xn = static_cast<T *>(d.x[cur ^ 1]);
    T *XTn = static_cast<T *>(d.xt[cur ^ 1]);
    const int64_t np = d.np, mp = d.mp;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int64_t col = col_base + j * 16, row = row_base + i * 16;
        f32x4 val;  // a*X is already in the accumulator
#pragma unroll
        for (int v = 0; v < 4; ++v) val[v] = acc[i][j][v] * inv;
        if constexpr (kStage) {
          stage_tile_put(lds, wm * kWaveM + i * 16 + 4 * g4, wn * kWaveN + j * 16 + r16, val);
          acc[i][j] = val;  // kept for the X'^T tile
        } else {
          Vec4<T>::st(XTn + col * mp + row, val);
#pragma unroll
          for (int v = 0; v < 4; ++v) WsType<T>::st(Xn, (row + v) * np + col, val[v]);
        }
      }
    if constexpr (kStage) {
      // X' tile (ti, tj), then X'^T tile (tj, ti) through the same LDS
      stage_tile_flush<kSwzRows>(lds, reinterpret_cast<uint16_t *>(Xn) + static_cast<int64_t>(ti) * kTile * np +
                                          static_cast<int64_t>(tj) * kTile, np, tid);
      lds_barrier();
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
          stage_tile_put_t(lds, wn * kWaveN + j * 16 + r16, wm * kWaveM + i * 16 + 4 * g4, acc[i][j]);
      stage_tile_flush<kSwzCols>(lds, reinterpret_cast<uint16_t *>(XTn) + static_cast<int64_t>(tj) * kTile * mp +
                                          static_cast<int64_t>(ti) * kTile, mp, tid);
    }
  } else {  // kModeFinal
    const float step = s.lr * d.scale;
    // (p, q): lane's four values are C[p + v][q] of the computed product.
    // Not swapped: p over m, q over n, P index (q, p + v) of the r x c = n x m
    // matrix.  Swapped: the product is C^T, p over n, q over m, P index
    // (q, p + v) of the m x n matrix.  Either way P[q][p .. p+3].
    const int64_t p_lim = swap ? d.n : d.m, q_lim = swap ? d.m : d.n;
    const T *Xsrc = static_cast<const T *>(swap ? d.x[cur] : d.xt[cur]);
    const int64_t xld = swap ? d.np : d.mp;
    const bool vec_ok = (d.cols & 3) == 0;  // rows of P start 4-element aligned
    // PT: the parameter's storage type.  Reads of a batch go first (X, and P
    // on the vector path); four fragment rows per batch when both are bf16.
    auto update = [&](auto ptag) {
      using PT = decltype(ptag);
      constexpr int kRows = sizeof(T) == 2 ? (sizeof(PT) == 2 ? 4 : 2) : 1;
      PT *const P = static_cast<PT *>(d.param);
      PT *const Orth = static_cast<PT *>(d.orth);
#pragma unroll
      for (int i0 = 0; i0 < kFragM; i0 += kRows) {
        typename Vec4<T>::Raw xraw[kRows][kFragN];
        typename Vec4<PT>::Raw praw[kRows][kFragN];
#pragma unroll
        for (int ii = 0; ii < kRows; ++ii)
#pragma unroll
          for (int j = 0; j < kFragN; ++j) {
            const int64_t q = col_base + j * 16, p = row_base + (i0 + ii) * 16;
            xraw[ii][j] = Vec4<T>::raw(Xsrc + q * xld + p);  // in the padded buffer
            if (vec_ok && p + 4 <= p_lim && q < q_lim) praw[ii][j] = Vec4<PT>::raw(P + q * d.cols + p);
          }
#pragma unroll
        for (int ii = 0; ii < kRows; ++ii)
#pragma unroll
          for (int j = 0; j < kFragN; ++j) {
            const int i = i0 + ii;
            const int64_t q = col_base + j * 16, p = row_base + i * 16;
            if (p >= p_lim || q >= q_lim) continue;
            const f32x4 xv = Vec4<T>::cvt(xraw[ii][j]);
            f32x4 o;
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = fmaf(s.a, xv[v], acc[i][j][v]) * inv;
            const int64_t pidx = q * d.cols + p;
            if (vec_ok && p + 4 <= p_lim) {
              const f32x4 pv = Vec4<PT>::cvt(praw[ii][j]);
              f32x4 nv;
#pragma unroll
              for (int v = 0; v < 4; ++v) nv[v] = fmaf(-step, o[v], pv[v]);
              Vec4<PT>::st(P + pidx, nv);
              if (Orth) Vec4<PT>::st(Orth + pidx, o);
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                if (p + v >= p_lim) break;
                if (Orth) store_elem(d.orth, d.param_dt, pidx + v, o[v]);
                store_elem(d.param, d.param_dt, pidx + v,
                           fmaf(-step, o[v], load_elem(d.param, d.param_dt, pidx + v)));
              }
            }
          }
      }
    };
    if (d.param_dt == kBF16)
      update(uint16_t{});
    else
      update(float{});
  }
}

template <typename T>
hipError_t launch_t(GemmMode mode, const MatDev *mats, const TileEntry *tiles, const StageXcd &xcd,
                    int32_t cur, int32_t first, StepScalars s, hipStream_t st) {
  int32_t longest = 0;
  for (int x = 0; x < kXcds; ++x) longest = xcd.count[x] > longest ? xcd.count[x] : longest;
  if (longest == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(longest) * kXcds), block(kThreads);
  switch (mode) {
    case kModeGram:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeGram>), grid, block, 0, st, mats, tiles, xcd, cur, first, s);
      break;
    case kModeSquare:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeSquare>), grid, block, 0, st, mats, tiles, xcd, cur, first, s);
      break;
    case kModeApply:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeApply>), grid, block, 0, st, mats, tiles, xcd, cur, first, s);
      break;
    default:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeFinal>), grid, block, 0, st, mats, tiles, xcd, cur, first, s);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_stage(GemmMode mode, bool fp32, const MatDev *mats, const TileEntry *tiles,
                           const StageXcd &xcd, int32_t cur, bool first, StepScalars s,
                           hipStream_t st) {
  const int32_t f = first ? 1 : 0;
  return fp32 ? launch_t<float>(mode, mats, tiles, xcd, cur, f, s, st)
              : launch_t<uint16_t>(mode, mats, tiles, xcd, cur, f, s, st);
}

}  // namespace dmuon
