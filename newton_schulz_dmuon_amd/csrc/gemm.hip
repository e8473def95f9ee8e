// Newton-Schulz stages of the owner's Muon step on gfx950 matrix cores.
//
// One iteration X <- a X + (b A + c A^2) X, A = X X^T, is three products,
// each a grouped launch over every matrix of the step.  The iterate is kept
// only as X^T (n_p x m_p, row-major):
//
//   Gram    A = X X^T        upper-triangle 256x256 tiles only, each tile also
//                            written mirrored (A is symmetric; a diagonal
//                            tile stores its upper triangle and the mirror
//                            of it, so the stored A is exactly symmetric,
//                            as is every Square output); both operands
//                            are column blocks of X^T (MN-major tiles)
//   Square  B = b A + c A A  A A = A A^T is again a Gram product of a
//                            symmetric matrix: upper tiles + mirror; the
//                            b A term is taken from the R tile in LDS (as
//                            (b/c) A, scaled by c in the epilogue).  The
//                            Gram-space chain also runs it with its own R
//                            (sq_r: A P^2, Q P, products of commuting
//                            symmetric matrices) and a diagonal term
//                            (P = a I + b A + c A A)
//   Apply   X' = a X + B X   full tiles, R operand = X^T (K-contiguous); the
//                            a X term is read from the R tile in LDS during the
//                            mainloop; X'^T is written
//   Final   the last Apply: P -= lr*scale*X' in the caller's orientation,
//           also stored to the packed slot when the step has one, and X'
//           to orth_out; no workspace write
//
// A launch can also hold Gram tiles of some matrices and Square tiles of
// others (the two chains of one step sharing a launch): its instance reads
// each tile's stage from the matrix's table row and runs that stage's tile
// function.  In a diagonal tile of Gram or Square, the waves whose quadrant
// lies below the diagonal skip their products.
//
// From six iterations on, B (and every P of the Gram-space chain) is kept
// as a bf16 hi + lo pair, hi = RNE(v), lo = RNE(v - hi): Square stores both
// halves, and a product that reads a pair runs its K loop over one more
// pass, (L, R) then (L, R_lo) and/or (L_lo, R), accumulating into the same
// tile.
//
// Every product is C[i][j] = sum_k L[i][k] R[j][k].  Square and Apply read
// both operands k-contiguous (row-major L and R), the layout the MFMA
// instructions take; Gram's operands have k down the rows and are turned
// into that layout by transposing LDS reads.  Operands are bf16 (v_mfma_f32_16x16x32_bf16) or
// fp32 in the checking mode (v_mfma_f32_16x16x4_f32); accumulation is fp32.
//
// Tiling: 256x256 output tile per work-group of 8 waves (2 x 4), each wave
// 128x64 = 8x4 MFMA 16x16 blocks.  K advances 128 bytes per step (64 bf16 or
// 32 fp32).  Operand tiles go straight from global memory into LDS with
// global_load_lds_dwordx4 (no register staging): each wave instruction fills
// one contiguous KB of LDS, and every lane picks the global 16-byte chunk that
// belongs at its LDS slot.  Two LDS stages (2 x 64 KB) form a ring, and the
// two halves of the work-group run the K loop in ping-pong: one half's waves
// read fragments (and issue the next stage's loads) while the other half's
// multiply, switching at every work-group barrier (the mainloop below).
//
// K-contiguous LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with
// (row / 2) mod 8.  A fragment read of 16 consecutive rows then touches 16
// distinct 16-byte bank groups of the 256-byte LDS line (two rows per line),
// which the bank-conflict counter confirms at zero.
//
// A bf16 Square launch with too few 256-tiles to fill the CUs runs 128x128
// tiles instead (ns_gemm_small_kernel): the same tile function with every
// extent halved, each wave 64x32 = 4x2 MFMA blocks, 2 x 32 KB of LDS, and
// two work-groups per CU, so four times the tiles share the CUs.
//
// Operands are zero-padded to multiples of 256 in the workspace, so no
// load or store is masked except the caller-visible writes of Final.

#include <type_traits>

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

typedef __attribute__((address_space(3))) char lds_char;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int chunk, int row) { return chunk ^ ((row >> 1) & 7); }

// Waits until this wave's LDS-bound global loads and LDS reads are complete,
// then synchronises the work-group.  The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// MN-major operand tiles (Gram reads X^T: K runs down the rows) are held as
// two 16 KB halves, columns 0-127 and 128-255 of the tile, so that each half
// of the work-group can load its own.  An LDS row of a half is one k: 128
// elements, 256 bytes (bf16) or 512 bytes (fp32); a stage holds kRowBytes /
// sizeof(T) rows.  The 16-byte chunk of a row is XORed with mn_swz(row),
// chosen so that the fragment reads below touch distinct banks: bf16 reads
// 16 rows x 32 bytes (bits 0-1 and 3 of the row pick one of 8 chunk pairs),
// fp32 reads 4 rows x 64 bytes (bits 2-3 pick the 64-byte group).
constexpr int kHalfBytes = kOperandBytes / 2;
template <typename T>
__device__ __forceinline__ int mn_swz(int row) {
  return sizeof(T) == 2 ? ((row & 3) | (((row >> 3) & 1) << 2)) << 1 : ((row >> 2) & 3) << 2;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4e+q gives the
// address of four consecutive elements Y[k0 + e][n0 + 4q .. n0 + 4q + 3] of
// a row-major Y; lane j of the group receives Y[k0 .. k0+3][n0 + j], i.e. four
// consecutive k of one column, the MFMA operand layout.  Issued as inline
// assembly: the compiler would otherwise wait for every LDS-bound global
// load before it (it cannot tell them apart), so the caller waits with
// wait_lds_tied() before using the result.
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t lds_addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}

// Synchronises the work-group once this wave's LDS reads are complete (its
// global stores may still be in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Synchronises the work-group once this wave's LDS-bound loads have landed.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// Eight consecutive elements of a caller's buffer: one 16-byte access for
// bf16, two for fp32; the address is 16-byte aligned.
template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  typedef u32x4 Raw;
  static __device__ __forceinline__ Raw raw(const uint16_t *p) { return *(const g_u32x4 *)p; }
  static __device__ __forceinline__ void cvt(const Raw &v, float (&o)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = __uint_as_float(v[k] << 16);
      o[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st(uint16_t *p, const float (&v)[8]) {
    u32x4 u;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      u[k] = static_cast<uint32_t>(f32_to_bf16_bits(v[2 * k])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * k + 1])) << 16);
    *(g_u32x4 *)p = u;
  }
};
template <> struct Vec8<float> {
  struct Raw {
    u32x4 a, b;
  };
  static __device__ __forceinline__ Raw raw(const float *p) {
    return Raw{*(const g_u32x4 *)p, *(const g_u32x4 *)(p + 4)};
  }
  static __device__ __forceinline__ void cvt(const Raw &v, float (&o)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[k] = __uint_as_float(v.a[k]);
      o[4 + k] = __uint_as_float(v.b[k]);
    }
  }
  static __device__ __forceinline__ void st(float *p, const float (&v)[8]) {
    *(g_u32x4 *)p = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    *(g_u32x4 *)(p + 4) =
        u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
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

// The low half of a bf16 hi + lo pair: v - RNE(v), exact in fp32 (it is
// rounded to bf16 when stored).
__device__ __forceinline__ f32x4 bf16_low_part(const f32x4 &v) {
  f32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = v[k] - bf16_bits_to_f32(f32_to_bf16_bits(v[k]));
  return r;
}

// The staged tile is TS x TS bf16 (TS = 256: 512-byte rows of 32 chunks;
// TS = 128: 256-byte rows of 16 chunks, the swizzles staying inside a row).
// Puts rows r0 .. r0+3 of column c (one lane's four values) as bf16.
template <int TS = 256>
__device__ __forceinline__ void stage_tile_put(lds_char *lds, int r0, int c, const f32x4 &v) {
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = r0 + k;
    const int off = row * (2 * TS) + tile_swz<kSwzRows>(row, c >> 3) * 16 + (c & 7) * 2;
    *(lds_u16 *)(lds + off) = f32_to_bf16_bits(v[k]);
  }
}

// Diagonal tiles of the symmetric outputs: the upper triangle (c >= row)
// of rows r0 .. r0+3 at column c, each value also at its mirror (c, row)
// when c > row.  Every element of the tile is written once, so the stored
// tile is exactly symmetric even when the product is only symmetric in
// exact arithmetic (A P^2 and Q P of the Gram-space chain).
template <int TS = 256>
__device__ __forceinline__ void stage_tile_put_sym(lds_char *lds, int r0, int c, const f32x4 &v) {
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  auto at = [](int row, int col) {
    return row * (2 * TS) + tile_swz<kSwzRows>(row, col >> 3) * 16 + (col & 7) * 2;
  };
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = r0 + k;
    const uint16_t bits = f32_to_bf16_bits(v[k]);
    if (c >= row) *(lds_u16 *)(lds + at(row, c)) = bits;
    if (c > row) *(lds_u16 *)(lds + at(c, row)) = bits;
  }
}

// Puts elements c0 .. c0+3 of row r (c0 a multiple of four) as bf16: the
// transposed placement of a lane's four values.
template <int TS = 256>
__device__ __forceinline__ void stage_tile_put_t(lds_char *lds, int r, int c0, const f32x4 &v) {
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  u32x2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16_bits(v[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16_bits(v[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
  *(lds_u32x2 *)(lds + r * (2 * TS) + tile_swz<kSwzCols>(r, c0 >> 3) * 16 + (c0 & 7) * 2) = u;
}

// Writes the staged tile to dst (row-major, leading dimension ld elements)
// with 16-byte stores: thread t moves chunks t, t + 512, ... (TS / 8 chunks
// per row).  All of a thread's LDS reads (16 for TS = 256, 4 for 128) are
// issued before its first store, so their latencies overlap instead of
// adding up.
// Starts with a barrier (the puts are visible); a later put into the same
// LDS needs lds_barrier() first (every wave's flush reads done).
template <int SW, int TS = 256>
__device__ __forceinline__ void stage_tile_flush(lds_char *lds, uint16_t *dst, int64_t ld, int tid) {
  constexpr int kChunksPerRow = TS / 8, kPerThread = TS * TS / 8 / 512;
  constexpr int kRowShift = TS == 256 ? 5 : 4;
  static_assert(kChunksPerRow == (1 << kRowShift), "chunks per row");
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // opaque: each flush rebuilds its addresses instead of keeping them live
  // across the epilogue's other flushes
  asm volatile("" : "+v"(tid));
  u32x4 v[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int f = q * 512 + tid;
    const int row = f >> kRowShift, chunk = f & (kChunksPerRow - 1);
    v[q] = *(const lds_u32x4 *)(lds + row * (2 * TS) + tile_swz<SW>(row, chunk) * 16);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int f = q * 512 + tid;
    const int row = f >> kRowShift, chunk = f & (kChunksPerRow - 1);
    *(g_u32x4 *)(dst + row * ld + chunk * 8) = v[q];
  }
}

// Role of a launch (a template argument, so that each kernel instance holds
// only its own code): whole tiles; pieces of split tiles (the mainloop over
// steps [k0, k1), fp32 accumulators to a partial slot); or the reduce
// entries of split tiles (the sum of their pieces' slots, then the tile's
// epilogue).
constexpr int kRoleWhole = 0, kRolePiece = 1, kRoleReduce = 2;

// One tile (or piece of a tile) of stage MODE: the work-group's whole work.
// lds: the work-group's 128 KB, [2 stages][L, R][256 rows][128 B].
// TS: the tile size, 256 (every stage) or 128 (Square, bf16 whole tiles,
// for launches with too few 256-tiles to fill the chip): the same 2 x 4
// waves, each computing (TS / 2) x (TS / 4), on a 64 KB operand ring.
template <typename T, int MODE, int ROLE, int TS = 256>
__device__ __forceinline__ void gemm_tile(lds_char *const lds, const MatDev &d, const TileEntry &e,
                                          const StepScalars &s, f32x4 *__restrict__ splitk) {
  static_assert(TS == 256 || (TS == 128 && MODE == kModeSquare && ROLE == kRoleWhole && sizeof(T) == 2),
                "128-tiles: bf16 Square, whole tiles");
  // the tile's geometry (shadowing the 256-tile constants)
  constexpr int kTile = TS;
  constexpr int kWaveM = kTile / kWavesM, kWaveN = kTile / kWavesN;
  constexpr int kFragM = kWaveM / 16, kFragN = kWaveN / 16;
  constexpr int kOperandBytes = kTile * kRowBytes, kHalfBytes = kOperandBytes / 2;
  constexpr int kStageBytes = 2 * kOperandBytes;
  const int32_t ti = e.ti, tj = e.tj;

  // Gram reads X^T (n_p x m_p): its operand tiles are MN-major, K = n runs
  // down the rows.  The other stages read K-contiguous rows.
  constexpr bool kMN = MODE == kModeGram;
  constexpr int kKStep = kRowBytes / static_cast<int>(sizeof(T));  // K elements per step
  const T *L, *R;
  const T *Llo = nullptr, *Rlo = nullptr;  // low halves of hi + lo operand pairs
  int64_t ld;  // elements; both operands have the same leading dimension
  if (MODE == kModeGram) {
    L = R = static_cast<const T *>(d.xt[0]);
    ld = d.mp;
  } else if (MODE == kModeSquare) {
    L = static_cast<const T *>(d.a);
    R = d.sq_r ? static_cast<const T *>(d.sq_r) : L;
    if constexpr (sizeof(T) == 2) {
      Llo = static_cast<const T *>(d.l_lo);
      Rlo = static_cast<const T *>(d.sq_r ? d.r_lo : d.l_lo);
    }
    ld = d.mp;
  } else {
    L = static_cast<const T *>(d.b);
    R = static_cast<const T *>(d.xt[0]);
    if constexpr (sizeof(T) == 2) Llo = static_cast<const T *>(d.l_lo);
    ld = d.mp;
  }
  const int64_t ld_bytes = ld * static_cast<int64_t>(sizeof(T));
  const int nkt = kMN ? static_cast<int>(d.np / kKStep) : static_cast<int>(ld_bytes / kRowBytes);
  // K-contiguous: the tile's 256 rows; MN-major: the tile's 256 columns
  const int64_t tile_stride = kMN ? kTile * static_cast<int64_t>(sizeof(T)) : kTile * ld_bytes;
  auto panel = [&](const T *base, int32_t t) {
    return reinterpret_cast<const char *>(base) + static_cast<int64_t>(t) * tile_stride;
  };
  // The K loop runs over one to three passes of the operand panels: (L, R),
  // then (L, R_lo) when R is a hi + lo pair, then (L_lo, R) when L is; all
  // accumulate into the same tile.  Pass s covers steps [s*nkt, (s+1)*nkt).
  const bool r_pair = Rlo != nullptr, l_pair = Llo != nullptr;
  const char *const gl = panel(L, ti), *const gr = panel(R, tj);
  const char *const gl_lo = l_pair ? panel(Llo, ti) : gl;
  const char *const gl1 = r_pair ? gl : gl_lo;
  const char *const gr1 = r_pair ? panel(Rlo, tj) : gr;
  // pass s reads L at gl + s1*dl1 + s2*dl2 (s1 = s >= 1, s2 = s >= 2), and
  // R likewise: byte distances, so that picking a pass is arithmetic
  const int64_t dl1 = gl1 - gl, dl2 = gl_lo - gl1, dr1 = gr1 - gr, dr2 = gr - gr1;
  const int ntot = (1 + r_pair + l_pair) * nkt;
  // split K: a piece runs steps [k0, k1) and leaves its accumulators in a
  // partial slot; a reduce entry runs no step and starts from the sum of
  // its pieces' slots
  constexpr bool kPiece = ROLE == kRolePiece, kReduce = ROLE == kRoleReduce;
  const int kbeg = kPiece ? e.k0 : 0, kend = kPiece ? e.k1 : ntot;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int wm = wave / kWavesN, wn = wave % kWavesN;

  // The four waves of half h (wm = h) load the rows of L that make the
  // tile's rows [128h, 128h + 128) (K-contiguous: L rows; MN-major: L's
  // column half h); waves 0-3 also load all of R.  Loader v = wn issues the
  // 1 KB instructions j*4 + v of each of its operand halves.
  // K-contiguous: KB b of the tile is LDS rows [8b, 8b + 8); lane l writes
  // LDS byte 16*l of it: row 8b + l/8, physical chunk l%8, which holds
  // logical chunk swz(l%8, row).  MN-major: KB b of a half is k rows
  // [4b, 4b + 4) (bf16, lane l: row 4b + l/16, physical chunk l%16) or
  // [2b, 2b + 2) (fp32: row 2b + l/32, chunk l%32), physical chunk c holding
  // logical chunk c ^ mn_swz(row).
  // Offsets within the operand's row block fit 32 bits: the step accepts
  // at most 2^22 elements per side, so 256 rows span < 2^32 bytes.
  constexpr int kRowsPerKB = kMN ? 1024 / (kHalfBytes / (kRowBytes / static_cast<int>(sizeof(T)))) : 8;
  constexpr int kChunksPerRow = 64 / kRowsPerKB;
  constexpr int kKBsPerHalf = kHalfBytes / 1024;  // 16
  constexpr int kPerLoader = kKBsPerHalf / 4;     // 4 instructions per half and loader
  // a row of a half: MN-major 128 elements of one k; K-contiguous a tile row
  const int lrow = wn * kRowsPerKB + lane / kChunksPerRow;
  const int lpc = lane % kChunksPerRow;
  const uint32_t goff0 = static_cast<uint32_t>(lrow) * static_cast<uint32_t>(ld_bytes);
  // rows between instruction j and j + 1 of a loader within one half
  const uint32_t goff_step = static_cast<uint32_t>(4 * kRowsPerKB) * static_cast<uint32_t>(ld_bytes);
  auto issue = [&](int slot, int kt) {
    lds_char *st = lds + slot * kStageBytes;
    const int s1 = kt >= nkt, s2 = kt >= 2 * nkt;  // pass of step kt (uniform)
    const int kk = kt - (s1 + s2) * nkt;
    const int64_t kofs = kMN ? static_cast<int64_t>(kk) * kKStep * ld_bytes : static_cast<int64_t>(kk) * kRowBytes;
    const char *const bl = gl + (kofs + s1 * dl1 + s2 * dl2);  // uniform
    const char *const br = gr + (kofs + s1 * dr1 + s2 * dr2);
    // opaque copy: the per-instruction offsets are rebuilt at every issue
    // instead of being kept live across the mainloop
    uint32_t g0 = goff0;
    asm volatile("" : "+v"(g0));
    // instruction j of half h of an operand (src, LDS operand op)
    auto load = [&](const char *src, int op, int h, int j) {
      const int row = lrow + j * 4 * kRowsPerKB;  // row within the half
      uint32_t go = g0 + static_cast<uint32_t>(j) * goff_step;
      if constexpr (kMN)
        go += static_cast<uint32_t>(h * (kHalfBytes / (kRowBytes / static_cast<int>(sizeof(T))))) +
              static_cast<uint32_t>(lpc ^ mn_swz<T>(row)) * 16;
      else
        go += static_cast<uint32_t>(h * (kTile / 2)) * static_cast<uint32_t>(ld_bytes) +
              static_cast<uint32_t>(swz(lpc, row)) * 16;
      __builtin_amdgcn_global_load_lds(
          (const void *)(src + go),
          (__attribute__((address_space(3))) void *)(st + op * kOperandBytes + h * kHalfBytes +
                                                     (j * 4 + wn) * 1024),
          16, 0, 0);
    };
#pragma unroll
    for (int j = 0; j < kPerLoader; ++j) load(bl, 0, wm, j);
    if (wm == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < kPerLoader; ++j) load(br, 1, h, j);
    }
  };

  const int r16 = lane & 15, g4 = lane >> 4;

  f32x4 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments of one K step: sub-step 0 covers k chunks 0-3, sub-step 1
  // chunks 4-7 of the 128-byte rows.
  // Transposed reads return 8-byte halves; they are kept as such until the
  // explicit wait, so that no register copy can read them before they land.
  constexpr bool kTr = kMN && sizeof(T) == 2;
  struct FragK {
    u32x4 l[kFragM], r[kFragN];
  };
  struct FragT {
    u32x2 l[kFragM][2], r[kFragN][2];
  };
  using Frag = std::conditional_t<kTr, FragT, FragK>;
  // MN-major bf16: lane l of 16-lane group g4 reads k rows 32*sub + 8*g4 +
  // 4*h + te (te = (l%16)/4) at column m0 + 4*tq (tq = l%4); rows & 3 = te and
  // bit 3 of the row = g4 & 1, so the swizzle is a lane constant.
  const int te = (lane & 15) >> 2, tq = lane & 3;
  const int tr_swz = mn_swz<T>(8 * g4 + te);
  const uint32_t tr_base = static_cast<uint32_t>((8 * g4 + te) * 256 + (tq & 1) * 8);
  auto tr_addr = [&](const lds_char *op, int sub, int h, int m0) -> uint32_t {
    // column m0 + 4*tq lies in half m0/128, chunk (m0%128)/8 + tq/2 of its
    // 256-byte row, XOR the swizzle (bits 1-3)
    const int chunk = ((m0 & 127) >> 3) + (tq >> 1);
    return (uint32_t)(uintptr_t)op + static_cast<uint32_t>((m0 >> 7) * kHalfBytes) + tr_base +
           static_cast<uint32_t>((32 * sub + 4 * h) * 256) + static_cast<uint32_t>((chunk ^ tr_swz) * 16);
  };
  auto read_frag = [&](const lds_char *st, int sub, Frag &f) {
    if constexpr (kTr) {
#pragma unroll
      for (int i = 0; i < kFragM; ++i) {
        const int m0 = wm * kWaveM + i * 16;
#pragma unroll
        for (int h = 0; h < 2; ++h) f.l[i][h] = ds_read_tr16(tr_addr(st, sub, h, m0));
      }
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int m0 = wn * kWaveN + j * 16;
#pragma unroll
        for (int h = 0; h < 2; ++h) f.r[j][h] = ds_read_tr16(tr_addr(st + kOperandBytes, sub, h, m0));
      }
    } else if constexpr (kMN) {  // fp32: lane (r16, g4) needs k = 16*sub + 4*g4 + t, t = 0..3, of column m
      typedef __attribute__((address_space(3))) uint32_t lds_u32;
      auto col = [&](const lds_char *op, int m) {
        u32x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = 16 * sub + 4 * g4 + t;
          v[t] = *(const lds_u32 *)(op + (m >> 7) * kHalfBytes + row * 512 +
                                    ((((m & 127) >> 2) ^ mn_swz<T>(row)) * 16) + (m & 3) * 4);
        }
        return v;
      };
#pragma unroll
      for (int i = 0; i < kFragM; ++i) f.l[i] = col(st, wm * kWaveM + i * 16 + r16);
#pragma unroll
      for (int j = 0; j < kFragN; ++j) f.r[j] = col(st + kOperandBytes, wn * kWaveN + j * 16 + r16);
    } else {
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
    }
  };
  // The transposed reads are not counted by the compiler: wait for them
  // explicitly, tied to every half so that no use (or copy) moves above the
  // wait, and keep the product block between the reads and the wait.
  auto tr_wait = [&](Frag &f) {
    if constexpr (kTr) {
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(f.l[0][0]), "+v"(f.l[0][1]), "+v"(f.l[1][0]), "+v"(f.l[1][1]), "+v"(f.l[2][0]),
                     "+v"(f.l[2][1]), "+v"(f.l[3][0]), "+v"(f.l[3][1]), "+v"(f.l[4][0]), "+v"(f.l[4][1]),
                     "+v"(f.l[5][0]), "+v"(f.l[5][1]), "+v"(f.l[6][0]), "+v"(f.l[6][1]), "+v"(f.l[7][0]),
                     "+v"(f.l[7][1]));
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(f.r[0][0]), "+v"(f.r[0][1]), "+v"(f.r[1][0]), "+v"(f.r[1][1]), "+v"(f.r[2][0]),
                     "+v"(f.r[2][1]), "+v"(f.r[3][0]), "+v"(f.r[3][1]));
    }
  };
  auto opnd = [&](const auto &x) -> u32x4 {  // one MFMA operand of a fragment
    if constexpr (kTr)
      return u32x4{x[0].x, x[0].y, x[1].x, x[1].y};
    else
      return x;
  };
  auto tr_fence = [&]() {
    if constexpr (kTr) __builtin_amdgcn_sched_barrier(0);
  };
  auto mfma_frag = [&](const Frag &f) {
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) Mfma<T>::run(acc[i][j], opnd(f.l[i]), opnd(f.r[j]));
  };

  // The aX term of Apply comes from the R operand, X^T: its rows are the tile's columns and its K range
  // [ti*256, ti*256 + 256) holds the tile's rows.  While the K steps of the
  // wave's 128 rows are in LDS, each lane reads its four values (four
  // consecutive k of one R row) and adds a*X to the accumulators.
  constexpr int kCapSteps = kWaveM / kKStep;                         // steps holding the wave's rows
  constexpr int kCapFrags = kKStep / 16;                             // fragment rows per step
  constexpr bool cap_ax = MODE == kModeApply || MODE == kModeFinal || MODE == kModeSquare;
  // Square's R operand is A and A is symmetric, so the same K steps hold
  // A[row][col] (= A[col][row]); it adds (b/c) A, the epilogue scales by c.
  // With c = 0 (or b/c not finite) it captures nothing and the epilogue
  // reads A instead.
  const float sq_w = d.cc != 0.f ? d.cb / d.cc : 0.f;
  const bool sq_cap = MODE == kModeSquare && d.cc != 0.f && __builtin_isfinite(sq_w);
  const float cap_w = MODE == kModeSquare ? (sq_cap ? sq_w : 0.f) : d.ca;
  const int cap_kt0 = ti * (kTile / kKStep) + wm * kCapSteps;
  // Only the first pass of the K loop captures: its R is R itself (later
  // passes read R_lo or run past kt = nkt, where c >= kCapSteps); the host
  // gives a capturing Square no hi + lo operand.
  // Step c of the wave's kCapSteps holds fragment rows [c*kCapFrags,
  // (c+1)*kCapFrags).  Every fragment row reads and adds at every capture
  // step, with weight a on its own step and 0 on the others (at an address
  // of the same step), so no accumulator is indexed by a run-time value.
  auto capture_ax = [&](const lds_char *st, int kt) {
    if constexpr (!cap_ax) return;
    const int c = kt - cap_kt0;  // uniform in the wave
    // a zero weight (the plain products of the Gram-space chain and its
    // X <- QX) adds nothing: skip the reads
    if (c < 0 || c >= kCapSteps || cap_w == 0.f) return;
#pragma unroll
    for (int i = 0; i < kFragM; ++i) {
      const float w = (i / kCapFrags == c) ? cap_w : 0.f;
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

  // In a diagonal tile of a symmetric output, rows 128-255 x columns 0-127
  // lie below the diagonal: the epilogue stores the upper triangle and its
  // mirror and never these values, so the two waves holding them (wm = 1,
  // wn < 2) skip their products and only keep the barrier schedule.
  constexpr bool kSymOut = MODE == kModeGram || MODE == kModeSquare;
  const bool lower_quadrant = kSymOut && ti == tj && wm == 1 && wn < 2;

  Frag fa, fb;
  // Waves 0-3 (the tile's rows 0-127) and waves 4-7 (rows 128-255) run the
  // same step: a read phase (next stage's loads issued, both sub-steps'
  // fragments read) then a product phase (the step's MFMAs), each ended by
  // a work-group barrier.  Waves 4-7 start one barrier late, so each SIMD
  // (one wave of each half) multiplies for one half while the other half
  // reads.  Step kt's stage takes step kt+2's loads only after both halves
  // have read it.  The loads of step kt+1 that a half issues in its read
  // phase of step kt are waited for at the end of its product phase: for
  // waves 0-3 (their L rows and R) before either half reads that stage,
  // for waves 4-7 (their L rows) before they read it.  No LDS-bound load
  // is in flight after the loop.  The last step re-loads its own K range
  // into the free stage, which keeps the loop body free of a branch
  // (measured faster than skipping that load).
  if constexpr (!kReduce) {
    issue(kbeg & 1, kbeg);
    stage_barrier();
    if (wm == 1) plain_barrier();
    for (int kt = kbeg; kt < kend; ++kt) {
      const lds_char *st = lds + (kt & 1) * kStageBytes;
      issue((kt + 1) & 1, min(kt + 1, kend - 1));
      capture_ax(st, kt);
      read_frag(st, 0, fa);
      read_frag(st, 1, fb);
      tr_fence();
      tr_wait(fa);
      tr_wait(fb);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (!lower_quadrant) {
        mfma_frag(fa);
        mfma_frag(fb);
      }
      __builtin_amdgcn_sched_barrier(0);
      dma_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (wm == 0) plain_barrier();
  }

  // Partial slots: fragment (i, j) of thread t at vector (i * kFragN + j) *
  // kThreads + t of the slot; the slot's base is uniform.
  constexpr int64_t kSlotVecs = kPartialSlotFloats / 4;
  if constexpr (kPiece) {
    f32x4 *const base = splitk + static_cast<int64_t>(e.slot) * kSlotVecs;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) base[(i * kFragN + j) * kThreads + tid] = acc[i][j];
    return;
  }
  if constexpr (kReduce) {
    // each element sums its pieces in slot order; one fragment row at a
    // time, so that few loads are in flight beside the accumulators
    const f32x4 *const base = splitk + static_cast<int64_t>(e.slot) * kSlotVecs;
#pragma unroll
    for (int i = 0; i < kFragM; ++i) {
#pragma unroll
      for (int j = 0; j < kFragN; ++j) acc[i][j] = base[(i * kFragN + j) * kThreads + tid];
      for (int32_t q = 1; q < e.k0; ++q)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) acc[i][j] += base[q * kSlotVecs + (i * kFragN + j) * kThreads + tid];
    }
  }

  // ---- epilogue: lane holds C[row0 + 4*g4 + v][col0 + r16], v = 0..3 ----
  // The four values of a lane are four consecutive rows of one column, i.e.
  // four consecutive elements of a row of the transposed matrix: transposed
  // reads and writes move them as one 8-byte (bf16) or 16-byte (fp32) vector.
  // Row-major bf16 outputs are staged through LDS (the 128 KB of the two
  // stages hold one 256 x 256 bf16 tile) and leave as 16-byte row segments.
  // rows of the computed product come from the L panel, columns from R
  const int64_t row_base = static_cast<int64_t>(ti) * kTile + wm * kWaveM + 4 * g4;
  const int64_t col_base = static_cast<int64_t>(tj) * kTile + wn * kWaveN + r16;
  constexpr bool kStage = sizeof(T) == 2;
  // fragment rows whose epilogue inputs are read in one batch: all of them
  // for bf16 (2 VGPRs per vector), two at a time for fp32 (4 per vector)
  constexpr int kReadRows = sizeof(T) == 2 ? kFragM : 2;
  // The loop's last barrier is passed by every wave after all of the
  // mainloop's LDS reads and LDS-bound loads: the LDS is free for staging.

  // The first iteration's X is U unnormalised (X0 = U * inv_norm): A0 picks
  // up inv_norm^2 and the first X' (or O) inv_norm.
  // A scalar load (written by an earlier kernel, uniform in the work-group):
  // as a vector load it would be counted with the LDS-bound loads, and the
  // compiler, which does not see the mainloop's own waits, would wait for
  // every outstanding vector load (Final's parameter reads included) at its
  // first use.
  const float inv = d.first_it ? *(const __attribute__((address_space(4))) float *)d.inv_norm : 1.f;
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
    if (MODE == kModeSquare && !sq_cap)
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
          if (sq_cap) {
#pragma unroll
            for (int v = 0; v < 4; ++v) val[v] = d.cc * val[v];  // b A is in the accumulator as (b/c) A
          } else {
            const f32x4 av = Vec4<T>::cvt(araw[ii][j]);
#pragma unroll
            for (int v = 0; v < 4; ++v) val[v] = fmaf(d.cb, av[v], d.cc * val[v]);
          }
          // diag I on the true diagonal only: the padding stays zero
          if (ti == tj && col < d.m)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (row + v == col) val[v] += d.cdiag;
        }
        if constexpr (kStage) {
          if (ti != tj)
            stage_tile_put<TS>(lds, wm * kWaveM + i * 16 + 4 * g4, wn * kWaveN + j * 16 + r16, val);
          else
            stage_tile_put_sym<TS>(lds, wm * kWaveM + i * 16 + 4 * g4, wn * kWaveN + j * 16 + r16, val);
          acc[i][j] = val;  // kept for the mirror tile
        } else if (ti != tj) {
#pragma unroll
          for (int v = 0; v < 4; ++v) WsType<T>::st(out, (row + v) * mp + col, val[v]);
          Vec4<T>::st(out + col * mp + row, val);
        } else {  // diagonal tile: upper triangle and its mirror, as above
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (col >= row + v) WsType<T>::st(out, (row + v) * mp + col, val[v]);
            if (col > row + v) WsType<T>::st(out, col * mp + row + v, val[v]);
          }
        }
      }
    }
    if constexpr (kStage) {
      const int64_t tile_ij = static_cast<int64_t>(ti) * kTile * mp + static_cast<int64_t>(tj) * kTile;
      const int64_t tile_ji = static_cast<int64_t>(tj) * kTile * mp + static_cast<int64_t>(ti) * kTile;
      // hi half (the output itself), then, for a hi + lo pair, the low half
      // lo = RNE(v - RNE(v)); each as the tile and, off the diagonal, its
      // mirror tile (tj, ti) staged the transposed way
      uint16_t *const o16 = reinterpret_cast<uint16_t *>(out);
      uint16_t *const lo16 = MODE == kModeSquare ? reinterpret_cast<uint16_t *>(d.out_lo) : nullptr;
      stage_tile_flush<kSwzRows, TS>(lds, o16 + tile_ij, mp, tid);
      if (ti != tj) {
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kFragM; ++i)
#pragma unroll
          for (int j = 0; j < kFragN; ++j)
            stage_tile_put_t<TS>(lds, wn * kWaveN + j * 16 + r16, wm * kWaveM + i * 16 + 4 * g4, acc[i][j]);
        stage_tile_flush<kSwzCols, TS>(lds, o16 + tile_ji, mp, tid);
      }
      if (lo16) {
        // The low halves go to the same LDS slots as the high ones: opaque
        // lane coordinates make the compiler rebuild those addresses here
        // rather than keep them live through the flushes above.
        int lo_lane = lane;
        asm volatile("" : "+v"(lo_lane));
        const int lr16 = lo_lane & 15, lg4 = lo_lane >> 4;
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kFragM; ++i)
#pragma unroll
          for (int j = 0; j < kFragN; ++j) {
            const f32x4 lo = bf16_low_part(acc[i][j]);
            if (ti != tj)
              stage_tile_put<TS>(lds, wm * kWaveM + i * 16 + 4 * lg4, wn * kWaveN + j * 16 + lr16, lo);
            else
              stage_tile_put_sym<TS>(lds, wm * kWaveM + i * 16 + 4 * lg4, wn * kWaveN + j * 16 + lr16, lo);
          }
        stage_tile_flush<kSwzRows, TS>(lds, lo16 + tile_ij, mp, tid);
        if (ti != tj) {
          lds_barrier();
#pragma unroll
          for (int i = 0; i < kFragM; ++i)
#pragma unroll
            for (int j = 0; j < kFragN; ++j)
              stage_tile_put_t<TS>(lds, wn * kWaveN + j * 16 + lr16, wm * kWaveM + i * 16 + 4 * lg4,
                               bf16_low_part(acc[i][j]));
          stage_tile_flush<kSwzCols, TS>(lds, lo16 + tile_ji, mp, tid);
        }
      }
    }
  } else if (MODE == kModeApply) {
    T *XTn = static_cast<T *>(d.xt[1]);
    const int64_t mp = d.mp;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int64_t col = col_base + j * 16, row = row_base + i * 16;
        f32x4 val;  // a*X is already in the accumulator
#pragma unroll
        for (int v = 0; v < 4; ++v) val[v] = acc[i][j][v] * inv;
        // X'^T[col][row .. row+3]: four consecutive elements of a row
        if constexpr (kStage)
          stage_tile_put_t<TS>(lds, wn * kWaveN + j * 16 + r16, wm * kWaveM + i * 16 + 4 * g4, val);
        else
          Vec4<T>::st(XTn + col * mp + row, val);
      }
    if constexpr (kStage)
      stage_tile_flush<kSwzCols, TS>(lds, reinterpret_cast<uint16_t *>(XTn) + static_cast<int64_t>(tj) * kTile * mp +
                                          static_cast<int64_t>(ti) * kTile, mp, tid);
  } else {  // kModeFinal
    // O = (aX + BX) * inv for the tile (rows over m, columns over n) goes
    // through LDS as fp32, one half of the rows at a time (the waves with
    // wm == h hold half h): row-major when P = O (m x n), transposed when
    // P = O^T (n x m).  Then all threads update P in eight-element pieces
    // along its rows (16-byte accesses: the epilogue is bound by the number
    // of memory instructions, not by bytes): P -= lr*scale*O, and
    // orth_out = O.  The aX term is already in the accumulators: it was
    // captured from the X^T tile in LDS during the mainloop, as in Apply.
    const float step = s.lr * d.scale;
    const bool tp = d.transposed != 0;
    // rows of P start 16-byte aligned (the buffers are: the host checks)
    const bool vec_ok = (d.cols & 7) == 0;
    // the tile lies wholly inside P and every piece is a full vector
    const bool whole = vec_ok && (tp ? (tj + 1) * kTile <= d.rows && (ti + 1) * kTile <= d.cols
                                     : (ti + 1) * kTile <= d.rows && (tj + 1) * kTile <= d.cols);
    typedef __attribute__((address_space(3))) float lds_f32;
    typedef __attribute__((address_space(3))) u32x4 lds_v4;
    // [128][256] fp32, 1 KB rows: chunk XOR 4 * ((row / 4) mod 4), so the four
    // rows of one put land in distinct 64-byte bank groups
    auto o_at = [&](int r, int c) { return r * 1024 + (((c >> 2) ^ (((r >> 2) & 3) << 2)) * 16) + (c & 3) * 4; };
    // [256][128] fp32, 512-byte rows: chunk XOR 4 * (row mod 4)
    auto ot_at = [&](int r, int c) { return r * 512 + (((c >> 2) ^ ((r & 3) << 2)) * 16); };
    // A piece's two 16-byte halves are read in the order (sw, 1 - sw): the 16
    // lanes of one LDS read pass hold 16 consecutive pieces of one row, and
    // with sw = bit 3 of the lane they touch 16 distinct bank groups.
    const int sw = (lane >> 3) & 1;
    auto update = [&](auto ptag) {
      using PT = decltype(ptag);
      PT *const P = static_cast<PT *>(d.param);
      PT *const Orth = static_cast<PT *>(d.orth);
      PT *const Packed = static_cast<PT *>(d.packed);  // nullable copy of the updated P
      // bf16 P: the 8 pieces of both halves are read before the first half
      // is staged, so their latency hides behind the staging and the first
      // half's update; fp32 P reads its pieces in batches of 2 after staging
      // (register budget)
      constexpr bool kPre = sizeof(PT) == 2;
      constexpr int kPieces = 8;
      constexpr int kBatch = kPre ? kPieces : 2;
      // Piece q of this thread in half h: staged block (r, c), P element
      // (pr, pc), n valid.
      struct Piece {
        int r, c, n;
        int64_t idx;
      };
      auto piece_of = [&](int h, int q) {
        Piece pc_;
        int64_t pr, pcol;
        if (tp) {
          pc_.r = q * 32 + (tid >> 4), pc_.c = (tid & 15) * 8;
          pr = static_cast<int64_t>(tj) * kTile + pc_.r;
          pcol = static_cast<int64_t>(ti) * kTile + h * kWaveM + pc_.c;
        } else {
          pc_.r = q * 16 + (tid >> 5), pc_.c = (tid & 31) * 8;
          pr = static_cast<int64_t>(ti) * kTile + h * kWaveM + pc_.r;
          pcol = static_cast<int64_t>(tj) * kTile + pc_.c;
        }
        pc_.n = (pr < d.rows && pcol < d.cols) ? static_cast<int>(min<int64_t>(8, d.cols - pcol)) : 0;
        pc_.idx = pr * d.cols + pcol;
        return pc_;
      };
      // O of half h into LDS (the previous half read first)
      auto stage_half = [&](int h) {
        if (h > 0) lds_barrier();
        if (wm == h) {
#pragma unroll
          for (int i = 0; i < kFragM; ++i)
#pragma unroll
            for (int j = 0; j < kFragN; ++j) {
              const int rl = i * 16 + 4 * g4, cl = wn * kWaveN + j * 16 + r16;
              f32x4 o;  // a*X is already in the accumulator
#pragma unroll
              for (int v = 0; v < 4; ++v) o[v] = acc[i][j][v] * inv;
              if (tp) {
                *(lds_v4 *)(lds + ot_at(cl, rl)) =
                    u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
              } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) *(lds_f32 *)(lds + o_at(rl + v, cl)) = o[v];
              }
            }
        }
        lds_barrier();
      };
      // the staged O of piece pp, its eight values in column order
      auto staged = [&](const Piece &pp, float (&o)[8]) {
        auto at = [&](int c) { return tp ? ot_at(pp.r, c) : o_at(pp.r, c); };
        const u32x4 u0 = *(const lds_v4 *)(lds + at(pp.c + 4 * sw));
        const u32x4 u1 = *(const lds_v4 *)(lds + at(pp.c + 4 - 4 * sw));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          o[v] = __uint_as_float(sw ? u1[v] : u0[v]);
          o[4 + v] = __uint_as_float(sw ? u0[v] : u1[v]);
        }
      };
      if constexpr (kPre) {
        if (whole) {
          // A whole tile runs with no branch from its parameter reads to
          // its last store, so that the compiler waits for each piece's
          // own read (a counted vmcnt).  With a branch in between it waits
          // for every outstanding access, the previous pieces' stores
          // included, and each piece pays a store's whole latency.
          typename Vec8<PT>::Raw pw[kWavesM][kPieces];
#pragma unroll
          for (int h = 0; h < kWavesM; ++h)
#pragma unroll
            for (int q = 0; q < kPieces; ++q) pw[h][q] = Vec8<PT>::raw(P + piece_of(h, q).idx);
#pragma unroll
          for (int h = 0; h < kWavesM; ++h) {
            stage_half(h);
#pragma unroll
            for (int q = 0; q < kPieces; ++q) {
              const Piece pp = piece_of(h, q);
              float o[8], pv[8], nv[8];
              staged(pp, o);
              Vec8<PT>::cvt(pw[h][q], pv);
#pragma unroll
              for (int v = 0; v < 8; ++v) nv[v] = fmaf(-step, o[v], pv[v]);
              Vec8<PT>::st(P + pp.idx, nv);
              if (Packed) Vec8<PT>::st(Packed + pp.idx, nv);
              if (Orth) Vec8<PT>::st(Orth + pp.idx, o);
            }
          }
          return;
        }
      }
      typename Vec8<PT>::Raw pre[kPre ? kWavesM : 1][kPre ? kPieces : 1];
      if constexpr (kPre) {
#pragma unroll
        for (int h = 0; h < kWavesM; ++h)
#pragma unroll
          for (int q = 0; q < kPieces; ++q) {
            const Piece pp = piece_of(h, q);
            if (vec_ok && pp.n == 8) pre[h][q] = Vec8<PT>::raw(P + pp.idx);
          }
      }
#pragma unroll
      for (int h = 0; h < kWavesM; ++h) {
        auto piece = [&](int q) { return piece_of(h, q); };
        stage_half(h);
#pragma unroll
        for (int q0 = 0; q0 < kPieces; q0 += kBatch) {
          typename Vec8<PT>::Raw praw[kBatch];
#pragma unroll
          for (int qq = 0; qq < kBatch; ++qq) {
            const Piece pp = piece(q0 + qq);
            if constexpr (kPre)
              praw[qq] = pre[h][q0 + qq];
            else if (vec_ok && pp.n == 8)
              praw[qq] = Vec8<PT>::raw(P + pp.idx);
          }
#pragma unroll
          for (int qq = 0; qq < kBatch; ++qq) {
            const Piece pp = piece(q0 + qq);
            if (pp.n == 0) continue;
            float o[8];
            staged(pp, o);
            if (vec_ok && pp.n == 8) {
              float pv[8], nv[8];
              Vec8<PT>::cvt(praw[qq], pv);
#pragma unroll
              for (int v = 0; v < 8; ++v) nv[v] = fmaf(-step, o[v], pv[v]);
              Vec8<PT>::st(P + pp.idx, nv);
              if (Packed) Vec8<PT>::st(Packed + pp.idx, nv);
              if (Orth) Vec8<PT>::st(Orth + pp.idx, o);
            } else {
              for (int v = 0; v < pp.n; ++v) {
                if (d.orth) store_elem(d.orth, d.param_dt, pp.idx + v, o[v]);
                const float nv1 = fmaf(-step, o[v], load_elem(d.param, d.param_dt, pp.idx + v));
                store_elem(d.param, d.param_dt, pp.idx + v, nv1);
                if (d.packed) store_elem(d.packed, d.param_dt, pp.idx + v, nv1);
              }
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

// The grouped launch of one stage: work-group w runs entry w / 8 of XCD
// (w % 8)'s tile list.  A launch of Gram and Square tiles of different
// matrices (kModeGramSquare) runs each tile with its matrix's stage.
template <typename T, int MODE, int ROLE>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(const MatDev *__restrict__ mats,
                                                           const TileEntry *__restrict__ tiles,
                                                           StageXcd xcd, StepScalars s,
                                                           f32x4 *__restrict__ splitk) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kOperandBytes];  // 128 KB
  // C cast: generic -> LDS address space
  lds_char *const lds = (lds_char *)smem;
  const int32_t w = static_cast<int32_t>(blockIdx.x);
  const int32_t xi = w % kXcds, k = w / kXcds;
  if (k >= xcd.count[xi]) return;  // whole group leaves before any barrier
  const TileEntry e = tiles[xcd.first[xi] + k];
  const MatDev &d = mats[e.mat];
  if constexpr (MODE == kModeGramSquare) {
    if (d.gemm_kind == kModeGram)
      gemm_tile<T, kModeGram, ROLE>(lds, d, e, s, splitk);
    else
      gemm_tile<T, kModeSquare, ROLE>(lds, d, e, s, splitk);
  } else {
    gemm_tile<T, MODE, ROLE>(lds, d, e, s, splitk);
  }
}

// Square launches of 128 x 128 tiles (bf16, whole tiles): the same work-group
// of 8 waves on a 64 KB operand ring, so that two work-groups fit on a CU.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void ns_gemm_small_kernel(const MatDev *__restrict__ mats, const TileEntry *__restrict__ tiles, StageXcd xcd,
                          StepScalars s) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * 128 * kRowBytes];  // 64 KB
  lds_char *const lds = (lds_char *)smem;
  const int32_t w = static_cast<int32_t>(blockIdx.x);
  const int32_t xi = w % kXcds, k = w / kXcds;
  if (k >= xcd.count[xi]) return;  // whole group leaves before any barrier
  const TileEntry e = tiles[xcd.first[xi] + k];
  gemm_tile<uint16_t, kModeSquare, kRoleWhole, 128>(lds, mats[e.mat], e, s, nullptr);
}

// One launch for all bf16 stages of a step (the chained mode).  Every matrix
// has all of its tiles, of every stage, in one XCD's queue, in the order of
// the stages; a work-group takes the next entry of its own XCD's queue (the
// hardware XCC id picks the queue), waits until the previous stage of that
// matrix has signalled all its tiles, runs the tile with its stage's code and
// signals.  An entry waits only on entries earlier in the same queue, which
// running work-groups took before it, so every wait ends; a wait that has not
// ended after kChainSpinLimit polls sets the timeout word and goes on (wrong
// values, never a hang).  A matrix's producers and consumers run on one XCD
// and share its L2: a producer signals once its stores have reached L2
// (vmcnt), and a consumer takes an agent-scope acquire after its wait,
// which drops its CU's L1 lines (a workgroup-scope invalidate let stale L1
// lines through; an agent-scope release, an L2 write-back per tile, is not
// needed on one L2 and cost a third of the step).
// Entry fields: k0 = counter waited on (-1: none), k1 = the count it waits
// for, slot = counter signalled.  sync: kXcds tickets, the timeout word at
// kXcds, counters from kChainCounters.
constexpr int32_t kChainSpinLimit = 1 << 20;

__device__ __forceinline__ int32_t xcc_id() {
  int32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
  return v;
}

__global__ __launch_bounds__(kThreads) void ns_gemm_chain_kernel(const MatDev *__restrict__ mats,
                                                                 const TileEntry *__restrict__ tiles, StageXcd xcd,
                                                                 StepScalars s, int32_t *__restrict__ sync) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes];
  __shared__ int32_t ticket;
  lds_char *const lds = (lds_char *)smem;
  const int32_t xi = xcc_id() & (kXcds - 1);
  if (threadIdx.x == 0) ticket = __hip_atomic_fetch_add(sync + xi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int32_t k = ticket;
  if (k >= xcd.count[xi]) return;  // the whole group leaves
  const TileEntry e = tiles[xcd.first[xi] + k];
  if (e.k0 >= 0) {
    if (threadIdx.x == 0) {
      int32_t *const c = sync + kChainCounters + e.k0;
      for (int32_t spins = 0; __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < e.k1;) {
        __builtin_amdgcn_s_sleep(8);
        if (++spins == kChainSpinLimit) {
          __hip_atomic_store(sync + kXcds, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  const MatDev &d = mats[e.mat];
  switch (d.gemm_kind) {
    case kModeGram:
      gemm_tile<uint16_t, kModeGram, kRoleWhole>(lds, d, e, s, nullptr);
      break;
    case kModeSquare:
      gemm_tile<uint16_t, kModeSquare, kRoleWhole>(lds, d, e, s, nullptr);
      break;
    case kModeApply:
      gemm_tile<uint16_t, kModeApply, kRoleWhole>(lds, d, e, s, nullptr);
      break;
    default:
      gemm_tile<uint16_t, kModeFinal, kRoleWhole>(lds, d, e, s, nullptr);
      break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have reached the XCD's L2
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(sync + kChainCounters + e.slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int ROLE>
hipError_t launch_role(GemmMode mode, const MatDev *mats, const TileEntry *tiles, const StageXcd &xcd,
                       StepScalars s, f32x4 *splitk, hipStream_t st) {
  int32_t longest = 0;
  for (int x = 0; x < kXcds; ++x) longest = xcd.count[x] > longest ? xcd.count[x] : longest;
  if (longest == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(longest) * kXcds), block(kThreads);
  switch (mode) {
    case kModeGram:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeGram, ROLE>), grid, block, 0, st, mats, tiles, xcd, s, splitk);
      break;
    case kModeSquare:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeSquare, ROLE>), grid, block, 0, st, mats, tiles, xcd, s, splitk);
      break;
    case kModeApply:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeApply, ROLE>), grid, block, 0, st, mats, tiles, xcd, s, splitk);
      break;
    case kModeGramSquare:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeGramSquare, ROLE>), grid, block, 0, st, mats, tiles, xcd, s,
                         splitk);
      break;
    default:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeFinal, ROLE>), grid, block, 0, st, mats, tiles, xcd, s, splitk);
      break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(GemmMode mode, int role, const MatDev *mats, const TileEntry *tiles, const StageXcd &xcd,
                    StepScalars s, float *splitk_f, hipStream_t st) {
  f32x4 *splitk = reinterpret_cast<f32x4 *>(splitk_f);
  switch (role) {
    case kRolePiece: return launch_role<T, kRolePiece>(mode, mats, tiles, xcd, s, splitk, st);
    case kRoleReduce: return launch_role<T, kRoleReduce>(mode, mats, tiles, xcd, s, splitk, st);
    default: return launch_role<T, kRoleWhole>(mode, mats, tiles, xcd, s, splitk, st);
  }
}

}  // namespace

hipError_t launch_ns_small_square(const MatDev *mats, const TileEntry *tiles, const StageXcd &xcd, StepScalars s,
                                  hipStream_t st) {
  int32_t longest = 0;
  for (int x = 0; x < kXcds; ++x) longest = xcd.count[x] > longest ? xcd.count[x] : longest;
  if (longest == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(longest) * kXcds), block(kThreads);
  hipLaunchKernelGGL(ns_gemm_small_kernel, grid, block, 0, st, mats, tiles, xcd, s);
  return hipGetLastError();
}

hipError_t launch_ns_chain(const MatDev *mats, const TileEntry *tiles, const StageXcd &xcd, StepScalars s,
                           int32_t *sync, hipStream_t st) {
  int32_t longest = 0;
  for (int x = 0; x < kXcds; ++x) longest = xcd.count[x] > longest ? xcd.count[x] : longest;
  if (longest == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(longest) * kXcds), block(kThreads);
  hipLaunchKernelGGL(ns_gemm_chain_kernel, grid, block, 0, st, mats, tiles, xcd, s, sync);
  return hipGetLastError();
}

hipError_t launch_ns_stage(GemmMode mode, bool fp32, int role, const MatDev *mats, const TileEntry *tiles,
                           const StageXcd &xcd, StepScalars s, float *splitk, hipStream_t st) {
  return fp32 ? launch_t<float>(mode, role, mats, tiles, xcd, s, splitk, st)
              : launch_t<uint16_t>(mode, role, mats, tiles, xcd, s, splitk, st);
}

}  // namespace dmuon
