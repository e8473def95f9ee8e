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
template <typename T> struct Vec4;
template <> struct Vec4<uint16_t> {
  static __device__ __forceinline__ f32x4 ld(const uint16_t *p) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                 __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
  }
  static __device__ __forceinline__ void st(uint16_t *p, const f32x4 &v) {
    uint2 u;
    u.x = static_cast<uint32_t>(f32_to_bf16_bits(v[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
    u.y = static_cast<uint32_t>(f32_to_bf16_bits(v[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
    *reinterpret_cast<uint2 *>(p) = u;
  }
};
template <> struct Vec4<float> {
  static __device__ __forceinline__ f32x4 ld(const float *p) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    return f32x4{v.x, v.y, v.z, v.w};
  }
  static __device__ __forceinline__ void st(float *p, const f32x4 &v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Upper-triangle tile t (row-major enumeration) of a tm x tm tile grid.
__device__ __forceinline__ void upper_tile(int32_t t, int32_t tm, int32_t &ti, int32_t &tj) {
  int32_t r = 0;
  while (t >= tm - r) { t -= tm - r; ++r; }
  ti = r;
  tj = r + t;
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(const MatDev *__restrict__ mats,
                                                           const StageEntry *__restrict__ stage,
                                                           int32_t nstage, int32_t cur,
                                                           StepScalars s) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kOperandBytes];  // 128 KB
  lds_char *const lds = (lds_char *)smem;  // C cast: generic -> LDS address space  // [2 stages][L, R][256][128 B]

  const int64_t w = blockIdx.x;
  const int32_t si = find_range(nstage, w, [&](int32_t i) { return stage[i].first; });
  const MatDev &d = mats[stage[si].mat];
  const int32_t t = static_cast<int32_t>(w - stage[si].first);

  int32_t ti, tj;
  constexpr bool kSym = (MODE == kModeGram || MODE == kModeSquare);
  if (kSym) {
    upper_tile(t, d.tm, ti, tj);
  } else {
    // column of tiles first: consecutive work-groups share the X^T panel
    ti = t % d.tm;
    tj = t / d.tm;
  }

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
  const char *gl = reinterpret_cast<const char *>(L) + static_cast<int64_t>(ti) * kTile * ld_bytes;
  const char *gr = reinterpret_cast<const char *>(R) + static_cast<int64_t>(tj) * kTile * ld_bytes;

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

  issue(0);
  for (int kt = 0; kt < nkt; ++kt) {
    stage_barrier();               // step kt is in LDS; step kt-1's stage is free
    if (kt + 1 < nkt) issue(kt + 1);
    const lds_char *sl = lds + (kt & 1) * kStageBytes;
    const lds_char *sr = sl + kOperandBytes;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int chunk = sub * 4 + g4;
      u32x4 fl[kFragM], fr[kFragN];
#pragma unroll
      for (int i = 0; i < kFragM; ++i) {
        const int row = wm * kWaveM + i * 16 + r16;
        fl[i] = *(const lds_u32x4 *)(sl + row * kRowBytes + swz(chunk, row) * 16);
      }
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int row = wn * kWaveN + j * 16 + r16;
        fr[j] = *(const lds_u32x4 *)(sr + row * kRowBytes + swz(chunk, row) * 16);
      }
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) Mfma<T>::run(acc[i][j], fl[i], fr[j]);
    }
  }

  // ---- epilogue: lane holds C[row0 + 4*g4 + v][col0 + r16], v = 0..3 ----
  // The four values of a lane are four consecutive rows of one column, i.e.
  // four consecutive elements of a row of the transposed matrix: transposed
  // reads and writes move them as one 8-byte (bf16) or 16-byte (fp32) vector.
  const int64_t row_base = static_cast<int64_t>(ti) * kTile + wm * kWaveM + 4 * g4;
  const int64_t col_base = static_cast<int64_t>(tj) * kTile + wn * kWaveN + r16;

  if (MODE == kModeGram || MODE == kModeSquare) {
    T *out = static_cast<T *>(MODE == kModeGram ? d.a : d.b);
    const T *prev = static_cast<const T *>(d.a);
    const int64_t mp = d.mp;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int64_t col = col_base + j * 16, row = row_base + i * 16;
        f32x4 val = acc[i][j];
        if (MODE == kModeSquare) {
          // A[row + v][col] = A[col][row + v]: A is exactly symmetric
          const f32x4 av = Vec4<T>::ld(prev + col * mp + row);
#pragma unroll
          for (int v = 0; v < 4; ++v) val[v] = fmaf(s.b, av[v], s.c * val[v]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) WsType<T>::st(out, (row + v) * mp + col, val[v]);
        if (ti != tj) Vec4<T>::st(out + col * mp + row, val);
      }
  } else if (MODE == kModeApply) {
    const T *XT = static_cast<const T *>(d.xt[cur]);
    T *Xn = static_cast<T *>(d.x[cur ^ 1]);
    T *XTn = static_cast<T *>(d.xt[cur ^ 1]);
    const int64_t np = d.np, mp = d.mp;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int64_t col = col_base + j * 16, row = row_base + i * 16;
        const f32x4 xv = Vec4<T>::ld(XT + col * mp + row);  // X[row + v][col]
        f32x4 val;
#pragma unroll
        for (int v = 0; v < 4; ++v) val[v] = fmaf(s.a, xv[v], acc[i][j][v]);
        Vec4<T>::st(XTn + col * mp + row, val);
#pragma unroll
        for (int v = 0; v < 4; ++v) WsType<T>::st(Xn, (row + v) * np + col, val[v]);
      }
  } else {  // kModeFinal
    const T *XT = static_cast<const T *>(d.xt[cur]);
    const int64_t mp = d.mp;
    const float step = s.lr * d.scale;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int64_t col = col_base + j * 16, row = row_base + i * 16;
        if (row >= d.m || col >= d.n) continue;
        const f32x4 xv = Vec4<T>::ld(XT + col * mp + row);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (row + v >= d.m) break;
          const float o = fmaf(s.a, xv[v], acc[i][j][v]);
          const int64_t pidx = d.transposed ? col * d.cols + row + v : (row + v) * d.cols + col;
          if (d.orth) store_elem(d.orth, d.param_dt, pidx, o);
          store_elem(d.param, d.param_dt, pidx,
                     fmaf(-step, o, load_elem(d.param, d.param_dt, pidx)));
        }
      }
  }
}

template <typename T>
hipError_t launch_t(GemmMode mode, const MatDev *mats, const StageEntry *stage, int32_t nstage,
                    int64_t total, int32_t cur, StepScalars s, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>(total)), block(kThreads);
  switch (mode) {
    case kModeGram:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeGram>), grid, block, 0, st, mats, stage, nstage, cur, s);
      break;
    case kModeSquare:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeSquare>), grid, block, 0, st, mats, stage, nstage, cur, s);
      break;
    case kModeApply:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeApply>), grid, block, 0, st, mats, stage, nstage, cur, s);
      break;
    default:
      hipLaunchKernelGGL((ns_gemm_kernel<T, kModeFinal>), grid, block, 0, st, mats, stage, nstage, cur, s);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_stage(GemmMode mode, bool fp32, const MatDev *mats, const StageEntry *stage,
                           int32_t nstage, int64_t total_tiles, int32_t cur, StepScalars s,
                           hipStream_t st) {
  if (total_tiles == 0) return hipSuccess;
  return fp32 ? launch_t<float>(mode, mats, stage, nstage, total_tiles, cur, s, st)
              : launch_t<uint16_t>(mode, mats, stage, nstage, total_tiles, cur, s, st);
}

}  // namespace dmuon
