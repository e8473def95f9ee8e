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
// 32 fp32).  Tiles are staged global -> registers -> LDS, double buffered
// (2 x 64 KB); the next K step's global loads are in flight while the
// current one runs on the matrix cores.  LDS rows are 128 bytes; the 16-byte
// chunk index is XOR-swizzled with the row so the fragment reads of 16
// consecutive rows spread over the banks.
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
constexpr int kLoadRounds = kOperandBytes / (kThreads * 16);  // 4

__device__ __forceinline__ int swz(int chunk, int row) { return chunk ^ (row & 7); }

template <typename T> struct Mfma;
template <> struct Mfma<uint16_t> {
  // one 16-byte chunk per lane = 8 bf16 along k = one 16x16x32 MFMA
  static __device__ __forceinline__ void run(f32x4 &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // one 16-byte chunk per lane = 4 fp32 along k = four 16x16x4 MFMAs
  static __device__ __forceinline__ void run(f32x4 &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
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
  __shared__ __attribute__((aligned(16))) char smem[4 * kOperandBytes];  // 128 KB
  char *lds_l = smem;                      // [2][256][128 B]
  char *lds_r = smem + 2 * kOperandBytes;  // [2][256][128 B]

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
  const int lrow = tid >> 3, lch = tid & 7;  // global -> LDS copy position
  uint4 rl[kLoadRounds], rr[kLoadRounds];

  auto load_regs = [&](int kt) {
#pragma unroll
    for (int q = 0; q < kLoadRounds; ++q) {
      const int64_t off = static_cast<int64_t>(q * 64 + lrow) * ld_bytes +
                          static_cast<int64_t>(kt) * kRowBytes + lch * 16;
      rl[q] = *reinterpret_cast<const uint4 *>(gl + off);
      rr[q] = *reinterpret_cast<const uint4 *>(gr + off);
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kLoadRounds; ++q) {
      const int row = q * 64 + lrow;
      const int off = buf * kOperandBytes + row * kRowBytes + swz(lch, row) * 16;
      *reinterpret_cast<uint4 *>(lds_l + off) = rl[q];
      *reinterpret_cast<uint4 *>(lds_r + off) = rr[q];
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int r16 = lane & 15, g4 = lane >> 4;

  f32x4 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_regs(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_regs(kt + 1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int chunk = sub * 4 + g4;
      uint4 fl[kFragM], fr[kFragN];
#pragma unroll
      for (int i = 0; i < kFragM; ++i) {
        const int row = wm * kWaveM + i * 16 + r16;
        fl[i] = *reinterpret_cast<const uint4 *>(lds_l + buf * kOperandBytes + row * kRowBytes +
                                                 swz(chunk, row) * 16);
      }
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int row = wn * kWaveN + j * 16 + r16;
        fr[j] = *reinterpret_cast<const uint4 *>(lds_r + buf * kOperandBytes + row * kRowBytes +
                                                 swz(chunk, row) * 16);
      }
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) Mfma<T>::run(acc[i][j], fl[i], fr[j]);
    }
    if (kt + 1 < nkt) store_lds(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[row0 + 4*g4 + v][col0 + r16], v = 0..3 ----
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
        const int64_t col = col_base + j * 16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = row_base + i * 16 + v;
          float val = acc[i][j][v];
          if (MODE == kModeSquare) val = fmaf(s.b, WsType<T>::ld(prev, row * mp + col), s.c * val);
          WsType<T>::st(out, row * mp + col, val);
          if (ti != tj) WsType<T>::st(out, col * mp + row, val);
        }
      }
  } else if (MODE == kModeApply) {
    const T *X = static_cast<const T *>(d.x[cur]);
    T *Xn = static_cast<T *>(d.x[cur ^ 1]);
    T *XTn = static_cast<T *>(d.xt[cur ^ 1]);
    const int64_t np = d.np, mp = d.mp;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int64_t col = col_base + j * 16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = row_base + i * 16 + v;
          const float val = fmaf(s.a, WsType<T>::ld(X, row * np + col), acc[i][j][v]);
          WsType<T>::st(Xn, row * np + col, val);
          WsType<T>::st(XTn, col * mp + row, val);
        }
      }
  } else {  // kModeFinal
    const T *X = static_cast<const T *>(d.x[cur]);
    const int64_t np = d.np;
    const float step = s.lr * d.scale;
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int64_t col = col_base + j * 16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = row_base + i * 16 + v;
          if (row < d.m && col < d.n) {
            const float o = fmaf(s.a, WsType<T>::ld(X, row * np + col), acc[i][j][v]);
            const int64_t pidx = d.transposed ? col * d.cols + row : row * d.cols + col;
            if (d.orth) store_elem(d.orth, d.param_dt, pidx, o);
            store_elem(d.param, d.param_dt, pidx,
                       fmaf(-step, o, load_elem(d.param, d.param_dt, pidx)));
          }
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
