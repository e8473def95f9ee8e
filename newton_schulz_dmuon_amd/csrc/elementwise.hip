// Memory-bound stages of the owner's Muon step on gfx950: momentum + sum of
// squares fused with the cast to the wide orientation (stored as X^T), the norm,
// the direct update (ns_steps = 0, with a flat momentum pass) and the
// packed-buffer copies.
//
// Every kernel here moves each byte once; they are bound by HBM bandwidth.
// Loads and stores are 16-byte vectors where the layout allows, consecutive
// lanes touch consecutive addresses, and the reductions run in a fixed order
// in fp64 so the result does not depend on scheduling.

#include "device_common.h"

namespace dmuon {

namespace {

constexpr int kEwThreads = 256;
constexpr int kOrientThreads = 1024;  // 8192 elements per group, eight per thread
constexpr int kEwPerThread = static_cast<int>(kEwChunk / kEwThreads);  // 32
static_assert(kEwPerThread % 4 == 0, "4-wide vectors");

__device__ __forceinline__ double block_sum_f64(double v, double *lds) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0)
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += lds[w];
  return s;  // valid in thread 0
}

typedef unsigned int vu32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) vu32x2 g_u32x2;
typedef unsigned int vu32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) vu32x4 g_u32x4;
typedef __attribute__((address_space(1))) double g_f64;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;

// Four consecutive bf16 or fp32 values at flat index i (i multiple of 4).
__device__ __forceinline__ f32x4 load_grad4(const void *g, int32_t dt, int64_t i) {
  f32x4 r;
  if (dt == kBF16) {
    const vu32x2 v = *(const g_u32x2 *)(static_cast<const uint16_t *>(g) + i);
    r[0] = __uint_as_float(v.x << 16);
    r[1] = __uint_as_float(v.x & 0xffff0000u);
    r[2] = __uint_as_float(v.y << 16);
    r[3] = __uint_as_float(v.y & 0xffff0000u);
  } else {
    r = *(const g_f32x4 *)(static_cast<const float *>(g) + i);
  }
  return r;
}

// M <- mu*M + G over one chunk; partial sum of U^2, U = M or G + mu*M.
__global__ __launch_bounds__(kEwThreads) void momentum_sumsq_kernel(
    const MatDev *__restrict__ mats, int32_t nmat, StepScalars s) {
  __shared__ double red[kEwThreads / 64];
  const int64_t w = blockIdx.x;
  const int32_t mi = find_range(nmat, w, [&](int32_t i) { return mats[i].ew_first; });
  const MatDev &d = mats[mi];
  const int64_t numel = d.rows * d.cols;
  const int64_t base = (w - d.ew_first) * kEwChunk;
  const float mu = s.mu;
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < kEwPerThread / 4; ++k) {
    const int64_t i = base + (static_cast<int64_t>(k) * kEwThreads + threadIdx.x) * 4;
    if (i + 4 <= numel) {
      f32x4 mv = *(const g_f32x4 *)(d.mom + i);
      const f32x4 g = load_grad4(d.grad, d.grad_dt, i);
      mv.x = fmaf(mu, mv.x, g[0]);
      mv.y = fmaf(mu, mv.y, g[1]);
      mv.z = fmaf(mu, mv.z, g[2]);
      mv.w = fmaf(mu, mv.w, g[3]);
      *(g_f32x4 *)(d.mom + i) = mv;
      float u0 = mv.x, u1 = mv.y, u2 = mv.z, u3 = mv.w;
      if (s.nesterov) {
        u0 = fmaf(mu, mv.x, g[0]); u1 = fmaf(mu, mv.y, g[1]);
        u2 = fmaf(mu, mv.z, g[2]); u3 = fmaf(mu, mv.w, g[3]);
      }
      acc += (double)u0 * u0 + (double)u1 * u1 + (double)u2 * u2 + (double)u3 * u3;
    } else {
      g_f32 *const mom = (g_f32 *)d.mom;
      for (int64_t j = i; j < numel && j < i + 4; ++j) {
        const float g = load_elem(d.grad, d.grad_dt, j);
        const float m = fmaf(mu, mom[j], g);
        mom[j] = m;
        const float u = s.nesterov ? fmaf(mu, m, g) : m;
        acc += (double)u * u;
      }
    }
  }
  const double tot = block_sum_f64(acc, red);
  if (threadIdx.x == 0) ((g_f64 *)d.partials)[w - d.ew_first] = tot;
}

// inv_norm = 1 / (sqrt(sum of the partials, in index order per thread) + eps)
__global__ __launch_bounds__(256) void finalize_norm_kernel(const MatDev *__restrict__ mats,
                                                            float eps) {
  __shared__ double red[4];
  const MatDev &d = mats[blockIdx.x];
  double acc = 0.0;
  for (int32_t i = threadIdx.x; i < d.part_count; i += 256) acc += ((const g_f64 *)d.partials)[i];
  const double tot = block_sum_f64(acc, red);
  if (threadIdx.x == 0) {
    *(g_f32 *)d.inv_norm = static_cast<float>(1.0 / (sqrt(tot) + (double)eps));
    // the squares are summed in fp64, where no finite fp32 U overflows: a
    // non-finite sum means a NaN or an Inf in U
    if (d.nonfinite) *(__attribute__((address_space(1))) int32_t *)d.nonfinite = __builtin_isfinite(tot) ? 0 : 1;
  }
}

// Fused momentum + sum of squares + wide orientation:
//   M <- mu*M + G on the caller's elements that map onto the group's block,
//   U = M (or G + mu*M), its sum of squares into partials[group],
//   U written unnormalised as X^T (n_p x m_p), zero in the padding.
// A tall matrix is its own X^T: group t takes its contiguous elements
// [8192 t, 8192 t + 8192) (long row runs keep HBM pages open).  Otherwise
// X^T = U^T and group t takes a 64 x 128 block of U, transposed through LDS,
// so that M is read in 512-byte and X^T written in 128-byte row segments.
// Every thread takes eight consecutive elements: M as two 16-byte vectors,
// a bf16 G and a bf16 X^T segment as one.  The 1/(||U||_F + eps) scale is
// applied by the first iteration's Gram and Apply epilogues, so M is read
// once.
struct MomPiece {
  int64_t ur, uc;
  bool full;  // eight valid elements with 16-byte aligned M: vector path
  f32x4 m[2];
  f32x4 g[2];
};

// Eight consecutive bf16 or fp32 values at flat index i (i multiple of 4;
// one 16-byte bf16 load when i is a multiple of 8).
__device__ __forceinline__ void load_grad8(const void *g, int32_t dt, int64_t i, f32x4 (&r)[2]) {
  if (dt == kBF16 && (i & 7) == 0) {
    const vu32x4 v = *(const g_u32x4 *)(static_cast<const uint16_t *>(g) + i);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r[h][0] = __uint_as_float(v[2 * h] << 16);
      r[h][1] = __uint_as_float(v[2 * h] & 0xffff0000u);
      r[h][2] = __uint_as_float(v[2 * h + 1] << 16);
      r[h][3] = __uint_as_float(v[2 * h + 1] & 0xffff0000u);
    }
  } else {
    r[0] = load_grad4(g, dt, i);
    r[1] = load_grad4(g, dt, i + 4);
  }
}

__device__ __forceinline__ MomPiece mom_load(const MatDev &d, int64_t ur, int64_t uc, bool vec) {
  MomPiece pc;
  pc.ur = ur;
  pc.uc = uc;
  pc.full = vec && ur < d.rows && uc + 8 <= d.cols;
  if (pc.full) {
    const int64_t idx = ur * d.cols + uc;
    pc.m[0] = *(const g_f32x4 *)(d.mom + idx);
    pc.m[1] = *(const g_f32x4 *)(d.mom + idx + 4);
    load_grad8(d.grad, d.grad_dt, idx, pc.g);
  }
  return pc;
}

__device__ __forceinline__ void momentum8(const MatDev &d, const MomPiece &pc, float mu, bool nesterov,
                                          float (&u)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) u[k] = 0.f;
  if (pc.ur >= d.rows || pc.uc >= d.cols) return;
  const int64_t idx = pc.ur * d.cols + pc.uc;
  if (pc.full) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 mv = pc.m[h];
      const f32x4 g = pc.g[h];
#pragma unroll
      for (int k = 0; k < 4; ++k) mv[k] = fmaf(mu, mv[k], g[k]);
      *(g_f32x4 *)(d.mom + idx + 4 * h) = mv;
#pragma unroll
      for (int k = 0; k < 4; ++k) u[4 * h + k] = nesterov ? fmaf(mu, mv[k], g[k]) : mv[k];
    }
  } else {
    g_f32 *const mom = (g_f32 *)d.mom;
    for (int k = 0; k < 8 && pc.uc + k < d.cols; ++k) {
      const float g = load_elem(d.grad, d.grad_dt, idx + k);
      const float m = fmaf(mu, mom[idx + k], g);
      mom[idx + k] = m;
      u[k] = nesterov ? fmaf(mu, m, g) : m;
    }
  }
}

// Eight consecutive elements of X^T in the matrix's workspace type: one
// 16-byte bf16 store, or two fp32 ones (the fp32 mode, and small matrices in
// a bf16 step).  idx is a multiple of 8.
__device__ __forceinline__ void store_xt8(const MatDev &d, int64_t idx, const float (&u)[8]) {
  if (d.ws_f32) {
    float *const p = static_cast<float *>(d.xt[0]) + idx;
    *(g_f32x4 *)p = f32x4{u[0], u[1], u[2], u[3]};
    *(g_f32x4 *)(p + 4) = f32x4{u[4], u[5], u[6], u[7]};
  } else {
    vu32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = f32_to_bf16_bits(u[2 * k]) | (static_cast<uint32_t>(f32_to_bf16_bits(u[2 * k + 1])) << 16);
    *(g_u32x4 *)(static_cast<uint16_t *>(d.xt[0]) + idx) = v;
  }
}

// The transpose tile: U[i0 + r][j0 + c] at LDS word r * kTrStride + c +
// 4 * (c / 64).  A row write (16 lanes per row, eight columns each, four
// rows per instruction) and a column read (eight lanes per column, eight
// rows each) then touch 64 distinct banks: the stride is 1 mod 8, and the
// four-word gap shifts the columns 64-127 of a row by half a bank octet.
constexpr int kTrStride = 137;
__device__ __forceinline__ int tr_pos(int r, int c) { return r * kTrStride + c + ((c >> 6) << 2); }

__global__ __launch_bounds__(kOrientThreads) void momentum_orient_kernel(
    const MatDev *__restrict__ mats, int32_t nmat, StepScalars s) {
  constexpr int TT = static_cast<int>(kTrTile);
  static_assert(2 * TT * TT == kOrientThreads * 8, "eight elements per thread and group");
  __shared__ float tile[TT * kTrStride];
  __shared__ double red[kOrientThreads / 64];
  const int64_t w = blockIdx.x;
  const int32_t mi = find_range(nmat, w, [&](int32_t i) { return mats[i].tr_first; });
  const MatDev &d = mats[mi];
  const int64_t t = w - d.tr_first;
  const float mu = s.mu;
  const int tid = threadIdx.x;
  const bool vec = (d.cols & 3) == 0;  // rows of M start 16-byte aligned
  double acc = 0.0;
  float u[8];
  if (d.transposed) {
    // 8192 contiguous elements of X^T per group, eight per thread (a run
    // of eight lies within one row: m_p is a multiple of 256)
    const int64_t e0 = t * (2 * TT * TT) + 8 * tid;
    const MomPiece pc = mom_load(d, e0 / d.mp, e0 % d.mp, vec);
    momentum8(d, pc, mu, s.nesterov, u);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (double)u[k] * u[k];
    store_xt8(d, e0, u);  // X^T[ur][uc .. uc+7], zeros in the padding
  } else {
    // block rows i0 .. i0+63 (m), columns j0 .. j0+127 (n); thread: row p,
    // columns q .. q+7
    const int64_t blocks_n = d.np / (2 * TT);
    const int64_t i0 = (t / blocks_n) * TT, j0 = (t % blocks_n) * (2 * TT);
    const int p = tid >> 4, q = (tid & 15) * 8;
    const MomPiece pc = mom_load(d, i0 + p, j0 + q, vec);
    momentum8(d, pc, mu, s.nesterov, u);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      tile[tr_pos(p, q) + k] = u[k];
      acc += (double)u[k] * u[k];
    }
    __syncthreads();
    // X^T row j0 + a (a < 128), elements i0 + b .. b+7
    const int a = tid >> 3, b = (tid & 7) * 8;
    float vt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) vt[k] = tile[tr_pos(b + k, a)];
    store_xt8(d, (j0 + a) * d.mp + i0 + b, vt);
  }
  const double tot = block_sum_f64(acc, red);
  if (tid == 0) ((g_f64 *)d.partials)[t] = tot;
}

// ns_steps = 0: O = U * inv_norm (already r x c), P -= lr*scale*O.
__global__ __launch_bounds__(kEwThreads) void update_direct_kernel(
    const MatDev *__restrict__ mats, int32_t nmat, StepScalars s) {
  const int64_t w = blockIdx.x;
  const int32_t mi = find_range(nmat, w, [&](int32_t i) { return mats[i].ew_first; });
  const MatDev &d = mats[mi];
  const int64_t numel = d.rows * d.cols;
  const int64_t base = (w - d.ew_first) * kEwChunk;
  const float inv = *(const g_f32 *)d.inv_norm;
  const float step = s.lr * d.scale;
  for (int k = 0; k < kEwPerThread; ++k) {
    const int64_t i = base + static_cast<int64_t>(k) * kEwThreads + threadIdx.x;
    if (i >= numel) break;
    float u = ((const g_f32 *)d.mom)[i];
    if (s.nesterov) u = fmaf(s.mu, u, load_elem(d.grad, d.grad_dt, i));
    const float o = u * inv;
    if (d.orth) store_elem(d.orth, d.param_dt, i, o);
    const float nv = fmaf(-step, o, load_elem(d.param, d.param_dt, i));
    store_elem(d.param, d.param_dt, i, nv);
    if (d.packed) store_elem(d.packed, d.param_dt, i, nv);
  }
}

// AdamW over a batch of tensors: one 4-wide vector per thread where the
// tensor's length allows.  Short work-groups (1024 elements) keep more HBM
// requests in flight than longer ones with 16-byte bf16 pieces (2048 and
// 4096 elements per group measured 3-5% slower).
__device__ __forceinline__ void adamw_elem(float &p, float g, float &m, float &v,
                                           const AdamScalars &s) {
  p *= s.decay;
  m = fmaf(s.beta1, m, (1.f - s.beta1) * g);
  v = fmaf(s.beta2, v, (1.f - s.beta2) * g * g);
  const float denom = fmaf(sqrtf(v), s.inv_sqrt_bc2, s.eps);
  p = fmaf(-s.step_size, m / denom, p);
}

__global__ __launch_bounds__(kEwThreads) void adamw_kernel(AdamBatch b, AdamScalars s) {
  const int64_t w = blockIdx.x;
  const int32_t ti = find_range(b.n, w, [&](int32_t i) { return b.first_block[i]; });
  const int64_t numel = b.numel[ti];
  const int64_t base = (w - b.first_block[ti]) * kAdamChunk;
  float *M = b.m[ti], *V = b.v[ti];
  void *P = b.param[ti];
  const void *G = b.grad[ti];
  const int32_t pdt = b.param_dt[ti], gdt = b.grad_dt[ti];
  static_assert(kAdamChunk % (4 * kEwThreads) == 0, "whole vectors per thread");
#pragma unroll
  for (int k = 0; k < static_cast<int>(kAdamChunk / (4 * kEwThreads)); ++k) {
    const int64_t i = base + (static_cast<int64_t>(k) * kEwThreads + threadIdx.x) * 4;
    if (i + 4 <= numel) {
      f32x4 mv = *(const g_f32x4 *)(M + i);
      f32x4 vv = *(const g_f32x4 *)(V + i);
      const f32x4 g = load_grad4(G, gdt, i);
      const f32x4 pv = load_grad4(P, pdt, i);
      float p[4] = {pv[0], pv[1], pv[2], pv[3]};
      { float m0 = mv.x, v0 = vv.x; adamw_elem(p[0], g[0], m0, v0, s); mv.x = m0; vv.x = v0; }
      { float m1 = mv.y, v1 = vv.y; adamw_elem(p[1], g[1], m1, v1, s); mv.y = m1; vv.y = v1; }
      { float m2 = mv.z, v2 = vv.z; adamw_elem(p[2], g[2], m2, v2, s); mv.z = m2; vv.z = v2; }
      { float m3 = mv.w, v3 = vv.w; adamw_elem(p[3], g[3], m3, v3, s); mv.w = m3; vv.w = v3; }
      *(g_f32x4 *)(M + i) = mv;
      *(g_f32x4 *)(V + i) = vv;
      if (pdt == kBF16) {
        vu32x2 u;
        u.x = f32_to_bf16_bits(p[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(p[1])) << 16);
        u.y = f32_to_bf16_bits(p[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(p[3])) << 16);
        *(g_u32x2 *)(static_cast<uint16_t *>(P) + i) = u;
      } else {
        *(g_f32x4 *)(static_cast<float *>(P) + i) = f32x4{p[0], p[1], p[2], p[3]};
      }
    } else {
      g_f32 *const Mg = (g_f32 *)M;
      g_f32 *const Vg = (g_f32 *)V;
      for (int64_t j = i; j < numel && j < i + 4; ++j) {
        float p = load_elem(P, pdt, j);
        float m = Mg[j], v = Vg[j];
        adamw_elem(p, load_elem(G, gdt, j), m, v, s);
        Mg[j] = m;
        Vg[j] = v;
        store_elem(P, pdt, j, p);
      }
    }
  }
}

// Zeroes n int32 (the chained mode's tickets and counters): a kernel, so
// that a captured step records no memset node.
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t *__restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) ((__attribute__((address_space(1))) int32_t *)p)[i] = 0;
}

constexpr int kPackThreads = 256;

// Byte copies of a batch of matrices; 16-byte vectors for the body, bytes
// for a tail shorter than 16.  Base pointers are 16-byte aligned.
__global__ __launch_bounds__(kPackThreads) void pack_copy_kernel(PackBatch b) {
  const int64_t w = blockIdx.x;
  const int32_t ci = find_range(b.n, w, [&](int32_t i) { return b.first_block[i]; });
  const int64_t begin = (w - b.first_block[ci]) * kPackBlockBytes;
  const int64_t end = min(begin + kPackBlockBytes, b.bytes[ci]);
  const char *src = static_cast<const char *>(b.src[ci]);
  char *dst = static_cast<char *>(b.dst[ci]);
  const int64_t vend = begin + ((end - begin) & ~static_cast<int64_t>(15));
  for (int64_t o = begin + static_cast<int64_t>(threadIdx.x) * 16; o < vend;
       o += kPackThreads * 16)
    *reinterpret_cast<uint4 *>(dst + o) = *reinterpret_cast<const uint4 *>(src + o);
  for (int64_t o = vend + threadIdx.x; o < end; o += kPackThreads) dst[o] = src[o];
}

}  // namespace

hipError_t launch_momentum_sumsq(const MatDev *mats, int32_t nmat, int64_t total_chunks,
                                 StepScalars s, hipStream_t st) {
  hipLaunchKernelGGL(momentum_sumsq_kernel, dim3((uint32_t)total_chunks), dim3(kEwThreads), 0,
                     st, mats, nmat, s);
  return hipGetLastError();
}

hipError_t launch_finalize_norm(const MatDev *mats, int32_t nmat, float eps, hipStream_t st) {
  hipLaunchKernelGGL(finalize_norm_kernel, dim3((uint32_t)nmat), dim3(256), 0, st, mats, eps);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_momentum_orient(const MatDev *mats, int32_t nmat, int64_t total_tiles,
                                  StepScalars s, hipStream_t st) {
  hipLaunchKernelGGL(momentum_orient_kernel, dim3((uint32_t)total_tiles), dim3(kOrientThreads), 0,
                     st, mats, nmat, s);
  return hipGetLastError();
}

hipError_t launch_update_direct(const MatDev *mats, int32_t nmat, int64_t total_chunks,
                                StepScalars s, hipStream_t st) {
  hipLaunchKernelGGL(update_direct_kernel, dim3((uint32_t)total_chunks), dim3(kEwThreads), 0,
                     st, mats, nmat, s);
  return hipGetLastError();
}

hipError_t launch_adamw_batch(const AdamBatch &b, AdamScalars s, hipStream_t st) {
  if (b.n == 0) return hipSuccess;
  hipLaunchKernelGGL(adamw_kernel, dim3((uint32_t)b.first_block[b.n]), dim3(kEwThreads), 0, st, b, s);
  return hipGetLastError();
}

hipError_t launch_pack_batch(const PackBatch &b, hipStream_t st) {
  if (b.n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_copy_kernel, dim3((uint32_t)b.first_block[b.n]), dim3(kPackThreads),
                     0, st, b);
  return hipGetLastError();
}

}  // namespace dmuon
