// HBM-bound phases of the MuonH step on gfx950: the init norm, the momentum
// update with its norm, the bf16/fp32 cast of the normalised momentum into
// both Newton-Schulz layouts, the trial update with its norm, and the
// projection back onto the sphere. Every kernel is one grouped launch over all
// matrices of all shape groups; blocks stream contiguous chunks with 16-byte
// accesses. Norms are deterministic two-level reductions: fp32 per thread, a
// fixed shuffle tree in fp64 per block, then a fixed-order fp64 sum of the
// per-block partials in a separate finalize kernel (no float atomics).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muonh_internal.h"

namespace muonh {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int group_of_block(const EwArgs& a, int b) {
  int gi = 0;
  for (int i = 1; i < a.ngroups; ++i)
    if (b >= a.g[i].block_begin) gi = i;
  return gi;
}

// Fixed-order block sum; the result is valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) t = (red[0] + red[1]) + (red[2] + red[3]);
  return t;
}

// Element range [lo, hi) of chunk `c` out of `bpm`, with lo a multiple of 4.
__device__ __forceinline__ void chunk_range(int64_t n, int bpm, int c, int64_t& lo, int64_t& hi) {
  int64_t len = (n + bpm - 1) / bpm;
  len = (len + 3) & ~int64_t(3);
  lo = (int64_t)c * len;
  hi = lo + len < n ? lo + len : n;
  if (lo > n) lo = n;
}

__device__ __forceinline__ bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// --------------------------------------------------------------------------
// init: partial sums of squares of W
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_sumsq(EwArgs a, float* const* W, double* partials) {
  __shared__ double red[4];
  const int gi = group_of_block(a, blockIdx.x);
  const EwGroup& g = a.g[gi];
  const int local = blockIdx.x - g.block_begin;
  const int m = local / g.bpm, c = local - m * g.bpm;
  const int mat = g.first + m;
  const float* w = W[mat];
  int64_t lo, hi;
  chunk_range(g.n, g.bpm, c, lo, hi);
  float acc = 0.f;
  int64_t mid = lo;
  if (aligned16(w)) {
    const int64_t n4 = (hi - lo) >> 2;
    const float4* w4 = reinterpret_cast<const float4*>(w + lo);
    for (int64_t i = threadIdx.x; i < n4; i += kThreads) {
      const float4 v = w4[i];
      acc = fmaf(v.x, v.x, acc);
      acc = fmaf(v.y, v.y, acc);
      acc = fmaf(v.z, v.z, acc);
      acc = fmaf(v.w, v.w, acc);
    }
    mid = lo + (n4 << 2);
  }
  for (int64_t e = mid + threadIdx.x; e < hi; e += kThreads) acc = fmaf(w[e], w[e], acc);
  const double t = block_sum((double)acc, red);
  if (threadIdx.x == 0) partials[(int64_t)mat * kMaxPartials + c] = t;
}

// --------------------------------------------------------------------------
// M <- beta*M + G, with partial sums of squares of the new M
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_momentum(EwArgs a, const float* const* G,
                                                       float* const* M, float beta,
                                                       double* partials) {
  __shared__ double red[4];
  const int gi = group_of_block(a, blockIdx.x);
  const EwGroup& g = a.g[gi];
  const int local = blockIdx.x - g.block_begin;
  const int m = local / g.bpm, c = local - m * g.bpm;
  const int mat = g.first + m;
  const float* gp = G[mat];
  float* mp = M[mat];
  int64_t lo, hi;
  chunk_range(g.n, g.bpm, c, lo, hi);
  float acc = 0.f;
  int64_t mid = lo;
  if (aligned16(gp) && aligned16(mp)) {
    const int64_t n4 = (hi - lo) >> 2;
    const float4* g4 = reinterpret_cast<const float4*>(gp + lo);
    float4* m4 = reinterpret_cast<float4*>(mp + lo);
    for (int64_t i = threadIdx.x; i < n4; i += kThreads) {
      const float4 gv = g4[i];
      float4 mv = m4[i];
      mv.x = fmaf(beta, mv.x, gv.x);
      mv.y = fmaf(beta, mv.y, gv.y);
      mv.z = fmaf(beta, mv.z, gv.z);
      mv.w = fmaf(beta, mv.w, gv.w);
      m4[i] = mv;
      acc = fmaf(mv.x, mv.x, acc);
      acc = fmaf(mv.y, mv.y, acc);
      acc = fmaf(mv.z, mv.z, acc);
      acc = fmaf(mv.w, mv.w, acc);
    }
    mid = lo + (n4 << 2);
  }
  for (int64_t e = mid + threadIdx.x; e < hi; e += kThreads) {
    const float v = fmaf(beta, mp[e], gp[e]);
    mp[e] = v;
    acc = fmaf(v, v, acc);
  }
  const double t = block_sum((double)acc, red);
  if (threadIdx.x == 0) partials[(int64_t)mat * kMaxPartials + c] = t;
}

// --------------------------------------------------------------------------
// norms[mat] = sqrt(sum_c partials[mat][c]) in a fixed order
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_finalize(EwArgs a, const double* partials,
                                                       double* norms, float* R) {
  const int first = a.g[0].first;
  const int last = a.g[a.ngroups - 1].first + a.g[a.ngroups - 1].count;
  const int64_t mat = (int64_t)first + (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (mat >= last) return;
  int gi = 0;
  for (int i = 1; i < a.ngroups; ++i)
    if (mat >= a.g[i].first) gi = i;
  const int bpm = a.g[gi].bpm;
  const double* p = partials + mat * kMaxPartials;
  double s = 0.0;
  for (int c = 0; c < bpm; ++c) s += p[c];
  const double nrm = sqrt(s);
  norms[mat] = nrm;
  if (R) R[mat] = (float)nrm;
}

// --------------------------------------------------------------------------
// X0 = M / (||M|| + eps): one 64x64 tile of the padded rp x cp domain per
// block; written straight to D and transposed (through LDS) to E. Entries
// outside rows x cols are written as zero.
// --------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T to_ns(float v);
template <>
__device__ __forceinline__ float to_ns<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 to_ns<__bf16>(float v) { return (__bf16)v; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_normcast(EwArgs a, const float* const* M,
                                                       const double* norms) {
  __shared__ float tile[64][65];
  const int gi = group_of_block(a, blockIdx.x);
  const EwGroup& g = a.g[gi];
  const int local = blockIdx.x - g.block_begin;
  const int m = local / g.tiles_per_mat, t = local - m * g.tiles_per_mat;
  const int mat = g.first + m;
  const int tcols = g.cp >> 6;
  const int r0 = (t / tcols) << 6, c0 = (t - (t / tcols) * tcols) << 6;
  const float scale = (float)(1.0 / (norms[mat] + kNsEps));
  const float* mp = M[mat];
  char* blk = g.ns_base + (int64_t)m * g.mat_bytes;
  T* D = reinterpret_cast<T*>(blk + g.offD);
  T* E = reinterpret_cast<T*>(blk + g.offE);
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int rr = i * 4 + ty;
    const int r = r0 + rr, c = c0 + tx;
    float v = 0.f;
    if (r < g.rows && c < g.cols) v = mp[(int64_t)r * g.cols + c] * scale;
    tile[rr][tx] = v;
    D[(int64_t)r * g.cp + c] = to_ns<T>(v);
  }
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int cc = i * 4 + ty;
    E[(int64_t)(c0 + cc) * g.rp + r0 + tx] = to_ns<T>(tile[tx][cc]);
  }
}

// --------------------------------------------------------------------------
// Trial update W' = W - lr*O (O read from D) and partial sums of squares of
// W'; the projection recomputes W' identically and rescales it.
// --------------------------------------------------------------------------
template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  __device__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <>
struct Vec4<__bf16> {
  __device__ static float4 load(const __bf16* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    float4 r;
    r.x = __uint_as_float(u.x << 16);
    r.y = __uint_as_float(u.x & 0xffff0000u);
    r.z = __uint_as_float(u.y << 16);
    r.w = __uint_as_float(u.y & 0xffff0000u);
    return r;
  }
};
__device__ __forceinline__ float ns_to_f(float v) { return v; }
__device__ __forceinline__ float ns_to_f(__bf16 v) { return (float)v; }

template <typename T, bool kProject>
__global__ __launch_bounds__(kThreads) void k_update(EwArgs a, float* const* W, float lr,
                                                     double* partials, const float* R,
                                                     const double* norms) {
  __shared__ double red[4];
  const int gi = group_of_block(a, blockIdx.x);
  const EwGroup& g = a.g[gi];
  const int local = blockIdx.x - g.block_begin;
  const int m = local / g.bpm, c = local - m * g.bpm;
  const int mat = g.first + m;
  float* w = W[mat];
  const T* D = reinterpret_cast<const T*>(g.ns_base + (int64_t)m * g.mat_bytes + g.offD);
  int64_t lo, hi;
  chunk_range(g.n, g.bpm, c, lo, hi);
  const float nlr = -lr;
  float scale = 1.f;
  if (kProject) {
    const double nrm = norms[mat];
    scale = nrm > 0.0 ? (float)((double)R[mat] / nrm) : 1.f;
  }
  float acc = 0.f;
  const int cols = g.cols;
  if ((cols & 3) == 0 && aligned16(w)) {
    // 4 consecutive elements share a row; walk (row, col) incrementally.
    const int64_t e0 = lo + 4 * (int64_t)threadIdx.x;
    int64_t r = e0 / cols;
    int col = (int)(e0 - r * cols);
    const int step = 4 * kThreads;
    const int dr = step / cols, dc = step - (step / cols) * cols;
    for (int64_t e = e0; e < hi; e += step) {
      float4 wv = *reinterpret_cast<const float4*>(w + e);
      const float4 ov = Vec4<T>::load(D + r * g.cp + col);
      wv.x = fmaf(nlr, ov.x, wv.x);
      wv.y = fmaf(nlr, ov.y, wv.y);
      wv.z = fmaf(nlr, ov.z, wv.z);
      wv.w = fmaf(nlr, ov.w, wv.w);
      if (kProject) {
        wv.x *= scale; wv.y *= scale; wv.z *= scale; wv.w *= scale;
        *reinterpret_cast<float4*>(w + e) = wv;
      } else {
        acc = fmaf(wv.x, wv.x, acc);
        acc = fmaf(wv.y, wv.y, acc);
        acc = fmaf(wv.z, wv.z, acc);
        acc = fmaf(wv.w, wv.w, acc);
      }
      col += dc;
      r += dr;
      if (col >= cols) { col -= cols; ++r; }
    }
  } else {
    for (int64_t e = lo + threadIdx.x; e < hi; e += kThreads) {
      const int64_t r = e / cols;
      const int col = (int)(e - r * cols);
      float v = fmaf(nlr, ns_to_f(D[r * g.cp + col]), w[e]);
      if (kProject) {
        w[e] = v * scale;
      } else {
        acc = fmaf(v, v, acc);
      }
    }
  }
  if (!kProject) {
    const double t = block_sum((double)acc, red);
    if (threadIdx.x == 0) partials[(int64_t)mat * kMaxPartials + c] = t;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_read_update(const T* D, int ldD, int rows, int cols,
                                                          float* dst) {
  const int64_t n = (int64_t)rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t r = e / cols;
    const int col = (int)(e - r * cols);
    dst[e] = ns_to_f(D[r * ldD + col]);
  }
}

}  // namespace

hipError_t launch_sumsq(const EwArgs& a, float* const* W, double* partials, hipStream_t s) {
  hipLaunchKernelGGL(k_sumsq, dim3(a.nblocks), dim3(kThreads), 0, s, a, W, partials);
  return hipGetLastError();
}

hipError_t launch_momentum(const EwArgs& a, const float* const* G, float* const* M, float beta,
                           double* partials, hipStream_t s) {
  hipLaunchKernelGGL(k_momentum, dim3(a.nblocks), dim3(kThreads), 0, s, a, G, M, beta, partials);
  return hipGetLastError();
}

hipError_t launch_finalize(const EwArgs& a, const double* partials, double* norms, float* R,
                           hipStream_t s) {
  const int64_t n = (int64_t)a.g[a.ngroups - 1].first + a.g[a.ngroups - 1].count - a.g[0].first;
  const int blocks = (int)((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(k_finalize, dim3(blocks), dim3(kThreads), 0, s, a, partials, norms, R);
  return hipGetLastError();
}

hipError_t launch_normcast(const EwArgs& a, bool fp32, const float* const* M, const double* norms,
                           hipStream_t s) {
  if (fp32)
    hipLaunchKernelGGL(k_normcast<float>, dim3(a.nblocks), dim3(kThreads), 0, s, a, M, norms);
  else
    hipLaunchKernelGGL(k_normcast<__bf16>, dim3(a.nblocks), dim3(kThreads), 0, s, a, M, norms);
  return hipGetLastError();
}

hipError_t launch_update_norm(const EwArgs& a, bool fp32, float* const* W, float lr,
                              double* partials, hipStream_t s) {
  if (fp32)
    hipLaunchKernelGGL((k_update<float, false>), dim3(a.nblocks), dim3(kThreads), 0, s, a, W, lr,
                       partials, nullptr, nullptr);
  else
    hipLaunchKernelGGL((k_update<__bf16, false>), dim3(a.nblocks), dim3(kThreads), 0, s, a, W, lr,
                       partials, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_project(const EwArgs& a, bool fp32, float* const* W, const float* R,
                          const double* norms, float lr, hipStream_t s) {
  if (fp32)
    hipLaunchKernelGGL((k_update<float, true>), dim3(a.nblocks), dim3(kThreads), 0, s, a, W, lr,
                       nullptr, R, norms);
  else
    hipLaunchKernelGGL((k_update<__bf16, true>), dim3(a.nblocks), dim3(kThreads), 0, s, a, W, lr,
                       nullptr, R, norms);
  return hipGetLastError();
}

hipError_t launch_read_update(bool fp32, const char* D, int ldD, int rows, int cols, float* dst,
                              hipStream_t s) {
  const int64_t n = (int64_t)rows * cols;
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (fp32)
    hipLaunchKernelGGL(k_read_update<float>, dim3((int)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<const float*>(D), ldD, rows, cols, dst);
  else
    hipLaunchKernelGGL(k_read_update<__bf16>, dim3((int)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<const __bf16*>(D), ldD, rows, cols, dst);
  return hipGetLastError();
}

}  // namespace muonh
