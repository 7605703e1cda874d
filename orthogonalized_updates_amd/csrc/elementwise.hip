// HBM-bound phases of the MuonH step on gfx950: the init norm, the momentum
// update with its norm (alone, or fused with the cast of the unscaled
// momentum into the Newton-Schulz operand layout), the normalised cast, the
// trial update with its norm, the projection back onto the sphere, and the
// Muon baseline's decayed update. G and M are fp32 or bf16 (St<BF>), W is
// fp32. Every kernel is one grouped launch over the matrices of up to 16
// shape groups; blocks stream contiguous chunks with 16-byte accesses
// (8-byte for bf16 G and M), non-temporal on the M and W streams. Norms are
// deterministic reductions: at most 16 squares summed in fp32 (relative error
// at most 16 fp32 ulps, about 1e-6, every term being positive), an fp64
// running sum per thread, a fixed shuffle tree in fp64 per block, then a
// fixed-order fp64 sum of the per-block partials in a separate finalize
// kernel (no float atomics). So a norm's relative error stays below about
// 5e-7 however many entries a matrix has.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muonh_internal.h"

namespace muonh {
namespace {

constexpr int kThreads = kEwThreads;

__device__ __forceinline__ int group_of_block(const EwArgs& a, int b) {
  int gi = 0;
  for (int i = 1; i < a.ngroups; ++i)
    if (b >= a.g[i].block_begin) gi = i;
  return gi;
}

// Sum of the squares of 4 values in fp32 (sq4f), widened for an fp64
// running sum (sq4).
__device__ __forceinline__ float sq4f(float4 v, float acc = 0.f) {
  return fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, acc))));
}
__device__ __forceinline__ double sq4(float4 v) { return (double)sq4f(v); }
__device__ __forceinline__ double sq1(float v) { return (double)v * (double)v; }

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

// Non-temporal 16- and 8-byte accesses, for the streams each thread touches
// once: M in the momentum pass (read-modify-write) and W in the updates. On
// MI355X such streams ran 7-9 % faster with the hint in isolation. Not used
// for write-only outputs, nor where a line is shared by two reads.
// The pointers are cast to the global address space: on a generic pointer
// the hint compiles to flat accesses, which also count against the LDS
// counter and so make every wait a full one.
typedef float nt_f4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u2 __attribute__((ext_vector_type(2)));
#define MUONH_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ float4 ld_nt(const float* q) {
  const nt_f4 x = __builtin_nontemporal_load((const MUONH_GLOBAL nt_f4*)q);
  return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_nt(float* q, const float4& v) {
  const nt_f4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, (MUONH_GLOBAL nt_f4*)q);
}
// Plain 16- and 8-byte global accesses (through the builtin vector types,
// which take an address space where HIP's vector classes do not).
__device__ __forceinline__ float4 ld_g4(const void* q) {
  const nt_f4 x = *(const MUONH_GLOBAL nt_f4*)q;
  return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ uint2 ld_g2(const void* q) {
  const nt_u2 x = *(const MUONH_GLOBAL nt_u2*)q;
  return make_uint2(x.x, x.y);
}
__device__ __forceinline__ void st_g4(void* q, const float4& v) {
  const nt_f4 x = {v.x, v.y, v.z, v.w};
  *(MUONH_GLOBAL nt_f4*)q = x;
}
__device__ __forceinline__ uint2 ld_nt(const uint2* q) {
  const nt_u2 x = __builtin_nontemporal_load((const MUONH_GLOBAL nt_u2*)q);
  return make_uint2(x.x, x.y);
}
__device__ __forceinline__ void st_nt(uint2* q, uint2 v) {
  const nt_u2 x = {v.x, v.y};
  __builtin_nontemporal_store(x, (MUONH_GLOBAL nt_u2*)q);
}

// 4 bf16 values (the low half of each pair first, as in memory) widened.
__device__ __forceinline__ float4 widen4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// beta*m + g rounded once to the nearest bf16 (ties to even), for a bf16 m:
// the value a bf16 momentum stores. beta*m has at most 24 + 8 significant
// bits, so the fp64 product is exact; the fp64 sum s is rounded and its
// error e recovered exactly (two-sum: s + e = beta*m + g). The step to fp32
// then rounds to odd (keep the value truncated toward zero, and set its last
// bit when anything was dropped), which leaves the final rounding to bf16,
// 16 bits shorter, the same as rounding the exact value. A plain fp32 fma
// followed by a bf16 conversion would round twice.
__device__ __forceinline__ float mom_bf16(float beta, float m, float g) {
  const double p = (double)beta * (double)m;
  const double gd = (double)g;
  const double s = p + gd;
  if (!isfinite(s)) return (float)(__bf16)(float)s;  // inf, NaN
  const double bv = s - p;
  const double e = (p - (s - bv)) + (gd - bv);
  const float r = (float)s;  // nearest
  const double rd = (double)r;
  uint32_t t = __float_as_uint(r);
  bool inexact = true;
  if (rd == s) {
    // s is an fp32 value: the exact sum lies beyond it (e with the sign of
    // s, truncation keeps r) or before it (truncation is r's predecessor)
    if (e == 0.0) inexact = false;
    else if ((e < 0.0) != (s < 0.0)) t -= 1u;
  } else if (fabs(rd) > fabs(s)) {
    t -= 1u;  // r was rounded away from zero (an fp32 overflow included)
  }
  if (inexact) t |= 1u;
  return (float)(__bf16)__uint_as_float(t);
}

// Storage of the gradient and the momentum: fp32, or bf16 (BF). Element i of
// a flat array; load4/load4_nt/store4_nt take 4 consecutive elements from i
// (a multiple of 4, the address aligned to kVecAlign). mom(beta, m, g) is the
// new momentum as stored: one fp32 fma, or for bf16 storage the exact value
// rounded once to bf16 (mom_bf16); the stores then write it unchanged, so
// that what the caller goes on with (the norm, the cast) is exactly the
// stored momentum.
template <bool BF>
struct St;
template <>
struct St<false> {
  static constexpr unsigned kVecAlign = 16;
  __device__ static float mom(float beta, float m, float g) { return fmaf(beta, m, g); }
  __device__ static float load(const void* p, int64_t i) {
    return ((const MUONH_GLOBAL float*)p)[i];
  }
  __device__ static float4 load4(const void* p, int64_t i) {
    return ld_g4(static_cast<const float*>(p) + i);
  }
  __device__ static float store(void* p, int64_t i, float v) {
    ((MUONH_GLOBAL float*)p)[i] = v;
    return v;
  }
  __device__ static float4 load4_nt(const void* p, int64_t i) {
    return ld_nt(static_cast<const float*>(p) + i);
  }
  __device__ static float4 store4_nt(void* p, int64_t i, float4 v) {
    st_nt(static_cast<float*>(p) + i, v);
    return v;
  }
};
template <>
struct St<true> {
  static constexpr unsigned kVecAlign = 8;
  __device__ static float mom(float beta, float m, float g) { return mom_bf16(beta, m, g); }
  __device__ static float load(const void* p, int64_t i) {
    return __uint_as_float((uint32_t)((const MUONH_GLOBAL uint16_t*)p)[i] << 16);
  }
  __device__ static float4 load4(const void* p, int64_t i) {
    return widen4(ld_g2(static_cast<const uint16_t*>(p) + i));
  }
  __device__ static float4 load4_nt(const void* p, int64_t i) {
    return widen4(ld_nt(reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i)));
  }
  __device__ static float4 store4_nt(void* p, int64_t i, float4 v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 h = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    st_nt(reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i), __builtin_bit_cast(uint2, h));
    return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
  }
  __device__ static float store(void* p, int64_t i, float v) {
    const __bf16 h = (__bf16)v;
    ((MUONH_GLOBAL __bf16*)p)[i] = h;
    return (float)h;
  }
};

template <bool BF>
__device__ __forceinline__ bool vec_aligned(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & (St<BF>::kVecAlign - 1)) == 0;
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
  double acc = 0.0;
  int64_t mid = lo;
  if (aligned16(w)) {
    const int64_t n4 = (hi - lo) >> 2;
    const float4* w4 = reinterpret_cast<const float4*>(w + lo);
    for (int64_t i = threadIdx.x; i < n4; i += kThreads) acc += sq4(w4[i]);
    mid = lo + (n4 << 2);
  }
  for (int64_t e = mid + threadIdx.x; e < hi; e += kThreads) acc += sq1(w[e]);
  const double t = block_sum(acc, red);
  if (threadIdx.x == 0) partials[(int64_t)mat * kMaxPartials + c] = t;
}

// --------------------------------------------------------------------------
// M <- beta*M + G, with partial sums of squares of the new (stored) M;
// G and M in fp32 or bf16 (GB, MB)
// --------------------------------------------------------------------------
template <bool GB, bool MB>
__global__ __launch_bounds__(kThreads) void k_momentum(EwArgs a, const void* const* G,
                                                       void* const* M, float beta,
                                                       double* partials) {
  __shared__ double red[4];
  const int gi = group_of_block(a, blockIdx.x);
  const EwGroup& g = a.g[gi];
  const int local = blockIdx.x - g.block_begin;
  const int m = local / g.bpm, c = local - m * g.bpm;
  const int mat = g.first + m;
  const void* gp = G[mat];
  void* mp = M[mat];
  int64_t lo, hi;
  chunk_range(g.n, g.bpm, c, lo, hi);
  double acc = 0.0;
  int64_t mid = lo;
  if (vec_aligned<GB>(gp) && vec_aligned<MB>(mp)) {
    const int64_t n4 = (hi - lo) >> 2;
    for (int64_t i = threadIdx.x; i < n4; i += kThreads) {
      const int64_t e = lo + 4 * i;
      const float4 gv = St<GB>::load4(gp, e);
      float4 mv = St<MB>::load4_nt(mp, e);
      mv.x = St<MB>::mom(beta, mv.x, gv.x);
      mv.y = St<MB>::mom(beta, mv.y, gv.y);
      mv.z = St<MB>::mom(beta, mv.z, gv.z);
      mv.w = St<MB>::mom(beta, mv.w, gv.w);
      mv = St<MB>::store4_nt(mp, e, mv);
      acc += sq4(mv);
    }
    mid = lo + (n4 << 2);
  }
  for (int64_t e = mid + threadIdx.x; e < hi; e += kThreads) {
    const float v = St<MB>::store(mp, e, St<MB>::mom(beta, St<MB>::load(mp, e), St<GB>::load(gp, e)));
    acc += sq1(v);
  }
  const double t = block_sum(acc, red);
  if (threadIdx.x == 0) partials[(int64_t)mat * kMaxPartials + c] = t;
}

// --------------------------------------------------------------------------
// norms[mat] = sqrt(sum_c partials[mat][c]) in a fixed order, for exactly the
// matrices of the launch's groups: one wave per matrix (the t-th of them),
// lane l summing partials l, l + 64, ... in order, then a fixed shuffle tree.
// The groups need not cover a contiguous range of matrices: launches for
// other matrices may run concurrently and own the rest of the arrays.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_finalize(EwArgs a, const double* partials,
                                                       double* norms, float* R, uint32_t* flags,
                                                       uint32_t bit) {
  int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int gi = 0;
  while (gi < a.ngroups && t >= a.g[gi].count) t -= a.g[gi++].count;
  if (gi >= a.ngroups) return;  // uniform for the wave
  const int64_t mat = (int64_t)a.g[gi].first + t;
  const int bpm = a.g[gi].bpm;
  const double* p = partials + mat * kMaxPartials;
  double s = 0.0;
  for (int c = lane; c < bpm; c += 64) s += p[c];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    const double nrm = sqrt(s);
    norms[mat] = nrm;
    if (R) R[mat] = (float)nrm;
    if (flags && !isfinite(nrm)) atomicOr(flags, bit);
  }
}

// --------------------------------------------------------------------------
// Newton-Schulz operand storage formats (see NsPrec): element (r, c) of a
// matrix with ld logical columns (rows and ld multiples of 256).
//   bf16:  panel-major, panels of 256 rows x 32 values (64-byte panel rows),
//          panel (r/256, c/32) at ((r/256) * (ld/32) + c/32) * 16 KB;
//   split: the same with 16 values per panel row: 16 hi (bf16(v)) then the
//          16 matching lo (bf16(v - hi));
//   fp32:  row-major, row pitch ld (the fp32 debug kernel's layout).
// --------------------------------------------------------------------------
template <int F>
struct Fmt;
template <>
struct Fmt<kBf16> {
  __device__ static int64_t off(int64_t r, int c, int ld) {
    return ((((r >> 8) * (ld >> 5)) + (c >> 5)) << 14) + ((r & 255) << 6) + ((c & 31) << 1);
  }
  __device__ static float load(const char* base, int64_t r, int c, int ld) {
    return (float)*(const MUONH_GLOBAL __bf16*)(base + off(r, c, ld));
  }
  // 4 consecutive elements of a row, c a multiple of 4 (one 8-byte load).
  __device__ static float4 load4(const char* base, int64_t r, int c, int ld) {
    return widen4(ld_g2(base + off(r, c, ld)));
  }
  __device__ static void store4(char* base, int64_t r, int c, int ld, float4 v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 h = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    *(MUONH_GLOBAL bf16x4*)(base + off(r, c, ld)) = h;
  }
};
template <>
struct Fmt<kSplitBf16> {
  __device__ static int64_t off(int64_t r, int c, int ld) {  // of the hi value; lo at +32
    return ((((r >> 8) * (ld >> 4)) + (c >> 4)) << 14) + ((r & 255) << 6) + ((c & 15) << 1);
  }
  __device__ static float load(const char* base, int64_t r, int c, int ld) {
    const MUONH_GLOBAL __bf16* p = (const MUONH_GLOBAL __bf16*)(base + off(r, c, ld));
    return (float)p[0] + (float)p[16];
  }
  __device__ static void store4(char* base, int64_t r, int c, int ld, float4 v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 h = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    const bf16x4 l = {(__bf16)(v.x - (float)h[0]), (__bf16)(v.y - (float)h[1]),
                      (__bf16)(v.z - (float)h[2]), (__bf16)(v.w - (float)h[3])};
    char* p = base + off(r, c, ld);
    *(MUONH_GLOBAL bf16x4*)p = h;
    *(MUONH_GLOBAL bf16x4*)(p + 32) = l;
  }
  __device__ static float4 load4(const char* base, int64_t r, int c, int ld) {
    const char* p = base + off(r, c, ld);
    return add4(widen4(ld_g2(p)), widen4(ld_g2(p + 32)));
  }
  __device__ static float4 add4(float4 h, float4 l) {
    return make_float4(h.x + l.x, h.y + l.y, h.z + l.z, h.w + l.w);
  }
};
template <>
struct Fmt<kFp32> {
  __device__ static int64_t off(int64_t r, int c, int ld) { return (r * ld + c) * 4; }
  __device__ static float load(const char* base, int64_t r, int c, int ld) {
    return *(const MUONH_GLOBAL float*)(base + off(r, c, ld));
  }
  __device__ static float4 load4(const char* base, int64_t r, int c, int ld) {
    return ld_g4(base + off(r, c, ld));
  }
  __device__ static void store4(char* base, int64_t r, int c, int ld, float4 v) {
    st_g4(base + off(r, c, ld), v);
  }
};

// --------------------------------------------------------------------------
// One 64x64 tile of the padded rp x cp domain of a matrix: X0 values written
// straight to D and/or transposed (through LDS) to E (an offset of -1 skips
// that output); entries outside rows x cols are written as zero. With
// kMomentum the tile first takes M <- beta*M + G (written back) and returns
// this thread's sum of squares of the new stored M; the values written are
// then scale * M. G and M are fp32 or bf16 (GB, MB). Each thread takes 4 consecutive columns of 4 rows: columns
// c0 + 4*(tid % 16), rows r0 + tid/16 + 16i. Every thread of the block must
// call it (it synchronises when E is written).
// --------------------------------------------------------------------------
template <int F, bool kMomentum, bool GB, bool MB>
__device__ __forceinline__ double cast_tile(const EwGroup& g, char* blk, const void* gp, void* mp,
                                           float beta, int r0, int c0, float scale,
                                           float (*tile)[65]) {
  const int tx = (threadIdx.x & 15) << 2, ty = threadIdx.x >> 4;
  const bool vec = (g.cols & 3) == 0 && vec_aligned<MB>(mp) && (!kMomentum || vec_aligned<GB>(gp));
  const bool trans = g.offE >= 0;
  float acc = 0.f;  // the squares of this thread's 16 values
  if (trans) __syncthreads();  // the previous tile's transposed reads are done
  // The vector loads of all four rows are issued before the first store.
  const int c = c0 + tx;
  const bool cvec = vec && c + 3 < g.cols;
  // Rows past the end reload the last row, so that the loads need no
  // branch of their own (each branch would end in a wait).
  float4 mv[4], gv[4];
  if (cvec) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = min(r0 + ty + 16 * i, g.rows - 1);
      const int64_t i0 = (int64_t)r * g.cols + c;
      if (kMomentum) {  // read-modify-write of M: non-temporal
        mv[i] = St<MB>::load4_nt(mp, i0);
        gv[i] = St<GB>::load4(gp, i0);
      } else {
        mv[i] = St<MB>::load4(mp, i0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = ty + 16 * i;
    const int r = r0 + rr;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < g.rows) {
      const int64_t i0 = (int64_t)r * g.cols + c;
      if (cvec) {
        v = mv[i];
        if (kMomentum) {
          v.x = St<MB>::mom(beta, v.x, gv[i].x);
          v.y = St<MB>::mom(beta, v.y, gv[i].y);
          v.z = St<MB>::mom(beta, v.z, gv[i].z);
          v.w = St<MB>::mom(beta, v.w, gv[i].w);
          v = St<MB>::store4_nt(mp, i0, v);
        }
      } else {
        float e[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (c + q < g.cols) {
            float m = St<MB>::load(mp, i0 + q);
            if (kMomentum) m = St<MB>::store(mp, i0 + q, St<MB>::mom(beta, m, St<GB>::load(gp, i0 + q)));
            e[q] = m;
          }
        }
        v = make_float4(e[0], e[1], e[2], e[3]);
      }
    }
    if (kMomentum) acc = sq4f(v, acc);
    v.x *= scale;
    v.y *= scale;
    v.z *= scale;
    v.w *= scale;
    if (g.offD >= 0) Fmt<F>::store4(blk + g.offD, r, c, g.cp, v);
    if (trans) {
      tile[rr][tx] = v.x;
      tile[rr][tx + 1] = v.y;
      tile[rr][tx + 2] = v.z;
      tile[rr][tx + 3] = v.w;
    }
  }
  if (trans) {
    __syncthreads();
    // transposed: row c0 + cc of E, its columns r0 + tx .. +3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cc = ty + 16 * i;
      const float4 v = make_float4(tile[tx][cc], tile[tx + 1][cc], tile[tx + 2][cc], tile[tx + 3][cc]);
      Fmt<F>::store4(blk + g.offE, c0 + cc, r0 + tx, g.rp, v);
    }
  }
  return (double)acc;
}

// X0 = M / (||M|| + eps): one tile per block.
template <int F, bool MB>
__global__ __launch_bounds__(kThreads) void k_normcast(EwArgs a, const void* const* M,
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
  cast_tile<F, false, false, MB>(g, g.ns_base + (int64_t)m * g.mat_bytes, nullptr,
                                 const_cast<void*>(M[mat]), 0.f, r0, c0, scale, tile);
}

// Fused momentum and unscaled cast: block c of a matrix takes tiles
// [c*tpb, (c+1)*tpb) of its padded domain and writes one partial sum.
template <int F, bool GB, bool MB>
__global__ __launch_bounds__(kThreads) void k_momentum_cast(EwArgs a, const void* const* G,
                                                            void* const* M, float beta,
                                                            double* partials) {
  __shared__ float tile[64][65];
  __shared__ double red[4];
  const int gi = group_of_block(a, blockIdx.x);
  const EwGroup& g = a.g[gi];
  const int local = blockIdx.x - g.block_begin;
  const int m = local / g.bpm, c = local - m * g.bpm;
  const int mat = g.first + m;
  char* blk = g.ns_base + (int64_t)m * g.mat_bytes;
  const int tcols = g.cp >> 6;
  const int t1 = min((c + 1) * g.tpb, g.tiles_per_mat);
  double acc = 0.0;
  for (int t = c * g.tpb; t < t1; ++t) {
    const int r0 = (t / tcols) << 6, c0 = (t - (t / tcols) * tcols) << 6;
    acc += cast_tile<F, true, GB, MB>(g, blk, G[mat], M[mat], beta, r0, c0, 1.f, tile);
  }
  const double tot = block_sum(acc, red);
  if (threadIdx.x == 0) partials[(int64_t)mat * kMaxPartials + c] = tot;
}

// Fallback of the deferred normalisation: 8 blocks per matrix; for the
// matrices whose norm fails xnorm_deferred, and for every matrix of a group
// that never defers, they rewrite X0 normalised.
template <int F, bool MB>
__global__ __launch_bounds__(kThreads) void k_cast_fallback(EwArgs a, const void* const* M,
                                                            const double* norms) {
  __shared__ float tile[64][65];
  int b = blockIdx.x, gi = 0;
  while (gi < a.ngroups && b >= a.g[gi].count * 8) b -= a.g[gi++].count * 8;
  if (gi >= a.ngroups) return;
  const EwGroup& g = a.g[gi];
  const int m = b >> 3, j = b & 7;
  const int mat = g.first + m;
  const double n = norms[mat];
  if (g.defer && xnorm_deferred(n)) return;  // uniform for the block
  const float scale = (float)(1.0 / (n + kNsEps));
  char* blk = g.ns_base + (int64_t)m * g.mat_bytes;
  const int tcols = g.cp >> 6;
  for (int t = j; t < g.tiles_per_mat; t += 8) {
    const int r0 = (t / tcols) << 6, c0 = (t - (t / tcols) * tcols) << 6;
    cast_tile<F, false, false, MB>(g, blk, nullptr, const_cast<void*>(M[mat]), 0.f, r0, c0, scale,
                                   tile);
  }
}

// --------------------------------------------------------------------------
// Updates that read O from D, by mode:
//   kTrialNorm  W' = W - lr*O, partial sums of squares of W' (W unchanged);
//   kProject    W <- (R / ||W'||) W', W' recomputed identically;
//   kDecay      W <- keep*W - lr*O with keep = 1 - lr*wd (Muon with
//               decoupled weight decay; no norm).
// --------------------------------------------------------------------------
enum UpdateMode : int { kTrialNorm = 0, kProjectMode = 1, kDecay = 2 };

template <int F, int kMode>
__global__ __launch_bounds__(kThreads) void k_update(EwArgs a, float* const* W, float lr,
                                                     double* partials, const float* R,
                                                     const double* norms, float keep) {
  constexpr bool kProject = kMode == kProjectMode;
  constexpr bool kWrite = kMode != kTrialNorm;
  __shared__ double red[4];
  const int gi = group_of_block(a, blockIdx.x);
  const EwGroup& g = a.g[gi];
  const int local = blockIdx.x - g.block_begin;
  const int m = local / g.bpm, c = local - m * g.bpm;
  const int mat = g.first + m;
  float* w = W[mat];
  const char* D = g.ns_base + (int64_t)m * g.mat_bytes + g.offD;
  const float nlr = -lr;
  float scale = 1.f;
  if (kProject) {
    const double nrm = norms[mat];
    scale = nrm > 0.0 ? (float)((double)R[mat] / nrm) : 1.f;
  }
  double acc = 0.0;
  const int cols = g.cols;
  if ((cols & 3) == 0 && aligned16(w)) {
    // Work unit: 4 consecutive columns of the row pair (2p, 2p + 1). The two
    // rows' O values share 128-byte lines of the panel layout (panel rows r
    // and r + 1 are adjacent 64-byte halves), so each line is read once.
    // Block c takes units [u0, u1); (pair, column group) walk incrementally.
    // A thread takes two units per iteration and issues all eight loads
    // before its first store, to keep enough bytes in flight per CU.
    const int cq = cols >> 2;
    const int64_t npairs = (int64_t)(g.rows + 1) >> 1;
    int64_t u0, u1;
    chunk_range(npairs * cq, g.bpm, c, u0, u1);
    int64_t u = u0 + threadIdx.x;
    int64_t pr = u / cq;
    int q = (int)(u - pr * cq);
    const int dpr = kThreads / cq, dq = kThreads - (kThreads / cq) * cq;
    for (; u < u1; u += 2 * kThreads) {
      int64_t prs[2] = {pr, pr + dpr};
      int qs[2] = {q, q + dq};
      if (qs[1] >= cq) { qs[1] -= cq; ++prs[1]; }
      const bool has1 = u + kThreads < u1;
      // The loads are unconditional, so that none of them waits for another:
      // a row past the end (the second row of the last pair of an odd row
      // count) reloads its own unit's first row, and a unit past the end
      // reloads the first unit's first row. Either way the address belongs
      // to one of this thread's own live units, so the store below rewrites
      // bytes only this thread writes, with the value it already computed.
      float4 wv[2][2], ov[2][2];
      float* wp[2][2];  // the load addresses, reused by the stores
      bool live[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool unit = j == 0 || has1;  // slot j holds a unit of this block
          const int64_t r = 2 * prs[j] + h;
          live[j][h] = unit && r < g.rows;
          const int64_t rl = live[j][h] ? r : 2 * (unit ? prs[j] : prs[0]);
          const int cl = (unit ? qs[j] : qs[0]) << 2;
          wp[j][h] = w + rl * cols + cl;
          wv[j][h] = ld_nt(wp[j][h]);
          // O plainly: rows r and r + 1 read the two halves of one 128-byte
          // line, and the second read is served from the cache only when the
          // first did not carry the non-temporal hint
          ov[j][h] = Fmt<F>::load4(D, rl, cl, g.cp);
        }
      // All four results first, then the stores: a store between two
      // results would make the next one wait for it.
      float part = 0.f;  // squares of this pass's (up to) 16 values
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float4 v = wv[j][h];
          const float4 o = ov[j][h];
          if (kMode == kDecay) {
            v.x *= keep; v.y *= keep; v.z *= keep; v.w *= keep;
          }
          v.x = fmaf(nlr, o.x, v.x);
          v.y = fmaf(nlr, o.y, v.y);
          v.z = fmaf(nlr, o.z, v.z);
          v.w = fmaf(nlr, o.w, v.w);
          if (kProject) {
            v.x *= scale; v.y *= scale; v.z *= scale; v.w *= scale;
          }
          if (!kWrite && live[j][h]) part = sq4f(v, part);
          wv[j][h] = v;
        }
      if (!kWrite) acc += (double)part;
      // Unconditional stores: a slot past the end holds the address and the
      // recomputed value of one of this thread's live units, so it rewrites
      // the same bytes with the same value (a store under a branch would
      // again cost a wait).
      if (kWrite) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) st_nt(wp[j][h], wv[j][h]);
      }
      pr = prs[1] + dpr;
      q = qs[1] + dq;
      if (q >= cq) { q -= cq; ++pr; }
    }
  } else {
    int64_t lo, hi;
    chunk_range(g.n, g.bpm, c, lo, hi);
    for (int64_t e = lo + threadIdx.x; e < hi; e += kThreads) {
      const int64_t r = e / cols;
      const int col = (int)(e - r * cols);
      const float wv = kMode == kDecay ? keep * w[e] : w[e];
      float v = fmaf(nlr, Fmt<F>::load(D, r, col, g.cp), wv);
      if (kWrite) {
        w[e] = kProject ? v * scale : v;
      } else {
        acc += sq1(v);
      }
    }
  }
  if (!kWrite) {
    const double t = block_sum(acc, red);
    if (threadIdx.x == 0) partials[(int64_t)mat * kMaxPartials + c] = t;
  }
}

template <int F>
__global__ __launch_bounds__(kThreads) void k_read_update(const char* D, int ldD, int rows,
                                                          int cols, float* dst) {
  const int64_t n = (int64_t)rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t r = e / cols;
    const int col = (int)(e - r * cols);
    dst[e] = Fmt<F>::load(D, r, col, ldD);
  }
}

}  // namespace

hipError_t launch_sumsq(const EwArgs& a, float* const* W, double* partials, hipStream_t s) {
  hipLaunchKernelGGL(k_sumsq, dim3(a.nblocks), dim3(kThreads), 0, s, a, W, partials);
  return hipGetLastError();
}

// Launches KERNEL<..., GB, MB> for the run-time storage formats of G and M.
#define MUONH_STATE_DISPATCH(SF, KERNEL, ...)                                   \
  do {                                                                          \
    if ((SF).g_bf16) {                                                          \
      if ((SF).m_bf16) hipLaunchKernelGGL(KERNEL(true, true), __VA_ARGS__);     \
      else hipLaunchKernelGGL(KERNEL(true, false), __VA_ARGS__);                \
    } else {                                                                    \
      if ((SF).m_bf16) hipLaunchKernelGGL(KERNEL(false, true), __VA_ARGS__);    \
      else hipLaunchKernelGGL(KERNEL(false, false), __VA_ARGS__);               \
    }                                                                           \
  } while (0)

#define K_MOMENTUM(GB, MB) (k_momentum<GB, MB>)

hipError_t launch_momentum(const EwArgs& a, StateFmt sf, const void* const* G, void* const* M,
                           float beta, double* partials, hipStream_t s) {
  MUONH_STATE_DISPATCH(sf, K_MOMENTUM, dim3(a.nblocks), dim3(kThreads), 0, s, a, G, M, beta,
                       partials);
  return hipGetLastError();
}

hipError_t launch_finalize(const EwArgs& a, const double* partials, double* norms, float* R,
                           hipStream_t s, uint32_t* flags, uint32_t bit) {
  int64_t n = 0;
  for (int i = 0; i < a.ngroups; ++i) n += a.g[i].count;
  const int per_block = kThreads / 64;  // one wave per matrix
  const int blocks = (int)((n + per_block - 1) / per_block);
  hipLaunchKernelGGL(k_finalize, dim3(blocks), dim3(kThreads), 0, s, a, partials, norms, R, flags,
                     bit);
  return hipGetLastError();
}

#define MUONH_PREC_DISPATCH(PREC, KERNEL, ...)                       \
  switch (PREC) {                                                    \
    case kBf16: hipLaunchKernelGGL(KERNEL(kBf16), __VA_ARGS__); break; \
    case kSplitBf16: hipLaunchKernelGGL(KERNEL(kSplitBf16), __VA_ARGS__); break; \
    case kFp32: hipLaunchKernelGGL(KERNEL(kFp32), __VA_ARGS__); break; \
  }

#define K_UPDATE(F) (k_update<F, kTrialNorm>)
#define K_PROJECT(F) (k_update<F, kProjectMode>)
#define K_DECAY(F) (k_update<F, kDecay>)
#define K_READ(F) k_read_update<F>

// Kernels templated on the operand format F and the momentum storage MB.
#define K_NORMCAST_M0(F) (k_normcast<F, false>)
#define K_NORMCAST_M1(F) (k_normcast<F, true>)
#define K_FALLBACK_M0(F) (k_cast_fallback<F, false>)
#define K_FALLBACK_M1(F) (k_cast_fallback<F, true>)

hipError_t launch_normcast(const EwArgs& a, NsPrec prec, StateFmt sf, const void* const* M,
                           const double* norms, hipStream_t s) {
  if (sf.m_bf16) {
    MUONH_PREC_DISPATCH(prec, K_NORMCAST_M1, dim3(a.nblocks), dim3(kThreads), 0, s, a, M, norms)
  } else {
    MUONH_PREC_DISPATCH(prec, K_NORMCAST_M0, dim3(a.nblocks), dim3(kThreads), 0, s, a, M, norms)
  }
  return hipGetLastError();
}

template <int F>
void launch_momentum_cast_f(const EwArgs& a, StateFmt sf, const void* const* G, void* const* M,
                            float beta, double* partials, hipStream_t s) {
#define K_MOMCAST(GB, MB) (k_momentum_cast<F, GB, MB>)
  MUONH_STATE_DISPATCH(sf, K_MOMCAST, dim3(a.nblocks), dim3(kThreads), 0, s, a, G, M, beta,
                       partials);
#undef K_MOMCAST
}

hipError_t launch_momentum_cast(const EwArgs& a, NsPrec prec, StateFmt sf, const void* const* G,
                                void* const* M, float beta, double* partials, hipStream_t s) {
  switch (prec) {
    case kBf16: launch_momentum_cast_f<kBf16>(a, sf, G, M, beta, partials, s); break;
    case kSplitBf16: launch_momentum_cast_f<kSplitBf16>(a, sf, G, M, beta, partials, s); break;
    case kFp32: launch_momentum_cast_f<kFp32>(a, sf, G, M, beta, partials, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_cast_fallback(const EwArgs& a, NsPrec prec, StateFmt sf, const void* const* M,
                                const double* norms, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < a.ngroups; ++i) blocks += (int64_t)a.g[i].count * 8;
  if (blocks == 0) return hipSuccess;
  if (sf.m_bf16) {
    MUONH_PREC_DISPATCH(prec, K_FALLBACK_M1, dim3((unsigned)blocks), dim3(kThreads), 0, s, a, M,
                        norms)
  } else {
    MUONH_PREC_DISPATCH(prec, K_FALLBACK_M0, dim3((unsigned)blocks), dim3(kThreads), 0, s, a, M,
                        norms)
  }
  return hipGetLastError();
}

hipError_t launch_update_norm(const EwArgs& a, NsPrec prec, float* const* W, float lr,
                              double* partials, hipStream_t s) {
  MUONH_PREC_DISPATCH(prec, K_UPDATE, dim3(a.nblocks), dim3(kThreads), 0, s, a, W, lr, partials,
                      nullptr, nullptr, 1.f)
  return hipGetLastError();
}

hipError_t launch_project(const EwArgs& a, NsPrec prec, float* const* W, const float* R,
                          const double* norms, float lr, hipStream_t s) {
  MUONH_PREC_DISPATCH(prec, K_PROJECT, dim3(a.nblocks), dim3(kThreads), 0, s, a, W, lr, nullptr,
                      R, norms, 1.f)
  return hipGetLastError();
}

hipError_t launch_decay_update(const EwArgs& a, NsPrec prec, float* const* W, float lr, float keep,
                               hipStream_t s) {
  MUONH_PREC_DISPATCH(prec, K_DECAY, dim3(a.nblocks), dim3(kThreads), 0, s, a, W, lr, nullptr,
                      nullptr, nullptr, keep)
  return hipGetLastError();
}

hipError_t launch_read_update(NsPrec prec, const char* D, int ldD, int rows, int cols, float* dst,
                              hipStream_t s) {
  const int64_t n = (int64_t)rows * cols;
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  MUONH_PREC_DISPATCH(prec, K_READ, dim3((int)blocks), dim3(kThreads), 0, s, D, ldD, rows, cols,
                      dst)
  return hipGetLastError();
}

}  // namespace muonh
