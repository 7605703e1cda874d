// Newton-Schulz GEMMs of the MuonH step on gfx950 MFMA.
//
// The digest page "Puro-2B trains for $6.9K, attention sinks hit 99%,
// LoopArena tops at 24.69%" (footnote 4) names the Newton-Schulz iterations as
// where Muon's cost goes. Per iteration, on the short-side-first operand X
// (s x l, zero-padded) the step computes
//   A = X X^T                  (symmetric: upper tiles only, mirrored)
//   B = b A + c A A            (A symmetric, so A A = A A^T: same kernel shape)
//   X <- a X + B X             (B X = B (X^T)^T: operands are B rows, X^T rows)
// so every product is C[i][j] = sum_k P[i][k] Q[j][k] with both operands read
// as K-contiguous rows. The apply step writes the new X in both layouts (X and
// X^T) so that the next Gram and the next apply again read K-contiguous rows.
//
// Kernel shape: one workgroup per output tile (grouped across all matrices of
// all shape groups in one launch), 4 waves in a 2x2 grid, 32x32 MFMA blocks,
// operands staged through a double-buffered LDS ring of 128-byte K-slab rows
// with an XOR swizzle of the 16-byte chunks, fp32 accumulation, fused
// epilogues. bf16: v_mfma_f32_32x32x16_bf16; fp32 debug: v_mfma_f32_32x32x2f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "muonh_internal.h"

namespace muonh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = 128;  // one K-slab row of an operand tile in LDS

// LDS byte offset of 16-byte chunk `chunk` (0..7) of tile row `row`. The XOR
// spreads the 8 rows that one ds_read_b128 phase touches over distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

// Register-staged global -> LDS copy of a ROWS x 128-byte operand slab.
template <int ROWS, int NTHR>
struct SlabLoader {
  static constexpr int kPer = ROWS * 8 / NTHR;
  static_assert(kPer * NTHR == ROWS * 8, "slab must split evenly over the threads");
  u32x4 v[kPer];
  __device__ __forceinline__ void load(const char* base, int64_t ld_bytes, int64_t k0_bytes,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + i * NTHR;
      const int row = q >> 3, c = q & 7;
      v[i] = *reinterpret_cast<const u32x4*>(base + row * ld_bytes + k0_bytes + (c << 4));
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + i * NTHR;
      const int row = q >> 3, c = q & 7;
      *reinterpret_cast<u32x4*>(lds + swz(row, c)) = v[i];
    }
  }
};

// One 128-byte K-slab of MFMAs for a wave's MT x NT grid of 32x32 blocks.
template <typename T, int MT, int NT>
__device__ __forceinline__ void mma_slab(const char* la, const char* lb, int wm0, int wn0,
                                         int lane, f32x16 (&acc)[MT][NT]) {
  const int r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = ks * 2 + g;
    if constexpr (std::is_same<T, __bf16>::value) {
      // Lane (r, g) holds k = 16*ks + 8*g .. +7 of row r: the operand layout of
      // the 32x32x16 bf16 MFMA.
      bf16x8 av[MT], bv[NT];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
        av[mi] = *reinterpret_cast<const bf16x8*>(la + swz(wm0 + mi * 32 + r, c));
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
        bv[ni] = *reinterpret_cast<const bf16x8*>(lb + swz(wn0 + ni * 32 + r, c));
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    } else {
      // fp32: lane (r, g) loads k = 8*ks + 4*g .. +3; MFMA j takes element j,
      // so lane group g stands for k = 8*ks + 4*g + j in both operands.
      f32x4 av[MT], bv[NT];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
        av[mi] = *reinterpret_cast<const f32x4*>(la + swz(wm0 + mi * 32 + r, c));
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
        bv[ni] = *reinterpret_cast<const f32x4*>(lb + swz(wn0 + ni * 32 + r, c));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
          for (int ni = 0; ni < NT; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mi][j], bv[ni][j], acc[mi][ni], 0, 0, 0);
    }
  }
}

template <typename T>
__device__ __forceinline__ float ld_f(const T* p) {
  return (float)*p;
}

template <typename T>
__device__ __forceinline__ void st_1(T* p, float v) {
  *p = (T)v;
}

// Stores 4 values that are consecutive along a row of the destination.
template <typename T>
__device__ __forceinline__ void st_4(T* p, float v0, float v1, float v2, float v3) {
  if constexpr (std::is_same<T, __bf16>::value) {
    bf16x4 w = {(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
    *reinterpret_cast<bf16x4*>(p) = w;
  } else {
    f32x4 w = {v0, v1, v2, v3};
    *reinterpret_cast<f32x4*>(p) = w;
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, int MODE>
__global__ __launch_bounds__(WGM * WGN * 64) void k_ns_gemm(GemmArgs args) {
  constexpr int NTHR = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int KE = kRowBytes / (int)sizeof(T);  // elements per K-slab
  constexpr bool kSym = (MODE != kApply);
  static_assert(BM == BN || !kSym, "symmetric modes need square tiles");

  __shared__ __attribute__((aligned(16))) char lds[2 * (BM + BN) * kRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;

  // ---- tile decode: group, matrix, (bi, bj)
  const int tile = blockIdx.x;
  int gi = 0;
  for (int i = 1; i < args.ngroups; ++i)
    if (tile >= args.g[i].tile_begin) gi = i;
  const GemmGroup& g = args.g[gi];
  const int local = tile - g.tile_begin;
  const int mat = local / g.tiles_per_mat;
  int t = local - mat * g.tiles_per_mat;
  int bi, bj;
  if (kSym) {
    int rowlen = g.tm;
    bi = 0;
    while (t >= rowlen) {
      t -= rowlen;
      ++bi;
      --rowlen;
    }
    bj = bi + t;
  } else {
    bi = t % g.tm;
    bj = t / g.tm;
  }

  const char* blk = g.base + (int64_t)mat * g.mat_bytes;
  const int64_t ldp_b = (int64_t)g.ldp * sizeof(T), ldq_b = (int64_t)g.ldq * sizeof(T);
  const char* P = blk + g.offP + (int64_t)bi * BM * ldp_b;
  const char* Q = blk + g.offQ + (int64_t)bj * BN * ldq_b;

  // Stage st of the LDS ring: A slab at st*kStage, B slab right after it.
  constexpr int kStage = (BM + BN) * kRowBytes;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x16{};

  SlabLoader<BM, NTHR> la;
  SlabLoader<BN, NTHR> lb;
  const int nk = g.K / KE;
  la.load(P, ldp_b, 0, tid);
  lb.load(Q, ldq_b, 0, tid);
  la.store(lds, tid);
  lb.store(lds + BM * kRowBytes, tid);
  __syncthreads();

  const int wm0 = wm * WTM, wn0 = wn * WTN;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(P, ldp_b, (int64_t)(kt + 1) * kRowBytes, tid);
      lb.load(Q, ldq_b, (int64_t)(kt + 1) * kRowBytes, tid);
    }
    char* st = lds + cur * kStage;
    mma_slab<T, MT, NT>(st, st + BM * kRowBytes, wm0, wn0, lane, acc);
    if (more) {
      char* nx = lds + (cur ^ 1) * kStage;
      la.store(nx, tid);
      lb.store(nx + BM * kRowBytes, tid);
    }
    __syncthreads();
  }

  // ---- epilogue. Accumulator element q of a 32x32 block sits at
  // row 8*(q/4) + 4*(lane/32) + q%4, column lane%32.
  const T* E = (MODE == kGram || g.offE < 0) ? nullptr : reinterpret_cast<const T*>(blk + g.offE);
  T* O1 = g.offO1 < 0 ? nullptr : reinterpret_cast<T*>(const_cast<char*>(blk) + g.offO1);
  T* O2 = g.offO2 < 0 ? nullptr : reinterpret_cast<T*>(const_cast<char*>(blk) + g.offO2);
  const float c0 = args.c0, c1 = args.c1;
  const bool mirror = kSym && bi != bj;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      const int col = bj * BN + wn0 + ni * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int row0 = bi * BM + wm0 + mi * 32 + 8 * rg + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a = acc[mi][ni][rg * 4 + q];
          if (MODE == kGram) {
            v[q] = a;
          } else if (MODE == kPoly) {
            v[q] = fmaf(c1, a, c0 * ld_f(E + (int64_t)(row0 + q) * g.lde + col));
          } else {
            v[q] = fmaf(c0, ld_f(E + (int64_t)(row0 + q) * g.lde + col), a);
          }
        }
        if (O1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) st_1(O1 + (int64_t)(row0 + q) * g.ldo1 + col, v[q]);
        }
        if (mirror) st_4(O1 + (int64_t)col * g.ldo1 + row0, v[0], v[1], v[2], v[3]);
        if (MODE == kApply && O2) st_4(O2 + (int64_t)col * g.ldo2 + row0, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

constexpr int kTile = 128;
constexpr int kWGM = 2, kWGN = 2;

template <typename T, int MODE>
hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_ns_gemm<T, kTile, kTile, kWGM, kWGN, MODE>), dim3(a.ntiles),
                     dim3(kWGM * kWGN * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int gemm_tile(bool /*fp32*/) { return kTile; }

hipError_t launch_gemm(GemmMode mode, bool fp32, const GemmArgs& a, hipStream_t s) {
  if (a.ntiles <= 0) return hipSuccess;
  if (fp32) {
    switch (mode) {
      case kGram: return launch_t<float, kGram>(a, s);
      case kPoly: return launch_t<float, kPoly>(a, s);
      case kApply: return launch_t<float, kApply>(a, s);
    }
  } else {
    switch (mode) {
      case kGram: return launch_t<__bf16, kGram>(a, s);
      case kPoly: return launch_t<__bf16, kPoly>(a, s);
      case kApply: return launch_t<__bf16, kApply>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace muonh
