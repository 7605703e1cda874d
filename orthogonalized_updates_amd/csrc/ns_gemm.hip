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
// Every launch covers one phase for all matrices of all shape groups: one
// workgroup per output tile, tiles dealt to the 8 XCDs in contiguous runs.
// bf16 (the product path): 256x256 tiles, 8 waves in two groups that take
// turns between MFMA clusters (v_mfma_f32_32x32x16_bf16, fp32 accumulation)
// and LDS fragment loads, operands streamed into a 2-stage LDS ring of
// 64-wide K slabs by LDS DMA (global_load_lds_dwordx4), the fp32 a*X or b*A
// term folded into the accumulators from the operand stream, and epilogues
// staged through LDS for coalesced stores of both output layouts.
// fp32 debug: a simpler 128x128 kernel on v_mfma_f32_32x32x2f32 with
// register-staged double buffering and direct epilogue stores.
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
__global__ __launch_bounds__(WGM * WGN * 64, (WGM * WGN) / 4) void k_ns_gemm(GemmArgs args) {
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

// ---------------------------------------------------------------------------
// bf16 pipeline: 256x256 tiles, 8 waves (2 x 4, wave tile 128x64), operands
// streamed straight from global memory into a 2-stage LDS ring of 64-wide K
// slabs (full 128-byte rows; global_load_lds_dwordx4, no staging
// registers). Each stage buffer is its own __shared__ object so that the
// compiler can tell the in-flight DMA writes of one buffer apart from the
// reads of the other.
// ---------------------------------------------------------------------------
namespace bf {

constexpr int kBM = 256, kBN = 256;
constexpr int kRow = 128;                            // bytes per slab row (64 bf16)
constexpr int kSlabA = kBM * kRow, kSlabB = kBN * kRow;
constexpr int kKS = kRow / 32;                       // 16-wide MFMA k steps per slab

// Wave grid WGM x WGN over the 256x256 tile; each wave owns MT x NT blocks
// of 32x32.
template <int WGM, int WGN>
struct Cfg {
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWTM = kBM / WGM, kWTN = kBN / WGN;
  static constexpr int kMT = kWTM / 32, kNT = kWTN / 32;
  static_assert(kWaves == 8, "the ping-pong schedule and the DMA split assume 8 waves");
};

// Chunk (16 B) c of slab row r sits at r*128 + ((c ^ ((r >> 1) & 7)) << 4).
// A ds_read_b128 is served 16 lanes at a time from 64 four-byte banks; the
// 16 consecutive rows one pass touches then fall on 16 distinct 16-byte bank
// groups ((r & 1) picks half of the 256-byte bank window, the swizzled chunk
// a slot within it).
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRow + ((chunk ^ ((row >> 1) & 7)) << 4);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14]; expcnt/lgkmcnt left at max.
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Phase barrier of the ping-pong schedule. __syncthreads() would also wait
// for every outstanding global load (its release fence covers the LDS DMA
// writes still in flight); here each wave has already waited for the loads
// it needs, and lgkmcnt(0) retires its LDS reads (so a buffer may be
// refilled after the barrier). The empty asm statements keep the compiler
// from moving memory accesses across, and the scheduling barriers keep any
// instruction (MFMAs included) from migrating from one phase to the next.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One stage is 64 global_load_lds instructions of 1 KB (8 rows x 128 B, full
// cache lines): waves 0-3 issue rows of A, waves 4-7 rows of B, 8 each.
// Instruction i of wave w covers rows 8*jj .. 8*jj+7, jj = 8*(w % 4) + i, of
// its operand; lane l fills LDS bytes l*16..l*16+15 of that 1 KB block: row
// 8*jj + l/8, position l%8, which must hold chunk (l%8) ^ swizzle(row). The
// swizzle (row >> 1) & 7 = (4*(jj & 1) + l/16) & 7 depends on jj only
// through its parity, so a lane needs two 32-bit offsets (voff[jj & 1]); the
// rest of the address is wave-uniform.
struct StageSrc {
  const char* base;  // operand rows of this wave's share, wave-uniform
  int64_t ld_b;      // operand row pitch in bytes
  int voff[2];       // per-lane offsets for even and odd instructions
};

__device__ __forceinline__ StageSrc stage_src(const char* P, const char* Q, int64_t ldp_b,
                                              int64_t ldq_b, int wave, int lane) {
  StageSrc t;
  const bool isA = wave < 4;
  const int jj0 = (wave & 3) * 8;
  t.ld_b = isA ? ldp_b : ldq_b;
  t.base = (isA ? P : Q) + (int64_t)(jj0 * 8) * t.ld_b;
#pragma unroll
  for (int par = 0; par < 2; ++par)
    t.voff[par] = (int)((lane >> 3) * t.ld_b) + (((lane & 7) ^ ((4 * par + (lane >> 4)) & 7)) << 4);
  return t;
}

// Issue this wave's 8 loads of the stage at K offset k0_b into slab buffer
// `buf` (A at +0, B at +kSlabA).
__device__ __forceinline__ void issue_stage(const StageSrc& t, int wave, int64_t k0_b, char* buf) {
  char* l = buf + (wave < 4 ? 0 : kSlabA) + (wave & 3) * 8 * 1024;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const char* g = t.base + (int64_t)(i * 8) * t.ld_b + k0_b;
    __builtin_amdgcn_global_load_lds(g + t.voff[i & 1], (lds_ptr)(l + i * 1024), 16, 0, 0);
  }
}

template <int MT, int NT>
struct Frags {
  bf16x8 a[MT], b[NT];
};

// Operand fragments of 16-wide k step ks of a slab. Fragment rows are
// (multiple of 32) + lane%32, so the swizzle depends only on the lane: lane
// offset loff[ks] = (lane%32)*128 + (((2ks + lane/32) ^ (((lane%32) >> 1) & 7)) << 4)
// serves every fragment of both operands; the row block is a uniform term.
template <int MT, int NT>
__device__ __forceinline__ void load_frags(const char* la, const char* lb, int wm0, int wn0,
                                           int loff, Frags<MT, NT>& f) {
  const char* pa = la + wm0 * kRow + loff;
  const char* pb = lb + wn0 * kRow + loff;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) f.a[mi] = *reinterpret_cast<const bf16x8*>(pa + mi * 32 * kRow);
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) f.b[ni] = *reinterpret_cast<const bf16x8*>(pb + ni * 32 * kRow);
}

template <int MT, int NT>
__device__ __forceinline__ void mfma_frags(const Frags<MT, NT>& f, f32x16 (&acc)[MT][NT]) {
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
}

}  // namespace bf

// Maps a block to (group, local tile). With xcd_map the 8 XCDs (blocks are
// dealt to them round-robin by block index) each take a contiguous eighth of
// every group's tile list, so concurrently resident tiles on one XCD belong to
// the same few matrices and share operand rows in that XCD's L2 (this halves
// the L2-miss traffic of the apply on the 2B-shaped set).
__device__ __forceinline__ bool map_tile(const GemmArgs& args, int b, int& gi, int& local) {
  if (args.xcd_map) {
    const int xcd = b & 7;
    int slot = b >> 3;
    for (int i = 0; i < args.ngroups; ++i) {
      const int64_t tot = (int64_t)args.g[i].count * args.g[i].tiles_per_mat;
      const int lo = (int)((xcd * tot) >> 3), hi = (int)(((xcd + 1) * tot) >> 3);
      if (slot < hi - lo) {
        gi = i;
        local = lo + slot;
        return true;
      }
      slot -= hi - lo;
    }
    return false;
  }
  gi = 0;
  for (int i = 1; i < args.ngroups; ++i)
    if (b >= args.g[i].tile_begin) gi = i;
  local = b - args.g[gi].tile_begin;
  return true;
}

// Tile coordinates of local tile t of a matrix. Symmetric modes walk the
// upper triangle row by row; the apply groups rows in bands of 4 tile rows
// (4 x 8 = 32 consecutive tiles share 4 B row-blocks and 8 X^T row-blocks).
template <bool kSym>
__device__ __forceinline__ void tile_coords(const GemmGroup& g, int t, int& bi, int& bj) {
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
    constexpr int kBand = 4;
    const int gsz = kBand * g.tn;
    const int band = t / gsz;
    const int first = band * kBand;
    const int gm = g.tm - first < kBand ? g.tm - first : kBand;
    const int rr = t - band * gsz;
    bi = first + rr % gm;
    bj = rr / gm;
  }
}

// 4x4 transpose of bf16 values within each quad of lanes. Lane k of a quad
// holds 4 consecutive rows of column k (d0 = rows 0|1, d1 = rows 2|3, low
// half first); afterwards it holds columns 0..3 of row k. Two rounds of DPP
// quad permutes: 2x2 transposes of 16-bit halves between lanes k and k^1,
// then an exchange of dwords between lanes k and k^2.
__device__ __forceinline__ void quad_transpose(uint32_t& d0, uint32_t& d1, int lane) {
  const int k = lane & 3;
  const uint32_t x0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  const uint32_t x1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0xB1, 0xF, 0xF, false);
  if ((k & 1) == 0) {
    d0 = (d0 & 0xFFFFu) | (x0 << 16);
    d1 = (d1 & 0xFFFFu) | (x1 << 16);
  } else {
    d0 = (x0 >> 16) | (d0 & 0xFFFF0000u);
    d1 = (x1 >> 16) | (d1 & 0xFFFF0000u);
  }
  const uint32_t send = (k & 2) ? d0 : d1;
  const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  if (k & 2) d0 = recv;
  else d1 = recv;
}

// Main loop of one group of the ping-pong schedule (see k_ns_gemm_bf16).
// Both groups execute the same sequence of barriers; G selects the role.
//
// Plain bf16: a slab is 64 logical k; chunk ch holds k steps 2ch and 2ch+1
// (fragments fa, fb); each 32x32 block takes 2 MFMAs per chunk.
// SPLIT (split-bf16 operands, each 128-byte slab row = 32 hi + 32 lo values
// of 32 logical k): chunk ch is k step ch, fa its hi and fb its lo
// fragments; each block takes hi*hi + hi*lo + lo*hi (3 MFMAs per chunk).
//
// With E_TERM, the fp32 term seed*E (apply: E = X, seed = a; polynomial:
// E = A, seed = b/c) is added to the accumulators on the way: element
// (i, j) of E is element (j, i) of the Q operand (X^T, or A itself, which
// is symmetric), so the E tile streams through the LDS ring as part of Q's
// slabs with k in [256*bi, 256*bi + 256). When a wave loads a chunk of that
// K range, it also reads, for the accumulator rows the chunk covers, its 4
// consecutive k values per column (one 8-byte LDS read per 4 elements, two
// with SPLIT: E = hi + lo).
template <int G, int MT, int NT, bool E_TERM, bool SPLIT>
__device__ __forceinline__ void pingpong(const bf::StageSrc& src, int wave, int nk, char* s0,
                                         char* s1, int wm0, int wn0, const int (&loff)[bf::kKS],
                                         int lane, int bi, float seed, f32x16 (&acc)[MT][NT]) {
  using namespace bf;
  constexpr int kW = SPLIT ? 16 : 32;   // logical k per chunk
  constexpr int kSW = SPLIT ? 32 : 64;  // logical k per slab
  Frags<MT, NT> fa, fb;
  auto take_e = [&](const char* buf, int kt, int ch) {
    // first accumulator row (relative to wm0) whose E value sits in this chunk
    const int r = kt * kSW + ch * kW - 256 * bi - wm0;
    if (r < 0 || r >= MT * 32) return;
    const char* lb = buf + kSlabA;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int row = mi * 32 + 8 * rg;  // rows row + 4*(lane/32) + q, q < 4
        if (row < r || row >= r + kW) continue;
        const int kk = ch * kW + (row - r) + 4 * (lane >> 5);  // logical k within the slab
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          const int qrow = wn0 + ni * 32 + (lane & 31);
          const bf16x4 hv =
              *reinterpret_cast<const bf16x4*>(lb + bf::swz(qrow, kk >> 3) + ((kk & 7) << 1));
          float e[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = (float)hv[q];
          if (SPLIT) {
            const bf16x4 lv =
                *reinterpret_cast<const bf16x4*>(lb + bf::swz(qrow, 4 + (kk >> 3)) + ((kk & 7) << 1));
#pragma unroll
            for (int q = 0; q < 4; ++q) e[q] += (float)lv[q];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[mi][ni][rg * 4 + q] = fmaf(seed, e[q], acc[mi][ni][rg * 4 + q]);
        }
      }
  };
  auto load = [&](const char* buf, int ch, int kt) {
    load_frags<MT, NT>(buf, buf + kSlabA, wm0, wn0, loff[SPLIT ? ch : 2 * ch], fa);
    load_frags<MT, NT>(buf, buf + kSlabA, wm0, wn0, loff[SPLIT ? ch + 2 : 2 * ch + 1], fb);
    if (E_TERM) take_e(buf, kt, ch);
  };
  auto mul = [&]() {
    if (SPLIT) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb.a[mi], fa.b[ni], acc[mi][ni], 0, 0, 0);
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa.a[mi], fb.b[ni], acc[mi][ni], 0, 0, 0);
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa.a[mi], fa.b[ni], acc[mi][ni], 0, 0, 0);
        }
    } else {
      mfma_frags<MT, NT>(fa, acc);
      mfma_frags<MT, NT>(fb, acc);
    }
  };
  // phase 0: group 0 loads chunk 0 of stage 0
  if (G == 0) load(s0, 0, 0);
  phase_barrier();
  auto stage = [&](int kt, char* buf, char* nxt) {
    if (G == 0) mul(); else load(buf, 0, kt);                   // 4s+1
    phase_barrier();
    if (G == 0) load(buf, 1, kt); else mul();                   // 4s+2
    phase_barrier();
    if (G == 0) mul(); else load(buf, 1, kt);                   // 4s+3
    wait_vmcnt<0>();
    phase_barrier();
    if (kt + 2 < nk) issue_stage(src, wave, (int64_t)(kt + 2) * kRow, buf);  // 4s+4
    if (G == 0) {
      if (kt + 1 < nk) load(nxt, 0, kt + 1);
    } else {
      mul();
    }
    phase_barrier();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    stage(kt, s0, s1);
    stage(kt + 1, s1, s0);
  }
}

template <int MODE, int WGM, int WGN, bool SPLIT>
__global__ __launch_bounds__(WGM * WGN * 64, (WGM * WGN) / 4) void k_ns_gemm_bf16(GemmArgs args) {
  using namespace bf;
  using C = Cfg<WGM, WGN>;
  constexpr int kWGN = WGN, kWTM = C::kWTM, kWTN = C::kWTN, kMT = C::kMT, kNT = C::kNT;
  constexpr bool kSym = (MODE != kApply);
  __shared__ __attribute__((aligned(1024))) char s0[kSlabA + kSlabB];
  __shared__ __attribute__((aligned(1024))) char s1[kSlabA + kSlabB];

  const int tid = threadIdx.x;
  // The wave index is uniform across a wave; readfirstlane lets the compiler
  // know, so that branches on it are scalar branches.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWGN, wn = wave - (wave / kWGN) * kWGN;

  int gi, local;
  if (!map_tile(args, blockIdx.x, gi, local)) return;
  const GemmGroup& g = args.g[gi];
  const int mat = local / g.tiles_per_mat;
  int bi, bj;
  tile_coords<kSym>(g, local - mat * g.tiles_per_mat, bi, bj);

  const char* blk = g.base + (int64_t)mat * g.mat_bytes;
  // Row pitch in bytes: 2 per logical element, 4 with split operands.
  constexpr int kEB = SPLIT ? 4 : 2;
  const int64_t ldp_b = (int64_t)g.ldp * kEB, ldq_b = (int64_t)g.ldq * kEB;
  const char* P = blk + g.offP + (int64_t)bi * kBM * ldp_b;
  const char* Q = blk + g.offQ + (int64_t)bj * kBN * ldq_b;

  f32x16 acc[kMT][kNT];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNT; ++ni) acc[mi][ni] = f32x16{};

  const int nk = g.K / (SPLIT ? 32 : 64);  // slabs; even, since K is a multiple of kPad
  const int wm0 = wm * kWTM, wn0 = wn * kWTN;
  // Ping-pong schedule. Stage s (a 64-wide K slab, full 128-byte rows) lives
  // in buffer s % 2 and is consumed in two chunks of two 16-wide k steps.
  // Waves 0-3 (group 0) and 4-7 (group 1) -- one of each per SIMD -- take
  // turns: in every phase one group issues a cluster of 16 MFMAs while the
  // other loads its next chunk's fragments from LDS, so each SIMD's matrix
  // core always has a wave feeding it. Phases are separated by barriers.
  // Phase 0: g0 loads chunk 0 of stage 0. Then per stage s:
  //   4s+1: g0 multiplies chunk 0, g1 loads chunk 0
  //   4s+2: g0 loads chunk 1, g1 multiplies chunk 0
  //   4s+3: g0 multiplies chunk 1, g1 loads chunk 1; every wave then waits
  //         for its loads of stage s+1, so the next barrier publishes it
  //   4s+4: loads of stage s+2 into buffer s % 2 (last read in 4s+3);
  //         g0 loads chunk 0 of stage s+1, g1 multiplies chunk 1.
  // Stage s+2's loads thus have one stage of time to land.
  int loff[kKS];
  {
    const int r = lane & 31, y = (lane >> 5) ^ ((r >> 1) & 7);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) loff[ks] = r * kRow + (((2 * ks) ^ y) << 4);
  }
  const StageSrc src = stage_src(P, Q, ldp_b, ldq_b, wave, lane);
  issue_stage(src, wave, 0, s0);
  issue_stage(src, wave, kRow, s1);
  wait_vmcnt<8>();
  phase_barrier();
  const float seed = MODE == kApply ? args.c0 : MODE == kPoly ? args.c0 / args.c1 : 0.f;
  if (wave < 4)
    pingpong<0, kMT, kNT, MODE != kGram, SPLIT>(src, wave, nk, s0, s1, wm0, wn0, loff, lane, bi,
                                                seed, acc);
  else
    pingpong<1, kMT, kNT, MODE != kGram, SPLIT>(src, wave, nk, s0, s1, wm0, wn0, loff, lane, bi,
                                                seed, acc);

  // ---- epilogue. The E term is already in the accumulators (the
  // polynomial's still needs its factor c). Outputs leave through the idle
  // LDS ring, one 256x256 bf16 pass per layout (row-major, then transposed;
  // with SPLIT one pass for the hi and one for the lo parts of each) so
  // that every global store is a coalesced 16-byte store.
  const float scale = MODE == kPoly ? args.c1 : 1.f;
  bf16x4 vh[kMT][kNT][4], vl[kMT][kNT][4];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNT; ++ni)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 h, l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = scale * acc[mi][ni][rg * 4 + q];
          h[q] = (__bf16)v;
          if (SPLIT) l[q] = (__bf16)(v - (float)h[q]);
        }
        vh[mi][ni][rg] = h;
        if (SPLIT) vl[mi][ni][rg] = l;
      }

  // The two 64 KB ring buffers hold 128 rows of 512 B each of the staging
  // tile; ring(q) is the 32 KB quarter holding rows [64q, 64q + 64).
  auto ring = [&](int q) -> char* { return (q < 2 ? s0 : s1) + (q & 1) * 32768; };
  char* O1 = g.offO1 < 0 ? nullptr : const_cast<char*>(blk) + g.offO1;
  char* O2 = g.offO2 < 0 ? nullptr : const_cast<char*>(blk) + g.offO2;
  char* OT = kSym ? (bi != bj ? O1 : nullptr) : O2;  // transposed destination
  const int64_t ld1_b = (int64_t)g.ldo1 * kEB, ldT_b = (int64_t)(kSym ? g.ldo1 : g.ldo2) * kEB;
  // Byte offset, within a row, of the 16-byte chunk holding logical columns
  // col .. col+7 (col a multiple of 8): plain rows are dense bf16; split rows
  // are 128-byte blocks of 32 hi then 32 lo values.
  auto col_off = [&](int col, bool lo) -> int64_t {
    if (!SPLIT) return (int64_t)col * 2;
    return (int64_t)(col >> 5) * 128 + ((col & 31) << 1) + (lo ? 64 : 0);
  };

  // Row-major pass into O1: LDS tile [row][col], 16-byte chunk c of row r
  // stored at position c ^ (r & 31). A quad transpose first gives each lane
  // 4 consecutive columns of one row, so the LDS writes are 8-byte writes.
  auto pass_rows = [&](const bf16x4 (&v)[kMT][kNT][4], bool lo) {
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNT; ++ni) {
        const int col = wn0 + ni * 32 + (lane & 28);  // first of the quad's 4 columns
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int row = wm0 + mi * 32 + 8 * rg + 4 * (lane >> 5) + (lane & 3);
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          u32x2 d = __builtin_bit_cast(u32x2, v[mi][ni][rg]);
          uint32_t d0 = d.x, d1 = d.y;
          quad_transpose(d0, d1, lane);
          d.x = d0;
          d.y = d1;
          char* base = ring(row >> 6) + (row & 63) * 512;
          const int off = ((((col >> 3) ^ (row & 31)) << 4) | ((col & 7) << 1));
          *reinterpret_cast<u32x2*>(base + off) = d;
        }
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = tid + i * C::kThreads;  // 0 .. 8191
      const int row = id >> 5, c = id & 31;
      const u32x4 d = *reinterpret_cast<const u32x4*>(ring(row >> 6) + (row & 63) * 512 +
                                                      ((c ^ (row & 31)) << 4));
      *reinterpret_cast<u32x4*>(O1 + (int64_t)(bi * kBM + row) * ld1_b +
                                col_off(bj * kBN + c * 8, lo)) = d;
    }
  };
  // Transposed pass into OT: LDS tile [col][row], 16-byte chunk c of LDS
  // row j stored at position c ^ (j & 31).
  auto pass_cols = [&](const bf16x4 (&v)[kMT][kNT][4], bool lo) {
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNT; ++ni) {
        const int col = wn0 + ni * 32 + (lane & 31);
        char* base = ring(col >> 6) + (col & 63) * 512;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int row0 = wm0 + mi * 32 + 8 * rg + 4 * (lane >> 5);
          const int off = ((((row0 >> 3) ^ (col & 31)) << 4) | ((row0 & 7) << 1));
          *reinterpret_cast<bf16x4*>(base + off) = v[mi][ni][rg];
        }
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = tid + i * C::kThreads;
      const int j = id >> 5, c = id & 31;
      const u32x4 d = *reinterpret_cast<const u32x4*>(ring(j >> 6) + (j & 63) * 512 +
                                                      ((c ^ (j & 31)) << 4));
      *reinterpret_cast<u32x4*>(OT + (int64_t)(bj * kBN + j) * ldT_b +
                                col_off(bi * kBM + c * 8, lo)) = d;
    }
  };
  if (O1) {
    pass_rows(vh, false);
    if (SPLIT) pass_rows(vl, true);
  }
  if (OT) {
    pass_cols(vh, false);
    if (SPLIT) pass_cols(vl, true);
  }
}

// fp32 debug path: the generic 128x128 kernel with 4 waves (2 x 2).
constexpr int kTile32 = 128;

template <typename T, int MODE>
hipError_t launch_t(const GemmArgs& a, hipStream_t s, bool split) {
  if constexpr (std::is_same<T, __bf16>::value) {
    // bf16: 256x256 tiles, 8 waves in a 2 x 4 grid (wave tile 128 x 64).
    if (split)
      hipLaunchKernelGGL((k_ns_gemm_bf16<MODE, 2, 4, true>), dim3(a.grid), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((k_ns_gemm_bf16<MODE, 2, 4, false>), dim3(a.grid), dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_ns_gemm<T, kTile32, kTile32, 2, 2, MODE>), dim3(a.ntiles), dim3(256), 0,
                       s, a);
  }
  return hipGetLastError();
}

}  // namespace

int gemm_tile(NsPrec prec) { return prec == kFp32 ? kTile32 : bf::kBM; }

hipError_t launch_gemm(GemmMode mode, NsPrec prec, const GemmArgs& a, hipStream_t s) {
  if (a.ntiles <= 0) return hipSuccess;
  const bool split = prec == kSplitBf16;
  if (prec == kFp32) {
    switch (mode) {
      case kGram: return launch_t<float, kGram>(a, s, false);
      case kPoly: return launch_t<float, kPoly>(a, s, false);
      case kApply: return launch_t<float, kApply>(a, s, false);
    }
  } else {
    switch (mode) {
      case kGram: return launch_t<__bf16, kGram>(a, s, split);
      case kPoly: return launch_t<__bf16, kPoly>(a, s, split);
      case kApply: return launch_t<__bf16, kApply>(a, s, split);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace muonh
