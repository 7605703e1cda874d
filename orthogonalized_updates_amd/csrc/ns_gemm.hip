// Newton-Schulz GEMMs of the MuonH step on gfx950 MFMA.
//
// The digest page "Puro-2B trains for $6.9K, attention sinks hit 99%,
// LoopArena tops at 24.69%" (footnote 4) names the Newton-Schulz iterations as
// where Muon's cost goes. Per iteration, on the short-side-first operand X
// (s x l, zero-padded) the step computes
//   A = X X^T                  (symmetric: upper tiles only, mirrored)
//   B = b A + c A A            (A symmetric, so A A = A A^T: same kernel shape)
//   X <- a X + B X             (operands: rows of B, and X itself read K-major)
// so every product is C[i][j] = sum_k P[i][k] Q[k][j].
//
// Every launch covers one phase for all matrices of up to 16 shape groups:
// one workgroup per output tile, tiles dealt to the 8 XCDs in contiguous runs.
// bf16 and split bf16 (the product path): operands stored panel-major (256
// rows x 64 bytes per panel), 256x256 tiles, 8 waves in two groups that take
// turns between MFMA clusters (bf16: v_mfma_f32_16x16x32_bf16; split:
// v_mfma_f32_32x32x16_bf16; fp32 accumulation) and LDS fragment loads plus
// LDS DMA refills (global_load_lds_dwordx4) of a 4-stage ring of 32 KB
// stages. The apply reads its X operand K-major with
// transposed LDS reads (ds_read_b64_tr_b16), so X has one layout; the fp32
// a*X or b*A term is folded into the accumulators from the operand stream.
// Row-major outputs are stored straight from registers; transposed ones
// (mirrored tiles, O of tall matrices) too in the bf16 kernel (after a lane
// exchange), and staged through the idle ring in the split one. Where the
// polynomial is folded (B' = a*I + B), the apply has no a*X term.
// In the bf16 kernel, diagonal tiles of the symmetric products compute three
// quadrants and mirror the fourth, and the last positions of every XCD's
// tile list are claimed at run time (tail balancing, see GemmArgs::sched).
// Phases with few tiles (a single matrix or a few small ones) run the same
// kernel on 128x128 tiles (GemmArgs::small): 4 waves in two groups, the same
// 64-byte panel rows (half of a 256-row panel per tile), a ring of 16 KB
// stages.
// fp32 debug: a simpler 128x128 kernel on v_mfma_f32_32x32x2f32 with
// register-staged double buffering and direct epilogue stores; it reads both
// operands along K, so that mode keeps X and X^T copies.
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
            if (g.fold && row0 + q == col) v[q] += args.diag;
          } else {
            v[q] = E ? fmaf(c0, ld_f(E + (int64_t)(row0 + q) * g.lde + col), a) : a;
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
// bf16 and split-bf16 pipeline.
//
// Operands are stored panel-major: a matrix of R x K logical elements (both
// multiples of 256) is a grid of (R/256) x (K/kPK) panels of 256 rows x 64
// bytes, panel (rb, kb) at (rb * (K/kPK) + kb) * 16 KB, panel row r at r*64.
// A 64-byte panel row holds kPK = 32 bf16 values, or in split mode 16 hi
// values followed by the 16 matching lo values (kPK = 16). One K-stage of a
// 256x256 tile is thus one contiguous 16 KB panel per operand: stages move
// into LDS in whole cache lines however small they are, and a 4-stage ring of
// 32 KB stages leaves each refill 4-5 phases to land.
//
// 8 waves (2 x 4, wave tile 128 x 64) form two groups of 4, one wave of each
// per SIMD. They take turns phase by phase: one group issues its MFMA cluster
// for a stage while the other reads the next stage's fragments from LDS and
// then issues a quarter of the ring refill (LDS DMA, global_load_lds_dwordx4,
// 4 instructions per wave). MFMA waves issue no memory instructions, so a DMA
// queue that backs up never holds back the matrix cores.
// ---------------------------------------------------------------------------
namespace bf {

constexpr int kBM = 256, kBN = 256;
constexpr int kPRow = 64;               // bytes per panel row
constexpr int kPanel = 256 * kPRow;     // 16 KB: one operand's share of a stage
constexpr int kStage = 2 * kPanel;      // A panel, then B panel
constexpr int kNBuf = 4;                // stages in the LDS ring

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

// Chunk (16 B) c of panel row r sits at r*64 + ((c ^ ((r >> SH) & 3)) << 4).
// The shift matches the fragment reads of each kernel, measured with an LDS
// probe (8 waves per CU, ds_read_b128): a 32x32x16 fragment read (32 rows,
// 2 chunks) is conflict-free with SH = 2, a 16x16x32 read (16 rows, 4
// chunks) with SH = 1, and each runs at half the rate (8 instead of 4.3
// cycles per instruction per CU, two-way bank conflicts) with the other.
template <int SH = 2>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kPRow + ((chunk ^ ((row >> SH) & 3)) << 4);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Phase barrier of the ping-pong schedule: wait until at most VM of this
// wave's vector memory operations are outstanding (63: no wait) and its LDS
// reads have retired (so a buffer may be refilled after the barrier), then
// s_barrier. __syncthreads() would also drain every DMA still in flight. The
// empty asm statements keep the compiler from moving memory accesses across,
// the scheduling barriers keep any instruction (MFMAs included) from
// migrating between phases.
template <int VM = 63>
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4));  // vmcnt(VM) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// phase_barrier with vmcnt(4n), n in {0, 1, 2} (wave-uniform).
__device__ __forceinline__ void phase_barrier_n(int n) {
  if (n >= 2) phase_barrier<8>();
  else if (n == 1) phase_barrier<4>();
  else phase_barrier<0>();
}

// One wave's share of a refill: 64 rows (4 KB) of one operand panel, as 4
// DMA instructions of 16 rows (1 KB, contiguous in the panel). Group 1
// (waves 4-7; 2-3 for 128-row tiles) refills the A panels, group 0 the B
// panels; wave w takes rows 64*(w%4) .. +63 (64*(w%2) for 128-row tiles,
// within the tile's half of the panel). Lane l fills LDS bytes 16l ..
// 16l+15 of an instruction's 1 KB block: panel row l/4 of the instruction's
// 16, position l%4, which must hold chunk (l%4) ^ ((row >> SH) & 3); for
// every instruction of every wave (row >> SH) & 3 = (l >> (2 + SH)) & 3, so
// the per-lane source offset is fixed.
struct DmaSrc {
  const char* g;  // per-lane source address of instruction 0, stage 0
  uint32_t lds;   // LDS offset of this wave's share within a stage buffer
};

// TM: tile rows (256, or 128 with 4 waves: group 1 is waves 2-3, a stage's
// B half starts at TM rows).
template <int SH = 2, int TM = 256>
__device__ __forceinline__ DmaSrc dma_src(const char* P, const char* Q, int wave, int lane) {
  constexpr int kWPG = TM / 64;  // waves per group
  const bool isA = wave >= kWPG;
  DmaSrc d;
  d.g = (isA ? P : Q) + (wave & (kWPG - 1)) * 4096 + (lane >> 2) * kPRow +
        (((lane & 3) ^ ((lane >> (2 + SH)) & 3)) << 4);
  d.lds = (uint32_t)((isA ? 0 : TM * kPRow) + (wave & (kWPG - 1)) * 4096);
  return d;
}

// Issue this wave's share of stage kt into the ring buffer at LDS offset
// `buf`. Written as inline asm: the compiler then does not track these LDS
// writes (its own tracking put full vmcnt waits in front of reads of other
// buffers); the schedule's explicit vmcnt waits and barriers order them. The
// instruction has no register results, so nothing in flight can land in a
// register the compiler has reused.
__device__ __forceinline__ void issue_share(const DmaSrc& d, int kt, uint32_t buf) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const char* g = d.g + (int64_t)kt * kPanel + i * 1024;
    const uint32_t m0 = buf + d.lds + i * 1024;
    // M0 (the LDS destination) is an input operand; the s_nop covers the
    // wait state an LDS DMA needs after M0 is written.
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
  }
}

// Q operand of the apply (QT: Q is X itself, read K-major). A stage holds
// rows k in [kPK*kt, kPK*kt + kPK) of X and the tile's 256 columns: 256/kPK
// pieces of kPK rows x 64 bytes, one per column panel, each contiguous in X
// (kPK*64 = 2 KB for bf16, 1 KB for split). Piece p lands at p*kPK*64 in the
// stage's B panel, rows unswizzled: a transposed fragment read (4 rows x 16
// columns per 16 lanes) then covers whole 256-byte bank windows. In split
// mode the two 16-lane groups of a read fall on consecutive pieces, so odd
// pieces store their two 32-byte halves swapped (chunk ^ 2) to keep the two
// groups on different banks. Group 0 refills these; wave w takes the 16
// 1 KB instructions 4*(w%4) .. 4*(w%4)+3 of the stage (128 columns: the 8
// instructions 4*(w%2) .. +3).
struct QtSrc {
  const char* g[2];  // per-lane source of even / odd instructions, tile column block included
  int64_t rbs;       // bytes per 256-row block of X
  uint32_t lds;      // LDS offset of this wave's instructions within a stage buffer
};

template <bool SPLIT>
__device__ __forceinline__ QtSrc qt_src(const char* X, int ldx, int bj, int wave, int lane) {
  constexpr int kPK = SPLIT ? 16 : 32;
  QtSrc d;
  const char* base = X + (int64_t)bj * (256 / kPK) * kPanel;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int lo = SPLIT ? (lane >> 2) * kPRow + (((lane & 3) ^ (2 * par)) << 4) : lane * 16;
    d.g[par] = base + lo;
  }
  d.rbs = (int64_t)(ldx / kPK) * kPanel;
  d.lds = (uint32_t)(kPanel + (wave & 3) * 4096);
  return d;
}

template <bool SPLIT, int TM = 256>
__device__ __forceinline__ void issue_share_qt(const QtSrc& d, int wave, int kt, uint32_t buf) {
  constexpr int kPK = SPLIT ? 16 : 32;
  const int k0 = kt * kPK;
  const int64_t row_part = (int64_t)(k0 >> 8) * d.rbs + (k0 & 255) * kPRow;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * (wave & (TM / 64 - 1)) + i;  // instruction of the stage
    // bf16: piece j/2, its half j%2 (16 rows each); split: piece j
    const int64_t piece = SPLIT ? (int64_t)j * kPanel : (int64_t)(j >> 1) * kPanel + (j & 1) * 1024;
    const char* g = d.g[i & 1] + row_part + piece;
    const uint32_t m0 = buf + d.lds + i * 1024;
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

// ds_read_b64_tr_b16: in each 16-lane group, lanes 4r .. 4r+3 name row r's
// 16 consecutive values (4 each); lane i receives column i of the 4 rows.
__device__ __forceinline__ bf16x4 read_tr(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(lds_ptr)p);
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 x, bf16x4 y) {
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

template <int MT, int NT>
struct Frags {
  bf16x8 a[MT], b[NT];
};

// Operand fragments of one k half of a stage. Fragment rows are (multiple
// of 32) + lane%32, so the swizzle depends only on the lane: the lane offset
// loff = (lane%32)*64 + ((c ^ ((lane%32 >> 2) & 3)) << 4), with chunk
// c = 2h + lane/32, serves every fragment of both operands.
template <int MT, int NT>
__device__ __forceinline__ void load_frags(const char* la, const char* lb, int wm0, int wn0,
                                           int loff, Frags<MT, NT>& f) {
  const char* pa = la + wm0 * kPRow + loff;
  const char* pb = lb + wn0 * kPRow + loff;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) f.a[mi] = *reinterpret_cast<const bf16x8*>(pa + mi * 32 * kPRow);
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) f.b[ni] = *reinterpret_cast<const bf16x8*>(pb + ni * 32 * kPRow);
}

// B fragments of a QT stage (see qt_src): lane l needs 8 consecutive k of
// column n = (wn0 + 32 ni) + l%32, k = 8*(l/32) + 16h (bf16, k half h) or
// 8*(l/32) (split: h = 0 hi, h = 1 lo). Two transposed reads give k .. k+3
// and k+4 .. k+7; qoff[h] is the lane's part of the address.
template <int NT, bool SPLIT>
__device__ __forceinline__ void load_frags_qt(const char* lb, int wn0, int qoff, bf16x8 (&b)[NT]) {
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) {
    const char* p = lb + (SPLIT ? ((wn0 + 32 * ni) >> 4) * 1024 : ((wn0 + 32 * ni) >> 5) * 2048) + qoff;
    b[ni] = cat8(read_tr(p), read_tr(p + 4 * kPRow));
  }
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
// upper triangle row by row; the apply groups rows in bands of 8 tile rows
// (8 x 4 = 32 consecutive tiles share 8 B row-blocks and 4 column blocks of
// X; for s = 2048 a band is a whole column of tiles, so each column block of
// X streams through the L2 once). With the conflict-free fragment reads this
// ran the apply 0.9 % faster in the 2B step than bands of 4 (1.6 % on the 84
// x 2048x6144 launches) for 2 % more HBM reads; before that change bands of 8
// were no faster and read 23 % more.
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
    constexpr int kBand = 8;
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
// A stage is one panel per operand: 32 logical k for bf16 (two 16-wide k
// steps: fragments fa and fb, 2 MFMAs per 32x32 block), 16 for split bf16
// (one k step: fa holds the hi, fb the lo parts; 3 MFMAs per block,
// hi*hi + hi*lo + lo*hi, the small terms first).
//
// With E_TERM, the fp32 term seed*E (apply: E = X, seed = a; polynomial:
// E = A, seed = b/c) is added to the accumulators on the way: element
// (i, j) of E is element (j, i) of the Q operand (X^T, or A itself, which
// is symmetric), so the E tile streams through the LDS ring as part of Q's
// panels with k in [256*bi, 256*bi + 256). When a wave loads a stage of that
// K range, it also reads, for the accumulator rows the stage covers, their 4
// consecutive k values per column (one 8-byte LDS read per 4 elements, two
// with split operands: E = hi + lo).
// Lane parts of the LDS addresses a wave reads (see k_ns_gemm_bf16).
struct LaneOffs {
  int f[2];   // A fragments (and B fragments unless QT), k half / hi-lo h
  int q[2];   // QT: transposed B fragment reads, h as above
  int e[2];   // QT: transposed E reads, hi and lo
};

template <int G, int MT, int NT, bool E_TERM, bool SPLIT, bool QT>
__device__ __forceinline__ void pingpong(const bf::DmaSrc& dsrc, const bf::QtSrc& qsrc, int nk,
                                         const char* ring, uint32_t ring_lds, int wave, int wm0,
                                         int wn0, const LaneOffs& lo, int lane, int bi, float seed,
                                         f32x16 (&acc)[MT][NT]) {
  using namespace bf;
  constexpr int kW = SPLIT ? 16 : 32;  // logical k per stage
  Frags<MT, NT> fa, fb;
  auto take_e = [&](const char* buf, int kt) {
    // first accumulator row (relative to wm0) whose E value sits in this stage
    const int r = kt * kW - 256 * bi - wm0;
    if (r < 0 || r >= MT * 32) return;
    const char* lb = buf + kPanel;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int row = mi * 32 + 8 * rg;  // rows row + 4*(lane/32) + q, q < 4
        if (row < r || row >= r + kW) continue;
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          float e[4];
          if (QT) {
            // E = X: stage row k = accumulator row, read 4 rows of the lane's
            // column with one transposed read (two with split operands)
            const char* pe = lb + (SPLIT ? ((wn0 + 32 * ni) >> 4) * 1024 : ((wn0 + 32 * ni) >> 5) * 2048) +
                             (row - r) * kPRow;
            const bf16x4 hv = read_tr(pe + lo.e[0]);
#pragma unroll
            for (int q = 0; q < 4; ++q) e[q] = (float)hv[q];
            if (SPLIT) {
              const bf16x4 lv = read_tr(pe + lo.e[1]);
#pragma unroll
              for (int q = 0; q < 4; ++q) e[q] += (float)lv[q];
            }
          } else {
            const int kk = (row - r) + 4 * (lane >> 5);  // logical k within the stage
            const int qrow = wn0 + ni * 32 + (lane & 31);
            const bf16x4 hv =
                *reinterpret_cast<const bf16x4*>(lb + bf::swz(qrow, kk >> 3) + ((kk & 7) << 1));
#pragma unroll
            for (int q = 0; q < 4; ++q) e[q] = (float)hv[q];
            if (SPLIT) {
              const bf16x4 lv = *reinterpret_cast<const bf16x4*>(
                  lb + bf::swz(qrow, 2 + (kk >> 3)) + ((kk & 7) << 1));
#pragma unroll
              for (int q = 0; q < 4; ++q) e[q] += (float)lv[q];
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[mi][ni][rg * 4 + q] = fmaf(seed, e[q], acc[mi][ni][rg * 4 + q]);
        }
      }
  };
  auto load = [&](int kt) {
    const char* buf = ring + (kt & (kNBuf - 1)) * kStage;
    if (QT) {
      const char* pa = buf + wm0 * kPRow;
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        fa.a[mi] = *reinterpret_cast<const bf16x8*>(pa + mi * 32 * kPRow + lo.f[0]);
        fb.a[mi] = *reinterpret_cast<const bf16x8*>(pa + mi * 32 * kPRow + lo.f[1]);
      }
      load_frags_qt<NT, SPLIT>(buf + kPanel, wn0, lo.q[0], fa.b);
      load_frags_qt<NT, SPLIT>(buf + kPanel, wn0, lo.q[1], fb.b);
    } else {
      load_frags<MT, NT>(buf, buf + kPanel, wm0, wn0, lo.f[0], fa);
      load_frags<MT, NT>(buf, buf + kPanel, wm0, wn0, lo.f[1], fb);
    }
    if (E_TERM && seed != 0.f) take_e(buf, kt);
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
  auto refill = [&](int kt) {
    const uint32_t buf = ring_lds + (kt & (kNBuf - 1)) * kStage;
    if (QT && G == 0) issue_share_qt<SPLIT>(qsrc, wave, kt, buf);
    else issue_share(dsrc, kt, buf);
  };
  // Phase 0: group 0 loads stage 0. Then per stage s:
  //   2s+1: g0 multiplies stage s; g1 loads stage s, then refills its half of
  //         stage s+3 (buffer of stage s-1, read by both groups before). At
  //         the end every wave waits for its share of stage s+1: the only
  //         refills it issued after that share are those of s+2 and s+3.
  //   2s+2: g0 loads stage s+1, then refills its half of stage s+4 (buffer of
  //         stage s, read by g1 in 2s+1); g1 multiplies stage s.
  // Stages 0-3 are issued before the loop; refills of stage t are issued in
  // phases 2t-6 (B half) and 2t-5 (A half) and waited for at the end of 2t-1.
  if (G == 0) load(0);
  phase_barrier<>();
  for (int s = 0; s < nk; ++s) {
    if (G == 0) {
      mul();
    } else {
      load(s);
      if (s >= 1 && s + 3 < nk) refill(s + 3);
    }
    phase_barrier_n((s + 2 < nk) + (s + 3 < nk));
    if (G == 0) {
      if (s + 1 < nk) load(s + 1);
      if (s + 4 < nk) refill(s + 4);
    } else {
      mul();
    }
    phase_barrier<>();
  }
}

// The 32x32x16 kernel. The library launches it for split-bf16 operands; the
// plain bf16 instantiation (SPLIT = false) is the reference the 16x16x32
// kernel below (k_ns_gemm_m16) was checked against, bit for bit.
template <int MODE, int WGM, int WGN, bool SPLIT>
__global__ __launch_bounds__(WGM * WGN * 64, (WGM * WGN) / 4) void k_ns_gemm_bf16(GemmArgs args) {
  using namespace bf;
  using C = Cfg<WGM, WGN>;
  constexpr int kWGN = WGN, kWTM = C::kWTM, kWTN = C::kWTN, kMT = C::kMT, kNT = C::kNT;
  constexpr bool kSym = (MODE != kApply);
  __shared__ __attribute__((aligned(1024))) char ring[kNBuf * kStage];

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
  // Bytes per logical element: 2, or 4 with split operands (hi + lo). A row
  // block of 256 rows is ld * 256 * kEB bytes of consecutive panels.
  constexpr int kEB = SPLIT ? 4 : 2;
  constexpr int kPK = SPLIT ? 16 : 32;  // logical k per panel
  // The apply reads its Q operand X K-major (QT): Q is then X's base and
  // the tile's column block is selected per piece.
  constexpr bool kQT = (MODE == kApply);
  const char* P = blk + g.offP + (int64_t)bi * kBM * g.ldp * kEB;
  const char* Q = blk + g.offQ + (kQT ? 0 : (int64_t)bj * kBN * g.ldq * kEB);

  f32x16 acc[kMT][kNT];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNT; ++ni) acc[mi][ni] = f32x16{};

  const int nk = g.K / kPK;  // stages; a multiple of 8, since K is a multiple of kPad
  const int wm0 = wm * kWTM, wn0 = wn * kWTN;
  // Lane parts of the LDS read addresses. Fragment reads (ds_read_b128):
  // row (multiple of 32) + lane%32, chunk 2h + lane/32, swizzled. QT
  // transposed reads: in 16-lane group gq = (lane/16)%2 of k group
  // kg = lane/32, lane i = lane%16 names row 8kg + i/4 (fragments, plus 16h
  // for bf16) or 4kg + i/4 (E), columns 16gq + 4(i%4) .. +3 of the tile's
  // column block: bf16 piece rows hold 32 columns; split pieces hold 16
  // (the group's own piece, hi then lo, halves swapped in odd pieces).
  LaneOffs lo;
  {
    const int r = lane & 31, f = (r >> 2) & 3, kg = lane >> 5, gq = (lane >> 4) & 1,
              i = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lo.f[h] = r * kPRow + (((2 * h + kg) ^ f) << 4);
      if (!SPLIT) {
        const int cb = (16 * gq + 4 * (i & 3)) * 2;
        lo.q[h] = (16 * h + 8 * kg + (i >> 2)) * kPRow + cb;
        lo.e[h] = (4 * kg + (i >> 2)) * kPRow + cb;
      } else {
        const int cb = gq * 1024 + (((((i & 3) >> 1) + 2 * h) ^ (2 * gq)) << 4) + (i & 1) * 8;
        lo.q[h] = (8 * kg + (i >> 2)) * kPRow + cb;
        lo.e[h] = (4 * kg + (i >> 2)) * kPRow + cb;
      }
    }
  }
  const DmaSrc dsrc = dma_src(P, Q, wave, lane);
  const QtSrc qsrc = qt_src<SPLIT>(Q, g.ldq, bj, wave, lane);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr)ring;
#pragma unroll
  for (int st = 0; st < kNBuf; ++st) {
    if (kQT && wave < 4) issue_share_qt<SPLIT>(qsrc, wave, st, ring_lds + st * kStage);
    else issue_share(dsrc, st, ring_lds + st * kStage);
  }
  phase_barrier<12>();  // this wave's share of stage 0 has landed
  // the E term: a*X in the apply (none where B carries a*I), (b/c)*A in the
  // polynomial
  const float seed = MODE == kApply ? (g.fold ? 0.f : args.c0)
                     : MODE == kPoly ? args.c0 / args.c1 : 0.f;
  if (wave < 4)
    pingpong<0, kMT, kNT, MODE != kGram, SPLIT, kQT>(dsrc, qsrc, nk, ring, ring_lds, wave, wm0,
                                                     wn0, lo, lane, bi, seed, acc);
  else
    pingpong<1, kMT, kNT, MODE != kGram, SPLIT, kQT>(dsrc, qsrc, nk, ring, ring_lds, wave, wm0,
                                                     wn0, lo, lane, bi, seed, acc);

  // ---- epilogue. The E term is already in the accumulators (the
  // polynomial's still needs its factor c). Every refill has landed (the last
  // wait of the main loop was vmcnt(0)). Outputs leave through the idle LDS
  // ring, one 256x256 bf16 pass per layout (row-major, then transposed; with
  // split operands one pass for the hi and one for the lo parts of each):
  // the tile's panels are one contiguous region of the output, written with
  // coalesced 16-byte stores.
  // The first iteration after the fused momentum + cast sees X0 unscaled:
  // A = sigma^2 Y Y^T, and the apply's a*Y + B*Y takes sigma.
  float scale = MODE == kPoly ? args.c1 : 1.f;
  if (MODE != kPoly && args.xnorm && g.defer) {
    const float sg = x0_sigma(args.xnorm[g.first + mat]);
    scale = MODE == kGram ? sg * sg : sg;
  }
  bf16x4 vh[kMT][kNT][4], vl[kMT][kNT][4];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNT; ++ni)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 h, l;
        const int row0 = wm0 + mi * 32 + 8 * rg + 4 * (lane >> 5);
        const int col = wn0 + ni * 32 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = scale * acc[mi][ni][rg * 4 + q];
          if (MODE == kPoly && g.fold && bi == bj && row0 + q == col) v += args.diag;
          h[q] = (__bf16)v;
          if (SPLIT) l[q] = (__bf16)(v - (float)h[q]);
        }
        vh[mi][ni][rg] = h;
        if (SPLIT) vl[mi][ni][rg] = l;
      }

  // The ring holds the 256 x 512 B staging tile: buffer q (32 KB) holds rows
  // [64q, 64q + 64).
  char* stg = const_cast<char*>(ring);
  auto srow = [&](int row) -> char* { return stg + (row >> 6) * kStage + (row & 63) * 512; };
  char* O1 = g.offO1 < 0 ? nullptr : const_cast<char*>(blk) + g.offO1;
  char* O2 = g.offO2 < 0 ? nullptr : const_cast<char*>(blk) + g.offO2;
  char* OT = kSym ? (bi != bj ? O1 : nullptr) : O2;  // transposed destination
  const int ldT = kSym ? g.ldo1 : g.ldo2;
  // Store a staged 256x256 tile to the panels of output rows 256*rb .. +255,
  // logical columns 256*cb .. +255, of a matrix with ld logical columns.
  auto store_tile = [&](char* O, int ld, int rb, int cb, bool lo) {
    char* region = O + (int64_t)rb * kBM * ld * kEB + (int64_t)cb * (256 / kPK) * kPanel;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = tid + i * C::kThreads;  // 16-byte chunk 0 .. 8191
      int row, c;
      char* dst;
      if (!SPLIT) {  // 8 panels of 256 rows x 64 B: the region is linear in id
        row = (id & 1023) >> 2;
        c = ((id >> 10) << 2) | (id & 3);
        dst = region + (int64_t)id * 16;
      } else {  // 16 panels; this pass fills the hi (or lo) 32 B of each row
        const int p = id >> 9, q = id & 511;
        row = q >> 1;
        c = (p << 1) | (q & 1);
        dst = region + (int64_t)p * kPanel + row * kPRow + ((q & 1) << 4) + (lo ? 32 : 0);
      }
      const u32x4 d = *reinterpret_cast<const u32x4*>(srow(row) + ((c ^ (row & 31)) << 4));
      *reinterpret_cast<u32x4*>(dst) = d;
    }
  };

  // Row-major pass, straight from registers: a quad transpose gives each
  // lane 4 consecutive columns (8 bytes) of one row; for one 32x32 block and
  // accumulator group, lanes 0-31 then hold 4 consecutive rows x 32 columns
  // and lanes 32-63 the next 4 rows, i.e. 8 consecutive 64-byte panel rows:
  // 512 contiguous bytes per store in the bf16 panel layout (split: the hi
  // or lo halves of the rows of two adjacent panels).
  auto pass_rows = [&](const bf16x4 (&v)[kMT][kNT][4], bool lo) {
    char* region = O1 + (int64_t)bi * kBM * g.ldo1 * kEB + (int64_t)bj * (256 / kPK) * kPanel;
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNT; ++ni) {
        const int col = wn0 + ni * 32 + (lane & 28);  // first of the lane's 4 columns
        const int64_t cpart = SPLIT ? (int64_t)(col >> 4) * kPanel + ((col & 15) << 1) + (lo ? 32 : 0)
                                    : (int64_t)(col >> 5) * kPanel + ((col & 31) << 1);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int row = wm0 + mi * 32 + 8 * rg + 4 * (lane >> 5) + (lane & 3);
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          u32x2 d = __builtin_bit_cast(u32x2, v[mi][ni][rg]);
          uint32_t d0 = d.x, d1 = d.y;
          quad_transpose(d0, d1, lane);
          d.x = d0;
          d.y = d1;
          *reinterpret_cast<u32x2*>(region + cpart + row * kPRow) = d;
        }
      }
  };
  // Transposed pass: LDS tile [col][row], 16-byte chunk c of LDS row j
  // stored at position c ^ (j & 31).
  auto pass_cols = [&](const bf16x4 (&v)[kMT][kNT][4], bool lo) {
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNT; ++ni) {
        const int col = wn0 + ni * 32 + (lane & 31);
        char* base = srow(col);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int row0 = wm0 + mi * 32 + 8 * rg + 4 * (lane >> 5);
          const int off = ((((row0 >> 3) ^ (col & 31)) << 4) | ((row0 & 7) << 1));
          *reinterpret_cast<bf16x4*>(base + off) = v[mi][ni][rg];
        }
      }
    __syncthreads();
    store_tile(OT, ldT, bj, bi, lo);
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

// ---------------------------------------------------------------------------
// bf16 kernel (the default operand format): the same tile, ring, DMA and
// ping-pong schedule as k_ns_gemm_bf16, on v_mfma_f32_16x16x32_bf16. One
// instruction takes a whole 32-k stage; a wave's 128 x 64 tile is 8 x 4
// blocks of 16 x 16, 32 instructions per stage (the work of 16
// 32x32x16). On random bf16 data this shape sustains about 16 % more
// throughput than 32x32x16 at the same occupancy (register-only loop: 2.0
// against 1.72 PFLOP/s; on all-zero data both reach ~2.47), and its results
// are bit for bit those of the 32x32x16 kernel (every launch of the Gram,
// polynomial and apply compared; the polynomial's mirrored quadrants of
// diagonal tiles assume a symmetric A, which the Gram's mirror guarantees). Lane layouts: A and B fragments, lane l
// holds row (column) l%16, k = 8(l/16) .. +7; accumulators, lane l holds
// rows 4(l/16) .. +3 of column l%16. Two differences from that kernel's ring:
// panels are swizzled with SH = 1 (see swz), and in the apply group 1
// issues the K-major Q refills and group 0 the A refills (the loading group
// of the second phase of a stage has less work then, measured 1 % faster).
// ---------------------------------------------------------------------------
namespace m16 {
using namespace bf;
// 16x16 blocks of a wave tile of (TM / 2) x 64: TM / 32 rows of kNT blocks
constexpr int kNT = 4;
template <int MT>
struct F { bf16x8 a[MT], b[kNT]; };
// Lane parts of LDS addresses: f row fragments (row l%16, chunk l/16,
// swizzled); q transposed B fragment reads of the apply (rows 8(l/16) +
// (l%16)/4, columns 4(l%4) .. +3 of a 16-column block); e transposed E reads
// (rows 4(l/16) + (l%16)/4).
struct Offs { int f, q, e; };

// QT stage for this kernel: as qt_src (bf16), but rows with bit 3 set hold
// their two 32-byte halves swapped, so that the two 16-lane groups of a
// transposed read (rows 8 apart, same columns) use different banks.
template <int TM = 256>
__device__ __forceinline__ QtSrc qt_src16(const char* X, int ldx, int bj, int wave, int lane) {
  QtSrc d;
  const char* base = X + (int64_t)bj * (TM / 32) * kPanel;
  const int lo = (lane >> 2) * kPRow + (((lane & 3) ^ (2 * ((lane >> 5) & 1))) << 4);
  d.g[0] = d.g[1] = base + lo;
  d.rbs = (int64_t)(ldx / 32) * kPanel;
  d.lds = (uint32_t)(TM * kPRow + (wave & (TM / 64 - 1)) * 4096);
  return d;
}

// After quad_transpose, lanes l and l^4 hold the two 4-column halves of 8
// columns of one row, for each of two blocks X and Y. Exchanging halves across
// the pair (DPP row shifts by 4 lanes) leaves lane l (bit 2 clear) with the 8
// columns of X and lane l^4 with those of Y: one 16-byte store each.
__device__ __forceinline__ u32x4 pair_halves(uint32_t x0, uint32_t x1, uint32_t y0, uint32_t y1, int lane) {
  const bool hi = (lane & 4) != 0;
  const uint32_t s0 = hi ? x0 : y0, s1 = hi ? x1 : y1;
  const uint32_t a0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x104, 0xF, 0xF, false);  // row_shl:4, from lane + 4
  const uint32_t a1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x104, 0xF, 0xF, false);
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x114, 0xF, 0xF, false);  // row_shr:4, from lane - 4
  const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x114, 0xF, 0xF, false);
  return hi ? u32x4{b0, b1, y0, y1} : u32x4{x0, x1, a0, a1};
}

// Main loop: as pingpong (same phases, barriers and refills), with one
// 32-k fragment set per stage. The E term: accumulator rows 16 mi .. +15 lie
// in one stage, read as 4 consecutive k of the lane's column (transposed
// read for the apply, a plain 8-byte read of A's row for the polynomial).
// NT: 16-column blocks the wave computes (kNT, or 2 for the second group on
// a diagonal tile of the symmetric modes).
template <int TM, int G, bool E_TERM, bool QT, int NT = kNT>
__device__ __forceinline__ void pingpong16(const DmaSrc& dsrc, const QtSrc& qsrc, int nk,
                                           const char* ring, uint32_t ring_lds, int wave, int wm0,
                                           int wn0, const Offs& o, int lane, int bi, float seed,
                                           f32x4 (&acc)[TM / 32][kNT]) {
  constexpr int kMT = TM / 32;
  constexpr int kStg = 2 * TM * kPRow;  // stage bytes: A rows, then B rows
  F<kMT> f;
  const int g = lane >> 4;
  auto take_e = [&](const char* buf, int kt) {
    // accumulator row rho (from wm0) takes its E value from stage row rho - r
    const int r = kt * 32 - TM * bi - wm0;  // a multiple of 32
    if (r < 0 || r >= kMT * 16) return;
    const char* lb = buf + TM * kPRow;
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi) {
      if (16 * mi < r || 16 * mi >= r + 32) continue;
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        const int n0 = wn0 + 16 * ni;
        bf16x4 hv;
        if (QT) {
          hv = read_tr(lb + (n0 >> 5) * 2048 + (16 * mi - r) * kPRow + o.e +
                       ((((n0 & 31) << 1) ^ (32 * ((g >> 1) & 1)))));
        } else {
          const int kk = 16 * mi - r + 4 * g;
          const int qrow = n0 + (lane & 15);
          hv = *reinterpret_cast<const bf16x4*>(lb + bf::swz<1>(qrow, kk >> 3) + ((kk & 7) << 1));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[mi][ni][q] = fmaf(seed, (float)hv[q], acc[mi][ni][q]);
      }
    }
  };
  auto load = [&](int kt) {
    const char* buf = ring + (kt & (kNBuf - 1)) * kStg;
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
      f.a[mi] = *reinterpret_cast<const bf16x8*>(buf + (wm0 + 16 * mi) * kPRow + o.f);
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      const int n0 = wn0 + 16 * ni;
      if (QT) {
        const char* p = buf + TM * kPRow + (n0 >> 5) * 2048 + o.q + ((((n0 & 31) << 1) ^ (32 * (g & 1))));
        f.b[ni] = cat8(read_tr(p), read_tr(p + 4 * kPRow));
      } else {
        f.b[ni] = *reinterpret_cast<const bf16x8*>(buf + TM * kPRow + n0 * kPRow + o.f);
      }
    }
    if (E_TERM && seed != 0.f) take_e(buf, kt);
  };
  auto mul = [&]() {
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
  };
  auto refill = [&](int kt) {
    const uint32_t buf = ring_lds + (kt & (kNBuf - 1)) * kStg;
    if (QT && G == 1) issue_share_qt<false, TM>(qsrc, wave, kt, buf);
    else issue_share(dsrc, kt, buf);
  };
  if (G == 0) load(0);
  phase_barrier<>();
  for (int s = 0; s < nk; ++s) {
    if (G == 0) {
      mul();
    } else {
      load(s);
      if (s >= 1 && s + 3 < nk) refill(s + 3);
    }
    phase_barrier_n((s + 2 < nk) + (s + 3 < nk));
    if (G == 0) {
      if (s + 1 < nk) load(s + 1);
      if (s + 4 < nk) refill(s + 4);
    } else {
      mul();
    }
    phase_barrier<>();
  }
}

// The kernel: tile mapping, operand pointers, DMA prologue and scaling as in
// k_ns_gemm_bf16; the epilogue stores row-major output from registers after
// a quad transpose and a pairwise exchange (lane: 8 columns of one row, 16
// bytes), and transposed output from registers after an exchange between
// lanes l and l^16 (lane: 8 rows of one column, 16 bytes).
template <int MODE, int TM>
__global__ __launch_bounds__(2 * TM, 2) void k_ns_gemm_m16(GemmArgs args) {
  constexpr bool kSym = (MODE != kApply);
  constexpr bool kQT = (MODE == kApply);
  constexpr int kMT = TM / 32;        // 16-row blocks of a wave tile
  constexpr int kWPG = TM / 64;       // waves per group
  constexpr int kStg = 2 * TM * kPRow;
  __shared__ __attribute__((aligned(1024))) char ring[kNBuf * kStg];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWPG, wn = wave - (wave / kWPG) * kWPG;
  int gi, local;
  int vb = blockIdx.x;  // position 8 * slot + XCD in the XCD lists
  if (args.sched) {
    // Tail balancing: XCDs run at different clocks under this load (their
    // last blocks finished up to 7 % apart with a fixed deal), so the last
    // positions of every list are claimed at run time, own list first.
    if (blockIdx.x < 8 && tid == 0) args.sched_clear[blockIdx.x] = 0;
    const int x = blockIdx.x & 7;
    if ((int)(blockIdx.x >> 3) >= args.xstatic[x]) {
      __shared__ int pick;
      if (tid < 64) {
        // lanes 0-7 look at lists x .. x+7; a failed claim marks its list
        // exhausted (the counter only grows), so at most 8 rounds fail and a
        // block gives up only when every tail position has been taken
        const int k8 = tid & 7, y = (x + k8) & 7;
        const int tail = args.xlen[y] - args.xstatic[y];
        uint32_t failed = 0;
        int p = -1;
        for (int round = 0; round < 9 && p < 0; ++round) {
          bool avail = false;
          if (tid < 8 && !((failed >> k8) & 1u))
            avail = __hip_atomic_load(args.sched + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < tail;
          const uint64_t m = __ballot(avail);
          if (m == 0) break;
          const int k = __builtin_ctzll(m);
          int got = -1;
          if (tid == 0) {
            const int yy = (x + k) & 7;
            const int at = atomicAdd(args.sched + yy, 1);
            if (at < args.xlen[yy] - args.xstatic[yy]) got = 8 * (args.xstatic[yy] + at) + yy;
          }
          p = __shfl(got, 0);
          failed |= 1u << k;
        }
        if (tid == 0) pick = p;
      }
      __syncthreads();
      vb = pick;
      if (vb < 0) return;
    }
  }
  if (!map_tile(args, vb, gi, local)) return;
  const GemmGroup& g = args.g[gi];
  const int mat = local / g.tiles_per_mat;
  int bi, bj;
  tile_coords<kSym>(g, local - mat * g.tiles_per_mat, bi, bj);
  const char* blk = g.base + (int64_t)mat * g.mat_bytes;
  // operand rows of the tile: a 256-row panel block, and for 128-row tiles
  // the half of it (panel rows are 64 bytes)
  const char* P;
  const char* Q;
  if constexpr (TM == 256) {
    P = blk + g.offP + (int64_t)bi * kBM * g.ldp * 2;
    Q = blk + g.offQ + (kQT ? 0 : (int64_t)bj * kBN * g.ldq * 2);
  } else {
    P = blk + g.offP + (int64_t)(bi >> 1) * 256 * g.ldp * 2 + (bi & 1) * TM * kPRow;
    Q = blk + g.offQ + (kQT ? 0 : (int64_t)(bj >> 1) * 256 * g.ldq * 2 + (bj & 1) * TM * kPRow);
  }
  f32x4 acc[kMT][kNT];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNT; ++ni) acc[mi][ni] = f32x4{};
  const int nk = g.K / 32;
  const int wm0 = wm * (TM / 2), wn0 = wn * 64;
  Offs o;
  {
    const int i = lane & 15, gg = lane >> 4;
    o.f = i * kPRow + ((gg ^ ((i >> 1) & 3)) << 4);
    o.q = (8 * gg + (i >> 2)) * kPRow + 8 * (i & 3);
    o.e = (4 * gg + (i >> 2)) * kPRow + 8 * (i & 3);
  }
  // apply: the first group refills the A panel (dma_src takes the second
  // group for A)
  const DmaSrc dsrc = dma_src<1, TM>(P, Q, kQT ? (wave ^ kWPG) : wave, lane);
  const QtSrc qsrc = qt_src16<TM>(Q, g.ldq, bj, wave, lane);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr)ring;
#pragma unroll
  for (int st = 0; st < kNBuf; ++st) {
    if (kQT && wave >= kWPG) issue_share_qt<false, TM>(qsrc, wave, st, ring_lds + st * kStg);
    else issue_share(dsrc, st, ring_lds + st * kStg);
  }
  phase_barrier<12>();
  // the E term: a*X in the apply (none where B carries a*I), (b/c)*A in the
  // polynomial
  const float seed = MODE == kApply ? (g.fold ? 0.f : args.c0)
                     : MODE == kPoly ? args.c0 / args.c1 : 0.f;
  // Diagonal tile of a symmetric product: its lower-left quadrant is the
  // transpose of the upper-right one, so the second group computes only the
  // lower-right quadrant (a (TM/2) x 32 strip per wave, half the MFMAs) and
  // the epilogue mirrors the upper-right quadrant (the first group's waves
  // on its right half).
  const bool diag = kSym && bi == bj;
  const bool half = diag && wave >= kWPG;
  const int wnc = half ? TM / 2 + 32 * (wave - kWPG) : wn0;  // first column of the wave's strip
  if (wave < kWPG)
    pingpong16<TM, 0, MODE != kGram, kQT>(dsrc, qsrc, nk, ring, ring_lds, wave, wm0, wn0, o, lane, bi, seed, acc);
  else if (!half)
    pingpong16<TM, 1, MODE != kGram, kQT>(dsrc, qsrc, nk, ring, ring_lds, wave, wm0, wn0, o, lane, bi, seed, acc);
  else
    pingpong16<TM, 1, MODE != kGram, kQT, 2>(dsrc, qsrc, nk, ring, ring_lds, wave, wm0, wnc, o, lane, bi, seed, acc);

  float scale = MODE == kPoly ? args.c1 : 1.f;
  if (MODE != kPoly && args.xnorm && g.defer) {
    const float sg = x0_sigma(args.xnorm[g.first + mat]);
    scale = MODE == kGram ? sg * sg : sg;
  }
  // B' = B + a*I on the diagonal of the polynomial's diagonal tiles
  const bool add_diag = MODE == kPoly && g.fold && diag;
  bf16x4 vh[kMT][kNT];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNT; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = scale * acc[mi][ni][q];
        if (add_diag && wm0 + 16 * mi + 4 * (lane >> 4) + q == wnc + 16 * ni + (lane & 15))
          v += args.diag;
        vh[mi][ni][q] = (__bf16)v;
      }
  char* O1 = g.offO1 < 0 ? nullptr : const_cast<char*>(blk) + g.offO1;
  char* O2 = g.offO2 < 0 ? nullptr : const_cast<char*>(blk) + g.offO2;
  char* OT = kSym ? (bi != bj ? O1 : nullptr) : O2;
  const int ldT = kSym ? g.ldo1 : g.ldo2;
  // output tile (r, c) of a panel-major buffer of leading dimension ld: its
  // 256-row panel block (and the half of it for 128-row tiles), then its
  // 32-column panels
  auto tile_at = [&](char* base, int r, int c, int ld) -> char* {
    if constexpr (TM == 256) return base + (int64_t)r * kBM * ld * 2 + (int64_t)c * 8 * kPanel;
    return base + (int64_t)(r >> 1) * 256 * ld * 2 + (r & 1) * TM * kPRow +
           (int64_t)c * (TM / 32) * kPanel;
  };
  if (O1) {
    // Blocks ni = 2p and 2p + 1 share one 64-byte panel row: after the
    // exchange, lane l holds columns 8 * (l/8 % 2) .. +7 of block 2p + (l/4 % 2)
    // in row 4 (l/16) + l%4 of the block row, so one store instruction writes
    // 16 whole panel rows (1 KB, contiguous). With 8-byte stores (half rows)
    // a CU wrote its 128 KB tile 3.5 times slower, and the L2 fetched part of
    // the partially written lines from HBM.
    char* region = tile_at(O1, bi, bj, g.ldo1);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int chunk = ((lane >> 1) & 2) | ((lane >> 3) & 1);  // 16-byte chunk of the panel row
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
      for (int p = 0; p < kNT / 2; ++p) {
        if (half && p > 0) break;
        const u32x2 x = __builtin_bit_cast(u32x2, vh[mi][2 * p]);
        const u32x2 y = __builtin_bit_cast(u32x2, vh[mi][2 * p + 1]);
        uint32_t x0 = x.x, x1 = x.y, y0 = y.x, y1 = y.y;
        quad_transpose(x0, x1, lane);
        quad_transpose(y0, y1, lane);
        const u32x4 d = pair_halves(x0, x1, y0, y1, lane);
        const int row = wm0 + 16 * mi + 4 * (lane >> 4) + (lane & 3);
        *reinterpret_cast<u32x4*>(region + (int64_t)((wnc + 32 * p) >> 5) * kPanel + row * kPRow + (chunk << 4)) = d;
      }
  }
  // Transposed outputs (the mirror of an off-diagonal Gram or polynomial
  // tile, the lower-left quadrant of a diagonal one, O of a tall matrix)
  // straight from registers. Element (R, C) of the tile goes to row C,
  // column R of the transposed tile: panel R/32, panel row C. For blocks
  // 2m and 2m+1 (tile rows 32m .. 32m+31 of the wave) and one block column,
  // lane l holds rows 4g .. 4g+3 of each (g = l/16) in column l%16; lanes l
  // and l^16 swap one block's values so that each holds 8 consecutive rows
  // of its column (g = 0, 1, 2, 3: rows 0-7, 16-23, 8-15, 24-31), and one
  // 16-byte store per lane writes 16 whole 64-byte panel rows (1 KB,
  // contiguous), as the row-major pass does. Staging through the ring cost
  // two barriers and an LDS round trip per tile.
  auto store_transposed = [&](char* region) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int g = lane >> 4;
    const bool odd = (g & 1) != 0;
    const int cbyte = ((g & 1) << 5) | ((g & 2) << 3);  // 0, 32, 16, 48
#pragma unroll
    for (int m = 0; m < kMT / 2; ++m)
#pragma unroll
      for (int ni = 0; ni < kNT; ++ni) {
        const u32x2 x = __builtin_bit_cast(u32x2, vh[2 * m][ni]);
        const u32x2 y = __builtin_bit_cast(u32x2, vh[2 * m + 1][ni]);
        const u32x2 send = odd ? x : y;
        const uint32_t r0 = (uint32_t)__shfl_xor((int)send.x, 16, 64);
        const uint32_t r1 = (uint32_t)__shfl_xor((int)send.y, 16, 64);
        const u32x4 d = odd ? u32x4{r0, r1, y.x, y.y} : u32x4{x.x, x.y, r0, r1};
        char* dst = region + (int64_t)((wm0 >> 5) + m) * kPanel +
                    (wnc + 16 * ni + (lane & 15)) * kPRow + cbyte;
        *reinterpret_cast<u32x4*>(dst) = d;
      }
  };
  // the mirror: waves of the first group on its right half
  const bool mirror = TM == 256 ? (wave == 2 || wave == 3) : (wave < kWPG && wn >= kWPG / 2);
  if (diag && O1 && mirror) store_transposed(tile_at(O1, bj, bi, g.ldo1));
  if (OT) store_transposed(tile_at(OT, bj, bi, ldT));
}
}  // namespace m16

// fp32 debug path: the generic 128x128 kernel with 4 waves (2 x 2).
constexpr int kTile32 = 128;

template <typename T, int MODE>
hipError_t launch_t(const GemmArgs& a, hipStream_t s, bool split) {
  if constexpr (std::is_same<T, __bf16>::value) {
    // 256x256 tiles, 8 waves in a 2 x 4 grid (wave tile 128 x 64): bf16 on
    // 16x16x32 MFMAs, split bf16 (hi + lo per 64-byte panel row, three
    // products per stage) on 32x32x16; bf16 launches with few tiles on
    // 128x128 tiles, 4 waves in a 2 x 2 grid (wave tile 64 x 64).
    if (split)
      hipLaunchKernelGGL((k_ns_gemm_bf16<MODE, 2, 4, true>), dim3(a.grid), dim3(512), 0, s, a);
    else if (a.small)
      hipLaunchKernelGGL((m16::k_ns_gemm_m16<MODE, 128>), dim3(a.grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((m16::k_ns_gemm_m16<MODE, 256>), dim3(a.grid), dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_ns_gemm<T, kTile32, kTile32, 2, 2, MODE>), dim3(a.ntiles), dim3(256), 0,
                       s, a);
  }
  return hipGetLastError();
}

}  // namespace

__global__ void k_zero_i32(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

int gemm_tile(NsPrec prec) { return prec == kFp32 ? kTile32 : bf::kBM; }

hipError_t launch_zero_i32(int* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, s, p, n);
  return hipGetLastError();
}

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
