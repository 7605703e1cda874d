// Internal interfaces between the host side of the MuonH library (plan,
// validation, launch sequence) and its HIP kernels. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muonh {

// Newton-Schulz quintic coefficients and the normalisation epsilon
// (see include/muonh.h for the step they belong to).
constexpr float kNsA = 3.4445f;
constexpr float kNsB = -4.7750f;
constexpr float kNsC = 2.0315f;
constexpr double kNsEps = 1e-7;

// Every Newton-Schulz operand is zero-padded to a multiple of this on both
// sides, so that the MFMA kernels never need bounds checks. Zero rows and
// columns stay exactly zero through every iteration.
constexpr int kPad = 256;

// Max number of per-matrix partial sums of a norm reduction.
constexpr int kMaxPartials = 256;

// Storage format of the Newton-Schulz operands (X, A, B; X^T in fp32 mode):
//   kBf16      bf16, panel-major: panels of 256 rows x 64 bytes (32 values
//              per panel row), panel (r/256, c/32) at
//              ((r/256) * (ld/32) + c/32) * 16 KB;
//   kSplitBf16 each value v as hi = bf16(v) and lo = bf16(v - hi); the same
//              panels with 16 hi then the 16 matching lo values per row;
//   kFp32      fp32, row-major (debug mode).
// Leading dimensions are always in logical elements; bytes per logical
// element: 2, 4 and 4.
enum NsPrec : int { kBf16 = 0, kSplitBf16 = 1, kFp32 = 2 };
constexpr int ns_elem_bytes(NsPrec p) { return p == kBf16 ? 2 : 4; }

// Deferred normalisation of X0 (bf16 and split operands with at least one
// iteration): the momentum kernel writes Y = M rounded to the operand format,
// unscaled, and the first iteration's GEMM epilogues apply
// sigma = 1 / (||M|| + eps) (Gram: sigma^2, apply: sigma). That is exact
// algebra (X0 = sigma * M), and safe while fp32 accumulation of Y neither
// overflows nor underflows: for ||M|| in [2^-40, 2^40], or 0 (Y = 0). Other
// norms (and non-finite ones) take a fallback that writes X0 normalised, and
// the epilogues then use sigma = 1.
__host__ __device__ inline bool xnorm_deferred(double n) {
  return n == 0.0 || (n >= 0x1p-40 && n <= 0x1p40);
}
__host__ __device__ inline float x0_sigma(double n) {
  return xnorm_deferred(n) ? (float)(1.0 / (n + kNsEps)) : 1.f;
}
// Matrices of at most this many entries follow the order of the step's
// definition exactly: their X0 is rounded after the normalisation (never
// deferred), and the apply adds a*X in fp32 (B is not folded, see
// GemmGroup::fold). For them the extra read of M costs nothing measurable,
// and with only a few singular values the place of a rounding shows in the
// result.
constexpr int64_t kSmallMatElems = 65536;

// Storage of the gradient and the momentum (plan flags MUONH_GRAD_BF16 and
// MUONH_MOM_BF16): fp32, or bf16. A bf16 momentum is the exact beta*M + G
// rounded once to the nearest bf16 (ties to even), and the stored value is
// the one the norm and Newton-Schulz see.
struct StateFmt {
  bool g_bf16 = false;
  bool m_bf16 = false;
};

// ---------------------------------------------------------------------------
// Elementwise / reduction kernels (elementwise.hip)
// ---------------------------------------------------------------------------
constexpr int kMaxEwGroups = 16;
// Threads per block of every elementwise kernel.
constexpr int kEwThreads = 256;

struct EwGroup {
  int rows, cols;       // matrix shape (row-major fp32)
  int count, first;     // number of matrices, global index of the first one
  int bpm;              // blocks per matrix (= partial sums per matrix in the
                        // kernels that take norms)
  int tpb;              // tiles per block (fused momentum + cast)
  int block_begin;      // first block of this group in the launch
  int64_t n;            // rows * cols
  // Newton-Schulz buffers of matrix m live at ns_base + m * mat_bytes.
  char* ns_base;
  int64_t mat_bytes;
  // Byte offsets (-1: absent) of a matrix in its own orientation, D (rows x
  // cols, leading dimension cp), and transposed, E (cols x rows, leading
  // dimension rp). The cast writes X0 to one or both; the update and the
  // projection read the final O from D.
  int64_t offD, offE;
  int rp, cp;           // padded rows / cols
  int tiles_per_mat;    // 64x64 tiles of the padded rp x cp domain
  int defer;            // 1: X0's normalisation may be deferred (more than
                        // kSmallMatElems entries)
};

struct EwArgs {
  EwGroup g[kMaxEwGroups];
  int ngroups;
  int nblocks;
};

// Norm partials: partials[mat * kMaxPartials + chunk] (double).
hipError_t launch_sumsq(const EwArgs& a, float* const* W, double* partials, hipStream_t s);
hipError_t launch_momentum(const EwArgs& a, StateFmt sf, const void* const* G, void* const* M,
                           float beta, double* partials, hipStream_t s);
// norms[mat] = sqrt(sum of partials) for the matrices of the batch `a`;
// if R != nullptr also R[mat] = (float)norms[mat]; if flags != nullptr, `bit`
// is or-ed into *flags when a norm is not finite.
hipError_t launch_finalize(const EwArgs& a, const double* partials, double* norms, float* R,
                           hipStream_t s, uint32_t* flags = nullptr, uint32_t bit = 0);
// X0 = M / (norm + eps) written to D (same orientation) and E (transposed).
hipError_t launch_normcast(const EwArgs& a, NsPrec prec, StateFmt sf, const void* const* M,
                           const double* norms, hipStream_t s);
// M <- beta*M + G with partial sums of squares, and Y = M (unscaled) written
// to D / E as X0 would be (tile launch; bpm blocks of tpb tiles per matrix).
hipError_t launch_momentum_cast(const EwArgs& a, NsPrec prec, StateFmt sf, const void* const* G,
                                void* const* M, float beta, double* partials, hipStream_t s);
// For the matrices whose norm fails xnorm_deferred, and every matrix of the
// groups that never defer: X0 = M / (norm + eps) written as launch_normcast
// would (8 blocks per matrix; the others return).
hipError_t launch_cast_fallback(const EwArgs& a, NsPrec prec, StateFmt sf, const void* const* M,
                                const double* norms, hipStream_t s);
hipError_t launch_update_norm(const EwArgs& a, NsPrec prec, float* const* W, float lr,
                              double* partials, hipStream_t s);
hipError_t launch_project(const EwArgs& a, NsPrec prec, float* const* W, const float* R,
                          const double* norms, float lr, hipStream_t s);
// W <- keep*W - lr*O (Muon with decoupled weight decay, keep = 1 - lr*wd).
hipError_t launch_decay_update(const EwArgs& a, NsPrec prec, float* const* W, float lr, float keep,
                               hipStream_t s);
// dst (rows x cols fp32) <- D of one matrix.
hipError_t launch_read_update(NsPrec prec, const char* D, int ldD, int rows, int cols, float* dst,
                              hipStream_t s);

// ---------------------------------------------------------------------------
// Newton-Schulz MFMA GEMM kernels (ns_gemm.hip)
//   C[i][j] = sum_k P[i][k] * Q[j][k]; the bf16 apply reads Q = X K-major
//   (C = B X), every other operand is read along its rows.
// ---------------------------------------------------------------------------
constexpr int kMaxGemmGroups = 16;

enum GemmMode : int {
  kGram = 0,   // O1 = P P^T              (symmetric; upper tiles, mirrored)
  kPoly = 1,   // O1 = c0*E + c1*(P P^T)  (symmetric; upper tiles, mirrored)
  kApply = 2,  // v = c0*E + P Q^T; O1[i][j] = v, O2[j][i] = v (either optional)
};

struct GemmGroup {
  const char* base;     // first matrix's Newton-Schulz block
  int64_t mat_bytes;    // stride between matrices
  int64_t offP, offQ, offE, offO1, offO2;  // byte offsets in a block (-1: absent)
  int ldp, ldq, lde, ldo1, ldo2;           // leading dimensions, in elements
  int K;                // contraction length (multiple of kPad)
  int tm, tn;           // tile grid (symmetric modes: tm == tn, upper triangle)
  int tiles_per_mat;
  int tile_begin;
  int count;
  int first;            // global index of the group's first matrix
  int defer;            // 1: the group's X0 may be unscaled (see EwGroup)
  // 1 (more than kSmallMatElems entries): the polynomial writes
  // B' = a*I + b*A + c*A*A and the apply computes X <- B' X with no a*X term.
  // The same algebra as a*X + B X; B' has eigenvalues p(sigma)/sigma near 1
  // instead of B's near -2.7, so its bf16 rounding costs less accuracy (a
  // bf16 emulation of 5 iterations: 1.07e-2 against 1.17e-2 on 512x1536).
  int fold;
};

struct GemmArgs {
  GemmGroup g[kMaxGemmGroups];
  int ngroups;
  int ntiles;
  int grid;      // blocks launched (>= ntiles when the XCD mapping pads)
  int xcd_map;   // 1: deal each group's tiles to the 8 XCDs in contiguous eighths
  float c0, c1;
  float diag;    // polynomial: added to the diagonal of B in groups that fold
  // First iteration after the fused momentum + cast: per-matrix ||M||; the
  // output is scaled by x0_sigma (Gram: squared). nullptr: no scaling.
  const double* xnorm;
  // Tail balancing (bf16 kernel with xcd_map; sched == nullptr: off). XCD x
  // has xlen[x] positions in its list; blocks of slot (blockIdx / 8) below
  // xstatic[x] take their own position, the others claim tail positions
  // [xstatic, xlen) of any list through the counters sched[0..7], which are
  // zero when the launch starts; block b < 8 zeroes sched_clear[b], the
  // counters of the next launch on the stream.
  int* sched;
  int* sched_clear;
  int xlen[8], xstatic[8];
  // bf16 launches that 256x256 tiles cannot spread over the CUs run
  // 128x128 tiles (the group's tm, tn and tiles_per_mat count those).
  int small;
};

// Sets the calling thread's muonh_last_error() message; returns `code`.
int set_error(int code, const char* msg);

// Tile edge (square tiles) used by the launchers for the given precision.
int gemm_tile(NsPrec prec);
hipError_t launch_gemm(GemmMode mode, NsPrec prec, const GemmArgs& a, hipStream_t s);
// Zeroes n ints at p (a kernel, so that the call may sit in a captured graph).
hipError_t launch_zero_i32(int* p, int n, hipStream_t s);

}  // namespace muonh
