// Host side of the MuonH C ABI (include/muonh.h): plan creation, argument
// validation, workspace layout and the fixed launch sequence of one step.
//
// Step sequence (all grouped launches over every matrix of the plan):
//   bf16 or split operands with ns_iters >= 1:
//     momentum + cast (M <- beta M + G stored, Y = M unscaled in the
//     operand layout, partial ||M||^2) -> finalize ||M|| -> cast fallback
//     (rewrites X0 normalised for norms outside [2^-40, 2^40] and for
//     matrices of at most 65536 entries); the first Gram and apply then
//     scale the others by 1/(||M||+eps)
//   otherwise: momentum -> finalize -> normcast (X0 = M/(||M||+eps))
//   ns_iters x { Gram A = X X^T ; Poly B = bA + cAA ; Apply X <- aX + BX }
//   MuonH: update (partial ||W - lr O||^2) -> finalize -> project
//          (W <- R W'/||W'||)
//   Muon baseline: decayed update (W <- (1 - lr wd) W - lr O)
// The projection onto the fixed sphere follows the digest page "Puro-2B
// trains for $6.9K, attention sinks hit 99%, LoopArena tops at 24.69%",
// section "The load-bearing tricks aren't in the abstract"; the absence of a
// weight-decay term follows the model card "Puro", section "Training".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/muonh.h"
#include "muonh_internal.h"

using namespace muonh;

namespace {
thread_local std::string g_last_error;
}  // namespace

// Shared with the other sources of the library (adamw.hip).
int muonh::set_error(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

namespace {

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MUONH_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct GroupPlan {
  int rows, cols, count, first;
  bool trans;
  int s, l, sp, lp;
  int64_t n;            // rows * cols
  int64_t off;          // workspace byte offset of the group's first matrix block
  int64_t mat_bytes;    // bytes per matrix block
  // Offsets within a matrix block. bf16 and split operands keep one layout of
  // X (s x l) in two buffers that alternate between iterations (offXs; the
  // apply reads X K-major); the fp32 debug kernel keeps X and two copies of
  // X^T (offX, offXt). A and B are s x s.
  int64_t offXs[2], offX, offXt[2], offA, offB;
  int bpm;              // streaming blocks per matrix
};

// Elements one streaming block handles (before the per-matrix partial cap).
constexpr int64_t kElemsPerBlock = 16384;

// GEMM tail balancing (GemmArgs::sched): fraction of every XCD list claimed
// at run time, and blocks launched per claimed position (the surplus lets an
// XCD that runs faster take positions of the others; extra blocks find no
// position left and exit). Used for launches of at least two rounds of
// tiles on kCUs compute units: in A/B runs of the 84 x 2048x6144 launches
// this took 0.7-1.2 % off the Gram, polynomial and apply.
constexpr double kTailFrac = 0.08, kTailBlocks = 1.5;
constexpr int64_t kCUs = 256;
// Index of the non-finite status word after the 16 tail counters.
constexpr int kStatusWord = 16;

}  // namespace

// Workspace of muonh_step_noalloc: a fixed device array. Every GPU the library
// runs on holds its own copy until the process ends. On the host the name is
// only a stand-in: host code reaches the memory through the address that
// hipGetSymbolAddress returns for the current device (noalloc_workspace).
static __device__ __align__(256) char scratch[MUONH_NOALLOC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The current device's address of `scratch`, looked up once per device.
int noalloc_workspace(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MUONH_EINVAL, "device %d out of [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MUONH_OK;
}
}  // namespace

struct muonh_plan {
  std::vector<GroupPlan> groups;
  int64_t n_mats = 0;
  int64_t n_params = 0;
  uint32_t flags = 0;
  NsPrec prec = kBf16;
  StateFmt sf;  // storage of G and M
  int esize = 2;  // workspace bytes per logical Newton-Schulz element
  int64_t off_partials = 0, off_norm_m = 0, off_norm_w = 0, off_sched = 0;
  size_t ws_bytes = 0;
};

namespace {

bool check_ws(const muonh_plan* p, const void* ws, size_t bytes, int* err) {
  if (!ws) {
    *err = fail(MUONH_EWORKSPACE, "workspace is NULL");
    return false;
  }
  if (reinterpret_cast<uintptr_t>(ws) & 255u) {
    *err = fail(MUONH_EWORKSPACE, "workspace must be 256-byte aligned");
    return false;
  }
  if (bytes < p->ws_bytes) {
    *err = fail(MUONH_EWORKSPACE, "workspace has %zu bytes, the plan needs %zu", bytes, p->ws_bytes);
    return false;
  }
  return true;
}

// Where O, the update of the last step, sits: in the matrix's own
// orientation (rows x cols, padded), for every group.
int64_t off_update(const muonh_plan* p, const GroupPlan& G) {
  if (p->prec != kFp32) return G.offXs[1];
  return G.trans ? G.offXt[0] : G.offX;
}

// Launch descriptors of the streaming kernels (kind kEwStream: bpm blocks per
// matrix, at most kMaxPartials), the writing updates (kEwOneShot: one pass of
// the block per unit of 2 rows x 4 columns and thread, two units per thread,
// so that no thread issues loads after its stores), the cast (kEwTile: one
// block per 64x64 tile of the padded domain) or the fused momentum + cast
// (kEwFused: blocks of tpb = ceil(tiles / 256) tiles, so at most 256 partial
// sums per matrix), in batches of at most kMaxEwGroups groups (the same
// batches for every kind).
// ns_iters < 0: D is O (the update and projection read it); otherwise D and
// E are what the normalising cast writes before ns_iters iterations: X0 in
// the buffer the first iteration reads (own orientation in D, transposed in
// E, -1 where nothing is written); with 0 iterations, O itself.
enum EwKind { kEwStream = 0, kEwTile = 1, kEwFused = 2, kEwOneShot = 3 };

std::vector<EwArgs> make_ew(const muonh_plan* p, char* ws, EwKind kind, int ns_iters) {
  std::vector<EwArgs> out;
  const size_t ng = p->groups.size();
  for (size_t g0 = 0; g0 < ng; g0 += kMaxEwGroups) {
    EwArgs a;
    std::memset(&a, 0, sizeof a);
    int64_t blocks = 0;
    const size_t g1 = std::min(ng, g0 + kMaxEwGroups);
    for (size_t gi = g0; gi < g1; ++gi) {
      const GroupPlan& G = p->groups[gi];
      EwGroup& e = a.g[gi - g0];
      e.rows = G.rows;
      e.cols = G.cols;
      e.count = G.count;
      e.first = G.first;
      e.bpm = G.bpm;
      e.n = G.n;
      e.ns_base = ws + G.off;
      e.mat_bytes = G.mat_bytes;
      const int rp = G.trans ? G.lp : G.sp;
      const int cp = G.trans ? G.sp : G.lp;
      e.rp = rp;
      e.cp = cp;
      // D holds the matrix's own orientation, E the transposed one.
      if (ns_iters < 0) {
        e.offD = off_update(p, G);
        e.offE = -1;
      } else if (p->prec == kFp32) {
        // X, and the X^T copy that the last apply lands in copy 0 from
        const int64_t xt = G.offXt[ns_iters & 1];
        e.offD = G.trans ? xt : G.offX;
        e.offE = G.trans ? G.offX : xt;
      } else if (ns_iters == 0) {
        e.offD = G.offXs[1];
        e.offE = -1;
      } else {
        // X0 (s x l) in the buffer from which the last apply lands in buffer 1
        const int64_t x0 = G.offXs[1 - (ns_iters & 1)];
        e.offD = G.trans ? -1 : x0;
        e.offE = G.trans ? x0 : -1;
      }
      e.tiles_per_mat = (rp / 64) * (cp / 64);
      e.defer = G.n > kSmallMatElems;
      e.tpb = 1;
      if (kind == kEwFused) {
        e.tpb = (e.tiles_per_mat + kMaxPartials - 1) / kMaxPartials;
        e.bpm = (e.tiles_per_mat + e.tpb - 1) / e.tpb;
      } else if (kind == kEwOneShot) {
        const int64_t units = (int64_t)((G.rows + 1) / 2) * ((G.cols + 3) / 4);
        e.bpm = (int)std::max<int64_t>(1, (units + 2 * kEwThreads - 1) / (2 * kEwThreads));
      }
      e.block_begin = (int)blocks;
      blocks += (int64_t)G.count * (kind == kEwTile ? e.tiles_per_mat : e.bpm);
    }
    a.ngroups = (int)(g1 - g0);
    a.nblocks = (int)blocks;
    out.push_back(a);
  }
  return out;
}

// GEMM descriptors for one Newton-Schulz phase, heaviest groups first.
std::vector<GemmArgs> make_gemm(const muonh_plan* p, char* ws, GemmMode mode, int it, int iters,
                                const double* xnorm = nullptr) {
  // bf16 phases whose 256x256 tiles would occupy at most half of the CUs
  // run 128x128 tiles (GemmArgs::small): four times as many, so that a
  // single matrix or a few small ones still spread over the chip
  int T = gemm_tile(p->prec);
  bool small = false;
  if (p->prec == kBf16) {
    int64_t big = 0;
    for (const GroupPlan& G : p->groups) {
      const int64_t ts = G.sp / 256, tl = G.lp / 256;
      big += (int64_t)G.count * (mode == kApply ? ts * tl : ts * (ts + 1) / 2);
    }
    if (2 * big <= kCUs) {
      T = 128;
      small = true;
    }
  }
  // bf16 / split: the buffer iteration `it` reads X from (X0 goes to buffer
  // 1 - iters%2, so that the last apply writes buffer 1)
  const int src = (1 - (iters & 1)) ^ (it & 1);
  std::vector<GemmGroup> all;
  for (const GroupPlan& G : p->groups) {
    GemmGroup q;
    std::memset(&q, 0, sizeof q);
    q.base = ws + G.off;
    q.mat_bytes = G.mat_bytes;
    q.count = G.count;
    q.first = G.first;
    q.offE = q.offO1 = q.offO2 = -1;
    q.defer = G.n > kSmallMatElems;
    q.fold = G.n > kSmallMatElems;
    const int ts = G.sp / T, tl = G.lp / T;
    const int64_t xcur = p->prec == kFp32 ? G.offX : G.offXs[src];
    if (mode == kGram) {
      q.offP = q.offQ = xcur;
      q.ldp = q.ldq = G.lp;
      q.K = G.lp;
      q.tm = q.tn = ts;
      q.tiles_per_mat = ts * (ts + 1) / 2;
      q.offO1 = G.offA;
      q.ldo1 = G.sp;
    } else if (mode == kPoly) {
      q.offP = q.offQ = G.offA;
      q.ldp = q.ldq = G.sp;
      q.K = G.sp;
      q.tm = q.tn = ts;
      q.tiles_per_mat = ts * (ts + 1) / 2;
      q.offE = G.offA;
      q.lde = G.sp;
      q.offO1 = G.offB;
      q.ldo1 = G.sp;
    } else if (p->prec != kFp32) {
      // X (s x l) from buffer src to buffer 1 - src; the last iteration
      // writes O in the matrix's own orientation into buffer 1.
      const bool last = it == iters - 1;
      const int64_t xin = G.offXs[src], xout = G.offXs[1 - src];
      q.offP = G.offB;
      q.ldp = G.sp;
      q.offQ = xin;  // read K-major (k along X's rows)
      q.ldq = G.lp;
      q.K = G.sp;
      q.tm = ts;
      q.tn = tl;
      q.tiles_per_mat = ts * tl;
      q.offE = q.fold ? -1 : xin;  // folded: B carries a*I
      q.lde = G.lp;
      if (last && G.trans) {
        q.offO2 = xout;
        q.ldo2 = G.sp;
      } else {
        q.offO1 = xout;
        q.ldo1 = G.lp;
      }
    } else {
      const bool last = it == iters - 1;
      const int xin = (iters - it) & 1, xout = (iters - 1 - it) & 1;
      q.offP = G.offB;
      q.ldp = G.sp;
      q.offQ = G.offXt[xin];
      q.ldq = G.sp;
      q.K = G.sp;
      q.tm = ts;
      q.tn = tl;
      q.tiles_per_mat = ts * tl;
      q.offE = q.fold ? -1 : G.offX;
      q.lde = G.lp;
      if (!(last && G.trans)) {
        q.offO1 = G.offX;
        q.ldo1 = G.lp;
      }
      if (!(last && !G.trans)) {
        q.offO2 = G.offXt[xout];
        q.ldo2 = G.sp;
      }
    }
    all.push_back(q);
  }
  std::stable_sort(all.begin(), all.end(),
                   [](const GemmGroup& x, const GemmGroup& y) { return x.K > y.K; });
  std::vector<GemmArgs> out;
  for (size_t g0 = 0; g0 < all.size(); g0 += kMaxGemmGroups) {
    GemmArgs a;
    std::memset(&a, 0, sizeof a);
    int64_t tiles = 0;
    const size_t g1 = std::min(all.size(), g0 + kMaxGemmGroups);
    for (size_t gi = g0; gi < g1; ++gi) {
      a.g[gi - g0] = all[gi];
      a.g[gi - g0].tile_begin = (int)tiles;
      tiles += (int64_t)all[gi].count * all[gi].tiles_per_mat;
    }
    a.ngroups = (int)(g1 - g0);
    a.ntiles = (int)tiles;
    a.small = small ? 1 : 0;
    a.xnorm = mode == kPoly ? nullptr : xnorm;
    a.xcd_map = p->prec == kFp32 ? 0 : 1;
    if (a.xcd_map) {
      // slots per XCD: the longest of the 8 per-XCD lists
      int64_t longest = 0;
      for (int x = 0; x < 8; ++x) {
        int64_t len = 0;
        for (int gi = 0; gi < a.ngroups; ++gi) {
          const int64_t tot = (int64_t)a.g[gi].count * a.g[gi].tiles_per_mat;
          len += ((x + 1) * tot >> 3) - (x * tot >> 3);
        }
        a.xlen[x] = (int)len;
        longest = std::max(longest, len);
      }
      a.grid = (int)(8 * longest);
      // bf16 launches of two or more rounds of tiles: the last kTailFrac of
      // every list is claimed at run time by kTailBlocks times as many
      // blocks (the step sets the counters; see GemmArgs::sched)
      if (p->prec == kBf16 && tiles >= 2 * kCUs) {
        int64_t slots = 0;
        for (int x = 0; x < 8; ++x) {
          const int tail = (int)std::ceil(a.xlen[x] * kTailFrac);
          a.xstatic[x] = a.xlen[x] - tail;
          slots = std::max<int64_t>(slots, a.xstatic[x] + (int64_t)std::ceil(tail * kTailBlocks));
        }
        a.grid = (int)(8 * slots);
        a.sched = reinterpret_cast<int*>(ws + p->off_sched);  // set per launch by the step
      }
    } else {
      a.grid = a.ntiles;
    }
    if (mode == kPoly) {
      a.c0 = kNsB;
      a.c1 = kNsC;
      a.diag = kNsA;
    } else if (mode == kApply) {
      a.c0 = kNsA;
      a.c1 = 1.f;
    } else {
      a.c0 = 0.f;
      a.c1 = 1.f;
    }
    out.push_back(a);
  }
  return out;
}

}  // namespace

extern "C" {

int32_t muonh_abi_version(void) { return MUONH_ABI_VERSION; }

int muonh_step_status(const muonh_plan* plan, const void* workspace, size_t workspace_bytes,
                      void* stream, uint32_t* flags) {
  if (!plan || !flags) return fail(MUONH_EINVAL, "plan and flags must not be NULL");
  int err = 0;
  if (!check_ws(plan, workspace, workspace_bytes, &err)) return err;
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(static_cast<const char*>(workspace) + plan->off_sched) +
      kStatusWord;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, src, sizeof v, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "step status");
  *flags = v;
  return MUONH_OK;
}

const char* muonh_status_string(int status) {
  switch (status) {
    case MUONH_OK: return "ok";
    case MUONH_EINVAL: return "invalid argument";
    case MUONH_ESHAPE: return "invalid shape or index";
    case MUONH_EWORKSPACE: return "invalid workspace";
    case MUONH_EHIP: return "HIP runtime error";
    case MUONH_ENOMEM: return "out of host memory";
    case MUONH_EALIAS: return "overlapping matrices";
    default: return "unknown status";
  }
}

const char* muonh_last_error(void) { return g_last_error.c_str(); }

int muonh_check_disjoint(const muonh_plan* plan, const void* const* W, const void* const* G,
                         const void* const* M) {
  if (!plan) return fail(MUONH_EINVAL, "plan is NULL");
  if (!W || !G || !M) return fail(MUONH_EINVAL, "W, G and M must be host arrays of pointers");
  struct Span {
    uintptr_t lo, hi;
    int kind;   // 0 W, 1 G, 2 M
    int64_t index;
  };
  std::vector<Span> spans;
  try {
    spans.reserve((size_t)plan->n_mats * 3);
  } catch (...) {
    return fail(MUONH_ENOMEM, "host allocation failed");
  }
  const uintptr_t gsz = plan->sf.g_bf16 ? 2 : 4, msz = plan->sf.m_bf16 ? 2 : 4;
  for (const GroupPlan& g : plan->groups)
    for (int i = 0; i < g.count; ++i) {
      const int64_t k = g.first + i;
      const uintptr_t n = (uintptr_t)g.n;
      const void* const* arr[3] = {W, G, M};
      const uintptr_t esz[3] = {4, gsz, msz};
      for (int t = 0; t < 3; ++t) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(arr[t][k]);
        spans.push_back(Span{lo, lo + n * esz[t], t, k});
      }
    }
  std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) {
    return a.lo != b.lo ? a.lo < b.lo : a.hi < b.hi;
  });
  // sorted by start: an overlap exists iff some span starts before the
  // furthest end seen so far
  static const char* const kName[3] = {"W", "G", "M"};
  size_t far = 0;
  for (size_t i = 1; i < spans.size(); ++i) {
    if (spans[i].lo < spans[far].hi)
      return fail(MUONH_EALIAS, "%s[%lld] overlaps %s[%lld]", kName[spans[i].kind],
                  (long long)spans[i].index, kName[spans[far].kind], (long long)spans[far].index);
    if (spans[i].hi > spans[far].hi) far = i;
  }
  return MUONH_OK;
}

int muonh_plan_create(muonh_plan** out, const muonh_group_desc* groups, int32_t n_groups,
                      uint32_t flags) {
  if (!out) return fail(MUONH_EINVAL, "out is NULL");
  *out = nullptr;
  if (!groups) return fail(MUONH_EINVAL, "groups is NULL");
  if (n_groups < 1 || n_groups > MUONH_MAX_GROUPS)
    return fail(MUONH_EINVAL, "n_groups=%d out of [1, %d]", n_groups, MUONH_MAX_GROUPS);
  if (flags & ~uint32_t(MUONH_NS_FP32 | MUONH_NS_SPLIT_BF16 | MUONH_GRAD_BF16 | MUONH_MOM_BF16))
    return fail(MUONH_EINVAL, "unknown flags 0x%x", flags);
  if ((flags & MUONH_NS_FP32) && (flags & MUONH_NS_SPLIT_BF16))
    return fail(MUONH_EINVAL, "MUONH_NS_FP32 and MUONH_NS_SPLIT_BF16 exclude each other");

  muonh_plan* p = new (std::nothrow) muonh_plan;
  if (!p) return fail(MUONH_ENOMEM, "plan allocation failed");
  p->flags = flags;
  p->prec = (flags & MUONH_NS_FP32) ? kFp32 : (flags & MUONH_NS_SPLIT_BF16) ? kSplitBf16 : kBf16;
  p->esize = ns_elem_bytes(p->prec);
  p->sf.g_bf16 = (flags & MUONH_GRAD_BF16) != 0;
  p->sf.m_bf16 = (flags & MUONH_MOM_BF16) != 0;

  int64_t n_mats = 0, total_tiles = 0;
  for (int32_t i = 0; i < n_groups; ++i) {
    const muonh_group_desc& d = groups[i];
    if (d.rows < 1 || d.rows > MUONH_MAX_DIM || d.cols < 1 || d.cols > MUONH_MAX_DIM) {
      delete p;
      return fail(MUONH_ESHAPE, "group %d: shape %dx%d out of [1, %d]", i, d.rows, d.cols,
                  MUONH_MAX_DIM);
    }
    if (d.count < 1) {
      delete p;
      return fail(MUONH_ESHAPE, "group %d: count=%d must be >= 1", i, d.count);
    }
    n_mats += d.count;
    if (n_mats > MUONH_MAX_MATRICES) {
      delete p;
      return fail(MUONH_ESHAPE, "more than %d matrices", MUONH_MAX_MATRICES);
    }
    // Elementwise launches index their blocks with 32-bit integers; the
    // largest per-matrix block count is the cast's 64x64 tiles of the padded
    // domain (every other kind needs fewer).
    const int64_t pr = round_up(d.rows, kPad), pc = round_up(d.cols, kPad);
    total_tiles += (int64_t)d.count * (pr / 64) * (pc / 64);
    if (total_tiles > INT32_MAX) {
      delete p;
      return fail(MUONH_ESHAPE, "plan too large: more than 2^31 elementwise tiles");
    }
  }
  try {
    p->groups.resize(n_groups);
  } catch (...) {
    delete p;
    return fail(MUONH_ENOMEM, "plan allocation failed");
  }

  // Workspace: norm partials, two per-matrix norm arrays, then per group the
  // matrix blocks [X buffer 0 | X buffer 1 | A | B] (fp32: [X | X^T (two
  // copies) | A | B]).
  int64_t off = 0;
  p->off_partials = off;
  off = round_up(off + n_mats * kMaxPartials * (int64_t)sizeof(double), 256);
  p->off_norm_m = off;
  off = round_up(off + n_mats * (int64_t)sizeof(double), 256);
  p->off_norm_w = off;
  off = round_up(off + n_mats * (int64_t)sizeof(double), 256);
  p->off_sched = off;  // two sets of 8 tail counters (GemmArgs::sched), then the status word
  off = round_up(off + (kStatusWord + 1) * (int64_t)sizeof(int), 256);

  int first = 0;
  int64_t params = 0;
  for (int32_t i = 0; i < n_groups; ++i) {
    const muonh_group_desc& d = groups[i];
    GroupPlan& G = p->groups[i];
    G.rows = d.rows;
    G.cols = d.cols;
    G.count = d.count;
    G.first = first;
    first += d.count;
    G.trans = d.rows > d.cols;
    G.s = std::min(d.rows, d.cols);
    G.l = std::max(d.rows, d.cols);
    G.sp = (int)round_up(G.s, kPad);
    G.lp = (int)round_up(G.l, kPad);
    G.n = (int64_t)d.rows * d.cols;
    params += G.n * d.count;
    const int64_t e = p->esize;
    const int64_t xs = round_up((int64_t)G.sp * G.lp * e, 256);
    const int64_t ss = round_up((int64_t)G.sp * G.sp * e, 256);
    const int nx = p->prec == kFp32 ? 3 : 2;  // s x l buffers per matrix
    G.offXs[0] = G.offX = 0;
    G.offXs[1] = G.offXt[0] = xs;
    G.offXt[1] = 2 * xs;
    G.offA = nx * xs;
    G.offB = nx * xs + ss;
    G.mat_bytes = nx * xs + 2 * ss;
    G.off = off;
    off += G.mat_bytes * d.count;
    int64_t bpm = (G.n + kElemsPerBlock - 1) / kElemsPerBlock;
    G.bpm = (int)std::max<int64_t>(1, std::min<int64_t>(bpm, kMaxPartials));
  }
  p->n_mats = n_mats;
  p->n_params = params;
  p->ws_bytes = (size_t)round_up(off, 256);
  *out = p;
  return MUONH_OK;
}

void muonh_plan_destroy(muonh_plan* plan) { delete plan; }

int64_t muonh_plan_num_matrices(const muonh_plan* plan) { return plan ? plan->n_mats : 0; }

int64_t muonh_plan_num_params(const muonh_plan* plan) { return plan ? plan->n_params : 0; }

size_t muonh_workspace_bytes(const muonh_plan* plan) { return plan ? plan->ws_bytes : 0; }

int muonh_init(const muonh_plan* plan, float* const* W, float* R, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MUONH_EINVAL, "plan is NULL");
  if (!W || !R) return fail(MUONH_EINVAL, "W and R must be device arrays");
  int err = 0;
  if (!check_ws(plan, workspace, workspace_bytes, &err)) return err;
  // set-up for muonh_step_noalloc on this device (its first call retries
  // and reports a failure)
  void* scratch_addr = nullptr;
  (void)noalloc_workspace(&scratch_addr);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  double* partials = reinterpret_cast<double*>(ws + plan->off_partials);
  double* norms = reinterpret_cast<double*>(ws + plan->off_norm_w);
  hipError_t e;
  // a workspace that no step has used yet reports no non-finite norm
  int* sched = reinterpret_cast<int*>(ws + plan->off_sched);
  if ((e = launch_zero_i32(sched, kStatusWord + 1, s)) != hipSuccess) return hip_fail(e, "init status");
  for (const EwArgs& a : make_ew(plan, ws, kEwStream, -1)) {
    if ((e = launch_sumsq(a, W, partials, s)) != hipSuccess) return hip_fail(e, "init sumsq");
    if ((e = launch_finalize(a, partials, norms, R, s)) != hipSuccess)
      return hip_fail(e, "init finalize");
  }
  return MUONH_OK;
}

}  // extern "C"

namespace {

// The update after Newton-Schulz: MuonH (trial update, its norm, projection
// onto the radius-R sphere), or Muon with decoupled weight decay.
struct Variant {
  bool muon_wd;
  float weight_decay;
};

int check_step_args(const muonh_plan* plan, float* const* W, const void* const* G,
                    void* const* M, const float* R, float lr, float beta, int32_t ns_iters,
                    void* const* events, int32_t n_events, Variant var) {
  if (!plan) return fail(MUONH_EINVAL, "plan is NULL");
  if (!W || !G || !M || (!R && !var.muon_wd))
    return fail(MUONH_EINVAL, var.muon_wd ? "W, G and M must be device arrays"
                                          : "W, G, M and R must be device arrays");
  if (var.muon_wd && (!std::isfinite(var.weight_decay) || var.weight_decay < 0.f))
    return fail(MUONH_EINVAL, "weight_decay=%g must be finite and >= 0", var.weight_decay);
  if (!std::isfinite(lr) || lr < 0.f) return fail(MUONH_EINVAL, "lr=%g must be finite and >= 0", lr);
  if (!std::isfinite(beta) || beta < 0.f || beta >= 1.f)
    return fail(MUONH_EINVAL, "beta=%g must be in [0, 1)", beta);
  if (ns_iters < 0 || ns_iters > MUONH_MAX_NS_ITERS)
    return fail(MUONH_EINVAL, "ns_iters=%d out of [0, %d]", ns_iters, MUONH_MAX_NS_ITERS);
  if (events) {
    if (n_events != 3 * ns_iters + 3)
      return fail(MUONH_EINVAL, "n_events=%d, expected 3*ns_iters+3 = %d", n_events,
                  3 * ns_iters + 3);
    for (int i = 0; i < n_events; ++i)
      if (!events[i]) return fail(MUONH_EINVAL, "events[%d] is NULL", i);
  }
  return MUONH_OK;
}

int step_impl(const muonh_plan* plan, float* const* W, const void* const* G, void* const* M,
              const float* R, float lr, float beta, int32_t ns_iters, void* workspace,
              size_t workspace_bytes, void* stream, void* const* events, int32_t n_events,
              Variant var = {false, 0.f}) {
  int err = check_step_args(plan, W, G, M, R, lr, beta, ns_iters, events, n_events, var);
  if (err != MUONH_OK) return err;
  if (!check_ws(plan, workspace, workspace_bytes, &err)) return err;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  double* partials = reinterpret_cast<double*>(ws + plan->off_partials);
  double* norm_m = reinterpret_cast<double*>(ws + plan->off_norm_m);
  double* norm_w = reinterpret_cast<double*>(ws + plan->off_norm_w);
  hipError_t e;
  int ev = 0;
  auto mark = [&]() -> hipError_t {
    if (!events) return hipSuccess;
    return hipEventRecord(reinterpret_cast<hipEvent_t>(events[ev++]), s);
  };
  // Tail counters (two sets of 8) and the non-finite flags, cleared by a
  // kernel (no memset, so the step can be captured in a graph); each
  // balanced GEMM launch uses one counter set and zeroes the other for the
  // next; the norm finalizes set the non-finite bits in the flags.
  int* sched = reinterpret_cast<int*>(ws + plan->off_sched);
  uint32_t* nf_flags = reinterpret_cast<uint32_t*>(sched + kStatusWord);
  if ((e = launch_zero_i32(sched, kStatusWord + 1, s)) != hipSuccess) return hip_fail(e, "step status");

  const std::vector<EwArgs> stream_args = make_ew(plan, ws, kEwStream, -1);
  const std::vector<EwArgs> write_args = make_ew(plan, ws, kEwOneShot, -1);
  // bf16 and split operands with at least one iteration: momentum and the
  // unscaled cast in one pass, normalisation deferred to the first GEMMs
  // (see xnorm_deferred); otherwise momentum, its norm, then the cast.
  const bool fused = plan->prec != kFp32 && ns_iters >= 1;

  if ((e = mark()) != hipSuccess) return hip_fail(e, "event record");
  if (fused) {
    for (const EwArgs& a : make_ew(plan, ws, kEwFused, ns_iters)) {
      if ((e = launch_momentum_cast(a, plan->prec, plan->sf, G, M, beta, partials, s)) != hipSuccess)
        return hip_fail(e, "momentum + cast");
      if ((e = launch_finalize(a, partials, norm_m, nullptr, s, nf_flags, MUONH_NONFINITE_MOMENTUM)) !=
          hipSuccess)
        return hip_fail(e, "momentum finalize");
      if ((e = launch_cast_fallback(a, plan->prec, plan->sf, M, norm_m, s)) != hipSuccess)
        return hip_fail(e, "cast fallback");
    }
  } else {
    for (const EwArgs& a : stream_args) {
      if ((e = launch_momentum(a, plan->sf, G, M, beta, partials, s)) != hipSuccess)
        return hip_fail(e, "momentum");
      if ((e = launch_finalize(a, partials, norm_m, nullptr, s, nf_flags, MUONH_NONFINITE_MOMENTUM)) !=
          hipSuccess)
        return hip_fail(e, "momentum finalize");
    }
    for (const EwArgs& a : make_ew(plan, ws, kEwTile, ns_iters))
      if ((e = launch_normcast(a, plan->prec, plan->sf, M, norm_m, s)) != hipSuccess)
        return hip_fail(e, "normcast");
  }
  if ((e = mark()) != hipSuccess) return hip_fail(e, "event record");

  int parity = 0;
  auto gemm = [&](GemmMode mode, GemmArgs a) -> hipError_t {
    if (a.sched) {
      a.sched = sched + 8 * parity;
      a.sched_clear = sched + 8 * (1 - parity);
      parity ^= 1;
    }
    return launch_gemm(mode, plan->prec, a, s);
  };
  for (int it = 0; it < ns_iters; ++it) {
    const double* xnorm = (fused && it == 0) ? norm_m : nullptr;
    for (const GemmArgs& a : make_gemm(plan, ws, kGram, it, ns_iters, xnorm))
      if ((e = gemm(kGram, a)) != hipSuccess) return hip_fail(e, "ns gram");
    if ((e = mark()) != hipSuccess) return hip_fail(e, "event record");
    for (const GemmArgs& a : make_gemm(plan, ws, kPoly, it, ns_iters))
      if ((e = gemm(kPoly, a)) != hipSuccess) return hip_fail(e, "ns poly");
    if ((e = mark()) != hipSuccess) return hip_fail(e, "event record");
    for (const GemmArgs& a : make_gemm(plan, ws, kApply, it, ns_iters, xnorm))
      if ((e = gemm(kApply, a)) != hipSuccess) return hip_fail(e, "ns apply");
    if ((e = mark()) != hipSuccess) return hip_fail(e, "event record");
  }

  if (var.muon_wd) {
    const float keep = (float)(1.0 - (double)lr * (double)var.weight_decay);
    for (const EwArgs& a : write_args)
      if ((e = launch_decay_update(a, plan->prec, W, lr, keep, s)) != hipSuccess)
        return hip_fail(e, "decayed update");
  } else {
    for (size_t b = 0; b < stream_args.size(); ++b) {
      const EwArgs& a = stream_args[b];
      if ((e = launch_update_norm(a, plan->prec, W, lr, partials, s)) != hipSuccess)
        return hip_fail(e, "update norm");
      if ((e = launch_finalize(a, partials, norm_w, nullptr, s, nf_flags, MUONH_NONFINITE_UPDATE)) !=
          hipSuccess)
        return hip_fail(e, "update finalize");
      if ((e = launch_project(write_args[b], plan->prec, W, R, norm_w, lr, s)) != hipSuccess)
        return hip_fail(e, "project");
    }
  }
  if ((e = mark()) != hipSuccess) return hip_fail(e, "event record");
  return MUONH_OK;
}

}  // namespace

extern "C" {

int muonh_step(const muonh_plan* plan, float* const* W, const void* const* G, void* const* M,
               const float* R, float lr, float beta, int32_t ns_iters, void* workspace,
               size_t workspace_bytes, void* stream) {
  return step_impl(plan, W, G, M, R, lr, beta, ns_iters, workspace, workspace_bytes, stream,
                   nullptr, 0);
}

int muonh_step_noalloc(const muonh_plan* plan, float* const* W, const void* const* G,
                       void* const* M, const float* R, float lr, float beta, int32_t ns_iters,
                       void* stream) {
  int err = check_step_args(plan, W, G, M, R, lr, beta, ns_iters, nullptr, 0, Variant{false, 0.f});
  if (err != MUONH_OK) return err;
  if (plan->ws_bytes > (size_t)MUONH_NOALLOC_WORKSPACE_BYTES)
    return fail(MUONH_EWORKSPACE,
                "the plan needs %zu bytes of workspace; muonh_step_noalloc has %zu "
                "(MUONH_NOALLOC_WORKSPACE_BYTES): use muonh_step with a caller workspace",
                plan->ws_bytes, (size_t)MUONH_NOALLOC_WORKSPACE_BYTES);
  void* ws = nullptr;
  if ((err = noalloc_workspace(&ws)) != MUONH_OK) return err;
  return step_impl(plan, W, G, M, R, lr, beta, ns_iters, ws, MUONH_NOALLOC_WORKSPACE_BYTES, stream,
                   nullptr, 0);
}

int muonh_step_timed(const muonh_plan* plan, float* const* W, const void* const* G,
                     void* const* M, const float* R, float lr, float beta, int32_t ns_iters,
                     void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                     int32_t n_events) {
  if (!events) return fail(MUONH_EINVAL, "events is NULL");
  return step_impl(plan, W, G, M, R, lr, beta, ns_iters, workspace, workspace_bytes, stream,
                   events, n_events);
}

int muonh_step_muon_wd(const muonh_plan* plan, float* const* W, const void* const* G,
                       void* const* M, float lr, float beta, float weight_decay,
                       int32_t ns_iters, void* workspace, size_t workspace_bytes, void* stream) {
  return step_impl(plan, W, G, M, nullptr, lr, beta, ns_iters, workspace, workspace_bytes, stream,
                   nullptr, 0, Variant{true, weight_decay});
}

int muonh_step_muon_wd_timed(const muonh_plan* plan, float* const* W, const void* const* G,
                             void* const* M, float lr, float beta, float weight_decay,
                             int32_t ns_iters, void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events, int32_t n_events) {
  if (!events) return fail(MUONH_EINVAL, "events is NULL");
  return step_impl(plan, W, G, M, nullptr, lr, beta, ns_iters, workspace, workspace_bytes, stream,
                   events, n_events, Variant{true, weight_decay});
}

int muonh_read_update(const muonh_plan* plan, int64_t index, float* dst, const void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MUONH_EINVAL, "plan is NULL");
  if (!dst) return fail(MUONH_EINVAL, "dst is NULL");
  if (index < 0 || index >= plan->n_mats)
    return fail(MUONH_ESHAPE, "index %lld out of [0, %lld)", (long long)index,
                (long long)plan->n_mats);
  int err = 0;
  if (!check_ws(plan, workspace, workspace_bytes, &err)) return err;
  const GroupPlan* G = nullptr;
  for (const GroupPlan& g : plan->groups)
    if (index >= g.first && index < g.first + g.count) G = &g;
  const char* blk = static_cast<const char*>(workspace) + G->off + (index - G->first) * G->mat_bytes;
  const char* D = blk + off_update(plan, *G);
  const int ld = G->trans ? G->sp : G->lp;
  hipError_t e = launch_read_update(plan->prec, D, ld, G->rows, G->cols, dst,
                                    reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read update");
  return MUONH_OK;
}

}  // extern "C"
