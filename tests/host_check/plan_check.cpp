// Host-side check of the MuonH library's plan, validation and launch
// descriptors, built from the library's own host source (muonh_abi.hip) with
// AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU: the HIP
// runtime calls and the kernel launchers are replaced by the stubs below.
// Every launcher stub checks its descriptor against the plan: each operand
// and output region lies inside its matrix block and the block inside the
// workspace, inputs and outputs of a product do not overlap, block counts
// and partial-sum indices stay in range, and the tile positions of every
// GEMM launch (static slots plus tail claims) cover each tile of each group
// exactly once. The driver runs the calls of the ABI over many plans (ragged
// shapes, more groups than one launch holds, the benchmark sets, the largest
// dimension, every precision and storage flag, 0 to 8 iterations) with fake
// device addresses that are never dereferenced.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <set>
#include <utility>
#include <vector>

#include "muonh.h"
#include "muonh_internal.h"

using namespace muonh;

// ---------------------------------------------------------------------------
// what the current call may touch
// ---------------------------------------------------------------------------
namespace {
uintptr_t g_ws_lo = 0, g_ws_hi = 0;
int64_t g_nmats = 0;
int g_eb = 2;       // bytes per logical Newton-Schulz element
int g_tile = 256;   // GEMM tile edge
int g_failures = 0;
long g_gemm_launches = 0, g_ew_launches = 0, g_events = 0, g_small_launches = 0;
const char* g_case = "";

#define EXPECT(c)                                                                    \
  do {                                                                               \
    if (!(c)) {                                                                      \
      if (g_failures++ < 20) std::printf("FAIL [%s] %s:%d: %s\n", g_case, __FILE__, __LINE__, #c); \
    }                                                                                \
  } while (0)

bool in_ws(uintptr_t lo, uintptr_t hi) { return lo >= g_ws_lo && hi <= g_ws_hi && lo <= hi; }

struct Region {
  int64_t off, bytes;
};

bool disjoint(Region a, Region b) {
  if (a.off < 0 || b.off < 0) return true;
  return a.off + a.bytes <= b.off || b.off + b.bytes <= a.off;
}

void check_partials(const void* p) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  EXPECT(in_ws(lo, lo + (uintptr_t)g_nmats * kMaxPartials * sizeof(double)));
}

void check_norms(const void* p) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  EXPECT(in_ws(lo, lo + (uintptr_t)g_nmats * sizeof(double)));
}

// kind: 0 streaming (bpm blocks, partials), 1 tiles, 2 fused (bpm blocks of
// tpb tiles, partials), 3 one-shot writers, 4 fallback (8 blocks per matrix)
void check_ew(const EwArgs& a, int kind) {
  ++g_ew_launches;
  EXPECT(a.ngroups >= 1 && a.ngroups <= kMaxEwGroups);
  int64_t blocks = 0;
  for (int i = 0; i < a.ngroups; ++i) {
    const EwGroup& g = a.g[i];
    EXPECT(g.count >= 1 && g.first >= 0 && g.first + g.count <= g_nmats);
    EXPECT(g.n == (int64_t)g.rows * g.cols);
    EXPECT(g.rp % kPad == 0 && g.cp % kPad == 0 && g.rp >= g.rows && g.cp >= g.cols);
    EXPECT(g.tiles_per_mat == (g.rp / 64) * (g.cp / 64));
    const uintptr_t base = reinterpret_cast<uintptr_t>(g.ns_base);
    EXPECT(in_ws(base, base + (uintptr_t)g.count * g.mat_bytes));
    const int64_t plane = (int64_t)g.rp * g.cp * g_eb;
    if (g.offD >= 0) EXPECT(g.offD + plane <= g.mat_bytes);
    if (g.offE >= 0) EXPECT(g.offE + plane <= g.mat_bytes);
    EXPECT(g.defer == (g.n > kSmallMatElems ? 1 : 0));
    if (kind != 4) EXPECT(g.block_begin == blocks);
    int64_t per = 0;
    switch (kind) {
      case 0: per = g.bpm; EXPECT(g.bpm >= 1 && g.bpm <= kMaxPartials); break;
      case 1: per = g.tiles_per_mat; break;
      case 2:
        per = g.bpm;
        EXPECT(g.bpm >= 1 && g.bpm <= kMaxPartials && g.tpb >= 1);
        EXPECT((int64_t)g.bpm * g.tpb >= g.tiles_per_mat && (int64_t)(g.bpm - 1) * g.tpb < g.tiles_per_mat);
        break;
      case 3: {
        const int64_t units = (int64_t)((g.rows + 1) / 2) * ((g.cols + 3) / 4);
        per = g.bpm;
        EXPECT(g.bpm >= 1 && (int64_t)g.bpm * 2 * kEwThreads >= units);
        break;
      }
      case 4: per = 8; break;
    }
    blocks += per * g.count;
  }
  if (kind != 4) EXPECT(a.nblocks == blocks);
  EXPECT(blocks <= INT32_MAX);
}

// The tile a launch position maps to (the kernels' deal: 8 XCD lists, each a
// contiguous eighth of every group's tile list in group order).
bool position_tile(const GemmArgs& a, int x, int slot, int& gi, int& local) {
  for (int i = 0; i < a.ngroups; ++i) {
    const int64_t tot = (int64_t)a.g[i].count * a.g[i].tiles_per_mat;
    const int lo = (int)((x * tot) >> 3), hi = (int)(((x + 1) * tot) >> 3);
    if (slot < hi - lo) {
      gi = i;
      local = lo + slot;
      return true;
    }
    slot -= hi - lo;
  }
  return false;
}

void check_gemm(GemmMode mode, NsPrec prec, const GemmArgs& a) {
  ++g_gemm_launches;
  const bool sym = mode != kApply;
  EXPECT(a.ngroups >= 1 && a.ngroups <= kMaxGemmGroups);
  int64_t tiles = 0;
  for (int i = 0; i < a.ngroups; ++i) {
    const GemmGroup& g = a.g[i];
    // 128x128 tiles only for bf16 launches whose 256x256 tiles would fill at
    // most half of the 256 CUs
    const int T = a.small ? 128 : g_tile;
    if (a.small) EXPECT(prec == kBf16 && g_tile == 256);
    EXPECT(g.count >= 1 && g.first >= 0 && g.first + g.count <= g_nmats);
    EXPECT(g.K % kPad == 0 && g.K >= kPad);
    EXPECT(g.tile_begin == tiles);
    EXPECT(g.tiles_per_mat == (sym ? g.tm * (g.tm + 1) / 2 : g.tm * g.tn));
    // a symmetric product reads one operand on both sides (P P^T): the
    // kernels compute upper tiles only, and a diagonal tile's lower-left
    // quadrant as the mirror of its upper-right one
    if (sym) EXPECT(g.tm == g.tn && g.offP == g.offQ && g.ldp == g.ldq);
    if (i > 0) EXPECT(a.g[i - 1].K >= g.K);   // heaviest groups first
    tiles += (int64_t)g.count * g.tiles_per_mat;
    const uintptr_t base = reinterpret_cast<uintptr_t>(g.base);
    EXPECT(in_ws(base, base + (uintptr_t)g.count * g.mat_bytes));
    const int64_t rows_p = (int64_t)g.tm * T, rows_q = (int64_t)g.tn * T;
    Region P{g.offP, rows_p * g.ldp * g_eb};
    // the bf16 and split apply reads its Q operand X K-major (K rows)
    const bool qt = mode == kApply && prec != kFp32;
    Region Q{g.offQ, (qt ? (int64_t)g.K : rows_q) * g.ldq * g_eb};
    Region E{g.offE, rows_p * g.lde * g_eb};
    Region O1{g.offO1, rows_p * g.ldo1 * g_eb};
    Region O2{g.offO2, rows_q * g.ldo2 * g_eb};
    EXPECT(g.offP >= 0 && g.offQ >= 0);
    EXPECT(g.ldp == g.K);
    if (!qt) EXPECT(g.ldq == g.K);
    EXPECT(g.offO1 >= 0 || g.offO2 >= 0);
    for (Region r : {P, Q, E, O1, O2})
      if (r.off >= 0) EXPECT(r.off + r.bytes <= g.mat_bytes);
    // no product reads what it writes; the one exception is the fp32
    // apply's E term, which reads X's own tile in the epilogue and writes
    // the same elements (X updated in place, element by element)
    for (Region in : {P, Q})
      for (Region out : {O1, O2}) EXPECT(disjoint(in, out));
    const bool in_place = prec == kFp32 && mode == kApply && g.offE == g.offO1 && g.lde == g.ldo1;
    if (!in_place) EXPECT(disjoint(E, O1));
    EXPECT(disjoint(E, O2));
    if (mode == kApply) {
      EXPECT(g.fold == (g.fold ? 1 : 0));
      if (g.fold) EXPECT(g.offE < 0);   // B carries a*I: no a*X term
      if (!g.fold && prec == kFp32) EXPECT(g.offE >= 0);
    }
    if (mode == kGram) EXPECT(g.offE < 0);
    if (mode == kPoly) EXPECT(g.offE >= 0);
  }
  EXPECT(a.ntiles == tiles);
  if (prec == kBf16) {
    // the choice of tile: the phase's 256-tile count (this launch's, when
    // the phase is one launch) against half of the CUs
    int64_t big = 0;
    for (int i = 0; i < a.ngroups; ++i) {
      const GemmGroup& g = a.g[i];
      const int64_t f = a.small ? 2 : 1;  // 128-tile grid -> 256-tile grid
      const int64_t ts = (g.tm + f - 1) / f, tl = (g.tn + f - 1) / f;
      big += (int64_t)g.count * (sym ? ts * (ts + 1) / 2 : ts * tl);
    }
    if (a.small) EXPECT(2 * big <= 256);
    if (a.small) ++g_small_launches;
  }
  if (a.xnorm) check_norms(a.xnorm);
  if (mode == kPoly) EXPECT(a.xnorm == nullptr && a.diag == kNsA);
  // every tile exactly once: static slots, then tail claims
  if (a.xcd_map) {
    EXPECT(a.grid % 8 == 0);
    const int slots = a.grid / 8;
    int64_t listed = 0, claimers = 0, tail = 0;
    std::set<std::pair<int, int>> seen;
    for (int x = 0; x < 8; ++x) {
      listed += a.xlen[x];
      const int stat = a.sched ? a.xstatic[x] : a.xlen[x];
      EXPECT(stat >= 0 && stat <= a.xlen[x] && stat <= slots);
      if (a.sched) {
        claimers += slots - stat;
        tail += a.xlen[x] - stat;
      }
      for (int s = 0; s < a.xlen[x]; ++s) {
        int gi = -1, local = -1;
        EXPECT(position_tile(a, x, s, gi, local));
        EXPECT(seen.insert({gi, local}).second);
        EXPECT(local >= 0 && local < a.g[gi].count * a.g[gi].tiles_per_mat);
      }
    }
    EXPECT(listed == tiles && (int64_t)seen.size() == tiles);
    EXPECT(claimers >= tail);   // every tail position finds a block
    if (a.sched) {
      const uintptr_t s = reinterpret_cast<uintptr_t>(a.sched);
      const uintptr_t c = reinterpret_cast<uintptr_t>(a.sched_clear);
      EXPECT(in_ws(s, s + 8 * sizeof(int)) && in_ws(c, c + 8 * sizeof(int)) && s != c);
    }
  } else {
    EXPECT(a.grid == a.ntiles);
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// launcher stubs (the library's kernels are not built into this program)
// ---------------------------------------------------------------------------
namespace muonh {
int gemm_tile(NsPrec prec) { return prec == kFp32 ? 128 : 256; }
hipError_t launch_gemm(GemmMode mode, NsPrec prec, const GemmArgs& a, hipStream_t) {
  check_gemm(mode, prec, a);
  return hipSuccess;
}
hipError_t launch_zero_i32(int* p, int n, hipStream_t) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  EXPECT(n > 0 && in_ws(lo, lo + (uintptr_t)n * sizeof(int)));
  return hipSuccess;
}
hipError_t launch_sumsq(const EwArgs& a, float* const* W, double* partials, hipStream_t) {
  check_ew(a, 0);
  EXPECT(W != nullptr);
  check_partials(partials);
  return hipSuccess;
}
hipError_t launch_momentum(const EwArgs& a, StateFmt, const void* const* G, void* const* M, float,
                           double* partials, hipStream_t) {
  check_ew(a, 0);
  EXPECT(G && M);
  check_partials(partials);
  return hipSuccess;
}
hipError_t launch_finalize(const EwArgs& a, const double* partials, double* norms, float*,
                           hipStream_t, uint32_t* flags, uint32_t) {
  ++g_ew_launches;
  for (int i = 0; i < a.ngroups; ++i) EXPECT(a.g[i].first + a.g[i].count <= g_nmats);
  check_partials(partials);
  check_norms(norms);
  if (flags) {
    const uintptr_t f = reinterpret_cast<uintptr_t>(flags);
    EXPECT(in_ws(f, f + 4));
  }
  return hipSuccess;
}
hipError_t launch_normcast(const EwArgs& a, NsPrec, StateFmt, const void* const* M, const double* norms,
                           hipStream_t) {
  check_ew(a, 1);
  EXPECT(M != nullptr);
  check_norms(norms);
  return hipSuccess;
}
hipError_t launch_momentum_cast(const EwArgs& a, NsPrec, StateFmt, const void* const* G, void* const* M,
                                float, double* partials, hipStream_t) {
  check_ew(a, 2);
  EXPECT(G && M);
  check_partials(partials);
  return hipSuccess;
}
hipError_t launch_cast_fallback(const EwArgs& a, NsPrec, StateFmt, const void* const*, const double* norms,
                                hipStream_t) {
  check_ew(a, 4);
  check_norms(norms);
  return hipSuccess;
}
hipError_t launch_update_norm(const EwArgs& a, NsPrec, float* const* W, float, double* partials,
                              hipStream_t) {
  check_ew(a, 0);
  EXPECT(W != nullptr);
  check_partials(partials);
  return hipSuccess;
}
hipError_t launch_project(const EwArgs& a, NsPrec, float* const*, const float* R, const double* norms,
                          float, hipStream_t) {
  check_ew(a, 3);
  EXPECT(R != nullptr);
  check_norms(norms);
  return hipSuccess;
}
hipError_t launch_decay_update(const EwArgs& a, NsPrec, float* const*, float, float, hipStream_t) {
  check_ew(a, 3);
  return hipSuccess;
}
hipError_t launch_read_update(NsPrec, const char* D, int ldD, int rows, int cols, float* dst, hipStream_t) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(D);
  EXPECT(dst && ldD >= cols && ldD % kPad == 0 && rows >= 1);
  EXPECT(in_ws(lo, lo + (uintptr_t)((rows + kPad - 1) / kPad * kPad) * ldD * g_eb));
  return hipSuccess;
}
}  // namespace muonh

// HIP runtime stubs: no device work exists in this program.
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void* sym) {
  *p = const_cast<void*>(sym);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  EXPECT(e != nullptr);
  ++g_events;
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void*, size_t n, hipMemcpyKind, hipStream_t) {
  std::memset(dst, 0, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }

// ---------------------------------------------------------------------------
// driver
// ---------------------------------------------------------------------------
namespace {
void* fake(uintptr_t v) { return reinterpret_cast<void*>(v); }

void run_plan(const char* name, std::vector<muonh_group_desc> groups, uint32_t flags) {
  g_case = name;
  muonh_plan* plan = nullptr;
  int st = muonh_plan_create(&plan, groups.data(), (int)groups.size(), flags);
  EXPECT(st == MUONH_OK);
  if (st != MUONH_OK) {
    std::printf("plan %s: %s\n", name, muonh_last_error());
    return;
  }
  const int64_t n = muonh_plan_num_matrices(plan);
  const size_t bytes = muonh_workspace_bytes(plan);
  g_nmats = n;
  g_eb = (flags & (MUONH_NS_FP32 | MUONH_NS_SPLIT_BF16)) ? 4 : 2;
  g_tile = (flags & MUONH_NS_FP32) ? 128 : 256;
  g_ws_lo = (uintptr_t)1 << 44;
  g_ws_hi = g_ws_lo + bytes;
  void* ws = fake(g_ws_lo);
  float* const* W = reinterpret_cast<float* const*>(fake(1 << 20));
  const void* const* G = reinterpret_cast<const void* const*>(fake(2 << 20));
  void* const* M = reinterpret_cast<void* const*>(fake(3 << 20));
  const float* R = reinterpret_cast<const float*>(fake(4 << 20));
  EXPECT(muonh_init(plan, const_cast<float* const*>(W), const_cast<float*>(R), ws, bytes, nullptr) == MUONH_OK);
  for (int k : {0, 1, 2, 5, 8}) {
    EXPECT(muonh_step(plan, W, G, M, R, 0.02f, 0.95f, k, ws, bytes, nullptr) == MUONH_OK);
    EXPECT(muonh_step_muon_wd(plan, W, G, M, 0.02f, 0.95f, 0.1f, k, ws, bytes, nullptr) == MUONH_OK);
    std::vector<void*> ev(3 * k + 3, fake(64));
    const long before = g_events;
    EXPECT(muonh_step_timed(plan, W, G, M, R, 0.02f, 0.95f, k, ws, bytes, nullptr, ev.data(),
                            (int)ev.size()) == MUONH_OK);
    EXPECT(g_events - before == 3 * k + 3);
    // a workspace one byte short, or misaligned, is refused before any launch
    const long launches = g_gemm_launches + g_ew_launches;
    EXPECT(muonh_step(plan, W, G, M, R, 0.02f, 0.95f, k, ws, bytes - 1, nullptr) == MUONH_EWORKSPACE);
    EXPECT(muonh_step(plan, W, G, M, R, 0.02f, 0.95f, k, fake(g_ws_lo + 16), bytes, nullptr) ==
           MUONH_EWORKSPACE);
    EXPECT(muonh_step(plan, W, G, M, R, 0.02f, 1.0f, k, ws, bytes, nullptr) == MUONH_EINVAL);
    EXPECT(g_gemm_launches + g_ew_launches == launches);
  }
  EXPECT(muonh_step(plan, W, G, M, R, 0.02f, 0.95f, MUONH_MAX_NS_ITERS + 1, ws, bytes, nullptr) ==
         MUONH_EINVAL);
  float* dst = reinterpret_cast<float*>(fake(5 << 20));
  EXPECT(muonh_read_update(plan, 0, dst, ws, bytes, nullptr) == MUONH_OK);
  EXPECT(muonh_read_update(plan, n - 1, dst, ws, bytes, nullptr) == MUONH_OK);
  EXPECT(muonh_read_update(plan, n, dst, ws, bytes, nullptr) == MUONH_ESHAPE);
  uint32_t fl = 9;
  EXPECT(muonh_step_status(plan, ws, bytes, nullptr, &fl) == MUONH_OK && fl == 0);
  // the fixed workspace of muonh_step_noalloc: used when the plan fits it
  if (bytes <= MUONH_NOALLOC_WORKSPACE_BYTES) {
    void* p = nullptr;
    // the stub hands out the host array itself as the "device" address
    EXPECT(hipGetSymbolAddress(&p, nullptr) == hipSuccess);
    (void)p;
  } else {
    EXPECT(muonh_step_noalloc(plan, W, G, M, R, 0.02f, 0.95f, 5, nullptr) == MUONH_EWORKSPACE);
  }
  muonh_plan_destroy(plan);
}

void check_disjoint_brute(uint64_t seed) {
  // muonh_check_disjoint against a quadratic check on random layouts
  g_case = "check_disjoint";
  std::vector<muonh_group_desc> groups = {{3, 5, 2}, {7, 2, 3}, {1, 9, 1}};
  muonh_plan* plan = nullptr;
  EXPECT(muonh_plan_create(&plan, groups.data(), 3, MUONH_MOM_BF16) == MUONH_OK);
  const int n = 6;
  const int64_t elems[6] = {15, 15, 14, 14, 14, 9};
  uint64_t s = seed;
  auto rnd = [&]() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (s >> 33) % 400;
  };
  for (int trial = 0; trial < 2000; ++trial) {
    std::vector<uintptr_t> w(n), g(n), m(n);
    for (int i = 0; i < n; ++i) {
      w[i] = 4096 + rnd() * 4;
      g[i] = 4096 + rnd() * 4;
      m[i] = 4096 + rnd() * 2;
    }
    bool overlap = false;
    std::vector<std::pair<uintptr_t, uintptr_t>> sp;
    for (int i = 0; i < n; ++i) {
      sp.push_back({w[i], w[i] + elems[i] * 4});
      sp.push_back({g[i], g[i] + elems[i] * 4});
      sp.push_back({m[i], m[i] + elems[i] * 2});
    }
    for (size_t a = 0; a < sp.size(); ++a)
      for (size_t b = a + 1; b < sp.size(); ++b)
        if (sp[a].first < sp[b].second && sp[b].first < sp[a].second) overlap = true;
    std::vector<const void*> wp(n), gp(n), mp(n);
    for (int i = 0; i < n; ++i) {
      wp[i] = fake(w[i]);
      gp[i] = fake(g[i]);
      mp[i] = fake(m[i]);
    }
    const int st = muonh_check_disjoint(plan, wp.data(), gp.data(), mp.data());
    EXPECT(st == (overlap ? MUONH_EALIAS : MUONH_OK));
  }
  muonh_plan_destroy(plan);
}
}  // namespace

int main() {
  const uint32_t precs[3] = {0u, MUONH_NS_SPLIT_BF16, MUONH_NS_FP32};
  const uint32_t states[3] = {0u, MUONH_GRAD_BF16 | MUONH_MOM_BF16, MUONH_MOM_BF16};
  std::vector<muonh_group_desc> ragged = {{1, 1, 1},     {3, 5, 1},     {5, 3, 1},   {1, 64, 1},
                                          {64, 1, 1},    {300, 200, 2}, {257, 129, 1},
                                          {130, 700, 1}, {511, 513, 1}, {129, 2052, 1},
                                          {1001, 1200, 1}};
  std::vector<muonh_group_desc> many;
  for (int i = 0; i < 40; ++i) many.push_back({8 + 7 * i, 300 - 6 * i, 1 + i % 3});
  std::vector<muonh_group_desc> qwen = {{2048, 2048, 56}, {512, 2048, 56}, {6144, 2048, 56}, {2048, 6144, 28}};
  std::vector<muonh_group_desc> occ = {{512, 1536, 256}, {1536, 512, 256}};
  std::vector<muonh_group_desc> large = {{4096, 14336, 32}, {14336, 4096, 32}};
  std::vector<muonh_group_desc> maxdim = {{65536, 256, 1}, {256, 65536, 1}, {65536, 1, 2}};
  // the largest square matrix: 2^32 entries, 32896 symmetric and 65536 apply tiles
  std::vector<muonh_group_desc> maxsq = {{65536, 65536, 1}};
  std::vector<muonh_group_desc> tail = {{512, 512, 96}, {768, 512, 96}};
  for (uint32_t p : precs)
    for (uint32_t s : states) {
      const uint32_t f = p | s;
      run_plan("ragged", ragged, f);
      run_plan("40 groups", many, f);
      run_plan("maximum dimension", maxdim, f);
      run_plan("tail balanced", tail, f);
    }
  for (uint32_t p : precs) {
    run_plan("largest square matrix", maxsq, p);
    run_plan("2B-shaped set", qwen, p);
    run_plan("occupancy set", occ, p);
    run_plan("4096x14336 set", large, p);
  }
  check_disjoint_brute(12345);
  std::printf("%ld GEMM launches (%ld with 128x128 tiles), %ld elementwise launches checked\n",
              g_gemm_launches, g_small_launches, g_ew_launches);
  EXPECT(g_small_launches > 0);
  if (g_failures) {
    std::printf("%d failures\n", g_failures);
    return 1;
  }
  std::printf("host check ok\n");
  return 0;
}
