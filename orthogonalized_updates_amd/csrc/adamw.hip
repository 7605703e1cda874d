// AdamW for the parameters outside the MuonH group (model card page "Puro",
// section "Training": those parameters use AdamW with weight decay 0.1).
//
// One grouped launch per batch of up to kMaxAdamTensors flat fp32 tensors (a
// model's whole non-matrix set fits one launch): each block takes
// kAdamBlockElems consecutive elements of one tensor, found by binary search
// over the batch's cumulative block counts, and
// applies, per element (decoupled decay, bias-corrected moments),
//   p <- p * (1 - lr*wd)
//   m <- beta1*m + (1 - beta1)*g
//   v <- beta2*v + (1 - beta2)*g^2
//   p <- p - (lr / (1 - beta1^t)) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
// in fp32, the step constants computed in fp64 on the host. Reads p, g, m, v
// and writes p, m, v: 28 bytes per element, HBM-bound. A full block whose four
// tensors are 16-byte aligned issues all of its loads first (two float4 per
// stream per thread), then computes and stores, with non-temporal loads and
// stores: on MI355X this read-modify-write stream runs about 6% faster with
// the hint on both sides (and no faster with it on one side only). Partial
// and misaligned blocks take plain vector or scalar accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/muonh.h"

namespace muonh {

// Defined in muonh_abi.hip: sets the thread's error message, returns `code`.
int set_error(int code, const char* msg);

namespace {

constexpr int kAdamThreads = 256;
constexpr int kAdamUnroll = 2;         // float4 per stream per thread (full blocks)
constexpr int kAdamBlockElems = kAdamThreads * 4 * kAdamUnroll;  // 2048
constexpr int kMaxAdamTensors = 128;  // kernel arguments stay near 2 KB

struct AdamArgs {
  int64_t n[kMaxAdamTensors];
  int64_t block_begin[kMaxAdamTensors + 1];  // cumulative block counts
  int first;                                // index of this batch's first tensor
  int count;
  float decay;      // 1 - lr*wd
  float beta1, one_minus_beta1, beta2, one_minus_beta2;
  float step_size;  // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
};

__device__ __forceinline__ float adam_elem(float& p, float g, float& m, float& v, const AdamArgs& a) {
  p *= a.decay;
  m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
  v = fmaf(a.beta2, v, a.one_minus_beta2 * g * g);
  const float den = sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
  p -= a.step_size * (m / den);
  return p;
}

typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_nt(const float* q) {
  const f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(q));
  return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void store_nt(const float4& a, float* q) {
  const f4v x = {a.x, a.y, a.z, a.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f4v*>(q));
}

__device__ __forceinline__ void adam4(float4& p, const float4& g, float4& m, float4& v,
                                      const AdamArgs& a) {
  adam_elem(p.x, g.x, m.x, v.x, a);
  adam_elem(p.y, g.y, m.y, v.y, a);
  adam_elem(p.z, g.z, m.z, v.z, a);
  adam_elem(p.w, g.w, m.w, v.w, a);
}

__global__ __launch_bounds__(kAdamThreads) void k_adamw(AdamArgs a, float* const* P,
                                                       const float* const* G, float* const* M,
                                                       float* const* V) {
  // First tensor whose block range ends after this block (empty tensors have
  // empty ranges and are never chosen); uniform for the block.
  const int64_t b = blockIdx.x;
  int t = 0, last = a.count - 1;
  while (t < last) {
    const int mid = (t + last) >> 1;
    if (a.block_begin[mid + 1] > b) last = mid; else t = mid + 1;
  }
  const int idx = a.first + t;
  const int64_t lo = (int64_t)(blockIdx.x - a.block_begin[t]) * kAdamBlockElems;
  const int64_t hi = lo + kAdamBlockElems < a.n[t] ? lo + kAdamBlockElems : a.n[t];
  float* p = P[idx];
  const float* g = G[idx];
  float* m = M[idx];
  float* v = V[idx];
  const bool vec = ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g) |
                     reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v)) & 15u) == 0;
  if (vec && hi - lo == kAdamBlockElems) {
    float4 pv[kAdamUnroll], gv[kAdamUnroll], mv[kAdamUnroll], vv[kAdamUnroll];
#pragma unroll
    for (int u = 0; u < kAdamUnroll; ++u) {
      const int64_t e = lo + 4 * (threadIdx.x + u * kAdamThreads);
      pv[u] = load_nt(p + e);
      gv[u] = load_nt(g + e);
      mv[u] = load_nt(m + e);
      vv[u] = load_nt(v + e);
    }
#pragma unroll
    for (int u = 0; u < kAdamUnroll; ++u) {
      const int64_t e = lo + 4 * (threadIdx.x + u * kAdamThreads);
      adam4(pv[u], gv[u], mv[u], vv[u], a);
      store_nt(pv[u], p + e);
      store_nt(mv[u], m + e);
      store_nt(vv[u], v + e);
    }
    return;
  }
  int64_t mid = lo;
  if (vec) {
    const int64_t n4 = (hi - lo) >> 2;
    for (int64_t i = threadIdx.x; i < n4; i += kAdamThreads) {
      const int64_t e = lo + 4 * i;
      float4 pv = *reinterpret_cast<const float4*>(p + e);
      const float4 gv = *reinterpret_cast<const float4*>(g + e);
      float4 mv = *reinterpret_cast<const float4*>(m + e);
      float4 vv = *reinterpret_cast<const float4*>(v + e);
      adam4(pv, gv, mv, vv, a);
      *reinterpret_cast<float4*>(p + e) = pv;
      *reinterpret_cast<float4*>(m + e) = mv;
      *reinterpret_cast<float4*>(v + e) = vv;
    }
    mid = lo + (n4 << 2);
  }
  for (int64_t e = mid + threadIdx.x; e < hi; e += kAdamThreads) {
    float pe = p[e], me = m[e], ve = v[e];
    adam_elem(pe, g[e], me, ve, a);
    p[e] = pe;
    m[e] = me;
    v[e] = ve;
  }
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return set_error(code, buf);
}

}  // namespace
}  // namespace muonh

extern "C" int muonh_adamw_step(int32_t n_tensors, const int64_t* sizes, float* const* P,
                                const float* const* G, float* const* M, float* const* V,
                                float lr, float beta1, float beta2, float eps,
                                float weight_decay, int32_t step, void* stream) {
  using namespace muonh;
  if (n_tensors < 0) return fail(MUONH_EINVAL, "n_tensors=%d must be >= 0", n_tensors);
  if (n_tensors == 0) return MUONH_OK;
  if (!sizes) return fail(MUONH_EINVAL, "sizes is NULL");
  if (!P || !G || !M || !V) return fail(MUONH_EINVAL, "P, G, M and V must be device arrays");
  if (!std::isfinite(lr) || lr < 0.f) return fail(MUONH_EINVAL, "lr=%g must be finite and >= 0", lr);
  if (!(beta1 >= 0.f && beta1 < 1.f)) return fail(MUONH_EINVAL, "beta1=%g must be in [0, 1)", beta1);
  if (!(beta2 >= 0.f && beta2 < 1.f)) return fail(MUONH_EINVAL, "beta2=%g must be in [0, 1)", beta2);
  if (!std::isfinite(eps) || eps < 0.f) return fail(MUONH_EINVAL, "eps=%g must be finite and >= 0", eps);
  if (!std::isfinite(weight_decay) || weight_decay < 0.f)
    return fail(MUONH_EINVAL, "weight_decay=%g must be finite and >= 0", weight_decay);
  if (step < 1) return fail(MUONH_EINVAL, "step=%d must be >= 1 (1-based)", step);
  for (int32_t i = 0; i < n_tensors; ++i)
    if (sizes[i] < 0 || sizes[i] > MUONH_MAX_TENSOR_ELEMS)
      return fail(MUONH_ESHAPE, "sizes[%d]=%lld out of [0, %lld]", i, (long long)sizes[i],
                  (long long)MUONH_MAX_TENSOR_ELEMS);

  AdamArgs a;
  a.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  a.beta1 = beta1;
  a.one_minus_beta1 = (float)(1.0 - (double)beta1);
  a.beta2 = beta2;
  a.one_minus_beta2 = (float)(1.0 - (double)beta2);
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  a.step_size = (float)((double)lr / bc1);
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  a.eps = eps;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t t0 = 0; t0 < n_tensors; t0 += kMaxAdamTensors) {
    const int cnt = std::min<int32_t>(kMaxAdamTensors, n_tensors - t0);
    a.first = t0;
    a.count = cnt;
    int64_t blocks = 0;
    for (int i = 0; i < cnt; ++i) {
      a.n[i] = sizes[t0 + i];
      a.block_begin[i] = blocks;
      blocks += (sizes[t0 + i] + kAdamBlockElems - 1) / kAdamBlockElems;
    }
    a.block_begin[cnt] = blocks;
    if (blocks == 0) continue;
    if (blocks > 0x7fffffff) return fail(MUONH_ESHAPE, "too many blocks in one launch");
    hipLaunchKernelGGL(k_adamw, dim3((unsigned)blocks), dim3(kAdamThreads), 0, s, a, P, G, M, V);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(MUONH_EHIP, "adamw launch: %s (%d)", hipGetErrorString(e), (int)e);
  }
  return MUONH_OK;
}
