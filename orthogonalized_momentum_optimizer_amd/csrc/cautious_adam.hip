// Cautious Adam for the non-matrix parameters: host validation and launches of the C ABI in
// include/cautious_adam.h, and its one fused elementwise kernel.
//
// The optimizer is the one the RecursiveFromBest record analysis (lqnn.cn, section 3.3)
// describes for the embedding-like parameters: Adam whose weight decay is applied only
// where the update and the parameter agree in sign, with a decay multiplier per tensor.
//
// The kernel is a single pass over HBM: each element is read once (p, g, m, v) and written
// once (p, m, v), 22 bytes per element for bf16 p and g with fp32 moments. Each block owns a
// chunk of kChunk contiguous elements of one tensor; each thread moves 8 consecutive
// elements per access (16-byte loads and stores) and issues all of its chunk's loads before
// any arithmetic, so a wavefront keeps several kilobytes in flight. Only the last chunk of
// a tensor takes the guarded path with a per-element tail.
#include <algorithm>
#include <cmath>
#include <vector>

#include "cautious_adam.h"
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                        // elements per thread per access
constexpr int kUnroll = 2;                     // accesses per thread per chunk
constexpr int kChunk = kThreads * kVec * kUnroll;  // 4096 elements per block
constexpr int kMaxPieces = 32;                 // tensor pieces per launch (passed by value)
constexpr int64_t kPieceElems = int64_t(1) << 29;  // longest piece of a tensor per launch
constexpr int64_t kMaxBlocks = kPieceElems / kChunk;  // blocks per launch
constexpr int64_t kMaxNumel = int64_t(1) << 40;

struct AdamLaunch {
  void* p[kMaxPieces];
  const void* g[kMaxPieces];
  float* m[kMaxPieces];
  float* v[kMaxPieces];
  int64_t numel[kMaxPieces];
  float lam[kMaxPieces];                       // weight_decay * wd_mul
  int chunk0[kMaxPieces + 1];                  // first block of each piece; [count] = grid
  int count;
  float lr, beta1, beta2, eps;
  float inv_bc1;                               // 1 / (1 - beta1^t)
  float inv_sqrt_bc2;                          // 1 / sqrt(1 - beta2^t)
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16-byte global accesses
template <typename T>
__device__ __forceinline__ T ld16(const T* p) { return *p; }
template <typename T>
__device__ __forceinline__ void st16(T* p, T v) { *p = v; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bfloat16 in one dword (lo = first), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8 consecutive elements of a bf16 (DT 0) or fp32 (DT 1) buffer.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t i, float x[8]) {
  if (DT == 0) {
    const u32x4 w = ld16(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + i));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(w[k]);
      x[2 * k + 1] = bf16_hi(w[k]);
    }
  } else {
    const f32x4* q = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
    const f32x4 a = ld16(q), b = ld16(q + 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a[k];
      x[4 + k] = b[k];
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t i, const float x[8]) {
  if (DT == 0) {
    const u32x4 w = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                     pack_bf16(x[6], x[7])};
    st16(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + i), w);
  } else {
    f32x4* q = reinterpret_cast<f32x4*>(static_cast<float*>(base) + i);
    st16(q, f32x4{x[0], x[1], x[2], x[3]});
    st16(q + 1, f32x4{x[4], x[5], x[6], x[7]});
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
  if (DT == 0) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[i]) << 16);
  return static_cast<const float*>(base)[i];
}

template <int DT>
__device__ __forceinline__ void store1(void* base, int64_t i, float x) {
  if (DT == 0) static_cast<uint16_t*>(base)[i] = uint16_t(pack_bf16(x, 0.f) & 0xffffu);
  else static_cast<float*>(base)[i] = x;
}

// The step on one element, in fp32; p, m and v are updated in place.
__device__ __forceinline__ void adam_elem(const AdamLaunch& L, float lam, float& p, float g,
                                          float& m, float& v) {
  m = fmaf(L.beta1, m, (1.f - L.beta1) * g);
  v = fmaf(L.beta2, v, (1.f - L.beta2) * (g * g));
  const float denom = fmaf(sqrtf(v), L.inv_sqrt_bc2, L.eps);
  float u = (m * L.inv_bc1) / denom;
  // cautious decay: only where the update and the parameter have the same (nonzero) sign
  const bool agree = (u > 0.f && p > 0.f) || (u < 0.f && p < 0.f);
  u = agree ? fmaf(lam, p, u) : u;
  p = fmaf(-L.lr, u, p);
}

template <int PDT, int GDT>
__global__ __launch_bounds__(kThreads) void cautious_adam_kernel(const AdamLaunch L) {
  const int b = blockIdx.x;
  int q = 0;
  while (q + 1 < L.count && L.chunk0[q + 1] <= b) ++q;
  void* const P = L.p[q];
  const void* const G = L.g[q];
  float* const M = L.m[q];
  float* const V = L.v[q];
  const float lam = L.lam[q];
  const int64_t n = L.numel[q];
  const int64_t base = int64_t(b - L.chunk0[q]) * kChunk;
  const int t = threadIdx.x;

  if (base + kChunk <= n) {
    // full chunk: every access is a whole 8-element vector
    float p[kUnroll][kVec], g[kUnroll][kVec], m[kUnroll][kVec], v[kUnroll][kVec];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + int64_t(u * kThreads + t) * kVec;
      load8<PDT>(P, i, p[u]);
      load8<GDT>(G, i, g[u]);
      load8<1>(M, i, m[u]);
      load8<1>(V, i, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + int64_t(u * kThreads + t) * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) adam_elem(L, lam, p[u][e], g[u][e], m[u][e], v[u][e]);
      store8<PDT>(P, i, p[u]);
      store8<1>(M, i, m[u]);
      store8<1>(V, i, v[u]);
    }
    return;
  }
  // the last chunk of a tensor: whole vectors where they fit, single elements after
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + int64_t(u * kThreads + t) * kVec;
    if (i + kVec <= n) {
      float p[kVec], g[kVec], m[kVec], v[kVec];
      load8<PDT>(P, i, p);
      load8<GDT>(G, i, g);
      load8<1>(M, i, m);
      load8<1>(V, i, v);
#pragma unroll
      for (int e = 0; e < kVec; ++e) adam_elem(L, lam, p[e], g[e], m[e], v[e]);
      store8<PDT>(P, i, p);
      store8<1>(M, i, m);
      store8<1>(V, i, v);
    } else {
      for (int64_t j = i; j < n; ++j) {
        float p = load1<PDT>(P, j), m = M[j], v = V[j];
        adam_elem(L, lam, p, load1<GDT>(G, j), m, v);
        store1<PDT>(P, j, p);
        M[j] = m;
        V[j] = v;
      }
    }
  }
}

typedef void (*AdamKernel)(AdamLaunch);

AdamKernel kernel_for(muon_dtype pdt, muon_dtype gdt) {
  if (pdt == MUON_DT_BF16)
    return gdt == MUON_DT_BF16 ? cautious_adam_kernel<0, 0> : cautious_adam_kernel<0, 1>;
  return gdt == MUON_DT_BF16 ? cautious_adam_kernel<1, 0> : cautious_adam_kernel<1, 1>;
}

size_t dt_bytes(muon_dtype d) { return d == MUON_DT_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_config(const muon_adam_config* cfg) {
  if (!cfg) return fail(MUON_ERR_INVALID_ARG, "cfg is NULL");
  if (!std::isfinite(cfg->lr) || !std::isfinite(cfg->eps) || !std::isfinite(cfg->weight_decay))
    return fail(MUON_ERR_INVALID_ARG, "lr, eps and weight_decay must be finite");
  if (cfg->eps < 0.f) return fail(MUON_ERR_INVALID_ARG, "eps must be >= 0");
  if (!(cfg->beta1 >= 0.f && cfg->beta1 < 1.f) || !(cfg->beta2 >= 0.f && cfg->beta2 < 1.f))
    return fail(MUON_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)");
  if (cfg->step < 1) return fail(MUON_ERR_INVALID_ARG, "step = %lld < 1", (long long)cfg->step);
  return MUON_OK;
}

int check_tensors(const muon_adam_tensor* ts, int64_t n) {
  std::vector<Range> rs;
  rs.reserve(4 * n);
  for (int64_t i = 0; i < n; ++i) {
    const muon_adam_tensor& T = ts[i];
    if (T.numel < 0 || T.numel > kMaxNumel)
      return fail(T.numel < 0 ? MUON_ERR_INVALID_ARG : MUON_ERR_UNSUPPORTED,
                  "tensor %lld: numel %lld outside [0, 2^40]", (long long)i, (long long)T.numel);
    if ((T.param_dtype != MUON_DT_BF16 && T.param_dtype != MUON_DT_F32) ||
        (T.grad_dtype != MUON_DT_BF16 && T.grad_dtype != MUON_DT_F32))
      return fail(MUON_ERR_INVALID_ARG, "tensor %lld: unknown dtype (%d, %d)", (long long)i,
                  (int)T.param_dtype, (int)T.grad_dtype);
    if (!std::isfinite(T.wd_mul))
      return fail(MUON_ERR_INVALID_ARG, "tensor %lld: wd_mul must be finite", (long long)i);
    if (T.numel == 0) continue;
    if (!T.param || !T.grad || !T.exp_avg || !T.exp_avg_sq)
      return fail(MUON_ERR_INVALID_ARG,
                  "tensor %lld: param, grad, exp_avg and exp_avg_sq must be non-NULL",
                  (long long)i);
    if (!aligned16(T.param) || !aligned16(T.grad) || !aligned16(T.exp_avg) ||
        !aligned16(T.exp_avg_sq))
      return fail(MUON_ERR_INVALID_ARG, "tensor %lld: buffers must be 16-byte aligned",
                  (long long)i);
    auto add = [&](const void* ptr, size_t bytes, bool w) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
      rs.push_back({lo, lo + bytes, w});
    };
    const size_t e = (size_t)T.numel;
    add(T.param, e * dt_bytes(T.param_dtype), true);
    add(T.grad, e * dt_bytes(T.grad_dtype), false);
    add(T.exp_avg, e * 4, true);
    add(T.exp_avg_sq, e * 4, true);
  }
  return check_overlaps(rs);
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

void muon_adam_config_default(muon_adam_config* cfg) {
  if (!cfg) return;
  cfg->lr = 1e-3f;
  cfg->beta1 = 0.9f;
  cfg->beta2 = 0.999f;
  cfg->eps = 1e-8f;
  cfg->weight_decay = 0.f;
  cfg->step = 1;
}

int muon_cautious_adam_step(const muon_adam_tensor* tensors, int64_t n,
                            const muon_adam_config* cfg, hipStream_t stream) {
  clear_error();
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (int st = check_config(cfg)) return st;
  if (n == 0) return MUON_OK;
  if (!tensors) return fail(MUON_ERR_INVALID_ARG, "tensors is NULL");
  if (int st = check_tensors(tensors, n)) return st;

  AdamLaunch L;
  L.lr = cfg->lr;
  L.beta1 = cfg->beta1;
  L.beta2 = cfg->beta2;
  L.eps = cfg->eps;
  const double t = (double)cfg->step;
  L.inv_bc1 = (float)(1.0 / (1.0 - std::pow((double)cfg->beta1, t)));
  L.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow((double)cfg->beta2, t)));

  // Tensors of one dtype pair share launches. A tensor longer than one launch's blocks can
  // cover is cut into pieces at chunk boundaries (so pieces stay 16-byte aligned).
  const int64_t piece_max = kPieceElems;
  for (int pdt = 0; pdt < 2; ++pdt)
    for (int gdt = 0; gdt < 2; ++gdt) {
      const AdamKernel k = kernel_for((muon_dtype)pdt, (muon_dtype)gdt);
      L.count = 0;
      int64_t blocks = 0;
      auto flush = [&]() -> int {
        if (L.count == 0) return MUON_OK;
        L.chunk0[L.count] = (int)blocks;
        hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, L);
        const hipError_t e = hipGetLastError();
        L.count = 0;
        blocks = 0;
        if (e != hipSuccess)
          return fail(MUON_ERR_HIP, "launch of the cautious Adam kernel failed: %s",
                      hipGetErrorString(e));
        return MUON_OK;
      };
      for (int64_t i = 0; i < n; ++i) {
        const muon_adam_tensor& T = tensors[i];
        if (T.numel == 0 || (int)T.param_dtype != pdt || (int)T.grad_dtype != gdt) continue;
        const float lam = cfg->weight_decay * T.wd_mul;
        if (!std::isfinite(lam))
          return fail(MUON_ERR_INVALID_ARG, "tensor %lld: weight_decay * wd_mul overflows",
                      (long long)i);
        for (int64_t off = 0; off < T.numel; off += piece_max) {
          const int64_t len = std::min(piece_max, T.numel - off);
          const int64_t nb = (len + kChunk - 1) / kChunk;
          if (L.count == kMaxPieces || blocks + nb > kMaxBlocks)
            if (int st = flush()) return st;
          const int c = L.count++;
          L.p[c] = static_cast<char*>(T.param) + off * dt_bytes(T.param_dtype);
          L.g[c] = static_cast<const char*>(T.grad) + off * dt_bytes(T.grad_dtype);
          L.m[c] = T.exp_avg + off;
          L.v[c] = T.exp_avg_sq + off;
          L.numel[c] = len;
          L.lam[c] = lam;
          L.chunk0[c] = (int)blocks;
          blocks += nb;
        }
      }
      if (int st = flush()) return st;
    }
  return MUON_OK;
}

}  // extern "C"
