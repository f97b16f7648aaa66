// Internal interfaces between the host plan (plan.hip) and the kernel launchers.
//
// Workspace matrices in bf16 (the bf16 rounds) use the tiled layout of toff(); in fp32 (the
// debug rounds) they are plain row-major.
// Every launcher enqueues on `stream`, returns the hipError_t of the launch, and assumes the
// host has validated shapes, pointers and the workspace layout.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace muon {

// Host-side error reporting shared by every entry point (muon_last_error reads it): fail
// stores the formatted message for this thread and returns `code`.
int fail(int code, const char* fmt, ...);
void clear_error();

// A byte range of a buffer an entry point receives.
struct Range {
  uintptr_t lo, hi;
  bool writable;
};
// MUON_OK, or MUON_ERR_INVALID_ARG when a written range overlaps any other range.
int check_overlaps(std::vector<Range>& rs);

constexpr int kPad = 128;        // wide shapes are padded to multiples of this

// Layout of the bf16 workspace matrices (X, A, B'; C columns, C a multiple of 32, rows a
// multiple of 16): 16 x 32 tiles of 1 KB, row-major inside a tile, tiles in row-major order.
// A 16-row by 32-column block, which one direct-to-LDS load instruction of the product
// kernels fetches, is then one contiguous kilobyte, and a 32-column step of K is +1 KB.
__host__ __device__ __forceinline__ size_t toff(int r, int c, int C) {
  return ((size_t)(r >> 4) * (size_t)(C >> 5) + (size_t)(c >> 5)) * 512u +
         (size_t)((r & 15) << 5) + (size_t)(c & 31);
}
constexpr int kTileBytes = 1024;  // one 16 x 32 bf16 tile
constexpr int kTile = 64;        // elementwise kernels work on 64x64 tiles
constexpr int kMaxPerLaunch = 48;  // matrices per elementwise launch (pointers travel by value)
constexpr int kRowParts = 8;       // row equaliser: partial row sums per slot (tall matrices)

// Elementwise launch over up to kMaxPerLaunch matrices of one shape and dtype pair.
// Matrix q of the launch owns slot (slot0 + q) of its group's workspace buffers.
struct ElemLaunch {
  const void* in[kMaxPerLaunch];   // K1: grad;  update: unused
  float* mom[kMaxPerLaunch];       // K1: momentum (nullptr = no momentum phase)
  void* param[kMaxPerLaunch];      // update: W (nullptr = write O only)
  void* out[kMaxPerLaunch];        // update: O destination (nullptr = none)
  int count;
  int rows, cols;                  // original orientation
  int tall;                        // rows > cols: the wide form is the transpose
  int mp, np;                      // padded wide shape (X is mp x np)
  int vec;                         // cols % 4 == 0: 4-wide vector access along rows
  void* x;                         // X buffer of slot0 (bf16 or f32), slot stride mp*np
  double* partials;                // K1: per-tile sums of squares of slot0
  const float* scales;             // per-slot {s1, s2, nu, 0} of slot0
  float beta;
  int nesterov;
  float lr;
  int apply_scale;                 // update: multiply X by s1 (ns_steps == 0)
  // row equaliser (per-slot arrays of np floats, slot0-based; nullptr = not used)
  float* rowvar[kMaxPerLaunch];    // finish: the caller's per-row state v
  float* rowsum;                   // rowstat: out; finish: in (kRowParts partial sums of O^2
                                   // per row, np floats each, per slot)
  float* rowf;                     // finish: out; update: per-row factor of O
  float row_beta, row_eps;
  const uint32_t* fault;           // update: nonzero word = the step's rounds failed (O := NaN)
};

// dtype codes: 0 = bf16, 1 = f32 (match muon_dtype)
hipError_t launch_momentum(const ElemLaunch& L, int grad_dt, int x_f32, hipStream_t s);
hipError_t launch_update(const ElemLaunch& L, int param_dt, int out_param_dt, int x_f32,
                         hipStream_t s);
// Row equaliser: rowstat writes each row's sum of O^2 (O in the caller's orientation, s1
// applied when apply_scale); finish updates the caller's row state and writes the per-row
// factors gamma / (sqrt(v_i) + eps) that the update kernel applies to O.
hipError_t launch_rowstat(const ElemLaunch& L, int x_f32, hipStream_t s);
hipError_t launch_roweq_finish(const ElemLaunch& L, hipStream_t s);
// Per-matrix norm finish: scales[4*i] = s1 = 1/(nu+eps), [4*i+1] = s1^2, [4*i+2] = nu. A
// matrix with nu outside [2^-40, 2^40] has its X0 (count matrices of mn elements at x0,
// bf16 or fp32) scaled in place by 2^-floor(log2 nu), and s1 = 2^floor(log2 nu) / (nu+eps).
hipError_t launch_norm(const double* partials, int tiles_per_mat, float* scales, int count,
                       float eps, void* x0, size_t mn, int x_f32, hipStream_t s);

// One batched Newton-Schulz product over a group of `batch` padded mp x np matrices.
struct NsGroup {
  void* x_in;          // X, batch x mp x np
  void* x_out;         // X', batch x mp x np
  void* a;             // A, batch x mp x mp
  void* b;             // B, batch x mp x mp
  const float* scales; // per matrix {s1, s2, nu, 0}; used when first != 0
  int batch, mp, np;
  int first;           // first round: fold the 1/nu normalisation into the epilogues
};
// bf16 storage, bf16 matrix cores with fp32 accumulation. The bf16 round folds a I into B:
// poly writes B' = aI + bA + cAA and apply forms s1 B' X. Each launcher takes one or more
// shape groups of a round (the step passes one group at a time, or all of them when they are
// too small to fill the device one by one). Gram and poly: groups with use_sym256
// (mp >= 1024) share 256x256-tile launches (ns_sym256_bf16.hip), smaller groups 128x128-tile
// launches (ns_gemm_bf16.hip); up to 8 groups per launch, tiles ordered longest first on
// every XCD. Apply: 256x256 tiles, groups of equal mp in one persistent launch, or 128x128
// tiles (one block each) when the 256x256 tiles number at most half the compute units
// (ns_apply_bf16.hip).
bool use_sym256(const NsGroup& g);
hipError_t launch_gram_bf16(const NsGroup* groups, int n, hipStream_t s);   // A = s2 X X^T
hipError_t launch_poly_bf16(const NsGroup* groups, int n, float a, float b, float c,
                            hipStream_t s);                                 // B' = aI+bA+cAA
hipError_t launch_apply_bf16(const NsGroup* groups, int n, hipStream_t s);  // X' = s1 B' X
int device_cus();  // compute units of the current device
hipError_t launch_gram256_bf16(const NsGroup* groups, int n, hipStream_t s);
// Four 128x128 blocks per work item (ns_quad_bf16.hip), for groups with mp a multiple of
// 256; mode 0 = gram, 1 = poly. quad_items: the group's work items.
bool use_quad(const NsGroup& g);
int quad_items(const NsGroup& g);
hipError_t launch_quad_bf16(const NsGroup* const* groups, int n, int mode, float a, float b,
                            float c, hipStream_t s);
hipError_t launch_poly256_bf16(const NsGroup* groups, int n, float a, float b, float c,
                               hipStream_t s);
// All rounds of a step as one persistent launch (ns_fused_bf16.hip): groups' X_0 in x_in,
// the result after `rounds` rounds in x_in for even rounds and x_out for odd; abc holds the
// rounds' (a, b, c); sync: fused_sync_words 4-byte words of workspace (cleared by the launch).
bool fused_rounds_ok(const NsGroup* groups, int n, int rounds);
size_t fused_sync_words(const NsGroup* groups, int n, int rounds);
hipError_t launch_fused_bf16(const NsGroup* groups, int n, int rounds, const float* abc,
                             uint32_t* sync, int max_polls, hipStream_t s);
// The word of a fused launch's sync area that is nonzero once one of its waits gave up.
inline uint32_t* fused_error_word(uint32_t* sync) { return sync + 8 * 16; }
// fp32 storage and arithmetic, the debug precision (ns_gemm_f32.hip): B = bA + cAA and
// X' = s1 (aX + BX), the round as written
hipError_t launch_gram_f32(const NsGroup& g, hipStream_t s);
hipError_t launch_poly_f32(const NsGroup& g, float b, float c, hipStream_t s);
hipError_t launch_apply_f32(const NsGroup& g, float a, hipStream_t s);

// The library's per-launch timing (muon_plan_set_profiling). While one launcher call of a
// step is timed, its first kernel launch records `start` when that kernel starts and every
// launch records `stop` when it ends, taken from the kernel dispatches themselves (no marker
// packets between the kernels, which would add their own latency to what is measured).
// Both are null when nothing is timed; then, and under stream capture, launches are plain.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTiming g_launch_timing;

template <typename... KArgs, typename... Args>
inline void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem,
                     hipStream_t s, Args... args) {
  if (g_launch_timing.stop) {
    hipEvent_t start = g_launch_timing.start;
    g_launch_timing.start = nullptr;  // later launches of the same call extend `stop` only
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, start, g_launch_timing.stop, 0u,
                          args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

}  // namespace muon
