// Device helpers shared by the bf16 Newton-Schulz product kernels (gfx950).
//
// Operand tiles move global -> LDS with 16-byte direct-to-LDS loads (global_load_lds):
// a wave instruction fills 1 KB of LDS linearly (lane l at byte 16 l), so the XOR swizzles
// below are applied by choosing which global 16-byte chunk each lane fetches. In global
// memory the bf16 matrices use the 16 x 32 tiled layout of toff() (muon_internal.h).
//
//  - K-contiguous tiles: ROWS rows x 32 K-values (4 chunks of 16 bytes per row); chunk c of
//    row r is stored at c ^ ((r >> 2) & 3). A fragment read (16 consecutive lanes = 16
//    consecutive rows, same chunk) then covers all 64 LDS banks (measured conflict-free;
//    keying on bits 1-2 of the row measured 2-way conflicted).
//  - N-contiguous tiles: 32 K-rows x COLS N-values (COLS/8 chunks per row); chunk c of K-row
//    k is stored at c ^ 2(k & 3). Fragments come from ds_read_b64_tr_b16: in each 16-lane
//    group, lanes 4e..4e+3 point at the 4 consecutive N-values of K-row e they cover, and lane
//    i receives the 4 K-values of column i; the 4 rows x 32 bytes of a group then fall on 8
//    distinct 16-byte bank groups.
#pragma once

#include <utility>

#include "muon_internal.h"

namespace muon {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

#define MUON_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 in one dword (lo = first), round to nearest even, NaN stays
// NaN: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Block id -> logical tile. Block ids are dealt to the 8 XCDs round robin (id % 8); the
// remap gives each XCD a contiguous logical range, so consecutive tiles of one matrix share
// an XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = w & 7, s = w >> 3;
  return (x < r) ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// One grid over the tiles of several shape groups. The groups are given longest tiles first;
// each XCD receives an even share of every group (q tiles, plus one of the group's r left
// over, dealt round robin over the XCDs continuing from the previous group's), contiguous
// within the group so that one XCD's L2 serves the matrices it works on, and an XCD takes
// its share of the first (longest) group first. Block ids reach the XCDs round robin
// (id % 8), in increasing order on each XCD.
constexpr int kMaxLaunchGroups = 8;
struct TileSplit {
  int n;                        // groups in the launch
  int q[kMaxLaunchGroups];      // tiles / 8
  int r[kMaxLaunchGroups];      // tiles % 8
  int off[kMaxLaunchGroups];    // first XCD of the group's left-over tiles
};

// Group of block `b` (returned) and the tile index within that group.
__device__ __forceinline__ int split_block(int b, const TileSplit& ts, int& tile) {
  const int x = b & 7;
  int s = b >> 3;
  for (int g = 0; g < ts.n; ++g) {
    const int q = ts.q[g], r = ts.r[g], off = ts.off[g];
    const int cnt = q + (((x - off) & 7) < r ? 1 : 0);
    if (s < cnt) {
      int before = 0;
      for (int y = 0; y < x; ++y) before += ((y - off) & 7) < r ? 1 : 0;
      tile = x * q + before + s;
      return g;
    }
    s -= cnt;
  }
  tile = 0;
  return 0;  // not reached: the grid is the groups' total tile count
}

// vmcnt <= N for this wave's outstanding vector-memory loads (lgkm and exp unconstrained).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ int kswz(int row) { return (row >> 2) & 3; }

// One K-contiguous fragment: 8 K-values (chunk c) of LDS row `row`.
__device__ __forceinline__ bf16x8 frag_k(const u32x4* stage, int row, int c) {
  return __builtin_bit_cast(bf16x8, stage[row * 4 + (c ^ kswz(row))]);
}

// ds_read_b64_tr_b16 and ds_read_b128 issued as inline assembly, from a byte address in LDS
// plus a compile-time offset (the instruction's 16-bit offset field, so that a run of reads
// shares one address register). Through the builtins the compiler waits for every
// outstanding direct-to-LDS load (vmcnt 0) before the read, which would drain the load
// pipeline; these results are valid only after an explicit lgkmcnt wait that names them.
template <int OFF>
__device__ __forceinline__ s16x4 ds_read_tr_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// 8-byte LDS write issued as inline assembly: while direct-to-LDS loads are outstanding,
// the compiler would otherwise wait for all of them (vmcnt 0) before any LDS access it
// cannot prove disjoint from their destinations.
__device__ __forceinline__ void ds_write_b64_at(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// A float at a wave-uniform global address, through the scalar cache (a scalar load: it
// does not count against vmcnt, so reading it never waits for outstanding vector loads).
__device__ __forceinline__ float scalar_load_f32(const float* p) {
  float v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Calls f(std::integral_constant<int, i>) for i = 0..N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace mfma
}  // namespace muon
