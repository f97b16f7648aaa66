// Batched Newton-Schulz products on CDNA4 bf16 matrix cores (gfx950).
//
// One round of the quintic iteration of page
// "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (section
// "Newton-Schulz正交化") is three products per matrix, each a launch over a whole shape
// group (batch x mp x np, padded to multiples of 128, padding kept at exact zeros):
//
//   gram   A  = s2 * X X^T          K = np   symmetric: upper 128x128 tiles, mirrored store
//   poly   B  = b A + c A A         K = mp   symmetric (A A = A A^T since A = A^T)
//   apply  X' = s1 * (a X + B X)    K = mp   full tiles
//
// s2 = 1/nu^2 and s1 = 1/nu fold the Frobenius normalisation into the first round; later
// rounds use 1. X, A and B are bf16 in HBM; products accumulate in fp32 on
// v_mfma_f32_32x32x16_bf16; epilogues run in fp32 and round to nearest even.
//
// Tiling: 256 threads (4 waves as 2x2), a 128x128 output tile per block, each wave 64x64
// (2x2 blocks of 32x32). K advances 64 at a time through double-buffered LDS (2 x 32 KB).
// Both operands sit in LDS as rows of 64 K-values (8 chunks of 16 bytes) with the chunk
// index XOR-swizzled by the row, so the 16-byte fragment reads of 8 consecutive rows and
// the 16-byte staging writes of one row both hit distinct banks.
//
// Operand layouts: gram and poly read both operands K-contiguous (rows of X, rows of A).
// apply's right operand X is read along its rows (K = row index of X), so each thread
// loads a 4(k) x 8(n) block with four 16-byte loads and transposes it in registers into
// eight 8-byte LDS writes of K-contiguous data.
//
// Block order: block ids are dealt to the 8 XCDs round robin, so the id is remapped such
// that consecutive tiles of one matrix land on the same XCD and share its L2.
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kChunks = BK / 8;  // 16-byte chunks per LDS row

enum Mode { GRAM = 0, POLY = 1, APPLY = 2 };

struct GemmArgs {
  const uint16_t* lhs;  // [batch][M][K]
  const uint16_t* rhs;  // GRAM/POLY: [batch][N][K]; APPLY: [batch][K][N]
  const uint16_t* epi;  // POLY: A, APPLY: X; laid out like out
  uint16_t* out;        // [batch][M][N]
  long long lhs_bs, rhs_bs, out_bs;
  int ld_lhs, ld_rhs, ld_out;
  int K;
  int tiles_m, tiles_n;
  int tiles_per_mat;
  int total_tiles;
  const float* scales;  // per matrix {s1, s2, nu, 0}, or null
  int scale_idx;        // 0: s1, 1: s2
  float alpha, beta;
};

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Block id -> logical tile so that each XCD (id % 8) receives a contiguous logical range.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = w & 7, s = w >> 3;
  return (x < r) ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// Stage a 128 x 64 K-contiguous tile: thread t moves chunk (t & 7) of rows (t >> 3) + 32 i.
__device__ __forceinline__ void load_kmajor(const uint16_t* src, int ld, uint4 reg[4]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 3) + 32 * i;
    reg[i] = *reinterpret_cast<const uint4*>(src + (size_t)r * ld + 8 * c);
  }
}

__device__ __forceinline__ void store_kmajor(uint4* lds, const uint4 reg[4]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 3) + 32 * i;
    lds[r * kChunks + (c ^ swz(r))] = reg[i];
  }
}

// Stage a 64(k) x 128(n) N-contiguous tile as 128 rows of 64 K-values: thread t loads rows
// 4p..4p+3 (p = t >> 4) at columns 8q..8q+7 (q = t & 15).
__device__ __forceinline__ void load_nmajor(const uint16_t* src, int ld, uint4 reg[4]) {
  const int t = threadIdx.x;
  const int p = t >> 4, q = t & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    reg[i] = *reinterpret_cast<const uint4*>(src + (size_t)(4 * p + i) * ld + 8 * q);
}

__device__ __forceinline__ uint32_t half_of(const uint4& v, int d, int h) {
  const uint32_t w = d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
  return h ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ void store_nmajor(uint4* lds, const uint4 reg[4]) {
  const int t = threadIdx.x;
  const int p = t >> 4, q = t & 15;
  uint2* l2 = reinterpret_cast<uint2*>(lds);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = 8 * q + 2 * d + h;  // LDS row
      uint2 v;
      v.x = half_of(reg[0], d, h) | (half_of(reg[1], d, h) << 16);
      v.y = half_of(reg[2], d, h) | (half_of(reg[3], d, h) << 16);
      const int chunk = (p >> 1) ^ swz(n);
      l2[n * (2 * kChunks) + 2 * chunk + (p & 1)] = v;
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void ns_gemm_bf16(GemmArgs g) {
  __shared__ uint4 sA[2][BM * kChunks];
  __shared__ uint4 sB[2][BN * kChunks];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  const int L = xcd_remap(blockIdx.x, g.total_tiles);
  const int bidx = L / g.tiles_per_mat;
  int tt = L - bidx * g.tiles_per_mat;
  int I, J;
  if (MODE == APPLY) {
    I = tt / g.tiles_n;
    J = tt - I * g.tiles_n;
  } else {
    I = 0;
    while (tt >= g.tiles_m - I) { tt -= g.tiles_m - I; ++I; }
    J = I + tt;
  }

  const uint16_t* lhs = g.lhs + bidx * g.lhs_bs + (size_t)(I * BM) * g.ld_lhs;
  const uint16_t* rhs = g.rhs + bidx * g.rhs_bs +
                        (MODE == APPLY ? (size_t)(J * BN) : (size_t)(J * BN) * g.ld_rhs);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[4], rb[4];
  const int KT = g.K / BK;

  load_kmajor(lhs, g.ld_lhs, ra);
  if (MODE == APPLY) load_nmajor(rhs, g.ld_rhs, rb);
  else load_kmajor(rhs, g.ld_rhs, rb);
  store_kmajor(sA[0], ra);
  if (MODE == APPLY) store_nmajor(sB[0], rb);
  else store_kmajor(sB[0], rb);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      const int k0 = (kt + 1) * BK;
      load_kmajor(lhs + k0, g.ld_lhs, ra);
      if (MODE == APPLY) load_nmajor(rhs + (size_t)k0 * g.ld_rhs, g.ld_rhs, rb);
      else load_kmajor(rhs + k0, g.ld_rhs, rb);
    }
    const uint4* A = sA[cur];
    const uint4* B = sB[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wr * 64 + i * 32 + (lane & 31);
        const uint4 v = A[row * kChunks + (c ^ swz(row))];
        af[i] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wc * 64 + j * 32 + (lane & 31);
        const uint4 v = B[row * kChunks + (c ^ swz(row))];
        bfr[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_kmajor(sA[cur ^ 1], ra);
      if (MODE == APPLY) store_nmajor(sB[cur ^ 1], rb);
      else store_kmajor(sB[cur ^ 1], rb);
    }
    __syncthreads();
  }

  // Epilogue. Accumulator element r of lane l in a 32x32 block sits at
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  float s = 1.f;
  if (g.scales) s = g.scales[4 * bidx + g.scale_idx];
  uint16_t* out = g.out + bidx * g.out_bs;
  const uint16_t* epi = (MODE == GRAM) ? nullptr : g.epi + bidx * g.out_bs;
  const int ld = g.ld_out;
  const bool diag = (MODE != APPLY) && (I == J);
  const bool mirror = (MODE != APPLY) && (I != J);

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gj = J * BN + wc * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int gi0 = I * BM + wr * 64 + i * 32 + 8 * rg + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gi = gi0 + r;
          const float a = acc[i][j][4 * rg + r];
          if (MODE == GRAM) {
            v[r] = a * s;
          } else if (MODE == POLY) {
            v[r] = fmaf(g.alpha, bf2f(epi[(size_t)gi * ld + gj]), g.beta * a);
          } else {
            v[r] = (fmaf(g.alpha, bf2f(epi[(size_t)gi * ld + gj]), a)) * s;
          }
        }
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = f2bf(v[r]);
        if (diag) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int gi = gi0 + r;
            if (gi <= gj) out[(size_t)gi * ld + gj] = (uint16_t)h[r];
            if (gi < gj) out[(size_t)gj * ld + gi] = (uint16_t)h[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) out[(size_t)(gi0 + r) * ld + gj] = (uint16_t)h[r];
          if (mirror) {
            uint2 w;
            w.x = h[0] | (h[1] << 16);
            w.y = h[2] | (h[3] << 16);
            *reinterpret_cast<uint2*>(out + (size_t)gj * ld + gi0) = w;
          }
        }
      }
    }
  }
}

GemmArgs base_args(int batch, int tiles_m, int tiles_n, bool sym) {
  GemmArgs a{};
  a.tiles_m = tiles_m;
  a.tiles_n = tiles_n;
  a.tiles_per_mat = sym ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  a.total_tiles = a.tiles_per_mat * batch;
  return a;
}

}  // namespace

hipError_t launch_gram_bf16(const NsGroup& G, hipStream_t s) {
  GemmArgs a = base_args(G.batch, G.mp / BM, G.mp / BN, true);
  a.lhs = static_cast<const uint16_t*>(G.x_in);
  a.rhs = a.lhs;
  a.out = static_cast<uint16_t*>(G.a);
  a.lhs_bs = a.rhs_bs = (long long)G.mp * G.np;
  a.out_bs = (long long)G.mp * G.mp;
  a.ld_lhs = a.ld_rhs = G.np;
  a.ld_out = G.mp;
  a.K = G.np;
  a.scales = G.first ? G.scales : nullptr;
  a.scale_idx = 1;
  hipLaunchKernelGGL(ns_gemm_bf16<GRAM>, dim3(a.total_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_poly_bf16(const NsGroup& G, float b, float c, hipStream_t s) {
  GemmArgs a = base_args(G.batch, G.mp / BM, G.mp / BN, true);
  a.lhs = static_cast<const uint16_t*>(G.a);
  a.rhs = a.lhs;
  a.epi = a.lhs;
  a.out = static_cast<uint16_t*>(G.b);
  a.lhs_bs = a.rhs_bs = a.out_bs = (long long)G.mp * G.mp;
  a.ld_lhs = a.ld_rhs = a.ld_out = G.mp;
  a.K = G.mp;
  a.alpha = b;
  a.beta = c;
  hipLaunchKernelGGL(ns_gemm_bf16<POLY>, dim3(a.total_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_apply_bf16(const NsGroup& G, float alpha, hipStream_t s) {
  GemmArgs a = base_args(G.batch, G.mp / BM, G.np / BN, false);
  a.lhs = static_cast<const uint16_t*>(G.b);
  a.rhs = static_cast<const uint16_t*>(G.x_in);
  a.epi = a.rhs;
  a.out = static_cast<uint16_t*>(G.x_out);
  a.lhs_bs = (long long)G.mp * G.mp;
  a.rhs_bs = a.out_bs = (long long)G.mp * G.np;
  a.ld_lhs = G.mp;
  a.ld_rhs = a.ld_out = G.np;
  a.K = G.mp;
  a.scales = G.first ? G.scales : nullptr;
  a.scale_idx = 0;
  a.alpha = alpha;
  hipLaunchKernelGGL(ns_gemm_bf16<APPLY>, dim3(a.total_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
