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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// fp32 staging tile of the epilogue: 128 rows of 32 chunks of 4 floats, chunk XOR row swizzle.
__device__ __forceinline__ int stage_idx(int row, int col) {
  return row * 128 + ((((col >> 2) ^ swz(row)) << 2) | (col & 3));
}

// Epilogue arithmetic on 8 consecutive outputs, one 16-byte store (and one 16-byte load of
// the epilogue operand): GRAM v = s*acc, POLY v = alpha*A + beta*acc, APPLY v = s*(alpha*X + acc).
template <int MODE>
__device__ __forceinline__ void store_chunk(uint16_t* dst, const uint16_t* epi, const float a[8],
                                            float s, float alpha, float beta) {
  u32x4 e4 = {0u, 0u, 0u, 0u};
  if (MODE != 0) e4 = *reinterpret_cast<const u32x4*>(epi);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v0, v1;
    if (MODE == 0) {
      v0 = a[2 * q] * s;
      v1 = a[2 * q + 1] * s;
    } else if (MODE == 1) {
      v0 = fmaf(alpha, bf2f(e4[q] & 0xffffu), beta * a[2 * q]);
      v1 = fmaf(alpha, bf2f(e4[q] >> 16), beta * a[2 * q + 1]);
    } else {
      v0 = fmaf(alpha, bf2f(e4[q] & 0xffffu), a[2 * q]) * s;
      v1 = fmaf(alpha, bf2f(e4[q] >> 16), a[2 * q + 1]) * s;
    }
    o[q] = f2bf(v0) | (f2bf(v1) << 16);
  }
  *reinterpret_cast<u32x4*>(dst) = o;
}

// Block id -> logical tile so that each XCD (id % 8) receives a contiguous logical range.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = w & 7, s = w >> 3;
  return (x < r) ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// Stage a 128 x 64 K-contiguous tile: thread t moves chunk (t & 7) of rows (t >> 3) + 32 i.
__device__ __forceinline__ void load_kmajor(const uint16_t* src, int ld, u32x4 reg[4]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 3) + 32 * i;
    reg[i] = *reinterpret_cast<const u32x4*>(src + (size_t)r * ld + 8 * c);
  }
}

__device__ __forceinline__ void store_kmajor(u32x4* lds, const u32x4 reg[4]) {
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
__device__ __forceinline__ void load_nmajor(const uint16_t* src, int ld, u32x4 reg[4]) {
  const int t = threadIdx.x;
  const int p = t >> 4, q = t & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    reg[i] = *reinterpret_cast<const u32x4*>(src + (size_t)(4 * p + i) * ld + 8 * q);
}

__device__ __forceinline__ uint32_t half_of(const u32x4& v, int d, int h) {
  const uint32_t w = v[d];
  return h ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ void store_nmajor(u32x4* lds, const u32x4 reg[4]) {
  const int t = threadIdx.x;
  const int p = t >> 4, q = t & 15;
  u32x2* l2 = reinterpret_cast<u32x2*>(lds);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = 8 * q + 2 * d + h;  // LDS row
      u32x2 v;
      v.x = half_of(reg[0], d, h) | (half_of(reg[1], d, h) << 16);
      v.y = half_of(reg[2], d, h) | (half_of(reg[3], d, h) << 16);
      const int chunk = (p >> 1) ^ swz(n);
      l2[n * (2 * kChunks) + 2 * chunk + (p & 1)] = v;
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void ns_gemm_bf16(GemmArgs g) {
  // operand tiles: A stages at [0, 2048), B stages at [2048, 4096) (16-byte units)
  __shared__ u32x4 smem[4 * BM * kChunks];
  constexpr int kStage = BM * kChunks;

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

  u32x4 ra[4], rb[4];
  const int KT = g.K / BK;

  load_kmajor(lhs, g.ld_lhs, ra);
  if (MODE == APPLY) load_nmajor(rhs, g.ld_rhs, rb);
  else load_kmajor(rhs, g.ld_rhs, rb);
  store_kmajor(smem, ra);
  if (MODE == APPLY) store_nmajor(smem + 2 * kStage, rb);
  else store_kmajor(smem + 2 * kStage, rb);
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
    const u32x4* A = smem + cur * kStage;
    const u32x4* B = smem + (2 + cur) * kStage;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wr * 64 + i * 32 + (lane & 31);
        const u32x4 v = A[row * kChunks + (c ^ swz(row))];
        af[i] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wc * 64 + j * 32 + (lane & 31);
        const u32x4 v = B[row * kChunks + (c ^ swz(row))];
        bfr[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_kmajor(smem + (cur ^ 1) * kStage, ra);
      if (MODE == APPLY) store_nmajor(smem + (2 + (cur ^ 1)) * kStage, rb);
      else store_kmajor(smem + (2 + (cur ^ 1)) * kStage, rb);
    }
    __syncthreads();
  }

  // Epilogue, staged through LDS so that every global access is a 16-byte row segment.
  // The fp32 tile (128 x 128, 64 KB) reuses the operand buffers; its 16-byte chunks are
  // XOR-swizzled by the row like the operand tiles. Accumulator element r of lane l in a
  // 32x32 block sits at row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wc * 64 + j * 32 + (lane & 31);
        st[stage_idx(row, col)] = acc[i][j][r];
      }
  __syncthreads();

  float s = 1.f;
  if (g.scales) s = g.scales[4 * bidx + g.scale_idx];
  uint16_t* out = g.out + bidx * g.out_bs;
  const uint16_t* epi = (MODE == GRAM) ? nullptr : g.epi + bidx * g.out_bs;
  const int ld = g.ld_out;
  const bool diag = (MODE != APPLY) && (I == J);

  // Row pass: output tile (I, J). Thread t takes 8-column chunks (t % 16) of rows t / 16 + 16k.
  // On a diagonal tile the lower triangle takes the upper triangle's values, so the stored
  // matrix is exactly symmetric.
#pragma unroll 2
  for (int k = 0; k < 8; ++k) {
    const int row = (t >> 4) + 16 * k, ch = t & 15;
    float a[8];
    if (diag) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = 8 * ch + e;
        a[e] = col >= row ? st[stage_idx(row, col)] : st[stage_idx(col, row)];
      }
    } else {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(st + stage_idx(row, 8 * ch));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(st + stage_idx(row, 8 * ch + 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) { a[e] = lo[e]; a[4 + e] = hi[e]; }
    }
    const size_t off = (size_t)(I * BM + row) * ld + J * BN + 8 * ch;
    store_chunk<MODE>(out + off, MODE == GRAM ? nullptr : epi + off, a, s, g.alpha, g.beta);
  }

  // Mirror pass: for an off-diagonal symmetric tile, tile (J, I) is the transpose.
  if (MODE != APPLY && I != J) {
#pragma unroll 2
    for (int k = 0; k < 8; ++k) {
      const int col = (t >> 4) + 16 * k, ch = t & 15;   // output row = col, columns = rows
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = st[stage_idx(8 * ch + e, col)];
      const size_t off = (size_t)(J * BN + col) * ld + I * BM + 8 * ch;
      store_chunk<MODE>(out + off, MODE == GRAM ? nullptr : epi + off, a, s, g.alpha, g.beta);
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
