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
// (2x2 blocks of 32x32). K advances 32 at a time through a ring of 4 LDS stages (16 KB
// each, 64 KB per block, two blocks per CU). Operand tiles go from global memory straight
// into LDS (16-byte direct-to-LDS loads, no staging registers), issued three stages ahead;
// each wave waits for its own loads with an explicit vmcnt before the block barrier.
//
// Operand layouts in LDS, both with an XOR swizzle of the 16-byte chunk index so that the
// fragment reads hit distinct banks (the direct loads fill LDS linearly, so the swizzle is
// applied by choosing which global chunk each lane fetches):
//  - K-contiguous tiles (both operands of gram and poly, the left operand of apply):
//    128 rows x 32 K-values (4 chunks per row), chunk c of row r stored at c ^ ((r>>2)&3);
//    a fragment is one 16-byte read of 8 K-values.
//  - apply's right operand X has N contiguous (its K index is X's row index): the tile is
//    kept as 32 K-rows x 128 N-values (16 chunks per row), chunk c of row k stored at
//    c ^ 2(k&3), and fragments come from two ds_read_b64_tr_b16 transposing reads. In each
//    16-lane group, lanes 4e..4e+3 point at the 4 consecutive N-values of K-row e that
//    they cover, and lane i receives the 4 K-values of column i.
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

constexpr int BM = 128, BN = 128, BK = 32, STAGES = 4;
constexpr int kStage = 1024;      // one stage: two 8 KB operand tiles, in 16-byte units
constexpr int kLoadsPerStage = 4; // direct-to-LDS loads per wave per stage

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


// fp32 staging tile of the epilogue: 128 rows of 32 chunks of 4 floats. Chunk q of row r is
// stored at q ^ f(r) ^ (q >> 4) with f(r) = (r ^ (r >> 3)) & 15, so that 16 lanes writing one
// chunk of 16 consecutive rows, reading the even (or odd) chunks of one row, or reading one
// column of rows 8 apart each touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int stage_idx(int row, int col) {
  const int q = col >> 2;
  const int pq = q ^ ((row ^ (row >> 3)) & 15) ^ ((q >> 4) & 1);
  return row * 128 + ((pq << 2) | (col & 3));
}

// Epilogue arithmetic on 8 consecutive outputs (e4: the 8 bf16 of the epilogue operand):
// GRAM v = s*acc, POLY v = alpha*A + beta*acc, APPLY v = s*(alpha*X + acc).
template <int MODE>
__device__ __forceinline__ void finish_chunk(const u32x4& e4, const float a[8], float s,
                                             float alpha, float beta, float v[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float x = bf2f(h ? (e4[q] >> 16) : (e4[q] & 0xffffu));
      const float acc = a[2 * q + h];
      if (MODE == 0) v[2 * q + h] = acc * s;
      else if (MODE == 1) v[2 * q + h] = fmaf(alpha, x, beta * acc);
      else v[2 * q + h] = fmaf(alpha, x, acc) * s;
    }
  }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float v[8]) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = f2bf(v[2 * q]) | (f2bf(v[2 * q + 1]) << 16);
  return o;
}

// Block id -> logical tile so that each XCD (id % 8) receives a contiguous logical range.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = w & 7, s = w >> 3;
  return (x < r) ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// vmcnt <= N for this wave's outstanding vector-memory loads (lgkm and exp unconstrained).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 64-byte rows: XOR the 16-byte chunk with bits 2-3 of the row. A fragment read (16
// consecutive lanes = 16 consecutive rows, one chunk each) then covers all 64 banks; keying
// on bits 1-2 instead leaves a measured 2-way conflict.
__device__ __forceinline__ int kswz(int row) { return (row >> 2) & 3; }

// K-contiguous 128 x 32 tile (rows of `src`, K from k0) into `stage` (1024 16-byte units
// at row*4 + chunk). Wave w issues 16-row blocks 2w and 2w+1; lane l of a block lands at
// unit 64*block + l, i.e. row 16*block + l/4, stored chunk l%4.
__device__ __forceinline__ void dma_kmajor(const uint16_t* src, int ld, int k0, u32x4* stage) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = 2 * w + i;
    const int row = 16 * blk + (lane >> 2);
    const int c = (lane & 3) ^ kswz(row);
    __builtin_amdgcn_global_load_lds(src + (size_t)row * ld + k0 + 8 * c, LDS_PTR(stage + 64 * blk),
                                     16, 0, 0);
  }
}

// N-contiguous 32(k) x 128(n) tile (rows k0.. of `src`, columns from `src`) into `stage`
// (units at k*16 + chunk). Wave w issues 4-row blocks 2w and 2w+1.
__device__ __forceinline__ void dma_nmajor(const uint16_t* src, int ld, int k0, u32x4* stage) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = 2 * w + i;
    const int k = 4 * blk + (lane >> 4);
    const int c = (lane & 15) ^ (2 * (k & 3));
    __builtin_amdgcn_global_load_lds(src + (size_t)(k0 + k) * ld + 8 * c,
                                     LDS_PTR(stage + 64 * blk), 16, 0, 0);
  }
}

// One K-contiguous fragment: 8 K-values (chunk c) of LDS row `row`.
__device__ __forceinline__ bf16x8 frag_k(const u32x4* stage, int row, int c) {
  return __builtin_bit_cast(bf16x8, stage[row * 4 + (c ^ kswz(row))]);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16 issued as inline assembly: through the builtin, the compiler waits for
// every outstanding direct-to-LDS load (vmcnt 0) before the read, which would empty the
// load pipeline each step. The result is only valid after lds_wait() below.
__device__ __forceinline__ s16x4 ds_read_tr(const uint16_t* p) {
  const unsigned addr = static_cast<unsigned>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// Waits for this wave's LDS reads; ties the fragments to the wait so no use moves above it.
__device__ __forceinline__ void lds_wait(bf16x8& x, bf16x8& y) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x), "+v"(y));
}

// One transposed fragment of the N-contiguous tile: lane l gets K-values kb + 8(l/32) + 0..7
// of column nb + l%32 (valid after lds_wait).
__device__ __forceinline__ bf16x8 frag_n(const u32x4* stage, int kb, int nb, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int n = nb + 16 * (g & 1) + 4 * (j & 3);
  const uint16_t* base = reinterpret_cast<const uint16_t*>(stage);
  s16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = kb + 8 * (g >> 1) + 4 * half + (j >> 2);
    const int c = (n >> 3) ^ (2 * (k & 3));
    h[half] = ds_read_tr(base + k * 128 + 8 * c + (n & 7));
  }
  const s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int MODE>
__global__ __launch_bounds__(256) void ns_gemm_bf16(GemmArgs g) {
  // STAGES ring buffers; stage s holds the left tile at units [1024 s, 1024 s + 512) and
  // the right tile at [1024 s + 512, 1024 (s + 1)).
  __shared__ u32x4 smem[STAGES * kStage];

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

  // The epilogue operand passes through LDS during the main loop and is captured there,
  // in the epilogue's layout (thread t: 8-column chunk t%16 of rows t/16 + 16k):
  //  - apply needs X[I-tile rows][J-tile cols]; the right-operand stages 4I..4I+3 hold
  //    exactly those rows (X's row is the contraction index), 32 rows each;
  //  - poly needs A[I-tile rows][J-tile cols]; the left-operand stages 4J..4J+3 hold A's
  //    I-tile rows at column block 4J + s, so chunk t%16 arrives at stage 4J + (t%16)/4.
  u32x4 epre[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) epre[k] = u32x4{0u, 0u, 0u, 0u};

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

  const int KT = g.K / BK;
  auto issue = [&](int kt) {
    u32x4* st = smem + (kt % STAGES) * kStage;
    dma_kmajor(lhs, g.ld_lhs, kt * BK, st);
    if (MODE == APPLY) dma_nmajor(rhs, g.ld_rhs, kt * BK, st + 512);
    else dma_kmajor(rhs, g.ld_rhs, kt * BK, st + 512);
  };
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s);

  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads of stage kt are done once at most the later stages' are pending
    if (kt + 2 < KT) vm_wait<2 * kLoadsPerStage>();
    else if (kt + 1 < KT) vm_wait<kLoadsPerStage>();
    else vm_wait<0>();
    // every wave's loads of stage kt are visible, and every wave is done with stage kt - 1
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves across the barrier
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);

    const u32x4* A = smem + (kt % STAGES) * kStage;
    const u32x4* B = A + 512;
    if (MODE == APPLY && (kt >> 2) == I) {
      const int sub = kt & 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = (t >> 4) + 16 * h;   // row within the stage: tile row 32 sub + kr
        epre[2 * sub + h] = B[kr * 16 + ((t & 15) ^ (2 * (kr & 3)))];
      }
    }
    if (MODE == POLY && (kt >> 2) == J && (kt & 3) == ((t & 15) >> 2)) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = (t >> 4) + 16 * k;
        epre[k] = A[row * 4 + ((t & 3) ^ kswz(row))];
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag_k(A, wr * 64 + i * 32 + (lane & 31), c);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (MODE == APPLY) bfr[j] = frag_n(B, 16 * ks, wc * 64 + j * 32, lane);
        else bfr[j] = frag_k(B, wc * 64 + j * 32 + (lane & 31), c);
      }
      if (MODE == APPLY) lds_wait(bfr[0], bfr[1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }
  // all waves are done reading the operand stages before the epilogue reuses them
  __syncthreads();

  // Epilogue, staged through LDS so that every global access is a 16-byte row segment.
  // The fp32 tile (128 x 128, 64 KB) reuses the operand stages. With the operands passed to
  // the MFMA as (right, left), block (i, j) holds the transposed product: element r of lane l
  // is C[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4], four consecutive columns per register
  // quad, so each quad is one 16-byte LDS write.
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wr * 64 + i * 32 + (lane & 31);
        const int col = wc * 64 + j * 32 + 8 * q + 4 * (lane >> 5);
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
        *reinterpret_cast<f32x4*>(st + stage_idx(row, col)) = v;
      }
  __syncthreads();

  float s = 1.f;
  if (g.scales) s = g.scales[4 * bidx + g.scale_idx];
  uint16_t* out = g.out + bidx * g.out_bs;
  const int ld = g.ld_out;
  const bool diag = (MODE != APPLY) && (I == J);
  const bool mirror = (MODE != APPLY) && (I != J);

  // Row pass: output tile (I, J), chunk t%16 of rows t/16 + 16k. On a diagonal tile the lower
  // triangle takes the upper triangle's accumulators (the epilogue operand is symmetric too),
  // so the stored matrix is exactly symmetric. Tiles that also store a mirror write their
  // final values back over their own staging slots.
#pragma unroll
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
    float v[8];
    const u32x4 e4 = (MODE == GRAM) ? u32x4{0u, 0u, 0u, 0u} : epre[k];
    finish_chunk<MODE>(e4, a, s, g.alpha, g.beta, v);
    *reinterpret_cast<u32x4*>(out + (size_t)(I * BM + row) * ld + J * BN + 8 * ch) =
        pack_bf16x8(v);
    if (mirror) {
      *reinterpret_cast<f32x4*>(st + stage_idx(row, 8 * ch)) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(st + stage_idx(row, 8 * ch + 4)) = f32x4{v[4], v[5], v[6], v[7]};
    }
  }

  // Mirror pass: tile (J, I) is the transpose of the finished tile (I, J).
  if (mirror) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int col = (t >> 4) + 16 * k, ch = t & 15;   // output row = col, columns = rows
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = st[stage_idx(8 * ch + e, col)];
      *reinterpret_cast<u32x4*>(out + (size_t)(J * BN + col) * ld + I * BM + 8 * ch) =
          pack_bf16x8(v);
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
