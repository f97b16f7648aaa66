// The apply product of a Newton-Schulz round on bf16 matrix cores (gfx950):
//
//   X' = s1 * (B' X),   B' = a I + b A + c A A
//
// Page "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (section
// "Newton-Schulz正交化") writes the round's last line as X = a X + B X; with the a I term
// folded into B' by the poly kernel (exact in real arithmetic), apply is a plain product
// with a scaling epilogue and no second operand to read. s1 = 1/nu on the first round (the
// Frobenius normalisation folded in), else 1.
//
// Tiling: 256 threads (4 waves as 2x2), a 256x256 output tile per block, each wave 128x128
// as 4x4 blocks of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane, in AGPRs).
// Per flop this moves half the global and LDS bytes of a 128x128 tile. K advances 32 at a
// time through a ring of 4 LDS stages of 32 KB (one block per CU, one wave per SIMD), so
// the loop is an explicit software pipeline (below). The left operand B' is
// K-contiguous; the right operand X is N-contiguous and read with transposing LDS loads
// (layouts in mfma_common.h). Output rows/columns beyond the padded shape (when mp or np is
// an odd multiple of 128) are computed from clamped loads and not stored.
//
// With the MFMA operands passed as (right, left), accumulator block (i, j) holds the
// transposed product: element r of lane l is C[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4],
// so each register quad is 4 consecutive columns of one row: one 8-byte store.
#include "mfma_common.h"

namespace muon {
namespace {

using namespace mfma;

constexpr int TM = 256, TN = 256, TK = 32, NSTAGE = 4;
constexpr int kUnitsA = TM * TK / 8;           // 1024 16-byte units
constexpr int kUnitsStage = kUnitsA + TK * TN / 8;
constexpr int kLoadsPerStage = (TM / 16) / 4 + (32 / 2) / 4;  // per wave: 4 + 4

struct ApplyArgs {
  const uint16_t* b;   // B', batch x mp x mp
  const uint16_t* x;   // X, batch x mp x np
  uint16_t* out;       // X', batch x mp x np
  const float* scales; // per matrix {s1, s2, nu, 0}, or null (scale 1)
  int mp, np;
  int tiles_m, tiles_n, total_tiles;
};

__global__ __launch_bounds__(256) void ns_apply_bf16(ApplyArgs g) {
  __shared__ u32x4 smem[NSTAGE * kUnitsStage];  // 128 KB

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  const int L = xcd_remap(blockIdx.x, g.total_tiles);
  const int per_mat = g.tiles_m * g.tiles_n;
  const int bidx = L / per_mat;
  const int tt = L - bidx * per_mat;
  const int I = tt / g.tiles_n, J = tt - (tt / g.tiles_n) * g.tiles_n;

  const size_t mm = (size_t)g.mp * g.mp, mn = (size_t)g.mp * g.np;
  const uint16_t* lhs = g.b + bidx * mm;
  const uint16_t* rhs = g.x + bidx * mn;
  const int row0 = I * TM, col0 = J * TN;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = g.mp / TK;
  auto issue = [&](int kt) {
    u32x4* st = smem + (kt % NSTAGE) * kUnitsStage;
    dma_kmajor<TM, 4>(lhs, g.mp, row0, g.mp, kt * TK, st);
    dma_nmajor<TN, 4>(rhs, g.np, kt * TK, col0, g.np, st + kUnitsA);
  };
  // Fragments of one 16-wide K slice (ks = 0, 1) of a stage.
  auto load = [&](int kt, int ks, bf16x8 (&af)[4], bf16x8 (&bf)[4]) {
    const u32x4* A = smem + (kt % NSTAGE) * kUnitsStage;
    const u32x4* B = A + kUnitsA;
    const int c = 2 * ks + (lane >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = frag_n<TN>(B, 16 * ks, wc * 128 + j * 32, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = frag_k(A, wr * 128 + i * 32 + (lane & 31), c);
  };
  auto wait_frags = [&](bf16x8 (&af)[4], bf16x8 (&bf)[4]) {
    lds_wait(bf[0], bf[1]);
    lds_wait(bf[2], bf[3]);
    lds_wait(af[0], af[1]);
    lds_wait(af[2], af[3]);
  };
  auto mma = [&](const bf16x8 (&af)[4], const bf16x8 (&bf)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
  };
  // Waits for this wave's loads of stage `next`, given how many later stages were issued,
  // then the block barrier: stage `next` is complete for every wave.
  auto stage_ready = [&](int later) {
    if (later >= 3) vm_wait<3 * kLoadsPerStage>();
    else if (later == 2) vm_wait<2 * kLoadsPerStage>();
    else if (later == 1) vm_wait<kLoadsPerStage>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves across the barrier
  };

  // Software pipeline: each stage's two K slices are read into registers one slice ahead of
  // the 16 MFMAs that use them, and the barrier for the next stage is taken right after a
  // batch of MFMAs is issued, so LDS reads, direct loads and the barrier all run in the
  // shadow of the matrix cores. Stages are prefetched four ahead (all four buffers in use).
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s)
    if (s < KT) issue(s);
  stage_ready(min(NSTAGE - 1, KT - 1));
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  load(0, 0, a0, b0);
  wait_frags(a0, b0);

  for (int kt = 0; kt < KT; ++kt) {
    load(kt, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    wait_frags(a1, b1);  // slice 1 is in registers: this wave is done reading stage kt
    if (kt + 1 < KT) {
      stage_ready(min(NSTAGE - 2, KT - 2 - kt));
      if (kt + NSTAGE < KT) issue(kt + NSTAGE);  // into stage kt's buffer, now free
      load(kt + 1, 0, a0, b0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < KT) wait_frags(a0, b0);
  }

  // Epilogue: scale, round to bf16 and stage the 256x256 tile in LDS (128 KB, the whole
  // operand ring), then store 16-byte chunks with 32 lanes per 512-byte row segment; stores
  // straight from the accumulator layout touch 32 rows per instruction and were measured to
  // take longer than the whole main loop. Chunk q (8 columns) of row r sits at
  // q ^ (r & 15): 16 lanes reading 16 chunks of one row, or writing one chunk of 16
  // consecutive rows, hit distinct 16-byte bank groups.
  const float s = g.scales ? g.scales[4 * bidx] : 1.f;
  __syncthreads();  // every wave is done with the operand stages
  u32x2* st2 = reinterpret_cast<u32x2*>(smem);  // 8-byte units: row * 64 + 2 * chunk + half
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wr * 128 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wc * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
        u32x2 w;
        w.x = pack_bf16(acc[i][j][4 * q] * s, acc[i][j][4 * q + 1] * s);
        w.y = pack_bf16(acc[i][j][4 * q + 2] * s, acc[i][j][4 * q + 3] * s);
        st2[row * 64 + 2 * ((col >> 3) ^ (row & 15)) + ((col >> 2) & 1)] = w;
      }
    }
  }
  __syncthreads();
  uint16_t* out = g.out + bidx * mn;
  const int ch = t & 31;
#pragma unroll 8
  for (int k = 0; k < 32; ++k) {
    const int row = (t >> 5) + 8 * k;
    const int grow = row0 + row, gcol = col0 + 8 * ch;
    if (grow < g.mp && gcol < g.np)
      *reinterpret_cast<u32x4*>(out + (size_t)grow * g.np + gcol) =
          smem[row * 32 + (ch ^ (row & 15))];
  }
}

}  // namespace

hipError_t launch_apply_bf16(const NsGroup& G, hipStream_t s) {
  ApplyArgs a{};
  a.b = static_cast<const uint16_t*>(G.b);
  a.x = static_cast<const uint16_t*>(G.x_in);
  a.out = static_cast<uint16_t*>(G.x_out);
  a.scales = G.first ? G.scales : nullptr;
  a.mp = G.mp;
  a.np = G.np;
  a.tiles_m = (G.mp + TM - 1) / TM;
  a.tiles_n = (G.np + TN - 1) / TN;
  a.total_tiles = a.tiles_m * a.tiles_n * G.batch;
  hipLaunchKernelGGL(ns_apply_bf16, dim3(a.total_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
