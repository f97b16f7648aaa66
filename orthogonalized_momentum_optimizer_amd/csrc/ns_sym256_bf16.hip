// The two symmetric products of a Newton-Schulz round, 256x256 output tiles (gfx950).
//
// Same products as ns_gemm_bf16.hip (page "深入解析KellerJordan/modded-nanogpt中的训练架构与
// 优化技术", section "Newton-Schulz正交化": A = X X^T, B = b A + c A A), for shape groups
// with mp >= 1024 (use_sym256 below):
//
//   gram   A  = s2 * X X^T              K = np
//   poly   B' = a I + b A + c A A       K = mp   (A A = A A^T since A is symmetric)
//
// A 128x128 tile moves 16 KB from L2 per 32-deep K step for 1 MFLOP; at two blocks per CU
// that rate of L2 traffic, not the matrix cores, bounds the smaller kernel. A 256x256 tile
// halves the bytes per flop and runs the software pipeline of the apply kernel: 4 waves as
// 2x2, each 128x128 as 4x4 v_mfma_f32_32x32x16_bf16 blocks (256 fp32 accumulators per lane,
// in AGPRs), a ring of 4 LDS stages of 32 KB (one block per CU), MFMAs interleaved by hand
// with the LDS reads of the next K slice and the direct-to-LDS refills. Both operands are
// K-contiguous (rows of X, or rows of A), so every fragment is one 16-byte LDS read.
//
// Only upper tiles (I <= J) are computed. The epilogue rounds the tile to bf16 once, stages
// it in LDS and writes it twice: rows of tile (I, J), and its transpose as tile (J, I), read
// with transposing LDS loads (ds_read_b64_tr_b16). A diagonal tile writes its upper triangle
// from its rows and its lower triangle from the transpose, so A and B' are exactly
// symmetric. POLY's b A term is the tile A[I-tile][J-tile], loaded into the ring by the last
// iterations of the K loop and combined in fp32 before the rounding.
#include <algorithm>
#include <vector>

#include "mfma_common.h"

namespace muon {
namespace {

using namespace mfma;

constexpr int TS = 256, TK = 32, NSTAGE = 4;
constexpr int kUnitsHalf = TS * TK / 8;        // one operand per stage: 1024 16-byte units
constexpr int kUnitsStage = 2 * kUnitsHalf;    // 32 KB
constexpr int kLoadsPerStage = 8;              // direct loads per wave per stage (4 + 4)

enum Mode { GRAM = 0, POLY = 1 };

struct Sym256Args {     // one shape group
  const uint16_t* in;   // GRAM: X (batch x mp x np); POLY: A (batch x mp x mp)
  uint16_t* out;        // batch x mp x mp
  const float* scales;  // GRAM first round: per matrix {s1, s2, nu, 0}; else null
  long long in_bs;
  int ld_in, K, mp;
  int tiles;            // tiles per side: ceil(mp / 256)
  int tiles_per_mat;
};

struct Sym256Launch {   // the shape groups of one launch, longest tiles (largest K) first
  TileSplit split;
  Sym256Args g[kMaxLaunchGroups];
  float a, b, c;        // POLY coefficients
};

// Fragments of one 16-wide K slice: 4 of the left operand (rows of the I tile) and 4 of the
// right (rows of the J tile).
struct Frags {
  u32x4 av[4];
  u32x4 bv[4];
};

// LDS read `OP` of a K slice: ops 0-3 right-operand fragment OP, ops 4-7 left-operand
// fragment OP - 4. `va`/`vb` are the lane's addresses of fragment 0 of the slice; fragment
// i is 32 rows (2048 bytes) further, and the row swizzle (bits 2-3 of the row) is the same.
template <int OP>
__device__ __forceinline__ void lds_op(uint32_t va, uint32_t vb, Frags& f) {
  if constexpr (OP < 4)
    f.bv[OP] = ds_read_b128_at<2048 * OP>(vb);
  else
    f.av[OP - 4] = ds_read_b128_at<2048 * (OP - 4)>(va);
}

// Byte offset of element (row, col) in the bf16 staging tile: 256 rows of 512 bytes, 16-byte
// chunk q of row r stored at q ^ (r & 15).
__device__ __forceinline__ uint32_t stage_byte(int row, int col) {
  return 512u * row + 16u * ((col >> 3) ^ (row & 15)) + 2u * (col & 7);
}

template <int MODE>
__global__ __launch_bounds__(256) void ns_sym256_bf16(Sym256Launch S) {
  __shared__ u32x4 smem[NSTAGE * kUnitsStage];  // 128 KB

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  int L;
  const Sym256Args g = S.g[split_block(blockIdx.x, S.split, L)];
  const int bidx = L / g.tiles_per_mat;
  int tt = L - bidx * g.tiles_per_mat;
  int I = 0;
  while (tt >= g.tiles - I) { tt -= g.tiles - I; ++I; }
  const int J = I + tt;
  const int row0 = I * TS, col0 = J * TS;
  const bool diag = I == J;

  const char* src = reinterpret_cast<const char*>(g.in + bidx * g.in_bs);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = g.K / TK;  // >= 4: K is a multiple of 128

  // ---- direct-to-LDS loads: 8 per wave per stage ----
  // Loads 0-3 fetch 16 rows each of the I tile, 4-7 of the J tile (4 lanes x 16 bytes per
  // row; lane l lands at 16 l of a 1 KB block, the K-major swizzle chosen through the global
  // chunk). Rows at or beyond mp come from row mp - 1 (never stored). Global address: the
  // stage's K origin (scalar) plus the lane's fixed byte offset.
  uint32_t doff[8];
#pragma unroll
  for (int op = 0; op < 8; ++op) {
    const int row = 16 * (4 * wave + (op & 3)) + (lane >> 2);
    const int c = (lane & 3) ^ kswz(row);
    const uint32_t grow = min((op < 4 ? row0 : col0) + row, g.mp - 1);
    doff[op] = 2u * (uint32_t)toff((int)grow, 8 * c, g.ld_in);
  }
  auto dma_op = [&](int kt, int op) {
    u32x4* st = smem + (kt & (NSTAGE - 1)) * kUnitsStage + (op >> 2) * kUnitsHalf;
    __builtin_amdgcn_global_load_lds(src + (size_t)kt * kTileBytes + doff[op],
                                     MUON_LDS_PTR(st + 64 * (4 * wave + (op & 3))), 16, 0, 0);
  };

  // ---- LDS read addresses (bytes): slice ks of fragment 0 ----
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(MUON_LDS_PTR(smem)));
  const int arow = wr * 128 + (lane & 31), brow = wc * 128 + (lane & 31);
  const uint32_t aoff0 = 64 * arow + 16 * ((lane >> 5) ^ kswz(arow));
  const uint32_t aoff1 = 64 * arow + 16 * ((2 + (lane >> 5)) ^ kswz(arow));
  const uint32_t boff0 = 16 * kUnitsHalf + 64 * brow + 16 * ((lane >> 5) ^ kswz(brow));
  const uint32_t boff1 = 16 * kUnitsHalf + 64 * brow + 16 * ((2 + (lane >> 5)) ^ kswz(brow));
  auto stage_base = [&](int kt) { return lds0 + (uint32_t)((kt & (NSTAGE - 1)) * kUnitsStage * 16); };

  auto ready = [&](Frags& f, bf16x8 (&af)[4], bf16x8 (&bf)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.av[0]), "+v"(f.av[1]), "+v"(f.av[2]), "+v"(f.av[3]),
                   "+v"(f.bv[0]), "+v"(f.bv[1]), "+v"(f.bv[2]), "+v"(f.bv[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = __builtin_bit_cast(bf16x8, f.av[i]);
      bf[i] = __builtin_bit_cast(bf16x8, f.bv[i]);
    }
  };
  auto mfma = [&](int m, const bf16x8 (&af)[4], const bf16x8 (&bf)[4]) {
    const int i = m >> 2, j = m & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
  };
  auto stage_ready = [&](int later) {
    if (later >= 3) vm_wait<3 * kLoadsPerStage>();
    else if (later == 2) vm_wait<2 * kLoadsPerStage>();
    else if (later == 1) vm_wait<kLoadsPerStage>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- software pipeline (the apply kernel's, with 8 reads per slice) ----
  // POLY keeps the refills going past the last operand stage: "stages" KT..KT+3 are the four
  // 64-row quarters of the tile A[I tile][J tile] that its b A term needs, so that tile is in
  // the ring when the loop ends. With KT a multiple of 4, quarter p lands in buffer p: the
  // tile's rows in order, 512 bytes each, 16-byte chunk p of row r holding chunk p ^ (r & 31).
  auto dma_a = [&](int part, int op) {
    const int blk = 8 * wave + op;
    const int r = 64 * part + 2 * blk + (lane >> 5);
    const int gch = (lane & 31) ^ (r & 31);
    const uint32_t grow = min(row0 + r, g.mp - 1), gcol = min(col0 + 8 * gch, g.mp - 8);
    __builtin_amdgcn_global_load_lds(src + 2 * toff((int)grow, (int)gcol, g.mp),
                                     MUON_LDS_PTR(smem + part * kUnitsStage + 64 * blk), 16, 0,
                                     0);
  };
  constexpr bool kAtile = MODE == POLY;
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  Frags f0, f1;
  // REFILL: 0 none, 1 operand stage kt + 4, 2 A-tile quarter kt + 4 - KT
  auto iteration = [&](int kt, auto refill_t, auto more_t) {
    constexpr int refill = decltype(refill_t)::value;
    constexpr bool more = decltype(more_t)::value;
    const uint32_t cur = stage_base(kt);
    const uint32_t va1 = cur + aoff1, vb1 = cur + boff1;
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto M) {
      constexpr int m = decltype(M)::value;
      mfma(m, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m < 8) lds_op<m>(va1, vb1, f1);
      __builtin_amdgcn_sched_barrier(0);
    });
    ready(f1, a1, b1);  // this wave is done reading stage kt
    if constexpr (more) {
      if constexpr (refill != 0) stage_ready(NSTAGE - 2);
      else stage_ready(min(NSTAGE - 2, KT - 2 - kt));
    } else if constexpr (refill != 0) {
      __builtin_amdgcn_s_barrier();  // every wave is done with the last stage's buffer
      asm volatile("" ::: "memory");
    }
    const uint32_t nxt = stage_base(kt + 1);
    const uint32_t va0 = nxt + aoff0, vb0 = nxt + boff0;
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto M) {
      constexpr int m = decltype(M)::value;
      mfma(m, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (refill == 1 && m < 8) dma_op(kt + NSTAGE, m);
      if constexpr (refill == 2 && m < 8) dma_a(kt + NSTAGE - KT, m);
      if constexpr (more && m >= 2 && m < 10) lds_op<m - 2>(va0, vb0, f0);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (more) ready(f0, a0, b0);
  };
  using R1 = std::integral_constant<int, 1>;
  using RT = std::integral_constant<int, kAtile ? 2 : 0>;

#pragma unroll
  for (int st = 0; st < NSTAGE; ++st)
#pragma unroll
    for (int op = 0; op < 8; ++op) dma_op(st, op);
  stage_ready(NSTAGE - 1);
  static_for<8>([&](auto OP) { lds_op<decltype(OP)::value>(lds0 + aoff0, lds0 + boff0, f0); });
  ready(f0, a0, b0);

  int kt = 0;
  for (; kt < KT - NSTAGE; ++kt) iteration(kt, R1{}, std::true_type{});
  for (; kt < KT - 1; ++kt) iteration(kt, RT{}, std::true_type{});
  iteration(KT - 1, RT{}, std::false_type{});

  // ---- epilogue ----
  // With the MFMA operands passed as (right, left), element r of lane l of block (i, j) is
  // C[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4] of the wave's 128x128 quarter.
  uint16_t* out = g.out + bidx * (size_t)g.mp * g.mp;
  const int mp = g.mp;
  u32x2* st2 = reinterpret_cast<u32x2*>(smem);

  if constexpr (MODE == POLY) {
    vm_wait<0>();
    __syncthreads();  // the A tile is in the ring
    // v = b A + c acc (+ a on the diagonal) in fp32, rounded once; held packed until every
    // wave is done reading the A tile
    uint32_t pk[4][4][8];
    const uint16_t* at = reinterpret_cast<const uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = wr * 128 + 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lc = wc * 128 + 32 * j + 8 * q + 4 * (lane >> 5);
          const u32x2 w = *reinterpret_cast<const u32x2*>(
              at + 256 * lr + 8 * ((lc >> 3) ^ (lr & 31)) + (lc & 7));
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t h = (e < 2 ? w.x : w.y) >> (16 * (e & 1));
            v[e] = fmaf(S.b, bf2f(h & 0xffffu), S.c * acc[i][j][4 * q + e]);
            if (diag && lr == lc + e) v[e] += S.a;
          }
          pk[i][j][2 * q] = pack_bf16(v[0], v[1]);
          pk[i][j][2 * q + 1] = pack_bf16(v[2], v[3]);
        }
    }
    __syncthreads();  // the A tile is no longer read
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = wr * 128 + 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lc = wc * 128 + 32 * j + 8 * q + 4 * (lane >> 5);
          st2[lr * 64 + 2 * ((lc >> 3) ^ (lr & 15)) + ((lc >> 2) & 1)] =
              u32x2{pk[i][j][2 * q], pk[i][j][2 * q + 1]};
        }
    }
  } else {
    __syncthreads();  // every wave is done with the operand stages
    const float s = g.scales ? g.scales[4 * bidx + 1] : 1.f;
    auto stage_out = [&](auto scaled_t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = wr * 128 + 32 * i + (lane & 31);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int lc = wc * 128 + 32 * j + 8 * q + 4 * (lane >> 5);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = decltype(scaled_t)::value ? acc[i][j][4 * q + e] * s : acc[i][j][4 * q + e];
            st2[lr * 64 + 2 * ((lc >> 3) ^ (lr & 15)) + ((lc >> 2) & 1)] =
                u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
          }
      }
    };
    if (g.scales) stage_out(std::true_type{});
    else stage_out(std::false_type{});
  }
  __syncthreads();

  // Output chunk (R, c0..c0+7) of a tile: a diagonal tile takes it from staged row R when
  // c0 >= R (upper) and from the transpose otherwise, merging the one chunk that the
  // diagonal crosses.
  // Row pass: tile (I, J), 16-byte chunk t%32 of rows t/32 + 8k, 8 rows in flight.
  {
    const int ch = t & 31;
#pragma unroll
    for (int kb = 0; kb < 32; kb += 8) {
      u32x4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = (t >> 5) + 8 * (kb + u);
        w[u] = smem[r * 32 + (ch ^ (r & 15))];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = (t >> 5) + 8 * (kb + u);
        if (row0 + r < mp && col0 + 8 * ch < mp && (!diag || 8 * ch >= r))
          *reinterpret_cast<u32x4*>(out + toff(row0 + r, col0 + 8 * ch, mp)) = w[u];
      }
    }
  }
  // Transpose pass: tile (J, I) row R = staged column R, 8 columns = staged rows r0..r0+7.
  // In each 16-lane group, lane 4e + q points at 4 staged columns c0 + 4q.. of row r0 + e
  // (then r0 + 4 + e), and the transposing read gives lane i column c0 + i of those rows.
  // One wave instruction covers 16 rows x 32 columns of the output; 4 in flight.
  {
    const int grp = lane >> 4, li = lane & 15;
#pragma unroll
    for (int ib = 0; ib < 32; ib += 4) {
      s16x4 lo[4], hi[4];
      u32x4 rowv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int combo = 32 * wave + ib + u;
        const int c0 = 16 * (combo >> 3), r0 = 32 * (combo & 7) + 8 * grp;
        const int ar = r0 + (li >> 2), acol = c0 + 4 * (li & 3);
        lo[u] = ds_read_tr_at<0>(lds0 + stage_byte(ar, acol));
        hi[u] = ds_read_tr_at<0>(lds0 + stage_byte(ar + 4, acol));
        // row R's own values of the chunk (used where a diagonal tile's chunk crosses the
        // diagonal); read unconditionally: a read issued on one path only would let the
        // compiler copy its not-yet-arrived result at the join
        rowv[u] = ds_read_b128_at<0>(lds0 + stage_byte(c0 + li, r0));
      }
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(lo[0]), "+v"(lo[1]), "+v"(lo[2]), "+v"(lo[3]), "+v"(hi[0]),
                     "+v"(hi[1]), "+v"(hi[2]), "+v"(hi[3]), "+v"(rowv[0]), "+v"(rowv[1]),
                     "+v"(rowv[2]), "+v"(rowv[3]));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int combo = 32 * wave + ib + u;
        const int c0 = 16 * (combo >> 3), r0 = 32 * (combo & 7) + 8 * grp;
        const int R = c0 + li;
        if (col0 + R >= mp || row0 + r0 >= mp || (diag && r0 >= R)) continue;
        const s16x8 tv = {lo[u][0], lo[u][1], lo[u][2], lo[u][3],
                          hi[u][0], hi[u][1], hi[u][2], hi[u][3]};
        u32x4 w = __builtin_bit_cast(u32x4, tv);
        if (diag && R <= r0 + 7) {  // the diagonal crosses this chunk: upper part from row R
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep_lo = r0 + 2 * e < R ? 0x0000ffffu : 0u;
            const uint32_t keep_hi = r0 + 2 * e + 1 < R ? 0xffff0000u : 0u;
            const uint32_t keep = keep_lo | keep_hi;
            w[e] = (w[e] & keep) | (rowv[u][e] & ~keep);
          }
        }
        *reinterpret_cast<u32x4*>(out + toff(col0 + R, row0 + r0, mp)) = w;
      }
    }
  }
}

}  // namespace

// The 256-tile kernel moves half the L2 bytes per flop but gives a group a quarter as many
// tiles: on GPT-2-124M's 768-wide groups (288 and 144 tiles per launch) the 128-tile kernel
// was measured faster, on GPT-2-1.5B's 1664-wide groups the 256-tile kernel (gram 16.1 vs
// 18.6 ms per step).
bool use_sym256(const NsGroup& G) { return G.mp >= 1024; }

namespace {

hipError_t launch_sym256(const NsGroup* groups, int n, int mode, float ca, float cb, float cc,
                         hipStream_t s) {
  // per-tile work is the K loop: np for GRAM, mp for POLY
  auto K = [&](const NsGroup* G) { return mode == GRAM ? G->np : G->mp; };
  std::vector<const NsGroup*> order(n);
  for (int i = 0; i < n; ++i) order[i] = groups + i;
  std::stable_sort(order.begin(), order.end(),
                   [&](const NsGroup* x, const NsGroup* y) { return K(x) > K(y); });
  for (int c0 = 0; c0 < n; c0 += kMaxLaunchGroups) {
    Sym256Launch a{};
    a.a = ca;
    a.b = cb;
    a.c = cc;
    int total = 0, left = 0;
    a.split.n = std::min(kMaxLaunchGroups, n - c0);
    for (int k = 0; k < a.split.n; ++k) {
      const NsGroup& G = *order[c0 + k];
      Sym256Args& g = a.g[k];
      g.in = static_cast<const uint16_t*>(mode == GRAM ? G.x_in : G.a);
      g.out = static_cast<uint16_t*>(mode == GRAM ? G.a : G.b);
      g.scales = (mode == GRAM && G.first) ? G.scales : nullptr;
      g.in_bs = mode == GRAM ? (long long)G.mp * G.np : (long long)G.mp * G.mp;
      g.ld_in = K(&G);
      g.K = K(&G);
      g.mp = G.mp;
      g.tiles = (G.mp + TS - 1) / TS;
      g.tiles_per_mat = g.tiles * (g.tiles + 1) / 2;
      const int tiles = g.tiles_per_mat * G.batch;
      a.split.q[k] = tiles / 8;
      a.split.r[k] = tiles % 8;
      a.split.off[k] = left % 8;
      left += tiles % 8;
      total += tiles;
    }
    if (mode == GRAM)
      launch_k(ns_sym256_bf16<GRAM>, dim3(total), dim3(256), 0, s, a);
    else
      launch_k(ns_sym256_bf16<POLY>, dim3(total), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gram256_bf16(const NsGroup* groups, int n, hipStream_t s) {
  return launch_sym256(groups, n, GRAM, 0.f, 0.f, 0.f, s);
}

hipError_t launch_poly256_bf16(const NsGroup* groups, int n, float ca, float cb, float cc,
                               hipStream_t s) {
  return launch_sym256(groups, n, POLY, ca, cb, cc, s);
}

}  // namespace muon
