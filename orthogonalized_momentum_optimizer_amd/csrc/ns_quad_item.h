// The four-block work item of the symmetric products of a Newton-Schulz round (gfx950),
// shared by the product kernel of ns_quad_bf16.hip and the fused kernel of
// ns_fused_bf16.hip.
//
// Products (page "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术", section
// "Newton-Schulz正交化": A = X X^T, B = b A + c A A):
//
//   gram   A  = s2 * X X^T              K = np
//   poly   B' = a I + b A + c A A       K = mp   (A A = A A^T since A is symmetric)
//
// Only the upper triangle of 128x128 blocks is computed: blocks (r, c), r <= c, of the
// mp / 128 panels (128 rows each) of a matrix. A work item is four such blocks, one per wave,
// each wave holding its block as the apply kernel's register tile (4x4
// v_mfma_f32_32x32x16_bf16 blocks, 256 fp32 accumulators per lane in AGPRs). The item's
// blocks draw on at most four panels ("slots"); a 32-deep K step moves 32 KB for 4 MFLOP,
// half the bytes per flop of a 128x128 tile, through a ring of 4 LDS stages of 32 KB (one
// block per CU), with the apply kernel's software pipeline: MFMAs interleaved by hand with
// the LDS reads of the next K slice and the direct-to-LDS refills.
//
// Items, with the panels taken in pairs (2I, 2I+1), I < mp / 256:
//  - pair items, I < J: the four blocks (2I+u, 2J+v), u, v in {0, 1}; slots 2I, 2I+1, 2J,
//    2J+1 (a 256x256 tile off the diagonal);
//  - triples: blocks (2I, 2I), (2I+1, 2I+1) and (2I, 2I+1), three blocks on two slots. The
//    triples, taken four at a time, make three items: triple j (j < 3) plus one block of the
//    fourth triple (its first diagonal block, its second, or its off-diagonal block for
//    j = 0, 1, 2). One to three triples left over make an item each, with the fourth wave
//    idle.
// A 768-wide group of 48 matrices is then 144 + 108 = 252 items, where 256x256 tiles would
// be 288 (and compute the lower block of every diagonal tile), and 128x128 tiles 1008 at half
// the work per byte.
//
// The epilogue rounds each block to bf16 once, stages it in LDS and writes it twice: rows of
// block (r, c), and its transpose as block (c, r), read with transposing LDS loads
// (ds_read_b64_tr_b16). A diagonal block writes its upper triangle from its rows and its
// lower triangle from the transpose, so A and B' are exactly symmetric. POLY's b A term is
// the wave's block of A, loaded into the ring by the last iterations of the K loop and
// combined in fp32 before the rounding.
#pragma once

#include "mfma_common.h"

namespace muon {
namespace quad {

using namespace mfma;

constexpr int TK = 32, NSTAGE = 4;
constexpr int kUnitsSlot = 128 * TK / 8;      // one panel's 32-deep slice: 512 16-byte units
constexpr int kUnitsStage = 4 * kUnitsSlot;   // 32 KB
constexpr int kLoadsPerStage = 8;             // wave w fills slot w: 8 loads of 1 KB

enum Mode { GRAM = 0, POLY = 1 };

// The items of `batch` matrices of mp / 256 = S panel pairs each.
struct QuadItems {
  int S;               // panel pairs per side: mp / 256
  int pairs_per_mat;   // S (S - 1) / 2
  int pair_items;      // batch * pairs_per_mat
  int triples;         // batch * S
};

__host__ __device__ inline QuadItems quad_items_of(int batch, int mp) {
  QuadItems q;
  q.S = mp / 256;
  q.pairs_per_mat = q.S * (q.S - 1) / 2;
  q.pair_items = batch * q.pairs_per_mat;
  q.triples = batch * q.S;
  return q;
}

// Items of a group: pair items, then three items per four triples, then left-over triples.
__host__ __device__ inline int quad_item_count(const QuadItems& q) {
  return q.pair_items + 3 * (q.triples >> 2) + (q.triples & 3);
}

__host__ __device__ __forceinline__ int pick4(int s, int v0, int v1, int v2, int v3) {
  return s == 0 ? v0 : s == 1 ? v1 : s == 2 ? v2 : v3;
}

// What wave `wave` of item L does: it loads slot `wave` (panel lpan of matrix lmat) and
// computes the block (rows of slot sa, columns of slot sb): panels (rpan, cpan) of matrix
// omat. An idle wave (active false) computes a copy of another block and stores nothing.
// Matrices are numbered within the item list (0 .. batch - 1).
struct QuadWave {
  int lmat, lpan, sa, sb, omat, rpan, cpan;
  bool active;
};

__host__ __device__ inline QuadWave quad_wave(const QuadItems& g, int L, int wave) {
  int m0, m2, p0, p1, p2, p3, sa, sb;
  bool active = true;
  if (L < g.pair_items) {
    const int b = L / g.pairs_per_mat;
    int u = L - b * g.pairs_per_mat;
    int I = 0;
    while (u >= g.S - 1 - I) { u -= g.S - 1 - I; ++I; }
    const int J = I + 1 + u;
    m0 = m2 = b;
    p0 = 2 * I; p1 = 2 * I + 1; p2 = 2 * J; p3 = 2 * J + 1;
    sa = wave >> 1;
    sb = 2 + (wave & 1);
  } else {
    const int v = L - g.pair_items;
    const int full = g.triples >> 2;
    int tri, j = -1;  // the item's triple; which block of triple 4k + 3 joins it
    if (v < 3 * full) {
      const int k = v / 3;
      j = v - 3 * k;
      tri = 4 * k + j;
    } else {
      tri = 4 * full + (v - 3 * full);
    }
    const int b = tri / g.S, I = tri - b * g.S;
    m0 = b;
    p0 = 2 * I; p1 = 2 * I + 1;
    if (j >= 0) {
      const int t4 = tri - j + 3;
      const int b4 = t4 / g.S, I4 = t4 - b4 * g.S;
      m2 = b4;
      p2 = 2 * I4 + (j == 1 ? 1 : 0);
      p3 = 2 * I4 + 1;
    } else {
      m2 = b;
      p2 = p0;
      p3 = p1;
      active = wave < 3;
    }
    // waves: (0, 0), (1, 1), (0, 1), then the joining block (2, 2) or, for j = 2, (2, 3)
    sa = pick4(wave, 0, 1, 0, 2);
    sb = pick4(wave, 0, 1, 1, j == 2 ? 3 : 2);
  }
  QuadWave q;
  q.lmat = wave < 2 ? m0 : m2;
  q.lpan = pick4(wave, p0, p1, p2, p3);
  q.sa = sa;
  q.sb = sb;
  q.omat = sa < 2 ? m0 : m2;
  q.rpan = pick4(sa, p0, p1, p2, p3);
  q.cpan = pick4(sb, p0, p1, p2, p3);
  q.active = active;
  return q;
}

// One wave's part of an item, resolved to addresses by the caller.
struct QuadWork {
  const uint16_t* lsrc;  // the matrix whose panel lpan this wave loads into slot `wave`
                         // (GRAM: X, ld = np; POLY: A, ld = mp)
  const uint16_t* asrc;  // POLY: the block's matrix of A (its b A term)
  uint16_t* out;         // the block's output matrix (mp x mp)
  int lpan, sa, sb, row0, col0;
  bool active;
  float scale;           // GRAM: s2 on the first round, else 1 (x * 1 is exact)
};

// Fragments of one 16-wide K slice: 4 of the left operand (rows of the block) and 4 of the
// right (its columns, i.e. rows of the column panel).
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

// Byte offset of element (row, col) of wave w's bf16 staging block: 128 rows of 256 bytes
// at 32 KB w, 16-byte chunk q of row r stored at q ^ (r & 15).
__device__ __forceinline__ uint32_t stage_byte(int w, int row, int col) {
  return 32768u * w + 256u * row + 16u * ((col >> 3) ^ (row & 15)) + 2u * (col & 7);
}

// The item, by all 4 waves of the block (every barrier is reached by every wave). smem: the
// 128 KB ring. On return every wave is done with the ring, and this wave's stores are issued
// (not waited for). K: the product's depth (a multiple of 128); ld_in: the row length of
// lsrc's matrix; mp: the output's side (and A's row length). ca, cb, cc: POLY's coefficients.
// kCpol: cache-policy bits of the operand loads (0; the fused launch, whose operands were
// written by other blocks of the same launch, passes device scope).
template <int MODE, int kCpol = 0>
__device__ __forceinline__ void quad_item(u32x4* smem, const QuadWork& w, int K, int ld_in,
                                          int mp, float ca, float cb, float cc) {
  int t = threadIdx.x;
  // opaque here, so that nothing derived from the lane index is computed ahead of the item
  // (in a loop over items, such values would stay live across every other kind of item)
  asm volatile("" : "+v"(t));
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int sa = w.sa, sb = w.sb, row0 = w.row0, col0 = w.col0;
  const bool diag = row0 == col0;
  const char* lsrc = reinterpret_cast<const char*>(w.lsrc);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / TK;  // >= 4: K is a multiple of 128

  // ---- direct-to-LDS loads: wave w fills slot w, 8 loads of 16 rows per stage ----
  // 4 lanes x 16 bytes per row; lane l lands at 16 l of a 1 KB block, the K-major swizzle
  // chosen through the global chunk. Global address: the stage's K origin (scalar) plus the
  // lane's fixed byte offset.
  uint32_t doff[8];
#pragma unroll
  for (int op = 0; op < 8; ++op) {
    const int row = 16 * op + (lane >> 2);
    const int c = (lane & 3) ^ kswz(row);
    doff[op] = 2u * (uint32_t)toff(128 * w.lpan + row, 8 * c, ld_in);
  }
  auto dma_op = [&](int kt, int op) {
    u32x4* st = smem + (kt & (NSTAGE - 1)) * kUnitsStage + wave * kUnitsSlot;
    __builtin_amdgcn_global_load_lds(lsrc + (size_t)kt * kTileBytes + doff[op],
                                     MUON_LDS_PTR(st + 64 * op), 16, 0, kCpol);
  };

  // ---- LDS read addresses (bytes): slice ks of fragment 0 ----
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(MUON_LDS_PTR(smem)));
  const int arow = sa * 128 + (lane & 31), brow = sb * 128 + (lane & 31);
  const uint32_t aoff0 = 64 * arow + 16 * ((lane >> 5) ^ kswz(arow));
  const uint32_t aoff1 = 64 * arow + 16 * ((2 + (lane >> 5)) ^ kswz(arow));
  const uint32_t boff0 = 64 * brow + 16 * ((lane >> 5) ^ kswz(brow));
  const uint32_t boff1 = 64 * brow + 16 * ((2 + (lane >> 5)) ^ kswz(brow));
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

  // ---- software pipeline ----
  // POLY keeps the refills going past the last operand stage: "stages" KT..KT+3 are the
  // four 32-row quarters of the wave's own block of A, which its b A term needs, so the
  // block is in the ring when the loop ends. With KT a multiple of 4, quarter p lands in
  // buffer p, wave w's rows at 8 KB w: row rr of the quarter is 256 bytes, 16-byte chunk q
  // holding the block's chunk q ^ (rr & 15).
  const char* asrc = reinterpret_cast<const char*>(w.asrc);
  auto dma_a = [&](int part, int op) {
    const int rr = 4 * op + (lane >> 4);
    const int gch = (lane & 15) ^ (rr & 15);
    __builtin_amdgcn_global_load_lds(
        asrc + 2 * toff(row0 + 32 * part + rr, col0 + 8 * gch, mp),
        MUON_LDS_PTR(smem + part * kUnitsStage + wave * kUnitsSlot + 64 * op), 16, 0, kCpol);
  };
  constexpr bool kAtile = MODE == POLY;
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  Frags f0, f1;
  // REFILL: 0 none, 1 operand stage kt + 4, 2 A-block quarter kt + 4 - KT
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
  // C[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4] of the wave's 128x128 block.
  uint16_t* out = w.out;
  u32x2* st2 = reinterpret_cast<u32x2*>(smem) + 4096 * wave;  // the wave's staging block

  if constexpr (MODE == POLY) {
    vm_wait<0>();
    __syncthreads();  // every wave's block of A is in the ring
    // v = b A + c acc (+ a on the diagonal) in fp32, rounded once; held packed until every
    // wave is done reading the ring
    uint32_t pk[4][4][8];
    const uint16_t* at = reinterpret_cast<const uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lc = 32 * j + 8 * q + 4 * (lane >> 5);
          // quarter i, wave's 8 KB, row lr & 31
          const u32x2 v2 = *reinterpret_cast<const u32x2*>(
              at + 8 * (i * kUnitsStage + wave * kUnitsSlot + 16 * (lr & 31) +
                        ((lc >> 3) ^ (lr & 15))) + (lc & 7));
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t h = (e < 2 ? v2.x : v2.y) >> (16 * (e & 1));
            v[e] = fmaf(cb, bf2f(h & 0xffffu), cc * acc[i][j][4 * q + e]);
            if (diag && lr == lc + e) v[e] += ca;
          }
          pk[i][j][2 * q] = pack_bf16(v[0], v[1]);
          pk[i][j][2 * q + 1] = pack_bf16(v[2], v[3]);
        }
    }
    __syncthreads();  // the ring's A blocks are no longer read
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lc = 32 * j + 8 * q + 4 * (lane >> 5);
          st2[lr * 32 + 2 * ((lc >> 3) ^ (lr & 15)) + ((lc >> 2) & 1)] =
              u32x2{pk[i][j][2 * q], pk[i][j][2 * q + 1]};
        }
    }
  } else {
    __syncthreads();  // every wave is done with the operand stages
    const float s = w.scale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lc = 32 * j + 8 * q + 4 * (lane >> 5);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] * s;
          st2[lr * 32 + 2 * ((lc >> 3) ^ (lr & 15)) + ((lc >> 2) & 1)] =
              u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        }
    }
  }
  __syncthreads();

  if (w.active) {
    // Row pass: block (r, c), 16-byte chunk lane%16 of rows lane/16 + 4k, 8 rows in flight. A
    // diagonal block writes here only the chunks that start on or above the diagonal.
    {
      const int ch = lane & 15;
      const u32x4* sw = smem + wave * kUnitsStage;
#pragma unroll
      for (int kb = 0; kb < 32; kb += 8) {
        u32x4 wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = (lane >> 4) + 4 * (kb + u);
          wv[u] = sw[r * 16 + (ch ^ (r & 15))];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = (lane >> 4) + 4 * (kb + u);
          if (!diag || 8 * ch >= r)
            *reinterpret_cast<u32x4*>(out + toff(row0 + r, col0 + 8 * ch, mp)) = wv[u];
        }
      }
    }
    // Transpose pass: block (c, r) row R = staged column R, 8 columns = staged rows
    // r0..r0+7. In each 16-lane group, lane 4e + q points at 4 staged columns c0 + 4q.. of
    // row r0 + e (then r0 + 4 + e), and the transposing read gives lane i column c0 + i of
    // those rows. One wave instruction covers 16 rows x 32 columns of the output; 4 in
    // flight.
    {
      const int grp = lane >> 4, li = lane & 15;
#pragma unroll
      for (int ib = 0; ib < 32; ib += 4) {
        s16x4 lo[4], hi[4];
        u32x4 rowv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int combo = ib + u;
          const int c0 = 16 * (combo >> 2), r0 = 32 * (combo & 3) + 8 * grp;
          const int ar = r0 + (li >> 2), acol = c0 + 4 * (li & 3);
          lo[u] = ds_read_tr_at<0>(lds0 + stage_byte(wave, ar, acol));
          hi[u] = ds_read_tr_at<0>(lds0 + stage_byte(wave, ar + 4, acol));
          // row R's own values of the chunk (used where a diagonal block's chunk crosses
          // the diagonal); read unconditionally: a read issued on one path only would let
          // the compiler copy its not-yet-arrived result at the join
          rowv[u] = ds_read_b128_at<0>(lds0 + stage_byte(wave, c0 + li, r0));
        }
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(lo[0]), "+v"(lo[1]), "+v"(lo[2]), "+v"(lo[3]), "+v"(hi[0]),
                       "+v"(hi[1]), "+v"(hi[2]), "+v"(hi[3]), "+v"(rowv[0]), "+v"(rowv[1]),
                       "+v"(rowv[2]), "+v"(rowv[3]));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int combo = ib + u;
          const int c0 = 16 * (combo >> 2), r0 = 32 * (combo & 3) + 8 * grp;
          const int R = c0 + li;
          if (diag && r0 >= R) continue;  // written by the row pass
          const s16x8 tv = {lo[u][0], lo[u][1], lo[u][2], lo[u][3],
                            hi[u][0], hi[u][1], hi[u][2], hi[u][3]};
          u32x4 wv = __builtin_bit_cast(u32x4, tv);
          if (diag && R <= r0 + 7) {  // the diagonal crosses this chunk: upper part from row R
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t keep_lo = r0 + 2 * e < R ? 0x0000ffffu : 0u;
              const uint32_t keep_hi = r0 + 2 * e + 1 < R ? 0xffff0000u : 0u;
              const uint32_t keep = keep_lo | keep_hi;
              wv[e] = (wv[e] & keep) | (rowv[u][e] & ~keep);
            }
          }
          *reinterpret_cast<u32x4*>(out + toff(col0 + R, row0 + r0, mp)) = wv;
        }
      }
    }
  }
}

}  // namespace quad
}  // namespace muon
