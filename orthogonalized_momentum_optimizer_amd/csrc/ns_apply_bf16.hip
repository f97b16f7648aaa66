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
// Tiling: 256 threads (4 waves as 2x2), a 256x256 output tile per block, each wave 128 rows
// (wr) by four 32-column blocks at 64j + 32wc, as 4x4 v_mfma_f32_32x32x16_bf16 blocks (256
// fp32 accumulators per lane, in AGPRs). Interleaving the waves' column blocks keeps each
// wave's LDS read addresses a fixed immediate offset apart (see the kernel's set-up), so
// the inner loop spends no vector instructions on addressing.
// Per flop this moves half the global and LDS bytes of a 128x128 tile. K advances 32 at a
// time through a ring of 4 LDS stages of 32 KB (one block per CU, one wave per SIMD), so
// the loop is an explicit software pipeline (below). The left operand B' is
// K-contiguous; the right operand X is N-contiguous and read with transposing LDS loads
// (layouts in mfma_common.h). Output rows/columns beyond the padded shape (when mp or np is
// an odd multiple of 128) are computed from clamped loads and not stored.
//
// With the MFMA operands passed as (right, left), accumulator block (i, j) holds the
// transposed product: element r of lane l is C[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4],
// so each register quad is 4 consecutive columns of one row. The epilogue pairs quads across
// the two lane halves (v_permlane32_swap) so that every lane stores 16 bytes, 8 columns of
// one row: with the tiled output layout that is a contiguous chunk, written straight from
// registers with no LDS staging and no barrier.
//
// Sets too small for 256x256 tiles to occupy half of the compute units (a single 768x768
// matrix has 9) run a 128x128-tile version of the same product instead (ns_apply128_bf16,
// below), bitwise equal to this one.
#include <algorithm>
#include <vector>

#include "mfma_common.h"

namespace muon {
namespace {

using namespace mfma;

constexpr int TM = 256, TN = 256, TK = 32, NSTAGE = 4;
constexpr int kUnitsA = TM * TK / 8;           // 1024 16-byte units
constexpr int kUnitsStage = kUnitsA + TK * TN / 8;
constexpr int kLoadsPerStage = (TM / 16) / 4 + (32 / 2) / 4;  // per wave: 4 + 4

struct ApplyGroup {     // one shape group
  const uint16_t* b;   // B', batch x mp x mp
  const uint16_t* x;   // X, batch x mp x np
  uint16_t* out;       // X', batch x mp x np
  const float* scales; // per matrix {s1, s2, nu, 0}, or null (scale 1)
  int np, tiles_n, per_mat;
  int first;           // the group's first tile in the launch's tile order
};

struct ApplyArgs {      // the shape groups of one launch, all of one mp
  ApplyGroup g[kMaxLaunchGroups];
  int n, mp, tiles_m, total_tiles;
};

// Fragments of one 16-wide K slice: 8 transposed half-fragments of the right operand and 4
// fragments of the left.
struct Frags {
  s16x4 bh[4][2];
  u32x4 av[4];
};

// LDS read `OP` of K slice `KS`: ops 0-7 are the transposing reads of right-operand
// fragment OP/2, half OP%2; ops 8-11 the left-operand fragments. `va` is the lane's
// left-operand address for slice KS of the stage and `vb` its right-operand address; every
// other read of the stage is a fixed offset from those (see the kernel's set-up).
template <int KS, int OP>
__device__ __forceinline__ void lds_op(uint32_t va, uint32_t vb, Frags& f) {
  if constexpr (OP < 8) {
    constexpr int j = OP >> 1, half = OP & 1;
    f.bh[j][half] = ds_read_tr_at<128 * j + 2 * 4 * TN * half + 2 * 16 * TN * KS>(vb);
  } else {
    constexpr int i = OP - 8;
    f.av[i] = ds_read_b128_at<2 * 32 * TK * i>(va);
  }
}

// The launch's arguments in the kernel-argument segment (constant memory): an element picked
// with a run-time index is read with a scalar load instead of copying the whole table.
template <typename T>
__device__ __forceinline__ const T* kernel_args() {
  return (const T*)__builtin_amdgcn_kernarg_segment_ptr();
}


// vmcnt <= 16 + extra for a wave-uniform even `extra` below 2 kN (a chain of immediates: the
// wait's count is an instruction field)
template <int kN>
__device__ __forceinline__ void vm_wait_16_plus(int extra) {
  static_for<kN>([&](auto E) {
    constexpr int e = 2 * decltype(E)::value;
    if (extra == e) vm_wait<16 + e>();
  });
}

// The kernel body. kMulti: the launch holds several groups (tile -> group lookup); a single
// group's tiles skip the lookup and the dependent argument load it needs. kScaled: the first
// round, whose output is scaled by s1 (every group of a launch has its scales, or none has).
// kDefer: how many of a wave's 32 output stores per tile are held back and issued two per
// iteration during the next tile's first iterations (0: all at the tile's end; see below).
template <bool kMulti, bool kScaled, int kDefer>
__device__ __forceinline__ void apply_tiles(const ApplyArgs& g) {
  __shared__ u32x4 smem[NSTAGE * kUnitsStage];  // 128 KB ring

  const int t = threadIdx.x;
  const int lane = t & 63;
  // wave-uniform, so every LDS destination of the direct loads is scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  // ---- persistent tile loop ----
  // Block k of XCD x (blockIdx % 8 = x) takes tiles lo + k, lo + k + nb, ... of the XCD's
  // contiguous range [lo, hi) of the group's tiles (nb = the XCD's block count), so the CUs
  // of one XCD work on neighbouring tiles of the same matrices at the same time.
  const int x = blockIdx.x & 7, k0 = blockIdx.x >> 3;
  const int T = g.total_tiles, G = gridDim.x;  // tiles of all groups, in group order
  const int lo = xcd_remap(x, T);  // first tile of XCD x
  const int nt = T / 8 + (x < (T & 7) ? 1 : 0);
  const int nb = G / 8 + (x < (G & 7) ? 1 : 0);
  const size_t mm = (size_t)g.mp * g.mp;
  const int KT = g.mp / TK;

  struct Tile {
    int bidx, row0, col0, np;
    const char* lhs;
    const char* rhs;
    size_t rhs_stage_bytes;  // one 32-row K step of X
    uint16_t* out;           // the matrix's X'
    const float* scale;      // the matrix's scale record, or null
    uint32_t doff[8];
  };
  // Direct-to-LDS loads, 8 per wave per stage, one instruction each: loads 0-3 fetch 16
  // left-operand rows each (4 lanes x 16 bytes per row), loads 4-7 two right-operand K-rows
  // each (32 lanes x 16 bytes per row); lane l lands at 16 l of a 1 KB LDS block, so the
  // swizzle is applied by choosing the global chunk a lane fetches. The global address is a
  // wave-uniform base (the operand's stage origin, in scalar registers) plus the lane's
  // 32-bit byte offset, fixed for the tile.
  auto setup = [&](int L, Tile& c) {
    // the tile's group: the last one whose first tile is at or below L; its record is
    // read from the kernel-argument segment (scalar loads), so only the chosen group's
    // fields occupy registers
    int k = 0;
    if constexpr (kMulti) {
#pragma unroll
      for (int j = 1; j < kMaxLaunchGroups; ++j)
        if (j < g.n && L >= g.g[j].first) k = j;
    }
    const ApplyGroup& q = kMulti ? kernel_args<ApplyArgs>()->g[k] : g.g[0];
    // A matrix's tiles go column by column (the tiles_m row tiles sharing one column panel
    // of X are consecutive), so the blocks an XCD runs at once share X's column panels and
    // B' (all of B' is used by every column): a wide matrix's X is then fetched about once.
    const int l = L - q.first;
    c.bidx = l / q.per_mat;
    const int tt = l - c.bidx * q.per_mat;
    const int J = tt / g.tiles_m, I = tt - J * g.tiles_m;
    const size_t mn = (size_t)g.mp * q.np;
    c.row0 = I * TM;
    c.col0 = J * TN;
    c.np = q.np;
    c.lhs = reinterpret_cast<const char*>(q.b + c.bidx * mm);
    c.rhs = reinterpret_cast<const char*>(q.x + c.bidx * mn);
    c.rhs_stage_bytes = (size_t)2 * TK * q.np;
    c.out = q.out + c.bidx * mn;
    c.scale = q.scales ? q.scales + 4 * c.bidx : nullptr;
#pragma unroll
    for (int op = 0; op < 4; ++op) {
      const int row = 16 * (4 * wave + op) + (lane >> 2);
      const int ch = (lane & 3) ^ kswz(row);
      const uint32_t grow = min(c.row0 + row, g.mp - 1);
      c.doff[op] = 2u * (uint32_t)toff((int)grow, 8 * ch, g.mp);
    }
#pragma unroll
    for (int op = 0; op < 4; ++op) {
      const int kk = 2 * (4 * wave + op) + (lane >> 5);
      const int ch = (lane & 31) ^ (2 * (kk & 3));
      const uint32_t gcol = min(c.col0 + 8 * ch, c.np - 8);
      c.doff[4 + op] = 2u * (uint32_t)toff(kk, (int)gcol, c.np);
    }
  };
  auto dma_op = [&](const Tile& c, int kt, int op) {
    u32x4* st = smem + (kt & (NSTAGE - 1)) * kUnitsStage;
    if (op < 4)
      __builtin_amdgcn_global_load_lds(c.lhs + (size_t)kt * kTileBytes + c.doff[op],
                                       MUON_LDS_PTR(st + 64 * (4 * wave + op)), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(c.rhs + (size_t)kt * c.rhs_stage_bytes + c.doff[op],
                                       MUON_LDS_PTR(st + kUnitsA + 64 * (4 * wave + op - 4)),
                                       16, 0, 0);
  };

  // ---- LDS read addresses ----
  // Left fragment i of slice ks: row wr*128 + 32i + l%32, chunk 2ks + l/32 (swizzled by
  // bits 2-3 of the row, which 32i leaves alone): base aoff[ks] plus 2048 i bytes.
  // Right fragment j, half h of slice ks: columns 64j + 32wc + (16-column group) of K-rows
  // 16ks + 8(group/2) + 4h + 0..3. Fragment j of a wave covers columns 64j + 32wc, so j
  // moves the chunk index by 8j, above the bits the row swizzle (chunk ^ 2(k & 3)) changes,
  // and h, ks move whole groups of 4 rows, leaving k & 3 alone: base boff plus
  // 128 j + 2048 h + 8192 ks bytes.
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(MUON_LDS_PTR(smem)));
  const int arow = wr * 128 + (lane & 31);
  const uint32_t aoff0 = 64 * arow + 16 * ((lane >> 5) ^ kswz(arow));
  const uint32_t aoff1 = 64 * arow + 16 * ((2 + (lane >> 5)) ^ kswz(arow));
  const int grp = lane >> 4, jj = lane & 15;
  const int bn = 32 * wc + 16 * (grp & 1) + 4 * (jj & 3);
  const int bk = 8 * (grp >> 1) + (jj >> 2);
  const uint32_t boff = 16 * kUnitsA + 2 * (bk * TN + 8 * ((bn >> 3) ^ (2 * (bk & 3))) + (bn & 7));
  auto stage_base = [&](int kt) { return lds0 + (uint32_t)((kt & (NSTAGE - 1)) * kUnitsStage * 16); };

  // Waits for the reads of `f` (and every earlier LDS read of this wave), then assembles the
  // MFMA operands; the assembly depends on the wait, so it cannot move above it.
  auto ready = [&](Frags& f, bf16x8 (&af)[4], bf16x8 (&bf)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.bh[0][0]), "+v"(f.bh[0][1]), "+v"(f.bh[1][0]), "+v"(f.bh[1][1]),
                   "+v"(f.bh[2][0]), "+v"(f.bh[2][1]), "+v"(f.bh[3][0]), "+v"(f.bh[3][1]),
                   "+v"(f.av[0]), "+v"(f.av[1]), "+v"(f.av[2]), "+v"(f.av[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const s16x8 v = {f.bh[j][0][0], f.bh[j][0][1], f.bh[j][0][2], f.bh[j][0][3],
                       f.bh[j][1][0], f.bh[j][1][1], f.bh[j][1][2], f.bh[j][1][3]};
      bf[j] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = __builtin_bit_cast(bf16x8, f.av[i]);
  };
  f32x16 acc[4][4];
  // FIRST: the tile's first K step, whose products start from a zero accumulator operand
  // (used where the step is unrolled; elsewhere the accumulators are zeroed before the tile)
  auto mfma = [&](int m, const bf16x8 (&af)[4], const bf16x8 (&bf)[4], auto first_t) {
    const int i = m >> 2, j = m & 3;
    if constexpr (decltype(first_t)::value)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], f32x16{}, 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
  };
  // Waits for this wave's loads of a stage, then the block barrier: that stage is complete
  // for every wave. The vector-memory counter completes loads and stores in issue order, so
  // the wait leaves pending exactly the operations issued after the stage's loads: `later`
  // stages of loads, plus `stores` output stores when the stage is one of a tile's first
  // four, which were prefetched before the previous tile's epilogue stored its output (32
  // per wave, 16 when the tile's right half lies outside the matrix, 0 when the wave's rows
  // do; `stores` is wave-uniform).
  auto wait_n = [&](auto n_t, int stores) {
    constexpr int n = decltype(n_t)::value;
    if (stores == 32) vm_wait<n + 32>();
    else if (stores == 16) vm_wait<n + 16>();
    else vm_wait<n>();
  };
  auto stage_ready = [&](int later, int stores) {
    if (later >= 3) wait_n(std::integral_constant<int, 3 * kLoadsPerStage>{}, stores);
    else if (later == 2) wait_n(std::integral_constant<int, 2 * kLoadsPerStage>{}, stores);
    else if (later == 1) wait_n(std::integral_constant<int, kLoadsPerStage>{}, stores);
    else wait_n(std::integral_constant<int, 0>{}, stores);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves across the barrier
  };

  // ---- software pipeline of one tile ----
  // Per stage, two batches of 16 MFMAs (one per K slice). While batch 0 runs, the 12 reads
  // of slice 1 are issued between its MFMAs; then (slice 1 in registers, so this wave is done
  // with the stage) the next stage's barrier; while batch 1 runs, the 8 direct loads of stage
  // kt + 4 (into this stage's buffer) and the 12 reads of the next stage's slice 0 are issued
  // between its MFMAs. sched_barrier fences pin that order. The stage loop is split where
  // the refills stop and before the last stage, so neither condition is a branch inside it.
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  Frags f0, f1;
  Tile cur;
  int stores = 0;  // output stores of the previous tile issued after this tile's prefetch

  // ---- deferred output (kDefer > 0) ----
  // All blocks reach a tile's end at about the same time, so storing every output tile at
  // its end sends the whole device's output out in one burst bound by HBM bandwidth (per-block
  // timestamps: 8.4k cycles per tile for the stores alone at K = 768, against ~29.5k in the
  // loop). With kDefer > 0 the tile's last kDefer chunks are kept in registers as bf16 and
  // issued two per iteration during the next tile's first kDefer / 2 iterations (the block's
  // last tile issues them after its loop). Chunk c (0..31) of a wave is accumulator block
  // (c / 8, (c / 2) % 4), register quads 4 (c % 2) and 4 (c % 2) + 1 paired across the lane
  // halves: 16 bytes per lane. A wave stores chunk c if its rows lie inside the matrix and,
  // for (c / 2) % 4 >= 2, if the tile's right half does too (`mode`: 0 no chunk, 1 all, 2
  // the left half only); the waits below count exactly the stores issued.
  constexpr int kImm = 32 - kDefer;
  constexpr int kHead = kDefer > 0 ? kDefer / 2 + 2 : 0;  // iterations whose waits count them
  uint32_t outv[4 * kDefer + 4];
  char* pseg = nullptr;  // the pending tile's lane address of chunk 0
  int p_np = 0;
  int mode = 0;
  auto chunk_addr = [&](int c) {
    return pseg + (size_t)64 * p_np * (c >> 3) + 2048 * ((c >> 1) & 3) + 16 * (2 * (c & 1));
  };
  auto chunk_stored = [&](int c) { return mode == 1 || (mode == 2 && ((c >> 1) & 3) < 2); };
  // deferred stores issued in iteration k of a tile (both of its chunks share (c / 2) % 4)
  auto deferred_in = [&](int k) {
    return (k >= 0 && k < kDefer / 2 && chunk_stored(kImm + 2 * k)) ? 2 : 0;
  };

  // One K step. DD: the first of this iteration's two deferred chunks (-1: none); extra:
  // stores issued after the loads of stage kt + 1, when kDefer > 0.
  using NoD = std::integral_constant<int, -1>;
  auto iteration = [&](int kt, auto refill_t, auto more_t, auto dd_t, int extra, auto first_t) {
    constexpr bool refill = decltype(refill_t)::value, more = decltype(more_t)::value;
    constexpr int dd = decltype(dd_t)::value;
    const uint32_t cb = stage_base(kt);
    const uint32_t va1 = cb + aoff1, vb = cb + boff;
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto M) {
      constexpr int m = decltype(M)::value;
      mfma(m, a0, b0, first_t);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m < 12) lds_op<1, m>(va1, vb, f1);
      if constexpr (dd >= 0 && (m == 12 || m == 14)) {
        constexpr int d = dd + (m == 14 ? 1 : 0);
        if (chunk_stored(kImm + d))
          *reinterpret_cast<u32x4*>(chunk_addr(kImm + d)) =
              u32x4{outv[4 * d], outv[4 * d + 1], outv[4 * d + 2], outv[4 * d + 3]};
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    ready(f1, a1, b1);  // slice 1 is in registers: this wave is done reading stage kt
    if constexpr (more) {
      if constexpr (kDefer > 0 && refill) {
        vm_wait_16_plus<(kImm + 6) / 2 + 1>(extra);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else {
        const int st = kt + 1 < NSTAGE ? stores : 0;  // stage kt + 1 was prefetched
        if constexpr (refill) stage_ready(NSTAGE - 2, st);
        else stage_ready(min(NSTAGE - 2, KT - 2 - kt), st);
      }
    }
    const uint32_t nxt = stage_base(kt + 1);
    const uint32_t va0n = nxt + aoff0, vbn = nxt + boff;
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto M) {
      constexpr int m = decltype(M)::value;
      mfma(m, a1, b1, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (refill && m < 8) dma_op(cur, kt + NSTAGE, m);
      if constexpr (more && m >= 2 && m < 14) lds_op<0, m - 2>(va0n, vbn, f0);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (more) ready(f0, a0, b0);
  };

  int L = lo + k0;
  const int hi = lo + nt;
  if (L < hi) {
    setup(L, cur);
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st)
#pragma unroll
      for (int op = 0; op < 8; ++op) dma_op(cur, st, op);  // KT >= 4: mp is a multiple of 128
  }
  for (; L < hi; L += nb) {
    if constexpr (kDefer == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }
    if constexpr (kDefer > 0) {  // stage 0: three stages of loads and the immediate stores later
      static_for<kImm + 1>([&](auto E) {
        if (stores == decltype(E)::value) vm_wait<3 * kLoadsPerStage + decltype(E)::value>();
      });
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      stage_ready(NSTAGE - 1, stores);
    }
    static_for<12>([&](auto OP) { lds_op<0, decltype(OP)::value>(lds0 + aoff0, lds0 + boff, f0); });
    ready(f0, a0, b0);

    int kt = 0;
    if constexpr (kDefer > 0) {
      // The wait for stage k + 1 leaves pending the two later stages' loads (16) and the
      // stores issued after that stage's loads: the previous tile's immediate stores when the
      // stage was prefetched (k + 1 < 4) and the deferred stores of iterations k - 2 .. k.
      static_for<kHead>([&](auto K) {
        constexpr int k = decltype(K)::value;
        const int extra = (k + 1 < NSTAGE ? stores : 0) + deferred_in(k - 2) +
                          deferred_in(k - 1) + deferred_in(k);
        iteration(k, std::true_type{}, std::true_type{},
                  std::integral_constant<int, (k < kDefer / 2) ? 2 * k : -1>{}, extra,
                  std::integral_constant<bool, k == 0>{});
      });
      kt = kHead;
    }
    using F = std::false_type;
    for (; kt < KT - NSTAGE; ++kt) iteration(kt, std::true_type{}, std::true_type{}, NoD{}, 0, F{});
    for (; kt < KT - 1; ++kt) iteration(kt, std::false_type{}, std::true_type{}, NoD{}, 0, F{});
    iteration(KT - 1, std::false_type{}, std::false_type{}, NoD{}, 0, F{});

    // every wave is done with the ring: the next tile's first stages load while this tile's
    // output is stored
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int row0 = cur.row0, col0 = cur.col0, np = cur.np;
    uint16_t* const out = cur.out;
    const float* const scale = cur.scale;
    if (L + nb < hi) {
      setup(L + nb, cur);
#pragma unroll
      for (int st = 0; st < NSTAGE; ++st)
#pragma unroll
        for (int op = 0; op < 8; ++op) dma_op(cur, st, op);
    }

    // Only the first round's kernels (kScaled) multiply by s1, read with a scalar load;
    // nothing below waits for the next tile's loads (the stores read registers only).
    const float s = kScaled ? scalar_load_f32(scale) : 1.f;
    // The tile is stored straight from the accumulators. Register quad q of lane l holds
    // columns 8q + 4(l/32) .. +3 of row l%32 of a block; converted to bf16, quads q and q + 1
    // (q even) are exchanged between the lane halves (v_permlane32_swap: the upper half of
    // the first operand trades places with the lower half of the second), after which lane l
    // holds columns 8q + 8(l/32) .. +7 of that row: one 16-byte segment of the tiled layout.
    // Addresses: in the tiled layout, with mp and np multiples of 128, lane l's segment of
    // block (i, j), quad pair q sits 64 np i + 2048 j + 16 q bytes after its segment of block
    // (0, 0); a wave's 128 rows and a tile's right 128 columns are each wholly inside the
    // padded matrix or wholly outside.
    const int half = lane >> 5;
    const bool rows_in = row0 + wr * 128 < g.mp, right_in = col0 + 128 < np;
    char* const seg0 = reinterpret_cast<char*>(
        out + toff(min(row0 + wr * 128 + (lane & 31), g.mp - 1), col0 + 32 * wc + 8 * half, np));
    if constexpr (kDefer > 0) {
      // the chunks in order c = 8i + 2j + q/2: the first kImm stored now, the rest kept
      mode = __builtin_amdgcn_readfirstlane(rows_in ? (right_in ? 1 : 2) : 0);
      pseg = seg0;
      p_np = np;
      stores = 0;
      static_for<32>([&](auto C) {
        constexpr int ch = decltype(C)::value;
        constexpr int i = ch >> 3, j = (ch >> 1) & 3, q = 2 * (ch & 1);
        __builtin_amdgcn_sched_barrier(0);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xv = acc[i][j][4 * q + e];
          v[e] = kScaled ? xv * s : xv;
        }
        uint32_t lo[2] = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        uint32_t hi[2] = {pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto r = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
          lo[d] = r[0];
          hi[d] = r[1];
        }
        if constexpr (ch < kImm) {
          if (chunk_stored(ch)) {
            *reinterpret_cast<u32x4*>(chunk_addr(ch)) = u32x4{lo[0], lo[1], hi[0], hi[1]};
            stores += 1;
          }
        } else {
          constexpr int d = ch - kImm;
          outv[4 * d] = lo[0];
          outv[4 * d + 1] = lo[1];
          outv[4 * d + 2] = hi[0];
          outv[4 * d + 3] = hi[1];
        }
      });
      stores = __builtin_amdgcn_readfirstlane(stores);
    } else {
      stores = rows_in ? (right_in ? 32 : 16) : 0;  // the stores issued below
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < 4; q += 2) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = acc[i][j][4 * q + e];
              v[e] = kScaled ? x * s : x;
            }
            uint32_t lo[2] = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            uint32_t hi[2] = {pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const auto r = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
              lo[d] = r[0];
              hi[d] = r[1];
            }
            if (rows_in && (j < 2 || right_in))
              *reinterpret_cast<u32x4*>(seg0 + (size_t)64 * np * i + 2048 * j + 16 * q) =
                  u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        }
    }
  }
  if constexpr (kDefer > 0) {  // the block's last tile: its kept chunks
    static_for<kDefer>([&](auto D) {
      constexpr int d = decltype(D)::value;
      if (chunk_stored(kImm + d))
        *reinterpret_cast<u32x4*>(chunk_addr(kImm + d)) =
            u32x4{outv[4 * d], outv[4 * d + 1], outv[4 * d + 2], outv[4 * d + 3]};
    });
  }
}

// Stores per wave held back to the next tile (24 of 32: the registers for 32 would spill), for
// launches of K >= 24 stages (mp >= 768: the held stores go out during the next tile's first
// 12 iterations) whose operands and output together fit the 256 MB Infinity Cache. When they
// do not (e.g. 96 matrices of 768 x 3072, 1 GB), the loads of the loop come from HBM and the
// held stores inside the loop slowed it more than the end-of-tile burst cost (per-block
// timestamps: ~38k against ~32k cycles per 24-step loop), so those launches store at the
// tile's end, and so does the first round (whose X0 comes from the momentum kernel: holding
// its stores measured 76.4 against 74.6 us per launch on the GPT-2-124M set).
constexpr int kDeferStores = 24;
constexpr int kDeferMinKt = 24;
constexpr size_t kDeferMaxBytes = size_t(256) << 20;

__global__ __launch_bounds__(256) void ns_apply_bf16(ApplyArgs g) {
  apply_tiles<false, false, 0>(g);
}

__global__ __launch_bounds__(256) void ns_apply_bf16_scaled(ApplyArgs g) {
  apply_tiles<false, true, 0>(g);
}

__global__ __launch_bounds__(256) void ns_apply_bf16_groups(ApplyArgs g) {
  apply_tiles<true, false, 0>(g);
}

__global__ __launch_bounds__(256) void ns_apply_bf16_groups_scaled(ApplyArgs g) {
  apply_tiles<true, true, 0>(g);
}

__global__ __launch_bounds__(256) void ns_apply_defer_bf16(ApplyArgs g) {
  apply_tiles<false, false, kDeferStores>(g);
}

__global__ __launch_bounds__(256) void ns_apply_defer_bf16_groups(ApplyArgs g) {
  apply_tiles<true, false, kDeferStores>(g);
}



// ---- 128x128 tiles, for sets whose 256x256 tiles would leave most compute units idle ----
// The same product on 128x128 output tiles, one tile per block (no persistent loop): 256
// threads as 2x2 waves of 64 rows by two 32-column blocks at 64j + 32wc (2x2
// v_mfma_f32_32x32x16_bf16 blocks, the 256-tile kernel's operand order and accumulator
// layout), K in steps of 32 through a ring of 4 LDS stages of 16 KB (64 KB, two blocks per
// CU). Per stage the left operand is 128 rows of B' x 32 K-values (K-contiguous, chunk
// swizzle kswz) and the right operand 32 K-rows of X x 128 columns (N-contiguous, chunk
// c of K-row k at c ^ 2(k & 3)), each filled by 2 direct-to-LDS loads per wave. Every output
// element accumulates the same K slices in the same order with the same instruction as in
// the 256-tile kernel, so the two kernels give bitwise the same X'.
constexpr int SM = 128, SN = 128;
constexpr int kSUnitsA = SM * TK / 8;                // 512 16-byte units
constexpr int kSUnitsStage = kSUnitsA + TK * SN / 8;  // 1024 units, 16 KB
constexpr int kSLoads = 4;                           // direct-to-LDS loads per wave per stage

template <bool kScaled>
__global__ __launch_bounds__(256) void ns_apply128_bf16(ApplyArgs g) {
  __shared__ u32x4 smem[NSTAGE * kSUnitsStage];  // 64 KB ring

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  // tile -> group (the last one whose first tile is at or below it), matrix and position
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int k = 0;
#pragma unroll
  for (int j = 1; j < kMaxLaunchGroups; ++j)
    if (j < g.n && L >= g.g[j].first) k = j;
  const ApplyGroup& q = g.g[k];
  const int l = L - q.first;
  const int bidx = l / q.per_mat;
  const int tt = l - bidx * q.per_mat;
  const int I = tt / q.tiles_n, J = tt - (tt / q.tiles_n) * q.tiles_n;
  const int mp = g.mp, np = q.np;
  const size_t mn = (size_t)mp * np;
  const char* lhs = reinterpret_cast<const char*>(q.b + bidx * (size_t)mp * mp);
  const char* rhs = reinterpret_cast<const char*>(q.x + bidx * mn);
  const size_t rhs_stage_bytes = (size_t)2 * TK * np;
  const int row0 = I * SM, col0 = J * SN;
  const int KT = mp / TK;  // >= 4: mp is a multiple of 128

  // Loads 0-1 of a wave: 16 left-operand rows each (4 lanes x 16 bytes per row); loads 2-3:
  // four right-operand K-rows each (16 lanes x 16 bytes per row). Lane l lands at 16 l of a
  // 1 KB LDS block; the swizzle is applied by the global chunk a lane fetches.
  uint32_t doff[4];
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const int row = 16 * (2 * wave + op) + (lane >> 2);
    const int ch = (lane & 3) ^ kswz(row);
    doff[op] = 2u * (uint32_t)toff(row0 + row, 8 * ch, mp);
  }
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const int kk = 4 * (2 * wave + op) + (lane >> 4);
    const int ch = (lane & 15) ^ (2 * (kk & 3));
    doff[2 + op] = 2u * (uint32_t)toff(kk, col0 + 8 * ch, np);
  }
  auto issue = [&](int kt) {
    u32x4* st = smem + (kt & (NSTAGE - 1)) * kSUnitsStage;
#pragma unroll
    for (int op = 0; op < 2; ++op)
      __builtin_amdgcn_global_load_lds(lhs + (size_t)kt * kTileBytes + doff[op],
                                       MUON_LDS_PTR(st + 64 * (2 * wave + op)), 16, 0, 0);
#pragma unroll
    for (int op = 0; op < 2; ++op)
      __builtin_amdgcn_global_load_lds(rhs + (size_t)kt * rhs_stage_bytes + doff[2 + op],
                                       MUON_LDS_PTR(st + kSUnitsA + 64 * (2 * wave + op)),
                                       16, 0, 0);
  };

  // LDS read addresses (bytes from the stage origin). Left fragment i of slice ks: row
  // wr*64 + 32i + l%32, chunk 2ks + l/32 (swizzled by bits 2-3 of the row, which 32i leaves
  // alone): aoff + 2048 i + 32 ks bytes before the swizzle, so each ks has its own base.
  // Right fragment j, half h of slice ks: columns 64j + 32wc + (16-column group), K-rows
  // 16ks + 8(group/2) + 4h + 0..3: boff + 128 j + 1024 h + 4096 ks (j moves the chunk index
  // by 8, above the bits the row swizzle changes; h and ks move whole groups of 4 rows).
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(MUON_LDS_PTR(smem)));
  const int arow = wr * 64 + (lane & 31);
  const uint32_t aoff0 = 64 * arow + 16 * ((lane >> 5) ^ kswz(arow));
  const uint32_t aoff1 = 64 * arow + 16 * ((2 + (lane >> 5)) ^ kswz(arow));
  const int grp = lane >> 4, jj = lane & 15;
  const int bn = 32 * wc + 16 * (grp & 1) + 4 * (jj & 3);
  const int bk = 8 * (grp >> 1) + (jj >> 2);
  const uint32_t boff =
      16 * kSUnitsA + 2 * (bk * SN + 8 * ((bn >> 3) ^ (2 * (bk & 3))) + (bn & 7));

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // One K slice: 2 left and 4 transposing right reads, one wait that names them, 4 MFMAs.
  auto slice = [&](uint32_t sb, auto ks_t) {
    constexpr int ks = decltype(ks_t)::value;
    const uint32_t va = sb + (ks ? aoff1 : aoff0), vb = sb + boff;
    u32x4 av0 = ds_read_b128_at<0>(va);
    u32x4 av1 = ds_read_b128_at<2048>(va);
    s16x4 b00 = ds_read_tr_at<4096 * ks>(vb);
    s16x4 b01 = ds_read_tr_at<1024 + 4096 * ks>(vb);
    s16x4 b10 = ds_read_tr_at<128 + 4096 * ks>(vb);
    s16x4 b11 = ds_read_tr_at<128 + 1024 + 4096 * ks>(vb);
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(av0), "+v"(av1), "+v"(b00), "+v"(b01), "+v"(b10), "+v"(b11));
    const bf16x8 af[2] = {__builtin_bit_cast(bf16x8, av0), __builtin_bit_cast(bf16x8, av1)};
    const s16x8 v0 = {b00[0], b00[1], b00[2], b00[3], b01[0], b01[1], b01[2], b01[3]};
    const s16x8 v1 = {b10[0], b10[1], b10[2], b10[3], b11[0], b11[1], b11[2], b11[3]};
    const bf16x8 bf[2] = {__builtin_bit_cast(bf16x8, v0), __builtin_bit_cast(bf16x8, v1)};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
  };
  // One stage: LATER of this wave's loads issued after stage kt's (two while refills run,
  // then one, then none) may still be pending; after the barrier every wave's loads of stage
  // kt are visible and every wave has its reads of stage kt - 1 in registers, so that
  // buffer takes stage kt + 3.
  auto stage = [&](int kt, auto later_t, auto refill_t) {
    constexpr int later = decltype(later_t)::value;
    vm_wait<later * kSLoads>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves across the barrier
    if constexpr (decltype(refill_t)::value) issue(kt + NSTAGE - 1);
    const uint32_t sb = lds0 + (uint32_t)((kt & (NSTAGE - 1)) * kSUnitsStage * 16);
    slice(sb, std::integral_constant<int, 0>{});
    slice(sb, std::integral_constant<int, 1>{});
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st) issue(st);
  int kt = 0;
  for (; kt < KT - (NSTAGE - 1); ++kt) stage(kt, I2{}, std::true_type{});
  stage(kt++, I2{}, std::false_type{});
  stage(kt++, I1{}, std::false_type{});
  stage(kt, I0{}, std::false_type{});

  // Epilogue, straight from the accumulators as in the 256-tile kernel: quads q and q + 1
  // (q even) are exchanged between the lane halves, after which lane l holds columns
  // 8q + 8(l/32) .. +7 of row l%32 of block (i, j): 16 contiguous bytes of the tiled layout.
  const float s = kScaled ? q.scales[4 * bidx] : 1.f;
  uint16_t* const out = q.out + bidx * mn;
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = row0 + wr * 64 + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int qq = 0; qq < 4; qq += 2) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = acc[i][j][4 * qq + e];
          v[e] = kScaled ? x * s : x;
        }
        uint32_t lo[2] = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        uint32_t hi[2] = {pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto pr = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
          lo[d] = pr[0];
          hi[d] = pr[1];
        }
        const int c = col0 + 64 * j + 32 * wc + 8 * qq + 8 * half;
        *reinterpret_cast<u32x4*>(out + toff(r, c, np)) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
  }
}

// launches the grid for a single group or for several, first round (scaled) or not
void launch_apply_grid(const ApplyArgs& a, bool scaled, dim3 grid, hipStream_t s) {
  size_t bytes = 0;  // B', X and X' of every matrix of the launch
  for (int k = 0; k < a.n; ++k) {
    const int end = k + 1 < a.n ? a.g[k + 1].first : a.total_tiles;
    const size_t batch = (size_t)(end - a.g[k].first) / a.g[k].per_mat;
    bytes += batch * 2 * ((size_t)a.mp * a.mp + 2 * (size_t)a.mp * a.g[k].np);
  }
  if (!scaled && a.mp / TK >= kDeferMinKt && bytes <= kDeferMaxBytes) {
    if (a.n > 1) launch_k(ns_apply_defer_bf16_groups, grid, dim3(256), 0, s, a);
    else launch_k(ns_apply_defer_bf16, grid, dim3(256), 0, s, a);
    return;
  }
  if (a.n > 1 && scaled) launch_k(ns_apply_bf16_groups_scaled, grid, dim3(256), 0, s, a);
  else if (a.n > 1) launch_k(ns_apply_bf16_groups, grid, dim3(256), 0, s, a);
  else if (scaled) launch_k(ns_apply_bf16_scaled, grid, dim3(256), 0, s, a);
  else launch_k(ns_apply_bf16, grid, dim3(256), 0, s, a);
}

}  // namespace

// Compute units of the current device (one persistent block each).
int device_cus() {
  static int cached[64] = {};
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
    n = 256;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

// All groups of a call with the same mp in one grid (their tiles all cost the same:
// K = mp): one persistent block per compute unit over 256x256 tiles, or, when those tiles
// would leave at least half of the compute units idle, one block per 128x128 tile (four
// times as many tiles, at most two blocks per compute unit). A step calls with one group at
// a time unless its groups are too small to fill the device on their own.
hipError_t launch_apply_bf16(const NsGroup* groups, int n, hipStream_t s) {
  const int cus = device_cus();
  std::vector<bool> done(n, false);
  for (int k0 = 0; k0 < n; ++k0) {
    if (done[k0]) continue;
    // a group that fills the device on its own gets a launch of its own; smaller groups
    // share one (every XCD's L2 then serves fewer matrices at a time)
    auto own_tiles = [&](int k) {
      return ((groups[k].mp + TM - 1) / TM) * ((groups[k].np + TN - 1) / TN) * groups[k].batch;
    };
    std::vector<const NsGroup*> set;
    for (int k = k0; k < n && (int)set.size() < kMaxLaunchGroups; ++k)
      if (!done[k] && groups[k].mp == groups[k0].mp) {
        const bool alone = own_tiles(k) >= cus;
        if (alone && !set.empty()) continue;
        done[k] = true;
        set.push_back(&groups[k]);
        if (alone) break;
      }
    auto fill = [&](int tm, int tn) {
      ApplyArgs a{};
      a.mp = groups[k0].mp;
      a.tiles_m = (a.mp + tm - 1) / tm;
      for (const NsGroup* G : set) {
        ApplyGroup& q = a.g[a.n++];
        q.b = static_cast<const uint16_t*>(G->b);
        q.x = static_cast<const uint16_t*>(G->x_in);
        q.out = static_cast<uint16_t*>(G->x_out);
        q.scales = G->first ? G->scales : nullptr;
        q.np = G->np;
        q.tiles_n = (G->np + tn - 1) / tn;
        q.per_mat = a.tiles_m * q.tiles_n;
        q.first = a.total_tiles;
        a.total_tiles += q.per_mat * G->batch;
      }
      return a;
    };
    const ApplyArgs a = fill(TM, TN);
    const bool scaled = a.g[0].scales != nullptr;
    if (2 * a.total_tiles <= cus) {
      const ApplyArgs h = fill(SM, SN);
      if (scaled) launch_k(ns_apply128_bf16<true>, dim3(h.total_tiles), dim3(256), 0, s, h);
      else launch_k(ns_apply128_bf16<false>, dim3(h.total_tiles), dim3(256), 0, s, h);
    } else {
      // persistent blocks: as few as give every block the same number of tiles (at most one
      // block per CU, a multiple of 8 for the XCDs); apply is power-limited, and CUs left
      // idle by a last, part-filled round of tiles measured ~1% slower on the GPT-2-124M set
      const int per = (a.total_tiles + cus - 1) / cus;  // tiles per block
      const int nb = ((a.total_tiles + per - 1) / per + 7) / 8 * 8;
      launch_apply_grid(a, scaled, dim3(std::min(nb, cus)), s);
    }
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

}  // namespace muon
