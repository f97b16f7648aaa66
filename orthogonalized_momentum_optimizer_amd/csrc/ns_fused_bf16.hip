// All Newton-Schulz rounds of a step as one persistent launch (gfx950).
//
// The rounds of page "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (section
// "Newton-Schulz正交化"), for every matrix of up to 4 shape groups: per round r,
//
//   gram    A   = s2 X_r X_r^T                (four-block items, ns_quad_item.h)
//   poly    B'  = a I + b A + c A A           (four-block items)
//   apply   X_{r+1} = s1 B' X_r               (256x256 tiles, the apply kernel's tile)
//
// with s1, s2 the first round's normalisation (1 afterwards), as the per-product kernels
// compute them: the same MFMA sequence per output block and the same epilogue arithmetic, so
// the results are bitwise theirs. Launched as separate kernels, every product ends in a tail where the device drains
// and a burst of stores that nothing overlaps, 3 x rounds times per group; here one block per
// compute unit takes work items from a queue in dependency order and starts each as soon as
// the matrices it reads are complete.
//
// Work and coherence. The matrices of a group are dealt to the 8 XCDs (matrix b to XCD b % 8)
// and each XCD has its own queue: per round, the Gram items of its matrices, then the
// polynomial items, then the apply tiles (groups in the order the host gives per phase).
// A block reads the XCD it runs on from the hardware (HW_REG_XCC_ID) and takes the next item
// of that XCD's queue with an atomic add, so every item that writes or reads a matrix runs
// on that matrix's XCD and its data passes through one L2: a producer waits for its stores
// (vmcnt 0) and then adds 1 to the matrix's completion counter for the phase and round (an
// atomic, performed in L2); a consumer polls the counter with atomics (answered by the L2)
// and loads the data with device-scope (sc1) loads, which the L2 answers and no compute
// unit's L1 does. (With plain loads after an L1 invalidation, buffer_inv sc0, results
// differed from run to run on the GPU: stale L1 lines were read.)
//
// Progress. Items are taken in queue order and an item waits only for items earlier in its
// XCD's queue, each already taken by a running block that waits only for earlier items in
// turn, so the earliest unfinished item never waits and every wait ends. Each wait also
// gives up after max_polls polls (the plan's default, 2^22, is a few seconds), sets the error
// flag, which ends every later wait at once, and goes on, so no wave can spin for long
// whatever happens; and no block makes more passes than the queue has items. A step whose
// launch set the flag makes its update write NaN to every W and O (the update kernels read
// the flag), so such a failure cannot pass unnoticed. Counters, queues and the flag are
// zeroed by a small kernel before the launch.
#include <algorithm>
#include <vector>

#include "ns_quad_item.h"

namespace muon {
namespace {

using namespace mfma;
using quad::NSTAGE;
using quad::TK;
using quad::kUnitsStage;

constexpr int kFusedMaxGroups = 4;
constexpr int kFusedMaxRounds = 16;
enum Phase { PH_GRAM = 0, PH_POLY = 1, PH_APPLY = 2 };

struct FusedGroup {
  uint16_t* x0;          // X_r for even r (X_0 on entry), written for odd r + 1
  uint16_t* x1;          // X_r for odd r
  uint16_t* a;           // A, batch x mp x mp
  uint16_t* b;           // B', batch x mp x mp
  const float* scales;   // per matrix {s1, s2, nu, 0}
  uint32_t* cnt;         // completion counters [3][rounds][batch]
  int batch, mp, np;
  int nblk;              // upper 128x128 blocks per matrix
  int tiles_m, tiles_n;  // 256x256 apply tiles per matrix side
};

struct FusedLaunch {
  FusedGroup g[kFusedMaxGroups];
  int ng, rounds;
  int ord[3][kFusedMaxGroups];       // group order in each phase of a round
  float coef[kFusedMaxRounds][3];    // (a, b, c) of each round
  uint32_t* queue;                   // per-XCD item counters, 64 bytes apart
  uint32_t* err;                     // 1 once a wait gave up
  int max_polls;                     // polls after which a wait gives up
};

// ---- the apply tile ----
// The persistent apply kernel's tile (ns_apply_bf16.hip) on its own: 4 waves as 2x2, each
// 128 rows by four 32-column blocks at 64j + 32wc, a ring of 4 LDS stages of 32 KB filled by
// direct-to-LDS loads (left operand B' K-contiguous, right operand X N-contiguous, read with
// transposing LDS loads), the same hand-interleaved schedule, and the epilogue that pairs
// register quads across the lane halves (v_permlane32_swap) and stores 16 bytes per lane
// straight from the accumulators. The tile's stages are not prefetched during the previous
// item's epilogue.
constexpr int TM = 256, TN = 256;
constexpr int kUnitsA = TM * TK / 8;  // 1024 16-byte units
constexpr int kLoadsPerStage = 8;

struct AFrags {
  s16x4 bh[4][2];
  u32x4 av[4];
};

template <int KS, int OP>
__device__ __forceinline__ void apply_lds_op(uint32_t va, uint32_t vb, AFrags& f) {
  if constexpr (OP < 8) {
    constexpr int j = OP >> 1, half = OP & 1;
    f.bh[j][half] = ds_read_tr_at<128 * j + 2 * 4 * TN * half + 2 * 16 * TN * KS>(vb);
  } else {
    constexpr int i = OP - 8;
    f.av[i] = ds_read_b128_at<2 * 32 * TK * i>(va);
  }
}

// Operand loads of a launch whose operands other blocks of it wrote: device-scope coherent
// (sc1), read from the L2 and never from a copy in this compute unit's L1.
constexpr int kCoherent = 16;

struct ApplyWork {
  const uint16_t* bmat;  // B' of the tile's matrix (mp x mp)
  const uint16_t* x;     // X_r of the matrix (mp x np)
  uint16_t* out;         // X_{r+1} of the matrix
  int row0, col0;
  float scale;           // s1 on the first round, else 1
};

// mp and np are multiples of 256 (every tile lies inside the matrix). On return every wave
// is done with the ring and this wave's stores are issued.
__device__ __forceinline__ void apply_tile(u32x4* smem, const ApplyWork& w, int mp, int np) {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));  // as in quad_item: nothing lane-derived outlives the tile
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int KT = mp / TK;
  const char* lhs = reinterpret_cast<const char*>(w.bmat);
  const char* rhs = reinterpret_cast<const char*>(w.x);
  const size_t rhs_stage_bytes = (size_t)2 * TK * np;

  uint32_t doff[8];
#pragma unroll
  for (int op = 0; op < 4; ++op) {
    const int row = 16 * (4 * wave + op) + (lane >> 2);
    const int ch = (lane & 3) ^ kswz(row);
    doff[op] = 2u * (uint32_t)toff(w.row0 + row, 8 * ch, mp);
  }
#pragma unroll
  for (int op = 0; op < 4; ++op) {
    const int kk = 2 * (4 * wave + op) + (lane >> 5);
    const int ch = (lane & 31) ^ (2 * (kk & 3));
    doff[4 + op] = 2u * (uint32_t)toff(kk, w.col0 + 8 * ch, np);
  }
  auto dma_op = [&](int kt, int op) {
    u32x4* st = smem + (kt & (NSTAGE - 1)) * kUnitsStage;
    if (op < 4)
      __builtin_amdgcn_global_load_lds(lhs + (size_t)kt * kTileBytes + doff[op],
                                       MUON_LDS_PTR(st + 64 * (4 * wave + op)), 16, 0, kCoherent);
    else
      __builtin_amdgcn_global_load_lds(rhs + (size_t)kt * rhs_stage_bytes + doff[op],
                                       MUON_LDS_PTR(st + kUnitsA + 64 * (4 * wave + op - 4)),
                                       16, 0, kCoherent);
  };

  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(MUON_LDS_PTR(smem)));
  const int arow = wr * 128 + (lane & 31);
  const uint32_t aoff0 = 64 * arow + 16 * ((lane >> 5) ^ kswz(arow));
  const uint32_t aoff1 = 64 * arow + 16 * ((2 + (lane >> 5)) ^ kswz(arow));
  const int grp = lane >> 4, jj = lane & 15;
  const int bn = 32 * wc + 16 * (grp & 1) + 4 * (jj & 3);
  const int bk = 8 * (grp >> 1) + (jj >> 2);
  const uint32_t boff = 16 * kUnitsA + 2 * (bk * TN + 8 * ((bn >> 3) ^ (2 * (bk & 3))) + (bn & 7));
  auto stage_base = [&](int kt) { return lds0 + (uint32_t)((kt & (NSTAGE - 1)) * kUnitsStage * 16); };

  auto ready = [&](AFrags& f, bf16x8 (&af)[4], bf16x8 (&bf)[4]) {
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
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
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

  bf16x8 a0[4], b0[4], a1[4], b1[4];
  AFrags f0, f1;
  auto iteration = [&](int kt, auto refill_t, auto more_t) {
    constexpr bool refill = decltype(refill_t)::value, more = decltype(more_t)::value;
    const uint32_t cb = stage_base(kt);
    const uint32_t va1 = cb + aoff1, vb = cb + boff;
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto M) {
      constexpr int m = decltype(M)::value;
      mfma(m, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m < 12) apply_lds_op<1, m>(va1, vb, f1);
      __builtin_amdgcn_sched_barrier(0);
    });
    ready(f1, a1, b1);  // slice 1 is in registers: this wave is done reading stage kt
    if constexpr (more) {
      if constexpr (refill) stage_ready(NSTAGE - 2);
      else stage_ready(min(NSTAGE - 2, KT - 2 - kt));
    }
    const uint32_t nxt = stage_base(kt + 1);
    const uint32_t va0n = nxt + aoff0, vbn = nxt + boff;
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto M) {
      constexpr int m = decltype(M)::value;
      mfma(m, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (refill && m < 8) dma_op(kt + NSTAGE, m);
      if constexpr (more && m >= 2 && m < 14) apply_lds_op<0, m - 2>(va0n, vbn, f0);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (more) ready(f0, a0, b0);
  };

#pragma unroll
  for (int st = 0; st < NSTAGE; ++st)
#pragma unroll
    for (int op = 0; op < 8; ++op) dma_op(st, op);  // KT >= 8: mp is a multiple of 256
  stage_ready(NSTAGE - 1);
  static_for<12>([&](auto OP) { apply_lds_op<0, decltype(OP)::value>(lds0 + aoff0, lds0 + boff, f0); });
  ready(f0, a0, b0);
  int kt = 0;
  for (; kt < KT - NSTAGE; ++kt) iteration(kt, std::true_type{}, std::true_type{});
  for (; kt < KT - 1; ++kt) iteration(kt, std::false_type{}, std::true_type{});
  iteration(KT - 1, std::false_type{}, std::false_type{});
  __builtin_amdgcn_s_barrier();  // every wave is done with the ring
  asm volatile("" ::: "memory");

  // Register quad q of lane l holds columns 8q + 4(l/32) .. +3 of row l%32 of a block;
  // converted to bf16, quads q and q + 1 (q even) are exchanged between the lane halves, after
  // which lane l holds columns 8q + 8(l/32) .. +7 of that row: one 16-byte segment of the
  // tiled layout, 64 np i + 2048 j + 16 q bytes after the lane's segment of block (0, 0).
  const float s = w.scale;
  const int half = lane >> 5;
  char* const seg0 = reinterpret_cast<char*>(
      w.out + toff(w.row0 + wr * 128 + (lane & 31), w.col0 + 32 * wc + 8 * half, np));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; q += 2) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[i][j][4 * q + e] * s;
        uint32_t lo[2] = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        uint32_t hi[2] = {pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto r = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
          lo[d] = r[0];
          hi[d] = r[1];
        }
        *reinterpret_cast<u32x4*>(seg0 + (size_t)64 * np * i + 2048 * j + 16 * q) =
            u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
}

// ---- the queue ----

// The queue's arithmetic is host-callable too, so that a host program can walk every XCD's
// queue and check the progress argument (tests/host_cpp/fused_queue_check.cpp).
__host__ __device__ __forceinline__ int local_batch(int batch, int x) {
  return batch > x ? (batch - x + 7) / 8 : 0;
}

// Items of group g in XCD x for phase ph (Gram and polynomial: four-block items; apply: tiles).
__host__ __device__ __forceinline__ int phase_items(const FusedGroup& G, int ph, int x) {
  const int bx = local_batch(G.batch, x);
  if (ph == PH_APPLY) return bx * G.tiles_m * G.tiles_n;
  return quad::quad_item_count(quad::quad_items_of(bx, G.mp));
}

// Waits until *c >= target (lane 0 of the calling wave polls with an atomic add of 0, which
// the L2 performs and answers: a plain load could keep returning a copy cached in the L1).
// Once any wait of the launch has given up, the flag makes every later wait return at once,
// so a launch whose counters never complete still ends within about one poll limit.
// max_polls 0 gives up at once, whatever the count (the failure path, for a test).
__device__ __forceinline__ void wait_count(uint32_t* c, uint32_t target, uint32_t* err,
                                           int max_polls) {
  if ((threadIdx.x & 63) != 0) return;
  if (max_polls == 0) {
    atomicOr(err, 1u);
    return;
  }
  int polls = 0;
  while (__hip_atomic_fetch_add(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if ((polls & 1023) == 0 &&
        __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
      break;
    __builtin_amdgcn_s_sleep(2);
    if (++polls >= max_polls) {
      atomicOr(err, 1u);
      break;
    }
  }
}

// This wave's stores are complete (in L2), then lane 0 counts them as done.
__device__ __forceinline__ void signal_done(uint32_t* c) {
  vm_wait<0>();
  if ((threadIdx.x & 63) == 0) atomicAdd(c, 1u);
}

struct Item {
  int r, ph, g, i;  // round, phase, group, item of the group's XCD share in that phase
};

__host__ __device__ __forceinline__ Item decode(const FusedLaunch& F, int idx, int per_round,
                                                int x) {
  Item it;
  it.r = idx / per_round;
  int rem = idx - it.r * per_round;
  it.ph = PH_APPLY;
  it.g = F.ord[PH_APPLY][F.ng - 1];
  it.i = 0;
  for (int ph = 0; ph < 3; ++ph)
    for (int k = 0; k < F.ng; ++k) {
      const int g = F.ord[ph][k];
      const int n = phase_items(F.g[g], ph, x);
      if (rem < n) {
        it.ph = ph;
        it.g = g;
        it.i = rem;
        return it;
      }
      rem -= n;
    }
  return it;  // not reached: idx < rounds * per_round
}

// The completion counters an item reads before it starts and the count each must reach:
// apply tiles the polynomial's counter of their matrix (every upper block stored), the
// polynomial's items the Gram counters of the matrices their waves load (m0 for waves 0-1,
// m2 for waves 2-3; one counter when they are one matrix), a later round's Gram items the
// previous round's apply counters of those matrices (4 per tile: each wave of a tile adds
// 1). The first round's Gram items read X_0, complete before the launch (n = 0).
struct Deps {
  uint32_t* c[2];
  uint32_t target;
  int n;
};

__host__ __device__ __forceinline__ Deps item_deps(const FusedLaunch& F, const Item& it, int x) {
  const FusedGroup& G = F.g[it.g];
  const size_t row = (size_t)G.batch;
  Deps d;
  d.n = 0;
  d.target = 0;
  d.c[0] = d.c[1] = nullptr;
  if (it.ph == PH_APPLY) {
    const int j = it.i / (G.tiles_m * G.tiles_n);
    d.c[0] = G.cnt + ((size_t)PH_POLY * F.rounds + it.r) * row + (x + 8 * j);
    d.target = G.nblk;
    d.n = 1;
  } else if (it.ph == PH_POLY || it.r > 0) {
    const quad::QuadItems qi = quad::quad_items_of(local_batch(G.batch, x), G.mp);
    const int m0 = x + 8 * quad::quad_wave(qi, it.i, 0).lmat;
    const int m2 = x + 8 * quad::quad_wave(qi, it.i, 3).lmat;
    uint32_t* c = it.ph == PH_POLY ? G.cnt + ((size_t)PH_GRAM * F.rounds + it.r) * row
                                   : G.cnt + ((size_t)PH_APPLY * F.rounds + it.r - 1) * row;
    d.c[0] = c + m0;
    d.c[1] = c + m2;
    d.target = it.ph == PH_POLY ? (uint32_t)G.nblk : 4u * G.tiles_m * G.tiles_n;
    d.n = m0 == m2 ? 1 : 2;
  }
  return d;
}

__global__ __launch_bounds__(256) void ns_fused_bf16(FusedLaunch) {
  __shared__ u32x4 smem[NSTAGE * kUnitsStage];  // 128 KB ring
  __shared__ int next_item;
  // the arguments are read where they lie, in the kernel-argument segment (scalar loads):
  // a group or round picked with a run-time index then costs no copy of the whole table
  const FusedLaunch& F = *(const FusedLaunch*)__builtin_amdgcn_kernarg_segment_ptr();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const int x = (int)(xcc & 7);

  int per_round = 0;
  for (int g = 0; g < F.ng; ++g)
    for (int ph = 0; ph < 3; ++ph) per_round += phase_items(F.g[g], ph, x);
  const int total = per_round * F.rounds;

  // Every pass takes a distinct item of the queue, so a block makes at most `total` passes;
  // the bound only guards the loop (a pass beyond it sets the error flag and ends the block).
  for (int pass = 0;; ++pass) {
    if (pass > total) {
      if (threadIdx.x == 0) atomicOr(F.err, 2u);
      break;
    }
    if (wave == 0) {
      int idx = 0;
      if (lane == 0) idx = (int)atomicAdd(F.queue + 16 * x, 1u);
      idx = __builtin_amdgcn_readfirstlane(idx);
      if (idx < total) {
        // wait for what the item reads (its loads then bypass the L1: kCoherent); the L1
        // invalidation is kept for any other read of the launch's own data
        const Deps d = item_deps(F, decode(F, idx, per_round, x), x);
        for (int k = 0; k < d.n; ++k) wait_count(d.c[k], d.target, F.err, F.max_polls);
        asm volatile("buffer_inv sc0" ::: "memory");
        vm_wait<0>();
      }
      if (lane == 0) next_item = idx;
    }
    __syncthreads();
    const int idx = __builtin_amdgcn_readfirstlane(next_item);
    if (idx >= total) break;
    const Item it = decode(F, idx, per_round, x);
    const FusedGroup& G = F.g[it.g];
    const size_t row = (size_t)G.batch;
    const uint16_t* xr = (it.r & 1) ? G.x1 : G.x0;
    uint16_t* xn = (it.r & 1) ? G.x0 : G.x1;
    if (it.ph == PH_APPLY) {
      const int tpm = G.tiles_m * G.tiles_n;
      const int j = it.i / tpm, tt = it.i - j * tpm;
      const int b = x + 8 * j;
      const int J = tt / G.tiles_m, I = tt - J * G.tiles_m;  // a matrix's tiles column by column
      const size_t mn = (size_t)G.mp * G.np;
      ApplyWork w;
      w.bmat = G.b + (size_t)b * G.mp * G.mp;
      w.x = xr + b * mn;
      w.out = xn + b * mn;
      w.row0 = I * TM;
      w.col0 = J * TN;
      w.scale = it.r == 0 ? G.scales[4 * b] : 1.f;
      apply_tile(smem, w, G.mp, G.np);
      signal_done(G.cnt + ((size_t)PH_APPLY * F.rounds + it.r) * row + b);
    } else {
      const quad::QuadItems qi = quad::quad_items_of(local_batch(G.batch, x), G.mp);
      const quad::QuadWave qw = quad::quad_wave(qi, it.i, wave);
      const int lb = x + 8 * qw.lmat, ob = x + 8 * qw.omat;
      const size_t mm = (size_t)G.mp * G.mp;
      quad::QuadWork w;
      w.lpan = qw.lpan;
      w.sa = qw.sa;
      w.sb = qw.sb;
      w.row0 = 128 * qw.rpan;
      w.col0 = 128 * qw.cpan;
      w.active = qw.active;
      if (it.ph == PH_GRAM) {
        w.lsrc = xr + (size_t)lb * G.mp * G.np;
        w.asrc = w.lsrc;
        w.out = G.a + ob * mm;
        w.scale = it.r == 0 ? G.scales[4 * ob + 1] : 1.f;
        quad::quad_item<quad::GRAM, kCoherent>(smem, w, G.np, G.np, G.mp, 0.f, 0.f, 0.f);
      } else {
        w.lsrc = G.a + lb * mm;
        w.asrc = G.a + ob * mm;
        w.out = G.b + ob * mm;
        w.scale = 1.f;
        quad::quad_item<quad::POLY, kCoherent>(smem, w, G.mp, G.mp, G.mp, F.coef[it.r][0],
                                               F.coef[it.r][1], F.coef[it.r][2]);
      }
      if (qw.active) signal_done(G.cnt + ((size_t)it.ph * F.rounds + it.r) * row + ob);
    }
  }
}

__global__ void fused_clear(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

// Whether one persistent launch can run these groups' rounds: every group 256-aligned on both
// sides (whole four-block items and 256x256 tiles), at most kFusedMaxGroups groups and
// kFusedMaxRounds rounds.
bool fused_rounds_ok(const NsGroup* groups, int n, int rounds) {
  if (n < 1 || n > kFusedMaxGroups || rounds < 1 || rounds > kFusedMaxRounds) return false;
  for (int k = 0; k < n; ++k)
    if (groups[k].mp % 256 != 0 || groups[k].np % 256 != 0 || groups[k].mp < 256) return false;
  return true;
}

// Counter words of the launch: 8 queues 16 words apart, the error flag, then per group
// 3 x rounds x batch completion counters.
size_t fused_sync_words(const NsGroup* groups, int n, int rounds) {
  size_t w = 8 * 16 + 16;
  for (int k = 0; k < n; ++k) w += (size_t)3 * rounds * groups[k].batch;
  return w;
}

namespace {

// The launch's arguments for groups that fused_rounds_ok accepts: per-group buffers and item
// counts, the completion counters laid out after the queues and the error flag in `sync`,
// and each phase's group order.
FusedLaunch make_fused_launch(const NsGroup* groups, int n, int rounds, const float* abc,
                              uint32_t* sync, int max_polls) {
  FusedLaunch F{};
  F.ng = n;
  F.rounds = rounds;
  F.max_polls = max_polls;
  for (int r = 0; r < rounds; ++r)
    for (int c = 0; c < 3; ++c) F.coef[r][c] = abc[3 * r + c];
  F.queue = sync;
  F.err = fused_error_word(sync);
  uint32_t* cnt = sync + 8 * 16 + 16;
  for (int k = 0; k < n; ++k) {
    const NsGroup& G = groups[k];
    FusedGroup& g = F.g[k];
    g.x0 = static_cast<uint16_t*>(G.x_in);
    g.x1 = static_cast<uint16_t*>(G.x_out);
    g.a = static_cast<uint16_t*>(G.a);
    g.b = static_cast<uint16_t*>(G.b);
    g.scales = G.scales;
    g.cnt = cnt;
    cnt += (size_t)3 * rounds * G.batch;
    g.batch = G.batch;
    g.mp = G.mp;
    g.np = G.np;
    const int T = G.mp / 128;
    g.nblk = T * (T + 1) / 2;
    g.tiles_m = G.mp / TM;
    g.tiles_n = G.np / TN;
  }
  // Gram items longest K first; then the polynomial items and the apply tiles shortest
  // Gram first, whose inputs are complete earliest
  std::vector<int> o(n);
  for (int k = 0; k < n; ++k) o[k] = k;
  std::stable_sort(o.begin(), o.end(), [&](int p, int q) { return groups[p].np > groups[q].np; });
  for (int k = 0; k < n; ++k) {
    F.ord[PH_GRAM][k] = o[k];
    F.ord[PH_POLY][k] = o[n - 1 - k];
    F.ord[PH_APPLY][k] = o[n - 1 - k];
  }
  return F;
}

}  // namespace

hipError_t launch_fused_bf16(const NsGroup* groups, int n, int rounds, const float* abc,
                             uint32_t* sync, int max_polls, hipStream_t s) {
  // the kernel's tiles and items assume these shapes: nothing is launched otherwise
  if (!fused_rounds_ok(groups, n, rounds) || max_polls < 0) return hipErrorInvalidValue;
  const FusedLaunch F = make_fused_launch(groups, n, rounds, abc, sync, max_polls);
  const int words = (int)fused_sync_words(groups, n, rounds);
  launch_k(fused_clear, dim3((words + 255) / 256), dim3(256), 0, s, sync, words);
  if (hipError_t e = hipGetLastError()) return e;
  launch_k(ns_fused_bf16, dim3(device_cus()), dim3(256), 0, s, F);
  return hipGetLastError();
}

}  // namespace muon
