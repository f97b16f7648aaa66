// The two symmetric products of a Newton-Schulz round on bf16 matrix cores (gfx950).
//
// One round of the quintic iteration of page
// "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (section
// "Newton-Schulz正交化") is A = X X^T, B = b A + c A A, X = a X + B X. Per shape group
// (batch x mp x np, padded to multiples of 128, padding kept at exact zeros):
//
//   gram   A  = s2 * X X^T              K = np
//   poly   B' = a I + b A + c A A       K = mp   (A A = A A^T since A is symmetric)
//
// and the apply kernel (ns_apply_bf16.hip) then forms X' = s1 * B' X. Folding a I into B'
// is exact in real arithmetic and makes apply a plain product. s2 = 1/nu^2 and s1 = 1/nu
// fold the Frobenius normalisation into the first round; later rounds use 1. X, A and B'
// are bf16 in HBM; products accumulate in fp32; epilogues run in fp32 and round to nearest
// even.
//
// Both outputs are symmetric: only the upper 128x128 tiles (I <= J) are computed. The
// epilogue rounds the tile to bf16 once, stages it in LDS and writes it twice (rows of tile
// (I, J), and its transpose as tile (J, I), read with transposing LDS loads); a diagonal
// tile takes its lower triangle from its upper one, so A and B' are exactly symmetric.
//
// Tiling: 256 threads (4 waves as 2x2), a 128x128 output tile per block, each wave 64x64
// (2x2 blocks of v_mfma_f32_32x32x16_bf16). K advances 32 at a time through a ring of 4 LDS
// stages of 16 KB (64 KB per block, two blocks per CU), filled with direct-to-LDS loads three
// stages ahead. Both operands are K-contiguous (rows of X, rows of A); X, A and B' are stored
// in the 16 x 32 tiled layout (toff), so each load instruction (16 rows x 32 columns) reads
// one contiguous kilobyte.
#include <algorithm>
#include <vector>

#include "mfma_common.h"

namespace muon {
namespace {

using namespace mfma;

constexpr int BM = 128, BN = 128, BK = 32, STAGES = 4;
constexpr int kStage = 1024;       // one stage: two 8 KB operand tiles, in 16-byte units
constexpr int kLoadsPerStage = 4;  // direct-to-LDS loads per wave per stage

enum Mode { GRAM = 0, POLY = 1 };

struct SymArgs {         // one shape group
  const uint16_t* in;   // GRAM: X (batch x mp x np); POLY: A (batch x mp x mp)
  uint16_t* out;        // batch x mp x mp
  const float* scales;  // GRAM first round: per matrix {s1, s2, nu, 0}; else null
  long long in_bs;
  int ld_in, K;
  int mp, tiles;        // tiles per side (mp / 128)
  int tiles_per_mat;
};

struct SymLaunch {      // the shape groups of one launch, longest tiles (largest K) first
  TileSplit split;
  SymArgs g[kMaxLaunchGroups];
  float a, b, c;        // POLY coefficients
};

// Byte offset of element (row, col) in the epilogue's bf16 staging tile: 128 rows of 256
// bytes, 16-byte chunk q of row r stored at q ^ (r & 15), so that 16 lanes reading the 16
// chunks of one row, or one chunk of 16 consecutive rows, touch 16 distinct bank groups.
__device__ __forceinline__ uint32_t stage_byte(int row, int col) {
  return 256u * row + 16u * ((col >> 3) ^ (row & 15)) + 2u * (col & 7);
}

// kMulti: the launch holds several groups (block -> group lookup); a single group's blocks
// skip the lookup and the dependent argument load it needs.
template <int MODE, bool kMulti>
__global__ __launch_bounds__(256) void ns_sym_bf16(SymLaunch S) {
  // STAGES ring buffers; stage s holds the left tile at units [1024 s, 1024 s + 512) and the
  // right tile at [1024 s + 512, 1024 (s + 1)). The epilogue reuses all 64 KB.
  __shared__ u32x4 smem[STAGES * kStage];

  const int t = threadIdx.x;
  const int lane = t & 63;
  // wave-uniform, so every LDS destination of the direct loads is scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  int L = 0;
  SymArgs g;
  if constexpr (kMulti) {
    g = S.g[split_block(blockIdx.x, S.split, L)];
  } else {
    g = S.g[0];
    L = xcd_remap(blockIdx.x, gridDim.x);
  }
  const int bidx = L / g.tiles_per_mat;
  int tt = L - bidx * g.tiles_per_mat;
  int I = 0;
  while (tt >= g.tiles - I) { tt -= g.tiles - I; ++I; }
  const int J = I + tt;

  const uint16_t* src = g.in + bidx * g.in_bs;

  // POLY's b A term: the elements of A[I-tile rows][J-tile cols] this lane's accumulators
  // hold (4 consecutive columns of one row per register quad, 8 bytes of the tiled layout).
  // They are loaded right after the last refill, so that they arrive while the last three
  // stages compute and the first stages' loads do not queue behind them; the tail stages'
  // waits leave these kPre loads pending (the memory clobbers keep the compiler from moving
  // them, and tests/test_asm_lds_waits.py checks that they compile to exactly kPre loads).
  u32x2 apre[2][2][4];
  constexpr int kPre = MODE == POLY ? 16 : 0;
  auto load_apre = [&]() {
    if constexpr (MODE == POLY) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            apre[i][j][q] = *reinterpret_cast<const u32x2*>(
                src + toff(I * BM + wr * 64 + 32 * i + (lane & 31),
                           J * BN + wc * 64 + 32 * j + 8 * q + 4 * (lane >> 5), g.ld_in));
      asm volatile("" ::: "memory");
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = g.K / BK;  // >= 4: K is a multiple of 128

  // Direct-to-LDS loads, 4 per wave per stage: loads 0-1 fetch 16 rows each of the left
  // tile (rows of block I), loads 2-3 of the right tile (block J); 4 lanes x 16 bytes per
  // row, lane l landing at 16 l of a 1 KB LDS block (the K-major swizzle is applied by the
  // global chunk a lane fetches). Rows at or beyond mp are fetched from row mp - 1 (their
  // products are never stored). The global address is the stage's K origin (scalar) plus the
  // lane's fixed 32-bit byte offset.
  const char* srcb = reinterpret_cast<const char*>(src);
  uint32_t doff[4];
#pragma unroll
  for (int op = 0; op < 4; ++op) {
    const int row = 16 * (2 * wave + (op & 1)) + (lane >> 2);
    const int c = (lane & 3) ^ kswz(row);
    const uint32_t grow = min((op < 2 ? I * BM : J * BN) + row, g.mp - 1);
    doff[op] = 2u * (uint32_t)toff((int)grow, 8 * c, g.ld_in);
  }
  // A diagonal tile (I == J) multiplies a row block by itself: it loads the block once and
  // reads both operands from it (half the stage traffic of an off-diagonal tile).
  auto run = [&](auto diag_t) {
    constexpr bool kDiag = decltype(diag_t)::value;
    constexpr int kLoads = kDiag ? 2 : kLoadsPerStage;  // direct loads per wave per stage
    auto issue = [&](int kt) {
      u32x4* st = smem + (kt & (STAGES - 1)) * kStage;
      const char* base = srcb + (size_t)kt * kTileBytes;  // next 32-column tile
#pragma unroll
      for (int op = 0; op < kLoads; ++op)
        __builtin_amdgcn_global_load_lds(base + doff[op],
                                         MUON_LDS_PTR(st + (op < 2 ? 0 : 512) +
                                                      64 * (2 * wave + (op & 1))),
                                         16, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s);

    // One stage of the main loop. LATER: this wave's loads issued after stage kt's (two
    // stages while refills run, then one, then none), so stage kt is in once at most LATER
    // stages' loads are pending (plus POLY's kPre loads once the refills are over); REFILL:
    // whether stage kt + 3 is loaded into the buffer that every wave finished with before
    // this stage's barrier.
    auto stage = [&](int kt, auto later_t, auto refill_t) {
      constexpr int later = decltype(later_t)::value;
      vm_wait<later * kLoads + (decltype(refill_t)::value ? 0 : kPre)>();
      // every wave's loads of stage kt are visible, and every wave is done with stage kt - 1
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");  // no LDS access moves across the barrier
      if constexpr (decltype(refill_t)::value) issue(kt + STAGES - 1);

      const u32x4* A = smem + (kt % STAGES) * kStage;
      const u32x4* B = kDiag ? A : A + 512;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int c = 2 * ks + (lane >> 5);
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = frag_k(A, wr * 64 + i * 32 + (lane & 31), c);
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[j] = frag_k(B, wc * 64 + j * 32 + (lane & 31), c);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int kt = 0;
    for (; kt < KT - STAGES; ++kt) stage(kt, I2{}, std::true_type{});
    stage(kt++, I2{}, std::true_type{});
    load_apre();
    stage(kt++, I2{}, std::false_type{});
    stage(kt++, I1{}, std::false_type{});
    stage(kt, I0{}, std::false_type{});
  };
  if (I == J) run(std::true_type{});
  else run(std::false_type{});
  // all waves are done reading the operand stages before the epilogue reuses them
  __syncthreads();

  // Epilogue. With the MFMA operands passed as (right, left), element r of lane l of block
  // (i, j) is C[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4] of the wave's 64x64 quarter. The
  // final values (Gram: s2 C; poly: b A + c C, plus a on the diagonal) are formed in fp32,
  // rounded to bf16 once and staged; the tile is then written twice: rows of tile (I, J),
  // and its transpose as tile (J, I), read with transposing LDS loads. A diagonal tile writes
  // its upper triangle from its rows and its lower triangle from the transpose, so A and B'
  // are exactly symmetric.
  uint16_t* out = g.out + bidx * (size_t)g.mp * g.mp;
  const int mp = g.mp, row0 = I * BM, col0 = J * BN;
  const bool diag = I == J;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(MUON_LDS_PTR(smem)));
  char* const stb = reinterpret_cast<char*>(smem);
  {
    const float s = (MODE == GRAM && g.scales) ? g.scales[4 * bidx + 1] : 1.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int lr = wr * 64 + 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lc = wc * 64 + 32 * j + 8 * q + 4 * (lane >> 5);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (MODE == GRAM) {
              v[e] = acc[i][j][4 * q + e] * s;
            } else {
              const uint32_t w = apre[i][j][q][e >> 1] >> (16 * (e & 1));
              v[e] = fmaf(S.b, bf2f(w & 0xffffu), S.c * acc[i][j][4 * q + e]);
              if (diag && lr == lc + e) v[e] += S.a;
            }
          }
          *reinterpret_cast<u32x2*>(stb + stage_byte(lr, lc)) =
              u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        }
    }
  }
  __syncthreads();

  // Row pass: tile (I, J), 16-byte chunk t%16 of rows t/16 + 16k. A diagonal tile writes
  // here only the chunks that start on or above the diagonal.
  {
    const int ch = t & 15;
    u32x4 w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = (t >> 4) + 16 * k;
      w[k] = smem[r * 16 + (ch ^ (r & 15))];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = (t >> 4) + 16 * k;
      if (!diag || 8 * ch >= r)
        *reinterpret_cast<u32x4*>(out + toff(row0 + r, col0 + 8 * ch, mp)) = w[k];
    }
  }
  // Transpose pass: tile (J, I) row R = staged column R, 8 columns = staged rows r0..r0+7.
  // In each 16-lane group, lane 4e + q points at 4 staged columns c0 + 4q.. of row r0 + e
  // (then r0 + 4 + e), and the transposing read gives lane i column c0 + i of those rows.
  // One wave instruction pair covers 16 rows x 32 columns of the output; 4 in flight.
  {
    const int grp = lane >> 4, li = lane & 15;
#pragma unroll
    for (int ib = 0; ib < 8; ib += 4) {
      s16x4 lo[4], hi[4];
      u32x4 rowv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int combo = 8 * wave + ib + u;
        const int c0 = 16 * (combo >> 2), r0 = 32 * (combo & 3) + 8 * grp;
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
        const int combo = 8 * wave + ib + u;
        const int c0 = 16 * (combo >> 2), r0 = 32 * (combo & 3) + 8 * grp;
        const int R = c0 + li;
        if (diag && r0 >= R) continue;  // written by the row pass
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

// Groups with use_sym256 go to the 256-tile kernel together (ns_sym256_bf16.hip); the rest
// run here, all groups of a call in one grid (a step calls with one group at a time unless
// its groups are too small to fill the device on their own).
namespace {

hipError_t launch_sym128(const NsGroup* const* groups, int n, int mode, float ca, float cb,
                         float cc, hipStream_t s) {
  // per-tile work is the K loop: np for GRAM, mp for POLY
  auto K = [&](const NsGroup* G) { return mode == GRAM ? G->np : G->mp; };
  std::vector<const NsGroup*> order(groups, groups + n);
  std::stable_sort(order.begin(), order.end(),
                   [&](const NsGroup* x, const NsGroup* y) { return K(x) > K(y); });
  for (int c0 = 0; c0 < n; c0 += kMaxLaunchGroups) {
    SymLaunch a{};
    a.a = ca;
    a.b = cb;
    a.c = cc;
    int total = 0, left = 0;
    a.split.n = std::min(kMaxLaunchGroups, n - c0);
    for (int k = 0; k < a.split.n; ++k) {
      const NsGroup& G = *order[c0 + k];
      SymArgs& g = a.g[k];
      g.in = static_cast<const uint16_t*>(mode == GRAM ? G.x_in : G.a);
      g.out = static_cast<uint16_t*>(mode == GRAM ? G.a : G.b);
      g.scales = (mode == GRAM && G.first) ? G.scales : nullptr;
      g.in_bs = mode == GRAM ? (long long)G.mp * G.np : (long long)G.mp * G.mp;
      g.ld_in = K(&G);
      g.K = K(&G);
      g.mp = G.mp;
      g.tiles = G.mp / BM;
      g.tiles_per_mat = g.tiles * (g.tiles + 1) / 2;
      const int tiles = g.tiles_per_mat * G.batch;
      a.split.q[k] = tiles / 8;
      a.split.r[k] = tiles % 8;
      a.split.off[k] = left % 8;
      left += tiles % 8;
      total += tiles;
    }
    const bool multi = a.split.n > 1;
    if (mode == GRAM && multi)
      launch_k((ns_sym_bf16<GRAM, true>), dim3(total), dim3(256), 0, s, a);
    else if (mode == GRAM)
      launch_k((ns_sym_bf16<GRAM, false>), dim3(total), dim3(256), 0, s, a);
    else if (multi)
      launch_k((ns_sym_bf16<POLY, true>), dim3(total), dim3(256), 0, s, a);
    else
      launch_k((ns_sym_bf16<POLY, false>), dim3(total), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

// Splits the groups of a call between the kernels. Groups below 1024 wide whose mp is a
// multiple of 256 go to the four-block kernel (ns_quad_bf16.hip) when together they give it
// about two items per compute unit or more; otherwise, and for other widths below 1024, this
// kernel runs them. With one item per unit every unit finishes at once and writes its four
// blocks (256 KB) in a burst that no computation overlaps: on the GPT-2-124M set's 48 x
// 768x768 group (252 items) the four-block kernel measured within 1% of this one per launch
// and its step 1.9% slower, on 96 x 768x3072 (504 items, K = 3072) its Gram product 6-8%
// faster.
hipError_t launch_sym(const NsGroup* groups, int n, int mode, float ca, float cb, float cc,
                      hipStream_t s) {
  std::vector<NsGroup> big;
  std::vector<const NsGroup*> small, quad;
  long long quad_total = 0;
  for (int i = 0; i < n; ++i) {
    if (use_sym256(groups[i])) {
      big.push_back(groups[i]);
    } else if (use_quad(groups[i])) {
      quad.push_back(groups + i);
      quad_total += quad_items(groups[i]);
    } else {
      small.push_back(groups + i);
    }
  }
  if (!quad.empty()) {
    const int cus = device_cus();
    if (quad_total >= 2 * cus - cus / 8) {
      if (hipError_t e = launch_quad_bf16(quad.data(), (int)quad.size(), mode, ca, cb, cc, s))
        return e;
    } else {
      small.insert(small.end(), quad.begin(), quad.end());
    }
  }
  if (!small.empty())
    if (hipError_t e = launch_sym128(small.data(), (int)small.size(), mode, ca, cb, cc, s))
      return e;
  if (big.empty()) return hipSuccess;
  return mode == GRAM ? launch_gram256_bf16(big.data(), (int)big.size(), s)
                      : launch_poly256_bf16(big.data(), (int)big.size(), ca, cb, cc, s);
}

}  // namespace

hipError_t launch_gram_bf16(const NsGroup* groups, int n, hipStream_t s) {
  return launch_sym(groups, n, GRAM, 0.f, 0.f, 0.f, s);
}

hipError_t launch_poly_bf16(const NsGroup* groups, int n, float ca, float cb, float cc,
                            hipStream_t s) {
  return launch_sym(groups, n, POLY, ca, cb, cc, s);
}

}  // namespace muon
