// The two symmetric products of a Newton-Schulz round as launches of four-block work items
// (gfx950), for shape groups whose mp is a multiple of 256 (use_quad below). The item, its
// pipeline and its epilogue are in ns_quad_item.h (page
// "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术", section "Newton-Schulz正交化":
// A = X X^T, B = b A + c A A); this file deals the items of up to 8 groups to blocks, one
// item per block, and resolves each wave's matrices to addresses.
#include <algorithm>
#include <vector>

#include "ns_quad_item.h"

namespace muon {
namespace {

using namespace mfma;
using namespace quad;

struct QuadArgs {        // one shape group
  const uint16_t* in;    // GRAM: X (batch x mp x np); POLY: A (batch x mp x mp)
  uint16_t* out;         // batch x mp x mp
  const float* scales;   // GRAM first round: per matrix {s1, s2, nu, 0}; else null
  long long in_bs;
  int ld_in, K, mp;
  QuadItems items;
};

struct QuadLaunch {      // the shape groups of one launch, longest items (largest K) first
  TileSplit split;
  QuadArgs g[kMaxLaunchGroups];
  float a, b, c;         // POLY coefficients
};

template <int MODE>
__global__ __launch_bounds__(256) void ns_quad_bf16(QuadLaunch S) {
  __shared__ u32x4 smem[NSTAGE * kUnitsStage];  // 128 KB

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int L;
  const QuadArgs g = S.g[split_block(blockIdx.x, S.split, L)];
  const QuadWave qw = quad_wave(g.items, L, wave);

  QuadWork w;
  w.lsrc = g.in + qw.lmat * g.in_bs;
  w.asrc = g.in + qw.omat * g.in_bs;
  w.out = g.out + qw.omat * (size_t)g.mp * g.mp;
  w.lpan = qw.lpan;
  w.sa = qw.sa;
  w.sb = qw.sb;
  w.row0 = 128 * qw.rpan;
  w.col0 = 128 * qw.cpan;
  w.active = qw.active;
  w.scale = (MODE == GRAM && g.scales) ? g.scales[4 * qw.omat + 1] : 1.f;
  quad_item<MODE>(smem, w, g.K, g.ld_in, g.mp, S.a, S.b, S.c);
}

}  // namespace

int quad_items(const NsGroup& G) { return quad_item_count(quad_items_of(G.batch, G.mp)); }

bool use_quad(const NsGroup& G) { return G.mp % 256 == 0; }

hipError_t launch_quad_bf16(const NsGroup* const* groups, int n, int mode, float ca, float cb,
                            float cc, hipStream_t s) {
  // per-item work is the K loop: np for GRAM, mp for POLY
  auto K = [&](const NsGroup* G) { return mode == GRAM ? G->np : G->mp; };
  std::vector<const NsGroup*> order(groups, groups + n);
  std::stable_sort(order.begin(), order.end(),
                   [&](const NsGroup* x, const NsGroup* y) { return K(x) > K(y); });
  for (int c0 = 0; c0 < n; c0 += kMaxLaunchGroups) {
    QuadLaunch a{};
    a.a = ca;
    a.b = cb;
    a.c = cc;
    int total = 0, left = 0;
    a.split.n = std::min(kMaxLaunchGroups, n - c0);
    for (int k = 0; k < a.split.n; ++k) {
      const NsGroup& G = *order[c0 + k];
      QuadArgs& g = a.g[k];
      g.in = static_cast<const uint16_t*>(mode == GRAM ? G.x_in : G.a);
      g.out = static_cast<uint16_t*>(mode == GRAM ? G.a : G.b);
      g.scales = (mode == GRAM && G.first) ? G.scales : nullptr;
      g.in_bs = mode == GRAM ? (long long)G.mp * G.np : (long long)G.mp * G.mp;
      g.ld_in = K(&G);
      g.K = K(&G);
      g.mp = G.mp;
      g.items = quad_items_of(G.batch, G.mp);
      const int items = quad_item_count(g.items);
      a.split.q[k] = items / 8;
      a.split.r[k] = items % 8;
      a.split.off[k] = left % 8;
      left += items % 8;
      total += items;
    }
    if (mode == GRAM)
      launch_k(ns_quad_bf16<GRAM>, dim3(total), dim3(256), 0, s, a);
    else
      launch_k(ns_quad_bf16<POLY>, dim3(total), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

}  // namespace muon
