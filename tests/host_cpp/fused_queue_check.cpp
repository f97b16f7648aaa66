// Host check of the single launch's queues (ns_fused_bf16.hip, compiled into this program with
// the library's flags): for many sets of shape groups and round counts, every XCD's queue is
// walked in claim order through the kernel's own decode and item_deps. Checked:
//  - every item decodes in range, and every matrix an item touches is one of its XCD's
//    (matrix b on XCD b % 8);
//  - every round's upper 128x128 blocks of A and B' and every 256x256 tile of X' is produced
//    exactly once;
//  - every counter an item waits for is the counter of the matrices it reads, its target is
//    the number of signals that counter receives, and every item that signals it comes
//    earlier in the same XCD's queue.
// The last point is the launch's progress argument: blocks take items in queue order, so the
// earliest unfinished item never waits, and every wait ends. Prints "fused queues ok".
#include <cstdio>
#include <map>
#include <random>
#include <vector>

#include "ns_fused_bf16.hip"

namespace muon {
thread_local LaunchTiming g_launch_timing;  // referenced by launch_k, unused here
int device_cus() { return 256; }
}  // namespace muon

using namespace muon;

static int fails = 0;
#define CHECK(c, ...)                              \
  do {                                             \
    if (!(c)) {                                    \
      if (++fails < 20) std::printf(__VA_ARGS__);  \
    }                                              \
  } while (0)

struct Counter {
  int signals = 0;       // adds the counter receives over the launch
  long long last = -1;   // queue position of the last item that adds to it
  int xcd = -1;
};

static long long check_set(const std::vector<NsGroup>& groups, int rounds) {
  const int n = (int)groups.size();
  std::vector<uint32_t> sync(fused_sync_words(groups.data(), n, rounds), 0u);
  std::vector<float> abc(3 * rounds, 1.f);
  const FusedLaunch F = make_fused_launch(groups.data(), n, rounds, abc.data(), sync.data(), 1);
  auto counter_id = [&](const uint32_t* c) { return (long long)(c - sync.data()); };

  // products of each (group, round): blocks of A and B' (phase 0, 1) and tiles of X' (phase 2)
  std::map<std::vector<int>, int> made;
  std::map<long long, Counter> counters;
  long long items = 0;
  for (int x = 0; x < 8; ++x) {
    int per_round = 0;
    for (int g = 0; g < n; ++g)
      for (int ph = 0; ph < 3; ++ph) per_round += phase_items(F.g[g], ph, x);
    const int total = per_round * rounds;
    // first pass: what every item produces and signals
    for (int idx = 0; idx < total; ++idx) {
      const Item it = decode(F, idx, per_round, x);
      CHECK(it.r >= 0 && it.r < rounds && it.ph >= 0 && it.ph < 3 && it.g >= 0 && it.g < n,
            "xcd %d item %d: decodes out of range\n", x, idx);
      if (!(it.r >= 0 && it.r < rounds && it.ph >= 0 && it.ph < 3 && it.g >= 0 && it.g < n))
        continue;
      const FusedGroup& G = F.g[it.g];
      CHECK(it.i >= 0 && it.i < phase_items(G, it.ph, x), "xcd %d item %d: index out of range\n",
            x, idx);
      const uint32_t* base = G.cnt + ((size_t)it.ph * rounds + it.r) * G.batch;
      auto signal = [&](int b, int adds) {
        CHECK(b >= 0 && b < G.batch && b % 8 == x, "xcd %d item %d: matrix %d not its own\n", x,
              idx, b);
        Counter& c = counters[counter_id(base + b)];
        c.signals += adds;
        c.last = idx;
        c.xcd = x;
      };
      if (it.ph == PH_APPLY) {
        const int tpm = G.tiles_m * G.tiles_n;
        const int j = it.i / tpm, tt = it.i - j * tpm;
        const int b = x + 8 * j;
        signal(b, 4);  // each wave of the tile adds 1
        ++made[{it.g, it.r, 2, b, tt % G.tiles_m, tt / G.tiles_m}];
      } else {
        const quad::QuadItems qi = quad::quad_items_of(local_batch(G.batch, x), G.mp);
        for (int w = 0; w < 4; ++w) {
          const quad::QuadWave qw = quad::quad_wave(qi, it.i, w);
          if (!qw.active) continue;
          const int ob = x + 8 * qw.omat;
          signal(ob, 1);
          ++made[{it.g, it.r, it.ph, ob, qw.rpan, qw.cpan}];
        }
      }
      ++items;
    }
    // second pass: every wait is for the matrices read, with the right target, on a counter
    // whose signalling items all come earlier in this queue
    for (int idx = 0; idx < total; ++idx) {
      const Item it = decode(F, idx, per_round, x);
      const FusedGroup& G = F.g[it.g];
      const Deps d = item_deps(F, it, x);
      std::vector<int> reads;  // matrices whose inputs the item reads
      if (it.ph == PH_APPLY) {
        reads.push_back(x + 8 * (it.i / (G.tiles_m * G.tiles_n)));
        CHECK(d.n == 1, "xcd %d item %d: apply tile waits on %d counters\n", x, idx, d.n);
      } else {
        const quad::QuadItems qi = quad::quad_items_of(local_batch(G.batch, x), G.mp);
        for (int w = 0; w < 4; ++w) {
          const quad::QuadWave qw = quad::quad_wave(qi, it.i, w);
          reads.push_back(x + 8 * qw.lmat);                      // the panel it loads
          if (it.ph == PH_POLY) reads.push_back(x + 8 * qw.omat);  // its b A term
        }
        const bool first_gram = it.ph == PH_GRAM && it.r == 0;
        CHECK(first_gram ? d.n == 0 : (d.n == 1 || d.n == 2), "xcd %d item %d: %d counters\n",
              x, idx, d.n);
      }
      if (d.n == 0) continue;
      // the phase and round whose outputs the item reads
      const int ph_in = it.ph == PH_GRAM ? PH_APPLY : it.ph - 1;
      const int r_in = it.ph == PH_GRAM ? it.r - 1 : it.r;
      const uint32_t* in_base = G.cnt + ((size_t)ph_in * rounds + r_in) * G.batch;
      for (int b : reads) {
        bool waited = false;
        for (int k = 0; k < d.n; ++k) waited = waited || d.c[k] == in_base + b;
        CHECK(waited, "xcd %d item %d (r %d ph %d): reads matrix %d without waiting for it\n", x,
              idx, it.r, it.ph, b);
      }
      for (int k = 0; k < d.n; ++k) {
        auto f = counters.find(counter_id(d.c[k]));
        CHECK(f != counters.end(), "xcd %d item %d: waits on a counter nothing signals\n", x, idx);
        if (f == counters.end()) continue;
        CHECK(f->second.xcd == x, "xcd %d item %d: waits on another XCD's counter\n", x, idx);
        CHECK(f->second.last < idx, "xcd %d item %d: waits on item %lld, later in the queue\n",
              x, idx, f->second.last);
        CHECK((int)d.target == f->second.signals,
              "xcd %d item %d: target %u but the counter receives %d signals\n", x, idx,
              d.target, f->second.signals);
      }
    }
  }
  // every product exactly once
  for (int g = 0; g < n; ++g) {
    const FusedGroup& G = F.g[g];
    const int T = G.mp / 128;
    for (int r = 0; r < rounds; ++r)
      for (int b = 0; b < G.batch; ++b) {
        for (int ph = 0; ph < 2; ++ph)
          for (int rp = 0; rp < T; ++rp)
            for (int cp = rp; cp < T; ++cp) {
              auto f = made.find({g, r, ph, b, rp, cp});
              CHECK(f != made.end() && f->second == 1,
                    "group %d round %d phase %d matrix %d block (%d, %d) made %d times\n", g, r,
                    ph, b, rp, cp, f == made.end() ? 0 : f->second);
            }
        for (int I = 0; I < G.tiles_m; ++I)
          for (int J = 0; J < G.tiles_n; ++J) {
            auto f = made.find({g, r, 2, b, I, J});
            CHECK(f != made.end() && f->second == 1,
                  "group %d round %d matrix %d tile (%d, %d) made %d times\n", g, r, b, I, J,
                  f == made.end() ? 0 : f->second);
          }
      }
  }
  size_t expected = 0;
  for (int g = 0; g < n; ++g) {
    const int T = F.g[g].mp / 128;
    expected += (size_t)rounds * F.g[g].batch * (T * (T + 1) + F.g[g].tiles_m * F.g[g].tiles_n);
  }
  CHECK(made.size() == expected, "%zu products made, %zu expected\n", made.size(), expected);
  return items;
}

int main() {
  long long items = 0;
  int sets = 0;
  // the GPT-2-124M set's groups, then seeded random sets of 1-4 groups
  {
    std::vector<NsGroup> gs(2);
    gs[0].batch = 48; gs[0].mp = 768; gs[0].np = 768;
    gs[1].batch = 24; gs[1].mp = 768; gs[1].np = 3072;
    for (int rounds : {1, 2, 5, 16}) {
      items += check_set(gs, rounds);
      ++sets;
    }
  }
  std::mt19937 rng(12345);
  for (int t = 0; t < 150; ++t) {
    const int n = 1 + (int)(rng() % 4);
    std::vector<NsGroup> gs(n);
    for (int k = 0; k < n; ++k) {
      gs[k].batch = 8 + (int)(rng() % 33);
      gs[k].mp = 256 * (1 + (int)(rng() % 6));
      gs[k].np = gs[k].mp + 256 * (int)(rng() % 8);
    }
    const int rounds = 1 + (int)(rng() % 16);
    if (!fused_rounds_ok(gs.data(), n, rounds)) {
      CHECK(false, "set %d: fused_rounds_ok refuses a valid set\n", t);
      continue;
    }
    items += check_set(gs, rounds);
    ++sets;
  }
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("fused queues ok: %d sets, %lld items\n", sets, items);
  return 0;
}
