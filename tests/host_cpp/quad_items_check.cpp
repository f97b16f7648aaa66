// Host check of the four-block item map of ns_quad_item.h (compiled into this program with
// ns_quad_bf16.hip, the library's flags): for a range of group sizes, every upper block (r <= c) of every
// matrix is computed and stored by exactly one wave, every index is in range, and the data a
// wave multiplies is what the waves of its item load (slot sa holds the block's row panel,
// slot sb its column panel, both of the block's matrix). Prints "quad items ok".
#include <cstdio>
#include <vector>

#include "ns_quad_bf16.hip"

namespace muon {
thread_local LaunchTiming g_launch_timing;  // referenced by launch_k, unused here
int device_cus() { return 256; }
}  // namespace muon

using muon::quad::QuadItems;

static int fails = 0;
#define CHECK(c, ...)                         \
  do {                                        \
    if (!(c)) {                               \
      if (++fails < 20) std::printf(__VA_ARGS__); \
    }                                         \
  } while (0)

int main() {
  long long checked = 0;
  for (int mp = 256; mp <= 2048; mp += 256) {
    for (int batch = 1; batch <= 50; ++batch) {
      const QuadItems g = muon::quad::quad_items_of(batch, mp);
      const int T = mp / 128;
      const int items = muon::quad::quad_item_count(g);
      muon::NsGroup G{};
      G.mp = mp;
      G.batch = batch;
      CHECK(muon::quad_items(G) == items, "mp %d batch %d: item counts differ\n", mp, batch);
      std::vector<int> hits((size_t)batch * T * T, 0);
      for (int L = 0; L < items; ++L) {
        muon::quad::QuadWave w[4];
        for (int k = 0; k < 4; ++k) w[k] = muon::quad::quad_wave(g, L, k);
        for (int k = 0; k < 4; ++k) {
          const muon::quad::QuadWave& q = w[k];
          CHECK(q.lmat >= 0 && q.lmat < batch && q.lpan >= 0 && q.lpan < T,
                "mp %d batch %d item %d wave %d: load slot out of range\n", mp, batch, L, k);
          CHECK(q.sa >= 0 && q.sa < 4 && q.sb >= 0 && q.sb < 4,
                "mp %d batch %d item %d wave %d: slot index out of range\n", mp, batch, L, k);
          if (q.sa < 0 || q.sa > 3 || q.sb < 0 || q.sb > 3) continue;
          const muon::quad::QuadWave& ra = w[q.sa];
          const muon::quad::QuadWave& rb = w[q.sb];
          CHECK(ra.lmat == q.omat && ra.lpan == q.rpan,
                "mp %d batch %d item %d wave %d: row slot holds the wrong panel\n", mp, batch, L, k);
          CHECK(rb.lmat == q.omat && rb.lpan == q.cpan,
                "mp %d batch %d item %d wave %d: column slot holds the wrong panel\n", mp, batch,
                L, k);
          CHECK(q.rpan <= q.cpan, "mp %d batch %d item %d wave %d: block below the diagonal\n",
                mp, batch, L, k);
          if (q.active && q.omat >= 0 && q.omat < batch && q.rpan >= 0 && q.cpan < T)
            ++hits[((size_t)q.omat * T + q.rpan) * T + q.cpan];
        }
      }
      for (int b = 0; b < batch; ++b)
        for (int r = 0; r < T; ++r)
          for (int c = 0; c < T; ++c) {
            const int h = hits[((size_t)b * T + r) * T + c];
            CHECK(h == (r <= c ? 1 : 0), "mp %d batch %d: block (%d, %d, %d) stored %d times\n",
                  mp, batch, b, r, c, h);
            ++checked;
          }
    }
  }
  // 48 matrices of 768 x 768: 144 pair items and 108 items from the 144 triples
  {
    muon::NsGroup G{};
    G.mp = 768;
    G.batch = 48;
    CHECK(muon::quad_items(G) == 252, "768 x 48: %d items, expected 252\n", muon::quad_items(G));
  }
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("quad items ok (%lld blocks)\n", checked);
  return 0;
}
