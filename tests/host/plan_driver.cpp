// Host build of the decode's chunk choice (choose_chunk in mla_checks.h).
// Mode "sweep": seeded length distributions (uniform, ragged, equal, mostly
// empty, one long sequence among short ones, up to 4096 sequences) at
// several CU counts, minimum chunks, overhead estimates and item capacities;
// every chosen chunk must be a multiple of 32 within [min_chunk, max_chunk],
// give at most max_items items, and cost no more under the planner's cost
// model than the best of the three k-candidates alone.  Prints "violations N
// cases M".  Mode "plan SLOTS MIN OVH ROVH": reads lengths from stdin and prints
// "chunk items rounds" for them.
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "../../mla_latent_kv_22_amd/csrc/mla_checks.h"

using namespace mla;

static long long items_of(const std::vector<int>& L, int ch) {
  long long it = 0;
  for (int l : L) it += (l + ch - 1) / ch;
  return it;
}

// the k-candidates alone (chunk = total / (k slots), k = 1, 2, 4)
static long long base_cost(const std::vector<int>& L, long long total, int slots, int mn, int mx, int ovh, int rovh,
                           int max_items) {
  long long best = -1;
  for (int k = 1; k <= 4; k <<= 1) {
    long long c = (total + (long long)k * slots - 1) / ((long long)k * slots);
    c = ((c + 31) / 32) * 32;
    const int ch = (int)(c < mn ? mn : (c > mx ? mx : c));
    const long long it = items_of(L, ch);
    if (k > 1 && it > max_items) continue;
    const long long cost = (it + slots - 1) / slots * (ch + rovh) + it * ovh / slots;
    if (best < 0 || cost < best) best = cost;
  }
  return best;
}

int main(int argc, char** argv) {
  const int kMaxChunk = 8192;
  if (argc >= 6 && !strcmp(argv[1], "plan")) {
    const int slots = atoi(argv[2]), mn = atoi(argv[3]), ovh = atoi(argv[4]), rovh = atoi(argv[5]);
    std::vector<int> L;
    long long total = 0;
    int v;
    while (scanf("%d", &v) == 1) {
      L.push_back(v);
      total += v;
    }
    const int B = (int)L.size();
    const long long by_len = (total + kMaxChunk - 1) / kMaxChunk;
    const int max_items = (int)((by_len > 4LL * slots ? by_len : 4LL * slots) + B);
    const int ch = choose_chunk(total, B, slots, mn, kMaxChunk, ovh, rovh, max_items,
                                [&](int c) { return items_of(L, c); });
    const long long it = items_of(L, ch);
    printf("%d %lld %lld\n", ch, it, (it + slots - 1) / slots);
    return 0;
  }
  std::mt19937_64 rng(2024);
  long long violations = 0, cases = 0;
  auto expect = [&](bool c, const char* what, int B, int slots) {
    ++cases;
    if (!c) {
      if (violations < 20) fprintf(stderr, "B=%d slots=%d: %s\n", B, slots, what);
      ++violations;
    }
  };
  const int Bs[] = {1, 2, 3, 16, 64, 100, 128, 257, 1000, 4096};
  const int slotss[] = {80, 256, 304};
  for (int dist = 0; dist < 5; ++dist)
    for (int B : Bs)
      for (int slots : slotss)
        for (int rep = 0; rep < 6; ++rep) {
          std::vector<int> L(B);
          const int top = (int)(rng() % 32768) + 1;
          for (int b = 0; b < B; ++b) {
            switch (dist) {
              case 0: L[b] = (int)(rng() % (top + 1)); break;                             // uniform 0..top
              case 1: L[b] = 512 + (int)(rng() % 32257); break;                           // ragged 512..32768
              case 2: L[b] = top; break;                                                  // equal
              case 3: L[b] = (rng() % 8 == 0) ? (int)(rng() % 100) : 0; break;             // mostly empty
              default: L[b] = (b == 0) ? 131072 : 1 + (int)(rng() % 64); break;           // one long
            }
          }
          long long total = 0;
          for (int l : L) total += l;
          for (int mn : {32, 256})
            for (int ovh : {0, 229, 457})
              for (int rovh : {0, 640})
              for (int small = 0; small < 2; ++small) {
                const long long by_len = (total + kMaxChunk - 1) / kMaxChunk;
                // the workspace's item capacity, or the smallest a no-alloc layout allows
                const long long base = by_len > 4LL * slots ? by_len : 4LL * slots;
                const long long need = (by_len > slots ? by_len : slots) + B;
                const int max_items = (int)(small ? need : base + B);
                const int ch = choose_chunk(total, B, slots, mn, kMaxChunk, ovh, rovh, max_items,
                                            [&](int c) { return items_of(L, c); });
                const long long it = items_of(L, ch);
                expect(ch % 32 == 0 && ch >= mn && ch <= kMaxChunk, "chunk range", B, slots);
                expect(it <= max_items, "items within capacity", B, slots);
                const long long cost = (it + slots - 1) / slots * (ch + rovh) + it * ovh / slots;
                expect(cost <= base_cost(L, total, slots, mn, kMaxChunk, ovh, rovh, max_items), "no worse than k-candidates",
                       B, slots);
              }
        }
  printf("violations %lld cases %lld\n", violations, cases);
  return violations == 0 ? 0 : 1;
}
