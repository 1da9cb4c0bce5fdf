// Host build of the device-side index checks (mla_checks.h): runs them over
// valid and corrupted block tables, slots and sequence offsets, and counts
// every result that would take an access outside the caller's buffers or
// change a valid value.  Prints "violations N cases M"; the CPU test suite
// compiles this file with g++ and expects N = 0.
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "../../mla_latent_kv_22_amd/csrc/mla_checks.h"

using namespace mla;

static long long violations = 0, cases = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    ++cases;                                                        \
    if (!(c)) {                                                     \
      if (violations < 20) fprintf(stderr, "line %d: %s\n", __LINE__, #c); \
      ++violations;                                                 \
    }                                                               \
  } while (0)

int main() {
  std::mt19937_64 rng(12345);
  auto uni = [&](long long lo, long long hi) { return lo + (long long)(rng() % (unsigned long long)(hi - lo + 1)); };

  // block-table entries
  for (int it = 0; it < 200000; ++it) {
    const int np = (int)uni(1, 5000);
    const int page = (int)uni(-20000, 20000) + (it % 7 == 0 ? 0x7fff0000 : 0);
    int err = 0;
    const int r = checked_page<true>(page, np, &err);
    EXPECT(r >= 0 && r < np);
    if (page >= 0 && page < np) EXPECT(r == page && err == 0);
    else EXPECT(r == 0 && err == MLA_DEVERR_PAGE);
    int err2 = 0;
    EXPECT(checked_page<false>(page, np, &err2) == page && err2 == 0);  // release: unchanged
  }
  // slots
  for (int it = 0; it < 200000; ++it) {
    const int np = (int)uni(1, 5000), P = (int)uni(1, 128);
    const long long slot = uni(-3, (long long)np * P + 3) + (it % 11 == 0 ? (1LL << 40) : 0);
    int err = 0;
    const long long r = checked_slot<true>(slot, np, P, &err);
    EXPECT(r >= -1 && r < (long long)np * P);
    if (slot >= -1 && slot < (long long)np * P) EXPECT(r == slot && err == 0);
    else EXPECT(r == -1 && err == MLA_DEVERR_SLOT);
  }
  // prefill offsets: consistent ones pass unchanged, corrupted ones stay in bounds
  for (int it = 0; it < 20000; ++it) {
    const int S = (int)uni(1, 9), P = 64;
    std::vector<int32_t> cq(S + 1), ck(S + 1);
    int max_q = 0, max_kv = 0;
    cq[0] = ck[0] = 0;
    for (int s = 0; s < S; ++s) {
      const int kv = (int)uni(0, 3000), q = (int)uni(0, kv);
      cq[s + 1] = cq[s] + q;
      ck[s + 1] = ck[s] + kv;
      max_q = q > max_q ? q : max_q;
      max_kv = kv > max_kv ? kv : max_kv;
    }
    const int total_q = cq[S], total_kv = ck[S];
    const bool corrupt = it % 2 == 1;
    if (corrupt) {
      const int k = (int)uni(0, 5);
      for (int j = 0; j <= k; ++j) {
        std::vector<int32_t>& v = (rng() & 1) ? cq : ck;
        v[uni(0, S)] = (int32_t)uni(-100000, 100000);
      }
    }
    const int mpps = (max_kv + P - 1) / P + (int)uni(0, 2);
    for (int s = 0; s < S; ++s) {
      int err = 0;
      const PrefillSeq r = prefill_seq<true>(cq.data(), ck.data(), s, total_q, total_kv, max_q, max_kv, &err);
      EXPECT(r.q0 >= 0 && r.q_len >= 0 && r.q0 + r.q_len <= total_q && r.q_len <= max_q);
      EXPECT(r.k0 >= 0 && r.kv_len >= 0 && r.k0 + r.kv_len <= total_kv && r.kv_len <= max_kv);
      EXPECT(r.q_len <= r.kv_len);
      if (!corrupt) {
        EXPECT(err == 0 && r.q0 == cq[s] && r.q_len == cq[s + 1] - cq[s] && r.k0 == ck[s] &&
               r.kv_len == ck[s + 1] - ck[s]);
      }
      // every key row the attention reads, and its block-table entry
      for (int t = 0; t < r.kv_len; t += 97) {
        EXPECT(r.k0 + t < total_kv);
        EXPECT((long long)s * mpps + t / P < (long long)(s + 1) * mpps);
      }
    }
    // key tokens of the up-projection: a search over cu_kv gives some s,
    // the position is clamped so that the entry stays in row s
    if (max_kv >= 1) {
      for (int n = 0; n < total_kv; n += 53) {
        const int s = (int)uni(0, S - 1);
        int err = 0;
        const int t = key_position<true>(n, ck[s], max_kv, &err);
        EXPECT(t >= 0 && t <= max_kv - 1);
        EXPECT((long long)s * mpps + t / P < (long long)(s + 1) * mpps);
        if (!corrupt && n >= ck[s] && n < ck[s + 1]) EXPECT(t == n - ck[s] && err == 0);
      }
    }
  }
  printf("violations %lld cases %lld\n", violations, cases);
  return violations == 0 ? 0 : 1;
}
