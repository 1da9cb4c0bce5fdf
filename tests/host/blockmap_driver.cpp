// Host build of the block map of the fused cache write + absorption launch
// (wa_role, wa_grid in mla_checks.h): for every slice count, feature-block
// count, head count and CU count the host can form, the grid must hold each
// write tile (fb, s) exactly once, the absorption ranks must be 0 ..
// n_ablocks - 1 exactly once, every head must fall to one rank, and no rank
// may take more than two heads.  Prints "violations N cases M".
#include <stdio.h>

#include <vector>

#include "../../mla_latent_kv_22_amd/csrc/mla_checks.h"

using namespace mla;

int main() {
  long long violations = 0, cases = 0;
  auto expect = [&](bool c, int S, int nfb, int H, int cus, const char* what) {
    ++cases;
    if (!c) {
      if (violations < 20) fprintf(stderr, "S=%d nfb=%d H=%d cus=%d: %s\n", S, nfb, H, cus, what);
      ++violations;
    }
  };
  const int heads[] = {1, 2, 3, 16, 40, 64, 127, 128};
  const int cuss[] = {1, 8, 64, 80, 120, 256, 304};
  for (int S = 1; S <= 16; ++S)
    for (int nfb = 1; nfb <= 64; ++nfb)
      for (int H : heads)
        for (int cus : cuss) {
          // the host's choice before the grid rule (k_project_mfma.hip)
          int na = cus - nfb * S;
          if (na > H) na = H;
          if (na < (H + 1) / 2) na = (H + 1) / 2;
          const int grid = wa_grid(S, nfb, na);
          expect(na >= (H + 1) / 2 && grid == nfb * S + na, S, nfb, H, cus, "grid size");
          std::vector<int> tile(nfb * S, 0), rank(na, 0), head(H, 0);
          for (int x = 0; x < grid; ++x) {
            const WaRole r = wa_role(x, S, nfb);
            if (r.write) {
              const bool ok = r.fb >= 0 && r.fb < nfb && r.s >= 0 && r.s < S;
              expect(ok, S, nfb, H, cus, "write tile in range");
              if (ok) ++tile[r.s * nfb + r.fb];
            } else {
              const bool ok = r.rank >= 0 && r.rank < na;
              expect(ok, S, nfb, H, cus, "rank in range");
              if (!ok) continue;
              ++rank[r.rank];
              int taken = 0;
              for (int h = r.rank; h < H; h += na, ++taken) ++head[h];
              expect(taken <= 2, S, nfb, H, cus, "at most two heads");
            }
          }
          for (int v : tile) expect(v == 1, S, nfb, H, cus, "each write tile once");
          for (int v : rank) expect(v == 1, S, nfb, H, cus, "each rank once");
          for (int v : head) expect(v == 1, S, nfb, H, cus, "each head once");
        }
  printf("violations %lld cases %lld\n", violations, cases);
  return violations == 0 ? 0 : 1;
}
