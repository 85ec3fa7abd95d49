// Host unit test of the pager's extent allocator (csrc/pw_arena.h): a
// randomized sequence of alloc / grow / shrink / release checked against a
// byte-granular occupancy map.  Prints "ok" and exits 0 on success.
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "pw_arena.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

struct Ext {
  size_t off, len;   // len already rounded
};

int main() {
  const size_t A = 256, S = 1 << 20;
  {
    // fixed cases
    pw::ExtentArena a(S + 100, A);   // size rounds down to the alignment
    CHECK(a.size() == S);
    size_t x = a.alloc(1);
    CHECK(x == 0 && a.used() == A);
    size_t y = a.alloc(3 * A);
    CHECK(y == A && a.used() == 4 * A);
    CHECK(!a.grow(x, A, 2 * A));            // y sits right after x
    CHECK(a.grow(y, 3 * A, 5 * A));         // free space after y
    CHECK(a.used() == 6 * A);
    a.release(y + 2 * A, 3 * A);            // shrink y back to two units
    CHECK(a.used() == 3 * A);
    CHECK(a.free_ranges() == 1);
    a.release(x, A);
    CHECK(a.free_ranges() == 2);
    a.release(y, 2 * A);                    // merges with both neighbours
    CHECK(a.free_ranges() == 1 && a.used() == 0 && a.largest_free() == S);
    CHECK(a.alloc(S + 1) == pw::ExtentArena::kNone);
    CHECK(a.alloc(0) == pw::ExtentArena::kNone);
    CHECK(a.alloc(S) == 0 && a.used() == S && a.free_ranges() == 0);
  }
  {
    // randomized against an occupancy map
    std::mt19937_64 rng(12345);
    pw::ExtentArena a(S, A);
    std::vector<unsigned char> occ(S, 0);
    std::vector<Ext> live;
    size_t used = 0;
    for (int it = 0; it < 20000; ++it) {
      const int op = (int)(rng() % 4);
      if (op == 0 || live.empty()) {
        const size_t n = 1 + rng() % (S / 16);
        const size_t off = a.alloc(n);
        if (off == pw::ExtentArena::kNone) {
          CHECK(a.largest_free() < a.round(n));
          continue;
        }
        const size_t len = a.round(n);
        CHECK(off % A == 0 && off + len <= S);
        for (size_t i = off; i < off + len; ++i) {
          CHECK(occ[i] == 0);
          occ[i] = 1;
        }
        live.push_back({off, len});
        used += len;
      } else if (op == 1) {
        const size_t k = rng() % live.size();
        Ext e = live[k];
        const size_t n = e.len + 1 + rng() % (S / 32);
        const size_t nl = a.round(n);
        const bool room = e.off + nl <= S && [&] {
          for (size_t i = e.off + e.len; i < e.off + nl; ++i)
            if (occ[i]) return false;
          return true;
        }();
        const bool ok = a.grow(e.off, e.len, n);
        CHECK(ok == room);
        if (ok) {
          for (size_t i = e.off + e.len; i < e.off + nl; ++i) occ[i] = 1;
          used += nl - e.len;
          live[k].len = nl;
        }
      } else if (op == 2) {
        const size_t k = rng() % live.size();
        Ext e = live[k];
        if (e.len <= A) continue;
        const size_t keep = A * (1 + rng() % (e.len / A - 1));
        a.release(e.off + keep, e.len - keep);
        for (size_t i = e.off + keep; i < e.off + e.len; ++i) occ[i] = 0;
        used -= e.len - keep;
        live[k].len = keep;
      } else {
        const size_t k = rng() % live.size();
        Ext e = live[k];
        a.release(e.off, e.len);
        for (size_t i = e.off; i < e.off + e.len; ++i) occ[i] = 0;
        used -= e.len;
        live[k] = live.back();
        live.pop_back();
      }
      CHECK(a.used() == used);
    }
    for (const Ext& e : live) a.release(e.off, e.len);
    CHECK(a.used() == 0 && a.free_ranges() == 1 && a.largest_free() == S);
  }
  printf("ok\n");
  return 0;
}
