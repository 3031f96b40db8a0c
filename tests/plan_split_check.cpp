// Host check of the key-axis split in the work plan (plan.h, compiled by the
// host compiler alone): for each plan given on the command line, every unit
// of every die's claim sequence is taken exactly once, the units decode to
// every (item, part) of the split items and to every other item exactly once,
// the parts of an item partition its key tiles, and the split items are the
// last items of the long group (entries with a predecessor) when there is one.
// Prints "ok" and exits 0, or prints the first violation and exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "plan.h"

using namespace chunkattn;

static int fail(const char* what, long long a, long long b) {
  std::printf("FAIL %s %lld %lld\n", what, a, b);
  return 1;
}

static int check(int n, int first_pred, int heads, int lq, int lown, int lpred, int bm, int n_xcd,
                 long long n_split, int parts) {
  Plan p = make_plan(n, first_pred, heads, lq, lown, lpred, bm, n_xcd);
  p = plan_with_split(p, n_split, parts);
  const long long n_items = p.n_items;
  const long long group_end = p.n_items_pred > 0 ? p.n_items_pred : n_items;
  const long long cnt = n_split < group_end ? n_split : group_end;
  if (parts >= 2 && cnt > 0) {
    if (p.split_count != cnt) return fail("split_count", p.split_count, cnt);
    if (p.split_from != group_end - cnt) return fail("split_from", p.split_from, group_end - cnt);
    if (p.n_units != n_items + cnt * (parts - 1)) return fail("n_units", p.n_units, n_items);
  } else if (p.n_units != n_items) {
    return fail("unsplit n_units", p.n_units, n_items);
  }
  // claims: every die drains its queue, then steals from the others in turn
  std::vector<int> unit_seen((size_t)p.n_units, 0);
  for (int x = 0; x < p.n_xcd; ++x) {
    for (unsigned long long old = 0;; ++old) {
      const long long u = claim_word_unit(p, x, old);
      if (u < 0) break;
      if (u >= p.n_units) return fail("unit range", u, p.n_units);
      if (unit_seen[(size_t)u]++) return fail("unit claimed twice", u, x);
    }
  }
  for (long long u = 0; u < p.n_units; ++u)
    if (!unit_seen[(size_t)u]) return fail("unit never claimed", u, 0);
  // decode: (item, part) coverage and tile ranges
  std::vector<int> whole(n_items, 0);
  std::vector<std::vector<int>> tiles(n_items);
  for (long long u = 0; u < p.n_units; ++u) {
    const Item it = decode_unit(p, u);
    // find the item index of this unit from its fields
    long long idx = -1;
    for (long long w = 0; w < n_items; ++w) {
      const Item ref = decode(p, w);
      if (ref.b == it.b && ref.h == it.h && ref.q0 == it.q0) { idx = w; break; }
    }
    if (idx < 0) return fail("unit decodes to no item", u, 0);
    const Item ref = decode(p, idx);
    const int T = ref.t_hi;
    if (it.part < 0) {
      if (it.t_lo != 0 || it.t_hi != T) return fail("whole item tiles", u, it.t_hi);
      if (whole[idx]++) return fail("item twice", idx, u);
      if (idx >= p.split_from && idx < p.split_from + p.split_count)
        return fail("split item run whole", idx, u);
    } else {
      if (idx < p.split_from || idx >= p.split_from + p.split_count)
        return fail("unsplit item cut", idx, u);
      if (it.split_idx != idx - p.split_from) return fail("split_idx", it.split_idx, idx);
      auto& tv = tiles[idx];
      if (tv.empty()) tv.assign((size_t)T, 0);
      if (it.t_lo >= it.t_hi) return fail("empty part", idx, it.part);
      for (int t = it.t_lo; t < it.t_hi; ++t)
        if (tv[(size_t)t]++) return fail("tile in two parts", idx, t);
    }
  }
  for (long long w = 0; w < n_items; ++w) {
    const bool split = w >= p.split_from && w < p.split_from + p.split_count;
    if (!split && whole[w] != 1) return fail("item missing", w, whole[w]);
    if (split)
      for (size_t t = 0; t < tiles[w].size(); ++t)
        if (tiles[w][t] != 1) return fail("tile missing", w, (long long)t);
    if (split && tiles[w].empty()) return fail("split item missing", w, 0);
  }
  return 0;
}

int main(int argc, char** argv) {
  // each case: n first_pred heads lq lown lpred bm n_xcd n_split parts
  if ((argc - 1) % 10 != 0) return 2;
  for (int i = 1; i + 9 < argc; i += 10) {
    int v[10];
    for (int k = 0; k < 10; ++k) v[k] = std::atoi(argv[i + k]);
    if (check(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], v[8], v[9])) return 1;
  }
  std::printf("ok\n");
  return 0;
}
