// Host check of the key-axis split in the work plan (plan.h, compiled by the
// host compiler alone): for each plan given on the command line, the work
// indices decode to every (entry, head, query tile) exactly once, the launch
// slots map onto the work indices one to one, each die's slots taking a
// contiguous run of the plan's order (head-major when asked, the plan allows
// it and has no split), every unit of every die's claim sequence is taken
// exactly once, the units decode to every (item, part) of the split
// items and to every other item exactly once, the parts of an item partition
// its key tiles, and the split items are the last items of the long group
// (entries with a predecessor) when there is one.
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
                 long long n_split, int parts, int head_major) {
  Plan p = make_plan(n, first_pred, heads, lq, lown, lpred, bm, n_xcd);
  if (head_major) p = plan_head_major(p);
  const int allowed = first_pred >= n;  // one group; entries are equal here
  if (p.head_major != (head_major && allowed)) return fail("head_major", p.head_major, allowed);
  p = plan_with_split(p, n_split, parts);
  const long long n_items = p.n_items;
  const long long group_end = p.n_items_pred > 0 ? p.n_items_pred : n_items;
  const long long cnt = n_split < group_end ? n_split : group_end;
  const bool split = parts >= 2 && cnt > 0;
  if (split && p.head_major) return fail("split plan left head-major", cnt, parts);
  const int nq = (lq + bm - 1) / bm;
  // items: work index w decodes to (entry, head, tile) with w = (b*heads + h)*nq + t
  if (n_items != (long long)n * heads * nq) return fail("n_items", n_items, 0);
  for (long long w = 0; w < n_items; ++w) {
    const Item it = decode(p, w);
    if (it.b < 0 || it.b >= n || it.h < 0 || it.h >= heads || it.q0 % bm || it.q0 >= lq)
      return fail("item out of range", w, it.b);
    const int t = it.q0 / bm;
    if (it.q_rows != (lq - it.q0 < bm ? lq - it.q0 : bm)) return fail("q_rows", w, it.q_rows);
    if (it.pred_rows != (it.b >= first_pred ? lpred : 0)) return fail("pred_rows", w, it.b);
    if (it.own_rows != lown) return fail("own_rows", w, it.own_rows);
    // one group: the plain (b, h, t) index; two: long group (b >= first_pred) first
    if (allowed && w != ((long long)it.b * heads + it.h) * nq + t) return fail("work index", w, it.b);
  }
  // launch slots: a bijection onto the work indices; with one group, each die's
  // slots x, x + n_xcd, ... take a contiguous run of the plan's order
  // ((h, b, t) when head-major, else (b, h, t))
  {
    std::vector<int> seen((size_t)n_items, 0);
    std::vector<long long> last((size_t)p.n_xcd, -1);
    for (long long slot = 0; slot < n_items; ++slot) {
      const long long w = plan_slot_work(p, slot);
      if (w < 0 || w >= n_items) return fail("slot work range", slot, w);
      if (seen[(size_t)w]++) return fail("slot work twice", slot, w);
      if (!allowed) continue;
      const Item it = decode(p, w);
      const long long o = p.head_major ? ((long long)it.h * n + it.b) * nq + it.q0 / bm
                                       : w;
      const int x = (int)(slot % p.n_xcd);
      if (last[(size_t)x] >= 0 && o != last[(size_t)x] + 1) return fail("die order", slot, o);
      last[(size_t)x] = o;
    }
  }
  if (split) {
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
  // each case: n first_pred heads lq lown lpred bm n_xcd n_split parts head_major
  if ((argc - 1) % 11 != 0) return 2;
  for (int i = 1; i + 10 < argc; i += 11) {
    int v[11];
    for (int k = 0; k < 11; ++k) v[k] = std::atoi(argv[i + k]);
    if (check(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], v[8], v[9], v[10])) return 1;
  }
  std::printf("ok\n");
  return 0;
}
