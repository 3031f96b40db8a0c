// Integer work plan of the chunk-attention launch: which (chunk, head, query
// tile) each workgroup computes, and which key/value rows it walks.
//
// One work item = one (batch item b, head h, query tile t) with query rows
// [t*BM, min(Lq, (t+1)*BM)).  Its logical key/value rows are [0, pred + own):
// logical row j < pred reads the predecessor segment (the cached K/V of the
// chunk processed just before, DualParal write-up section 三), j >= pred reads
// row j - pred of the item's own K/V.  Nothing is concatenated in memory.
//
// The last batch entry may have fewer query and own rows than the others
// (lq_last, lown_last): the last window of a window step has no next chunk.
//
// Order.  Items of batch entries that have a predecessor (chunks 1..n-1 of a
// queue step) come first, because they walk the most key rows; entries without
// one (chunk 0) fill the tail of the launch.  Within a group the order is
// (b, h, t) with t fastest, so consecutive items share one chunk/head's K/V.
// A plan of one group whose entries are all the same size may run its items
// head-major instead, (h, b, t) (plan_head_major): when every entry attends
// over one shared K/V (per-chunk cross-attention to the text tokens), the
// items a die runs at one time then read one head's K/V rather than one per
// concurrent (b, h).  The work index, which decode() takes, stays (b, h, t);
// plan_slot_work() maps launch positions onto it in the plan's order.
//
// Die-aware launch order.  Workgroup ids are handed to the accelerator dies
// round-robin (id % n_xcd), and each die runs its own ids in increasing order.
// slot_to_work() renumbers so that every die gets an equal share of the long
// items (those with a predecessor) and an equal share of the short ones, each
// share a contiguous range of the work order, long share first.  The query
// tiles of one (chunk, head) then run together on one die and share that die's
// L2 copy of the K/V tiles, and all dies walk about the same number of key
// rows (one contiguous range per die would leave the short items of chunk 0
// to the last die, which then idles for half the launch).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define CA_HD __host__ __device__ __forceinline__
#else
#define CA_HD inline
#endif

namespace chunkattn {

struct Plan {
  int n_batch;     // chunks (queue step) or batch items (full attention)
  int first_pred;  // batch entries b >= first_pred have a predecessor segment
  int heads;
  int lq;          // query rows per batch entry
  int lown;        // own key/value rows per batch entry
  int lpred;       // predecessor rows (entries b >= first_pred)
  int bm;          // query rows per work item
  int n_qtiles;    // ceil(lq / bm)
  int lq_last;     // query rows of the last entry (b = n_batch - 1)
  int lown_last;   // own key/value rows of the last entry
  int n_qtiles_last;
  int n_xcd;       // dies for the launch-order renumbering (>= 1)
  int64_t n_items;
  int64_t n_items_pred;  // items of entries with a predecessor (scheduled first)
  // Key-axis split (split_parts = 1: none).  Items [split_from, split_from +
  // split_count) of the work order are each cut into split_parts units along
  // their key tiles; the launch runs n_units units.
  int64_t split_from;
  int split_parts;
  int64_t n_units;
  int64_t split_count;
  int head_major;  // 1: items run in (h, b, t) order (plan_head_major)
};

struct Item {
  int b, h, q0, q_rows, pred_rows, own_rows;
  // key tiles [t_lo, t_hi) of the item's walk; part >= 0 for a unit of a
  // split item (split_idx: its index among the split items), -1 otherwise
  int t_lo, t_hi, part, split_idx;
};

CA_HD Plan make_plan(int n_batch, int first_pred, int heads, int lq, int lown, int lpred,
                     int bm, int n_xcd, int lq_last, int lown_last) {
  Plan p;
  p.n_batch = n_batch;
  p.first_pred = first_pred < n_batch ? first_pred : n_batch;
  p.heads = heads;
  p.lq = lq;
  p.lown = lown;
  p.lpred = lpred;
  p.bm = bm;
  p.n_qtiles = (lq + bm - 1) / bm;
  p.lq_last = lq_last;
  p.lown_last = lown_last;
  p.n_qtiles_last = (lq_last + bm - 1) / bm;
  p.n_xcd = n_xcd < 1 ? 1 : n_xcd;
  const int64_t per_entry = (int64_t)heads * p.n_qtiles;
  const int64_t per_last = (int64_t)heads * p.n_qtiles_last;
  p.n_items = n_batch > 0 ? (int64_t)(n_batch - 1) * per_entry + per_last : 0;
  const int n_pred = n_batch - p.first_pred;  // the last entry is among them if n_pred > 0
  p.n_items_pred = n_pred > 0 ? (int64_t)(n_pred - 1) * per_entry + per_last : 0;
  p.split_from = p.n_items;
  p.split_parts = 1;
  p.n_units = p.n_items;
  p.split_count = 0;
  p.head_major = 0;
  return p;
}

// The same plan run head-major when it has one group (no predecessor
// segments), every entry the same size and fewer than 2^31 items (the order
// map divides in 32 bits); otherwise unchanged.
CA_HD Plan plan_head_major(Plan p) {
  if (p.first_pred >= p.n_batch && p.lq_last == p.lq && p.lown_last == p.lown &&
      p.n_items <= 0x7fffffff)
    p.head_major = 1;
  return p;
}

// The same plan with n_split items cut into `parts` units each along the key
// axis: the last n_split items of the long group (entries with a
// predecessor) when the plan has one, else the last n_split of the work order.
// The short items then stay whole: they cost a fraction of a long item and
// fill the end of the launch better than quarter units of themselves, whose
// start and finish would weigh as much as their few tiles.
CA_HD Plan plan_with_split(Plan p, int64_t n_split, int parts) {
  const int64_t group_end = p.n_items_pred > 0 ? p.n_items_pred : p.n_items;
  if (n_split > group_end) n_split = group_end;
  if (parts < 2 || n_split <= 0) return p;
  p.head_major = 0;  // a split plan claims units in (b, h, t) order
  p.split_from = group_end - n_split;
  p.split_count = n_split;
  p.split_parts = parts;
  p.n_units = p.n_items + n_split * (parts - 1);
  return p;
}
// Every entry the same size.
CA_HD Plan make_plan(int n_batch, int first_pred, int heads, int lq, int lown, int lpred,
                     int bm, int n_xcd) {
  return make_plan(n_batch, first_pred, heads, lq, lown, lpred, bm, n_xcd, lq, lown);
}

// First index of die x's share when m items are split over n_xcd dies as
// evenly as possible (the first m % n_xcd dies take one more).
CA_HD int64_t die_share_start(int64_t m, int64_t x, int n_xcd) {
  const int64_t per = m / n_xcd, extra = m % n_xcd;
  return x * per + (x < extra ? x : extra);
}

// Launch slot (workgroup id) -> work index, a bijection on [0, n).  Work
// indices [0, n_first) are the long items, [n_first, n) the short ones.  Die x
// (= slot % n_xcd) owns the slots x, x + n_xcd, ...; the first F_x of them take
// its share of the long items and the rest a contiguous range of short items.
// The short count of a die, S_x - F_x, is never negative: S_x and F_x are
// even splits of n >= n_first.
CA_HD int64_t slot_to_work(int64_t slot, int64_t n, int64_t n_first, int n_xcd) {
  if (n_xcd <= 1) return slot;
  const int64_t x = slot % n_xcd, local = slot / n_xcd;
  const int64_t s0 = die_share_start(n, x, n_xcd);
  const int64_t f0 = die_share_start(n_first, x, n_xcd);
  const int64_t fx = die_share_start(n_first, x + 1, n_xcd) - f0;
  if (local < fx) return f0 + local;
  return n_first + (s0 - f0) + (local - fx);
}

// The work index of launch slot `slot` under plan p.  A head-major plan
// places position o = (h * n_batch + b) * n_qtiles + t of its order at work
// index (b * heads + h) * n_qtiles + t.
CA_HD int64_t plan_slot_work(const Plan& p, int64_t slot) {
  const int64_t o = slot_to_work(slot, p.n_items, p.n_items_pred, p.n_xcd);
  if (!p.head_major) return o;
  const uint32_t nq = (uint32_t)p.n_qtiles;
  const uint32_t per_head = (uint32_t)p.n_batch * nq;
  const uint32_t h = (uint32_t)o / per_head;
  const uint32_t bt = (uint32_t)o - h * per_head;  // b * n_qtiles + t
  const uint32_t b = bt / nq;
  return ((int64_t)b * p.heads + h) * nq + (bt - b * nq);
}

// Persistent launch: each die x owns the work of its launch slots
// x, x + n_xcd, ... (count die_share_start(n, x+1) - die_share_start(n, x)) as
// a queue, longest items first.  Its claim word counts the claims made on it,
// by its own workgroups and, once theirs is used up, by other dies'.  `old` is
// the word's value before this claim added 1: the claim gets queue position
// old while old < count, so every item is taken exactly once, and -1 once the
// queue is used up.  Taking stolen items from the front too keeps each die's
// short items for the end of the launch, where they even out the finish.
CA_HD int64_t claim_word_item(const Plan& p, int x, unsigned long long old) {
  const int64_t count = die_share_start(p.n_items, x + 1, p.n_xcd) -
                        die_share_start(p.n_items, x, p.n_xcd);
  if ((int64_t)old >= count) return -1;
  return plan_slot_work(p, x + (int64_t)old * p.n_xcd);
}

CA_HD Item decode(const Plan& p, int64_t w) {
  // group: entries [first_pred, n_batch) first, then [0, first_pred)
  int64_t idx = w;
  int b0 = p.first_pred, count = p.n_batch - p.first_pred;
  if (w >= p.n_items_pred) {
    idx = w - p.n_items_pred;
    b0 = 0;
    count = p.first_pred;
  }
  // the group's entries are regular except the last entry of the queue
  const int regular = b0 + count == p.n_batch ? count - 1 : count;
  const int64_t per_entry = (int64_t)p.heads * p.n_qtiles;
  int64_t b, rem;
  int nq, lq, lown;
  if (idx < (int64_t)regular * per_entry) {
    b = b0 + idx / per_entry;
    rem = idx % per_entry;
    nq = p.n_qtiles;
    lq = p.lq;
    lown = p.lown;
  } else {
    b = p.n_batch - 1;
    rem = idx - (int64_t)regular * per_entry;
    nq = p.n_qtiles_last;
    lq = p.lq_last;
    lown = p.lown_last;
  }
  Item it;
  it.b = (int)b;
  it.h = (int)(rem / nq);
  const int t = (int)(rem % nq);
  it.q0 = t * p.bm;
  const int left = lq - it.q0;
  it.q_rows = left < p.bm ? left : p.bm;
  it.pred_rows = b >= p.first_pred ? p.lpred : 0;
  it.own_rows = lown;
  it.t_lo = 0;
  it.t_hi = (it.pred_rows + it.own_rows + 63) / 64;
  it.part = -1;
  it.split_idx = -1;
  return it;
}

// Work unit u of a plan with a key-axis split: units [0, split_from) are the
// items themselves; unit split_from + s (s < split_count * split_parts) is
// part s % split_parts of item split_from + s / split_parts, whose key tiles
// [T*part/parts, T*(part+1)/parts) it walks (T: the item's tiles); the units
// after those are the items after the split range, whole.
CA_HD Item decode_unit(const Plan& p, int64_t u) {
  if (u < p.split_from) return decode(p, u);
  const int64_t s = u - p.split_from;
  const int64_t su = p.split_count * p.split_parts;
  if (s >= su) return decode(p, p.split_from + p.split_count + (s - su));
  Item it = decode(p, p.split_from + s / p.split_parts);
  const int part = (int)(s % p.split_parts);
  const int t = it.t_hi;
  it.t_lo = (int)((int64_t)t * part / p.split_parts);
  it.t_hi = (int)((int64_t)t * (part + 1) / p.split_parts);
  it.part = part;
  it.split_idx = (int)(s / p.split_parts);
  return it;
}

// Persistent claim over units.  Without a split it is claim_word_item.  With
// one, die x's queue holds its even share of the unsplit long items, then of
// the unsplit short items before the split range and after it, then of the
// split units (each a contiguous range of units), so the small units come
// last on every die.
CA_HD int64_t claim_word_unit(const Plan& p, int x, unsigned long long old) {
  if (p.split_parts <= 1) return claim_word_item(p, x, old);
  const int64_t a = p.n_items_pred < p.split_from ? p.n_items_pred : p.split_from;
  const int64_t su_end = p.split_from + p.split_count * p.split_parts;
  const int64_t sizes[4] = {a, p.split_from - a, p.n_units - su_end, su_end - p.split_from};
  const int64_t starts[4] = {0, a, su_end, p.split_from};
  int64_t pos = (int64_t)old;
  for (int k = 0; k < 4; ++k) {
    const int64_t s0 = die_share_start(sizes[k], x, p.n_xcd);
    const int64_t cnt = die_share_start(sizes[k], x + 1, p.n_xcd) - s0;
    if (pos < cnt) return starts[k] + s0 + pos;
    pos -= cnt;
  }
  return -1;
}

}  // namespace chunkattn
