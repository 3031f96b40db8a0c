// Host-side bookkeeping of the streaming chunk queue (DualParal write-up,
// section 二): chunks of frames in a first-in-first-out queue, noise falling
// from the tail to the head; every diffusion step processes all live chunks
// (tail first), a new noisy chunk joins at the tail and the clean chunk at the
// head leaves, so each chunk spends exactly `depth` steps in the queue and the
// video can grow without bound.
//
// Storage is a ring of `slots` chunk buffers owned by the caller: chunk number
// g (in order of arrival) lives in slot g mod slots, so nothing is ever copied
// when the queue advances; slots >= depth keeps live chunks in distinct slots.
// With the live chunks in processing order (c = 0 the tail, the newest),
// chunk c is in slot (tail - c) mod slots and its predecessor c-1 (processed
// just before it) in the next slot up, which the attention kernel reads in
// place.
#pragma once

#include <stdint.h>

#include <deque>

namespace chunkattn {

class Fifo {
 public:
  Fifo(int slots, int depth) : slots_(slots), depth_(depth) {}

  int slots() const { return slots_; }
  int depth() const { return depth_; }
  int live() const { return (int)queue_.size(); }
  int64_t next_id() const { return next_id_; }
  bool full() const { return (int)queue_.size() == depth_; }
  bool head_clean() const { return !queue_.empty() && queue_.front().done >= depth_; }
  int slot_of(int64_t id) const { return (int)(id % slots_); }
  // slot of the tail (newest chunk); the queue must not be empty
  int tail_slot() const { return slot_of(queue_.back().id); }

  // A new chunk joins at the tail; returns its slot.  The queue must not be full.
  int push() {
    queue_.push_back(Rec{next_id_, 0});
    return slot_of(next_id_++);
  }
  // Every live chunk has done one more step.
  void advance() {
    for (Rec& r : queue_) ++r.done;
  }
  // The clean head leaves; returns its slot.  head_clean() must hold.
  int pop() {
    const int s = slot_of(queue_.front().id);
    queue_.pop_front();
    return s;
  }
  // Live chunk c in processing order (0 = tail): number, slot, steps done.
  void at(int c, int64_t* id, int* slot, int* done) const {
    const Rec& r = queue_[queue_.size() - 1 - (size_t)c];
    *id = r.id;
    *slot = slot_of(r.id);
    *done = r.done;
  }

 private:
  struct Rec {
    int64_t id;
    int done;
  };
  int slots_, depth_;
  int64_t next_id_ = 0;
  std::deque<Rec> queue_;  // head at the front
};

}  // namespace chunkattn
