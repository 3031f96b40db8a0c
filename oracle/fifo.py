"""Plain simulation of the DualParal chunk queue (TEST INFRASTRUCTURE).

Follows "双重并行：让AI视频生成突破时长限制" (techwalker write-up of DualParal),
section 二: chunks of frames sit in a first-in-first-out queue with noise
decreasing from the tail to the head; every diffusion step processes all of
them (tail first), then a new noisy chunk joins at the tail and the clean chunk
at the head leaves, so a chunk spends exactly `depth` steps in the queue (one
per noise level) and the video can grow without bound.

Bookkeeping used with a ring of `slots` buffers: chunk number g (0, 1, 2, ...
in order of arrival) lives in slot g mod slots; slots >= depth keeps the live
chunks in distinct slots.  Listing the live chunks in processing order
(c = 0 the tail, the newest), chunk c is in slot (tail - c) mod slots.

Only the tests import this module.
"""
from collections import deque


class Fifo:
    def __init__(self, slots: int, depth: int):
        if depth < 1 or slots < depth:
            raise ValueError("need depth >= 1 and slots >= depth")
        self.slots = slots
        self.depth = depth
        self.next_id = 0          # number of the next chunk to arrive
        self.queue = deque()      # [chunk number, steps done], head on the left

    def push(self) -> int:
        """A new noisy chunk joins at the tail; returns its slot."""
        if len(self.queue) == self.depth:
            raise ValueError("queue full")
        g = self.next_id
        self.next_id += 1
        self.queue.append([g, 0])
        return g % self.slots

    def step(self) -> None:
        """One diffusion step over every live chunk."""
        if not self.queue:
            raise ValueError("queue empty")
        for rec in self.queue:
            rec[1] += 1

    def pop(self) -> int:
        """The clean chunk leaves at the head; returns its slot."""
        if not self.queue or self.queue[0][1] < self.depth:
            raise ValueError("head not clean")
        g, _ = self.queue.popleft()
        return g % self.slots

    def live(self):
        """(chunk number, slot, steps done) of the live chunks, tail first."""
        return [(g, g % self.slots, done) for g, done in reversed(self.queue)]

    def tail_slot(self) -> int:
        return self.queue[-1][0] % self.slots


def run(total: int, slots: int, depth: int):
    """The whole schedule for a video of `total` chunks: each step pushes the
    next chunk while any are left, processes the queue and lets a clean head
    leave.  Returns one record per step: (pushed slot or -1, live list before
    the step's processing, popped slot or -1)."""
    f = Fifo(slots, depth)
    out = []
    while f.next_id < total or f.queue:
        pushed = f.push() if f.next_id < total else -1
        live = f.live()
        f.step()
        popped = f.pop() if f.queue and f.queue[0][1] == depth else -1
        out.append((pushed, live, popped))
    return out
