"""The rolling frame-window KV cache, modelled frame by frame (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: frames are generated and evicted in a sliding window, and every layer
reads and writes a rolling KV cache ("Amazon and Reactor tune Trainium for
real-time video generation", section "Three problems for generic compilers";
the yomu.fyi digest "A kernel-centric path to real-time video generation on
Trainium", FAQ on the Rolling Forcing model).  The pages give no data
structure; the reading here is a ring of ``W`` frame slots:

* frame ``t`` (absolute latent frame index) lives in slot ``t mod W``;
* the valid window is frames ``first .. first+count-1``;
* ``roll(t0, n)`` writes frames ``t0 .. t0+n-1`` and needs
  ``first <= t0 <= first+count`` and ``1 <= n <= W``.  A frame already in the
  window is overwritten in place; a later one is appended, and an append to
  a full ring evicts the oldest frame (whose slot is the one being written);
* slots that are not written keep their contents.

The model keeps, per slot, the frame index last written there and the raw
(un-rotated) data the caller handed in, so tests can build the expected ring
contents with ``rope3d.rope_spec_bits``.
"""


class RingError(ValueError):
    pass


class RingModel:
    def __init__(self, capacity):
        if capacity < 1:
            raise RingError("capacity must be >= 1")
        self.capacity = capacity
        self.first = 0
        self.count = 0
        self.slot_frame = [None] * capacity   # frame index last written to each slot
        self.slot_data = [None] * capacity    # caller data of that write

    def slot(self, t):
        return t % self.capacity

    def window(self):
        return list(range(self.first, self.first + self.count))

    def check_roll(self, t0, n):
        if not (1 <= n <= self.capacity):
            raise RingError("n must be in 1..capacity")
        if self.count == 0:
            return
        if not (self.first <= t0 <= self.first + self.count):
            raise RingError("t0 must lie in first..first+count")

    def roll(self, t0, n, data=None):
        """Write frames t0..t0+n-1; ``data`` is a list of n per-frame payloads.

        Returns the list of evicted frame indices.  An empty ring accepts any
        ``t0`` and starts its window there.
        """
        self.check_roll(t0, n)
        if self.count == 0:
            self.first = t0
        evicted = []
        for i in range(n):
            t = t0 + i
            if t >= self.first + self.count:          # append
                if self.count == self.capacity:
                    evicted.append(self.first)
                    self.first += 1
                else:
                    self.count += 1
            s = self.slot(t)
            self.slot_frame[s] = t
            self.slot_data[s] = None if data is None else data[i]
        return evicted

    def contains(self, t0, n):
        """True when frames t0..t0+n-1 all lie in the valid window."""
        return n >= 1 and self.first <= t0 and t0 + n <= self.first + self.count
