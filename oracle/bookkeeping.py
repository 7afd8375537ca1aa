"""Oracle bookkeeping of the ConvKV KV memory (integers only; test infrastructure).

Follows the pages' statement of the memory:
  * a recent window of exact KV frames, older frames compressed at a fixed 5:1 ratio into
    a fixed-length long-term memory (news summary "SoulX-LiveAct - Soul App ...", section
    "technical principle", ConvKV Memory bullet; press release digi.china.com, the
    technical-principle paragraph: rolling compression at a fixed ratio);
  * append-only reuse of cached KV, compression once between blocks, blocks 1-2 not
    compressed (walkthrough "SoulX-LiveAct", sections "ConvKV Memory" and "Streaming
    Pipeline");
  * positions reset so they stay bounded (press release: RoPE Reset).

Readings (the pages are silent on them): the memory is a FIFO of groups, each group built
once from r consecutive evicted frames; up to r-1 evicted frames wait as "pending" until
their group is complete and are not attended; reset temporal positions are the ranks in
[reference | memory oldest..newest | window oldest..newest | current].  The reference
segment (walkthrough, "ConvKV Memory": the reference-image part of the context) is a
fixed set of ref_frames frames that every step attends first, so its positions are
always 0..ref_frames-1.
"""


class OracleStateError(Exception):
    pass


class OracleCapacityError(Exception):
    pass


SEG_MEMORY, SEG_WINDOW, SEG_CURRENT, SEG_REF = 0, 1, 2, 3


class Bookkeeping:
    def __init__(self, window_frames, mem_slots, ratio, max_block_frames, ref_frames=0):
        self.ref = ref_frames
        self.W = window_frames
        self.M = mem_slots
        self.r = ratio
        self.B_max = max_block_frames
        self.R = self.W + self.B_max + self.r - 1   # raw slots: pending + window + new block
        self.F = 0          # frames appended
        self.G = 0          # groups compressed
        self.version = 0

    # derived counters
    @property
    def E(self):
        """Frames that have left the window."""
        return max(0, self.F - self.W)

    @property
    def pending(self):
        return self.E - self.r * self.G

    @property
    def win_len(self):
        return self.F - self.E

    @property
    def mem_len(self):
        return min(self.G, self.M)

    def raw_slot(self, f):
        return f % self.R

    def append(self, n):
        """New block of n frames; returns [(absolute frame, raw slot)]."""
        if not 1 <= n <= self.B_max:
            raise OracleCapacityError(f"block of {n} frames, limit {self.B_max}")
        if self.pending >= self.r:
            raise OracleStateError("a complete group is waiting: compress before appending")
        placed = [(f, self.raw_slot(f)) for f in range(self.F, self.F + n)]
        self.F += n
        self.version += 1
        return placed

    def compress(self):
        """Consume every complete group of evicted frames; returns the group ids in order.
        Group g covers frames [r*g, r*g + r) and lands in memory slot g mod M."""
        groups = []
        while self.E - self.r * self.G >= self.r:
            groups.append(self.G)
            self.G += 1
        if groups:
            self.version += 1
        return groups

    def keys(self, n_cur):
        """Key frames in attention order: dicts with segment, slot, id, t_pos."""
        out = [dict(segment=SEG_REF, slot=i, id=i) for i in range(self.ref)]
        if self.M > 0:
            for g in range(max(0, self.G - self.M), self.G):
                out.append(dict(segment=SEG_MEMORY, slot=g % self.M, id=g))
        for f in range(self.E, self.F):
            out.append(dict(segment=SEG_WINDOW, slot=self.raw_slot(f), id=f))
        for i in range(n_cur):
            out.append(dict(segment=SEG_CURRENT, slot=i, id=self.F + i))
        for rank, kf in enumerate(out):
            kf["t_pos"] = rank
        return out

    def state(self):
        return dict(F=self.F, E=self.E, G=self.G, win_len=self.win_len, mem_len=self.mem_len,
                    pending=self.pending, ring_slots=self.R, version=self.version)
