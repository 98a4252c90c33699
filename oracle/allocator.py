"""Plain model of the paged KV block allocator -- TEST INFRASTRUCTURE.

Only tests/ may use it.  It restates the allocator's contract with Python
lists, for comparison with the native allocator on the same calls:

* ForgeEngine README, "What it implements": the KV cache is a paged block
  allocator with deterministic cleanup; "Loading": one worker owns KV-cache
  mutation; measurements table: zero allocated KV blocks after a workload of
  eight requests, six finished and two cancelled.
* Readings (the pages give no algorithm): free blocks form a stack, 0 on top
  at the start; a sequence's new tokens take the blocks they need from the
  top, in order; releasing a sequence puts its blocks back in reverse token
  order; token t of a sequence lives at slot blocks[t // BS] * BS + t % BS;
  an append that does not fit changes nothing.
"""


class CapacityError(Exception):
    pass


class AllocatorModel:
    def __init__(self, num_blocks, block_size, max_seqs, max_blocks_per_seq):
        self.bs = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.num_blocks = num_blocks
        self.free = list(range(num_blocks - 1, -1, -1))  # last element = top = block 0
        self.blocks = [[] for _ in range(max_seqs)]
        self.length = [0] * max_seqs

    def append(self, seq, n):
        """Slots of n new tokens of seq, or CapacityError (nothing changes)."""
        old, new = self.length[seq], self.length[seq] + n
        if new > self.max_blocks_per_seq * self.bs:
            raise CapacityError("sequence block limit")
        need = -(-new // self.bs) - (-(-old // self.bs))
        if need > len(self.free):
            raise CapacityError("free blocks")
        for _ in range(need):
            self.blocks[seq].append(self.free.pop())
        self.length[seq] = new
        return [self.blocks[seq][t // self.bs] * self.bs + t % self.bs for t in range(old, new)]

    def release(self, seq):
        for b in reversed(self.blocks[seq]):
            self.free.append(b)
        self.blocks[seq] = []
        self.length[seq] = 0

    @property
    def num_allocated(self):
        return self.num_blocks - len(self.free)
