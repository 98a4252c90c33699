"""The paged KV block allocator (host code, no GPU).

The plain model in oracle/allocator.py is pinned by invariants and by the
ForgeEngine README's measurements table (zero allocated KV blocks after an
eight-request workload with six finished and two cancelled requests, at a
concurrency of four); the native allocator in libfe.so must then make
exactly the model's choices on the same seeded call sequences.
"""
import os
import random

import numpy as np
import pytest

from oracle.allocator import AllocatorModel, CapacityError
from paged_kv_gqa_slot_amd import binding

BS = 16


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("libfe.so not built")
    return binding.load_library()


def check_invariants(m: AllocatorModel):
    owned = [b for blocks in m.blocks for b in blocks]
    assert len(owned) == len(set(owned)), "a block is owned twice"
    assert not set(owned) & set(m.free), "a block is both free and owned"
    assert sorted(owned + m.free) == list(range(m.num_blocks)), "blocks lost or invented"
    for blocks, L in zip(m.blocks, m.length):
        assert len(blocks) == -(-L // m.bs), "block count does not match the length"


def serving_run(alloc_append, alloc_release, num_allocated, seed=0):
    """Eight requests, at most four running: each appends its prompt, then one
    token per step until it finishes; requests 2 and 5 are cancelled midway.
    Returns the allocated-block count at the end."""
    rng = random.Random(seed)
    reqs = [dict(id=i, prompt=rng.randint(20, 300), gen=rng.randint(5, 60), cancel_at=(rng.randint(1, 4)
                 if i in (2, 5) else None)) for i in range(8)]
    waiting, running, seq_of = list(reqs), [], {}
    free_seqs = list(range(4))
    finished = cancelled = 0
    while waiting or running:
        while waiting and len(running) < 4:
            r = waiting.pop(0)
            seq = free_seqs.pop(0)
            seq_of[r["id"]] = seq
            alloc_append(seq, r["prompt"])
            r["done"] = 0
            running.append(r)
        for r in list(running):
            seq = seq_of[r["id"]]
            if r["cancel_at"] is not None and r["done"] >= r["cancel_at"]:
                alloc_release(seq)
                cancelled += 1
            elif r["done"] >= r["gen"]:
                alloc_release(seq)
                finished += 1
            else:
                alloc_append(seq, 1)
                r["done"] += 1
                continue
            running.remove(r)
            free_seqs.append(seq)
    assert (finished, cancelled) == (6, 2)
    return num_allocated()


# -- the model ---------------------------------------------------------------------

def test_model_invariants_under_random_calls():
    rng = random.Random(1)
    m = AllocatorModel(200, BS, 8, 40)
    for _ in range(3000):
        seq = rng.randrange(8)
        if rng.random() < 0.2:
            m.release(seq)
        else:
            try:
                slots = m.append(seq, rng.choice([1, 1, 1, 5, 16, 17, 40]))
                assert len(set(slots)) == len(slots)
            except CapacityError:
                pass
        check_invariants(m)


def test_model_slots_follow_blocks():
    m = AllocatorModel(10, BS, 2, 10)
    assert m.append(0, 20) == list(range(0, 20))           # blocks 0, 1 from the top
    assert m.append(1, 3) == [32, 33, 34]                  # block 2
    assert m.append(0, 13) == list(range(20, 32)) + [48]   # fills block 1, then block 3
    m.release(0)                                           # pushes 3, 1, 0: block 0 on top
    assert m.append(1, 14)[-1] == 0 * BS + 0               # block 2 full at 16 tokens: next block is 0
    check_invariants(m)


def test_model_append_is_all_or_nothing():
    m = AllocatorModel(3, BS, 2, 10)
    m.append(0, 40)                                        # 3 blocks
    with pytest.raises(CapacityError):
        m.append(1, 1)
    assert m.length[1] == 0 and m.num_allocated == 3
    m2 = AllocatorModel(10, BS, 1, 2)
    with pytest.raises(CapacityError):
        m2.append(0, 33)                                   # over the 2-block limit
    assert m2.num_allocated == 0


def test_model_serving_run_leaks_nothing():
    """The pages' figure: final allocated KV blocks 0."""
    m = AllocatorModel(400, BS, 4, 32)
    assert serving_run(m.append, m.release, lambda: m.num_allocated) == 0
    check_invariants(m)


class _LeakyModel(AllocatorModel):
    def release(self, seq):  # planted mistake: the last block is not returned
        self.blocks[seq] = self.blocks[seq][:-1]
        super().release(seq)


class _GreedyModel(AllocatorModel):
    def append(self, seq, n):  # planted mistake: a fresh block at every exact block boundary
        if n and self.length[seq] % self.bs == 0 and self.length[seq] and self.free:
            self.blocks[seq].append(self.free.pop())
        return super().append(seq, n)


def test_planted_allocator_mistakes_are_caught():
    m = _LeakyModel(400, BS, 4, 32)
    assert serving_run(m.append, m.release, lambda: m.num_allocated) != 0
    g = _GreedyModel(50, BS, 2, 20)
    g.append(0, 16)
    g.append(0, 1)
    with pytest.raises(AssertionError):
        check_invariants(g)


# -- the native allocator against the model -------------------------------------

def test_native_matches_model(lib):
    rng = random.Random(2)
    a = binding.KVAllocator(150, BS, 6, 30)
    m = AllocatorModel(150, BS, 6, 30)
    for step in range(4000):
        seq = rng.randrange(6)
        if rng.random() < 0.15:
            a.release(seq)
            m.release(seq)
        else:
            n = rng.choice([0, 1, 1, 1, 2, 15, 16, 17, 64, 200])
            try:
                want = m.append(seq, n)
            except CapacityError:
                with pytest.raises(binding.FeError, match="FE_ERR_CAPACITY"):
                    a.append(seq, n)
            else:
                assert a.append(seq, n).tolist() == want, step
        assert a.num_allocated == m.num_allocated and a.num_free == len(m.free)
        assert a.seq_len(seq) == m.length[seq]
        if step % 97 == 0:
            seqs = list(range(6))
            bt, cl = a.batch(seqs, row_len=30, pad_block=0)
            for i, s in enumerate(seqs):
                assert cl[i] == m.length[s]
                assert bt[i, :len(m.blocks[s])].tolist() == m.blocks[s]
                assert np.all(bt[i, len(m.blocks[s]):] == 0)


def test_native_serving_run_leaks_nothing(lib):
    a = binding.KVAllocator(400, BS, 4, 32)
    assert serving_run(a.append, a.release, lambda: a.num_allocated) == 0
    assert a.num_free == 400


def test_native_is_deterministic(lib):
    def run():
        a = binding.KVAllocator(120, BS, 4, 40)
        rng = random.Random(3)
        out = []
        for _ in range(500):
            s = rng.randrange(4)
            if rng.random() < 0.2:
                a.release(s)
            else:
                try:
                    out.append(a.append(s, rng.randint(1, 30)).tolist())
                except binding.FeError:
                    out.append("full")
        return out
    assert run() == run()


def test_native_errors(lib):
    a = binding.KVAllocator(4, BS, 2, 3)
    with pytest.raises(binding.FeError, match="FE_ERR_INVALID_ARG"):
        a.append(2, 1)
    with pytest.raises(binding.FeError, match="FE_ERR_INVALID_ARG"):
        a.append(0, -1)
    with pytest.raises(binding.FeError, match="FE_ERR_CAPACITY"):
        a.append(0, 49)                      # above the 3-block limit of a sequence
    assert a.seq_len(0) == 0 and a.num_allocated == 0
    a.append(0, 48)
    a.append(1, 10)
    with pytest.raises(binding.FeError, match="FE_ERR_CAPACITY"):
        a.append(1, 7)                       # needs a 5th block
    assert a.seq_len(1) == 10
    with pytest.raises(binding.FeError, match="FE_ERR_CAPACITY"):
        a.batch([0], row_len=2)              # 3 blocks do not fit a row of 2
    a.release(1)
    a.release(1)                             # releasing an empty sequence is a no-op
    assert a.num_allocated == 3
    with pytest.raises(ValueError):
        binding.KVAllocator(0, BS, 1, 1)
