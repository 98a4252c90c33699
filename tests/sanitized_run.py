"""Run inside a process that preloads the AddressSanitizer runtime (see
tests/test_sanitizers.py): exercise a sanitized g++ build of the oracle or of
the host block allocator and exit non-zero on any mismatch.

  python tests/sanitized_run.py oracle <liboracle built with sanitizers>
  python tests/sanitized_run.py allocator <allocator library built with sanitizers>
"""
import ctypes
import os
import random
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))


def run_oracle(path):
    import oracle
    import test_oracle

    oracle.use_library(path)
    for pin in test_oracle.PINS:
        pin()
        print("pin ok:", pin.__name__, flush=True)


def run_allocator(path):
    from oracle.allocator import AllocatorModel, CapacityError
    import test_allocator

    lib = ctypes.CDLL(path)
    H, I, P = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    lib.fe_kv_allocator_create.argtypes = [I, I, I, I]
    lib.fe_kv_allocator_create.restype = H
    lib.fe_kv_allocator_destroy.argtypes = [H]
    lib.fe_kv_allocator_append.argtypes = [H, I, I, P]
    lib.fe_kv_allocator_release.argtypes = [H, I]
    lib.fe_kv_allocator_seq_len.argtypes = [H, I]
    lib.fe_kv_allocator_num_allocated.argtypes = [H]
    lib.fe_kv_allocator_num_free.argtypes = [H]
    lib.fe_kv_allocator_batch.argtypes = [H, P, I, P, I, ctypes.c_int32, P]
    for name in ("fe_kv_allocator_append", "fe_kv_allocator_release", "fe_kv_allocator_seq_len",
                 "fe_kv_allocator_num_allocated", "fe_kv_allocator_num_free", "fe_kv_allocator_batch"):
        getattr(lib, name).restype = I
    assert not lib.fe_kv_allocator_create(0, 16, 1, 1)
    assert not lib.fe_kv_allocator_create(1 << 30, 16, 1, 1)

    def append(h, seq, n):
        out = (ctypes.c_int32 * max(n, 1))()
        rc = lib.fe_kv_allocator_append(h, seq, n, out)
        return rc, list(out)[:n]

    rng = random.Random(7)
    h = lib.fe_kv_allocator_create(150, 16, 6, 30)
    m = AllocatorModel(150, 16, 6, 30)
    for step in range(4000):
        seq = rng.randrange(-1, 7)  # out-of-range sequence ids too
        if rng.random() < 0.15:
            rc = lib.fe_kv_allocator_release(h, seq)
            if 0 <= seq < 6:
                m.release(seq)
                assert rc == 0
            else:
                assert rc < 0
        else:
            n = rng.choice([-1, 0, 1, 1, 2, 15, 16, 17, 64, 200])
            rc, slots = append(h, seq, n)
            if not (0 <= seq < 6) or n < 0:
                assert rc < 0, (step, seq, n)
                continue
            try:
                want = m.append(seq, n)
            except CapacityError:
                assert rc == -7, (step, rc)
            else:
                assert rc == 0 and slots == want, step
        assert lib.fe_kv_allocator_num_allocated(h) == m.num_allocated
        if step % 53 == 0:
            seqs = (ctypes.c_int * 6)(*range(6))
            for row_len in (1, 30):
                bt = (ctypes.c_int32 * (6 * row_len))()
                cl = (ctypes.c_int32 * 6)()
                rc = lib.fe_kv_allocator_batch(h, seqs, 6, bt, row_len, 0, cl)
                fits = all(len(b) <= row_len for b in m.blocks)
                assert (rc == 0) == fits, (step, rc)
                if fits:
                    for i in range(6):
                        assert cl[i] == m.length[i]
                        assert list(bt)[i * row_len: i * row_len + len(m.blocks[i])] == m.blocks[i]
    lib.fe_kv_allocator_destroy(h)
    h = lib.fe_kv_allocator_create(400, 16, 4, 32)
    left = test_allocator.serving_run(lambda s, n: append(h, s, n), lambda s: lib.fe_kv_allocator_release(h, s),
                                      lambda: lib.fe_kv_allocator_num_allocated(h))
    assert left == 0
    lib.fe_kv_allocator_destroy(h)
    lib.fe_kv_allocator_destroy(None)
    print("allocator ok", flush=True)


if __name__ == "__main__":
    {"oracle": run_oracle, "allocator": run_allocator}[sys.argv[1]](sys.argv[2])
