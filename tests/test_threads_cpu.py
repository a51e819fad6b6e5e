"""rope_last_error is per thread: concurrent calls that fail different
checks each read back their own message (the header documents the text as
that of the last non-OK status on the calling thread). No GPU is used: the
calls fail validation before any HIP call."""
import threading

import transformer_positional_encoding_amd as rp

FAKE = 0x10000
TS, TT = (1, 4, 1, 32), (128, 32, 32, 1)

CASES = [
    # (x_shape, slice, x pointer, expected status, expected message)
    ((2, 4, 3, 63), (0, 32), FAKE, rp.ROPE_ERR_INVALID, "D must be even"),
    ((2, 4, 3, 2048), (0, 32), FAKE, rp.ROPE_ERR_INVALID, "D exceeds 1024"),
    ((2, 4, 3, 64), (0, 32), None, rp.ROPE_ERR_NULLPTR, "x is NULL"),
    ((2, 4, 3, 64), (0, 31), FAKE, rp.ROPE_ERR_INVALID, "slice length end-start must be even"),
]


def test_last_error_is_per_thread():
    errors = []
    start = threading.Barrier(len(CASES))

    def worker(case):
        x_shape, sl, x, status, msg = case
        try:
            start.wait()
            for _ in range(3000):
                st = rp.raw_check(x, x_shape, 2, FAKE, TS, TT, FAKE, TS, TT, 2, 1, sl)
                got = rp.last_error()
                if st != status or got != msg:
                    errors.append((msg, st, got))
                    return
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append((msg, "exception", repr(e)))

    threads = [threading.Thread(target=worker, args=(c,)) for c in CASES]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:4]


def test_success_leaves_the_thread_message_alone():
    """A later OK call does not clear or change this thread's last message."""
    st = rp.raw_check(FAKE, (2, 4, 3, 63), 2, FAKE, TS, TT, FAKE, TS, TT, 2, 1, (0, 32))
    assert st == rp.ROPE_ERR_INVALID and rp.last_error() == "D must be even"
    assert rp.raw_check(FAKE, (2, 4, 3, 64), 2, FAKE, TS, TT, FAKE, TS, TT, 2, 1, (0, 32)) == rp.ROPE_OK
    assert rp.last_error() == "D must be even"
