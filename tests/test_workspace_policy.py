"""Host-side test of the workspace pool's policy (bpt_ws_choose, a pure
function of the pool's state; no GPU).  What it must guarantee: a call never
takes a buffer that another call is still filling on the host (busy), and
never uses a buffer whose last use may still run on the GPU without first
waiting for it -- whatever the stream handles are (a recycled handle of a
destroyed stream, or hipStreamPerThread, which names a different stream on
every host thread, look the same as the caller's own)."""
import ctypes
import itertools
import os

import pytest

import barrier_pipelined_tiled_amd as pkg


@pytest.fixture(scope="module")
def choose():
    if not os.path.exists(pkg.LIB_PATH):
        from barrier_pipelined_tiled_amd import build
        build.build()
    f = pkg.lib().bpt_ws_choose
    i64p, ip = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int)
    f.argtypes = [ctypes.c_int, i64p, ip, ip, ip, ctypes.c_int64, ctypes.c_int, ip, ip]
    f.restype = ctypes.c_int

    def call(slots, need, cap=4):
        n = len(slots)
        arr = lambda t, k: (t * max(n, 1))(*[s[k] for s in slots])
        wait, grow = ctypes.c_int(-1), ctypes.c_int(-1)
        i = f(n, arr(ctypes.c_int64, 0), arr(ctypes.c_int, 1), arr(ctypes.c_int, 2), arr(ctypes.c_int, 3),
              need, cap, ctypes.byref(wait), ctypes.byref(grow))
        return i, wait.value, grow.value
    return call


# slot = (bytes, busy, state, same): state 0 never used, 1 last use done, 2 may still run
MiB = 1 << 20


def test_empty_pool_makes_a_buffer(choose):
    assert choose([], 8 * MiB) == (0, 0, 0)


def test_idle_buffer_is_taken_without_wait(choose):
    assert choose([(16 * MiB, 0, 1, 0)], 8 * MiB) == (0, 0, 0)
    assert choose([(16 * MiB, 0, 0, 0)], 8 * MiB) == (0, 0, 0)


def test_same_handle_still_waits(choose):
    # a recycled handle looks like the caller's own: the event wait is what
    # orders it, so even the caller's handle gets wait = 1
    assert choose([(16 * MiB, 0, 2, 1)], 8 * MiB) == (0, 1, 0)


def test_other_stream_gets_its_own_buffer_while_the_pool_has_room(choose):
    assert choose([(16 * MiB, 0, 2, 0)], 8 * MiB) == (1, 0, 0)


def test_full_pool_orders_by_waiting(choose):
    slots = [(16 * MiB, 0, 2, 0)] * 4
    assert choose(slots, 8 * MiB) == (0, 1, 0)


def test_busy_buffers_are_never_taken(choose):
    slots = [(16 * MiB, 1, 1, 1)] * 4
    i, wait, grow = choose(slots, 8 * MiB)
    assert i == 4 and grow == 0          # a new buffer beyond the pool size


def test_too_small_buffer_grows(choose):
    i, wait, grow = choose([(4 * MiB, 0, 1, 1)] * 4, 8 * MiB)
    assert (i, grow) == (0, 1)


def test_exhaustive_small_pools_are_safe(choose):
    """Every state of pools of up to 3 slots: the chosen slot is never busy,
    and a slot whose last use may still run is only taken with a wait (or
    grown, which gives it a new buffer)."""
    kinds = [(b, busy, st, same) for b in (4 * MiB, 16 * MiB) for busy in (0, 1) for st in (0, 1, 2)
             for same in ((0, 1) if st == 2 else (0,))]
    for n in range(0, 4):
        for slots in itertools.product(kinds, repeat=n):
            for cap in (1, 2, 4):
                i, wait, grow = choose(list(slots), 8 * MiB, cap)
                assert 0 <= i <= n
                if i == n:
                    assert wait == 0 and grow == 0
                    continue
                b, busy, st, same = slots[i]
                assert not busy
                if grow:
                    assert b < 8 * MiB and wait == 0
                else:
                    assert b >= 8 * MiB
                    assert wait == (1 if st == 2 else 0)
