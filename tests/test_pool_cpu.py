"""The host page pool of the C ABI (kitty_pool_*): order of page ids,
reservation by token count, all-or-nothing exhaustion, release and reuse,
argument errors, and a seeded random workload that checks that mapped and
free pages always partition the pool.  No GPU is involved."""
import ctypes
import os

import numpy as np
import pytest

from mixed_precision_bit_kitty_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libkitty.so not built")


def row(n):
    return np.full(n, -1, np.int32)


def test_init_and_order():
    pool = B.PagePool(5)
    assert pool.n_free == 5
    r = row(4)
    pool.reserve(r, 31)  # no full page yet
    assert (r == -1).all() and pool.n_free == 5
    pool.reserve(r, 32)
    assert r.tolist() == [0, -1, -1, -1]
    pool.reserve(r, 100)  # 3 pages: 0 kept, 1 and 2 added
    assert r.tolist() == [0, 1, 2, -1] and pool.n_free == 2
    pool.reserve(r, 95)  # fewer tokens never unmaps
    assert r.tolist() == [0, 1, 2, -1]


def test_all_or_nothing():
    pool = B.PagePool(3)
    a, b = row(4), row(4)
    pool.reserve(a, 64)
    with pytest.raises(B.KittyError) as e:
        pool.reserve(b, 64)
    assert e.value.code == B.KITTY_ERR_NO_PAGES
    assert (b == -1).all() and pool.n_free == 1
    assert "free" in B.load().kitty_last_error().decode()
    pool.reserve(b, 32)
    assert b.tolist() == [2, -1, -1, -1] and pool.n_free == 0


def test_release_and_reuse():
    pool = B.PagePool(6)
    a, b = row(3), row(3)
    pool.reserve(a, 96)
    pool.reserve(b, 64)
    assert a.tolist() == [0, 1, 2] and b.tolist() == [3, 4, -1]
    pool.release(a)
    assert (a == -1).all() and pool.n_free == 4
    c = row(3)
    pool.reserve(c, 96)  # the pages just released come back first, last one first
    assert c.tolist() == [2, 1, 0]
    assert set(c.tolist()).isdisjoint(b.tolist())


def test_argument_errors():
    lib = B.load()
    pool = B.PagePool(4)
    r = row(2)
    with pytest.raises(B.KittyError) as e:
        pool.reserve(r, 96)  # 3 pages > max_pages 2
    assert e.value.code == B.KITTY_ERR_INVALID_ARG
    with pytest.raises(B.KittyError):
        pool.reserve(r, -1)
    bad = np.array([7, -1], np.int32)  # 7 is not a page of a 4-page pool
    with pytest.raises(B.KittyError):
        pool.reserve(bad, 32)
    bad = np.array([-2, -1], np.int32)
    with pytest.raises(B.KittyError):
        pool.release(bad)
    # releasing the same pages twice overflows the pool and changes nothing
    pool.reserve(r, 64)
    saved = r.copy()
    pool.release(r)
    assert pool.n_free == 4
    with pytest.raises(B.KittyError) as e:
        pool.release(saved)
    assert e.value.code == B.KITTY_ERR_INVALID_ARG
    assert pool.n_free == 4 and saved.tolist() == [0, 1]
    p = B.kitty_pool_t()
    fl = np.empty(4, np.int32)
    assert lib.kitty_pool_init(None, fl.ctypes.data, 4) == B.KITTY_ERR_INVALID_ARG
    assert lib.kitty_pool_init(ctypes.byref(p), None, 4) == B.KITTY_ERR_INVALID_ARG
    assert lib.kitty_pool_init(ctypes.byref(p), fl.ctypes.data, 0) == B.KITTY_ERR_INVALID_ARG
    assert lib.kitty_pool_init(ctypes.byref(p), fl.ctypes.data, 1 << 31) == B.KITTY_ERR_INVALID_ARG
    assert lib.kitty_pool_reserve(ctypes.byref(p), None, 2, 0) == B.KITTY_ERR_INVALID_ARG


def test_random_workload_partitions_the_pool():
    rng = np.random.default_rng(11)
    n_pages, n_rows, max_pages = 40, 7, 9
    pool = B.PagePool(n_pages)
    rows = [row(max_pages) for _ in range(n_rows)]
    lens = [0] * n_rows
    for _ in range(2000):
        i = int(rng.integers(n_rows))
        op = rng.random()
        if op < 0.15:
            pool.release(rows[i])
            lens[i] = 0
        else:
            want = min(lens[i] + int(rng.integers(0, 40)), 32 * max_pages)
            try:
                pool.reserve(rows[i], want)
                lens[i] = want
            except B.KittyError as e:
                assert e.value.code == B.KITTY_ERR_NO_PAGES
                need = sum(1 for j in range(want // 32) if rows[i][j] < 0)
                assert need > pool.n_free
        mapped = [int(x) for r in rows for x in r if x >= 0]
        free = pool.free_list[:pool.n_free].tolist()
        assert len(mapped) == len(set(mapped))
        assert sorted(mapped + free) == list(range(n_pages))
        for r, n in zip(rows, lens):  # every row maps exactly the pages its length needs
            assert all(r[j] >= 0 for j in range(n // 32))
            assert all(r[j] < 0 for j in range(n // 32, max_pages))
