"""The page allocator (csa_page_pool) and the paged entry points' argument
checks, on the CPU ("LLM Atlas: DeepSeek" §19: serving depends on the
sequence-length distribution and the page allocator).  No kernel runs here."""
import ctypes
import threading

import numpy as np
import pytest

import compressed_sparse_attention_06_amd as csa
from compressed_sparse_attention_06_amd._lib import CompressJob, PageTableC

INVALID, NO_PAGES = -1, -5
P = ctypes.c_void_p(0x10000)


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(csa.LIB_PATH):
        from compressed_sparse_attention_06_amd import build
        build.build()
    return csa.lib()


def test_alloc_release_and_exhaustion(lib):
    pool = csa.PagePool(6)
    a = pool.alloc(4)
    assert sorted(a) == [0, 1, 2, 3] and pool.available() == 2
    with pytest.raises(csa.CsaError, match="out of pages"):
        pool.alloc(3)                       # all or nothing
    assert pool.available() == 2
    pool.release(a[:2])
    assert pool.available() == 4
    b = pool.alloc(4)
    assert len(set(b) | set(a[2:])) == 6     # no page handed out twice


def test_release_is_all_or_nothing(lib):
    pool = csa.PagePool(8)
    a = pool.alloc(3)
    for bad in ([a[0], a[0]], [a[0], 7], [a[1], -1], [a[2], 8]):
        with pytest.raises(csa.CsaError, match="invalid argument"):
            pool.release(bad)
        assert pool.available() == 5        # nothing was released
    pool.release(a)
    with pytest.raises(csa.CsaError):
        pool.release(a[:1])                 # double free
    assert pool.available() == 8


def test_reserve_grows_a_sequence_page_by_page(lib):
    pool = csa.PagePool(5)
    row = np.full(4, -1, np.int32)
    pool.reserve(row, 64, 1)
    assert (row >= 0).sum() == 1
    first = row[0]
    pool.reserve(row, 64, 64)                # still one page
    assert (row >= 0).sum() == 1 and row[0] == first
    pool.reserve(row, 64, 65)
    assert (row >= 0).sum() == 2 and row[0] == first
    pool.reserve(row, 64, 256)
    assert (row >= 0).sum() == 4 and pool.available() == 1
    with pytest.raises(csa.CsaError, match="invalid argument"):
        pool.reserve(row, 64, 257)           # beyond max_pages
    other = np.full(4, -1, np.int32)
    with pytest.raises(csa.CsaError, match="out of pages"):
        pool.reserve(other, 64, 129)         # needs 3, one free: nothing taken
    assert (other == -1).all() and pool.available() == 1
    pool.release_row(row)
    assert (row == -1).all() and pool.available() == 5


def test_concurrent_alloc_release_never_shares_a_page(lib):
    pool = csa.PagePool(4096)
    held, errors = [], []
    lock = threading.Lock()

    def worker(seed):
        rng = np.random.default_rng(seed)
        mine = []
        try:
            for _ in range(300):
                if mine and rng.random() < 0.4:
                    k = int(rng.integers(1, len(mine) + 1))
                    pool.release(mine[:k])
                    mine = mine[k:]
                else:
                    mine += list(pool.alloc(int(rng.integers(1, 8))))
        except Exception as e:  # noqa: BLE001
            errors.append(e)
        with lock:
            held.extend(mine)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors
    assert len(held) == len(set(held))
    assert pool.available() + len(held) == 4096


def _pt(pages=P, max_pages=4, page_rows=256, pool_pages=64):
    return PageTableC(pages, max_pages, page_rows, pool_pages)


@pytest.mark.parametrize("bad", [dict(pages=None), dict(max_pages=0), dict(page_rows=32), dict(page_rows=384),
                                 dict(pool_pages=0)])
def test_paged_entry_points_reject_bad_tables(lib, bad):
    pt = _pt(**bad)
    assert lib.csa_index_score_paged(P, P, P, 1, P, 2, 1, 64, 128, ctypes.byref(pt), 4, P, None) == INVALID
    assert lib.csa_sparse_attn_paged(P, P, ctypes.byref(pt), P, 512, P, 128, 128, P, P, 1, 0.04, 64, 1e4, 2, 1, 64,
                                     512, P, 0, P, 1 << 30, None) == INVALID
    assert lib.hca_attn_paged(P, P, ctypes.byref(pt), 128, P, 128, 128, P, P, 1, 0.04, 64, 1e4, 2, 1, 64, 512, P, 0,
                              P, 1 << 30, None) == INVALID
    job = CompressJob(P, P, None, None, 1, P, 2, 8, 8 * 512, 512, 4, 1, 64, 1e4, 1e-6, 0, 0, 0, P, P, 1, 0, 0,
                      None, 0)
    assert lib.csa_compress_paged(ctypes.byref(job), ctypes.byref(pt), 1, None) == INVALID
    # a bad table behind a good one in the same launch
    jobs = (CompressJob * 2)(job, job)
    tabs = (PageTableC * 2)(_pt(), pt)
    assert lib.csa_compress_paged(jobs, tabs, 2, None) == INVALID
    assert lib.csa_compress_paged(None, ctypes.byref(_pt()), 1, None) == INVALID
    assert lib.csa_compress_paged(ctypes.byref(job), None, 1, None) == INVALID
    assert lib.csa_compress_paged(jobs, tabs, 17, None) == INVALID   # more than CSA_MAX_COMPRESS_JOBS
    assert lib.csa_index_score_paged(P, P, P, 1, P, 2, 1, 64, 128, None, 4, P, None) == INVALID
