"""Host-side plan of the many-row (prefill) path, through the library's own
planning code (an internal, non-ABI call; no GPU needed): key ranges cover
every key of every row, and the workspace holds every sub-list and count the
kernels address."""
import ctypes

import pytest

import dsa_top_token_amd as dsa

SHAPES = [
    # (batch, n_q, n_k, q_pos0, top_k)
    (1, 1024, 1024, 0, 64),
    (1, 65536, 65536, 0, 1536),
    (1, 131072, 131072, 0, 2048),
    (2, 40000, 40000, 0, 1024),
    (2, 700, 50000, 49300, 512),
    (1, 500, 70000, 69500, 2048),
    (2, 9, 12000, 11991, 333),
    (1, 3001, 5000, 1999, 500),
    (3, 17, 4194304, 4194287, 4096),
    (1, 16383, 40000, 23617, 700),
    (1, 16384, 40000, 23616, 700),
]


def plan(B, n_q, n_k, q_pos0, k):
    p = dsa.make_problem(B, n_q, n_k, q_pos0, 128, "fp8", k, 2)
    f = dsa.load().dsa_internal_prefill_plan
    f.argtypes = [ctypes.POINTER(dsa.Problem), ctypes.c_void_p]
    f.restype = ctypes.c_int32
    out = (ctypes.c_int64 * 6)()
    assert f(ctypes.byref(p), out) == 0
    return p, [int(v) for v in out]


@pytest.mark.parametrize("shape", SHAPES)
def test_ranges_cover_every_key(shape):
    B, n_q, n_k, q_pos0, k = shape
    _, (slabs, slab_rows, nr, rk, cap, ws) = plan(*shape)
    maxlen = min(n_k, q_pos0 + n_q)
    assert nr >= 1 and rk % 128 == 0 and nr * rk >= maxlen
    assert (nr - 1) * rk < maxlen  # no range starts past every key
    assert slabs * slab_rows >= n_q and (slabs - 1) * slab_rows < n_q
    # every row's keys [0, len) fall in ranges 0 .. ceil(len / rk) - 1 < nr
    for pos in (q_pos0, q_pos0 + n_q // 2, q_pos0 + n_q - 1):
        n = min(n_k, pos + 1)
        assert -(-n // rk) <= nr
    # thresholds, counts [rows][nr], sub-lists [nr][rows][cap], fallback list
    # and counter, fallback score rows: all inside the prefill workspace
    r = B * slab_rows
    al = lambda x: (x + 255) // 256 * 256
    need = al(r * 4) + al(r * nr * 4) + al(r * nr * cap * 8) + al(r * 4) + al(4) + al(256 * n_k * 4)
    assert ws >= need


def test_many_rows_take_one_range_and_few_rows_split():
    assert plan(1, 65536, 65536, 0, 1536)[1][2] == 1
    assert plan(1, 131072, 131072, 0, 2048)[1][2] == 1
    assert plan(2, 700, 50000, 49300, 512)[1][2] == 4
    assert plan(1, 1024, 1024, 0, 64)[1][2] == 1
