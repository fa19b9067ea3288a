"""Host logic: the W4A4 GEMM's row split (nvfp4_gemm_plan) against a brute
force over every split, each timed by simulating greedy in-order dispatch of
the tiles onto the CUs (a 256 x 192 tile takes 4 time units, a 192 x 192
tile 3).  CPU only."""
import ctypes as C
import heapq
import random

import pytest


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_quantization_amd as m

    m.lib()
    return m


def finish(n1, n2, cus):
    free = [0] * cus
    for _ in range(n1):
        heapq.heappush(free, heapq.heappop(free) + 4)
    for _ in range(n2):
        heapq.heappush(free, heapq.heappop(free) + 3)
    return max(free)


def brute(M, N, cus):
    tn, kfull = -(-N // 192), -(-M // 256)
    base = finish(kfull * tn, 0, cus)
    best, plan = base, (M, kfull * tn)
    for k1 in range(kfull - 1, -1, -1):
        k2 = -(-(M - 256 * k1) // 192)
        t = finish(k1 * tn, k2 * tn, cus)
        if t < best and t * 100 < base * 97:
            best, plan = t, (256 * k1, (k1 + k2) * tn)
    return plan


def test_gemm_plan_known_shapes(nv):
    # 7040 x 3072 on 256 CUs: a round of 256 tiles of 256 rows, a round of
    # 256 tiles of 192 rows
    assert nv.gemm_plan(7040, 3072, 256) == (4096, 512)
    assert nv.gemm_plan(7040, 14336, 256) == (21 * 256, 30 * 75)
    # one CU: two 192-row tiles (6 units) would take longer than one 256-row
    # tile (4)
    assert nv.gemm_plan(256, 192, 1) == (256, 1)
    assert nv.gemm_plan(0, 3072, 256) == (0, 0)
    assert nv.gemm_plan(7040, 0, 256) == (7040, 0)


def test_gemm_plan_matches_brute_force(nv):
    rng = random.Random(7)
    for _ in range(150):
        M = rng.choice([rng.randint(1, 300), rng.randint(300, 4000), rng.randint(4000, 9000)])
        N = rng.choice([16, 192, 200, 3072, rng.randint(16, 6000)])
        cus = rng.choice([1, 3, 8, 64, 80, 256, 304])
        assert nv.gemm_plan(M, N, cus) == brute(M, N, cus), (M, N, cus)


def test_gemm_plan_rejects(nv):
    L = nv.lib()
    r, g = C.c_int64(), C.c_int64()
    assert L.nvfp4_gemm_plan(-1, 16, 256, C.byref(r), C.byref(g)) == -1
    assert L.nvfp4_gemm_plan(16, 16, 0, C.byref(r), C.byref(g)) == -1
    assert L.nvfp4_gemm_plan(16, 16, 256, None, C.byref(g)) == -1
