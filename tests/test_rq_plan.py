"""The rotate-quantize launch plan (rq_plan, host arithmetic in liboq.so), on the CPU.

rq_plan picks the kernel (one wavefront per token, or a workgroup per token
group), its workgroup size, grid and LDS bytes from (d, h, dtype, bits, T, G).
A plan the kernels cannot run would fault or race on the GPU, so its bounds
are checked here without one: every supported shape gets a plan whose LDS
fits a gfx950 CU (160 KB), whose workgroup is whole wavefronts of at most
1024 threads, and whose kernel choice matches the kernels' own limits (the
wavefront kernel: d = 1024 J, h in {64, 256}, a search grid, and with codes
of at most 6 bits at most 256 grid cells, since it takes a cell index as one
byte)."""

import ctypes
import itertools

import pytest

from free_bit_quantization_amd import oq


class RqPlan(ctypes.Structure):
    _fields_ = [("ns", ctypes.c_int), ("tpw", ctypes.c_int), ("threads", ctypes.c_int), ("grid", ctypes.c_int),
                ("lds", ctypes.c_size_t), ("wave_j", ctypes.c_int), ("wpb", ctypes.c_int), ("pad", ctypes.c_int)]


@pytest.fixture(scope="module")
def plan_fn():
    lib = ctypes.CDLL(oq.LIB_PATH)
    try:
        f = lib["_ZN2oq7rq_planEiibiliPNS_6RqPlanE"]   # oq::rq_plan(int, int, bool, int, long, int, RqPlan*)
    except AttributeError:
        pytest.skip("rq_plan not exported under the expected C++ name")
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_bool, ctypes.c_int, ctypes.c_long, ctypes.c_int,
                  ctypes.POINTER(RqPlan)]
    f.restype = ctypes.c_bool

    def plan(d, log2h, bf16, bits, T, G):
        p = RqPlan()
        ok = f(d, log2h, bf16, bits, T, G, ctypes.byref(p))
        return ok, p
    return plan


def _supported(d, log2h):
    ns = d // 16
    return d % 16 == 0 and d % (1 << log2h) == 0 and ((ns % 64 == 0 and ns <= 768) or
                                                        (ns < 64 and ns & (ns - 1) == 0))


DS = [16, 32, 64, 256, 512, 1024, 2048, 3072, 4096, 5120, 6144, 8192, 12288, 1536, 2560, 768]
LOG2HS = [1, 4, 5, 6, 7, 8]
CASES = list(itertools.product(DS, LOG2HS, [True, False], [2, 4, 6, 8], [1, 100, 3072, 4608, 32760], [0, 32, 256, 512]))


def test_every_supported_shape_gets_a_plan_that_fits(plan_fn):
    for d, lg, bf16, bits, T, G in CASES:
        if d % (1 << lg):
            continue
        ok, p = plan_fn(d, lg, bf16, bits, T, G)
        if not _supported(d, lg):
            assert not ok, (d, lg, bf16, bits, T, G)   # no kernel for this (d, h)
        if not ok:
            continue   # also: a supported (d, h) whose tables exceed the LDS (OQ_EUNSUPPORTED)
        where = (d, lg, bf16, bits, T, G, p.wave_j, p.wpb, p.threads, p.lds)
        assert p.lds <= 160 * 1024, where
        assert 64 <= p.threads <= 1024 and p.threads % 64 == 0, where
        assert p.grid >= 1, where
        if p.wave_j > 0:
            assert d == 1024 * p.wave_j and lg in (6, 8) and G > 0, where
            assert bits > 6 or G <= 256, where
            assert p.wave_j <= (5 if bf16 else 2), where
            assert p.threads == 64 * p.wpb and 64 * p.wpb * 16 >= d, where
            assert p.grid == (T + p.wpb - 1) // p.wpb, where
        else:
            assert p.threads == p.ns * p.tpw and p.ns == d // 16, where
            assert p.grid == (T + p.tpw - 1) // p.tpw, where


def test_the_workload_widths_are_supported(plan_fn):
    for d in (256, 1024, 3072, 5120, 12288):
        for bf16 in (True, False):
            for bits in (2, 3, 4, 6, 8):
                for G in (0, 32, 512):
                    ok, p = plan_fn(d, 8 if d >= 256 else 6, bf16, bits, 4608, G)
                    assert ok, (d, bf16, bits, G)


def test_workload_shapes_take_the_wavefront_kernel(plan_fn):
    # FLUX 3072-wide bf16 rows, 4-bit codes, a 32-cell grid: one wavefront per
    # token, 12 per workgroup from 3072 tokens on, 8 below
    ok, p = plan_fn(3072, 8, True, 4, 4608, 32)
    assert ok and p.wave_j == 3 and p.wpb == 12, (p.wave_j, p.wpb)
    ok, p = plan_fn(3072, 8, True, 4, 1024, 32)
    assert ok and p.wave_j == 3 and p.wpb == 8
    # 8-bit codes with a 512-cell grid keep it; 4-bit codes with more than 256
    # cells (thresholds closer than the library's codebooks) and fp32 rows of
    # 12288 take the workgroup kernel
    assert plan_fn(3072, 8, True, 8, 4608, 512)[1].wave_j == 3
    assert plan_fn(3072, 8, True, 4, 4608, 512)[1].wave_j == 0
    assert plan_fn(12288, 8, False, 4, 4608, 64)[1].wave_j == 0
    # no grid (binary search): workgroup kernel
    assert plan_fn(3072, 8, True, 4, 4608, 0)[1].wave_j == 0
