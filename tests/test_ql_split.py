"""The codebook GEMM's work split, checked on the CPU.

ql_split.h holds the arithmetic the kernel uses to divide a launch among its
persistent workgroups: whole tiles first, then the last partial round of tiles
cut along K (stream-K) when the caller gives a workspace.  tests/ql_split_check.cpp
compiles that header with the host compiler and enumerates what every
workgroup computes, checking that each (tile, K stage) is computed once, that
each split tile has one finisher whose contributor list is exactly the
workgroups that left it a partial (at most 4, all with lower indices, so no
wait can be on a workgroup dispatched after the waiter), and that a workgroup
leaves at most one partial (one workspace slot each)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "free_bit_quantization_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "ql_split_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("qlsplit") / "ql_split_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-Werror", f"-I{CSRC}", SRC, "-o", exe], check=True)
    return exe


def _run(exe, *args):
    r = subprocess.run([exe] + [str(a) for a in args], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout
    return r.stdout


def _tiles(T, N):
    return ((T + 255) // 256) * ((N + 255) // 256)


def _stages(K, bits_a):
    return K // (64 if bits_a in (6, 8) else 128)


# every linear of the five workloads, and the shapes of the GPU stream-K tests
SHAPES = [
    (64, 256, 256, 4),                                            # single linear
    (4608, 3072, 9216, 4),                                        # FLUX QKV
    (4608, 3072, 12288, 4), (4608, 12288, 3072, 4),               # FLUX MLP pair
    (32760, 5120, 13824, 4),                                      # Wan FFN
    (8192, 3072, 9216, 8), (8192, 3072, 3072, 8), (8192, 3072, 12288, 8), (8192, 12288, 3072, 8),
    (1024, 3072, 9216, 8), (1024, 3072, 3072, 8), (1024, 3072, 12288, 8), (1024, 12288, 3072, 8),
    (1024, 3072, 3072, 8), (1024, 12288, 3072, 8), (2100, 1024, 300, 4), (1000, 1024, 2000, 4),
    (512, 1024, 1024, 4), (2048, 512, 1024, 4), (1024, 1024, 1024, 6), (520, 1024, 777, 4),
    (2100, 3072, 300, 4), (1000, 3072, 2000, 4), (512, 3072, 1024, 4), (1024, 2048, 512, 4), (520, 3072, 777, 4),
    (4608, 3072, 9216, 6), (8192, 12288, 3072, 6),
    (700, 3072, 1030, 4),
]


def _weight(bits_a):
    return 70 if bits_a == 8 else 105 if bits_a == 6 else 100


@pytest.mark.parametrize("T,K,N,bits_a", SHAPES)
@pytest.mark.parametrize("cus", [256, 304, 80])
def test_split_of_workload_shapes(checker, T, K, N, bits_a, cus):
    _run(checker, _tiles(T, N), _stages(K, bits_a), cus, cus, _weight(bits_a))


def test_plan_follows_the_measured_split_gains(checker):
    # FLUX QKV: 648 tiles of 24 stages, a tail of 136 tiles: the split lost
    # 4.5 %, so whole tiles; the MLP down projection at 1024 tokens (48 tiles of
    # 96 stages) gained 109 % from the split; 288 tiles of 24 stages (a tail of
    # 32) gained 9 %; 216 tiles of 96 stages lost 2 %
    out = _run(checker, _tiles(4608, 9216), _stages(3072, 4), 256)
    assert "n_dp=648 sk_tiles=0 grid=256" in out, out
    out = _run(checker, _tiles(1024, 3072), _stages(12288, 4), 256)
    assert "n_dp=0 sk_tiles=48 grid=256 classes=8" in out, out
    out = _run(checker, _tiles(2048, 9216), _stages(3072, 4), 256)
    assert "n_dp=256 sk_tiles=32 grid=256 classes=8" in out, out
    out = _run(checker, _tiles(4608, 3072), _stages(12288, 4), 256)
    assert "n_dp=216 sk_tiles=0" in out, out
    # W6A6 FLUX QKV (48 stages of 64, a tail of 136): +7.5 % split; W4A8 8192 x
    # 3072 -> 3072 (a tail of 128): +2 %; W4A8 1024 x 3072 -> 9216 (144): even, whole
    out = _run(checker, _tiles(4608, 9216), _stages(3072, 6), 256, 256, _weight(6))
    assert "n_dp=512 sk_tiles=136" in out, out
    out = _run(checker, _tiles(8192, 3072), _stages(3072, 8), 256, 256, _weight(8))
    assert "n_dp=256 sk_tiles=128" in out, out
    out = _run(checker, _tiles(1024, 9216), _stages(3072, 8), 256, 256, _weight(8))
    assert "sk_tiles=0" in out, out


# Split against whole tiles on MI355X (256 CUs), current kernel: HIP events,
# median of 6 alternating runs in one process, a library build that splits
# every tail of >= 8 tiles.  (T, K, N, activation bits, gain of the split in %)
MEASURED_GAINS = [
    (256, 3072, 9216, 4, 34.8), (512, 3072, 9216, 4, 5.7), (1024, 3072, 9216, 4, -5.9),
    (1536, 3072, 9216, 4, -14.3), (2048, 3072, 9216, 4, 11.9), (3072, 3072, 9216, 4, -8.9),
    (3840, 3072, 9216, 4, 8.0), (4608, 3072, 9216, 4, -4.6), (5120, 3072, 9216, 4, -6.4),
    (5632, 3072, 9216, 4, 5.4), (6400, 3072, 9216, 4, -2.7), (512, 12288, 3072, 4, 150.0),
    (1024, 12288, 3072, 4, 121.2), (2048, 12288, 3072, 4, 47.4), (3072, 12288, 3072, 4, 10.4),
    (4096, 12288, 3072, 4, 3.2), (4608, 12288, 3072, 4, -1.2), (5120, 12288, 3072, 4, -2.1),
    (6144, 12288, 3072, 4, 32.4), (8192, 12288, 3072, 4, 7.0), (4608, 3072, 12288, 4, -0.2),
    (8192, 3072, 3072, 8, -0.5), (8192, 12288, 3072, 8, 11.7), (1024, 3072, 9216, 8, -1.3),
    (1024, 12288, 3072, 8, 141.0), (8192, 3072, 9216, 8, 0.7), (4608, 3072, 9216, 6, 8.1),
    (4608, 3072, 9216, 3, -3.1), (1024, 3072, 3072, 8, 45.3), (1024, 3072, 12288, 8, -4.4),
]


@pytest.mark.parametrize("T,K,N,bits_a,gain", MEASURED_GAINS)
def test_plan_agrees_with_every_measured_gain(checker, T, K, N, bits_a, gain):
    # the cost model splits where the split measured faster by more than 1 %
    # and keeps whole tiles where it measured slower by more than 1 %; within
    # 1 % either choice is allowed (box-to-box spread is larger than that)
    out = _run(checker, _tiles(T, N), _stages(K, bits_a), 256, 256, _weight(bits_a))
    split = "sk_tiles=0" not in out
    if gain > 1.0:
        assert split, (T, K, N, bits_a, gain, out)
    elif gain < -1.0:
        assert not split, (T, K, N, bits_a, gain, out)


def test_no_split_without_slots(checker):
    out = _run(checker, _tiles(1024, 3072), _stages(12288, 4), 256, 0)
    assert "n_dp=48 sk_tiles=0 grid=48" in out, out


def test_sweep_of_tile_counts_stages_and_cu_counts(checker):
    _run(checker, "sweep")


def test_launch_generation_protocol(checker):
    # epoch-tagged flags over a sequence of launches on one workspace, one of
    # them losing a producer's flag, starting also near the 32-bit wrap
    _run(checker, "protocol")
