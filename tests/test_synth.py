"""The seeded input generators: shapes, determinism, bf16 exactness."""

import numpy as np

from free_bit_quantization_amd import synth


def test_workloads_shapes():
    w = synth.workloads()
    assert list(w) == synth.WORKLOAD_ORDER
    q = w["flux_qkv_w4a4"].linears[0]
    assert (q.T, q.d_in, q.d_out, q.h, q.bits_w, q.bits_a) == (4608, 3072, 9216, 256, 4, 4)
    assert (q.act_outliers, q.w_outliers) == (31, 15)
    f = w["wan_ffn_w4a4"].linears[0]
    assert (f.T, f.d_in, f.d_out, f.act_outliers, f.w_outliers) == (32760, 5120, 13824, 51, 0)
    b = w["flux_block_w4a8_b2"].linears
    assert len(b) == 8 and {l.bits_a for l in b} == {8}
    assert [l.act_outliers for l in b if l.d_in == 12288] == [123, 123]


def test_generators_deterministic_and_bf16_exact():
    lin = synth.workloads()["flux_qkv_w4a4"].linears[0]
    x1, w1 = synth.gen_linear(lin, 0, 0, T=16)
    x2, w2 = synth.gen_linear(lin, 0, 0, T=16)
    assert np.array_equal(x1, x2) and np.array_equal(w1, w2)
    assert x1.shape == (16, 3072) and w1.shape == (9216, 3072)
    assert np.all((x1.view(np.uint32) & 0xFFFF) == 0)     # bf16-representable
    x3, _ = synth.gen_linear(lin, 1, 0, T=16)
    assert not np.array_equal(x1, x3)


def test_bf16_round_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    np.testing.assert_array_equal(synth.bf16_round(v), np.array([1.0, 1.0, 1.0 + 2 ** -7, -2.5, 1.0], dtype=np.float32))
