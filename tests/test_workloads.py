"""The seeded input generator: rounding, slicing, distribution (CPU only)."""
import numpy as np

import workloads as wl


def test_bf16_rounding_nearest_even():
    L = wl.lib()
    assert L.gen_bf16_from_double(1.0) == 0x3F80
    assert L.gen_bf16_from_double(-2.0) == 0xC000
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even (1.0)
    assert L.gen_bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    assert L.gen_bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the halfway point rounds up
    assert L.gen_bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    # rounding that carries into the exponent
    assert L.gen_bf16_from_double(2.0 - 2.0 ** -10) == 0x4000
    # smallest subnormal and zero
    assert L.gen_bf16_from_double(2.0 ** -133) == 0x0001
    assert L.gen_bf16_from_double(0.0) == 0x0000


def test_slices_equal_whole():
    whole = wl.normal_bf16(123, 4, 0.02, 0, 100_003)
    part = wl.normal_bf16(123, 4, 0.02, 50_001, 20_000, nthreads=3)
    assert np.array_equal(part, whole[50_001:70_001])
    u = wl.uniform_f32(5, 2, -0.1, 0.1, 0, 1000)
    assert np.array_equal(wl.uniform_f32(5, 2, -0.1, 0.1, 300, 10), u[300:310])
    assert u.min() >= -0.1 and u.max() <= 0.1


def test_thread_count_does_not_change_bytes():
    a = wl.normal_bf16(9, 0, 1.0, 0, 1 << 20, nthreads=1)
    b = wl.normal_bf16(9, 0, 1.0, 0, 1 << 20, nthreads=7)
    assert np.array_equal(a, b)


def test_normal_distribution_and_table():
    L = wl.lib()
    q = np.array([L.gen_normal_quantile(i) for i in range(65536)])
    assert np.all(np.diff(q) > 0)
    assert np.allclose(q, -q[::-1], atol=1e-9)  # symmetric about 0
    assert abs(q[-1] - 4.3249) < 1e-3  # PhiInv(1 - 2^-17): reach of a 16-bit quantile table
    v = (wl.normal_bf16(1, 0, 1.0, 0, 1 << 21).astype(np.uint32) << 16).view(np.float32)
    assert abs(v.mean()) < 3e-3 and abs(v.std() - 1.0) < 3e-3


def test_seeds_and_tensors_differ():
    a = wl.normal_bf16(1, 3, 0.02, 0, 4096)
    assert not np.array_equal(a, wl.normal_bf16(2, 3, 0.02, 0, 4096))
    assert not np.array_equal(a, wl.normal_bf16(1, 4, 0.02, 0, 4096))
