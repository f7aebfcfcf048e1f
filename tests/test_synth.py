"""The seeded generator: splitmix64 known answers, determinism, distributions."""
import ctypes
import math

import numpy as np

import synth


def test_splitmix64_reference_output():
    # splitmix64 seeded with 0 first returns 0xE220A8397B1DCDAF (Steele, Lea and
    # Flood 2014; the widely used reference implementation).
    L = synth.lib()
    L.synth_splitmix64_next.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    L.synth_splitmix64_next.restype = ctypes.c_uint64
    L.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
    L.synth_key.restype = ctypes.c_uint64
    st = ctypes.c_uint64(0)
    assert L.synth_splitmix64_next(ctypes.byref(st)) == 0xE220A8397B1DCDAF
    # counter form: word i of a stream is output i+1 of splitmix64 seeded with the stream key
    key = L.synth_key(9, 2)
    st = ctypes.c_uint64(key)
    for i in range(5):
        assert L.synth_splitmix64_next(ctypes.byref(st)) == synth.word(9, 2, i)


def test_uniform_and_box_muller_from_words():
    # uniform = ((word >> 11) + 1) * 2^-53; normals by Box-Muller on consecutive pairs
    for i in range(6):
        assert synth.uniform(3, 1, i) == ((synth.word(3, 1, i) >> 11) + 1) * 2.0 ** -53
    u0, u1 = synth.uniform(3, 1, 4), synth.uniform(3, 1, 5)
    r = math.sqrt(-2.0 * math.log(u0))
    assert synth.normal(3, 1, 4) == r * math.cos(2 * math.pi * u1)
    assert synth.normal(3, 1, 5) == r * math.sin(2 * math.pi * u1)


def test_same_seed_same_bits_and_layout_independence():
    lens = np.array([7, 3], np.int32)
    g1 = synth.packed_token_major_geometry(lens, 2, 8)
    g2 = synth.packed_head_major_geometry(lens, 2, 8)
    a = synth.fill(5, synth.T_K, g1)
    b = synth.fill(5, synth.T_K, g1)
    np.testing.assert_array_equal(a, b)
    c = synth.fill(5, synth.T_K, g2)
    for bb in range(2):
        for kh in range(2):
            for t in range(lens[bb]):
                r1 = a[g1.seq_offset[bb] + kh * g1.stride_h + t * g1.stride_t:][:8]
                r2 = c[g2.seq_offset[bb] + kh * g2.stride_h + t * g2.stride_t:][:8]
                np.testing.assert_array_equal(r1, r2)
    d = synth.fill(6, synth.T_K, g1)
    assert not np.array_equal(a, d)


def test_normal_moments_and_bf16_rounding():
    geom = synth.dense_geometry(2, 2, 4096, 64)
    x = synth.fill(7, synth.T_V, geom, fmt=synth.F32)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    y = synth.fill(7, synth.T_V, geom, fmt=synth.BF16)
    yf = synth.bf16_bits_to_f32(y)
    assert np.all(np.abs(yf - x) <= np.abs(x) * 2.0 ** -8)


def test_unit_direction_lognormal_values():
    geom = synth.dense_geometry(1, 1, 2000, 128)
    v = synth.bf16_bits_to_f32(synth.fill(5, synth.T_V, geom, kind=synth.UNIT_DIR_LOGNORMAL)).reshape(2000, 128)
    n = np.log(np.linalg.norm(v.astype(np.float64), axis=1))
    assert abs(n.mean()) < 0.1 and abs(n.std() - 1) < 0.1


def test_outlier_channels_and_lengths():
    ch = synth.outlier_channels(4, 0, 8, 128)
    assert all(len(set(c)) == 2 for c in ch)
    m = synth.outlier_multipliers(4, 0, 8, 128)
    assert np.all((m == 10).sum(axis=1) == 2)
    lens = synth.loguniform_lengths(3, 32)
    assert lens.min() >= 512 and lens.max() <= 131072
    assert len(set(lens.tolist())) > 20
    np.testing.assert_array_equal(lens, synth.loguniform_lengths(3, 32))
