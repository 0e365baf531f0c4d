"""The seeded input generator: Philox4x32-10 known-answer vectors (Random123
distribution, Salmon et al. SC'11), host C vs NumPy implementations, and the
draw recipes."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("ctr,key,expect", [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
])
def test_philox_kat(ctr, key, expect):
    out = synth.philox4x32_10(np.array([ctr], np.uint32), key)[0]
    assert tuple(int(x) for x in out) == expect


def test_fnv1a():
    # FNV-1a 32-bit reference values: "" -> offset basis, "a" -> 0xe40c292c
    assert synth.fnv1a32("") == 0x811C9DC5
    assert synth.fnv1a32("a") == 0xE40C292C


def test_stream_offsets_consistent():
    a = synth.stream_u32(5, "t", 37)
    b = synth.stream_u32(5, "t", 20, 13)
    assert np.array_equal(a[13:33], b)


def test_c_matches_numpy():
    if synth._c() is None:
        synth.build_host_generator()
    for dt in ("f32", "bf16"):
        a = synth.normal(3, "w", (1001, 7), 0.02, mean=0.5, dtype=dt)
        b = synth.normal(3, "w", (1001, 7), 0.02, mean=0.5, dtype=dt, use_c=False)
        assert np.array_equal(a, b)
    assert np.array_equal(synth.token_ids(1, "ids", 999, 248320),
                          synth.token_ids(1, "ids", 999, 248320, use_c=False))


def test_normal_moments_and_bf16():
    x = synth.normal(0, "m", (200000,), 0.02, dtype="bf16")
    v = synth.bf16_bits_to_f32(x)
    assert abs(v.std() - 0.02) < 2e-4 and abs(v.mean()) < 2e-4
    # bf16 rounding is nearest-even of the float32 value
    f = synth.normal(0, "m", (200000,), 0.02, dtype="f32")
    assert np.array_equal(synth.f32_to_bf16_bits(f), x)
    assert np.all(np.abs(v - f) <= np.abs(f) * 2.0 ** -8)


def test_token_ids_range():
    ids = synth.token_ids(1, "ids", 100000, 1000)
    assert ids.min() >= 0 and ids.max() < 1000
    assert abs(np.bincount(ids, minlength=1000).std() / 100 - 0.1) < 0.05


@pytest.mark.parametrize("use_c", [True, False])
def test_normal_slice_matches_whole(use_c):
    if use_c and synth._c() is None:
        synth.build_host_generator()
    whole = synth.normal(2, "kv", (4099,), 1.0, dtype="bf16", use_c=use_c)
    part = synth.normal(2, "kv", (1000,), 1.0, dtype="bf16", use_c=use_c, start=1537)
    assert np.array_equal(whole[1537:2537], part)
