"""The seeded input generator (host side): Philox known answers, table, slicing."""
import numpy as np
import pytest

from workloads import CONFIGS, TINY, M130, B28, LONG, DECODE, inputs, philox


# Known-answer vectors of Philox4x32-10 published with the Random123 library
# (Salmon et al., SC'11): counter, key -> output.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = philox.philox4x32_10(*[np.uint32(c) for c in ctr], *key)
    assert tuple(int(g) for g in got) == want


def test_draw_slices_are_consistent():
    full = philox.draw_u16(7, 9, 3, 0, 0, 1000)
    for start, count in [(0, 1), (1, 7), (5, 16), (8, 8), (123, 300), (999, 1)]:
        assert np.array_equal(philox.draw_u16(7, 9, 3, 0, start, count), full[start:start + count])
    assert not np.array_equal(philox.draw_u16(7, 9, 4, 0, 0, 64), full[:64])   # another stream
    assert not np.array_equal(philox.draw_u16(7, 9, 3, 1, 0, 64), full[:64])   # another step


def test_normal_table():
    t = inputs._normal_f64()
    assert t.shape == (65536,)
    assert np.all(np.diff(t) > 0)
    assert np.allclose(t, -t[::-1], atol=1e-12)
    assert abs(t.mean()) < 1e-12 and abs(t.std() - 1.0) < 2e-3
    t16 = inputs.table("bf16")
    t32 = inputs.table("f32")
    assert t16.dtype == np.uint16 and t32.dtype == np.float32
    half = inputs.table("f32", 0.5)
    assert np.array_equal(half, t32 * np.float32(0.5))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.0, 0.0, 3.3895314e38], dtype=np.float32)])
    ours = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_bits_to_f32(ours), torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_configs_are_the_five_workloads():
    assert [c.index for c in CONFIGS] == [1, 2, 3, 4, 5]
    assert (TINY.batch, TINY.dim, TINY.dstate, TINY.seqlen, TINY.io) == (1, 16, 4, 64, "f32")
    assert (M130.batch, M130.dim, M130.dstate, M130.seqlen, M130.io) == (8, 1536, 16, 2048, "f32")
    assert (B28.batch, B28.dim, B28.dstate, B28.seqlen, B28.io) == (8, 5120, 16, 2048, "bf16")
    assert (LONG.batch, LONG.dim, LONG.seqlen) == (1, 2048, 1 << 20)
    assert (DECODE.batch, DECODE.dim, DECODE.steps) == (256, 5120, 128)


def test_params_recipe():
    A, dskip, bias = inputs.params(M130)
    assert A.shape == (1536, 16) and np.array_equal(A[5], -np.arange(1, 17, dtype=np.float32))
    u = np.log1p(np.exp(bias.astype(np.float64)))      # softplus(dt_bias) = u
    assert u.min() >= 0.999e-3 and u.max() <= 1.001e-1
    assert abs(dskip.mean() - 1.0) < 0.02 and 0.07 < dskip.std() < 0.13
    _, d1, _ = inputs.params(B28)
    assert np.all(d1 == 1.0)


def test_channel_subset_equals_full_draw():
    full = inputs.scan_inputs_full(TINY)
    chans = [(0, 3), (0, 11)]
    sub = inputs.scan_inputs(TINY, channels=chans, t0=5, t1=40)
    for name in ("x", "dt", "z"):
        for i, (b, d) in enumerate(chans):
            assert np.array_equal(sub[name][i], full[name][b, d, 5:40])
    assert np.array_equal(sub["B"], full["B"][..., 5:40])
    x = inputs.raw_to_f64(full["x"], "f32")
    assert abs(x.mean()) < 0.1 and abs(x.std() - 1) < 0.1
    dt = inputs.raw_to_f64(full["dt"], "f32")
    assert abs(dt.std() - 0.5) < 0.05


def test_decode_inputs_subset():
    chans = [(0, 0), (3, 17), (255, 5119)]
    step = 5
    full = inputs.decode_inputs(DECODE, step)
    sub = inputs.decode_inputs(DECODE, step, channels=chans)
    for i, (b, d) in enumerate(chans):
        assert sub["x"][i] == full["x"][b, d]
    s0 = inputs.decode_state0(DECODE, channels=chans)
    assert s0.shape == (3, 16) and s0.dtype == np.float32
