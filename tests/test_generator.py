"""The seeded input generator: its definition, determinism, slices and quantisation (CPU)."""
import math

import numpy as np
import pytest

import ssmgen

M64 = 2**64 - 1
GAMMA = 0x9E3779B97F4A7C15


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_splitmix64_reference_vector():
    # SplitMix64 from state 0: its published first outputs
    state, outs = 0, []
    for _ in range(3):
        state = (state + GAMMA) & M64
        outs.append(_mix(state))
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_raw_stream_definition():
    for seed, tid, i in [(0, 0, 0), (123, 4, 99), (ssmgen.SEED_BASE + 2, 6, 2**33 + 5)]:
        key = _mix((seed + tid * GAMMA) & M64)
        assert ssmgen.raw(seed, tid, i) == _mix((key + (i + 1) * GAMMA) & M64)


def test_uniform_and_normal_from_definition():
    seed, tid = 77, 3
    u = ssmgen.fill(seed, tid, ssmgen.UNIFORM, 0.0, 1.0, 10, ssmgen.F64)
    for i in range(10):
        assert u[i] == (ssmgen.raw(seed, tid, i) >> 11) * 2.0**-53
    n = ssmgen.fill(seed, tid, ssmgen.NORMAL, 0.0, 1.0, 10, ssmgen.F64)
    for i in range(10):
        p = i // 2
        r = math.sqrt(-2.0 * math.log(1.0 - u[2 * p]))
        th = 2.0 * math.pi * u[2 * p + 1]
        ref = r * (math.sin(th) if i % 2 else math.cos(th))
        assert abs(n[i] - ref) <= 1e-15 * max(1.0, abs(ref))


def test_moments():
    n = ssmgen.fill(5, 1, ssmgen.NORMAL, 0.0, 1.0, 1 << 20, ssmgen.F64)
    assert abs(n.mean()) < 5e-3 and abs(n.var() - 1.0) < 5e-3
    u = ssmgen.fill(5, 2, ssmgen.UNIFORM, 1.0, 16.0, 1 << 20, ssmgen.F64)
    assert u.min() >= 1.0 and u.max() < 16.0 and abs(u.mean() - 8.5) < 0.02


def test_slices_equal_bulk_and_threads_do_not_matter():
    bulk = ssmgen.fill(9, 4, ssmgen.NORMAL, 0.0, 0.5, 300000, ssmgen.BF16, nthreads=7)
    one = ssmgen.fill(9, 4, ssmgen.NORMAL, 0.0, 0.5, 300000, ssmgen.BF16, nthreads=1)
    part = ssmgen.fill(9, 4, ssmgen.NORMAL, 0.0, 0.5, 1000, ssmgen.BF16, start=123456)
    assert np.array_equal(bulk, one)
    assert np.array_equal(bulk[123456:124456], part)


def test_bf16_round_to_nearest_even():
    f = ssmgen.f32_to_bf16_bits
    assert f(1.0) == 0x3F80
    assert f(1.0 + 2.0**-8) == 0x3F80            # tie -> even (down)
    assert f(1.0 + 3 * 2.0**-8) == 0x3F82        # tie -> even (up)
    assert f(1.0 + 2.0**-8 + 2.0**-20) == 0x3F81  # above the tie -> up
    assert f(-2.5) == 0xC020
    assert f(float("inf")) == 0x7F80
    nan = f(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_bias_recipe_inverts_softplus():
    b = ssmgen.fill(1, 7, ssmgen.INV_SOFTPLUS_UNIFORM, 0.001, 0.1, 10000, ssmgen.F64)
    sp = np.log1p(np.exp(b))
    assert sp.min() >= 0.001 * (1 - 1e-12) and sp.max() < 0.1 * (1 + 1e-12)


def test_config_table():
    c = ssmgen.CONFIGS
    assert c[2].algorithmic_bytes() == 1_076_133_888
    assert c[1].algorithmic_bytes() == 202_485_760
    assert c[3].algorithmic_bytes() == 17_247_125_504
    assert c[4].algorithmic_bytes() == 826_294_784
    assert c[0].algorithmic_bytes() == 233_984
    assert c[3].tokch == 2**31


def test_channel_slice_matches_full_tensors():
    cfg = ssmgen.with_shape(ssmgen.CONFIGS[4], batch=2, dim=256, L=64, N=8)
    full = ssmgen.make_inputs(cfg)
    b, d = 1, 133
    ch = ssmgen.make_channel(cfg, b, d)
    assert np.array_equal(ch["x"][0, 0], full["x"][b, d])
    assert np.array_equal(ch["delta"][0, 0], full["delta"][b, d // 64])
    assert np.array_equal(ch["B"][0, 0], full["B"][b, 0])
    assert ch["A"][0] == full["A"][d // 64] and ch["D"][0] == full["D"][d]
    assert ch["delta_bias"][0] == full["delta_bias"][d // 64]


def test_batch_entry_is_a_slice_of_the_whole_tensors():
    cfg = ssmgen.with_shape(ssmgen.CONFIGS[1], batch=3, dim=16, L=40)
    whole = ssmgen.make_inputs(cfg)
    for b in range(cfg.batch):
        one = ssmgen.make_batch_entry(cfg, b)
        assert set(one) == set(whole)
        for name, arr in one.items():
            if name in ("x", "delta", "B", "C", "z"):
                assert np.array_equal(arr[0], whole[name][b]), name
            else:
                assert np.array_equal(arr, whole[name]), name


@pytest.mark.parametrize("mode", ["diag", "head"])
def test_channel_block_equals_slice_of_full_tensors(mode):
    """A block of channels regenerated alone has exactly the bits of the same slice of the full
    tensors (the full-size parity tests rely on it)."""
    cfg = ssmgen.ScanConfig(name="blk", batch=3, dim=256, L=40, N=8, ngroups=2,
                            headdim=32 if mode == "head" else 1, a_mode=mode, seed=91)
    full = ssmgen.make_inputs(cfg)
    b, d0, d1 = 2, 128, 192
    blk = ssmgen.make_channel_block(cfg, b, d0, d1)
    sub = ssmgen.block_config(cfg, d0, d1)
    assert set(blk) == set(sub.shapes())
    r0, r1 = (d0 // 32, d1 // 32) if mode == "head" else (d0, d1)
    g = d0 // (cfg.dim // cfg.ngroups)
    assert np.array_equal(blk["x"][0], full["x"][b, d0:d1])
    assert np.array_equal(blk["z"][0], full["z"][b, d0:d1])
    assert np.array_equal(blk["delta"][0], full["delta"][b, r0:r1])
    assert np.array_equal(blk["B"][0, 0], full["B"][b, g])
    assert np.array_equal(blk["C"][0, 0], full["C"][b, g])
    assert np.array_equal(blk["A"], full["A"][r0:r1])
    assert np.array_equal(blk["D"], full["D"][d0:d1])
    assert np.array_equal(blk["delta_bias"], full["delta_bias"][r0:r1])
    for k, shp in sub.shapes().items():
        assert blk[k].shape == shp, k
    with pytest.raises(ValueError):
        ssmgen.make_channel_block(cfg, 0, 100, 140)   # crosses the group boundary at 128
