"""The seeded input generator: determinism, chunk invariance, rounding, distributions."""
import numpy as np

from bidirectional_mamba_state_amd import configs, inputs


def test_bf16_rounding_is_nearest_even():
    # exact ties between two bf16 neighbours round to the even mantissa
    one = 1.0
    ulp = 2.0 ** -7
    v = np.array([one + ulp / 2, one + 3 * ulp / 2, -(one + ulp / 2), 3.0e-3, 1e-40, 0.0])
    bits = inputs.round_bf16_bits(v)
    back = inputs.bf16_bits_to_f32(bits).astype(np.float64)
    assert back[0] == 1.0
    assert back[1] == one + 2 * ulp
    assert back[2] == -1.0
    assert abs(back[3] - 3.0e-3) <= 3.0e-3 * 2.0 ** -8
    assert back[5] == 0.0
    # against a brute-force nearest search on random values
    rng = np.random.default_rng(0)
    r = rng.standard_normal(2000) * 10.0 ** rng.uniform(-5, 3, 2000)
    b = inputs.round_bf16_bits(r)
    f = inputs.bf16_bits_to_f32(b).astype(np.float64)
    up = inputs.bf16_bits_to_f32(b + 1).astype(np.float64)
    dn = inputs.bf16_bits_to_f32(b - 1).astype(np.float64)
    assert np.all(np.abs(f - r) <= np.abs(up - r)) and np.all(np.abs(f - r) <= np.abs(dn - r))


def test_deterministic_and_chunk_invariant():
    cfg = configs.get(1)
    P = inputs.PREFIX
    a = inputs.draw(cfg, 0, P, 0, inputs.FWD, 0, 5000)      # crosses a piece boundary
    parts = [inputs.draw(cfg, 0, P, 0, inputs.FWD, 0, 40),
             inputs.draw(cfg, 0, P, 0, inputs.FWD, 40, 4100),
             inputs.draw(cfg, 0, P, 0, inputs.FWD, 4100, 5000)]
    for i in range(4):
        assert np.array_equal(a[i], np.concatenate([p[i] for p in parts]))
    c = inputs.draw(cfg, 0, P, 0, inputs.FWD, 0, 5000)
    assert all(np.array_equal(a[i], c[i]) for i in range(4))
    d = inputs.draw(cfg, 1, P, 0, inputs.FWD, 0, 96)
    assert not np.array_equal(a[0][:96], d[0])               # streams differ
    e = inputs.draw(cfg, 0, inputs.BLOCK(0), 0, inputs.REV, 0, 96)
    assert not np.array_equal(a[0][:96], e[0])               # segments and directions differ
    f = inputs.draw(cfg, 0, inputs.BLOCK(0), 0, inputs.FWD, 0, 96)
    assert not np.array_equal(e[0], f[0])
    seg = inputs.prefix(cfg, streams=[0], length=5000)
    assert np.array_equal(seg.x[0], a[0]) and np.array_equal(seg.dt[0], a[1])


def test_shapes_dtypes_and_distributions():
    cfg = configs.get(1)
    s = inputs.prefix(cfg, length=2048)
    assert s.x.shape == (1, 2048, 48, 64) and s.x.dtype == np.uint16
    assert s.dt.shape == (1, 2048, 48)
    assert s.B.shape == (1, 2048, 1, 128) and s.C.shape == (1, 2048, 1, 128)
    x = inputs.as_f32(s.x, cfg.in_dtype)
    dt = inputs.as_f32(s.dt, cfg.in_dtype)
    B = inputs.as_f32(s.B, cfg.in_dtype)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert abs(B.std() - 0.25) < 0.01
    assert dt.min() >= np.float32(1e-3) * (1 - 2 ** -8) and dt.max() <= 0.1 * (1 + 2 ** -8)
    assert 0.015 < np.median(dt) < 0.022
    assert 0.02 < np.mean(dt >= 0.0995) < 0.07  # a few percent sit at the upper clip
    A, D = inputs.params(cfg)
    assert A.dtype == np.float32 and np.all(A <= -1.0) and np.all(A >= -16.0)
    c0 = configs.get(0)
    s0 = inputs.block(c0, 0, 0, inputs.REV)
    assert s0.x.dtype == np.float32 and s0.x.shape == (1, 16, 4, 16)
