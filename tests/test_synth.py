"""The seeded input generators: determinism and the structure each recipe
plants (checked with plain numpy in fp64, not with the oracle)."""
from __future__ import annotations

import numpy as np

import synth


def sylvester16() -> np.ndarray:
    h = np.ones((1, 1))
    for _ in range(4):
        h = np.block([[h, h], [h, -h]])
    return h / 4.0


def test_same_seed_same_bytes():
    a = synth.make("t3_lognormal_16384x8192", rows=32)
    b = synth.make("t3_lognormal_16384x8192", rows=32)
    assert a.sha256() == b.sha256()
    c = synth.make("t3_lognormal_16384x8192", rows=32, seed=1)
    assert a.sha256() != c.sha256()


def test_row_slices_are_prefixes():
    small = synth.make("gauss_1pct_cols_4096x4096", rows=8)
    big = synth.make("gauss_1pct_cols_4096x4096", rows=16)
    assert np.array_equal(small.x, big.x[:8])


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -30, -2.5,
                     0.0, -0.0, 3.0e38, 2.0 ** -130])
    bits = synth.round_bf16(vals)
    back = synth.bf16_to_f32(bits).astype(np.float64)
    assert back[0] == 1.0
    assert back[1] == 1.0                       # tie -> even
    assert back[2] == 1.0 + 4 * 2 ** -8         # tie -> even (up)
    assert back[3] == 1.0 + 2 * 2 ** -8         # above the tie
    assert back[4] == -2.5
    assert bits[5] == 0 and bits[6] == 0x8000
    assert np.isfinite(back[7])
    assert back[8] == 2.0 ** -130               # bf16 subnormal, exact


def test_normal_moments():
    z = synth.normal_f64(1 << 20, seed=5)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3


def test_outlier_columns():
    w = synth.make("gauss_outliers_128x1024")
    xf = synth.bf16_to_f32(w.x).astype(np.float64)
    cols = w.meta["outlier_cols"]
    assert len(set(cols)) == 4
    std = xf.std(0)
    assert np.all(std[cols] > 30) and np.median(std) < 1.2
    w2 = synth.make("gauss_1pct_cols_4096x4096", rows=256)
    assert len(set(w2.meta["outlier_cols"])) == 41
    s2 = synth.bf16_to_f32(w2.x).astype(np.float64).std(0)
    assert np.all(s2[w2.meta["outlier_cols"]] > 7)


def test_silu_ties_planted_blocks():
    H = sylvester16()
    for rotate in (False, True):
        w = synth.make("silu_ties_32768x14336", rotate=rotate, rows=256)
        xb = synth.bf16_to_f32(w.x).astype(np.float64).reshape(-1, 16)
        flags = w.meta["tie_flags"]
        assert 0.5 / 1024 < flags.mean() < 2.0 / 1024
        y = xb @ H if rotate else xb
        ties = y[flags.astype(bool)]
        mids = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0}
        assert all(abs(v) in mids for v in ties.reshape(-1))
        assert np.all(np.abs(ties).max(1) == 6.0)
        anchor = y[w.meta["anchor_block"]]
        assert np.abs(anchor).max() == 168.0
        others = np.delete(np.abs(y), w.meta["anchor_block"], axis=0)
        assert others.max() < 168.0


def test_kv_heads_planted_blocks():
    w = synth.make("kv_heads_65536x8x128_f32", rows=4096)
    kind = w.meta["block_kind"]
    xb = w.x.reshape(-1, 16)
    assert np.all(xb[kind == 1] == 0) and np.all(np.signbit(xb[kind == 1]) == 0)
    assert np.all(xb[kind == 2] == 0) and np.all(np.signbit(xb[kind == 2]))
    dom = xb[kind == 3]
    assert len(dom) > 0 and np.all(dom == dom[0])
    nat = np.abs(xb[kind == 0]).max()
    H = sylvester16()
    assert np.abs(dom[0].astype(np.float64) @ H).max() > 2 * nat
    assert np.abs(dom[0]).max() > 2 * nat
