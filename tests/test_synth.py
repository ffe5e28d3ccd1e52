"""The seeded generators: the jump-ahead LCG equals the step-by-step recurrence of the oxinfer
tests' `rnd` helper (multiplier 6364136223846793005, increment 1442695040888963407), draws are
deterministic, and the value recipes produce the documented ranges."""
import numpy as np

import synth


def test_lcg_jump_ahead_equals_recurrence():
    M = (1 << 64) - 1
    for seed, stream, n in [(1, 0, 5), (1003, 2, 70000), (7, 6, 131073)]:
        st = synth.lcg_states(seed, stream, n)
        x = synth._splitmix64(((seed & 0xFFFFFFFFFFFF) << 16) | stream)
        for i in range(n):
            x = (x * 6364136223846793005 + 1442695040888963407) & M
            if i < 50 or i % 9973 == 0 or i == n - 1:
                assert int(st[i]) == x


def test_determinism_and_ranges():
    a = synth.make_dense("q4a", 64, 256, 8, "bf16", 1.0, 1234)
    b = synth.make_dense("q4a", 64, 256, 8, "bf16", 1.0, 1234)
    for k in ("codes", "scales", "offsets", "X"):
        assert np.array_equal(a[k], b[k])
    d = a["scales"].view(np.float16).astype(np.float64)
    assert d.min() >= 0.01 - 1e-5 and d.max() <= 0.05 + 1e-5
    nib = np.concatenate([a["codes"] & 15, a["codes"] >> 4])
    assert set(np.unique(nib)) == set(range(16))
    q = synth.make_dense("q8", 64, 256, 1, "f32", 1.0, 5)
    assert q["codes"].min() >= -127 and q["codes"].max() <= 127
    s = q["scales"]
    assert s.min() >= 0.002 and s.max() <= 0.01
    z = synth.normal(3, 3, 200000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01


def test_streams_differ():
    assert not np.array_equal(synth.uniform(1000, 0, 100), synth.uniform(1000, 1, 100))
    assert not np.array_equal(synth.uniform(1000, 0, 100), synth.uniform(1001, 0, 100))
