"""CPU checks of the seeded input recipes (no arithmetic of the method):
the Zipf router bias and the churning ragged batch."""

import numpy as np

from persistent_megakernel_03_amd import configs, synth


def test_zipf_bias_slope_and_determinism():
    b1, alpha, slope = synth.zipf_router_bias(configs.A3B)
    b2, _, _ = synth.zipf_router_bias(configs.A3B)
    assert abs(slope + 1.1) < 0.02 and alpha > 0
    assert len(b1) == configs.A3B["n_layers"]
    for x, y in zip(b1, b2):
        assert x.dtype == np.float32 and x.shape == (128,)
        assert np.array_equal(x, y)
        # b_e = -alpha s ln(rank): the ranks are a permutation of 1..E
        rank = np.exp(-x.astype(np.float64) / (alpha * 1.1))
        assert np.array_equal(np.sort(np.rint(rank)), np.arange(1, 129))


def test_churn_workload_draws():
    w = synth.ChurnWorkload(32, 1000, seed=3)
    ctx0 = [c for c, _ in w.initial]
    assert len(ctx0) == 32 and min(ctx0) >= 128 and max(ctx0) <= 32768
    assert len(set(ctx0)) > 20     # log-uniform spread, not a constant
    w2 = synth.ChurnWorkload(32, 1000, seed=3)
    for step in range(1, 41):
        ev, ev2 = w.after_step(step), w2.after_step(step)
        assert ev == ev2
        assert (len(ev) == 4) == (step % 8 == 0)
        assert [s for s, _, _ in ev] == sorted({s for s, _, _ in ev})
        for slot, ctx, tok in ev:
            assert 0 <= slot < 32 and 128 <= ctx <= 2048 and 0 <= tok < 1000
