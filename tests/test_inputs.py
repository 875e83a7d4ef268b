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


def test_ragged_batch_pages_and_churn():
    rb = synth.RaggedBatch(32, 20000, 16, 2200, 1000, seed=3)
    ctx0 = list(rb.pos)
    assert min(ctx0) >= 128 and max(ctx0) <= 32768
    seen_ids = set(rb.ids)
    for step in range(1, 41):
        joined = rb.advance()
        assert (len(joined) == 4) == (step % 8 == 0)
        for b in joined:
            assert 128 <= rb.pos[b] <= 2048 and rb.ids[b] not in seen_ids
        seen_ids |= set(rb.ids)
        # every sequence holds exactly the pages its next slot needs, no page twice
        owned = [p for pg in rb.pages for p in pg]
        assert len(owned) == len(set(owned))
        assert not set(owned) & set(rb.free)
        for b in range(32):
            assert len(rb.pages[b]) == rb.pos[b] // 16 + 1
        bt = rb.tables()
        assert bt.shape == (32, 2200)
