"""The step entry point that allocates nothing (mk_decode_step_noalloc),
called through the C ABI, against mk_decode_step: the same inputs give the
same logits and the same KV cache bit for bit, on two calls in a row, the
second with a smaller batch (a different kernel build: three tokens run the
matrix-core schedule, two the two-token one). A handle whose step needs more
than the library's static scratch is refused before anything is enqueued."""

import numpy as np
import pytest
import torch

from persistent_megakernel_03_amd import configs, mk, synth
from tests.gpu_setup import Setup

pytestmark = pytest.mark.gpu

CFG = configs.TINY
V = CFG["vocab"]
PAGES = 7
N_PAGES = 4 * PAGES + 4


def test_noalloc_step_equals_the_workspace_step():
    s = Setup(CFG, n_pages=N_PAGES, seed=0)
    bts = synth.make_block_tables(4, PAGES, N_PAGES, seed=77, shuffle=True)
    calls = [([5, 70, 33], bts[:3], [11, 700, 95]), ([40, 2], bts[1:3], [3, 1000])]
    k1, v1 = s.fresh_pools()
    k2, v2 = s.fresh_pools()
    d1 = mk.Decoder(CFG, s.w_dev, k1, v1, max_batch=4, max_pages_per_seq=PAGES)
    d2 = mk.Decoder(CFG, s.w_dev, k2, v2, max_batch=4, max_pages_per_seq=PAGES)
    stream = torch.cuda.current_stream().cuda_stream
    for i, (pos, bt, toks) in enumerate(calls):
        B = len(pos)
        print(f"noalloc call {i}: batch {B}", flush=True)
        t = torch.tensor(toks, dtype=torch.int32, device="cuda")
        l1 = torch.full((B, V), float("nan"), device="cuda")
        l2 = torch.full((B, V), float("nan"), device="cuda")
        d1.step(pos, bt, t, l1)
        mk.mk_decode_step_noalloc(d2.handle, B, None, pos, np.ascontiguousarray(bt, np.int32), t.data_ptr(),
                                  l2.data_ptr(), stream)
        assert d1.sync_check() == mk.MK_OK and d2.sync_check() == mk.MK_OK
        assert torch.isfinite(l1).all()
        assert torch.equal(l1, l2)
        assert torch.equal(k1, k2) and torch.equal(v1, v2)
    d1.close()
    d2.close()


def test_a_step_larger_than_the_scratch_is_refused():
    # attention partials for 64 sequences x 4 heads x 512 chunks x 64 dims x 2 layers: 67 MB > 64 MiB
    s = Setup(CFG, n_pages=8, seed=0)
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, s.w_dev, k, v, max_batch=64, max_pages_per_seq=4096)
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.full((1, V), 7.0, device="cuda")
    with pytest.raises(mk.MkError) as e:
        mk.mk_decode_step_noalloc(dec.handle, 1, None, [3], np.zeros((1, 4096), np.int32), t.data_ptr(),
                                  lg.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert e.value.status == mk.MK_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((lg == 7.0).all())
    assert dec.sync_check() == mk.MK_OK
    dec.close()
