"""GPU test of the host continuous-batching scheduler driving the megakernel:
requests with prompts of 1 to 70 tokens and 2 to 10 new tokens, more
requests than slots (queueing), prompts longer than a step's rows (chunked
prefill), decode rows and prompt chunks in the same launches
(mk_forward_step), greedy tokens chosen on the device.

Each finished request is checked against the oracle: its prompt and the
tokens the device generated, fed to the oracle's prefill from an empty
cache (the plain definition), give logits within 5e-2 of the device's at
every row that chose a token, and every chosen token is the oracle's argmax
unless the oracle's top two are within 1e-3 (a near tie either side may take).
"""

import numpy as np
import pytest
import torch

from oracle import PagedKV, prefill
from persistent_megakernel_03_amd import configs, mk, synth
from tests.gpu_setup import Setup

pytestmark = pytest.mark.gpu

CFG = configs.TINY
P = CFG["page_size"]


@pytest.mark.parametrize("mode", [mk.MK_MODE_MEGAKERNEL, mk.MK_MODE_PEROP])
def test_scheduler_serves_requests_that_match_the_oracle(mode):
    n_pages, max_pages, rows = 96, 8, 24
    s = Setup(CFG, n_pages=n_pages, seed=0)
    rng = np.random.default_rng(21)
    lens = [1, 5, 17, 40, 70, 3, 25, 9]
    news = [6, 4, 8, 3, 5, 10, 2, 7]
    prompts = {r: [int(x) for x in rng.integers(0, CFG["vocab"], size=n)] for r, n in enumerate(lens)}
    sch = mk.Scheduler(4, rows, P, max_pages, n_pages, reserve_full=True,
                       page_order=np.random.default_rng(5).permutation(n_pages))
    for r in prompts:
        sch.submit(r, prompts[r], news[r])
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, s.w_dev, k, v, max_batch=rows, max_pages_per_seq=max_pages, mode=mode,
                     validate_plans=True)
    tokens = torch.empty(rows, dtype=torch.int32, device="cuda")
    logits = torch.empty(rows, CFG["vocab"], device="cuda")
    dev_logits = {r: [] for r in prompts}
    steps = 0
    while True:
        n = sch.next()
        if n == 0:
            break
        steps += 1
        tokens[:n].copy_(torch.from_numpy(sch.tokens[:n].copy()))
        dec.forward(sch.seq_ids[:n].copy(), sch.positions[:n].copy(), sch.block_tables[:n].copy(), tokens[:n],
                    logits[:n])
        assert dec.sync_check() == mk.MK_OK
        lg = logits[:n].cpu().numpy()
        for b in range(n):
            if sch.sample[b]:
                dev_logits[int(sch.request_ids[b])].append(lg[b])
        sch.commit(np.argmax(lg, axis=1).astype(np.int32))
        assert steps < 200
    st = sch.stats()
    print(f"scheduler: {steps} steps, {st}", flush=True)
    assert st["finished"] == len(prompts) and st["free_pages"] == n_pages and st["prompt_rows"] == sum(lens)
    dec.close()
    model = s.oracle_model()
    for r, prompt in prompts.items():
        toks = sch.tokens_of(r)
        gen = toks[len(prompt):]
        assert len(gen) == news[r]
        kv = PagedKV(synth.bits(s.k0).copy(), synth.bits(s.v0.transpose(-1, -2)).copy(), P)
        ol, _ = prefill(model, kv, 0, list(range(max_pages)), toks[:-1])
        for i, g in enumerate(gen):
            row = ol[len(prompt) - 1 + i]
            assert np.max(np.abs(row - dev_logits[r][i])) <= 5e-2, ("logits", r, i)
            top2 = np.sort(row.astype(np.float64))[-2:]
            if g != int(np.argmax(row)):
                assert top2[1] - top2[0] < 1e-3, ("token", r, i)
    sch.close()
