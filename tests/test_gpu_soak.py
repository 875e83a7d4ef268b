"""Protocol soak and checkpoint/resume at full scale.

* Soak: the churning 30B batch (32 requests, contexts log-uniform on
  [128, 32768], 4 replaced every 8 steps, Zipf router bias) for 256 steps,
  driven by the host scheduler, with the megakernel and the per-op build in
  lock-step on their own copies of the cache. The per-op build orders every
  level by kernel boundaries; the megakernel only by its counters. At every
  step the logits, the whole residual stream and the routing must agree bit
  for bit, so a counter protocol that let a tile read stale data would show
  up as a mismatch. Stops at the first one.
* Resume: a greedy chain run for 16 steps on one handle equals, bit for bit,
  8 steps, a copy of the cache and the next tokens, a new handle on that
  copy, and the 8 remaining steps.
"""

import numpy as np
import pytest
import torch

from persistent_megakernel_03_amd import configs, mk, synth
from tests.gpu_setup import route_ids, x_layers

pytestmark = pytest.mark.gpu

CFG = configs.A3B
P = CFG["page_size"]


@pytest.fixture(scope="module")
def weights():
    print("soak: generating weights on the device", flush=True)
    return synth.make_model(CFG, 0, "cuda")


def test_megakernel_and_perop_in_lock_step_on_the_churning_batch(weights):
    B, steps = 32, 256
    biases, _, _ = synth.zipf_router_bias(CFG)
    w = dict(weights)
    for l, b in enumerate(biases):
        w[f"layers.{l}.router_bias"] = torch.as_tensor(b).cuda()
    max_pages = 32768 // P + steps // P + 2
    # pool: the workload's peak page use, from a host-only dry run of the scheduler
    dry = mk.Scheduler(B, B, P, max_pages, 1 << 22, reserve_full=False)
    run = synth.ChurnRun(dry, synth.ChurnWorkload(B, CFG["vocab"]), max_len=max_pages * P)
    low = 1 << 22
    for _ in range(steps + 1):
        n = dry.next()
        low = min(low, dry.stats()["free_pages"])
        dry.commit(np.zeros(n, np.int32))
        run.advance()
    dry.close()
    n_pages = (1 << 22) - low + 16
    print(f"soak: pool of {n_pages} pages", flush=True)
    k, v = synth.make_kv_pool(CFG, n_pages, 1, "cuda")
    v = v.transpose(-1, -2).contiguous()
    k2, v2 = k.clone(), v.clone()
    sch = mk.Scheduler(B, B, P, max_pages, n_pages, reserve_full=False,
                       page_order=np.random.default_rng(9).permutation(n_pages))
    run = synth.ChurnRun(sch, synth.ChurnWorkload(B, CFG["vocab"]), max_len=max_pages * P)
    mkd = mk.Decoder(CFG, w, k, v, max_batch=B, max_pages_per_seq=max_pages, mode=mk.MK_MODE_MEGAKERNEL)
    pod = mk.Decoder(CFG, w, k2, v2, max_batch=B, max_pages_per_seq=max_pages, mode=mk.MK_MODE_PEROP)
    tokens = torch.empty(B, dtype=torch.int32, device="cuda")
    la = torch.empty(B, CFG["vocab"], device="cuda")
    lb = torch.empty(B, CFG["vocab"], device="cuda")
    for st in range(steps):
        n = sch.next()
        ids, pos, bts = sch.seq_ids[:n].copy(), sch.positions[:n].copy(), sch.block_tables[:n].copy()
        tokens[:n].copy_(torch.from_numpy(sch.tokens[:n].copy()))
        mkd.forward(ids, pos, bts, tokens[:n], la[:n])
        pod.forward(ids, pos, bts, tokens[:n], lb[:n])
        assert mkd.sync_check() == mk.MK_OK and pod.sync_check() == mk.MK_OK
        same = (torch.equal(la[:n], lb[:n]) and torch.equal(x_layers(mkd)[:, :n], x_layers(pod)[:, :n])
                and torch.equal(route_ids(mkd)[:, :n], route_ids(pod)[:, :n]))
        if not same:
            pytest.fail(f"step {st}: megakernel and per-op differ (positions {pos.min()}..{pos.max()})")
        if st % 32 == 0:
            print(f"soak: step {st} equal, contexts {pos.min()}..{pos.max()}", flush=True)
        sch.commit(torch.argmax(la[:n], dim=1).to(torch.int32).cpu().numpy())
        run.advance()
    assert torch.equal(k, k2) and torch.equal(v, v2)
    mkd.close()
    pod.close()
    sch.close()


@pytest.mark.parametrize("B", [1, 3])
def test_resume_from_a_cache_copy_is_bit_identical(weights, B):
    ctx, n1, n2 = 4096, 8, 8
    pages = (ctx + n1 + n2) // P + 2
    n_pages = B * pages + 3
    k0, v0 = synth.make_kv_pool(CFG, n_pages, 2, "cuda")
    v0 = v0.transpose(-1, -2).contiguous()
    bts = synth.make_block_tables(B, pages, n_pages, seed=5, shuffle=True)
    tok0 = torch.tensor(synth.make_tokens(B, CFG["vocab"], seed=6), dtype=torch.int32, device="cuda")

    def steps(dec, tokens, first, n, out):
        logits = torch.empty(B, CFG["vocab"], device="cuda")
        for i in range(n):
            dec.step([ctx + first + i] * B, bts, tokens, logits)
            out.append(logits.clone())
            tokens.copy_(torch.argmax(logits, dim=1).to(torch.int32))
        assert dec.sync_check() == mk.MK_OK

    # one handle, 16 steps
    ka, va = k0.clone(), v0.clone()
    a = mk.Decoder(CFG, weights, ka, va, max_batch=B, max_pages_per_seq=pages)
    ta, la = tok0.clone(), []
    steps(a, ta, 0, n1 + n2, la)
    a.close()
    # 8 steps, checkpoint (cache and next tokens), a new handle on a copy, 8 steps
    kb, vb = k0.clone(), v0.clone()
    b = mk.Decoder(CFG, weights, kb, vb, max_batch=B, max_pages_per_seq=pages)
    tb, lb = tok0.clone(), []
    steps(b, tb, 0, n1, lb)
    b.close()
    ck, cv, ct = kb.clone(), vb.clone(), tb.clone()
    del kb, vb, b
    c = mk.Decoder(CFG, weights, ck, cv, max_batch=B, max_pages_per_seq=pages)
    steps(c, ct, n1, n2, lb)
    c.close()
    for i in range(n1 + n2):
        assert torch.equal(la[i], lb[i]), ("step", i)
    assert torch.equal(ka, ck) and torch.equal(va, cv) and torch.equal(ta, ct)
