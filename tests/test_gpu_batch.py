"""GPU parity of batched decode steps (3 to 64 sequences, the matrix-core
tiles) on the tiny MoE decoder, through the C ABI, against the CPU oracle.

Same bar as the one-sequence tests, per row: logits max-abs <= 5e-2,
residual stream after every block relative L2 <= 1e-2, routing ids
bit-exact (a decision whose oracle margin is below 1e-4 may differ, and that
row's layer comparison stops there), every sequence's new KV slot written
and nothing else, the new entries within one BF16 ulp of the oracle's
rounding where not tiny and within BF16 noise overall, and the megakernel
equal to the per-op build bit for bit.

Batches are ragged: seeded positions from 0 (empty cache) to 95, pages
drawn from a shuffled pool. A batch of 64 identical sequences sends all 64
tokens to the same two experts, which takes the expert tiles' widest token
blocks (33-64 columns). A churning batch (sequences leaving and joining,
pages recycled through a free list) runs with a Zipf router bias.
"""

import numpy as np
import pytest
import torch

from oracle import bf16_to_f32, decode_step
from persistent_megakernel_03_amd import configs, mk, synth
from tests.gpu_setup import Setup, rel_l2, route_ids, routing_margin, x_layers

pytestmark = pytest.mark.gpu

CFG = configs.TINY
PAGES_PER_SEQ = 7
N_PAGES = 64 * PAGES_PER_SEQ + 8


@pytest.fixture(scope="module")
def setup():
    torch.manual_seed(0)
    return Setup(CFG, n_pages=N_PAGES, seed=0)


def _batch(B, seed):
    rng = np.random.default_rng(1000 + seed)
    positions = [int(x) for x in rng.integers(0, 96, size=B)]
    positions[0] = 0
    bts = synth.make_block_tables(B, PAGES_PER_SEQ, N_PAGES, seed=seed, shuffle=True).tolist()
    toks = [int(t) for t in synth.make_tokens(B, CFG["vocab"], seed=seed)]
    return positions, bts, toks


def _run(s, positions, bts, toks, mode=mk.MK_MODE_MEGAKERNEL, steps=1, shared=0, mfma_min_batch=0, row_blocks=0):
    B = len(positions)
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, s.w_dev, k, v, max_batch=max(B, 3), max_pages_per_seq=PAGES_PER_SEQ, mode=mode,
                     shared_levels=shared, validate_plans=True, mfma_min_batch=mfma_min_batch,
                     mm_row_blocks=row_blocks)
    tokens = torch.tensor(toks, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, CFG["vocab"], device="cuda")
    print(f"batch B={B} mode={mode} shared={shared} steps={steps} mfma_min_batch={mfma_min_batch} "
          f"row_blocks={row_blocks}", flush=True)
    for st in range(steps):
        dec.step([p + st for p in positions], bts, tokens, logits, seq_ids=list(range(100, 100 + B)))
        assert dec.sync_check() == mk.MK_OK
    out = dict(logits=logits.cpu().numpy(), xs=x_layers(dec).cpu().numpy(), ids=route_ids(dec).cpu().numpy(),
               k=k, v=v)
    dec.close()
    return out


def _check_rows(s, positions, bts, toks, g):
    model, kv = s.oracle_model(), s.oracle_kv()
    ol, tr, _ = decode_step(model, kv, positions, bts, toks)
    L = CFG["n_layers"]
    for b in range(len(positions)):
        assert np.max(np.abs(g["logits"][b] - ol[b])) <= 5e-2, ("logits", b)
        for l in range(L):
            lt = tr[b].layers[l]
            assert rel_l2(g["xs"][2 * l + 1, b], lt.x_attn) < 1e-2, ("x_attn", b, l)
            if not np.array_equal(g["ids"][l, b], lt.ids):
                assert routing_margin(lt.router_logits, CFG["top_k"]) < 1e-4, ("routing", b, l)
                break
            assert rel_l2(g["xs"][2 * l + 2, b], lt.x_out) < 1e-2, ("x_out", b, l)
    # the pool changed exactly at every sequence's new slot, to the oracle's rounding
    kb, vb = synth.bits(s.k0), synth.bits(s.v0)
    ka, va = synth.bits(g["k"]), synth.bits(g["v"])
    ck = {tuple(int(t) for t in x) for x in np.argwhere(np.any(ka != kb, axis=(2, 4)))}
    cv = {tuple(int(t) for t in x) for x in np.argwhere(np.any(va != vb, axis=(2, 3)))}
    want = {(l, bts[b][p // 16], p % 16) for l in range(L) for b, p in enumerate(positions)}
    assert ck <= want and cv <= want
    new = np.zeros(kb.shape, bool)
    for b, p in enumerate(positions):
        new[:, bts[b][p // 16], :, p % 16, :] = True
    for got, want_ in ((ka, kv.k), (synth.bits(g["v"].transpose(-1, -2)), kv.v)):
        assert np.array_equal(got[~new], want_[~new])
        gv, wv = got[new], want_[new]
        wf = bf16_to_f32(wv)
        big = np.abs(wf) >= 0.1 * np.max(np.abs(wf))
        assert np.abs(gv.astype(np.int32) - wv.astype(np.int32))[big].max() <= 1
        assert rel_l2(bf16_to_f32(gv), wf) <= 5e-3


@pytest.mark.parametrize("B", [3, 8, 17, 64])
def test_batch_step_matches_oracle(setup, B):
    positions, bts, toks = _batch(B, B)
    g = _run(setup, positions, bts, toks)
    _check_rows(setup, positions, bts, toks, g)


@pytest.mark.parametrize("B", [1, 2])
def test_matrix_core_schedule_at_one_and_two_tokens(setup, B):
    """mfma_min_batch = 1: one- and two-token batches on the matrix-core
    schedule (every weight product on MFMA, routing and expert-sum levels)
    match the oracle at the same bars, in both modes, and the megakernel
    equals the per-op build bit for bit."""
    positions, bts, toks = _batch(B, 40 + B)
    a = _run(setup, positions, bts, toks, mfma_min_batch=1)
    _check_rows(setup, positions, bts, toks, a)
    b = _run(setup, positions, bts, toks, mk.MK_MODE_PEROP, mfma_min_batch=1)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["xs"], b["xs"])


def test_batch_megakernel_equals_perop_bitwise(setup):
    positions, bts, toks = _batch(8, 5)
    a = _run(setup, positions, bts, toks, mk.MK_MODE_MEGAKERNEL, steps=2)
    b = _run(setup, positions, bts, toks, mk.MK_MODE_PEROP, steps=2)
    assert np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["xs"], b["xs"])
    assert np.array_equal(a["ids"], b["ids"])
    assert torch.equal(a["k"], b["k"]) and torch.equal(a["v"], b["v"])


@pytest.mark.parametrize("B", [3, 17, 64])
def test_expert_row_blocks_bitwise(setup, B):
    """Expert tiles of two row blocks per activation load (gate/up: 16 rows,
    down: 32 rows) sum each output row's products in the same order as tiles
    of one block, so the step is the same bit for bit, in both modes."""
    positions, bts, toks = _batch(B, 13)
    a = _run(setup, positions, bts, toks, mk.MK_MODE_MEGAKERNEL, steps=2, row_blocks=1)
    for mode in (mk.MK_MODE_MEGAKERNEL, mk.MK_MODE_PEROP):
        b = _run(setup, positions, bts, toks, mode, steps=2, row_blocks=2)
        assert np.array_equal(a["logits"], b["logits"])
        assert np.array_equal(a["xs"], b["xs"])
        assert np.array_equal(a["ids"], b["ids"])
        assert torch.equal(a["k"], b["k"]) and torch.equal(a["v"], b["v"])


@pytest.mark.parametrize("B", [8, 64])
def test_shared_levels_equal_static_lists_bitwise(setup, B):
    """Tiles claimed from shared pools compute exactly what the same tiles
    compute from fixed lists (placement decides only where a tile runs), and
    the shared-level step matches the oracle."""
    positions, bts, toks = _batch(B, 11)
    a = _run(setup, positions, bts, toks, mk.MK_MODE_MEGAKERNEL, steps=2, shared=-1)
    b = _run(setup, positions, bts, toks, mk.MK_MODE_MEGAKERNEL, steps=2, shared=2)
    assert np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["xs"], b["xs"])
    assert np.array_equal(a["ids"], b["ids"])
    assert torch.equal(a["k"], b["k"]) and torch.equal(a["v"], b["v"])
    g = _run(setup, positions, bts, toks, shared=2)
    _check_rows(setup, positions, bts, toks, g)


def test_identical_sequences_share_experts(setup):
    """64 copies of one sequence at position 0: every row computes the same
    values, so every token picks the same two experts (64 columns in one
    expert tile); the rows must agree with each other bit for bit and with
    the oracle."""
    B = 64
    positions = [0] * B
    bts = synth.make_block_tables(B, PAGES_PER_SEQ, N_PAGES, seed=9, shuffle=True).tolist()
    toks = [77] * B
    g = _run(setup, positions, bts, toks)
    for b in range(1, B):
        assert np.array_equal(g["logits"][b], g["logits"][0])
        assert np.array_equal(g["ids"][:, b], g["ids"][:, 0])
    _check_rows(setup, positions, bts, toks, g)


def test_batch_greedy_chain(setup):
    """Four greedy steps of a ragged batch of 5, the device's argmax fed back
    on the device; the oracle is teacher-forced with the same tokens."""
    s = setup
    B = 5
    positions, bts, toks = _batch(B, 21)
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, s.w_dev, k, v, max_batch=B, max_pages_per_seq=PAGES_PER_SEQ)
    model, kv = s.oracle_model(), s.oracle_kv()
    tokens = torch.tensor(toks, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, CFG["vocab"], device="cuda")
    for st in range(4):
        pos = [p + st for p in positions]
        cur = [int(t) for t in tokens.cpu().tolist()]
        print(f"batch greedy step={st}", flush=True)
        dec.step(pos, bts, tokens, logits)
        assert dec.sync_check() == mk.MK_OK
        ol, _, _ = decode_step(model, kv, pos, bts, cur)
        assert np.max(np.abs(logits.cpu().numpy() - ol)) <= 5e-2
        tokens.copy_(torch.argmax(logits, dim=1).to(torch.int32))
    dec.close()


def test_churning_batch_with_zipf_bias(setup):
    """Eight slots over 12 steps, driven by the host scheduler: every 4 steps
    three requests end and new ones (new ids, pages recycled through the
    scheduler's free list, fresh first tokens) take their slots; the router
    carries a Zipf(1.1) bias. Each step is compared with the oracle
    teacher-forced on the device's tokens and cache."""
    s = setup
    B = 8
    biases, _, _ = synth.zipf_router_bias(CFG)
    w = dict(s.w_dev)
    for l, b in enumerate(biases):
        w[f"layers.{l}.router_bias"] = torch.as_tensor(b).cuda()
    sch = mk.Scheduler(B, B, 16, PAGES_PER_SEQ, N_PAGES, reserve_full=False,
                       page_order=np.random.default_rng(4).permutation(N_PAGES))
    run = synth.ChurnRun(sch, synth.ChurnWorkload(B, CFG["vocab"], seed=4, ctx_lo=2, ctx_hi=80, join_lo=0,
                                                  join_hi=40, every=4, churn=3), max_len=PAGES_PER_SEQ * 16)
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, w, k, v, max_batch=B, max_pages_per_seq=PAGES_PER_SEQ)
    model = s.oracle_model(weights=w)
    tokens = torch.empty(B, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, CFG["vocab"], device="cuda")
    for st in range(12):
        n = sch.next()
        assert n == B
        pos, bts, ids = sch.positions[:n].tolist(), sch.block_tables[:n].tolist(), sch.seq_ids[:n].tolist()
        cur = sch.tokens[:n].tolist()
        tokens.copy_(torch.tensor(cur, dtype=torch.int32))
        kv = s.oracle_kv(k, v)            # the cache as the device holds it before this step
        print(f"churn step={st} requests={sch.request_ids[:n].tolist()}", flush=True)
        dec.forward(ids, pos, bts, tokens, logits)
        assert dec.sync_check() == mk.MK_OK
        ol, tr, _ = decode_step(model, kv, pos, bts, cur)
        gl = logits.cpu().numpy()
        xs, rid = x_layers(dec).cpu().numpy(), route_ids(dec).cpu().numpy()
        for b in range(B):
            assert np.max(np.abs(gl[b] - ol[b])) <= 5e-2, ("logits", st, b)
            for l in range(CFG["n_layers"]):
                lt = tr[b].layers[l]
                if not np.array_equal(rid[l, b], lt.ids):
                    assert routing_margin(lt.router_logits, CFG["top_k"]) < 1e-4, ("routing", st, b, l)
                    break
                assert rel_l2(xs[2 * l + 2, b], lt.x_out) < 1e-2, ("x_out", st, b, l)
        sch.commit(np.argmax(gl, axis=1).astype(np.int32))
        run.advance()
    dec.close()
    sch.close()


def test_longer_sequence_joins_a_reserved_slot(setup):
    """A sequence of 500 cached tokens takes the slot of one of 10 in the
    next step. The plan built for the first step reserved 3 chunks of 128
    tokens for that slot (256 tokens of lookahead), so the step reuses it and
    the new sequence spreads its 501 tokens over those 3 chunks (192 tokens
    each). Both steps against the oracle, teacher-forced on the device's
    cache."""
    s = setup
    pps = 40
    bts = synth.make_block_tables(4, pps, N_PAGES, seed=31, shuffle=True).tolist()
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, s.w_dev, k, v, max_batch=3, max_pages_per_seq=pps)
    model = s.oracle_model()
    logits = torch.empty(3, CFG["vocab"], device="cuda")
    steps = [([10, 20, 30], [bts[0], bts[1], bts[2]], [5, 6, 7], [1, 2, 3]),
             ([500, 21, 31], [bts[3], bts[1], bts[2]], [9, 8, 4], [4, 2, 3])]
    for pos, bt, toks, ids in steps:
        kv = s.oracle_kv(k, v)
        print(f"reserved-slot step pos={pos}", flush=True)
        dec.step(pos, bt, torch.tensor(toks, dtype=torch.int32, device="cuda"), logits, seq_ids=ids)
        assert dec.sync_check() == mk.MK_OK
        ol, _, _ = decode_step(model, kv, pos, bt, toks)
        assert np.max(np.abs(logits.cpu().numpy() - ol)) <= 5e-2
    dec.close()
