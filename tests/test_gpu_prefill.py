"""GPU parity of multi-token steps (mk_forward_step): rows of one sequence
at consecutive positions in one launch, attending causally over the cached
prefix and the rows before them, against the oracle's prefill (the plain
definition: the same tokens decoded one after another).

Bars as for decode, per row: logits max-abs <= 5e-2, the residual after
every block relative L2 <= 1e-2, routing ids bit-exact unless the oracle's
float64 margin is below 1e-4 (then that row and the rows after it in its
run are not compared past that layer: a flip changes the KV they read), the
pool changed exactly at the written slots and within one BF16 ulp of the
oracle where not tiny. The megakernel equals the per-op build bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import bf16_to_f32, decode_step, prefill
from persistent_megakernel_03_amd import configs, mk, synth
from tests.gpu_setup import Setup, rel_l2, route_ids, routing_margin, x_layers

pytestmark = pytest.mark.gpu

CFG = configs.TINY
P = CFG["page_size"]
PAGES_PER_SEQ = 8
N_PAGES = 16 * PAGES_PER_SEQ


@pytest.fixture(scope="module")
def setup():
    return Setup(CFG, n_pages=N_PAGES, seed=0)


def _tables(n_seqs, seed):
    return synth.make_block_tables(n_seqs, PAGES_PER_SEQ, N_PAGES, seed=seed, shuffle=True).tolist()


def _rows(runs, tables):
    """runs: [(seq, first position, n rows, first token seed)] -> per-row
    seq ids, positions, block tables, tokens."""
    ids, pos, bts, toks = [], [], [], []
    for seq, p0, n, ts in runs:
        t = [int(x) for x in synth.make_tokens(n, CFG["vocab"], seed=ts)]
        for i in range(n):
            ids.append(seq)
            pos.append(p0 + i)
            bts.append(tables[seq])
            toks.append(t[i])
    return ids, pos, bts, toks


def _run(s, ids, pos, bts, toks, mode=mk.MK_MODE_MEGAKERNEL, max_batch=None):
    B = len(pos)
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, s.w_dev, k, v, max_batch=max_batch or max(B, 3), max_pages_per_seq=PAGES_PER_SEQ,
                     mode=mode, validate_plans=True)
    tokens = torch.tensor(toks, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, CFG["vocab"], device="cuda")
    print(f"forward step: {B} rows, runs {sorted(set(ids))}, mode {mode}", flush=True)
    dec.forward(ids, pos, bts, tokens, logits)
    assert dec.sync_check() == mk.MK_OK
    out = dict(logits=logits.cpu().numpy(), xs=x_layers(dec).cpu().numpy(), ids=route_ids(dec).cpu().numpy(),
               k=k, v=v)
    dec.close()
    return out


def _check(s, ids, pos, bts, toks, g):
    """Each run through the oracle's prefill (a run of one row is a decode
    step), on one oracle cache, then the per-row comparison."""
    model, kv = s.oracle_model(), s.oracle_kv()
    L = CFG["n_layers"]
    rows = {}
    b = 0
    while b < len(pos):
        e = b
        while e + 1 < len(pos) and ids[e + 1] == ids[b]:
            e += 1
        if e == b:
            lg, tr, _ = decode_step(model, kv, [pos[b]], [bts[b]], [toks[b]])
        else:
            lg, tr = prefill(model, kv, pos[b], bts[b], toks[b:e + 1])
        for i in range(e - b + 1):
            rows[b + i] = (lg[i], tr[i], b)
        b = e + 1
    flipped = {}   # run start -> (first row with a near-tie flip, layer)
    for b in range(len(pos)):
        ol, tr, start = rows[b]
        fr = flipped.get(start)
        stop = L if fr is None else fr[1]
        for l in range(stop):
            lt = tr.layers[l]
            assert rel_l2(g["xs"][2 * l + 1, b], lt.x_attn) < 1e-2, ("x_attn", b, l)
            if not np.array_equal(g["ids"][l, b], lt.ids):
                assert routing_margin(lt.router_logits, CFG["top_k"]) < 1e-4, ("routing", b, l)
                flipped.setdefault(start, (b, l))
                break
            assert rel_l2(g["xs"][2 * l + 2, b], lt.x_out) < 1e-2, ("x_out", b, l)
        if fr is None and flipped.get(start) is None:
            assert np.max(np.abs(g["logits"][b] - ol)) <= 5e-2, ("logits", b)
    # the pool changed exactly at the written slots, to the oracle's rounding
    kb, vb = synth.bits(s.k0), synth.bits(s.v0)
    ka, va = synth.bits(g["k"]), synth.bits(g["v"])
    ck = {tuple(int(t) for t in x) for x in np.argwhere(np.any(ka != kb, axis=(2, 4)))}
    cv = {tuple(int(t) for t in x) for x in np.argwhere(np.any(va != vb, axis=(2, 3)))}
    want = {(l, bts[b][p // P], p % P) for l in range(L) for b, p in enumerate(pos)}
    assert ck <= want and cv <= want
    if not flipped:
        new = np.zeros(kb.shape, bool)
        for b, p in enumerate(pos):
            new[:, bts[b][p // P], :, p % P, :] = True
        for got, ref in ((ka, kv.k), (synth.bits(g["v"].transpose(-1, -2)), kv.v)):
            assert np.array_equal(got[~new], ref[~new])
            gv, wv = got[new], ref[new]
            wf = bf16_to_f32(wv)
            big = np.abs(wf) >= 0.1 * np.max(np.abs(wf))
            assert np.abs(gv.astype(np.int32) - wv.astype(np.int32))[big].max() <= 1
            assert rel_l2(bf16_to_f32(gv), wf) <= 5e-3
    return flipped


def test_prompt_block_after_a_cached_prefix(setup):
    """One sequence: 20 new tokens at positions 37..56 (three pages) after 37
    cached ones, one launch, matrix-core schedule."""
    tables = _tables(1, 3)
    ids, pos, bts, toks = _rows([(0, 37, 20, 5)], tables)
    g = _run(setup, ids, pos, bts, toks)
    _check(setup, ids, pos, bts, toks, g)


def test_prompt_from_an_empty_cache(setup):
    """A 33-token prompt from position 0: every key the rows read was written
    in the same launch."""
    tables = _tables(1, 4)
    ids, pos, bts, toks = _rows([(0, 0, 33, 6)], tables)
    g = _run(setup, ids, pos, bts, toks)
    _check(setup, ids, pos, bts, toks, g)


def test_mixed_prompts_and_decode_rows(setup):
    """Two prompt blocks and three decode rows in one batch (continuous
    batching: requests joining while others decode), both modes equal bit
    for bit and equal to the oracle."""
    tables = _tables(5, 7)
    runs = [(3, 50, 4, 11), (0, 17, 1, 12), (1, 0, 6, 13), (4, 90, 1, 14), (2, 33, 1, 15)]
    ids, pos, bts, toks = _rows(runs, tables)
    a = _run(setup, ids, pos, bts, toks)
    _check(setup, ids, pos, bts, toks, a)
    b = _run(setup, ids, pos, bts, toks, mk.MK_MODE_PEROP)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["xs"], b["xs"])
    assert torch.equal(a["k"], b["k"]) and torch.equal(a["v"], b["v"])


def test_two_token_block_on_the_dot_product_schedule(setup):
    """Two rows of one sequence on the one- and two-token schedule."""
    tables = _tables(1, 9)
    ids, pos, bts, toks = _rows([(0, 30, 2, 16)], tables)
    g = _run(setup, ids, pos, bts, toks, max_batch=2)
    _check(setup, ids, pos, bts, toks, g)


def test_malformed_runs_are_rejected_before_launch(setup):
    k, v = setup.fresh_pools()
    dec = mk.Decoder(CFG, setup.w_dev, k, v, max_batch=8, max_pages_per_seq=PAGES_PER_SEQ)
    tables = _tables(2, 10)
    tok = torch.zeros(4, dtype=torch.int32, device="cuda")
    lg = torch.empty(4, CFG["vocab"], device="cuda")
    bad = [([0, 0, 1, 0], [5, 6, 9, 7]),       # sequence 0's rows not adjacent
           ([0, 0, 0, 1], [5, 6, 8, 9]),       # positions not consecutive
           ]
    for ids, pos in bad:
        with pytest.raises(mk.MkError) as e:
            dec.forward(ids, pos, [tables[i] for i in ids], tok, lg)
        assert e.value.status == mk.MK_ERR_INVALID
    bts = [tables[0], [tables[0][0], tables[1][1]] + tables[0][2:], tables[1], tables[1]]
    with pytest.raises(mk.MkError):
        dec.forward([0, 0, 1, 1], [5, 20, 0, 1], bts, tok, lg)      # also not consecutive
    bts = [tables[0], list(tables[0]), tables[1], tables[1]]
    bts[1][0] = tables[1][5]                                        # a shared page that differs
    with pytest.raises(mk.MkError):
        dec.forward([0, 0, 1, 1], [5, 6, 0, 1], bts, tok, lg)
    assert dec.sync_check() == mk.MK_OK
    dec.close()
