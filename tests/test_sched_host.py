"""CPU tests of the host continuous-batching scheduler (include/mk_sched.h),
driven with a stand-in for the model (the next token is a fixed function of
the fed token and position), so every invariant of the host state can be
checked step by step: disjoint pages, runs of consecutive positions, the
tokens fed, admission and finishing, capacity errors."""

import numpy as np
import pytest

from persistent_megakernel_03_amd import mk

V = 1000
P = 16


def fake_next(tok, pos):
    return (int(tok) * 31 + int(pos) * 7 + 3) % V


def drive(sch, n_pages, max_steps=500, on_step=None):
    """Run the scheduler to completion with the stand-in model. Returns
    {request: generated tokens} and the per-step row counts."""
    gen, rows_per_step = {}, []
    for step in range(max_steps):
        n = sch.next()
        if n == 0:
            break
        rows_per_step.append(n)
        ids, pos = sch.seq_ids[:n].copy(), sch.positions[:n].copy()
        bts, toks, smp, rid = (sch.block_tables[:n].copy(), sch.tokens[:n].copy(), sch.sample[:n].copy(),
                               sch.request_ids[:n].copy())
        check_rows(ids, pos, bts, rid, n_pages)
        nxt = np.array([fake_next(t, p) for t, p in zip(toks, pos)], np.int32)
        for b in range(n):
            if smp[b]:
                gen.setdefault(int(rid[b]), []).append(int(nxt[b]))
        if on_step:
            on_step(step, n, ids, pos, bts, toks, smp, rid)
        sch.commit(nxt)
    return gen, rows_per_step


def check_rows(ids, pos, bts, rid, n_pages):
    n = len(ids)
    owner = {}
    b = 0
    while b < n:
        e = b
        while e + 1 < n and ids[e + 1] == ids[b]:
            e += 1
        # one run: one request, consecutive positions, one table
        assert len(set(rid[b:e + 1].tolist())) == 1
        assert np.array_equal(pos[b:e + 1], np.arange(pos[b], pos[b] + e - b + 1))
        for i in range(b, e + 1):
            assert np.array_equal(bts[i], bts[b])
        used = bts[b][:pos[e] // P + 1]
        assert np.all((used >= 0) & (used < n_pages))
        assert len(set(used.tolist())) == len(used)
        for pg in used.tolist():
            assert owner.setdefault(pg, int(rid[b])) == int(rid[b]), "page shared by two requests"
        b = e + 1
    # runs have distinct seq ids
    starts = [0] + [i for i in range(1, n) if ids[i] != ids[i - 1]]
    assert len({int(ids[i]) for i in starts}) == len(starts)


def reference(prompt, max_new, cached=0):
    """The tokens the stand-in model generates for one request fed alone."""
    toks, out = list(prompt), []
    for i in range(len(prompt) + max_new - 1):
        if i >= len(toks):
            break
        nxt = fake_next(toks[i], cached + i)
        if i >= len(prompt) - 1 and len(out) < max_new:
            out.append(nxt)
            toks.append(nxt)
    return out


def make(n_pages=4096, max_seqs=8, max_rows=32, max_pages=64, reserve=True, order=None):
    return mk.Scheduler(max_seqs, max_rows, P, max_pages, n_pages, reserve_full=reserve, page_order=order)


def test_requests_generate_what_they_would_alone():
    rng = np.random.default_rng(0)
    sch = make()
    reqs = {}
    for r in range(20):
        plen, mnew = int(rng.integers(1, 90)), int(rng.integers(1, 40))
        prompt = [int(x) for x in rng.integers(0, V, size=plen)]
        reqs[r] = (prompt, mnew)
        sch.submit(r, prompt, mnew)
    gen, rows = drive(sch, 4096)
    assert max(rows) <= 32
    for r, (prompt, mnew) in reqs.items():
        assert gen[r] == reference(prompt, mnew), r
        assert sch.tokens_of(r) == prompt + gen[r]
    st = sch.stats()
    assert st["finished"] == 20 and st["running"] == 0 and st["queued"] == 0 and st["free_pages"] == 4096
    assert st["prompt_rows"] == sum(len(p) for p, _ in reqs.values())


def test_long_prompts_are_chunked_and_decode_rows_keep_running():
    sch = make(max_seqs=4, max_rows=16)
    sch.submit(0, [5], 30)                       # decodes from the first step
    sch.submit(1, list(range(100)), 3)           # 100-token prompt: chunks of what the rows leave
    seen = []
    drive(sch, 4096, on_step=lambda step, n, ids, pos, bts, toks, smp, rid: seen.append((n, rid.tolist())))
    # request 0 has a decode row in every step until it finishes; the prompt fills the rest
    for n, rid in seen[:6]:
        assert n == 16 and rid.count(0) == 1
    assert sum(rid.count(1) for _, rid in seen) == 100 + 2


def test_admission_is_first_come_and_waits_for_pages():
    # 10 pages: request 0 reserves 4, request 1 (needs 8) must wait, and blocks request 2 behind it
    sch = make(n_pages=10, max_seqs=4, reserve=True)
    sch.submit(0, list(range(40)), 20)           # 59 positions -> 4 pages
    sch.submit(1, list(range(100)), 20)          # 119 -> 8 pages
    sch.submit(2, [1], 1)                        # 1 page, but queued behind 1
    n = sch.next()
    assert set(sch.request_ids[:n].tolist()) == {0}
    st = sch.stats()
    assert st["running"] == 1 and st["queued"] == 2
    sch.commit(np.zeros(n, np.int32))
    gen, _ = drive(sch, 10)
    assert sch.stats()["finished"] == 3


def test_without_reservation_a_full_pool_is_a_capacity_error_until_release():
    sch = make(n_pages=6, max_seqs=4, reserve=False)
    sch.submit(0, [1] * 30, 200)                 # grows a page every 16 tokens
    sch.submit(1, [2] * 30, 200)
    with pytest.raises(mk.MkError) as e:
        for _ in range(100):
            n = sch.next()
            sch.commit(np.zeros(n, np.int32))
    assert e.value.status == mk.MK_ERR_CAPACITY
    sch.release(1)
    n = sch.next()
    assert n == 1 and sch.request_ids[0] == 0


def test_released_slots_are_reused_by_joining_requests():
    sch = make(max_seqs=3)
    for r in range(3):
        sch.submit(r, [r + 1], 100, cached_len=50 + r)
    n = sch.next()
    assert sch.seq_ids[:n].tolist() == [0, 1, 2] and sch.positions[:n].tolist() == [50, 51, 52]
    sch.commit(np.zeros(n, np.int32))
    sch.release(1)
    sch.submit(7, [9], 5, cached_len=300)
    n = sch.next()
    assert sch.request_ids[:n].tolist() == [0, 7, 2] and sch.positions[:n].tolist() == [51, 300, 53]
    assert sch.tokens[1] == 9


def test_pages_follow_the_given_order_and_come_back():
    order = np.random.default_rng(3).permutation(64)
    sch = make(n_pages=64, max_seqs=2, reserve=False, order=order)
    sch.submit(0, [1], 3, cached_len=40)         # positions 0..40: pages order[0..2]
    n = sch.next()
    assert sch.block_tables[0][:3].tolist() == order[:3].tolist()
    sch.commit(np.zeros(n, np.int32))
    sch.release(0)
    assert sch.stats()["free_pages"] == 64


@pytest.mark.parametrize("bad", ["dup", "len", "cap"])
def test_bad_submissions(bad):
    sch = make(max_pages=4)
    sch.submit(0, [1], 1)
    with pytest.raises(mk.MkError) as e:
        if bad == "dup":
            sch.submit(0, [1], 1)
        elif bad == "len":
            sch.submit(1, [], 1)
        else:
            sch.submit(2, [1] * 60, 10)          # 69 positions > 4 pages
    assert e.value.status == (mk.MK_ERR_CAPACITY if bad == "cap" else mk.MK_ERR_INVALID)


def test_commit_needs_a_pending_step_and_pending_requests_cannot_be_released():
    sch = make()
    with pytest.raises(mk.MkError):
        sch.commit([])
    sch.submit(0, [1, 2], 2)
    n = sch.next()
    with pytest.raises(mk.MkError):
        sch.release(0)
    sch.commit(np.zeros(n, np.int32))
    sch.release(0)


def test_churn_run_keeps_slots_and_positions():
    """The churning workload on the scheduler: 32 rows every step, in slot
    order; after each churn the new requests sit in the released slots at
    their drawn contexts with their first tokens."""
    from persistent_megakernel_03_amd import synth
    w = synth.ChurnWorkload(32, V, seed=3)
    ref = synth.ChurnWorkload(32, V, seed=3)
    sch = make(n_pages=40000, max_seqs=32, max_rows=32, max_pages=2200, reserve=False,
               order=np.random.default_rng(1).permutation(40000))
    run = synth.ChurnRun(sch, w, max_len=2200 * P)
    expect = {b: (ctx, tok) for b, (ctx, tok) in enumerate(ref.initial)}
    pos = {b: ctx for b, (ctx, _) in expect.items()}
    for step in range(1, 34):
        n = sch.next()
        assert n == 32 and sch.seq_ids[:n].tolist() == list(range(32))
        assert [int(sch.positions[b]) for b in range(32)] == [pos[b] for b in range(32)]
        check_rows(sch.seq_ids[:n], sch.positions[:n], sch.block_tables[:n], sch.request_ids[:n], 40000)
        for b in range(32):
            if pos[b] == expect[b][0]:
                assert sch.tokens[b] == expect[b][1]     # the request's first token
        sch.commit(np.arange(n, dtype=np.int32))
        pos = {b: p + 1 for b, p in pos.items()}
        joined = run.advance()
        for slot, ctx, tok in ref.after_step(step):
            assert slot in joined
            expect[slot] = (ctx, tok)
            pos[slot] = ctx
