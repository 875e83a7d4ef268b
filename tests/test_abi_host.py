"""CPU tests of the C ABI library: it loads, exports every declared entry
point, and its host task-graph builder produces valid, deadlock-free plans.
No device code runs here."""

import re
import os
import random
from collections import defaultdict

import numpy as np
import pytest

from persistent_megakernel_03_amd import configs, mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
(OP_EMBED, OP_QKV, OP_ATTN, OP_COMBINE, OP_OPROJ, OP_ROUTER, OP_ROUTE, OP_GATEUP, OP_DOWN, OP_MOESUM,
 OP_LMHEAD, OP_CLAIM, OP_FNORM) = range(13)
LEVELS_PER_LAYER = 9


def header_functions():
    import glob
    text = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = mk.load()
    names = header_functions()
    assert set(names) == set(mk.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_and_pool_sizes():
    d = mk.make_dims(configs.A3B, 1, 520, 520)
    assert mk.mk_kv_pool_bytes(d) == 48 * 520 * 4 * 16 * 128 * 2
    ws = mk.mk_workspace_bytes(d, mk.make_options())
    assert ws > 0
    # unsupported shapes report 0 bytes
    bad = dict(configs.A3B, head_dim=96)
    assert mk.mk_workspace_bytes(mk.make_dims(bad, 1, 520, 520), mk.make_options()) == 0


def simulate(tasks, offs, targets, rng):
    """Run the per-workgroup lists with a random interleaving and the counter
    protocol; a claim task takes tiles from its level's pool (past the lists)
    in pool order until none is left. Returns the final counters and the
    number of tiles run, or raises on deadlock."""
    n_wg = len(offs) - 1
    ctr = defaultdict(int)
    claimed = defaultdict(int)   # claim counter per level
    nxt = [int(offs[w]) for w in range(n_wg)]
    cur = [None] * n_wg  # pool tile a claim task is running
    stage = [0] * n_wg  # 0: before pre-wait, 1: before compute wait
    live = [w for w in range(n_wg) if nxt[w] < offs[w + 1]]
    steps = 0

    def advance(w):
        nxt[w] += 1
        if nxt[w] >= offs[w + 1]:
            live.remove(w)

    while live:
        progressed = False
        rng.shuffle(live)
        for w in list(live):
            t = tasks[nxt[w]]
            if int(t[0]) == OP_CLAIM and cur[w] is None:
                j = claimed[int(t[4])]
                claimed[int(t[4])] += 1
                progressed = True
                if j >= int(t[3]):
                    advance(w)
                    continue
                cur[w] = int(t[2]) + j
            tile = tasks[cur[w]] if cur[w] is not None else t
            op, layer, a0, a1, a2, a3, pre_c, pre_t, c, tg, sig, lvl = [int(v) for v in tile]
            if stage[w] == 0:
                if pre_c >= 0 and ctr[pre_c] < pre_t:
                    continue
                stage[w] = 1
            if c >= 0 and ctr[c] < tg:
                continue
            # run the tile
            if sig >= 0:
                ctr[sig] += 1
            stage[w] = 0
            progressed = True
            steps += 1
            if cur[w] is not None:
                cur[w] = None
            else:
                advance(w)
        if not progressed:
            raise RuntimeError("deadlock")
    return ctr, steps


@pytest.mark.parametrize("cfg_name,batch,positions,n_wg", [
    ("TINY", 1, [64], 16),
    ("TINY", 2, [5, 70], 7),
    ("TINY", 1, [0], 512),
    ("A3B", 1, [8192], 512),
    ("A3B", 2, [100, 3000], 256),
    ("TINY", 3, [64, 0, 17], 16),
    ("TINY", 8, [5, 70, 64, 63, 1, 0, 127, 300], 512),
    ("A3B", 4, [8192, 100, 3000, 5], 512),
])
@pytest.mark.parametrize("shared", [-1, 0, 2])
def test_plan_is_valid_and_deadlock_free(cfg_name, batch, positions, n_wg, shared):
    cfg = configs.dims_of(cfg_name)
    d = mk.make_dims(cfg, max(2, batch), 600, 1200)
    info, tasks, offs, targets = mk.mk_plan_build(d, mk.make_options(shared_levels=shared), n_wg, positions)
    assert info.n_tasks == len(tasks) and offs[-1] <= len(tasks)
    # each workgroup list is in non-decreasing dependency level
    for w in range(n_wg):
        lv = tasks[offs[w]:offs[w + 1], 11]
        assert np.all(np.diff(lv) >= 0)
    # claim tasks (batches of 3+ only) name pools past the lists
    claims = tasks[:offs[-1]][tasks[:offs[-1], 0] == OP_CLAIM]
    assert np.all(claims[:, 2] >= offs[-1])
    if shared != 0:
        assert (len(claims) > 0) == (shared > 0 and batch > 2)
    if shared == 0 and len(claims):   # ragged contexts only
        assert OP_ATTN in set(tasks[claims[:, 2], 0])
    n_tiles = len(tasks) - len(claims)
    # the counters reach exactly their targets, whatever the interleaving
    for seed in range(1 if batch > 2 and cfg_name == "A3B" else (2 if cfg_name == "A3B" else 5)):
        ctr, steps = simulate(tasks, offs, targets, random.Random(seed))
        assert steps == n_tiles
        for c, t in enumerate(targets):
            assert ctr[c] == t, (c, ctr[c], t)
    # attention chunks cover every cached token plus the new one
    chunk = info.chunk_tokens
    for b in range(batch):
        att = tasks[(tasks[:, 0] == OP_ATTN) & (tasks[:, 2] == b) & (tasks[:, 1] == 0)]
        n = -(-(positions[b] + 1) // chunk)
        assert len(att) == cfg["n_kv_heads"] * n
        assert set(att[:, 5]) == {n}


def test_plan_counts_for_the_30b_shape():
    d = mk.make_dims(configs.A3B, 1, 520, 520)
    info, tasks, offs, targets = mk.mk_plan_build(d, mk.make_options(), 512, [8192])
    ops = np.bincount(tasks[:, 0], minlength=13)
    assert ops[OP_CLAIM] == 0                  # one- and two-token plans are fully static
    assert ops[OP_EMBED] == 1
    assert ops[OP_QKV] == 48 * 4 * 54          # 1280 rows per KV group, 24 per tile
    assert ops[OP_ATTN] == 48 * 4 * 65         # 8193 tokens in 128-token chunks
    assert ops[OP_COMBINE] == 48 * 32          # one merge per query head
    assert ops[OP_OPROJ] == 48 * 256
    assert ops[OP_ROUTER] == 48 * 16
    assert ops[OP_GATEUP] == 48 * 8 * 64       # 8 slots x 768 rows / 12: one per workgroup
    assert ops[OP_DOWN] == 48 * 256            # 2048 rows / 8: 8 experts x 8 rows per tile held in registers
    # every workgroup one gate/up tile per layer, the down tiles on the lower half
    wg = np.repeat(np.arange(512), np.diff(offs))
    for l in (0, 20, 47):
        gu = wg[(tasks[:, 0] == OP_GATEUP) & (tasks[:, 1] == l)]
        dn = wg[(tasks[:, 0] == OP_DOWN) & (tasks[:, 1] == l)]
        assert sorted(gu.tolist()) == list(range(512))
        assert sorted(dn.tolist()) == list(range(256))
    assert ops[OP_LMHEAD] == -(-151936 // 64)
    assert ops[OP_ROUTE] == 0 and ops[OP_MOESUM] == 0 and ops[OP_FNORM] == 0
    assert info.n_levels == 3 + LEVELS_PER_LAYER * 48   # the final-norm level is empty here


@pytest.mark.parametrize("batch", [4, 16, 64])
def test_plan_counts_for_30b_batches(batch):
    # batches of 3+: every weight product in 16-row matrix-core blocks, one
    # routing tile; router tiles are (8 expert rows, one 16-token block)
    # pairs. Gate/up tiles are (rb 8-row blocks, slot group) pairs and down
    # tiles (rb 16-row blocks, slot group): rb = 2 where the expected distinct
    # experts, 128 (1 - (120/128)^B), reach 7 per gate/up slot group (126 at
    # B = 64 over 16 groups), else 1 (83 at B = 16 over 8 groups)
    rb = 2 if batch == 64 else 1
    d = mk.make_dims(configs.A3B, batch, 520, 520 * batch)
    info, tasks, offs, targets = mk.mk_plan_build(d, mk.make_options(), 512, [8192] * batch)
    ops = np.bincount(tasks[:, 0], minlength=13)
    assert ops[OP_EMBED] == -(-batch // 4)
    assert ops[OP_QKV] == 48 * 4 * 80          # 1280 rows per KV group, 16 per tile
    assert ops[OP_COMBINE] == 48 * 32 * batch
    assert ops[OP_OPROJ] == 48 * 256           # 8 rows per tile
    assert ops[OP_ROUTER] == 48 * 16 * -(-batch // 16)
    rt = tasks[(tasks[:, 0] == OP_ROUTER) & (tasks[:, 1] == 0)]
    assert set((rt[:, 4] >> 16).tolist()) == set(range(-(-batch // 16)))   # token blocks
    assert set((rt[:, 4] & 0xffff).tolist()) == set(range(0, 256, 16))   # 8-element groups of the expert input
    assert ops[OP_ROUTE] == 48
    assert ops[OP_GATEUP] == 48 * (96 // rb) * (8 * rb)     # 8 rb rows per tile x 8 rb slot groups
    assert ops[OP_DOWN] == 48 * (128 // rb) * (4 * rb)      # 16 rb rows per tile x 4 rb slot groups
    assert ops[OP_MOESUM] == 48 * 128
    assert ops[OP_FNORM] == batch                  # the final norm, one tile per token
    assert ops[OP_LMHEAD] == -(-151936 // 32)
    att = tasks[tasks[:, 0] == OP_ATTN]
    assert len(att) == 48 * batch * 4 * att[0, 5]
    # down slot groups: every slot in exactly one group
    dn = tasks[(tasks[:, 0] == OP_DOWN) & (tasks[:, 1] == 0)]
    assert set(dn[:, 5]) == {4 * rb} and set(dn[:, 4]) == set(range(4 * rb))
    assert set((dn[:, 3] - dn[:, 2]).tolist()) == {16 * rb}
    gu = tasks[(tasks[:, 0] == OP_GATEUP) & (tasks[:, 1] == 0)]
    assert set(gu[:, 5]) == {8 * rb} and set(gu[:, 4]) == set(range(8 * rb))
    assert set((gu[:, 3] - gu[:, 2]).tolist()) == {8 * rb}


@pytest.mark.parametrize("rb", [1, 2])
def test_plan_row_blocks_option(rb):
    # forced row blocks per matrix-core expert tile: gate/up tiles of 8 rb
    # rows, down tiles of 16 rb rows (the last one partial where the size is
    # not a multiple), every tile still covering each slot group exactly once
    d = mk.make_dims(configs.TINY, 8, 8, 64)
    pos = [5, 9, 33, 70, 1, 0, 2, 3]
    o = mk.make_options(mm_row_blocks=rb)
    info, tasks, offs, targets = mk.mk_plan_build(d, o, 64, pos)
    gu = tasks[(tasks[:, 0] == OP_GATEUP) & (tasks[:, 1] == 0)]
    dn = tasks[(tasks[:, 0] == OP_DOWN) & (tasks[:, 1] == 0)]
    assert set((gu[:, 3] - gu[:, 2]).tolist()) == {8 * rb}
    assert set((dn[:, 3] - dn[:, 2]).tolist()) == {16 * rb}
    mk.mk_plan_check(d, o, 64, pos, tasks, offs)


@pytest.mark.parametrize("batch,rb", [(32, 1), (33, 2)])
def test_row_block_choice_at_its_threshold(batch, rb):
    # two row blocks per gate/up tile once the expected distinct experts,
    # 128 (1 - (120/128)^B), reach 7 per slot group of the two-block plan
    # (16 groups): 111.77 at B = 32, 112.79 at B = 33
    expected = 128 * (1 - (120 / 128) ** batch)
    assert (expected >= 7 * 16) == (rb == 2)
    d = mk.make_dims(configs.A3B, batch, 520, 520 * batch)
    info, tasks, offs, targets = mk.mk_plan_build(d, mk.make_options(), 512, [8192] * batch)
    gu = tasks[(tasks[:, 0] == OP_GATEUP) & (tasks[:, 1] == 0)]
    assert set((gu[:, 3] - gu[:, 2]).tolist()) == {8 * rb}
    assert len(gu) == (96 // rb) * (8 * rb)


def test_plan_rejects_bad_row_blocks():
    d = mk.make_dims(configs.TINY, 8, 8, 64)
    for bad in (-1, 3):
        with pytest.raises(mk.MkError) as e:
            mk.mk_plan_build(d, mk.make_options(mm_row_blocks=bad), 64, [5] * 8)
        assert e.value.status == mk.MK_ERR_INVALID


def test_plan_rejects_bad_input():
    d = mk.make_dims(configs.TINY, 1, 8, 16)
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_build(d, mk.make_options(), 8, [1, 2])   # batch above max_batch
    assert e.value.status == mk.MK_ERR_CAPACITY
    bad = mk.make_dims(dict(configs.TINY, page_size=32), 1, 8, 16)
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_build(bad, mk.make_options(), 8, [1])
    assert e.value.status == mk.MK_ERR_UNSUPPORTED


@pytest.mark.parametrize("cfg_name,batch,positions,shared", [
    ("A3B", 1, [8192], 0), ("TINY", 2, [5, 70], 0), ("TINY", 8, [5, 70, 64, 63, 1, 0, 127, 300], 2),
    ("A3B", 4, [8192, 100, 3000, 5], 0)])
def test_plan_check_accepts_built_plans_and_finds_missing_dependencies(cfg_name, batch, positions, shared):
    """mk_plan_check passes the builder's own plans; planted mistakes that keep
    every counter target and level order intact (so only the read-coverage
    rule can see them) are rejected: an attention tile waiting on another KV
    group's QKV counter, a down tile waiting on the router instead of the
    gate/up tiles, a merge tile waiting on another group's attention."""
    cfg = configs.dims_of(cfg_name)
    d = mk.make_dims(cfg, max(2, batch), 600, 1200)
    o = mk.make_options(shared_levels=shared)
    info, tasks, offs, targets = mk.mk_plan_build(d, o, 512, positions)
    mk.mk_plan_check(d, o, 512, positions, tasks, offs)
    Hkv, L = cfg["n_kv_heads"], cfg["n_layers"]
    per = 2 * Hkv + 7
    qkv_ctr = lambda l, g: 1 + l * per + g
    attn_ctr = lambda l, g: 1 + l * per + Hkv + g
    router_ctr = lambda l: 1 + l * per + 2 * Hkv + 2
    l = L - 1

    def planted(pick, change):
        t = tasks.copy()
        idx = [i for i in range(len(t)) if pick(t[i])]
        assert idx
        change(t[idx[0]])
        with pytest.raises(mk.MkError) as e:
            mk.mk_plan_check(d, o, 512, positions, t, offs)
        assert e.value.status == mk.MK_ERR_INVALID and "reads" in str(e.value)

    def other_group(t):
        t[8] = qkv_ctr(t[1], (t[3] + 1) % Hkv)

    planted(lambda t: t[0] == OP_ATTN and t[1] == l and t[8] == qkv_ctr(l, t[3]), other_group)

    def to_other_attn(t):
        g = t[8] - (1 + t[1] * per + Hkv)
        t[8] = attn_ctr(t[1], (g + 1) % Hkv)
        t[9] = int(targets[t[8]])

    planted(lambda t: t[0] == OP_COMBINE and t[1] == l, to_other_attn)
    if batch <= 2:
        def down_on_router(t):
            t[8], t[9] = router_ctr(t[1]), int(targets[router_ctr(t[1])])
        planted(lambda t: t[0] == OP_DOWN and t[1] == l, down_on_router)


@pytest.mark.parametrize("cfg_name", ["TINY", "A3B"])
@pytest.mark.parametrize("max_batch", [1, 2, 3, 8])
@pytest.mark.parametrize("mmb", [0, 1, 3])
def test_every_plan_fits_the_task_capacity(cfg_name, max_batch, mmb):
    # the task buffer a handle reserves is sized once, for any batch and
    # context; the plans of every batch up to max_batch at the longest and
    # shortest contexts fit it on every workgroup count
    cfg = configs.dims_of(cfg_name)
    max_pages = 520 if cfg_name == "A3B" else 40
    d = mk.make_dims(cfg, max_batch, max_pages, max_pages * max_batch)
    o = mk.make_options(mfma_min_batch=mmb)
    longest = max_pages * cfg["page_size"] - 1
    for n_wg in (7, 64, 256, 512):
        for b in sorted({1, 2, max_batch} & set(range(1, max_batch + 1))):
            for pos in ([0] * b, [longest] * b, [longest] + [0] * (b - 1)):
                info, tasks, offs, targets = mk.mk_plan_build(d, o, n_wg, pos)
                assert 0 < info.n_tasks <= info.cap_tasks, (n_wg, b, pos[0], info.n_tasks, info.cap_tasks)


def test_plan_check_rejects_router_token_blocks():
    # batches above 16 tokens: router tiles per 16-token block; a tile moved
    # to another block leaves its own block's expert rows uncovered
    d = mk.make_dims(configs.A3B, 32, 520, 520 * 32)
    o = mk.make_options()
    positions = [8192] * 32
    info, tasks, offs, targets = mk.mk_plan_build(d, o, 512, positions)
    mk.mk_plan_check(d, o, 512, positions, tasks, offs)
    t = tasks.copy()
    i = int(np.flatnonzero((t[:, 0] == OP_ROUTER) & ((t[:, 4] >> 16) == 1))[0])
    t[i, 4] &= 0xffff
    t[i, 5] &= 0xffff
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_check(d, o, 512, positions, t, offs)
    assert e.value.status == mk.MK_ERR_INVALID
