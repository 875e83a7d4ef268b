"""The exchange-buffer poison mode (mk_options.poison_exchange) as a
read-before-write detector: every float buffer that carries data between
tiles is filled with NaN before the step, so a tile that read such data
before its producer wrote it in this step would make the outputs NaN. With
every read covered by a wait, the poisoned step equals the plain one bit for
bit. Tiny MoE decoder, through the C ABI: one and two tokens (the GEMV
tiles), ragged batches of 8 and 17 (the matrix-core tiles, shared levels),
a prompt block after a cached prefix, both modes.
"""

import numpy as np
import pytest
import torch

from persistent_megakernel_03_amd import configs, mk, synth
from tests.gpu_setup import Setup, x_layers

pytestmark = pytest.mark.gpu

CFG = configs.TINY
PAGES_PER_SEQ = 7
N_PAGES = 24 * PAGES_PER_SEQ + 8


@pytest.fixture(scope="module")
def setup():
    torch.manual_seed(0)
    return Setup(CFG, n_pages=N_PAGES, seed=0)


def _run(s, positions, bts, toks, poison, mode, seq_ids=None, forward=False):
    B = len(positions)
    k, v = s.fresh_pools()
    dec = mk.Decoder(CFG, s.w_dev, k, v, max_batch=max(B, 3), max_pages_per_seq=PAGES_PER_SEQ, mode=mode,
                     validate_plans=True, poison_exchange=poison)
    tokens = torch.tensor(toks, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, CFG["vocab"], device="cuda")
    print(f"poison={poison} mode={mode} rows={B} forward={forward}", flush=True)
    if forward:
        dec.forward(seq_ids, positions, bts, tokens, logits)
    else:
        dec.step(positions, bts, tokens, logits)
    assert dec.sync_check() == mk.MK_OK
    out = dict(logits=logits.cpu().numpy(), xs=x_layers(dec).cpu().numpy()[:, :B], k=synth.bits(k.cpu()),
               v=synth.bits(v.cpu()))
    dec.close()
    return out


def _same(a, b):
    assert np.all(np.isfinite(a["logits"])) and np.all(np.isfinite(a["xs"]))
    assert np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["xs"], b["xs"])
    assert np.array_equal(a["k"], b["k"]) and np.array_equal(a["v"], b["v"])


def _batch(B, seed):
    rng = np.random.default_rng(2000 + seed)
    positions = [int(x) for x in rng.integers(0, 96, size=B)]
    bts = synth.make_block_tables(B, PAGES_PER_SEQ, N_PAGES, seed=seed, shuffle=True).tolist()
    toks = [int(t) for t in synth.make_tokens(B, CFG["vocab"], seed=seed)]
    return positions, bts, toks


@pytest.mark.parametrize("B", [1, 2, 8, 17])
@pytest.mark.parametrize("mode", [mk.MK_MODE_MEGAKERNEL, mk.MK_MODE_PEROP])
def test_poisoned_step_equals_plain_step(setup, B, mode):
    positions, bts, toks = _batch(B, B)
    _same(_run(setup, positions, bts, toks, True, mode), _run(setup, positions, bts, toks, False, mode))


def test_poisoned_prompt_block_equals_plain(setup):
    # a 6-token prompt block after 40 cached tokens, and one decode row
    bts = synth.make_block_tables(2, PAGES_PER_SEQ, N_PAGES, seed=5, shuffle=True).tolist()
    ids = [0] * 6 + [1]
    pos = [40 + i for i in range(6)] + [70]
    toks = [int(t) for t in synth.make_tokens(7, CFG["vocab"], seed=9)]
    rows_bt = [bts[i] for i in ids]
    a = _run(setup, pos, rows_bt, toks, True, mk.MK_MODE_MEGAKERNEL, seq_ids=ids, forward=True)
    b = _run(setup, pos, rows_bt, toks, False, mk.MK_MODE_MEGAKERNEL, seq_ids=ids, forward=True)
    _same(a, b)
