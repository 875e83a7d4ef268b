"""Pins for the oracle's multi-token entry points, prefill and
decode_sequence (CPU only).

Both are written as decode steps in order. They are pinned here against an
independent formulation: a float64 torch forward of the whole block of new
tokens at once, with the cached prefix read out of the pool and a causal
mask over the block, attention by torch's scaled_dot_product_attention and
routing by torch.topk. It shares no code with the oracle. Agreement of every
row's logits and of the written KV slots fixes the positions each token is
fed at, the slot it writes, that token i sees new tokens 0..i and no later
one, and (for decode_sequence) that each fed token is the argmax of the
previous step. Planted mistakes (a position that does not advance, a
one-token-late chain) are shown to fail the same comparison.
"""

import numpy as np
import pytest
import torch

from oracle import DenseModel, PagedKV, bf16_to_f32, decode_sequence, decode_step, prefill
from persistent_megakernel_03_amd import configs, synth


def _np_model(dims, seed=0):
    t = synth.make_model(dims, seed, "cpu")
    return {k: synth.bits(v) for k, v in t.items()}


def _np_pool(dims, n_pages, seed=1):
    k, v = synth.make_kv_pool(dims, n_pages, seed, "cpu")
    return synth.bits(k), synth.bits(v)


def _bf16_rne64(x: torch.Tensor) -> torch.Tensor:
    """float64 -> BF16 (nearest, ties to even) -> float64, via torch's own
    conversion chain (float64 -> float32 -> bfloat16)."""
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _block_forward(d, tensors, kp, vp, pos0, bt, tokens):
    """All T tokens at once in float64. Returns (logits [T][V], new keys
    [L][T][Hkv][D] and values, both BF16-rounded)."""
    f = {k: torch.from_numpy(bf16_to_f32(v).astype(np.float64)) for k, v in tensors.items()}
    H, hq, hkv, D = d["hidden"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"]
    E, K, P = d["n_experts"], d["top_k"], d["page_size"]
    eps, theta = d["rms_eps"], d["rope_theta"]
    T = len(tokens)
    n_ctx = pos0 + T

    def norm(x, g):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * g

    pos = torch.arange(pos0, pos0 + T, dtype=torch.float64)
    inv = theta ** (-2.0 * torch.arange(D // 2, dtype=torch.float64) / D)
    ang = pos[:, None] * inv[None, :]
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rot(u):  # [T][heads][D]
        a, b = u[..., :D // 2], u[..., D // 2:]
        return torch.cat([a * cos - b * sin, a * sin + b * cos], -1)

    # causal mask over [prefix | block]: row i sees the prefix and block 0..i
    mask = torch.ones(T, n_ctx, dtype=torch.bool)
    mask[:, pos0:] = torch.tril(torch.ones(T, T, dtype=torch.bool))
    x = f["embed"][torch.as_tensor(np.asarray(tokens, np.int64))]
    ks, vs = [], []
    for l in range(d["n_layers"]):
        p = f"layers.{l}."
        h = norm(x, f[p + "attn_norm"])
        qkv = h @ f[p + "wqkv"].T
        q = rot(qkv[:, :hq * D].reshape(T, hq, D))
        k = _bf16_rne64(rot(qkv[:, hq * D:(hq + hkv) * D].reshape(T, hkv, D)))
        v = _bf16_rne64(qkv[:, (hq + hkv) * D:].reshape(T, hkv, D))
        ks.append(k)
        vs.append(v)
        pk = torch.from_numpy(bf16_to_f32(np.stack([kp[l, bt[t // P], :, t % P, :] for t in range(pos0)]
                                                   or [np.zeros((hkv, D), np.uint16)])).astype(np.float64))[:pos0]
        pv = torch.from_numpy(bf16_to_f32(np.stack([vp[l, bt[t // P], :, t % P, :] for t in range(pos0)]
                                                   or [np.zeros((hkv, D), np.uint16)])).astype(np.float64))[:pos0]
        keys = torch.cat([pk, k], 0).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)   # [hq][n_ctx][D]
        vals = torch.cat([pv, v], 0).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        o = torch.nn.functional.scaled_dot_product_attention(q.permute(1, 0, 2), keys, vals, attn_mask=mask)
        x = x + o.permute(1, 0, 2).reshape(T, hq * D) @ f[p + "wo"].T
        h2 = norm(x, f[p + "ffn_norm"])
        r = h2 @ f[p + "router"].T
        top, ids = torch.topk(r, K, dim=-1)
        w = torch.softmax(top, -1)
        y = torch.zeros_like(x)
        for t in range(T):
            for j in range(K):
                e = int(ids[t, j])
                g_ = f[p + "w_gate"][e] @ h2[t]
                u_ = f[p + "w_up"][e] @ h2[t]
                y[t] += w[t, j] * (f[p + "w_down"][e] @ (g_ / (1 + torch.exp(-g_)) * u_))
        x = x + y
    logits = norm(x, f["final_norm"]) @ f["lm_head"].T
    return logits.numpy(), torch.stack(ks).numpy(), torch.stack(vs).numpy()


@pytest.fixture(scope="module")
def tiny():
    d = configs.TINY
    return d, _np_model(d, seed=0)


CASE = dict(pos0=37, T=21, bt=[6, 2, 9, 0, 4], n_pages=10)   # the block crosses three pages


def _slots_written(before, after):
    return {(int(a), int(b), int(c)) for a, b, c in np.argwhere(np.any(before != after, axis=(2, 4)))}


def test_prefill_matches_the_causal_block_forward(tiny):
    d, tensors = tiny
    P, pos0, T, bt = d["page_size"], CASE["pos0"], CASE["T"], CASE["bt"]
    kp, vp = _np_pool(d, CASE["n_pages"])
    toks = [int(t) for t in synth.make_tokens(T, d["vocab"], seed=21)]
    kv = PagedKV(kp.copy(), vp.copy(), P)
    lg, tr = prefill(DenseModel.from_dict(d, tensors, np.float64), kv, pos0, bt, toks, np.float64)
    ref, knew, vnew = _block_forward(d, tensors, kp, vp, pos0, bt, toks)
    assert lg.shape == (T, d["vocab"]) and len(tr) == T
    err = np.max(np.abs(lg - ref)) / np.max(np.abs(ref))
    assert err < 1e-9, err
    # the block wrote exactly its T slots in every layer, with the block forward's BF16 keys and values
    want = {(l, bt[(pos0 + i) // P], (pos0 + i) % P) for l in range(d["n_layers"]) for i in range(T)}
    assert _slots_written(kp, kv.k) == want and _slots_written(vp, kv.v) == want
    for l in range(d["n_layers"]):
        for i in range(T):
            t = pos0 + i
            assert np.array_equal(bf16_to_f32(kv.k[l, bt[t // P], :, t % P, :]).astype(np.float64), knew[l, i])
            assert np.array_equal(bf16_to_f32(kv.v[l, bt[t // P], :, t % P, :]).astype(np.float64), vnew[l, i])


def test_prefill_float32_is_sequential_decode_at_float32(tiny):
    """The default precision: float32 over BF16 weights, the block's rows
    within float32 rounding of the float64 block forward."""
    d, tensors = tiny
    P, pos0, T, bt = d["page_size"], 16, 9, [3, 1, 0]
    kp, vp = _np_pool(d, 5)
    toks = [5, 900, 77, 5, 5, 1023, 0, 64, 300]
    lg, _ = prefill(DenseModel.from_dict(d, tensors), PagedKV(kp.copy(), vp.copy(), P), pos0, bt, toks)
    ref, _, _ = _block_forward(d, tensors, kp, vp, pos0, bt, toks)
    assert lg.dtype == np.float32
    assert np.max(np.abs(lg - ref)) <= 1e-3 * np.max(np.abs(ref))


def test_a_block_forward_with_shifted_positions_is_rejected(tiny):
    """The comparison above is sharp: feeding the same block one position
    later (a prefill that skipped a slot) moves every row's logits."""
    d, tensors = tiny
    P, pos0, T, bt = d["page_size"], 20, 6, [0, 1, 2]
    kp, vp = _np_pool(d, 3)
    toks = [1, 2, 3, 4, 5, 6]
    lg, _ = prefill(DenseModel.from_dict(d, tensors, np.float64), PagedKV(kp.copy(), vp.copy(), P), pos0, bt, toks,
                    np.float64)
    bad, _, _ = _block_forward(d, tensors, kp, vp, pos0 + 1, bt, toks)
    assert np.min(np.max(np.abs(lg - bad), axis=1)) > 1e-6


def test_decode_sequence_is_the_greedy_chain(tiny):
    d, tensors = tiny
    P, pos0, n, bt = d["page_size"], 45, 7, [2, 0, 4, 1]
    kp, vp = _np_pool(d, 5)
    kv = PagedKV(kp.copy(), vp.copy(), P)
    logits, toks, traces = decode_sequence(DenseModel.from_dict(d, tensors, np.float64), kv, pos0, bt, 17, n,
                                           np.float64)
    assert len(toks) == n + 1 and toks[0] == 17 and logits.shape == (n, d["vocab"]) and len(traces) == n
    for i in range(n):
        assert toks[i + 1] == int(np.argmax(logits[i]))
    # step i ran at position pos0 + i on token i: the block forward of the fed tokens reproduces every row
    ref, knew, _ = _block_forward(d, tensors, kp, vp, pos0, bt, toks[:n])
    assert np.max(np.abs(logits - ref)) / np.max(np.abs(ref)) < 1e-9
    want = {(l, bt[(pos0 + i) // P], (pos0 + i) % P) for l in range(d["n_layers"]) for i in range(n)}
    assert _slots_written(kp, kv.k) == want
    for i, tr in enumerate(traces):
        assert {(lt.kv_page, lt.kv_slot) for lt in tr.layers} == {(bt[(pos0 + i) // P], (pos0 + i) % P)}


def test_planted_chain_mistakes_fail_the_block_comparison(tiny):
    """Two plausible bugs of a greedy loop, planted on the CPU: a position
    that never advances (every step rewrites one slot) disagrees with the
    block forward of the tokens it fed; a chain that feeds each token one
    step late fails the argmax check of test_decode_sequence_is_the_greedy_chain."""
    d, tensors = tiny
    P, pos0, n, bt = d["page_size"], 30, 4, [1, 3, 0]
    kp, vp = _np_pool(d, 4)
    model = DenseModel.from_dict(d, tensors, np.float64)

    def chain(advance, lag):
        kv = PagedKV(kp.copy(), vp.copy(), P)
        toks, rows, fed = [9], [], []
        for i in range(n):
            tok = toks[max(0, len(toks) - 1 - lag)]
            fed.append(tok)
            lg, _, _ = decode_step(model, kv, [pos0 + (i if advance else 0)], [bt], [tok], np.float64)
            rows.append(lg[0])
            toks.append(int(np.argmax(lg[0])))
        return np.stack(rows), fed

    good, fed = chain(True, 0)
    ref, _, _ = _block_forward(d, tensors, kp, vp, pos0, bt, fed)
    assert np.max(np.abs(good - ref)) / np.max(np.abs(ref)) < 1e-9
    stuck, fed_stuck = chain(False, 0)
    ref_stuck, _, _ = _block_forward(d, tensors, kp, vp, pos0, bt, fed_stuck)
    assert np.max(np.abs(stuck - ref_stuck)) / np.max(np.abs(ref_stuck)) > 1e-3
    late, fed_late = chain(True, 1)
    assert any(fed_late[i + 1] != int(np.argmax(late[i])) for i in range(n - 1))


def test_decode_sequence_resolves_an_exact_tie_to_the_lowest_index(tiny):
    """An LM head whose only non-zero rows are 5 and 9, both equal to c * e_0:
    logits 5 and 9 are the same product (exactly equal), the rest are 0. The
    next token is 5 when that product is positive, else 0 (the lowest of the
    zeros)."""
    d, tensors = tiny
    P, pos0, bt = d["page_size"], 10, [0, 1]
    t2 = dict(tensors)
    lm = np.zeros_like(tensors["lm_head"])
    lm[5, 0] = lm[9, 0] = 0x4000   # BF16 2.0
    t2["lm_head"] = lm
    kp, vp = _np_pool(d, 2)
    logits, toks, traces = decode_sequence(DenseModel.from_dict(d, t2), PagedKV(kp, vp, P), pos0, bt, 3, 3)
    for i in range(3):
        assert logits[i][5] == logits[i][9]
        assert np.count_nonzero(logits[i]) == (2 if logits[i][5] != 0 else 0)
        assert toks[i + 1] == (5 if logits[i][5] > 0 else 0)
