"""Pins for the oracle's whole decode step (CPU only).

* a pure-Python float64 brute force of a micro model, written with explicit
  loops over a contiguous (unpaged) cache;
* invariants: paged == contiguous, batch == one sequence at a time,
  determinism and idempotence, the step writes exactly one KV slot per layer;
* byte accounting: the oracle's counted bytes equal the closed form.
"""

import math
import struct

import numpy as np
import pytest

from oracle import (DenseModel, PagedKV, attention_block, bf16_to_f32, decode_sequence, decode_step, final_logits,
                    moe_block, rope_cos_sin, route_weights)
from oracle.decode import LayerTrace
from persistent_megakernel_03_amd import configs, sol, synth


def _np_model(dims, seed=0, router_bias=None):
    t = synth.make_model(dims, seed, "cpu", router_bias)
    out = {}
    for k, v in t.items():
        out[k] = synth.bits(v) if v.dtype.is_floating_point and v.element_size() == 2 else v.numpy()
    return out


def _np_pool(dims, n_pages, seed=1):
    k, v = synth.make_kv_pool(dims, n_pages, seed, "cpu")
    return synth.bits(k), synth.bits(v)


# ------------------------------------------------------------ brute force ---

def _bf16_round(x: float) -> float:
    """float64 -> float32 (nearest) -> BF16 (nearest, ties to even), back to float."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def _brute_step(d, W, cache, pos, token):
    """Explicit-loop decode of one token. ``W`` holds nested Python lists of
    floats; ``cache[l]`` is a list of (k, v) per cached position, each
    [Hkv][D], already post-RoPE. Appends the new position's entries."""
    H, hq, hkv, D = d["hidden"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"]
    E, K, I = d["n_experts"], d["top_k"], d["moe_inter"]
    eps, theta = d["rms_eps"], d["rope_theta"]

    def rms(v, g):
        s = 0.0
        for a in v:
            s += a * a
        inv = 1.0 / math.sqrt(s / len(v) + eps)
        return [v[i] * inv * g[i] for i in range(len(v))]

    def mv(M, v):
        return [sum(M[i][j] * v[j] for j in range(len(v))) for i in range(len(M))]

    def rot(u):
        half = D // 2
        out = list(u)
        for i in range(half):
            ang = pos * theta ** (-2.0 * i / D)
            c, s = math.cos(ang), math.sin(ang)
            out[i] = u[i] * c - u[i + half] * s
            out[i + half] = u[i] * s + u[i + half] * c
        return out

    x = list(W["embed"][token])
    for l in range(d["n_layers"]):
        p = f"layers.{l}."
        h = rms(x, W[p + "attn_norm"])
        qkv = mv(W[p + "wqkv"], h)
        q = [rot(qkv[hh * D:(hh + 1) * D]) for hh in range(hq)]
        k = [rot(qkv[hq * D + g * D: hq * D + (g + 1) * D]) for g in range(hkv)]
        v = [qkv[(hq + hkv) * D + g * D: (hq + hkv) * D + (g + 1) * D] for g in range(hkv)]
        cache[l].append(([[_bf16_round(a) for a in kk] for kk in k],
                         [[_bf16_round(a) for a in vv] for vv in v]))
        o = []
        for hh in range(hq):
            g = hh // (hq // hkv)
            s = [sum(q[hh][i] * kt[g][i] for i in range(D)) / math.sqrt(D) for kt, _ in cache[l]]
            m = max(s)
            e = [math.exp(a - m) for a in s]
            z = sum(e)
            o.extend(sum(e[t] / z * cache[l][t][1][g][i] for t in range(len(e))) for i in range(D))
        ao = mv(W[p + "wo"], o)
        x = [x[i] + ao[i] for i in range(H)]
        h2 = rms(x, W[p + "ffn_norm"])
        r = mv(W[p + "router"], h2)
        if p + "router_bias" in W:
            r = [r[e] + W[p + "router_bias"][e] for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-r[e], e))[:K]
        m = max(r[e] for e in sel)
        ex = [math.exp(r[e] - m) for e in sel]
        w = [a / sum(ex) for a in ex]
        for j, e in enumerate(sel):
            g_ = mv(W[p + "w_gate"][e], h2)
            u_ = mv(W[p + "w_up"][e], h2)
            a = [g_[i] / (1.0 + math.exp(-g_[i])) * u_[i] for i in range(I)]
            y = mv(W[p + "w_down"][e], a)
            x = [x[i] + w[j] * y[i] for i in range(H)]
    hf = rms(x, W["final_norm"])
    return mv(W["lm_head"], hf), x


def _to_lists(tensors):
    out = {}
    for k, v in tensors.items():
        f = bf16_to_f32(v).astype(np.float64) if v.dtype == np.uint16 else v.astype(np.float64)
        out[k] = f.tolist()
    return out


@pytest.mark.parametrize("with_bias", [False, True])
def test_micro_model_matches_bruteforce(with_bias):
    d = configs.MICRO
    bias = None
    if with_bias:
        bias = [np.random.default_rng(20 + l).standard_normal(d["n_experts"]).astype(np.float32)
                for l in range(d["n_layers"])]
    tensors = _np_model(d, seed=5, router_bias=bias)
    n_pages, cached = 6, 3
    kp, vp = _np_pool(d, n_pages, seed=6)
    bt = [4, 1, 5]            # shuffled page table: tokens 0,1 -> page 4, 2,3 -> page 1
    token = 11
    # brute force: contiguous cache built from the same pool entries
    W = _to_lists(tensors)
    P = d["page_size"]
    cache = []
    for l in range(d["n_layers"]):
        cl = []
        for t in range(cached):
            cl.append((bf16_to_f32(kp[l, bt[t // P], :, t % P, :]).astype(np.float64).tolist(),
                       bf16_to_f32(vp[l, bt[t // P], :, t % P, :]).astype(np.float64).tolist()))
        cache.append(cl)
    ref_logits, ref_x = _brute_step(d, W, cache, cached, token)
    ref_logits = np.array(ref_logits)

    for dtype, tol in ((np.float64, 1e-10), (np.float32, 2e-4)):
        model = DenseModel.from_dict(d, tensors, dtype)
        kv = PagedKV(kp.copy(), vp.copy(), P)
        logits, tr, _ = decode_step(model, kv, [cached], [bt], [token], dtype)
        err = np.max(np.abs(logits[0] - ref_logits)) / np.max(np.abs(ref_logits))
        assert err < tol, (dtype, err)
        assert np.max(np.abs(tr[0].x_final - np.array(ref_x))) / np.max(np.abs(ref_x)) < tol


def test_micro_model_catches_a_planted_mistake():
    """The brute-force comparison is sharp enough to see a small change in the
    oracle's inputs (a stand-in for a dropped term): flip one weight."""
    d = configs.MICRO
    tensors = _np_model(d, seed=5)
    kp, vp = _np_pool(d, 6, seed=6)
    W = _to_lists(tensors)
    cache = [[] for _ in range(d["n_layers"])]
    ref, _ = _brute_step(d, W, cache, 0, 3)
    bad = {k: v.copy() for k, v in tensors.items()}
    bad["layers.0.wo"][2, 5] ^= np.uint16(0x8000)   # sign flip of one O-projection weight
    model = DenseModel.from_dict(d, bad, np.float64)
    logits, _, _ = decode_step(model, PagedKV(kp.copy(), vp.copy(), 2), [0], [[0]], [3], np.float64)
    assert np.max(np.abs(logits[0] - np.array(ref))) > 1e-6


# -------------------------------------------------------------- invariants --

@pytest.fixture(scope="module")
def tiny():
    d = configs.TINY
    return d, _np_model(d, seed=0)


def test_paged_equals_contiguous_step(tiny):
    d, tensors = tiny
    P, T = d["page_size"], 64
    n = T // P + 1
    kp, vp = _np_pool(d, n, seed=1)
    model = DenseModel.from_dict(d, tensors)
    l1, _, _ = decode_step(model, PagedKV(kp.copy(), vp.copy(), P), [T], [list(range(n))], [7])
    perm = np.random.default_rng(3).permutation(23)[:n]
    kp2, vp2 = _np_pool(d, 23, seed=9)
    kp2[:, perm], vp2[:, perm] = kp, vp
    l2, _, _ = decode_step(model, PagedKV(kp2, vp2, P), [T], [list(perm)], [7])
    assert np.array_equal(l1, l2)


def test_step_writes_exactly_one_slot_per_layer(tiny):
    d, tensors = tiny
    P, T = d["page_size"], 37
    bt = [5, 2, 7, 0]
    kp, vp = _np_pool(d, 8, seed=1)
    kv = PagedKV(kp.copy(), vp.copy(), P)
    _, tr, _ = decode_step(DenseModel.from_dict(d, tensors), kv, [T], [bt], [100])
    for pool_before, pool_after in ((kp, kv.k), (vp, kv.v)):
        changed = {(int(a), int(b), int(c)) for a, b, c in np.argwhere(np.any(pool_before != pool_after, axis=(2, 4)))}
        assert changed == {(l, bt[T // P], T % P) for l in range(d["n_layers"])}
    for lt in tr[0].layers:
        assert (lt.kv_page, lt.kv_slot) == (bt[T // P], T % P)


def test_step_is_deterministic_and_idempotent(tiny):
    d, tensors = tiny
    P, T = d["page_size"], 64
    bt = list(range(T // P + 1))
    kp, vp = _np_pool(d, len(bt), seed=1)
    model = DenseModel.from_dict(d, tensors)
    kv = PagedKV(kp.copy(), vp.copy(), P)
    a, _, _ = decode_step(model, kv, [T], [bt], [9])
    b, _, _ = decode_step(model, kv, [T], [bt], [9])       # re-run on the written cache
    c, _, _ = decode_step(model, PagedKV(kp.copy(), vp.copy(), P), [T], [bt], [9])
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_batch_equals_sequences_one_at_a_time(tiny):
    d, tensors = tiny
    P = d["page_size"]
    Ts = [5, 40, 17]
    bts = synth.make_block_tables(3, 4, 12, shuffle=True)
    kp, vp = _np_pool(d, 12, seed=1)
    model = DenseModel.from_dict(d, tensors)
    kv = PagedKV(kp.copy(), vp.copy(), P)
    batched, _, _ = decode_step(model, kv, Ts, bts, [1, 2, 3])
    for b in range(3):
        kv1 = PagedKV(kp.copy(), vp.copy(), P)
        one, _, _ = decode_step(model, kv1, [Ts[b]], [bts[b]], [b + 1])
        assert np.array_equal(one[0], batched[b])


def test_routing_weights_sum_to_one_and_ids_distinct(tiny):
    d, tensors = tiny
    P, T = d["page_size"], 64
    bt = list(range(5))
    kp, vp = _np_pool(d, 5)
    logits, toks, traces = decode_sequence(DenseModel.from_dict(d, tensors), PagedKV(kp, vp, P), T, bt, 17, 4)
    assert np.all(np.isfinite(logits))
    for tr in traces:
        for lt in tr.layers:
            assert abs(float(np.sum(lt.weights, dtype=np.float64)) - 1.0) < 1e-6
            assert len(set(lt.ids.tolist())) == d["top_k"]


def test_blocks_compose_to_the_step_and_forced_routing_reproduces_top_k(tiny):
    """The per-block entry points (used to adopt another implementation's
    routing) are the step: composing them with the oracle's own top-k ids
    forced gives the step's logits bit for bit."""
    d, tensors = tiny
    P, T = d["page_size"], 40
    bt = [3, 0, 2]
    kp, vp = _np_pool(d, 4, seed=1)
    model = DenseModel.from_dict(d, tensors)
    want, tr, _ = decode_step(model, PagedKV(kp.copy(), vp.copy(), P), [T], [bt], [21])
    kv = PagedKV(kp.copy(), vp.copy(), P)
    cos, sin = rope_cos_sin(T, d["head_dim"], d["rope_theta"])
    x = model.rows("embed", 21).astype(np.float32)
    for l in range(d["n_layers"]):
        x, lt = attention_block(model, kv, l, x, T, bt, cos, sin)
        x = moe_block(model, l, x, lt, force_ids=tr[0].layers[l].ids)
        assert np.array_equal(lt.weights, tr[0].layers[l].weights)
    assert np.array_equal(final_logits(model, x), want[0])


def test_route_weights_is_the_renormalised_full_softmax():
    rng = np.random.default_rng(5)
    r = rng.normal(size=32).astype(np.float32)
    ids = [7, 3, 30, 12]
    full = np.exp(r.astype(np.float64) - r.max()) / np.sum(np.exp(r.astype(np.float64) - r.max()))
    want = full[ids] / full[ids].sum()
    got = route_weights(r, ids)
    assert np.allclose(got, want, rtol=1e-6, atol=0)
    # the order of ids is the order of the weights
    assert np.allclose(route_weights(r, ids[::-1]), want[::-1], rtol=1e-6, atol=0)


# ----------------------------------------------------------------- bytes ----

@pytest.mark.parametrize("Ts,toks", [([64], [7]), ([5, 40, 17], [1, 2, 1])])
def test_counted_bytes_equal_closed_form(tiny, Ts, toks):
    d, tensors = tiny
    P = d["page_size"]
    bts = synth.make_block_tables(len(Ts), 5, 16, shuffle=True)
    kp, vp = _np_pool(d, 16)
    model = DenseModel.from_dict(d, tensors)
    _, traces, touched = decode_step(model, PagedKV(kp, vp, P), Ts, bts, toks)
    distinct = [len({int(e) for tr in traces for e in tr.layers[l].ids}) for l in range(d["n_layers"])]
    want = sol.step_bytes(d, Ts, distinct, distinct_tokens=len(set(toks)))
    assert touched == want


def test_counted_bytes_with_router_bias():
    d = configs.MICRO
    bias = [np.zeros(d["n_experts"], np.float32)]
    tensors = _np_model(d, seed=5, router_bias=bias)
    kp, vp = _np_pool(d, 6)
    _, traces, touched = decode_step(DenseModel.from_dict(d, tensors), PagedKV(kp, vp, 2), [3], [[0, 1, 2]], [4])
    distinct = [len(set(traces[0].layers[0].ids.tolist()))]
    assert touched == sol.step_bytes(d, [3], distinct, router_bias=True)
