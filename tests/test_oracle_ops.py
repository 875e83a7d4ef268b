"""Pins for the oracle's individual operations (CPU only).

Each test ties an oracle function to something other than itself: an
exhaustive enumeration, a closed form, an invariant, or a library routine on
a special case.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import (attention_decode, bf16_to_f32, f32_to_bf16_rne, gather_pages,
                    moe_combine, rms_norm, rope_cos_sin, rope_rotate, route_topk,
                    swiglu_expert)


# ---------------------------------------------------------------- BF16 -----

def test_bf16_decode_exhaustive_matches_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f32(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_roundtrip_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = f32_to_bf16_rne(bf16_to_f32(codes))
    f = bf16_to_f32(codes)
    ok = ~np.isnan(f)
    assert np.array_equal(back[ok], codes[ok])
    assert np.all(np.isnan(bf16_to_f32(back[~ok])))


def test_bf16_rne_ties_by_hand():
    # 1 + 2^-8 sits half-way between 1 and 1 + 2^-7: ties go to the even code (1.0)
    # 1 + 3*2^-8 sits half-way between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    # 1 + 2^-8 + 2^-20 is just above the tie: rounds up
    # the largest BF16 (0x7F7F) stays; half an ulp above it is a tie that rounds to
    # the even neighbour, which is infinity
    big = np.array([0x7F7F0000, 0x7F7F8000], dtype=np.uint32).view(np.float32)
    x = np.concatenate([np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8),
                                  np.inf, -np.inf], dtype=np.float32), big])
    want = np.array([0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x7F80, 0xFF80, 0x7F7F, 0x7F80], dtype=np.uint16)
    assert np.array_equal(f32_to_bf16_rne(x), want)


def test_bf16_rne_matches_torch_random():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(x), ref)


# ------------------------------------------------------------- RMSNorm -----

def test_rmsnorm_constant_vector_closed_form():
    c, H, eps = 3.0, 64, 1e-6
    g = np.linspace(0.5, 1.5, H)
    out = rms_norm(np.full(H, c), g, eps, np.float64)
    assert np.allclose(out, g * c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype,tol", [(np.float64, 1e-13), (np.float32, 1e-6)])
def test_rmsnorm_matches_torch(dtype, tol):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2048) * 3
    g = 1 + 0.02 * rng.standard_normal(2048)
    ref = F.rms_norm(torch.tensor(x), (2048,), weight=torch.tensor(g), eps=1e-6).numpy()
    out = rms_norm(x.astype(dtype), g.astype(dtype), 1e-6, dtype)
    assert np.max(np.abs(out - ref) / np.max(np.abs(ref))) < tol


# ---------------------------------------------------------------- RoPE -----

def test_rope_position_zero_is_identity():
    u = np.random.default_rng(2).standard_normal((4, 128))
    c, s = rope_cos_sin(0, 128, 10000.0, np.float64)
    assert np.array_equal(rope_rotate(u, c, s), u)


def test_rope_matches_complex_multiply_and_preserves_norm():
    rng = np.random.default_rng(3)
    D, pos = 128, 12345
    u = rng.standard_normal((3, D))
    c, s = rope_cos_sin(pos, D, 10000.0, np.float64)
    out = rope_rotate(u, c, s)
    i = np.arange(D // 2)
    phi = pos * 10000.0 ** (-2.0 * i / D)
    z = (u[:, :D // 2] + 1j * u[:, D // 2:]) * np.exp(1j * phi)
    assert np.allclose(out[:, :D // 2], z.real, atol=1e-12)
    assert np.allclose(out[:, D // 2:], z.imag, atol=1e-12)
    assert np.allclose(np.linalg.norm(out, axis=1), np.linalg.norm(u, axis=1), rtol=1e-13)


def test_rope_dot_product_depends_on_offset_only():
    rng = np.random.default_rng(4)
    D = 64
    q, k = rng.standard_normal(D), rng.standard_normal(D)

    def dot(p, t):
        cq, sq = rope_cos_sin(p, D, 10000.0, np.float64)
        ck, sk = rope_cos_sin(t, D, 10000.0, np.float64)
        return rope_rotate(q, cq, sq) @ rope_rotate(k, ck, sk)

    assert abs(dot(10, 3) - dot(107, 100)) < 1e-9
    assert abs(dot(5000, 4990) - dot(10, 0)) < 1e-9
    assert abs(dot(10, 3) - dot(10, 4)) > 1e-6  # and it does depend on the offset


# ---------------------------------------------------------- Attention -----

def _pool(n_pages, hkv, P, D, seed):
    return np.random.default_rng(seed).integers(0, 2 ** 16, (n_pages, hkv, P, D)).astype(np.uint16) & np.uint16(0xBFFF)


def test_paged_gather_equals_contiguous_under_shuffle():
    P, hkv, D, T = 16, 2, 8, 70
    n = (T + P - 1) // P
    contiguous = _pool(n, hkv, P, D, 5)
    perm = np.random.default_rng(6).permutation(40)[:n]
    shuffled = _pool(40, hkv, P, D, 7)
    for i in range(n):
        shuffled[perm[i]] = contiguous[i]
    a = gather_pages(contiguous, list(range(n)), T, P)
    b = gather_pages(shuffled, list(perm), T, P)
    assert np.array_equal(a, b)
    # page lookup: token t is block_table[t // P], slot t % P
    for t in (0, 15, 16, 69):
        assert np.array_equal(b[t], shuffled[perm[t // P], :, t % P, :])


def test_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(8)
    hq, hkv, D, T = 8, 2, 32, 37
    q = rng.standard_normal((hq, D))
    K = rng.standard_normal((T, hkv, D))
    V = rng.standard_normal((T, hkv, D))
    out = attention_decode(q, K, V, np.float64)
    rep = hq // hkv
    kt = torch.tensor(K).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
    vt = torch.tensor(V).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
    ref = F.scaled_dot_product_attention(torch.tensor(q)[None, :, None, :], kt, vt)[0, :, 0, :].numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_attention_special_cases():
    rng = np.random.default_rng(9)
    hq, hkv, D = 4, 2, 16
    q = rng.standard_normal((hq, D))
    # one cached token: output is that token's value
    K1, V1 = rng.standard_normal((1, hkv, D)), rng.standard_normal((1, hkv, D))
    o = attention_decode(q, K1, V1, np.float64)
    for h in range(hq):
        assert np.allclose(o[h], V1[0, h // 2], atol=1e-15)
    # identical keys: uniform weights, output is the mean of the values
    T = 11
    K = np.repeat(rng.standard_normal((1, hkv, D)), T, axis=0)
    V = rng.standard_normal((T, hkv, D))
    o, probs = attention_decode(q, K, V, np.float64, return_probs=True)
    for h in range(hq):
        assert np.allclose(o[h], V[:, h // 2].mean(0), atol=1e-14)
    # probabilities sum to one
    Kr = rng.standard_normal((T, hkv, D)) * 5
    _, probs = attention_decode(q, Kr, V, np.float32, return_probs=True)
    for p in probs:
        assert abs(float(np.sum(p, dtype=np.float64)) - 1.0) < 1e-6


def test_attention_gqa_head_mapping():
    # q head h must read kv head h // (Hq/Hkv): make kv heads distinguishable
    hq, hkv, D, T = 6, 3, 4, 5
    rng = np.random.default_rng(10)
    q = rng.standard_normal((hq, D))
    K = rng.standard_normal((T, hkv, D))
    V = np.zeros((T, hkv, D))
    for g in range(hkv):
        V[:, g, :] = g + 1.0
    o = attention_decode(q, K, V, np.float64)
    assert np.allclose(o[:, 0], [1, 1, 2, 2, 3, 3])


# -------------------------------------------------------------- Router -----

def test_topk_matches_bruteforce_sort_and_ties():
    r = np.array([0.5, 2.0, -1.0, 2.0, 0.5, 3.0, 2.0, -7.0], dtype=np.float32)
    ids, w = route_topk(r, 4)
    brute = sorted(range(len(r)), key=lambda e: (-float(r[e]), e))[:4]
    assert list(ids) == brute == [5, 1, 3, 6]
    assert abs(float(np.sum(w, dtype=np.float64)) - 1.0) < 1e-6
    rng = np.random.default_rng(11)
    for _ in range(200):
        r = rng.standard_normal(128).astype(np.float32)
        ids, w = route_topk(r, 8)
        assert list(ids) == sorted(range(128), key=lambda e: (-float(r[e]), e))[:8]
        assert abs(float(np.sum(w, dtype=np.float64)) - 1.0) < 1e-6
        assert np.all(np.diff(w) <= 0)


def test_topk_full_softmax_and_single_expert():
    r = np.random.default_rng(12).standard_normal(16)
    ids, w = route_topk(r, 16, np.float64)
    assert np.allclose(w, scipy.special.softmax(r)[ids], rtol=1e-13)
    ids, w = route_topk(np.array([0.3], dtype=np.float32), 1)
    assert list(ids) == [0] and w[0] == np.float32(1.0)
    # renormalised full softmax over the selection gives the same weights
    r = np.random.default_rng(13).standard_normal(32)
    ids, w = route_topk(r, 4, np.float64)
    full = scipy.special.softmax(r)
    assert np.allclose(w, full[ids] / full[ids].sum(), rtol=1e-13)


# ----------------------------------------------------------------- MoE -----

def test_swiglu_matches_torch():
    rng = np.random.default_rng(14)
    H, I = 32, 12
    h = rng.standard_normal(H)
    wg, wu, wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    ref = (F.silu(torch.tensor(wg) @ torch.tensor(h)) * (torch.tensor(wu) @ torch.tensor(h))) @ torch.tensor(wd).T
    out = swiglu_expert(h, wg, wu, wd, np.float64)
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_sparse_moe_equals_dense_masked_mixture():
    rng = np.random.default_rng(15)
    E, k, H, I = 8, 3, 16, 8
    h = rng.standard_normal(H)
    Wg, Wu, Wd = rng.standard_normal((E, I, H)), rng.standard_normal((E, I, H)), rng.standard_normal((E, H, I))
    r = rng.standard_normal(E)
    ids, w = route_topk(r, k, np.float64)
    sparse = moe_combine([swiglu_expert(h, Wg[e], Wu[e], Wd[e], np.float64) for e in ids], w, np.float64)
    # dense: every expert runs, weighted by the full softmax masked to the top-k
    th = torch.tensor(h)
    ys = torch.stack([(F.silu(torch.tensor(Wg[e]) @ th) * (torch.tensor(Wu[e]) @ th)) @ torch.tensor(Wd[e]).T
                      for e in range(E)])
    mask = torch.zeros(E, dtype=torch.float64)
    top = torch.topk(torch.tensor(r), k).indices
    p = torch.softmax(torch.tensor(r), 0)
    mask[top] = p[top] / p[top].sum()
    dense = (mask[:, None] * ys).sum(0).numpy()
    assert np.max(np.abs(sparse - dense)) < 1e-12


def test_one_expert_moe_is_the_dense_mlp_exactly():
    rng = np.random.default_rng(16)
    H, I = 16, 8
    h = rng.standard_normal(H).astype(np.float32)
    wg, wu, wd = (rng.standard_normal(s).astype(np.float32) for s in ((I, H), (I, H), (H, I)))
    ids, w = route_topk(np.array([1.7], dtype=np.float32), 1)
    y = moe_combine([swiglu_expert(h, wg, wu, wd)], w)
    assert np.array_equal(y, swiglu_expert(h, wg, wu, wd))
