"""Seeded synthetic inputs: weights, paged KV prefill, page tables, tokens.

This module only draws random numbers and lays them out; it holds none of the
decode arithmetic. Both the HIP path's tests and benchmark and the CPU
reference take their inputs from here.

Recipe (the pages give no model, so all inputs are synthetic):
* matrices and embeddings: float32 N(0, 0.02), rounded to BF16 by torch;
* norm gains: 1 + N(0, 0.02), rounded to BF16;
* KV cache prefill: N(0, 1) rounded to BF16 over the whole pool (pages no
  sequence owns are filled too, so a stray read shows up);
* each tensor has its own generator seeded from (seed, tensor name);
* page tables: sequential, or a seeded permutation of the pool;
* first tokens: seeded uniform integers in [0, vocab).
"""

from __future__ import annotations

import zlib
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch


def tensor_seed(seed: int, name: str) -> int:
    return (zlib.crc32(name.encode()) * 1000003 + int(seed) * 7919) % (2 ** 62)


def _gen(device, seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, name))
    return g


def gen_bf16(shape, std: float, seed: int, name: str, device="cpu", mean: float = 0.0,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """N(mean, std) drawn in float32, stored as BF16. Tensors above 2^26
    elements are drawn in slices along the first axis, each slice with its
    own generator, so the float32 staging stays small."""
    shape = tuple(int(s) for s in shape)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    numel = int(np.prod(shape))
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    sliced = numel > (1 << 26)
    per = max(1, (1 << 26) // row) if sliced else shape[0]
    for s0 in range(0, shape[0], per):
        s1 = min(shape[0], s0 + per)
        g = _gen(device, seed, f"{name}#{s0}" if sliced else name)
        t = torch.randn((s1 - s0,) + shape[1:], generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        if mean != 0.0:
            t.add_(mean)
        out[s0:s1].copy_(t)
        del t
    return out


def tensor_names(dims: dict) -> List[str]:
    names = ["embed", "final_norm", "lm_head"]
    for l in range(dims["n_layers"]):
        for k in ("attn_norm", "wqkv", "wo", "ffn_norm", "router", "w_gate", "w_up", "w_down"):
            names.append(f"layers.{l}.{k}")
    return names


def tensor_shape(dims: dict, name: str):
    H, V = dims["hidden"], dims["vocab"]
    hq, hkv, D = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    E, I = dims["n_experts"], dims["moe_inter"]
    kind = name.split(".")[-1]
    return {
        "embed": (V, H), "lm_head": (V, H), "final_norm": (H,),
        "attn_norm": (H,), "ffn_norm": (H,),
        "wqkv": ((hq + 2 * hkv) * D, H), "wo": (H, hq * D),
        "router": (E, H), "w_gate": (E, I, H), "w_up": (E, I, H), "w_down": (E, H, I),
    }[kind]


def make_model(dims: dict, seed: int = 0, device="cpu",
               router_bias: Optional[Sequence[np.ndarray]] = None) -> Dict[str, torch.Tensor]:
    """All weights as BF16 torch tensors on ``device`` (norm gains 1+N(0,.02),
    everything else N(0,.02)). ``router_bias``, if given, is one float32
    vector of length E per layer."""
    out = {}
    for name in tensor_names(dims):
        shp = tensor_shape(dims, name)
        if name.endswith("norm"):
            out[name] = gen_bf16(shp, 0.02, seed, name, device, mean=1.0)
        else:
            out[name] = gen_bf16(shp, 0.02, seed, name, device)
    if router_bias is not None:
        for l, b in enumerate(router_bias):
            out[f"layers.{l}.router_bias"] = torch.as_tensor(
                np.asarray(b, dtype=np.float32)).to(device)
    return out


def make_kv_pool(dims: dict, n_pages: int, seed: int = 1, device="cpu"):
    """K and V pools ``[L][n_pages][Hkv][P][D]`` BF16, filled with N(0,1)."""
    shp = (dims["n_layers"], n_pages, dims["n_kv_heads"], dims["page_size"], dims["head_dim"])
    k = torch.empty(shp, dtype=torch.bfloat16, device=device)
    v = torch.empty(shp, dtype=torch.bfloat16, device=device)
    for l in range(shp[0]):
        gen_bf16(shp[1:], 1.0, seed, f"kpool.{l}", device, out=k[l])
        gen_bf16(shp[1:], 1.0, seed, f"vpool.{l}", device, out=v[l])
    return k, v


def make_block_tables(n_seqs: int, pages_per_seq: int, n_pages: int, seed: int = 2,
                      shuffle: bool = False) -> np.ndarray:
    """int32 ``[n_seqs][pages_per_seq]``: disjoint page ids, either
    sequential or drawn from a seeded permutation of the pool."""
    need = n_seqs * pages_per_seq
    if need > n_pages:
        raise ValueError("pool too small")
    if shuffle:
        perm = np.random.default_rng(tensor_seed(seed, "pages")).permutation(n_pages)[:need]
    else:
        perm = np.arange(need)
    return perm.reshape(n_seqs, pages_per_seq).astype(np.int32)


def make_tokens(n: int, vocab: int, seed: int = 3) -> np.ndarray:
    return np.random.default_rng(tensor_seed(seed, "tokens")).integers(0, vocab, size=n).astype(np.int32)


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> uint16 numpy array of its bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def zipf_router_bias(dims: dict, seed: int = 5, s: float = 1.1, n_tokens: int = 4096):
    """Per-layer float32 router bias b_e = -alpha * s * ln(rank_e), rank_e a
    seeded permutation of 1..E per layer, for a workload whose expert
    popularity follows Zipf(s). alpha is set once by bisection so that, for
    router logits drawn N(0, sigma^2) with sigma = 0.02 sqrt(H) (the spread a
    N(0, 0.02) router gives a unit-RMS input), the selection counts of the
    top-k experts, ordered by rank, fall off with a log-log slope of -s.
    Returns (biases, alpha, fitted slope)."""
    E, K, L, H = dims["n_experts"], dims["top_k"], dims["n_layers"], dims["hidden"]
    sigma = 0.02 * float(np.sqrt(H))
    rng = np.random.default_rng(tensor_seed(seed, "zipf.calib"))
    logits = rng.standard_normal((n_tokens, E)) * sigma
    lr = np.log(np.arange(1, E + 1, dtype=np.float64))

    def slope(alpha):
        z = logits - alpha * s * lr[None, :]
        top = np.argpartition(-z, K - 1, axis=1)[:, :K]
        cnt = np.bincount(top.ravel(), minlength=E).astype(np.float64)
        keep = cnt > 0
        return float(np.polyfit(lr[keep], np.log(cnt[keep]), 1)[0])

    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if slope(mid) > -s:
            lo = mid
        else:
            hi = mid
    alpha = 0.5 * (lo + hi)
    biases = []
    for l in range(L):
        rank = np.random.default_rng(tensor_seed(seed, f"zipf.rank.{l}")).permutation(E) + 1
        biases.append((-alpha * s * np.log(rank)).astype(np.float32))
    return biases, alpha, slope(alpha)


class ChurnWorkload:
    """Seeded draws of a churning batch, as a serving loop would see it:
    `n_seqs` requests with initial contexts log-uniform on [ctx_lo, ctx_hi]
    (their cache pages hold the pool's random prefill) and seeded first
    tokens; after every `every` steps, `churn` seeded-random slots finish and
    new requests with contexts uniform on [join_lo, join_hi] and seeded first
    tokens take them. Draws only: the scheduler (mk.Scheduler) owns slots,
    pages and positions."""

    def __init__(self, n_seqs: int, vocab: int, seed: int = 7, ctx_lo: int = 128, ctx_hi: int = 32768,
                 join_lo: int = 128, join_hi: int = 2048, every: int = 8, churn: int = 4):
        self.rng = np.random.default_rng(tensor_seed(seed, "ragged"))
        self.n_seqs, self.vocab, self.every, self.churn, self.join = n_seqs, vocab, every, churn, (join_lo, join_hi)
        ctx = [int(np.exp(self.rng.uniform(np.log(ctx_lo), np.log(ctx_hi)))) for _ in range(n_seqs)]
        toks = [int(t) for t in self.rng.integers(0, vocab, size=n_seqs)]
        self.initial = list(zip(ctx, toks))

    def after_step(self, step: int):
        """Slots replaced after `step` steps (counted from 1): [(slot,
        context, first token)] in ascending slot order, or []."""
        if step % self.every:
            return []
        out = []
        for b in sorted(self.rng.choice(self.n_seqs, size=self.churn, replace=False).tolist()):
            out.append((int(b), int(self.rng.integers(self.join[0], self.join[1] + 1)),
                        int(self.rng.integers(0, self.vocab))))
        return out


class ChurnRun:
    """A ChurnWorkload played on a scheduler: request b (b < n_seqs) starts
    in slot b; every churn releases the requests of the chosen slots and
    submits the new ones, which the scheduler admits into those slots (lowest
    free slot first, in submission order). Each request's length limit is
    max_len positions; it ends earlier only by churn."""

    def __init__(self, sched, workload: ChurnWorkload, max_len: int):
        self.sched, self.w, self.max_len = sched, workload, max_len
        self.step_no, self.next_id = 0, 0
        self.req_of_slot = {}
        for b, (ctx, tok) in enumerate(workload.initial):
            self._submit(b, ctx, tok)

    def _submit(self, slot, ctx, tok):
        self.sched.submit(self.next_id, [tok], self.max_len - ctx, cached_len=ctx)
        self.req_of_slot[slot] = self.next_id
        self.next_id += 1

    def advance(self):
        """After a committed step: apply the workload's churn. Returns the
        slots that new requests took."""
        self.step_no += 1
        ev = self.w.after_step(self.step_no)
        for slot, _, _ in ev:
            self.sched.release(self.req_of_slot[slot])
        for slot, ctx, tok in ev:
            self._submit(slot, ctx, tok)
        return [slot for slot, _, _ in ev]
