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
