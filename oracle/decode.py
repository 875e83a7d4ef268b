"""Plain, slow CPU definition of one MoE-transformer decode step.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What is computed, and where it comes from:

* The pages say a decode step streams the active weights plus the KV cache
  ("Cohere Publishes One-Kernel Server for North Mini Code, Claims 1.58x vLLM
  Speedup", section "The delay is between operations"), that the work is
  normalization, projections, attention and mixture-of-experts routing (same
  section; "Cohere fuses an entire decode step into one GPU program",
  paragraph 2) and that the KV cache is kept in pages (opening section of the
  first page; third page, paragraph 4). They give no architecture; the model
  below is the plainest reading: pre-norm RMSNorm, fused QKV projection with
  rotate-half RoPE, grouped-query attention over a paged BF16 KV cache, a
  softmax-over-selected top-k router and SwiGLU experts, final RMSNorm and an
  untied LM head.
* The megakernel is a scheduling change, not a change of the arithmetic
  (first page, opening section and section "A hand-built approach to a
  specialized server"), so this file is that plain definition: no blocking,
  fusion or reordering.

Precision: float32 over BF16 weights by default; ``dtype=np.float64`` gives the
same steps in float64. Rotary angles are formed in float64 and their cos/sin
rounded to the working precision. Values written to the KV cache are rounded
to BF16 (round-to-nearest-even) and read back from the cache.

Every public function is pinned by tests in tests/test_oracle_*.py.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# BF16 encoding
# ---------------------------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    """Decode BF16 bit patterns (uint16) exactly: the 16 bits become the high
    half of an IEEE float32. Pinned exhaustively over all 65,536 codes."""
    u = np.asarray(bits, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x) -> np.ndarray:
    """Round float32 values to BF16, nearest with ties to even, returning the
    uint16 bit patterns. NaN stays NaN (quiet), infinities stay infinite,
    finite values past the largest BF16 round to infinity."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    rounded = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        sign = ((b >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        out = np.where(nan, sign | np.uint16(0x7FC0), out)
    return out


# ---------------------------------------------------------------------------
# Ops
# ---------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float, dtype=np.float32) -> np.ndarray:
    """RMSNorm: x / sqrt(mean(x^2) + eps), times the per-channel gain."""
    x = np.asarray(x, dtype=dtype)
    ms = np.mean(x * x, dtype=dtype)
    inv = dtype(1.0) / np.sqrt(ms + dtype(eps))
    return (x * inv) * np.asarray(gain, dtype=dtype)


def rope_cos_sin(pos: int, head_dim: int, theta: float, dtype=np.float32):
    """Angles phi_i = pos * theta^(-2i/D) for i < D/2, formed in float64;
    returns (cos, sin) rounded to ``dtype``."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / np.float64(head_dim))
    ang = np.float64(pos) * inv_freq
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope_rotate(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the last axis: the pair (u_i, u_{i+D/2}) turns by
    phi_i. ``u`` may carry leading head axes."""
    half = u.shape[-1] // 2
    a = u[..., :half]
    b = u[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def gather_pages(pool_layer: np.ndarray, block_table: Sequence[int], n_tokens: int,
                 page_size: int) -> np.ndarray:
    """Read tokens 0..n_tokens-1 of one sequence out of a paged pool
    ``[n_pages][Hkv][P][D]``: token t lives in page block_table[t // P],
    slot t % P. Returns ``[n_tokens][Hkv][D]`` with the pool's dtype."""
    hkv, d = pool_layer.shape[1], pool_layer.shape[3]
    out = np.empty((n_tokens, hkv, d), dtype=pool_layer.dtype)
    for t in range(n_tokens):
        out[t] = pool_layer[block_table[t // page_size], :, t % page_size, :]
    return out


def attention_decode(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     dtype=np.float32, return_probs: bool = False):
    """Single-query attention for every q head over cached tokens.

    q: ``[Hq][D]``; keys, values: ``[T][Hkv][D]`` (already decoded to float).
    Query head h reads KV head h // (Hq / Hkv). Scores are q.k / sqrt(D),
    softmax is max-subtracted. Returns ``[Hq][D]`` (and the probabilities)."""
    hq, d = q.shape
    hkv = keys.shape[1]
    group = hq // hkv
    scale = dtype(1.0 / math.sqrt(d))
    out = np.empty((hq, d), dtype=dtype)
    probs = []
    for h in range(hq):
        g = h // group
        k = np.asarray(keys[:, g, :], dtype=dtype)
        v = np.asarray(values[:, g, :], dtype=dtype)
        s = (k @ np.asarray(q[h], dtype=dtype)) * scale
        e = np.exp(s - np.max(s))
        a = e / np.sum(e, dtype=dtype)
        out[h] = a @ v
        probs.append(a)
    if return_probs:
        return out, probs
    return out


def route_weights(logits: np.ndarray, ids: Sequence[int], dtype=np.float32) -> np.ndarray:
    """Routing weights of the selected experts ``ids`` (in that order): a
    softmax over their logits, which equals the full softmax renormalised
    over the selection."""
    sel = np.asarray(logits, dtype=dtype)[np.asarray(ids, dtype=np.int64)]
    e = np.exp(sel - np.max(sel))
    return (e / np.sum(e, dtype=dtype)).astype(dtype)


def route_topk(logits: np.ndarray, k: int, dtype=np.float32):
    """Top-k expert selection and routing weights.

    Selection order is (logit descending, expert index ascending), so ties go
    to the lower index; the weights are route_weights of the selection."""
    r = np.asarray(logits, dtype=dtype)
    order = np.argsort(-r, kind="stable")[:k]
    return order.astype(np.int32), route_weights(r, order, dtype)


def swiglu_expert(h: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                  w_down: np.ndarray, dtype=np.float32) -> np.ndarray:
    """One SwiGLU expert: W_down (SiLU(W_gate h) * (W_up h)), with
    SiLU(z) = z / (1 + exp(-z))."""
    g = np.asarray(w_gate, dtype=dtype) @ h
    u = np.asarray(w_up, dtype=dtype) @ h
    a = (g / (dtype(1.0) + np.exp(-g))) * u
    return np.asarray(w_down, dtype=dtype) @ a


def moe_combine(ys: Sequence[np.ndarray], w: np.ndarray, dtype=np.float32) -> np.ndarray:
    """sum_j w_j y_j, accumulated in rank order."""
    acc = np.zeros_like(np.asarray(ys[0], dtype=dtype))
    for j, y in enumerate(ys):
        acc = acc + dtype(w[j]) * np.asarray(y, dtype=dtype)
    return acc


# ---------------------------------------------------------------------------
# Model and KV containers
# ---------------------------------------------------------------------------

@dataclass
class Dims:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    moe_inter: int
    vocab: int
    page_size: int
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @staticmethod
    def of(d) -> "Dims":
        if isinstance(d, Dims):
            return d
        keys = Dims.__dataclass_fields__.keys()
        return Dims(**{k: d[k] for k in keys if k in d})


class DenseModel:
    """Weights as BF16 bit patterns (uint16 numpy arrays), decoded lazily and
    cached. ``source(name)`` returns the array for a tensor name; expert
    tensors may instead come from ``expert_source(layer, kind, e)`` so that a
    large model only materialises the experts a step touches.

    Tensor names: ``embed`` [V][H], ``final_norm`` [H], ``lm_head`` [V][H];
    per layer l, ``layers.l.attn_norm`` [H], ``layers.l.wqkv``
    [(Hq+2Hkv)D][H] (q rows, then k rows, then v rows), ``layers.l.wo``
    [H][Hq D], ``layers.l.ffn_norm`` [H], ``layers.l.router`` [E][H],
    optional ``layers.l.router_bias`` float32 [E], ``layers.l.w_gate`` and
    ``layers.l.w_up`` [E][I][H], ``layers.l.w_down`` [E][H][I].
    """

    def __init__(self, dims, source: Callable[[str], Optional[np.ndarray]],
                 expert_source: Optional[Callable[[int, str, int], np.ndarray]] = None,
                 dtype=np.float32):
        self.dims = Dims.of(dims)
        self._source = source
        self._expert_source = expert_source
        self.dtype = dtype
        self._cache: Dict[Tuple, np.ndarray] = {}
        self.touched: Dict[Tuple, int] = {}

    @staticmethod
    def from_dict(dims, tensors: Dict[str, np.ndarray], dtype=np.float32) -> "DenseModel":
        return DenseModel(dims, lambda n: tensors.get(n), None, dtype)

    def _touch(self, key, nbytes):
        self.touched[key] = int(nbytes)

    def _decoded(self, key, raw: np.ndarray) -> np.ndarray:
        if key not in self._cache:
            self._cache[key] = bf16_to_f32(raw).astype(self.dtype, copy=False)
        return self._cache[key]

    def tensor(self, name: str) -> np.ndarray:
        raw = self._source(name)
        if raw is None:
            raise KeyError(name)
        self._touch((name,), raw.size * 2)
        return self._decoded((name,), raw)

    def rows(self, name: str, idx: int) -> np.ndarray:
        raw = self._source(name)
        self._touch((name, "row", int(idx)), raw.shape[1] * 2)
        return bf16_to_f32(raw[int(idx)]).astype(self.dtype)

    def router_bias(self, layer: int) -> Optional[np.ndarray]:
        b = self._source(f"layers.{layer}.router_bias")
        if b is None:
            return None
        b = np.asarray(b, dtype=np.float32)
        self._touch((f"layers.{layer}.router_bias",), b.size * 4)
        return b.astype(self.dtype)

    def expert(self, layer: int, e: int):
        mats = []
        for kind in ("w_gate", "w_up", "w_down"):
            key = (f"layers.{layer}.{kind}", int(e))
            if key not in self._cache:
                if self._expert_source is not None:
                    raw = self._expert_source(layer, kind, int(e))
                else:
                    raw = self._source(f"layers.{layer}.{kind}")[int(e)]
                self._cache[key] = bf16_to_f32(raw).astype(self.dtype, copy=False)
            arr = self._cache[key]
            self._touch(key, arr.size * 2)
            mats.append(arr)
        return tuple(mats)

    def reset_touched(self):
        self.touched = {}

    def touched_bytes(self) -> int:
        return int(sum(self.touched.values()))


class PagedKV:
    """Paged BF16 KV cache: ``k`` and ``v`` are uint16 arrays
    ``[L][n_pages][Hkv][P][D]``. The oracle writes into them in place, so
    callers hand it its own copy."""

    def __init__(self, k_pool: np.ndarray, v_pool: np.ndarray, page_size: int):
        self.k = k_pool
        self.v = v_pool
        self.page_size = page_size
        self.bytes_read = 0
        self.bytes_written = 0

    def append(self, layer: int, block_table, pos: int, k_bf16: np.ndarray, v_bf16: np.ndarray):
        page = block_table[pos // self.page_size]
        slot = pos % self.page_size
        self.k[layer, page, :, slot, :] = k_bf16
        self.v[layer, page, :, slot, :] = v_bf16
        self.bytes_written += k_bf16.nbytes + v_bf16.nbytes

    def read(self, layer: int, block_table, n_tokens: int):
        kk = gather_pages(self.k[layer], block_table, n_tokens, self.page_size)
        vv = gather_pages(self.v[layer], block_table, n_tokens, self.page_size)
        self.bytes_read += kk.nbytes + vv.nbytes
        return bf16_to_f32(kk), bf16_to_f32(vv)


# ---------------------------------------------------------------------------
# The decode step
# ---------------------------------------------------------------------------

@dataclass
class LayerTrace:
    x_attn: np.ndarray = None      # residual after the attention block
    x_out: np.ndarray = None       # residual after the MoE block
    h2: np.ndarray = None          # normalised FFN input
    router_logits: np.ndarray = None
    ids: np.ndarray = None
    weights: np.ndarray = None
    kv_page: int = -1
    kv_slot: int = -1


@dataclass
class SeqTrace:
    layers: List[LayerTrace] = field(default_factory=list)
    x_final: np.ndarray = None


def attention_block(model: DenseModel, kv: PagedKV, l: int, x: np.ndarray, pos: int, block_table,
                    cos: np.ndarray, sin: np.ndarray, dtype=np.float32) -> Tuple[np.ndarray, LayerTrace]:
    """Layer l's attention block for one sequence: RMSNorm, QKV projection,
    RoPE at position pos, append of the new K/V (BF16) to the paged cache,
    attention over positions 0..pos, output projection plus residual.
    Returns the residual after the block and a trace with the KV slot."""
    d = model.dims
    hq, hkv, D = d.n_q_heads, d.n_kv_heads, d.head_dim
    qd, kvd = hq * D, hkv * D
    lt = LayerTrace()
    pre = f"layers.{l}."
    h = rms_norm(x, model.tensor(pre + "attn_norm"), d.rms_eps, dtype)
    qkv = model.tensor(pre + "wqkv") @ h
    q = qkv[:qd].reshape(hq, D)
    k = qkv[qd:qd + kvd].reshape(hkv, D)
    v = qkv[qd + kvd:qd + 2 * kvd].reshape(hkv, D)
    q = rope_rotate(q, cos, sin)
    k = rope_rotate(k, cos, sin)
    kv.append(l, block_table, pos, f32_to_bf16_rne(k.astype(np.float32)),
              f32_to_bf16_rne(v.astype(np.float32)))
    lt.kv_page, lt.kv_slot = int(block_table[pos // d.page_size]), pos % d.page_size
    keys, vals = kv.read(l, block_table, pos + 1)
    o = attention_decode(q, keys, vals, dtype)
    x = x + model.tensor(pre + "wo") @ o.reshape(qd)
    lt.x_attn = x.copy()
    return x, lt


def moe_block(model: DenseModel, l: int, x: np.ndarray, lt: LayerTrace, dtype=np.float32,
              force_ids: Optional[Sequence[int]] = None) -> np.ndarray:
    """Layer l's mixture-of-experts block for one sequence: RMSNorm, router
    (plus bias), top-k routing, SwiGLU experts combined in rank order, plus
    residual. ``force_ids`` replaces the top-k selection by the given
    experts (in that order; weights by route_weights), for comparisons that
    adopt another implementation's routing. Fills lt and returns the new
    residual."""
    d = model.dims
    pre = f"layers.{l}."
    h2 = rms_norm(x, model.tensor(pre + "ffn_norm"), d.rms_eps, dtype)
    r = model.tensor(pre + "router") @ h2
    bias = model.router_bias(l)
    if bias is not None:
        r = r + bias
    if force_ids is None:
        ids, w = route_topk(r, d.top_k, dtype)
    else:
        ids = np.asarray(force_ids, dtype=np.int32)
        w = route_weights(r, ids, dtype)
    ys = []
    for e in ids:
        wg, wu, wd = model.expert(l, int(e))
        ys.append(swiglu_expert(h2, wg, wu, wd, dtype))
    x = x + moe_combine(ys, w, dtype)
    lt.x_out = x.copy()
    lt.h2, lt.router_logits, lt.ids, lt.weights = h2, r, ids, w
    return x


def final_logits(model: DenseModel, x: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Final RMSNorm and LM head."""
    hf = rms_norm(x, model.tensor("final_norm"), model.dims.rms_eps, dtype)
    return (model.tensor("lm_head") @ hf).astype(dtype)


def _decode_one(model: DenseModel, kv: PagedKV, pos: int, block_table, token: int,
                dtype) -> Tuple[np.ndarray, SeqTrace]:
    d = model.dims
    tr = SeqTrace()
    x = model.rows("embed", token).astype(dtype)
    cos, sin = rope_cos_sin(pos, d.head_dim, d.rope_theta, dtype)
    for l in range(d.n_layers):
        x, lt = attention_block(model, kv, l, x, pos, block_table, cos, sin, dtype)
        x = moe_block(model, l, x, lt, dtype)
        tr.layers.append(lt)
    tr.x_final = x.copy()
    return final_logits(model, x, dtype), tr


def decode_step(model: DenseModel, kv: PagedKV, positions: Sequence[int],
                block_tables: Sequence[Sequence[int]], tokens: Sequence[int],
                dtype=np.float32):
    """One decode step for a batch, run one sequence at a time (no sequence
    reads another's state).

    Sequence b holds ``positions[b]`` cached tokens; its new token goes to
    position p = positions[b], written into page ``block_tables[b][p // P]``,
    slot ``p % P``, and attention covers positions 0..p inclusive.

    Returns ``(logits [B][V], traces, touched_bytes)`` where touched_bytes is
    the number of bytes the step read or wrote: every weight tensor it used
    (each counted once per step; experts once per distinct (layer, expert)),
    the embedding rows, the KV it read and wrote, and the float32 logits."""
    model.reset_touched()
    kv.bytes_read = kv.bytes_written = 0
    out, traces = [], []
    for b in range(len(tokens)):
        lg, tr = _decode_one(model, kv, int(positions[b]), block_tables[b],
                             int(tokens[b]), dtype)
        out.append(lg)
        traces.append(tr)
    logits = np.stack(out)
    touched = model.touched_bytes() + kv.bytes_read + kv.bytes_written + logits.shape[0] * logits.shape[1] * 4
    return logits, traces, touched


def prefill(model: DenseModel, kv: PagedKV, pos0: int, block_table, tokens: Sequence[int],
            dtype=np.float32):
    """A block of T new tokens of one sequence at positions pos0 .. pos0+T-1
    (a prompt being ingested, or any step that feeds a sequence several
    tokens at once).

    The pages describe a server that takes new requests into a running batch
    over a paged KV cache ("Cohere Publishes One-Kernel Server for North Mini
    Code, Claims 1.58x vLLM Speedup", opening section; "Cohere fuses an entire
    decode step into one GPU program", paragraph 4), so a prompt has to be
    written into the cache before its sequence decodes. They say nothing of
    how; the plainest reading is causal attention over the block: token i
    writes its K/V slot pos0+i and attends over positions 0..pos0+i (the
    cached prefix and new tokens 0..i). That is exactly T decode steps in
    order, which is how it is written here.

    Returns ``(logits [T][V], traces)``: every token's logits (the last row
    predicts the token after the block)."""
    out, traces = [], []
    for i, tok in enumerate(tokens):
        lg, tr = _decode_one(model, kv, int(pos0) + i, block_table, int(tok), dtype)
        out.append(lg)
        traces.append(tr)
    return np.stack(out), traces


def decode_sequence(model: DenseModel, kv: PagedKV, pos0: int, block_table,
                    token0: int, n_steps: int, dtype=np.float32):
    """Free-running greedy decode of one sequence: step i feeds token i at
    position pos0 + i (writing that KV slot), and token i+1 is the argmax of
    step i's logits (lowest index on ties). Returns (logits [n][V], the
    n + 1 tokens, traces)."""
    toks, all_logits, traces = [int(token0)], [], []
    pos = int(pos0)
    for _ in range(n_steps):
        lg, tr, _ = decode_step(model, kv, [pos], [block_table], [toks[-1]], dtype)
        all_logits.append(lg[0])
        traces.append(tr[0])
        toks.append(int(np.argmax(lg[0])))
        pos += 1
    return np.stack(all_logits), toks, traces

