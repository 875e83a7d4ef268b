"""Shared set-up for the GPU tests: seeded inputs on the device, the matching
oracle state on the host, and views of the library's per-step results."""

from __future__ import annotations

import numpy as np
import torch

from oracle import DenseModel, PagedKV
from persistent_megakernel_03_amd import configs, mk, synth


class Setup:
    """Weights and KV for one model on both sides. The device V pool is the
    oracle's pool with each page stored dimension-major (the library's V
    layout); everything else is bit-identical."""

    def __init__(self, cfg: dict, n_pages: int, seed: int = 0, device_gen: bool = False, weights=None):
        self.cfg = cfg
        self.n_pages = n_pages
        if device_gen:
            self.w_dev = weights if weights is not None else synth.make_model(cfg, seed, "cuda")
            k, v = synth.make_kv_pool(cfg, n_pages, seed + 1, "cuda")
        else:
            w_cpu = synth.make_model(cfg, seed, "cpu")
            self.w_dev = {n: t.cuda() for n, t in w_cpu.items()}
            k, v = synth.make_kv_pool(cfg, n_pages, seed + 1, "cpu")
            k, v = k.cuda(), v.cuda()
        self.k0 = k                                   # [L][N][Hkv][P][D]
        self.v0 = v.transpose(-1, -2).contiguous()    # [L][N][Hkv][D][P]
        del v

    def fresh_pools(self):
        return self.k0.clone(), self.v0.clone()

    def oracle_model(self, dtype=np.float32, lazy_experts: bool = False, weights=None) -> DenseModel:
        """weights: another name -> device tensor dict (default: this set-up's)."""
        cache = {}
        wd = self.w_dev if weights is None else weights

        def src(name):
            if name not in wd:
                return None
            if name not in cache:
                t = wd[name]
                cache[name] = synth.bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()
            return cache[name]

        if not lazy_experts:
            return DenseModel(self.cfg, src, None, dtype)

        def esrc(layer, kind, e):
            return synth.bits(wd[f"layers.{layer}.{kind}"][e])

        def src_dense(name):
            if name.split(".")[-1] in ("w_gate", "w_up", "w_down"):
                raise KeyError(name)
            return src(name)

        return DenseModel(self.cfg, src_dense, esrc, dtype)

    def oracle_kv(self, k_dev=None, v_dev=None) -> PagedKV:
        k = self.k0 if k_dev is None else k_dev
        v = self.v0 if v_dev is None else v_dev
        return PagedKV(synth.bits(k), synth.bits(v.transpose(-1, -2)), self.cfg["page_size"])


def workspace_view(dec: mk.Decoder, ptr: int, count: int, dtype) -> torch.Tensor:
    """A tensor over `count` elements of the decoder's workspace at device address `ptr`."""
    base = dec.workspace.data_ptr()
    off = ptr - base
    item = torch.empty((), dtype=dtype).element_size()
    assert 0 <= off and off + count * item <= dec.workspace.numel()
    return dec.workspace[off:off + count * item].view(dtype)


def pad64(n: int) -> int:
    return (n + 63) // 64 * 64


def x_layers(dec: mk.Decoder) -> torch.Tensor:
    c = dec.cfg
    B = dec.dims.max_batch
    stride = pad64(B * c["hidden"])
    n = (2 * c["n_layers"] + 1) * stride
    v = workspace_view(dec, dec.debug().x_layers, n, torch.float32).view(2 * c["n_layers"] + 1, stride)
    return v[:, :B * c["hidden"]].reshape(2 * c["n_layers"] + 1, B, c["hidden"])


def route_ids(dec: mk.Decoder) -> torch.Tensor:
    c = dec.cfg
    B = dec.dims.max_batch
    n = c["n_layers"] * B * c["top_k"]
    return workspace_view(dec, dec.debug().route_ids, n, torch.int32).view(c["n_layers"], B, c["top_k"])


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def routing_margin(logits: np.ndarray, k: int) -> float:
    """Smallest gap between adjacent logits among the top k+1 (float64)."""
    s = np.sort(np.asarray(logits, np.float64))[::-1][:k + 1]
    return float(np.min(s[:-1] - s[1:]))
