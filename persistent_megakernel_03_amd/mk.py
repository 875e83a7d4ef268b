"""ctypes binding of libmk (include/mk.h): the same entry points, argument
marshalling only. Every step of the decode runs in the HIP library; torch is
used here only to own device memory and streams.

``load()`` must run after ``import torch`` so that torch and libmk share one
HIP runtime (both name ``libamdhip64.so.7``; the dynamic linker reuses the one
torch loaded). It raises if the library is missing -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import sys
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK = 0
MK_ERR_INVALID = -1
MK_ERR_UNSUPPORTED = -2
MK_ERR_CAPACITY = -3
MK_ERR_BAD_PAGE = -4
MK_ERR_HIP = -5
MK_ERR_TIMEOUT = -6
MK_ERR_DEVICE = -7
MK_MODE_MEGAKERNEL = 0
MK_MODE_PEROP = 1

STATUS_NAMES = {0: "MK_OK", -1: "MK_ERR_INVALID", -2: "MK_ERR_UNSUPPORTED", -3: "MK_ERR_CAPACITY",
                -4: "MK_ERR_BAD_PAGE", -5: "MK_ERR_HIP", -6: "MK_ERR_TIMEOUT", -7: "MK_ERR_DEVICE"}

# Every function declared in include/mk.h.
EXPORTS = ["mk_kv_pool_bytes", "mk_workspace_bytes", "mk_create", "mk_decode_step", "mk_forward_step",
           "mk_decode_step_noalloc", "mk_set_mode",
           "mk_sync_check", "mk_get_debug_ptrs", "mk_plan_build", "mk_plan_check", "mk_get_trace", "mk_get_plan", "mk_kernel_time",
           "mk_destroy", "mk_last_error",
           # include/mk_sched.h
           "mk_sched_create", "mk_sched_destroy", "mk_sched_submit", "mk_sched_release", "mk_sched_next",
           "mk_sched_commit", "mk_sched_get_stats", "mk_sched_tokens"]


class MkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class mk_dims(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("moe_inter", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_batch", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("n_pages", ctypes.c_int64)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class mk_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PP), ("wqkv", _PP), ("wo", _PP), ("ffn_norm", _PP), ("router", _PP),
                ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP), ("router_bias", _PP)]


class mk_options(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("trace", ctypes.c_int32), ("watchdog_ns", ctypes.c_int64),
                ("wg_per_cu", ctypes.c_int32), ("split_kv_tokens", ctypes.c_int32),
                ("n_cu_override", ctypes.c_int32), ("time_kernels", ctypes.c_int32),
                ("shared_levels", ctypes.c_int32), ("validate_plans", ctypes.c_int32),
                ("mfma_min_batch", ctypes.c_int32), ("poison_exchange", ctypes.c_int32),
                ("mm_row_blocks", ctypes.c_int32), ("reserved0", ctypes.c_int32)]


class mk_debug_ptrs(ctypes.Structure):
    _fields_ = [("x_layers", ctypes.c_void_p), ("route_ids", ctypes.c_void_p), ("route_w", ctypes.c_void_p),
                ("router_logits", ctypes.c_void_p), ("trace", ctypes.c_void_p),
                ("trace_capacity", ctypes.c_int64)]


class mk_plan_info(ctypes.Structure):
    _fields_ = [("n_wg", ctypes.c_int32), ("n_tasks", ctypes.c_int32), ("n_counters", ctypes.c_int32),
                ("n_levels", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32), ("cap_tasks", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


class mk_sched_config(ctypes.Structure):
    _fields_ = [("max_seqs", ctypes.c_int32), ("max_rows", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("n_pages", ctypes.c_int64), ("reserve_full", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 3)]


class mk_sched_stats(ctypes.Structure):
    _fields_ = [("queued", ctypes.c_int32), ("running", ctypes.c_int32), ("free_pages", ctypes.c_int32),
                ("reserved_pages", ctypes.c_int32), ("admitted", ctypes.c_int64), ("finished", ctypes.c_int64),
                ("steps", ctypes.c_int64), ("rows", ctypes.c_int64), ("prompt_rows", ctypes.c_int64)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open libmk.so (built in-tree by persistent_megakernel_03_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if "torch" not in sys.modules:
        import torch  # noqa: F401  (share torch's HIP runtime)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m persistent_megakernel_03_amd.build`")
    lib = ctypes.CDLL(path)
    c = ctypes
    lib.mk_kv_pool_bytes.argtypes = [c.POINTER(mk_dims)]
    lib.mk_kv_pool_bytes.restype = c.c_size_t
    lib.mk_workspace_bytes.argtypes = [c.POINTER(mk_dims), c.POINTER(mk_options)]
    lib.mk_workspace_bytes.restype = c.c_size_t
    lib.mk_create.argtypes = [c.POINTER(mk_dims), c.POINTER(mk_weights), c.c_void_p, c.c_void_p, c.c_void_p,
                              c.c_size_t, c.POINTER(mk_options), c.c_int, c.POINTER(c.c_void_p)]
    lib.mk_create.restype = c.c_int
    lib.mk_decode_step.argtypes = [c.c_void_p, c.c_int32, c.POINTER(c.c_int32), c.POINTER(c.c_int32),
                                   c.POINTER(c.c_int32), c.c_void_p, c.c_void_p, c.c_void_p]
    lib.mk_decode_step.restype = c.c_int
    lib.mk_forward_step.argtypes = lib.mk_decode_step.argtypes
    lib.mk_forward_step.restype = c.c_int
    lib.mk_decode_step_noalloc.argtypes = lib.mk_decode_step.argtypes
    lib.mk_decode_step_noalloc.restype = c.c_int
    lib.mk_set_mode.argtypes = [c.c_void_p, c.c_int32]
    lib.mk_set_mode.restype = c.c_int
    lib.mk_sync_check.argtypes = [c.c_void_p, c.c_void_p]
    lib.mk_sync_check.restype = c.c_int
    lib.mk_get_debug_ptrs.argtypes = [c.c_void_p, c.POINTER(mk_debug_ptrs)]
    lib.mk_get_debug_ptrs.restype = c.c_int
    lib.mk_plan_build.argtypes = [c.POINTER(mk_dims), c.POINTER(mk_options), c.c_int32, c.c_int32,
                                  c.POINTER(c.c_int32), c.POINTER(mk_plan_info), c.POINTER(c.c_int32), c.c_int64,
                                  c.POINTER(c.c_int32), c.POINTER(c.c_int32)]
    lib.mk_plan_build.restype = c.c_int
    lib.mk_plan_check.argtypes = [c.POINTER(mk_dims), c.POINTER(mk_options), c.c_int32, c.c_int32,
                                  c.POINTER(c.c_int32), c.POINTER(c.c_int32), c.c_int64, c.POINTER(c.c_int32)]
    lib.mk_plan_check.restype = c.c_int
    lib.mk_get_trace.argtypes = [c.c_void_p, c.c_void_p, c.c_size_t, c.POINTER(c.c_size_t)]
    lib.mk_get_trace.restype = c.c_int
    lib.mk_get_plan.argtypes = [c.c_void_p, c.POINTER(c.c_int32), c.c_int64, c.POINTER(c.c_int64)]
    lib.mk_get_plan.restype = c.c_int
    lib.mk_kernel_time.argtypes = [c.c_void_p, c.POINTER(c.c_float)]
    lib.mk_kernel_time.restype = c.c_int
    lib.mk_destroy.argtypes = [c.c_void_p]
    lib.mk_destroy.restype = None
    lib.mk_last_error.argtypes = []
    lib.mk_last_error.restype = c.c_char_p
    I32P, I64P = c.POINTER(c.c_int32), c.POINTER(c.c_int64)
    lib.mk_sched_create.argtypes = [c.POINTER(mk_sched_config), I32P, c.POINTER(c.c_void_p)]
    lib.mk_sched_destroy.argtypes = [c.c_void_p]
    lib.mk_sched_destroy.restype = None
    lib.mk_sched_submit.argtypes = [c.c_void_p, c.c_int64, c.c_int32, I32P, c.c_int32, c.c_int32]
    lib.mk_sched_release.argtypes = [c.c_void_p, c.c_int64]
    lib.mk_sched_next.argtypes = [c.c_void_p, I32P, I32P, I32P, I32P, I32P, I32P, I64P]
    lib.mk_sched_commit.argtypes = [c.c_void_p, I32P, I32P, I64P, c.c_int32]
    lib.mk_sched_get_stats.argtypes = [c.c_void_p, c.POINTER(mk_sched_stats)]
    lib.mk_sched_tokens.argtypes = [c.c_void_p, c.c_int64, I32P, c.c_int32, I32P]
    for n in ("mk_sched_create", "mk_sched_submit", "mk_sched_release", "mk_sched_next", "mk_sched_commit",
              "mk_sched_get_stats", "mk_sched_tokens"):
        getattr(lib, n).restype = c.c_int
    _lib = lib
    return lib


def _check(st: int):
    if st != MK_OK:
        raise MkError(st, load().mk_last_error().decode())


def _i32(a) -> ctypes.Array:
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def make_dims(cfg: dict, max_batch: int, max_pages_per_seq: int, n_pages: int) -> mk_dims:
    return mk_dims(cfg["n_layers"], cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                   cfg["n_experts"], cfg["top_k"], cfg["moe_inter"], cfg["vocab"], cfg["page_size"],
                   cfg.get("rms_eps", 1e-6), cfg.get("rope_theta", 10000.0), max_batch, max_pages_per_seq,
                   n_pages)


def make_options(mode: int = MK_MODE_MEGAKERNEL, trace: bool = False, watchdog_ns: int = 0, wg_per_cu: int = 0,
                 split_kv_tokens: int = 0, n_cu_override: int = 0, time_kernels: bool = False,
                 shared_levels: int = 0, validate_plans: bool = False, mfma_min_batch: int = 0,
                 poison_exchange: bool = False, mm_row_blocks: int = 0) -> mk_options:
    o = mk_options()
    o.mode, o.trace, o.watchdog_ns = mode, int(bool(trace)), watchdog_ns
    o.wg_per_cu, o.split_kv_tokens, o.n_cu_override = wg_per_cu, split_kv_tokens, n_cu_override
    o.time_kernels = int(bool(time_kernels))
    o.shared_levels = int(shared_levels)
    o.validate_plans = int(bool(validate_plans))
    o.mfma_min_batch = int(mfma_min_batch)
    o.poison_exchange = int(bool(poison_exchange))
    o.mm_row_blocks = int(mm_row_blocks)
    return o


# ----------------------------------------------------------- thin wrappers --

def mk_kv_pool_bytes(dims: mk_dims) -> int:
    return int(load().mk_kv_pool_bytes(ctypes.byref(dims)))


def mk_workspace_bytes(dims: mk_dims, opts: mk_options) -> int:
    return int(load().mk_workspace_bytes(ctypes.byref(dims), ctypes.byref(opts)))


def mk_create(dims: mk_dims, weights: mk_weights, k_pool: int, v_pool: int, workspace: int, workspace_bytes: int,
              opts: mk_options, device: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(load().mk_create(ctypes.byref(dims), ctypes.byref(weights), ctypes.c_void_p(k_pool),
                            ctypes.c_void_p(v_pool), ctypes.c_void_p(workspace), workspace_bytes,
                            ctypes.byref(opts), device, ctypes.byref(h)))
    return h.value


def mk_decode_step(h: int, batch: int, seq_ids, positions, block_tables, tokens: int, logits: int,
                   stream: int) -> None:
    s_arr, s_p = _i32(seq_ids) if seq_ids is not None else (None, None)
    p_arr, p_p = _i32(positions)
    b_arr, b_p = _i32(block_tables)
    _check(load().mk_decode_step(ctypes.c_void_p(h), batch, s_p, p_p, b_p, ctypes.c_void_p(tokens),
                                 ctypes.c_void_p(logits), ctypes.c_void_p(stream)))


def mk_forward_step(h: int, batch: int, seq_ids, positions, block_tables, tokens: int, logits: int,
                    stream: int) -> None:
    s_arr, s_p = _i32(seq_ids)
    p_arr, p_p = _i32(positions)
    b_arr, b_p = _i32(block_tables)
    _check(load().mk_forward_step(ctypes.c_void_p(h), batch, s_p, p_p, b_p, ctypes.c_void_p(tokens),
                                  ctypes.c_void_p(logits), ctypes.c_void_p(stream)))


def mk_decode_step_noalloc(h: int, batch: int, seq_ids, positions, block_tables, tokens: int, logits: int,
                           stream: int) -> None:
    s_arr, s_p = _i32(seq_ids) if seq_ids is not None else (None, None)
    p_arr, p_p = _i32(positions)
    b_arr, b_p = _i32(block_tables)
    _check(load().mk_decode_step_noalloc(ctypes.c_void_p(h), batch, s_p, p_p, b_p, ctypes.c_void_p(tokens),
                                         ctypes.c_void_p(logits), ctypes.c_void_p(stream)))


def mk_set_mode(h: int, mode: int) -> None:
    _check(load().mk_set_mode(ctypes.c_void_p(h), mode))


def mk_sync_check(h: int, stream: int) -> int:
    """Returns the status (MK_OK, MK_ERR_TIMEOUT, MK_ERR_DEVICE) instead of raising for device errors."""
    st = load().mk_sync_check(ctypes.c_void_p(h), ctypes.c_void_p(stream))
    if st in (MK_OK, MK_ERR_TIMEOUT, MK_ERR_DEVICE):
        return st
    _check(st)
    return st


def mk_get_debug_ptrs(h: int) -> mk_debug_ptrs:
    out = mk_debug_ptrs()
    _check(load().mk_get_debug_ptrs(ctypes.c_void_p(h), ctypes.byref(out)))
    return out


def mk_plan_build(dims: mk_dims, opts: mk_options, n_wg: int, positions: Sequence[int]):
    """Returns (info, tasks [n_tasks][12] int32, wg_offsets, counter_targets)."""
    lib = load()
    p_arr, p_p = _i32(positions)
    info = mk_plan_info()
    _check(lib.mk_plan_build(ctypes.byref(dims), ctypes.byref(opts), n_wg, len(p_arr), p_p, ctypes.byref(info),
                             None, 0, None, None))
    tasks = np.zeros((info.n_tasks, 12), np.int32)
    offs = np.zeros(info.n_wg + 1, np.int32)
    targets = np.zeros(info.n_counters, np.int32)
    _check(lib.mk_plan_build(ctypes.byref(dims), ctypes.byref(opts), n_wg, len(p_arr), p_p, ctypes.byref(info),
                             tasks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), info.n_tasks,
                             offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                             targets.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return info, tasks, offs, targets


def mk_plan_check(dims: mk_dims, opts: mk_options, n_wg: int, positions: Sequence[int], tasks: np.ndarray,
                  offs: np.ndarray) -> None:
    """Raises MkError(MK_ERR_INVALID) naming the first rule the task table breaks."""
    p_arr, p_p = _i32(positions)
    t_arr = np.ascontiguousarray(tasks, dtype=np.int32)
    o_arr, o_p = _i32(offs)
    _check(load().mk_plan_check(ctypes.byref(dims), ctypes.byref(opts), n_wg, len(p_arr), p_p,
                                t_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), t_arr.shape[0], o_p))


def mk_get_trace(h: int) -> np.ndarray:
    lib = load()
    n = ctypes.c_size_t()
    _check(lib.mk_get_trace(ctypes.c_void_p(h), None, 0, ctypes.byref(n)))
    buf = np.zeros(n.value // 8, np.uint64)
    _check(lib.mk_get_trace(ctypes.c_void_p(h), buf.ctypes.data_as(ctypes.c_void_p), n.value, ctypes.byref(n)))
    return buf.reshape(-1, 8)


def mk_get_plan(h: int) -> np.ndarray:
    """Task table [n_tasks][12] int32 of the plan the last step ran."""
    lib = load()
    n = ctypes.c_int64()
    _check(lib.mk_get_plan(ctypes.c_void_p(h), None, 0, ctypes.byref(n)))
    tasks = np.zeros((n.value, 12), np.int32)
    _check(lib.mk_get_plan(ctypes.c_void_p(h), tasks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value,
                           ctypes.byref(n)))
    return tasks


def mk_kernel_time(h: int) -> float:
    ms = ctypes.c_float()
    _check(load().mk_kernel_time(ctypes.c_void_p(h), ctypes.byref(ms)))
    return float(ms.value)


def mk_destroy(h: int) -> None:
    load().mk_destroy(ctypes.c_void_p(h))


# ------------------------------------------------------------ convenience --

def check_step_args(dims: mk_dims, vocab: int, positions, block_tables, tokens, logits, device, seq_ids=None):
    """Shapes, dtypes and placement of one step's arguments, checked before
    the C ABI sees raw pointers (it trusts them: block-table rows are read
    max_pages_per_seq entries long, logits are written batch x vocab floats).
    Returns the positions and block tables as contiguous int32 arrays.
    Raises MkError(MK_ERR_INVALID)."""
    import torch

    def bad(msg):
        raise MkError(MK_ERR_INVALID, msg)

    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(-1))
    B = int(pos.shape[0])
    if B <= 0:
        bad("batch must be positive")
    if np.any(pos > np.iinfo(np.int32).max):
        bad("position out of int32 range")
    bt = np.asarray(block_tables)
    if bt.ndim != 2 or bt.shape[0] < B or bt.shape[1] != dims.max_pages_per_seq:
        bad(f"block_tables must be [batch >= {B}][max_pages_per_seq = {dims.max_pages_per_seq}], got {bt.shape}")
    if not np.issubdtype(bt.dtype, np.integer):
        bad("block_tables must hold integers")
    if seq_ids is not None and len(seq_ids) < B:
        bad(f"seq_ids holds {len(seq_ids)} entries for a batch of {B}")
    for name, t, dt, n in (("tokens", tokens, torch.int32, B), ("logits", logits, torch.float32, B * vocab)):
        if not isinstance(t, torch.Tensor):
            bad(f"{name} must be a torch tensor")
        if t.dtype != dt:
            bad(f"{name} must be {dt}, got {t.dtype}")
        if t.device != torch.device(device):
            bad(f"{name} must be on {device}, got {t.device}")
        if not t.is_contiguous():
            bad(f"{name} must be contiguous")
        if t.numel() < n:
            bad(f"{name} holds {t.numel()} elements, the step needs {n}")
    if logits.dim() == 2 and logits.shape[1] != vocab:
        bad(f"logits rows must be vocab = {vocab} wide, got {logits.shape[1]}")
    return pos.astype(np.int32), np.ascontiguousarray(bt[:B], dtype=np.int32)


class Decoder:
    """Owns the torch tensors a handle points into (weights dict, KV pools,
    workspace) and forwards calls to the C ABI. No arithmetic happens here."""

    def __init__(self, cfg: dict, weights: Dict[str, "torch.Tensor"], k_pool, v_pool, max_batch: int,
                 max_pages_per_seq: int, mode: int = MK_MODE_MEGAKERNEL, trace: bool = False,
                 watchdog_ns: int = 0, wg_per_cu: int = 0, split_kv_tokens: int = 0, device: int = 0,
                 time_kernels: bool = False, shared_levels: int = 0, validate_plans: bool = False,
                 mfma_min_batch: int = 0, poison_exchange: bool = False, mm_row_blocks: int = 0):
        import torch
        self.cfg = dict(cfg)
        self.dims = make_dims(cfg, max_batch, max_pages_per_seq, k_pool.shape[1])
        self.opts = make_options(mode, trace, watchdog_ns, wg_per_cu, split_kv_tokens, 0, time_kernels, shared_levels,
                                 validate_plans, mfma_min_batch, poison_exchange, mm_row_blocks)
        L = cfg["n_layers"]
        self._keep: List = [weights, k_pool, v_pool]

        def arr(kind):
            a = (ctypes.c_void_p * L)(*[weights[f"layers.{l}.{kind}"].data_ptr() for l in range(L)])
            self._keep.append(a)
            return ctypes.cast(a, _PP)

        w = mk_weights()
        w.embed = weights["embed"].data_ptr()
        w.lm_head = weights["lm_head"].data_ptr()
        w.final_norm = weights["final_norm"].data_ptr()
        w.attn_norm, w.wqkv, w.wo = arr("attn_norm"), arr("wqkv"), arr("wo")
        w.ffn_norm, w.router = arr("ffn_norm"), arr("router")
        w.w_gate, w.w_up, w.w_down = arr("w_gate"), arr("w_up"), arr("w_down")
        if f"layers.0.router_bias" in weights:
            w.router_bias = arr("router_bias")
        self.weights_struct = w
        nbytes = mk_workspace_bytes(self.dims, self.opts)
        if nbytes == 0:
            raise MkError(MK_ERR_UNSUPPORTED, load().mk_last_error().decode() or "unsupported dims")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=k_pool.device)
        self.k_pool, self.v_pool = k_pool, v_pool
        self.handle = mk_create(self.dims, w, k_pool.data_ptr(), v_pool.data_ptr(), self.workspace.data_ptr(),
                                nbytes, self.opts, device)

    def step(self, positions, block_tables, tokens, logits, stream=None, seq_ids=None):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        positions, block_tables = check_step_args(self.dims, self.cfg["vocab"], positions, block_tables, tokens,
                                                  logits, self.k_pool.device, seq_ids)
        mk_decode_step(self.handle, len(positions), seq_ids, positions, block_tables,
                       tokens.data_ptr(), logits.data_ptr(), stream)

    def forward(self, seq_ids, positions, block_tables, tokens, logits, stream=None):
        """A multi-token step (mk_forward_step): rows of one sequence are
        adjacent with equal seq_ids at consecutive positions."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        if seq_ids is None:
            raise MkError(MK_ERR_INVALID, "a multi-token step needs seq_ids")
        positions, block_tables = check_step_args(self.dims, self.cfg["vocab"], positions, block_tables, tokens,
                                                  logits, self.k_pool.device, seq_ids)
        mk_forward_step(self.handle, len(positions), seq_ids, positions, block_tables,
                        tokens.data_ptr(), logits.data_ptr(), stream)

    def set_mode(self, mode: int):
        mk_set_mode(self.handle, mode)

    def sync_check(self, stream=None) -> int:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return mk_sync_check(self.handle, stream)

    def kernel_ms(self) -> float:
        return mk_kernel_time(self.handle)

    def debug(self) -> mk_debug_ptrs:
        return mk_get_debug_ptrs(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            mk_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------- scheduler --

class Scheduler:
    """The host continuous-batching scheduler (include/mk_sched.h): request
    queue, admission, page allocator and the rows of each step. Argument
    marshalling only; the policy lives in libmk."""

    def __init__(self, max_seqs: int, max_rows: int, page_size: int, max_pages_per_seq: int, n_pages: int,
                 reserve_full: bool = True, page_order=None):
        cfg = mk_sched_config(max_seqs, max_rows, page_size, max_pages_per_seq, n_pages, int(bool(reserve_full)))
        self.max_rows, self.max_pages = max_rows, max_pages_per_seq
        order = None
        if page_order is not None:
            self._order, order = _i32(page_order)
        h = ctypes.c_void_p()
        _check(load().mk_sched_create(ctypes.byref(cfg), order, ctypes.byref(h)))
        self.handle = h.value
        R, M = max_rows, max_pages_per_seq
        self.seq_ids = np.zeros(R, np.int32)
        self.positions = np.zeros(R, np.int32)
        self.block_tables = np.zeros((R, M), np.int32)
        self.tokens = np.zeros(R, np.int32)
        self.sample = np.zeros(R, np.int32)
        self.request_ids = np.zeros(R, np.int64)
        self._fin = np.zeros(R, np.int64)

    @staticmethod
    def _p(a):
        return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32 if a.dtype == np.int32 else ctypes.c_int64))

    def submit(self, request_id: int, prompt, max_new_tokens: int, cached_len: int = 0) -> None:
        arr, ptr = _i32(prompt)
        _check(load().mk_sched_submit(ctypes.c_void_p(self.handle), int(request_id), int(cached_len), ptr, len(arr),
                                      int(max_new_tokens)))

    def release(self, request_id: int) -> None:
        _check(load().mk_sched_release(ctypes.c_void_p(self.handle), int(request_id)))

    def next(self) -> int:
        """Lay out the next step; returns the number of rows (views of the
        arrays above hold them)."""
        n = ctypes.c_int32()
        _check(load().mk_sched_next(ctypes.c_void_p(self.handle), ctypes.byref(n), self._p(self.seq_ids),
                                    self._p(self.positions), self._p(self.block_tables), self._p(self.tokens),
                                    self._p(self.sample), self._p(self.request_ids)))
        return int(n.value)

    def commit(self, next_tokens) -> list:
        """next_tokens: one per row of the step (read where sample == 1).
        Returns the ids of the requests that finished."""
        arr, ptr = _i32(next_tokens)
        nf = ctypes.c_int32()
        _check(load().mk_sched_commit(ctypes.c_void_p(self.handle), ptr, ctypes.byref(nf), self._p(self._fin),
                                      len(self._fin)))
        return [int(x) for x in self._fin[:min(nf.value, len(self._fin))]]

    def stats(self) -> dict:
        st = mk_sched_stats()
        _check(load().mk_sched_get_stats(ctypes.c_void_p(self.handle), ctypes.byref(st)))
        return {k: int(getattr(st, k)) for k, _ in mk_sched_stats._fields_}

    def tokens_of(self, request_id: int) -> list:
        n = ctypes.c_int32()
        _check(load().mk_sched_tokens(ctypes.c_void_p(self.handle), int(request_id), None, 0, ctypes.byref(n)))
        out = np.zeros(max(1, n.value), np.int32)
        _check(load().mk_sched_tokens(ctypes.c_void_p(self.handle), int(request_id), self._p(out), n.value,
                                      ctypes.byref(n)))
        return [int(x) for x in out[:n.value]]

    def close(self):
        if getattr(self, "handle", None):
            load().mk_sched_destroy(ctypes.c_void_p(self.handle))
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass
