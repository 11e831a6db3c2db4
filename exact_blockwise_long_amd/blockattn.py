"""Thin ctypes binding of libblockattn.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels.  PyTorch is
used only to own device memory and to name the current stream; this module
turns tensors into pointers, strides and sizes, allocates the workspace the
library asks for, and raises ``BlockAttnError`` on a non-zero status.  There
is no CPU path: if the built library is missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libblockattn.so")

BA_F32, BA_BF16 = 0, 1
MAX_VISITS = 32
MAX_MERGE_PARTS = 64
STATIC_SCRATCH_BYTES = 64 << 20   # BLOCKATTN_STATIC_SCRATCH_BYTES

STATUS = {0: "BA_OK", 1: "BA_ERR_NULL", 2: "BA_ERR_SHAPE", 3: "BA_ERR_UNSUPPORTED",
          4: "BA_ERR_ORDER", 5: "BA_ERR_WORKSPACE", 6: "BA_ERR_HIP"}


class BlockAttnError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{func}: {self.name}: {msg}")


class Problem(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_len", ctypes.c_int32), ("q_pos0", ctypes.c_int64),
        ("q_stride_token", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("split_mode", ctypes.c_int32), ("batch", ctypes.c_int32), ("q_stride_batch", ctypes.c_int64),
    ]


class KVBlock(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_int32), ("pos0", ctypes.c_int64),
        ("k_stride_token", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("k_stride_batch", ctypes.c_int64), ("v_stride_batch", ctypes.c_int64),
    ]


class State(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("l", ctypes.c_void_p), ("o", ctypes.c_void_p)]


class Fanout(ctypes.Structure):
    _fields_ = [
        ("n_branches", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("prefix_len", ctypes.c_int32), ("suffix_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class FanoutPrefill(ctypes.Structure):
    _fields_ = [
        ("n_branches", ctypes.c_int32), ("n_new", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("prefix_len", ctypes.c_int32),
        ("suffix_len", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


class KVPages(ctypes.Structure):
    _fields_ = [
        ("prefix_pages", ctypes.c_void_p), ("suffix_pages", ctypes.c_void_p), ("page_len", ctypes.c_int32),
        ("n_pool_pages", ctypes.c_int32),
    ]


EXPORTS = [
    "blockattn_fwd_block", "blockattn_fwd_block_finalize", "blockattn_fwd_workspace_bytes",
    "blockattn_shard_states", "blockattn_shard_workspace_bytes", "blockattn_merge_states", "blockattn_finalize",
    "fanout_prefix_decode", "fanout_workspace_bytes", "fanout_prefix_decode_noalloc", "fanout_prefix_prefill",
    "fanout_prefill_workspace_bytes",
    "fanout_prefix_decode_paged", "fanout_prefix_prefill_paged", "blockattn_workspace_bytes",
    "blockattn_bwd_delta", "blockattn_bwd_block", "blockattn_status_str", "blockattn_last_error",
    "blockattn_abi_version",
]

_lib = None


def hip_runtimes_loaded() -> List[str]:
    """Paths of every libamdhip64 mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and "libamdhip64" in parts[5]:
                paths.add(parts[5])
    return sorted(paths)


def load():
    """Load the library (after torch, so both use torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_blockwise_long_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    lib.blockattn_fwd_block.argtypes = [P(Problem), vp, P(KVBlock), i32, P(i32), i32, State, i32, vp, sz, vp]
    lib.blockattn_fwd_block.restype = i32
    lib.blockattn_fwd_block_finalize.argtypes = [P(Problem), vp, P(KVBlock), i32, P(i32), i32, State, i32, vp, i32,
                                                 i64, vp, vp, sz, vp]
    lib.blockattn_fwd_block_finalize.restype = i32
    lib.blockattn_fwd_workspace_bytes.argtypes = [P(Problem), P(KVBlock), i32, P(i32), i32]
    lib.blockattn_fwd_workspace_bytes.restype = sz
    lib.blockattn_shard_states.argtypes = [P(Problem), vp, P(KVBlock), i32, P(State), vp, sz, vp]
    lib.blockattn_shard_states.restype = i32
    lib.blockattn_shard_workspace_bytes.argtypes = [P(Problem), P(KVBlock), i32]
    lib.blockattn_shard_workspace_bytes.restype = sz
    lib.blockattn_merge_states.argtypes = [i32, P(State), i64, i32, State, vp]
    lib.blockattn_merge_states.restype = i32
    lib.blockattn_finalize.argtypes = [State, i64, i32, vp, i32, i64, vp, vp]
    lib.blockattn_finalize.restype = i32
    lib.fanout_prefix_decode.argtypes = [P(Fanout), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fanout_prefix_decode.restype = i32
    lib.fanout_workspace_bytes.argtypes = [P(Fanout)]
    lib.fanout_workspace_bytes.restype = sz
    lib.fanout_prefix_decode_noalloc.argtypes = [P(Fanout), vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fanout_prefix_decode_noalloc.restype = i32
    lib.blockattn_bwd_delta.argtypes = [i64, i32, vp, i32, i64, vp, i64, vp, vp]
    lib.blockattn_bwd_delta.restype = i32
    lib.blockattn_bwd_block.argtypes = [P(Problem), vp, vp, vp, vp, P(KVBlock), i32, P(i32), i32, vp,
                                        P(ctypes.c_void_p), P(ctypes.c_void_p), vp]
    lib.blockattn_bwd_block.restype = i32
    lib.fanout_prefix_prefill.argtypes = [P(FanoutPrefill), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fanout_prefix_prefill.restype = i32
    lib.fanout_prefill_workspace_bytes.argtypes = [P(FanoutPrefill)]
    lib.fanout_prefill_workspace_bytes.restype = sz
    lib.blockattn_workspace_bytes.argtypes = [P(Problem), P(Fanout)]
    lib.blockattn_workspace_bytes.restype = sz
    lib.fanout_prefix_decode_paged.argtypes = [P(Fanout), P(KVPages), vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fanout_prefix_decode_paged.restype = i32
    lib.fanout_prefix_prefill_paged.argtypes = [P(FanoutPrefill), P(KVPages), vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fanout_prefix_prefill_paged.restype = i32
    lib.blockattn_status_str.argtypes = [i32]
    lib.blockattn_status_str.restype = ctypes.c_char_p
    lib.blockattn_last_error.argtypes = []
    lib.blockattn_last_error.restype = ctypes.c_char_p
    lib.blockattn_abi_version.argtypes = []
    lib.blockattn_abi_version.restype = i32
    _lib = lib
    return lib


def _check(status: int, func: str):
    if status != 0:
        raise BlockAttnError(status, func, load().blockattn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# Debug canary: when set, every buffer this module allocates (workspaces,
# states from new_state, outputs) is filled with 0xFF bytes -- NaN as fp32 and
# as bf16 -- before the call, so a kernel that reads a slot before writing it,
# or lets a key outside its range into a result, shows NaN instead of stale
# values.
_poison = False


def set_poison(enabled: bool) -> bool:
    """Turns the NaN canary on or off; returns the previous setting."""
    global _poison
    prev, _poison = _poison, bool(enabled)
    return prev


def _empty(shape, dtype, device, stream=None) -> torch.Tensor:
    """Uninitialised device memory for a call enqueued on ``stream``.

    The allocation is made on that stream, so the caching allocator hands the
    memory to other work only in that stream's order: a buffer dropped on return
    (an auto-sized workspace) is not reused while the call still runs.
    """
    if stream is None or stream == torch.cuda.current_stream(device):
        t = torch.empty(shape, dtype=dtype, device=device)
        if _poison:
            t.view(torch.uint8).fill_(0xFF)
        return t
    with torch.cuda.stream(stream):
        t = torch.empty(shape, dtype=dtype, device=device)
        if _poison:
            t.view(torch.uint8).fill_(0xFF)
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BA_BF16
    if t.dtype == torch.float32:
        return BA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dim_contig(t: torch.Tensor, name: str, batched: bool = False):
    if t.dim() != (4 if batched else 3) or t.stride(-1) != 1:
        shape = "[batch, tokens, heads, head_dim]" if batched else "[tokens, heads, head_dim]"
        raise ValueError(f"{name} must be {shape} with a contiguous head_dim axis")


def _qshape(q: torch.Tensor):
    """(batch, q_len, n_q_heads, head_dim, batched) of a query block: [T, Hq, D]
    is one sequence, [B, T, Hq, D] a batch of B sequences."""
    if q.dim() == 3:
        T, Hq, D = q.shape
        return 1, T, Hq, D, False
    if q.dim() == 4:
        B, T, Hq, D = q.shape
        return B, T, Hq, D, True
    raise ValueError("q must be [tokens, heads, head_dim] or [batch, tokens, heads, head_dim]")


def _rows(q: torch.Tensor) -> int:
    """State rows of a query block: batch * q_len * n_q_heads."""
    B, T, Hq, _, _ = _qshape(q)
    return B * T * Hq


def _check_state(state, rows: int, head_dim: int, name: str = "state"):
    """The library reads and writes the first rows entries of m and l and the
    first rows x head_dim of o: the tensors must be contiguous fp32 holding at
    least that (o with rows of exactly head_dim)."""
    m, l, o = state
    for t, n in ((m, "m"), (l, "l")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < rows:
            raise ValueError(f"{name}.{n} must be contiguous fp32 with at least {rows} entries")
    if o.dtype != torch.float32 or not o.is_contiguous() or o.dim() != 2 or o.shape[1] != head_dim or \
            o.shape[0] < rows:
        raise ValueError(f"{name}.o must be contiguous fp32 [>= {rows}, {head_dim}]")


def _check_blocks(blocks, n_kv_heads: int, head_dim: int, dtype, batch: int = 1):
    """Every K/V block must carry n_kv_heads heads of head_dim in the problem's
    dtype: [len, Hkv, D], or [batch, len, Hkv, D] for a batched problem (a
    3-D block is then shared by all its sequences)."""
    for i, (k, v, _) in enumerate(blocks):
        for t, n in ((k, "k"), (v, "v")):
            ok_shape = (t.dim() == 3 or (t.dim() == 4 and batch > 1 and t.shape[0] == batch)) and \
                t.shape[-2] == n_kv_heads and t.shape[-1] == head_dim
            if not ok_shape or t.dtype != dtype:
                raise ValueError(f"block {i}: {n} must be [len, {n_kv_heads}, {head_dim}]"
                                 f"{f' or [{batch}, len, {n_kv_heads}, {head_dim}]' if batch > 1 else ''} {dtype}, "
                                 f"got {tuple(t.shape)} {t.dtype}")


def from_host(storage, bf16: bool, device="cuda") -> torch.Tensor:
    """A host array as a device tensor: uint16 bf16 bit patterns become
    bfloat16 (bf16=True), float32 values stay float32."""
    import numpy as np
    arr = np.ascontiguousarray(storage)
    if bf16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def new_state(rows: int, head_dim: int, device="cuda", stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Uninitialised fp32 state buffers (m [rows], l [rows], o [rows, D])."""
    return (_empty(rows, torch.float32, device, stream),
            _empty(rows, torch.float32, device, stream),
            _empty((rows, head_dim), torch.float32, device, stream))


def _state(st) -> State:
    m, l, o = st
    return State(m.data_ptr(), l.data_ptr(), o.data_ptr())


def make_problem(q: torch.Tensor, n_kv_heads: int, q_pos0: int = 0, causal: bool = False,
                 scale: float = 0.0, split_mode: int = 0) -> Problem:
    """q [T, Hq, D] (one sequence) or [B, T, Hq, D] (a batch of B sequences)."""
    B, T, Hq, D, batched = _qshape(q)
    _dim_contig(q, "q", batched)
    st = q.stride()
    qsb, qst, qsh = (st[0], st[1], st[2]) if batched else (0, st[0], st[1])
    return Problem(Hq, n_kv_heads, D, T, q_pos0, qst, qsh, _dtype_code(q), scale, 1 if causal else 0, split_mode,
                   B if batched else 0, qsb)


def make_blocks(blocks: Sequence[Tuple[torch.Tensor, torch.Tensor, int]]):
    """Blocks (k, v, pos0), k and v [len, Hkv, D] or [batch, len, Hkv, D]; a 3-D
    block has batch stride 0 (shared by the sequences of a batched problem)."""
    arr = (KVBlock * max(1, len(blocks)))()
    for i, (k, v, pos0) in enumerate(blocks):
        batched = k.dim() == 4
        _dim_contig(k, "k", batched)
        _dim_contig(v, "v", batched)
        if k.shape != v.shape:
            raise ValueError("k and v blocks must have the same shape")
        ks, vs = k.stride(), v.stride()
        if batched:
            arr[i] = KVBlock(k.data_ptr(), v.data_ptr(), k.shape[1], pos0, ks[1], ks[2], vs[1], vs[2], ks[0], vs[0])
        else:
            arr[i] = KVBlock(k.data_ptr(), v.data_ptr(), k.shape[0], pos0, ks[0], ks[1], vs[0], vs[1], 0, 0)
    return arr


def fwd_block(q: torch.Tensor, blocks: Sequence[Tuple[torch.Tensor, torch.Tensor, int]],
              order: Optional[Sequence[int]], state, reset: bool, *, n_kv_heads: int, q_pos0: int = 0,
              causal: bool = False, scale: float = 0.0, split_mode: int = 0,
              workspace: Optional[torch.Tensor] = None, stream=None):
    """blockattn_fwd_block: walk ``blocks`` in ``order`` updating ``state`` (m, l, o) in place."""
    lib = load()
    p = make_problem(q, n_kv_heads, q_pos0, causal, scale, split_mode)
    B, T, Hq, D, _ = _qshape(q)
    _check_blocks(blocks, n_kv_heads, D, q.dtype, B)
    _check_state(state, B * T * Hq, D)
    arr = make_blocks(blocks)
    n_visit = len(order) if order is not None else len(blocks)
    order_arr = (ctypes.c_int32 * max(1, n_visit))(*(order or []))
    order_ptr = order_arr if order is not None else None
    need = lib.blockattn_fwd_workspace_bytes(ctypes.byref(p), arr, len(blocks), order_ptr, n_visit)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.blockattn_fwd_block(ctypes.byref(p), _ptr(q), arr, len(blocks), order_ptr, n_visit,
                                   _state(state), 1 if reset else 0, _ptr(workspace), ws_bytes,
                                   _stream(stream)), "blockattn_fwd_block")
    return state


def fwd_block_finalize(q: torch.Tensor, blocks: Sequence[Tuple[torch.Tensor, torch.Tensor, int]],
                       order: Optional[Sequence[int]], state, reset: bool, *, n_kv_heads: int, q_pos0: int = 0,
                       causal: bool = False, scale: float = 0.0, split_mode: int = 0,
                       out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None, want_lse: bool = True,
                       lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """blockattn_fwd_block_finalize: the visits of fwd_block, then the finalised
    (A [rows, D], lse [rows] or None) in one call; ``state`` is read when not
    ``reset`` and left unspecified."""
    lib = load()
    p = make_problem(q, n_kv_heads, q_pos0, causal, scale, split_mode)
    B, T, Hq, D, _ = _qshape(q)
    rows = B * T * Hq
    _check_blocks(blocks, n_kv_heads, D, q.dtype, B)
    _check_state(state, rows, D)
    if out is None:
        out = _empty((rows, D), out_dtype, q.device, stream)
    elif out.dim() != 2 or out.shape[0] != rows or out.shape[1] != D or out.stride(1) != 1 or \
            out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"out must be bf16 or fp32 [{rows}, {D}] with contiguous rows")
    if lse is None and want_lse:
        lse = _empty(rows, torch.float32, q.device, stream)
    elif lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != rows):
        raise ValueError(f"lse must be contiguous fp32 with {rows} entries")
    arr = make_blocks(blocks)
    n_visit = len(order) if order is not None else len(blocks)
    order_arr = (ctypes.c_int32 * max(1, n_visit))(*(order or []))
    order_ptr = order_arr if order is not None else None
    need = lib.blockattn_fwd_workspace_bytes(ctypes.byref(p), arr, len(blocks), order_ptr, n_visit)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = BA_BF16 if out.dtype == torch.bfloat16 else BA_F32
    _check(lib.blockattn_fwd_block_finalize(ctypes.byref(p), _ptr(q), arr, len(blocks), order_ptr, n_visit,
                                            _state(state), 1 if reset else 0, _ptr(out), code, out.stride(0),
                                            _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)),
           "blockattn_fwd_block_finalize")
    return out, lse


def fwd_workspace_bytes(q, blocks, order, *, n_kv_heads, q_pos0=0, causal=False, split_mode=0) -> int:
    lib = load()
    p = make_problem(q, n_kv_heads, q_pos0, causal, 0.0, split_mode)
    arr = make_blocks(blocks)
    n_visit = len(order) if order is not None else len(blocks)
    order_arr = (ctypes.c_int32 * max(1, n_visit))(*(order or []))
    return lib.blockattn_fwd_workspace_bytes(ctypes.byref(p), arr, len(blocks),
                                             order_arr if order is not None else None, n_visit)


def shard_states(q: torch.Tensor, blocks, states_out, *, n_kv_heads: int, q_pos0: int = 0,
                 causal: bool = False, scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                 stream=None):
    """blockattn_shard_states: one partial state per block into ``states_out``."""
    lib = load()
    p = make_problem(q, n_kv_heads, q_pos0, causal, scale, 0)
    B, T, Hq, D, _ = _qshape(q)
    _check_blocks(blocks, n_kv_heads, D, q.dtype, B)
    if len(states_out) != len(blocks):
        raise ValueError("one output state per block")
    for i, st in enumerate(states_out):
        _check_state(st, B * T * Hq, D, f"states_out[{i}]")
    arr = make_blocks(blocks)
    sts = (State * max(1, len(blocks)))(*[_state(s) for s in states_out])
    need = lib.blockattn_shard_workspace_bytes(ctypes.byref(p), arr, len(blocks))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.blockattn_shard_states(ctypes.byref(p), _ptr(q), arr, len(blocks), sts, _ptr(workspace),
                                      ws_bytes, _stream(stream)), "blockattn_shard_states")
    return states_out


def merge_states(parts, out, stream=None):
    """blockattn_merge_states over a list of (m, l, o) states into ``out``."""
    lib = load()
    rows, D = out[2].shape
    _check_state(out, rows, D, "out")
    for i, st in enumerate(parts):
        _check_state(st, rows, D, f"parts[{i}]")
    arr = (State * max(1, len(parts)))(*[_state(s) for s in parts])
    _check(lib.blockattn_merge_states(len(parts), arr, rows, D, _state(out), _stream(stream)),
           "blockattn_merge_states")
    return out


def finalize(state, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None, want_lse: bool = True,
             lse: Optional[torch.Tensor] = None, stream=None):
    """blockattn_finalize: returns (A [rows, D], lse [rows] or None)."""
    lib = load()
    m, l, o = state
    rows, D = o.shape
    _check_state(state, rows, D)
    if out is None:
        out = _empty((rows, D), out_dtype, o.device, stream)
    elif out.dim() != 2 or out.shape[0] != rows or out.shape[1] != D or out.stride(1) != 1 or \
            out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"out must be bf16 or fp32 [{rows}, {D}] with contiguous rows")
    if lse is None and want_lse:
        lse = _empty(rows, torch.float32, o.device, stream)
    elif lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != rows):
        raise ValueError(f"lse must be contiguous fp32 with {rows} entries")
    code = BA_BF16 if out.dtype == torch.bfloat16 else BA_F32
    _check(lib.blockattn_finalize(_state(state), rows, D, _ptr(out), code, out.stride(0), _ptr(lse),
                                  _stream(stream)), "blockattn_finalize")
    return out, lse


def _check_fanout(q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse, rows_shape, Hkv, D, P, S):
    """Shapes the fan-out entry points read and write: q and out are
    rows_shape + [D] (out bf16), lse rows_shape (fp32), the prefix [P, Hkv, D]
    and each suffix [nb, S, Hkv, D]; all contiguous."""
    nb = rows_shape[0]
    want = {"prefix_k": (prefix_k, (P, Hkv, D)), "prefix_v": (prefix_v, (P, Hkv, D)),
            "suffix_k": (suffix_k, (nb, S, Hkv, D)), "suffix_v": (suffix_v, (nb, S, Hkv, D))}
    for name, (t, shape) in want.items():
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if (prefix_k is None) != (prefix_v is None) or (suffix_k is None) != (suffix_v is None):
        raise ValueError("k and v come in pairs (prefix and suffix)")
    if out is not None and (tuple(out.shape) != tuple(rows_shape) + (D,) or out.dtype != torch.bfloat16
                            or not out.is_contiguous()):
        raise ValueError(f"out must be contiguous bf16 of shape {tuple(rows_shape) + (D,)}")
    if lse is not None and (tuple(lse.shape) != tuple(rows_shape) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError(f"lse must be contiguous fp32 of shape {tuple(rows_shape)}")


def fanout_prefix_decode(q, prefix_k, prefix_v, suffix_k, suffix_v, scale: float = 0.0,
                         workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """fanout_prefix_decode: q [nb, Hq, D]; prefix [P, Hkv, D]; suffix [nb, S, Hkv, D] (all contiguous bf16)."""
    lib = load()
    nb, Hq, D = q.shape
    Hkv = prefix_k.shape[1] if prefix_k is not None else suffix_k.shape[2]
    P = prefix_k.shape[0] if prefix_k is not None else 0
    S = suffix_k.shape[1] if suffix_k is not None else 0
    for name, t in (("q", q), ("prefix_k", prefix_k), ("prefix_v", prefix_v), ("suffix_k", suffix_k),
                    ("suffix_v", suffix_v)):
        if t is not None and (not t.is_contiguous() or t.dtype != torch.bfloat16):
            raise ValueError(f"{name} must be contiguous bf16")
    _check_fanout(q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse, (nb, Hq), Hkv, D, P, S)
    f = Fanout(nb, Hq, Hkv, D, P, S, scale)
    need = lib.fanout_workspace_bytes(ctypes.byref(f))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = _empty((nb, Hq, D), torch.bfloat16, q.device, stream)
    if lse is None and want_lse:
        lse = _empty((nb, Hq), torch.float32, q.device, stream)
    _check(lib.fanout_prefix_decode(ctypes.byref(f), _ptr(q), _ptr(prefix_k), _ptr(prefix_v), _ptr(suffix_k),
                                    _ptr(suffix_v), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                    _stream(stream)), "fanout_prefix_decode")
    return out, lse


def fanout_prefix_decode_noalloc(q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse=None, scale: float = 0.0,
                                 stream=None):
    """fanout_prefix_decode_noalloc: fanout_prefix_decode with the library's static
    per-device scratch instead of a workspace.  ``out`` [nb, Hq, D] bf16 (and
    ``lse`` [nb, Hq] fp32, optional) are the caller's; this wrapper allocates
    nothing, so it can run under graph capture."""
    lib = load()
    nb, Hq, D = q.shape
    Hkv = prefix_k.shape[1] if prefix_k is not None else suffix_k.shape[2]
    P = prefix_k.shape[0] if prefix_k is not None else 0
    S = suffix_k.shape[1] if suffix_k is not None else 0
    for name, t in (("q", q), ("prefix_k", prefix_k), ("prefix_v", prefix_v), ("suffix_k", suffix_k),
                    ("suffix_v", suffix_v)):
        if t is not None and (not t.is_contiguous() or t.dtype != torch.bfloat16):
            raise ValueError(f"{name} must be contiguous bf16")
    if out is None:
        raise ValueError("out is required (the allocation-free entry point allocates nothing)")
    _check_fanout(q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse, (nb, Hq), Hkv, D, P, S)
    f = Fanout(nb, Hq, Hkv, D, P, S, scale)
    _check(lib.fanout_prefix_decode_noalloc(ctypes.byref(f), _ptr(q), _ptr(prefix_k), _ptr(prefix_v),
                                            _ptr(suffix_k), _ptr(suffix_v), _ptr(out), _ptr(lse), _stream(stream)),
           "fanout_prefix_decode_noalloc")
    return out, lse


def fanout_workspace_bytes(n_branches, n_q_heads, n_kv_heads, head_dim, prefix_len, suffix_len) -> int:
    f = Fanout(n_branches, n_q_heads, n_kv_heads, head_dim, prefix_len, suffix_len, 0.0)
    return load().fanout_workspace_bytes(ctypes.byref(f))


def fanout_prefix_prefill(q, prefix_k, prefix_v, suffix_k, suffix_v, scale: float = 0.0,
                          workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """fanout_prefix_prefill: q [nb, T, Hq, D] (each branch's T newest tokens); prefix [P, Hkv, D];
    suffix [nb, S, Hkv, D] whose last T tokens are the new ones (all contiguous bf16).
    Returns out [nb, T, Hq, D] bf16 and lse [nb, T, Hq]."""
    lib = load()
    nb, T, Hq, D = q.shape
    Hkv = prefix_k.shape[1] if prefix_k is not None else suffix_k.shape[2]
    P = prefix_k.shape[0] if prefix_k is not None else 0
    S = suffix_k.shape[1] if suffix_k is not None else 0
    for name, t in (("q", q), ("prefix_k", prefix_k), ("prefix_v", prefix_v), ("suffix_k", suffix_k),
                    ("suffix_v", suffix_v)):
        if t is not None and (not t.is_contiguous() or t.dtype != torch.bfloat16):
            raise ValueError(f"{name} must be contiguous bf16")
    _check_fanout(q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse, (nb, T, Hq), Hkv, D, P, S)
    f = FanoutPrefill(nb, T, Hq, Hkv, D, P, S, scale)
    need = lib.fanout_prefill_workspace_bytes(ctypes.byref(f))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = _empty((nb, T, Hq, D), torch.bfloat16, q.device, stream)
    if lse is None and want_lse:
        lse = _empty((nb, T, Hq), torch.float32, q.device, stream)
    _check(lib.fanout_prefix_prefill(ctypes.byref(f), _ptr(q), _ptr(prefix_k), _ptr(prefix_v), _ptr(suffix_k),
                                     _ptr(suffix_v), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                     _stream(stream)), "fanout_prefix_prefill")
    return out, lse


def fanout_prefill_workspace_bytes(nb, T, Hq, Hkv, D, P, S) -> int:
    return load().fanout_prefill_workspace_bytes(ctypes.byref(FanoutPrefill(nb, T, Hq, Hkv, D, P, S, 0.0)))


def bwd_delta(out: torch.Tensor, dout: torch.Tensor, delta: Optional[torch.Tensor] = None, stream=None):
    """blockattn_bwd_delta: delta[r] = sum_d dout[r, d] * out[r, d] over rows in state-row order.

    out: the forward's output ([rows, D] or [T, Hq, D], bf16 or fp32, rows contiguous);
    dout: bf16 of the same shape."""
    lib = load()
    D = out.shape[-1]
    o2 = out.reshape(-1, D)
    g2 = dout.reshape(-1, D)
    if o2.stride(1) != 1 or g2.stride(1) != 1 or dout.dtype != torch.bfloat16:
        raise ValueError("out and dout need a contiguous last axis; dout must be bf16")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be bf16 or fp32")
    rows = o2.shape[0]
    if g2.shape != o2.shape:
        raise ValueError(f"dout {tuple(g2.shape)} must match out {tuple(o2.shape)} row for row")
    if delta is None:
        delta = _empty(rows, torch.float32, out.device, stream)
    elif delta.dtype != torch.float32 or not delta.is_contiguous() or delta.numel() != rows:
        raise ValueError(f"delta must be contiguous fp32 with {rows} entries")
    code = BA_BF16 if out.dtype == torch.bfloat16 else BA_F32
    _check(lib.blockattn_bwd_delta(rows, D, _ptr(o2), code, o2.stride(0), _ptr(g2), g2.stride(0), _ptr(delta),
                                   _stream(stream)), "blockattn_bwd_delta")
    return delta


def bwd_block(q: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor, delta: torch.Tensor,
              blocks: Sequence[Tuple[torch.Tensor, torch.Tensor, int]], order: Optional[Sequence[int]],
              dq: torch.Tensor, dkv: Sequence[Tuple[torch.Tensor, torch.Tensor]], *, n_kv_heads: int,
              q_pos0: int = 0, causal: bool = False, scale: float = 0.0, stream=None):
    """blockattn_bwd_block: accumulate dq [rows, D] and each visited block's (dk, dv) [len, Hkv, D]
    ([batch, len, Hkv, D] for a batched q, one gradient per sequence), all fp32, over the visits
    of one forward call.  dout has q's shape and strides (bf16)."""
    lib = load()
    if dout.shape != q.shape or dout.stride() != q.stride() or dout.dtype != torch.bfloat16:
        raise ValueError("dout must be bf16 with q's shape and strides")
    p = make_problem(q, n_kv_heads, q_pos0, causal, scale, 0)
    B, T, Hq, D, batched = _qshape(q)
    _check_blocks(blocks, n_kv_heads, D, q.dtype, B)
    rows = B * T * Hq
    if dq.dtype != torch.float32 or not dq.is_contiguous() or dq.numel() != rows * D:
        raise ValueError("dq must be contiguous fp32 with batch * q_len * n_q_heads * head_dim elements")
    for name, t in (("lse", lse), ("delta", delta)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != rows:
            raise ValueError(f"{name} must be contiguous fp32 with one entry per (sequence, token, query head)")
    if len(dkv) != len(blocks):
        raise ValueError("one (dk, dv) pair per block")
    for (kb, _, _), (dk, dv) in zip(blocks, dkv):
        n = kb.shape[-3]
        want = (B, n, n_kv_heads, D) if batched else (n, n_kv_heads, D)
        if dk.dtype != torch.float32 or dv.dtype != torch.float32 or not dk.is_contiguous() or not dv.is_contiguous():
            raise ValueError("dk and dv must be contiguous fp32")
        if tuple(dk.shape) != want or tuple(dv.shape) != want:
            raise ValueError(f"dk and dv of a block of {n} keys must have shape {want}")
    arr = make_blocks(blocks)
    n_visit = len(order) if order is not None else len(blocks)
    order_arr = (ctypes.c_int32 * max(1, n_visit))(*(order or []))
    dks = (ctypes.c_void_p * max(1, len(blocks)))(*[t[0].data_ptr() for t in dkv])
    dvs = (ctypes.c_void_p * max(1, len(blocks)))(*[t[1].data_ptr() for t in dkv])
    _check(lib.blockattn_bwd_block(ctypes.byref(p), _ptr(q), _ptr(dout), _ptr(lse), _ptr(delta), arr, len(blocks),
                                   order_arr if order is not None else None, n_visit, _ptr(dq), dks, dvs,
                                   _stream(stream)), "blockattn_bwd_block")
    return dq, dkv


def _paged_args(q, k_pool, v_pool, prefix_pages, suffix_pages, prefix_len, suffix_len, rows_shape, out, lse):
    """Checks the pools and page tables of the paged fan-out and returns
    (n_kv_heads, head_dim, KVPages)."""
    if k_pool.dim() != 4 or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool must be [n_pool_pages, page_len, n_kv_heads, head_dim], same shape")
    n_pool, PL, Hkv, D = k_pool.shape
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be contiguous bf16")
    if q.shape[-1] != D:
        raise ValueError(f"q head_dim {q.shape[-1]} != pool head_dim {D}")
    nb = rows_shape[0]
    per_branch = -(-suffix_len // PL) if PL > 0 else 0
    for name, t, need in (("prefix_pages", prefix_pages, -(-prefix_len // PL) if PL > 0 else 0),
                          ("suffix_pages", suffix_pages, nb * per_branch)):
        if need == 0:
            continue
        if t is None or t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < need:
            raise ValueError(f"{name} must be contiguous int32 with at least {need} entries")
    if suffix_len > 0 and suffix_pages.dim() == 2 and tuple(suffix_pages.shape) != (nb, per_branch):
        raise ValueError(f"suffix_pages must be [{nb}, {per_branch}]")
    if out is not None and (tuple(out.shape) != tuple(rows_shape) + (D,) or out.dtype != torch.bfloat16
                            or not out.is_contiguous()):
        raise ValueError(f"out must be contiguous bf16 of shape {tuple(rows_shape) + (D,)}")
    if lse is not None and (tuple(lse.shape) != tuple(rows_shape) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError(f"lse must be contiguous fp32 of shape {tuple(rows_shape)}")
    pages = KVPages(prefix_pages.data_ptr() if prefix_pages is not None else None,
                    suffix_pages.data_ptr() if suffix_pages is not None else None, PL, n_pool)
    return Hkv, D, pages


def fanout_prefix_decode_paged(q, k_pool, v_pool, prefix_pages, suffix_pages, prefix_len: int, suffix_len: int,
                               scale: float = 0.0, workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """fanout_prefix_decode_paged: q [nb, Hq, D]; pools [n_pool, page_len, Hkv, D] bf16; prefix_pages int32
    [>= ceil(P / page_len)] and suffix_pages int32 [nb, ceil(S / page_len)] (device).  Returns (out, lse)."""
    lib = load()
    nb, Hq, D = q.shape
    Hkv, D, pages = _paged_args(q, k_pool, v_pool, prefix_pages, suffix_pages, prefix_len, suffix_len, (nb, Hq),
                                out, lse)
    f = Fanout(nb, Hq, Hkv, D, prefix_len, suffix_len, scale)
    need = lib.fanout_workspace_bytes(ctypes.byref(f))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = _empty((nb, Hq, D), torch.bfloat16, q.device, stream)
    if lse is None and want_lse:
        lse = _empty((nb, Hq), torch.float32, q.device, stream)
    _check(lib.fanout_prefix_decode_paged(ctypes.byref(f), ctypes.byref(pages), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                          _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)),
           "fanout_prefix_decode_paged")
    return out, lse


def fanout_prefix_prefill_paged(q, k_pool, v_pool, prefix_pages, suffix_pages, prefix_len: int, suffix_len: int,
                                scale: float = 0.0, workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """fanout_prefix_prefill_paged: q [nb, T, Hq, D] (each branch's T newest tokens, the last T of its suffix);
    pools and page tables as fanout_prefix_decode_paged.  Returns (out [nb, T, Hq, D], lse [nb, T, Hq])."""
    lib = load()
    nb, T, Hq, D = q.shape
    Hkv, D, pages = _paged_args(q, k_pool, v_pool, prefix_pages, suffix_pages, prefix_len, suffix_len,
                                (nb, T, Hq), out, lse)
    f = FanoutPrefill(nb, T, Hq, Hkv, D, prefix_len, suffix_len, scale)
    need = lib.fanout_prefill_workspace_bytes(ctypes.byref(f))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = _empty((nb, T, Hq, D), torch.bfloat16, q.device, stream)
    if lse is None and want_lse:
        lse = _empty((nb, T, Hq), torch.float32, q.device, stream)
    _check(lib.fanout_prefix_prefill_paged(ctypes.byref(f), ctypes.byref(pages), _ptr(q), _ptr(k_pool),
                                           _ptr(v_pool), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                           _stream(stream)), "fanout_prefix_prefill_paged")
    return out, lse
