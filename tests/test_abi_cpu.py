"""The C-ABI library loads, exports every declared entry point, shares
torch's HIP runtime, and rejects bad arguments on the host before any launch.

No GPU is needed: every call here fails validation before anything is
enqueued (pointers are never dereferenced on the host).
"""

import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch  # noqa: F401  (load torch's HIP runtime first)

from exact_blockwise_long_amd import blockattn as ba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockattn.h")

FAKE = 0x100000  # a 256-byte aligned non-null address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:blockattn|fanout)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ba.LIB_PATH):
        pytest.skip("libblockattn.so not built")
    return ba.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "blockattn_fwd_block" in names and "fanout_prefix_decode" in names
    assert set(names) == set(ba.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_single_hip_runtime(lib):
    loaded = ba.hip_runtimes_loaded()
    assert len(loaded) == 1, loaded


def test_version_and_status_strings(lib):
    assert lib.blockattn_abi_version() == 2
    for s in range(7):
        assert lib.blockattn_status_str(s)
    assert lib.blockattn_status_str(99) == b"unknown status"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_struct_layouts_match_the_header(tmp_path):
    """Every field of the public structs sits at the same offset in the
    header (compiled as C) and in the binding's ctypes declarations."""
    exe = str(tmp_path / "abi_layout")
    subprocess.run(["gcc", "-std=c11", "-Wall", f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "abi_layout.c"), "-o", exe], check=True)
    lines = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=60).stdout.split("\n")
    py = {"ba_problem": ba.Problem, "ba_kv_block": ba.KVBlock, "ba_state": ba.State, "ba_fanout": ba.Fanout,
          "ba_fanout_prefill": ba.FanoutPrefill, "ba_kv_pages": ba.KVPages}
    seen = {n: set() for n in py}
    for ln in filter(None, lines):
        struct, field, value = ln.split()
        cls = py[struct]
        if field == "sizeof":
            assert ctypes.sizeof(cls) == int(value), (struct, ctypes.sizeof(cls), value)
        else:
            assert getattr(cls, field).offset == int(value), (struct, field)
            seen[struct].add(field)
    for n, cls in py.items():
        assert seen[n] == {f for f, _ in cls._fields_}, n


def _problem(**kw):
    p = ba.Problem(8, 2, 128, 16, 0, 8 * 128, 128, ba.BA_BF16, 0.0, 0, 0)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _blocks(n, length=64):
    arr = (ba.KVBlock * n)()
    for i in range(n):
        arr[i] = ba.KVBlock(FAKE, FAKE, length, i * length, 2 * 128, 128, 2 * 128, 128)
    return arr


def _state():
    return ba.State(FAKE, FAKE, FAKE)


def _fwd(lib, p, blocks, n_blocks, order, n_visit, ws=None, ws_bytes=0, state=None, q=FAKE):
    o = None
    if order is not None:
        o = (ctypes.c_int32 * len(order))(*order)
    return lib.blockattn_fwd_block(ctypes.byref(p) if p is not None else None, q, blocks, n_blocks, o, n_visit,
                                   state or _state(), 1, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(head_dim=96), 2), (dict(n_q_heads=6, n_kv_heads=4), 2), (dict(n_kv_heads=0), 2),
    (dict(q_len=-1), 2), (dict(dtype=7), 3), (dict(q_stride_token=0), 2), (dict(split_mode=5), 2),
    (dict(q_stride_head=12), 2), (dict(batch=-1), 2), (dict(batch=2, q_stride_batch=0), 2),
    (dict(batch=2, q_stride_batch=12), 2), (dict(batch=1 << 24, q_stride_batch=16 * 8 * 128), 2),
])
def test_fwd_rejects_bad_problem(lib, kw, expect):
    assert _fwd(lib, _problem(**kw), _blocks(2), 2, [0, 1], 2) == expect
    assert lib.blockattn_last_error()


def test_fwd_null_arguments(lib):
    assert _fwd(lib, None, _blocks(1), 1, None, 1) == 1
    assert _fwd(lib, _problem(), _blocks(1), 1, None, 1, q=None) == 1
    assert _fwd(lib, _problem(), None, 1, None, 1) == 1
    assert _fwd(lib, _problem(split_mode=1), _blocks(1), 1, None, 1, state=ba.State(FAKE, None, FAKE)) == 1
    bad = _blocks(1)
    bad[0].k = None
    assert _fwd(lib, _problem(), bad, 1, None, 1) == 1


@pytest.mark.parametrize("order,n_blocks", [([0, 0], 2), ([0, 2], 2), ([-1], 2), (list(range(33)), 40)])
def test_fwd_rejects_bad_order(lib, order, n_blocks):
    assert _fwd(lib, _problem(), _blocks(n_blocks), n_blocks, order, len(order)) == 4


def test_fwd_rejects_bad_batch_strides(lib):
    p = _problem(batch=3, q_stride_batch=16 * 8 * 128)
    for field, value in (("k_stride_batch", -8), ("v_stride_batch", -8), ("k_stride_batch", 12)):
        b = _blocks(2)
        setattr(b[1], field, value)
        assert _fwd(lib, p, b, 2, None, 2) == 2, field
    # batch strides are not read without a batch, and 0 (shared keys) is valid with one
    b = _blocks(2)
    b[0].k_stride_batch = -8
    assert lib.blockattn_fwd_workspace_bytes(ctypes.byref(_problem(split_mode=2)), b, 2, None, 2) > 0
    assert lib.blockattn_fwd_workspace_bytes(ctypes.byref(_problem(split_mode=2, batch=3,
                                                                   q_stride_batch=16 * 8 * 128)),
                                             _blocks(2), 2, None, 2) > 0


def test_batch_scales_the_workspace(lib):
    """Split partial states cover every sequence's rows."""
    one = lib.blockattn_fwd_workspace_bytes(ctypes.byref(_problem(split_mode=2)), _blocks(3), 3, None, 3)
    three = lib.blockattn_fwd_workspace_bytes(
        ctypes.byref(_problem(split_mode=2, batch=3, q_stride_batch=16 * 8 * 128)), _blocks(3), 3, None, 3)
    assert one > 0 and three > one


def test_fwd_rejects_misaligned(lib):
    bad = _blocks(1)
    bad[0].k = FAKE + 2
    assert _fwd(lib, _problem(), bad, 1, None, 1) == 2
    assert _fwd(lib, _problem(), _blocks(1), 1, None, 1, q=FAKE + 4) == 2
    assert _fwd(lib, _problem(split_mode=1), _blocks(1), 1, None, 1, state=ba.State(FAKE, FAKE, FAKE + 4)) == 2


def test_split_needs_workspace(lib):
    p = _problem(split_mode=2)
    need = lib.blockattn_fwd_workspace_bytes(ctypes.byref(p), _blocks(3), 3, None, 3)
    assert need > 0
    assert _fwd(lib, p, _blocks(3), 3, None, 3) == 5
    assert _fwd(lib, p, _blocks(3), 3, None, 3, ws=FAKE, ws_bytes=need - 1) == 5
    # walk mode needs none
    assert lib.blockattn_fwd_workspace_bytes(ctypes.byref(_problem(split_mode=1)), _blocks(3), 3, None, 3) == 0
    # the f32 path splits a query block too small to fill the GPU as well, unless told not to
    f32 = _problem(dtype=ba.BA_F32, split_mode=0, q_stride_token=8 * 128)
    need32 = lib.blockattn_fwd_workspace_bytes(ctypes.byref(f32), _blocks(3), 3, None, 3)
    assert need32 > 0
    assert _fwd(lib, f32, _blocks(3), 3, None, 3) == 5
    assert lib.blockattn_fwd_workspace_bytes(ctypes.byref(_problem(dtype=ba.BA_F32, split_mode=1)),
                                             _blocks(3), 3, None, 3) == 0


def test_shard_states_validation(lib):
    p = _problem()
    sts = (ba.State * 2)(_state(), _state())
    assert lib.blockattn_shard_states(ctypes.byref(p), FAKE, _blocks(2), 0, sts, None, 0, None) == 4
    assert lib.blockattn_shard_states(ctypes.byref(p), FAKE, _blocks(2), 2, sts, None, 0, None) == 5
    assert lib.blockattn_shard_workspace_bytes(ctypes.byref(p), _blocks(2), 2) > 0
    # fp32 problems take the fp32 split kernel: the same workspace rule
    f32 = _problem(dtype=ba.BA_F32)
    assert lib.blockattn_shard_states(ctypes.byref(f32), FAKE, _blocks(2), 2, sts, None, 0, None) == 5
    assert lib.blockattn_shard_workspace_bytes(ctypes.byref(f32), _blocks(2), 2) > 0


def test_merge_validation(lib):
    parts = (ba.State * 2)(_state(), _state())
    assert lib.blockattn_merge_states(0, parts, 10, 128, _state(), None) == 2
    assert lib.blockattn_merge_states(65, parts, 10, 128, _state(), None) == 2
    assert lib.blockattn_merge_states(2, None, 10, 128, _state(), None) == 1
    assert lib.blockattn_merge_states(2, parts, 10, 100, _state(), None) == 2
    assert lib.blockattn_merge_states(2, parts, 10, 128, ba.State(None, FAKE, FAKE), None) == 1
    # zero rows is a valid no-op that launches nothing
    assert lib.blockattn_merge_states(2, parts, 0, 128, _state(), None) == 0


def test_finalize_validation(lib):
    assert lib.blockattn_finalize(_state(), 4, 128, None, ba.BA_BF16, 128, None, None) == 1
    assert lib.blockattn_finalize(_state(), 4, 128, FAKE, ba.BA_BF16, 64, None, None) == 2
    assert lib.blockattn_finalize(_state(), 4, 128, FAKE, 9, 128, None, None) == 3
    assert lib.blockattn_finalize(_state(), 0, 128, FAKE, ba.BA_BF16, 128, None, None) == 0


def test_fwd_block_finalize_validation(lib):
    """The fused forward-and-finalise call checks the problem, the state and
    the output before any launch; every call here fails one of those checks."""
    def call(p=None, out=FAKE, dtype=ba.BA_BF16, stride=128, state=None, ws=None, ws_bytes=0):
        p = p if p is not None else _problem()
        order = (ctypes.c_int32 * 2)(1, 0)
        return lib.blockattn_fwd_block_finalize(ctypes.byref(p), FAKE, _blocks(2), 2, order, 2, state or _state(), 1,
                                                out, dtype, stride, None, ws, ws_bytes, None)
    assert call(p=_problem(head_dim=96)) == 2
    assert call(p=_problem(n_kv_heads=3)) == 2
    assert call(state=ba.State(FAKE, None, FAKE)) == 1
    assert call(out=None) == 1
    assert call(dtype=9) == 3
    assert call(stride=64) == 2
    assert call(stride=130) == 2
    assert call(out=FAKE + 4) == 2                        # bf16 rows need 8-byte alignment
    assert call(out=FAKE + 8, dtype=ba.BA_F32) == 2       # fp32 rows need 16
    # 16 query tokens split over keys: the workspace is checked before any launch
    assert call() == 5
    assert call(ws=FAKE, ws_bytes=16) == 5
    assert call(p=_problem(q_len=0)) == 0                 # nothing to do: no launch


def test_fanout_validation(lib):
    def call(f, ws=None, ws_bytes=0, **ptrs):
        a = dict(q=FAKE, pk=FAKE, pv=FAKE, sk=FAKE, sv=FAKE, out=FAKE)
        a.update(ptrs)
        return lib.fanout_prefix_decode(ctypes.byref(f), a["q"], a["pk"], a["pv"], a["sk"], a["sv"], a["out"],
                                        None, ws, ws_bytes, None)
    assert call(ba.Fanout(4, 8, 3, 128, 100, 10, 0.0)) == 2
    assert call(ba.Fanout(4, 8, 2, 128, 0, 0, 0.0)) == 2
    assert call(ba.Fanout(4, 8, 2, 128, 100, 10, 0.0), q=None) == 1
    assert call(ba.Fanout(4, 8, 2, 128, 100, 10, 0.0), pk=None) == 1
    f = ba.Fanout(4, 8, 2, 128, 100, 10, 0.0)
    need = lib.fanout_workspace_bytes(ctypes.byref(f))
    assert need > 0
    assert call(f) == 5
    assert call(f, ws=FAKE, ws_bytes=need - 16) == 5
    assert call(ba.Fanout(0, 8, 2, 128, 100, 10, 0.0)) == 0   # no branches: no-op


def test_fanout_noalloc_rejects_more_than_its_scratch(lib):
    # decode shapes whose partial states exceed the static scratch: rejected on
    # the host before the scratch is looked up or anything is enqueued
    f = ba.Fanout(2048, 64, 8, 128, 65536, 512, 0.0)
    assert lib.fanout_workspace_bytes(ctypes.byref(f)) > ba.STATIC_SCRATCH_BYTES
    assert lib.fanout_prefix_decode_noalloc(ctypes.byref(f), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 5
    assert b"static scratch" in lib.blockattn_last_error()
    # the full-size 64K decode (16 branches) fits
    f = ba.Fanout(16, 64, 8, 128, 65536, 512, 0.0)
    assert 0 < lib.fanout_workspace_bytes(ctypes.byref(f)) <= ba.STATIC_SCRATCH_BYTES
    # shape errors come first, as for fanout_prefix_decode
    assert lib.fanout_prefix_decode_noalloc(ctypes.byref(ba.Fanout(4, 8, 3, 128, 100, 10, 0.0)), FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, None, None) == 2


def test_fanout_prefill_validation(lib):
    def call(f, ws=None, ws_bytes=0, **ptrs):
        a = dict(q=FAKE, pk=FAKE, pv=FAKE, sk=FAKE, sv=FAKE, out=FAKE)
        a.update(ptrs)
        return lib.fanout_prefix_prefill(ctypes.byref(f), a["q"], a["pk"], a["pv"], a["sk"], a["sv"], a["out"],
                                         None, ws, ws_bytes, None)
    P = ba.FanoutPrefill
    assert call(P(4, 20, 8, 3, 128, 100, 64, 0.0)) == 2          # heads
    assert call(P(4, 0, 8, 2, 128, 100, 64, 0.0)) == 2           # n_new < 1
    assert call(P(4, 65, 8, 2, 128, 100, 64, 0.0)) == 2          # n_new > suffix_len
    assert call(P(4, 20, 8, 2, 96, 100, 64, 0.0)) == 2           # head_dim
    assert call(P(4, 20, 8, 2, 128, 100, 64, 0.0), q=None) == 1
    assert call(P(4, 20, 8, 2, 128, 100, 64, 0.0), sv=None) == 1
    assert lib.fanout_prefix_prefill(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    f = P(8, 20, 64, 8, 128, 65536, 512, 0.0)
    need = lib.fanout_prefill_workspace_bytes(ctypes.byref(f))
    assert need > 0 and need % 256 == 0
    assert call(f) == 5
    assert call(f, ws=FAKE, ws_bytes=need - 16) == 5
    assert call(P(0, 20, 8, 2, 128, 100, 64, 0.0)) == 0           # no branches: no-op
    # one new token per branch needs exactly the decode's workspace
    dec = lib.fanout_workspace_bytes(ctypes.byref(ba.Fanout(16, 64, 8, 128, 65536, 512, 0.0)))
    pre = lib.fanout_prefill_workspace_bytes(ctypes.byref(P(16, 1, 64, 8, 128, 65536, 512, 0.0)))
    assert dec == pre


def test_workspace_sizes_are_deterministic(lib):
    f = ba.Fanout(16, 64, 8, 128, 65536, 512, 0.0)
    a = lib.fanout_workspace_bytes(ctypes.byref(f))
    b = lib.fanout_workspace_bytes(ctypes.byref(f))
    assert a == b and a % 256 == 0


def _bwd(lib, p=None, q=FAKE, dout=FAKE, lse=FAKE, delta=FAKE, blocks=None, n_blocks=2, order=None, n_visit=2,
         dq=FAKE, dk=(FAKE, FAKE), dv=(FAKE, FAKE), dk_arr=True):
    p = _problem() if p is None else p
    blocks = _blocks(n_blocks) if blocks is None else blocks
    o = None if order is None else (ctypes.c_int32 * len(order))(*order)
    dka = (ctypes.c_void_p * len(dk))(*dk) if dk_arr else None
    dva = (ctypes.c_void_p * len(dv))(*dv)
    return lib.blockattn_bwd_block(ctypes.byref(p), q, dout, lse, delta, blocks, n_blocks, o, n_visit, dq, dka, dva,
                                   None)


def test_bwd_block_validation(lib):
    assert lib.blockattn_bwd_block(None, FAKE, FAKE, FAKE, FAKE, _blocks(1), 1, None, 1, FAKE, None, None, None) == 1
    assert _bwd(lib, p=_problem(dtype=ba.BA_F32)) == 3           # bf16 only
    assert _bwd(lib, p=_problem(head_dim=96)) == 2
    assert _bwd(lib, order=[0, 0]) == 4
    assert _bwd(lib, dout=None) == 1
    assert _bwd(lib, lse=None) == 1
    assert _bwd(lib, delta=None) == 1
    assert _bwd(lib, dq=None) == 1
    assert _bwd(lib, dout=FAKE + 2) == 2
    assert _bwd(lib, dq=FAKE + 4) == 2
    assert _bwd(lib, dk_arr=False) == 1
    assert _bwd(lib, dk=(FAKE, None)) == 1
    assert _bwd(lib, dv=(FAKE + 4, FAKE)) == 2
    assert _bwd(lib, p=_problem(q_stride_token=1 << 28)) == 2   # beyond 32-bit offsets
    # nothing to do: no rows, no visits, or every visited key in the causal future
    assert _bwd(lib, p=_problem(q_len=0)) == 0
    assert _bwd(lib, order=[], n_visit=0) == 0
    future = _blocks(2)
    for i in range(2):
        future[i].pos0 = 1000 + 64 * i
    assert _bwd(lib, p=_problem(causal=1), blocks=future, dk=(None, None), dv=(None, None)) == 0


def test_bwd_delta_validation(lib):
    def call(rows=16, D=128, out=FAKE, dtype=ba.BA_BF16, os_=128, dout=FAKE, gs=128, delta=FAKE):
        return lib.blockattn_bwd_delta(rows, D, out, dtype, os_, dout, gs, delta, None)
    assert call(D=96) == 2
    assert call(rows=-1) == 2
    assert call(dtype=7) == 3
    assert call(rows=0) == 0
    assert call(out=None) == 1
    assert call(delta=None) == 1
    assert call(os_=64) == 2
    assert call(gs=132) == 2
    assert call(dout=FAKE + 8) == 2


def test_bf16_blocks_beyond_32bit_offsets_are_rejected(lib):
    """One KV head of a bf16 block must span less than 4 GiB (the kernels'
    buffer offsets are 32-bit): 2^21 + 1 keys at 1024 elements per key span
    4 GiB + 256 B and are rejected.  (Only rejected calls here: nothing may
    reach a kernel launch with the fake pointers.)"""
    big = _blocks(1, length=(1 << 21) + 1)
    big[0].k_stride_token = big[0].v_stride_token = 1024
    assert _fwd(lib, _problem(), big, 1, None, 1) == 2
    assert b"4 GiB" in lib.blockattn_last_error()
    assert _bwd(lib, blocks=big, n_blocks=1, order=None, n_visit=1, dk=(FAKE,), dv=(FAKE,)) == 2
    f = ba.Fanout(4, 64, 8, 128, (1 << 21) + 1, 16, 0.0)
    assert lib.fanout_prefix_decode(ctypes.byref(f), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 2


def test_fanout_paged_validation(lib):
    f = ba.Fanout(4, 64, 8, 128, 1000, 100, 0.0)
    fp = ba.FanoutPrefill(4, 20, 64, 8, 128, 1000, 100, 0.0)

    def call(pages=True, prefix_pages=FAKE, suffix_pages=FAKE, page_len=256, n_pool=64, k=FAKE, v=FAKE,
             prefill=False, desc=None):
        pg = ba.KVPages(prefix_pages, suffix_pages, page_len, n_pool)
        pp = ctypes.byref(pg) if pages else None
        if prefill:
            return lib.fanout_prefix_prefill_paged(ctypes.byref(desc or fp), pp, FAKE, k, v, FAKE, None, None, 0,
                                                   None)
        return lib.fanout_prefix_decode_paged(ctypes.byref(desc or f), pp, FAKE, k, v, FAKE, None, None, 0, None)

    for prefill in (False, True):
        assert call(pages=False, prefill=prefill) == 1
        assert call(page_len=100, prefill=prefill) == 2
        assert call(page_len=0, prefill=prefill) == 2
        assert call(n_pool=0, prefill=prefill) == 2
        assert call(prefix_pages=None, prefill=prefill) == 1
        assert call(suffix_pages=None, prefill=prefill) == 1
        assert call(k=None, prefill=prefill) == 1
        assert call(v=FAKE + 8, prefill=prefill) == 2
        assert call(prefill=prefill) == 5                   # valid; no workspace given
    # a prefix of 4M tokens is fine when paged (each page is its own 32-bit range)
    assert call(desc=ba.Fanout(4, 64, 8, 128, 1 << 22, 100, 0.0)) == 5
    assert call(desc=ba.Fanout(4, 64, 8, 128, 1000, 0, 0.0), suffix_pages=None) == 5


def test_workspace_bound_covers_every_call(lib):
    """blockattn_workspace_bytes(p, NULL) bounds blockattn_fwd_workspace_bytes
    over random block sets and visit orders of the problem; (NULL, f) is the
    fan-out decode's requirement.  Host-side sizing only."""
    import numpy as np
    g = np.random.Generator(np.random.PCG64(5))
    for trial in range(200):
        Hkv = int(g.choice([1, 2, 8]))
        Hq = Hkv * int(g.choice([1, 4, 8]))
        T = int(g.choice([1, 7, 64, 300, 2000]))
        mode = int(g.choice([0, 2]))
        p = _problem(n_q_heads=Hq, n_kv_heads=Hkv, q_len=T, q_stride_token=Hq * 128, split_mode=mode,
                     causal=int(g.integers(0, 2)), q_pos0=int(g.integers(0, 5000)))
        n = int(g.integers(1, 33))
        blocks = (ba.KVBlock * n)()
        pos = 0
        for i in range(n):
            ln = int(g.integers(0, 40000))
            blocks[i] = ba.KVBlock(FAKE, FAKE, ln, pos, Hkv * 128, 128, Hkv * 128, 128)
            pos += ln
        bound = lib.blockattn_workspace_bytes(ctypes.byref(p), None)
        order = (ctypes.c_int32 * n)(*g.permutation(n).tolist())
        exact = lib.blockattn_fwd_workspace_bytes(ctypes.byref(p), blocks, n, order, n)
        assert exact <= bound, (trial, exact, bound)
    f = ba.Fanout(16, 64, 8, 128, 65536, 512, 0.0)
    assert lib.blockattn_workspace_bytes(None, ctypes.byref(f)) == lib.fanout_workspace_bytes(ctypes.byref(f))
    assert lib.blockattn_workspace_bytes(None, None) == 0
