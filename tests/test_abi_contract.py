"""C-ABI contract tests that need no GPU.

The library must load, export every entry point include/*.h declares, and
decline every host-knowable problem before any HIP call, with a status code and
a reason (pull request 3705, section Execution and supported scope: alignment,
capacity and overlap are validated before launch; pull request 3527, Notes for
reviewers / Scope: explicit declines with reasons, never a silent fallback).
All pointers below are fake, aligned addresses: validation never dereferences
them, and every call here returns before a kernel would be launched.
"""

import ctypes
import os
import re

import pytest

from scaled_dot_product_02_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, ALIGN, OVERLAP, WORKSPACE = 0, 1, 2, 3, 4, 5
GiB = 1 << 30


@pytest.fixture(scope="module")
def L(lib_path):
    return B.lib()


def declared_functions():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert set(decl) == set(B.EXPORTED)
    for name in decl:
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.attn_abi_version() == 4
    for code, name in B.STATUS.items():
        assert L.attn_status_str(code).decode() == name
    assert L.attn_status_str(42).decode() == "ATTN_E_UNKNOWN"


def dense_problem(b=2, sq=256, skv=256, hq=4, hkv=2, d=128, dtype=0, mask=1):
    p = B.AttnProblem()
    p.abi_version = 4
    p.window_left = -1  # no sliding window (ctypes zero-fills, and 0 is a window)
    p.dtype, p.mask, p.scale = dtype, mask, d ** -0.5
    p.batch, p.heads_q, p.heads_kv, p.head_dim = b, hq, hkv, d
    p.max_seqlen_q, p.max_seqlen_kv = sq, skv
    p.q_stride[:] = (sq * hq * d, hq * d, d)
    p.o_stride[:] = (sq * hq * d, hq * d, d)
    p.k_stride[:] = (skv * hkv * d, hkv * d, d)
    p.v_stride[:] = (skv * hkv * d, hkv * d, d)
    return p


def packed_problem(tq=1000, tkv=1000, nseq=4, hq=4, hkv=4, d=64):
    p = dense_problem(b=nseq, sq=600, skv=600, hq=hq, hkv=hkv, d=d)
    p.cu_seqlens_q, p.cu_seqlens_kv = 0x7000_0000, 0x7000_1000
    p.total_q, p.total_kv = tq, tkv
    p.q_stride[:] = (hq * d, d, 0)
    p.o_stride[:] = (hq * d, d, 0)
    p.k_stride[:] = (hkv * d, d, 0)
    p.v_stride[:] = (hkv * d, d, 0)
    return p


# fake, disjoint, 256-byte aligned device addresses, 1 GiB apart
Q, K, V, O, LSE, WS, DO, DQ, DK, DV = (0x1_0000_0000 + i * GiB for i in range(10))


def fwd(L, p, q=Q, k=K, v=V, o=O, lse=LSE, ws=WS, ws_bytes=1 << 20):
    return L.attn_fwd(ctypes.byref(p) if p is not None else None, q, k, v, o, lse, ws, ws_bytes, None)


def bwd(L, p, q=Q, k=K, v=V, o=O, do=DO, lse=LSE, dq=DQ, dk=DK, dv=DV, ws=WS, ws_bytes=1 << 30):
    return L.attn_bwd(ctypes.byref(p), q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, None)


def expect(L, status, want, fragment):
    assert status == want, (B.STATUS.get(status), L.attn_last_error())
    assert fragment in L.attn_last_error().decode()


def test_null_problem(L):
    expect(L, fwd(L, None), INVALID, "NULL")


@pytest.mark.parametrize("field,value,want,frag", [
    ("abi_version", 2, UNSUPPORTED, "abi_version"),
    ("abi_version", 3, UNSUPPORTED, "abi_version"),
    ("abi_version", 5, UNSUPPORTED, "abi_version"),
    ("flags", 8, INVALID, "unknown flags"),
    ("window_left", -2, INVALID, "window_left"),
    ("head_dim_v", -8, INVALID, "head_dim_v"),
    ("head_dim_v", 100, UNSUPPORTED, "head_dim_v 100"),
    ("head_dim_v", 520, UNSUPPORTED, "head_dim_v 520"),
    ("dtype", 7, UNSUPPORTED, "dtype"),
    ("mask", 3, UNSUPPORTED, "mask"),
    ("mask", -1, UNSUPPORTED, "mask"),
    ("head_dim", 100, UNSUPPORTED, "head_dim 100"),
    ("head_dim", 4, UNSUPPORTED, "head_dim 4"),
    ("head_dim", 520, UNSUPPORTED, "head_dim 520"),
    ("head_dim", 0, INVALID, "head_dim"),
    ("heads_q", 3, INVALID, "multiple"),
    ("heads_kv", 0, INVALID, "head counts"),
    ("batch", -1, INVALID, "batch"),
    ("batch", 1 << 30, UNSUPPORTED, "launch grid"),
    ("scale", float("inf"), INVALID, "scale"),
    ("scale", float("nan"), INVALID, "scale"),
    ("scale", 0.0, UNSUPPORTED, "not positive"),
    ("scale", -0.125, UNSUPPORTED, "not positive"),
    ("max_seqlen_q", -5, INVALID, "max_seqlen"),
])
def test_declines_bad_fields(L, field, value, want, frag):
    p = dense_problem()
    setattr(p, field, value)
    expect(L, fwd(L, p), want, frag)
    expect(L, bwd(L, p), want, frag)


def test_declines_half_packed(L):
    p = dense_problem()
    p.cu_seqlens_q = 0x7000_0000
    expect(L, fwd(L, p), INVALID, "both")


@pytest.mark.parametrize("which", ["q_stride", "k_stride", "v_stride", "o_stride"])
def test_stride_alignment(L, which):
    p = dense_problem()
    getattr(p, which)[1] = 132  # not a multiple of 8 elements
    expect(L, fwd(L, p), ALIGN, which)
    p = dense_problem()
    getattr(p, which)[0] = -8
    expect(L, fwd(L, p), INVALID, "negative")


@pytest.mark.parametrize("which", ["q_stride", "k_stride", "v_stride", "o_stride"])
def test_row_stride_limit(L, which):
    p = dense_problem()
    getattr(p, which)[1] = 1 << 24
    expect(L, fwd(L, p), UNSUPPORTED, "row stride")
    getattr(p, which)[1] = (1 << 24) - 8
    p2 = dense_problem(b=0)  # same strides, nothing to launch: accepted
    getattr(p2, which)[1] = (1 << 24) - 8
    assert fwd(L, p2) == OK


@pytest.mark.parametrize("arg", ["q", "k", "v", "o"])
def test_pointer_alignment_and_null(L, arg):
    p = dense_problem()
    kw = {arg: {"q": Q, "k": K, "v": V, "o": O}[arg] + 8}
    expect(L, fwd(L, p, **kw), ALIGN, arg)
    expect(L, fwd(L, p, **{arg: None}), INVALID, f"{arg} is NULL")


def test_lse_alignment_and_null(L):
    p = dense_problem()
    expect(L, fwd(L, p, lse=LSE + 2), ALIGN, "lse")
    expect(L, fwd(L, p, lse=None), INVALID, "lse")


def test_output_overlap(L):
    p = dense_problem()
    expect(L, fwd(L, p, o=Q + 4096), OVERLAP, "o overlaps")
    expect(L, fwd(L, p, lse=O + 64), OVERLAP, "o overlaps lse")
    expect(L, fwd(L, p, lse=K + 64), OVERLAP, "lse overlaps")
    expect(L, bwd(L, p, dk=DQ + 1024), OVERLAP, "dq overlaps dk")
    expect(L, bwd(L, p, dv=DO), OVERLAP, "dv overlaps")
    expect(L, bwd(L, p, ws=DK), OVERLAP, "overlaps")


def test_workspace_sizes(L):
    p = dense_problem(b=2, sq=256, hq=4)
    assert L.attn_fwd_workspace_bytes(ctypes.byref(p)) == 0
    nq = 2 * 256
    assert L.attn_bwd_workspace_bytes(ctypes.byref(p)) == 256 + 2 * ((nq * 4 * 4 + 255) // 256 * 256)
    pk = packed_problem(tq=1000, hq=4)
    assert L.attn_fwd_workspace_bytes(ctypes.byref(pk)) == 256
    assert L.attn_bwd_workspace_bytes(ctypes.byref(pk)) == 256 + 2 * ((1000 * 4 * 4 + 255) // 256 * 256)
    bad = dense_problem(d=96)
    assert L.attn_fwd_workspace_bytes(ctypes.byref(bad)) == 0


def test_workspace_capacity_and_alignment(L):
    pk = packed_problem()
    expect(L, fwd(L, pk, ws_bytes=128), WORKSPACE, "workspace")
    expect(L, fwd(L, pk, ws=WS + 64), WORKSPACE, "aligned")
    p = dense_problem()
    need = L.attn_bwd_workspace_bytes(ctypes.byref(p))
    expect(L, bwd(L, p, ws_bytes=need - 1), WORKSPACE, "required")
    expect(L, bwd(L, p, ws=None), WORKSPACE, "NULL")


def test_cu_seqlens_alignment(L):
    pk = packed_problem()
    pk.cu_seqlens_q = 0x7000_0002
    expect(L, fwd(L, pk), ALIGN, "cu_seqlens")


def test_empty_batch_is_a_no_op(L):
    p = dense_problem(b=0)
    assert fwd(L, p) == OK
    assert bwd(L, p) == OK
    p = dense_problem(sq=0, skv=0)
    assert fwd(L, p) == OK


def test_last_error_is_thread_local(L):
    import threading
    p = dense_problem(d=100)
    fwd(L, p)
    mine = L.attn_last_error().decode()
    other = {}

    def run():
        q = dense_problem()
        q.mask = 9
        fwd(L, q)
        other["msg"] = L.attn_last_error().decode()

    t = threading.Thread(target=run)
    t.start()
    t.join()
    assert "head_dim" in mine and "mask" in other["msg"]
    assert L.attn_last_error().decode() == mine


def test_binding_rejects_host_tensors(lib_path):
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        B.attn_fwd(q, q, q)


def test_problem_struct_layout():
    # attn_problem_t: 10 x int32, 2 pointers, 2 x int64, 4 x int64[3], window_left, head_dim_v, flags (int32),
    # padded to the 8-byte alignment of its int64 members
    assert ctypes.sizeof(B.AttnProblem) == 40 + 16 + 16 + 4 * 24 + 12 + 4
    assert B.AttnProblem.cu_seqlens_q.offset == 40
    assert B.AttnProblem.q_stride.offset == 72
    assert B.AttnProblem.window_left.offset == 168
    assert B.AttnProblem.head_dim_v.offset == 172
    assert B.AttnProblem.flags.offset == 176


def test_window_needs_a_causal_mask(L):
    p = dense_problem(mask=0)
    p.window_left = 16
    expect(L, fwd(L, p), UNSUPPORTED, "causal mask")
    expect(L, bwd(L, p), UNSUPPORTED, "causal mask")
    for mask in (1, 2):
        p = dense_problem(b=0, mask=mask)
        p.window_left = 0
        assert fwd(L, p) == OK


# ---- attn_merge (validation only: every call below returns before a launch)
def merge(L, p, n=2, o_parts=None, lse_parts=None, o=O, lse=LSE):
    o_parts = o_parts if o_parts is not None else [Q, K][:n] + [V] * max(0, n - 2)
    lse_parts = lse_parts if lse_parts is not None else [DO + i * (1 << 24) for i in range(n)]
    oa = (ctypes.c_void_p * max(1, n))(*o_parts[:n]) if n > 0 else None
    la = (ctypes.c_void_p * max(1, n))(*lse_parts[:n]) if n > 0 else None
    return L.attn_merge(ctypes.byref(p) if p is not None else None, n, oa, la, o, lse, None)


def test_merge_declines(L):
    p = dense_problem()
    expect(L, merge(L, None), INVALID, "NULL")
    expect(L, merge(L, p, n=0), INVALID, "n_parts")
    expect(L, merge(L, p, n=9), INVALID, "n_parts")
    bad = dense_problem(d=96)
    bad.head_dim_v = 100
    expect(L, merge(L, bad), UNSUPPORTED, "head_dim_v")
    bad = dense_problem()
    bad.dtype = 5
    expect(L, merge(L, bad), UNSUPPORTED, "dtype")
    al = dense_problem()
    al.o_stride[1] = 132
    expect(L, merge(L, al), ALIGN, "o_stride")
    expect(L, merge(L, p, o=O + 8), ALIGN, "o")
    expect(L, merge(L, p, lse=LSE + 2), ALIGN, "lse")
    expect(L, merge(L, p, o_parts=[Q + 8, K]), ALIGN, "o_parts")
    big = dense_problem(b=1 << 24, sq=1 << 10)  # 2^34 rows x 4 heads: past the 32-bit grid
    expect(L, merge(L, big), UNSUPPORTED, "launch grid")


def test_declines_extents_past_2_62_bytes(L):
    # a batch stride no allocation can have: the extent is computed without overflow and refused
    p = dense_problem()
    p.q_stride[0] = 1 << 62
    expect(L, fwd(L, p), UNSUPPORTED, "q spans more than 2^62 bytes")
    expect(L, bwd(L, p), UNSUPPORTED, "q spans more than 2^62 bytes")


def test_declines_packed_totals_beyond_batch_times_max(L):
    p = packed_problem(tq=1000, nseq=4)
    p.max_seqlen_q = 200  # 4 sequences of at most 200 tokens cannot hold 1000
    expect(L, fwd(L, p), INVALID, "exceed batch x max_seqlen")
    expect(L, bwd(L, p), INVALID, "exceed batch x max_seqlen")


def test_declines_grids_past_32_bits_without_overflowing(L):
    # batch x heads x tiles far beyond 2^63 must still be declined cleanly (no 64-bit overflow)
    p = dense_problem(b=(1 << 31) - 1, sq=(1 << 31) - 1, skv=(1 << 31) - 1, hq=1 << 30, hkv=1 << 30)
    expect(L, fwd(L, p), UNSUPPORTED, "launch grid")
    expect(L, bwd(L, p), UNSUPPORTED, "launch grid")


def test_merge_overlap_rules(L):
    p = dense_problem()
    expect(L, merge(L, p, o=Q + 4096), OVERLAP, "partially overlaps o_parts")
    expect(L, merge(L, p, lse=DO + 64), OVERLAP, "partially overlaps lse_parts")
    expect(L, merge(L, p, o=DO), OVERLAP, "o overlaps lse_parts")
    expect(L, merge(L, p, lse=Q + 64), OVERLAP, "lse overlaps o_parts")
    expect(L, merge(L, p, lse=O + 64), OVERLAP, "o overlaps lse")


def test_merge_empty_is_a_no_op(L):
    assert merge(L, dense_problem(b=0)) == OK
    assert merge(L, dense_problem(sq=0, skv=0)) == OK
    # exact aliasing of an output with a part is accepted (nothing to launch here)
    assert merge(L, dense_problem(b=0), o=Q, lse=DO) == OK


def test_head_dims_that_are_multiples_of_8_are_accepted(L):
    # validation only: the empty batch returns OK after every check and before any launch
    for d, dv in [(8, 0), (96, 0), (192, 128), (264, 0), (504, 512), (512, 8), (40, 328)]:
        p = dense_problem(b=0, d=d)
        p.head_dim_v = dv
        assert fwd(L, p) == OK, (d, dv, L.attn_last_error())
        assert bwd(L, p) == OK, (d, dv, L.attn_last_error())


def test_extents_use_each_tensors_head_dim(L):
    # O of a (64, 512) problem is 8x wider than Q: an O that would overlap K only at its wide width is refused,
    # and the same placement with a symmetric problem passes
    p = dense_problem(b=1, sq=256, skv=256, hq=4, hkv=2, d=64)
    p.head_dim_v = 512
    p.o_stride[:] = (256 * 4 * 512, 4 * 512, 512)
    p.v_stride[:] = (256 * 2 * 512, 2 * 512, 512)
    q_bytes = 256 * 4 * 64 * 2
    o_bytes_wide = 256 * 4 * 512 * 2
    k_addr = O + q_bytes + 4096          # past a D=64 O, inside a D=512 O
    assert k_addr < O + o_bytes_wide
    expect(L, fwd(L, p, k=k_addr), OVERLAP, "o overlaps an input")


def test_mfma_probe_declines(L):
    """The matrix-core probe validates its arguments before launching (no GPU needed for these)."""
    out, ticks = 1 << 20, 1 << 24  # fake aligned device addresses, never dereferenced
    nout, nticks = 4 * 256 * 4, 4 * 16

    def call(blocks=4, iters=10, x=0.5, y=0.0, o=out, ob=nout, t=ticks, tb=nticks):
        return L.attn_mfma_probe(blocks, iters, x, y, o, ob, t, tb, None)

    cases = [
        (dict(blocks=0), INVALID, "blocks"), (dict(blocks=65537), INVALID, "blocks"),
        (dict(iters=0), INVALID, "iters"), (dict(iters=(1 << 24) + 1), INVALID, "iters"),
        (dict(x=float("nan")), INVALID, "finite"), (dict(y=float("inf")), INVALID, "finite"),
        (dict(o=None), INVALID, "NULL"), (dict(t=None), INVALID, "NULL"),
        (dict(o=out + 2), ALIGN, "out"), (dict(t=ticks + 4), ALIGN, "ticks"),
        (dict(ob=nout - 4), WORKSPACE, "out holds"), (dict(tb=nticks - 8), WORKSPACE, "ticks holds"),
        (dict(t=out + 64), OVERLAP, "overlaps"),
    ]
    for kw, want, frag in cases:
        assert call(**kw) == want, kw
        assert frag in L.attn_last_error().decode(), (kw, L.attn_last_error())


def test_lds_probe_declines(L):
    """The LDS read probe validates its kind, iteration count, buffers and every lane address on the host
    before launching (no GPU needed for these)."""
    out = 1 << 20  # fake aligned device address, never dereferenced

    def call(kind=0, addrs=None, iters=4, o=out, ob=256):
        arr = (ctypes.c_int32 * 64)(*(addrs if addrs is not None else [16 * l for l in range(64)]))
        return L.attn_lds_probe(kind, arr, iters, o, ob, None)

    lane5 = lambda a: [a if l == 5 else -1 for l in range(64)]
    cases = [
        (dict(kind=3), INVALID, "kind"), (dict(kind=-1), INVALID, "kind"),
        (dict(iters=0), INVALID, "iters"), (dict(iters=(1 << 20) + 1), INVALID, "iters"),
        (dict(o=None), INVALID, "NULL"), (dict(o=out + 2), ALIGN, "out"), (dict(ob=252), WORKSPACE, "out holds"),
        (dict(addrs=lane5(8)), ALIGN, "lane 5"), (dict(kind=1, addrs=lane5(4)), ALIGN, "lane 5"),
        (dict(addrs=lane5(32768 - 8)), ALIGN, "lane 5"), (dict(addrs=lane5(32768)), INVALID, "passes"),
        (dict(kind=2, addrs=lane5(32768 - 4)), ALIGN, "lane 5"), (dict(kind=2, addrs=lane5(32768)), INVALID, "passes"),
    ]
    for kw, want, frag in cases:
        assert call(**kw) == want, kw
        assert frag in L.attn_last_error().decode(), (kw, L.attn_last_error())


@pytest.mark.parametrize("entry", sorted(set(B.BWD_PASSES.values())))
def test_every_backward_entry_point_validates(L, entry):
    """Each backward entry point (attn_bwd and the single passes, the fused dQ + preprocess pass
    included) runs the same host checks before any launch."""
    fn = getattr(L, entry)

    def call(p, ws_bytes=1 << 30, dq=DQ):
        return fn(ctypes.byref(p), Q, K, V, O, DO, LSE, dq, DK, DV, WS, ws_bytes, None)

    bad = dense_problem()
    bad.head_dim = 100
    expect(L, call(bad), UNSUPPORTED, "head_dim 100")
    p = dense_problem()
    need = L.attn_bwd_workspace_bytes(ctypes.byref(p))
    expect(L, call(p, ws_bytes=need - 256), WORKSPACE, "workspace")
    expect(L, call(p, dq=DQ + 2), ALIGN, "dq")
    expect(L, call(p, dq=DK), OVERLAP, "overlap")


def test_noalloc_declines_before_any_hip_call(L):
    """attn_bwd_noalloc checks the problem and its workspace need against ATTN_NOALLOC_MAX_WORKSPACE on the
    host, before it looks up its device array or launches anything."""
    def call(p):
        return L.attn_bwd_noalloc(ctypes.byref(p), Q, K, V, O, DO, LSE, DQ, DK, DV, None)

    bad = dense_problem()
    bad.head_dim = 100
    expect(L, call(bad), UNSUPPORTED, "head_dim 100")
    big = dense_problem(b=2, sq=262144, skv=64, hq=8, hkv=8, d=64)  # 2 x 262144 x 8 rows x 8 bytes = 32 MiB
    assert L.attn_bwd_workspace_bytes(ctypes.byref(big)) > B.NOALLOC_MAX_WORKSPACE
    expect(L, call(big), WORKSPACE, "attn_bwd_noalloc holds")
    fits = dense_problem(b=1, sq=131072, skv=64, hq=15, hkv=15, d=64)  # 15 MiB of rows: inside the array
    assert 0 < L.attn_bwd_workspace_bytes(ctypes.byref(fits)) <= B.NOALLOC_MAX_WORKSPACE


def test_single_pass_backward_flag(L):
    """ATTN_FLAG_BWD_ATOMIC_DQ: unknown bits are refused; the flag adds 4 * head_dim bytes per query row
    and q-head to the backward workspace; head dims past 128 and the fused dQ + preprocess pass are
    declined with a reason, before any launch."""
    p = dense_problem()
    p.flags = 8
    expect(L, bwd(L, p), INVALID, "unknown flags")
    p = dense_problem(b=2, sq=256, hq=4, d=128)
    base = L.attn_bwd_workspace_bytes(ctypes.byref(p))
    p.flags = B.FLAG_BWD_ATOMIC_DQ
    assert L.attn_bwd_workspace_bytes(ctypes.byref(p)) == base + 2 * 256 * 4 * 128 * 4
    expect(L, L.attn_bwd_dq_preprocess(ctypes.byref(p), Q, K, V, O, DO, LSE, DQ, DK, DV, WS, 1 << 30, None),
           UNSUPPORTED, "attn_bwd_dq_preprocess")
    wide = dense_problem(d=256)
    wide.flags = B.FLAG_BWD_ATOMIC_DQ
    expect(L, bwd(L, wide), UNSUPPORTED, "head dims up to 128")
    need = L.attn_bwd_workspace_bytes(ctypes.byref(p))
    expect(L, bwd(L, p, ws_bytes=need - 256), WORKSPACE, "workspace")


def test_exp_split_flag(L):
    """ATTN_FLAG_FWD_EXP_SPLIT: the forward declines it past head dim 256 with a reason before any launch;
    it changes no workspace size."""
    for d, dv in ((512, 0), (64, 512), (512, 128)):
        p = dense_problem(d=d)
        p.head_dim_v = dv
        p.flags = B.FLAG_FWD_EXP_SPLIT
        expect(L, fwd(L, p), UNSUPPORTED, "head dims up to 256")
    p = dense_problem(b=2, sq=256, hq=4, d=128)
    base_f, base_b = L.attn_fwd_workspace_bytes(ctypes.byref(p)), L.attn_bwd_workspace_bytes(ctypes.byref(p))
    p.flags = B.FLAG_FWD_EXP_SPLIT
    assert L.attn_fwd_workspace_bytes(ctypes.byref(p)) == base_f
    assert L.attn_bwd_workspace_bytes(ctypes.byref(p)) == base_b
    p.flags = B.FLAG_FWD_EXP_SPLIT | 8
    expect(L, fwd(L, p), INVALID, "unknown flags")


def test_stored_ds_flag(L):
    """ATTN_FLAG_BWD_STORED_DS: the flag adds a dtype [Hq x query tokens x max_seqlen_kv rounded up to 64]
    dS array to the backward workspace (dense and packed); head dims up to 256 and the fused dQ +
    preprocess pass are declined with a reason before any launch, and a workspace one 256-byte block short
    is refused."""
    p = dense_problem(b=2, sq=256, skv=300, hq=4, hkv=2, d=512)
    base = L.attn_bwd_workspace_bytes(ctypes.byref(p))
    p.flags = B.FLAG_BWD_STORED_DS
    ds = 2 * 4 * (2 * 256) * 320  # bf16 x heads x tokens x (300 keys rounded up to 64)
    assert L.attn_bwd_workspace_bytes(ctypes.byref(p)) == base + (ds + 255) // 256 * 256
    expect(L, L.attn_bwd_dq_preprocess(ctypes.byref(p), Q, K, V, O, DO, LSE, DQ, DK, DV, WS, 1 << 30, None),
           UNSUPPORTED, "attn_bwd_dq_preprocess")
    need = L.attn_bwd_workspace_bytes(ctypes.byref(p))
    expect(L, bwd(L, p, ws_bytes=need - 256), WORKSPACE, "workspace")
    for d, dv in ((256, 0), (128, 256), (64, 0)):
        narrow = dense_problem(d=d)
        narrow.head_dim_v = dv
        narrow.flags = B.FLAG_BWD_STORED_DS
        expect(L, bwd(L, narrow), UNSUPPORTED, "head dims above 256")
    for d, dv in ((64, 512), (512, 96), (264, 0)):  # any head above 256 on either side takes the mode
        wide = dense_problem(d=d)
        wide.head_dim_v = dv
        wide.flags = B.FLAG_BWD_STORED_DS
        assert L.attn_bwd_workspace_bytes(ctypes.byref(wide)) > 0
    both = dense_problem(d=512)
    both.flags = B.FLAG_BWD_STORED_DS | B.FLAG_BWD_ATOMIC_DQ
    expect(L, bwd(L, both), UNSUPPORTED, "head dims up to 128")
    # the dQ product addresses a workgroup's dS rows with 32-bit offsets: key lengths stay below 2^24
    long_keys = dense_problem(b=1, sq=64, skv=(1 << 24) - 8, hq=1, hkv=1, d=512)
    long_keys.flags = B.FLAG_BWD_STORED_DS
    far = [(1 << 44) + i * (1 << 40) for i in range(10)]  # buffers 1 TiB apart: no extent overlaps
    expect(L, bwd(L, long_keys, *far[:9], ws=far[9], ws_bytes=1 << 62), UNSUPPORTED, "key lengths below 2^24")
    # a dS array beyond 2^62 bytes is declined when the problem is checked (workspace size 0)
    huge = dense_problem(b=1 << 16, sq=1 << 16, skv=1 << 20, hq=64, hkv=64, d=512)
    huge.flags = B.FLAG_BWD_STORED_DS
    assert L.attn_bwd_workspace_bytes(ctypes.byref(huge)) == 0
    # the forward ignores the flag: no workspace change
    p0 = dense_problem(b=2, sq=256, skv=300, hq=4, hkv=2, d=512)
    f0 = L.attn_fwd_workspace_bytes(ctypes.byref(p0))
    p0.flags = B.FLAG_BWD_STORED_DS
    assert L.attn_fwd_workspace_bytes(ctypes.byref(p0)) == f0
