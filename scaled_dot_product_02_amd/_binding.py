"""ctypes binding of the C-ABI in include/attn.h (argument marshalling only).

Every step of attention runs in the HIP kernels of libsdpa02.so. This module
only turns torch tensors (device memory) and the current torch stream into the
pointers, strides and sizes the C entry points take, allocates outputs and
workspace with torch when the caller does not pass them, and raises AttnError
with the library's status and reason when a call is declined. There is no
fallback: if the library is missing, the first call raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libsdpa02.so"

ABI_VERSION = 4
FLAG_BWD_ATOMIC_DQ = 1  # ATTN_FLAG_BWD_ATOMIC_DQ
FLAG_FWD_EXP_SPLIT = 2  # ATTN_FLAG_FWD_EXP_SPLIT
FLAG_BWD_STORED_DS = 4  # ATTN_FLAG_BWD_STORED_DS
STATUS = {0: "ATTN_OK", 1: "ATTN_E_INVALID", 2: "ATTN_E_UNSUPPORTED", 3: "ATTN_E_ALIGN", 4: "ATTN_E_OVERLAP",
          5: "ATTN_E_WORKSPACE", 6: "ATTN_E_HIP"}
MASK_CODES = {"none": 0, "causal_tl": 1, "causal_br": 2}
EXPORTED = ("attn_fwd", "attn_bwd", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_preprocess",
            "attn_bwd_noalloc", "attn_merge", "attn_mfma_probe", "attn_lds_probe", "attn_tile_order_probe",
            "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes", "attn_status_str", "attn_last_error",
            "attn_abi_version")
MERGE_MAX_PARTS = 8
BWD_PASSES = {"all": "attn_bwd", "preprocess": "attn_bwd_preprocess", "dkdv": "attn_bwd_dkdv", "dq": "attn_bwd_dq",
              "dq_preprocess": "attn_bwd_dq_preprocess"}


class AttnProblem(ctypes.Structure):
    """Mirror of attn_problem_t."""
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_kv", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_kv", ctypes.c_void_p),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("window_left", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class AttnError(RuntimeError):
    def __init__(self, status, reason):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        self.reason = reason
        super().__init__(f"{self.status_name}: {reason}")


_LIB = None


def library_path():
    return os.path.join(HERE, LIB_NAME)


def lib():
    """Load libsdpa02.so once. Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run __graft_entry__.build() or "
                               "python -m scaled_dot_product_02_amd.build")
        L = ctypes.CDLL(path)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        pp = ctypes.POINTER(AttnProblem)
        L.attn_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_fwd.restype = ctypes.c_int
        for name in BWD_PASSES.values():
            getattr(L, name).argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
            getattr(L, name).restype = ctypes.c_int
        L.attn_bwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_bwd_noalloc.restype = ctypes.c_int
        L.attn_merge.argtypes = [pp, ctypes.c_int32, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp]
        L.attn_merge.restype = ctypes.c_int
        L.attn_mfma_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float, vp, sz, vp, sz,
                                      vp]
        L.attn_mfma_probe.restype = ctypes.c_int
        L.attn_lds_probe.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, vp, sz, vp]
        L.attn_lds_probe.restype = ctypes.c_int
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.attn_tile_order_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p, i32p, sz]
        L.attn_tile_order_probe.restype = ctypes.c_int
        L.attn_fwd_workspace_bytes.argtypes = [pp]
        L.attn_fwd_workspace_bytes.restype = sz
        L.attn_bwd_workspace_bytes.argtypes = [pp]
        L.attn_bwd_workspace_bytes.restype = sz
        L.attn_status_str.argtypes = [ctypes.c_int]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        L.attn_abi_version.argtypes = []
        L.attn_abi_version.restype = ctypes.c_int32
        _LIB = L
    return _LIB


def _dtype_code(t):
    import torch
    return {torch.bfloat16: 0, torch.float16: 1}.get(t.dtype, 99)  # 99: the library declines it


def _strides(t, packed):
    if t is None:
        return (0, 0, 0)
    st = t.stride()
    if packed:
        return (st[0], st[1], 0)
    return (st[0], st[1], st[2])


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("attention tensors must be GPU tensors (the HIP kernels read them directly)")
        if t is not None and t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous (stride 1)")


def _shape_of(t):
    return tuple(t.shape)


def _check_tensors(q, k, v, packed, cu_seqlens_q=None, cu_seqlens_kv=None, o=None, do=None, lse=None, dq=None,
                   dk=None, dv=None):
    """Every tensor must agree with q before any pointer reaches the library, which sizes every extent from
    the problem it builds out of q, k and v: one 16-bit dtype (bf16 or fp16) for Q, K, V, O, dO, dQ, dK, dV;
    the documented shapes (dense Q [B,Sq,Hq,Dqk], K [B,Skv,Hkv,Dqk], V [B,Skv,Hkv,Dv], O and dO
    [B,Sq,Hq,Dv]; packed Q [Tq,Hq,Dqk], K [Tkv,Hkv,Dqk], V [Tkv,Hkv,Dv], O and dO [Tq,Hq,Dv]); dQ, dK, dV the
    shapes of Q, K, V; LSE contiguous float32 [B,Hq,Sq] or [Tq,Hq]; cu_seqlens contiguous 1-D int32 of one
    length; all on one device. Raises ValueError naming the first mismatch."""
    import torch
    nd = 3 if packed else 4
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != nd:
            raise ValueError(f"{n} must be {'[T,H,D]' if packed else '[B,S,H,D]'}; got shape {_shape_of(t)}")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"q must be bfloat16 or float16; got {q.dtype}")
    if packed:
        tq, hq, dqk = q.shape
        tk, hkv, dk_ = k.shape
        if dk_ != dqk:
            raise ValueError(f"k head dim {dk_} differs from q's {dqk}")
        if tuple(v.shape[:2]) != (tk, hkv):
            raise ValueError(f"v shape {_shape_of(v)} does not match k's tokens and heads {(tk, hkv)}")
        dvh = v.shape[2]
        o_shape, lse_shape = (tq, hq, dvh), (tq, hq)
    else:
        b, sq, hq, dqk = q.shape
        if k.shape[0] != b or k.shape[3] != dqk:
            raise ValueError(f"k shape {_shape_of(k)} does not match q's batch {b} and head dim {dqk}")
        _, skv, hkv, _ = k.shape
        if tuple(v.shape[:3]) != (b, skv, hkv):
            raise ValueError(f"v shape {_shape_of(v)} does not match k's {(b, skv, hkv)}")
        dvh = v.shape[3]
        o_shape, lse_shape = (b, sq, hq, dvh), (b, hq, sq)
    expect = {"k": (k, None), "v": (v, None), "o": (o, o_shape), "do": (do, o_shape), "dq": (dq, tuple(q.shape)),
              "dk": (dk, tuple(k.shape)), "dv": (dv, tuple(v.shape))}
    for n, (t, shape) in expect.items():
        if t is None:
            continue
        if t.dtype != q.dtype:
            raise ValueError(f"{n} has dtype {t.dtype}; every attention tensor must have q's dtype {q.dtype}")
        if shape is not None and _shape_of(t) != shape:
            raise ValueError(f"{n} must have shape {shape}; got {_shape_of(t)}")
    if lse is not None:
        if lse.dtype != torch.float32:
            raise ValueError(f"lse must be float32; got {lse.dtype}")
        if _shape_of(lse) != lse_shape:
            raise ValueError(f"lse must have shape {lse_shape}; got {_shape_of(lse)}")
        if not lse.is_contiguous():
            raise ValueError("lse must be contiguous")
    if packed:
        for n, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
            if c is None:
                raise ValueError("packed batches need both cu_seqlens_q and cu_seqlens_kv")
            if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
                raise ValueError(f"{n} must be a contiguous 1-D int32 tensor")
        if cu_seqlens_q.numel() != cu_seqlens_kv.numel() or cu_seqlens_q.numel() < 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_kv must both hold batch + 1 >= 1 entries")
    elif cu_seqlens_kv is not None:
        raise ValueError("cu_seqlens_kv given without cu_seqlens_q")
    ts = [t for t in (q, k, v, o, do, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_kv) if t is not None]
    if any(t.device != q.device for t in ts):
        raise ValueError("all attention tensors must be on one device")
    _check_device(*ts)


def make_problem(q, k, v, o_like, mask, scale, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                 window_left=-1, flags=0):
    packed = cu_seqlens_q is not None
    p = AttnProblem()
    p.abi_version = ABI_VERSION
    p.dtype = _dtype_code(q)
    p.mask = MASK_CODES[mask] if isinstance(mask, str) else int(mask)
    d = q.shape[-1]
    p.scale = float(scale) if scale is not None else d ** -0.5
    p.heads_q = q.shape[-2]
    p.heads_kv = k.shape[-2]
    p.head_dim = d
    p.head_dim_v = 0 if v.shape[-1] == d else v.shape[-1]  # V/O head dim when it differs from Q/K's
    if packed:
        p.batch = cu_seqlens_q.numel() - 1
        p.total_q = q.shape[0]
        p.total_kv = k.shape[0]
        p.cu_seqlens_q = cu_seqlens_q.data_ptr()
        p.cu_seqlens_kv = cu_seqlens_kv.data_ptr()
        if max_seqlen_q is None or max_seqlen_kv is None:
            raise ValueError("packed batches need max_seqlen_q and max_seqlen_kv (host-known upper bounds)")
        p.max_seqlen_q, p.max_seqlen_kv = int(max_seqlen_q), int(max_seqlen_kv)
    else:
        p.batch = q.shape[0]
        p.max_seqlen_q = q.shape[1]
        p.max_seqlen_kv = k.shape[1]
    p.q_stride[:] = _strides(q, packed)
    p.k_stride[:] = _strides(k, packed)
    p.v_stride[:] = _strides(v, packed)
    p.o_stride[:] = _strides(o_like, packed)
    p.window_left = int(window_left)
    p.flags = int(flags)
    return p


def _raise(status):
    L = lib()
    raise AttnError(status, L.attn_last_error().decode())


def _stream(stream):
    import torch
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def _workspace(nbytes, device, workspace):
    import torch
    if nbytes == 0:
        return workspace
    if workspace is not None:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_fwd_workspace_bytes(p):
    return lib().attn_fwd_workspace_bytes(ctypes.byref(p))


def attn_bwd_workspace_bytes(p):
    return lib().attn_bwd_workspace_bytes(ctypes.byref(p))


def attn_fwd(q, k, v, mask="causal_tl", scale=None, cu_seqlens_q=None, cu_seqlens_kv=None, max_seqlen_q=None,
             max_seqlen_kv=None, out=None, lse=None, workspace=None, stream=None, window_left=-1, exp_split=False):
    """Forward through the C-ABI. Returns (O, LSE).

    Dense q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D]; packed q [Tq,Hq,D], k/v [Tkv,Hkv,D] with int32
    cu_seqlens on the device. V (and O) may have their own head dim D_v; O is then [..., Hq, D_v].
    LSE is fp32 [B,Hq,Sq] (dense) or [Tq,Hq] (packed). ``exp_split`` sets ATTN_FLAG_FWD_EXP_SPLIT (a quarter
    of the exponentials on interior tiles by a VALU polynomial; head dims up to 256).
    """
    import torch
    packed = cu_seqlens_q is not None
    _check_tensors(q, k, v, packed, cu_seqlens_q, cu_seqlens_kv, o=out, lse=lse)
    if out is None:
        out = torch.empty(q.shape[:-1] + v.shape[-1:], dtype=q.dtype, device=q.device)
    if lse is None:
        shape = (q.shape[0], q.shape[1]) if packed else (q.shape[0], q.shape[2], q.shape[1])
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    p = make_problem(q, k, v, out, mask, scale, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                     window_left, FLAG_FWD_EXP_SPLIT if exp_split else 0)
    L = lib()
    need = L.attn_fwd_workspace_bytes(ctypes.byref(p))
    ws = _workspace(need, q.device, workspace)
    st = L.attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
                    0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if st != 0:
        _raise(st)
    return out, lse


def attn_bwd(q, k, v, o, do, lse, mask="causal_tl", scale=None, cu_seqlens_q=None, cu_seqlens_kv=None,
             max_seqlen_q=None, max_seqlen_kv=None, dq=None, dk=None, dv=None, workspace=None, stream=None,
             passes=("all",), window_left=-1, atomic_dq=False, stored_ds=False):
    """Backward through the C-ABI from the forward's O and LSE. Returns (dQ, dK, dV).

    dO must have O's strides; dQ/dK/dV are allocated with Q/K/V's shapes (contiguous) unless given.
    ``passes`` lists the entry points to call in order: "all" (attn_bwd) or any of "preprocess",
    "dkdv", "dq", "dq_preprocess" (attn_bwd_preprocess / attn_bwd_dkdv / attn_bwd_dq /
    attn_bwd_dq_preprocess, which share the workspace; "dq_preprocess" then "dkdv" is what
    attn_bwd runs for head dims up to 256). ``atomic_dq`` sets ATTN_FLAG_BWD_ATOMIC_DQ (the single-pass
    backward, head dims up to 128): then "preprocess", "dkdv", "dq" is what attn_bwd runs. ``stored_ds`` sets
    ATTN_FLAG_BWD_STORED_DS (dS stored by the dK/dV pass, dQ as its product with K; head dims above 256;
    the workspace then holds Hq x tokens x max_seqlen_kv (rounded up to 64) dS values): "preprocess",
    "dkdv", "dq" again.
    """
    import torch
    _check_tensors(q, k, v, cu_seqlens_q is not None, cu_seqlens_q, cu_seqlens_kv, o=o, do=do, lse=lse, dq=dq,
                   dk=dk, dv=dv)
    if do.stride() != o.stride():
        raise ValueError("dO must have the same strides as O")
    if dq is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    if dk is None:
        dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    if dv is None:
        dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("dQ/dK/dV must have the strides of Q/K/V")
    p = make_problem(q, k, v, o, mask, scale, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                     window_left, (FLAG_BWD_ATOMIC_DQ if atomic_dq else 0) | (FLAG_BWD_STORED_DS if stored_ds else 0))
    L = lib()
    need = L.attn_bwd_workspace_bytes(ctypes.byref(p))
    ws = _workspace(need, q.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    sptr = _stream(stream)
    for name in passes:
        st = getattr(L, BWD_PASSES[name])(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nbytes, sptr)
        if st != 0:
            _raise(st)
    return dq, dk, dv


NOALLOC_MAX_WORKSPACE = 16 << 20  # ATTN_NOALLOC_MAX_WORKSPACE


def attn_bwd_noalloc(q, k, v, o, do, lse, mask="causal_tl", scale=None, cu_seqlens_q=None, cu_seqlens_kv=None,
                     max_seqlen_q=None, max_seqlen_kv=None, dq=None, dk=None, dv=None, stream=None, window_left=-1,
                     stored_ds=False):
    """attn_bwd_noalloc through the C-ABI: attn_bwd with the library's own per-device scratch array as the
    workspace (no workspace argument; problems needing more than NOALLOC_MAX_WORKSPACE bytes are declined).
    ``stored_ds`` sets ATTN_FLAG_BWD_STORED_DS as in attn_bwd (its dS array must fit the scratch array too).
    Returns (dQ, dK, dV); dQ/dK/dV are allocated here unless given (the library allocates nothing)."""
    import torch
    _check_tensors(q, k, v, cu_seqlens_q is not None, cu_seqlens_q, cu_seqlens_kv, o=o, do=do, lse=lse, dq=dq,
                   dk=dk, dv=dv)
    if do.stride() != o.stride():
        raise ValueError("dO must have the same strides as O")
    if dq is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    if dk is None:
        dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    if dv is None:
        dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("dQ/dK/dV must have the strides of Q/K/V")
    p = make_problem(q, k, v, o, mask, scale, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                     window_left, FLAG_BWD_STORED_DS if stored_ds else 0)
    st = lib().attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                _ptr(dk), _ptr(dv), _stream(stream))
    if st != 0:
        _raise(st)
    return dq, dk, dv


def merge_problem(o_like, cu_seqlens_q=None, max_seqlen_q=None):
    """The query-side problem attn_merge reads: dense O [B,Sq,Hq,D] or packed O [Tq,Hq,D] (cu_seqlens_q
    marks the packed layout; the merge does not read it)."""
    packed = cu_seqlens_q is not None
    p = AttnProblem()
    p.abi_version = ABI_VERSION
    p.dtype = _dtype_code(o_like)
    p.heads_q = o_like.shape[-2]
    p.heads_kv = o_like.shape[-2]
    p.head_dim = o_like.shape[-1]
    p.scale = 1.0
    if packed:
        p.batch = cu_seqlens_q.numel() - 1
        p.total_q = o_like.shape[0]
        p.cu_seqlens_q = cu_seqlens_q.data_ptr()
        p.max_seqlen_q = int(max_seqlen_q) if max_seqlen_q is not None else 0
    else:
        p.batch = o_like.shape[0]
        p.max_seqlen_q = o_like.shape[1]
    p.o_stride[:] = _strides(o_like, packed)
    p.window_left = -1
    return p


def attn_merge(o_parts, lse_parts, cu_seqlens_q=None, max_seqlen_q=None, out=None, lse=None, stream=None):
    """Merge per-chunk forward results of the same queries over disjoint key sets (attn_merge).

    o_parts: up to MERGE_MAX_PARTS tensors with one layout (dense [B,Sq,Hq,D] or packed [Tq,Hq,D]);
    lse_parts: their fp32 Stats ([B,Hq,Sq] or [Tq,Hq]). ``out`` / ``lse`` may be one of the parts
    (in-place). Returns (O, LSE).
    """
    import torch
    o_parts, lse_parts = list(o_parts), list(lse_parts)
    if not o_parts or len(o_parts) != len(lse_parts):
        raise ValueError("o_parts and lse_parts must be non-empty and of equal length")
    ref = o_parts[0]
    packed = cu_seqlens_q is not None
    if ref.dim() != (3 if packed else 4):
        raise ValueError(f"o_parts must be {'[Tq,Hq,D]' if packed else '[B,Sq,Hq,D]'}; got shape {tuple(ref.shape)}")
    if ref.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"o_parts must be bfloat16 or float16; got {ref.dtype}")
    for x in o_parts:
        if x.shape != ref.shape or x.stride() != ref.stride() or x.dtype != ref.dtype:
            raise ValueError("all parts of O must share shape, strides and dtype")
    lse_shape = (ref.shape[0], ref.shape[1]) if packed else (ref.shape[0], ref.shape[2], ref.shape[1])
    for x in lse_parts + ([lse] if lse is not None else []):
        if x.dtype != torch.float32 or tuple(x.shape) != lse_shape or not x.is_contiguous():
            raise ValueError(f"every LSE must be contiguous float32 of shape {lse_shape}")
    if out is not None and (out.shape != ref.shape or out.dtype != ref.dtype):
        raise ValueError("out must have the parts' shape and dtype")
    if packed and (cu_seqlens_q.dtype != torch.int32 or cu_seqlens_q.dim() != 1):
        raise ValueError("cu_seqlens_q must be a 1-D int32 tensor")
    ts = [t for t in (*o_parts, *lse_parts, out, lse, cu_seqlens_q) if t is not None]
    if any(t.device != ref.device for t in ts):
        raise ValueError("all tensors must be on one device")
    _check_device(*ts)
    if out is None:
        out = torch.empty_like(ref)
    if out.stride() != ref.stride():
        raise ValueError("out must have the parts' strides")
    if lse is None:
        lse = torch.empty_like(lse_parts[0])
    p = merge_problem(ref, cu_seqlens_q, max_seqlen_q)
    n = len(o_parts)
    oa = (ctypes.c_void_p * n)(*[x.data_ptr() for x in o_parts])
    la = (ctypes.c_void_p * n)(*[x.data_ptr() for x in lse_parts])
    st = lib().attn_merge(ctypes.byref(p), n, oa, la, _ptr(out), _ptr(lse), _stream(stream))
    if st != 0:
        _raise(st)
    return out, lse


LDS_READ_KINDS = {"b128": 0, "b64_tr_b16": 1, "b64": 2}  # ATTN_LDS_READ_*
LDS_PROBE_BYTES = 32768  # ATTN_LDS_PROBE_BYTES


def attn_lds_probe(kind, lane_addr, iters, out, stream=None):
    """LDS read probe (attn_lds_probe): one wave reads 8 * iters times at lane_addr[l] (64 byte addresses,
    negative = lane inactive) with the read `kind` ("b128", "b64_tr_b16", "b64"); `out` is a device int32
    tensor of at least 64 elements. Asynchronous on `stream`."""
    if len(lane_addr) != 64:
        raise ValueError("lane_addr needs 64 entries")
    arr = (ctypes.c_int32 * 64)(*[int(a) for a in lane_addr])
    st = lib().attn_lds_probe(LDS_READ_KINDS[kind], arr, int(iters), _ptr(out), out.numel() * out.element_size(),
                              _stream(stream))
    if st != 0:
        _raise(st)


ORDERS = {"tile_major": 0, "query": 1, "grouped": 2}


def attn_tile_order_probe(units, tiles, reverse=False, order="query"):
    """The kernels' workgroup order (attn_tile_order_probe, evaluated on the host): two lists of
    units * tiles ints, the unit and the tile of each workgroup index. order "query" is that of the
    forward and the dQ pass, "grouped" of the dense dK/dV passes, "tile_major" of the packed ones."""
    n = int(units) * int(tiles)
    u = (ctypes.c_int32 * max(n, 1))()
    t = (ctypes.c_int32 * max(n, 1))()
    st = lib().attn_tile_order_probe(int(units), int(tiles), int(bool(reverse)), ORDERS[order], u, t, n)
    if st != 0:
        _raise(st)
    return list(u)[:n], list(t)[:n]


def attn_mfma_probe(blocks, iters, x=0.5, y=1.0 / 512, device="cuda:0", stream=None):
    """Matrix-core rate probe (attn_mfma_probe): launches it on `stream` and returns (out, ticks), a
    float32 [blocks * 256] checksum tensor and an int64 [blocks, 2] tensor of (shader-clock ticks,
    100 MHz ticks) per workgroup, both on `device`. One call executes blocks * 4 * iters * 4 * 32768 FLOP."""
    import torch
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    ticks = torch.empty((blocks, 2), dtype=torch.int64, device=device)
    st = lib().attn_mfma_probe(int(blocks), int(iters), float(x), float(y), _ptr(out), out.numel() * 4, _ptr(ticks),
                               ticks.numel() * 8, _stream(stream))
    if st != 0:
        _raise(st)
    return out, ticks
