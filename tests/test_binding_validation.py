"""CPU: the Python binding refuses tensors that disagree with q before any library call.

The C-ABI sizes every extent from the problem the binding builds out of q, k and v, so a
K with a smaller batch, a V with fewer tokens, a float32 dO, a bf16 LSE or a dQ with Q's
strides but fewer rows would let the kernels read or write past the caller's buffers.
The binding checks shapes, dtypes and devices first and raises ValueError; these tests use
CPU tensors, which the binding refuses last ("must be GPU tensors"), so every other
mismatch is seen before that and nothing reaches the library.
"""

import pytest
import torch

import scaled_dot_product_02_amd as sd

BF = torch.bfloat16


def dense(b=2, sq=40, skv=56, hq=4, hkv=2, d=64, dv=64, dtype=BF):
    q = torch.zeros(b, sq, hq, d, dtype=dtype)
    k = torch.zeros(b, skv, hkv, d, dtype=dtype)
    v = torch.zeros(b, skv, hkv, dv, dtype=dtype)
    o = torch.zeros(b, sq, hq, dv, dtype=dtype)
    lse = torch.zeros(b, hq, sq, dtype=torch.float32)
    return q, k, v, o, lse


def packed(tq=30, tkv=44, hq=4, hkv=2, d=64, dv=64, nseq=3):
    q = torch.zeros(tq, hq, d, dtype=BF)
    k = torch.zeros(tkv, hkv, d, dtype=BF)
    v = torch.zeros(tkv, hkv, dv, dtype=BF)
    o = torch.zeros(tq, hq, dv, dtype=BF)
    lse = torch.zeros(tq, hq, dtype=torch.float32)
    cq = torch.tensor([0, 10, 20, tq][:nseq + 1], dtype=torch.int32)
    ck = torch.tensor([0, 14, 30, tkv][:nseq + 1], dtype=torch.int32)
    return q, k, v, o, lse, cq, ck


def fwd_raises(match, *a, **kw):
    with pytest.raises(ValueError, match=match):
        sd.attn_fwd(*a, **kw)


def bwd_raises(match, *a, **kw):
    with pytest.raises(ValueError, match=match):
        sd.attn_bwd(*a, **kw)


def test_consistent_cpu_tensors_reach_only_the_device_check():
    q, k, v, o, lse = dense()
    fwd_raises("GPU tensors", q, k, v, out=o, lse=lse)
    bwd_raises("GPU tensors", q, k, v, o, o.clone(), lse, dq=torch.zeros_like(q), dk=torch.zeros_like(k),
               dv=torch.zeros_like(v))
    q, k, v, o, lse, cq, ck = packed()
    fwd_raises("GPU tensors", q, k, v, out=o, lse=lse, cu_seqlens_q=cq, cu_seqlens_kv=ck, max_seqlen_q=10,
               max_seqlen_kv=16)


def test_dense_shape_mismatches():
    q, k, v, o, lse = dense()
    fwd_raises("k shape", q, k[:1], v[:1])                          # K with a smaller batch
    fwd_raises("v shape", q, k, v[:, :50])                          # V with fewer keys than K
    fwd_raises("v shape", q, k, torch.zeros(2, 56, 1, 64, dtype=BF))  # V with other heads
    fwd_raises("k head dim|k shape", q, torch.zeros(2, 56, 2, 32, dtype=BF), v)
    fwd_raises("o must have shape", q, k, v, out=o[:, :39])
    fwd_raises("lse must have shape", q, k, v, lse=lse[:1])
    fwd_raises("q must be", q[0], k, v)                              # 3-D Q without cu_seqlens
    bwd_raises("do must have shape", q, k, v, o, o[:, :20], lse)
    bwd_raises("dq must have shape", q, k, v, o, o.clone(), lse, dq=q[:1])
    bwd_raises("dk must have shape", q, k, v, o, o.clone(), lse, dk=k[:, :50])
    bwd_raises("dv must have shape", q, k, v, o, o.clone(), lse, dv=torch.zeros(2, 56, 2, 32, dtype=BF))


def test_dtype_mismatches():
    q, k, v, o, lse = dense()
    fwd_raises("q must be bfloat16 or float16", q.float(), k.float(), v.float())
    fwd_raises("k has dtype", q, k.half(), v)
    fwd_raises("v has dtype", q, k, v.half())
    bwd_raises("do has dtype", q, k, v, o, o.float(), lse)           # dO in fp32
    bwd_raises("lse must be float32", q, k, v, o, o.clone(), lse.to(BF))
    bwd_raises("dq has dtype", q, k, v, o, o.clone(), lse, dq=torch.zeros_like(q, dtype=torch.float16))


def test_lse_must_be_contiguous():
    q, k, v, o, lse = dense()
    strided = torch.zeros(2, 4, 80, dtype=torch.float32)[:, :, ::2]
    bwd_raises("lse must be contiguous", q, k, v, o, o.clone(), strided)


def test_asymmetric_head_dims_follow_v():
    q, k, v, o, lse = dense(d=64, dv=32)
    fwd_raises("GPU tensors", q, k, v, out=o)                        # O takes V's head dim
    fwd_raises("o must have shape", q, k, v, out=torch.zeros(2, 40, 4, 64, dtype=BF))


def test_packed_mismatches():
    q, k, v, o, lse, cq, ck = packed()
    kw = dict(max_seqlen_q=10, max_seqlen_kv=16)
    fwd_raises("v shape", q, k, v[:40], cu_seqlens_q=cq, cu_seqlens_kv=ck, **kw)
    fwd_raises("int32", q, k, v, cu_seqlens_q=cq.long(), cu_seqlens_kv=ck, **kw)
    fwd_raises("batch \\+ 1", q, k, v, cu_seqlens_q=cq, cu_seqlens_kv=ck[:3], **kw)
    fwd_raises("both cu_seqlens", q, k, v, cu_seqlens_q=cq, **kw)
    fwd_raises("lse must have shape", q, k, v, lse=lse.t().contiguous(), cu_seqlens_q=cq, cu_seqlens_kv=ck, **kw)
    fwd_raises("T,H,D", torch.zeros(1, 30, 4, 64, dtype=BF), k, v, cu_seqlens_q=cq, cu_seqlens_kv=ck, **kw)


def test_merge_mismatches():
    o = torch.zeros(2, 40, 4, 64, dtype=BF)
    l = torch.zeros(2, 4, 40, dtype=torch.float32)
    with pytest.raises(ValueError, match="LSE"):
        sd.attn_merge([o, o.clone()], [l, l.to(BF)])
    with pytest.raises(ValueError, match="LSE"):
        sd.attn_merge([o], [l[:, :, :20]])
    with pytest.raises(ValueError, match="share shape"):
        sd.attn_merge([o, o[:, :20]], [l, l])
    with pytest.raises(ValueError, match="out must have"):
        sd.attn_merge([o], [l], out=o.half())
    with pytest.raises(ValueError, match="GPU tensors"):
        sd.attn_merge([o], [l])
