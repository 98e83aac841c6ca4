"""Seeded synthetic attention workloads (inputs only; no attention arithmetic).

The pages measure on synthetic shapes, not on a dataset: pull request 3527
("cuDNN FROST attention backend for head_dim in (256, 512], with context
parallelism", section Performance) times b2 hq8 hkv4 d512 causal bf16, and
pull request 3705 (FROST forward provider for context-parallel attention,
section "Current-software original-method CP results") times BF16 causal
compact-THD batches with Hq32/Hkv8, D128. The workloads below keep that
structure (GQA ratios, packed variable-length batches, causal masks, a
rectangular bottom-right block for the single-rank context-parallel share)
at the sizes this engine is measured on. Values are N(0, 1).

Recipe (identical for every consumer, GPU path and oracle alike):
  gen = torch.Generator("cpu").manual_seed(seed)
  packed batches first draw their lengths: randint(lo, hi + 1, (nseq,))
  then Q, K, V, dO are drawn in that order as float32 N(0, 1) and rounded to
  the dtype (round to nearest even). Those dtype tensors are the inputs.
  Q and K have head dim d; V and dO have d_v (= d unless set).
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
MASKS = ("none", "causal_tl", "causal_br")


@dataclass(frozen=True)
class Workload:
    name: str
    hq: int
    hkv: int
    d: int
    dtype: str
    mask: str
    seed: int
    batch: int = 1
    sq: int = 0
    skv: int = 0
    # packed (THD) batches: number of sequences and the inclusive length range
    nseq: int = 0
    len_range: Tuple[int, int] = (0, 0)
    # explicit packed lengths (tests); overrides len_range when given
    seqlens: Optional[Tuple[int, ...]] = None
    seqlens_kv: Optional[Tuple[int, ...]] = None
    # sliding window below the causal diagonal (keys i+delta-W .. i+delta); -1 = none
    window_left: int = -1
    # head dim of V, O, dO when it differs from d (the Q/K head dim); 0 = same as d
    dv: int = 0
    note: str = field(default="", compare=False)

    @property
    def packed(self):
        return self.nseq > 0 or self.seqlens is not None

    @property
    def d_v(self):
        return self.dv or self.d

    @property
    def scale(self):
        return 1.0 / (self.d ** 0.5)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]


WORKLOADS = {
    "tiny": Workload("tiny", batch=1, hq=2, hkv=2, sq=128, skv=128, d=64, dtype="fp16", mask="causal_tl", seed=0,
                     note="B1 H2/2 S128 D64 fp16 causal top-left"),
    "dense_d128": Workload("dense_d128", batch=2, hq=16, hkv=16, sq=8192, skv=8192, d=128, dtype="bf16",
                           mask="causal_tl", seed=1, note="B2 H16/16 S8192 D128 bf16 causal top-left (MHA)"),
    "thd_d128": Workload("thd_d128", nseq=16, len_range=(256, 4096), hq=32, hkv=8, d=128, dtype="bf16",
                         mask="causal_tl", seed=2, note="16 packed sequences, lengths U{256..4096}, Hq32/Hkv8 D128 bf16"),
    "dense_d512": Workload("dense_d512", batch=1, hq=16, hkv=4, sq=8192, skv=8192, d=512, dtype="bf16",
                           mask="causal_tl", seed=3, note="B1 Hq16/Hkv4 S8192 D512 bf16 causal"),
    "cp_share_d256": Workload("cp_share_d256", batch=1, hq=16, hkv=8, sq=4096, skv=16384, d=256, dtype="fp16",
                              mask="causal_br", seed=4, note="single-rank CP share: Sq4096 vs Skv16384 BR, D256 fp16"),
    "cp_share_d512": Workload("cp_share_d512", batch=1, hq=16, hkv=8, sq=4096, skv=16384, d=512, dtype="fp16",
                              mask="causal_br", seed=4, note="single-rank CP share: Sq4096 vs Skv16384 BR, D512 fp16"),
    # a local (sliding-window) layer at D=256, the other half of the hybrid model pull request 3527 motivates
    "window_d256": Workload("window_d256", batch=1, hq=16, hkv=8, sq=8192, skv=8192, d=256, dtype="bf16",
                            mask="causal_tl", window_left=1023, seed=5,
                            note="B1 Hq16/Hkv8 S8192 D256 bf16 causal with a 1024-key sliding window"),
    # the asymmetric head pair (Q/K 192, V/O 128) that pull request 3527 says the forward engine lists,
    # at the dense D=128 shape; it runs on the D=256 kernels with padded columns
    "asym_d192": Workload("asym_d192", batch=2, hq=16, hkv=16, sq=8192, skv=8192, d=192, dv=128, dtype="bf16",
                          mask="causal_tl", seed=6, note="B2 H16/16 S8192 Dqk192/Dv128 bf16 causal top-left"),
    # many short sequences: every pass moves more bytes per FLOP than the chip's balance point
    # (2.5 PFLOP/s / 8 TB/s), so HBM bandwidth, not the matrix cores, bounds it
    "short_d128": Workload("short_d128", batch=128, hq=16, hkv=16, sq=256, skv=256, d=128, dtype="bf16",
                           mask="causal_tl", seed=7, note="B128 H16/16 S256 D128 bf16 causal top-left (HBM-bound)"),
}


def make_inputs(w: Workload, with_do: bool = True):
    """Draw the workload's inputs on the CPU. Returns a dict of tensors.

    Keys: q, k, v, do (dtype tensors, dense [B,S,H,D] or packed [T,H,D]),
    seqlens_q, seqlens_kv (python lists), cu_seqlens_q, cu_seqlens_kv (int32
    tensors, zero-based cumulative, or None for dense), max_seqlen_q/kv.
    """
    gen = torch.Generator("cpu").manual_seed(w.seed)
    dt = w.torch_dtype
    if w.packed:
        if w.seqlens is not None:
            lq = list(w.seqlens)
        else:
            lo, hi = w.len_range
            lq = torch.randint(lo, hi + 1, (w.nseq,), generator=gen).tolist()
        lk = list(w.seqlens_kv) if w.seqlens_kv is not None else list(lq)
        cq = torch.zeros(len(lq) + 1, dtype=torch.int32)
        ck = torch.zeros(len(lk) + 1, dtype=torch.int32)
        cq[1:] = torch.cumsum(torch.tensor(lq, dtype=torch.int64), 0).to(torch.int32)
        ck[1:] = torch.cumsum(torch.tensor(lk, dtype=torch.int64), 0).to(torch.int32)
        lead_q, lead_k = (int(cq[-1]),), (int(ck[-1]),)
    else:
        lq, lk = [w.sq] * w.batch, [w.skv] * w.batch
        cq = ck = None
        lead_q, lead_k = (w.batch, w.sq), (w.batch, w.skv)
    q = torch.randn(lead_q + (w.hq, w.d), generator=gen, dtype=torch.float32).to(dt)
    k = torch.randn(lead_k + (w.hkv, w.d), generator=gen, dtype=torch.float32).to(dt)
    v = torch.randn(lead_k + (w.hkv, w.d_v), generator=gen, dtype=torch.float32).to(dt)
    do = torch.randn(lead_q + (w.hq, w.d_v), generator=gen, dtype=torch.float32).to(dt) if with_do else None
    return dict(q=q, k=k, v=v, do=do, seqlens_q=lq, seqlens_kv=lk, cu_seqlens_q=cq, cu_seqlens_kv=ck,
                max_seqlen_q=max(lq) if lq else 0, max_seqlen_kv=max(lk) if lk else 0)


def draw_device(shape, seed, dtype, device="cuda:0"):
    """N(0,1) in float32 from torch's seeded generator on the device, rounded to dtype: inputs too large
    to draw on the host and copy up (the tests read back the slices they check)."""
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    out = x.to(dtype)
    del x
    return out


def small(name="small", *, batch=1, hq=2, hkv=2, sq=64, skv=64, d=64, dtype="bf16", mask="causal_tl", seed=0,
          seqlens=None, seqlens_kv=None, window_left=-1, dv=0):
    """A test-sized workload with the same recipe."""
    return Workload(name, batch=batch, hq=hq, hkv=hkv, sq=sq, skv=skv, d=d, dtype=dtype, mask=mask, seed=seed,
                    seqlens=tuple(seqlens) if seqlens is not None else None,
                    seqlens_kv=tuple(seqlens_kv) if seqlens_kv is not None else None, window_left=window_left,
                    dv=dv)
