"""Benchmark: fused attention forward + backward TFLOP/s on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense_d128]

One step is the whole hot path over one batch already resident in HBM: attn_fwd,
then the backward passes exactly as attn_bwd runs them, each a single kernel
launch on the current stream: attn_bwd_dq_preprocess (the dQ pass with the
preprocess folded in) and attn_bwd_dkdv for head dims up to 256,
attn_bwd_preprocess, attn_bwd_dkdv and attn_bwd_dq for wider heads.
Credited FLOPs (algorithmic, exact allowed-pair counts): forward 4*D per allowed
(query, key) pair and q-head, backward 10*D (S recompute, dV, dP, dK, dQ). The
value is (F_fwd + F_bwd) / step time. HIP events bracket every launch inside the
timed region (mean, median and minimum per kernel); the kernel with the largest
per-step time is reported under
"roofline". Each kernel is placed on the roofline by its algorithmic FLOPs per launch
(forward 4D, dK/dV pass 8D, dQ pass 2D per pair, which sum to the 14D credited per
step; the dQ pass's second S/dP recompute is not credited) over its compulsory HBM
bytes: below the balance point 2.5 PFLOP/s / 8 TB/s it is HBM-bound and "achieved"
is compulsory bytes per second against 8 TB/s, else MFMA-bound and "achieved" is
algorithmic FLOP/s against 2.5 PFLOP/s ("kernel_roofline" lists every kernel of the step).
"cpu_baseline" times the float64 CPU oracle on a bounded sample of the same
workload. The default run also times, under "cases", every other named case
(tiny B1 H2 S128 D64 fp16; the packed GQA batch thd_d128; dense_d512; the two
single-rank context-parallel shares at D=256 and D=512): forward, backward and
combined ms, TFLOP/s and fraction of peak, compulsory-byte GB/s, per-kernel
times, and the float64 oracle timed on a bounded slice of the same case (the D=512 cases also with the
stored-dS backward, ATTN_FLAG_BWD_STORED_DS, under "stored_ds"). Under
"extra" it reports attn_merge (two forward results combined, the ring step) on
the dense D=128 query side against the HBM peak, and the HBM-bound
short-sequence workload (B128 S256 D128), also with the 256 MB memory-side
cache overwritten before every step; "sustained_mfma" (the rate and engine clock of
attn_mfma_probe, MFMAs from registers only), "hbm_copy" (a plain 1 GiB device
copy) and "telemetry" (rocm-smi clocks,
power and temperature before and after the timed steps) give context for the
fractions of peak. Prints one JSON line on stdout; diagnostics go to stderr.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s at D=128/512 bf16; % of MFMA bf16 peak"
PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated against a plain device
# copy of known size (profiles/dense_d128_hbm_traffic.md). Each entry is valid only for the kernel it was
# measured on: "traffic" is null once that kernel's source fingerprint (kernel_fingerprint) has changed.
TRAFFIC = {
    ("dense_d128", "fwd"): {"fingerprint": "244e429d5eb0", "bytes": 852121147},
    ("dense_d128", "bwd_dq"): {"fingerprint": "c7bbbc9b6b9e", "bytes": 915104803},
    ("dense_d128", "bwd_dkdv"): {"fingerprint": "56ff48a21ae8", "bytes": 693965439},
}
KERNEL_OF = {"fwd": "attn_fwd_kernel", "bwd_dq": "attn_bwd_dq_kernel", "bwd_dkdv": "attn_bwd_dkdv_kernel"}


def _code_only(text):
    """The source without its comments and blank lines (a comment edit leaves a fingerprint unchanged)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_fingerprint(kernel):
    """sha1 prefix of what decides one kernel's code, comments left out: attn_device.h, attn_internal.h, the
    shared part of attn_kernels.hip before its first kernel, the kernel's own definition, and the tile-size
    helpers the launchers instantiate it with."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "scaled_dot_product_02_amd", "csrc")
    src = open(os.path.join(csrc, "attn_kernels.hip")).read()
    parts = [_code_only(open(os.path.join(csrc, f)).read()) for f in ("attn_device.h", "attn_internal.h")]
    parts.append(_code_only(src[:src.index("__global__")]))
    m = re.search(r"__global__ void[^\n]*\b" + re.escape(kernel) + r"\(.*?\n}\n", src, re.S)
    parts.append(_code_only(m.group(0)) if m else "")
    parts += re.findall(r"template <int D> constexpr int \w+\(\) \{[^\n]*\}", src)
    return hashlib.sha1("\n".join(parts).encode()).hexdigest()[:12]


def traffic_for(workload, kernel):
    t = TRAFFIC.get((workload, kernel))
    return t["bytes"] if t and kernel in KERNEL_OF and t["fingerprint"] == kernel_fingerprint(KERNEL_OF[kernel]) else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def allowed_pairs(lq, lk, mask, window_left=-1):
    """Allowed (query, key) pairs of one head, summed over sequences (closed forms).

    Causal with diagonal delta (0 TL, Skv - Sq BR): row i sees keys up to i + delta, and with a
    sliding window W >= 0 only from i + delta - W on.
    """
    total = 0
    for sq, skv in zip(lq, lk):
        if mask == "none":
            total += sq * skv
            continue
        delta = skv - sq if mask == "causal_br" else 0

        def upto(n):  # sum over rows i < n of min(skv, max(0, i + delta + 1)): keys at or below the diagonal
            n = max(0, min(n, sq))
            lo = max(0, -delta)                 # first row with at least one key
            full = max(lo, min(n, skv - delta))  # rows i >= full see all skv keys
            t = 0
            if full > lo:
                a, b = lo + delta + 1, full - 1 + delta + 1
                t += (a + b) * (full - lo) // 2
            t += max(0, n - full) * skv
            return t
        total += upto(sq)
        if window_left >= 0:
            # keys before the window: min(skv, max(0, i + delta - W)) for each row = the same sum with
            # the diagonal moved down by W + 1
            d2 = delta - window_left - 1
            lo2 = max(0, -d2)
            full2 = max(lo2, min(sq, skv - d2))
            if full2 > lo2:
                a, b = lo2 + d2 + 1, full2 - 1 + d2 + 1
                total -= (a + b) * (full2 - lo2) // 2
            total -= max(0, sq - full2) * skv
    return total


def flop_per_pair(w):
    """Algorithmic FLOPs per allowed (query, key) pair and q-head, with Q/K head dim Dqk and V/O head
    dim Dv (both D for a symmetric head): forward QK^T + PV; backward S recompute, dV, dP, dQ, dK;
    per kernel: the dK/dV pass S, dP, dV, dK and the dQ pass its dQ product (its second S/dP recompute
    is executed but not credited)."""
    dqk, dv = w.d, w.d_v
    return {"fwd": 2.0 * (dqk + dv), "bwd": 6.0 * dqk + 4.0 * dv, "bwd_dkdv": 4.0 * (dqk + dv), "bwd_dq": 2.0 * dqk,
            "bwd_fused": 6.0 * dqk + 4.0 * dv}


def fused_backward(w):
    """Whether attn_bwd runs the dQ pass with the preprocess folded in (kernels up to head dim 256)."""
    return max(w.d, w.d_v) <= 256


def compulsory_bytes(w, x, nrows):
    """Bytes each kernel must move to or from HBM at least: its inputs read once, its outputs written once.

    forward   Q, K, V read; O, LSE written
    pre       O, dO, LSE read; D and LSE*log2(e) written (fp32)
    dK/dV     Q, dO, K, V, D, LSE*log2(e) read; dK, dV written
    dQ        Q, dO, K, V, D, LSE*log2(e) read; dQ written; with the preprocess folded in, O and LSE
              read and D, LSE*log2(e) written instead of read
    """
    el = 2  # bf16 / fp16
    nkv = sum(x["seqlens_kv"]) if w.packed else w.batch * w.skv
    q, o = nrows * w.hq * w.d * el, nrows * w.hq * w.d_v * el
    k, v = nkv * w.hkv * w.d * el, nkv * w.hkv * w.d_v * el
    row = nrows * w.hq * 4
    dq = q + o + k + v + q + (o + row + 2 * row if fused_backward(w) else 2 * row)
    acc = 2 * q  # the fp32 dQ buffer of the single-pass backward (4 bytes per element)
    return {"fwd": q + k + v + o + row, "bwd_pre": 2 * o + row + 2 * row,
            "bwd_dkdv": q + o + k + v + 2 * row + k + v, "bwd_dq": dq,
            # single-pass backward: preprocess also zeroes the buffer; the fused kernel writes it once at
            # least; the conversion reads it and writes dQ
            "bwd_pre_zero": 2 * o + row + 2 * row + acc, "bwd_fused": q + o + k + v + 2 * row + k + v + acc,
            "bwd_dq_convert": acc + q}


def kernel_roofline(w, x, nrows, pairs, kern_ms):
    """Roofline of each kernel: bound by HBM when its algorithmic FLOPs per compulsory byte are below
    the chip's balance point (peak FLOP/s over peak bytes/s), else by the matrix cores."""
    fp = flop_per_pair(w)
    nbytes = compulsory_bytes(w, x, nrows)
    balance = PEAK_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    out = {}
    for n, ms in kern_ms.items():
        flops = fp.get(n, 0) * pairs
        if flops / nbytes[n] < balance:
            ach = nbytes[n] / (ms * 1e-3) / 1e9
            out[n] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                      "bytes": nbytes[n]}
        else:
            ach = flops / (ms * 1e-3) / 1e12
            out[n] = {"bound": "mfma", "achieved": ach, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": ach / PEAK_TFLOPS}
        out[n]["flop_per_byte"] = flops / nbytes[n]
    return out


def cpu_baseline(w, x, budget_s=15.0, max_units=16):
    """Time the float64 oracle (forward + backward) on whole (sequence, kv-head) units."""
    import numpy as np
    from oracle import MASK_CAUSAL_BR, MASK_CAUSAL_TL, MASK_NONE, sdpa_bwd, sdpa_fwd
    mask = {"none": MASK_NONE, "causal_tl": MASK_CAUSAL_TL, "causal_br": MASK_CAUSAL_BR}[w.mask]
    f64 = {n: x[n].float().numpy().astype(np.float64) for n in ("q", "k", "v", "do")}
    cu_q = x["cu_seqlens_q"].numpy() if w.packed else None
    cu_k = x["cu_seqlens_kv"].numpy() if w.packed else None
    grp = w.hq // w.hkv
    done, flops, t_total, t_fwd = [], 0.0, 0.0, 0.0
    nseq = len(x["seqlens_q"])
    order = [(b, g) for b in range(nseq) for g in range(w.hkv)]
    for unit in order[:max_units]:
        b, g = unit
        t0 = time.perf_counter()
        sdpa_fwd(f64["q"], f64["k"], f64["v"], mask, w.scale, cu_q, cu_k, units=[unit], window_left=w.window_left)
        t_fwd += time.perf_counter() - t0
        sdpa_bwd(f64["q"], f64["k"], f64["v"], f64["do"], mask, w.scale, cu_q, cu_k, units=[unit],
                 window_left=w.window_left)
        t_total += time.perf_counter() - t0
        fp = flop_per_pair(w)
        flops += (fp["fwd"] + fp["bwd"]) * grp * allowed_pairs([x["seqlens_q"][b]], [x["seqlens_kv"][b]], w.mask,
                                                              w.window_left)
        done.append(unit)
        if t_total >= budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count()
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "fwd_s": round(t_fwd, 3), "bwd_s": round(t_total - t_fwd, 3),
            "sample": f"{len(done)} of {len(order)} (sequence, kv-head) units of {w.name} ({grp} q-heads each), "
                      f"forward+backward, numpy float64, {t_total:.1f} s; credited FLOPs as for the GPU value"}


def oracle_sample(w, x, rows=512):
    """The float64 oracle timed beside the GPU on a bounded slice of the workload: the last `rows` query rows
    of the last sequence's last q-head against all of that sequence's keys. Under a causal mask those rows are
    the bottom-right causal problem of themselves against every key (the slice keeps every allowed pair of the
    rows it holds), so the seconds per allowed pair are the oracle's own. Returns fwd/bwd seconds and rates."""
    import numpy as np
    from oracle import MASK_CAUSAL_BR, MASK_NONE, head_backward, head_forward
    b = len(x["seqlens_q"]) - 1
    h = w.hq - 1
    g = h // (w.hq // w.hkv)
    lq, lk = x["seqlens_q"][b], x["seqlens_kv"][b]
    r = min(rows, lq)
    if w.packed:
        q0, k0 = int(x["cu_seqlens_q"][b]), int(x["cu_seqlens_kv"][b])
        qs, ks = slice(q0 + lq - r, q0 + lq), slice(k0, k0 + lk)
        pick_q = lambda t: t[qs, h]  # noqa: E731
        pick_k = lambda t: t[ks, g]  # noqa: E731
    else:
        pick_q = lambda t: t[b, lq - r:, h]  # noqa: E731
        pick_k = lambda t: t[b, :, g]  # noqa: E731
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    qh, doh, kh, vh = f(pick_q(x["q"])), f(pick_q(x["do"])), f(pick_k(x["k"])), f(pick_k(x["v"]))
    mask = MASK_NONE if w.mask == "none" else MASK_CAUSAL_BR
    head_forward(qh, kh, vh, w.scale, mask, w.window_left)  # untimed: the first call starts the BLAS threads
    t0 = time.perf_counter()
    head_forward(qh, kh, vh, w.scale, mask, w.window_left)
    t1 = time.perf_counter()
    head_backward(qh, kh, vh, doh, w.scale, mask, w.window_left)
    t2 = time.perf_counter()
    pairs = allowed_pairs([r], [lk], "none" if w.mask == "none" else "causal_br", w.window_left)
    fp = flop_per_pair(w)
    return {"kind": "oracle", "sample": f"last {r} query rows of sequence {b}, q-head {h}, against its {lk} keys",
            "pairs": pairs, "fwd_s": round(t1 - t0, 4), "bwd_s": round(t2 - t1, 4),
            "fwd_tflops": round(fp["fwd"] * pairs / (t1 - t0) / 1e12, 5),
            "bwd_tflops": round(fp["bwd"] * pairs / (t2 - t1) / 1e12, 5)}


def atomic_supported(w):
    """Whether the single-pass backward (ATTN_FLAG_BWD_ATOMIC_DQ) is built for w's head dims."""
    return max(w.d, w.d_v) <= 128


def run(w, steps, warmup, want_events=True, flush_mall=False, atomic=False, exp_split=False, stored_ds=False):
    """Time `steps` steps of workload w. With flush_mall, a 512 MiB buffer is overwritten before every
    timed step (outside the per-kernel events), so no input is still in the 256 MB memory-side cache
    when a step starts; ms_step then includes the fill and only the per-kernel times are meaningful."""
    import torch
    import scaled_dot_product_02_amd as sd
    from scaled_dot_product_02_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    x = make_inputs(w)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    kw = dict(mask=w.mask, scale=w.scale, window_left=w.window_left)
    if w.packed:
        kw.update(cu_seqlens_q=x["cu_seqlens_q"].to(dev), cu_seqlens_kv=x["cu_seqlens_kv"].to(dev),
                  max_seqlen_q=x["max_seqlen_q"], max_seqlen_kv=x["max_seqlen_kv"])
    o = torch.empty(q.shape[:-1] + v.shape[-1:], dtype=q.dtype, device=dev)  # O has V's head dim
    p = sd.make_problem(q, k, v, o, w.mask, w.scale, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_kv"),
                        x["max_seqlen_q"], x["max_seqlen_kv"], w.window_left)
    lse_shape = (q.shape[0], q.shape[1]) if w.packed else (q.shape[0], q.shape[2], q.shape[1])
    lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsf = torch.empty(max(sd.attn_fwd_workspace_bytes(p), 256), dtype=torch.uint8, device=dev)
    wsb = torch.empty(sd.attn_bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)
    # the launches attn_bwd makes: the dQ pass with the preprocess folded in, then dK/dV (head dims up
    # to 256); preprocess, dK/dV, dQ for wider heads
    fused = fused_backward(w)
    names = ["fwd", "bwd_dq", "bwd_dkdv"] if fused else ["fwd", "bwd_pre", "bwd_dkdv", "bwd_dq"]
    seq = ["dq_preprocess", "dkdv"] if fused else ["preprocess", "dkdv", "dq"]
    if atomic:  # single-pass backward: preprocess (+ zeroing), the fused kernel, the dQ conversion
        names = ["fwd", "bwd_pre_zero", "bwd_fused", "bwd_dq_convert"]
        seq = ["preprocess", "dkdv", "dq"]
        p.flags = sd.FLAG_BWD_ATOMIC_DQ
        wsb = torch.empty(sd.attn_bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)
        kw["atomic_dq"] = True
    if stored_ds:  # stored-dS backward (head dims above 256): preprocess, dK/dV storing dS, dQ = dS K
        p.flags = sd.FLAG_BWD_STORED_DS
        wsb = torch.empty(sd.attn_bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)
        kw["stored_ds"] = True

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        sd.attn_fwd(q, k, v, out=o, lse=lse, workspace=wsf, exp_split=exp_split,
                    **{n: a for n, a in kw.items() if n not in ("atomic_dq", "stored_ds")})
        for i, pas in enumerate(seq):
            mark(1 + i)
            sd.attn_bwd(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=wsb, passes=(pas,), **kw)
        mark(1 + len(seq))

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if flush_mall else None
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)] if want_events else None
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            scratch.zero_()
        step(evs[i] if evs else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    kern_ms, kern_med, kern_min = {}, {}, {}
    if evs:
        for j, n in enumerate(names):
            per = sorted(e[j].elapsed_time(e[j + 1]) for e in evs)
            kern_ms[n] = sum(per) / steps
            kern_med[n] = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
            kern_min[n] = per[0]
    pairs = allowed_pairs(x["seqlens_q"], x["seqlens_kv"], w.mask, w.window_left) * w.hq
    return dict(x=x, ms_step=ms_step, kern_ms=kern_ms, kern_med=kern_med, kern_min=kern_min, pairs=pairs,
                nrows=p.total_q if w.packed else w.batch * w.sq)


def mfma_probe_measure(blocks=512, iters=150000, reps=5):
    """Sustained matrix-core rate as context for the fraction-of-peak figures: attn_mfma_probe runs
    independent bf16 32x32x16 MFMA chains from registers only (blocks x 4 waves, four chains per wave),
    timed with HIP events on the launch stream; the best of `reps` calls. Also reports the engine clock
    the probe read meanwhile (shader-clock ticks over 100 MHz reference ticks, mean over workgroups)."""
    import torch
    import scaled_dot_product_02_amd as sd
    sd.attn_mfma_probe(blocks, 1000)
    torch.cuda.synchronize()
    flops = blocks * 4 * iters * 4 * 32768
    rates, clocks = [], []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        _, ticks = sd.attn_mfma_probe(blocks, iters)
        e.record()
        torch.cuda.synchronize()
        rates.append(flops / (s.elapsed_time(e) * 1e-3) / 1e12)
        t = ticks.double().cpu()
        clocks.append(float((t[:, 0] / t[:, 1]).mean()) * 0.1)
    best = max(rates)
    return {"what": "attn_mfma_probe: independent bf16 32x32x16 MFMA chains from registers, no memory traffic",
            "tflops": round(best, 1), "frac_of_published_peak": round(best / PEAK_TFLOPS, 4),
            "clock_ghz": round(clocks[rates.index(best)], 3), "blocks": blocks, "iters": iters, "reps": reps}


def copy_rate(nbytes=1 << 30, reps=5):
    """Measured HBM ceiling as context for the HBM-bound kernels: a plain device-to-device copy of
    `nbytes` (torch's copy kernel), timed with HIP events on the current stream; bytes moved = read +
    write. Returns the best of `reps`."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (s.elapsed_time(e) * 1e-3) / 1e9)
    del src, dst
    return {"what": "device copy of 1 GiB (read + write counted)", "GB/s": round(best, 1),
            "frac_of_published_peak": round(best / PEAK_HBM_GBS, 4)}


def telemetry():
    """Engine clock, power and temperature as rocm-smi reports them (read-only; a child process).
    Returns the fields of the first card whose names mention a clock, power or temperature, or the
    error text when rocm-smi is unavailable."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showtemp", "--json"], capture_output=True,
                           text=True, timeout=30)
        cards = json.loads(r.stdout)
        card = next(v for k, v in cards.items() if k.startswith("card"))
        return {k: v for k, v in card.items() if re.search(r"sclk|mclk|power|temperature", k, re.I)}
    except Exception as e:  # telemetry is context only: never fail the run for it
        return {"error": f"{type(e).__name__}: {e}"[:200]}


def merge_measure(w, parts=2, steps=20, warmup=3):
    """attn_merge of `parts` forward results over w's query side (the ring step's combination).

    HBM-bound: per (row, head) it reads parts x (2*Dv + 4) bytes and writes 2*Dv + 4. Returns the
    average launch time (HIP events on the launch stream) and the achieved GB/s against 8 TB/s.
    """
    import torch
    import scaled_dot_product_02_amd as sd
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(7)
    shape = (w.batch, w.sq, w.hq, w.d_v)
    o_parts = [torch.randn(shape, generator=g).to(w.torch_dtype).to(dev) for _ in range(parts)]
    lse_parts = [(torch.randn(w.batch, w.hq, w.sq, generator=g) * 4).to(dev) for _ in range(parts)]
    out = torch.empty(shape, dtype=w.torch_dtype, device=dev)
    lse = torch.empty(w.batch, w.hq, w.sq, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        sd.attn_merge(o_parts, lse_parts, out=out, lse=lse)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        sd.attn_merge(o_parts, lse_parts, out=out, lse=lse)
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    nbytes = w.batch * w.sq * w.hq * (parts + 1) * (2 * w.d_v + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"what": f"attn_merge of {parts} forward results, query side of {w.name}", "parts": parts,
            "us": round(ms * 1e3, 2), "bytes": nbytes, "GB/s": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def case_measure(w, steps, warmup, oracle_rows=512):
    """One named case: forward, backward and combined time and TFLOP/s (algorithmic FLOPs over the exact
    allowed pairs) with the per-kernel launch times, the compulsory-byte rates (GB/s against the HBM peak;
    the measure that matters for latency-bound tiny cases) and the oracle timed on a bounded slice."""
    r = run(w, steps, warmup)
    fp = flop_per_pair(w)
    km = r["kern_ms"]
    fwd_ms = km["fwd"]
    bwd_ms = sum(t for n, t in km.items() if n != "fwd")
    pairs = r["pairs"]
    f_fwd, f_bwd = fp["fwd"] * pairs, fp["bwd"] * pairs
    nb = compulsory_bytes(w, r["x"], r["nrows"])
    bwd_bytes = sum(nb[n] for n in km if n != "fwd")
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12  # noqa: E731
    out = {"config": w.note, "steps": steps, "warmup": warmup, "allowed_pairs": pairs,
           "ms_per_step": round(r["ms_step"], 4),
           "fwd": {"ms": round(fwd_ms, 4), "us": round(fwd_ms * 1e3, 2), "tflops": round(tf(f_fwd, fwd_ms), 2),
                   "frac_of_peak": round(tf(f_fwd, fwd_ms) / PEAK_TFLOPS, 4),
                   "GB/s": round(nb["fwd"] / (fwd_ms * 1e-3) / 1e9, 1)},
           "bwd": {"ms": round(bwd_ms, 4), "us": round(bwd_ms * 1e3, 2), "tflops": round(tf(f_bwd, bwd_ms), 2),
                   "frac_of_peak": round(tf(f_bwd, bwd_ms) / PEAK_TFLOPS, 4),
                   "GB/s": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9, 1)},
           "fwd_bwd": {"tflops": round(tf(f_fwd + f_bwd, fwd_ms + bwd_ms), 2),
                       "frac_of_peak": round(tf(f_fwd + f_bwd, fwd_ms + bwd_ms) / PEAK_TFLOPS, 4)},
           "kernel_ms": {n: round(t, 4) for n, t in km.items()},
           "kernel_ms_min": {n: round(t, 4) for n, t in r["kern_min"].items()}}
    if w.packed:
        out["seqlens"] = list(map(int, r["x"]["seqlens_q"]))
    if oracle_rows:
        out["oracle"] = oracle_sample(w, r["x"], oracle_rows)
    return out


def graph_step_us(w, replays=50):
    """Device time of one whole step (forward + the backward launches attn_bwd makes) captured once in a HIP
    graph and replayed back to back: the figure that matters for a latency-bound case, where the HIP events
    around each eager launch also hold the host-side launch path. Every buffer is allocated before capture
    (the library allocates nothing)."""
    import torch
    import scaled_dot_product_02_amd as sd
    from scaled_dot_product_02_amd.workloads import make_inputs
    dev = torch.device("cuda:0")
    x = make_inputs(w)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    kw = dict(mask=w.mask, scale=w.scale, window_left=w.window_left)
    if w.packed:
        kw.update(cu_seqlens_q=x["cu_seqlens_q"].to(dev), cu_seqlens_kv=x["cu_seqlens_kv"].to(dev),
                  max_seqlen_q=x["max_seqlen_q"], max_seqlen_kv=x["max_seqlen_kv"])
    o = torch.empty(q.shape[:-1] + v.shape[-1:], dtype=q.dtype, device=dev)
    p = sd.make_problem(q, k, v, o, w.mask, w.scale, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_kv"),
                        x["max_seqlen_q"], x["max_seqlen_kv"], w.window_left)
    lse_shape = (q.shape[0], q.shape[1]) if w.packed else (q.shape[0], q.shape[2], q.shape[1])
    lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsf = torch.empty(max(sd.attn_fwd_workspace_bytes(p), 256), dtype=torch.uint8, device=dev)
    wsb = torch.empty(sd.attn_bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)

    def step():
        sd.attn_fwd(q, k, v, out=o, lse=lse, workspace=wsf, **kw)
        sd.attn_bwd(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=wsb, **kw)

    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1e3 / replays, 2)


def single_pass_measure(w, steps, warmup):
    """The same workload with the single-pass backward (ATTN_FLAG_BWD_ATOMIC_DQ): backward ms, TFLOP/s
    (the same credited FLOPs) and per-kernel times, the step with the default forward."""
    r = run(w, steps, warmup, atomic=True)
    fp = flop_per_pair(w)
    km = r["kern_ms"]
    bwd_ms = sum(t for n, t in km.items() if n != "fwd")
    f_fwd, f_bwd = fp["fwd"] * r["pairs"], fp["bwd"] * r["pairs"]
    kroof = kernel_roofline(w, r["x"], r["nrows"], r["pairs"], km)
    return {"what": "single-pass backward (ATTN_FLAG_BWD_ATOMIC_DQ): preprocess with the zeroing of the fp32 dQ "
                    "buffer, the dK/dV kernel that also adds dQ with fp32 atomics, the dQ conversion",
            "bwd": {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
                    "frac_of_peak": round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_TFLOPS, 4)},
            "fwd_bwd": {"tflops": round((f_fwd + f_bwd) / ((km["fwd"] + bwd_ms) * 1e-3) / 1e12, 2),
                        "ms_per_step": round(r["ms_step"], 4)},
            "kernel_ms": {n: round(t, 4) for n, t in km.items()},
            "kernel_ms_min": {n: round(t, 4) for n, t in r["kern_min"].items()},
            "kernel_roofline": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in e.items()}
                                for n, e in kroof.items()}}


def stored_ds_measure(w, steps, warmup):
    """The same workload with the stored-dS backward (ATTN_FLAG_BWD_STORED_DS, head dims above 256): the
    dK/dV pass also stores dS and the dQ pass is the product dS K. Backward ms and TFLOP/s (the same
    credited FLOPs), per-kernel times, the dQ product's rate at its 2*D FLOP per pair, and the dS bytes
    it stores and reads back (dtype, one per allowed pair and q-head)."""
    r = run(w, steps, warmup, stored_ds=True)
    fp = flop_per_pair(w)
    km = r["kern_ms"]
    bwd_ms = sum(t for n, t in km.items() if n != "fwd")
    f_fwd, f_bwd = fp["fwd"] * r["pairs"], fp["bwd"] * r["pairs"]
    f_dq = 2 * w.d * r["pairs"]
    return {"what": "stored-dS backward (ATTN_FLAG_BWD_STORED_DS): preprocess, the dK/dV pass that also stores dS, "
                    "dQ = scale * dS K",
            "bwd": {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
                    "frac_of_peak": round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_TFLOPS, 4)},
            "fwd_bwd": {"tflops": round((f_fwd + f_bwd) / ((km["fwd"] + bwd_ms) * 1e-3) / 1e12, 2),
                        "frac_of_peak": round((f_fwd + f_bwd) / ((km["fwd"] + bwd_ms) * 1e-3) / 1e12 / PEAK_TFLOPS, 4),
                        "ms_per_step": round(r["ms_step"], 4)},
            "dq_product": {"tflops": round(f_dq / (km["bwd_dq"] * 1e-3) / 1e12, 2),
                           "frac_of_peak": round(f_dq / (km["bwd_dq"] * 1e-3) / 1e12 / PEAK_TFLOPS, 4),
                           "ds_bytes": int(2 * r["pairs"])},
            "kernel_ms": {n: round(t, 4) for n, t in km.items()},
            "kernel_ms_min": {n: round(t, 4) for n, t in r["kern_min"].items()}}


def exp_split_measure(w, steps, warmup):
    """The same workload with the forward's exp split (ATTN_FLAG_FWD_EXP_SPLIT: a quarter of the exponentials
    on interior tiles by a VALU polynomial), the default backward: forward ms and TFLOP/s."""
    r = run(w, steps, warmup, exp_split=True)
    fp = flop_per_pair(w)
    km = r["kern_ms"]
    f_fwd = fp["fwd"] * r["pairs"]
    return {"what": "forward with ATTN_FLAG_FWD_EXP_SPLIT (one in four exponentials of each lane on interior tiles "
                    "by a degree-5 polynomial on the VALU), default backward",
            "fwd": {"ms": round(km["fwd"], 4), "tflops": round(f_fwd / (km["fwd"] * 1e-3) / 1e12, 2),
                    "frac_of_peak": round(f_fwd / (km["fwd"] * 1e-3) / 1e12 / PEAK_TFLOPS, 4)},
            "ms_per_step": round(r["ms_step"], 4)}


# The named cases timed in every default run besides the headline (dense_d128): the tiny case, the packed
# GQA batch, the D=512 layer and the two single-rank context-parallel shares.
CASES = ("tiny", "thd_d128", "dense_d512", "cp_share_d256", "cp_share_d512")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_d128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-pass-only", action="store_true",
                    help="time only the workload with the single-pass backward and print its line")
    ap.add_argument("--stored-ds-only", action="store_true",
                    help="time only the workload with the stored-dS backward (heads above 256) and print its line")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other named cases and the informational merge and short-sequence lines")
    ap.add_argument("--merge-only", action="store_true",
                    help="only time attn_merge of two forward results (dense_d128 query side) and print its line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (calibrates HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: this engine runs on one GPU; --gpus {args.gpus} is not supported (no multi-GPU path "
              "is built: sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    import scaled_dot_product_02_amd as sd
    from scaled_dot_product_02_amd.workloads import WORKLOADS

    if not os.path.exists(sd.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    w = WORKLOADS[args.workload]
    if args.merge_only:
        print(json.dumps({"merge": merge_measure(w, steps=args.steps, warmup=args.warmup)}), flush=True)
        return
    log(f"workload {w.name}: {w.note}")
    if args.single_pass_only:
        print(json.dumps({"workload": w.name, "single_pass": single_pass_measure(w, args.steps, args.warmup)}),
              flush=True)
        return
    if args.stored_ds_only:
        print(json.dumps({"workload": w.name, "stored_ds": stored_ds_measure(w, args.steps, args.warmup)}), flush=True)
        return
    tele_before = telemetry() if not args.no_extra else None
    r = run(w, args.steps, args.warmup)
    tele_after = telemetry() if not args.no_extra else None
    d, pairs = w.d, r["pairs"]
    fp = flop_per_pair(w)
    f_fwd, f_bwd = fp["fwd"] * pairs, fp["bwd"] * pairs
    value = (f_fwd + f_bwd) / (r["ms_step"] * 1e-3) / 1e12
    km = r["kern_ms"]
    kroof = kernel_roofline(w, r["x"], r["nrows"], pairs, km)
    dom = max(km, key=km.get)
    roof = {kk: kroof[dom][kk] for kk in ("bound", "achieved", "peak", "unit", "frac")}
    roof["kernel"] = dom
    roof["avg_launch_ms"] = km[dom]
    roof["traffic"] = traffic_for(w.name, dom)
    fwd_ms = km["fwd"]
    bwd_ms = sum(t for n, t in km.items() if n != "fwd")
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch if not w.packed else len(r["x"]["seqlens_q"]),
                   "heads_q": w.hq, "heads_kv": w.hkv, "seq_q": w.sq or r["x"]["max_seqlen_q"],
                   "seq_kv": w.skv or r["x"]["max_seqlen_kv"], "head_dim": d, "head_dim_v": w.d_v,
                   "mask": w.mask,
                   "layout": "thd" if w.packed else "bshd", "window_left": w.window_left, "allowed_pairs": pairs,
                   "seed": w.seed, **({"seqlens": list(map(int, r["x"]["seqlens_q"])), "total_q": int(r["nrows"])}
                                      if w.packed else {})},
        "frac_of_peak": round(value / PEAK_TFLOPS, 4),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                "frac_of_peak": round(f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
                "frac_of_peak": round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_TFLOPS, 4)},
        "kernel_ms": {n: round(t, 4) for n, t in km.items()},
        "kernel_ms_median": {n: round(t, 4) for n, t in r["kern_med"].items()},
        "kernel_ms_min": {n: round(t, 4) for n, t in r["kern_min"].items()},
        "roofline": {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in roof.items()},
        "kernel_roofline": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in e.items()}
                            for n, e in kroof.items()},
    }
    if not args.no_extra:
        out["telemetry"] = {"before": tele_before, "after": tele_after}
        out["sustained_mfma"] = mfma_probe_measure()
        out["hbm_copy"] = copy_rate()
    if not args.no_extra and atomic_supported(w):
        log("single-pass backward on the same workload")
        out["single_pass"] = single_pass_measure(w, args.steps, args.warmup)
        if max(w.d, w.d_v) <= 256:  # the exp split is built for head dims up to 256
            out["exp_split"] = exp_split_measure(w, max(5, args.steps // 2), 3)
    if not args.no_extra and w.name == "dense_d128":
        out["cases"] = {}
        for name in CASES:
            wc = WORKLOADS[name]
            log(f"case {name}: {wc.note}")
            out["cases"][name] = case_measure(wc, max(5, args.steps // 2), 3)
            if name == "tiny":  # latency-bound: the device time of a whole step, launched as one graph
                out["cases"][name]["graph_us_per_step"] = graph_step_us(wc)
            if atomic_supported(wc):
                out["cases"][name]["single_pass"] = single_pass_measure(wc, max(5, args.steps // 2), 3)
            if max(wc.d, wc.d_v) > 256:  # the stored-dS backward serves the heads above 256
                out["cases"][name]["stored_ds"] = stored_ds_measure(wc, max(5, args.steps // 2), 3)
        out["extra"] = {"merge": merge_measure(w)}
        w3 = WORKLOADS["short_d128"]
        r3 = run(w3, max(5, args.steps // 3), 3)
        kr3 = kernel_roofline(w3, r3["x"], r3["nrows"], r3["pairs"], r3["kern_ms"])
        out["extra"]["short_d128"] = {
            "ms_per_step": round(r3["ms_step"], 4), "kernel_ms": {n: round(t, 4) for n, t in r3["kern_ms"].items()},
            "kernel_roofline": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in e.items()}
                                for n, e in kr3.items()}}
        # the same HBM-bound workload with the memory-side cache overwritten before every step
        r4 = run(w3, max(5, args.steps // 3), 3, flush_mall=True)
        kr4 = kernel_roofline(w3, r4["x"], r4["nrows"], r4["pairs"], r4["kern_ms"])
        out["extra"]["short_d128_mall_flushed"] = {
            "kernel_ms": {n: round(t, 4) for n, t in r4["kern_ms"].items()},
            "kernel_hbm_frac": {n: round(e["frac"], 4) for n, e in kr4.items()}}
    if not args.no_cpu_baseline:
        log("timing the float64 CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(w, r["x"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
