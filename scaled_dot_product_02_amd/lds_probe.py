"""LDS bank and pass structure of gfx950, measured with attn_lds_probe under the bank-conflict counter.

The attention kernels stage tiles in LDS with their 16-byte chunks permuted per row (sw_key in
csrc/attn_device.h) and read them back as matrix-core operands with ds_read_b128 (16 bytes per lane)
and ds_read_b64_tr_b16 (the 8-byte transpose read). Whether a read takes extra cycles depends on how the
LDS serves it: the bank of an address, and which lanes share a cycle. This module measures both, and the
kernels' own read patterns under the swizzle keys, with single-wave dispatches of attn_lds_probe:

  run <manifest>                 issue every test in order (one dispatch each) and write the manifest
  summarize <counter csv> <manifest>
                                 read rocprofv3's per-dispatch SQ_LDS_BANK_CONFLICT and print the results

The run is meant to execute under
  rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS -d <dir> -o run --output-format csv -- \\
      python3 -m scaled_dot_product_02_amd.lds_probe run <dir>/manifest.txt
(the counter is read per dispatch; this module only issues the reads). The fitted model, predicted(),
is what the swizzle keys are checked against on the CPU.
"""
import csv
import os
import re
import sys

ITERS = 64  # 8 * ITERS reads per dispatch
HERE = os.path.dirname(os.path.abspath(__file__))


# ---- the model the measurements fit (see summarize) ----
def b128_pass(lane):
    """ds_read_b128: 4 passes of 16 lanes, picked by lane bit 5 and the parity of lane bits 2..4."""
    return (lane >> 5) & 1, ((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1


def b64_pass(lane):
    """8-byte reads (ds_read_b64, ds_read_b64_tr_b16): 2 passes of 32 consecutive lanes."""
    return lane >> 5


def predicted(addrs, kind):
    """Extra cycles of one wave-wide read: 64 banks of 4 bytes, bank = (address / 4) % 64; per pass,
    every additional distinct dword address on one bank costs a cycle (equal addresses are one access)."""
    width = 16 if kind == "b128" else 8
    passes = {}
    for lane, a in enumerate(addrs):
        if a < 0:
            continue
        p = b128_pass(lane) if kind == "b128" else b64_pass(lane)
        for i in range(width // 4):
            dw = a // 4 + i
            passes.setdefault(p, {}).setdefault(dw % 64, set()).add(dw)
    return sum(max(len(s) for s in banks.values()) - 1 for banks in passes.values())


# ---- swizzle keys ----
def current_keys():
    """The two sw_key branches of csrc/attn_device.h (D >= 128, D = 64) as Python functions of the row.
    The C expressions use only &, |, ^, <<, >> on a non-negative int, which Python evaluates the same."""
    src = open(os.path.join(HERE, "csrc", "attn_device.h")).read()
    m = re.search(r"int sw_key\(int r\) \{\s*if constexpr \(D >= 128\) return (.*?);\s*else return (.*?);\s*\}", src, re.S)
    if not m:
        raise RuntimeError("sw_key not found in attn_device.h")
    wide, narrow = m.group(1), m.group(2)
    return (lambda r, e=wide: eval(e, {}, {"r": r})), (lambda r, e=narrow: eval(e, {}, {"r": r}))


def earlier_key_wide(r):  # key bits (3 2 1 0) = (r1, r0, r2, r3)
    return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1)


def earlier_key_narrow(r):  # row XOR, D = 64
    return r & 7


# ---- the kernels' read patterns (byte addresses of one wave-wide read, tile at LDS offset 0) ----
# Operand rows for the 16x16x32 products (both backward passes): lane (G = lane/16, r = lane%16) reads
# row 16kb + r, logical chunk 4kk + G.
def rows_16x16(D, key, kk, kb):
    return [2 * ((l & 15) * D + 16 * kb * D + ((32 * kk) ^ ((key(l & 15) ^ (l >> 4)) << 3))) for l in range(64)]


# Operand rows for the 32x32x16 products (forward): lane reads row 32kb + lane%32, chunk 2kk + lane/32.
def rows_32x32(D, key, kk, kb):
    return [((2 * ((l & 31) * D + ((key(l & 31) ^ (l >> 5)) << 3))) ^ (32 * kk)) + 64 * kb * D for l in range(64)]


# Transpose reads for the 16x16x32 products: lane (G, rr = lane/4 % 4, cc = lane%4) reads row 4G + rr
# (+16 for the second read of a pair), chunk 2dt + cc/2, 8-byte half cc%2.
def transpose_16x16(D, key, dt, hi):
    out = []
    for l in range(64):
        G, rr, cc = l >> 4, (l >> 2) & 3, l & 3
        row = (4 * G + rr) * D + 4 * (cc & 1)
        x = (key(4 * G + rr) ^ (cc >> 1)) << 3
        out.append(2 * (row + ((16 * dt) ^ x) + hi * 16 * D))
    return out


# Transpose reads for the 32x32x16 products (the forward's V): lane (hh = lane/32, G, rr, c4 = lane%4)
# reads key row 8cp + 4hh + rr (+16), chunk 4dt + 2(G%2) + c4/2, half c4%2.
def transpose_32x32(D, key, dt, cp):
    out = []
    for l in range(64):
        hh, G, rr, c4 = l >> 5, l >> 4, (l >> 2) & 3, l & 3
        row = (4 * hh + rr) * D + 4 * (c4 & 1)
        x = (key(8 * cp + 4 * hh + rr) ^ (2 * (G & 1) + (c4 >> 1))) << 3
        out.append((2 * (row + 8 * D * cp + x)) ^ (64 * dt))
    return out


def kernel_patterns(D, key):
    """(name, kind, list of wave-wide address lists) for the four read shapes of the kernels at head dim D."""
    return [
        ("16x16x32 operand rows", "b128", [rows_16x16(D, key, kk, kb) for kk in range(D // 32) for kb in range(2)]),
        ("32x32x16 operand rows", "b128", [rows_32x32(D, key, kk, kb) for kk in range(D // 16) for kb in range(2)]),
        ("16x16x32 transpose reads", "b64_tr_b16", [transpose_16x16(D, key, dt, hi) for dt in range(D // 16) for hi in range(2)]),
        ("32x32x16 transpose reads", "b64_tr_b16", [transpose_32x32(D, key, dt, cp) for dt in range(D // 32) for cp in range(2)]),
    ]


def tests():
    """Every dispatch of the run, in order: (kind, test, p1, p2, lane addresses)."""
    out = []
    for kind, step in (("b128", 16), ("b64", 8)):
        for y in range(step, 16384, step):  # bank function: lane 0 at 0, lane 1 at y
            t = [-1] * 64
            t[0], t[1] = 0, y
            out.append((kind, "bank", 0, y, t))
        for b in range(1, 64):  # passes: lane 0 at 0, lane b at 256 (same banks, other address)
            t = [-1] * 64
            t[0], t[b] = 0, 256
            out.append((kind, "pass", b, 256, t))
    out.append(("b128", "linear", 0, 0, [16 * l for l in range(64)]))
    out.append(("b64", "linear", 0, 0, [8 * l for l in range(64)]))
    out.append(("b64_tr_b16", "linear", 0, 0, [8 * l for l in range(64)]))
    out.append(("b128", "8 rows at one chunk", 0, 0, [256 * (l & 7) for l in range(64)]))
    wide, narrow = current_keys()
    for D in (64, 128):
        for kname, key in (("earlier", earlier_key_wide if D >= 128 else earlier_key_narrow),
                           ("current", wide if D >= 128 else narrow)):
            for name, kind, reads in kernel_patterns(D, key):
                for i, addrs in enumerate(reads):
                    out.append((kind, f"D{D} {kname} key: {name}", i, 0, addrs))
    return out


def run(manifest):
    import torch
    from ._binding import attn_lds_probe
    out = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    ts = tests()
    with open(manifest, "w") as f:
        for i, (kind, name, p1, p2, addrs) in enumerate(ts):
            attn_lds_probe(kind, addrs, ITERS, out)
            torch.cuda.synchronize()
            f.write(f"{i}\t{kind}\t{name}\t{p1}\t{p2}\n")
            if i % 500 == 0:
                print(f"dispatch {i} of {len(ts)}", flush=True)
    print(f"done: {len(ts)} dispatches", flush=True)


def summarize(counter_csv, manifest):
    rows = {}
    for r in csv.DictReader(open(counter_csv)):
        if "lds_probe_kernel" in r["Kernel_Name"] and r["Counter_Name"] == "SQ_LDS_BANK_CONFLICT":
            rows[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    conf = [rows[d] / (8 * ITERS) for d in sorted(rows)]
    man = [line.rstrip("\n").split("\t") for line in open(manifest)]
    if len(man) != len(conf):
        raise SystemExit(f"{len(man)} tests in the manifest, {len(conf)} probe dispatches in the counters")
    ts = tests()
    for kind in ("b128", "b64"):
        hits = [int(m[4]) for m, c in zip(man, conf) if m[1] == kind and m[2] == "bank" and c > 0.5]
        n = sum(1 for m in man if m[1] == kind and m[2] == "bank")
        print(f"{kind} bank test ({n} addresses y in (0, 16384), lane 0 at 0, lane 1 at y): conflict at "
              f"{len(hits)} of them; all multiples of 256: {all(y % 256 == 0 for y in hits)}; "
              f"every multiple of 256 conflicts: {len(hits) == 16384 // 256 - 1}")
        lanes = [int(m[3]) for m, c in zip(man, conf) if m[1] == kind and m[2] == "pass" and c > 0.5]
        print(f"{kind} pass test (lane 0 at 0, lane b at 256): lanes sharing lane 0's pass: {lanes}")
    print("| pattern | read | measured extra cycles per read (mean over the pattern's reads) | model |")
    print("|---|---|---|---|")
    groups = {}
    for (kind, name, p1, p2, addrs), m, c in zip(ts, man, conf):
        if m[2] in ("bank", "pass"):
            continue
        g = groups.setdefault(name, [kind, [], []])
        g[1].append(c)
        g[2].append(predicted(addrs, kind))
    for name, (kind, meas, pred) in groups.items():
        print(f"| {name} | {kind} | {sum(meas) / len(meas):.2f} | {sum(pred) / len(pred):.2f} |")


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "run":
        run(sys.argv[2])
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
