"""Benchmark: one step = one causal GQA prefill (B=1, Hq=64, Hkv=8, N=8192,
d=128, bf16, the 70B-layer shape), one paged GQA decode (64 sequences,
lengths ~ U{512..32768}, Hq=64, Hkv=8, d=128, 16-token pages in a seeded
random permutation), one paged chunked prefill (8 sequences, the last
1024 tokens of caches of U{2048..16384} tokens as queries, same heads) and
one causal sliding-window prefill (the prefill's inputs, each query seeing
its last 4097 keys), one causal block-sparse prefill (the prefill's
inputs, each 128-query block attending to the first key block and the 16
key blocks ending at its own), one backward of the causal prefill (its
inputs, O and LSE, and a seeded N(0,1) dO), one backward of the block-sparse
prefill (same mask, its O and LSE, the same dO) and one FP8 causal prefill (the
prefill's inputs block-quantized to E4M3 by fa_quantize_fp8 before timing),
all through the C ABI on one GPU.

Prints one JSON line. `value` is the prefill's attention TFLOP/s (FLOPs =
4*B*Hq*Nq*Nk*d, halved for causal); the decode's HBM GB/s (algorithmic bytes:
K and V of every cached token, q, O, LSE, the used block-table entries and
seq_lens) is reported under "decode", the chunked prefill's TFLOP/s (4*d*Hq
per visible query-key pair) under "paged_prefill", the windowed and
block-sparse prefills' (same count) under "window" and "block_sparse", the
backward's TFLOP/s (2.5x the forward's FLOPs, the usual count for the five
products of a backward) under "backward" and "backward_block_sparse", the FP8
prefill's TFLOP/s against
the FP8 MFMA peak under "fp8". The K timed steps run as K passes of each
kernel back to back (prefill, windowed prefill, block-sparse prefill, FP8
prefill, backward, block-sparse backward, decode, chunked prefill, then the
cold-cache prefill and the two other prefill shapes), so
each kernel is timed in its steady state. Each kernel's time is the mean
(median and min also given) of HIP events recorded around it on its launch
stream. Inputs are generated and copied to device memory before timing
starts; warm-ups run before the timed region.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (% bf16 MFMA peak); paged decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense FP8 MFMA: twice the bf16 rate

PREFILL = dict(B=1, Hq=64, Hkv=8, N=8192, d=128, causal=True, seed=1003, sigma=1.0)
# The other two prefill shapes of the workload set: causal MHA B=4 Hq=16
# N=2048 (seed 1002) and the 64K-token causal GQA 32/8 with N(0, 0.5^2)
# inputs (seed 1004), each timed as its own leg with the same kernel.
CONFIG2 = dict(B=4, Hq=16, Hkv=16, N=2048, d=128, causal=True, seed=1002, sigma=1.0)
CONFIG4 = dict(B=1, Hq=32, Hkv=8, N=65536, d=128, causal=True, seed=1004, sigma=0.5)
FLUSH_BYTES = 1 << 30   # read-modify-write between cold prefill passes: evicts L2 and the 256 MB MALL
DECODE = dict(B=64, Hq=64, Hkv=8, d=128, page=16, len_lo=512, len_hi=32768, max_pages=2048, seed=1005)
# Chunked prefill over the paged cache: each sequence's last `chunk` tokens
# are queries against its whole cache.
PAGED = dict(B=8, Hq=64, Hkv=8, d=128, page=16, chunk=1024, len_lo=2048, len_hi=16384, max_pages=1024,
             seed=1006, causal=True)
# Sliding window over the prefill's inputs: query i sees keys [i - left, i].
WINDOW = dict(left=4096, causal=True)
# Block-sparse mask over the prefill's inputs (128 x 128 blocks): local + global.
SPARSE = dict(local=16, n_global=1, causal=True)
COPY_CALIB_BYTES = 1 << 30


def prefill_flops(B, Hq, Nq, Nk, d, causal):
    f = 4.0 * B * Hq * Nq * Nk * d
    return f / 2 if causal else f


def prefill_min_bytes(B, Hq, Hkv, Nq, Nk, d):
    return 2 * (B * Hq * Nq * d * 2 + B * Hkv * Nk * d * 2) + 4 * B * Hq * Nq


def paged_prefill_flops(seq_lens, q_lens, Hq, d, causal):
    """4*d flop per visible (query, key) pair and query head; a chunk of n
    queries at the end of L tokens sees n*(L-n) + n*(n+1)/2 pairs causally."""
    f = 0.0
    for L, n in zip(np.asarray(seq_lens, dtype=np.int64), np.asarray(q_lens, dtype=np.int64)):
        pairs = n * (L - n) + n * (n + 1) // 2 if causal else n * L
        f += 4.0 * Hq * d * float(pairs)
    return f


def window_flops(B, Hq, Nq, Nk, d, left, causal):
    """4*d flop per visible (query, key) pair and query head; query i sits at
    key position p = i + Nk - Nq and sees keys [max(0, p - left), p] causally
    (up to Nk - 1 without the right bound)."""
    p = np.arange(Nq, dtype=np.int64) + (Nk - Nq)
    lo = np.maximum(0, p - left) if left >= 0 else np.zeros_like(p)
    hi = np.minimum(p, Nk - 1) if causal else np.full_like(p, Nk - 1)
    return 4.0 * B * Hq * d * float(np.maximum(0, hi - lo + 1).sum())


def block_sparse_flops(B, Hq, Nq, Nk, d, mask, causal, block=128):
    """4*d flop per visible (query, key) pair and query head under a
    [n_qblocks, n_kblocks] block mask shared by all heads (and the causal
    mask, bottom-right aligned)."""
    pairs = 0
    for qb in range(mask.shape[0]):
        i = np.arange(qb * block, min(Nq, qb * block + block), dtype=np.int64)
        for kb in np.nonzero(mask[qb])[0]:
            j0, j1 = kb * block, min(Nk, kb * block + block)
            if causal:
                hi = np.minimum(i + (Nk - Nq), j1 - 1)
                pairs += int(np.maximum(0, hi - j0 + 1).sum())
            else:
                pairs += i.size * (j1 - j0)
    return 4.0 * B * Hq * d * float(pairs)


def decode_bytes(seq_lens, B, Hq, Hkv, d, page=16):
    L = np.asarray(seq_lens, dtype=np.int64)
    kv = int(L.sum()) * Hkv * d * 2 * 2
    table = int(((L + page - 1) // page).sum()) * 4
    return kv + B * Hq * d * 2 * 2 + B * Hq * 4 + table + B * 4


def decode_overhead_bytes(seq_lens, B, Hq, Hkv, d, max_seq_len, page=16):
    """HBM bytes the decode moves beyond the algorithmic ones: the slots past
    each sequence's end in its last page (K and V are read page by page), and
    the split-K partials (fp32 row + LSE per split of a sequence with several
    splits) written by the split kernel and read back by the combine. The
    split length follows the library's launch rule: 4096 tokens at d = 128
    when B * Hkv * ceil(G/16) * ceil(max_seq_len/4096) >= 2048, else 2048."""
    L = np.asarray(seq_lens, dtype=np.int64)
    tail = int((((L + page - 1) // page) * page - L).sum()) * Hkv * d * 2 * 2
    n_hgrp = (Hq // Hkv + 15) // 16
    long_split = d == 128 and B * Hkv * n_hgrp * -(-max_seq_len // 4096) >= 2048
    split = 4096 if long_split else 2048
    n = (L + split - 1) // split
    part = int(n[n > 1].sum()) * Hq * (d * 4 + 4) * 2
    return {"tail_slots": tail, "split_partials": part, "split_tokens": split}


def decode_flops(seq_lens, Hq, d):
    return 4.0 * Hq * d * float(np.asarray(seq_lens, dtype=np.int64).sum())


def source_hash(names):
    """Hash of kernel sources with comments and layout whitespace removed, so
    that the counter summary stays attached to the code it measured and only
    a change of the code itself detaches it."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_attention_03_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on different kernel source."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
        e = t[kernel_key]
        return e["bytes_per_launch"] if e.get("source_hash") == src_hash else None
    except (OSError, KeyError, ValueError):
        return None


def load_traffic_sum(kernel_keys, src_hash):
    """Summed HBM bytes per call of several kernels run as one step, or None
    if any of them has no current summary."""
    parts = [load_traffic(k, src_hash) for k in kernel_keys]
    return None if any(x is None for x in parts) else sum(parts)


def pmc_summary(fetch_csv, write_csv, out_path):
    """Per-launch HBM bytes of each kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by what the
    same counter reads for the plain device copy of COPY_CALIB_BYTES made by
    --copy-calib in the same run (factor = known bytes / counted bytes)."""
    import csv
    import collections

    def per_kernel(path, counter):
        acc = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc[(r["Kernel_Name"], r["Dispatch_Id"])].append(float(r["Counter_Value"]))
        by_name = collections.defaultdict(list)
        for (name, _), vals in acc.items():
            by_name[name].append(sum(vals))
        return by_name

    fetch_all = per_kernel(fetch_csv, "FETCH_SIZE")
    write_all = per_kernel(write_csv, "WRITE_SIZE")
    fetch = {k: sum(v) / len(v) for k, v in fetch_all.items()}
    write = {k: sum(v) / len(v) for k, v in write_all.items()}

    def calib(d_all):
        copies = [max(v) for k, v in d_all.items() if "copy" in k.lower() and max(v) > 0.25 * COPY_CALIB_BYTES / 1024]
        if not copies:
            raise SystemExit("no calibration copy kernel found in the counter CSV")
        return COPY_CALIB_BYTES / (max(copies) * 1024.0)

    fr, wr = calib(fetch_all), calib(write_all)
    keys = {"fa_fwd_kernel<128, true, false, false, false>": ("fa_fwd_kernel<128,true>", "fa_prefill.hip"),
            "fa_fwd_kernel<128, true, true, false, false>": ("fa_fwd_kernel<128,true,paged>", "fa_prefill.hip"),
            "fa_fwd_kernel<128, true, false, true, false>": ("fa_fwd_kernel<128,true,window>", "fa_prefill.hip"),
            "fa_fwd_kernel<128, true, false, false, true>": ("fa_fwd_kernel<128,true,sparse>", "fa_prefill.hip"),
            "fa_bwd_dq<128, true, false, false>": ("fa_bwd_dq<128,true>", "fa_backward.hip"),
            "fa_bwd_dkdv<128, true, false, false>": ("fa_bwd_dkdv<128,true>", "fa_backward.hip"),
            "fa_bwd_dq<128, true, false, true>": ("fa_bwd_dq<128,true,sparse>", "fa_backward.hip"),
            "fa_bwd_dkdv<128, true, false, true>": ("fa_bwd_dkdv<128,true,sparse>", "fa_backward.hip"),
            "fa_bwd_pre<128>": ("fa_bwd_pre<128>", "fa_backward.hip"),
            "fa_fwd_fp8_kernel<128, true>": ("fa_fwd_fp8_kernel<128,true>", "fa_prefill_fp8.hip"),
            "fa_quantize_fp8_incoherent_kernel<128>": ("fa_quantize_fp8_incoherent_kernel<128>", "fa_prefill_fp8.hip"),
            "fa_decode_split_kernel<128, 4096>": ("fa_decode_split_kernel<128,4096>", "fa_decode.hip"),
            "fa_decode_combine_kernel<128>": ("fa_decode_combine_kernel<128>", "fa_decode.hip")}
    out = {"about": "HBM bytes per launch = (FETCH_SIZE + WRITE_SIZE counted per dispatch, KiB x 1024) "
                    "x calibration factor from a plain %d-byte device copy in the same run" % COPY_CALIB_BYTES,
           "fetch_factor": fr, "write_factor": wr}
    for name in set(fetch) | set(write):
        for pat, (key, src) in keys.items():
            if pat in name:
                f = fetch.get(name, 0.0) * 1024 * fr
                w = write.get(name, 0.0) * 1024 * wr
                out[key] = {"fetch_bytes": f, "write_bytes": w, "bytes_per_launch": f + w,
                            "source_hash": source_hash([src])}
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def host_cpu():
    """The host's CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_fields():
    """cores = the threads the oracle's matrix products actually use (numpy's
    BLAS pool; its elementwise passes run on one); with the host's CPU model
    and affinity core count beside it."""
    return dict({"cores": blas_threads()}, **host_cpu())


def cpu_baseline_prefill(case, budget_s):
    """The oracle, as is, on whole query heads' sampled rows until the budget
    is spent. Rate uses the same FLOP convention as the metric (visible keys)."""
    import gen
    import oracle
    q = oracle.bf16_bits_to_f64(case["q_bits"][:, :1])  # placeholder to import cost out of timing
    del q
    B, Hq, Hkv, N, d = case["B"], case["Hq"], case["Hkv"], case["N"], case["d"]
    G = Hq // Hkv
    rows_per_head = 2048
    flops = 0.0
    t0 = time.perf_counter()
    heads = 0
    for h in range(Hq):
        rows = gen.row_sample(case["seed"], N, rows_per_head, salt=h)
        qh = oracle.bf16_bits_to_f64(case["q_bits"][:, h:h + 1])
        kh = oracle.bf16_bits_to_f64(case["k_bits"][:, h // G:h // G + 1])
        vh = oracle.bf16_bits_to_f64(case["v_bits"][:, h // G:h // G + 1])
        oracle.attention_naive(qh, kh, vh, case["scale"], True, rows=rows)
        flops += 4.0 * d * float((rows + 1).sum())
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **cpu_fields(), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": "fp64 naive three-pass oracle on %d sampled rows (rows 0, N-1 and a seeded "
                      "draw) of each of %d of the %d query heads of the prefill workload, all Nk "
                      "keys masked causally; FLOPs counted as 4*d*(visible keys) per row"
                      % (rows_per_head, heads, Hq)}


def cpu_baseline_decode(dc, budget_s):
    import oracle
    t0 = time.perf_counter()
    done = []
    for b in range(dc["B"]):
        oracle.paged_decode(dc["q_bits"][b:b + 1], dc["k_bits"], dc["v_bits"], dc["table"][b:b + 1],
                            dc["seq_lens"][b:b + 1], dc["scale"], dc["page"])
        done.append(b)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    sl = dc["seq_lens"][done]
    by = decode_bytes(sl, len(done), dc["Hq"], dc["Hkv"], dc["d"], dc["page"])
    return {"value": by / dt / 1e9, "unit": "GB/s", **cpu_fields(), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": "fp64 oracle (page gather + naive attention) on the first %d of the %d "
                      "sequences of the decode workload; algorithmic bytes as for the GPU" % (len(done), dc["B"])}


def cpu_baseline_config4(cfg, budget_s):
    """The oracle on the 64K-token workload's sampled rows (256 per query
    head: rows 0, N-1 and seeded draws), head by head until the budget is
    spent; reports the fraction of the full causal work the sample covers
    and the full-oracle time that fraction extrapolates to."""
    import gen
    import oracle
    B, Hq, Hkv, N, d, seed = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["d"], cfg["seed"]
    G = Hq // Hkv
    scale = float(np.float32(1.0 / math.sqrt(d)))
    full = 4.0 * d * B * Hq * N * (N + 1) / 2.0      # visible pairs of the whole launch, 4*d flop each
    flops = 0.0
    heads = 0
    dt = 0.0
    for h in range(Hq):
        rows = gen.row_sample(seed, N, 256, salt=h)
        g = h // G
        per_head = (B, 1, N, d)
        qh = oracle.bf16_bits_to_f64(gen.normal_bf16(seed, gen.STREAM_Q, per_head, cfg["sigma"], offset=h * N * d))
        kh = oracle.bf16_bits_to_f64(gen.normal_bf16(seed, gen.STREAM_K, per_head, cfg["sigma"], offset=g * N * d))
        vh = oracle.bf16_bits_to_f64(gen.normal_bf16(seed, gen.STREAM_V, per_head, cfg["sigma"], offset=g * N * d))
        t0 = time.perf_counter()
        oracle.attention_naive(qh, kh, vh, scale, True, rows=rows)
        dt += time.perf_counter() - t0
        flops += 4.0 * d * float((rows + 1).sum())
        heads += 1
        if dt >= budget_s:
            break
    frac = flops / full
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **cpu_fields(), "kind": "oracle",
            "seconds": round(dt, 2), "fraction_of_full_work": frac,
            "extrapolated_full_oracle_seconds": round(dt / frac, 1),
            "sample": "fp64 naive three-pass oracle on 256 sampled rows (rows 0, N-1 and seeded draws) of each "
                      "of %d of the %d query heads of the 64K-token causal GQA workload; the full-oracle time is an extrapolation by the covered "
                      "fraction of visible pairs" % (heads, Hq)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds per CPU-baseline leg")
    ap.add_argument("--copy-calib", action="store_true",
                    help="a counter run: also run one plain 1 GiB device copy (for HBM counter calibration), "
                         "and leave out the cold-cache and other-shape prefill legs")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs into profiles/hbm_traffic.json and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], os.path.join(ROOT, "profiles", "hbm_traffic.json"))
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import gen
    from __graft_entry__ import _ensure_built
    _ensure_built()
    import exact_attention_03_amd as fa
    fa.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs (host generation, then resident in HBM) ----
    P = PREFILL
    pscale = float(np.float32(1.0 / math.sqrt(P["d"])))
    pc = dict(B=P["B"], Hq=P["Hq"], Hkv=P["Hkv"], N=P["N"], d=P["d"], seed=P["seed"], scale=pscale)
    pc["q_bits"] = gen.normal_bf16(P["seed"], gen.STREAM_Q, (P["B"], P["Hq"], P["N"], P["d"]), P["sigma"])
    pc["k_bits"] = gen.normal_bf16(P["seed"], gen.STREAM_K, (P["B"], P["Hkv"], P["N"], P["d"]), P["sigma"])
    pc["v_bits"] = gen.normal_bf16(P["seed"], gen.STREAM_V, (P["B"], P["Hkv"], P["N"], P["d"]), P["sigma"])
    q, k, v = dev_bf16(pc["q_bits"]), dev_bf16(pc["k_bits"]), dev_bf16(pc["v_bits"])
    o = torch.empty_like(q)
    lse = torch.empty((P["B"], P["Hq"], P["N"]), dtype=torch.float32, device=dev)

    D = DECODE
    dscale = float(np.float32(1.0 / math.sqrt(D["d"])))
    seq_lens, table, total = gen.decode_layout(D["seed"], D["B"], D["len_lo"], D["len_hi"], D["page"], D["max_pages"])
    dc = dict(B=D["B"], Hq=D["Hq"], Hkv=D["Hkv"], d=D["d"], page=D["page"], scale=dscale,
              seq_lens=seq_lens, table=table)
    dc["q_bits"] = gen.normal_bf16(D["seed"], gen.STREAM_Q, (D["B"], D["Hq"], D["d"]))
    dc["k_bits"] = gen.normal_bf16(D["seed"], gen.STREAM_K, (total, D["Hkv"], D["page"], D["d"]))
    dc["v_bits"] = gen.normal_bf16(D["seed"], gen.STREAM_V, (total, D["Hkv"], D["page"], D["d"]))
    dq, dk, dv = dev_bf16(dc["q_bits"]), dev_bf16(dc["k_bits"]), dev_bf16(dc["v_bits"])
    dbt = torch.from_numpy(table).to(dev)
    dsl = torch.from_numpy(seq_lens).to(dev)
    do_ = torch.empty((D["B"], D["Hq"], D["d"]), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((D["B"], D["Hq"]), dtype=torch.float32, device=dev)
    max_seq_len = D["max_pages"] * D["page"]
    ws = torch.empty(fa.fa_paged_decode_workspace_size(D["B"], D["Hq"], D["d"], D["page"], max_seq_len),
                     dtype=torch.uint8, device=dev)

    C = PAGED
    cscale = float(np.float32(1.0 / math.sqrt(C["d"])))
    c_lens, c_table, c_total = gen.decode_layout(C["seed"], C["B"], C["len_lo"], C["len_hi"], C["page"],
                                                 C["max_pages"])
    c_qlens = np.full(C["B"], C["chunk"], dtype=np.int32)
    c_cu = np.concatenate([[0], np.cumsum(c_qlens)]).astype(np.int32)
    cq = dev_bf16(gen.normal_bf16(C["seed"], gen.STREAM_Q, (int(c_cu[-1]), C["Hq"], C["d"])))
    ck = dev_bf16(gen.normal_bf16(C["seed"], gen.STREAM_K, (c_total, C["Hkv"], C["page"], C["d"])))
    cv = dev_bf16(gen.normal_bf16(C["seed"], gen.STREAM_V, (c_total, C["Hkv"], C["page"], C["d"])))
    cbt, csl, ccu = (torch.from_numpy(x).to(dev) for x in (c_table, c_lens, c_cu))
    co = torch.empty_like(cq)
    clse = torch.empty((int(c_cu[-1]), C["Hq"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def prefill(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_forward(q, k, v, o, lse, P["causal"], pscale)
        if ev is not None:
            ev[1].record()

    # The same prefill with cold inputs: a 1 GiB read-modify-write (untimed)
    # right before each timed pass leaves none of Q, K, V in L2 or the MALL.
    flush = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def prefill_cold(ev=None):
        flush.add_(1)
        prefill(ev)

    def shape_inputs(cfg):
        qb = dev_bf16(gen.normal_bf16(cfg["seed"], gen.STREAM_Q, (cfg["B"], cfg["Hq"], cfg["N"], cfg["d"]), cfg["sigma"]))
        kb = dev_bf16(gen.normal_bf16(cfg["seed"], gen.STREAM_K, (cfg["B"], cfg["Hkv"], cfg["N"], cfg["d"]), cfg["sigma"]))
        vb = dev_bf16(gen.normal_bf16(cfg["seed"], gen.STREAM_V, (cfg["B"], cfg["Hkv"], cfg["N"], cfg["d"]), cfg["sigma"]))
        return qb, kb, vb, torch.empty_like(qb), torch.empty((cfg["B"], cfg["Hq"], cfg["N"]), dtype=torch.float32,
                                                                device=dev)

    c2_in = shape_inputs(CONFIG2)
    c4_in = shape_inputs(CONFIG4)
    c2_scale = float(np.float32(1.0 / math.sqrt(CONFIG2["d"])))
    c4_scale = float(np.float32(1.0 / math.sqrt(CONFIG4["d"])))

    def config2(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_forward(*c2_in, CONFIG2["causal"], c2_scale)
        if ev is not None:
            ev[1].record()

    def config4(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_forward(*c4_in, CONFIG4["causal"], c4_scale)
        if ev is not None:
            ev[1].record()

    W = WINDOW
    wo = torch.empty_like(q)
    wlse = torch.empty_like(lse)

    def window(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_forward_window(q, k, v, wo, wlse, W["causal"], W["left"], -1, pscale)
        if ev is not None:
            ev[1].record()

    SP = SPARSE
    nqb = -(-P["N"] // 128)
    sp_mask = gen.local_global_block_mask(nqb, nqb, SP["local"], SP["n_global"])
    smask = torch.from_numpy(sp_mask[None, None].copy()).to(dev)
    so = torch.empty_like(q)
    slse = torch.empty_like(lse)

    def block_sparse(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_forward_block_sparse(q, k, v, so, slse, SP["causal"], smask, pscale)
        if ev is not None:
            ev[1].record()

    dout = dev_bf16(gen.normal_bf16(P["seed"], gen.STREAM_DO, (P["B"], P["Hq"], P["N"], P["d"])))
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(fa.fa_backward_workspace_size(P["B"], P["Hq"], P["N"]), dtype=torch.uint8, device=dev)
    sbws = torch.empty(fa.fa_backward_block_sparse_workspace_size(P["B"], P["Hq"], P["Hkv"], P["N"], P["N"], P["d"]),
                       dtype=torch.uint8, device=dev)

    nqb = -(-P["N"] // fa.FP8_SCALE_ROWS)
    cq8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    ck8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    cv8 = torch.empty(v.shape, dtype=torch.uint8, device=dev)
    sq8 = torch.empty((P["B"], P["Hq"], nqb), dtype=torch.float32, device=dev)
    sk8 = torch.empty((P["B"], P["Hkv"], nqb), dtype=torch.float32, device=dev)
    sv8 = torch.empty((P["B"], P["Hkv"], 1), dtype=torch.float32, device=dev)
    fa.fa_quantize_fp8(q, cq8, sq8, fa.FP8_SCALE_ROWS)
    fa.fa_quantize_fp8(k, ck8, sk8, fa.FP8_SCALE_ROWS)
    fa.fa_quantize_fp8(v, cv8, sv8, P["N"])
    o8 = torch.empty_like(q)
    lse8 = torch.empty_like(lse)

    def fp8(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_forward_fp8(cq8, sq8, ck8, sk8, cv8, sv8.reshape(P["B"], P["Hkv"]), o8, lse8, P["causal"], pscale)
        if ev is not None:
            ev[1].record()

    def backward(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_backward(q, k, v, o, lse, dout, gq, gk, gv, P["causal"], pscale, bws)
        if ev is not None:
            ev[1].record()

    def backward_sparse(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_backward_block_sparse(q, k, v, so, slse, dout, gq, gk, gv, SP["causal"], smask, pscale, sbws)
        if ev is not None:
            ev[1].record()

    def decode(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_paged_decode(dq, dk, dv, dbt, dsl, do_, dlse, max_seq_len, dscale, ws, page_size=D["page"])
        if ev is not None:
            ev[1].record()

    def chunked(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_paged_prefill(cq, ck, cv, cbt, csl, ccu, co, clse, C["chunk"], C["causal"], cscale,
                            page_size=C["page"])
        if ev is not None:
            ev[1].record()

    # K steps = K passes of each kernel. Each kernel's passes run back to back
    # so each is timed in its steady state: the prefill's 170 MB of Q/K/V stay
    # in the 256 MB MALL between passes (as when a projection has just written
    # them; its warm-ups run last, right before it, and the windowed prefill
    # reads the same inputs right after it); the decode's 4.7 GB pool never
    # fits.
    prefill()  # O and LSE for the backward
    block_sparse()  # O and LSE for the block-sparse backward
    # A counter run (--copy-calib) leaves out the legs that launch the
    # prefill kernel on other inputs (cold caches, other shapes), so that the
    # prefill kernel's counters are the headline prefill's alone.
    extra = () if args.copy_calib else (prefill_cold, config2, config4)
    for fn in extra + (decode, chunked, backward_sparse, backward, fp8, block_sparse, window, prefill):
        for _ in range(args.warmup):
            fn()
    legs = (prefill, window, block_sparse, fp8, backward, backward_sparse, decode, chunked) + extra
    evs = {fn: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
           for fn in legs}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for fn in legs:
        for i in range(args.steps):
            fn(evs[fn][i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_pre, ev_dec, ev_chk = evs[prefill], evs[decode], evs[chunked]
    t_pre = [e[0].elapsed_time(e[1]) for e in ev_pre]   # ms
    t_dec = [e[0].elapsed_time(e[1]) for e in ev_dec]
    t_chk = [e[0].elapsed_time(e[1]) for e in ev_chk]
    t_win = [e[0].elapsed_time(e[1]) for e in evs[window]]
    ms_win = float(np.mean(t_win))
    t_sp = [e[0].elapsed_time(e[1]) for e in evs[block_sparse]]
    ms_sp = float(np.mean(t_sp))
    t_bw = [e[0].elapsed_time(e[1]) for e in evs[backward]]
    ms_bw = float(np.mean(t_bw))
    t_bs = [e[0].elapsed_time(e[1]) for e in evs[backward_sparse]]
    ms_bs = float(np.mean(t_bs))
    t_f8 = [e[0].elapsed_time(e[1]) for e in evs[fp8]]
    ms_f8 = float(np.mean(t_f8))
    # the quantizer (not part of any step): Q of the prefill, timed alone
    qz0, qz1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qz0.record()
    fa.fa_quantize_fp8(q, cq8, sq8, fa.FP8_SCALE_ROWS)
    qz1.record()
    torch.cuda.synchronize()
    ms_qz = qz0.elapsed_time(qz1)
    # incoherent processing + quantization of the same Q (not part of any
    # step either): mean of 5 launches
    signs = torch.from_numpy(gen.random_signs(P["seed"] + 1, P["d"])).to(dev)
    fa.fa_quantize_fp8_incoherent(q, signs, cq8, sq8, fa.FP8_SCALE_ROWS)
    qi = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for e in qi:
        e[0].record()
        fa.fa_quantize_fp8_incoherent(q, signs, cq8, sq8, fa.FP8_SCALE_ROWS)
        e[1].record()
    torch.cuda.synchronize()
    ms_qi = float(np.mean([e[0].elapsed_time(e[1]) for e in qi]))
    qi_bytes = P["B"] * P["Hq"] * P["N"] * P["d"] * 3 + sq8.numel() * 4 + P["d"]  # bf16 in, E4M3 out, scales, signs
    ms_pre = float(np.mean(t_pre))
    ms_dec = float(np.mean(t_dec))
    ms_chk = float(np.mean(t_chk))
    if extra:
        t_cold = [e[0].elapsed_time(e[1]) for e in evs[prefill_cold]]
        t_c2 = [e[0].elapsed_time(e[1]) for e in evs[config2]]
        t_c4 = [e[0].elapsed_time(e[1]) for e in evs[config4]]
    del flush

    if args.copy_calib:
        a = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    pf = prefill_flops(P["B"], P["Hq"], P["N"], P["N"], P["d"], P["causal"])
    tflops = pf / (ms_pre * 1e-3) / 1e12
    db = decode_bytes(seq_lens, D["B"], D["Hq"], D["Hkv"], D["d"], D["page"])
    gbps = db / (ms_dec * 1e-3) / 1e9
    pre_hash = source_hash(["fa_prefill.hip"])
    dec_hash = source_hash(["fa_decode.hip"])
    cf = paged_prefill_flops(c_lens, c_qlens, C["Hq"], C["d"], C["causal"])
    ctflops = cf / (ms_chk * 1e-3) / 1e12
    wf = window_flops(P["B"], P["Hq"], P["N"], P["N"], P["d"], W["left"], W["causal"])
    wtflops = wf / (ms_win * 1e-3) / 1e12
    sf = block_sparse_flops(P["B"], P["Hq"], P["N"], P["N"], P["d"], sp_mask, SP["causal"])
    stflops = sf / (ms_sp * 1e-3) / 1e12
    bf = 2.5 * pf
    btflops = bf / (ms_bw * 1e-3) / 1e12
    bsf = 2.5 * sf
    bstflops = bsf / (ms_bs * 1e-3) / 1e12
    f8tflops = pf / (ms_f8 * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal GQA prefill B=1 Hq=64 Hkv=8 N=8192 d=128 + paged GQA decode "
                        "64 seqs L~U{512..32768} Hq=64 Hkv=8 d=128 page=16 + paged chunked prefill "
                        "8 seqs x 1024-token chunks, caches L~U{2048..16384} + causal sliding-window "
                        "prefill (prefill inputs, left window 4096) + causal block-sparse prefill (prefill "
                        "inputs, local 16 + global 1 blocks of 128) + causal backward (prefill inputs) + "
                        "causal block-sparse backward (same mask) + FP8 E4M3 causal prefill (prefill inputs "
                        "quantized per 128-row block)",
            "prefill": {"B": P["B"], "Hq": P["Hq"], "Hkv": P["Hkv"], "Nq": P["N"], "Nk": P["N"],
                        "d": P["d"], "causal": P["causal"], "seed": P["seed"], "flops": pf},
            "decode": {"B": D["B"], "Hq": D["Hq"], "Hkv": D["Hkv"], "d": D["d"], "page_size": D["page"],
                       "seed": D["seed"], "tokens": int(seq_lens.astype(np.int64).sum()),
                       "pages": int(total), "bytes": db},
            "paged_prefill": {"B": C["B"], "Hq": C["Hq"], "Hkv": C["Hkv"], "d": C["d"], "page_size": C["page"],
                              "chunk": C["chunk"], "causal": C["causal"], "seed": C["seed"],
                              "cached_tokens": int(c_lens.astype(np.int64).sum()), "flops": cf},
            "window": {"inputs": "prefill", "window_left": W["left"], "window_right": -1,
                       "causal": W["causal"], "flops": wf},
            "block_sparse": {"inputs": "prefill", "block": 128, "local_blocks": SP["local"],
                             "global_blocks": SP["n_global"], "causal": SP["causal"],
                             "mask_density": round(float(sp_mask.mean()), 4), "flops": sf},
            "fp8": {"inputs": "prefill, quantized to E4M3 (Q, K per 128-row block, V per head)",
                    "causal": P["causal"], "flops": pf},
            "backward": {"inputs": "prefill", "causal": P["causal"], "dout_seed": P["seed"], "flops": bf,
                         "flops_convention": "2.5 x forward (5 products of 2*d flop per visible pair)"},
            "backward_block_sparse": {"inputs": "prefill, the block-sparse prefill's O and LSE, the backward's dO",
                                      "mask": "as block_sparse", "causal": SP["causal"], "flops": bsf,
                                      "flops_convention": "2.5 x the block-sparse forward's"},
        },
        "roofline": {
            "kernel": "fa_fwd_kernel<128, causal>",
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "ms": round(ms_pre, 4),
            "ms_median": round(float(np.median(t_pre)), 4), "ms_min": round(float(np.min(t_pre)), 4),
            "traffic": load_traffic("fa_fwd_kernel<128,true>", pre_hash),
            "min_bytes": prefill_min_bytes(P["B"], P["Hq"], P["Hkv"], P["N"], P["N"], P["d"]),
        },
        "decode": {
            "metric": "paged decode HBM GB/s",
            "value": round(gbps, 1), "unit": "GB/s", "ms": round(ms_dec, 4),
            "ms_median": round(float(np.median(t_dec)), 4), "ms_min": round(float(np.min(t_dec)), 4),
            "roofline": {
                "kernel": "fa_decode_split_kernel<128, 4096> + fa_decode_combine_kernel<128>",
                "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": load_traffic_sum(["fa_decode_split_kernel<128,4096>", "fa_decode_combine_kernel<128>"], dec_hash),
            },
            "tflops": round(decode_flops(seq_lens, D["Hq"], D["d"]) / (ms_dec * 1e-3) / 1e12, 2),
            "overhead_bytes": decode_overhead_bytes(seq_lens, D["B"], D["Hq"], D["Hkv"], D["d"], max_seq_len,
                                                    D["page"]),
        },
        "paged_prefill": {
            "metric": "paged chunked prefill TFLOP/s",
            "value": round(ctflops, 2), "unit": "TFLOP/s", "ms": round(ms_chk, 4),
            "ms_median": round(float(np.median(t_chk)), 4), "ms_min": round(float(np.min(t_chk)), 4),
            "roofline": {
                "kernel": "fa_fwd_kernel<128, causal, paged>",
                "bound": "mfma", "achieved": round(ctflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ctflops / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic("fa_fwd_kernel<128,true,paged>", pre_hash),
            },
        },
        "window": {
            "metric": "sliding-window prefill TFLOP/s",
            "value": round(wtflops, 2), "unit": "TFLOP/s", "ms": round(ms_win, 4),
            "ms_median": round(float(np.median(t_win)), 4), "ms_min": round(float(np.min(t_win)), 4),
            "roofline": {
                "kernel": "fa_fwd_kernel<128, causal, window>",
                "bound": "mfma", "achieved": round(wtflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(wtflops / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic("fa_fwd_kernel<128,true,window>", pre_hash),
            },
        },
        "block_sparse": {
            "metric": "block-sparse prefill TFLOP/s",
            "value": round(stflops, 2), "unit": "TFLOP/s", "ms": round(ms_sp, 4),
            "ms_median": round(float(np.median(t_sp)), 4), "ms_min": round(float(np.min(t_sp)), 4),
            "roofline": {
                "kernel": "fa_fwd_kernel<128, causal, block-sparse>",
                "bound": "mfma", "achieved": round(stflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(stflops / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic("fa_fwd_kernel<128,true,sparse>", pre_hash),
            },
        },
        "fp8": {
            "metric": "FP8 attention forward TFLOP/s",
            "value": round(f8tflops, 2), "unit": "TFLOP/s", "ms": round(ms_f8, 4),
            "ms_median": round(float(np.median(t_f8)), 4), "ms_min": round(float(np.min(t_f8)), 4),
            "quantize_q_ms": round(ms_qz, 4),
            "quantize_incoherent_q": {
                "kernel": "fa_quantize_fp8_incoherent_kernel<128>", "ms": round(ms_qi, 4),
                "bound": "hbm", "achieved": round(qi_bytes / ms_qi / 1e6, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(qi_bytes / ms_qi / 1e6 / PEAK_HBM_GBPS, 4),
                "traffic": load_traffic("fa_quantize_fp8_incoherent_kernel<128>", source_hash(["fa_prefill_fp8.hip"])),
            },
            "roofline": {
                "kernel": "fa_fwd_fp8_kernel<128, causal>",
                "bound": "mfma", "achieved": round(f8tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(f8tflops / PEAK_FP8_TFLOPS, 4),
                "traffic": load_traffic("fa_fwd_fp8_kernel<128,true>", source_hash(["fa_prefill_fp8.hip"])),
            },
        },
        "backward": {
            "metric": "attention backward TFLOP/s",
            "value": round(btflops, 2), "unit": "TFLOP/s", "ms": round(ms_bw, 4),
            "ms_median": round(float(np.median(t_bw)), 4), "ms_min": round(float(np.min(t_bw)), 4),
            "roofline": {
                "kernel": "fa_bwd_pre<128> + fa_bwd_dq<128, causal> + fa_bwd_dkdv<128, causal>",
                "bound": "mfma", "achieved": round(btflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(btflops / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic_sum(["fa_bwd_pre<128>", "fa_bwd_dq<128,true>", "fa_bwd_dkdv<128,true>"],
                                            source_hash(["fa_backward.hip"])),
            },
        },
        "backward_block_sparse": {
            "metric": "block-sparse attention backward TFLOP/s",
            "value": round(bstflops, 2), "unit": "TFLOP/s", "ms": round(ms_bs, 4),
            "ms_median": round(float(np.median(t_bs)), 4), "ms_min": round(float(np.min(t_bs)), 4),
            "roofline": {
                "kernel": "fa_bwd_pre<128> + fa_bwd_dq<128, causal, block-sparse> + "
                          "fa_bwd_dkdv<128, causal, block-sparse>",
                "bound": "mfma", "achieved": round(bstflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(bstflops / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic_sum(["fa_bwd_pre<128>", "fa_bwd_dq<128,true,sparse>",
                                             "fa_bwd_dkdv<128,true,sparse>"], source_hash(["fa_backward.hip"])),
            },
        },
    }
    def prefill_leg(name, cfg, times, extra=None):
        f = prefill_flops(cfg["B"], cfg["Hq"], cfg["N"], cfg["N"], cfg["d"], cfg["causal"])
        ms = float(np.mean(times))
        tf = f / (ms * 1e-3) / 1e12
        leg = {"metric": "attn fwd TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
               "ms_median": round(float(np.median(times)), 4), "ms_min": round(float(np.min(times)), 4),
               "config": {"B": cfg["B"], "Hq": cfg["Hq"], "Hkv": cfg["Hkv"], "Nq": cfg["N"], "Nk": cfg["N"],
                          "d": cfg["d"], "causal": cfg["causal"], "seed": cfg["seed"], "sigma": cfg["sigma"],
                          "flops": f},
               "roofline": {"kernel": "fa_fwd_kernel<128, causal>", "bound": "mfma", "achieved": round(tf, 2),
                            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                            "traffic": None}}
        if extra:
            leg.update(extra)
        out[name] = leg

    if extra:
        prefill_leg("prefill_cold", P, t_cold, {"note": "the headline prefill with a 1 GiB read-modify-write "
                                                        "(untimed) before every pass: Q, K, V start outside L2 and "
                                                        "the MALL"})
        prefill_leg("config2", CONFIG2, t_c2, {"note": "135 MB working set: MALL-resident across back-to-back passes"})
        prefill_leg("config4", CONFIG4, t_c4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(pc, args.cpu_budget)
        out["decode"]["cpu_baseline"] = cpu_baseline_decode(dc, args.cpu_budget)
        if extra:
            out["config4"]["cpu_baseline"] = cpu_baseline_config4(CONFIG4, args.cpu_budget / 2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
