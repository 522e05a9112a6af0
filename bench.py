"""Benchmark of the KV-streams hot path on one MI355X.

One step = one pass of every hot-path stage over one batch of synthetic input:
  training side (4 x 32k-token summary-compaction traces, 32 q / 8 kv heads,
  D = 128, bf16): RoPE at logical positions on Q and K, eviction-masked
  attention forward, then backward;
  inference side (64 paged caches, 32 q / 8 kv heads): 1-6 rounds of
  block-table compaction, the append of the new token (its key rotated at
  its logical position), one paged GQA decode step with the query rotated
  in the kernel's prologue.

Prints one JSON line.  `value` is the masked attention fwd+bwd throughput in
TFLOP/s of useful work (4*D flops forward and 10*D backward per live
(query, key) pair per query head; masked pairs are not counted), timed with
HIP events on the stream the kernels run on.  The decode side's HBM GB/s is
reported beside it.  `single_token_blocks` times the same decode step with
one pool slot per token (token tables, token-run compaction), and
`toy_stack` reports the trainer/generator mismatch KL of a random-weight
3-layer model built on the path, and `reprefill_counterfactual` times,
outside the step, the
attention that re-prefill compaction would run on the same rollouts.
`long_mixed_64k` times the fwd+bwd of 8 x 64k traces under three compaction
strategies and their continuation by 256 decode steps with a forced event.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same workload
on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (a known-size "
                         "reference for HBM byte counters)")
    return ap.parse_args()


def live_pairs(e: np.ndarray) -> int:
    """sum over queries of |{j <= i : e_j > i}| for a batch of traces."""
    tot = 0
    for row in e.astype(np.int64):
        N = row.size
        hist = np.zeros(N + 1, dtype=np.int64)
        np.add.at(hist, row[row < N], 1)
        gone = np.cumsum(hist)[:N]
        tot += int(((np.arange(N) + 1) - gone).sum())
    return tot


def executed_flops(e: np.ndarray, Hq: int, Hkv: int, D: int, kt: int = 64):
    """MFMA flops the attention kernels execute (tile granularity) for a batch
    of traces, following their tiling: the forward and dQ kernels visit, per
    query tile of BM rows and query head, every key tile t with t <= last row
    / kt and max e over the tile > first row; dK/dV workgroups of 256 keys
    (8 waves x 32 keys) visit 32-row query chunks of each of the G heads up to
    the largest e of their keys, each wave skipping chunks none of its keys
    sees.  Returns (forward, dQ, dK/dV) flops."""
    G = Hq // Hkv
    hpw = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)   # query heads per wave
    bm = 32 * (8 // hpw)
    fwd = dq = dkdv = 0
    for row in e.astype(np.int64):
        N = row.size
        nt = (N + kt - 1) // kt
        emax = np.array([row[t * kt:(t + 1) * kt].max() for t in range(nt)])
        for i0 in range(0, N, bm):
            i1 = min(N, i0 + bm)
            tmax = (i1 - 1) // kt
            live = int((emax[:tmax + 1] > i0).sum())
            fwd += live * 4 * D * bm * kt * Hq
            dq += live * 6 * D * bm * kt * Hq
        for j0 in range(0, N, 256):
            c_begin = j0 // 32
            c_end = (min(N, int(row[j0:j0 + 256].max())) + 31) // 32
            for w in range(8):
                kw0 = j0 + 32 * w
                keys = row[kw0:min(N, kw0 + 32)]
                if keys.size == 0:
                    continue
                wq1 = min(N, int(keys.max()))
                c = np.arange(c_begin, c_end) * 32
                visited = int(((c < wq1) & (c + 32 > kw0)).sum())
                dkdv += visited * G * 8 * D * 32 * 32 * Hkv
    return fwd, dq, dkdv


# HIP sources each entry point's kernels are built from (a stored counter
# summary applies only to the kernels it was taken on)
ENTRY_SOURCES = {
    "ks_evict_attn_fwd_rope": ("ks_common.h", "attn_common.h", "attn_fwd.hip", "rope.hip"),
    "ks_evict_attn_bwd_rope": ("ks_common.h", "attn_common.h", "attn_fwd.hip", "attn_bwd.hip",
                               "rope.hip"),
    "ks_paged_decode": ("ks_common.h", "decode.hip"),
    "ks_paged_decode_bs1": ("ks_common.h", "decode.hip"),
    "ks_compact_block_table_rounds": ("ks_common.h", "compact.hip"),
}


def kernel_sources_hash(entry: str) -> str:
    """sha256 over the code of the HIP sources of one entry point's kernels
    (comments and blank space removed, so editing a comment keeps a stored
    counter summary valid)."""
    import hashlib
    import re
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kv_cache_compaction_amd",
                        "csrc")
    h = hashlib.sha256()
    for name in sorted(ENTRY_SOURCES[entry]):
        with open(os.path.join(root, name)) as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or it was taken on other kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "hbm_traffic_attn32k_decode64.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get("entry_points", {}).get(kernel)
    if ent is None or kernel not in ENTRY_SOURCES:
        return None
    if ent.get("sources_sha256") != kernel_sources_hash(kernel):
        return None
    return ent.get("hbm_bytes_per_launch")


class Timer:
    """HIP-event timing of one stage on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        return ev

    def stop(self, ev0, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.pairs.append((name, ev0, ev))

    def totals(self):
        out = {}
        for name, a, b in self.pairs:
            out[name] = out.get(name, 0.0) + a.elapsed_time(b)
        return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the path "
              "would shard by (trace, kv group) for training and by sequence for decode, "
              "with no exchange inside a step", file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_compaction_amd as ks
    from workloads import (PAGED_DECODE, SUMMARY_32K, build_decode_batch, config_trace_batch,
                           normal_tensor, stacked_e, workload_rng)

    dev = "cuda"
    torch.cuda.set_device(0)
    bf = torch.bfloat16

    # ---------------- training-side inputs (32k summary traces) ----------------
    trn = SUMMARY_32K
    traces, seeds = config_trace_batch(trn)
    e_np = stacked_e(traces)
    B, N, Hq, Hkv, D = trn.batch, trn.N, trn.Hq, trn.Hkv, trn.D
    q = normal_tensor((B, N, Hq, D), seeds["q"], trn.value_scale, bf, dev)
    k = normal_tensor((B, N, Hkv, D), seeds["k"], trn.value_scale, bf, dev)
    v = normal_tensor((B, N, Hkv, D), seeds["v"], trn.value_scale, bf, dev)
    do = normal_tensor((B, N, Hq, D), seeds["do"], trn.value_scale, bf, dev)
    e = torch.from_numpy(e_np).to(dev)
    pos = torch.arange(N, dtype=torch.int32, device=dev)[None].repeat(B, 1).contiguous()
    # q and k are the raw projections: the attention entry points rotate
    # them at their logical positions (k once into k_rot, q in the forward
    # kernel, which stores q_rot for the backward) and leave them unchanged
    q_rot, k_rot = torch.empty_like(q), torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lib = ks.load_library()
    ws_f = torch.empty(lib.ks_evict_attn_fwd_rope_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(lib.ks_evict_attn_bwd_rope_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                       dtype=torch.uint8, device=dev)
    pairs = live_pairs(e_np)
    ex_fwd, ex_dq, ex_dkdv = executed_flops(e_np, Hq, Hkv, D)
    # live pairs summed over the traces; every query head sees its trace's mask
    flops_fwd = 4.0 * D * pairs * Hq
    flops_bwd = 10.0 * D * pairs * Hq
    causal_pairs = B * N * (N + 1) // 2

    # ---------------- inference-side inputs (paged decode) ----------------
    dec = PAGED_DECODE
    db = build_decode_batch(workload_rng(dec), dec.batch)
    DB, MB = db.table0.shape
    NB = db.num_pool_blocks
    Hq_d, Hkv_d = dec.Hq, dec.Hkv
    kp = normal_tensor((NB, Hkv_d, 16, D), 4001, 0.5, bf, dev)
    vp = normal_tensor((NB, Hkv_d, 16, D), 4002, 0.5, bf, dev)
    q4 = normal_tensor((DB, 1, Hq_d, D), 4003, 0.5, bf, dev)
    k4 = normal_tensor((DB, Hkv_d, D), 4004, 0.5, bf, dev)
    v4 = normal_tensor((DB, Hkv_d, D), 4005, 0.5, bf, dev)
    pos4 = torch.from_numpy(db.pos[:, None].astype(np.int32)).to(dev)
    pos4f = pos4[:, 0].contiguous()
    table0 = torch.from_numpy(db.table0).to(dev)
    nblk0 = torch.from_numpy(db.nblk0).to(dev)
    keeps_all = torch.from_numpy(np.ascontiguousarray(db.keeps)).to(dev)  # [R, B, MB]
    tbufs = [torch.empty_like(table0), torch.empty_like(table0)]
    nbufs = [torch.empty_like(nblk0), torch.empty_like(nblk0)]
    seq_lens = torch.from_numpy((db.live_len + 1).astype(np.int32)).to(dev)
    out4 = torch.empty((DB, Hq_d, D), dtype=bf, device=dev)
    lse4 = torch.empty((DB, Hq_d), dtype=torch.float32, device=dev)
    ws_d = torch.empty(ks.ks_paged_decode_workspace(DB, Hq_d, D, MB), dtype=torch.uint8,
                       device=dev)
    L = db.live_len.astype(np.int64) + 1
    # decode step bytes: K/V of every live token once, q (read once, rotated
    # in the kernel), the appended token's k/v (read + write), output, lse,
    # table entries and lengths
    dec_bytes = int((L * Hkv_d * D * 2 * 2).sum()) + DB * Hq_d * D * 2 + \
        2 * 2 * DB * Hkv_d * D * 2 + DB * Hq_d * D * 2 + DB * Hq_d * 4 + \
        int(((L + 15) // 16).sum()) * 4 + DB * 4
    # compaction bytes: the table rows and every event's keep flags read once,
    # the compacted rows and lengths written once
    R = db.keeps.shape[0]
    comp_bytes = DB * MB * 4 + R * DB * MB + DB * MB * 4 + DB * 8

    stream = torch.cuda.current_stream()

    def step(tm=None):
        def t0():
            return tm.start() if tm else None

        def t1(ev, name):
            if tm:
                tm.stop(ev, name)
        ev = t0()
        ks.ks_evict_attn_fwd_rope(q, k, v, e, pos, q_rot=q_rot, k_rot=k_rot, out=o, lse=lse,
                                  ws=ws_f, stream=stream)
        t1(ev, "attn_fwd")
        ev = t0()
        ks.ks_evict_attn_bwd_rope(q_rot, k_rot, v, e, pos, o, lse, do, dq=dq, dk=dk, dv=dv,
                                  ws=ws_b, stream=stream)
        t1(ev, "attn_bwd")
        ev = t0()
        # the step's compaction events, applied together in one launch
        ks.ks_compact_block_table_rounds(table0, nblk0, keeps_all, tbufs[0], nbufs[0],
                                         stream=stream)
        src = tbufs[0]
        t1(ev, "compact")
        ev = t0()
        # the new token's k rotated and written by the append, the query
        # rotated inside the decode kernel
        ks.ks_append_kv(k4, v4, pos4f, src, seq_lens, kp, vp, stream=stream)
        ks.ks_paged_decode_rope(q4[:, 0], pos4f, kp, vp, src, seq_lens, out=out4, lse=lse4,
                                ws=ws_d, stream=stream)
        t1(ev, "decode")

    # q4[:, 0] is a view of a contiguous [B, 1, Hq, D] tensor: contiguous as [B, Hq, D]
    assert q4[:, 0].is_contiguous()

    if args.copy_calibration_mib > 0:
        nb = args.copy_calibration_mib << 20
        src_c = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst_c = torch.empty_like(src_c)
        torch.cuda.synchronize()
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tm = Timer(torch)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step(tm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    tot = tm.totals()

    # standalone compaction scan of 2^26 table entries (16384 rows x 4096),
    # one event, 70% of blocks kept: a bandwidth-meaningful size for the
    # prefix-scan kernel (not part of the step)
    crng = np.random.default_rng(4242)
    CB, CM = 16384, 4096
    ctab = torch.from_numpy(crng.integers(0, 2**31 - 1, size=(CB, CM), dtype=np.int32)).to(dev)
    ckeep = torch.from_numpy((crng.random((CB, CM)) < 0.7).astype(np.uint8)).to(dev)
    cn = torch.full((CB,), CM, dtype=torch.int32, device=dev)
    cout, cnout = torch.empty_like(ctab), torch.empty_like(cn)
    ks.ks_compact_block_table(ctab, cn, ckeep, cout, cnout, stream=stream)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        ks.ks_compact_block_table(ctab, cn, ckeep, cout, cnout, stream=stream)
    c1.record()
    torch.cuda.synchronize()
    scan_ms = c0.elapsed_time(c1) / 10
    scan_bytes = CB * CM * (4 + 1 + 4) + CB * 8
    del ctab, ckeep, cout
    K = args.steps
    ms = {kk: vv / K for kk, vv in tot.items()}
    attn_ms = ms["attn_fwd"] + ms["attn_bwd"]
    tflops = (flops_fwd + flops_bwd) / (attn_ms * 1e-3) / 1e12
    dec_gbs = (dec_bytes + comp_bytes) / ((ms["decode"] + ms["compact"]) * 1e-3) / 1e9
    parts = {
        "attn_fwd": {"bound": "mfma", "ms": ms["attn_fwd"],
                     "achieved": flops_fwd / (ms["attn_fwd"] * 1e-3) / 1e12,
                     "unit": "TFLOP/s"},
        "attn_bwd": {"bound": "mfma", "ms": ms["attn_bwd"],
                     "achieved": flops_bwd / (ms["attn_bwd"] * 1e-3) / 1e12,
                     "unit": "TFLOP/s"},
        "decode": {"bound": "hbm", "ms": ms["decode"],
                   "achieved": dec_bytes / (ms["decode"] * 1e-3) / 1e9, "unit": "GB/s"},
        "compact": {"bound": "hbm", "ms": ms["compact"],
                    "achieved": comp_bytes / (ms["compact"] * 1e-3) / 1e9, "unit": "GB/s"},
        "compact_2^26": {"bound": "hbm", "ms": scan_ms,
                         "achieved": scan_bytes / (scan_ms * 1e-3) / 1e9, "unit": "GB/s"},
    }
    for p in parts.values():
        peak = MFMA_BF16_PEAK_TFLOPS if p["bound"] == "mfma" else HBM_PEAK_GBS
        p["frac"] = p["achieved"] / peak
    # executed MFMA work (tile granularity) next to the useful work
    parts["attn_fwd"]["executed_tflop"] = ex_fwd / 1e12
    parts["attn_fwd"]["executed_over_useful"] = ex_fwd / flops_fwd
    parts["attn_fwd"]["executed_tflops_per_s"] = ex_fwd / (ms["attn_fwd"] * 1e-3) / 1e12
    parts["attn_bwd"]["executed_tflop"] = (ex_dq + ex_dkdv) / 1e12
    parts["attn_bwd"]["executed_over_useful"] = (ex_dq + ex_dkdv) / flops_bwd
    parts["attn_bwd"]["executed_tflops_per_s"] = (ex_dq + ex_dkdv) / (ms["attn_bwd"] * 1e-3) / 1e12
    dom = max(("attn_fwd", "attn_bwd"), key=lambda x: ms[x])
    result = {
        "metric": "eviction-masked attn fwd+bwd TFLOP/s @32k trace; paged-decode HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded traces and N(0,1)*0.5 tensors; no dataset or weights)",
        "config": {
            "workload": "4 x 32768-token summary-compaction traces (P=512, B=8192, o=1024, "
                        "s=512), 32 q / 8 kv heads, D=128, fwd+bwd; plus paged decode of 64 "
                        "compacted caches (4k-16k live tokens, 1-6 events), 32 q / 8 kv heads",
            "global_batch": B, "seq_len": N, "parallelism": "single GPU",
            "live_pairs_per_head": pairs, "causal_fraction": round(pairs / causal_pairs, 4),
        },
        "decode_hbm_gbs": round(dec_gbs, 1),
        "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "stage_ms": {kk: round(vv, 4) for kk, vv in ms.items()},
        "roofline": {
            "kernel": f"ks_{'evict_attn_bwd' if dom == 'attn_bwd' else 'evict_attn_fwd'}_rope",
            "bound": "mfma",
            "achieved": round(parts[dom]["achieved"], 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(parts[dom]["frac"], 4),
            "traffic": stored_traffic(
                f"ks_{'evict_attn_bwd' if dom == 'attn_bwd' else 'evict_attn_fwd'}_rope"),
        },
        "stages": {kk: {x: (round(y, 4) if isinstance(y, float) else y) for x, y in vv.items()}
                   for kk, vv in parts.items()},
    }
    mfma = mfma_rate(ks, torch, stream)
    result["mfma_reference"] = mfma
    result["roofline"]["peak_measured"] = mfma["tflops"]
    result["roofline"]["frac_of_measured"] = round(parts[dom]["achieved"] / mfma["tflops"], 4)
    for p in parts.values():
        if p["bound"] == "mfma":
            p["frac_of_measured"] = round(p["achieved"] / mfma["tflops"], 4)
    result["fused_dq_atomics_probe"] = dq_atomics_probe(ks, torch, stream, e_np, trn,
                                                      ms["attn_bwd"])
    result["hbm_reference"] = hbm_reference(torch, stream)
    result["single_token_blocks"] = token_granular_decode(ks, torch, stream, dec)
    result["toy_stack"] = toy_stack_mismatch(torch)
    result["reprefill_counterfactual"] = reprefill_counterfactual(
        ks, torch, traces, q, k, v, do, stream, ms, pairs, trn)
    result["long_mixed_64k"] = long_mixed_64k(ks, torch, stream)
    if not args.no_cpu_baseline:
        small = small_configs_gpu(ks, torch, stream)
        result["cpu_baseline"] = cpu_baseline(traces, seeds, trn, args.cpu_seconds)
        dec_gpu = dict(db=db, kp=kp, vp=vp, q=q4[:, 0], k_new=k4, v_new=v4, pos=db.pos,
                       out=out4, lse=lse4, table=tbufs[0], ms=ms["compact"] + ms["decode"])
        result["cpu_baseline"]["per_config"] = cpu_per_config(
            small, result["cpu_baseline"], traces, trn, attn_ms, dec_gpu,
            result["long_mixed_64k"])
        for key in ("_n", "_heads", "_seconds"):
            result["cpu_baseline"].pop(key)
    print(json.dumps(result), flush=True)


def hbm_reference(torch, stream, nbytes=2 << 30, reps=5):
    """What plain library kernels reach on this GPU's HBM, as context for the
    decode and compaction figures: a device-to-device copy (read + write) and
    a full read of 2 GiB (fp32 sums of 4096 rows, the fastest of torch's
    reductions here; a flat sum to one value reads at about two thirds of it)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    rows = src.view(4096, -1)
    out = {}
    for name, fn, traffic in (("copy", lambda: dst.copy_(src), 2 * nbytes),
                              ("read", lambda: rows.sum(dim=1), nbytes)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[f"{name}_gbs"] = round(traffic / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)
    del src, dst
    return out


def token_granular_decode(ks, torch, stream, cfg, reps=5):
    """The decode step of the 64-sequence batch with single-token blocks (the
    SGLang setup: token tables, no padding): every event compacts the token
    tables (all events in one launch, rows of up to 65k entries), then RoPE of q,
    append of the new token and the decode.  Timed apart from the step; HBM
    bytes as for the 16-token decode, with one table entry per token."""
    from workloads import build_decode_batch, normal_tensor, workload_rng

    db = build_decode_batch(workload_rng(cfg), cfg.batch, block=1)
    B, MT = db.table0.shape
    NT = db.num_pool_blocks
    Hq, Hkv, D = cfg.Hq, cfg.Hkv, cfg.D
    bf = torch.bfloat16
    dev = "cuda"
    kp = normal_tensor((NT, Hkv, D), 8001, 0.5, bf, dev)
    vp = normal_tensor((NT, Hkv, D), 8002, 0.5, bf, dev)
    q = normal_tensor((B, 1, Hq, D), 8003, 0.5, bf, dev)
    k_new = normal_tensor((B, Hkv, D), 8004, 0.5, bf, dev)
    v_new = normal_tensor((B, Hkv, D), 8005, 0.5, bf, dev)
    pos = torch.from_numpy(db.pos.astype(np.int32)).to(dev)
    table0 = torch.from_numpy(db.table0).to(dev)
    n0 = torch.from_numpy(db.nblk0).to(dev)
    keeps = torch.from_numpy(np.ascontiguousarray(db.keeps)).to(dev)     # [R, B, MT]
    R = keeps.shape[0]
    tb, nb = torch.empty_like(table0), torch.empty_like(n0)
    seq_lens = torch.from_numpy((db.live_len + 1).astype(np.int32)).to(dev)
    out = torch.empty((B, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(ks.ks_paged_decode_bs1_workspace(B, Hq, D, MT), dtype=torch.uint8,
                     device=dev)
    q0 = q[:, 0]

    def compact():
        # the pending events applied together in one launch
        ks.ks_compact_block_table_rounds(table0, n0, keeps, tb, nb, stream=stream)
        return tb

    def decode(tab):
        ks.ks_append_kv_bs1(k_new, v_new, pos, tab, seq_lens, kp, vp, stream=stream)
        ks.ks_paged_decode_rope(q0, pos, kp, vp, tab, seq_lens, out=out, lse=lse, ws=ws,
                                stream=stream)
    tab = compact()
    decode(tab)
    torch.cuda.synchronize()
    # steps back to back on the stream, as the 16-token step runs (no host
    # synchronisation between them, so no launch latency inside the stages)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record(stream)
        tab = compact()
        ev[r][1].record(stream)
        decode(tab)
        ev[r][2].record(stream)
    torch.cuda.synchronize()
    t_c = sum(x[0].elapsed_time(x[1]) for x in ev) / reps
    t_d = sum(x[1].elapsed_time(x[2]) for x in ev) / reps
    L = db.live_len.astype(np.int64) + 1
    dec_bytes = int((L * Hkv * D * 2 * 2).sum()) + B * Hq * D * 2 + \
        2 * 2 * B * Hkv * D * 2 + B * Hq * D * 2 + B * Hq * 4 + int(L.sum()) * 4 + B * 4
    # the table rows and every event's keep flags read once, the rows and
    # lengths written once
    comp_bytes = B * MT * 4 + R * B * MT + B * MT * 4 + B * 8
    return {
        "workload": "64 token-table caches (4k-16k live tokens at any length, 1-6 events "
                    "of token runs, applied in one launch), 32 q / 8 kv heads, D=128",
        "events": R,
        "table_entries": int(MT),
        "compact_ms": round(t_c, 4),
        "decode_ms": round(t_d, 4),
        "compact_gbs": round(comp_bytes / (t_c * 1e-3) / 1e9, 1),
        "decode_gbs": round(dec_bytes / (t_d * 1e-3) / 1e9, 1),
        "decode_plus_compact_frac": round((dec_bytes + comp_bytes) / ((t_c + t_d) * 1e-3)
                                          / 1e9 / HBM_PEAK_GBS, 4),
    }


def toy_stack_mismatch(torch):
    """A 3-layer random-weight decoder over the path: the masked training pass
    and token-by-token generation over compacted paged caches on one 1024-token
    trace (2+ events); the KL divergence of their next-token distributions is
    the trainer/generator mismatch the pages quote (about 0.001 for theirs)."""
    from kv_cache_compaction_amd.toy_stack import ToyStack
    from workloads import ToyShape, build_trace, toy_tokens, toy_weights

    shape = ToyShape()
    tr = build_trace(np.random.default_rng(21), 1024, 64, 512, "recent", turn_len=(48, 160))
    w = toy_weights(shape, 21)
    stack = ToyStack(w, shape.Hq, shape.Hkv, shape.D)
    tok = torch.from_numpy(toy_tokens(shape, tr.N, 21)).cuda()
    e = torch.from_numpy(tr.e.astype(np.int32)).cuda()
    stack.train_logits(tok, e)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    lt = stack.train_logits(tok, e)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ld = stack.decode_logits(tok, tr.evicted)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    lp, lq = torch.log_softmax(lt.double(), -1), torch.log_softmax(ld.double(), -1)
    kl = (lp.exp() * (lp - lq)).sum(-1)
    return {
        "model": f"{shape.layers} layers, d_model {shape.d_model}, {shape.Hq} q / {shape.Hkv} kv "
                 f"heads, D {shape.D}, random weights",
        "tokens": int(tr.N), "events": len(tr.events),
        "mismatch_kl_mean": float(kl.mean()), "mismatch_kl_max": float(kl.max()),
        "train_pass_ms": round((t1 - t0) * 1e3, 2), "generation_ms": round((t2 - t1) * 1e3, 1),
    }


def reprefill_counterfactual(ks, torch, traces, q, k, v, do, stream, ms, pairs, cfg,
                             reps=3):
    """Time what re-prefill compaction would run on the same rollouts (paper
    page, Fig. 2A and Fig. 3): after every event the kept tokens are processed
    again, as the start of a new causal trace.  The segments are packed end to
    end (each key evicted at its segment's end), so one masked fwd+bwd launch
    computes every segment's causal attention; compared with the single
    masked pass over the rollout that the step times."""
    from workloads import reprefill_pack, reprefill_segments

    B, N, Hq, Hkv, D = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    packs = [reprefill_pack(tr) for tr in traces]
    L = max(len(p[0]) for p in packs)
    packs = [reprefill_pack(tr, L) for tr in traces]
    dev = q.device
    idx = torch.from_numpy(np.stack([p[0] for p in packs])).to(dev)
    ep = torch.from_numpy(np.stack([p[1] for p in packs])).to(dev)
    gather = lambda t: torch.stack([t[b, idx[b]] for b in range(B)]).contiguous()
    qp, kp, vp, dop = gather(q), gather(k), gather(v), gather(do)
    op = torch.empty_like(qp)
    lsep = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    dqp, dkp, dvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
    # the same fused entry points as the step; kept tokens keep their
    # original (logical) positions in every segment
    posp = idx.to(torch.int32).contiguous()
    qr, kr = torch.empty_like(qp), torch.empty_like(kp)
    lib = ks.load_library()
    wsf = torch.empty(lib.ks_evict_attn_fwd_rope_workspace(B, L, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=dev)
    wsb = torch.empty(lib.ks_evict_attn_bwd_rope_workspace(B, L, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=dev)

    def run():
        ks.ks_evict_attn_fwd_rope(qp, kp, vp, ep, posp, q_rot=qr, k_rot=kr, out=op, lse=lsep,
                                  ws=wsf, stream=stream)
        ks.ks_evict_attn_bwd_rope(qr, kr, vp, ep, posp, op, lsep, dop, dq=dqp, dk=dkp, dv=dvp,
                                  ws=wsb, stream=stream)
    run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_rp = ev0.elapsed_time(ev1) / reps
    segs = [reprefill_segments(tr) for tr in traces]
    pairs_rp = sum(len(x) * (len(x) + 1) // 2 for sg in segs for x in sg)
    toks = sum(len(x) for sg in segs for x in sg)
    t_ks = ms["attn_fwd"] + ms["attn_bwd"]
    ev = [len(tr.events) for tr in traces]
    return {
        "what": "masked fwd+bwd over every re-prefill segment (kept tokens processed "
                "again after each event) vs one masked pass over the rollout",
        "packed_len": int(L),
        "events_per_trace": ev,
        "fig3_factor": round(N / (cfg.budget - (cfg.overlap + cfg.summary)), 3),
        "tokens_ratio": round(toks / (B * N), 4),
        "live_pairs_ratio": round(pairs_rp / pairs, 4),
        "ms_fwd_bwd": round(t_rp, 3),
        "ms_fwd_bwd_kv_streams": round(t_ks, 3),
        "time_ratio": round(t_rp / t_ks, 4),
        "tflops_useful": round(14.0 * D * pairs_rp * Hq / (t_rp * 1e-3) / 1e12, 2),
    }


def long_mixed_64k(ks, torch, stream, reps=5):
    """Masked fwd+bwd of the long mixed workload: 8 traces of 65,536 tokens
    compacted by sliding window, prompt+recent and summary in turn, 64 q /
    8 kv heads, D = 128.  Median over reps of each pass, timed with HIP
    events on the library's stream; useful TFLOP/s with the step's
    convention (RoPE fused into the timed forward and backward).  Then the
    traces continued by 256 decode steps (long_mixed_decode)."""
    from workloads import LONG_MIXED_64K, config_trace_batch, normal_tensor, stacked_e

    cfg = LONG_MIXED_64K
    traces, seeds = config_trace_batch(cfg)
    e_np = stacked_e(traces)
    B, N, Hq, Hkv, D = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    dev, bf = "cuda", torch.bfloat16
    q = normal_tensor((B, N, Hq, D), seeds["q"], cfg.value_scale, bf, dev)
    k = normal_tensor((B, N, Hkv, D), seeds["k"], cfg.value_scale, bf, dev)
    v = normal_tensor((B, N, Hkv, D), seeds["v"], cfg.value_scale, bf, dev)
    do = normal_tensor((B, N, Hq, D), seeds["do"], cfg.value_scale, bf, dev)
    e = torch.from_numpy(e_np).to(dev)
    pos = torch.arange(N, dtype=torch.int32, device=dev)[None].repeat(B, 1).contiguous()
    q_rot, k_rot = torch.empty_like(q), torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lib = ks.load_library()
    wsf = torch.empty(lib.ks_evict_attn_fwd_rope_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=dev)
    wsb = torch.empty(lib.ks_evict_attn_bwd_rope_workspace(B, N, Hq, Hkv, D, ks.KS_BF16),
                      dtype=torch.uint8, device=dev)
    fwd = lambda: ks.ks_evict_attn_fwd_rope(q, k, v, e, pos, q_rot=q_rot, k_rot=k_rot, out=o,
                                            lse=lse, ws=wsf, stream=stream)
    bwd = lambda: ks.ks_evict_attn_bwd_rope(q_rot, k_rot, v, e, pos, o, lse, do, dq=dq, dk=dk,
                                            dv=dv, ws=wsb, stream=stream)
    fwd()
    bwd()
    torch.cuda.synchronize()
    t_f, t_b = [], []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        fwd()
        ev[1].record(stream)
        bwd()
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_f.append(ev[0].elapsed_time(ev[1]))
        t_b.append(ev[1].elapsed_time(ev[2]))
    mf, mb = float(np.median(t_f)), float(np.median(t_b))
    pairs = live_pairs(e_np)
    useful_f = 4.0 * D * pairs * Hq
    useful_b = 10.0 * D * pairs * Hq
    ex_f, ex_q, ex_kv = executed_flops(e_np, Hq, Hkv, D)
    out = {
        "workload": "8 x 65536-token traces (sliding window, prompt+recent, summary "
                    "o=2048 s=1024; P=512, B=16384), 64 q / 8 kv heads, D=128, fwd+bwd",
        "events_per_trace": [len(tr.events) for tr in traces],
        "live_pairs_per_head": int(pairs),
        "ms_fwd": round(mf, 3),
        "ms_bwd": round(mb, 3),
        "useful_tflop": round((useful_f + useful_b) / 1e12, 2),
        "tflops_useful": round((useful_f + useful_b) / ((mf + mb) * 1e-3) / 1e12, 2),
        "frac_of_bf16_peak": round((useful_f + useful_b) / ((mf + mb) * 1e-3) / 2516.6e12, 4),
        "fwd_tflops_useful": round(useful_f / (mf * 1e-3) / 1e12, 2),
        "bwd_tflops_useful": round(useful_b / (mb * 1e-3) / 1e12, 2),
        "executed_over_useful": round((ex_f + ex_q + ex_kv) / (useful_f + useful_b), 4),
    }
    del q, do, o, dq, dk, dv, wsf, wsb, q_rot
    torch.cuda.empty_cache()
    # the traces continued by 256 decoded tokens with a forced event after 128
    out["decode_256"] = long_mixed_decode(ks, torch, stream, traces, cfg, k_rot, v)
    del k, v, k_rot
    torch.cuda.empty_cache()
    return out


def long_mixed_decode(ks, torch, stream, traces, cfg, k_rot, v, ndec=256, event_after=128,
                      reps=3):
    """The long mixed traces continued by decoding, as the decode step runs:
    each trace's live set (keys as the training pass rotated them) in a
    16-token-block pool with ndec / 16 fresh blocks, then ndec steps over all
    traces of ks_append_kv (the new key rotated at position N + s) and
    ks_paged_decode_rope (the query rotated in the kernel), with the forced
    compaction event after event_after tokens (ks_compact_block_table).  The
    ndec steps run back to back on the stream between two HIP events (median
    of reps); tokens, lengths and positions are resident before the timed
    region, and the tables are reset between reps outside it."""
    from workloads import BLOCK, continuation_layout, normal_tensor

    B, N, Hq, Hkv, D = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    dev, bf = "cuda", torch.bfloat16
    lay = continuation_layout(traces, N, ndec, event_after, np.random.default_rng(5005))
    NB, MB = lay.num_pool_blocks, lay.table0.shape[1]
    kp = torch.zeros((NB, Hkv, BLOCK, D), dtype=bf, device=dev)
    vp = torch.zeros_like(kp)
    for b in range(B):
        L = int(lay.live_len[b])
        blk = torch.from_numpy(np.repeat(lay.table0[b, :L // BLOCK], BLOCK).astype(np.int64)).to(dev)
        slot = torch.arange(L, device=dev) % BLOCK
        tok = torch.from_numpy(lay.live_tok[b].astype(np.int64)).to(dev)
        kp[blk, :, slot] = k_rot[b, tok]
        vp[blk, :, slot] = v[b, tok]
    qn = normal_tensor((ndec, B, Hq, D), 7001, 0.5, bf, dev)
    kn = normal_tensor((ndec, B, Hkv, D), 7002, 0.5, bf, dev)
    vn = normal_tensor((ndec, B, Hkv, D), 7003, 0.5, bf, dev)
    lens = np.empty((ndec, B), np.int64)
    length = lay.live_len.astype(np.int64)
    for s in range(ndec):
        if s == event_after:
            length = length - lay.ev_tokens
        length = length + 1
        lens[s] = length
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    posn = torch.arange(N, N + ndec, dtype=torch.int32, device=dev)[:, None].repeat(1, B)
    table0 = torch.from_numpy(lay.table0).to(dev)
    nblk0 = torch.from_numpy(lay.nblk0).to(dev)
    keep = torch.from_numpy(lay.keep).to(dev)
    tab, nblk = torch.empty_like(table0), torch.empty_like(nblk0)
    tab2, nblk2 = torch.empty_like(table0), torch.empty_like(nblk0)
    out = torch.empty((B, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(ks.ks_paged_decode_workspace(B, Hq, D, MB * BLOCK), dtype=torch.uint8,
                     device=dev)

    def steps():
        t = tab
        for s in range(ndec):
            if s == event_after:
                ks.ks_compact_block_table(tab, nblk, keep, tab2, nblk2, stream=stream)
                t = tab2
            ks.ks_append_kv(kn[s], vn[s], posn[s], t, seq[s], kp, vp, stream=stream)
            ks.ks_paged_decode_rope(qn[s], posn[s], kp, vp, t, seq[s], out=out, lse=lse, ws=ws,
                                    stream=stream)

    times = []
    for r in range(reps + 1):                    # the first pass is a warm-up
        tab.copy_(table0)
        nblk.copy_(nblk0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        steps()
        e1.record(stream)
        torch.cuda.synchronize()
        if r:
            times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    # per step as for the 64-sequence decode: K and V of every live token,
    # q, the new k and v (read and written), out, lse, table entries, lengths
    per_step = [int((Ls * Hkv * D * 2 * 2).sum()) + B * Hq * D * 2 + 2 * 2 * B * Hkv * D * 2 +
                B * Hq * D * 2 + B * Hq * 4 + int(((Ls + 15) // 16).sum()) * 4 + B * 4
                for Ls in lens]
    dec_bytes = sum(per_step)
    del kp, vp, ws
    return {"steps": ndec, "event_after": event_after,
            "evicted_tokens_per_trace": [int(x) for x in lay.ev_tokens],
            "ms_total": round(ms, 3), "us_per_step": round(ms * 1e3 / ndec, 1),
            "hbm_gbs": round(dec_bytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(dec_bytes / (ms * 1e-3) / 8e12, 4)}


def mfma_rate(ks, torch, stream, workgroups=2048, iters=2500):
    """bf16 MFMA rate of a loop of nothing but 32x32x16 MFMAs at the attention
    kernels' occupancy (8 waves per workgroup, 2 per SIMD), timed with HIP
    events: the rate this GPU sustains at the clock it holds under such a
    load, beside the published dense peak."""
    seed = torch.full((1024,), 0.01, dtype=torch.bfloat16, device="cuda")
    sink = torch.empty(workgroups * 512, dtype=torch.float32, device="cuda")
    run = lambda: ks.ks_measure_mfma_bf16(seed, sink, workgroups, iters, stream=stream)
    run()
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = ks.ks_measure_mfma_flops(workgroups, iters)
    return {"what": "v_mfma_f32_32x32x16_bf16 only, 4 independent chains per wave, "
                    "2 waves per SIMD", "workgroups": workgroups, "ms": round(ms, 3),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_published_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                            4)}


def dq_atomics_probe(ks, torch, stream, e_np, cfg, bwd_ms, reps=3):
    """The dQ adds a single-pass backward would issue from the dK/dV walk on
    the same traces (every 256-key workgroup adding a 32 x 128 fp32 partial
    per query chunk and head, global fp32 atomics), timed alone: the case
    against fusing dQ into the dK/dV kernel."""
    B, N, Hq, Hkv = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv
    G = Hq // Hkv
    nkt = (N + 255) // 256
    cend = np.zeros((B, nkt), np.int32)
    for b in range(B):
        em = np.maximum.reduceat(e_np[b].astype(np.int64), np.arange(0, N, 256))
        cend[b] = (np.minimum(N, em) + 31) // 32
    units = int(sum(max(0, int(cend[b, t]) - 8 * t) for b in range(B) for t in range(nkt))) * G * Hkv
    acc = torch.zeros((B, N, Hq, 128), dtype=torch.float32, device="cuda")
    cg = torch.from_numpy(cend).cuda()
    run = lambda: ks.ks_measure_dq_atomics(acc, cg, Hkv, stream=stream)
    ms = _median_ms(torch, stream, run, reps)
    nbytes = units * 32 * 128 * 4
    del acc
    torch.cuda.empty_cache()
    return {"what": "fp32 atomic dQ adds of a dK/dV-walk backward (256-key workgroups, "
                    "32-row chunks), nothing else", "chunk_head_units": units,
            "atomic_bytes": nbytes, "ms": round(ms, 3),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "backward_ms_two_kernels": round(bwd_ms, 3)}


def _median_ms(torch, stream, fn, reps):
    fn()
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    return float(np.median(t))


def small_configs_gpu(ks, torch, stream, reps=20):
    """The two small workloads on the GPU, timed (median of reps) and kept
    for the oracle beside them: the 512-token fp32 trace (RoPE, forward,
    compaction of its 32-block table) and the 4k bf16 trace (RoPE, forward,
    backward).  Inputs are drawn on the host (numpy), as the tests draw them."""
    from workloads import TINY_F32, TRAIN_4K, config_trace_batch, normal_tensor, stacked_e
    from workloads import trace_blocks_keep

    out = {}
    for cfg in (TINY_F32, TRAIN_4K):
        traces, seeds = config_trace_batch(cfg)
        e_np = stacked_e(traces)
        B, N, Hq, Hkv, D = cfg.batch, cfg.N, cfg.Hq, cfg.Hkv, cfg.D
        dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        raw = {nm: normal_tensor(shp, seeds[nm], cfg.value_scale, dt)
               for nm, shp in (("q", (B, N, Hq, D)), ("k", (B, N, Hkv, D)),
                               ("v", (B, N, Hkv, D)), ("do", (B, N, Hq, D)))}
        g = {nm: t.cuda() for nm, t in raw.items()}
        qg, kg = g["q"].clone(), g["k"].clone()
        e = torch.from_numpy(e_np).cuda()
        pos = torch.arange(N, dtype=torch.int32, device="cuda")[None].repeat(B, 1).contiguous()
        o = torch.empty_like(qg)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(g["v"])
        rec = {"cfg": cfg, "traces": traces, "raw": raw}
        if cfg.backward:
            # the step's fused entry points (qg, kg receive the rotated q, k;
            # dq, dk are gradients of the unrotated projections)
            def run():
                ks.ks_evict_attn_fwd_rope(g["q"], g["k"], g["v"], e, pos, q_rot=qg, k_rot=kg,
                                          out=o, lse=lse, stream=stream)
                ks.ks_evict_attn_bwd_rope(qg, kg, g["v"], e, pos, o, lse, g["do"], dq=dq, dk=dk,
                                          dv=dv, stream=stream)
        else:
            perm = np.random.default_rng(7).permutation(32).astype(np.int32)[None]
            keep = trace_blocks_keep(traces[0])[None]
            tg, ng = torch.from_numpy(perm).cuda(), torch.tensor([32], dtype=torch.int32).cuda()
            kpg = torch.from_numpy(keep).cuda()
            tout, nout = torch.empty_like(tg), torch.empty_like(ng)
            rec.update(table=perm, keep=keep)

            def run():
                qg.copy_(g["q"])
                kg.copy_(g["k"])
                ks.ks_rope_logical(qg, kg, pos, stream=stream)
                ks.ks_evict_attn_fwd(qg, kg, g["v"], e, out=o, lse=lse, stream=stream)
                ks.ks_compact_block_table(tg, ng, kpg, tout, nout, stream=stream)
        rec["gpu_ms"] = _median_ms(torch, stream, run, reps)
        rec["o"], rec["lse"] = o.cpu(), lse.cpu()
        if cfg.backward:
            rec["dq"], rec["dk"], rec["dv"] = dq.cpu(), dk.cpu(), dv.cpu()
        else:
            rec["table_out"], rec["n_out"] = tout.cpu().numpy(), nout.cpu().numpy()
        out[cfg.name] = rec
    return out


def oracle_formed_entries(e_row, n, chunk=512):
    """(row, key) entries the oracle forms for one query head over rows
    [0, n) of a trace: per chunk of rows [i0, i1) it forms the key columns
    live for some row of the chunk, {j < i1 : e_j > i0}.  Its time per head
    follows this count, which scales a sample to a full configuration."""
    e_row = np.asarray(e_row, dtype=np.int64)
    tot = 0
    for i0 in range(0, n, chunk):
        i1 = min(n, i0 + chunk)
        tot += (i1 - i0) * int((e_row[:i1] > i0).sum())
    return tot


def cpu_per_config(small, base, traces, cfg3, gpu3_ms, dec, mixed):
    """The fp64 oracle beside the GPU on every workload: the 512-token, 4k and
    decode workloads in full (with the GPU's error against it), the 32k and
    64k workloads extrapolated from a sample by the oracle's formed entries."""
    import torch

    import oracle as O
    from workloads import LONG_MIXED_64K, config_trace_batch, stacked_e

    f64 = lambda t: t.to(torch.float64).numpy()
    res = {}
    # --- 512-token fp32 trace: RoPE, forward, compaction of its 32-block table
    r = small["tiny-f32"]
    c = r["cfg"]
    e = stacked_e(r["traces"]).astype(np.int64)
    t0 = time.perf_counter()
    pos = np.arange(c.N)[None]
    qr, kr = O.rope(f64(r["raw"]["q"]), pos), O.rope(f64(r["raw"]["k"]), pos)
    ro, rl = O.attn_fwd(qr, kr, f64(r["raw"]["v"]), e)
    rt, rn = O.compact_block_table(r["table"], np.array([32]), r["keep"])
    el = time.perf_counter() - t0
    res["tiny-f32"] = {
        "work": "RoPE + masked forward of 512 fp32 tokens + compaction of a 32-block table",
        "oracle_s": round(el, 4), "oracle_measured": "full", "gpu_ms": round(r["gpu_ms"], 4),
        "gpu_max_abs_err": {"o": float(np.abs(f64(r["o"]) - ro).max()),
                            "lse": float(np.abs(f64(r["lse"]) - rl).max())},
        "table_bit_exact": bool(np.array_equal(r["table_out"], rt)
                                and np.array_equal(r["n_out"], rn)),
    }
    # --- 4k bf16 trace: RoPE, forward, backward (every head)
    r = small["train-4k"]
    c = r["cfg"]
    e = stacked_e(r["traces"]).astype(np.int64)
    t0 = time.perf_counter()
    pos = np.arange(c.N)[None]
    qr, kr = O.rope(f64(r["raw"]["q"]), pos), O.rope(f64(r["raw"]["k"]), pos)
    vv, dd = f64(r["raw"]["v"]), f64(r["raw"]["do"])
    ro, rl = O.attn_fwd(qr, kr, vv, e)
    rdq, rdk, rdv = O.attn_bwd(qr, kr, vv, e, dd)
    el = time.perf_counter() - t0
    # the GPU's dq, dk are gradients of the unrotated projections
    rdq, rdk = O.rope(rdq, pos, inverse=True), O.rope(rdk, pos, inverse=True)
    err = {nm: float(np.abs(f64(r[nm]) - ref).max())
           for nm, ref in (("o", ro), ("lse", rl), ("dq", rdq), ("dk", rdk), ("dv", rdv))}
    res["train-4k"] = {"work": "RoPE + masked forward + backward, 4096 tokens, 8 q / 2 kv heads",
                       "oracle_s": round(el, 3), "oracle_measured": "full",
                       "gpu_ms": round(r["gpu_ms"], 4), "gpu_max_abs_err": err}
    # --- 32k summary traces: from the sample the headline baseline timed
    full = sum(oracle_formed_entries(tr.e, cfg3.N) for tr in traces) * cfg3.Hq
    samp = oracle_formed_entries(traces[0].e, base["_n"]) * base["_heads"]
    est = base["_seconds"] * full / samp
    res["summary-32k"] = {
        "work": "RoPE + masked forward + backward, 4 x 32768 tokens, 32 q / 8 kv heads",
        "oracle_s": round(est, 1),
        "oracle_measured": f"extrapolated from the timed sample ({base['_n']} tokens of trace 0, "
                           f"{base['_heads']} heads: {base['_seconds']:.1f} s) by the oracle's "
                           f"formed (row, key) entries, x{full / samp:.1f}",
        "gpu_ms": round(gpu3_ms, 3)}
    # --- paged decode: the step's compaction events, append, decode (all 64)
    db = dec["db"]
    B, MB = db.table0.shape
    Hq, Hkv, D = dec["q"].shape[1], dec["kp"].shape[1], dec["q"].shape[2]
    L = (db.live_len + 1).astype(np.int64)
    t0 = time.perf_counter()
    rt, rn = db.table0, db.nblk0
    for x in range(db.keeps.shape[0]):
        rt, rn = O.compact_block_table(rt, rn, db.keeps[x])
    el_c = time.perf_counter() - t0
    need = [rt[b, :(int(L[b]) + 15) // 16] for b in range(B)]
    ids = np.unique(np.concatenate(need))
    idx = torch.from_numpy(ids.astype(np.int64)).cuda()
    kh = dec["kp"].index_select(0, idx).float().cpu().numpy()
    vh = dec["vp"].index_select(0, idx).float().cpu().numpy()
    where = {int(p): i for i, p in enumerate(ids)}
    rt2 = np.full_like(rt, -1)
    for b in range(B):
        rt2[b, :len(need[b])] = [where[int(p)] for p in need[b]]
    q_raw = dec["q"].float().cpu().numpy().astype(np.float64)
    k_raw = dec["k_new"].float().cpu().numpy().astype(np.float64)
    v_new = dec["v_new"].float().cpu().numpy()
    t0 = time.perf_counter()
    posd = db.pos.astype(np.int64)
    qrot = O.rope(q_raw[:, None], posd[:, None])[:, 0]
    krot = O.rope(k_raw[:, None], posd[:, None])[:, 0]
    for b in range(B):                      # the append: token L-1 of each sequence
        blk, slot = int(rt2[b, (L[b] - 1) // 16]), int((L[b] - 1) % 16)
        kh[blk, :, slot] = krot[b]
        vh[blk, :, slot] = v_new[b]
    ro, rl = O.paged_decode(qrot, kh, vh, rt2, L)
    el = el_c + time.perf_counter() - t0
    res["paged-decode"] = {
        "work": "1-6 compaction events + append + one decode step, 64 caches of 4k-16k tokens, "
                "32 q / 8 kv heads",
        "oracle_s": round(el, 3), "oracle_measured": "full",
        "gpu_ms": round(dec["ms"], 4),
        "gpu_max_abs_err": {"out": float(np.abs(dec["out"].float().cpu().numpy() - ro).max()),
                            "lse": float(np.abs(dec["lse"].cpu().numpy() - rl).max())},
        "table_bit_exact": bool(np.array_equal(dec["table"].cpu().numpy(), rt)),
    }
    del kh, vh
    # --- 64k mixed: one query head of trace 0 over its first 16384 tokens
    cfg5 = LONG_MIXED_64K
    tr5, seeds5 = config_trace_batch(cfg5)
    n = 16384
    rng = np.random.default_rng(5005)
    x = {nm: rng.standard_normal((1, n, 1, cfg5.D)) * cfg5.value_scale
         for nm in ("q", "k", "v", "do")}
    e5 = tr5[0].e[None, :n].astype(np.int64)
    t0 = time.perf_counter()
    pos = np.arange(n)[None]
    qr, kr = O.rope(x["q"], pos), O.rope(x["k"], pos)
    O.attn_fwd(qr, kr, x["v"], e5)
    O.attn_bwd(qr, kr, x["v"], e5, x["do"])
    el = time.perf_counter() - t0
    full5 = sum(oracle_formed_entries(tr.e, cfg5.N) for tr in tr5) * cfg5.Hq
    samp5 = oracle_formed_entries(tr5[0].e, n)
    res["long-mixed-64k"] = {
        "work": "masked forward + backward, 8 x 65536 tokens, 64 q / 8 kv heads",
        "oracle_s": round(el * full5 / samp5, 1),
        "oracle_measured": f"extrapolated from one query head over the first {n} tokens of "
                           f"trace 0 ({el:.1f} s) by the oracle's formed (row, key) entries, "
                           f"x{full5 / samp5:.0f}",
        "gpu_ms": round(mixed["ms_fwd"] + mixed["ms_bwd"], 2)}
    for v in res.values():
        v["gpu_speedup"] = round(v["oracle_s"] * 1e3 / v["gpu_ms"], 1)
    return res


def cpu_baseline(traces, seeds, cfg, budget_s):
    """Time the fp64 oracle (forward + backward on a prefix of one trace, one
    query head at a time, until about budget_s seconds have passed) on the
    host; report useful TFLOP/s with the GPU figure's flop convention."""
    import torch
    from threadpoolctl import threadpool_info

    import oracle as O
    from workloads import normal_tensor

    N, D, Hq, Hkv = cfg.N, cfg.D, cfg.Hq, cfg.Hkv
    G = Hq // Hkv
    tr = traces[0]
    e = tr.e[None].astype(np.int64)
    # raw projections of trace 0, kv head 0 (the generator draws whole tensors)
    bf = torch.bfloat16
    qa = normal_tensor((1, N, Hq, D), seeds["q"], cfg.value_scale, bf, "cuda")
    ka = normal_tensor((1, N, Hkv, D), seeds["k"], cfg.value_scale, bf, "cuda")
    va = normal_tensor((1, N, Hkv, D), seeds["v"], cfg.value_scale, bf, "cuda")
    da = normal_tensor((1, N, Hq, D), seeds["do"], cfg.value_scale, bf, "cuda")
    qh, kh, vh, dh = qa[:, :, :G], ka[:, :, :1], va[:, :, :1], da[:, :, :G]
    f = lambda t: t.to("cpu", torch.float64).numpy()
    q, k, v, do = f(qh), f(kh), f(vh), f(dh)
    # the GPU path on the same trace (whole trace, every head), for the error
    # of the sampled rows against the oracle
    import kv_cache_compaction_amd as ks
    eg = torch.from_numpy(tr.e[None].astype(np.int32)).cuda()
    pg = torch.arange(N, dtype=torch.int32, device="cuda")[None].contiguous()
    go, glse, qrg, krg = ks.ks_evict_attn_fwd_rope(qa, ka, va, eg, pg)
    gdq, gdk, gdv = ks.ks_evict_attn_bwd_rope(qrg, krg, va, eg, pg, go, glse, da)
    del qrg, krg
    torch.cuda.synchronize()
    pos = np.arange(N)[None]
    q, k = O.rope(q, pos), O.rope(k, pos)
    # prefix of the trace: rows < n only see keys < n, so the prefix is a
    # complete masked-attention problem of its own
    n = min(N, 16384)
    en = e[:, :n]
    pairs_n = int(O.eviction_mask(en[0], np.arange(n), n).sum())
    done_pairs = 0
    heads_used = 0
    ref = []
    t0 = time.perf_counter()
    while heads_used < G and (heads_used == 0 or time.perf_counter() - t0 < budget_s):
        h = heads_used
        qh1, doh1 = q[:, :n, h:h + 1], do[:, :n, h:h + 1]
        ro, rl = O.attn_fwd(qh1, k[:, :n], v[:, :n], en)
        rdq, rdk, rdv = O.attn_bwd(qh1, k[:, :n], v[:, :n], en, doh1)
        done_pairs += pairs_n
        heads_used += 1
        ref.append((ro, rl, rdq))
        rdk_sum = rdk if heads_used == 1 else rdk_sum + rdk
        rdv_sum = rdv if heads_used == 1 else rdv_sum + rdv
    el = time.perf_counter() - t0
    # rows < n of the GPU's full-trace outputs against the oracle's prefix;
    # the GPU's dq, dk are gradients of the unrotated projections
    unrot = lambda x: O.rope(x, pos[:, :n], inverse=True)
    ref = [(ro, rl, unrot(rdq)) for ro, rl, rdq in ref]
    if heads_used == G:
        rdk_sum = unrot(rdk_sum)
    err = {"o": 0.0, "lse": 0.0, "dq": 0.0}
    scale_ref = {"o": 0.0, "lse": 0.0, "dq": 0.0}
    for h, (ro, rl, rdq) in enumerate(ref):
        for name, got, want in (("o", go[0, :n, h], ro[0, :, 0]), ("lse", glse[0, h, :n], rl[0, 0]),
                                ("dq", gdq[0, :n, h], rdq[0, :, 0])):
            g = got.to("cpu", torch.float64).numpy()
            err[name] = max(err[name], float(np.abs(g - want).max()))
            scale_ref[name] = max(scale_ref[name], float(np.abs(want).max()))
    # dK, dV of the keys whose every query lies inside the prefix (evicted by
    # token n), summed over the kv group's query heads when all were timed
    if heads_used == G:
        done = np.flatnonzero(e[0, :n] <= n)
        for name, got, want in (("dk", gdk[0, done, 0], rdk_sum[0, done, 0]),
                                ("dv", gdv[0, done, 0], rdv_sum[0, done, 0])):
            g = got.to("cpu", torch.float64).numpy()
            err[name] = float(np.abs(g - want).max())
            scale_ref[name] = float(np.abs(want).max())
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(14.0 * D * done_pairs / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "host": f"{model}; {len(os.sched_getaffinity(0))} logical CPUs available",
        "sample": f"fp64 oracle forward + backward (dQ, dK, dV) of the first {n} tokens "
                  f"of trace 0, {heads_used} query head(s) of kv group 0: {done_pairs} live "
                  f"pairs in {el:.1f} s",
        "_n": n, "_heads": heads_used, "_seconds": el,
        "gpu_vs_oracle_on_sample": {
            "rows": n, "heads": heads_used,
            "keys_compared": int((e[0, :n] <= n).sum()) if heads_used == G else 0,
            "max_abs": {kk: round(vv, 6) for kk, vv in err.items()},
            "max_abs_of_reference": {kk: round(vv, 4) for kk, vv in scale_ref.items()},
        },
    }


if __name__ == "__main__":
    main()
