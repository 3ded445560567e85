#!/usr/bin/env python3
"""Benchmark of the AB-Attention sparse attention layer on one MI355X.

A step is one pass of the whole hot path over one synthetic layer with its
inputs resident in HBM:

    aba_score  (IBCS: k-means clustering, key pooling, block scores)
    aba_sample (SIP: inclusion probabilities, Philox draws, list compaction)
    aba_attend (block-sparse flash attention with inverse-inclusion weights)

The workload is the 32K-token single video DiT layer (batch 1, 12 heads,
head_dim 128, bf16, 21x30x52 latent grid, 10% key-block density); the steps
cycle through three seeded input sets so that no step finds its q and k in the
MALL.  ``value`` is the effective (dense-equivalent) throughput 4*B*H*N^2*D /
step time.  Printed as one JSON line, with the roofline of the dominant call
(aba_attend, measured with HIP events on the stream it runs on), untimed
selection diagnostics (dense attention mass kept by the ideal, IBCS, mean-pool
and sampled selections on sampled query blocks, and the attention error of the
sampled lists against hard top-K lists), the rate the bf16 matrix cores sustain
on register operands alone (the practical ceiling beside the quoted peak), and
the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload single_layer]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_sparse_attention_38_amd import aba, synth  # noqa: E402
from block_sparse_attention_38_amd.workloads import ALL, CLUSTERS, KMEANS_ITERS  # noqa: E402

METRIC = "ms/call and effective TFLOP/s of sparse attention, 32K-token video layer"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (vector)
ATTEND_SRC = os.path.join(ROOT, "block_sparse_attention_38_amd", "csrc", "attend.hip")
TRAFFIC_FILES = {128: os.path.join(ROOT, "profiles", "attend_single_layer_traffic.json"),
                 4: os.path.join(ROOT, "profiles", "attend_single_layer_4token_traffic.json")}


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def mfma_rate(iters: int, reps: int = 3) -> dict:
    """Sustained bf16 matrix-core rate (aba_mfma_rate: MFMAs on register operands
    only, two wavefronts per SIMD), on random operands and on zeros; the median
    of the reps after one untimed call each."""
    dev = torch.device("cuda:0")
    out = torch.empty(aba.MFMA_RATE_THREADS, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    res = {}
    for name, random in (("random", True), ("zero", False)):
        aba.mfma_rate(iters, random, out)
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            aba.mfma_rate(iters, random, out)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        res[f"{name}_tflops"] = iters * aba.MFMA_RATE_FLOP_PER_ITER / (float(np.median(ms)) * 1e-3) / 1e12
        res[f"{name}_ms"] = ms
    res["iters"] = iters
    res["random_frac_of_peak"] = res["random_tflops"] / PEAK_BF16_TFLOPS
    log(f"[bench] sustained bf16 MFMA (register operands only): random {res['random_tflops']:.0f} TFLOP/s "
        f"({res['random_frac_of_peak']:.3f} of peak), zeros {res['zero_tflops']:.0f} TFLOP/s")
    return res


def kept_flops(p, cnt: np.ndarray, idx: np.ndarray) -> float:
    """4 * D * sum over kept (query block, key block) pairs of valid queries x valid keys."""
    N, NB, NBk, kb = p.seq_len, p.n_blocks, p.n_key_blocks, p.key_block
    valid_q = np.minimum(128, N - 128 * np.arange(NB)).astype(np.float64)    # valid tokens per query block
    valid_k = np.minimum(kb, N - kb * np.arange(NBk)).astype(np.float64)     # valid tokens per key block
    total = 0.0
    flat_c = cnt.reshape(-1, NB)
    flat_i = idx.reshape(-1, NB, idx.shape[-1])
    for r in range(flat_c.shape[0]):
        for qb in range(NB):
            c = int(flat_c[r, qb])
            total += valid_q[qb] * valid_k[flat_i[r, qb, :c]].sum()
    return 4.0 * p.head_dim * total


def source_digest(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_entry(key_block: int = 128, path: str = None):
    """HBM traffic per attend call (bytes) of the 32K bf16 layer from the committed
    rocprofv3 counter runs for that key block size, if the kernel source has not
    changed since they were taken."""
    path = path or TRAFFIC_FILES.get(key_block)
    if path is None or not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("attend_src_sha256_16") != source_digest(ATTEND_SRC) or rec.get("key_block", 128) != key_block:
        return None
    return rec.get("bytes_per_launch")


def summarize_traffic(fetch_dir: str, write_dir: str, key_block: int, commands: list, out_dir: str = None):
    """Turn two rocprofv3 counter runs of ``bench.py --copy-calibration`` (one with
    FETCH_SIZE, one with WRITE_SIZE, KiB per dispatch) into the per-kernel HBM
    bytes of the 32K-token layer: each counter is scaled by what it reads for the
    run's plain 1 GiB device copy.  Writes profiles/hbm_traffic_single_layer*.md
    and the aba_attend record that traffic_entry() reads (tied to the hash of
    attend.hip)."""
    import csv
    import glob
    import re

    def load(d, counter):
        per, grid = {}, {}
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = re.sub(r"\(.*", "", r["Kernel_Name"].replace("aba::(anonymous namespace)::", "aba::"))
                per.setdefault(name, []).append(float(r["Counter_Value"]))
                grid[name] = r.get("Grid_Size", "")
        return per, grid

    fetch, grid = load(fetch_dir, "FETCH_SIZE")
    write, _ = load(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)

    def copy_kib(per):   # the calibration copy: the largest copy dispatch of the run
        vals = [v for n, vs in per.items() if "copyBuffer" in n for v in vs]
        return max(vals) if vals else 0.0

    f_copy, w_copy = copy_kib(fetch), copy_kib(write)
    if f_copy < gib_kib / 4 or w_copy < gib_kib / 4:
        raise SystemExit("no 1 GiB calibration copy in the counter runs (run bench.py with --copy-calibration)")
    fs, ws = gib_kib / f_copy, gib_kib / w_copy
    sfx = "" if key_block == 128 else "_4token"
    rows = []
    kernels = {}
    attend_kernels = ("aba::order_kernel",
                      "void aba::attend_bf16_kernel<128, false>" if key_block == 128 else "void aba::attend_fine_kernel<128>")
    for name in sorted(fetch, key=lambda n: -sum(fetch[n]) / len(fetch[n])):
        if "copyBuffer" in name:
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write.get(name, [0.0])) / max(1, len(write.get(name, [])))
        rows.append(f"| `{name}` | {grid.get(name, '')} | {fk:.0f} | {wk:.0f} | {fk * 1024 * fs / 1e6:.1f} | "
                    f"{wk * 1024 * ws / 1e6:.1f} |")
        if name in attend_kernels:
            kernels[name] = {"read_bytes": fk * 1024 * fs, "write_bytes": wk * 1024 * ws}
    if len(kernels) != 2:
        raise SystemExit(f"the counter runs lack the aba_attend kernels {attend_kernels}")
    md = [f"# HBM traffic per launch, single 32K layer, {key_block}-token key blocks", "",
          "Counter passes (each its own run, from /tmp with TMPDIR=/tmp; R = repository root), then the summary:", "",
          "```", *commands, "```", "",
          f"Scale factors from the plain 1 GiB device copy in the same runs (`--copy-calibration`): FETCH_SIZE reads "
          f"{f_copy:.0f} KiB for 1 GiB read (x{fs:.4f}), WRITE_SIZE reads {w_copy:.0f} KiB for 1 GiB written "
          f"(x{ws:.4f}).", "",
          "| kernel | grid | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | read MB (scaled) | written MB (scaled) |",
          "|---|---|---|---|---|---|", *rows]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    md_path = os.path.join(out_dir, f"hbm_traffic_single_layer{sfx}.md")
    json_path = os.path.join(out_dir, os.path.basename(TRAFFIC_FILES[key_block]))
    open(md_path, "w").write("\n".join(md) + "\n")
    rd = sum(k["read_bytes"] for k in kernels.values())
    wr = sum(k["write_bytes"] for k in kernels.values())
    rec = {"call": "aba_attend", "key_block": key_block, "kernels": kernels, "workload": "single_layer",
           "read_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr, "fetch_scale": fs, "write_scale": ws,
           "attend_src_sha256_16": source_digest(ATTEND_SRC),
           "source": "profiles/" + os.path.basename(md_path)}
    json.dump(rec, open(json_path, "w"), indent=1)
    print(f"wrote {md_path} and {json_path}: aba_attend reads {rd / 1e9:.3f} GB, writes {wr / 1e9:.3f} GB per call")
    return rec


def cpu_baseline(w, p, q, k, v, seed: int, target_s: float):
    """The oracle (as it stands) on a bounded sample: whole heads when it is fast
    enough, else evenly spaced query blocks of head 0."""
    import oracle

    N, NB, D = w.seq_len, w.n_blocks, w.head_dim
    NBk, kb = p.n_key_blocks, p.key_block
    valid = np.minimum(128, N - 128 * np.arange(NB))

    def run(h, blocks):
        qh, kh, vh = (np.ascontiguousarray(x[:1, h:h + 1].float().numpy()) for x in (q, k, v))
        t0 = time.perf_counter()
        cents, wts = [], []
        for qb in blocks:
            c, wt, _, _ = oracle.kmeans_block(qh[0, 0, qb * 128:qb * 128 + valid[qb]], C=p.n_clusters,
                                              T=p.kmeans_iters)
            cents.append(c)
            wts.append(wt)
        kbar = oracle.pool(kh, N, blk=kb)
        s = oracle.score(np.stack(cents)[None, None], np.stack(wts)[None, None], kbar, p.softmax_scale)
        idx_s, cnt_s, w_s, _ = oracle.sample(s.astype(np.float32), p.budget, seed)
        idx = np.zeros((1, 1, NB, NBk), np.int32)
        cnt = np.zeros((1, 1, NB), np.int32)
        wl = np.zeros((1, 1, NB, NBk), np.float32)
        for r, qb in enumerate(blocks):
            idx[0, 0, qb], cnt[0, 0, qb], wl[0, 0, qb] = idx_s[0, 0, r], cnt_s[0, 0, r], w_s[0, 0, r]
        oracle.attend(qh, kh, vh, N, idx, cnt, wl, items=[(0, 0, qb) for qb in blocks], scale=p.softmax_scale,
                      kblk=kb)
        return time.perf_counter() - t0

    probe = list(range(0, NB, max(1, NB // 16)))[:16]
    per_block = run(0, probe) / len(probe)
    n_blocks = target_s / max(per_block, 1e-6)
    total_t, rows, what = 0.0, 0, ""
    if n_blocks >= NB:
        heads = 0
        while heads < w.heads and total_t < target_s:
            total_t += run(heads, list(range(NB)))
            heads += 1
        rows = heads * float(valid.sum())
        what = f"every query block of heads 0..{heads - 1} ({heads} of {w.heads} heads)"
    else:
        blocks = sorted(set(np.linspace(0, NB - 1, max(len(probe), int(n_blocks))).astype(int).tolist()))
        total_t = run(0, blocks)
        rows = float(valid[blocks].sum())
        what = f"{len(blocks)} of {NB} query blocks of head 0 (of {w.heads} heads)"
    flops = 4.0 * D * N * rows          # dense-equivalent work of the sampled query rows
    return {
        "value": flops / total_t / 1e12,
        "unit": "TFLOP/s (effective, dense-equivalent)",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"full layer pass (k-means, pooling, scores, sampling, attention) for {what}; "
                  f"{total_t:.1f} s on {oracle.max_threads()} threads ({platform.machine()})",
        "seconds": total_t,
    }


def selection_diagnostics(w, p, qkv, ws, n_blocks: int, seed: int, softmax_scale: float = 0.0):
    """How much dense attention mass the selections keep, on sampled query blocks
    (dense mass per key block from aba_block_mass), and the attention error of the
    sampled lists and of hard top-K lists of the same scores against dense
    attention (outputs of aba_attend against aba_attend_full), as an RMS over the
    sampled rows divided by the RMS of v.  Untimed.  softmax_scale > 0 runs the
    whole layer (scores, lists, attention) at that scale instead of the plan's:
    1.0 is the peaked variant (logits x sqrt(D) at D = 128)."""
    qd, kd, vd = qkv
    B, H, NB, K = p.batch, p.heads, p.n_blocks, p.budget
    if softmax_scale > 0:
        p = aba.plan(B, H, w.seq_len, w.head_dim, w.dtype, p.n_clusters, p.kmeans_iters, K, softmax_scale=softmax_scale,
                     key_block=p.key_block)
    scores = aba.score(p, qd, kd, ws=ws)
    idx, cnt, wt = aba.sample(p, scores, seed, ws=ws)
    rng = np.random.default_rng(5)
    items = sorted({(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(NB))) for _ in range(4 * n_blocks)})
    items = items[:max(n_blocks, 32)]
    mass = aba.block_mass(p, qd, kd, items).double().cpu().numpy()                 # [n, NB]
    it = np.array(items)
    ideal = np.sort(mass, axis=1)[:, ::-1][:, :K].sum(axis=1)

    def top_k_mass(sc):
        top = np.argsort(-sc[it[:, 0], it[:, 1], it[:, 2]], axis=1, kind="stable")[:, :K]
        return np.take_along_axis(mass, top, axis=1).sum(axis=1)

    ibcs = top_k_mass(scores.double().cpu().numpy())
    p1 = aba.plan(B, H, w.seq_len, w.head_dim, w.dtype, 1, p.kmeans_iters, K, softmax_scale=p.softmax_scale,
                  key_block=p.key_block)                                          # one cluster: mean-pool scorer
    meanpool = top_k_mass(aba.score(p1, qd, kd, ws=aba.workspace(p1, qd.device)).double().cpu().numpy())
    idx_h, cnt_h, wt_h = (x.cpu().numpy() for x in (idx, cnt, wt))
    kept, ht = [], []
    for r, (b, h, qb) in enumerate(items):
        c = int(cnt_h[b, h, qb])
        sel = idx_h[b, h, qb, :c]
        kept.append(mass[r, sel].sum())
        ht.append((mass[r, sel] * wt_h[b, h, qb, :c]).sum())
    # hard top-K lists of the same scores, ascending, unit weights
    top = torch.topk(scores, K, dim=-1).indices.sort(dim=-1).values.to(torch.int32)
    idx_t = torch.zeros_like(idx)
    idx_t[..., :K] = top
    cnt_t = torch.full_like(cnt, K)
    wt_t = torch.ones_like(wt)
    dense = aba.attend_full(p, qd, kd, vd, ws=ws)
    o_sip = aba.attend(p, qd, kd, vd, idx, cnt, wt, ws=ws)
    o_top = aba.attend(p, qd, kd, vd, idx_t, cnt_t, wt_t, ws=ws)
    torch.cuda.synchronize()
    errs = attention_errors(w, items, vd, dense, {"sip": o_sip, "hard_topk": o_top})
    return {
        "softmax_scale": float(p.softmax_scale),
        "query_blocks": len(items),
        "ideal_topk_mass": float(ideal.mean()),
        "ibcs_topk_mass": float(ibcs.mean()),
        "meanpool_topk_mass": float(meanpool.mean()),
        "recall_gap": {"ibcs": float((ideal - ibcs).mean()), "meanpool": float((ideal - meanpool).mean())},
        "sip_kept_mass": float(np.mean(kept)),
        "sip_ht_weighted_mass": float(np.mean(ht)),
        "mean_kept_blocks": float(cnt_h.mean()),
        "attention_rms_err_over_rms_v": errs,
        "dense_output_rms_over_rms_v": errs.pop("dense_scale"),
    }


def attention_errors(w, items, vd, dense, outs):
    """RMS of (out - dense) over the sampled query blocks' valid rows, divided by
    the RMS of v over the same heads (the scale of an output that attends to one
    key); also the dense output's own RMS on that scale."""
    rows = {name: [] for name in outs}
    ref, vs = [], []
    for b, h, qb in items:
        n = min(128, w.seq_len - 128 * qb)
        d = dense[b, h, 128 * qb:128 * qb + n].float()
        ref.append(d)
        vs.append(vd[b, h, :w.seq_len].float().pow(2).mean())
        for name, o in outs.items():
            rows[name].append(o[b, h, 128 * qb:128 * qb + n].float() - d)
    rms_v = float(torch.stack(vs).mean().sqrt())
    res = {name: float(torch.cat(r).pow(2).mean().sqrt()) / rms_v for name, r in rows.items()}
    res["dense_scale"] = float(torch.cat(ref).pow(2).mean().sqrt()) / rms_v
    return res


def fine_leg(args, w, sets, density, coarse_plan, coarse_lists, dense_ms, n_diag: int, diagnostics: bool):
    """The same layer with 4-token key blocks (the page's kernel paragraph) at the
    number of 128-key tiles of the 128-token budget: score, sample and attend timed
    over the same input sets, kept work, and (untimed) the dense attention mass the
    ideal, IBCS and sampled selections keep at either granularity on the same
    query blocks, with the attention error of both sampled lists against dense."""
    dev = torch.device("cuda:0")
    p = aba.plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, CLUSTERS, KMEANS_ITERS, w.fine_budget(density),
                 key_block=aba.FINE_BLOCK)
    B, H, NB, NBk, cap = p.batch, p.heads, p.n_blocks, p.n_key_blocks, p.list_cap
    ws = aba.workspace(p, dev)
    scores = torch.empty(B, H, NB, NBk, dtype=torch.float32, device=dev)
    lists = (torch.empty(B, H, NB, cap, dtype=torch.int32, device=dev),
             torch.empty(B, H, NB, dtype=torch.int32, device=dev),
             torch.empty(B, H, NB, cap, dtype=torch.float32, device=dev))
    out = torch.empty_like(sets[0][0])
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        qd, kd, vd = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        aba.score(p, qd, kd, out=scores, ws=ws)
        if ev is not None:
            ev[1].record(stream)
        aba.sample(p, scores, args.seed + i % len(sets), out=lists, ws=ws)
        if ev is not None:
            ev[2].record(stream)
        aba.attend(p, qd, kd, vd, *lists, out=out, ws=ws)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n = max(10, args.steps // 2)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(n):
        step(i, evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n
    st = {k: float(np.mean([e[a].elapsed_time(e[b]) for e in evs]))
          for k, a, b in (("score", 0, 1), ("sample", 1, 2), ("attend", 2, 3))}
    kfl, kept = [], []
    set_lists = []
    for i in range(len(sets)):
        qd, kd, vd = sets[i]
        s_i = aba.score(p, qd, kd, ws=ws)
        l_i = aba.sample(p, s_i, args.seed + i, ws=ws)
        idx, cnt, _ = (x.cpu().numpy() for x in l_i)
        kfl.append(kept_flops(p, cnt, idx))
        kept.append(float(cnt.mean()))
        set_lists.append((s_i, l_i))
    kflops = float(np.mean(kfl))
    res = {
        "key_block": p.key_block, "key_blocks": NBk, "budget_blocks": p.budget, "ms_per_step": ms,
        "effective_tflops": w.dense_flops / (ms * 1e-3) / 1e12, "stages_ms": st,
        "mean_kept_blocks": float(np.mean(kept)), "realised_density": float(np.mean(kept)) / NBk,
        "kept_tflop_per_call": kflops / 1e12, "attend_kept_tflops": kflops / (st["attend"] * 1e-3) / 1e12,
        "attend_kept_mfma_frac": kflops / (st["attend"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "attend_traffic_bytes": traffic_entry(aba.FINE_BLOCK) if w.name == "single_layer" else None,
        "speedup_vs_dense": {"layer": dense_ms / ms, "attention": dense_ms / st["attend"]} if dense_ms else None,
    }
    log(f"[bench] 4-token key blocks: {ms:.3f} ms/step (score {st['score']:.3f}, sample {st['sample']:.3f}, "
        f"attend {st['attend']:.3f}); kept {res['mean_kept_blocks']:.1f} of {NBk}; "
        f"attention {res['attend_kept_tflops']:.0f} TFLOP/s on kept blocks")
    if not diagnostics:
        return res

    # selection quality at both granularities on the same sampled query blocks
    qd, kd, vd = sets[0]
    rng = np.random.default_rng(5)
    items = sorted({(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(NB))) for _ in range(4 * n_diag)})
    items = items[:max(n_diag, 32)]
    it = np.array(items)
    K, Kf = coarse_plan.budget, p.budget
    mass_c = aba.block_mass(coarse_plan, qd, kd, items).double().cpu().numpy()
    mass_f = aba.block_mass(p, qd, kd, items).double().cpu().numpy()
    ideal_c = np.sort(mass_c, axis=1)[:, ::-1][:, :K].sum(axis=1)
    ideal_f = np.sort(mass_f, axis=1)[:, ::-1][:, :Kf].sum(axis=1)
    sc_f = set_lists[0][0].double().cpu().numpy()[it[:, 0], it[:, 1], it[:, 2]]
    ibcs_f = np.take_along_axis(mass_f, np.argsort(-sc_f, axis=1, kind="stable")[:, :Kf], axis=1).sum(axis=1)
    sc_c = coarse_lists[0].double().cpu().numpy()[it[:, 0], it[:, 1], it[:, 2]]
    ibcs_c = np.take_along_axis(mass_c, np.argsort(-sc_c, axis=1, kind="stable")[:, :K], axis=1).sum(axis=1)

    def sip_mass(mass, lists_):
        idx, cnt, _ = (x.cpu().numpy() for x in lists_)
        return float(np.mean([mass[r, idx[b, h, qb, :cnt[b, h, qb]]].sum() for r, (b, h, qb) in enumerate(items)]))

    dense = aba.attend_full(p, qd, kd, vd, ws=ws)
    o_f = aba.attend(p, qd, kd, vd, *set_lists[0][1], ws=ws)
    o_c = aba.attend(coarse_plan, qd, kd, vd, *coarse_lists[1], ws=aba.workspace(coarse_plan, dev))
    torch.cuda.synchronize()
    errs = attention_errors(w, items, vd, dense, {"128_token": o_c, "4_token": o_f})

    res["diagnostics"] = {
        "query_blocks": len(items),
        "ideal_topk_mass": {"128_token": float(ideal_c.mean()), "4_token": float(ideal_f.mean())},
        "ibcs_topk_mass": {"128_token": float(ibcs_c.mean()), "4_token": float(ibcs_f.mean())},
        "sip_kept_mass": {"128_token": sip_mass(mass_c, coarse_lists[1]), "4_token": sip_mass(mass_f, set_lists[0][1])},
        "attention_rms_err_over_rms_v": {"128_token": errs["128_token"], "4_token": errs["4_token"]},
        "dense_output_rms_over_rms_v": errs["dense_scale"],
        # the peaked variant (softmax scale 1) at 4-token granularity: ideal, IBCS, mean-pool and sampled
        # selections, and sampled against hard top-K lists, as the 128-token diagnostics report them
        "peaked": selection_diagnostics(w, p, sets[0], ws, n_diag, args.seed, softmax_scale=1.0),
    }
    log(f"[bench] 4-token diagnostics: {json.dumps(res['diagnostics'])}")
    return res


def run_sweep(args, w):
    """The denoising sweep: w.steps steps, each with fresh q/k/v (centres drifting
    per step), each re-running score, sample and attend.  Also timed, on the same
    inputs: the plan refreshed every args.plan_every steps and reused in between
    (attend every step), and that schedule with dense attention for the first
    args.dense_frac of the steps.  One JSON line."""
    dev = torch.device("cuda:0")
    steps = w.steps
    t0 = time.perf_counter()
    sets = [tuple(x.to(dev) for x in synth.make_inputs(w, seed=1001, step=s)) for s in range(steps)]
    log(f"[bench] sweep: {steps} steps of inputs ready in {time.perf_counter() - t0:.1f} s")
    density = w.densities[0] if args.density is None else args.density
    p = aba.plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, CLUSTERS, KMEANS_ITERS, w.budget(density))
    B, H, NB, cap = p.batch, p.heads, p.n_blocks, p.list_cap
    ws = aba.workspace(p, dev)
    scores = torch.empty(B, H, NB, NB, dtype=torch.float32, device=dev)
    lists = (torch.empty(B, H, NB, cap, dtype=torch.int32, device=dev),
             torch.empty(B, H, NB, dtype=torch.int32, device=dev),
             torch.empty(B, H, NB, cap, dtype=torch.float32, device=dev))
    out = torch.empty_like(sets[0][0])
    stream = torch.cuda.current_stream()

    def sweep(plan_every: int, dense_steps: int, record: bool):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for s in range(steps):
            qd, kd, vd = sets[s]
            e = evs[s]
            e[0].record(stream)
            if s < dense_steps:
                e[1].record(stream)
                e[2].record(stream)
                aba.attend_full(p, qd, kd, vd, out=out, ws=ws)
            else:
                if (s - dense_steps) % plan_every == 0:
                    aba.score(p, qd, kd, out=scores, ws=ws)
                    e[1].record(stream)
                    aba.sample(p, scores, args.seed + s, out=lists, ws=ws)
                else:
                    e[1].record(stream)
                e[2].record(stream)
                aba.attend(p, qd, kd, vd, *lists, out=out, ws=ws)
            e[3].record(stream)
        torch.cuda.synchronize()
        per = [evs[s][0].elapsed_time(evs[s][3]) for s in range(steps)]
        parts = {"score": float(sum(evs[s][0].elapsed_time(evs[s][1]) for s in range(steps))),
                 "sample": float(sum(evs[s][1].elapsed_time(evs[s][2]) for s in range(steps))),
                 "attend": float(sum(evs[s][2].elapsed_time(evs[s][3]) for s in range(steps)))}
        return per, parts

    for _ in range(max(1, args.warmup // 5)):
        sweep(1, 0, False)
    per, parts = sweep(1, 0, True)
    total = float(sum(per))
    log(f"[bench] sweep, plan every step: total {total:.2f} ms ({np.mean(per):.3f} ms/step; score {parts['score']:.2f}, "
        f"sample {parts['sample']:.2f}, attend {parts['attend']:.2f})")
    per_r, parts_r = sweep(args.plan_every, 0, True)
    total_r = float(sum(per_r))
    dense_steps = int(round(args.dense_frac * steps))
    per_d, parts_d = sweep(args.plan_every, dense_steps, True)
    total_d = float(sum(per_d))
    log(f"[bench] sweep, plan every {args.plan_every}: total {total_r:.2f} ms; with {dense_steps} dense steps first: "
        f"{total_d:.2f} ms")
    dense_flops = w.dense_flops
    result = {
        "metric": METRIC,
        "value": steps * dense_flops / (total * 1e-3) / 1e12,
        "unit": "TFLOP/s (effective, dense-equivalent)",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": total / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian-mixture video tokens, fresh per step, centres drifting; no model weights)",
        "config": {"workload": w.name, "batch": B, "heads": H, "seq_len": w.seq_len, "head_dim": w.head_dim,
                   "steps": steps, "drift": w.drift, "density": density, "budget_blocks": p.budget},
        "sweep": {
            "per_step_ms": per,
            "total_ms": total,
            "stages_total_ms": parts,
            "score_sample_over_attend": (parts["score"] + parts["sample"]) / parts["attend"],
            "plan_reuse": {"plan_every": args.plan_every, "total_ms": total_r, "stages_total_ms": parts_r,
                           "speedup": total / total_r},
            "plan_reuse_dense_first": {"plan_every": args.plan_every, "dense_steps": dense_steps,
                                        "total_ms": total_d, "per_step_ms": per_d},
        },
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def _smi_sample(exe: str):
    """One amd-smi reading of GPU 0: (socket power W, mean graphics clock MHz over the XCDs), or None."""
    import subprocess
    r = subprocess.run(["timeout", "10", exe, "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True, text=True)
    try:
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [v["clk"]["value"] for name, v in g["clock"].items()
                if name.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk", {}).get("value"), (int, float))]
        return float(g["power"]["socket_power"]["value"]), float(np.mean(clks))
    except (ValueError, KeyError, IndexError, TypeError):
        return None


def power_trace(args):
    """Socket power and graphics clock (amd-smi, sampled from a host thread) while
    one kind of call runs back to back for a few seconds: the sparse and dense
    attention of the layer, the matrix-core rate loop on random operands and on
    zeros, and the score stage; idle first.  For each phase: median power and
    clock, time per call, and for the attention and the loop their bf16 rate
    against the quoted peak and against the peak at the clock the phase ran at."""
    import shutil
    import threading
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe) or _smi_sample(exe) is None:
        print("amd-smi is not available or reads no power: no power trace", file=sys.stderr)
        sys.exit(2)
    w = ALL[args.workload]
    density = w.densities[0] if args.density is None else args.density
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in synth.make_inputs(w, seed=1001))
    p = aba.plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, CLUSTERS, KMEANS_ITERS, w.budget(density))
    ws = aba.workspace(p, dev)
    sc = aba.score(p, qd, kd, ws=ws)
    lists = aba.sample(p, sc, args.seed, ws=ws)
    out = torch.empty_like(qd)
    kept = int(lists[1].clamp(min=0).sum().item())
    kept_flop = kept_flops(p, lists[1].cpu().numpy(), lists[0].cpu().numpy())
    dense_flop = 4.0 * w.batch * w.heads * float(w.seq_len) ** 2 * w.head_dim
    rate_out = torch.empty(aba.MFMA_RATE_THREADS, dtype=torch.float32, device=dev)
    rate_iters = 2000
    rate_flop = float(aba.MFMA_RATE_FLOP_PER_ITER) * rate_iters
    torch.cuda.synchronize()
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            t0 = time.time()
            r = _smi_sample(exe)
            if r is not None:
                samples.append(((t0 + time.time()) / 2, *r))

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    phases = []

    def run(name, fn, flop):
        if fn is None:
            t0 = time.time()
            time.sleep(args.power_seconds / 2)
            phases.append((name, t0, time.time(), 0, flop))
            return
        fn()
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        while time.time() - t0 < args.power_seconds:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            n += 10
        phases.append((name, t0, time.time(), n, flop))
        log(f"[bench] power trace: {name} {n} calls")
        time.sleep(1.0)

    run("idle", None, 0.0)
    run("sparse_attend", lambda: aba.attend(p, qd, kd, vd, *lists, out=out, ws=ws), kept_flop)
    run("dense_attend", lambda: aba.attend_full(p, qd, kd, vd, out=out, ws=ws), dense_flop)
    run("mfma_rate_random", lambda: aba.mfma_rate(rate_iters, True, rate_out), rate_flop)
    run("mfma_rate_zeros", lambda: aba.mfma_rate(rate_iters, False, rate_out), rate_flop)
    run("score", lambda: aba.score(p, qd, kd, out=sc, ws=ws), 0.0)
    stop.set()
    th.join(timeout=15)
    res = {}
    for name, a, b, n, flop in phases:
        sel = [x for x in samples if a + 0.5 < x[0] < b - 0.1]   # skip the first half second of a phase
        pw = np.array([x[1] for x in sel]) if sel else np.array([np.nan])
        ck = np.array([x[2] for x in sel]) if sel else np.array([np.nan])
        e = {"samples": len(sel), "socket_power_w_median": float(np.median(pw)), "socket_power_w_max": float(pw.max()),
             "gfx_clock_mhz_median": float(np.median(ck))}
        if n:
            ms = (b - a) / n * 1e3
            e["ms_per_call"] = ms
            if flop:
                tf = flop / (ms * 1e-3) / 1e12
                e["bf16_tflops"] = tf
                e["frac_of_peak"] = tf / PEAK_BF16_TFLOPS
                e["frac_of_peak_at_clock"] = tf / (PEAK_BF16_TFLOPS * np.median(ck) / 2400.0)
        res[name] = e
    print(json.dumps({"power_trace": res, "workload": w.name, "kept_blocks": kept,
                      "seconds_per_phase": args.power_seconds, "sample_period_s":
                      float(np.mean(np.diff([x[0] for x in samples]))) if len(samples) > 1 else None}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="single_layer", choices=sorted(ALL))
    ap.add_argument("--density", type=float, default=None)
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--dense-reps", type=int, default=5)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--input-sets", type=int, default=3, help="input sets the steps cycle through")
    ap.add_argument("--windows", type=int, default=5,
                    help="windows of K steps timed in all (the first gives value; the rest its spread)")
    ap.add_argument("--plan-every", type=int, default=4, help="sweep: steps between plan refreshes (the page: 4)")
    ap.add_argument("--dense-frac", type=float, default=0.2,
                    help="sweep: share of the first steps run dense (the page: 10 of 50)")
    ap.add_argument("--no-diagnostics", action="store_true")
    ap.add_argument("--diag-blocks", type=int, default=32, help="sampled query blocks for the selection diagnostics")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--key-block", type=int, default=128, choices=(128, 4),
                    help="key block size of the timed layer (4: the page's fine-grained selection)")
    ap.add_argument("--no-fine", action="store_true",
                    help="skip the 4-token key block measurement that follows the 128-token one")
    ap.add_argument("--head-shard", default=None, metavar="I/N",
                    help="time one GPU's share of the layer sharded by heads over N GPUs: heads "
                         "[I*H/N, (I+1)*H/N), drawn with their global head offset (no 4-token leg, diagnostics "
                         "or CPU baseline)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script "
                         "with --copy-calibration into profiles/ for --key-block")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize-traffic: a command line that produced the counters (recorded verbatim)")
    ap.add_argument("--no-mfma-rate", action="store_true",
                    help="skip the sustained matrix-core rate measurement (aba_mfma_rate) reported beside the roofline")
    ap.add_argument("--mfma-rate-iters", type=int, default=10000,
                    help="rounds of the matrix-core rate loop per timed call (2^30 flop each; 10^4: ~6 ms)")
    ap.add_argument("--mfma-rate-only", action="store_true",
                    help="only measure the sustained matrix-core rate and print it (for its counter profile)")
    ap.add_argument("--power-only", action="store_true",
                    help="only sample socket power and graphics clock (amd-smi) while each kind of call runs back to "
                         "back (sparse and dense attention, the matrix-core rate loop, the score stage)")
    ap.add_argument("--power-seconds", type=float, default=4.0, help="--power-only: seconds per phase")
    args = ap.parse_args()
    if args.power_only:
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(2)
        power_trace(args)
        return
    if args.mfma_rate_only:
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"mfma_sustained": mfma_rate(args.mfma_rate_iters)}), flush=True)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.key_block, args.command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer shards over heads with no exchange, and no multi-GPU "
              "figure is produced (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    w = ALL[args.workload]
    if w.steps > 1:
        run_sweep(args, w)
        return
    density = w.densities[0] if args.density is None else args.density
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: {w.description}; density {density}")
    # One GPU's share of a layer sharded by heads: the inputs are the layer's own
    # (generated whole, then sliced), and the draws use the global head index.
    h0, shard = 0, None
    if args.head_shard:
        si, sn = (int(x) for x in args.head_shard.split("/"))
        if not (sn >= 1 and 0 <= si < sn and w.heads >= sn):
            raise SystemExit(f"--head-shard {args.head_shard}: need 0 <= I < N <= heads ({w.heads})")
        h0, h1 = si * w.heads // sn, (si + 1) * w.heads // sn
        shard = {"shard": f"{si}/{sn}", "layer_heads": w.heads, "head_offset": h0}
        args.no_fine = args.no_diagnostics = args.no_cpu_baseline = True
        log(f"[bench] head shard {si}/{sn}: heads {h0}..{h1 - 1} of {w.heads}")
    # Several input sets, used in turn: one set's q and k (201 MB at the single
    # layer) would otherwise stay in the 256 MB MALL from one step to the next.
    t0 = time.perf_counter()
    host_sets = [synth.make_inputs(w, seed=1001 + 10 * i) for i in range(args.input_sets)]
    if shard:
        host_sets = [tuple(x[:, h0:h1].contiguous() for x in hs) for hs in host_sets]
        w = dataclasses.replace(w, heads=h1 - h0)
    sets = [tuple(x.to(dev) for x in hs) for hs in host_sets]
    log(f"[bench] {len(sets)} input sets ready in {time.perf_counter() - t0:.1f} s")

    fine_main = args.key_block == aba.FINE_BLOCK
    p = aba.plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, CLUSTERS, KMEANS_ITERS,
                 w.fine_budget(density) if fine_main else w.budget(density), key_block=args.key_block)
    B, H, NB, cap, D = p.batch, p.heads, p.n_blocks, p.list_cap, p.head_dim
    scores = torch.empty(B, H, NB, p.n_key_blocks, dtype=torch.float32, device=dev)
    ws = aba.workspace(p, dev)
    lists = (torch.empty(B, H, NB, cap, dtype=torch.int32, device=dev),
             torch.empty(B, H, NB, dtype=torch.int32, device=dev),
             torch.empty(B, H, NB, cap, dtype=torch.float32, device=dev))
    out = torch.empty_like(sets[0][0])
    stream = torch.cuda.current_stream()

    def step(i, ev=None, att=None):
        qd, kd, vd = sets[i % len(sets)]
        seed = args.seed + i % len(sets)
        if ev is not None:
            ev[0].record(stream)
        aba.score(p, qd, kd, out=scores, ws=ws)
        if ev is not None:
            ev[1].record(stream)
        aba.sample(p, scores, seed, out=lists, ws=ws, head_offset=h0)
        if ev is not None:
            ev[2].record(stream)
        if att is not None:
            att[0].record(stream)
        aba.attend(p, qd, kd, vd, *lists, out=out, ws=ws)
        if att is not None:
            att[1].record(stream)
        if ev is not None:
            ev[3].record(stream)

    t_warm = time.perf_counter()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warm-up steps in {time.perf_counter() - t_warm:.3f} s")
    # the dense path between the warm-up and the timed steps: its own
    # measurement, and it leaves the GPU at its loaded clock, so that the
    # timed steps do not include the ramp from idle (the warm-up's first calls
    # spend host time in which the chip idles, and a first window after 0.5 s
    # of idle runs ~13% slower than the windows after it)
    dense_ms = None
    if not args.no_dense:
        qd, kd, vd = sets[0]
        aba.attend_full(p, qd, kd, vd, out=out, ws=ws)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.dense_reps):
            aba.attend_full(p, qd, kd, vd, out=out, ws=ws)
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / args.dense_reps
        log(f"[bench] dense attention: {dense_ms:.3f} ms")

    # the timed region: K steps, events only around each aba_attend call (the
    # dominant call, for the roofline)
    att_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i, att=att_ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    attend_each = np.array([a.elapsed_time(b) for a, b in att_ev])
    attend_timed_ms = float(attend_each.mean())
    # the same K steps again with events around every call, for the per-stage
    # times (the events themselves add a little to these)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    score_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sample_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    attend_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, aba_attend {attend_timed_ms:.3f} ms; per stage "
        f"(a second, evented pass) score {score_ms:.3f}, sample {sample_ms:.3f}, attend {attend_ms:.3f}")
    # stability: the same K steps timed again in further windows (after the
    # timed region above, which alone gives `value`)
    window_ms = [ms_per_step]
    for _ in range(max(0, args.windows - 1)):
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for i in range(args.steps):
            step(i)
        w1.record(stream)
        torch.cuda.synchronize()
        window_ms.append(w0.elapsed_time(w1) / args.steps)
    log(f"[bench] {len(window_ms)} windows of {args.steps} steps: median {np.median(window_ms):.3f} ms/step, "
        f"range {min(window_ms):.3f} .. {max(window_ms):.3f}")

    # kept work per call, averaged over the input sets the steps cycle through
    kflops_sets, dens_sets, set_lists = [], [], []
    for i in range(len(sets)):
        qd, kd, vd = sets[i]
        s_i = aba.score(p, qd, kd, ws=ws)
        l_i = aba.sample(p, s_i, args.seed + i, ws=ws, head_offset=h0)
        idx, cnt, wt = (x.cpu().numpy() for x in l_i)
        kflops_sets.append(kept_flops(p, cnt, idx))
        dens_sets.append(float(cnt.mean() / p.n_key_blocks))
        set_lists.append((s_i, l_i))
    kflops = float(np.mean(kflops_sets))
    dense_flops = w.dense_flops
    realised_density = float(np.mean(dens_sets))

    diagnostics = None
    if not args.no_diagnostics and w.dtype == "bf16" and not fine_main:
        diagnostics = {
            "literal": selection_diagnostics(w, p, sets[0], ws, args.diag_blocks, args.seed),
            # the same inputs with logits x sqrt(D): reported beside the workload, never in place of it
            "peaked": selection_diagnostics(w, p, sets[0], ws, args.diag_blocks, args.seed, softmax_scale=1.0),
        }
        log(f"[bench] diagnostics: {json.dumps(diagnostics)}")

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB device-to-device copy done")

    # scoring-stage bytes: q and k read once, centroids/weights/pooled keys written and re-read, scores written
    elem = 2 if w.dtype == "bf16" else 4
    rows, krows = B * H * NB, B * H * p.n_key_blocks
    score_bytes = (2 * B * H * w.seq_len * D * elem + 2 * 4 * rows * (p.n_clusters * D + p.n_clusters)
                   + 2 * 4 * krows * D + 4 * rows * p.n_key_blocks)
    # scoring-stage fp32 work: T Lloyd rounds per query block (the assignment's
    # 2 n C D and the update's n D), then the centroid x pooled-key products 2 C NBk D
    n_valid = np.minimum(128, w.seq_len - 128 * np.arange(NB)).astype(np.float64)
    C, T = p.n_clusters, p.kmeans_iters
    kmeans_flops = B * H * float((T * (2.0 * n_valid * C * D + n_valid * D)).sum())
    score_flops = kmeans_flops + rows * 2.0 * C * p.n_key_blocks * D
    attend_tflops = kflops / (attend_timed_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": dense_flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s (effective, dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian-mixture video tokens; no model weights)",
        "config": {
            "workload": w.name, "batch": B, "heads": H, "seq_len": w.seq_len, "seq_pad": p.seq_pad,
            "head_dim": D, "grid": list(w.grid), "density": density, "budget_blocks": p.budget,
            "clusters": p.n_clusters, "kmeans_iters": p.kmeans_iters, "block": 128, "key_block": p.key_block,
            "seed": args.seed, "input_sets": len(sets), **(shard or {}),
        },
        "stages_ms": {"score": score_ms, "sample": sample_ms, "attend": attend_ms},
        "attend_ms_timed_region": attend_timed_ms,
        "dense_attention_ms": dense_ms,
        "speedup_vs_dense": {"layer": dense_ms / ms_per_step, "attention": dense_ms / attend_timed_ms} if dense_ms else None,
        "realised_density": realised_density,
        "kept_tflop_per_call": kflops / 1e12,
        "attend_kept_tflops": attend_tflops,
        "timing": {
            "evented_step_ms_median": float(np.median(step_ms)), "evented_step_ms_p10": float(np.percentile(step_ms, 10)),
            "evented_step_ms_p90": float(np.percentile(step_ms, 90)),
            "attend_ms_timed_median": float(np.median(attend_each)),
            "attend_ms_timed_p10": float(np.percentile(attend_each, 10)),
            "attend_ms_timed_p90": float(np.percentile(attend_each, 90)),
            "windows_ms_per_step": window_ms, "windows_median": float(np.median(window_ms)),
        },
        "score_stage_gbs": score_bytes / (score_ms * 1e-3) / 1e9,
        "score_stage_hbm_frac": score_bytes / (score_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        # the stage is bound by its fp32 arithmetic (k-means dominates), not by HBM
        "score_stage_fp32_tflops": score_flops / (score_ms * 1e-3) / 1e12,
        "score_stage_fp32_frac": score_flops / (score_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
        "score_stage_algorithmic_gflop": score_flops / 1e9,
        "roofline": {
            # the whole aba_attend call: the work order is part of it
            "kernel": (("aba_attend: order_kernel + attend_fine_kernel<128>" if fine_main else
                        "aba_attend: order_kernel + attend_bf16_kernel<128,false>")
                       if w.dtype == "bf16" else "aba_attend: attend_f32_kernel<64,false>"),
            "bound": "mfma",
            "achieved": attend_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": attend_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic_entry(p.key_block) if w.name == "single_layer" and w.dtype == "bf16" and not shard else None,
        },
        "diagnostics": diagnostics,
        "fine_key_blocks": None,
        "cpu_baseline": None,
    }
    if not fine_main and not args.no_fine and w.dtype == "bf16":
        result["fine_key_blocks"] = fine_leg(args, w, sets, density, p, set_lists[0], dense_ms, args.diag_blocks,
                                             not args.no_diagnostics)
    if not args.no_mfma_rate and w.dtype == "bf16":
        rate = mfma_rate(args.mfma_rate_iters)
        result["mfma_sustained"] = rate
        result["roofline"]["sustained_peak"] = rate["random_tflops"]
        result["roofline"]["frac_of_sustained"] = attend_tflops / rate["random_tflops"]
        if result["fine_key_blocks"]:
            fk = result["fine_key_blocks"]
            fk["attend_kept_frac_of_sustained"] = fk["attend_kept_tflops"] / rate["random_tflops"]
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        q, k, v = host_sets[0]
        result["cpu_baseline"] = cpu_baseline(w, p, q, k, v, args.seed, args.cpu_seconds)
        log(f"[bench] CPU oracle: {result['cpu_baseline']['value']:.4g} TFLOP/s effective")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
