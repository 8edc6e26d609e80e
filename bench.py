#!/usr/bin/env python3
"""Benchmark: MTGR HSTU encoder forward (bf16, fp32 accumulation) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large-bf16] [--no-cpu-baseline]
                    [--mask dynamic|causal|full] [--norm group|shared] [--block-bwd] [--front-end]

--mask / --norm select the ablation variants (plain causal or full mask in place of the dynamic
mask, one shared LayerNorm in place of GroupLN); the defaults are the method itself.

One step = one mtgr_encoder_fwd over the whole synthetic batch (all L blocks + the candidate
head), inputs and weights resident in HBM, workspace preallocated.  Prints ONE JSON line.

Besides the headline tokens/s the line carries
  * "roofline": the dominant kernel (the fused attention) -- algorithmic FLOPs per launch
    (4 * d_model per visible (query, key) pair) over its average launch duration, measured with
    HIP events on the library's stream in a replay of the per-layer kernel sequence;
  * "mfma_util": algorithmic FLOPs of the GEMM + attention launches over their summed durations
    and the bf16 dense MFMA peak;
  * "cpu_baseline": the fp64 CPU oracle timed on this host on a bounded sample of users.

--block-bwd measures the backward pass of one block instead (layer 0 of the workload): one step =
one mtgr_block_bwd over the whole batch (forward recompute, then dX and every parameter gradient)
from a synthetic upstream gradient; its roofline entry is the attention backward (the gate, dK/dV
and dQ launches) at 10 * d_model algorithmic FLOPs per visible pair, with the 14 * d_model the
kernels execute (dQ recomputes S and dP) reported beside it.

--front-end measures the embedding front end instead: one step = one mtgr_tokenize over the whole
batch (field IDs -> dedup -> hash-store lookup -> per-group MLP -> encoder input x), with 64-wide
bf16 embeddings; its roofline entry is the store's lookup kernel on a separate stream of 4M random
keys over an 8M-row store (HBM-bound: key, index slot, value row read, value row written).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "encoder tokens/sec (fwd, bf16) and MFMA-util % on one MI355X"
ATTN_SRC = os.path.join(ROOT, "generative_recommendation_ranking_amd", "csrc", "attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_large-bf16_traffic.md")
COPY_BYTES = 1 << 30        # size of the plain copy used to calibrate the traffic counters


def attention_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in (ATTN_SRC, os.path.join(os.path.dirname(ATTN_SRC), "common.h")):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    or None when the attention source changed after they were taken."""
    try:
        fields = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
        if fields.get("attention source sha256/16") != attention_source_hash():
            return None
        return float(fields["calibrated bytes per launch"])
    except (OSError, KeyError, ValueError):
        return None


def visible_pairs_per_user(b, mask="dynamic") -> np.ndarray:
    """Exact count of (query, key) pairs the mask lets through, per user.  Dynamic: every query
    sees the n_U+n_S static keys; R and C queries also see the strictly earlier R keys; every
    token sees itself (static rows already count themselves among the static keys).  Causal:
    n(n+1)/2.  Full: n^2."""
    n_all = np.diff(np.asarray(b.offsets, dtype=np.int64))
    if mask == "causal":
        return n_all * (n_all + 1) // 2
    if mask == "full":
        return n_all * n_all
    out = np.zeros(b.num_users, dtype=np.int64)
    for u in range(b.num_users):
        lo = int(b.offsets[u])
        n = int(b.offsets[u + 1]) - lo
        ns = int(b.n_u[u] + b.n_s[u])
        nr = int(b.n_r[u])
        t = b.timestamps[lo + ns:lo + n]
        tr = np.sort(t[:nr])
        earlier = np.searchsorted(tr, t, side="left")   # R keys strictly earlier than each R/C row
        out[u] = n * ns + int(earlier.sum()) + (n - ns)
    return out


def flops_per_layer(b, d, h, mask="dynamic"):
    T = b.num_tokens
    pairs = int(visible_pairs_per_user(b, mask).sum())
    return {"qkvu": 2.0 * T * d * 4 * d, "mlp1": 2.0 * T * d * h, "mlp2": 2.0 * T * h * d,
            "attention": 4.0 * d * pairs, "pairs": pairs}


def cpu_baseline_block_bwd(b, p, dout, mask="dynamic", norm="group", budget_s=12.0, max_s=30.0):
    """The oracle's block backward (fp64 numpy) on whole users of the same batch, in index order,
    until at least `budget_s` seconds of work; tokens of the sample per second."""
    from oracle import mtgr_oracle as O
    lay = O.params_layers(p)[0]
    done, users, t0 = 0, [], time.perf_counter()
    for u in range(b.num_users):
        lo, hi = int(b.offsets[u]), int(b.offsets[u + 1])
        O.block_backward(b.x[lo:hi], b.group_ids[lo:hi], b.timestamps[lo:hi], lay, p.H, dout[lo:hi],
                         p.ln_eps, mask_mode=mask, shared_norm=(norm == "shared"))
        done += hi - lo
        users.append(u)
        el = time.perf_counter() - t0
        if el >= budget_s or el >= max_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"users {users[0]}..{users[-1]} ({len(users)} users, {done} tokens) of the "
                      f"same batch, backward of block 0 (forward recompute included), fp64 numpy",
            "seconds": round(el, 2), "host": host_cpu()}


def host_cpu():
    """model name and logical CPU count of the host (lscpu, else /proc/cpuinfo)"""
    model = None
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def baseline_user_order(b):
    """users in the order the baseline samples them: the first user whose long-term history sits at
    the workload's 3000-item cap (when there is one), then users 0, 1, 2, ..."""
    tail = np.flatnonzero(np.asarray(b.n_s) == 3000)
    first = [int(tail[0])] if tail.size else []
    return first + [u for u in range(b.num_users) if u not in first]


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return int(os.cpu_count())


def cpu_baseline(b, p, mask="dynamic", norm="group", budget_s=20.0, max_s=30.0):
    """The oracle (fp64 numpy, as it stands) on whole users of the same batch -- the first user at
    the 3000-item history cap, then users 0, 1, 2, ... (the start of the subset users 0-7 plus that
    user, which takes about 100 s in full) -- until at least `budget_s` seconds of work; tokens of
    the sample per second."""
    from generative_recommendation_ranking_amd import synth
    from oracle import mtgr_oracle as O
    layers, head = O.params_layers(p), O.params_head(p)
    done, users, t0 = 0, [], time.perf_counter()
    for u in baseline_user_order(b):
        s = synth.subset(b, [u])
        O.encoder_forward(s.offsets, s.group_ids, s.timestamps, s.x, layers, head, p.H, p.ln_eps,
                          mask_mode=mask, shared_norm=(norm == "shared"))
        done += s.num_tokens
        users.append(u)
        el = time.perf_counter() - t0
        if el >= budget_s or el >= max_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"users {users} ({len(users)} users, {done} tokens) of the same batch, all "
                      f"{p.num_layers} blocks + head, fp64 numpy",
            "seconds": round(el, 2), "host": host_cpu()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large-bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mask", choices=["dynamic", "causal", "full"], default="dynamic")
    ap.add_argument("--norm", choices=["group", "shared"], default="group")
    ap.add_argument("--replay-steps", type=int, default=5)
    ap.add_argument("--block-bwd", action="store_true",
                    help="time the backward pass of one block (mtgr_block_bwd) instead of the encoder")
    ap.add_argument("--front-end", action="store_true",
                    help="time the tokenizer front end (mtgr_tokenize) and the hash-store lookup instead")
    ap.add_argument("--profile-kernel", choices=["attention", "copy", "layer"], default=None,
                    help="run only this kernel (attention, a plain copy) or one layer's kernel sequence "
                         "(layer) --steps times, for rocprofv3 counter runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); users are independent, "
              "so more GPUs would each run their own share of users with no exchange step.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from generative_recommendation_ranking_amd import mtgr as M
    from generative_recommendation_ranking_amd import synth

    torch.cuda.set_device(0)
    if args.profile_kernel == "copy":
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_kernel": "copy", "bytes_read": COPY_BYTES,
                          "bytes_written": COPY_BYTES, "launches": args.steps}), flush=True)
        return
    b, p = synth.make_workload(args.workload)
    db, dm = M.DeviceBatch(b), M.DeviceModel(p, mask_mode=args.mask, norm_mode=args.norm)
    mask_c, norm_c = M.MASK_MODES[args.mask], M.NORM_MODES[args.norm]
    ws = M.workspace(M.mtgr_encoder_workspace_size(dm, db))
    hidden = torch.empty_like(db.x)
    logits = torch.empty(db.num_candidates, 2, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    print(f"[bench] workload {args.workload}: users {b.num_users} tokens {b.num_tokens} "
          f"candidates {db.num_candidates}", file=sys.stderr, flush=True)

    def step():
        M.mtgr_encoder_fwd(dm, db, db.x, hidden, logits, ws)

    if args.block_bwd:
        bench_block_bwd(args, b, p, db, dm, M, torch)
        return
    if args.front_end:
        bench_front_end(args, b, p, db, M, torch, synth)
        return

    if args.profile_kernel == "attention":
        # layer 0's QKVU from one real block pass, then the attention launch alone
        d_, H_ = p.d, p.H
        lay0 = dm.layers[0]
        xt0 = torch.empty(b.num_tokens, d_, dtype=torch.bfloat16, device="cuda")
        q0 = torch.empty(b.num_tokens, 4 * d_, dtype=torch.bfloat16, device="cuda")
        y0 = torch.empty(b.num_tokens, d_, dtype=torch.bfloat16, device="cuda")
        M.mtgr_groupln_fwd(db, d_, 0, 1, 1, norm_c, lay0["gln1_gamma"], lay0["gln1_beta"], p.ln_eps, db.x, xt0)
        M.mtgr_linear_fwd(b.num_tokens, 4 * d_, d_, M.MTGR_BF16, M.MTGR_EPI_STORE, xt0,
                          lay0["w_qkvu"], lay0["b_qkvu"], None, q0)
        aws0 = M.workspace(M.mtgr_attention_workspace_size(db, d_, H_))
        for _ in range(args.steps):
            M.mtgr_attention_fwd(db, d_, H_, M.MTGR_BF16, mask_c, q0, y0, aws0)
        torch.cuda.synchronize()
        print(json.dumps({"profile_kernel": "attention", "launches": args.steps,
                          "attention_source_sha256_16": attention_source_hash()}), flush=True)
        return

    if args.profile_kernel != "layer":
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        ms_per_step = elapsed / args.steps * 1e3
        tokens_per_s = b.num_tokens * args.steps / elapsed
        print(f"[bench] {ms_per_step:.2f} ms/step, {tokens_per_s / 1e6:.3f} M tokens/s",
              file=sys.stderr, flush=True)

    # ---- replay of one layer's kernel sequence through the kernel-level entries, timed with
    # HIP events on the same stream (layer 0's weights; every layer has the same shapes)
    d, H, h = p.d, p.H, p.h
    T = b.num_tokens
    lay = dm.layers[0]
    bf = torch.bfloat16
    xt = torch.empty(T, d, dtype=bf, device="cuda")
    big = torch.empty(T, max(4 * d, h), dtype=bf, device="cuda")
    yb = torch.empty(T, d, dtype=bf, device="cuda")
    xo = torch.empty_like(db.x)
    aws = M.workspace(M.mtgr_attention_workspace_size(db, d, H))
    seq = [
        ("gln1", lambda: M.mtgr_groupln_fwd(db, d, 0, 1, 1, norm_c, lay["gln1_gamma"], lay["gln1_beta"], p.ln_eps, db.x, xt)),
        ("qkvu", lambda: M.mtgr_linear_fwd(T, 4 * d, d, M.MTGR_BF16, M.MTGR_EPI_STORE, xt, lay["w_qkvu"], lay["b_qkvu"], None, big)),
        ("attention", lambda: M.mtgr_attention_fwd(db, d, H, M.MTGR_BF16, mask_c, big, yb, aws)),
        ("gln2", lambda: M.mtgr_groupln_fwd(db, d, 1, 1, 1, norm_c, lay["gln2_gamma"], lay["gln2_beta"], p.ln_eps, yb, xt)),
        ("mlp1", lambda: M.mtgr_linear_fwd(T, h, d, M.MTGR_BF16, M.MTGR_EPI_SILU, xt, lay["w_mlp1"], lay["b_mlp1"], None, big)),
        ("mlp2", lambda: M.mtgr_linear_fwd(T, d, h, M.MTGR_BF16, M.MTGR_EPI_RESIDUAL_F32, big, lay["w_mlp2"], lay["b_mlp2"], db.x, xo)),
    ]
    for _, fn in seq:
        fn()
    torch.cuda.synchronize()
    if args.profile_kernel == "layer":
        for _ in range(args.steps):
            for _, fn in seq:
                fn()
        torch.cuda.synchronize()
        print(json.dumps({"profile_kernel": "layer", "launches_each": args.steps + 1,
                          "kernels": [k for k, _ in seq]}), flush=True)
        return
    # Back-to-back replay: one event between consecutive launches on the library's stream and a
    # single synchronisation per layer, so every kernel runs in the same steady state as inside
    # the timed encoder steps (no idle gap, warm caches and clocks) and the per-kernel averages
    # match those of a rocprofv3 kernel trace of the same run.
    times = {k: 0.0 for k, _ in seq}
    for _ in range(args.replay_steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)]
        ev[0].record(stream)
        for i, (k, fn) in enumerate(seq):
            fn()
            ev[i + 1].record(stream)
        ev[-1].synchronize()
        for i, (k, _) in enumerate(seq):
            times[k] += ev[i].elapsed_time(ev[i + 1])
    ms = {k: v / args.replay_steps for k, v in times.items()}
    fl = flops_per_layer(b, d, h, args.mask)
    gemm_ms = ms["qkvu"] + ms["mlp1"] + ms["mlp2"]
    gemm_fl = fl["qkvu"] + fl["mlp1"] + fl["mlp2"]
    att_tflops = fl["attention"] / (ms["attention"] * 1e-3) / 1e12
    util_all = (gemm_fl + fl["attention"]) / ((gemm_ms + ms["attention"]) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    norm_bytes = {"gln1": T * d * (4 + 2), "gln2": T * d * (2 + 2)}
    kernels = {k: {"ms": round(v, 4)} for k, v in ms.items()}
    for k in ("qkvu", "mlp1", "mlp2", "attention"):
        kernels[k]["tflops"] = round(fl[k] / (ms[k] * 1e-3) / 1e12, 1)
    for k, by in norm_bytes.items():
        kernels[k]["gbs"] = round(by / (ms[k] * 1e-3) / 1e9, 1)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "users": b.num_users, "tokens": T,
                   "candidates": db.num_candidates, "layers": p.num_layers, "d_model": d,
                   "heads": H, "mlp_hidden": h, "mask": args.mask, "norm": args.norm,
                   "visible_pairs_per_layer": fl["pairs"]},
        "roofline": {"bound": "mfma", "kernel": "attention (fused masked silu + U gate)",
                     "achieved": round(att_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic() if args.mask == "dynamic" else None,
                     "flops_per_launch": fl["attention"], "launch_ms": round(ms["attention"], 4)},
        "mfma_util": {"gemm_plus_attention": round(util_all, 4),
                      "gemm": round(gemm_fl / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "attention": round(att_tflops / PEAK_BF16_TFLOPS, 4)},
        "kernels_per_layer": kernels,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample of users", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(b, p, args.mask, args.norm)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def cpu_baseline_tokenize(ids, groups, spec, tabs, pids, vals, budget_s=10.0):
    """The oracle's tokenizer (per-token Python/numpy) on a prefix of the batch's tokens until at
    least `budget_s` seconds of work; tokens per second."""
    from oracle import embedding_oracle as EO
    store = EO.EmbeddingStore(len(tabs), vals.shape[1])
    store.insert([EO.merged_key(t, i) for t, i in zip(tabs.tolist(), pids.tolist())], vals, 0)
    done, t0, chunk = 0, time.perf_counter(), 256
    while time.perf_counter() - t0 < budget_s and done < len(groups):
        EO.tokenize(ids[done:done + chunk], groups[done:done + chunk], spec.field_tables, store, spec.mlps)
        done += min(chunk, len(groups) - done)
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"the batch's first {done} tokens, per-token dict lookups + fp64 numpy MLP",
            "seconds": round(el, 2), "host": host_cpu()}


def bench_front_end(args, b, p, db, M, torch, synth):
    T, d, e = b.num_tokens, p.d, 64
    rng = np.random.default_rng(11)
    spec, ids, counts, tabs, pids, vals = synth.make_tokenizer_inputs(b, rng, d, e)
    store = M.DeviceHashTable(len(tabs), e, M.MTGR_BF16)
    M.mtgr_hash_init(store)
    M.mtgr_hash_insert(store, torch.from_numpy(M.tok_key(tabs, pids)).cuda(),
                       torch.from_numpy(vals).cuda().to(torch.bfloat16), 0, None,
                       M.workspace(M.mtgr_hash_insert_workspace_size(len(tabs))))
    tok = M.DeviceTokenizer(spec)
    ws = M.workspace(M.mtgr_tokenize_workspace_size(tok, db, store, counts))
    idd = torch.from_numpy(ids).cuda()
    x = torch.empty(T, d, dtype=torch.float32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(i):
        M.mtgr_tokenize(tok, db, counts, idd, store, i, x, flags, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = T * args.steps / elapsed
    assert int(flags.item()) == 0
    print(f"[bench] tokenizer {ms_per_step:.3f} ms/step, {tokens_per_s / 1e6:.2f} M tokens/s",
          file=sys.stderr, flush=True)
    n_keys = int(sum(counts[g] * len(spec.field_tables[g]) for g in range(4)))

    # store lookup: 8M rows of 64 bf16, index at 1/2 load; 4M random keys of the live set
    rows, n_look = 8 << 20, 4 << 20
    big = M.DeviceHashTable(rows, e, M.MTGR_BF16, index_cap=2 * rows)
    M.mtgr_hash_init(big)
    keys_all = torch.randint(0, 1 << 62, (rows,), dtype=torch.int64, device="cuda")
    init = torch.randn(rows, e, device="cuda").to(torch.bfloat16)
    M.mtgr_hash_insert(big, keys_all, init, 0, None, M.workspace(M.mtgr_hash_insert_workspace_size(rows)))
    ins_ws = M.workspace(M.mtgr_hash_insert_workspace_size(rows))
    ins = 0.0
    for _ in range(2):                                 # init + insert of all 8M keys, timed
        M.mtgr_hash_init(big)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        M.mtgr_hash_insert(big, keys_all, init, 0, None, ins_ws)
        e1.record(torch.cuda.current_stream())
        e1.synchronize()
        ins = e0.elapsed_time(e1)
    look = keys_all[torch.randint(0, rows, (n_look,), device="cuda")].contiguous()
    out = torch.empty(n_look, e, dtype=torch.bfloat16, device="cuda")
    M.mtgr_hash_lookup(big, look, -1, out, None)
    torch.cuda.synchronize()
    assert M.mtgr_hash_get_stats(big)["live"] == len(torch.unique(keys_all))
    stream = torch.cuda.current_stream()
    tot = 0.0
    for _ in range(args.replay_steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        M.mtgr_hash_lookup(big, look, -1, out, None)
        e1.record(stream)
        e1.synchronize()
        tot += e0.elapsed_time(e1)
    look_ms = tot / args.replay_steps
    row_bytes = e * 2
    look_bytes = n_look * (8 + 16 + 2 * row_bytes)     # key, slot, value read, value written
    gbs = look_bytes / (look_ms * 1e-3) / 1e9
    out_json = {
        "metric": "tokenizer front-end tokens/sec (bf16; key dedup + hash-store lookup + per-group MLP) "
                  "on one MI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "users": b.num_users, "tokens": T, "d_model": d, "emb_dim": e,
                   "group_tokens": [int(c) for c in counts], "field_keys": n_keys, "store_rows": len(tabs)},
        "roofline": {"bound": "hbm", "kernel": "hash-store lookup (8M-row store, 4M random keys)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": look_bytes, "launch_ms": round(look_ms, 4),
                     "lookups_per_s": round(n_look / (look_ms * 1e-3), 1)},
        "store_insert": {"keys": rows, "ms": round(ins, 4), "inserts_per_s": round(rows / (ins * 1e-3), 1)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle's tokenizer on a prefix of the tokens", file=sys.stderr, flush=True)
        out_json["cpu_baseline"] = cpu_baseline_tokenize(ids, b.group_ids, spec, tabs, pids, vals)
    else:
        out_json["cpu_baseline"] = None
    print(json.dumps(out_json), flush=True)


def bench_block_bwd(args, b, p, db, dm, M, torch):
    T, d, H, h = b.num_tokens, p.d, p.H, p.h
    blk = dm.blocks[0]
    ws = M.workspace(M.mtgr_block_bwd_workspace_size(blk, db))
    rng = np.random.default_rng(7)
    dout = rng.standard_normal((T, d)).astype(np.float32)
    dxo = torch.from_numpy(dout).cuda()
    dxi = torch.empty_like(dxo)
    shapes = {"gln1_gamma": (4, d), "gln1_beta": (4, d), "w_qkvu": (4 * d, d), "b_qkvu": (4 * d,),
              "gln2_gamma": (4, d), "gln2_beta": (4, d), "w_mlp1": (h, d), "b_mlp1": (h,),
              "w_mlp2": (d, h), "b_mlp2": (d,)}
    grads = {k: torch.empty(s_, dtype=torch.float32, device="cuda") for k, s_ in shapes.items()}

    def step():
        M.mtgr_block_bwd(blk, db, db.x, dxo, dxi, grads, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = T * args.steps / elapsed
    print(f"[bench] block backward {ms_per_step:.2f} ms/step, {tokens_per_s / 1e6:.3f} M tokens/s",
          file=sys.stderr, flush=True)

    # attention backward alone (prep, gate, dK/dV, dQ) on layer 0's activations, HIP events on the
    # library's stream
    stream = torch.cuda.current_stream()
    bf = torch.bfloat16
    lay = dm.layers[0]
    xt = torch.empty(T, d, dtype=bf, device="cuda")
    qkvu = torch.empty(T, 4 * d, dtype=bf, device="cuda")
    mask_c, norm_c = M.MASK_MODES[args.mask], M.NORM_MODES[args.norm]
    M.mtgr_groupln_fwd(db, d, 0, 1, 1, norm_c, lay["gln1_gamma"], lay["gln1_beta"], p.ln_eps, db.x, xt)
    M.mtgr_linear_fwd(T, 4 * d, d, M.MTGR_BF16, M.MTGR_EPI_STORE, xt, lay["w_qkvu"], lay["b_qkvu"], None, qkvu)
    vt = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda().to(bf)
    dy = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda().to(bf)
    dq = torch.empty(T, 4 * d, dtype=bf, device="cuda")
    aws = M.workspace(M.mtgr_attention_bwd_workspace_size(db, d, H, M.MTGR_BF16))
    M.mtgr_attention_bwd(db, d, H, M.MTGR_BF16, mask_c, qkvu, vt, dy, dq, aws)
    torch.cuda.synchronize()
    att = 0.0
    for _ in range(args.replay_steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        M.mtgr_attention_bwd(db, d, H, M.MTGR_BF16, mask_c, qkvu, vt, dy, dq, aws)
        e1.record(stream)
        e1.synchronize()
        att += e0.elapsed_time(e1)
    att_ms = att / args.replay_steps
    pairs = int(visible_pairs_per_user(b, args.mask).sum())
    # algorithmic: S, dP, dV, dQ, dK, 2 d FLOPs each per visible pair; the kernels execute 14 d
    # (the dQ pass recomputes S and dP so that dQ is written without atomics)
    att_fl = 10.0 * d * pairs
    att_fl_exec = 14.0 * d * pairs
    att_tflops = att_fl / (att_ms * 1e-3) / 1e12
    out = {
        "metric": "block backward tokens/sec (bf16; forward recompute + dX + parameter gradients of "
                  "one HSTU block) on one MI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "block": 0, "users": b.num_users, "tokens": T,
                   "d_model": d, "heads": H, "mlp_hidden": h, "mask": args.mask, "norm": args.norm,
                   "visible_pairs": pairs},
        "roofline": {"bound": "mfma", "kernel": "attention backward (gate + dK/dV + dQ launches)",
                     "achieved": round(att_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": att_fl, "launch_ms": round(att_ms, 4),
                     "executed_flops_per_launch": att_fl_exec,
                     "executed_tflops": round(att_fl_exec / (att_ms * 1e-3) / 1e12, 1)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle's block backward on a sample of users", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_block_bwd(b, p, dout, args.mask, args.norm)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
