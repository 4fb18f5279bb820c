#!/usr/bin/env python3
"""Benchmark of sharded paged decode attention on one MI355X.

Default workload (mla_bf16_b64_bimodal): absorbed-MLA decode with a bf16
latent cache, batch 64, 64 query heads over a 576-wide latent (value = first
512 columns), block size 64, D = 8 interleaved shards, context lengths drawn as
stratified quantiles of the agentic-trace statistics (median ~67K, 53 % above
64K, ~8 % above 128K, ~3 % above 256K; sum 5,065,388 tokens, max 769,505).

One step = one dcp_decode_all_shards call over the whole batch: work plan,
attention over all D shards, and the LSE merge -- one decode token per
sequence through one attention layer, inputs already resident in HBM.

`--q-len N` times multi-token (draft) decode instead: N query tokens per
sequence, each seeing the positions up to its own; `value` still counts each
cached byte once per step and tok/s counts every query token.

Prints one JSON line. `value` is KV GB/s: bytes of cached latent rows the step
must read (sum of lengths x 1152 B) divided by the wall time of a step.
`roofline.achieved` divides the same bytes by the attention kernel's own
average duration, measured with HIP events recorded on its stream around
every timed launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
PROFILES = ROOT / "profiles"
# Sources whose change can move the attention kernel's HBM traffic: the kernels,
# the work plan that assigns their block ranges, and the launch code.
KERNEL_SOURCES = ["mla.hip", "gqa.hip", "dcp_internal.hpp", "plan_merge.hip", "api.hip"]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "decode_attention_sequence_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def traffic_from_counters(workload: str):
    """HBM bytes per attention launch from committed counter runs, if current."""
    path = PROFILES / f"{workload}_hbm_traffic.json"
    if not path.exists():
        return None
    rec = json.loads(path.read_text())
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None  # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def _oracle_pass(w, picks, budget_s, o_gpu=None, lse_gpu=None):
    """Run the oracle sequence by sequence over `picks` until `budget_s` seconds
    of oracle time are spent; returns (sequences done, tokens, seconds, errors)."""
    import oracle

    done, tokens, t_used, errs = [], 0, 0.0, []
    for b in picks:
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.decode_reference(w, batch_indices=[b])
        t_used += time.perf_counter() - t0
        done.append(b)
        tokens += int(w.seq_lens[b])
        if o_gpu is not None:
            diff = o_gpu[b].astype(np.float64) - o_ref[b]
            errs.append((np.linalg.norm(diff) / np.linalg.norm(o_ref[b]), np.abs(diff).max(),
                         np.abs(lse_gpu[b] - lse_ref[b]).max()))
        if t_used >= budget_s:
            break
    return done, tokens, t_used, errs


def cpu_baseline(w, o_gpu, lse_gpu, budget_s: float):
    """Time the fp64 oracle on a stratified sample of the workload's sequences,
    with the host's BLAS threads and again on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    order = np.argsort(w.seq_lens, kind="stable")
    # Stratified over the sorted lengths: passes over every 8th sequence, each pass
    # starting at a different offset inside the groups of 8, so that any prefix of the
    # visit order spans the whole length range. Stops once the budget is spent or
    # every sequence was visited.
    picks = [int(order[i]) for off in (4, 0, 6, 2, 5, 1, 7, 3)
             for i in range(off, len(order), 8)]
    done, tokens, t_used, errs = _oracle_pass(w, picks, budget_s, o_gpu, lse_gpu)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    per_tok = w.spec.kv_bytes_per_token()
    kv = tokens * per_tok
    rate = kv / t_used / 1e9
    sample = (f"fp64 oracle on {len(done)} of {w.spec.batch} sequences (stratified by length), "
              f"{tokens} tokens = {kv / 1e9:.3f} GB of cached rows in {t_used:.1f} s")
    # One-thread leg: the same visit order on a third of the budget.
    with threadpool_limits(limits=1):
        done1, tokens1, t1, _ = _oracle_pass(w, picks, budget_s / 3)
    kv1 = tokens1 * per_tok
    parity = {"sequences": len(done), "worst_rel_l2": float(max(e[0] for e in errs)),
              "max_abs": float(max(e[1] for e in errs)), "lse_abs": float(max(e[2] for e in errs))}
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"value": rate, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "blas_threads": int(threads),
            "single_thread": {"value": kv1 / t1 / 1e9, "unit": "GB/s", "cores": 1,
                              "sample": f"fp64 oracle on one thread, {len(done1)} sequences, "
                                        f"{tokens1} tokens = {kv1 / 1e9:.3f} GB in {t1:.1f} s"}}, parity


def components(dcp, desc, dev, w, ws, iters: int = 20):
    """The path's calls one by one, at the workload's real shapes: the
    ownership remap, one shard's partial (the share one GPU of D would run;
    shard 0, and the slowest shard), and the LSE merge of the D partials.
    Wall time per call over `iters` back-to-back calls, bracketed by
    synchronisation."""
    import torch

    spec = w.spec
    D = spec.num_shards

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(iters):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / iters

    remap_ms = timed(lambda: dcp.block_remap(dev.block_table, dev.seq_lens, spec.block_size, D))
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, spec.block_size, D)
    o_parts = torch.empty((D, spec.batch, spec.num_q_heads, spec.v_dim), dtype=torch.float32,
                          device="cuda")
    lse_parts = torch.empty((D, spec.batch, spec.num_q_heads), dtype=torch.float32, device="cuda")
    per_token = spec.kv_bytes_per_token()
    shard_tokens = ll.sum(dim=1).cpu().numpy().astype(np.int64)
    shard_ms = []
    for r in range(D):
        ltr, llr = lt[r].contiguous(), ll[r].contiguous()
        shard_ms.append(timed(lambda: dcp.decode_partial(
            desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale, ltr, llr, workspace=ws,
            o_partial=o_parts[r], lse_partial=lse_parts[r])))
    out = torch.empty((spec.batch, spec.num_q_heads, spec.v_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device="cuda")
    merge_ms = timed(lambda: dcp.lse_merge(o_parts, lse_parts, out=out, lse_out=lse))
    merge_bytes = (o_parts.numel() + lse_parts.numel() + out.numel() + lse.numel()) * 4
    slow = int(np.argmax(shard_ms))

    def shard(r, ms=None):
        ms = shard_ms[r] if ms is None else ms
        b = int(shard_tokens[r]) * per_token
        return {"shard": r, "ms": round(ms, 4), "kv_bytes": b,
                "GBps": round(b / (ms * 1e-3) / 1e9, 1)}

    # Plan once per decode step, run per layer: the same shards' partials run
    # on a plan made before the timed calls (every layer of a step shares the
    # lengths, hence the plan).
    ws_plan = dcp.alloc_workspace(desc, torch.device("cuda"))
    run_ms = {}
    for r in sorted({0, slow}):
        ltr, llr = lt[r].contiguous(), ll[r].contiguous()
        dcp.decode_partial_plan(desc, llr, ws_plan)
        run_ms[r] = timed(lambda: dcp.decode_partial_run(
            desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale, ltr, ws_plan,
            o_partial=o_parts[r], lse_partial=lse_parts[r]))
    # Token-level ownership (position t on shard t % D): shard 0's partial read
    # in place from the global table, every D-th row of each block.
    lens_h = dev.seq_lens.cpu().numpy().astype(np.int64)
    tok_bytes = int(((lens_h + D - 1) // D).sum()) * per_token
    try:
        tok_ms = timed(lambda: dcp.decode_partial_token(
            desc, 0, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale, dev.block_table, dev.seq_lens,
            workspace=ws, o_partial=o_parts[0], lse_partial=lse_parts[0]))
        token0 = {"shard": 0, "ms": round(tok_ms, 4), "kv_bytes": tok_bytes,
                  "GBps": round(tok_bytes / (tok_ms * 1e-3) / 1e9, 1)}
    except dcp.DcpValueError:  # (blocks not a multiple of D tokens)
        token0 = None
    dcp.decode_all_shards_plan(desc, dev.seq_lens, ws_plan)
    fused_out = torch.empty((spec.batch, spec.num_q_heads, spec.v_dim),
                            dtype=torch.float32 if desc.out_dtype == dcp.F32 else torch.bfloat16,
                            device="cuda")
    fused_run_ms = timed(lambda: dcp.decode_all_shards_run(
        desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale, dev.block_table, ws_plan,
        out=fused_out, want_lse=False))
    fused_bytes = int(shard_tokens.sum()) * per_token

    # A decode step's cache maintenance: one new token per sequence, written at
    # the last position each table row maps, into a scratch pool of one block
    # per sequence (so the workload's cache stays as generated), and the
    # incremental table update from L - 1 to L tokens.
    B, bs = spec.batch, spec.block_size
    kind_rows = (B, spec.num_kv_heads, spec.qk_dim) if spec.kind == "gqa" else (B, spec.qk_dim)
    new_dt = torch.float32 if spec.kv_dtype == "f32" else torch.bfloat16
    k_new = torch.randn(kind_rows, device="cuda").to(new_dt)
    v_new = (torch.randn((B, spec.num_kv_heads, spec.v_dim), device="cuda").to(new_dt)
             if spec.kind == "gqa" else None)
    pool_k = torch.empty((B,) + tuple(dev.k_cache.shape[1:]), dtype=dev.k_cache.dtype, device="cuda")
    pool_v = torch.empty_like(pool_k) if dev.v_cache is not None else None
    pool_s = (torch.empty((B, bs), dtype=torch.float32, device="cuda")
              if dev.kv_scale is not None else None)
    scratch_table = torch.arange(B, dtype=torch.int32, device="cuda")[:, None].expand(
        B, dev.block_table.shape[1]).contiguous()
    sdesc = dcp.make_desc(desc.kv_kind, dev.q, pool_k, scratch_table, num_shards=D,
                          v_dim=spec.v_dim, softmax_scale=spec.softmax_scale)
    pos = (dev.seq_lens - 1).clamp(min=0).to(torch.int32).contiguous()
    append_ms = timed(lambda: dcp.kv_append(sdesc, pos, k_new, v_new, scratch_table, pool_k,
                                             pool_v, pool_s))
    lt_u, ll_u = lt.clone(), ll.clone()
    upd_ms = timed(lambda: dcp.block_remap_update(dev.block_table, pos, dev.seq_lens,
                                                  spec.block_size, D, lt_u, ll_u))
    return {
        "note": ("per call, wall time of back-to-back calls; each dcp_decode_partial includes its own "
                 "plan and piece merge; the *_run entries run on a plan made once before them "
                 "(dcp_decode_partial_plan / dcp_decode_all_shards_plan), as every layer of a "
                 "decode step can; decode_partial_token_shard0 is shard 0 under token-level "
                 "ownership (its plan included)"),
        "block_remap_ms": round(remap_ms, 4),
        "block_remap_update_ms": round(upd_ms, 4),
        "kv_append_ms": round(append_ms, 4),
        "decode_partial_shard0": shard(0),
        "decode_partial_slowest": shard(slow),
        "decode_partial_run_shard0": shard(0, run_ms[0]),
        "decode_partial_run_slowest": shard(slow, run_ms[slow]),
        "decode_partial_token_shard0": token0,
        "decode_all_shards_run": {"ms": round(fused_run_ms, 4), "kv_bytes": fused_bytes,
                                  "GBps": round(fused_bytes / (fused_run_ms * 1e-3) / 1e9, 1)},
        "lse_merge": {"partials": D, "ms": round(merge_ms, 4), "bytes": merge_bytes,
                      "GBps": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1)},
    }


def copy_probe(mib: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch

    n = mib * (1 << 20) // 4
    x = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copy probe: 3 copies of {mib} MiB (read {mib} MiB + write {mib} MiB each)")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # A step is about a millisecond. In a fresh process the attention kernel's
    # launches 3 to about 20 run up to 45 % slower than later ones when
    # launched back to back (a transient of the GPU's power management), so the
    # defaults time 100 steps after 20 warm-up steps; `--steps 20 --warmup 5`
    # reads about 5-8 % below this sustained rate.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=W.HEADLINE, choices=sorted(W.SPECS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true",
                    help="skip the per-call timings of remap, one shard's partial and the merge")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (multi-token decode when > 1)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the "
              "D shards are simulated on one device and no cross-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_attention_sequence_amd as dcp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dcp.lib()
    spec = W.SPECS[args.workload]
    if args.q_len > 1:
        from dataclasses import replace

        spec = replace(spec, name=f"{spec.name}_q{args.q_len}", q_len=args.q_len)
    log(f"generating {spec.name} inputs on the host")
    t0 = time.perf_counter()
    w = W.make(spec)
    log(f"generated {w.num_blocks} blocks in {time.perf_counter() - t0:.1f} s; uploading")
    dev = W.to_torch(w, "cuda")
    torch.cuda.synchronize()
    kind = dcp.KV_LATENT if spec.kind == "mla" else dcp.KV_SEPARATE
    desc = dcp.make_desc(kind, dev.q, dev.k_cache, dev.block_table, num_shards=spec.num_shards,
                         v_dim=spec.v_dim, softmax_scale=spec.softmax_scale,
                         max_seq_len=int(w.seq_lens.max()), q_len=spec.q_len)
    ws = dcp.alloc_workspace(desc, "cuda")
    rows = spec.q_len * spec.num_q_heads
    out = torch.empty((spec.batch, rows, spec.v_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((spec.batch, rows), dtype=torch.float32, device="cuda")

    def step(events=None):
        dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                              dev.block_table, dev.seq_lens, workspace=ws, out=out, lse_out=lse,
                              attn_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    evs = [(dcp.HipEvent(), dcp.HipEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    attn_ms = float(np.mean([b.elapsed_ms(e) for b, e in evs]))
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, attention kernel {attn_ms:.3f} ms")

    kv_bytes = w.kv_bytes()
    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (attn_ms * 1e-3) / 1e9
    traffic = traffic_from_counters(spec.name)
    result = {
        "metric": "decode-attn KV HBM GB/s (% of peak) + tok/s per layer, MLA batch 64, D=8",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.kv_dtype,
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tok_per_s_per_layer": round(spec.batch * spec.q_len / (ms_per_step * 1e-3), 1),
        "config": {
            "workload": spec.name,
            "batch": spec.batch,
            "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads,
            "qk_dim": spec.qk_dim,
            "v_dim": spec.v_dim,
            "block_size": spec.block_size,
            "num_shards": spec.num_shards,
            "q_len": spec.q_len,
            "sum_seq_len": int(w.seq_lens.sum()),
            "max_seq_len": int(w.seq_lens.max()),
            "kv_bytes": kv_bytes,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_ms": round(attn_ms, 4),
        },
    }
    if not args.no_components and spec.q_len == 1:
        log("timing the path's calls one by one")
        result["components"] = components(dcp, desc, dev, w, ws)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        base, parity = cpu_baseline(w, out.cpu().numpy(), lse.cpu().numpy(), args.cpu_seconds)
        result["cpu_baseline"] = base
        result["parity_sample"] = parity
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
