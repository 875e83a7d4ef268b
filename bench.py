"""Decode throughput of the persistent MoE megakernel on one MI355X.

Workload (default): synthetic 30B-total / 3.3B-active MoE decoder (48 layers,
hidden 2048, 32 q / 4 kv heads of 128, 128 experts top-8 SwiGLU with width
768, vocab 151936, untied LM head), BF16 weights drawn N(0, 0.02), batch 1
at 8K context (8192 cached tokens, N(0,1) BF16 KV in 16-token pages), greedy
decode. A "step" is one whole decode step: embedding through logits, one
launch of the persistent kernel, plus the caller's greedy argmax.

Prints one JSON line: decode tok/s, the per-op (one launch per operation)
build of the same tiles in the same harness, the roofline of the megakernel
(algorithmic bytes per step / measured kernel time vs the 8 TB/s HBM peak) and
the CPU oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-schedule]
                       [--sweep 4,16,64 [--sweep-steps K]] [--long 32768,131072,262144]
                       [--ragged] [--prefill 512,2048 [--prefill-prefix N]]

"schedule" is one traced step of the same workload after the timed ones:
the fraction of workgroup time spent waiting on dependency counters (with
the loads issued before each wait), the fraction computing, the fraction of
compute units with a workgroup computing, and the time each dependency level
adds to a layer.

--long adds, under "long_context", batch 1 at other context lengths (e.g.
32768,131072,262144; 32 timed steps each): megakernel and per-op tok/s, kernel
time, algorithmic bytes per step and % of 8 TB/s.

--ragged adds, under "ragged", the churning batch: 32 sequences with contexts
log-uniform on [128, 32768], 4 of them replaced every 8 steps by new ones
(contexts uniform on [128, 2048]), a Zipf(1.1) router bias, 256 timed steps;
the megakernel (its default: the ragged contexts make it share the
attention, merge, output-projection and expert levels, whose tiles workgroups
then claim from per-level pools), the megakernel with fixed per-workgroup
lists only, and the per-op build.

--prefill adds, under "prefill", prompt ingestion: each prompt length in
multi-token steps of up to 64 rows of one sequence (one launch per block,
causal attention over the cache and the earlier rows), prompt tok/s over the
whole prompt and the blocks' bytes against 8 TB/s, megakernel and per-op.

--sweep adds, under "batch_sweep", the same measurement at other batch sizes
(each sequence at the same context, pages from a shuffled pool, per-sequence
seeded first tokens): megakernel and per-op tok/s, kernel time, algorithmic
bytes per step with the counted distinct experts, and % of 8 TB/s.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s at batch 1, 8K ctx + % of HBM speed-of-light (bytes/step÷BW)"
PEAK_GBS = 8000.0


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha256() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "persistent_megakernel_03_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(batch: int, ctx: int):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter
    summary for this workload, or None when there is none or the kernel
    sources have changed since the counters were taken."""
    if batch != 1 or ctx != 8192:
        return None
    path = os.path.join(ROOT, "profiles", "k_persistent_a3b_b1_ctx8192_hbm_counters.md")
    try:
        text = open(path).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    if data.get("source_sha256") != kernel_source_sha256():
        return None
    return int(data["traffic_bytes_per_launch"])


def distinct_experts(route_ids: np.ndarray, B: int) -> list:
    return [len(set(route_ids[l, :B].reshape(-1).tolist())) for l in range(route_ids.shape[0])]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--context", type=int, default=8192)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-steps", type=int, default=8)
    ap.add_argument("--no-perop", action="store_true")
    ap.add_argument("--no-schedule", action="store_true", help="skip the traced step (wait-stall and busy fractions)")
    ap.add_argument("--wg-per-cu", type=int, default=0, help="persistent workgroups per compute unit (0 = auto, 2)")
    ap.add_argument("--mfma-min-batch", type=int, default=0,
                    help="smallest batch on the matrix-core schedule (0 = default 3; 1 or 2 move those batches to it)")
    ap.add_argument("--mm-row-blocks", type=int, default=0,
                    help="row blocks per matrix-core expert tile (0 = chosen per step; 1 or 2 force it)")
    ap.add_argument("--sweep", type=str, default="", help="comma-separated batch sizes to measure as well")
    ap.add_argument("--sweep-steps", type=int, default=32)
    ap.add_argument("--long", type=str, default="", help="comma-separated batch-1 context lengths to measure as well")
    ap.add_argument("--long-steps", type=int, default=32)
    ap.add_argument("--ragged", action="store_true", help="also measure the churning 32-sequence batch")
    ap.add_argument("--ragged-steps", type=int, default=256)
    ap.add_argument("--prefill", type=str, default="",
                    help="prompt lengths to ingest (multi-token steps of up to 64 rows), e.g. 512,2048")
    ap.add_argument("--prefill-prefix", type=int, default=0, help="tokens already cached before each prompt")
    ap.add_argument("--calib-lmhead", action="store_true",
                    help="also run one per-op step, whose LM-head level is a single dispatch reading exactly the "
                         "V x H BF16 LM-head matrix through the kernels' own weight loads (HBM counter calibration)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from persistent_megakernel_03_amd import configs, mk, sol, synth

    cfg = configs.A3B
    B, ctx = args.batch, args.context
    P = cfg["page_size"]
    t0 = time.time()
    log(f"generating weights ({cfg['n_layers']} layers) on device")
    weights = synth.make_model(cfg, 0, "cuda")

    def make_inputs(B, steps, warmup, ctx=ctx):
        total_tokens = ctx + warmup + steps + 16 + 1  # + the per-step kernel timing pass
        pages_per_seq = -(-total_tokens // P)
        n_pages = pages_per_seq * B + 1
        log(f"batch {B}: KV for {B} x {ctx} tokens ({n_pages} pages, {2 * k_bytes(n_pages) / 1e9:.1f} GB) on device")
        k_pool, v_oracle_layout = synth.make_kv_pool(cfg, n_pages, 1, "cuda")
        v_pool = v_oracle_layout.transpose(-1, -2).contiguous()
        del v_oracle_layout
        torch.cuda.synchronize()
        block_tables = synth.make_block_tables(B, pages_per_seq, n_pages, shuffle=B > 1)
        tok0 = synth.make_tokens(B, cfg["vocab"], seed=3)
        return pages_per_seq, k_pool, v_pool, block_tables, tok0

    def k_bytes(n_pages):
        return cfg["n_layers"] * n_pages * cfg["n_kv_heads"] * P * cfg["head_dim"] * 2

    pages_per_seq, k_pool, v_pool, block_tables, tok0 = make_inputs(B, args.steps, args.warmup)
    log(f"inputs ready in {time.time() - t0:.1f}s")

    def run(mode: int, steps: int, warmup: int, k, v, B=B, pages_per_seq=pages_per_seq, block_tables=block_tables,
            tok0=tok0, ctx=ctx):
        dec = mk.Decoder(cfg, weights, k, v, max_batch=B, max_pages_per_seq=pages_per_seq, mode=mode,
                         wg_per_cu=args.wg_per_cu, mfma_min_batch=args.mfma_min_batch,
                         mm_row_blocks=args.mm_row_blocks, time_kernels=True)
        tokens = torch.tensor(tok0, dtype=torch.int32, device="cuda")
        logits = torch.empty(B, cfg["vocab"], dtype=torch.float32, device="cuda")
        pos = [ctx] * B
        stream = torch.cuda.current_stream()

        def one():
            dec.step(pos, block_tables, tokens, logits)
            tokens.copy_(torch.argmax(logits, dim=1).to(torch.int32))
            for b in range(B):
                pos[b] += 1

        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        assert dec.sync_check() == mk.MK_OK
        start = time.perf_counter()
        for _ in range(steps):
            one()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - start
        st = dec.sync_check()
        if st != mk.MK_OK:
            raise RuntimeError(f"device status {st}")
        # kernel-only time per step: HIP events bracketing the step's kernels,
        # one step at a time
        kms = []
        for _ in range(min(16, steps)):
            one()
            kms.append(dec.kernel_ms())
        dbg = dec.debug()
        off = dbg.route_ids - dec.workspace.data_ptr()
        n = cfg["n_layers"] * B * cfg["top_k"]
        rid = dec.workspace[off:off + 4 * n].view(torch.int32).view(cfg["n_layers"], B, cfg["top_k"]).cpu().numpy()
        dec.close()
        return elapsed, float(np.median(kms)), rid, list(pos)

    log(f"megakernel: {args.warmup} warmup + {args.steps} timed steps")
    k1, v1 = k_pool.clone(), v_pool.clone()
    el, kms, rid, pos_end = run(mk.MK_MODE_MEGAKERNEL, args.steps, args.warmup, k1, v1)
    del k1, v1
    ms_per_step = 1e3 * el / args.steps
    tok_s = B * args.steps / el
    # algorithmic bytes of the last timed step (contexts just before it, counted experts)
    ctx_last = [p - 1 for p in pos_end]
    bytes_step = sol.step_bytes(cfg, ctx_last, distinct_experts(rid, B), distinct_tokens=B)
    achieved = bytes_step / (kms * 1e-3) / 1e9
    log(f"megakernel: {tok_s:.1f} tok/s, {ms_per_step:.3f} ms/step, kernel {kms:.3f} ms, "
        f"{achieved:.0f} GB/s ({100 * achieved / PEAK_GBS:.1f}% of 8 TB/s)")

    if args.calib_lmhead:
        k2, v2 = k_pool.clone(), v_pool.clone()
        run(mk.MK_MODE_PEROP, 1, 0, k2, v2)
        del k2, v2
        log(f"calibration: two per-op steps run; each LM-head level dispatch reads "
            f"{cfg['vocab'] * cfg['hidden'] * 2} bytes of weights")

    perop = None
    if not args.no_perop:
        k2, v2 = k_pool.clone(), v_pool.clone()
        steps2 = max(8, args.steps // 4)
        el2, kms2, _, _ = run(mk.MK_MODE_PEROP, steps2, 3, k2, v2)
        del k2, v2
        eager = {"value": round(B * steps2 / el2, 2), "ms_per_step": round(1e3 * el2 / steps2, 4),
                 "kernel_ms": round(kms2, 4), "steps": steps2}
        log(f"per-op: {eager['value']:.1f} tok/s, kernels {kms2:.3f} ms/step")
        k2, v2 = k_pool.clone(), v_pool.clone()
        try:
            graph = perop_graph(cfg, weights, k2, v2, block_tables, tok0, ctx, B, pages_per_seq, steps2, 3)
            log(f"per-op as a HIP graph: {graph['value']:.1f} tok/s, {graph['ms_per_step']:.3f} ms/step")
        except RuntimeError as e:   # capture refused: the eager figure stands
            graph = {"value": 0.0, "error": str(e)[:200]}
            log(f"per-op as a HIP graph: not measured ({graph['error']})")
        del k2, v2
        best = graph if graph["value"] > eager["value"] else eager
        perop = {"value": best["value"], "unit": "tok/s", "ms_per_step": best["ms_per_step"],
                 "kind": "per-op launches, same tiles; the better of eager launches and one captured HIP graph "
                         "per step", "eager": eager, "graph": graph}

    sched = None
    if not args.no_schedule:
        k3, v3 = k_pool.clone(), v_pool.clone()
        sched = schedule_stats(cfg, weights, k3, v3, block_tables, tok0, ctx, B, pages_per_seq)
        del k3, v3

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, weights, k_pool, v_pool, block_tables, tok0, ctx, B, args.cpu_steps)

    sweep = []
    if args.sweep:
        del k_pool, v_pool
        torch.cuda.empty_cache()
        for Bs in [int(x) for x in args.sweep.split(",") if x]:
            steps_s, warm_s = args.sweep_steps, 5
            pps, kp, vp, bts, tk = make_inputs(Bs, steps_s, warm_s)
            k1, v1 = kp.clone(), vp.clone()
            el_s, kms_s, rid_s, pe_s = run(mk.MK_MODE_MEGAKERNEL, steps_s, warm_s, k1, v1, Bs, pps, bts, tk)
            del k1, v1
            k2, v2 = kp.clone(), vp.clone()
            el_p, kms_p, _, _ = run(mk.MK_MODE_PEROP, max(8, steps_s // 2), 3, k2, v2, Bs, pps, bts, tk)
            del k2, v2
            k2, v2 = kp.clone(), vp.clone()
            g_p = graph_or_none(cfg, weights, k2, v2, bts, tk, ctx, Bs, pps, max(8, steps_s // 2))
            del k2, v2, kp, vp
            torch.cuda.empty_cache()
            nexp = distinct_experts(rid_s, Bs)
            by = sol.step_bytes(cfg, [p - 1 for p in pe_s], nexp, distinct_tokens=Bs)
            ach = by / (kms_s * 1e-3) / 1e9
            rec = {"batch": Bs, "value": round(Bs * steps_s / el_s, 2), "unit": "tok/s",
                   "ms_per_step": round(1e3 * el_s / steps_s, 4), "kernel_ms": round(kms_s, 4),
                   "bytes_per_step": by, "distinct_experts_mean": round(float(np.mean(nexp)), 2),
                   "achieved_gbs": round(ach, 1), "frac": round(ach / PEAK_GBS, 4),
                   "sol_tok_s": round(sol.sol_tokens_per_s(by, Bs), 1),
                   "perop_eager_value": round(Bs * max(8, steps_s // 2) / el_p, 2), "perop_kernel_ms": round(kms_p, 4),
                   "perop_graph_value": g_p, "steps": steps_s}
            rec["perop_value"] = max(rec["perop_eager_value"], g_p or 0.0)
            log(f"batch {Bs}: {rec['value']:.1f} tok/s (kernel {kms_s:.3f} ms, {100 * rec['frac']:.1f}% of 8 TB/s, "
                f"{rec['distinct_experts_mean']} experts/layer); per-op {rec['perop_value']:.1f} tok/s "
                f"(kernels {kms_p:.3f} ms)")
            sweep.append(rec)

    long_ctx = []
    if args.long:
        if not args.sweep:
            del k_pool, v_pool
            torch.cuda.empty_cache()
        for T in [int(x) for x in args.long.split(",") if x]:
            steps_l, warm_l = args.long_steps, 3
            pps, kp, vp, bts, tk = make_inputs(1, steps_l, warm_l, ctx=T)
            el_l, kms_l, rid_l, pe_l = run(mk.MK_MODE_MEGAKERNEL, steps_l, warm_l, kp, vp, 1, pps, bts, tk, ctx=T)
            del kp, vp
            torch.cuda.empty_cache()
            # the per-op build on a fresh pool of the same contents (the megakernel run appended to the first)
            pps, kp, vp, bts, tk = make_inputs(1, steps_l, warm_l, ctx=T)
            el_p, kms_p, _, _ = run(mk.MK_MODE_PEROP, max(4, steps_l // 4), 2, kp, vp, 1, pps, bts, tk, ctx=T)
            g_p = graph_or_none(cfg, weights, kp, vp, bts, tk, T, 1, pps, max(4, steps_l // 4))
            del kp, vp
            torch.cuda.empty_cache()
            by = sol.step_bytes(cfg, [p - 1 for p in pe_l], distinct_experts(rid_l, 1), distinct_tokens=1)
            ach = by / (kms_l * 1e-3) / 1e9
            rec = {"context": T, "value": round(steps_l / el_l, 2), "unit": "tok/s",
                   "ms_per_step": round(1e3 * el_l / steps_l, 4), "kernel_ms": round(kms_l, 4),
                   "bytes_per_step": by, "achieved_gbs": round(ach, 1), "frac": round(ach / PEAK_GBS, 4),
                   "sol_tok_s": round(sol.sol_tokens_per_s(by, 1), 1),
                   "perop_eager_value": round(max(4, steps_l // 4) / el_p, 2), "perop_kernel_ms": round(kms_p, 4),
                   "perop_graph_value": g_p, "steps": steps_l}
            rec["perop_value"] = max(rec["perop_eager_value"], g_p or 0.0)
            log(f"context {T}: {rec['value']:.1f} tok/s (kernel {kms_l:.3f} ms, {100 * rec['frac']:.1f}% of 8 TB/s); "
                f"per-op {rec['perop_value']:.1f} tok/s (kernels {kms_p:.3f} ms)")
            long_ctx.append(rec)

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"30B-A3B synthetic MoE decode, batch {B}, {ctx} cached tokens, greedy",
                   "batch": B, "context": ctx, "layers": cfg["n_layers"], "experts": cfg["n_experts"],
                   "top_k": cfg["top_k"], "parallelism": "single GPU",
                   **({"wg_per_cu": args.wg_per_cu} if args.wg_per_cu else {}),
                   **({"mfma_min_batch": args.mfma_min_batch} if args.mfma_min_batch else {}),
                   **({"mm_row_blocks": args.mm_row_blocks} if args.mm_row_blocks else {}),
                   "precision": "BF16 weights and KV; fp32 activations, entering weight products as two BF16 parts; fp32 accumulation"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": (measured_traffic(B, ctx)
                                 if not (args.wg_per_cu or args.mfma_min_batch or args.mm_row_blocks) else None),
                     "kernel": "k_persistent (one launch per step)", "bytes_per_launch": bytes_step,
                     "kernel_ms": round(kms, 4)},
        "sol": {"bytes_per_step": bytes_step, "sol_tok_s": round(sol.sol_tokens_per_s(bytes_step, B), 1),
                "pct_sol_step": round(100 * tok_s / sol.sol_tokens_per_s(bytes_step, B), 2)},
        "perop_baseline": perop,
        "schedule": sched,
        "cpu_baseline": cpu,
    }
    if sweep:
        out["batch_sweep"] = sweep
    if long_ctx:
        out["long_context"] = long_ctx
    if args.ragged:
        if not args.sweep and not args.long:
            del k_pool, v_pool
            torch.cuda.empty_cache()
        out["ragged"] = run_ragged(cfg, weights, args.ragged_steps)
    if args.prefill:
        try:
            del k_pool, v_pool
        except NameError:
            pass
        torch.cuda.empty_cache()
        out["prefill"] = [run_prefill(cfg, weights, int(T), args.prefill_prefix)
                          for T in args.prefill.split(",") if T]
    print(json.dumps(out), flush=True)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy of 1 GiB done (3 launches)")


def churn_pool_pages(cfg, B, max_pages, steps, seed_pages=(1 << 22)):
    """Pages the churning workload holds at its peak, from a dry run of the
    host scheduler (host bookkeeping only), plus a margin."""
    from persistent_megakernel_03_amd import mk, synth

    sch = mk.Scheduler(B, B, cfg["page_size"], max_pages, seed_pages, reserve_full=False)
    run = synth.ChurnRun(sch, synth.ChurnWorkload(B, cfg["vocab"]), max_len=max_pages * cfg["page_size"])
    low = seed_pages
    for _ in range(steps):
        n = sch.next()
        low = min(low, sch.stats()["free_pages"])
        sch.commit(np.zeros(n, np.int32))
        run.advance()
    sch.close()
    return seed_pages - low + 64


def run_ragged(cfg, weights, steps, warmup=8, B=32):
    """The churning batch (see the module docstring), megakernel then per-op,
    each over the same schedule from the same initial state. The host
    continuous-batching scheduler (mk.Scheduler) owns the requests, slots and
    pages; the workload's draws (synth.ChurnWorkload) say which requests end
    and which join. Throughput is tokens over wall time of the timed steps
    (host scheduling, plan rebuilds and joins included)."""
    import torch

    from persistent_megakernel_03_amd import mk, sol, synth

    biases, alpha, slope = synth.zipf_router_bias(cfg)
    w2 = dict(weights)
    for l, b in enumerate(biases):
        w2[f"layers.{l}.router_bias"] = torch.as_tensor(b).cuda()
    P = cfg["page_size"]
    max_pages = 32768 // P + (steps + warmup) // P + 2
    n_pages = churn_pool_pages(cfg, B, max_pages, steps + warmup + 2)
    log(f"ragged: Zipf bias alpha {alpha:.4f} (fitted slope {slope:.3f}); pool of {n_pages} pages")
    k_pool, v_oracle_layout = synth.make_kv_pool(cfg, n_pages, 1, "cuda")
    v_pool = v_oracle_layout.transpose(-1, -2).contiguous()
    del v_oracle_layout
    order = np.random.default_rng(synth.tensor_seed(7, "ragged.pages")).permutation(n_pages)
    res = {}
    for name, mode, shared in (("megakernel", mk.MK_MODE_MEGAKERNEL, 0),
                               ("megakernel_fixed_lists", mk.MK_MODE_MEGAKERNEL, -1),
                               ("perop", mk.MK_MODE_PEROP, 0)):
        nsteps = steps
        k, v = k_pool.clone(), v_pool.clone()
        sch = mk.Scheduler(B, B, P, max_pages, n_pages, reserve_full=False, page_order=order)
        run = synth.ChurnRun(sch, synth.ChurnWorkload(B, cfg["vocab"]), max_len=max_pages * P)
        dec = mk.Decoder(cfg, w2, k, v, max_batch=B, max_pages_per_seq=max_pages, mode=mode, time_kernels=True,
                         shared_levels=shared)
        tokens = torch.empty(B, dtype=torch.int32, device="cuda")
        logits = torch.empty(B, cfg["vocab"], dtype=torch.float32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        host_next = torch.empty(B, dtype=torch.int32, pin_memory=True)

        def one():
            n = sch.next()
            tokens[:n].copy_(torch.from_numpy(sch.tokens[:n]), non_blocking=False)
            dec.forward(sch.seq_ids[:n], sch.positions[:n], sch.block_tables[:n], tokens[:n], logits[:n])
            nxt[:n].copy_(torch.argmax(logits[:n], dim=1).to(torch.int32))
            host_next[:n].copy_(nxt[:n])
            sch.commit(host_next[:n].numpy())
            run.advance()
            return n

        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        assert dec.sync_check() == mk.MK_OK
        t0 = time.perf_counter()
        toks = 0
        for _ in range(nsteps):
            toks += one()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if dec.sync_check() != mk.MK_OK:
            raise RuntimeError("device status after the ragged run")
        n = sch.next()
        ctx = [int(x) for x in sch.positions[:n]]
        tokens[:n].copy_(torch.from_numpy(sch.tokens[:n]))
        dec.forward(sch.seq_ids[:n], sch.positions[:n], sch.block_tables[:n], tokens[:n], logits[:n])
        kms = dec.kernel_ms()
        dbg = dec.debug()
        off = dbg.route_ids - dec.workspace.data_ptr()
        n_ids = cfg["n_layers"] * B * cfg["top_k"]
        rid = dec.workspace[off:off + 4 * n_ids].view(torch.int32).view(cfg["n_layers"], B, cfg["top_k"]).cpu().numpy()
        st = sch.stats()
        dec.close()
        sch.close()
        del k, v
        nexp = distinct_experts(rid, n)
        by = sol.step_bytes(cfg, ctx, nexp, distinct_tokens=n)
        res[name] = {"value": round(toks / el, 2), "unit": "tok/s", "steps": nsteps,
                     "ms_per_step": round(1e3 * el / nsteps, 4), "kernel_ms_sample": round(kms, 4),
                     "bytes_per_step_sample": by, "distinct_experts_mean": round(float(np.mean(nexp)), 2),
                     "frac_sample": round(by / (kms * 1e-3) / 1e9 / PEAK_GBS, 4),
                     "mean_context": round(float(np.mean(ctx)), 1),
                     "scheduler": {"admitted": st["admitted"], "released": st["finished"], "steps": st["steps"]}}
        log(f"ragged {name}: {res[name]['value']:.1f} tok/s over {nsteps} steps ({res[name]['ms_per_step']:.2f} ms/step); "
            f"sample step kernel {kms:.3f} ms, {res[name]['distinct_experts_mean']} experts/layer, "
            f"{100 * res[name]['frac_sample']:.1f}% of 8 TB/s")
    res["zipf"] = {"s": 1.1, "alpha": round(alpha, 5), "fitted_slope": round(slope, 4)}
    res["workload"] = ("32 sequences, contexts log-uniform [128, 32768], 4 replaced every 8 steps (contexts [128, 2048]); "
                       "requests, slots and pages owned by the host scheduler (libmk mk_sched)")
    return res


def run_prefill(cfg, weights, T, prefix, block=64):
    """Ingest one prompt of T tokens after `prefix` cached ones, in
    multi-token steps of up to `block` rows (mk_forward_step: one launch per
    block, the rows attending causally over the cache and each other), then
    decode nothing. Reports prompt tokens per second over the whole prompt
    (wall time, blocks back to back), per-block kernel time, and the
    algorithmic bytes of the blocks (weights and routed experts once per
    block, the sequence's cache read once per block) against 8 TB/s; the
    per-op build in the same harness."""
    import torch

    from persistent_megakernel_03_amd import mk, sol, synth

    P = cfg["page_size"]
    pages = (prefix + T) // P + 2
    k_pool, v_oracle_layout = synth.make_kv_pool(cfg, pages + 1, 1, "cuda")
    v_pool = v_oracle_layout.transpose(-1, -2).contiguous()
    del v_oracle_layout
    bt = synth.make_block_tables(1, pages, pages + 1, shuffle=True)[0]
    prompt = synth.make_tokens(T, cfg["vocab"], seed=17)
    blocks = [(s0, min(T, s0 + block)) for s0 in range(0, T, block)]
    res = {"prompt_tokens": T, "prefix": prefix, "block_rows": block}
    for name, mode in (("megakernel", mk.MK_MODE_MEGAKERNEL), ("perop", mk.MK_MODE_PEROP)):
        dec = mk.Decoder(cfg, weights, k_pool.clone(), v_pool.clone(), max_batch=block, max_pages_per_seq=pages,
                         mode=mode, time_kernels=True)
        logits = torch.empty(block, cfg["vocab"], dtype=torch.float32, device="cuda")
        toks = torch.tensor(prompt, dtype=torch.int32, device="cuda")

        def one(s0, s1):
            n = s1 - s0
            dec.forward([0] * n, [prefix + s0 + i for i in range(n)], [bt] * n, toks[s0:s1], logits[:n])

        for s0, s1 in blocks:       # warm pass (plans built, code paged in)
            one(s0, s1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s0, s1 in blocks:
            one(s0, s1)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if dec.sync_check() != mk.MK_OK:
            raise RuntimeError("device status after the prefill run")
        kms, by = [], []
        for s0, s1 in blocks:
            one(s0, s1)
            kms.append(dec.kernel_ms())
            dbg = dec.debug()
            off = dbg.route_ids - dec.workspace.data_ptr()
            n_ids = cfg["n_layers"] * block * cfg["top_k"]
            rid = dec.workspace[off:off + 4 * n_ids].view(torch.int32).view(cfg["n_layers"], block,
                                                                           cfg["top_k"]).cpu().numpy()
            by.append(sol.forward_step_bytes(cfg, [(prefix + s0, s1 - s0)], distinct_experts(rid, s1 - s0),
                                             distinct_tokens=len(set(prompt[s0:s1].tolist()))))
        dec.close()
        ach = sum(by) / (sum(kms) * 1e-3) / 1e9
        res[name] = {"value": round(T / el, 1), "unit": "prompt tok/s", "ms_per_prompt": round(1e3 * el, 3),
                     "kernel_ms_per_block": [round(x, 4) for x in kms], "bytes_per_block": by,
                     "achieved_gbs": round(ach, 1), "frac": round(ach / PEAK_GBS, 4)}
        log(f"prefill {name}: {T} tokens after {prefix}: {res[name]['value']:.0f} prompt tok/s, "
            f"{sum(kms):.2f} ms of kernels in {len(blocks)} blocks, {100 * ach / PEAK_GBS:.1f}% of 8 TB/s")
    return res


def graph_or_none(cfg, weights, k_pool, v_pool, block_tables, tok0, ctx, B, pages_per_seq, steps):
    """tok/s of the per-op build as a replayed HIP graph, or None if the
    capture was refused."""
    try:
        return perop_graph(cfg, weights, k_pool, v_pool, block_tables, tok0, ctx, B, pages_per_seq, steps, 2)["value"]
    except RuntimeError as e:
        log(f"per-op graph not measured: {str(e)[:200]}")
        return None


def perop_graph(cfg, weights, k_pool, v_pool, block_tables, tok0, ctx, B, pages_per_seq, steps, warmup):
    """The per-op build's step captured once as a HIP graph (its staging copy
    and every level's launch), then replayed: each replay is the captured
    step at the same positions (the same cache slot rewritten), with the
    caller's greedy argmax between replays as in the eager loop."""
    import torch

    from persistent_megakernel_03_amd import mk

    dec = mk.Decoder(cfg, weights, k_pool, v_pool, max_batch=B, max_pages_per_seq=pages_per_seq,
                     mode=mk.MK_MODE_PEROP)
    tokens = torch.tensor(tok0, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, cfg["vocab"], dtype=torch.float32, device="cuda")
    pos = [ctx] * B
    dec.step(pos, block_tables, tokens, logits)   # builds and uploads the plan outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        dec.step(pos, block_tables, tokens, logits)
    torch.cuda.synchronize()

    def one():
        g.replay()
        tokens.copy_(torch.argmax(logits, dim=1).to(torch.int32))

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    if dec.sync_check() != mk.MK_OK:
        raise RuntimeError("device status after the per-op graph replays")
    del g
    dec.close()
    return {"value": round(B * steps / el, 2), "ms_per_step": round(1e3 * el / steps, 4), "steps": steps}


OP_NAMES = ["embed", "qkv", "attention", "merge", "o_proj", "router", "routing", "gate_up", "down", "expert_sum",
            "lm_head", "claim", "final_norm"]
OP_CLAIM = 11


def schedule_stats(cfg, weights, k_pool, v_pool, block_tables, tok0, ctx, B, pages_per_seq, warmup=3):
    """One traced megakernel step after a few untraced ones (the in-kernel
    trace: per task its start, the end of its last counter wait and its end,
    100 MHz wall clock). Reports, over the step's span and all workgroups,
    the fraction of workgroup time spent before a task's last counter wait
    ended (waiting, plus the weight loads issued before it), the fraction
    after it (compute, stores, signal), the fraction of compute units with a
    workgroup past its wait (workgroups w and w + n_wg/2 share a unit), and
    per tile kind the median over the middle layers of the time from the
    previous level's last tile to the level's last tile."""
    import torch

    from persistent_megakernel_03_amd import mk

    dec = mk.Decoder(cfg, weights, k_pool, v_pool, max_batch=B, max_pages_per_seq=pages_per_seq, trace=True)
    tokens = torch.tensor(tok0, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, cfg["vocab"], dtype=torch.float32, device="cuda")
    pos = [ctx] * B
    for _ in range(warmup + 1):
        dec.step(pos, block_tables, tokens, logits)
        tokens.copy_(torch.argmax(logits, dim=1).to(torch.int32))
        pos = [p + 1 for p in pos]
    torch.cuda.synchronize()
    if dec.sync_check() != mk.MK_OK:
        raise RuntimeError("device status after the traced step")
    tr = mk.mk_get_trace(dec.handle)
    tasks = mk.mk_get_plan(dec.handle)
    dec.close()
    return schedule_from_trace(tr, tasks, cfg["n_layers"])


def schedule_from_trace(tr, tasks, L):
    """The schedule figures of one traced step from its trace records
    ({task | workgroup << 32, start, end of last wait, 4 marks, end}, 100 MHz
    ticks) and the task table they index (see schedule_stats). Records of
    claim tasks (which span the tiles they drain) are left out."""
    tr = tr[tasks[(tr[:, 0] & 0xffffffff).astype(np.int64), 0] != OP_CLAIM]
    idx = (tr[:, 0] & 0xffffffff).astype(np.int64)
    wg = (tr[:, 0] >> 32).astype(np.int64)
    t0 = int(tr[:, 1].min())
    st = (tr[:, 1].astype(np.int64) - t0) / 100.0
    wt = (tr[:, 2].astype(np.int64) - t0) / 100.0
    en = (tr[:, 7].astype(np.int64) - t0) / 100.0
    span = float(en.max())
    n_wg = int(wg.max()) + 1
    wait = float(np.sum(wt - st)) / (n_wg * span)
    busy = float(np.sum(en - wt)) / (n_wg * span)
    # compute units with a workgroup past its wait: union of the two
    # workgroups' busy intervals per unit
    half = n_wg // 2
    cu = wg % half if n_wg % 2 == 0 else wg
    busy_cu = 0.0
    for c in np.unique(cu):
        m = np.where(cu == c)[0]
        iv = sorted(zip(wt[m], en[m]))
        cur0, cur1 = iv[0]
        for a, b in iv[1:]:
            if a > cur1:
                busy_cu += cur1 - cur0
                cur0, cur1 = a, b
            else:
                cur1 = max(cur1, b)
        busy_cu += cur1 - cur0
    n_cu = len(np.unique(cu))
    op, layer, level = tasks[idx, 0], tasks[idx, 1], tasks[idx, 11]
    ends = {}
    for lv in np.unique(level):
        ends[int(lv)] = float(en[level == lv].max())
    order = sorted(ends)
    per = {}
    for i, lv in enumerate(order[1:], 1):
        m = level == lv
        o, l = int(op[m][0]), int(layer[m][0])
        if L // 6 <= l < L - L // 6 and o not in (0, 10, 12):
            per.setdefault(OP_NAMES[o], []).append(ends[lv] - ends[order[i - 1]])
    return {"traced_step_us": round(span, 1), "wait_stall_frac": round(wait, 4), "busy_wg_frac": round(busy, 4),
            "busy_cu_frac": round(float(busy_cu) / (n_cu * span), 4), "n_wg": n_wg,
            "level_us": {k: round(float(np.median(v)), 2) for k, v in per.items()},
            "kind": "one traced step after the timed steps; layers %d-%d for level_us" % (L // 6, L - L // 6 - 1)}


def cpu_baseline(cfg, weights, k_pool, v_pool, block_tables, tok0, ctx, B, n_steps):
    """The CPU oracle, as it stands, on the first steps of the same workload:
    one untimed pass pulls and decodes the weights it touches, then
    n_steps greedy steps are timed (compute only)."""
    import torch

    from oracle import DenseModel, PagedKV, decode_step
    from persistent_megakernel_03_amd import synth

    log("cpu oracle: pulling weights and KV to the host")
    cache = {}

    def src(name):
        if name not in weights:
            return None
        if name not in cache:
            cache[name] = synth.bits(weights[name])
        return cache[name]

    def esrc(layer, kind, e):
        return synth.bits(weights[f"layers.{layer}.{kind}"][e])

    model = DenseModel(cfg, src, esrc, np.float32)
    kv = PagedKV(synth.bits(k_pool), synth.bits(v_pool.transpose(-1, -2)), cfg["page_size"])
    toks = list(int(t) for t in tok0)
    pos = [ctx] * B
    # untimed warm pass: decodes dense weights and the first step's experts
    kv_k, kv_v = kv.k.copy(), kv.v.copy()
    decode_step(model, PagedKV(kv_k, kv_v, cfg["page_size"]), pos, block_tables, toks)
    del kv_k, kv_v
    cores_visible = len(os.sched_getaffinity(0))
    threads, blas_threads, blas_lib = cores_visible, None, None
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            blas_threads = max(int(i.get("num_threads", 0)) for i in blas)
            blas_lib = blas[0].get("internal_api")
            threads = blas_threads
    except Exception:
        pass
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    t0 = time.perf_counter()
    for _ in range(n_steps):
        lg, _, _ = decode_step(model, kv, pos, block_tables, toks)
        toks = [int(np.argmax(lg[b])) for b in range(B)]
        pos = [p + 1 for p in pos]
    el = time.perf_counter() - t0
    log(f"cpu oracle: {B * n_steps / el:.3f} tok/s over {n_steps} steps ({el:.1f}s, {threads} cores)")
    return {"value": round(B * n_steps / el, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_steps} greedy steps of the same workload from its first position, after one untimed "
                      f"pass that decodes the touched weights; numpy float32",
            "cpu_model": cpu_model, "cores_visible": cores_visible, "blas_threads": blas_threads,
            "blas": blas_lib}


if __name__ == "__main__":
    main()
