#!/usr/bin/env python3
"""Benchmark one DSA layer decode step (indexer -> top-k -> sparse MLA) on one
MI355X, on seeded synthetic caches shaped like the serving workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  `value` is the algorithmic HBM throughput of the whole
step (GB/s: bytes the method must move / the median step time, inputs resident
in HBM); µs per step, query tokens/s and the per-stage split ride along.

Timing protocol: W untimed warm-up steps, then K timed steps, each preceded by
a 1 GiB read-modify-write scrub on the same stream (outside the step's events)
so that no step finds the previous step's data in L2 or the 256 MB MALL; every
step is bracketed by HIP events on the launch stream, and the median, p10 and
p90 over the K steps are reported (the back-to-back mean without scrubs rides
along as `warm_us`).  Besides the headline workload, the other reference
workloads are timed the same way under `workloads`.  `roofline` covers the
headline's dominant kernel; `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the headline workload, with all host cores and with one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA layer decode µs/step & achieved HBM GB/s (indexer+top-k+MLA), 64K–1M ctx"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="tp8_spec_decode_64k")
    ap.add_argument("--others", type=int, default=1,
                    help="also time the other reference workloads under `workloads` (0 = skip)")
    ap.add_argument("--scrub-mib", type=int, default=1024, help="cache scrub before every timed step (0 = none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target length of the oracle sample (0 disables the CPU baseline)")
    ap.add_argument("--shards", type=int, default=8,
                    help="context shards of the sharded top-k merge measurement (0 or 1 = skip)")
    ap.add_argument("--msa", type=int, default=1, help="also time the MSA block-sparse variant (0 = skip)")
    ap.add_argument("--prefix", type=int, default=1,
                    help="also time the shared-prefix indexer on a 64-request FP4 batch (0 = skip)")
    ap.add_argument("--prefix-group", type=int, default=64, help="requests per shared-prefix group")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times), to scale "
                         "the HBM byte counters of a profiler against a known size")
    return ap.parse_args()


def copy_calibration(nbytes: int):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "repeats": 5}))


def measured_traffic(workload: str, stage: str):
    """HBM bytes (read + written) per launch of `stage`'s kernels on `workload`,
    from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs summarised in
    profiles/traffic.json (already scaled by the copy calibration).  None when
    no such run exists or the library sources changed since it was taken."""
    from sparse_attention_03_amd import build as B
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256_16") != B.source_digest():
        return None
    st = rec.get("workloads", {}).get(workload, {}).get(stage)
    if not st:
        return None
    return int(st["fetch_bytes"] + st["write_bytes"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_run(inp, wl, seconds, bytes_of_rows):
    from oracle import dsa as O
    rts = wl.req_token_start.cpu().tolist()
    done_rows, elapsed, reqs = [], 0.0, 0
    for r in range(wl.R):
        rows = list(range(rts[r], rts[r + 1]))
        t0 = time.perf_counter()
        O.layer(inp, k=wl.spec.k, tokens=rows, want_scores=False)
        elapsed += time.perf_counter() - t0
        done_rows += rows
        reqs += 1
        if elapsed >= seconds:
            break
    return reqs, done_rows, elapsed, bytes_of_rows(reqs, done_rows) / elapsed / 1e9


def cpu_baseline(wl, seconds, bytes_of_rows):
    """Time the oracle, request by request, until `seconds` have elapsed: once
    with the BLAS pool at every host core, once on a single thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from tests.helpers import oracle_inputs
    inp = oracle_inputs(wl)
    ncpu = os.cpu_count() or 1
    with threadpool_limits(limits=ncpu):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        reqs, rows, el, gbs = _oracle_run(inp, wl, seconds, bytes_of_rows)
    with threadpool_limits(limits=1):
        reqs1, rows1, el1, gbs1 = _oracle_run(inp, wl, seconds, bytes_of_rows)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": ncpu,
            "one_thread": {"value": round(gbs1, 4), "cores": 1, "requests": reqs1, "rows": len(rows1),
                           "seconds": round(el1, 2)},
            "sample": f"{reqs} of {wl.R} requests ({len(rows)} query rows), fp64 NumPy with {threads} BLAS "
                      f"threads, {el:.2f} s; same algorithmic-byte accounting as value"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the DSA layer path here runs on a single MI355X "
              "(no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_03_amd as dsa
    import synth
    from sparse_attention_03_amd import bytemodel as BM

    dsa.load()
    dev = torch.device("cuda:0")
    E = torch.cuda.Event
    K = args.steps
    scrub = torch.zeros(args.scrub_mib * (1 << 20) // 4, dtype=torch.float32, device=dev) if args.scrub_mib else None

    def build(spec):
        t0 = time.time()
        wl = synth.make_workload(spec, device=dev)
        torch.cuda.synchronize()
        print(f"[bench] workload {spec.name} generated in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
        step = dsa.make_step(key_pool=wl.key_pool, lat_pool=wl.lat_pool, page_size=wl.P, key_fmt=spec.key_fmt,
                             lat_fmt=spec.lat_fmt, req_row_start=wl.req_token_start, tok_req=wl.tok_req,
                             tok_vis=wl.tok_vis, block_table=wl.block_table, q_idx=wl.q_idx, w=wl.w,
                             q_mla=wl.q_mla, k=spec.k, sm_scale=spec.sm_scale, q_idx_scale=wl.q_idx_scale,
                             prefill=spec.q_per_req > 64, max_vis=spec.N, max_rows_per_req=spec.q_per_req)
        return wl, step

    def time_step(step, n=K, warmup=args.warmup):
        """n scrubbed steps with per-stage events; then n back-to-back steps."""
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev = [[E(enable_timing=True) for _ in range(4)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            if scrub is not None:
                scrub.add_(1.0)  # reads and writes 1 GiB: evicts L2 and the MALL
            ev[i][0].record()
            step.indexer()
            ev[i][1].record()
            step.topk()
            ev[i][2].record()
            step.mla()
            ev[i][3].record()
        torch.cuda.synchronize()
        per = {nm: [ev[i][a].elapsed_time(ev[i][b]) for i in range(n)]
               for nm, a, b in (("indexer", 0, 1), ("topk", 1, 2), ("mla", 2, 3), ("step", 0, 3))}
        w0, w1 = E(enable_timing=True), E(enable_timing=True)
        w0.record()
        for _ in range(n):
            step()
        w1.record()
        torch.cuda.synchronize()
        return per, w0.elapsed_time(w1) / n

    def pct(xs, q):
        ys = sorted(xs)
        return ys[min(len(ys) - 1, max(0, int(round(q * (len(ys) - 1)))))]

    def summarise(spec, wl, per, warm_ms):
        vis = wl.tok_vis.cpu().tolist()
        rts = wl.req_token_start.cpu().tolist()
        req_vis = [max(vis[rts[r]:rts[r + 1]]) for r in range(wl.R)]
        page = 0 if spec.page == 0 else wl.P
        B = BM.step_bytes(req_vis_max=req_vis, row_vis=vis, k=spec.k, H=spec.H, key_fmt=spec.key_fmt,
                          lat_fmt=spec.lat_fmt, q_fmt=spec.q_fmt, page=page)
        F = BM.step_flops(row_vis=vis, k=spec.k, H=spec.H)
        med = pct(per["step"], 0.5)
        stages = {n: pct(per[n], 0.5) for n in ("indexer", "topk", "mla")}
        rec = {"us_median": round(med * 1e3, 2), "us_p10": round(pct(per["step"], 0.1) * 1e3, 2),
               "us_p90": round(pct(per["step"], 0.9) * 1e3, 2), "warm_us": round(warm_ms * 1e3, 2),
               "tokens_per_s": round(wl.T / (med * 1e-3), 1), "alg_bytes": B["total"],
               "alg_GB_per_s": round(B["total"] / (med * 1e-3) / 1e9, 2),
               "roofline_frac": round(B["total"] / (PEAK_HBM_GBS * 1e9) / (med * 1e-3), 4),
               "literal_formula_roofline_us": round(BM.literal_formula_bytes(wl.T, spec.N, spec.k) / 8e12 * 1e6, 2),
               "stages_us_median": {n: round(v * 1e3, 2) for n, v in stages.items()},
               "indexer_flop": F["indexer"], "mla_flop": F["mla"]}
        if spec.q_per_req > 64:
            # the prefill chunk is bound by the FP8 matrix instructions of its indexer
            rec["indexer_fp8_mfma_frac"] = round(F["indexer"] / (stages["indexer"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)
            rec["mla_bf16_mfma_frac"] = round(F["mla"] / (stages["mla"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        return rec, B, F, vis, req_vis, page, stages, med

    spec = synth.CONFIGS[args.workload]
    wl, step = build(spec)
    prefill = spec.q_per_req > 64
    per, warm_ms = time_step(step)
    head, B, F, vis, req_vis, page, st_med, ms_step = summarise(spec, wl, per, warm_ms)
    st = st_med
    value = B["total"] / (ms_step * 1e-3) / 1e9
    # with fewer than 100 timed steps, the same statistics over 100 more
    # scrubbed steps (after the timed region; not part of `value`)
    head100 = None
    if K < 100:
        per100, warm100 = time_step(step, n=100, warmup=0)
        head100 = summarise(spec, wl, per100, warm100)[0]

    # dominant kernel and its roofline (median launch durations over the K
    # scrubbed steps)
    dom = max(st, key=st.get)
    t_dom = st[dom] * 1e-3
    if dom == "indexer":
        peak_f = PEAK_FP8_TFLOPS if spec.q_fmt == "fp8" else PEAK_BF16_TFLOPS
        t_mem, t_cmp = B["indexer"] / (PEAK_HBM_GBS * 1e9), F["indexer"] / (peak_f * 1e12)
        if t_cmp > t_mem:
            roof = {"bound": "mfma", "achieved": F["indexer"] / t_dom / 1e12, "peak": peak_f, "unit": "TFLOP/s",
                    "traffic": None}
        else:
            roof = {"bound": "hbm", "achieved": B["indexer"] / t_dom / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "traffic": None}
    elif dom == "mla":
        t_mem, t_cmp = B["mla"] / (PEAK_HBM_GBS * 1e9), F["mla"] / (PEAK_BF16_TFLOPS * 1e12)
        if t_cmp > t_mem:
            roof = {"bound": "mfma", "achieved": F["mla"] / t_dom / 1e12, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "traffic": None}
        else:
            roof = {"bound": "hbm", "achieved": B["mla"] / t_dom / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "traffic": None}
    else:
        nbytes = sum(vis) * 4
        roof = {"bound": "hbm", "achieved": nbytes / t_dom / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "traffic": None}
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(spec.name, dom)
    roof["achieved"] = round(roof["achieved"], 2)
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["launch_us_median"] = round(t_dom * 1e6, 2)

    # The step's front end, timed apart from the step (not part of the metric):
    # every query row's own token is the newest visible one of its request, so
    # one step quantises T index queries and inserts T keys and latents.
    fe = None
    if not prefill:
        g = torch.Generator(device=dev)
        g.manual_seed(4242)
        key_new = torch.randn(wl.T, 128, generator=g, device=dev).to(torch.bfloat16)
        lat_new = torch.randn(wl.T, 576, generator=g, device=dev).to(torch.bfloat16)
        pos_new = (wl.tok_vis - 1).to(torch.int32).contiguous()
        q_fmt_fe = "fp8" if spec.key_fmt == "fp8" else "mxfp4"

        def front_end():
            dsa.quantize_q(wl.q_idx if wl.q_idx.dtype == torch.bfloat16 else key_new.new_zeros(wl.T, 32, 128),
                           wl.w, q_fmt_fe, fold=(q_fmt_fe == "fp8"))
            dsa.cache_insert(wl.tok_req, pos_new, wl.R, wl.block_table, wl.P, key_vals=key_new,
                             key_pool=wl.key_pool, key_fmt=spec.key_fmt, lat_vals=lat_new, lat_pool=wl.lat_pool,
                             lat_fmt=spec.lat_fmt)

        for _ in range(3):
            front_end()
        torch.cuda.synchronize()
        # Two small launches take less GPU time than the host needs to queue
        # them, so the GPU is first given a backlog of whole steps (not timed);
        # the front ends queued behind it then run back to back.
        n_busy = max(1, int(1.5 * K * 40e-3 / ms_step) + 1)
        f0, f1 = E(enable_timing=True), E(enable_timing=True)
        for _ in range(n_busy):
            step()
        h0 = time.perf_counter()
        f0.record()
        for _ in range(K):
            front_end()
        f1.record()
        host_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        fe_ms = f0.elapsed_time(f1) / K
        backlog_ok = host_ms < n_busy * ms_step
        key_b = BM.KEY_B[spec.key_fmt]
        lat_b = {"bf16": 1152, "fp8": 580, "nvfp4": 352}[spec.lat_fmt]
        q_out = 32 * (128 + 4 + 4) if q_fmt_fe == "fp8" else 32 * (64 + 4)
        fe_bytes = wl.T * (32 * 128 * 2 + 32 * 4 + q_out + 128 * 2 + 576 * 2 + 8 + key_b + lat_b)
        fe = {"us": round(fe_ms * 1e3, 2), "q_fmt": q_fmt_fe, "tokens": wl.T, "alg_bytes": fe_bytes,
              "GB_per_s": round(fe_bytes / (fe_ms * 1e-3) / 1e9, 2), "gpu_bound_timing": backlog_ok}

    # The exact sharded top-k merge (context shards emulated on this device),
    # timed apart from the step on the step's own scores: each shard's share
    # of every row in the interleaved layout, eight shards.
    shard = None
    if not prefill and args.shards > 1:
        W = args.shards
        ld_l = -(-(-(-spec.N // W)) // 4) * 4
        full = torch.zeros(wl.T, ld_l * W, dtype=torch.float32, device=dev)
        n_cols = min(step.scores.shape[1], ld_l * W)
        full[:, :n_cols] = step.scores[:, :n_cols]
        local = full.view(wl.T, ld_l, W).permute(2, 0, 1).contiguous()
        del full
        st_op = dsa.ShardedTopk(local, wl.tok_vis, spec.N, spec.k)
        torch.cuda.synchronize()
        for _ in range(3):
            st_op()
        torch.cuda.synchronize()
        # (queued behind a backlog of steps, as the front end: a call's seven or
        # more launches can take the host longer than the GPU)
        n_busy = max(1, int(2.0 * K * 150e-3 / ms_step) + 1)
        s0, s1 = E(enable_timing=True), E(enable_timing=True)
        for _ in range(n_busy):
            step()
        h0 = time.perf_counter()
        s0.record()
        for _ in range(K):
            st_op()
        s1.record()
        sh_host_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        sh_ms = s0.elapsed_time(s1) / K
        same = bool(torch.equal(st_op.idx, step.idx))
        resent = st_op.resend.cpu().numpy()
        cand = min(spec.k, -(-3 * spec.k // (2 * W)))
        n_loc = [[max(0, -(-(v - r) // W)) for r in range(W)] for v in vis]
        sent = sum(min(cand, n) for row in n_loc for n in row)
        sent += sum(min(spec.k, n_loc[t][r]) for t in range(wl.T) for r in range(W) if resent[t, r])
        generic = sum(min(spec.k, n) for row in n_loc for n in row)
        shard = {"shards": W, "cand": cand, "us": round(sh_ms * 1e3, 2), "unsharded_topk_us": round(st["topk"] * 1e3, 2),
                 "equals_unsharded": same, "rows_resent": int((resent.sum(axis=1) > 0).sum()),
                 "exchange_bytes": 8 * sent, "generic_exchange_bytes": 8 * generic,
                 "gpu_bound_timing": sh_host_ms < n_busy * ms_step}
        del local, st_op

    # The MSA block-sparse variant on its own workload (apart from the metric):
    # 128-token blocks, FP8 index keys of one shared head, FP8 K/V of 4 heads.
    msa = None
    if args.msa and not prefill:
        import synth.msa as SM
        mspec = SM.MSA_CONFIGS["msa_decode_128k"]
        minp = SM.make_inputs(mspec, device=dev)
        mop = dsa.MsaDecode(req_row_start=minp["req_row_start"], tok_req=minp["tok_req"], tok_vis=minp["tok_vis"],
                            block_table=minp["block_table"], idx_pool=minp["idx_pool"], kv_pool=minp["kv_pool"],
                            q_idx=minp["q_idx"], q=minp["q"], max_vis=mspec.N, max_rows_per_req=mspec.rows,
                            top_blocks=mspec.top_blocks, k_scale=mspec.k_scale, v_scale=mspec.v_scale)
        for _ in range(3):
            mop()
        torch.cuda.synchronize()
        m0, m1 = E(enable_timing=True), E(enable_timing=True)
        m0.record()
        for _ in range(K):
            mop()
        m1.record()
        torch.cuda.synchronize()
        msa_ms = m0.elapsed_time(m1) / K
        mvis = minp["tok_vis"].cpu().tolist()
        T_m = len(mvis)
        sel = mop.sel.cpu()
        kv_tok = 0
        for t in range(T_m):
            for g_ in range(mspec.hkv):
                for b_ in sel[t, g_].tolist():
                    if b_ >= 0:
                        kv_tok += min(128, mvis[t] - 128 * b_)
        mbytes = (mspec.R * 128 * mspec.N + T_m * mspec.hkv * 256 + T_m * mspec.hq * 256 + kv_tok * 256
                  + T_m * mspec.hq * (512 + 4) + mspec.R * (-(-mspec.N // 128)) * 4)
        msa = {"workload": mspec.name, "requests": mspec.R, "context": mspec.N, "kv_heads": mspec.hkv,
               "q_heads": mspec.hq, "top_blocks": mspec.top_blocks, "us": round(msa_ms * 1e3, 2),
               "alg_bytes": mbytes, "GB_per_s": round(mbytes / (msa_ms * 1e-3) / 1e9, 1),
               "roofline_frac": round(mbytes / (msa_ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)}
        del minp, mop

    # Shared-prefix indexer on a high-concurrency FP4 batch (apart from the
    # metric): 64 single-row requests at 256K whose first 192K tokens are one
    # shared prefix (the same physical pages), plain call against the call
    # that streams the shared pages once for the whole group.
    pre = None
    if args.prefix and not prefill:
        pspec = synth.CONFIGS["fp4_decode_256k"]
        pwl = synth.make_workload(pspec, device=dev)
        L = 196608
        gsz = args.prefix_group  # requests per group (one request = one row here)
        bt = pwl.block_table.clone()
        for a0 in range(0, pwl.R, gsz):
            bt[a0:a0 + gsz, :L // pwl.P] = bt[a0, :L // pwl.P].clone()
        pwl.block_table = bt.contiguous()
        pst = dsa.make_step(key_pool=pwl.key_pool, lat_pool=pwl.lat_pool, page_size=pwl.P, key_fmt=pspec.key_fmt,
                            lat_fmt=pspec.lat_fmt, req_row_start=pwl.req_token_start, tok_req=pwl.tok_req,
                            tok_vis=pwl.tok_vis, block_table=pwl.block_table, q_idx=pwl.q_idx, w=pwl.w,
                            q_mla=pwl.q_mla, k=pspec.k, sm_scale=pspec.sm_scale, q_idx_scale=pwl.q_idx_scale,
                            max_vis=pspec.N, max_rows_per_req=pspec.q_per_req)
        starts = list(range(0, pwl.R, gsz))
        grs = torch.tensor(starts + [pwl.T], dtype=torch.int32, device=dev)
        gfr = torch.tensor(starts, dtype=torch.int32, device=dev)
        pargs, pws = dsa.indexer_prefix_args(dsa.IndexerArgs.from_buffer_copy(pst.iargs), grs, gfr, L, gsz, dev)

        def timed(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            a0, a1 = E(enable_timing=True), E(enable_timing=True)
            a0.record()
            for _ in range(K):
                fn()
            a1.record()
            torch.cuda.synchronize()
            return a0.elapsed_time(a1) / K

        plain_ms = timed(pst.indexer)
        ref = pst.scores.clone()
        pre_ms = timed(lambda: dsa.dsa_indexer_scores_prefix(pargs))
        pvis = pwl.tok_vis.cpu().tolist()
        diff = max(float((pst.scores[t, :v] - ref[t, :v]).abs().max() / ref[t, :v].abs().max())
                   for t, v in enumerate(pvis))
        kb = 68
        plain_bytes = sum(pvis) * kb
        # the shared pages are streamed once per pass of at most 12 rows
        n_pass = sum(-(-min(gsz, pwl.R - a0) // 12) for a0 in starts)
        shared_bytes = n_pass * L * kb + sum(v - L for v in pvis) * kb
        pre = {"workload": f"fp4_decode_256k, groups of {gsz} requests sharing a 196,608-token prefix",
               "plain_us": round(plain_ms * 1e3, 2),
               "prefix_us": round(pre_ms * 1e3, 2), "plain_key_bytes": plain_bytes, "prefix_key_bytes": shared_bytes,
               "max_rel_diff": diff}
        del pwl, pst, ref

    cpu = None
    if args.cpu_seconds > 0:
        def bytes_of_rows(nreq, rows):
            b = BM.step_bytes(req_vis_max=req_vis[:nreq], row_vis=[vis[t] for t in rows], k=spec.k, H=spec.H,
                              key_fmt=spec.key_fmt, lat_fmt=spec.lat_fmt, q_fmt=spec.q_fmt, page=page)
            return b["total"]
        cpu = cpu_baseline(wl, args.cpu_seconds, bytes_of_rows)
    del step, wl
    torch.cuda.empty_cache()

    # the other reference workloads, timed by the same protocol
    others = {}
    if args.others:
        extra = dict(synth.CONFIGS)
        # the FP4 workload with MXFP4 index queries: the indexer on the FP4
        # matrix instruction (no dequantisation), everything else as above
        extra["fp4_decode_256k_mxfp4_q"] = synth.CONFIGS["fp4_decode_256k"].replace(
            name="fp4_decode_256k_mxfp4_q", q_fmt="mxfp4")
        # the 64K speculative workload with FP8 index queries (the front end's
        # FP8 output, head weight and scale folded): the multi-row indexer on
        # the FP8 matrix instruction over raw keys
        extra["tp8_spec_decode_64k_fp8_q"] = synth.CONFIGS["tp8_spec_decode_64k"].replace(
            name="tp8_spec_decode_64k_fp8_q", q_fmt="fp8")
        for name, ospec in extra.items():
            if name == spec.name:
                continue
            owl, ostep = build(ospec)
            oper, owarm = time_step(ostep, n=max(K, 100))
            orec = summarise(ospec, owl, oper, owarm)[0]
            orec["config"] = {"requests": ospec.R, "rows_per_request": ospec.q_per_req, "context": ospec.N,
                              "key_fmt": ospec.key_fmt, "latent_fmt": ospec.lat_fmt, "index_q_fmt": ospec.q_fmt,
                              "mla_heads": ospec.H, "topk": ospec.k}
            others[name] = orec
            print(f"[bench] {name}: {orec['us_median']} us median", file=sys.stderr, flush=True)
            del owl, ostep
            torch.cuda.empty_cache()

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "requests": spec.R, "rows_per_request": spec.q_per_req,
                   "context": spec.N, "page": spec.page, "key_fmt": spec.key_fmt, "latent_fmt": spec.lat_fmt,
                   "index_q_fmt": spec.q_fmt, "mla_heads": spec.H, "topk": spec.k},
        "timing": {"statistic": "median of K steps, each after a cache scrub", "scrub_mib": args.scrub_mib,
                   "us_p10": head["us_p10"], "us_p90": head["us_p90"], "warm_us": head["warm_us"],
                   "steps_100": None if head100 is None else
                   {k2: head100[k2] for k2 in ("us_median", "us_p10", "us_p90", "warm_us", "stages_us_median")}},
        "us_per_step": head["us_median"],
        "tokens_per_s": head["tokens_per_s"],
        "alg_bytes": B["total"],
        "step_roofline_frac": head["roofline_frac"],
        "literal_formula_roofline_us": head["literal_formula_roofline_us"],
        "stages_us": head["stages_us_median"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": others,
        "front_end": fe,
        "sharded_topk": shard,
        "msa": msa,
        "shared_prefix_indexer": pre,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
