"""GPU parity: every libdsa entry point against the fp64 oracle on the same
seeded inputs.

Tolerances:
  * indexer scores (tests.helpers.assert_scores_close): |gpu - oracle| <=
    1e-5 * max_s |oracle score| per row for BF16 queries (bf16 products are
    exact, fp32 accumulation of 4096 terms); for FP8 / MXFP4 queries the
    per-element worst-case bound of an fp32 sum of the score's 160 terms in
    any order (160 * 2^-23 * sum of |terms|), since the low-precision matrix
    instructions do not document their internal summation; -inf exactly where
    the oracle has it (tokens on absent pages);
  * top-k: bit-exact index sets when the scores are the same fp32 values or a
    gap is planted at rank k; otherwise every selected score >= tau - 1e-3|tau|;
  * attention: max-abs-err <= 1e-2 * max|oracle o| (BF16/FP8 latents), 3e-2 (FP4);
    lse within 1e-3 absolute.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import synth
from oracle import dsa as O
from tests.helpers import assert_scores_close, gpu_step, oracle_inputs

pytestmark = pytest.mark.gpu


def _wl(spec, gpu):
    return synth.make_workload(spec, device=gpu)


def _check_scores(step, wl, inp, tokens=None):
    sc = step.scores.cpu().numpy()
    vis = wl.tok_vis.cpu().numpy()
    res = O.layer(inp, k=wl.spec.k, tokens=tokens)
    keys = {}
    for t, ref in zip(res["t"], res["scores"]):
        kk = None
        if inp["q_fmt"] != "bf16":
            r = int(wl.tok_req[t])
            if r not in keys:
                keys.clear()
                keys[r] = O.request_keys(inp["key_pool"], inp["key_fmt"], inp["P"], inp["block_table"], r,
                                         int(vis[inp["req_token_start"][r]:inp["req_token_start"][r + 1]].max()))
            kk = keys[r]
        assert_scores_close(sc[t, : vis[t]], ref, inp, t, keys=kk)
    return res


def _check_topk_sets(step, wl, res, exact):
    idx = step.idx.cpu().numpy()
    rows = step.rows.cpu().numpy()
    cnt = step.count.cpu().numpy()
    k = wl.spec.k
    for j, t in enumerate(res["t"]):
        K = len(res["idx"][j])
        assert cnt[t] == K
        got = idx[t, :K]
        assert np.all(idx[t, K:] == -1)
        assert np.all(np.diff(got) > 0), "indices must be ascending and distinct"
        if exact:
            assert np.array_equal(got, res["idx"][j]), f"row {t}: top-k set differs"
            assert np.array_equal(rows[t, :K], res["rows"][j])
        else:
            sc = res["scores"][j]
            tau = res["tau"][j]
            assert np.all(got < len(sc))
            assert np.all(sc[got] >= tau - 1e-3 * abs(tau)), f"row {t}: selected score below tau"
        assert np.all(rows[t, K:] == -1)


def _check_attention(out, lse, ref_o, ref_lse, fp4=False):
    tol = (3e-2 if fp4 else 1e-2) * np.abs(ref_o).max()
    err = np.abs(out - ref_o).max()
    assert err <= tol, f"attention err {err} > {tol}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - ref_lse[fin]).max() <= 1e-3


# ----------------------------------------------------------------- end to end
CASES = {
    # tiny decode: non-paged BF16 latents, one row (the 8K reference shape)
    "tiny_8k_bf16": synth.CONFIGS["tiny_decode_8k"],
    # speculative rows sharing keys, paged FP8, ragged last page, 12 heads
    "spec_fp8_paged": synth.CONFIGS["tp8_spec_decode_64k"].replace(R=3, N=12345, seed=5),
    # FP4 formats
    "fp4_paged": synth.CONFIGS["fp4_decode_256k"].replace(R=3, N=9000, seed=6),
    # NVFP4 index keys: one row per request (streaming kernel) and speculative rows
    "nvfp4_keys_row": synth.CONFIGS["fp4_decode_256k"].replace(R=3, N=9000, key_fmt="nvfp4", seed=8),
    "nvfp4_keys_spec": synth.CONFIGS["tp8_spec_decode_64k"].replace(R=3, N=12345, key_fmt="nvfp4", seed=9),
    # MXFP4 index queries against MXFP4 keys on the FP4 matrix instruction:
    # one row per request, and three rows per request (scored in turn)
    "fp4_native_row": synth.CONFIGS["fp4_decode_256k"].replace(R=3, N=9000, q_fmt="mxfp4", seed=12),
    "fp4_native_spec": synth.CONFIGS["fp4_decode_256k"].replace(R=3, q_per_req=3, N=7001, q_fmt="mxfp4",
                                                                 seed=13),
    # FP8 index queries on the FP8 instruction over raw keys: speculative rows
    # and one row per request (the multi-row decode kernel)
    "fp8q_spec": synth.CONFIGS["tp8_spec_decode_64k"].replace(R=3, N=12345, q_fmt="fp8", seed=14),
    "fp8q_row": synth.CONFIGS["tp8_spec_decode_64k"].replace(R=4, q_per_req=1, N=9000, q_fmt="fp8", seed=15),
    # eight rows per request: two row passes (6 + 2) of the multi-row FP8 kernel
    "fp8q_8rows": synth.CONFIGS["tp8_spec_decode_64k"].replace(R=2, q_per_req=8, N=7000, q_fmt="fp8", seed=16),
    # 96 heads (two head groups), planted gap
    "h96_gap": synth.CONFIGS["long_decode_1m"].replace(R=2, N=20000, seed=7),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_end_to_end(name, gpu):
    spec = CASES[name]
    print(f"[gpu] case {name}: {spec}", flush=True)
    wl = _wl(spec, gpu)
    inp = oracle_inputs(wl)
    step = gpu_step(wl)
    out, lse = step()
    torch.cuda.synchronize()
    res = _check_scores(step, wl, inp)
    _check_topk_sets(step, wl, res, exact=spec.plant_gap)
    # attention end to end on every row whose selected set equals the
    # oracle's (all rows when a gap is planted); near-tie rows are covered by
    # the top-k tolerance check above and by the attention-alone tests
    idx = step.idx.cpu().numpy()
    same = [j for j, t in enumerate(res["t"]) if np.array_equal(idx[t, : len(res["idx"][j])], res["idx"][j])]
    if spec.plant_gap:
        assert len(same) == len(res["t"])
    assert len(same) >= len(res["t"]) // 2, "too many rows with a different top-k set"
    ts = [res["t"][j] for j in same]
    _check_attention(out.cpu().numpy()[ts], lse.cpu().numpy()[ts], np.stack([res["o"][j] for j in same]),
                     np.stack([res["lse"][j] for j in same]), fp4=spec.lat_fmt == "nvfp4")


@pytest.mark.parametrize("name", ["tiny_8k_bf16", "spec_fp8_paged", "fp4_paged", "nvfp4_keys_row",
                                  "nvfp4_keys_spec", "fp4_native_row", "fp4_native_spec", "fp8q_spec"])
def test_layer_end_to_end_planted(name, gpu):
    spec = CASES[name].replace(plant_gap=True, seed=CASES[name].seed + 100)
    print(f"[gpu] planted case {name}", flush=True)
    wl = _wl(spec, gpu)
    inp = oracle_inputs(wl)
    step = gpu_step(wl)
    out, lse = step()
    torch.cuda.synchronize()
    res = _check_scores(step, wl, inp)
    _check_topk_sets(step, wl, res, exact=True)
    for t in range(wl.T):
        assert np.array_equal(step.idx[t].cpu().numpy(), wl.hot[t].cpu().numpy())
    _check_attention(out.cpu().numpy(), lse.cpu().numpy(), np.stack(res["o"]), np.stack(res["lse"]),
                     fp4=spec.lat_fmt == "nvfp4")


# ----------------------------------------------------------------- top-k alone
def _topk_alone(scores, vis, k, gpu):
    import sparse_attention_03_amd as dsa
    T, ld = scores.shape
    sc = scores.to(gpu)
    tv = torch.tensor(vis, dtype=torch.int32, device=gpu)
    tr = torch.zeros(T, dtype=torch.int32, device=gpu)
    rs = torch.tensor([0, T], dtype=torch.int32, device=gpu)
    b = dsa.batch_view(rs, tr, tv, None, ld, T)
    idx = torch.empty(T, k, dtype=torch.int32, device=gpu)
    cnt = torch.empty(T, dtype=torch.int32, device=gpu)
    a = dsa.topk_args(b, sc, k, idx, count=cnt)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.OP_TOPK, a), gpu)
    dsa.dsa_topk(dsa.topk_args(b, sc, k, idx, count=cnt, ws=ws))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("ld", [100000, 40000, 30000, 8192, 8000])
@pytest.mark.parametrize("kind", ["random", "ties", "all_equal", "short_rows", "k1", "negative", "sampled_high",
                                  "row_sampled_high", "one_slice_high"])
def test_topk_exact_on_same_scores(kind, ld, gpu):
    # ld 100000: threshold / filter / finalize kernels; ld 40000, 30000, 8192
    # and 8000: the one-workgroup-per-row kernel (16 float4 per thread at
    # 40000, 8 at 30000, 4 at 8192 and 8000; sampled threshold at 40000 and
    # 30000, every score kept at 8192 and 8000).  "all_equal" overflows the candidate buffers; "sampled_high" and
    # "row_sampled_high" put large scores only where the threshold sample of
    # the multi-kernel path (the first 32 of every 256) or of the per-row
    # kernel (group (p >> 12) & m == (p >> 2) & m of four, m = 15, or 7 for
    # rows up to 32K) looks, so the sampled threshold comes out too high and
    # the whole row is selected from.
    # "one_slice_high" puts 1800 of the top scores in one 8192-score slice of
    # the filter pass, more than a slice's candidate region (1024) holds.
    g = np.random.default_rng(42)
    T, k = 6, 2048
    if kind == "random":
        s = g.standard_normal((T, ld)).astype(np.float32) * 50 + 100
    elif kind == "ties":
        s = g.integers(0, 700, (T, ld)).astype(np.float32)
    elif kind == "all_equal":
        s = np.full((T, ld), 3.5, np.float32)
    elif kind == "short_rows":
        s = g.standard_normal((T, ld)).astype(np.float32)
    elif kind == "k1":
        s = g.integers(0, 5, (T, ld)).astype(np.float32)
        k = 1
    elif kind == "negative":
        s = -np.abs(g.standard_normal((T, ld)).astype(np.float32))
        s[:, ::7] = 0.0
        s[:, 3::7] = -0.0
    elif kind == "sampled_high":
        s = g.standard_normal((T, ld)).astype(np.float32)
        s[:, (np.arange(ld) % 256) < 32] += 1000.0
    elif kind == "row_sampled_high":
        s = g.standard_normal((T, ld)).astype(np.float32)
        pos = np.arange(ld)
        m = 7 if ld <= 32768 else 15
        s[:, ((pos >> 12) & m) == ((pos >> 2) & m)] += 1000.0
    else:
        s = g.standard_normal((T, ld)).astype(np.float32)
        s[:, 3 * 8192 // 4: 3 * 8192 // 4 + 1800] += 5.0 if ld < 8192 * 4 else 0.0
        s[:, 3 * 8192: 3 * 8192 + 1800] += 5.0 if ld >= 8192 * 4 else 0.0
    if ld == 100000:
        vis = [ld, ld - 1, 30001, 2049, 2048, 17] if kind == "short_rows" else [ld, ld - 3, 70001, 65537, 8193, 4097]
    elif ld in (40000, 30000):
        vis = [ld, ld - 1, 30001 if ld > 30001 else 20001, 2049, 2048, 17] if kind == "short_rows" else \
            [ld, ld - 3, ld, 12345, 8193, 4097]
    else:
        vis = [ld, ld - 1, 5001, 2049, 2048, 17] if kind == "short_rows" else [ld, ld - 3, min(ld, 8000), 6345, 4097, 2049]
    idx, cnt = _topk_alone(torch.from_numpy(s), vis, k, gpu)
    for t in range(T):
        ref, _ = O.topk(s[t, : vis[t]].astype(np.float64), k)
        K = len(ref)
        assert cnt[t] == K
        assert np.array_equal(idx[t, :K], ref), f"{kind} row {t}"
        assert np.all(idx[t, K:] == -1)


@pytest.mark.parametrize("kind", ["random", "ties", "all_equal", "negative", "binade"])
@pytest.mark.parametrize("k", [2048, 384, 1])
def test_topk_many_short_rows(kind, k, gpu):
    """>= 512 rows of <= 8192 scores: the one-workgroup short-row kernel (keys
    in registers), against the oracle row by row; ragged lengths, rows that
    keep everything, ties, +-0, and scores of one binade (shared leading
    digits)."""
    print(f"[gpu] topk short rows {kind} k={k}", flush=True)
    g = np.random.default_rng(7 + k)
    T, ld = 600, 8192
    if kind == "random":
        s = g.standard_normal((T, ld)).astype(np.float32)
    elif kind == "ties":
        s = g.integers(0, 40, (T, ld)).astype(np.float32)
    elif kind == "all_equal":
        s = np.full((T, ld), -2.25, np.float32)
    elif kind == "negative":
        s = -np.abs(g.standard_normal((T, ld)).astype(np.float32))
        s[:, ::5] = 0.0
        s[:, 2::5] = -0.0
    else:
        s = (1.0 + g.random((T, ld))).astype(np.float32)
    vis = g.integers(1, ld + 1, T)
    vis[:8] = [ld, ld - 1, k, k + 1, max(1, k - 1), 1, 4097, 33]
    idx, cnt = _topk_alone(torch.from_numpy(s), vis.tolist(), k, gpu)
    for t in range(T):
        ref, _ = O.topk(s[t, : vis[t]].astype(np.float64), k)
        K = len(ref)
        assert cnt[t] == K
        assert np.array_equal(idx[t, :K], ref), f"{kind} row {t}"
        assert np.all(idx[t, K:] == -1)


def test_topk_candidate_overflow_path(gpu):
    # > 8192 scores share the threshold bin: the finalize pass rescans the row
    g = np.random.default_rng(3)
    T, ld = 2, 100000
    s = (64.0 + g.integers(0, 1 << 16, (T, ld)) * (8.0 / (1 << 16))).astype(np.float32)
    idx, cnt = _topk_alone(torch.from_numpy(s), [ld, ld - 11], 2048, gpu)
    for t, v in enumerate([ld, ld - 11]):
        ref, _ = O.topk(s[t, :v].astype(np.float64), 2048)
        assert np.array_equal(idx[t], ref)


# ----------------------------------------------------------------- attention alone
@pytest.mark.parametrize("lat_fmt,H,splits", [("bf16", 16, 0), ("fp8", 12, 0), ("fp8", 12, 1),
                                              ("fp8", 96, 0), ("nvfp4", 12, 0), ("nvfp4", 40, 3)])
def test_mla_on_generated_rows(lat_fmt, H, splits, gpu):
    import sparse_attention_03_amd as dsa
    spec = synth.Spec("mla", R=2, q_per_req=3, N=3000, page=64, lat_fmt=lat_fmt, H=H, seed=9)
    wl = _wl(spec, gpu)
    inp = oracle_inputs(wl)
    rows = synth.workloads.random_rows(wl, 2048)
    rows[1, 1000:] = -1              # a short list
    rows[2, :] = -1                  # an empty list
    rows[3, 5] = wl.num_pages * wl.P + 7   # an entry outside the pool is skipped
    out = torch.empty(wl.T, H, 512, device=gpu)
    lse = torch.empty(wl.T, H, device=gpu)
    lat = dsa.cache_view(wl.lat_pool, wl.P, dsa.LAT_FMT[lat_fmt])
    a = dsa.mla_args(wl.q_mla, lat, rows, out, lse, spec.sm_scale, splits)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.OP_MLA_DECODE, a), gpu)
    dsa.sparse_mla_decode(dsa.mla_args(wl.q_mla, lat, rows, out, lse, spec.sm_scale, splits, ws))
    torch.cuda.synchronize()
    rr = rows.cpu().numpy().copy()
    rr[rr >= wl.num_pages * wl.P] = -1
    ref_o, ref_lse = O.mla_on_rows(inp, rr)
    _check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_lse, fp4=lat_fmt == "nvfp4")
    assert np.all(out[2].cpu().numpy() == 0) and np.all(np.isneginf(lse[2].cpu().numpy()))


def test_mla_padded_heads_bit_identical(gpu):
    import sparse_attention_03_amd as dsa
    spec = synth.Spec("pad", R=1, q_per_req=4, N=5000, page=64, lat_fmt="fp8", H=16, seed=10)
    wl = _wl(spec, gpu)
    rows = synth.workloads.random_rows(wl, 2048)
    lat = dsa.cache_view(wl.lat_pool, wl.P, dsa.LAT_FMT["fp8"])
    outs = []
    for H in (12, 16):
        q = wl.q_mla[:, :H].contiguous()
        out = torch.empty(wl.T, H, 512, device=gpu)
        lse = torch.empty(wl.T, H, device=gpu)
        dsa.sparse_mla_decode(dsa.mla_args(q, lat, rows, out, lse, spec.sm_scale, 1))
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0][:, :12]) and torch.equal(outs[0][1], outs[1][1][:, :12])


def test_translate_matches_oracle(gpu):
    import sparse_attention_03_amd as dsa
    spec = synth.CONFIGS["tp8_spec_decode_64k"].replace(R=4, N=5000, seed=12)
    wl = _wl(spec, gpu)
    idx = synth.workloads.random_logical(wl, 2048)
    idx[0, 3] = 10 ** 6   # past the request's block-table row -> -1
    rows = torch.empty_like(idx)
    b = dsa.batch_view(wl.req_token_start, wl.tok_req, wl.tok_vis, wl.block_table, spec.N, spec.q_per_req)
    dsa.dsa_translate_pages(idx, 2048, b, wl.P.bit_length() - 1, wl.num_pages, rows)
    torch.cuda.synchronize()
    bt = wl.block_table.cpu().numpy()
    ii = idx.cpu().numpy()
    ii[0, 3] = -1
    for t in range(wl.T):
        assert np.array_equal(rows[t].cpu().numpy(), O.translate(ii[t], bt, int(wl.tok_req[t]), wl.P))


# ----------------------------------------------------------------- properties
def test_determinism_and_batch_invariance(gpu):
    spec = synth.CONFIGS["tp8_spec_decode_64k"].replace(R=4, N=9000, seed=13)
    wl = _wl(spec, gpu)
    step = gpu_step(wl, num_splits=4)
    outs = []
    for _ in range(3):
        o, l = step()
        outs.append((o.clone(), l.clone(), step.idx.clone()))
    torch.cuda.synchronize()
    for o, l, i in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1]) and torch.equal(i, outs[0][2])
    # request 2 alone gives the same bits as inside the batch
    one = synth.make_workload(spec, device=gpu)
    sl = slice(2 * 6, 3 * 6)
    one.req_token_start = torch.tensor([0, 6], dtype=torch.int32, device=gpu)
    one.tok_req = torch.zeros(6, dtype=torch.int32, device=gpu)
    one.tok_vis = wl.tok_vis[sl].contiguous()
    one.block_table = wl.block_table[2:3].contiguous()
    one.q_idx, one.w, one.q_mla = wl.q_idx[sl].contiguous(), wl.w[sl].contiguous(), wl.q_mla[sl].contiguous()
    one.spec = spec.replace(R=1)
    s1 = gpu_step(one, num_splits=4)
    o1, l1 = s1()
    torch.cuda.synchronize()
    assert torch.equal(s1.idx, outs[0][2][sl])
    assert torch.equal(o1, outs[0][0][sl]) and torch.equal(l1, outs[0][1][sl])
    for j in range(6):
        v = int(one.tok_vis[j])
        assert torch.equal(s1.scores[j, :v], step.scores[2 * 6 + j, :v])


# ----------------------------------------------------------------- indexer: rows per request
def _keep_last_rows(wl, counts):
    """The workload restricted to the last counts[r] query rows of each
    request (their causal visible counts unchanged), as a ragged batch."""
    q = wl.spec.q_per_req
    sel = torch.cat([torch.arange(r * q + q - n, r * q + q) for r, n in enumerate(counts)]).to(wl.tok_vis.device)
    starts = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=wl.tok_vis.device)
    pick = lambda x: None if x is None else x.index_select(0, sel).contiguous()
    return dataclasses.replace(wl, req_token_start=starts, tok_req=pick(wl.tok_req), tok_vis=pick(wl.tok_vis),
                               q_idx=pick(wl.q_idx), q_idx_scale=pick(wl.q_idx_scale), w=pick(wl.w),
                               q_mla=pick(wl.q_mla), hot=pick(wl.hot), spec=wl.spec.replace(q_per_req=max(counts)))


@pytest.mark.parametrize("key_fmt,counts,N", [
    # two passes (9 rows = 6 + 3), one row, odd halves; chunks of 1024 keys
    # (several ring rounds per workgroup) with a ragged last chunk
    ("fp8", [1, 9, 5, 4], 140001),
    ("mxfp4", [6, 3, 2, 7], 140001),
    ("nvfp4", [6, 3, 2, 7], 140001),
    # short context: one round per workgroup, a ragged last page
    ("mxfp4", [6, 1], 1000),
    ("nvfp4", [6, 1], 1000),
])
def test_indexer_rows_per_request(key_fmt, counts, N, gpu):
    print(f"[gpu] indexer rows {key_fmt} {counts} N={N}", flush=True)
    spec = synth.CONFIGS["tp8_spec_decode_64k"].replace(R=len(counts), q_per_req=max(counts), N=N,
                                                          key_fmt=key_fmt, seed=50 + N % 7)
    wl = _keep_last_rows(synth.make_workload(spec, device=gpu), counts)
    step = gpu_step(wl)
    step.indexer()
    torch.cuda.synchronize()
    inp = oracle_inputs(wl)
    rts = inp["req_token_start"]
    sc = step.scores.cpu().numpy()
    for r in range(len(counts)):
        nmax = int(inp["tok_vis"][rts[r]:rts[r + 1]].max())
        keys = O.request_keys(inp["key_pool"], key_fmt, wl.P, inp["block_table"], r, nmax)
        for t in range(rts[r], rts[r + 1]):
            n = int(inp["tok_vis"][t])
            ref = O.indexer_scores(O.dequant_q_idx(inp, t), inp["w"][t], keys[:n])
            assert_scores_close(sc[t, :n], ref, inp, t, keys=keys, what=f"request {r}")


# ----------------------------------------------------------------- FP8 queries / prefill
PREFILL = {
    # causal prefill: 300 new rows (ragged against 16-row groups) after a prefix
    "prefill_h96": synth.CONFIGS["prefill_chunk_32k"].replace(q_per_req=300, N=5300, seed=40),
    # two requests of 40 rows, 8 heads, FP8 query rows in decode-sized groups
    "prefill_2req": synth.CONFIGS["prefill_chunk_32k"].replace(R=2, q_per_req=40, N=3000, H=8, seed=41),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_end_to_end(name, gpu):
    spec = PREFILL[name]
    print(f"[gpu] prefill case {name}", flush=True)
    wl = _wl(spec, gpu)
    inp = oracle_inputs(wl)
    step = gpu_step(wl, prefill=True)
    out, lse = step()
    torch.cuda.synchronize()
    res = _check_scores(step, wl, inp)
    _check_topk_sets(step, wl, res, exact=False)
    idx = step.idx.cpu().numpy()
    same = [j for j, t in enumerate(res["t"]) if np.array_equal(idx[t, : len(res["idx"][j])], res["idx"][j])]
    assert len(same) >= len(res["t"]) // 2
    ts = [res["t"][j] for j in same]
    _check_attention(out.cpu().numpy()[ts], lse.cpu().numpy()[ts], np.stack([res["o"][j] for j in same]),
                     np.stack([res["lse"][j] for j in same]))


def test_fp8_query_decode_planted(gpu):
    spec = synth.CONFIGS["tp8_spec_decode_64k"].replace(R=2, N=14000, q_fmt="fp8", plant_gap=True, seed=42)
    wl = _wl(spec, gpu)
    inp = oracle_inputs(wl)
    step = gpu_step(wl)
    out, lse = step()
    torch.cuda.synchronize()
    res = _check_scores(step, wl, inp)
    _check_topk_sets(step, wl, res, exact=True)
    _check_attention(out.cpu().numpy(), lse.cpu().numpy(), np.stack(res["o"]), np.stack(res["lse"]))
