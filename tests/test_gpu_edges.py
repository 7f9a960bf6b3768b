"""GPU parity on the layer's edges, against the fp64 oracle.

  * absent pages: block-table entries set to -1 and past the pool, with signed
    head weights, through indexer -> top-k (fused translation) -> MLA, on the
    single-row and multi-row BF16 indexers for FP8, MXFP4 and NVFP4 keys and
    on the FP8-query indexer; one request with every page absent;
  * rows past the host bound: a request with more rows than max_rows_per_req
    promised still has every row scored;
  * the standalone translation maps absent pages to -1.
Tolerances as in test_gpu_parity (scores: tests.helpers.assert_scores_close).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import dsa as O
from tests.helpers import assert_scores_close, gpu_step, oracle_inputs
from tests.test_gpu_parity import _check_attention

pytestmark = pytest.mark.gpu

ABSENT = {
    # one row per request: the streaming single-row indexer
    "row_fp8": synth.Spec("row_fp8", R=4, q_per_req=1, N=5000, key_fmt="fp8", lat_fmt="fp8", H=12, k=512, seed=61),
    "row_mxfp4": synth.Spec("row_mxfp4", R=4, q_per_req=1, N=5000, key_fmt="mxfp4", lat_fmt="nvfp4", H=12, k=512,
                            seed=62),
    "row_nvfp4": synth.Spec("row_nvfp4", R=4, q_per_req=1, N=5000, key_fmt="nvfp4", lat_fmt="nvfp4", H=12, k=512,
                            seed=63),
    # speculative rows: the multi-row indexer
    "spec_fp8": synth.Spec("spec_fp8", R=4, q_per_req=4, N=5000, key_fmt="fp8", lat_fmt="fp8", H=16, k=512,
                           seed=64),
    "spec_mxfp4": synth.Spec("spec_mxfp4", R=4, q_per_req=4, N=5000, key_fmt="mxfp4", lat_fmt="fp8", H=16, k=512,
                             seed=65),
    "spec_nvfp4": synth.Spec("spec_nvfp4", R=4, q_per_req=4, N=5000, key_fmt="nvfp4", lat_fmt="nvfp4", H=16,
                             k=512, seed=66),
    # MXFP4 query rows on the FP4 matrix instruction
    "row_fp4q": synth.Spec("row_fp4q", R=4, q_per_req=1, N=5000, key_fmt="mxfp4", lat_fmt="nvfp4", q_fmt="mxfp4",
                           H=12, k=512, seed=70),
    # FP8 query rows (the prefill indexer), causal rows
    "fp8q": synth.Spec("fp8q", R=2, q_per_req=40, N=3000, key_fmt="fp8", lat_fmt="fp8", q_fmt="fp8", H=8,
                       k=512, seed=67),
    # FP8 query rows of speculative requests (the multi-row FP8 kernel)
    "fp8q_spec": synth.Spec("fp8q_spec", R=4, q_per_req=4, N=5000, key_fmt="fp8", lat_fmt="fp8", q_fmt="fp8",
                            H=12, k=512, seed=71),
}


def _damaged(spec, gpu, n_entries, all_absent_req=None):
    wl = synth.make_workload(spec.replace(w_signed=True), device=gpu)
    bt, hit = synth.mark_absent(wl, n_entries, seed=spec.seed + 1)
    if all_absent_req is not None:
        bt[all_absent_req, :] = -1
    wl.block_table = bt.contiguous()
    return wl


def _check_layer(wl, step, out, lse, prefill=False):
    inp = oracle_inputs(wl)
    res = O.layer(inp, k=wl.spec.k)
    sc = step.scores.cpu().numpy()
    idx = step.idx.cpu().numpy()
    rows = step.rows.cpu().numpy()
    cnt = step.count.cpu().numpy()
    vis = wl.tok_vis.cpu().numpy()
    assert inp["w"].min() < 0, "the head weights must include negative ones"
    same = []
    for j, t in enumerate(res["t"]):
        ref = res["scores"][j]
        assert_scores_close(sc[t, : vis[t]], ref, inp, t, what=wl.spec.name)
        K = len(res["idx"][j])
        assert cnt[t] == K and np.all(idx[t, K:] == -1) and np.all(rows[t, K:] == -1)
        sel = idx[t, :K]
        assert np.all(np.diff(sel) > 0)
        tau = res["tau"][j]
        if np.isfinite(tau):
            assert np.all(ref[sel] >= tau - 1e-3 * abs(tau)), f"row {t}: selected score below tau"
        else:
            # fewer present tokens than K: all of them, then the lowest-index absent ones
            assert np.array_equal(sel, res["idx"][j]), f"row {t}: set with -inf ties differs"
        if np.array_equal(sel, res["idx"][j]):
            same.append(j)
            assert np.array_equal(rows[t, :K], res["rows"][j]), f"row {t}: translated rows differ"
    assert len(same) >= max(1, len(res["t"]) // 2)
    ts = [res["t"][j] for j in same]
    _check_attention(out.cpu().numpy()[ts], lse.cpu().numpy()[ts], np.stack([res["o"][j] for j in same]),
                     np.stack([res["lse"][j] for j in same]), fp4=wl.spec.lat_fmt == "nvfp4")
    return res


@pytest.mark.parametrize("name", list(ABSENT))
def test_absent_pages_through_the_layer(name, gpu):
    spec = ABSENT[name]
    print(f"[gpu] absent pages {name}", flush=True)
    # 25 damaged (request, page) entries out of 4 x 79, and request 1 with
    # every page absent when there are more than two requests
    wl = _damaged(spec, gpu, 25, all_absent_req=1 if spec.R > 2 else None)
    prefill = spec.q_per_req > 8
    step = gpu_step(wl, prefill=prefill)
    out, lse = step()
    torch.cuda.synchronize()
    res = _check_layer(wl, step, out, lse, prefill)
    if spec.R > 2:
        # the all-absent request: every score -inf, the lowest K indices, no row, o = 0, lse = -inf
        for j, t in enumerate(res["t"]):
            if int(wl.tok_req[t]) == 1:
                assert np.all(np.isneginf(step.scores[t, : int(wl.tok_vis[t])].cpu().numpy()))
                assert np.all(step.rows[t].cpu().numpy() == -1)
                assert np.all(out[t].cpu().numpy() == 0) and np.all(np.isneginf(lse[t].cpu().numpy()))


def test_translate_maps_absent_pages_to_minus_one(gpu):
    import sparse_attention_03_amd as dsa
    spec = synth.Spec("tr", R=3, q_per_req=2, N=3000, H=4, k=256, seed=68)
    wl = _damaged(spec, gpu, 12)
    idx = synth.workloads.random_logical(wl, 256, seed=3)
    rows = torch.empty_like(idx)
    b = dsa.batch_view(wl.req_token_start, wl.tok_req, wl.tok_vis, wl.block_table, spec.N, 2)
    dsa.dsa_translate_pages(idx, 256, b, wl.P.bit_length() - 1, wl.num_pages, rows)
    torch.cuda.synchronize()
    bt = wl.block_table.cpu().numpy()
    got, ii = rows.cpu().numpy(), idx.cpu().numpy()
    for t in range(wl.T):
        ref = O.translate(ii[t], bt, int(wl.tok_req[t]), wl.P, num_pages=wl.num_pages)
        assert np.array_equal(got[t], ref)
    assert (got == -1).sum() > (ii == -1).sum(), "some selected index must fall on a damaged page"


@pytest.mark.parametrize("key_fmt", ["fp8", "mxfp4", "nvfp4"])
def test_rows_past_the_host_bound_are_scored(key_fmt, gpu):
    """max_rows_per_req = 1 selects the single-row kernel; requests that hold
    three rows anyway get all three scored."""
    import sparse_attention_03_amd as dsa
    spec = synth.Spec("extra", R=3, q_per_req=3, N=7000, key_fmt=key_fmt, lat_fmt="fp8", H=4, k=256, seed=69)
    print(f"[gpu] rows past the bound {key_fmt}", flush=True)
    wl = synth.make_workload(spec, device=gpu)
    step = dsa.make_step(key_pool=wl.key_pool, lat_pool=wl.lat_pool, page_size=wl.P, key_fmt=key_fmt,
                         lat_fmt="fp8", req_row_start=wl.req_token_start, tok_req=wl.tok_req, tok_vis=wl.tok_vis,
                         block_table=wl.block_table, q_idx=wl.q_idx, w=wl.w, q_mla=wl.q_mla, k=256,
                         sm_scale=spec.sm_scale, max_vis=spec.N, max_rows_per_req=1)
    step.scores.fill_(7.0)
    step.indexer()
    torch.cuda.synchronize()
    inp = oracle_inputs(wl)
    sc = step.scores.cpu().numpy()
    for r in range(spec.R):
        keys = O.request_keys(inp["key_pool"], key_fmt, wl.P, inp["block_table"], r, spec.N)
        for t in range(3 * r, 3 * r + 3):
            n = int(inp["tok_vis"][t])
            ref = O.indexer_scores(O.dequant_q_idx(inp, t), inp["w"][t], keys[:n])
            assert_scores_close(sc[t, :n], ref, inp, t, keys=keys, what=key_fmt)
