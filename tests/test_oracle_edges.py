"""Pins for the oracle's edges (CPU only): quantised index queries, absent
block-table pages, NVFP4 index keys, signed head weights, NVFP4 block scales
and the byte model's constants.

  dequant_q_idx (FP8)    -> torch's float8_e4m3fn decoder x the stored scale,
                            scored by the pure-Python brute force
  dequant_q_idx (MXFP4)  -> the OCP E2M1 golden table x torch's E8M0 decoder
  absent pages           -> a dictionary of present tokens + brute force:
                            absent tokens score -inf, rank last (lower index
                            first), translate to -1 and are never attended
  NVFP4 keys             -> a hand-written page (closed form), and insertion
                            decodes back to the quantised values
  signed head weights    -> brute force (fsum) over w in (-1, 1)
  nvfp4_blocks           -> hand-worked non-unit, subnormal, tie and
                            saturating block scales
  bytemodel              -> every byte figure the pages print
                            (tests/golden/page_constants.json)
"""
import json
import math
import os

import numpy as np
import torch

import synth
from oracle import brute, codecs as OC, dsa as O, quant as Q
from sparse_attention_03_amd import bytemodel as BM
from tests.helpers import oracle_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(codes) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _brute_scores(q, w, keys):
    return [brute.score(q.tolist(), w.tolist(), keys[s].tolist()) for s in range(keys.shape[0])]


# ------------------------------------------------------------------ quantised queries
def test_fp8_query_layer_matches_bruteforce():
    spec = synth.Spec("fp8q", R=2, q_per_req=2, N=90, page=16, k=20, H=2, q_fmt="fp8", seed=41)
    wl = synth.make_workload(spec)
    inp = oracle_inputs(wl)
    res = O.layer(inp, k=20)
    for t in range(wl.T):
        # independent decode of the query: torch's E4M3 table x the per-head scale
        q = _torch_e4m3(inp["q_idx"][t]) * inp["q_idx_scale"][t].astype(np.float64)[:, None]
        assert np.array_equal(O.dequant_q_idx(inp, t), q)
        r, n = int(wl.tok_req[t]), int(wl.tok_vis[t])
        keys = O.request_keys(inp["key_pool"], "fp8", 16, inp["block_table"], r, n)
        ref = _brute_scores(q, inp["w"][t], keys)
        assert np.allclose(res["scores"][t], ref, rtol=1e-12, atol=1e-12)
        assert res["idx"][t].tolist() == brute.topk_dominance(ref, 20)


def test_mxfp4_query_decode():
    g = np.random.default_rng(42)
    codes = g.integers(0, 256, (3, 32, 64)).astype(np.uint8)
    e8 = g.integers(100, 150, (3, 32, 4)).astype(np.uint8)
    inp = {"q_fmt": "mxfp4", "q_idx": codes, "q_idx_scale": e8}
    table = np.array(json.load(open(os.path.join(GOLD, "e2m1_ocp.json")))["codes_0_to_15"])
    e8v = torch.from_numpy(e8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for t in range(3):
        got = O.dequant_q_idx(inp, t)
        for h in (0, 7, 31):
            for i in (0, 1, 31, 32, 63, 64, 127):
                byte = int(codes[t, h, i // 2])
                nib = byte & 0xF if i % 2 == 0 else byte >> 4
                assert got[h, i] == table[nib] * e8v[t, h, i // 32]


# ------------------------------------------------------------------ absent pages
def _present_dictionary(inp, r, n):
    """(logical token -> dequantised key) for the tokens whose block-table
    entry names a page of the pool, built page by page."""
    P, bt = inp["P"], inp["block_table"]
    pool = inp["key_pool"]
    out = {}
    for lp in range((n + P - 1) // P):
        pg = int(bt[r, lp])
        if 0 <= pg < pool.shape[0]:
            vals = O.key_pages(pool, inp["key_fmt"], P, np.array([pg]))
            for slot in range(P):
                if lp * P + slot < n:
                    out[lp * P + slot] = vals[slot]
    return out


def test_absent_pages_score_minus_inf_rank_last_and_are_not_attended():
    spec = synth.Spec("absent", R=3, q_per_req=2, N=200, page=16, k=40, H=2, seed=43, w_signed=True)
    wl = synth.make_workload(spec)
    bt, hit = synth.mark_absent(wl, 9, seed=44)
    wl.block_table = bt
    inp = oracle_inputs(wl)
    num_pages = inp["key_pool"].shape[0]
    assert any(int(bt[r, lp]) < 0 for r, lp in hit) and any(int(bt[r, lp]) >= num_pages for r, lp in hit)
    res = O.layer(inp, k=40)
    for t in range(wl.T):
        r, n = int(wl.tok_req[t]), int(wl.tok_vis[t])
        have = _present_dictionary(inp, r, n)
        q = OC.bf16(inp["q_idx"][t])
        ref = [brute.score(q.tolist(), inp["w"][t].tolist(), have[s].tolist()) if s in have else -math.inf
               for s in range(n)]
        got = res["scores"][t]
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(got), fin)
        assert np.allclose(got[fin], np.array(ref)[fin], rtol=1e-12, atol=1e-12)
        sel = brute.topk_dominance(ref, 40)
        assert res["idx"][t].tolist() == sel
        # absent tokens translate to -1; present ones through the table
        for i, row in zip(sel, res["rows"][t]):
            pg = int(bt[r, i // 16])
            assert row == (pg * 16 + i % 16 if i in have else -1)
        lat = O.lat_rows(inp["lat_pool"], "fp8", 16, np.array([row for row in res["rows"][t] if row >= 0]))
        qm = OC.bf16(inp["q_mla"][t])
        for h in range(2):
            bo, blse = brute.attention(qm[h].tolist(), lat.tolist(), spec.sm_scale, 512)
            assert np.allclose(res["o"][t][h], bo, rtol=1e-11, atol=1e-13)
            assert abs(res["lse"][t][h] - blse) < 1e-11


def test_request_with_every_page_absent():
    spec = synth.Spec("allabsent", R=2, q_per_req=1, N=70, page=16, k=8, H=1, seed=45)
    wl = synth.make_workload(spec)
    bt = wl.block_table.clone()
    bt[1, :] = -1
    wl.block_table = bt
    res = O.layer(oracle_inputs(wl), k=8)
    assert np.all(res["scores"][1] == -math.inf)
    assert res["idx"][1].tolist() == list(range(8))         # ties at -inf: lowest indices
    assert np.all(res["rows"][1] == -1)
    assert np.all(res["o"][1] == 0) and np.all(res["lse"][1] == -math.inf)
    assert np.all(np.isfinite(res["scores"][0]))


def test_translate_absent_and_out_of_pool_pages():
    bt = np.array([[3, -1, 7, 2]])
    idx = np.array([0, 17, 33, 63, 48, -1])
    assert O.translate(idx, bt, 0, 16, num_pages=5).tolist() == [48, -1, -1, 47, 32, -1]
    assert O.translate(idx, bt, 0, 16).tolist() == [48, -16 + 1, 7 * 16 + 1, 47, 32, -1]


# ------------------------------------------------------------------ NVFP4 keys
def test_nvfp4_key_page_closed_form():
    P = 4
    pool = np.zeros((1, 72 * P), np.uint8)
    pool[0, 64:128] = 0x3A          # token 1: low nibble 0xA = -1.0, high nibble 0x3 = 1.5
    pool[0, 64 * P + 8: 64 * P + 16] = [0x38, 0x40, 0x30, 0x48, 0x01, 0x7E, 0x00, 0xB8]
    k = O.key_pages(pool, "nvfp4", P, np.array([0]))
    assert np.all(k[0] == 0) and np.all(k[2:] == 0)
    scales = [1.0, 2.0, 0.5, 4.0, 2.0 ** -9, 448.0, 0.0, -1.0]
    for b, s in enumerate(scales):
        seg = k[1, 16 * b: 16 * b + 16]
        assert np.all(seg[0::2] == -1.0 * s) and np.all(seg[1::2] == 1.5 * s)


def test_nvfp4_key_insert_decodes_back():
    g = np.random.default_rng(46)
    P = 16
    pool = g.integers(0, 256, (3, 72 * P)).astype(np.uint8)
    kv = torch.from_numpy(g.standard_normal((1, 128)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    kp, _ = Q.cache_insert(pool, "nvfp4", None, "fp8", P, np.array([[2]]), np.array([0]), np.array([5]), kv, None, 3)
    x = Q.bf16_to_f32(kv[0]).astype(np.float64)
    got = O.key_pages(kp, "nvfp4", P, np.array([2]))[5]
    # within each 16-block: the block maximum maps near 6 x scale, and every
    # element is within half an E2M1 step (x scale) of its input
    sc = OC.e4m3(kp[2, 64 * P + 5 * 8: 64 * P + 6 * 8])
    for b in range(8):
        xs = x[16 * b:16 * b + 16]
        assert sc[b] == OC.e4m3(Q.e4m3_encode(np.float32(np.abs(xs).max() / 6.0)))
        assert np.all(np.abs(got[16 * b:16 * b + 16] - xs) <= sc[b] * 1.0 + 1e-12)
    untouched = np.ones(72 * P, bool)
    untouched[5 * 64:6 * 64] = False
    untouched[64 * P + 40:64 * P + 48] = False
    assert np.array_equal(kp[2, untouched], pool[2, untouched])
    assert np.array_equal(kp[[0, 1]], pool[[0, 1]])


# ------------------------------------------------------------------ signed head weights
def test_signed_head_weights_match_bruteforce():
    spec = synth.Spec("signed", R=1, q_per_req=2, N=60, page=16, k=12, H=1, seed=47, w_signed=True)
    wl = synth.make_workload(spec)
    inp = oracle_inputs(wl)
    assert inp["w"].min() < 0 < inp["w"].max()
    res = O.layer(inp, k=12)
    for t in range(wl.T):
        keys = O.request_keys(inp["key_pool"], "fp8", 16, inp["block_table"], 0, int(wl.tok_vis[t]))
        ref = _brute_scores(OC.bf16(inp["q_idx"][t]), inp["w"][t], keys)
        assert np.allclose(res["scores"][t], ref, rtol=1e-12, atol=1e-12)
        assert min(ref) < 0   # negative weights do give negative scores
        assert res["idx"][t].tolist() == brute.topk_dominance(ref, 12)


# ------------------------------------------------------------------ NVFP4 block scales
def test_nvfp4_blocks_hand_worked_scales():
    def one(block):
        x = np.zeros(16, np.float32)
        x[: len(block)] = block
        packed, sc = Q.nvfp4_blocks(x[None], 16)
        vals = OC.e2m1_packed(packed)[0] * OC.e4m3(sc)[0, 0]
        return int(sc[0, 0]), vals[: len(block)].tolist()

    # amax 3 -> scale 0.5 (0x30), elements 6, 3, 0.5, -1.5 exactly
    assert one([3.0, 1.5, 0.25, -0.75]) == (0x30, [3.0, 1.5, 0.25, -0.75])
    # amax 7 -> 7/6 = 1.1667 rounds to 1.125 (0x39); 7/1.125 = 6.22 saturates to 6 -> 6.75
    assert one([7.0, -2.25]) == (0x39, [6.75, -2.25])
    # amax 6.375 -> 1.0625 is the midpoint of 1.0 and 1.125: ties to the even code 0x38
    assert one([6.375, 1.0]) == (0x38, [6.0, 1.0])
    # amax 6 * 2^-8 -> scale 2^-8 = 2 x 2^-9, a subnormal E4M3 (code 2)
    assert one([6 * 2.0 ** -8, 2.0 ** -9]) == (0x02, [6 * 2.0 ** -8, 2.0 ** -9])
    # amax below half the smallest subnormal scale: scale code 0, every element 0
    assert one([2.0 ** -13, -2.0 ** -14]) == (0x00, [0.0, 0.0])
    # amax 3000 -> 500 saturates to 448 (0x7E); 3000/448 = 6.7 saturates to 6 -> 2688
    assert one([3000.0, -448.0]) == (0x7E, [2688.0, -448.0])


# ------------------------------------------------------------------ byte model
def test_bytemodel_reproduces_the_pages_byte_figures():
    g = json.load(open(os.path.join(GOLD, "page_constants.json")))
    assert BM.KEY_B["fp8"] == g["fp8_index_key_bytes"]["value"]
    assert BM.KEY_B["mxfp4"] == g["mxfp4_index_key_bytes"]["value"]
    assert round(100 * BM.index_key_saving("fp8", "mxfp4"), 1) == g["mxfp4_index_saving_pct"]["value"]
    assert BM.LAT_B_PAGE_FORMULA["fp8"] == g["fp8_latent_bytes"]["value"]
    assert BM.LAT_B["nvfp4"] == g["nvfp4_latent_bytes"]["value"]
    assert BM.TOPK == g["topk"]["value"]
    assert BM.step_flops(row_vis=[1], k=1, H=0)["indexer"] == 2 * g["indexer_heads"]["value"] * 128
    # about 23% of dense MLA's bytes at long context (1M tokens)
    assert round(100 * BM.dense_vs_sparse_ratio(1 << 20)) == g["decode_bytes_vs_dense_pct"]["value"]
    # latents plus index keys of 1M FP8 tokens: about 0.7 GB
    assert round(BM.cache_bytes_per_token("fp8", "fp8") * 1e6 / 1e9, 1) == \
        g["dcp_prefill_workspace_gb_per_1m_tokens_fp8"]["value"]
    # 2,048 candidates: score + id 16 KiB, scores only 8 KiB
    assert [BM.candidate_exchange_bytes(2048, ids=True) / 1024, BM.candidate_exchange_bytes(2048, ids=False) / 1024] \
        == g["candidate_bytes_per_query_kib"]["value"]
    m = g["mla_payload_gb"]
    assert round(BM.latent_cache_bytes(m["layers"], m["tokens"], m["bytes"]) / 1e9, 2) == m["value"]
    assert round(BM.latent_cache_bytes(m["layers"], m["tokens"], m["bytes"]) / 8 / 1e6) == \
        g["mla_payload_dcp8_mb"]["value"]
    ph = g["padded_heads"]
    assert BM.padded_heads(ph["real"]) == ph["padded"]


def test_bytemodel_step_terms_on_a_hand_counted_step():
    # 2 requests of 100 and 3000 tokens, 1 row each, k = 2048, 12 heads, FP8 / FP8, page 64
    b = BM.step_bytes(req_vis_max=[100, 3000], row_vis=[100, 3000], k=2048, H=12, key_fmt="fp8", lat_fmt="fp8")
    assert b["keys"] == 3100 * 132
    assert b["latents"] == (100 + 2048) * 580
    bt = (2 + 47) * 4
    small = 2 * 8192 + 2 * 128 + 2 * 12 * 1152 + 2 * 12 * (2048 + 4) + bt
    assert b["small"] == small and b["total"] == 3100 * 132 + 2148 * 580 + small
    assert BM.literal_formula_bytes(2, 3000) == 2 * (3000 * 132 + 2048 * 576)
    f = BM.step_flops(row_vis=[100, 3000], k=2048, H=12)
    assert f["indexer"] == 3100 * 8192 and f["mla"] == (100 + 2048) * 2 * 12 * 1088
