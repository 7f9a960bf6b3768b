"""Pins for the fp64 oracle (CPU only).

Each test ties one oracle function to something other than itself: a library
routine, a closed form, an invariant the pages state, a value the pages print,
or a pure-Python brute force on tiny inputs.

  codecs          -> torch's float8/bfloat16 decoders, OCP E2M1 table (golden)
  key/lat decode  -> paged vs non-paged layouts of the same values; closed forms
  indexer_scores  -> brute force (fsum), one-hot closed form, homogeneity,
                     head-permutation invariance
  topk            -> pairwise-dominance brute force, all-equal ties, k >= n,
                     planted gap
  sparse_mla      -> brute force, dense == sparse (scipy softmax/logsumexp),
                     padded heads, LSE merge, q = 0, identical rows, one row,
                     permutation, V = first 512 dims
  translate       -> dictionary brute force
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

import synth
from oracle import brute, codecs as OC, dsa as O
from tests.helpers import oracle_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ codecs
def test_e4m3_table_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(OC.E4M3_TABLE)
    assert np.array_equal(ref[~both_nan], OC.E4M3_TABLE[~both_nan])
    assert both_nan.sum() == 2          # 0x7F and 0xFF only
    assert np.nanmax(OC.E4M3_TABLE) == 448.0


def test_e2m1_table_matches_ocp_golden():
    g = json.load(open(os.path.join(GOLD, "e2m1_ocp.json")))["codes_0_to_15"]
    assert np.array_equal(OC.E2M1_TABLE, np.array(g))
    # low nibble first
    assert np.array_equal(OC.e2m1_packed(np.array([[0x71]], np.uint8)), [[0.5, 6.0]])


def test_e8m0_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(ref[:255], OC.E8M0_TABLE[:255])
    assert math.isnan(OC.E8M0_TABLE[255])


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(3)
    bits = torch.randint(-32768, 32767, (4096,), generator=g, dtype=torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = OC.bf16(bits.numpy())
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], got[fin])


def test_bf16_rounding_example_from_page():
    g = json.load(open(os.path.join(GOLD, "page_constants.json")))["bf16_rounding_example"]
    b = synth.codecs.bf16_bits(torch.tensor([g["input"]]))
    assert OC.bf16(b.view(torch.int16).numpy())[0] == g["bf16"]


# ------------------------------------------------------------------ indexer
def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_scores_match_bruteforce():
    q, keys = _rand((32, 128), 1), _rand((24, 128), 2)
    w = np.random.default_rng(3).uniform(size=32)
    got = O.indexer_scores(q, w, keys)
    for s in range(24):
        ref = brute.score(q.tolist(), w.tolist(), keys[s].tolist())
        assert abs(got[s] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_scores_one_hot_closed_form():
    q = _rand((32, 128), 4)
    for h, j, ks in [(0, 0, 1.0), (5, 77, 0.25), (31, 127, 3.0), (17, 3, 2.0)]:
        w = np.zeros(32)
        w[h] = 1.0
        key = np.zeros((1, 128))
        key[0, j] = ks
        assert O.indexer_scores(q, w, key)[0] == ks * max(0.0, q[h, j])


def test_scores_homogeneity_and_head_permutation():
    q, keys = _rand((32, 128), 5), _rand((50, 128), 6)
    w = np.random.default_rng(7).uniform(size=32)
    base = O.indexer_scores(q, w, keys)
    # per-token scale pulls out of the ReLU (scale > 0)
    assert np.allclose(O.indexer_scores(q, w, 2.0 * keys), 2.0 * base, rtol=1e-14, atol=0)
    assert np.allclose(O.indexer_scores(q, 3.0 * w, keys), 3.0 * base, rtol=1e-14, atol=0)
    perm = np.random.default_rng(8).permutation(32)
    assert np.allclose(O.indexer_scores(q[perm], w[perm], keys), base, rtol=1e-13, atol=0)
    # keys anti-aligned with every head contribute nothing
    assert np.all(O.indexer_scores(np.abs(q), w, -np.abs(keys)) == 0.0)


def test_paged_and_nonpaged_decode_the_same_values():
    base = synth.Spec("t", R=2, q_per_req=1, N=300, page=64, key_fmt="fp8",
                      lat_fmt="fp8", H=4, k=16, seed=11)
    for kf, lf in [("fp8", "fp8"), ("mxfp4", "nvfp4"), ("fp8", "bf16")]:
        a = oracle_inputs(synth.make_workload(base.replace(key_fmt=kf, lat_fmt=lf)))
        b = oracle_inputs(synth.make_workload(base.replace(key_fmt=kf, lat_fmt=lf, page=0)))
        for r in range(2):
            ka = O.request_keys(a["key_pool"], kf, a["P"], a["block_table"], r, 300)
            kb = O.request_keys(b["key_pool"], kf, b["P"], b["block_table"], r, 300)
            assert np.array_equal(ka, kb)
            idx = np.arange(0, 300, 7)
            la = O.lat_rows(a["lat_pool"], lf, a["P"], O.translate(idx, a["block_table"], r, a["P"]))
            lb = O.lat_rows(b["lat_pool"], lf, b["P"], O.translate(idx, b["block_table"], r, b["P"]))
            assert np.array_equal(la, lb)


def test_key_decode_closed_form_fp8():
    # one page of 4 tokens written by hand: codes 0x38 (=1.0) and 0xB8 (=-1.0)
    P = 4
    pool = np.zeros((1, 132 * P), np.uint8)
    pool[0, :128] = 0x38
    pool[0, 128:256] = 0xB8
    pool[0, 128 * P: 128 * P + 16] = np.array([0.5, 2.0, 1.0, 1.0], "<f4").view(np.uint8)
    k = O.key_pages(pool, "fp8", P, np.array([0]))
    assert np.all(k[0] == 0.5) and np.all(k[1] == -2.0) and np.all(k[2:] == 0)


def test_key_decode_closed_form_mxfp4():
    P = 4
    pool = np.zeros((1, 68 * P), np.uint8)
    pool[0, :64] = 0x72            # pairs (1.0, 6.0)
    pool[0, 64 * P: 64 * P + 4] = [127, 128, 126, 130]
    k = O.key_pages(pool, "mxfp4", P, np.array([0]))[0]
    for blk, e in enumerate([0, 1, -1, 3]):
        seg = k[32 * blk: 32 * blk + 32]
        assert np.all(seg[0::2] == 2.0 ** e) and np.all(seg[1::2] == 6.0 * 2.0 ** e)


def test_lat_decode_closed_form_nvfp4():
    P = 2
    pool = np.zeros((1, 384 * P), np.uint8)
    pool[0, 384:640] = 0x1F            # row 1 codes: low nibble 0xF = -6.0, high nibble 0x1 = 0.5
    pool[0, 384 + 256: 384 + 288] = 0x40   # row 1 block scales: E4M3 0x40 = 2.0
    pool[0, 384 + 288: 384 + 352] = 0xB8   # row 1 rope: E4M3 0xB8 = -1.0
    pool[0, 384 + 352: 768] = 0x7E         # row 1 padding: never read
    lat = O.lat_rows(pool, "nvfp4", P, np.array([1, 0]))
    assert np.all(lat[0, 0:512:2] == -12.0) and np.all(lat[0, 1:512:2] == 1.0)
    assert np.all(lat[0, 512:] == -1.0) and np.all(lat[1] == 0.0)


def test_lat_decode_closed_form_fp8():
    P = 2
    pool = np.zeros((1, 640 * P), np.uint8)
    pool[0, 0:576] = 0x38                  # row 0 codes: E4M3 0x38 = 1.0
    pool[0, 576:580] = np.frombuffer(np.float32(0.25).tobytes(), np.uint8)
    pool[0, 580:640] = 0x7E                # row 0 padding: never read
    pool[0, 640:640 + 576] = 0xC0          # row 1 codes: E4M3 0xC0 = -2.0
    pool[0, 640 + 576:640 + 580] = np.frombuffer(np.float32(3.0).tobytes(), np.uint8)
    lat = O.lat_rows(pool, "fp8", P, np.array([1, 0]))
    assert np.all(lat[0] == -6.0) and np.all(lat[1] == 0.25)


# ------------------------------------------------------------------ top-k
def test_topk_matches_pairwise_dominance_with_ties():
    rng = np.random.default_rng(9)
    for trial in range(30):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        sc = rng.integers(0, 5, size=n).astype(np.float64)   # many ties
        sel, tau = O.topk(sc, k)
        assert sel.tolist() == brute.topk_dominance(sc.tolist(), k)
        assert np.all(sc[sel] >= tau)
        rest = np.setdiff1d(np.arange(n), sel)
        assert np.all(sc[rest] <= tau)


def test_topk_all_equal_keeps_lowest_indices():
    sel, tau = O.topk(np.full(5000, 1.25), 2048)
    assert np.array_equal(sel, np.arange(2048)) and tau == 1.25


def test_topk_k_at_least_n_keeps_all():
    sc = _rand(100, 10)
    sel, _ = O.topk(sc, 2048)
    assert np.array_equal(sel, np.arange(100))


def test_topk_zero_and_negative_zero_tie():
    sel, _ = O.topk(np.array([0.0, -0.0, 0.0, 1.0]), 2)
    assert sel.tolist() == [0, 3]


def test_planted_gap_selects_planted_set():
    spec = synth.Spec("gap", R=2, q_per_req=3, N=5000, page=64, k=256, H=4,
                      plant_gap=True, seed=21)
    wl = synth.make_workload(spec)
    inp = oracle_inputs(wl)
    res = O.layer(inp, k=256)
    for t in range(wl.T):
        assert np.array_equal(res["idx"][t], wl.hot[t].numpy())
        s = np.sort(res["scores"][t])[::-1]
        assert s[255] >= 1.05 * s[256]


# ------------------------------------------------------------------ sparse MLA
def test_attention_matches_bruteforce():
    q, lat = _rand((3, 576), 12), _rand((9, 576), 13) / 24
    o, lse = O.sparse_mla(q, lat, 1 / math.sqrt(192))
    for h in range(3):
        bo, blse = brute.attention(q[h].tolist(), lat.tolist(), 1 / math.sqrt(192), 512)
        assert np.allclose(o[h], bo, rtol=1e-12, atol=1e-14)
        assert abs(lse[h] - blse) < 1e-12


def test_sparse_equals_dense_when_k_covers_context():
    q, lat = _rand((16, 576), 14), _rand((700, 576), 15) / 24
    sc = 1 / math.sqrt(192)
    sel, _ = O.topk(_rand(700, 16), 2048)
    o, lse = O.sparse_mla(q, lat[sel], sc)
    logits = sc * q @ lat.T
    ref_o = sps.softmax(logits, axis=1) @ lat[:, :512]
    ref_lse = sps.logsumexp(logits, axis=1)
    assert np.allclose(o, ref_o, rtol=1e-12, atol=1e-15)
    assert np.allclose(lse, ref_lse, rtol=1e-13, atol=0)


def test_padded_heads_leave_real_heads_bit_identical():
    q, lat = _rand((12, 576), 16), _rand((300, 576), 17) / 24
    o, lse = O.sparse_mla(q, lat, 0.1)
    for pad in (np.zeros((4, 576)), q[:4].copy()):
        o2, lse2 = O.sparse_mla(np.concatenate([q, pad]), lat, 0.1)
        assert np.array_equal(o2[:12], o) and np.array_equal(lse2[:12], lse)


def test_lse_merge_equals_unsplit():
    q, lat = _rand((16, 576), 18), _rand((2048, 576), 19) / 24
    o, lse = O.sparse_mla(q, lat, 0.07)
    rng = np.random.default_rng(20)
    for nsplit in (2, 3, 8, 64):
        cuts = np.sort(rng.choice(np.arange(1, 2048), nsplit - 1, replace=False))
        parts = np.split(np.arange(2048), cuts)
        parts.append(np.arange(0))          # an empty split drops out
        po, pl = zip(*[O.sparse_mla(q, lat[p], 0.07) for p in parts])
        mo, ml = O.lse_merge(np.stack(po), np.stack(pl))
        assert np.allclose(mo, o, rtol=1e-12, atol=1e-15)
        assert np.allclose(ml, lse, rtol=1e-13, atol=0)


def test_uniform_softmax_and_degenerate_rows():
    lat = _rand((37, 576), 21)
    o, lse = O.sparse_mla(np.zeros((2, 576)), lat, 0.1)
    assert np.allclose(o, lat[:, :512].mean(0)[None], rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, math.log(37))
    same = np.repeat(lat[:1], 20, axis=0)
    o, _ = O.sparse_mla(_rand((4, 576), 22), same, 0.3)
    assert np.allclose(o, lat[0, :512][None], rtol=1e-13, atol=1e-15)
    q = _rand((4, 576), 23)
    o, lse = O.sparse_mla(q, lat[5:6], 0.3)
    assert np.array_equal(o, np.repeat(lat[5:6, :512], 4, 0))
    assert np.allclose(lse, 0.3 * q @ lat[5], rtol=1e-14)


def test_attention_permutation_invariant_and_value_slice():
    q, lat = _rand((8, 576), 24), _rand((128, 576), 25) / 24
    o, lse = O.sparse_mla(q, lat, 0.05)
    p = np.random.default_rng(26).permutation(128)
    o2, lse2 = O.sparse_mla(q, lat[p], 0.05)
    assert np.allclose(o2, o, rtol=1e-12, atol=1e-15) and np.allclose(lse2, lse, rtol=1e-14)
    # V = dims 0..511: with q = 0 the rope dims 512..575 must not reach o
    lat2 = lat.copy()
    lat2[:, 512:] *= -7
    a, _ = O.sparse_mla(np.zeros((1, 576)), lat, 0.05)
    b, _ = O.sparse_mla(np.zeros((1, 576)), lat2, 0.05)
    assert np.array_equal(a, b)
    # and the rope dims do reach the logits
    c, _ = O.sparse_mla(q[:1], lat2, 0.05)
    assert not np.allclose(c, o[:1])


def test_empty_selection():
    o, lse = O.sparse_mla(_rand((3, 576), 27), np.zeros((0, 576)), 0.1)
    assert np.all(o == 0) and np.all(lse == -math.inf)


# ------------------------------------------------------------------ translation
def test_translate_matches_dictionary():
    rng = np.random.default_rng(28)
    P, R, npg = 64, 3, 9
    bt = rng.permutation(R * npg).reshape(R, npg)
    where = {}
    for r in range(R):
        for j in range(npg):
            for s in range(P):
                where[(r, j * P + s)] = bt[r, j] * P + s
    idx = np.concatenate([rng.choice(npg * P, 50, replace=False), [-1, -1]])
    for r in range(R):
        got = O.translate(idx, bt, r, P)
        ref = [where[(r, int(i))] if i >= 0 else -1 for i in idx]
        assert got.tolist() == ref


def test_layer_composes_the_stages():
    spec = synth.Spec("tiny", R=2, q_per_req=2, N=200, page=16, k=24, H=3, seed=30)
    wl = synth.make_workload(spec)
    inp = oracle_inputs(wl)
    res = O.layer(inp, k=24)
    for t in range(wl.T):
        r = int(wl.tok_req[t])
        n = int(wl.tok_vis[t])
        keys = O.request_keys(inp["key_pool"], "fp8", 16, inp["block_table"], r, n)
        q = OC.bf16(inp["q_idx"][t])
        sc = [brute.score(q.tolist(), inp["w"][t].tolist(), keys[s].tolist()) for s in range(n)]
        sel = brute.topk_dominance(sc, 24)
        assert res["idx"][t].tolist() == sel
        lat = O.lat_rows(inp["lat_pool"], "fp8", 16, O.translate(np.array(sel), inp["block_table"], r, 16))
        qm = OC.bf16(inp["q_mla"][t])
        for h in range(3):
            bo, blse = brute.attention(qm[h].tolist(), lat.tolist(), spec.sm_scale, 512)
            assert np.allclose(res["o"][t][h], bo, rtol=1e-11, atol=1e-13)
            assert abs(res["lse"][t][h] - blse) < 1e-11
