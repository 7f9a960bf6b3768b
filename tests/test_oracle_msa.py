"""Pins of the MSA block-sparse oracle (oracle/msa.py).

Checked against things other than itself: pure-Python loops (math.fsum dot
products, sorted tuples, explicit softmax) on a tiny paged input, the
selection rules worked out by hand, and invariants the method fixes (every
block kept when there are at most top_blocks of them, groups independent of
each other's K/V and index queries, q = 0 giving the mean of the values,
paging invisible).
"""
import math

import numpy as np
import pytest

import synth.msa as S
from oracle import codecs as C
from oracle import msa as M


def _tiny(seed=0, N=300, rows=2, hkv=2, hq=4, top=2):
    spec = S.MsaSpec("tiny", R=2, rows=rows, N=N, hkv=hkv, hq=hq, top_blocks=top, seed=seed)
    return spec, S.oracle_view(S.make_inputs(spec), spec)


def _brute_row(inp, t):
    """Everything written out with Python loops."""
    r, n = int(inp["tok_req"][t]), int(inp["tok_vis"][t])
    hkv, hq, top = inp["hkv"], inp["hq"], inp["top_blocks"]
    G = hq // hkv
    bt = inp["block_table"]
    E = C.E4M3_TABLE

    def key(s):
        page, slot = int(bt[r, s // 128]), s % 128
        return [float(E[c]) for c in inp["idx_pool"][page, slot * 128:(slot + 1) * 128]]

    def kv(s, which, g):
        page, slot = int(bt[r, s // 128]), s % 128
        row = inp["kv_pool"][page].reshape(128, 2, hkv, 128)[slot, which, g]
        sc = inp["k_scale"] if which == 0 else inp["v_scale"]
        return [sc * float(E[c]) for c in row]

    sel_all, o, lse = [], np.zeros((hq, 128)), np.zeros(hq)
    nb = (n + 127) // 128
    for g in range(hkv):
        q = [float(x) for x in inp["q_idx"][t, g]]
        bs = []
        for b in range(nb):
            bs.append(max(math.fsum(a * c for a, c in zip(q, key(s))) for s in range(b * 128, min(n, b * 128 + 128))))
        if nb <= top:
            sel = list(range(nb))
        else:
            others = sorted(range(nb - 1), key=lambda b: (-bs[b], b))[:top - 1]
            sel = sorted(others + [nb - 1])
        sel_all.append(sel)
        toks = [s for b in sel for s in range(b * 128, min(n, b * 128 + 128))]
        for h in range(g * G, (g + 1) * G):
            qh = [float(x) for x in inp["q"][t, h]]
            lg = [inp["sm_scale"] * math.fsum(a * c for a, c in zip(qh, kv(s, 0, g))) for s in toks]
            mx = max(lg)
            e = [math.exp(x - mx) for x in lg]
            z = math.fsum(e)
            vs = [kv(s, 1, g) for s in toks]
            for d in range(128):
                o[h, d] = math.fsum(e[i] * vs[i][d] for i in range(len(toks))) / z
            lse[h] = mx + math.log(z)
    return sel_all, o, lse


def test_brute_force_tiny():
    spec, inp = _tiny()
    for t in range(2):
        sel, o, lse, _ = M.msa_row(inp, t)
        bsel, bo, blse = _brute_row(inp, t)
        for g in range(spec.hkv):
            got = [int(x) for x in sel[g] if x >= 0]
            assert got == bsel[g]
        assert np.allclose(o, bo, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse, blse, rtol=1e-12, atol=1e-12)


def test_selection_rules_by_hand():
    # 6 blocks, keep 3: the last (5) always, then the best two others: scores
    # 1, 9, 9, 3, 8, -50 -> blocks 1 and 2 (tie at 9 broken to the lower id,
    # both kept), 4 loses to them; last block kept although lowest.
    assert M.select_blocks(np.array([1, 9, 9, 3, 8, -50.0]), 3).tolist() == [1, 2, 5]
    assert M.select_blocks(np.array([1, 9, 9, 3, 8, -50.0]), 2).tolist() == [1, 5]
    assert M.select_blocks(np.array([4.0, 4.0, 4.0]), 2).tolist() == [0, 2]
    assert M.select_blocks(np.array([4.0, -1.0]), 16).tolist() == [0, 1]
    assert M.select_blocks(np.array([7.0]), 1).tolist() == [0]
    # block max ignores positions past n: the last block holds 2 of 128
    s = np.arange(258, dtype=np.float64)[None]
    assert M.block_max(s).tolist() == [[127.0, 255.0, 257.0]]


def test_dense_when_every_block_fits():
    # N = 300 -> 3 blocks <= top 16: the result is dense attention over every
    # visible key of the group
    spec, inp = _tiny(seed=3, top=16)
    for t in range(2):
        sel, o, lse, _ = M.msa_row(inp, t)
        n, r = int(inp["tok_vis"][t]), int(inp["tok_req"][t])
        G = spec.hq // spec.hkv
        for g in range(spec.hkv):
            k, v = M.request_kv(inp["kv_pool"], inp["block_table"], r, np.arange((n + 127) // 128), n, spec.hkv, g,
                                spec.k_scale, spec.v_scale)
            assert k.shape[0] == n
            lg = inp["sm_scale"] * inp["q"][t, g * G:(g + 1) * G] @ k.T
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            ref = (p / p.sum(axis=1, keepdims=True)) @ v
            assert np.allclose(o[g * G:(g + 1) * G], ref, rtol=1e-12, atol=1e-12)


def test_groups_are_independent():
    spec, inp = _tiny(seed=4, N=700, top=3)
    sel, o, lse, bs = M.msa_row(inp, 1)
    inp2 = dict(inp)
    kv = inp["kv_pool"].copy().reshape(inp["kv_pool"].shape[0], 128, 2, spec.hkv, 128)
    kv[:, :, :, 1] = np.random.default_rng(0).integers(0, 120, kv[:, :, :, 1].shape)  # group 1's K and V
    inp2["kv_pool"] = kv.reshape(inp["kv_pool"].shape)
    qi = inp["q_idx"].copy()
    qi[:, 1] = -qi[:, 1]                                   # group 1's index query
    inp2["q_idx"] = qi
    sel2, o2, lse2, _ = M.msa_row(inp2, 1)
    G = spec.hq // spec.hkv
    assert np.array_equal(sel[0], sel2[0])
    assert np.array_equal(o[:G], o2[:G]) and np.array_equal(lse[:G], lse2[:G])
    assert not np.array_equal(o[G:], o2[G:])


def test_zero_query_gives_mean_of_values():
    spec, inp = _tiny(seed=5, N=500, top=2)
    inp["q"] = np.zeros_like(inp["q"])
    sel, o, lse, _ = M.msa_row(inp, 0)
    n, r = int(inp["tok_vis"][0]), int(inp["tok_req"][0])
    for g in range(spec.hkv):
        blocks = sel[g][sel[g] >= 0]
        _, v = M.request_kv(inp["kv_pool"], inp["block_table"], r, blocks, n, spec.hkv, g, spec.k_scale,
                            spec.v_scale)
        G = spec.hq // spec.hkv
        assert np.allclose(o[g * G], v.mean(axis=0), rtol=1e-12, atol=1e-13)
        assert lse[g * G] == pytest.approx(math.log(v.shape[0]))


def test_paging_is_invisible():
    spec, inp = _tiny(seed=6, N=600, top=3)
    ref = M.msa_row(inp, 0)
    nb = inp["idx_pool"].shape[0]
    perm = np.random.default_rng(1).permutation(nb)
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["idx_pool"] = inp["idx_pool"][perm]
    inp2["kv_pool"] = inp["kv_pool"][perm]
    inp2["block_table"] = inv[inp["block_table"]]
    got = M.msa_row(inp2, 0)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)


def test_planted_blocks_are_selected():
    spec = S.MsaSpec("p", R=1, rows=1, N=128 * 40 + 17, hkv=2, hq=4, top_blocks=16, planted=True, seed=9)
    inp = S.oracle_view(S.make_inputs(spec), spec)
    sel, _, _, bs = M.msa_row(inp, 0)
    for g in range(2):
        top = np.sort(bs[g][:-1])[::-1]
        assert top[14] > 2 * max(top[15], 0) + 100  # the gap below the 15 planted blocks
        assert sel[g][-1] == 40


def test_absent_blocks():
    # block 2 of request 0 absent: its score is -inf, it is never attended;
    # a row whose every selected block is absent gives o = 0, lse = -inf
    spec, inp = _tiny(seed=11, N=128 * 6, rows=1, top=3)
    inp["block_table"] = inp["block_table"].copy()
    inp["block_table"][0, 2] = -1
    sel, o, lse, bs = M.msa_row(inp, 0)
    assert np.all(bs[:, 2] == -np.inf)
    for g in range(spec.hkv):
        assert 2 not in sel[g].tolist() and sel[g][-1] == 5
    inp["block_table"][0, :] = -1
    sel, o, lse, bs = M.msa_row(inp, 0)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    assert [x for x in sel[0] if x >= 0] == [0, 1, 5]     # ties at -inf: the lower ids
