"""GPU parity of the sharded top-k merge (dsa_topk_sharded) through the C ABI.

The selected indices, counts and re-send flags are integers and compare bit
for bit with the oracle's merge (oracle/merge.py) on the same fp32 scores, and
the indices also with the unsharded top-k of the same rows (dsa_topk), which
the merge must reproduce exactly.
"""
import numpy as np
import pytest
import torch

import sparse_attention_03_amd as dsa
from oracle import merge as M

pytestmark = pytest.mark.gpu


def _local_layout(full: np.ndarray, W: int):
    """Full rows [T, n] -> the interleaved shard layout [W, T, ld]."""
    T, n = full.shape
    ld = -(-(-(-n // W)) // 4) * 4
    pad = np.zeros((T, ld * W), np.float32)
    pad[:, :n] = full
    return np.ascontiguousarray(pad.reshape(T, ld, W).transpose(2, 0, 1))


def _topk_full(full: np.ndarray, vis, k, gpu):
    T, n = full.shape
    ld = -(-n // 4) * 4
    sc = torch.zeros(T, ld, dtype=torch.float32)
    sc[:, :n] = torch.from_numpy(full)
    sc = sc.to(gpu)
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


def _run(full, vis, W, k, cand, gpu, check_unsharded=True):
    T, n = full.shape
    local = _local_layout(full, W)
    loc_t = torch.from_numpy(local).to(gpu)
    vis_t = torch.tensor(vis, dtype=torch.int32, device=gpu)
    idx, cnt, rs = dsa.topk_sharded(loc_t, vis_t, max(1, n), k, cand)
    torch.cuda.synchronize()
    idx, cnt, rs = idx.cpu().numpy(), cnt.cpu().numpy(), rs.cpu().numpy()
    ri, rc, rf, _ = M.sharded_topk_rows(local, np.asarray(vis), W, k, cand or None)
    assert np.array_equal(cnt, rc)
    assert np.array_equal(rs, rf), np.nonzero(rs != rf)
    assert np.array_equal(idx, ri), np.nonzero((idx != ri).any(axis=1))
    if check_unsharded and n >= 4:
        ui, uc = _topk_full(full, vis, k, gpu)
        assert np.array_equal(idx, ui) and np.array_equal(cnt, uc)
    return rs


def _rows(kind, T, n, seed):
    g = np.random.default_rng(seed)
    if kind == "random":
        return g.standard_normal((T, n)).astype(np.float32)
    if kind == "ties":
        return g.integers(-4, 5, (T, n)).astype(np.float32)
    if kind == "zeros":
        x = np.zeros((T, n), np.float32)
        x[g.random((T, n)) < 0.5] = -0.0
        return x
    if kind == "shard0_high":                 # every 4th token scores high: shard 0 of W=4 (and 2) holds the top
        x = g.standard_normal((T, n)).astype(np.float32)
        x[:, ::4] += 20.0
        return x
    if kind == "decreasing":
        return np.tile(-np.arange(n, dtype=np.float32), (T, 1))
    raise ValueError(kind)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("kind", ["random", "ties", "zeros", "shard0_high", "decreasing"])
def test_sharded_matches_oracle_and_unsharded(W, kind, gpu):
    print(f"[gpu] topk_sharded W={W} {kind}", flush=True)
    n = 9000
    vis = [0, 1, 3, W + 1, 100, 2047, 2048, 2049, 5000, 8999, 9000]
    full = _rows(kind, len(vis), n, 11 + W)
    _run(full, vis, W, 2048, 0, gpu)


@pytest.mark.parametrize("W,k,cand", [(4, 16, 3), (8, 64, 1), (2, 300, 7), (16, 2048, 2048), (3, 5, 5)])
def test_sharded_custom_candidates(W, k, cand, gpu):
    print(f"[gpu] topk_sharded custom W={W} k={k} cand={cand}", flush=True)
    vis = [0, 2, 17, 64, 299, 1000, 4000]
    for kind in ("random", "ties", "shard0_high"):
        full = _rows(kind, len(vis), 4000, 3 * W + k)
        _run(full, vis, W, k, cand, gpu)


def test_resend_cases_are_exercised(gpu):
    """The hand-worked oracle rows on the GPU: all shards re-send (equal
    scores), and only shard 0 re-sends (shard 0 holds the top)."""
    print("[gpu] topk_sharded resend cases", flush=True)
    full = np.ones((1, 100), np.float32)
    rs = _run(full, [100], 4, 16, 3, gpu)
    assert rs.tolist() == [[1, 1, 1, 1]]
    full = np.where(np.arange(1000) % 4 == 0, 1.0, 0.0).astype(np.float32)[None]
    rs = _run(full, [1000], 4, 8, 3, gpu)
    assert rs.tolist() == [[1, 0, 0, 0]]


def test_long_local_rows(gpu):
    """Local rows longer than the single-workgroup top-k handles (the
    threshold / filter / finalize path inside the shard step)."""
    print("[gpu] topk_sharded long local rows", flush=True)
    n = 200000
    vis = [200000, 150001, 70000]
    for kind in ("random", "shard0_high"):
        full = _rows(kind, len(vis), n, 5)
        _run(full, vis, 2, 2048, 0, gpu)


@pytest.mark.parametrize("shape", ["long_decode_1m", "tp8_spec_decode_64k"])
def test_full_size(shape, gpu):
    """The merge at the decode workloads' full sizes, eight shards: 4 rows of
    1,048,576 tokens, and 32 x 6 speculative rows of 65,531..65,536 tokens."""
    print(f"[gpu] topk_sharded full size {shape}", flush=True)
    if shape == "long_decode_1m":
        T, n = 4, 1 << 20
        vis = [n] * T
    else:
        T, n = 192, 65536
        vis = [n - 5 + (t % 6) for t in range(T)]
    full = np.random.default_rng(77).standard_normal((T, n)).astype(np.float32)
    _run(full, vis, 8, 2048, 0, gpu)
