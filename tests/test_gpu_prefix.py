"""GPU parity of the shared-prefix indexer (dsa_indexer_scores_prefix): groups
of requests whose block tables share their first pages get the scores of the
plain indexer call on the same batch (within fp32 summation order) and of the
oracle (1e-5 of the row maximum, as every BF16-q score)."""
import numpy as np
import pytest
import torch

import sparse_attention_03_amd as dsa
import synth
from oracle import dsa as O
from tests.helpers import gpu_step, oracle_inputs

pytestmark = pytest.mark.gpu


def _shared(spec, groups, L, gpu):
    wl = synth.make_workload(spec, device=gpu)
    P = wl.P
    bt = wl.block_table.clone()
    for a, b in groups:
        bt[a:b, :L // P] = bt[a, :L // P].clone()
    wl.block_table = bt.contiguous()
    return wl


@pytest.mark.parametrize("key_fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("rows", [1, 3])
@pytest.mark.parametrize("L", [0, 64 * 40, 64 * 140])
def test_prefix_indexer(key_fmt, rows, L, gpu):
    print(f"[gpu] prefix indexer {key_fmt} rows={rows} L={L}", flush=True)
    spec = synth.CONFIGS["tp8_spec_decode_64k"].replace(R=8, q_per_req=rows, N=9000, key_fmt=key_fmt,
                                                        seed=300 + rows + L // 64)
    groups = [(0, 3), (3, 4), (4, 8)]
    wl = _shared(spec, groups, L, gpu)
    step = gpu_step(wl)
    step.indexer()
    plain = step.scores.clone()
    got = torch.full_like(step.scores, float("nan"))
    base = dsa.IndexerArgs.from_buffer_copy(step.iargs)
    base.scores = got.data_ptr()
    grs = torch.tensor([a * rows for a, _ in groups] + [8 * rows], dtype=torch.int32, device=gpu)
    gfr = torch.tensor([a for a, _ in groups], dtype=torch.int32, device=gpu)
    args, ws = dsa.indexer_prefix_args(base, grs, gfr, L, 5 * rows, gpu)
    dsa.dsa_indexer_scores_prefix(args)
    torch.cuda.synchronize()
    inp = oracle_inputs(wl)
    vis = inp["tok_vis"]
    g_np, p_np = got.cpu().numpy(), plain.cpu().numpy()
    rts = inp["req_token_start"]
    for r in range(spec.R):
        n = int(vis[rts[r]:rts[r + 1]].max())
        keys = O.request_keys(inp["key_pool"], spec.key_fmt, wl.P, inp["block_table"], r, n)
        for t in range(rts[r], rts[r + 1]):
            v = int(vis[t])
            ref = O.indexer_scores(O.dequant_q_idx(inp, t), inp["w"][t], keys[:v])
            tol = 1e-5 * np.abs(ref).max()
            assert np.abs(g_np[t, :v] - ref).max() <= tol, (r, t)
            assert np.abs(g_np[t, :v] - p_np[t, :v]).max() <= tol, (r, t)


def test_prefix_indexer_full_size(gpu):
    """At 64K with 32 requests of 6 rows in two groups sharing 48K tokens:
    the prefix call's scores against the plain call's, every row."""
    print("[gpu] prefix indexer 64K", flush=True)
    spec = synth.CONFIGS["tp8_spec_decode_64k"]
    L = 49152
    groups = [(0, 16), (16, 32)]
    wl = _shared(spec, groups, L, gpu)
    step = gpu_step(wl)
    step.indexer()
    plain = step.scores.clone()
    base = dsa.IndexerArgs.from_buffer_copy(step.iargs)
    grs = torch.tensor([0, 16 * 6, 32 * 6], dtype=torch.int32, device=gpu)
    gfr = torch.tensor([0, 16], dtype=torch.int32, device=gpu)
    args, ws = dsa.indexer_prefix_args(base, grs, gfr, L, 16 * 6, gpu)
    dsa.dsa_indexer_scores_prefix(args)   # writes step.scores in place
    torch.cuda.synchronize()
    vis = wl.tok_vis.cpu().numpy()
    d = (step.scores - plain).abs().cpu().numpy()
    mx = plain.abs().cpu().numpy()
    for t in range(wl.T):
        assert d[t, :vis[t]].max() <= 1e-5 * mx[t, :vis[t]].max(), t
