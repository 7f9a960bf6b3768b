"""Parity at the full reference workload sizes, in the launch configuration the
benchmark times (DecodeStep with automatic splits), on sampled query rows the
oracle recomputes one by one.

  tiny_decode_8k       every row (one)
  tp8_spec_decode_64k  rows of 3 requests (all 6 speculative rows each)
  long_decode_1m       2 of 4 rows (planted gap: bit-exact top-k sets)
  prefill_chunk_32k    8 rows spread over the chunk (first, last, ragged tail)
  fp4_decode_256k      4 of 64 rows (and 3 rows each of the same workload
                       with NVFP4 index keys, and with MXFP4 index queries)
Tolerances as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dsa as O
from tests.helpers import assert_scores_close, gpu_step, oracle_inputs
from tests.test_gpu_parity import _check_attention

pytestmark = pytest.mark.gpu

SAMPLES = {
    "tiny_decode_8k": [0],
    "tp8_spec_decode_64k": list(range(0, 6)) + list(range(90, 96)) + list(range(186, 192)),
    "long_decode_1m": [0, 3],
    "prefill_chunk_32k": [0, 1, 517, 2048, 3001, 4094, 4095, 2],
    "fp4_decode_256k": [0, 17, 40, 63],
    # the FP4 workload with NVFP4 index keys (72 B per key) in place of MXFP4
    "fp4_decode_256k_nvfp4_keys": [0, 33, 63],
    # the FP4 workload with MXFP4 index queries on the FP4 matrix instruction
    "fp4_decode_256k_mxfp4_q": [1, 30, 62],
    # the 64K speculative workload with FP8 index queries (multi-row FP8 kernel)
    "tp8_spec_decode_64k_fp8_q": [0, 5, 96, 191],
}
SPECS = dict(synth.CONFIGS)
SPECS["fp4_decode_256k_nvfp4_keys"] = synth.CONFIGS["fp4_decode_256k"].replace(
    name="fp4_decode_256k_nvfp4_keys", key_fmt="nvfp4", seed=1006)
SPECS["fp4_decode_256k_mxfp4_q"] = synth.CONFIGS["fp4_decode_256k"].replace(
    name="fp4_decode_256k_mxfp4_q", q_fmt="mxfp4", seed=1007)
SPECS["tp8_spec_decode_64k_fp8_q"] = synth.CONFIGS["tp8_spec_decode_64k"].replace(
    name="tp8_spec_decode_64k_fp8_q", q_fmt="fp8", seed=1008)


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_sampled(name, gpu):
    spec = SPECS[name]
    print(f"[gpu] full-size {name}", flush=True)
    wl = synth.make_workload(spec, device=gpu)
    step = gpu_step(wl, prefill=spec.q_per_req > 64)
    out, lse = step()
    torch.cuda.synchronize()
    rows = SAMPLES[name]
    inp = oracle_inputs(wl)
    res = O.layer(inp, k=spec.k, tokens=rows)
    sc = step.scores
    idx = step.idx.cpu().numpy()
    cnt = step.count.cpu().numpy()
    same = []
    for j, t in enumerate(res["t"]):
        n = int(wl.tok_vis[t])
        ref = res["scores"][j]
        assert_scores_close(sc[t, :n].cpu().numpy(), ref, inp, t, what=name)
        K = len(res["idx"][j])
        assert cnt[t] == K and np.all(idx[t, K:] == -1)
        sel = idx[t, :K]
        assert np.all(np.diff(sel) > 0)
        if spec.plant_gap:
            assert np.array_equal(sel, res["idx"][j]), f"row {t} top-k set"
            assert np.array_equal(sel, wl.hot[t].cpu().numpy())
        else:
            tau = res["tau"][j]
            assert np.all(ref[sel] >= tau - 1e-3 * abs(tau)), f"row {t} top-k tolerance"
        if np.array_equal(sel, res["idx"][j]):
            same.append(j)
    assert len(same) >= max(1, len(res["t"]) // 2)
    ts = [res["t"][j] for j in same]
    _check_attention(out[ts].cpu().numpy(), lse[ts].cpu().numpy(), np.stack([res["o"][j] for j in same]),
                     np.stack([res["lse"][j] for j in same]), fp4=spec.lat_fmt == "nvfp4")
