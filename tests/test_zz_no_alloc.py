"""sparse_mla_decode_noalloc (the allocation-free decode entry point) against
sparse_mla_decode on the same inputs, through the C ABI.

Two calls in a row share the library's device scratch, the second on a
smaller input: each must equal sparse_mla_decode bit for bit (same kernels,
same split plan) and the oracle within the attention tolerance.  A third call
whose automatic split count would overflow the scratch runs with fewer splits
(equal to sparse_mla_decode within the attention tolerance), and an explicit split count
that cannot fit is rejected on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_03_amd as dsa
import synth
from oracle import dsa as O
from tests.helpers import oracle_inputs
from tests.test_gpu_parity import _check_attention

pytestmark = pytest.mark.gpu


def _case(spec, gpu, k):
    wl = synth.make_workload(spec, device=gpu)
    rows = synth.workloads.random_rows(wl, k, seed=spec.seed)
    lats = dsa.cache_view(wl.lat_pool, wl.P, dsa.LAT_FMT[spec.lat_fmt])
    return wl, rows, lats


def _both(wl, rows, lats, sm_scale, num_splits=0):
    T, H = wl.T, wl.q_mla.shape[1]
    dev = wl.q_mla.device
    o_ref = torch.empty(T, H, 512, dtype=torch.float32, device=dev)
    l_ref = torch.empty(T, H, dtype=torch.float32, device=dev)
    a = dsa.mla_args(wl.q_mla, lats, rows, o_ref, l_ref, sm_scale, num_splits)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.OP_MLA_DECODE, a), dev)
    a = dsa.mla_args(wl.q_mla, lats, rows, o_ref, l_ref, sm_scale, num_splits, ws)
    dsa.sparse_mla_decode(a)
    o = torch.full((T, H, 512), float("nan"), device=dev)
    lse = torch.full((T, H), float("nan"), device=dev)
    b = dsa.mla_args(wl.q_mla, lats, rows, o, lse, sm_scale, num_splits)   # no workspace
    assert b.workspace is None and b.workspace_bytes == 0
    dsa.sparse_mla_decode_noalloc(b)
    torch.cuda.synchronize()
    return o_ref.cpu().numpy(), l_ref.cpu().numpy(), o.cpu().numpy(), lse.cpu().numpy()


def _vs_oracle(wl, rows, o, lse):
    inp = oracle_inputs(wl)
    ro, rl = O.mla_on_rows(inp, rows.cpu().numpy().astype(np.int64))
    _check_attention(o, lse, ro, rl, fp4=wl.spec.lat_fmt == "nvfp4")


def test_noalloc_equals_decode_on_two_calls_in_a_row(gpu):
    # call 1: 192 rows x 12 heads, FP8 latents (5 automatic splits: 23.6 MB of partials)
    s1 = synth.CONFIGS["tp8_spec_decode_64k"].replace(R=32, N=3000, seed=81)
    # call 2: a smaller input, 10 rows x 40 heads, NVFP4 latents
    s2 = synth.Spec("small", R=5, q_per_req=2, N=2500, key_fmt="mxfp4", lat_fmt="nvfp4", H=40, k=1024, seed=82)
    for spec, k in ((s1, 2048), (s2, 1024)):
        print(f"[gpu] noalloc {spec.name} T={spec.R * spec.q_per_req} H={spec.H}", flush=True)
        wl, rows, lats = _case(spec, gpu, k)
        o_ref, l_ref, o, lse = _both(wl, rows, lats, spec.sm_scale)
        assert np.array_equal(o, o_ref), "output differs from sparse_mla_decode"
        assert np.array_equal(np.isfinite(lse), np.isfinite(l_ref)) and np.array_equal(lse, l_ref)
        _vs_oracle(wl, rows, o, lse)


def test_noalloc_lowers_automatic_splits_to_fit(gpu):
    # 64 rows x 128 heads: two automatic splits would need 33.6 MB > 32 MiB
    spec = synth.Spec("wide", R=64, q_per_req=1, N=2100, lat_fmt="fp8", H=128, k=2048, seed=83)
    print("[gpu] noalloc with lowered splits", flush=True)
    wl, rows, lats = _case(spec, gpu, 2048)
    o_ref, l_ref, o, lse = _both(wl, rows, lats, spec.sm_scale)
    assert np.all(np.isfinite(o))
    # another split plan rounds the bf16 softmax weights against other running
    # maxima: equal to sparse_mla_decode within the attention tolerance
    assert np.abs(o - o_ref).max() <= 1e-2 * np.abs(o_ref).max()
    assert np.abs(lse - l_ref).max() <= 1e-3
    _vs_oracle(wl, rows, o, lse)


def test_noalloc_rejects_explicit_splits_that_do_not_fit(gpu):
    spec = synth.Spec("wide2", R=64, q_per_req=1, N=2100, lat_fmt="fp8", H=128, k=2048, seed=84)
    wl, rows, lats = _case(spec, gpu, 2048)
    o = torch.empty(64, 128, 512, device=gpu)
    a = dsa.mla_args(wl.q_mla, lats, rows, o, None, spec.sm_scale, num_splits=8)
    st = dsa.load().sparse_mla_decode_noalloc(ctypes.byref(a), None)
    assert st == dsa.DSA_ERR_WORKSPACE
    assert b"scratch" in dsa.load().dsa_last_error()
