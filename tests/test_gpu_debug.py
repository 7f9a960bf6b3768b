"""The debug library (libdsa_debug.so, DSA_DEBUG=1) on the GPU: its kernels
note the metadata they clamp or skip, dsa_check_debug_flag() reads and clears
the notes, and its results still match the fp64 oracle.

  * a clean decode batch leaves no note;
  * absent block-table pages note DSA_DEBUG_ABSENT_PAGE (results checked as
    in test_gpu_edges);
  * a visible count above the host bound notes DSA_DEBUG_VIS_CLAMPED;
  * a row whose request id names no request notes DSA_DEBUG_REQ_OUTSIDE and
    gets no translated rows (-1), so attention reads nothing for it.
"""
import contextlib

import numpy as np
import pytest
import torch

import synth
import sparse_attention_03_amd as dsa
from tests.helpers import gpu_step
from tests.test_gpu_edges import _check_layer, _damaged

pytestmark = pytest.mark.gpu

SPEC = synth.Spec("debug", R=4, q_per_req=1, N=5000, key_fmt="fp8", lat_fmt="fp8", H=12, k=512, seed=81)


@contextlib.contextmanager
def debug_library():
    """Route the binding through libdsa_debug.so for the block's calls."""
    saved = dsa._lib
    dsa._lib = None
    try:
        lib = dsa.load(dsa.DEBUG_LIB_PATH)
        yield lib
    finally:
        dsa._lib = saved


def test_release_library_reports_no_debug_build(gpu):
    assert dsa.dsa_check_debug_flag() == -1


def test_clean_batch_leaves_no_note(gpu):
    print("[gpu] debug library: clean batch", flush=True)
    with debug_library():
        dsa.dsa_check_debug_flag()  # clear what earlier calls left
        wl = synth.make_workload(SPEC, device=gpu)
        step = gpu_step(wl)
        step()
        assert dsa.dsa_check_debug_flag() == 0


def test_absent_pages_are_noted_and_results_hold(gpu):
    print("[gpu] debug library: absent pages", flush=True)
    with debug_library():
        dsa.dsa_check_debug_flag()
        wl = _damaged(SPEC, gpu, 12)
        step = gpu_step(wl)
        out, lse = step()
        flag = dsa.dsa_check_debug_flag()
        assert flag & dsa.DEBUG_ABSENT_PAGE, f"flag {flag}"
        assert not flag & (dsa.DEBUG_VIS_CLAMPED | dsa.DEBUG_REQ_OUTSIDE), f"flag {flag}"
        _check_layer(wl, step, out, lse)
        assert dsa.dsa_check_debug_flag() == 0, "the call clears the notes"


def test_visible_count_above_the_bound_is_noted(gpu):
    print("[gpu] debug library: visible count above max_vis", flush=True)
    with debug_library():
        dsa.dsa_check_debug_flag()
        wl = synth.make_workload(SPEC, device=gpu)
        step = gpu_step(wl)
        # rows see at most N keys by the host bound; one row claims 7 more
        wl.tok_vis[2] = SPEC.N + 7
        step.indexer()
        step.topk()
        torch.cuda.synchronize()
        flag = dsa.dsa_check_debug_flag()
        assert flag & dsa.DEBUG_VIS_CLAMPED, f"flag {flag}"
        assert int(step.count[2]) == min(SPEC.k, SPEC.N)


def test_row_without_a_request_is_noted_and_reads_nothing(gpu):
    print("[gpu] debug library: request id outside the batch", flush=True)
    with debug_library():
        dsa.dsa_check_debug_flag()
        wl = synth.make_workload(SPEC, device=gpu)
        step = gpu_step(wl)
        wl.tok_req[1] = SPEC.R + 3
        out, lse = step()
        flag = dsa.dsa_check_debug_flag()
        assert flag & dsa.DEBUG_REQ_OUTSIDE, f"flag {flag}"
        rows = step.rows.cpu().numpy()
        assert np.all(rows[1] == -1)
        assert np.all(out[1].cpu().numpy() == 0) and np.all(np.isneginf(lse[1].cpu().numpy()))
        assert np.all(rows[0, : int(step.count[0])] >= 0)
