"""Test-side glue: turn a synthetic workload (torch tensors) into the plain
NumPy inputs the oracle reads."""
from __future__ import annotations

import numpy as np
import torch


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def oracle_inputs(wl) -> dict:
    s = wl.spec
    q_idx = wl.q_idx
    if q_idx.dtype == torch.bfloat16:
        q_idx = q_idx.view(torch.int16)
    return {
        "P": wl.P,
        "key_fmt": s.key_fmt,
        "lat_fmt": s.lat_fmt,
        "q_fmt": s.q_fmt,
        "sm_scale": s.sm_scale,
        "req_token_start": _np(wl.req_token_start).astype(np.int64),
        "tok_vis": _np(wl.tok_vis).astype(np.int64),
        "block_table": None if wl.block_table is None else _np(wl.block_table).astype(np.int64),
        "key_pool": _np(wl.key_pool),
        "lat_pool": _np(wl.lat_pool),
        "q_idx": _np(q_idx),
        "q_idx_scale": _np(wl.q_idx_scale),
        "w": _np(wl.w).astype(np.float64),
        "q_mla": _np(wl.q_mla.view(torch.int16)),
    }


def gpu_step(wl, k=None, prefill=False, num_splits=0):
    """libdsa DecodeStep over a synthetic workload that lives on the GPU."""
    import sparse_attention_03_amd as dsa
    s = wl.spec
    return dsa.make_step(key_pool=wl.key_pool, lat_pool=wl.lat_pool, page_size=wl.P,
                         key_fmt=s.key_fmt, lat_fmt=s.lat_fmt, req_row_start=wl.req_token_start,
                         tok_req=wl.tok_req, tok_vis=wl.tok_vis, block_table=wl.block_table,
                         q_idx=wl.q_idx, w=wl.w, q_mla=wl.q_mla, k=k or s.k, sm_scale=s.sm_scale,
                         q_idx_scale=wl.q_idx_scale, prefill=prefill, num_splits=num_splits,
                         max_vis=s.N, max_rows_per_req=s.q_per_req)


def quantised_q_score_tolerance(inp, t, keys):
    """Per-element bound on the error of a GPU score computed from a quantised
    (FP8 or MXFP4) index query on the low-precision matrix instructions.

    Every product of two quantised values is exact in fp32; what the
    instruction does not document is the order and width of its internal
    additions.  Whatever they are, an fp32 sum of n terms in any order, with
    each addition rounded or truncated (unit 2^-23), is off by at most about
    n * 2^-23 * sum|terms| (the classical worst-case summation bound).  A score
    adds 128 products per head, then 32 weighted heads and a scale: n = 160
    covers them.  Returns [n_keys] bounds for query row t over `keys` [n, 128]
    (the dequantised keys, the key scale included)."""
    import numpy as np
    from oracle import dsa as O
    q = np.abs(O.dequant_q_idx(inp, t))                 # [32, 128]
    w = np.abs(np.asarray(inp["w"][t], np.float64))     # [32]
    terms = (np.abs(keys) @ q.T) @ w                    # sum_h |w_h| sum_i |q_hi k_i|
    return 160 * 2.0 ** -23 * terms


def assert_scores_close(got, ref, inp, t, keys=None, what=""):
    """GPU scores of row t against the oracle's: -inf (a token on an absent
    page) exactly where the oracle has it; elsewhere within 1e-5 x the row's
    largest |score| for BF16 queries (exact products, fp32 sums of 4096
    terms), or within the per-element bound of quantised_q_score_tolerance
    for FP8 / MXFP4 queries.  `keys`: the request's dequantised keys [>= n,
    128] (looked up when None and needed)."""
    import numpy as np
    from oracle import dsa as O
    got = np.asarray(got, np.float64)
    n = ref.shape[0]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what} row {t}: -inf pattern differs"
    assert np.all(got[~fin] == -np.inf) and np.all(ref[~fin] == -np.inf)
    if not fin.any():
        return
    err = np.abs(got[fin] - ref[fin])
    if inp["q_fmt"] == "bf16":
        tol = 1e-5 * np.abs(ref[fin]).max()
    else:
        if keys is None:
            rts = np.asarray(inp["req_token_start"])
            r = int(np.searchsorted(rts, t, side="right") - 1)
            keys = O.request_keys(inp["key_pool"], inp["key_fmt"], inp["P"], inp["block_table"], r, n)
        tol = quantised_q_score_tolerance(inp, t, keys[:n])[fin]
    bad = err > tol
    assert not bad.any(), f"{what} row {t}: score err {err[bad].max()} above its bound"
