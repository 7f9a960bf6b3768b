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
