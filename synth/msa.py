"""Seeded synthetic inputs for the MSA block-sparse decode step (MiniMax M3.1
page, "MSA primer"): 128-token blocks, FP8 index keys of one shared head
(128 bytes per token), FP8 K and V of Hkv heads (2 * Hkv * 128 bytes per
token), one BF16 index query per GQA group and BF16 query heads.

Only encoding (value -> code) happens here; decoding belongs to the oracle and
to the kernels.  Optionally a planted gap: for every (row, group), 15 random
earlier blocks get one key along the group's index query, far above every
other score, so the block selection is checkable bit for bit.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import codecs

BLOCK = 128
DIM = 128


@dataclass
class MsaSpec:
    name: str
    R: int                 # requests
    rows: int              # query rows per request (row j sees N - rows + 1 + j tokens)
    N: int                 # context length of every request
    hkv: int = 4           # KV heads = GQA groups = index queries per row
    hq: int = 64           # query heads
    top_blocks: int = 16
    k_scale: float = 0.5
    v_scale: float = 0.25
    planted: bool = False
    seed: int = 2001

    def replace(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return MsaSpec(**d)


MSA_CONFIGS = {
    "msa_decode_128k": MsaSpec("msa_decode_128k", R=32, rows=1, N=131072),
}


def make_inputs(spec: MsaSpec, device="cpu") -> dict:
    """Tensors on `device` (codes uint8, queries bf16, indices int32)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(spec.seed)
    R, rows, N, hkv, hq = spec.R, spec.rows, spec.N, spec.hkv, spec.hq
    T = R * rows
    nb = -(-N // BLOCK)
    pool_blocks = R * nb
    perm = torch.randperm(pool_blocks, generator=g).to(torch.int32)
    block_table = perm.view(R, nb)
    tok_req = torch.arange(R, dtype=torch.int32).repeat_interleave(rows)
    tok_vis = torch.tensor([N - rows + 1 + j for _ in range(R) for j in range(rows)], dtype=torch.int32)
    req_row_start = torch.arange(0, T + 1, rows, dtype=torch.int32)
    q_idx = torch.randn(T, hkv, DIM, generator=g)
    q = torch.randn(T, hq, DIM, generator=g)
    idx_vals = torch.randn(pool_blocks * BLOCK, DIM, generator=g)
    if spec.planted:
        # one key per planted block along the group's index query (|q|-scaled,
        # length 4 sqrt(128) before FP8 rounding): scores ~ 4 * 128 * |q|
        for t in range(T):
            r, vis = int(tok_req[t]), int(tok_vis[t])
            last = (vis - 1) // BLOCK
            for gg in range(hkv):
                cand = torch.randperm(last, generator=g)[:spec.top_blocks - 1]
                u = q_idx[t, gg] / q_idx[t, gg].norm()
                for b in cand.tolist():
                    slot = int(torch.randint(0, BLOCK, (1,), generator=g))
                    tok = int(block_table[r, b]) * BLOCK + slot
                    idx_vals[tok] = 4.0 * (DIM ** 0.5) * u
    idx_pool = codecs.e4m3_encode(idx_vals).view(pool_blocks, BLOCK * DIM)
    kv_vals = torch.randn(pool_blocks * BLOCK, 2, hkv, DIM, generator=g) * 2.0
    kv_pool = codecs.e4m3_encode(kv_vals).view(pool_blocks, BLOCK * 2 * hkv * DIM)
    out = dict(block_table=block_table, tok_req=tok_req, tok_vis=tok_vis, req_row_start=req_row_start,
               q_idx=codecs.bf16_bits(q_idx), q=codecs.bf16_bits(q), idx_pool=idx_pool, kv_pool=kv_pool)
    return {k: v.to(device) for k, v in out.items()}


def oracle_view(inp: dict, spec: MsaSpec) -> dict:
    """NumPy copies in the oracle's terms (queries as float64 of their bf16
    values, codes as uint8)."""
    d = {k: v.cpu() for k, v in inp.items()}
    return dict(block_table=d["block_table"].numpy().astype(np.int64), tok_req=d["tok_req"].numpy(),
                tok_vis=d["tok_vis"].numpy(), q_idx=d["q_idx"].float().numpy().astype(np.float64),
                q=d["q"].float().numpy().astype(np.float64), idx_pool=d["idx_pool"].numpy(),
                kv_pool=d["kv_pool"].numpy(), hkv=spec.hkv, hq=spec.hq, top_blocks=spec.top_blocks,
                k_scale=spec.k_scale, v_scale=spec.v_scale, sm_scale=1.0 / DIM ** 0.5)
