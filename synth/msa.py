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
    """Tensors on `device` (codes uint8, queries bf16, indices int32).  The
    pools are drawn in chunks of blocks on `device` (seed, chunk) so that a
    full-size cache never exists in fp32."""
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
    q_idx = codecs.bf16_bits(torch.randn(T, hkv, DIM, generator=g))
    q = codecs.bf16_bits(torch.randn(T, hq, DIM, generator=g))
    idx_pool = torch.empty(pool_blocks, BLOCK * DIM, dtype=torch.uint8, device=device)
    kv_pool = torch.empty(pool_blocks, BLOCK * 2 * hkv * DIM, dtype=torch.uint8, device=device)
    gd = torch.Generator(device=device)
    chunk = 256
    for i, b0 in enumerate(range(0, pool_blocks, chunk)):
        b1 = min(pool_blocks, b0 + chunk)
        gd.manual_seed(spec.seed * 1000 + i)
        iv = torch.randn((b1 - b0) * BLOCK, DIM, generator=gd, device=device)
        idx_pool[b0:b1] = codecs.e4m3_encode(iv).view(b1 - b0, BLOCK * DIM)
        kv = torch.randn((b1 - b0) * BLOCK, 2 * hkv * DIM, generator=gd, device=device) * 2.0
        kv_pool[b0:b1] = codecs.e4m3_encode(kv).view(b1 - b0, BLOCK * 2 * hkv * DIM)
    if spec.planted:
        # for every (row, group): one key in each of top_blocks - 1 random
        # earlier blocks along the group's index query, length 4 sqrt(128)
        # before FP8 rounding, so its score (~ 4 sqrt(128) |q|) dwarfs the rest
        qf = q_idx.float()
        for t in range(T):
            r, vis = int(tok_req[t]), int(tok_vis[t])
            last = (vis - 1) // BLOCK
            for gg in range(hkv):
                cand = torch.randperm(last, generator=g)[:spec.top_blocks - 1]
                u = qf[t, gg] / qf[t, gg].norm()
                code = codecs.e4m3_encode(4.0 * (DIM ** 0.5) * u).to(device)
                for bb in cand.tolist():
                    slot = int(torch.randint(0, BLOCK, (1,), generator=g))
                    page = int(block_table[r, bb])
                    idx_pool[page, slot * DIM:(slot + 1) * DIM] = code
    out = dict(block_table=block_table, tok_req=tok_req, tok_vis=tok_vis, req_row_start=req_row_start,
               q_idx=q_idx, q=q)
    out = {k: v.to(device) for k, v in out.items()}
    out.update(idx_pool=idx_pool, kv_pool=kv_pool)
    return out


def oracle_view(inp: dict, spec: MsaSpec) -> dict:
    """NumPy copies in the oracle's terms (queries as float64 of their bf16
    values, codes as uint8)."""
    d = {k: v.cpu() for k, v in inp.items()}
    return dict(block_table=d["block_table"].numpy().astype(np.int64), tok_req=d["tok_req"].numpy(),
                tok_vis=d["tok_vis"].numpy(), q_idx=d["q_idx"].float().numpy().astype(np.float64),
                q=d["q"].float().numpy().astype(np.float64), idx_pool=d["idx_pool"].numpy(),
                kv_pool=d["kv_pool"].numpy(), hkv=spec.hkv, hq=spec.hq, top_blocks=spec.top_blocks,
                k_scale=spec.k_scale, v_scale=spec.v_scale, sm_scale=1.0 / DIM ** 0.5)
