"""Seeded synthetic inputs for one DSA layer, laid out in the paged-cache
format the kernels read.

Nothing here computes any step of DSA (no scoring, selection or attention):
it draws random values, quantises them with ``synth.codecs`` and writes the
bytes into pages.  Both the oracle and the HIP path consume exactly these
bytes.

Workload shapes follow the pages' settings: 32 indexer heads x 128 dims and
top-2048 (Kimi K3.1 Pro day-0 page, "Sparse attention in K3.1 Pro"); 576-byte
FP8 / 352-byte NVFP4 latents and 132-byte FP8 / 68-byte MXFP4 index keys ("One
KV cache, three states"); 12 TP8 heads padded to 16 ("Prefill: shard attention
by token"; MI355X Kimi K3 page, section 4 "MLA"); speculative verify rows that
share keys (AMD section "native MXFP4 indexer").

Page layout.  Index keys are streamed page by page, so their pages are
structure-of-arrays (every region 16-byte aligned for P a multiple of 4):

  key  FP8     [P x 128 E4M3 codes][P x fp32 scale]                 132 B/token
  key  MXFP4   [P x 64 B packed E2M1][P x 4 E8M0 (one per 32)]        68 B/token
  key  NVFP4   [P x 64 B packed E2M1][P x 8 E4M3 (one per 16)]        72 B/token

Latent rows are gathered one by one, so a latent page is P rows, each padded
to a whole number of 128-byte lines with all of the row's bytes inside it:

  lat  BF16    row 1152 B: [576 bf16]                               1152 B/token
  lat  FP8     row  640 B: [576 E4M3 codes][fp32 scale][60 B pad]    580 B/token
  lat  NVFP4   row  384 B: [256 B packed E2M1 (dims 0..511)]
                           [32 E4M3 block scales (one per 16 dims)]
                           [64 E4M3 rope dims 512..575, unscaled]
                           [32 B pad]                                352 B/token

Keys and latents of a token sit in the pages with the same physical id.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

from . import codecs

HI = 32          # indexer heads
DI = 128         # indexer dims
D_LAT = 576      # latent dims (512 nope + 64 rope)
D_V = 512        # value dims
TOPK = 2048

KEY_FP8, KEY_MXFP4, KEY_NVFP4 = "fp8", "mxfp4", "nvfp4"
LAT_BF16, LAT_FP8, LAT_NVFP4 = "bf16", "fp8", "nvfp4"
Q_BF16, Q_FP8, Q_MXFP4 = "bf16", "fp8", "mxfp4"

KEY_TOKEN_BYTES = {KEY_FP8: 132, KEY_MXFP4: 68, KEY_NVFP4: 72}
LAT_TOKEN_BYTES = {LAT_BF16: 1152, LAT_FP8: 580, LAT_NVFP4: 352}   # data bytes per token
LAT_ROW_STRIDE = {LAT_BF16: 1152, LAT_FP8: 640, LAT_NVFP4: 384}    # bytes per row in a page


def key_regions(fmt: str, P: int):
    """(codes offset, codes bytes/token, scales offset, scale bytes/token)."""
    if fmt == KEY_FP8:
        return 0, 128, 128 * P, 4
    if fmt == KEY_MXFP4:
        return 0, 64, 64 * P, 4
    if fmt == KEY_NVFP4:
        return 0, 64, 64 * P, 8
    raise ValueError(fmt)


def lat_fields(fmt: str):
    """Byte offsets inside a latent row: (codes, scales, rope)."""
    if fmt == LAT_BF16:
        return 0, None, None
    if fmt == LAT_FP8:
        return 0, 576, None
    if fmt == LAT_NVFP4:
        return 0, 256, 288
    raise ValueError(fmt)


@dataclasses.dataclass
class Spec:
    name: str
    R: int                      # requests
    q_per_req: int              # query tokens per request
    N: int                      # context length (tokens visible to the last query row)
    page: int = 64              # tokens per page; 0 = non-paged (one page per request)
    key_fmt: str = KEY_FP8
    lat_fmt: str = LAT_FP8
    q_fmt: str = Q_BF16
    H: int = 16                 # real MLA heads
    k: int = TOPK
    causal_rows: bool = True    # row j of a request sees N - (q_per_req-1) + j tokens
    lat_std: float = 1.0        # std of latent values before quantisation
    plant_gap: bool = False     # plant a score gap at rank k (per query row)
    w_signed: bool = False      # head weights U(-1, 1) instead of U(0, 1)
    sm_scale: float = 1.0 / math.sqrt(192.0)
    seed: int = 0

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The five reference workloads (sizes as the pages' serving settings give them).
CONFIGS = {
    "tiny_decode_8k": Spec("tiny_decode_8k", R=1, q_per_req=1, N=8192, page=0,
                           key_fmt=KEY_FP8, lat_fmt=LAT_BF16, H=16,
                           lat_std=1.0 / math.sqrt(576.0), seed=1001),
    "tp8_spec_decode_64k": Spec("tp8_spec_decode_64k", R=32, q_per_req=6, N=65536,
                                page=64, key_fmt=KEY_FP8, lat_fmt=LAT_FP8, H=12,
                                seed=1002),
    "long_decode_1m": Spec("long_decode_1m", R=4, q_per_req=1, N=1 << 20, page=64,
                           key_fmt=KEY_FP8, lat_fmt=LAT_FP8, H=96, plant_gap=True,
                           seed=1003),
    "prefill_chunk_32k": Spec("prefill_chunk_32k", R=1, q_per_req=4096, N=32768,
                              page=64, key_fmt=KEY_FP8, lat_fmt=LAT_FP8,
                              q_fmt=Q_FP8, H=96, seed=1004),
    "fp4_decode_256k": Spec("fp4_decode_256k", R=64, q_per_req=1, N=262144, page=64,
                            key_fmt=KEY_MXFP4, lat_fmt=LAT_NVFP4, H=12, seed=1005),
}


@dataclasses.dataclass
class Workload:
    spec: Spec
    P: int                              # tokens per page (power of two)
    num_pages: int
    req_token_start: torch.Tensor       # int32 [R+1]
    tok_req: torch.Tensor               # int32 [T]
    tok_vis: torch.Tensor               # int32 [T]
    block_table: Optional[torch.Tensor] # int32 [R, pages_per_req] or None (non-paged)
    key_pool: torch.Tensor              # uint8 [num_pages, P*key_bytes]
    lat_pool: torch.Tensor              # uint8 [num_pages, P*lat_row_stride]
    q_idx: torch.Tensor                 # bf16 [T,32,128], uint8 E4M3 codes, or uint8 E2M1 pairs [T,32,64]
    q_idx_scale: Optional[torch.Tensor] # fp32 [T,32] (FP8 q), uint8 E8M0 [T,32,4] (MXFP4 q)
    w: torch.Tensor                     # fp32 [T,32]
    q_mla: torch.Tensor                 # bf16 [T,H,576]
    hot: Optional[torch.Tensor]         # int64 [T, k] planted top-k sets (sorted), or None

    @property
    def T(self) -> int:
        return int(self.tok_vis.numel())

    @property
    def R(self) -> int:
        return self.spec.R


def _next_pow2(n: int) -> int:
    return 1 << max(0, (n - 1).bit_length())


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _write_key_rows(pool, fmt, P, phys_pages, vals):
    """Quantise vals [n,128] (n = len(phys_pages)*P or less) into pages."""
    n = vals.shape[0]
    npg = (n + P - 1) // P
    if n < npg * P:
        vals = torch.cat([vals, vals.new_zeros(npg * P - n, vals.shape[1])])
    vals = vals.reshape(npg, P, DI)
    c_off, c_b, s_off, s_b = key_regions(fmt, P)
    if fmt == KEY_FP8:
        codes, scale = codecs.fp8_rowwise(vals)
        pool[phys_pages, c_off:c_off + P * c_b] = codes.reshape(npg, P * c_b)
        pool[phys_pages, s_off:s_off + P * s_b] = scale.contiguous().view(torch.uint8).reshape(npg, P * s_b)
    elif fmt == KEY_MXFP4:
        codes, e8 = codecs.mxfp4_blocks(vals, 32)
        pool[phys_pages, c_off:c_off + P * c_b] = codes.reshape(npg, P * c_b)
        pool[phys_pages, s_off:s_off + P * s_b] = e8.reshape(npg, P * s_b)
    else:
        codes, sc = codecs.nvfp4_blocks(vals, 16)
        pool[phys_pages, c_off:c_off + P * c_b] = codes.reshape(npg, P * c_b)
        pool[phys_pages, s_off:s_off + P * s_b] = sc.reshape(npg, P * s_b)


def _write_lat_rows(pool, fmt, P, phys_pages, vals):
    n = vals.shape[0]
    npg = (n + P - 1) // P
    if n < npg * P:
        vals = torch.cat([vals, vals.new_zeros(npg * P - n, vals.shape[1])])
    vals = vals.reshape(npg, P, D_LAT)
    stride = LAT_ROW_STRIDE[fmt]
    c_off, s_off, r_off = lat_fields(fmt)
    rows = torch.zeros(npg, P, stride, dtype=torch.uint8, device=pool.device)
    if fmt == LAT_BF16:
        rows[:] = codecs.bf16_bits(vals).contiguous().view(torch.uint8).reshape(npg, P, 1152)
    elif fmt == LAT_FP8:
        codes, scale = codecs.fp8_rowwise(vals)
        rows[..., c_off:c_off + 576] = codes
        rows[..., s_off:s_off + 4] = scale.contiguous().view(torch.uint8).reshape(npg, P, 4)
    else:
        codes, sc = codecs.nvfp4_blocks(vals[..., :D_V], 16)
        rope = codecs.e4m3_encode(vals[..., D_V:])
        rows[..., c_off:c_off + 256] = codes
        rows[..., s_off:s_off + 32] = sc
        rows[..., r_off:r_off + 64] = rope
    pool[phys_pages, :] = rows.reshape(npg, P * stride)


def make_workload(spec: Spec, device="cpu", seed: Optional[int] = None) -> Workload:
    """Draw one workload.  Draw order: q_idx, w, q_mla, planted sets, then per
    request key values and latent values; the block-table permutation comes
    from its own seeded stream so paged and non-paged variants of one spec hold
    the same values."""
    seed = spec.seed if seed is None else seed
    g = _gen(device, seed)
    R, Tq, N, k = spec.R, spec.q_per_req, spec.N, spec.k
    T = R * Tq
    if spec.page == 0:
        P = _next_pow2(N)
        pages_per_req = 1
    else:
        P = spec.page
        assert P & (P - 1) == 0
        pages_per_req = (N + P - 1) // P
    num_pages = R * pages_per_req

    # token metadata
    rts = torch.arange(0, T + 1, Tq, dtype=torch.int32)
    tok_req = torch.arange(R, dtype=torch.int32).repeat_interleave(Tq)
    j = torch.arange(Tq, dtype=torch.int32).repeat(R)
    if spec.causal_rows:
        tok_vis = N - (Tq - 1) + j
    else:
        tok_vis = torch.full((T,), N, dtype=torch.int32)
    assert int(tok_vis.min()) >= 1

    # physical pages: random permutation (paged) or identity (non-paged)
    if spec.page == 0:
        block_table = None
        phys = torch.arange(R, dtype=torch.int64).reshape(R, 1)
    else:
        # separate stream: the values do not depend on whether the cache is paged
        perm = torch.randperm(num_pages, generator=_gen(device, seed ^ 0x5A5A5A), device=device).cpu()
        phys = perm.reshape(R, pages_per_req)
        block_table = phys.to(torch.int32)

    # queries and head weights
    qf = torch.randn(T, HI, DI, generator=g, device=device)
    if spec.q_fmt == Q_BF16:
        q_idx = codecs.bf16_bits(qf)
        q_idx_scale = None
        q_eff = q_idx.float()
    elif spec.q_fmt == Q_FP8:
        q_idx, q_idx_scale = codecs.fp8_rowwise(qf)
        q_eff = codecs.e4m3_value(q_idx) * q_idx_scale.unsqueeze(-1)
    else:
        # MXFP4 query (E2M1 pairs + E8M0 per 32 dims); the planting direction
        # only needs an approximation of the query, so the BF16 values serve
        q_idx, q_idx_scale = codecs.mxfp4_blocks(qf, 32)
        q_eff = codecs.bf16_bits(qf).float()
    w = torch.rand(T, HI, generator=g, device=device)
    if spec.w_signed:
        w = 2.0 * w - 1.0
    q_mla = codecs.bf16_bits(torch.randn(T, spec.H, D_LAT, generator=g, device=device))

    # planted sets: row t gets its own k keys (disjoint within a request),
    # all visible to every row of the request
    hot = None
    if spec.plant_gap:
        vis_min = N - (Tq - 1) if spec.causal_rows else N
        assert Tq * k <= vis_min, "cannot plant disjoint sets"
        hot_rows = []
        for r in range(R):
            pick = torch.randperm(vis_min, generator=g, device=device)[: Tq * k]
            hot_rows.append(pick.reshape(Tq, k))
        hot = torch.sort(torch.cat(hot_rows), dim=1).values

    key_pool = torch.zeros(num_pages, P * KEY_TOKEN_BYTES[spec.key_fmt], dtype=torch.uint8, device=device)
    lat_pool = torch.zeros(num_pages, P * LAT_ROW_STRIDE[spec.lat_fmt], dtype=torch.uint8, device=device)
    phys_d = phys.to(device)
    for r in range(R):
        kv = torch.randn(N, DI, generator=g, device=device)
        if hot is not None:
            # A planted key points along u = sum_h w_h q_h of its row, with a
            # random length in [1, 1.5) x sqrt(128) plus small noise.
            for jj in range(Tq):
                t = r * Tq + jj
                u = (w[t].unsqueeze(-1) * q_eff[t]).sum(0)
                u = u / u.norm()
                ln = math.sqrt(DI) * (1.0 + 0.5 * torch.rand(k, 1, generator=g, device=device))
                kv[hot[t]] = ln * u + 0.05 * torch.randn(k, DI, generator=g, device=device)
        _write_key_rows(key_pool, spec.key_fmt, P, phys_d[r], kv)
        del kv
        lv = spec.lat_std * torch.randn(N, D_LAT, generator=g, device=device)
        _write_lat_rows(lat_pool, spec.lat_fmt, P, phys_d[r], lv)
        del lv

    dev = torch.device(device)
    return Workload(spec=spec, P=P, num_pages=num_pages,
                    req_token_start=rts.to(dev), tok_req=tok_req.to(dev),
                    tok_vis=tok_vis.to(dev),
                    block_table=None if block_table is None else block_table.to(dev),
                    key_pool=key_pool, lat_pool=lat_pool, q_idx=q_idx,
                    q_idx_scale=q_idx_scale, w=w, q_mla=q_mla, hot=hot)


def random_rows(wl: Workload, k: int, seed: int = 7, device=None):
    """Seeded selection lists for testing attention on its own: for query row
    t, min(k, vis_t) distinct physical rows drawn uniformly from the whole
    latent pool (ascending, -1 padded)."""
    device = wl.tok_vis.device if device is None else device
    g = _gen("cpu", seed)
    T = wl.T
    total = wl.num_pages * wl.P
    rows = torch.full((T, k), -1, dtype=torch.int32)
    vis = wl.tok_vis.cpu()
    for t in range(T):
        m = min(k, int(vis[t]), total)
        pick = torch.randperm(total, generator=g)[:m]
        rows[t, :m] = torch.sort(pick).values.to(torch.int32)
    return rows.to(device)


def random_logical(wl: Workload, k: int, seed: int = 11, device=None):
    """Seeded logical index lists (ascending, -1 padded): min(k, vis_t)
    distinct positions below vis_t for each query row."""
    device = wl.tok_vis.device if device is None else device
    g = _gen("cpu", seed)
    idx = torch.full((wl.T, k), -1, dtype=torch.int32)
    vis = wl.tok_vis.cpu()
    for t in range(wl.T):
        n = int(vis[t])
        m = min(k, n)
        idx[t, :m] = torch.sort(torch.randperm(n, generator=g)[:m]).values.to(torch.int32)
    return idx.to(device)


def mark_absent(wl: Workload, n_entries: int, seed: int = 5):
    """Seeded damage to the block table for tests of absent pages: n_entries
    distinct (request, logical page) entries are set, alternately, to -1 and
    to num_pages + j (outside the pool).  Returns the new block table (int32,
    on the workload's device) and the list of (request, logical page) hit."""
    assert wl.block_table is not None
    g = _gen("cpu", seed)
    bt = wl.block_table.cpu().clone()
    R, npg = bt.shape
    pick = torch.randperm(R * npg, generator=g)[:n_entries]
    hit = []
    for j, e in enumerate(pick.tolist()):
        r, lp = divmod(e, npg)
        bt[r, lp] = -1 if j % 2 == 0 else wl.num_pages + j
        hit.append((r, lp))
    return bt.to(wl.block_table.device), hit
