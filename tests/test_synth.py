"""The seeded generators write what they claim: encoders round-trip through the
oracle's independent decoders with round-to-nearest-even, scales never encode
NaN, and workloads have the advertised shapes and page structure."""
import numpy as np
import torch

import synth
from oracle import codecs as OC
from synth import codecs as SC


def _nearest_even(x, table, mant_bit_of):
    """Brute-force RNE onto a finite value table (index = code)."""
    fin = [(c, v) for c, v in enumerate(table) if np.isfinite(v)]
    out = []
    for xv in x:
        best = min(abs(v - xv) for _, v in fin)
        cands = [c for c, v in fin if abs(v - xv) == best]
        cands.sort(key=lambda c: (mant_bit_of(c), c & 0x80 != 0 if table is OC.E4M3_TABLE else c & 8 != 0))
        out.append(table[cands[0]])
    return np.array(out)


def test_e4m3_encoder_round_trips_every_code():
    vals = torch.tensor(OC.E4M3_TABLE[np.isfinite(OC.E4M3_TABLE)], dtype=torch.float32)
    codes = SC.e4m3_encode(vals).numpy()
    assert np.array_equal(OC.e4m3(codes), vals.numpy().astype(np.float64))


def test_e4m3_encoder_is_rne_and_saturating():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(3000) * 30, [448, 460, 500, -1e6, 1e-7, -3e-3]])
    got = OC.e4m3(SC.e4m3_encode(torch.tensor(x, dtype=torch.float32)).numpy())
    xc = np.clip(x.astype(np.float32).astype(np.float64), -448, 448)
    ref = _nearest_even(xc, OC.E4M3_TABLE, lambda c: c & 1)
    assert np.array_equal(np.abs(got), np.abs(ref))


def test_e2m1_encoder_is_rne_and_saturating():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x = np.concatenate([np.random.default_rng(2).uniform(-8, 8, 4000), mids, [-m for m in mids], [7.0, -100.0]])
    nib = SC.e2m1_encode_nibbles(torch.tensor(x, dtype=torch.float32)).numpy()
    got = OC.E2M1_TABLE[nib]
    ref = _nearest_even(np.clip(x, -6, 6), OC.E2M1_TABLE, lambda c: c & 1)
    assert np.array_equal(got, ref)
    # exact midpoints go to the even mantissa
    assert OC.E2M1_TABLE[SC.e2m1_encode_nibbles(torch.tensor(mids)).numpy()].tolist() == [0, 1, 1, 2, 2, 4, 4]


def test_mxfp4_blocks_bound_and_scales():
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(3)) * 5
    x[0] = 0
    codes, e8 = SC.mxfp4_blocks(x, 32)
    assert int(e8.max()) < 255
    deq = OC.e2m1_packed(codes.numpy()) * np.repeat(OC.e8m0(e8.numpy()), 32, axis=-1)
    X = np.repeat(e8.numpy().astype(np.int64) - 127, 32, axis=-1)
    assert np.all(np.abs(deq - x.numpy()) <= 2.0 ** (X + 1))
    assert np.all(deq[0] == 0)


def test_nvfp4_blocks_bound():
    x = torch.randn(64, 512, generator=torch.Generator().manual_seed(4))
    codes, sc = SC.nvfp4_blocks(x, 16)
    s = np.repeat(OC.e4m3(sc.numpy()), 16, axis=-1)
    assert np.all(np.isfinite(s))
    deq = OC.e2m1_packed(codes.numpy()) * s
    assert np.all(np.abs(deq - x.numpy()) <= 1.0 * s + 1e-12)


def test_fp8_rowwise_scale_is_amax_over_448():
    x = torch.randn(10, 128, generator=torch.Generator().manual_seed(5))
    codes, scale = SC.fp8_rowwise(x)
    assert torch.allclose(scale, x.abs().amax(-1) / 448)
    deq = OC.e4m3(codes.numpy()) * scale.numpy()[:, None]
    assert np.all(np.abs(deq - x.numpy()) <= 2 ** -4 * np.abs(x.numpy()) + scale.numpy()[:, None] * 2 ** -10)


def test_workload_structure():
    spec = synth.CONFIGS["tp8_spec_decode_64k"].replace(R=3, N=1000)
    wl = synth.make_workload(spec)
    assert wl.T == 18 and wl.P == 64 and wl.num_pages == 3 * 16
    assert wl.key_pool.shape == (48, 64 * 132) and wl.lat_pool.shape == (48, 64 * 640)
    assert sorted(wl.block_table.flatten().tolist()) == list(range(48))
    assert wl.tok_vis.tolist() == [995, 996, 997, 998, 999, 1000] * 3
    assert wl.q_mla.shape == (18, 12, 576) and wl.q_mla.dtype == torch.bfloat16
    c1 = synth.make_workload(synth.CONFIGS["tiny_decode_8k"])
    assert c1.block_table is None and c1.P == 8192 and c1.lat_pool.shape == (1, 8192 * 1152)


def test_same_seed_same_bytes():
    spec = synth.CONFIGS["fp4_decode_256k"].replace(R=2, N=700)
    a, b = synth.make_workload(spec), synth.make_workload(spec)
    assert torch.equal(a.key_pool, b.key_pool) and torch.equal(a.lat_pool, b.lat_pool)
    assert torch.equal(a.q_idx, b.q_idx) and torch.equal(a.block_table, b.block_table)
