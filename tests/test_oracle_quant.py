"""Pins for the oracle's front-end quantisers (CPU only).

  e4m3_encode   -> every finite code round-trips through the (pinned) decoder;
                   torch's float8_e4m3fn conversion (nearest even) on random
                   values and on every midpoint; saturation at 448
  e2m1_encode   -> the eight magnitudes round-trip; every midpoint goes to the
                   even code; saturation at 6
  fp8_row       -> the row maximum lands on +-448; all-zero rows; error bound
  mx_e8m0       -> the exponent rule on closed-form block maxima
  nvfp4_blocks  -> unit scale for a block maximum of 6; zero blocks
  quantize_q    -> folded weights give the same scores (ReLU homogeneity)
  cache_insert  -> the inserted bytes decode, through the pinned page decoders
                   of oracle.dsa, to the quantised values at (page, slot);
                   bytes elsewhere and skipped tokens are untouched
"""
import numpy as np
import pytest
import torch

from oracle import codecs as OC, dsa as O, quant as Q


def _finite_e4m3_codes():
    return [c for c in range(256) if c not in (0x7F, 0xFF, 0x80)]


def test_e4m3_encode_round_trips_every_code():
    codes = np.array(_finite_e4m3_codes(), np.uint8)
    vals = OC.e4m3(codes).astype(np.float32)
    assert np.array_equal(Q.e4m3_encode(vals), codes)
    assert np.array_equal(Q.e4m3_value(codes).astype(np.float64), OC.e4m3(codes))


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    c = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    c[c == 0x80] = 0  # a zero result is stored as +0
    return c


def test_e4m3_encode_matches_torch_and_ties_go_to_even():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * 50, g.standard_normal(20000) * 2e-3,
                        g.uniform(-448, 448, 20000)]).astype(np.float32)
    assert np.array_equal(Q.e4m3_encode(x), _torch_e4m3(x))
    # midpoints between neighbouring codes of one sign: ties to the even code
    pos = np.array([c for c in range(0x7F)], np.int64)  # 0 .. 0x7E
    v = OC.e4m3(pos.astype(np.uint8))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)  # exact in fp32
    want = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:]).astype(np.uint8)
    assert np.array_equal(Q.e4m3_encode(mids), want)
    assert np.array_equal(Q.e4m3_encode(-mids), np.where(want == 0, 0, want | 0x80).astype(np.uint8))
    assert np.array_equal(Q.e4m3_encode(mids), _torch_e4m3(mids))


def test_e4m3_encode_saturates_and_zero_is_positive():
    x = np.array([448, 449, 479.9, 480, 1e30, -500, -1e30, 0.0, -0.0, -1e-9], np.float32)
    assert Q.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0, 0, 0]


def test_e2m1_encode_round_trip_ties_saturation():
    mags = Q.E2M1_MAGS
    assert Q.e2m1_encode(mags.astype(np.float32)).tolist() == list(range(8))
    assert Q.e2m1_encode(-mags[1:].astype(np.float32)).tolist() == [8 + c for c in range(1, 8)]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    # the even code of each pair: 0 | 2 | 2 | 4 | 4 | 6 | 6
    assert Q.e2m1_encode(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]
    eps = np.float32(1e-3)
    assert Q.e2m1_encode(mids + eps).tolist() == [1, 2, 3, 4, 5, 6, 7]
    assert Q.e2m1_encode(mids - eps).tolist() == [0, 1, 2, 3, 4, 5, 6]
    assert Q.e2m1_encode(np.array([6.0, 7.0, 1e9, -100.0, -0.0, -0.2], np.float32)).tolist() == [7, 7, 7, 15, 0, 0]
    # against the pinned decoder table
    nib = Q.e2m1_encode(np.linspace(-7, 7, 2801).astype(np.float32))
    back = np.array([OC.E2M1_TABLE[c] for c in nib])
    grid = np.concatenate([-mags[::-1], mags])
    x = np.linspace(-7, 7, 2801)
    xs = np.clip(x, -6, 6)
    assert np.all(np.abs(back - xs) <= np.min(np.abs(grid[None, :] - xs[:, None]), axis=1) + 1e-12)


def test_fp8_row_maps_the_maximum_to_448():
    g = np.random.default_rng(1)
    x = (g.standard_normal((500, 128)) * np.exp(g.uniform(-8, 8, (500, 1)))).astype(np.float32)
    codes, scale = Q.fp8_row(x)
    assert scale.dtype == np.float32
    assert np.array_equal(scale, (np.abs(x).max(1) / np.float32(448)).astype(np.float32))
    j = np.abs(x).argmax(1)
    top = codes[np.arange(500), j]
    assert np.all((top == 0x7E) | (top == 0xFE))
    deq = OC.e4m3(codes) * scale[:, None].astype(np.float64)
    bound = np.abs(x) * 2.0 ** -4 + scale[:, None] * 2.0 ** -10 + 1e-30
    assert np.all(np.abs(deq - x) <= bound)
    zc, zs = Q.fp8_row(np.zeros((3, 128), np.float32))
    assert np.all(zc == 0) and np.all(zs == 1.0)


def test_mx_e8m0_exponent_rule():
    amax = np.array([6.0, 0.75, 1.0, 7.9, 8.0, 0.0, 1e-40, 2.0 ** 127], np.float32)
    # floor(log2 amax) - 2 + 127, clamped: 6 -> 2, 0.75 -> -1, 1 -> 0, 7.9 -> 2, 8 -> 3
    assert Q.mx_e8m0(amax).tolist() == [127, 124, 125, 127, 128, 0, 0, 252]
    g = np.random.default_rng(2)
    x = (g.standard_normal((64, 128)) * np.exp(g.uniform(-6, 6, (64, 1)))).astype(np.float32)
    packed, e8 = Q.mxfp4_blocks(x, 32)
    assert packed.shape == (64, 64) and e8.shape == (64, 4)
    deq = OC.e2m1_packed(packed).reshape(64, 4, 32) * OC.e8m0(e8)[..., None]
    xb = x.reshape(64, 4, 32).astype(np.float64)
    # the block maximum / 2^X lies in [4, 8): it rounds to 4 or 6 (saturating)
    top = np.abs(deq).max(-1) / OC.e8m0(e8)
    assert np.all((top == 4.0) | (top == 6.0))
    assert np.all(np.abs(deq - xb) <= 0.25 * np.abs(xb) + OC.e8m0(e8)[..., None] * 0.25 + 2.0 * OC.e8m0(e8)[..., None] * (np.abs(xb) / OC.e8m0(e8)[..., None] > 6))


def test_nvfp4_block_rule():
    x = np.array([[6.0, -3.0, 1.5, 0.5] + [0.0] * 12, [0.0] * 16], np.float32)
    packed, sc = Q.nvfp4_blocks(x, 16)
    assert sc.reshape(2).tolist() == [0x38, 0]  # E4M3(6/6) = 1.0; zero block -> scale 0
    deq = OC.e2m1_packed(packed).reshape(2, 16) * OC.e4m3(sc.reshape(2))[:, None]
    assert np.array_equal(deq, x.astype(np.float64))


def test_folded_weights_give_the_same_scores():
    g = np.random.default_rng(3)
    qb = torch.from_numpy(g.standard_normal((4, 32, 128)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    w = g.uniform(-1, 1, (4, 32)).astype(np.float32)
    codes, scale, wf = Q.quantize_q(qb, w, "fp8")
    assert np.array_equal(wf, (w * scale).astype(np.float32))
    keys = g.standard_normal((300, 128))
    q8 = OC.e4m3(codes)
    for t in range(4):
        a = O.indexer_scores(q8[t] * scale[t][:, None].astype(np.float64), w[t].astype(np.float64), keys)
        b = O.indexer_scores(q8[t], wf[t].astype(np.float64), keys)
        # w' is rounded to fp32: each term moves by at most 2^-24 of itself
        terms = np.abs(wf[t].astype(np.float64)) @ np.maximum(q8[t] @ keys.T, 0)
        assert np.all(np.abs(a - b) <= 2.0 ** -23 * terms + 1e-12)


@pytest.mark.parametrize("key_fmt,lat_fmt", [("fp8", "fp8"), ("mxfp4", "nvfp4"), ("fp8", "bf16")])
def test_cache_insert_decodes_back_at_the_right_rows(key_fmt, lat_fmt):
    g = np.random.default_rng(4)
    P, npg, R = 16, 12, 3
    kbytes = {"fp8": 132, "mxfp4": 68}[key_fmt] * P
    lbytes = Q.LAT_ROW_STRIDE[lat_fmt] * P
    kpool = g.integers(0, 256, (npg, kbytes)).astype(np.uint8)
    lpool = g.integers(0, 256, (npg, lbytes)).astype(np.uint8)
    bt = np.stack([g.permutation(npg)[:4] for _ in range(R)]).astype(np.int64)
    bt[2, 3] = -1  # an absent page: tokens there are skipped
    tok_req = np.array([0, 0, 1, 2, 2, 1])
    tok_pos = np.array([0, 15, 33, 47, 50, 63])
    kv = torch.from_numpy(g.standard_normal((6, 128)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    lv = torch.from_numpy(g.standard_normal((6, 576)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    kp, lp = Q.cache_insert(kpool, key_fmt, lpool, lat_fmt, P, bt, tok_req, tok_pos, kv, lv, npg)
    touched = np.zeros((npg, P), bool)
    for i in range(6):
        r, pos = tok_req[i], tok_pos[i]
        page = bt[r, pos // P]
        if page < 0:
            continue
        touched[page, pos % P] = True
        row = np.array([page * P + pos % P])
        kx = Q.bf16_to_f32(kv[i])
        if key_fmt == "fp8":
            c, s = Q.fp8_row(kx)
            want = OC.e4m3(c) * float(s)
        else:
            c, e8 = Q.mxfp4_blocks(kx, 32)
            want = (OC.e2m1_packed(c).reshape(4, 32) * OC.e8m0(e8)[:, None]).reshape(128)
        got = O.key_pages(kp, key_fmt, P, np.array([page])).reshape(P, 128)[pos % P]
        assert np.array_equal(got, want)
        lx = Q.bf16_to_f32(lv[i])
        if lat_fmt == "fp8":
            c, s = Q.fp8_row(lx)
            want = OC.e4m3(c) * float(s)
        elif lat_fmt == "bf16":
            want = lx.astype(np.float64)
        else:
            c, sc = Q.nvfp4_blocks(lx[:512], 16)
            want = np.concatenate([(OC.e2m1_packed(c).reshape(32, 16) * OC.e4m3(sc)[:, None]).reshape(512),
                                   OC.e4m3(Q.e4m3_encode(lx[512:]))])
        assert np.array_equal(O.lat_rows(lp, lat_fmt, P, row)[0], want)
    # untouched slots keep their bytes (codes, scales, rows)
    kc = {"fp8": 128, "mxfp4": 64}[key_fmt]
    ls = Q.LAT_ROW_STRIDE[lat_fmt]
    for page in range(npg):
        for slot in range(P):
            if touched[page, slot]:
                continue
            assert np.array_equal(kp[page, slot * kc:(slot + 1) * kc], kpool[page, slot * kc:(slot + 1) * kc])
            assert np.array_equal(kp[page, P * kc + 4 * slot:P * kc + 4 * slot + 4],
                                  kpool[page, P * kc + 4 * slot:P * kc + 4 * slot + 4])
            assert np.array_equal(lp[page, slot * ls:(slot + 1) * ls], lpool[page, slot * ls:(slot + 1) * ls])
