"""q8_0 K blocks over the whole range of their f16 scale, through prefill,
decode and store-then-read, against the CPU oracle.

A q8_0 block is 32 int8 codes and one f16 scale, any finite f16 value
("KV Cache Design — cells, format, sessions", section 3), so a block's
largest value reaches 127 * 65504 ~ 8.3e6.  The pools here are written byte
by byte: every live (token, kv head, block) gets codes drawn from [-127, 127]
(one of them +-127, as the quantizer always produces) and a scale drawn from
one binade band, from f16 subnormals up to 65504.  The attention scale of a
call is chosen against its band so that the scores stay O(1) and the
softmax is well conditioned; the mixed case puts every band in one pool.

Tolerance: max-abs 2e-3 on out and lse (f16/q8_0 inputs, f32 accumulation).
"""

import numpy as np
import pytest

import oracle
import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

from gpu_util import Dev, compare, log

pytestmark = pytest.mark.gpu

# binade exponents of the scale bands; "sub" = f16 subnormal scales
BANDS = ["sub", -14, -4, 6, 9, 12, 15]


def _scales(rng, band, shape):
    if band == "sub":
        return (rng.integers(1, 1024, size=shape) * 2.0 ** -24).astype(np.float16)
    s = rng.uniform(1.0, 2.0, size=shape) * 2.0 ** band
    s = np.minimum(s, 65504.0).astype(np.float16)
    if band == 15:
        s.flat[:: 7] = np.float16(65504.0)  # the largest f16 value itself
    return s


def _band_exp(band):
    return -15 if band == "sub" else band


def _write_q8_pool(w, kh, rng, bands):
    """Overwrite the live rows of the q8_0 K pool kh ([blocks, kv heads,
    block size, seg] uint8) with random codes and scales from `bands`
    (chosen per row at random); dead rows keep their NaN scales."""
    nb = w.head_dim // 32
    nblk, hkv, bs, _ = kh.shape
    shape = (nblk, hkv, bs, nb)
    band_of = rng.integers(0, len(bands), size=shape)
    sc = np.zeros(shape, dtype=np.float16)
    for i, b in enumerate(bands):
        sel = band_of == i
        sc[sel] = _scales(rng, b, int(sel.sum()))
    codes = rng.integers(-127, 128, size=shape + (32,)).astype(np.int8)
    first = np.where(rng.integers(0, 2, size=shape) == 1, 127, -127).astype(np.int8)
    codes[..., 0] = first
    blk = np.concatenate([sc[..., None].view(np.uint8).reshape(shape + (2,)), codes.view(np.uint8)], axis=-1)
    live = wgen.referenced_rows(w).reshape(nblk, bs)  # row = block * bs + slot
    live = np.broadcast_to(live[:, None, :, None, None], shape + (34,))
    view = kh[..., : nb * 34].reshape(shape + (34,))
    view[...] = np.where(live, blk, view)
    return kh


def _dev_with_pool(w, rng, bands):
    import torch

    d = Dev(w)
    d.kh = _write_q8_pool(w, d.kh.copy(), rng, bands)
    d.k = torch.from_numpy(d.kh).cuda()
    return d


@pytest.mark.parametrize("band", BANDS)
def test_q8_scale_band_prefill_and_decode(band):
    e = _band_exp(band)
    rng = np.random.default_rng(100 + BANDS.index(band))
    for kind, mode in (("prefill", "kv_map"), ("prefill", "causal"), ("decode", "span")):
        w = wgen.make_custom(seed=300 + BANDS.index(band), n_seqs=5, n_q_heads=8, n_kv_heads=2, head_dim=128,
                             block_size=32, fmts=("f16", "q8_0", "f16"), ctx=(30, 400), mode=mode, n_runs=4,
                             kind=kind, q_per_seq=(1, 70), hole_frac=0.05)
        w.scale = float(2.4e-3 * 2.0 ** -e)
        log(f"q8_0 scale band 2^{e} ({band}): {kind} {mode}, attention scale {w.scale:.3g}")
        d = _dev_with_pool(w, rng, [band])
        out, lse = d.prefill() if kind == "prefill" else d.decode()
        ro, rl = d.oracle()
        compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, 2e-3, f"band {band} {kind} {mode}")


@pytest.mark.parametrize("hd,bs", [(64, 16), (128, 16), (256, 16), (128, 32)])
def test_q8_all_bands_in_one_pool(hd, bs):
    """Every band in one pool: the largest scales dominate the softmax, the
    tiny ones must still give finite, exact-enough contributions."""
    rng = np.random.default_rng(hd + bs)
    for kind in ("prefill", "decode"):
        w = wgen.make_custom(seed=hd * 3 + bs, n_seqs=4, n_q_heads=8, n_kv_heads=2, head_dim=hd, block_size=bs,
                             fmts=("f16", "q8_0", "f16"), ctx=(20, 300), mode="causal", kind=kind,
                             q_per_seq=(1, 50), hole_frac=0.05)
        w.scale = float(2.4e-3 * 2.0 ** -15)
        log(f"q8_0 all bands: hd {hd} bs {bs} {kind}")
        d = _dev_with_pool(w, rng, BANDS)
        out, lse = d.prefill() if kind == "prefill" else d.decode()
        ro, rl = d.oracle()
        compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, 2e-3, f"all bands hd{hd} bs{bs} {kind}")


@pytest.mark.parametrize("e", [-20, 0, 9, 16, 22])
def test_q8_store_then_prefill_large_values(e):
    """f32 rows of magnitude ~2^e stored through the q8_0 quantizer (amax up
    to 127 * 65504 at e = 22), then read by prefill and decode: the stored
    bytes equal the oracle's quantizer, and attention over them matches the
    oracle."""
    import torch

    rng = np.random.default_rng(1000 + e)
    for kind in ("prefill", "decode"):
        w = wgen.make_custom(seed=500 + e, n_seqs=4, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=32,
                             fmts=("f16", "q8_0", "f16"), ctx=(30, 260), mode="causal", kind=kind,
                             q_per_seq=(1, 60), hole_frac=0.0)
        w.scale = float(2.4e-3 * 2.0 ** -(e - 7))
        d = Dev(w)
        # every live position of every sequence, stored in one call
        seq_ids, pos = [], []
        for s in range(w.n_seqs):
            seq_ids += [s] * int(w.seq_lens[s])
            pos += list(range(int(w.seq_lens[s])))
        seq_ids, pos = np.array(seq_ids, np.int32), np.array(pos, np.int32)
        n = len(pos)
        x = rng.standard_normal((n, 2, 128)).astype(np.float32) * np.float32(2.0 ** e)
        amax_cap = np.float32(127.0 * 65504.0)
        x = np.clip(x, -amax_cap, amax_cap)
        vx = rng.standard_normal((n, 2, 128)).astype(np.float32)
        rk, rv, skipped = oracle.store_rows(d.kh.copy(), d.vh.copy(), "q8_0", "f16", x, vx, seq_ids, pos,
                                            w.block_table)
        dk, dv = d.k.clone(), d.v.clone()
        pkv.kv_store(torch.from_numpy(x).cuda(), torch.from_numpy(vx).cuda(), torch.from_numpy(pos).cuda(), dk, dv,
                     d.table, seq_ids=torch.from_numpy(seq_ids).cuda())
        assert np.array_equal(dk.cpu().numpy(), rk), f"stored q8_0 bytes differ (e = {e})"
        d.k, d.v, d.kh, d.vh = dk, dv, rk, rv
        log(f"q8_0 store of 2^{e} values then {kind}: {n} tokens")
        out, lse = d.prefill() if kind == "prefill" else d.decode()
        ro, rl = d.oracle()
        compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, 2e-3, f"store 2^{e} then {kind}")


@pytest.mark.parametrize("band", ["sub", 15])
def test_q8_scale_band_f32_queries(band):
    """The f32-query combination (q f32, K q8_0, V f32) at the ends of the
    scale range: decode, and prefill (which runs f32 queries through the
    decode kernels), against the oracle."""
    e = _band_exp(band)
    rng = np.random.default_rng(700 + BANDS.index(band))
    for kind, mode in (("decode", "causal"), ("prefill", "kv_map")):
        w = wgen.make_custom(seed=710 + BANDS.index(band), n_seqs=4, n_q_heads=8, n_kv_heads=2, head_dim=128,
                             block_size=16, fmts=("f32", "q8_0", "f32"), ctx=(30, 300), mode=mode, n_runs=4,
                             kind=kind, q_per_seq=(1, 30), hole_frac=0.05)
        w.scale = float(2.4e-3 * 2.0 ** -e)
        log(f"q8_0 scale band 2^{e} ({band}), f32 q and V: {kind} {mode}, attention scale {w.scale:.3g}")
        d = _dev_with_pool(w, rng, [band])
        out, lse = d.prefill() if kind == "prefill" else d.decode()
        ro, rl = d.oracle()
        compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, 2e-3, f"f32 band {band} {kind} {mode}")
