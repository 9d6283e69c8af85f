"""int4 cold-block codec on the GPU: bit-exact against the oracle."""

import json
import os

import numpy as np
import pytest

import oracle
import paged_kv_cache_table_amd as pkv

from gpu_util import log

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pool(rng, nb, shape, dtype, scale_exp=None):
    x = rng.standard_normal((nb, *shape)).astype(np.float32)
    if scale_exp is not None:
        x *= (2.0 ** rng.integers(*scale_exp, size=(nb,) + (1,) * len(shape))).astype(np.float32)
    return x.astype(dtype)


@pytest.mark.parametrize("hkv,bs,hd", [(1, 16, 64), (8, 16, 128), (8, 32, 128), (8, 16, 256), (8, 32, 256),
                                       (3, 16, 64), (2, 1, 32)])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_encode_decode_bit_exact(hkv, bs, hd, dtype):
    import torch

    rng = np.random.default_rng(hkv * 1000 + bs * 10 + hd + (dtype == np.float32))
    nb = 24
    ph = _pool(rng, nb, (hkv, bs, hd), dtype, scale_exp=(-20, 6))
    ph[3] = 0  # an all-zero block
    blocks = np.array([5, 3, 0, 23, 7, 7, 11, 40, -2], dtype=np.int32)  # repeats; ids outside the pool
    pool = torch.from_numpy(ph).cuda()
    dblocks = torch.from_numpy(blocks).cuda()
    blobs = pkv.int4_encode(pool, dblocks)
    torch.cuda.synchronize()
    nbytes = oracle.blob_bytes(hkv * bs * hd)
    got = blobs.cpu().numpy()
    for i, b in enumerate(blocks):
        want = oracle.encode_block(ph[b]) if 0 <= b < nb else np.zeros(nbytes, dtype=np.uint8)
        assert np.array_equal(got[i, :nbytes], want), f"block {b}"
    # decode the blobs of the valid, distinct ids into other blocks
    src = [0, 1, 2, 3, 4, 6]  # blobs of blocks 5, 3, 0, 23, 7, 11 (index 5 repeats 7)
    dst = np.array([12, 13, 14, 15, 16, 17], dtype=np.int32)
    out = torch.from_numpy(ph.copy()).cuda()
    pkv.int4_decode(blobs[src].contiguous(), out, torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    oh = out.cpu().numpy()
    fmt = "f16" if dtype == np.float16 else "f32"
    for j, i in enumerate(src):
        want = oracle.decode_block(got[i], hkv * bs * hd, fmt).reshape(hkv, bs, hd)
        assert np.array_equal(oh[dst[j]].view(np.uint8), want.view(np.uint8)), f"decode {j}"
    untouched = [b for b in range(nb) if b not in dst]
    assert np.array_equal(oh[untouched].view(np.uint8), ph[untouched].view(np.uint8))


def test_edge_values_bit_exact():
    """The hand-worked blocks (padded with zeros to a block), values on and
    beside code boundaries, tiny and subnormal magnitudes."""
    import torch

    with open(os.path.join(GOLDEN, "int4_block_worked.json")) as f:
        cases = json.load(f)["cases"]
    rng = np.random.default_rng(21)
    n = 2 * 16 * 64
    blocks = []
    for c in cases:
        x = np.zeros(n, dtype=np.float32)
        v = np.array([float.fromhex(t) for t in c["x"]], dtype=np.float32)
        x[: v.size] = v
        blocks.append(x)
    for _ in range(12):
        amax = np.float32(rng.uniform(0.1, 10))
        s = np.float32(amax / np.float32(7))
        x = ((rng.integers(-7, 7, size=n) + 0.5) * np.float64(s)).astype(np.float32)
        step = rng.integers(-1, 2, size=n)
        x = np.where(step > 0, np.nextafter(x, np.float32(np.inf)),
                     np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
        x[0] = amax
        blocks.append(x)
    for e in (-126, -130, -140, -149):
        blocks.append((rng.standard_normal(n) * 2.0 ** e).astype(np.float32))
    ph = np.stack(blocks).reshape(len(blocks), 2, 16, 64)
    pool = torch.from_numpy(ph).cuda()
    ids = torch.arange(len(blocks), dtype=torch.int32, device="cuda")
    got = pkv.int4_encode(pool, ids).cpu().numpy()
    nbytes = oracle.blob_bytes(n)
    for i in range(len(blocks)):
        assert np.array_equal(got[i, :nbytes], oracle.encode_block(ph[i])), f"block {i}"


def test_round_trip_cosine_about_099():
    """The page's figure on N(0, 1) blocks of the 7B-class layer shape."""
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    pool = torch.randn((256, 8, 16, 128), generator=g, device="cuda").half()
    ids = torch.arange(256, dtype=torch.int32, device="cuda")
    out = torch.empty_like(pool)
    pkv.int4_decode(pkv.int4_encode(pool, ids), out, ids)
    a, b = pool.float().reshape(256, -1), out.float().reshape(256, -1)
    cos = (a * b).sum(1) / (a.norm(dim=1) * b.norm(dim=1))
    log(f"  int4 round trip cosine: mean {cos.mean().item():.4f}, min {cos.min().item():.4f}")
    # the mean is the page's figure; single blocks with an outlier amax fall a little lower
    assert 0.97 <= cos.min().item() and abs(cos.mean().item() - 0.99) < 0.006


def test_refusals():
    import torch

    pool = torch.zeros((4, 2, 16, 64), dtype=torch.float16, device="cuda")
    ids = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        pkv.int4_encode(pool.to(torch.uint8), ids)
    bad = torch.zeros((4, 1, 1, 12), dtype=torch.float16, device="cuda")  # 12 values: not a multiple of 8
    with pytest.raises(pkv.PkvError):
        pkv.int4_encode(bad, ids)
    small = torch.zeros((2, 100), dtype=torch.uint8, device="cuda")  # stride below the blob size
    with pytest.raises(pkv.PkvError):
        pkv.int4_encode(pool, ids, small)
    big = torch.zeros((2, 8, 32, 512), dtype=torch.float16, device="cuda")  # 131072 values per block
    with pytest.raises(pkv.PkvError):
        pkv.int4_encode(big, ids)
