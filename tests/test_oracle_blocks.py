"""Pins of the oracle's blocks layout (64 x 64 weight blocks as tiles).

The layout is a format choice: the pages ask for independently decodable
tiles and leave their shape open; blocks let a matrix product decode each
block of W straight into its operand (API reference, "CompressedLinear").
What is pinned, each against the layout's definition rather than against the
oracle's own encoder:
  * decode equals direct quantization (rANS and the layout are lossless);
  * tile t decodes exactly the block (t // KB, t % KB), KB = ceil(cols / 64),
    and touches nothing else;
  * inside a tile, local vector i = 8 * (block row) + (vector column) belongs
    to state i mod 64: a single heavy vector makes its state's pair emit the
    most words, read from the stream bytes;
  * the header's layout byte and tile count, the argument rules, the rate.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_tile_interleaved_amd import workloads as W

B = oracle.LAYOUT_BLOCKS


def blocks(x, target=4.0, **kw):
    blob, rc, a = oracle.compress(x, target, layout=B, **kw)
    assert rc == 0, rc
    return blob, a


@pytest.mark.parametrize("rows,cols", [(64, 64), (200, 136), (130, 520), (65, 8), (1, 72), (257, 1024)])
def test_decode_equals_direct_quantization(rows, cols):
    x = W.gaussian(rows, cols, 0.02, seed=rows + 17 * cols)
    blob, a = blocks(x, fixed_a=0.3)
    _, v = oracle.quantize_matrix(x, a)
    assert np.array_equal(oracle.decode_symbols(blob), v)


@pytest.mark.parametrize("rows,cols", [(200, 136), (64, 200), (130, 72)])
def test_each_tile_decodes_exactly_its_block(rows, cols):
    x = W.gaussian(rows, cols, 0.02, seed=3 * rows + cols)
    blob, a = blocks(x, fixed_a=0.3)
    d = oracle.info(blob)
    kb_n, nb_n = math.ceil(cols / 64), math.ceil(rows / 64)
    assert d["layout"] == B and d["n_tiles"] == kb_n * nb_n
    full = oracle.decompress_raw(blob)
    sentinel = np.uint16(0x7fc1)  # a BF16 NaN the decoder never writes
    for t in range(d["n_tiles"]):
        out = np.full((rows, cols), sentinel, np.uint16)
        oracle.decompress_tile_range(blob, t, t + 1, out=out)
        nb, kb = divmod(t, kb_n)
        mask = np.zeros((rows, cols), bool)
        mask[64 * nb:64 * nb + 64, 64 * kb:64 * kb + 64] = True
        assert np.array_equal(out != sentinel, mask), f"tile {t} wrote outside block ({nb}, {kb})"
        assert np.array_equal(out[mask], full[mask])


def pair_counts(blob: np.ndarray, tile: int) -> np.ndarray:
    """The 32 pair-count bytes of a 64-state tile, read from the stream."""
    off_to = int(blob[88:96].view(np.uint64)[0])
    off_w = int(blob[96:104].view(np.uint64)[0])
    first = int(blob[off_to + 4 * tile:off_to + 4 * tile + 4].view(np.uint32)[0])
    at = off_w + 2 * first
    return blob[at:at + 32].astype(int)


@pytest.mark.parametrize("r,c", [(0, 0), (0, 7), (5, 3), (13, 6), (63, 7), (40, 1)])
def test_state_of_a_vector_is_its_index_mod_64(r, c):
    """One heavy vector at block row r, vector column c of tile 0: its state
    q = (8 r + c) mod 64 codes far more bits than any other, so pair q // 2
    holds the most words.  The rows are 1024 wide so that the vector is a
    small part of its row's RMS, and the resolution is coarse enough that the
    other coordinates quantize to 0 while the heavy ones do not."""
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(64, 1024, generator=g) * 0.02).float()
    x[r, 8 * c:8 * c + 8] = torch.tensor([3.0, -2.5, 2.0, -3.5, 2.25, -1.75, 3.25, -2.0])
    blob, _ = blocks(x.to(torch.bfloat16), fixed_a=8.0)
    v = oracle.decode_symbols(blob)
    assert np.count_nonzero(v[r, 8 * c:8 * c + 8]) >= 6
    pc = pair_counts(blob, 0)
    q = (8 * r + c) % 64
    assert int(np.argmax(pc)) == q // 2, (pc, q)
    assert pc[q // 2] > 2 * np.sort(pc)[-2] + 1


def test_layout_rules():
    x = W.gaussian(64, 64, 0.02, seed=1)
    with pytest.raises(oracle.OracleError) as e:
        oracle.compress(x.to(torch.float16), 4.0, layout=B)
    assert e.value.rc == oracle.ERR_ARG
    with pytest.raises(oracle.OracleError) as e:
        oracle.compress(W.gaussian(64, 60, 0.02, seed=1), 4.0, layout=B)
    assert e.value.rc == oracle.ERR_SHAPE
    for kw in ({"n_states": 16}, {"tile_vecs": 1024}):
        with pytest.raises(oracle.OracleError) as e:
            oracle.compress(x, 4.0, layout=B, **kw)
        assert e.value.rc == oracle.ERR_ARG
    with pytest.raises(oracle.OracleError) as e:
        oracle.compress(x, 4.0, layout=2)
    assert e.value.rc == oracle.ERR_ARG


@pytest.mark.parametrize("rows,cols,target", [(512, 1024, 4.0), (300, 640, 2.75), (256, 3840, 3.0)])
def test_rate_and_one_encode(rows, cols, target):
    x = W.rowscale_gaussian(rows, cols, seed=rows + cols)
    blob, _ = blocks(x, target)
    assert oracle.last_encode_count() == 1
    bpp = 8 * blob.size / (rows * cols)
    assert abs(bpp - target) <= 0.02 * target, bpp
