"""Host-side layout helpers of the binding (no GPU): the row-major view of the tile-major FP8 head
codes against the layout as the C header defines it."""
import numpy as np
import torch

import quantized_weight_streaming_amd as qws
from quantized_weight_streaming_amd import _lib

from .helpers import fp8_tile_major


def test_fp8_codes_rowmajor_inverts_the_tile_major_layout():
    rng = np.random.default_rng(5)
    for rows, cols in ((1, 32), (17, 96), (40, 544)):
        codes = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
        d = _lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, rows, cols, None, None)
        head = qws.LMHead(torch.from_numpy(fp8_tile_major(codes)), None, d)
        assert np.array_equal(qws.fp8_codes_rowmajor(head).numpy(), codes)


def test_tile_major_places_chunks_as_defined():
    # one worked case: rows 0 .. 16 x 64 columns; codes encode (row, column) so each byte's place
    # can be read back: tile 0 holds rows 0 .. 15, chunk c of row i at byte 16 (16 c + i)
    rows, cols = 17, 64
    codes = ((np.arange(rows)[:, None] * 7 + np.arange(cols)[None, :]) % 251).astype(np.uint8)
    t = fp8_tile_major(codes)
    assert t.size == 32 * 64
    assert t[16 * (16 * 2 + 5) + 3] == codes[5, 2 * 16 + 3]           # tile 0, chunk 2, row 5, byte 3
    assert t[16 * 64 + 16 * (16 * 1 + 0) + 15] == codes[16, 31]       # tile 1, chunk 1, row 16
    assert not t[16 * 64 + 16 * 1:16 * 64 + 16 * 16].any()            # chunk 0 of the pad rows 17 .. 31
