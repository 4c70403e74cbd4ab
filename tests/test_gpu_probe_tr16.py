"""The lane layout of gfx950's transposed LDS read (ds_read_b64_tr_b16) that the
adjoint walk's fragment transposes assume (tr_frag, gdr_device.h): within each
16-lane row of a wavefront, lane 4a + e receives element e of the 8-byte pieces
that lanes a, 4 + a, 8 + a and 12 + a address, in that order.  Checked with one
in-bounds read of a 512-value LDS block (probe library, two address patterns)."""
import ctypes

import numpy as np
import pytest
import torch


def expected(mode):
    out = np.zeros((64, 4), dtype=np.int64)
    for lane in range(64):
        base, a, e = 16 * (lane // 16), (lane % 16) // 4, lane % 4
        for j in range(4):
            src = base + 4 * j + a  # the lane whose address supplies element j
            piece = src if mode == 0 else 63 - src
            out[lane, j] = 4 * piece + e
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 1], ids=["own_piece", "reversed_pieces"])
def test_transposed_lds_read_lane_layout(mode):
    from chunked_gated_delta_14_amd import _build

    L = ctypes.CDLL(_build.PROBE_PATH)
    L.gdr_probe_tr16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    out = torch.full((256,), -1, dtype=torch.int16, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.gdr_probe_tr16(ctypes.c_void_p(out.data_ptr()), mode, st) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(64, 4) & 0xFFFF
    assert np.array_equal(got, expected(mode))
