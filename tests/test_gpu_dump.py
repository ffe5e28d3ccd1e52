"""Bit-exact staged tiles: the dump kernel (same block loader and decoder as the MFMA kernels)
against the oracle's staged values, every format x staged type."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import dev

pytestmark = pytest.mark.gpu

STAGED = {"f32": qg.QG_X_F32, "f16": qg.QG_X_F16, "bf16": qg.QG_X_BF16}


@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8", "q8a"])
@pytest.mark.parametrize("staged", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(64, 256, 5, 64, 37, 128), (48, 96, 0, 0, 48, 96), (4096, 4096, 4000, 3968, 96, 128)])
def test_dump_bit_exact(orc, fmt, staged, shape):
    N, K, n0, k0, rows, cols = shape
    w = synth.make_dense(fmt, N, K, 1, "f32", 1.0, 77 + N, group=32 if K == 96 else 64)
    group = w["group"]
    codes, scales = dev(w["codes"]), dev(w["scales"])
    offs = dev(w["offsets"]) if fmt in ("q4a", "q8a") else None
    out = torch.empty((rows, cols), dtype=torch.float32 if staged == "f32" else torch.int16, device="cuda")
    qg.qg_dequant_dump(fmt, codes, scales, offs, group, N, K, n0, k0, rows, cols, STAGED[staged], out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = orc.dequant_tile(fmt, w["codes"], w["scales"], w.get("offsets"), group, N, K, n0, k0, rows, cols, staged)
    if staged == "f32":
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    else:
        assert np.array_equal(got.view(np.uint16), ref)


def test_dump_extreme_scales(orc):
    """Scales at the f16 extremes (subnormal, largest finite) and codes hitting every nibble."""
    N, K = 32, 64
    nib = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    codes = qg.pack_q4(nib).reshape(-1)
    sc = np.array([0x0001, 0x03FF, 0x0400, 0x7BFF, 0x3C00, 0xBC00, 0x1400, 0x5BFF], np.uint16)
    scales = np.resize(sc, N * K // 32)
    offs = np.resize(np.array([0x0001, 0x3F80, 0xC2F7, 0x7F7F, 0x0000, 0x8000], np.uint16), N * K // 64)
    for fmt in ("q4", "q4a"):
        for staged in ("f32", "f16", "bf16"):
            out = torch.empty((N, K), dtype=torch.float32 if staged == "f32" else torch.int16, device="cuda")
            qg.qg_dequant_dump(fmt, dev(codes), dev(scales), dev(offs) if fmt == "q4a" else None, 64, N, K, 0, 0,
                               N, K, STAGED[staged], out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            ref = orc.dequant_tile(fmt, codes, scales, offs if fmt == "q4a" else None, 64, N, K, 0, 0, N, K, staged)
            if staged == "f32":
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (fmt, staged)
            else:
                assert np.array_equal(got.view(np.uint16), ref), (fmt, staged)
