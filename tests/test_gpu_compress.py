"""GPU parity: compressor (projections, softmax fold, RoPE).  Bar: 1e-4 x RMS.  Float32
inputs (and a scalar Z) take the float64 kernel, which also agrees with the oracle to
float32 rounding; bf16 inputs take the MFMA kernel (fp32 accumulation)."""
import numpy as np
import pytest
import torch

from helpers import dev, dev_bf16
from oracle.codecs import f64_to_bf16
from oracle.csa2 import compress

pytestmark = pytest.mark.gpu


def bd():
    from kv_cache_compression_03_amd import binding
    return binding


@pytest.mark.parametrize("B,T,dm,d,dz,m,pos0,r,bf16", [
    (1, 333, 96, 128, 128, 2, 0, 64, False),
    (2, 64, 64, 256, 256, 1, 7, 64, False),
    (1, 130, 80, 128, 1, 4, 24576, 64, False),
    (1, 96, 64, 512, 512, 2, 24576, 64, True),
    (1, 40, 32, 64, 64, 2, 0, 0, False),
    (2, 600, 128, 256, 256, 1, 0, 64, True),
    (1, 300, 192, 128, 128, 4, 8, 64, True),
    (1, 1030, 320, 512, 512, 2, 24576, 64, True),
    (1, 200, 128, 128, 1, 2, 0, 64, True),
    (1, 64, 64, 64, 64, 1, 3, 0, True),
    # a few tokens in all (a decode step's new blocks): the split-reduction kernel
    (3, 2, 256, 512, 512, 2, 24576, 64, True),
    (64, 1, 512, 512, 512, 1, 1000, 64, True),
    (5, 4, 384, 256, 256, 4, 0, 64, True),
    (2, 16, 128, 128, 128, 1, 7, 0, True),
])
def test_compress(B, T, dm, d, dz, m, pos0, r, bf16):
    rng = np.random.default_rng(T + d)
    H = rng.standard_normal((B, T, dm)).astype(np.float32)
    Wkv = (rng.standard_normal((dm, d)) / np.sqrt(dm)).astype(np.float32)
    Wz = (rng.standard_normal((dm, dz)) / np.sqrt(dm)).astype(np.float32)
    if bf16:
        H, Wkv, Wz = f64_to_bf16(H), f64_to_bf16(Wkv), f64_to_bf16(Wz)
        to = dev_bf16
    else:
        to = dev
    out = bd().csa2_compress(to(H), to(Wkv), to(Wz), m, pos0=pos0, rope_dim=r).cpu().numpy()
    for b in range(B):
        ref = compress(H[b], Wkv, Wz, m, pos0=pos0, rope_dim=r)
        rms = np.sqrt(np.mean(ref ** 2))
        assert out.shape[1] == T // m
        assert np.max(np.abs(out[b] - ref)) <= 1e-4 * rms
        if not bf16 or dz == 1:
            # float64 sums: within a float32 rounding of the oracle almost everywhere
            close = np.abs(out[b] - ref) <= np.abs(ref) * 2.0 ** -23 + 1e-30
            assert close.mean() > 0.999
