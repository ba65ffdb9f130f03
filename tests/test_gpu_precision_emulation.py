"""GPU parity: precision emulation (replayssm_emulate_precision) against the oracle's
read-copy formats, bit for bit -- both sides round the same fp32 values to nearest
even, and the fp8 scales come from the same fp32 divisions.  Rows cover several
magnitudes, zero rows, ties, fp16 subnormals and fp16 overflow, and row lengths that
are not multiples of the 64-lane wave."""

import numpy as np
import pytest
import torch

from hybrid_model_ssm_amd import replayssm as rs
from oracle import readcopy as orc
from tests.gpu_helpers import DEV, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def rows_of(n_rows, row_len, seed):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n_rows, row_len)).astype(np.float32)
    h *= (10.0 ** rng.uniform(-6, 4, size=(n_rows, 1))).astype(np.float32)
    h[0] = 0.0                                                   # a zero row
    if n_rows > 1:
        h[1] = 0.0
        h[1, row_len // 2] = -3.5                                # one nonzero value
    if n_rows > 2:
        # exact bf16 ties: the low 16 bits are 0x8000
        bits = rng.integers(0x3F000000, 0x40000000, size=row_len, dtype=np.uint32)
        h[2] = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)
    if n_rows > 3:
        h[3] = np.linspace(-7e4, 7e4, row_len, dtype=np.float32)   # beyond the fp16 range
    if n_rows > 4:
        h[4] = np.linspace(-2e-6, 2e-6, row_len, dtype=np.float32)  # fp16 subnormals
    return h


SHAPES = [(1, 4), (7, 36), (300, 128), (5, 260)]


def run(h, dtype, with_scale=False):
    d = torch.from_numpy(h).to(DEV)
    sc = torch.full((h.shape[0],), -1.0, device=DEV) if with_scale else None
    rs.emulate_precision(d, dtype, sc)
    torch.cuda.synchronize()
    return d.cpu().numpy(), (sc.cpu().numpy() if with_scale else None)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_bf16_and_f16_rounding(shape):
    h = rows_of(*shape, seed=71)
    got, _ = run(h, rs.BF16)
    assert np.array_equal(got, orc.bf16_copy(h).astype(np.float32))
    got, _ = run(h, rs.F16)
    with np.errstate(over="ignore"):
        want = orc.f16_copy(h).astype(np.float32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_fp8_row_scaled_rounding(shape):
    h = rows_of(*shape, seed=73)
    codes, scale = orc.fp8_copy(h)
    want = orc.fp8_values(codes, scale).astype(np.float32)
    got, sc = run(h, rs.FP8_E4M3, with_scale=True)
    assert np.array_equal(sc, scale)
    assert np.array_equal(got, want)
    got2, _ = run(h, rs.FP8_E4M3)          # no scale output
    assert np.array_equal(got2, want)


def test_f32_is_identity_and_rounding_is_idempotent():
    h = rows_of(9, 64, seed=75)
    got, _ = run(h, rs.F32)
    assert np.array_equal(got, h)
    for dt in (rs.BF16, rs.F16):
        once, _ = run(h, dt)
        finite = np.isfinite(once)
        twice, _ = run(np.where(finite, once, 0).astype(np.float32), dt)
        assert np.array_equal(twice[finite], once[finite])
    # fp8: the codes come back; the new row scale may differ from the old in its last bit
    once, _ = run(h, rs.FP8_E4M3)
    twice, _ = run(once, rs.FP8_E4M3)
    assert np.allclose(twice, once, rtol=2.0 ** -21, atol=0.0)
