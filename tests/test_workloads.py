"""The input generators' bf16 storage: round to nearest, ties to even, as
PyTorch's own float32 -> bfloat16 conversion does, on a sweep of bit patterns
covering every exponent, both signs, ties, subnormals, infinities and NaN."""
import numpy as np
import torch

from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def test_bf16_rounding_matches_torch():
    pats = np.arange(0, 2 ** 32, 65521, dtype=np.uint64).astype(np.uint32)
    ties = (np.arange(0, 2 ** 16, dtype=np.uint32) << 16) | np.uint32(0x8000)   # exact halfway cases
    near = (np.arange(0, 2 ** 16, dtype=np.uint32) << 16) | np.uint32(0x7FFF)
    a = np.concatenate([pats, ties, near]).view(np.float32)
    finite = ~np.isnan(a)
    got = f32_to_bf16_bits(a)
    want = torch.from_numpy(a.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[finite], want[finite])
    assert np.all(np.isnan(bf16_bits_to_f32(got[~finite])))


def test_bf16_widening_is_exact():
    b = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(b)
    ok = ~np.isnan(f)
    assert np.array_equal(f32_to_bf16_bits(f[ok]), b[ok])
