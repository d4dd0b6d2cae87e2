"""The comparison helpers against values fixed by the bf16 format (CPU)."""
import numpy as np
import torch

from tests.util import bf16_bits_to_f32, bf16_rne_bits


def test_bf16_rne_hand_values():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing just above 1.0
    x = np.array([one, one + ulp / 2, one + 1.5 * ulp, one + 0.75 * ulp, -one - ulp / 2, 0.0, -0.0,
                  3.0e38, 1e-40], dtype=np.float32)
    got = bf16_rne_bits(x).tolist()
    # 1.0; a tie rounds down to the even 1.0; a tie rounds up to the even 1+2ulp;
    # above half an ulp rounds up; the negative tie; both zeros; a large finite
    # value; an fp32 subnormal keeps its top bits
    assert got[:7] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x0000, 0x8000]
    assert got[7] == 0x7F62 and got[8] == int(np.array([1e-40], np.float32).view(np.uint32)[0] + 0x7FFF) >> 16


def test_bf16_rne_matches_torch_cpu_conversion():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_rne_bits(x), ref)
    back = bf16_bits_to_f32(ref)
    assert np.all(np.abs(back.astype(np.float64) - x) <= np.abs(x.astype(np.float64)) * 2.0 ** -8)
