"""Pins of the exact bf16 rounding helper used by the output-rounding GPU tests
(CPU only): hand-worked ties and near-ties, the bit patterns of a few values,
and agreement with torch's float32 -> bfloat16 conversion (round to nearest
even) on every constructed column sum, each of which is exact in float32."""
from fractions import Fraction as F

import torch

from bf16_rounding import bf16_bits, halfway_columns, rne_bf16


def test_hand_worked_ties_and_near_ties():
    u = F(1, 256)  # half an ulp of 1.0 in bf16
    assert rne_bf16(1 + u) == 1                      # tie, 1.0000000b is even
    assert rne_bf16(1 + 3 * u) == 1 + 4 * u          # tie between ...001 and ...010 -> even
    assert rne_bf16(1 + u + u / 16) == 1 + 2 * u     # just above the tie
    assert rne_bf16(1 + u - u / 16) == 1             # just below the tie
    assert rne_bf16(2 - u / 2) == 2                  # carries into the next binade
    assert rne_bf16(-(1 + 3 * u)) == -(1 + 4 * u)
    assert rne_bf16(F(3, 1)) == 3 and rne_bf16(F(0)) == 0


def test_bit_patterns():
    assert bf16_bits(F(1)) == 0x3F80
    assert bf16_bits(F(-2)) == 0xC000
    assert bf16_bits(1 + F(1, 128)) == 0x3F81
    assert bf16_bits(F(1, 8)) == 0x3E00


def test_agrees_with_torch_rne_on_the_constructed_sums():
    cols = halfway_columns(128)
    kinds = set()
    for addends, x in cols:
        assert sum(addends) == x
        f = torch.tensor([float(x)], dtype=torch.float64).to(torch.float32)
        assert F(f.item()) == x, "the sum must be exact in float32"
        got = int(f.to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        assert got == bf16_bits(rne_bf16(x)), (x, hex(got))
        for a in addends:  # every addend is a bf16 value
            assert F(torch.tensor([float(a)]).to(torch.bfloat16).double().item()) == a
        kinds.add(rne_bf16(x) != rne_bf16(x + F(1, 2 ** 40)))
    assert kinds == {True, False}  # both exact ties and non-ties are present
