"""Planted mistakes in the oracle (built on the CPU with -DDFKV_ORACLE_MUTANT=k) must each fail a pin.

Mutants: 1 off-by-one clamp, 2 dummy slot neither skipped nor reset, 3 RoPE halves' sin terms swapped,
4 wrong layer stride in the paged store, 5 transposed GEMM weight index, 6 RMSNorm sum instead of mean,
7 YaRN ramp reversed, 8 block placement past the allocation, 9 page count rounded down, 10 bonus token not counted, 11 row-store page bound off by one,
12 cos/sin angle formed in fp32.
"""
import os

import pytest

import oracle
from pins import ALL_PINS

MUTANTS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12]


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(mutant, tmp_path):
    lib = oracle.build(out=os.path.join(str(tmp_path), f"libdfkv_oracle_m{mutant}.so"), mutant=mutant, openmp=False)
    o = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, IndexError) as e:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant} passed every pin"
