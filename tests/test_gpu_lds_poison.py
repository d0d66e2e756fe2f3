"""The LDS-poison A/B build (build variant "poison") on every kernel instance.

That build fills each kernel's LDS with NaN bits before the first load or
write reaches it, and the epilogue's staging region and the split-K
reduction region the same way before they are written.  Any fragment read
of a slot that the loads of its stage have not filled (a read before its
write, a stage handed over too early, an edge chunk skipped instead of
zero-filled) then puts NaN into the products that use it.  On integer inputs
the result is unique, so every instance must still match the oracle bit for
bit ("Lds Optimization", "LDS Instruction Model": LDS accesses complete in
order only within a wave; "Verification Checklist": every read must see the
write it depends on).  The cases are those of the every-kernel test.
"""
import pytest

import lds_staged_matrix_amd as lsm
from test_gpu_every_kernel import ALL_LAYOUTS, CASES16, CASES8, DTYPES16, DTYPES8, check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def poison():
    lib = lsm.ablation_library("poison")
    h = lib.gemm_create()
    yield lib, h
    lib.gemm_destroy(h)


@pytest.mark.parametrize("case", CASES16, ids=lambda c: c[0])
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gd", DTYPES16)
def test_poison_build_16bit(poison, case, la, lb, gd):
    cls, M, N, K = case
    check(cls, M, N, K, la, lb, gd, 900 + 10 * gd, "int", lib=poison, what="lds-poison")


@pytest.mark.parametrize("case", CASES8, ids=lambda c: c[0])
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gd", DTYPES8)
def test_poison_build_8bit(poison, case, la, lb, gd):
    cls, M, N, K = case
    check(cls, M, N, K, la, lb, gd, 950 + 10 * gd, "int", lib=poison, what="lds-poison")
