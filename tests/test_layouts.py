"""CPU checks of the operand layouts the GPU models assume (test code only).

The FP8 MFMA model of the kernel's row sum and PV (tests/fp8_model.py)
groups a 128-key tile's P codes as the kernel's operands hold them, and the
V^T layout (include/sage.h, sage_quant_v) permutes keys within 64-key groups
so that PV needs no shuffles. These tests pin that the two descriptions fit
together, so the GPU model tests cannot pass on a layout mistake that
cancels out.
"""
import numpy as np

from fp8_model import rowsum_key_groups
from gpu_common import kappa


def test_rowsum_groups_partition_the_tile():
    g = rowsum_key_groups()
    assert g.shape == (16, 8)
    assert sorted(g.ravel().tolist()) == list(range(128))


def test_vt_slots_of_each_group_are_one_operand_run():
    """MFMA w of a tile reads V^T bytes [64 w + 32 h, +32) for lane half h,
    and the P operand's bytes in the same order; a group is 8 consecutive
    bytes of those 32. So the V^T slots of a group's keys must be 8
    consecutive slots starting at a multiple of 8, inside one lane half's
    run of 32."""
    slot_of = {}
    for p in range(64):
        slot_of[kappa(p)] = p
    for gi, keys in enumerate(rowsum_key_groups()):
        w = keys[0] // 64
        assert all(k // 64 == w for k in keys), gi
        slots = [64 * w + slot_of[k % 64] for k in keys]
        assert slots == list(range(slots[0], slots[0] + 8)), (gi, slots)
        assert slots[0] % 8 == 0
        h = (slots[0] % 64) // 32
        assert gi == 8 * w + 4 * h + (slots[0] % 32) // 8, gi


def test_kappa_is_a_permutation_of_each_64_key_group():
    assert sorted(kappa(p) for p in range(64)) == list(range(64))
