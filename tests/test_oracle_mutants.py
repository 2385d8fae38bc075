"""Each planted mistake in the oracle (built on the CPU with -DORC_PLANT=n)
must fail at least one pin: evidence the pins can see such mistakes.

Planted mistakes: 1 gate/up rows swapped, 2 ties to the higher expert index,
3 W_down read transposed, 4 unstable permutation, 5 MXFP4 nibble order
swapped, 6 silu sign error, 7 routing weights not normalised, 8 NaN logits
compared raw, 20 quantizer
ties to the odd code, 21 quantizer shared exponent one octave high, 22
quantizer keeps negative zero, 30 silu derivative missing a term, 31 W_down
gradient written transposed, 32 router gradient without the softmax mean
term, 40 packed order: up rows taken from the gate half, 41 packed order:
chunk base from the chunk's own width, 42 packed order: scale slots with
(g, t) swapped."""
import pytest

import oracle
from tests import oracle_pins

PLANTS = {1: "gate_up_swapped", 2: "tie_to_higher_index", 3: "down_transposed", 4: "unstable_permute",
          5: "nibble_order_swapped", 6: "silu_sign", 7: "weights_unnormalised", 8: "nan_logits_raw",
          20: "quant_ties_odd",
          21: "quant_exponent_high", 22: "quant_negative_zero", 30: "bwd_silu_grad", 31: "bwd_down_transposed",
          32: "bwd_router_mean", 40: "pack_up_rows", 41: "pack_chunk_base", 42: "pack_scale_slots"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_mistake_is_caught(plant, tmp_path):
    path = oracle.build(plant=plant, out=str(tmp_path / f"liboracle_plant{plant}.so"))
    mutant = oracle.Oracle(path)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {PLANTS[plant]} passed every pin"
