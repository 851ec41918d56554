"""A plausible mistake planted in the oracle (on the CPU, in a throw-away build)
makes at least one pin fail. This shows the pins constrain the oracle."""
import os

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

PLANTS = ["quant_round_away", "drop_sk", "alpha_sign", "no_alpha", "l_no_rescale", "transpose_v",
          "causal_off_by_one", "gqa_wrong_head", "v_head_no_batch", "lut_half_step", "lut_round_index",
          "lut_no_clip", "lut_no_query_scale", "v_channel_no_head", "v_channel_transposed",
          "cols_no_group", "q4_qmax_8", "fwht_sign", "fwht_no_norm", "no_log2e", "bias_sign",
          "no_bias_nudge"]


@pytest.mark.parametrize("plant", PLANTS)
def test_planted_mistake_is_caught(plant, tmp_path):
    path = obuild.build(out=os.path.join(str(tmp_path), "liboracle_%s.so" % plant), plant=plant)
    L = oracle.lib(path)
    failed = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(L)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, "planted mistake %r passed every pin" % plant
