"""CPU checks of the GPU tests' comparison helpers (no GPU): the re-rotation
choices reproduce the oracle's own rounding, a difference is accepted only at
an element marked ambiguous and only as its other fp16 neighbour, and a
requantized group is accepted only as the quantization of such a choice."""
import numpy as np
import pytest

from oracle import cache as oc
from oracle import quant, rope
from tiered_quantized_kv_amd import synth

from .gpu_helpers import adopt_fp16_rerope, adopt_group_rerope, rerope_choices


def _cfg():
    return oc.Config(head_dim=64, n_q_heads=8, n_kv_heads=2, n_sink=4, recent_window=8, int4_budget=10,
                     rope_theta=1e4)


def test_choices_reproduce_oracle_rounding():
    c = _cfg()
    x = synth.normal(synth.rng(7), 2, 50, 64).astype(np.float16)
    old = np.arange(1000, 1050)
    new = np.arange(10, 60)
    y16, nb, amb = rerope_choices(x, old, new, c)
    assert np.array_equal(y16.view(np.uint16), rope.rerope_fp16(x, old, new, c.freqs()).view(np.uint16))
    # neighbours are one fp16 step away on the side of the float64 value
    assert np.all(np.abs(nb.astype(np.float64) - y16.astype(np.float64)) > 0)
    assert amb.mean() < 1e-3


def test_fp16_difference_accepted_only_where_ambiguous():
    c = _cfg()
    x = synth.normal(synth.rng(8), 2, 20, 64).astype(np.float16)
    y16, nb, amb = rerope_choices(x, np.arange(500, 520), np.arange(4, 24), c)
    amb = np.zeros_like(amb)
    amb[1, 3, 5] = True
    gpu = y16.copy()
    gpu[1, 3, 5] = nb[1, 3, 5]
    got = adopt_fp16_rerope(gpu, y16, (y16, nb, amb))
    assert got[1, 3, 5] == nb[1, 3, 5]
    gpu[0, 0, 0] = nb[0, 0, 0]                    # not ambiguous
    with pytest.raises(AssertionError):
        adopt_fp16_rerope(gpu, y16, (y16, nb, amb))


def test_group_requantization_accepted_only_as_a_choice():
    c = _cfg()
    x = synth.normal(synth.rng(9), 2, 6, 64).astype(np.float16)
    y16, nb, amb = rerope_choices(x, np.arange(300, 306), np.arange(4, 10), c)
    amb = np.zeros_like(amb)
    # make the group's largest element ambiguous so its flip moves the scale
    j = int(np.argmax(np.abs(y16[0, 2, :32].astype(np.float64))))
    amb[0, 2, j] = True
    u, s = quant.quantize(y16, 4, 32)
    z = y16.copy()
    z[0, 2, j] = nb[0, 2, j]
    gu, gs = quant.quantize(z, 4, 32)
    packed = quant.pack(gu, 4)
    ou, os_ = adopt_group_rerope(packed, gs, u, s, (y16, nb, amb), 4)
    assert np.array_equal(ou, gu) and np.array_equal(os_.view(np.uint16), gs.view(np.uint16))
    # a change in a group without an ambiguous element is refused
    bad = gu.copy()
    bad[1, 0, 0] = (int(bad[1, 0, 0]) % 15) + 1
    with pytest.raises(AssertionError):
        adopt_group_rerope(quant.pack(bad, 4), gs, u, s, (y16, nb, amb), 4)
