"""CPU pins of the oracle's fp64 paged attention and its split/combine form."""

import numpy as np

import oracle
import pins


def test_attention_pins():
    pins.pins_attention(oracle.attention, oracle.assign)


def test_fp8_gather_pins():
    pins.pins_attention_fp8(oracle.attention, oracle.e4m3)


def test_e4m3_pins():
    pins.pins_e4m3(oracle.e4m3)


def test_bf16_widening_matches_torch():
    import torch
    x = torch.randn(4096) * 100
    bits = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.attention.bf16_bits_to_f64(bits), ref)
