"""The CPU oracle against facts fixed outside it (closed forms, IEEE 754,
brute force, library routines). See tests/pins.py for each fact."""

import types

import pytest

import oracle
from tests import pins


def oracle_ns():
    return types.SimpleNamespace(
        quantize_groups=oracle.quantize_groups,
        dequantize=oracle.dequantize,
        flush_pages=oracle.flush_pages,
        sequence_cache=oracle.sequence_cache,
        dequantized_sequence=oracle.dequantized_sequence,
        decode_attention=oracle.decode_attention,
    )


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle_ns())
