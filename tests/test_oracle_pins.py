"""The CPU oracle against its pins (hand-derived example, closed forms, library
routines on special cases, brute-force enumeration). CPU only."""
import types

import pytest

import oracle
import pins


def oracle_ns():
    return types.SimpleNamespace(
        OracleTrie=oracle.OracleTrie, expand_request=oracle.expand_request,
        masked_log_softmax=oracle.masked_log_softmax, decode=oracle.decode,
        lmhead_logits=oracle.lmhead_logits, widen_logits=oracle.widen_logits,
        decode_sampled=oracle.decode_sampled, noise_uniform=oracle.noise_uniform,
        splitmix64=oracle.splitmix64, gumbel=oracle.gumbel, score_catalog=oracle.score_catalog)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle_ns())
