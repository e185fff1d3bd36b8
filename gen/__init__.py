"""Seeded synthetic inputs for the DSpark draft -> schedule -> verify round.

This package is shared test and benchmark infrastructure.  It draws the
inputs of a round (base logits, Markov factors, anchors, confidences, cost
table, target logits and every uniform the round consumes) and holds none of
the method's arithmetic: no softmax, no sampling, no scheduling.
"""

from .configs import CONFIGS, config
from .inputs import make_inputs, bf16_bits_from_f32

__all__ = ["CONFIGS", "config", "make_inputs", "bf16_bits_from_f32"]
