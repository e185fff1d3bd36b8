"""Seeded synthetic weights of the RNN head (the gated recurrent alternative to
the Markov head).  No trained head is available, so the weights are random with
the same storage type as the Markov factors; the scales keep the gates away
from saturation and the state bias comparable to the Markov bias.  Nothing
here is the head's arithmetic."""

import numpy as np

from .inputs import bf16_bits_from_f32

TID_RNN_WX, TID_RNN_WS, TID_RNN_B = 201, 202, 203


def make_rnn_weights(r, w_dtype, seed=0, scale_x=6.0, scale_s=1.5):
    """Wx, Ws [3, r, r] (update, reset, candidate gates; N(0, scale/sqrt(r))),
    bias float32 [3, r] (update N(0, 0.5), reset N(1, 0.5), candidate N(0, 0.3)).
    bf16 weights are returned as uint16 bit patterns, like W1/W2."""
    Wx = np.random.default_rng([seed, TID_RNN_WX]).normal(0.0, scale_x / np.sqrt(r), (3, r, r)).astype(np.float32)
    Ws = np.random.default_rng([seed, TID_RNN_WS]).normal(0.0, scale_s / np.sqrt(r), (3, r, r)).astype(np.float32)
    rb = np.random.default_rng([seed, TID_RNN_B])
    bias = np.stack([rb.normal(0.0, 0.5, r), rb.normal(1.0, 0.5, r), rb.normal(0.0, 0.3, r)]).astype(np.float32)
    if w_dtype == "bf16":
        Wx, Ws = bf16_bits_from_f32(Wx), bf16_bits_from_f32(Ws)
    return dict(Wx=Wx, Ws=Ws, bias=bias)
