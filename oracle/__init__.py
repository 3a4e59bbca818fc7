"""fp64 CPU oracle of the BERT-style encoder forward (and of the decoder forward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package; the library never does, and this package
imports nothing of the library.  See ``oracle/fp64_encoder.py`` for what it computes
and which passage each function follows; ``oracle/fp64_decoder.py`` for the decoder.
"""
from .fp64_encoder import (LN_EPS, linear, split_heads, merge_heads, scaled_scores,
                      key_valid, masked_softmax, context, layer_norm, gelu_tanh,
                      encoder_layer, layer_steps, encoder, encoder_rows)
from .fp64_decoder import (DECODER_WEIGHT_NAMES, causal_softmax, decoder_layer_steps,
                           decoder_layer, decoder)

__all__ = ["LN_EPS", "linear", "split_heads", "merge_heads", "scaled_scores",
           "key_valid", "masked_softmax", "context", "layer_norm", "gelu_tanh",
           "encoder_layer", "layer_steps", "encoder", "encoder_rows",
           "DECODER_WEIGHT_NAMES", "causal_softmax", "decoder_layer_steps", "decoder_layer",
           "decoder"]
