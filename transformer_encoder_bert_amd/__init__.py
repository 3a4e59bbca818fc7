"""ftx: forward pass of a BERT-style Transformer encoder (and of a decoder built from the
same kernels) on AMD MI355X (gfx950).

The compute path is libftx.so (hand-written HIP kernels behind a C ABI, see
include/ftx.h and include/ftx_decoder.h); ``transformer_encoder_bert_amd.ftx`` is its
ctypes binding (``Encoder``, ``Decoder``).  Importing
this package does not load the library; the binding loads it on first use and raises
if it has not been built.  ``transformer_encoder_bert_amd.torch_op`` registers the forward
as the PyTorch operator ``torch.ops.ftx.encoder_forward``.
"""
__all__ = ["ftx", "torch_op"]
