"""D-Quant decode attention for MI355X (gfx950).

``decode_attention_dq_amd.dq`` is the Python binding of the C-ABI library
``libdq.so`` (hand-written HIP kernels); ``synth`` holds the seeded input
generators. Importing the package does not load the library; importing
``dq`` does, and fails loudly when the library is missing.
"""
