"""CPU oracle for the D-Quant codec and its decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package. The product
path (the HIP library and its Python binding) never imports, calls or links
anything here, and nothing here comes from the HIP path.

Source: "D-Quant: Driftable Entropy Coding for KV Cache Quantization"
(Su, Liu, Yu, Zhu; arXiv 2609.19880). Section references below are to that
paper. The code is plain fp64 NumPy with exact integers for the rANS coder.
It is vectorised across independent streams only; every per-symbol step is
written out in the order the method takes it.

Modules
  tables     O1   static N(0,1)-derived entropy table (sections 3.1, 4.4)
  codec      O2-O10  rotation, normalisation, quantisation, drift, rANS
             encode/decode, reconstruction (sections 3.1, 4.1-4.3)
  attention  O11  fp64 GQA decode attention over reconstructed K/V
  means      O12  windowed INT8 channel-mean removal for keys (sections 3.2, 5)
  token      O13-O17  the per-token format: one 1024-value stream per token over
             all 8 KV heads, min-max affine grid, drift, rANS, least-squares
             refit with fp16 (o, s) (sections 4.2-4.5, 5.1; appendix
             "Compared configurations")
  measures   entropy, cross-entropy, coding gain, normal gap, NMSE (section 3.1/3.2)

Parity status: every function is pinned by the tests in ``tests/`` against
closed forms, library special cases, brute force or invariants the paper
states. No function here is "parity unpinned"; the absolute grid step and
therefore absolute NMSE values are engineering choices the paper leaves open.
"""
from .tables import (Table, make_table, default_step, FLUSH_BITS, STATE_LOW, STATE_BYTES,
                     COST_ONE)
from .codec import (fwht, normalize, nearest_level, drift_candidates, rans_encode, rans_enc_step, rans_dec_step,
                    rans_decode, encode_streams, decode_streams, reconstruct, EncodeResult)
from .attention import attention, attention_rotated
from .means import block_means, dequantize as dequantize_means, BLOCK as MEAN_BLOCK
from .token import (make_token_table, encode_tokens, decode_tokens, reconstruct_tokens, TokenEncodeResult,
                    TOKEN_N, TOKEN_HEADS)
from . import measures

__all__ = [
    "Table", "make_table", "default_step", "FLUSH_BITS", "STATE_LOW", "STATE_BYTES", "COST_ONE",
    "fwht", "normalize", "nearest_level", "drift_candidates", "rans_encode", "rans_decode",
    "rans_enc_step", "rans_dec_step",
    "encode_streams", "decode_streams", "reconstruct", "EncodeResult",
    "attention", "attention_rotated", "measures", "block_means", "dequantize_means", "MEAN_BLOCK",
    "make_token_table", "encode_tokens", "decode_tokens", "reconstruct_tokens", "TokenEncodeResult", "TOKEN_N",
    "TOKEN_HEADS",
]
