"""few_row_vocab_amd -- the few-row draft-head vocabulary projection on MI355X (gfx950).

The product is the C-ABI library libdh.so (include/dh.h) built from csrc/*.hip; this package
holds it, its build script and a thin Python binding (dh.py).
"""
from . import dh
from .dh import (BF16, FP8_BLOCK32, FP8_ROW, OUT_ADD_BF16, OUT_BF16, OUT_F32, DHError, Head,
                 draft, draft_lowrank, draft_mapped, gather_rows, gemv, linear, quantize,
                 rescore, sample, topk, topk_mapped, topk_softmax, workspace, workspace_bytes)

__all__ = ["dh", "BF16", "FP8_BLOCK32", "FP8_ROW", "OUT_ADD_BF16", "OUT_BF16", "OUT_F32",
           "DHError", "Head", "draft", "draft_lowrank", "draft_mapped", "gather_rows", "gemv",
           "linear", "quantize", "rescore", "sample", "topk", "topk_mapped", "topk_softmax",
           "workspace", "workspace_bytes"]
