"""Seeded synthetic inputs for the five workloads, shared by the tests, the
bench and the oracle.  This module holds none of the method's arithmetic:
it draws random numbers, casts them to the storage dtypes and lays out page
tables.  Both the oracle and the HIP path consume exactly these arrays.

Shapes follow the pages' workloads: Llama-2-7B attention shapes
(32 heads x d128, fp16 KV) from the Quest page (§0 and §2, eq. (9)-(12)),
page sizes and budgets from the same page (§2 and §2.2), and the 64K
context / FP8 E4M3 KV / BF16 query / neighbouring-query overlap structure of
the PageWeaver notes.  No dataset or model weights are used: real-model
keys are replaced by i.i.d. draws with the stated distributions.

RNG: numpy ``default_rng(SeedSequence([seed, stream, index...]))`` drawing
float32 (or float64 for Student-t), then cast with round-to-nearest-even:
numpy for fp16, torch CPU casts for bf16 and float8_e4m3fn.
"""
from .cases import (DecodeCase, ChunkCase, tiny_single_head, llama2_7b_layer, batched_gqa_append,
                    multiquery_chunk, stress_long_context, corrupt_lists, worked_example_case,
                    figure2_case, layer_queries, STEP_STREAM)

__all__ = ["DecodeCase", "ChunkCase", "tiny_single_head", "llama2_7b_layer", "batched_gqa_append",
           "multiquery_chunk", "stress_long_context", "corrupt_lists", "worked_example_case",
           "figure2_case", "layer_queries", "STEP_STREAM"]
