"""CPU oracle for the int4 KIVI paged KV cache -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct numpy model of what the GPU
library computes. It exists to check the GPU path and nothing else:

* only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
  ``bench.py`` may import it;
* it shares no code, header, table or constant with the HIP library under
  ``int4_kivi_quantized_amd/`` and neither side imports the other;
* the product path never falls back to it.

Sources (cited by page title and section):

* S4 KV product page, "int4 KV-Cache-Kompression fuer vLLM" (abyo.net/de/s4/s4-kv),
  header paragraph and "Funktionsweise" step 1: the cache is stored as
  asymmetric int4 in KIVI style, KEY quantized per channel, VALUE per token;
  models with head_dim 128 and standard attention.
* PagedAttention explainers (gyaansetu.com "KV-Cache und PagedAttention",
  section "Wie PagedAttention das loest"; polaris7.io signal page, "Wichtigste
  Kernpunkte & Evidenz"): the cache is cut into fixed-size token pages
  (16 tokens) reached through a page table.

* ``oracle.fp8``: the FP8 (E4M3) KV-cache variant with per-KV-head scales,
  from the KV-quantization guide on adechristanto.de (sections on attention
  arithmetic in the quantized domain and on default / calibrated scales) and
  the OCP E4M3 format definition.

Where the pages leave a step open, the oracle takes one plain reading; each
reading is named in the docstring of the function that takes it.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
against closed forms, special cases, brute force or library routines.
"""

from .quant import QMAX, quantize_groups, dequantize, flush_pages, dequantize_pages
from .cache import PAGE, sequence_cache, dequantized_sequence
from .attention import decode_attention, decode_attention_batch, multiquery_attention

__all__ = [
    "QMAX",
    "PAGE",
    "quantize_groups",
    "dequantize",
    "flush_pages",
    "dequantize_pages",
    "sequence_cache",
    "dequantized_sequence",
    "decode_attention",
    "decode_attention_batch",
    "multiquery_attention",
]
