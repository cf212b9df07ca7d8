"""Plain, slow, fp64 CPU oracle for the MFA decode-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call or link anything under ``oracle/``.  Only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  The oracle shares no code with the GPU path: it has its own storage
decoders, its own block-table walk and its own softmax.

What it computes, and which passage each function follows:

* :func:`decode_attention` -- softmax attention of one new query token per
  slot over that slot's cached keys/values.  MFA case: 64 query heads sharing
  one K head and one V head of width 256 ("Step-3 is Large yet Affordable",
  section 2 "Step-3 model card" and Table 1).  GQA / window case: head ``h``
  reads KV group ``floor(h / (Hq/Hkv))`` and the scaled-dot-product softmax
  equation of "Step-5-Preview: Sparse GQA, Indexer und KV-Speicher", section
  "Die eigentliche Attention liest weiterhin originale K/V"; the sliding window
  counts the current token (same page, backbone table).  The context length
  includes the token just appended (duck-llm chapter 7 "decode fixed cost
  reduction", section 7.6, the active-length off-by-one).
* :func:`query_proj` -- the low-rank query path: down-projection to the
  2048 rank, normalisation, up-projection to 64 x 256 (Step-3 report,
  section 2).
* :func:`kv_append` -- the step before decode attention: write each slot's
  new K/V token at its current length and advance the length on the device
  (duck-llm chapter 7, sections 7.5 and 7.6); :func:`e4m3fn_encode` is the
  brute-force nearest-code FP8 encoder it uses for FP8 caches.
* :func:`decode_attention_mtp` -- several new query tokens per sequence (MTP
  drafts or a speculative verify, Step-3 report section 5.2), causal among
  themselves: token t of Tq attends the first L - (Tq - 1 - t) keys.
* :mod:`oracle.sparse` -- Step-5 sparse global attention for a decode token
  ("Step-5-Preview" page, indexer and attention sections): coordinatewise
  block summaries, weighted-ReLU scores on E4M3-rounded operands, causal
  top-512 selection with ties to the lower id plus the current block, and
  softmax attention over the selected original K/V.
* :mod:`oracle.codecs` -- bf16 and OCP FP8 E4M3 (E4M3FN) storage decoders.

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: brute-force loops on tiny inputs, torch's CPU scaled-dot-product
attention in float64, closed forms (L = 1 returns V, q = 0 returns the mean of
V, RMSNorm mean square), invariants (block permutation, 64 independent
single-head attentions, window >= L equals dense), all 256 E4M3 codes
against torch's float8_e4m3fn, and the pages' own printed byte/FLOP figures
for the accounting model.
"""

from .codecs import bf16_bits_to_f64, e4m3fn_codes_to_f64, decode_storage
from .attention import decode_attention
from .query_proj import query_proj, rms_norm
from .kv_append import e4m3fn_encode, kv_append
from .mtp import decode_attention_mtp, mtp_lengths

__all__ = [
    "bf16_bits_to_f64",
    "e4m3fn_codes_to_f64",
    "decode_storage",
    "decode_attention",
    "query_proj",
    "rms_norm",
    "e4m3fn_encode",
    "kv_append",
    "decode_attention_mtp",
    "mtp_lengths",
]
