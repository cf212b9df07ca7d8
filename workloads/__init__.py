"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module draws random numbers, rounds them to the storage formats and lays
them out in the cache formats.  It holds none of the attention or projection
arithmetic.
"""

from .gen import (
    DecodeCase,
    QueryInputs,
    bf16_round_bits,
    config_case,
    config_query_inputs,
    make_decode_case,
    make_mtp_queries,
    make_query_inputs,
    make_sparse_indexer_inputs,
    SparseIndexerInputs,
    ragged_lengths,
    v_by_subblock,
    CONFIG_NAMES,
)

__all__ = [
    "DecodeCase",
    "QueryInputs",
    "bf16_round_bits",
    "config_case",
    "config_query_inputs",
    "make_decode_case",
    "make_mtp_queries",
    "make_query_inputs",
    "make_sparse_indexer_inputs",
    "SparseIndexerInputs",
    "ragged_lengths",
    "v_by_subblock",
    "CONFIG_NAMES",
]
