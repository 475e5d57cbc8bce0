"""fp64 CPU oracle (test infrastructure only; see ``oracle.fp64``)."""
from .fp64 import (BLOCK_KEYS, CHUNK_KEYS, attention, attention_chunked, attention_flops,
                        chunk_partials, dequantize_e4m3, e4m3fn_table, gather_pages, paged_decode,
                        visible)

__all__ = ["BLOCK_KEYS", "CHUNK_KEYS", "attention", "attention_chunked", "attention_flops",
           "chunk_partials", "dequantize_e4m3", "e4m3fn_table", "gather_pages", "paged_decode",
           "visible"]
