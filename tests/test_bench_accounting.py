"""The algorithmic work that bench.py divides by its timings, counted by hand
on tiny inputs: decode bytes (K and V of every visible token, Q, O, the page
table entries in use and the context lengths) for both cache dtypes."""
import bench
import synth


def test_decode_bytes_bf16_by_hand():
    inp = synth.decode_inputs(1, 3, 4, 2, 64, context_lens=[1, 17, 40], spare_pages=2)
    kv = (1 + 17 + 40) * 2 * 64 * 2 * 2          # tokens x Hkv x D x 2 B x (K, V)
    q = o = 3 * 4 * 64 * 2                          # B x Hq x D x 2 B
    pages = (1 + 2 + 3) * 4                         # ceil(ctx / 16) entries of 4 B
    assert bench.decode_bytes(inp) == kv + q + o + pages + 3 * 4


def test_decode_bytes_fp8_halves_cache_and_query():
    inp = synth.decode_inputs(2, 2, 8, 1, 128, context_lens=[16, 33], spare_pages=1, dtype="fp8")
    kv = (16 + 33) * 1 * 128 * 1 * 2
    q = 2 * 8 * 128 * 1
    o = 2 * 8 * 128 * 2                             # the output stays bf16
    pages = (1 + 3) * 4
    assert bench.decode_bytes(inp) == kv + q + o + pages + 2 * 4
