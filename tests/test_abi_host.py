"""CPU tests of the C-ABI boundary: the library loads, exports every entry point
that include/detattn.h declares, and rejects malformed arguments on the host
with the documented status before any HIP call (so these run without a GPU:
no call here reaches a launch)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "detattn.h")

DA_OK, DA_EINVAL, DA_EUNSUPPORTED, DA_EWORKSPACE, DA_ELAUNCH = range(5)
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def lib():
    import deterministic_flash_attention_amd as dfa
    if not os.path.exists(dfa.library_path()):
        from deterministic_flash_attention_amd import build
        build.build()
    return dfa.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    assert names == sorted(["attn_status_str", "attn_num_chunks", "attn_partials_bytes",
                            "attn_extend_workspace_bytes",
                            "attn_prefill_fwd", "attn_decode_split_fwd",
                            "attn_paged_extend_fwd", "attn_chunk_merge",
                            "attn_decode_fwd_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    import deterministic_flash_attention_amd as dfa
    out = subprocess.run(["nm", "-D", "--defined-only", dfa.library_path()], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\sT\s(attn_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_small_helpers(lib):
    assert lib.attn_num_chunks(0) == 0 and lib.attn_num_chunks(1) == 1
    assert lib.attn_num_chunks(512) == 1 and lib.attn_num_chunks(513) == 2
    assert lib.attn_num_chunks(32768) == 64
    assert lib.attn_partials_bytes(8192, 32, 16, 128) == 8192 * 32 * 16 * 130 * 4
    assert lib.attn_partials_bytes(-1, 32, 16, 128) == 0
    lib.attn_extend_workspace_bytes.restype = ctypes.c_size_t
    assert lib.attn_extend_workspace_bytes(11, 32, 8, 64, 128) == (1 << 18) + 11 * 32 * 64 * 130 * 4
    assert lib.attn_extend_workspace_bytes(-1, 32, 8, 64, 128) == 0
    for s in range(5):
        assert lib.attn_status_str(s).decode().startswith("DA_")


def _prefill_args(**over):
    a = dict(dtype=0, q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, batch=1, max_q=300,
             max_k=300, total_q=300, total_k=300, hq=2, hkv=1, d=64, scale=0.125, causal=1,
             wl=-1, wr=-1, qd=1.0, kd=1.0, vd=1.0, schedule=0, o=FAKE, lse=None, part=None,
             part_bytes=0, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), DA_EINVAL),
    (dict(schedule=5), DA_EINVAL),
    (dict(causal=2), DA_EINVAL),
    (dict(d=80), DA_EUNSUPPORTED),
    (dict(hq=3, hkv=2), DA_EINVAL),
    (dict(hkv=0), DA_EINVAL),
    (dict(q=None), DA_EINVAL),
    (dict(cu_k=None), DA_EINVAL),
    (dict(o=None), DA_EINVAL),
    (dict(q=FAKE + 8), DA_EINVAL),          # misaligned
    (dict(scale=0.0), DA_EINVAL),
    (dict(scale=float("nan")), DA_EINVAL),
    (dict(qd=0.5), DA_EINVAL),              # descales must be 1 for bf16
    (dict(dtype=1, qd=0.0), DA_EINVAL),     # fp8 descales must be finite and positive
    (dict(batch=-1), DA_EINVAL),
    (dict(schedule=1, part=None), DA_EINVAL),
    (dict(schedule=1, part=FAKE, part_bytes=1024), DA_EWORKSPACE),
    (dict(max_q=1 << 30), DA_EUNSUPPORTED),  # beyond 32-bit descriptor offsets
    (dict(wl=-2), DA_EINVAL),               # windows are >= 0 or -1 (unbounded)
    (dict(wr=-5), DA_EINVAL),
])
def test_prefill_validation(lib, over, status):
    assert lib.attn_prefill_fwd(*_prefill_args(**over)) == status


def _decode_args(**over):
    a = dict(dtype=0, q=FAKE, kc=FAKE, vc=FAKE, num_pages=100, page_stride=16 * 8 * 128,
             token_stride=8 * 128, head_stride=128, table=FAKE, max_pages=64, ctx=FAKE,
             max_ctx=1024, wl=-1, batch=4, page_size=16, hq=32, hkv=8, d=128, scale=0.088,
             qd=1.0, kd=1.0, vd=1.0, schedule=1, part=FAKE, part_bytes=1 << 40, o=None, lse=None,
             stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(page_size=32), DA_EUNSUPPORTED),
    (dict(hq=64, hkv=1), DA_EUNSUPPORTED),   # more than 32 query heads per kv head
    (dict(max_ctx=64 * 16 + 1), DA_EINVAL),  # context beyond the page table
    (dict(num_pages=0), DA_EINVAL),
    (dict(token_stride=0), DA_EINVAL),
    (dict(head_stride=100), DA_EINVAL),      # 200-byte stride is not a multiple of 16
    (dict(table=None), DA_EINVAL),
    (dict(part=None), DA_EINVAL),
    (dict(part_bytes=4096), DA_EWORKSPACE),
    (dict(schedule=0, o=None), DA_EINVAL),
    (dict(d=96), DA_EUNSUPPORTED),
    (dict(vd=2.0), DA_EINVAL),
    (dict(wl=-3), DA_EINVAL),
])
def test_decode_validation(lib, over, status):
    assert lib.attn_decode_split_fwd(*_decode_args(**over)) == status


def _noalloc_args(**over):
    a = dict(dtype=0, q=FAKE, kc=FAKE, vc=FAKE, num_pages=100, page_stride=16 * 8 * 128,
             token_stride=8 * 128, head_stride=128, table=FAKE, max_pages=64, ctx=FAKE,
             max_ctx=1024, wl=-1, batch=4, page_size=16, hq=32, hkv=8, d=128, scale=0.088,
             qd=1.0, kd=1.0, vd=1.0, o=FAKE, lse=None, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(page_size=32), DA_EUNSUPPORTED),
    (dict(max_ctx=64 * 16 + 1), DA_EINVAL),
    (dict(o=None), DA_EINVAL),
    (dict(o=FAKE + 2), DA_EINVAL),
    (dict(d=96), DA_EUNSUPPORTED),
    (dict(vd=2.0), DA_EINVAL),
    # partials of 64 rows x 32 heads x 256 chunks x 130 x 4 B exceed the static scratch
    (dict(batch=64, max_pages=8192, max_ctx=8192 * 16), DA_EWORKSPACE),
])
def test_decode_noalloc_validation(lib, over, status):
    """The allocation-free decode rejects before any HIP call, so these run on
    the CPU; an oversized request is DA_EWORKSPACE."""
    assert lib.attn_decode_fwd_noalloc(*_noalloc_args(**over)) == status


def test_decode_noalloc_limit_matches_header(lib):
    import deterministic_flash_attention_amd as dfa
    text = open(HEADER).read()
    assert re.search(r"#define DA_DECODE_SCRATCH_BYTES \(\(size_t\)128 << 20\)", text)
    assert dfa.DECODE_SCRATCH_BYTES == 128 << 20
    # the full paged decode workload (64 sequences, contexts up to 32768) fits
    assert lib.attn_partials_bytes(64, 32, 64, 128) <= dfa.DECODE_SCRATCH_BYTES


def _extend_args(**over):
    a = dict(dtype=0, q=FAKE, cu_q=FAKE, kc=FAKE, vc=FAKE, num_pages=100,
             page_stride=16 * 8 * 128, token_stride=8 * 128, head_stride=128, table=FAKE,
             max_pages=64, ctx=FAKE, batch=4, max_q=300, max_ctx=1024, total_q=600,
             page_size=16, hq=32, hkv=8, d=128, scale=0.088, causal=1, wl=-1, wr=-1, qd=1.0,
             kd=1.0, vd=1.0, schedule=0, o=FAKE, lse=None, part=None, part_bytes=0, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(dtype=3), DA_EINVAL),
    (dict(schedule=2), DA_EINVAL),
    (dict(causal=-1), DA_EINVAL),
    (dict(page_size=8), DA_EUNSUPPORTED),
    (dict(d=256), DA_EUNSUPPORTED),
    (dict(hq=30, hkv=8), DA_EINVAL),
    (dict(max_ctx=64 * 16 + 1), DA_EINVAL),   # context beyond the page table
    (dict(num_pages=0), DA_EINVAL),
    (dict(page_stride=-5), DA_EINVAL),
    (dict(token_stride=4), DA_EINVAL),        # 8-byte stride is not a multiple of 16
    (dict(token_stride=64), DA_EINVAL),       # tokens closer than one head row (D = 128)
    (dict(token_stride=1 << 26), DA_EUNSUPPORTED),  # a page beyond 32-bit offsets
    (dict(cu_q=None), DA_EINVAL),
    (dict(table=None), DA_EINVAL),
    (dict(ctx=None), DA_EINVAL),
    (dict(kc=FAKE + 4), DA_EINVAL),           # misaligned cache
    (dict(o=None), DA_EINVAL),
    (dict(scale=float("inf")), DA_EINVAL),
    (dict(kd=3.0), DA_EINVAL),                # descales must be 1 for bf16
    (dict(schedule=1, part=None), DA_EINVAL),
    (dict(schedule=1, part=FAKE, part_bytes=4096), DA_EWORKSPACE),
    (dict(part=FAKE, part_bytes=4096), DA_EWORKSPACE),   # monolithic, workspace too small
    (dict(part=FAKE + 4, part_bytes=1 << 30), DA_EINVAL),  # monolithic, misaligned workspace
    (dict(part=FAKE, part_bytes=1 << 40, batch=70000, hkv=1, hq=1), DA_EUNSUPPORTED),  # > 65536 counters
    (dict(max_q=1 << 28), DA_EUNSUPPORTED),   # beyond 32-bit descriptor offsets
    (dict(wl=-7), DA_EINVAL),
    (dict(batch=0), DA_OK),                   # no work: nothing launched
])
def test_paged_extend_validation(lib, over, status):
    assert lib.attn_paged_extend_fwd(*_extend_args(**over)) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, 1 << 40, -1, 32, 4, 128, 1.0, FAKE, None, None), DA_EINVAL),
    ((FAKE, 1 << 40, 64, 0, 4, 128, 1.0, FAKE, None, None), DA_EINVAL),
    ((FAKE, 1 << 40, 64, 32, 4, 100, 1.0, FAKE, None, None), DA_EUNSUPPORTED),
    ((FAKE, 1 << 40, 64, 32, 4, 128, 0.0, FAKE, None, None), DA_EINVAL),
    ((FAKE, 1 << 40, 64, 32, 4, 128, 1.0, None, None, None), DA_EINVAL),
    ((FAKE, 100, 64, 32, 4, 128, 1.0, FAKE, None, None), DA_EWORKSPACE),
    ((None, 1 << 40, 64, 32, 4, 128, 1.0, FAKE, None, None), DA_EINVAL),
])
def test_merge_validation(lib, args, status):
    assert lib.attn_chunk_merge(*args) == status


def test_zero_work_calls_return_ok_without_launch(lib):
    # batch 0 and zero rows are no-ops that succeed before any HIP call
    assert lib.attn_prefill_fwd(*_prefill_args(batch=0)) == DA_OK
    assert lib.attn_chunk_merge(None, 0, 0, 32, 0, 128, 1.0, None, None, None) == DA_OK


# ---------------------------------------------------------------- GEMM boundary
GEMM_HEADER = os.path.join(ROOT, "include", "detgemm.h")


def gemm_declared_functions():
    text = open(GEMM_HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(det_gemm_\w+)\s*\(", text,
                                 re.M)))


def test_gemm_header_declares_entry_points_and_library_exports_them(lib):
    import deterministic_flash_attention_amd as dfa
    names = gemm_declared_functions()
    assert names == sorted(["det_gemm_num_chunks", "det_gemm_workspace_bytes",
                            "det_gemm_num_configs", "det_gemm_config_tile", "det_gemm_fwd"])
    out = subprocess.run(["nm", "-D", "--defined-only", dfa.library_path()], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\sT\s(det_gemm_\w+)", out))
    for name in names:
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_gemm_small_helpers(lib):
    import deterministic_flash_attention_amd as dfa
    assert [dfa.det_gemm_num_chunks(k) for k in (0, 1, 1024, 1025, 4096)] == [0, 1, 1, 2, 4]
    assert dfa.det_gemm_workspace_bytes(8, 1536, 4096) == 4 * 8 * 1536 * 4
    assert dfa.det_gemm_workspace_bytes(8, 1536, 0) == 0
    assert dfa.det_gemm_workspace_bytes(-1, 8, 8) == 0
    n = dfa.det_gemm_num_configs()
    assert n >= 1
    tiles = [dfa.det_gemm_config_tile(c) for c in range(n)]
    assert all(bm % 32 == 0 and bn % 32 == 0 for bm, bn in tiles)
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.det_gemm_config_tile(n, ctypes.byref(bm), ctypes.byref(bn)) == DA_EINVAL
    assert lib.det_gemm_config_tile(-1, ctypes.byref(bm), ctypes.byref(bn)) == DA_EINVAL


def _gemm_args(**over):
    args = dict(a=FAKE, lda=4096, w=FAKE, ldw=4096, layout=0, c=FAKE, ldc=6144, m=4096, n=6144,
                k=4096, schedule=0, config=-1, ws=None, ws_bytes=0, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("over,status", [
    (dict(layout=2), DA_EINVAL),
    (dict(schedule=2), DA_EINVAL),
    (dict(m=-1), DA_EINVAL),
    (dict(k=-8), DA_EINVAL),
    (dict(config=99), DA_EINVAL),
    (dict(config=-2), DA_EINVAL),
    (dict(n=6140, ldc=6144), DA_EUNSUPPORTED),      # N not a multiple of 8
    (dict(k=4092, lda=4096, ldw=4096), DA_EUNSUPPORTED),  # K not a multiple of 8
    (dict(a=None), DA_EINVAL),
    (dict(w=None), DA_EINVAL),
    (dict(c=None), DA_EINVAL),
    (dict(a=FAKE + 8), DA_EINVAL),                  # misaligned
    (dict(lda=4000), DA_EINVAL),                    # lda < K
    (dict(lda=4100), DA_EINVAL),                    # lda not a multiple of 8
    (dict(ldw=4000), DA_EINVAL),                    # [N, K] weight: ldw < K
    (dict(layout=1, ldw=4096), DA_EINVAL),          # [K, N] weight: ldw < N
    (dict(ldc=6000), DA_EINVAL),                    # ldc < N
    (dict(schedule=1), DA_EINVAL),                  # split without workspace
    (dict(schedule=1, ws=FAKE, ws_bytes=100), DA_EWORKSPACE),
    (dict(lda=1 << 24), DA_EUNSUPPORTED),           # a tile's byte extent beyond 2^31
])
def test_gemm_validation(lib, over, status):
    assert lib.det_gemm_fwd(*_gemm_args(**over)) == status


def test_gemm_zero_work_returns_ok_without_launch(lib):
    assert lib.det_gemm_fwd(*_gemm_args(m=0, a=None, c=None)) == DA_OK
    assert lib.det_gemm_fwd(*_gemm_args(n=0, w=None, c=None)) == DA_OK


def test_cache_layout_strides():
    """The Python mirror's element strides for the two paged-cache layouts."""
    import torch
    import deterministic_flash_attention_amd as dfa
    nhd = torch.empty(10, 16, 8, 128)
    hnd = torch.empty(10, 8, 16, 128)
    assert dfa._cache_geometry(nhd, "NHD") == (10, 16, 8, 128, 16 * 8 * 128, 8 * 128, 128)
    assert dfa._cache_geometry(hnd, "HND") == (10, 16, 8, 128, 8 * 16 * 128, 128, 16 * 128)
    with pytest.raises(ValueError):
        dfa._cache_geometry(nhd, "NDH")
