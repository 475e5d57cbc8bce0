"""Batch-invariant GEMM on the GPU (RL-Kernel page "MFMA batch-invariant GEMM and
chunked Triton attention", section 1): parity with the fp64 oracle under the
derived one-rounding bound, and the page's invariance claims as bitwise
checks: every tile configuration, both weight layouts ([N, K] view and [K, N]
prepared), M (sub-batches), strided rows and the split-K decode schedule give
the same bits.  Row-stride padding is NaN-poisoned where it must not be read."""
import numpy as np
import pytest
import torch

import synth
from gpu_utils import assert_bitwise, compare_gemm, gemm_views, note, oracle_gemm, run_gemm

pytestmark = pytest.mark.gpu

MONO, SPLIT = 0, 1


def _dfa():
    import deterministic_flash_attention_amd as dfa
    return dfa


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
@pytest.mark.parametrize("kn", [False, True])
@pytest.mark.parametrize("m,n,k", [(1, 8, 8), (37, 40, 64), (300, 200, 1000), (130, 264, 2504),
                                   (65, 136, 1032), (513, 392, 4096)])
def test_gemm_parity(m, n, k, kn, schedule):
    inp = synth.gemm_inputs(101, m, n, k, weight_kn=kn)
    note(f"gemm parity m={m} n={n} k={k} kn={kn} schedule={schedule}")
    c = run_gemm(inp, schedule)
    ref, absprod = oracle_gemm(inp)
    compare_gemm(c, ref, absprod, k, label=f"C {m}x{n}x{k} kn={kn} s={schedule}")


def test_all_configs_layouts_schedules_bitwise():
    """Every tile configuration x weight layout x schedule: identical bits."""
    dfa = _dfa()
    m, n, k = 300, 264, 2600
    nk = synth.gemm_inputs(103, m, n, k, weight_kn=False)
    kn = synth.GemmInputs(nk.a, nk.w.t().contiguous(), m, n, k, True, nk.seed)
    base = run_gemm(nk, MONO, config=0)
    ref, absprod = oracle_gemm(nk)
    compare_gemm(base, ref, absprod, k, label="config 0 NK mono")
    for cfg in range(dfa.det_gemm_num_configs()):
        for inp in (nk, kn):
            for sched in (MONO, SPLIT):
                note(f"config {cfg} {dfa.det_gemm_config_tile(cfg)} kn={inp.weight_kn} s={sched}")
                c = run_gemm(inp, sched, config=cfg)
                assert_bitwise(c, base, f"config {cfg} kn={inp.weight_kn} schedule {sched}")


@pytest.mark.parametrize("kn", [False, True])
def test_rows_do_not_depend_on_m_or_offset(kn):
    """A row's result is the same in the full batch, in any sub-batch (at any
    offset inside a tile) and alone."""
    m, n, k = 777, 136, 2056
    inp = synth.gemm_inputs(105, m, n, k, weight_kn=kn)
    full = run_gemm(inp, MONO)
    a, _ = gemm_views(inp)
    for r0, r1 in [(0, 1), (5, 70), (13, 14), (300, 777), (1, 600)]:
        for sched in (MONO, SPLIT):
            sub = run_gemm(inp, sched, a=a[r0:r1])
            assert_bitwise(sub, full[r0:r1], f"rows {r0}:{r1} schedule {sched}")


@pytest.mark.parametrize("kn", [False, True])
def test_strided_rows_and_poisoned_padding(kn):
    """Operands with padded row strides (padding = NaN) and an output written
    into a wider buffer: same bits as the packed call, padding never read,
    cells outside C untouched."""
    m, n, k = 200, 264, 1000
    packed = synth.gemm_inputs(107, m, n, k, weight_kn=kn)
    padded = synth.gemm_inputs(107, m, n, k, weight_kn=kn, pad_a=24, pad_w=40, poison=True)
    assert torch.equal(padded.a[:, :k], packed.a)
    c0 = run_gemm(packed, MONO)
    big = torch.full((m + 5, n + 16), 3.0, dtype=torch.bfloat16, device="cuda")
    for sched in (MONO, SPLIT):
        big.fill_(3.0)
        run_gemm(padded, sched, out=big[:m, :n])
        assert_bitwise(big[:m, :n], c0, f"strided rows schedule {sched}")
        assert torch.all(big[m:] == 3.0) and torch.all(big[:, n:] == 3.0), "wrote outside C"


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
def test_k_zero_gives_positive_zero(schedule):
    dfa = _dfa()
    a = torch.empty(70, 0, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(40, 0, dtype=torch.bfloat16, device="cuda")
    c = torch.full((70, 40), 5.0, dtype=torch.bfloat16, device="cuda")
    dfa.gemm(a, w, schedule=schedule, out=c)
    torch.cuda.synchronize()
    assert torch.all(c.view(torch.int16) == 0), "K = 0 must give +0"


def test_empty_m_and_n_write_nothing():
    dfa = _dfa()
    w = torch.randn(16, 64, device="cuda").to(torch.bfloat16)
    c = torch.empty(0, 16, dtype=torch.bfloat16, device="cuda")
    dfa.gemm(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), w, out=c)
    a = torch.randn(5, 64, device="cuda").to(torch.bfloat16)
    w0 = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    c0 = torch.empty(5, 0, dtype=torch.bfloat16, device="cuda")
    dfa.gemm(a, w0, out=c0)
    torch.cuda.synchronize()


def test_chunk_boundary_values():
    """Integer-valued operands whose exact sums are representable: the result
    is exact (closed form of the oracle's pin), across chunk boundaries."""
    m, n, k = 48, 64, 3072
    a = torch.zeros(m, k)
    w = torch.zeros(n, k)
    a[:, ::64] = 1.0                       # one non-zero per 64-block
    w[:, ::64] = torch.arange(n)[:, None].float()
    want = (k // 64) * torch.arange(n).float()[None, :].expand(m, n)
    inp = synth.GemmInputs(a.to(torch.bfloat16), w.to(torch.bfloat16), m, n, k, False, 0)
    for sched in (MONO, SPLIT):
        c = run_gemm(inp, sched)
        assert torch.equal(c.float().cpu(), want.to(torch.bfloat16).float()), f"schedule {sched}"


@pytest.mark.parametrize("name,m,n,k", synth.GEMM_SHAPES)
def test_full_shapes_and_schedules(name, m, n, k):
    """The benchmark's layer shapes at full size: every element against the
    oracle, and monolithic = split bit for bit."""
    inp = synth.gemm_inputs(0, m, n, k)
    note(f"full gemm {name} {m}x{n}x{k}")
    c_mono = run_gemm(inp, MONO)
    c_split = run_gemm(inp, SPLIT)
    assert_bitwise(c_mono, c_split, f"{name} monolithic vs split")
    ref, absprod = oracle_gemm(inp)
    compare_gemm(c_mono, ref, absprod, k, label=f"{name} all {ref.size} elements")
