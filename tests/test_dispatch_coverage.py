"""Host-side check (no GPU) that the GPU parity tests reach every kernel
instantiation the C-ABI can launch.

qg_kernel_for reports, by name, the instantiation the launchers pick for a
call; it runs the same selection function the launchers run.  Sweeping it over
shapes that straddle every boundary of that selection (M against the GEMV's
row counts and the 64- and 128-row tiles, N against the 128 x 512 tile's
chip-filling rule, K against the GEMV's LDS budget) gives the reachable set.
Mapping the shapes of the GPU tests through it gives the covered set; the
first must be inside the second.
"""
import itertools

import pytest

import synth
import quantized_prefill_gemm_codec_amd as qg

import test_gpu_cross as cross
import test_gpu_limits as limits
import test_gpu_parity as par

ENTRIES = ["prefill", "heads", "swiglu", "geglu", "gemv"]


def _name(entry, codec, m, n, k):
    try:
        return qg.qg_kernel_for(entry, codec, m, n, k)
    except qg.QGError as e:
        assert e.status == -3       # sizes the entry point rejects
        return None


def reachable():
    ms = [1, 2, 3, 4, 5, 33, 64, 65, 127, 128, 129, 255, 512, 2048, 4096]
    ns = [1, 200, 8192, 14336, 65536]
    ks = [256, 2048, 4096, 1 << 14, 1 << 18]
    names = set()
    for codec, entry, m, n, k in itertools.product(range(1, 9), ENTRIES, ms, ns, ks):
        nm = _name(entry, codec, m, n, k)
        if nm:
            names.add(nm)
    return names


def covered():
    cases = []   # (entry, codec, m, n, k)
    cases += [(e, c, m, cross.N, cross.K) for c, e, m in cross.cross_cases()]
    cases += [("prefill", c, m, n, k) for c, m, n, k in par.GEMM_SHAPES]
    cases += [("heads", c, m, n, k) for c, m, n, k, _ in par.HEADS_SHAPES]
    cases += [("swiglu", c, m, n, k) for c, m, n, k in par.SWIGLU_SHAPES]
    cases += [("geglu", c, m, n, k) for c, m, n, k in par.GEGLU_SHAPES]
    cases += [("gemv", c, m, n, k) for c, m, n, k in par.GEMV_SHAPES]
    cases += [("prefill", c, 1921, 7681, 256) for c in range(1, 9)]          # test_prefill_wide_tile_ragged
    for wl in synth.WORKLOADS.values():                                       # test_full_workload_sampled
        cases.append((wl.op, wl.codec, wl.m, wl.n, wl.k))
    cases += [("prefill", c, m, n, k) for c, m, n, k in limits.DEGENERATE]
    cases += [("prefill", 1, 257, 256, 1 << 18), ("prefill", 1, 1, 131072, 8192), ("prefill", 1, 300, 131072, 8192)]
    return {nm for nm in (_name(*c) for c in cases) if nm}


def test_every_reachable_instantiation_is_tested():
    r, c = reachable(), covered()
    missing = sorted(r - c)
    assert not missing, f"{len(missing)} reachable kernel instantiations have no GPU parity test: {missing}"


def test_reachable_set_size():
    """Per codec: plain 128 x 512, 128 x 256 and 64 x 64 split-k tiles; gated
    128 x 256 and 64 x 64 split-k tiles (SwiGLU and GeGLU each); GEMV at 1, 2
    and 4 rows -- ten; Q8_0's gated small-M calls run the register-staged
    64 x 64 and 128 x 128 kernels instead of the split-k tile -- twelve.  A
    change to the dispatch that adds or drops an instantiation shows up here
    first.  (Codec 8, the 2-bit ternary layout, runs the Q2_0 kernels.)"""
    names = reachable()
    assert len(names) == 6 * 10 + 12, sorted(names)


@pytest.mark.parametrize("entry,codec,m,n,k,want", [
    ("prefill", 1, 1, 14336, 4096, "gemv_kernel<1, 1>"),
    ("prefill", 1, 3, 14336, 4096, "gemv_kernel<1, 4>"),
    ("gemv", 1, 64, 14336, 4096, "gemm_dma_kernel<1, 64, 64, 1, 1, 4, 0, 3, 1>"),
    ("prefill", 1, 65, 14336, 4096, "gemm_dma_kernel<1, 64, 64, 1, 1, 4, 0, 3, 1>"),
    ("prefill", 1, 2048, 8192, 2048, "gemm_dma_kernel<1, 128, 512, 1, 8, 1, 0, 3, 1>"),
    ("prefill", 3, 2048, 4096, 4096, "gemm_dma_kernel<3, 128, 256, 1, 8, 1, 0, 2, 2>"),
    ("swiglu", 2, 2048, 14336, 4096, "gemm_dma_kernel<2, 128, 256, 1, 8, 1, 1, 3, 1>"),
    ("geglu", 4, 64, 200, 512, "gemm_kernel<4, 64, 64, 2, 2, 2>"),
    ("gemv", 1, 2, 200, 1 << 18, "gemm_dma_kernel<1, 64, 64, 1, 1, 4, 0, 3, 1>"),   # X too large to stage
])
def test_named_choices(entry, codec, m, n, k, want):
    assert qg.qg_kernel_for(entry, codec, m, n, k) == want


def test_kernel_for_rejects_what_the_entry_points_reject():
    for args in [("gemv", 1, 65, 200, 512), ("prefill", 1, 5, 200, 48), ("prefill", 1, 0, 200, 512)]:
        with pytest.raises(qg.QGError) as e:
            qg.qg_kernel_for(*args)
        assert e.value.status == -3
    with pytest.raises(qg.QGError) as e:
        qg.qg_kernel_for("prefill", 9, 5, 200, 512)
    assert e.value.status == -2
