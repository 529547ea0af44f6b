"""The measurement kernels bench.py judges the loss kernels against, on the GPU.

The streaming copy of librlpl_bench.so is the HBM ceiling of the roofline
lines, so it must copy exactly the bytes it is asked to, in each of its eight
variants (plain or non-temporal; four or eight 16-byte words in flight per
lane; grid-stride or one chunk per workgroup) and at any grid, including
grids with more workgroups than 16-byte words: every destination word equal
to its source word, and the bytes just past the destination untouched.
"""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GUARD = 256                         # bytes past the destination that must stay untouched


@pytest.fixture(scope="module")
def lib():
    import bench
    return bench.bench_lib()


@pytest.mark.parametrize("variant", range(8))
@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, (16 << 20) + 16])
@pytest.mark.parametrize("grid", [0, 7, 1024, 8192])
def test_copy_moves_exactly_the_requested_bytes(lib, variant, nbytes, grid):
    g = torch.Generator(device="cpu").manual_seed(nbytes * 131 + variant * 7 + grid)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(DEV)
    dst = torch.full((nbytes + GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    pairs = (ctypes.c_uint64 * 2)(dst.data_ptr(), src.data_ptr())
    stream = torch.cuda.current_stream(DEV).cuda_stream
    st = lib.rlpl_bench_copy(1, pairs, nbytes, grid, variant, 1, 0, stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())


def test_copy_rejects_sizes_that_are_not_whole_words(lib):
    dst = torch.zeros(64, dtype=torch.uint8, device=DEV)
    pairs = (ctypes.c_uint64 * 2)(dst.data_ptr(), dst.data_ptr())
    assert lib.rlpl_bench_copy(1, pairs, 24, 0, 0, 1, 0, None) != 0
    assert lib.rlpl_bench_copy(1, pairs, 16, 0, 8, 1, 0, None) != 0
