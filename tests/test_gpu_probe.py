"""The calibration kernels behind the measured peaks of the benchmark (not
part of a DDTree round): the read stream reads every vector it is given, and
the MFMA loop performs exactly `iters` accumulations."""
import numpy as np
import pytest
import torch

from draft_tree_build_amd import api
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _read_fold(words: np.ndarray, grid: int) -> np.ndarray:
    """Host replay of the read probe's folding (grid-strided 16-byte vectors,
    eight per thread per step, XOR of the words, OR over a wave, XOR over the
    four waves of a workgroup)."""
    vec = words.reshape(-1, 4)
    nvec = vec.shape[0]
    stride = grid * 256
    out = np.zeros(grid, dtype=np.uint32)
    for g in range(grid):
        per_wave = []
        for w in range(4):
            acc = 0
            for lane in range(64):
                t = g * 256 + w * 64 + lane
                x = 0
                base = t
                while base < nvec:
                    for j in range(8):
                        v = vec[min(base + j * stride, nvec - 1)]
                        x ^= int(v[0]) ^ int(v[1]) ^ int(v[2]) ^ int(v[3])
                    base += 8 * stride
                acc |= x
            per_wave.append(acc)
        out[g] = per_wave[0] ^ per_wave[1] ^ per_wave[2] ^ per_wave[3]
    return out


@pytest.mark.parametrize("nvec,grid", [(5000, 3), (256, 1), (70001, 2)])
def test_probe_read_folds_every_vector(nvec, grid):
    g = torch.Generator().manual_seed(nvec)
    words = torch.randint(0, 2**31 - 1, (nvec * 4,), generator=g, dtype=torch.int64)
    words = words.to(torch.int32)
    note("probe read nvec=%d grid=%d" % (nvec, grid))
    src = words.to(DEV)
    out = torch.zeros(grid, dtype=torch.int32, device=DEV)
    api.ddtree_probe_hbm_read(src, out, grid)
    torch.cuda.synchronize()
    ref = _read_fold(words.numpy().view(np.uint32), grid)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref)


def test_probe_mfma_accumulates_iters_times():
    grid = 4
    o1 = torch.zeros(grid * 256, dtype=torch.float32, device=DEV)
    o4 = torch.zeros_like(o1)
    note("probe mfma grid=%d iters=1,4" % grid)
    api.ddtree_probe_mfma_bf16(o1, grid, 1)
    api.ddtree_probe_mfma_bf16(o4, grid, 4)
    torch.cuda.synchronize()
    a, b = o1.cpu().numpy(), o4.cpu().numpy()
    assert np.all(np.isfinite(a)) and np.any(a != 0)
    np.testing.assert_array_equal(b, 4 * a)   # operands are exact in bf16; sums exact in fp32
