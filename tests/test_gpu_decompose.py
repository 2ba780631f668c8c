"""GPU parity of fp4q_error_decompose against the oracle: the 320-bit exact
sums bit for bit (and so the additive identity), the counts exactly, and the
FP64 sums of squares within rounding."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import workload, need_gpu, say, to_dev
from workloads import CONFIGS, bf16_bits, dense_case

pytestmark = pytest.mark.gpu


def _to_int(limbs):
    v = 0
    for i, l in enumerate(limbs):
        v |= (int(l) & ((1 << 64) - 1)) << (64 * i)
    return v - (1 << 320) if v >> 319 else v


def _check(orc, x):
    need_gpu()
    ref = orc.error_decompose(x)
    got = fq.error_decompose(1, to_dev(x))
    assert got["exact"] == ref["exact"]
    t, sb, dz, gn = (_to_int(l) for l in got["exact"])
    assert sb + dz + gn == t
    assert got["n_elems"] == ref["n_elems"]
    assert got["n_deadzone"] == ref["n_deadzone"]
    assert got["n_clipped"] == ref["n_clipped"] == 0
    for c in range(4):
        assert np.isclose(got["sum"][c], ref["sum"][c], rtol=1e-12, atol=0)
        assert np.isclose(got["sumsq"][c], ref["sumsq"][c], rtol=1e-9, atol=0)
    assert np.isclose(got["cross_sb_gn"], ref["cross_sb_gn"], rtol=1e-9, atol=1e-300)
    return got


def test_small_and_special(orc):
    say("decompose small + special values")
    rng = np.random.default_rng(8)
    x = bf16_bits(rng.standard_t(4, (40, 256)).astype(np.float32))
    x[0] = 0
    x[1, :64] = np.arange(64, dtype=np.uint16) + 1         # subnormals
    x[2, :32] = 0x7F7F                                       # huge
    x[2, 32:64] = bf16_bits(np.float32(1e-38))
    x[3, :32] = bf16_bits(np.array([6.0 * 2 ** -3] + [1e-20] * 31, np.float32))  # wide span
    _check(orc, x)


def test_ragged_rows(orc):
    x = dense_case(3, 96, 8, seed=3)["x"]
    _check(orc, x)
    _check(orc, x[:1].copy())


def test_workload_activations_and_weights(orc):
    """MXFP4 workload: X [8192 x 4096] and W^T [14336 x 4096]."""
    say("decompose MXFP4 workload X and W^T")
    d = workload("prefill_mxfp4")
    gx = _check(orc, d["x"])
    gw = _check(orc, d["wt"])
    say(f"  X: n_deadzone {gx['n_deadzone']}, sums {gx['sum']}")
    say(f"  W: n_deadzone {gw['n_deadzone']}, sums {gw['sum']}")


def _check_nv(orc, x):
    need_gpu()
    ref = orc.error_decompose(x, fmt=0)
    got = fq.error_decompose(0, to_dev(x))
    assert got["exact"] == ref["exact"]
    t, sb, dz, gn = (_to_int(l) for l in got["exact"])
    assert sb + dz + gn == t
    assert got["n_elems"] == ref["n_elems"]
    assert got["n_deadzone"] == ref["n_deadzone"]
    assert got["n_clipped"] == ref["n_clipped"]
    for c in range(4):
        assert np.isclose(got["sum"][c], ref["sum"][c], rtol=1e-12, atol=0)
        assert np.isclose(got["sumsq"][c], ref["sumsq"][c], rtol=1e-9, atol=0)
    assert np.isclose(got["cross_sb_gn"], ref["cross_sb_gn"], rtol=1e-9, atol=1e-300)
    return got


def test_nvfp4_small_and_special(orc):
    """NVFP4: heavy tails, an all-zero row, subnormals and huge values in one
    tensor (blocks whose scale underflows are all deadzone), a block whose
    E4M3 scale rounds down (clipping), and a wide exponent span."""
    say("decompose NVFP4 small + special values")
    rng = np.random.default_rng(9)
    x = bf16_bits(rng.standard_t(4, (40, 256)).astype(np.float32))
    x[0] = 0
    x[1, :64] = np.arange(64, dtype=np.uint16) + 1
    x[2, :16] = 0x7F7F
    x[2, 32:48] = bf16_bits(np.float32(1e-38))
    x[3, :16] = bf16_bits(np.array([6.0 * 2 ** -3] + [1e-20] * 15, np.float32))
    x[4, 16:20] = bf16_bits(np.array([0.96875, 0.5, -0.25, 0.9375], np.float32))
    g = _check_nv(orc, x)
    assert g["n_clipped"] > 0


@pytest.mark.parametrize("rows,cols", [(3, 48), (1, 16), (65, 80)])
def test_nvfp4_ragged(orc, rows, cols):
    """Column counts that are not a multiple of 32 (odd numbers of 16-blocks)."""
    say(f"decompose NVFP4 {rows}x{cols}")
    _check_nv(orc, dense_case(rows, cols, 8, n_out=1, seed=rows + cols)["x"])


def test_nvfp4_workload_activations(orc):
    """NVFP4 workload activations: prefill X [8192 x 4096] and decode X [64 x 2048]."""
    say("decompose NVFP4 workload X")
    gx = _check_nv(orc, workload("prefill_nvfp4")["x"])
    gd = _check_nv(orc, workload("decode_nvfp4")["x"])
    say(f"  prefill X: deadzone {gx['n_deadzone']}, clipped {gx['n_clipped']}")
    say(f"  decode X: deadzone {gd['n_deadzone']}, clipped {gd['n_clipped']}")
