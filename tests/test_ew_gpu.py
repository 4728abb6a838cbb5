"""GPU parity of the elementwise chain y = relu(scale * x + bias), fused and
as three launches, against the fp64 oracle.

Bounds from the arithmetic (fp32 compute, bf16 round to nearest even: an
8-bit significand, so at most 2^-8 relative): fused, one rounding of the fp32
result:
    |dy| <= 2^-8 |y| + 2^-22 (|t1| + |bias|);
three launches, rounding t1 = scale*x and t2 = t1 + bias to bf16 before the
activation (which is 1-Lipschitz):
    |dy| <= 2^-8 (1 + 2^-8) |t1| + 2^-8 |t2| + 2^-22 (|t1| + |bias|),
with t1, t2, y the oracle's exact intermediates.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SCALE = 1.7


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_124_amd as ea
    ea.load_library()
    return ea


def check(y, x, b, oracle_mod, fused, what):
    ref, t1, t2 = oracle_mod.elementwise_chain(x, SCALE, b)
    got = y.double().cpu().numpy()
    ba = np.abs(b.double().numpy())[None, :]
    if fused:
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -22 * (np.abs(t1) + ba)
    else:
        bound = 2.0 ** -8 * (1 + 2.0 ** -8) * np.abs(t1) + 2.0 ** -8 * np.abs(t2) + 2.0 ** -22 * (np.abs(t1) + ba)
    err = np.abs(got - ref)
    ratio = (err / np.maximum(bound, 1e-300)).max() if err.any() else 0.0
    say(f"  {what}: max|dy|={err.max():.3e} max err/bound={ratio:.3f}")
    assert np.isfinite(got).all() and ratio <= 1.0, what


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 24), (1000, 768), (4097, 3072), (7, 8200)])
def test_small_full(ea, oracle_mod, rows, cols, fused):
    from exact_attention_124_amd.workloads import make_chain
    x, b = make_chain(rows, cols, seed=rows)
    say(f"[ew] rows={rows} cols={cols} fused={fused}")
    y = ea.elementwise_chain(x.cuda(), b.cuda(), SCALE, fused=fused)
    torch.cuda.synchronize()
    check(y, x, b, oracle_mod, fused, f"{rows}x{cols}")


@pytest.mark.parametrize("fused", [True, False])
def test_in_place(ea, oracle_mod, fused):
    from exact_attention_124_amd.workloads import make_chain
    x, b = make_chain(513, 1024, seed=5)
    xd = x.cuda()
    (ea.ew_chain_fused if fused else ea.ew_chain_unfused)(xd, xd, b.cuda(), SCALE)
    torch.cuda.synchronize()
    check(xd, x, b, oracle_mod, fused, "in place")


def test_bench_size_sampled_rows(ea, oracle_mod):
    """The benchmarked shape (65536 x 4096, 512 MiB of bf16), both forms,
    checked on 64 sampled rows."""
    from exact_attention_124_amd.workloads import make_chain
    rows, cols = 65536, 4096
    x, b = make_chain(rows, cols, seed=0)
    xd, bd = x.cuda(), b.cuda()
    pick = torch.randperm(rows, generator=torch.Generator().manual_seed(3))[:64].sort().values
    for fused in (True, False):
        y = ea.elementwise_chain(xd, bd, SCALE, fused=fused)
        torch.cuda.synchronize()
        check(y[pick.cuda()], x[pick], b, oracle_mod, fused, f"{rows}x{cols} fused={fused}")
