"""Largest matrices the GEMMs address (the padded iterate just under 4 GiB of
bf16), checked exactly where the mathematics allows it at any size.

A signed injection G (one entry +-g per row, in distinct columns) has every
singular value equal to g, so the Newton-Schulz output is G/g times the
scalar map p_K(...p_1(1/sqrt(m))) of the normalised singular value.  Every row
then goes through the same arithmetic on the device, so all nonzero outputs
must have the same magnitude, every other entry must be exactly zero, and
the magnitude must match the scalar map within the bf16 tolerance.  A wrong
offset anywhere in the addressing of a 30720 x 65536 matrix would break the
pattern."""
import math

import numpy as np
import pytest
import torch

import orthogonalising_matrix_optimizer_amd as mo
from oracle import muon_oracle as orc
from tests.gpu_helpers import TOL_BF16, announce
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mo._lib.load()


@pytest.mark.parametrize("rows,cols", [(30720, 65536), (65536, 30720)])
def test_signed_injection_at_the_offset_limit(rows, cols):
    announce(f"max-size signed injection {rows}x{cols}")
    assert mo.workspace_bytes([(rows, cols)]) > 0        # planned: under the limit
    m, n = min(rows, cols), max(rows, cols)
    dev = torch.device("cuda")
    gtr = torch.Generator(device=dev)
    gtr.manual_seed(2024)
    cols_of_rows = torch.randperm(n, generator=gtr, device=dev)[:m]
    signs = torch.randint(0, 2, (m,), generator=gtr, device=dev).float().mul_(2).sub_(1)
    g = 1.0 / 64
    G = torch.zeros((m, n), dtype=torch.bfloat16, device=dev)
    G[torch.arange(m, device=dev), cols_of_rows] = (signs * g).to(torch.bfloat16)
    if rows > cols:
        G = G.T.contiguous()
    out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    steps = 5
    ws = mo.orthogonalize([G], [out], coeffs="quintic", steps=steps)
    torch.cuda.synchronize()
    del ws
    nz = G != 0
    assert int(nz.sum()) == m
    vals = out[nz]
    mags = vals.abs()
    # one magnitude for every row, signs as in G, exact zeros elsewhere
    assert float(mags.max()) == float(mags.min())
    assert torch.equal(torch.sign(vals), torch.sign(G[nz].float()))
    off = out.masked_fill(nz, 0.0)
    assert int(torch.count_nonzero(off)) == 0
    # the scalar map on the normalised singular value: 1 / (sqrt(m) + eps/g)
    x = g / (g * math.sqrt(m) + 1e-7)
    want = orc.ns_poly_scalar(x, gen.coeff_table("quintic", steps))
    assert abs(float(mags[0]) - want) <= TOL_BF16 * want, (float(mags[0]), want)
