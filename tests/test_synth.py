"""The seeded input generators (CPU): shapes the parity tests draw."""
import torch

from warp_specialized_pipelined_amd import synth
from tests.helpers import Problem


def test_empty_e4m3_operands_are_drawn():
    # K = 0 leaves an e4m3 operand with no entries: there is nothing to
    # scale, and the draw must still give an empty e4m3 tensor.
    g = torch.Generator().manual_seed(1)
    x = synth.random_matrix(g, (0, 888), synth.E4M3)
    assert x.shape == (0, 888) and x.dtype == torch.float8_e4m3fn
    p = Problem.random(g, 867, 888, 0, "row", "row", dtype=synth.E4M3)
    assert p.K == 0 and p.B.numel() == 0


def test_draws_repeat_with_the_seed():
    a = synth.random_matrix(torch.Generator().manual_seed(7), (64, 48), synth.E4M3)
    b = synth.random_matrix(torch.Generator().manual_seed(7), (64, 48), synth.E4M3)
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
