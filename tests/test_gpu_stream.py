"""The plain HBM stream kernel (muon_hbm_stream, the ceiling that
`bench.py --hbm-ceiling` measures) moves every byte as documented: output k
receives input k (or input 0 with one input), and two inputs into one output
give their bitwise XOR; with and without the nontemporal hint."""
import pytest
import torch

import newton_schulz_03_amd as nsa

pytestmark = pytest.mark.gpu

N = 3 * 16384 + 16384  # a few blocks of 4 KiB per stream, a multiple of 16384


def _rand(seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(0, 256, (N,), dtype=torch.uint8, generator=g).cuda()


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("n_in,n_out", [(1, 1), (1, 2), (2, 1), (2, 2)])
def test_stream_moves_every_byte(n_in, n_out, nt):
    ins = [_rand(10 + k) for k in range(n_in)]
    outs = [torch.zeros(N, dtype=torch.uint8, device="cuda") for _ in range(n_out)]
    nsa.hbm_stream(ins, outs, nontemporal=nt)
    torch.cuda.synchronize()
    if n_in == 2 and n_out == 1:
        assert torch.equal(outs[0], ins[0] ^ ins[1])
    else:
        for k in range(n_out):
            assert torch.equal(outs[k], ins[k % n_in])
