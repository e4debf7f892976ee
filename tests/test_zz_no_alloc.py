"""The allocation-free entry point against the workspace entry point, on the GPU.

muon_ns_batched_noalloc runs the same kernels as muon_ns_batched on the
library's own scratch array, so its outputs must equal the workspace call's bit
for bit, and each must be within the tolerance of the oracle per 256 x 256
block.  Two calls in a row, the second over smaller matrices (the array keeps
the first call's contents, which the second must not depend on), in bf16 and
fp32, and with e4m3 steps; and a batch too large for the array is refused
without touching the outputs.
"""
import numpy as np
import pytest
import torch

import newton_schulz_03_amd as nsa
import oracle
from parity_util import TOL, check_blocks, host_f64

pytestmark = pytest.mark.gpu

FIRST = [(700, 1300), (1300, 700), (513, 257), (33, 65), (256, 768)]
SECOND = [(300, 500), (64, 96), (1, 300)]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def _inputs(shapes, dtype, seed):
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).to(tdt).cuda()
            for sh in shapes]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_equals_workspace_call(dtype):
    for call, shapes in enumerate((FIRST, SECOND)):
        xs = _inputs(shapes, dtype, 100 + call)
        ref = nsa.ns_batched(xs, steps=5)
        got = [torch.full_like(x, 7.0) for x in xs]
        nsa.ns_batched_noalloc(xs, got, steps=5)
        torch.cuda.synchronize()
        for i, sh in enumerate(shapes):
            assert torch.equal(got[i], ref[i]), (dtype, call, sh)
            check_blocks(host_f64(got[i]), oracle.newton_schulz(host_f64(xs[i]), 5), TOL[dtype],
                         what=f"noalloc {dtype} call {call} {sh}")


def test_noalloc_with_e4m3_steps():
    """The e4m3 steps on the library's array (its e4m3 buffers included) equal
    the workspace call's, two calls in a row, the second smaller."""
    for call, shapes in enumerate((FIRST, SECOND)):
        xs = _inputs(shapes, "bf16", 200 + call)
        ref = nsa.ns_batched(xs, steps=5, fp8_steps=2)
        got = [torch.full_like(x, 7.0) for x in xs]
        nsa.ns_batched_noalloc(xs, got, steps=5, fp8_steps=2)
        torch.cuda.synchronize()
        for i, sh in enumerate(shapes):
            assert torch.equal(got[i], ref[i]), (call, sh)


def test_noalloc_in_stream_order_and_too_large():
    """Calls in order on one stream reuse the array safely; an oversize batch
    raises MUON_ERR_WORKSPACE and leaves the outputs untouched."""
    xs = _inputs(FIRST, "bf16", 7)
    ys = _inputs(SECOND, "bf16", 8)
    out_x = [torch.empty_like(x) for x in xs]
    out_y = [torch.empty_like(y) for y in ys]
    nsa.ns_batched_noalloc(xs, out_x, steps=5)
    nsa.ns_batched_noalloc(ys, out_y, steps=3, coeffs=oracle.CUBIC)
    ref_x = nsa.ns_batched(xs, steps=5)
    ref_y = nsa.ns_batched(ys, steps=3, coeffs=oracle.CUBIC)
    torch.cuda.synchronize()
    for a, b in zip(out_x + out_y, ref_x + ref_y):
        assert torch.equal(a, b)
    big = torch.zeros(8192, 8192, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(big, 3.0)
    with pytest.raises(nsa.MuonError) as e:
        nsa.ns_batched_noalloc([big], [out])
    assert e.value.status == nsa.MUON_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def test_noalloc_replays_from_a_graph():
    """The allocation-free call captured into a HIP graph (torch.cuda.CUDAGraph):
    the capture holds only kernel launches (the descriptor table travels as
    kernel arguments, the claim counters are zeroed by a kernel, no memset).
    Three replays, each after eager work that overwrites the outputs and the
    library's array (an allocation-free call over other matrices), each equal
    bit for bit to the workspace call's result."""
    xs = _inputs(FIRST, "bf16", 300)
    ys = _inputs(SECOND, "bf16", 301)
    ref = nsa.ns_batched(xs, steps=5)
    out = [torch.empty_like(x) for x in xs]
    out_y = [torch.empty_like(y) for y in ys]
    nsa.ns_batched_noalloc(xs, out, steps=5)  # eager first: the array's address is resolved
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nsa.ns_batched_noalloc(xs, out, steps=5)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in out:
            o.fill_(5.0)
        nsa.ns_batched_noalloc(ys, out_y, steps=3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, sh in enumerate(FIRST):
            assert torch.equal(out[i], ref[i]), (rep, sh)
