"""The allocation-free layer entry point against coli_moe_layer (GPU): the
same routing and output bit for bit, on two calls in a row sharing the
device scratch, the second with fewer tokens; over-size calls are refused
before any launch."""
import ctypes

import numpy as np
import pytest

import synth
from tests.gpu_util import build_table

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def both(table, w, T, seed, accumulate):
    x, lg, b = synth.activations(w, T, seed), synth.logits(w, T, seed), synth.router_bias(w)
    y0 = synth.normal(seed + 7, T * w.D, 1.0).reshape(T, w.D)
    ref = to_dev(y0)
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                     device=dev)
    coli.coli_moe_layer(table, to_dev(x), to_dev(lg), to_dev(b), w.k, ref, ws,
                        accumulate=accumulate)
    got = to_dev(y0)
    coli.coli_moe_layer_noalloc(table, to_dev(x), to_dev(lg), to_dev(b), w.k, got,
                                accumulate=accumulate)
    torch.cuda.synchronize()
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    g, r = got.cpu().numpy(), ref.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), \
        f"T={T}: {np.count_nonzero(g != r)} outputs differ"


@pytest.fixture(scope="module")
def tiny():
    w = synth.WORKLOADS[0]
    return w, build_table(w)


@pytest.mark.parametrize("sizes", [(64, 5), (300, 17), (9, 1)])
def test_noalloc_matches_layer_tiny(tiny, sizes):
    """Two calls in a row, the second smaller: grouped then GEMV path, fused
    front or not, accumulate on and off."""
    w, table = tiny
    for i, T in enumerate(sizes):
        both(table, w, T, 50 + T, accumulate=bool(i))


def test_noalloc_matches_layer_page_shape():
    """Decode and verify at the page shape (4.86 GB table): 4 tokens, then 1."""
    w = synth.WORKLOADS[2]
    table = build_table(w)
    both(table, w, 4, 60, accumulate=False)
    both(table, w, 1, 61, accumulate=True)
    del table
    torch.cuda.empty_cache()


def test_noalloc_limits(tiny):
    """A call needing more than the scratch is refused before any launch; an
    empty call does nothing."""
    w, table = tiny
    L = coli.lib()
    T = 1
    while coli.coli_moe_layer_workspace_bytes(table, T, w.k) <= coli.COLI_NOALLOC_BYTES:
        T *= 2
    x = torch.empty((1, w.D), dtype=torch.float32, device=dev)
    p = ctypes.c_void_p(x.data_ptr())
    rc = L.coli_moe_layer_noalloc(table.ref(), p, p, None, T, w.k, 1.0, p, 0, None)
    assert rc == coli.COLI_E_WORKSPACE
    assert L.coli_moe_layer_noalloc(table.ref(), p, p, None, 0, w.k, 1.0, p, 0, None) == coli.COLI_OK
