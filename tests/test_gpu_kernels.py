"""Per-kernel parity of the HIP path against the oracle (GPU)."""
import numpy as np
import pytest

import oracle
import synth
from tests import oracle_pins
from tests.gpu_util import assert_bitexact, build_table, decode_table_expert, stream_ptr

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_device_generator_matches_host():
    for sid, off, n, sigma in ((synth.stream_id(1, 1, 0, 5), 0, 100003, 0.02),
                               (synth.stream_id(2, 0, 3, 7), 2**33 + 17, 4097, 1.0),
                               (synth.stream_id(4, 1, 39, 0), 123456789, 256, 0.1)):
        out = torch.empty(n, dtype=torch.float32, device=dev)
        synth.normal_device(sid, n, sigma, out.data_ptr(), stream_ptr(), offset=off)
        assert_bitexact(f"synth {sid:x}", out.cpu().numpy(), synth.normal(sid, n, sigma, offset=off))


def quant_act(x):
    x = np.ascontiguousarray(x, np.float32)
    xd = to_dev(x)
    q = torch.empty(x.shape, dtype=torch.int8, device=dev)
    d = torch.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=torch.float32, device=dev)
    coli.coli_quant_act_q8(xd, q, d)
    return q.cpu().numpy(), d.cpu().numpy()


@pytest.mark.parametrize("T,D", [(1, 6144), (4, 256), (3, 32), (2048, 6144)])
def test_quant_act_q8(T, D):
    x = synth.normal(synth.stream_id(2, 9, 0, T), T * D, 1.0).reshape(T, D)
    q, d = quant_act(x)
    rq, rd = oracle.q8_quant(x)
    assert_bitexact("q", q, rq)
    assert_bitexact("d", d, rd)


def test_quant_act_q8_edges():
    blocks = []
    for name in ("rint_ties_q8.txt", "rint_ties_q8_d255.txt"):
        rows = oracle_pins.load_golden(name)
        scale = 2.0 ** -5 if name == "rint_ties_q8.txt" else 255.0
        blocks.append(np.array([m for m, _ in rows], np.float32) * np.float32(scale))
    blocks.append(np.zeros(32, np.float32))                       # zero block
    blocks.append(np.full(32, -3.25, np.float32))                 # constant block
    blocks.append(np.float32([1e-30] * 16 + [-1e-30] * 16))        # tiny values
    blocks.append(np.float32([3e38] + [-1.0] * 31))                # huge max
    x = np.concatenate(blocks)[None, :]
    q, d = quant_act(x)
    rq, rd = oracle.q8_quant(x)
    assert_bitexact("q", q, rq)
    assert_bitexact("d", d, rd)
    for i, name in enumerate(("rint_ties_q8.txt", "rint_ties_q8_d255.txt")):
        assert q[0, 32 * i:32 * i + 32].tolist() == [e for _, e in oracle_pins.load_golden(name)]


@pytest.mark.parametrize("rows,k", [(2048, 6144), (6144, 2048), (128, 256), (7, 32)])
def test_quant_weight_q4(rows, k):
    w = synth.normal(synth.stream_id(1, 9, 1, rows), rows * k, 0.02).reshape(rows, k)
    w[0, :] = 0.0                      # an all-zero row
    w[-1, :] = np.float32(0.37)        # a constant row
    wd = to_dev(w)
    q = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    s = torch.empty(rows, dtype=torch.float32, device=dev)
    coli.coli_quant_weight_q4(wd, q, s)
    rq, rs = oracle.q4_quant(w)
    assert_bitexact("packs", q.cpu().numpy(), rq)
    assert_bitexact("scales", s.cpu().numpy(), rs)


def test_quant_weight_q4_ties():
    rows = oracle_pins.load_golden("rint_ties_q4.txt")
    w = np.array([m for m, _ in rows], np.float32) * np.float32(2.0 ** -3)
    w = np.concatenate([w, np.zeros(16, np.float32)])[None, :]
    q = torch.empty((1, 16), dtype=torch.uint8, device=dev)
    s = torch.empty(1, dtype=torch.float32, device=dev)
    coli.coli_quant_weight_q4(to_dev(w), q, s)
    codes = oracle.unpack_q4(q.cpu().numpy())[0, :len(rows)]
    assert codes.tolist() == [e for _, e in rows]
    assert s.item() == 2.0 ** -3


def test_table_layout_tiny():
    w = synth.WORKLOADS[0]
    table = build_table(w)
    arrs = [t.cpu().numpy() for t in (table.gu_q, table.gu_s, table.dn_q, table.dn_s)]
    from tests.gpu_util import OracleExperts
    ox = OracleExperts(w)
    for e in range(w.E + w.S):
        gate, up, gs, us, down, ds = decode_table_expert(w, *arrs, e)
        ex = ox[e]
        assert_bitexact(f"gate codes e{e}", gate, oracle.unpack_q4(ex.gate_q).astype(np.int64))
        assert_bitexact(f"up codes e{e}", up, oracle.unpack_q4(ex.up_q).astype(np.int64))
        assert_bitexact(f"down codes e{e}", down, oracle.unpack_q4(ex.down_q).astype(np.int64))
        assert_bitexact(f"gate s e{e}", gs, ex.gate_s)
        assert_bitexact(f"up s e{e}", us, ex.up_s)
        assert_bitexact(f"down s e{e}", ds, ex.down_s)


def route(logits, bias, k, scale=1.0):
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    coli.coli_route_topk(to_dev(logits), None if bias is None else to_dev(bias), k, idx, w,
                         routed_scale=scale)
    return idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("wl,T", [(0, 4), (1, 64), (3, 2048)])
def test_route_topk(wl, T):
    w = synth.WORKLOADS[wl]
    lg, b = synth.logits(w, T), synth.router_bias(w)
    idx, wt = route(lg, b, w.k)
    ridx, rw = oracle.route(lg, b, w.k)
    assert_bitexact("idx", idx, ridx)
    assert_bitexact("w", wt, rw)


def lane_heavy_logits():
    """256 experts whose top-8 sit in few wavefront lanes (expert e is held by
    lane e % 64): a four-way tie inside lane 3, a tie across lanes 7 and 3,
    one more winner in lane 7, and the 8th taken among 248 equal scores;
    row 1 puts all eight winners into lanes 3 and 7 with distinct scores."""
    lg = np.full((2, 256), -2.0, np.float32)
    lg[0, [3, 67, 131, 195, 7, 71]] = 1.0
    lg[0, 135] = 0.5
    lg[1, [3, 67, 131, 195, 7, 71, 135, 199]] = np.float32([5, 1, 4, 2, 8, 3, 7, 6]) / 4
    return lg


def test_route_topk_edges():
    cases = [
        (np.float32([[1.0, 2.0, 1.0, 2.0, 2.0, 0.0]]), None, 4, 1.0),      # exact ties
        (np.zeros((3, 16), np.float32), np.zeros(16, np.float32), 16, 1.0),  # k = E, all equal
        (np.float32([[2.0, 1.0, -3.0]]), np.float32([0.0, 0.5, 0.0]), 2, 2.5),  # bias flip
        (np.float32([[0.7]]), None, 1, 1.0),                                  # E = 1
        (-np.abs(synth.normal(77, 5 * 256, 3.0)).reshape(5, 256), None, 64, 1.0),  # k = 64
        (lane_heavy_logits(), None, 8, 1.0),     # winners stacked in a few lanes, with ties
        (lane_heavy_logits(), np.linspace(-0.01, 0.01, 256, dtype=np.float32), 8, 1.0),
    ]
    for lg, b, k, sc in cases:
        bb = np.zeros(lg.shape[1], np.float32) if b is None else b
        idx, wt = route(lg, b, k, sc)
        ridx, rw = oracle.route(lg, bb, k, sc)
        assert_bitexact("idx", idx, ridx)
        assert_bitexact("w", wt, rw)


def dispatch(idx, E, S):
    T, k = idx.shape
    counts = torch.full((E + S,), -7, dtype=torch.int32, device=dev)
    lists = torch.full((E + S, T), -1, dtype=torch.int32, device=dev)
    na = torch.zeros(1, dtype=torch.int32, device=dev)
    active = torch.full((E + S,), -1, dtype=torch.int32, device=dev)
    err = torch.full((1,), 99, dtype=torch.int32, device=dev)
    coli.coli_dispatch(to_dev(idx), E, S, counts, lists, na, active, err)
    return counts.cpu().numpy(), lists.cpu().numpy(), int(na.item()), active.cpu().numpy(), \
        int(err.item())


@pytest.mark.parametrize("wl,T", [(0, 4), (2, 4), (3, 2048), (3, 2500)])
def test_dispatch(wl, T):
    w = synth.WORKLOADS[wl]
    ridx, _ = oracle.route(synth.logits(w, T), synth.router_bias(w), w.k)
    counts, lists, na, active, err = dispatch(ridx, w.E, w.S)
    rc, rl, rna, ract = oracle.dispatch(ridx, w.E, w.S)
    assert err == 0
    assert_bitexact("counts", counts, rc)
    assert na == rna
    assert_bitexact("active", active[:na], ract)
    for e in range(w.E + w.S):
        assert_bitexact(f"list {e}", lists[e, :counts[e]], rl[e, :rc[e]])


def _bad_routings():
    yield np.int32([[0, 16], [1, 2]]), 16
    yield np.int32([[-1, 3]]), 16
    yield np.int32([[5, 5], [1, 2]]), 16
    yield np.int32([[5, 5], [5, 4]]), 16
    rng = np.random.default_rng(5)
    for T, E, k in ((300, 256, 8), (700, 16, 2), (65, 64, 4), (2301, 256, 8), (1030, 32, 3)):
        idx = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
        idx[::2, -1] = idx[::2, 0]
        yield idx, E


def test_dispatch_drops_bad_indices():
    """Out-of-range and repeated entries are left out of every list (the
    oracle's keep rule), the lists of the rest are exact, and the flag is set;
    the larger cases span several 1024-token sweeps with a ragged tail."""
    for bad, E in _bad_routings():
        counts, lists, na, active, err = dispatch(bad, E, 1)
        assert err == coli.COLI_E_INDEX
        keep, dropped = oracle.keep_entries(bad, E)
        assert dropped > 0
        rc, rl, rna, ract = oracle.dispatch(bad, E, 1, keep=keep)
        assert_bitexact("counts", counts, rc)
        assert na == rna
        assert_bitexact("active", active[:na], ract)
        for e in range(E + 1):
            assert_bitexact(f"list {e}", lists[e, :counts[e]], rl[e, :rc[e]])


def test_rmsnorm_q8():
    w = synth.WORKLOADS[4]
    h = synth.hidden0(w, 8) * np.float32(3.0)
    h[1] = 0.0                                   # zero row: r = 1/sqrt(eps), codes 0
    h[2] = np.float32(-0.75)                     # constant row
    T, D = h.shape
    q = torch.empty((T, D), dtype=torch.int8, device=dev)
    d = torch.empty((T, D // 32), dtype=torch.float32, device=dev)
    r = torch.empty(T, dtype=torch.float32, device=dev)
    coli.coli_rmsnorm_q8(to_dev(h), 1e-6, q, d, r)
    xh, rr = oracle.rmsnorm(h, np.float32(1e-6))
    rq, rd = oracle.q8_quant(xh)
    assert_bitexact("r", r.cpu().numpy(), rr)
    assert_bitexact("q", q.cpu().numpy(), rq)
    assert_bitexact("d", d.cpu().numpy(), rd)
