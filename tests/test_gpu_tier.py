"""Expert tier (HBM slots over a pinned host store) against the oracle (GPU).

Every plan's decisions -- slot of each expert, expert of each slot, stamps,
pins, usage counts, the load list and the hit count -- are compared bit for
bit with the oracle's tier after each pass, over Zipf-skewed routings with
1-4 tokens per pass and interleaved prefetch plans.  The forward through the
tier (experts read through the slot map) must equal the forward through the
fully resident table bit for bit.  Also: a pass that does not fit, a forward
that selects a non-resident expert, usage-learned pinning, an int8 tier and a
page-shape layer.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import OracleExperts, assert_bitexact, build_table

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"
ZIPF_TINY = replace(synth.WORKLOADS[4], name="tiny zipf layer d256 f128 e16+1 top2", D=256, F=128,
                    E=16, k=2, family=0, tag=6, layers=1)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def route(w, T, token0, layer=0):
    lg = to_dev(synth.logits(w, T, token0, layer))
    idx = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    coli.coli_route_topk(lg, to_dev(np.zeros(w.E, np.float32)), w.k, idx, wt)
    return idx, wt


def check_state(tier, ref, step):
    st = {k: v.cpu().numpy() for k, v in tier.st.items()}
    assert_bitexact(f"slot_of step {step}", st["slot_of"], ref.slot_of)
    assert_bitexact(f"expert_in step {step}", st["expert_in"], ref.expert_in)
    assert_bitexact(f"stamp step {step}", st["stamp"], ref.stamp)
    assert_bitexact(f"pinned step {step}", st["pinned"], ref.pinned)
    assert_bitexact(f"usage step {step}", st["usage"], ref.usage)
    assert int(st["counters"][0]) == ref.step and int(st["counters"][3]) == 0
    return st


class Layer:
    """Resident table, its pinned host store, and a tier over the store."""

    def __init__(self, w, slots, bits=4, layer=0):
        self.w = w
        self.table = build_table(w, layer, bits=bits)
        self.store = self.table.to_host_store()
        self.tier = coli.ExpertTier(w.E, w.S, w.D, w.F, slots, weight_bits=bits)

    def forward(self, table, xq, xd, idx, wt):
        T = idx.shape[0]
        ws = torch.empty(coli.coli_moe_workspace_bytes(table, T, self.w.k), dtype=torch.uint8,
                         device=dev)
        y = torch.empty((T, self.w.D), dtype=torch.float32, device=dev)
        coli.coli_moe_forward(table, xq, xd, idx, wt, y, ws)
        return y, coli.coli_moe_status(ws)


def quant(w, T, token0):
    xq = torch.empty((T, w.D), dtype=torch.int8, device=dev)
    xd = torch.empty((T, w.D // 32), dtype=torch.float32, device=dev)
    coli.coli_quant_act_q8(to_dev(synth.activations(w, T, token0)), xq, xd)
    return xq, xd


@pytest.fixture(scope="module")
def tiny():
    return Layer(ZIPF_TINY, slots=12)   # 1 shared + 2 pinned + up to 8 per pass + 1


def test_tier_plans_and_forward_match(tiny):
    """48 passes of 1-4 tokens, every 5th preceded by a prefetch plan: the
    tier's state after each plan equals the oracle's, and the forward through
    the tier equals the resident forward."""
    w, L = ZIPF_TINY, tiny
    pin = [5, 9]
    L.tier.init(L.store, pin)
    ref = oracle.Tier(oracle.get(), w.E, w.S, 12, pin)
    st = check_state(L.tier, ref, "init")
    assert_bitexact("init loads", st["loads"][1:1 + st["loads"][0]], ref.init_loads)
    hits = 0
    for step in range(48):
        T = 1 + step % 4
        if step % 5 == 4:   # prefetch the next pass's routing (no usage counted)
            pidx, _ = route(w, T, 100 * step + 50)
            L.tier.plan(pidx, count_usage=False)
            loads, hp = ref.plan(pidx.cpu().numpy(), count_usage=False)
            hits += hp                     # the hit counter counts every plan
            st = check_state(L.tier, ref, f"{step} prefetch")
            assert_bitexact("prefetch loads", st["loads"][1:1 + st["loads"][0]], loads)
            L.tier.fetch(L.store)
        idx, wt = route(w, T, 100 * step + 50)
        L.tier.plan(idx)
        loads, h = ref.plan(idx.cpu().numpy())
        hits += h
        st = check_state(L.tier, ref, step)
        assert_bitexact(f"loads {step}", st["loads"][1:1 + st["loads"][0]], loads)
        assert int(st["counters"][1]) == hits
        L.tier.fetch(L.store)
        xq, xd = quant(w, T, 100 * step)
        y_tier, s1 = L.forward(L.tier, xq, xd, idx, wt)
        y_res, s2 = L.forward(L.table, xq, xd, idx, wt)
        assert s1 == coli.COLI_OK and s2 == coli.COLI_OK
        assert_bitexact(f"y through the tier, step {step}", y_tier.cpu().numpy(),
                        y_res.cpu().numpy())
    assert L.tier.status() == coli.COLI_OK
    # the forward through the tier also equals the oracle (last pass)
    ox = OracleExperts(w)
    xq_h, xd_h = oracle.q8_quant(synth.activations(w, T, 100 * 47))
    idx_h, wt_h = idx.cpu().numpy(), wt.cpu().numpy()
    yr, _ = oracle.moe_layer(ox.table_for(idx_h), w.E, w.S, xq_h, xd_h, idx_h, wt_h)
    assert_bitexact("y vs oracle", y_tier.cpu().numpy(), yr)


def test_tier_learned_pins(tiny):
    """Usage-learned pinning: the rank of the usage counts and a tier
    re-initialised with those pins match the oracle."""
    w, L = ZIPF_TINY, tiny
    L.tier.init(L.store)
    ref = oracle.Tier(oracle.get(), w.E, w.S, 12)
    for step in range(30):
        idx, _ = route(w, 2, 10 * step + 7)
        L.tier.plan(idx)
        ref.plan(idx.cpu().numpy())
    usage = L.tier.st["usage"].cpu().numpy()
    assert_bitexact("usage", usage, ref.usage)
    top = coli.coli_tier_rank(usage[: w.E], 3)
    assert_bitexact("rank", top, ref.pin_top(3))
    L.tier.init(L.store, top)
    ref2 = oracle.Tier(oracle.get(), w.E, w.S, 12, top)
    check_state(L.tier, ref2, "re-init")


def test_tier_pass_that_does_not_fit(tiny):
    w, L = ZIPF_TINY, tiny
    L.tier.init(L.store, [3, 4, 5, 7, 8, 9, 10, 11])   # 1 shared + 8 pinned: 3 free
    idx = to_dev(np.array([[0, 1], [2, 6]], np.int32))
    before = {k: v.clone() for k, v in L.tier.st.items()}
    L.tier.plan(idx)
    assert L.tier.status() == coli.COLI_E_TIER
    for k in ("slot_of", "expert_in", "stamp", "usage"):
        assert torch.equal(L.tier.st[k], before[k]), k


def test_forward_with_non_resident_expert(tiny):
    """Selecting an expert that is not in the tier reports COLI_E_TIER; the
    kernels skip it instead of reading outside the tier."""
    w, L = ZIPF_TINY, tiny
    L.tier.init(L.store)
    L.tier.plan(to_dev(np.array([[0, 1]], np.int32)))
    L.tier.fetch(L.store)
    xq, xd = quant(w, 1, 0)
    idx = to_dev(np.array([[0, 2]], np.int32))          # 2 is not resident
    wt = to_dev(np.array([[0.5, 0.5]], np.float32))
    _, status = L.forward(L.tier, xq, xd, idx, wt)
    assert status == coli.COLI_E_TIER


def test_int8_tier():
    """An int8 head layer through a tier equals its resident forward."""
    w = ZIPF_TINY
    L = Layer(w, slots=10, bits=8, layer=78)
    L.tier.init(L.store, [1])
    ref = oracle.Tier(oracle.get(), w.E, w.S, 10, [1])
    for step in range(12):
        T = 1 + step % 3
        idx, wt = route(w, T, 31 * step)
        L.tier.plan(idx)
        ref.plan(idx.cpu().numpy())
        check_state(L.tier, ref, step)
        L.tier.fetch(L.store)
        xq, xd = quant(w, T, 31 * step)
        y_tier, s1 = L.forward(L.tier, xq, xd, idx, wt)
        y_res, s2 = L.forward(L.table, xq, xd, idx, wt)
        assert s1 == s2 == coli.COLI_OK
        assert_bitexact(f"int8 y step {step}", y_tier.cpu().numpy(), y_res.cpu().numpy())


def test_page_shape_tier():
    """A 6144 x 2048, 256 + 1 expert layer with 48 HBM slots over its pinned
    host store (4.86 GB): Zipf decode and verify passes through the tier equal
    the resident forward; decisions equal the oracle's."""
    w = replace(synth.WORKLOADS[4], layers=1)
    L = Layer(w, slots=48)
    L.tier.init(L.store)
    ref = oracle.Tier(oracle.get(), w.E, w.S, 48)
    for step in range(16):
        T = 4 if step % 4 == 3 else 1
        idx, wt = route(w, T, 13 * step)
        L.tier.plan(idx)
        ref.plan(idx.cpu().numpy())
        check_state(L.tier, ref, step)
        L.tier.fetch(L.store)
        xq, xd = quant(w, T, 13 * step)
        y_tier, s1 = L.forward(L.tier, xq, xd, idx, wt)
        y_res, s2 = L.forward(L.table, xq, xd, idx, wt)
        assert s1 == s2 == coli.COLI_OK
        assert_bitexact(f"page-shape y step {step}", y_tier.cpu().numpy(), y_res.cpu().numpy())
    del L
    torch.cuda.empty_cache()
