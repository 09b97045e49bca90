"""Pins of the oracle against facts that do not come from the oracle itself.

Each pin_* function takes an oracle.Oracle and raises AssertionError when the
oracle disagrees with: the pages' stated invariants (nibble packs identical
to the int8 container, lrintf / np.rint half-to-even rounding), closed forms,
brute force in int64 / fp64 written independently here, a library routine
(Python's sorted, numpy's float64 exp), or error bounds.

The same functions run against deliberately mutated oracle builds
(test_oracle_mutants.py), which must each fail at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL_REL = 1e-5   # |y - ref| <= 1e-5 * sum|terms| + 1e-6
TOL_ABS = 1e-6


# ---------------------------------------------------------------- helpers
def signed_lo(b):
    """Low nibble as signed int4 by arithmetic-shift sign extension."""
    return (np.left_shift(b.astype(np.uint8), 4).view(np.int8) >> 4).astype(np.int64)


def signed_hi(b):
    return (b.astype(np.uint8).view(np.int8) >> 4).astype(np.int64)


def unpack_ref(packed):
    """[..., k/2] bytes -> [..., k] int64, low nibble = even column."""
    lo, hi = signed_lo(packed), signed_hi(packed)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def ulp_dist(a, b):
    """|a - b| in units of float32 ulp of b (b computed in float64)."""
    b32 = np.float32(b)
    spacing = np.spacing(np.abs(b32)).astype(np.float64)
    return np.abs(np.float64(a) - np.float64(b)) / spacing


def load_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((float(a), int(b)))
    return rows


def unpack2_ref(packed):
    """[..., k/4] bytes -> [..., k] int64: 2-bit fields, lowest bits first,
    sign-extended by shifting the field to the top of an int32 and back."""
    b = packed.astype(np.int64)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 4,), dtype=np.int64)
    for j in range(4):
        f = ((b >> (2 * j)) & 3).astype(np.int32)
        out[..., j::4] = (np.left_shift(f, 30) >> 30).astype(np.int64)
    return out


def codes_of(Wq, bits=4):
    """The integer codes of a weight container: nibbles (bits 4), 2-bit
    fields (bits 2) or int8 (bits 8)."""
    if bits == 4:
        return unpack_ref(Wq)
    if bits == 2:
        return unpack2_ref(Wq)
    return Wq.view(np.int8).astype(np.int64)


def dot_ref64(Wq, Ws, xq, xd, bits=4):
    """fp64 dequantised matmul and its sum of |terms|, from int64 brute force."""
    qw = codes_of(Wq, bits)                     # rows x k
    rows, k = qw.shape
    P = (qw.reshape(rows, k // 32, 32) * xq.astype(np.int64).reshape(1, k // 32, 32)).sum(-1)
    terms = Ws.astype(np.float64)[:, None] * xd.astype(np.float64)[None, :] * P
    return terms.sum(1), np.abs(terms).sum(1), P


def within_tol(y, ref, absterm, what):
    err = np.abs(np.float64(y) - ref)
    bound = TOL_REL * absterm + TOL_ABS
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"{what}: {bad.size} outside tolerance, first {bad[:5]}, " \
                          f"err {err[bad[:5]]}, bound {bound[bad[:5]]}"


# ---------------------------------------------------------------- pins
def pin_nibble_codec(orc):
    # all 16 codes in both positions
    codes = np.arange(-8, 8, dtype=np.int8)
    pairs = np.array([(a, b) for a in codes for b in codes], dtype=np.int8).reshape(-1)
    packed = orc.pack_q4(pairs)
    assert np.array_equal(orc.unpack_q4(packed), pairs), "pack/unpack of all 256 code pairs"
    # explicit bytes: low nibble is the even column, two's complement
    for (a, b), byte in {(-1, 0): 0x0F, (0, -1): 0xF0, (-8, 7): 0x78, (7, -8): 0x87,
                         (1, 2): 0x21, (-7, 3): 0x39}.items():
        assert int(orc.pack_q4(np.array([a, b], np.int8))[0]) == byte, (a, b, byte)
    # all 256 bytes decode like arithmetic-shift sign extension and re-encode to themselves
    allb = np.arange(256, dtype=np.uint8)
    un = orc.unpack_q4(allb)
    assert np.array_equal(un.astype(np.int64), unpack_ref(allb)), "unpack of all 256 bytes"
    assert np.array_equal(orc.pack_q4(un), allb), "re-pack of all 256 bytes"
    # the pages' invariant: a dot over the packed form equals the dot over the int8 container
    rng = np.random.default_rng(1)
    for k in (32, 256, 6144):
        q = rng.integers(-8, 8, size=k).astype(np.int8)
        x = rng.integers(-127, 128, size=k).astype(np.int8)
        P = orc.row_partials(orc.pack_q4(q), x)
        ref = (q.astype(np.int64) * x.astype(np.int64)).reshape(-1, 32).sum(1)
        assert np.array_equal(P.astype(np.int64), ref), f"packed dot != int8 container dot, k={k}"


def pin_rint_ties(orc):
    rows = load_golden("rint_ties_q4.txt")
    for start in range(0, len(rows), 8):
        chunk = rows[start:start + 8]
        mult = [m for m, _ in chunk]
        if max(abs(m) for m in mult) != 7.0:
            mult = mult + [7.0]
            chunk = chunk + [(7.0, 7)]
        w = np.array(mult, dtype=np.float32) * np.float32(2.0 ** -3)
        q, s = orc.q4_quant_row(w)
        assert s == 2.0 ** -3, f"q4 scale {s}"
        assert [int(v) for v in q] == [e for _, e in chunk], f"q4 ties {mult} -> {list(q)}"
    rows = load_golden("rint_ties_q8.txt")
    assert len(rows) == 32
    x = np.array([m for m, _ in rows], dtype=np.float32) * np.float32(2.0 ** -5)
    q, d = orc.q8_quant(x)
    assert d[0] == np.float32(2.0 ** -5), f"q8 scale {d[0]}"
    assert [int(v) for v in q] == [e for _, e in rows], f"q8 ties -> {list(q)}"
    rows = load_golden("rint_ties_q8_d255.txt")
    assert len(rows) == 32
    x = np.array([m for m, _ in rows], dtype=np.float32) * np.float32(255.0)
    q, d = orc.q8_quant(x)
    assert d[0] == np.float32(255.0), f"q8 scale {d[0]}"
    assert [int(v) for v in q] == [e for _, e in rows], f"q8 ties, d=255 -> {list(q)}"


def pin_quant_closed_forms(orc):
    # Q8: a constant block maps to +-127 with d = |c| / 127
    for c in (1.0, -3.25, 1e-20, 7e30, -0.015625):
        x = np.full(64, c, dtype=np.float32)
        q, d = orc.q8_quant(x)
        assert np.all(q == (127 if c > 0 else -127)), f"q8 constant {c}"
        assert np.all(d == np.float32(abs(np.float32(c))) / np.float32(127.0)), f"q8 d {c}"
    q, d = orc.q8_quant(np.zeros(32, np.float32))
    assert np.all(q == 0) and d[0] == 0.0, "q8 zero block"
    # Q8 on random data: the largest magnitude maps to +-127, |q| <= 127 and q is the
    # nearest integer to the fp32 quotient x/d, ties to even
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(32 * 200) * rng.choice([1e-3, 1.0, 50.0], 32 * 200)).astype(np.float32)
    q, d = orc.q8_quant(x)
    xb, qb = x.reshape(-1, 32), q.reshape(-1, 32).astype(np.int64)
    am = np.argmax(np.abs(xb), axis=1)
    assert np.all(np.abs(qb[np.arange(len(am)), am]) == 127), "q8 max element -> 127"
    assert np.all(np.abs(qb) <= 127)
    ratio = (xb / d[:, None]).astype(np.float32).astype(np.float64)   # the fp32 quotient
    assert np.all(np.abs(ratio - qb) <= 0.5), "q8 not nearest"
    tie = np.abs(ratio - qb) == 0.5
    assert np.all(qb[tie] % 2 == 0), "q8 tie not to even"
    # Q4: constant row -> +-7, zero row -> 0, nearest-integer property
    for c in (0.02, -1.5, 3e-30):
        q, s = orc.q4_quant_row(np.full(48, c, np.float32))
        assert np.all(q == (7 if c > 0 else -7)) and s == np.float32(abs(np.float32(c))) / np.float32(7)
    q, s = orc.q4_quant_row(np.zeros(64, np.float32))
    assert s == 0.0 and np.all(q == 0), "q4 zero row"
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    packed, sc = orc.q4_quant(w)
    qi = unpack_ref(packed)
    assert np.all(np.abs(qi) <= 7) and np.all(np.abs(qi).max(1) == 7), "q4 range / max -> 7"
    ratio = (w / sc[:, None]).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(ratio - qi) <= 0.5), "q4 not nearest"
    assert np.all(qi[np.abs(ratio - qi) == 0.5] % 2 == 0), "q4 tie not to even"
    assert np.all(sc == np.abs(w).max(1) / np.float32(7)), "q4 scale"
    # constant weights and constant activations: P = 32 * 7 * 127 per block
    P = orc.row_partials(orc.pack_q4(np.full(64, 7, np.int8)), np.full(64, 127, np.int8))
    assert np.all(P == 32 * 7 * 127)
    P = orc.row_partials(orc.pack_q4(np.full(64, -8, np.int8)), np.full(64, -127, np.int8))
    assert np.all(P == 32 * 8 * 127), "code 8 decodes to -8"


def pin_partials_bruteforce(orc):
    rng = np.random.default_rng(3)
    for rows, k in ((7, 32), (33, 256), (64, 2048)):
        q = rng.integers(-8, 8, size=(rows, k)).astype(np.int8)
        Wq = orc.pack_q4(q)
        Ws = rng.uniform(0.5, 2.0, rows).astype(np.float32)
        xq = rng.integers(-127, 128, size=k).astype(np.int8)
        xd = rng.uniform(0.01, 0.1, k // 32).astype(np.float32)
        _, P, _ = orc.matvec(Wq, Ws, xq, xd, want_partials=True)
        ref = np.einsum("rbj,bj->rb", q.astype(np.int64).reshape(rows, -1, 32),
                        xq.astype(np.int64).reshape(-1, 32))
        assert np.array_equal(P.astype(np.int64), ref), f"partials {rows}x{k}"


def pin_dot_fp64(orc):
    rng = np.random.default_rng(4)
    for rows, k in ((16, 256), (64, 6144)):
        w = (rng.standard_normal((rows, k)) * 0.02).astype(np.float32)
        Wq, Ws = orc.q4_quant(w)
        x = rng.standard_normal(k).astype(np.float32)
        xq, xd = orc.q8_quant(x)
        y, _, A = orc.matvec(Wq, Ws, xq, xd, want_absterm=True)
        ref, absterm, _ = dot_ref64(Wq, Ws, xq, xd)
        within_tol(y, ref, absterm, f"matvec {rows}x{k}")
        assert np.allclose(A, absterm, rtol=1e-12), "oracle absterm != sum |terms|"
    # a single block is a closed form: fl(fl(P * d) * s)
    for P, d, s in ((28448, 0.0078125, 0.5), (-12345, 3.1e-3, 7.7e-3), (1, 1e-30, 1e10)):
        ref = np.float32(np.float32(np.float64(P) * np.float64(np.float32(d))) * np.float32(s))
        got = orc.rescale(np.array([P], np.int32), np.array([d], np.float32), np.float32(s))
        assert np.float32(got) == ref, (P, d, s, got, ref)


def pin_exp(orc):
    xs = np.concatenate([np.linspace(-87.0, 88.5, 400001, dtype=np.float32),
                         np.linspace(-1.0, 1.0, 100001, dtype=np.float32),
                         np.float32([0.0, -0.0, 1e-30, -1e-30, 1e-8])])
    e = orc.expf_vec(xs)
    ref = np.exp(xs.astype(np.float64))
    u = ulp_dist(e, ref)
    assert u.max() <= 1.0, f"exp max ulp error {u.max()} at x={xs[np.argmax(u)]}"
    assert orc.expf(0.0) == 1.0
    for n in range(-125, 128):
        v = orc.expf(np.float32(n * math.log(2.0)))
        assert ulp_dist(v, math.exp(float(np.float32(n * math.log(2.0))))) <= 1.0, n
    srt = np.sort(xs)
    assert np.all(np.diff(orc.expf_vec(srt).astype(np.float64)) >= 0), "exp not monotone"
    assert orc.expf(100.0) == orc.expf(88.5) and np.isfinite(orc.expf(1000.0))
    assert orc.expf(-100.0) == orc.expf(-87.0) and orc.expf(-87.0) > 0
    # sigmoid and silu against float64
    xs = np.linspace(-30.0, 30.0, 200001, dtype=np.float32)
    sg = orc.sigmoidf_vec(xs)
    sref = 1.0 / (1.0 + np.exp(-xs.astype(np.float64)))
    # exp (<= 1 ulp), the add and the divide (<= 1/2 ulp each) compound to < 3 ulp
    assert ulp_dist(sg, sref).max() <= 3.0, "sigmoid"
    assert orc.sigmoidf(0.0) == 0.5
    assert np.all(np.diff(sg.astype(np.float64)) >= 0), "sigmoid not monotone"
    sl = orc.siluf_vec(xs)
    lref = xs.astype(np.float64) * sref
    assert ulp_dist(sl, lref).max() <= 3.0, "silu"
    assert orc.siluf(0.0) == 0.0


def _route_ref(logits, bias, k, routed_scale):
    """float64 reference for inputs whose selection scores have no near ties."""
    T, E = logits.shape
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    c = s + bias.astype(np.float64)[None, :]
    idx = np.array([sorted(range(E), key=lambda e: (-c[t, e], e))[:k] for t in range(T)])
    sel = np.take_along_axis(s, idx, 1)
    w = sel / sel.sum(1, keepdims=True) * routed_scale
    return idx, w, c


def pin_route(orc):
    # distinct logits, no bias: sigmoid is monotone, so the order is argsort
    lg = np.array([[0.3, -1.2, 2.5, 0.9, -0.1, 1.7, -2.2, 0.05]], np.float32)
    idx, w = orc.route(lg, np.zeros(8, np.float32), 3)
    assert idx.tolist() == [[2, 5, 3]], idx
    # exact ties go to the lower index
    lg = np.array([[1.0, 2.0, 1.0, 2.0, 2.0, 0.0]], np.float32)
    idx, w = orc.route(lg, np.zeros(6, np.float32), 4)
    assert idx.tolist() == [[1, 3, 4, 0]], idx
    # a bias flips the order but does not enter the weights
    lg = np.array([[2.0, 1.0, -3.0]], np.float32)
    b = np.array([0.0, 0.5, 0.0], np.float32)
    idx, w = orc.route(lg, b, 2)
    assert idx.tolist() == [[1, 0]], idx
    s1, s0 = 1 / (1 + math.exp(-1.0)), 1 / (1 + math.exp(-2.0))
    assert abs(w[0, 0] - s1 / (s0 + s1)) < 1e-6 and abs(w[0, 1] - s0 / (s0 + s1)) < 1e-6
    # all-equal scores: the first k experts, equal weights (exact for logit 0)
    idx, w = orc.route(np.zeros((2, 16), np.float32), np.zeros(16, np.float32), 8)
    assert idx.tolist() == [list(range(8))] * 2 and np.all(w == 0.125)
    # k = E with negative logits is a full sort
    rng = np.random.default_rng(5)
    lg = -np.abs(rng.standard_normal((3, 16))).astype(np.float32) - 0.5
    idx, w = orc.route(lg, np.zeros(16, np.float32), 16)
    for t in range(3):
        assert idx[t].tolist() == sorted(range(16), key=lambda e: (-float(lg[t, e]), e))
    # random scale-256 routing against float64, where no near tie makes it ambiguous
    T, E, k = 64, 256, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    for scale in (1.0, 2.5):
        idx, w = orc.route(lg, b, k, scale)
        ridx, rw, c = _route_ref(lg, b, k, scale)
        cs = np.sort(c, 1)[:, ::-1]
        clear = np.min(np.abs(np.diff(cs[:, : k + 1], axis=1)), axis=1) > 1e-5
        assert clear.sum() > T // 2
        assert np.array_equal(idx[clear], ridx[clear]), "route vs float64"
        assert np.all(ulp_dist(w[clear], rw[clear]) <= 4), "weights vs float64"
        assert np.all(np.abs(w.astype(np.float64).sum(1) - scale) <= k * 1.2e-7 * scale)


def _tiny_expert(orc, rng, D, F, sigma=0.02, bits=4):
    from oracle import Expert
    ws = [(rng.standard_normal(shape) * sigma).astype(np.float32)
          for shape in ((F, D), (F, D), (D, F))]
    return Expert.quantize(*ws, orc=orc, bits=bits)


def _silu64(g):
    return g / (1.0 + np.exp(-g))


def pin_expert_fp64(orc):
    for bits, seed in ((4, 6), (8, 16), (2, 26)):
        _expert_fp64(orc, bits, np.random.default_rng(seed))


def _expert_fp64(orc, bits, rng):
    D, F = 256, 128
    ex = _tiny_expert(orc, rng, D, F, bits=bits)
    x = rng.standard_normal(D).astype(np.float32)
    xq, xd = orc.q8_quant(x)
    r = orc.expert_forward(ex, xq, xd, want_partials=True)
    g64, ga, Pg = dot_ref64(ex.gate_q, ex.gate_s, xq, xd, bits)
    u64, ua, Pu = dot_ref64(ex.up_q, ex.up_s, xq, xd, bits)
    assert np.array_equal(r["P_gate"], Pg) and np.array_equal(r["P_up"], Pu)
    within_tol(r["g"], g64, ga, "gate")
    within_tol(r["u"], u64, ua, "up")
    # h = silu(g) u, from the oracle's own fp32 g, u (isolates the activation step)
    h64 = _silu64(r["g"].astype(np.float64)) * r["u"].astype(np.float64)
    assert np.all(np.abs(r["h"] - h64) <= 4 * np.spacing(np.abs(np.float32(h64))) + 1e-30), "h"
    # Q8(h): nearest-integer property and scale
    hb = r["h"].reshape(-1, 32)
    assert np.all(r["hd"] == np.abs(hb).max(1) / np.float32(127))
    ratio = (hb / r["hd"][:, None]).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(ratio - r["hq"].reshape(-1, 32)) <= 0.5)
    # the down projection of the oracle's Q8(h), in fp64
    o64, oa, Pd = dot_ref64(ex.down_q, ex.down_s, r["hq"], r["hd"], bits)
    assert np.array_equal(r["P_down"], Pd)
    within_tol(r["o"], o64, oa, "down")
    assert np.allclose(r["abs_o"], oa, rtol=1e-12)


def pin_moe_invariants(orc):
    rng = np.random.default_rng(7)
    D, F, E, k, T = 256, 128, 16, 2, 6
    shared = _tiny_expert(orc, rng, D, F)
    same = _tiny_expert(orc, rng, D, F)
    distinct = {e: _tiny_expert(orc, rng, D, F) for e in range(E)}
    x = rng.standard_normal((T, D)).astype(np.float32)
    xq, xd = orc.q8_quant(x)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    idx, w = orc.route(lg, b, k)
    # (a) every routed expert identical: y = o_shared + (sum w) * o  (fp64, tolerance)
    table = {e: same for e in range(E)}
    table[E] = shared
    y, A = orc.moe_layer(table, E, 1, xq, xd, idx, w)
    for t in range(T):
        os_ = orc.expert_forward(shared, xq[t], xd[t])
        o = orc.expert_forward(same, xq[t], xd[t])
        ref = os_["o"].astype(np.float64) + w[t].astype(np.float64).sum() * o["o"].astype(np.float64)
        within_tol(y[t], ref, A[t], "identical experts")
        assert np.allclose(A[t], os_["abs_o"] + np.abs(w[t]).sum() * o["abs_o"])
    # (b) distinct experts: brute-force combine in fp64 over the oracle's expert outputs
    table = dict(distinct)
    table[E] = shared
    y, A = orc.moe_layer(table, E, 1, xq, xd, idx, w)
    for t in range(T):
        ref = orc.expert_forward(shared, xq[t], xd[t])["o"].astype(np.float64)
        for j in range(k):
            ref = ref + float(w[t, j]) * orc.expert_forward(distinct[int(idx[t, j])], xq[t],
                                                            xd[t])["o"].astype(np.float64)
        within_tol(y[t], ref, A[t], "combine")
    # (c) permuting tokens permutes outputs bit for bit
    perm = rng.permutation(T)
    yp, _ = orc.moe_layer(table, E, 1, xq[perm], xd[perm], idx[perm], w[perm])
    assert np.array_equal(yp, y[perm]), "token permutation"
    # (d) zero routing weights leave exactly the shared expert's output
    y0, _ = orc.moe_layer(table, E, 1, xq, xd, idx, np.zeros_like(w))
    for t in range(T):
        assert np.array_equal(y0[t], orc.expert_forward(shared, xq[t], xd[t])["o"])
    # (e) accumulate adds the layer output to the residual in fp32
    res = rng.standard_normal((T, D)).astype(np.float32)
    ya, _ = orc.moe_layer(table, E, 1, xq, xd, idx, w, out=res, accumulate=True)
    assert np.array_equal(ya, res + y), "residual accumulate"
    # (f) no shared expert, k = 1, w = 1: the routed expert's output exactly
    y1, _ = orc.moe_layer(distinct, E, 0, xq, xd, idx[:, :1], np.ones((T, 1), np.float32))
    for t in range(T):
        assert np.array_equal(y1[t], orc.expert_forward(distinct[int(idx[t, 0])], xq[t], xd[t])["o"])


def pin_dropped_entries(orc):
    """Routings a caller hands to the forward may hold an index outside [0, E)
    or the same expert twice in one token; the rule: an entry is served when it
    is in range and no earlier slot of its token holds the same expert.
    Pinned against a brute-force reading of that rule, and the layer with
    dropped entries against the strict layer run on each token's kept slots."""
    def brute(idx, E):
        keep = np.zeros(idx.shape, np.uint8)
        for t in range(idx.shape[0]):
            seen = set()
            for j in range(idx.shape[1]):
                e = int(idx[t, j])
                if 0 <= e < E and e not in seen:
                    keep[t, j] = 1
                seen.add(e)
        return keep
    hand = [(np.int32([[5, 5]]), 16, [[1, 0]]),
            (np.int32([[0, 16], [3, -2]]), 16, [[1, 0], [1, 0]]),
            (np.int32([[3, -1, 3, 7]]), 16, [[1, 0, 0, 1]]),
            (np.int32([[2, 2, 2, 2], [1, 0, 1, 0]]), 4, [[1, 0, 0, 0], [1, 1, 0, 0]]),
            (np.int32([[7, 8, 7, 9]]), 8, [[1, 0, 0, 0]])]
    for idx, E, ref in hand:
        keep, n = orc.keep_entries(idx, E)
        assert keep.tolist() == ref, (idx.tolist(), keep.tolist())
        assert n == int((keep == 0).sum())
    rng = np.random.default_rng(21)
    for T, E, k in ((40, 16, 4), (9, 8, 8), (64, 256, 8)):
        idx = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
        idx[::3, 1] = idx[::3, 0]                 # plenty of repeats
        keep, _ = orc.keep_entries(idx, E)
        assert np.array_equal(keep, brute(idx, E)), (T, E, k)
        counts, lists, na, active = orc.dispatch(idx, E, 1, keep=keep)
        for e in range(E + 1):
            ref = [t * (k + 1) + (k if e == E else j) for t in range(T) for j in range(k)
                   if (e == E and j == 0) or (e < E and keep[t, j] and idx[t, j] == e)]
            assert counts[e] == len(ref) and lists[e, : counts[e]].tolist() == ref, (T, E, e)
        assert active.tolist() == [e for e in range(E + 1) if counts[e] > 0]
    # the layer: dropped entries contribute nothing, kept ones keep their order
    D, F, E, k, T = 256, 128, 16, 4, 6
    table = {e: _tiny_expert(orc, rng, D, F) for e in range(E + 1)}
    x = rng.standard_normal((T, D)).astype(np.float32)
    xq, xd = orc.q8_quant(x)
    idx = np.int32([[3, 3, 5, 9], [16, 2, -1, 2], [7, 1, 7, 1], [4, 4, 4, 4], [0, 1, 2, 3],
                    [-5, 20, 16, 99]])
    w = rng.uniform(0.05, 0.5, size=(T, k)).astype(np.float32)
    keep, _ = orc.keep_entries(idx, E)
    y, _ = orc.moe_layer(table, E, 1, xq, xd, idx, w, keep=keep)
    for t in range(T):
        J = [j for j in range(k) if keep[t, j]]
        ys, _ = orc.moe_layer(table, E, 1, xq[t:t + 1], xd[t:t + 1],
                              idx[t:t + 1, J].reshape(1, len(J)), w[t:t + 1, J].reshape(1, len(J)))
        assert np.array_equal(y[t], ys[0]), f"token {t} with dropped entries"
    assert np.array_equal(y[5], orc.expert_forward(table[E], xq[5], xd[5])["o"]), "all dropped"


def pin_rmsnorm(orc):
    eps = np.float32(1e-6)
    for c in (1.0, -0.37, 25.0, 1e-4):
        h = np.full((1, 256), c, np.float32)
        out, r = orc.rmsnorm(h, eps)
        c32 = float(np.float32(c))
        rr = np.float32(1.0 / math.sqrt(c32 * c32 + float(eps)))
        assert r[0] == rr, (c, r[0], rr)
        assert np.all(out == np.float32(c) * rr)
    rng = np.random.default_rng(8)
    h = rng.standard_normal((5, 6144)).astype(np.float32) * 3
    out, r = orc.rmsnorm(h, eps)
    ref = 1.0 / np.sqrt((h.astype(np.float64) ** 2).mean(1) + float(eps))
    assert np.all(ulp_dist(r, ref) <= 0.5 + 1e-6), "rmsnorm scale vs float64"
    # unit root-mean-square after the norm
    assert np.allclose(np.sqrt((out.astype(np.float64) ** 2).mean(1)), 1.0, atol=1e-5)


def pin_router_logits(orc):
    """Router projection: closed form, exact small-integer dots, and the
    correctly rounded exact sum (math.fsum) within half an fp32 ulp plus the
    fp64 rounding of the ascending sum."""
    # constant inputs: 6144 * 0.5 * 0.25 = 768 exactly
    lg = orc.router_logits(np.full((2, 6144), 0.25, np.float32), np.full((3, 6144), 0.5, np.float32))
    assert lg.shape == (2, 3) and np.all(lg == 768.0)
    # small integers: every partial sum is an exact integer
    rng = np.random.default_rng(21)
    xi = rng.integers(-3, 4, size=(3, 1000))
    wi = rng.integers(-3, 4, size=(5, 1000))
    lg = orc.router_logits(xi.astype(np.float32), wi.astype(np.float32))
    assert np.array_equal(lg, (xi @ wi.T).astype(np.float32)), "integer router logits"
    # random fp32 inputs at the page shape (T != E, so a transposed operand fails)
    x = rng.standard_normal((3, 6144)).astype(np.float32)
    w = (rng.standard_normal((7, 6144)) * 0.02).astype(np.float32)
    lg = orc.router_logits(x, w)
    ref = np.array([[math.fsum((x[t].astype(np.float64) * w[e].astype(np.float64)).tolist())
                     for e in range(7)] for t in range(3)])
    assert np.all(ulp_dist(lg, ref) <= 0.5 + 1e-3), "router logits vs the exact sum"


def pin_dispatch(orc):
    rng = np.random.default_rng(9)
    for T, E, k, S in ((4, 16, 2, 1), (37, 256, 8, 1), (5, 16, 3, 0)):
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, lists, na, active = orc.dispatch(idx, E, S)
        for e in range(E + S):
            ref = [t * (k + S) + (k if e == E else j)
                   for t in range(T) for j in range(k) if (e == E and j == 0) or
                   (e < E and idx[t, j] == e)]
            assert counts[e] == len(ref) and lists[e, : counts[e]].tolist() == ref, (T, E, e)
        assert active.tolist() == [e for e in range(E + S) if counts[e] > 0]
    for bad in (np.array([[0, 16]], np.int32), np.array([[-1, 2]], np.int32),
                np.array([[3, 3]], np.int32)):
        try:
            orc.dispatch(bad, 16, 1)
        except ValueError:
            continue
        raise AssertionError(f"dispatch accepted {bad}")


def pin_int8_quant(orc):
    """Per-row int8 weights: scale 2^-3 makes every quotient exact, so the
    codes of half-integer multiples are the textbook round-half-to-even."""
    mult = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 125.5, 126.5, -126.5, 127.0, -3.0]
    want = [0, 2, 2, 4, 0, -2, -2, 126, 126, -126, 127, -3]
    q, s = orc.q8w_quant_row(np.array(mult, np.float32) * np.float32(2.0 ** -3))
    assert s == 2.0 ** -3, f"int8 scale {s}"
    assert [int(v) for v in q] == want, f"int8 ties -> {list(q)}"
    for c in (0.02, -1.5, 3e-30):
        q, s = orc.q8w_quant_row(np.full(48, c, np.float32))
        assert np.all(q == (127 if c > 0 else -127))
        assert s == np.float32(abs(np.float32(c))) / np.float32(127)
    q, s = orc.q8w_quant_row(np.zeros(64, np.float32))
    assert s == 0.0 and np.all(q == 0), "int8 zero row"
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    qi, sc = orc.q8w_quant(w)
    qi = qi.astype(np.int64)
    assert np.all(np.abs(qi) <= 127) and np.all(np.abs(qi).max(1) == 127), "int8 range / max"
    ratio = (w / sc[:, None]).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(ratio - qi) <= 0.5), "int8 not nearest"
    assert np.all(qi[np.abs(ratio - qi) == 0.5] % 2 == 0), "int8 tie not to even"
    assert np.all(sc == np.abs(w).max(1) / np.float32(127)), "int8 scale"
    # each row is the same rule applied alone
    q0, s0 = orc.q8w_quant_row(w[5])
    assert np.array_equal(q0.astype(np.int64), qi[5]) and s0 == sc[5]


def pin_int8_container(orc):
    """The int8 container through the dot: brute-force int64 partials over the
    full code range, fp64 dequantised matvec, and the pages' invariant that the
    nibble container and the int8 container holding the same codes give
    identical results, from the partials up to the layer output."""
    from oracle import Expert
    rng = np.random.default_rng(18)
    for rows, k in ((7, 32), (33, 256), (64, 2048)):
        q = rng.integers(-127, 128, size=(rows, k)).astype(np.int8)
        Ws = rng.uniform(0.5, 2.0, rows).astype(np.float32)
        xq = rng.integers(-127, 128, size=k).astype(np.int8)
        xd = rng.uniform(0.01, 0.1, k // 32).astype(np.float32)
        _, P, _ = orc.matvec(q, Ws, xq, xd, want_partials=True, bits=8)
        ref = np.einsum("rbj,bj->rb", q.astype(np.int64).reshape(rows, -1, 32),
                        xq.astype(np.int64).reshape(-1, 32))
        assert np.array_equal(P.astype(np.int64), ref), f"int8 partials {rows}x{k}"
    P = orc.row_partials(np.full(64, 127, np.int8), np.full(64, -127, np.int8), bits=8)
    assert np.all(P == -32 * 127 * 127), "int8 extreme block"
    for rows, k in ((16, 256), (64, 6144)):
        w = (rng.standard_normal((rows, k)) * 0.02).astype(np.float32)
        Wq, Ws = orc.q8w_quant(w)
        xq, xd = orc.q8_quant(rng.standard_normal(k).astype(np.float32))
        y, _, _ = orc.matvec(Wq, Ws, xq, xd, bits=8)
        ref, absterm, _ = dot_ref64(Wq, Ws, xq, xd, bits=8)
        within_tol(y, ref, absterm, f"int8 matvec {rows}x{k}")
    # same codes in both containers -> identical results
    D, F, E, k, T = 256, 128, 6, 2, 5
    pair = {}
    for e in range(E + 1):
        mats = [rng.integers(-8, 8, size=shape).astype(np.int8) for shape in ((F, D), (F, D), (D, F))]
        sc = [rng.uniform(1e-3, 1e-2, m.shape[0]).astype(np.float32) for m in mats]
        pair[e] = (Expert(orc.pack_q4(mats[0]), sc[0], orc.pack_q4(mats[1]), sc[1],
                          orc.pack_q4(mats[2]), sc[2], bits=4),
                   Expert(mats[0], sc[0], mats[1], sc[1], mats[2], sc[2], bits=8))
    xq, xd = orc.q8_quant(rng.standard_normal((T, D)).astype(np.float32))
    r4 = orc.expert_forward(pair[0][0], xq[0], xd[0], want_partials=True)
    r8 = orc.expert_forward(pair[0][1], xq[0], xd[0], want_partials=True)
    for key in r4:
        assert np.array_equal(r4[key], r8[key]), f"container identity: {key}"
    idx, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), np.zeros(E, np.float32), k)
    y4, _ = orc.moe_layer({e: p[0] for e, p in pair.items()}, E, 1, xq, xd, idx, w)
    y8, _ = orc.moe_layer({e: p[1] for e, p in pair.items()}, E, 1, xq, xd, idx, w)
    assert np.array_equal(y4, y8), "container identity: layer output"


def _lru_reference(refs, capacity):
    """Textbook LRU over single references: a recency list, most recent last.
    Returns the hit flags and the resident set after each reference."""
    recency, hits, sets = [], [], []
    for r in refs:
        if r in recency:
            recency.remove(r)
            hits.append(True)
        else:
            if len(recency) == capacity:
                recency.pop(0)
            hits.append(False)
        recency.append(r)
        sets.append(set(recency))
    return hits, sets


def pin_tier(orc):
    """Expert tier: a hand-worked LRU sequence (slots and loads written out),
    an independent recency-list LRU on one-expert passes, the LRU inclusion
    property, invariants with several experts per pass, pinned and shared
    experts, usage counts, and the pin ranking against Python's sorted."""
    from oracle import Tier
    # hand-worked: capacity 3, references 0 1 2 0 3 0 4 2 3 0 (one token, k = 1, no shared)
    t = Tier(orc, 8, 0, 3)
    refs = [0, 1, 2, 0, 3, 0, 4, 2, 3, 0]
    want_loads = [[0], [1], [2], [], [1], [], [2], [1], [0], [2]]
    got = [t.plan(np.array([[r]], np.int32)) for r in refs]
    assert [list(l) for l, _ in got] == want_loads, [list(l) for l, _ in got]
    assert [h for _, h in got] == [0, 0, 0, 1, 0, 1, 0, 0, 0, 0]
    assert t.expert_in.tolist() == [3, 2, 0] and t.slot_of[[0, 2, 3]].tolist() == [2, 1, 0]
    assert np.all(t.slot_of[[1, 4, 5, 6, 7]] == -1)
    # one expert per pass: identical to the recency-list LRU; hits grow with capacity
    rng = np.random.default_rng(41)
    p = 1.0 / np.arange(1, 33) ** 1.1
    refs = rng.choice(32, size=400, p=p / p.sum())
    prev = None
    for cap in (2, 5, 9, 16):
        t = Tier(orc, 32, 0, cap)
        hits = [t.plan(np.array([[r]], np.int32))[1] == 1 for r in refs]
        ref_hits, _ = _lru_reference(list(refs), cap)
        assert hits == ref_hits, f"LRU hits differ at capacity {cap}"
        resident = set(int(e) for e in t.expert_in if e >= 0)
        assert resident == _lru_reference(list(refs), cap)[1][-1]
        if prev is not None:
            assert all(h or not ph for h, ph in zip(hits, prev)), "LRU inclusion"
        prev = hits
    # several experts per pass, a shared expert and pinned experts
    E, S, k, T, slots = 16, 1, 2, 3, 12
    pin = [5, 2]
    t = Tier(orc, E, S, slots, pin)
    assert t.init_loads.tolist() == [0, 1, 2] and t.expert_in[:3].tolist() == [E, 5, 2]
    usage = np.zeros(E + S, np.int64)
    for step in range(60):
        idx = np.stack([rng.choice(E, k, replace=False, p=None) for _ in range(T)]).astype(np.int32)
        before = t.expert_in.copy()
        loads, hits = t.plan(idx)
        need = set(idx.reshape(-1).tolist()) | {E}
        assert hits + len(loads) == len(need)
        assert hits == len(need & set(int(e) for e in before if e >= 0))
        assert all(t.slot_of[e] >= 0 and t.expert_in[t.slot_of[e]] == e for e in need)
        assert t.expert_in[:3].tolist() == [E, 5, 2], "pinned slots evicted"
        assert len(set(loads.tolist())) == len(loads) and all(t.pinned[s] == 0 for s in loads)
        assert all(t.stamp[t.slot_of[e]] == step for e in need)
        np.add.at(usage, idx.reshape(-1), 1)
        usage[E] += T
    assert np.array_equal(t.usage, usage), "usage counts"
    # a prefetch plan moves experts in without counting usage
    u0 = t.usage.copy()
    t.plan(np.array([[0, 1]], np.int32), count_usage=False)
    assert np.array_equal(t.usage, u0)
    # too many experts for the unpinned slots
    t = Tier(orc, 16, 1, 4, [3])
    t.plan(np.array([[0, 1]], np.int32))
    state = [a.copy() for a in (t.slot_of, t.expert_in, t.stamp, t.usage)]
    try:
        t.plan(np.array([[0, 1], [2, 4]], np.int32))   # 0, 1 hit; 2, 4 need 2 more slots
    except ValueError:
        pass
    else:
        raise AssertionError("tier accepted more experts than slots")
    assert all(np.array_equal(a, b) for a, b in zip(state, (t.slot_of, t.expert_in, t.stamp,
                                                             t.usage))), "rejected plan changed the tier"
    t.plan(np.array([[0, 3], [1, 3]], np.int32))          # fits: 3 is pinned
    # pin ranking
    u = rng.integers(0, 5, size=40).astype(np.int32)
    t = Tier(orc, 40, 0, 4)
    t.usage[:] = u
    assert t.pin_top(12).tolist() == sorted(range(40), key=lambda e: (-int(u[e]), e))[:12]


def pin_int2(orc):
    """The 2-bit container: all 256 bytes decode like sign extension and
    re-encode to themselves, a hand-packed byte, textbook ties of the int2
    quantiser at s = 2^-2, brute-force partials over the full field range,
    the fp64 dequantised matvec, and the same codes in the 2-bit, nibble and
    int8 containers giving identical results (the pages' invariant)."""
    from oracle import Expert
    allb = np.arange(256, dtype=np.uint8)
    un = orc.unpack_q2(allb)
    assert np.array_equal(un.astype(np.int64), unpack2_ref(allb)), "unpack of all 256 bytes"
    assert np.array_equal(orc.pack_q2(un), allb), "re-pack of all 256 bytes"
    # codes 1, -1, 0, -2 -> fields 01, 11, 00, 10 from the lowest bits up
    assert int(orc.pack_q2(np.array([1, -1, 0, -2], np.int8))[0]) == 0b10_00_11_01
    mult = [0.5, -0.5, 0.75, -0.25, 1.0, -1.0, 0.0, 0.25]
    q, sc = orc.q2_quant_row(np.array(mult, np.float32) * np.float32(0.25))
    assert sc == 0.25 and [int(v) for v in q] == [0, 0, 1, 0, 1, -1, 0, 0], (sc, list(q))
    q, sc = orc.q2_quant_row(np.full(32, -3.5, np.float32))
    assert sc == 3.5 and np.all(q == -1)
    q, sc = orc.q2_quant_row(np.zeros(32, np.float32))
    assert sc == 0.0 and np.all(q == 0)
    rng = np.random.default_rng(27)
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    packed, sc = orc.q2_quant(w)
    qi = unpack2_ref(packed)
    assert np.all(np.abs(qi) <= 1) and np.all(np.abs(qi).max(1) == 1), "int2 range / max"
    ratio = (w / sc[:, None]).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(ratio - qi) <= 0.5), "int2 not nearest"
    assert np.all(qi[np.abs(ratio - qi) == 0.5] % 2 == 0), "int2 tie not to even"
    assert np.all(sc == np.abs(w).max(1)), "int2 scale"
    for rows, k in ((7, 32), (33, 256), (64, 2048)):
        q = rng.integers(-2, 2, size=(rows, k)).astype(np.int8)
        xq = rng.integers(-127, 128, size=k).astype(np.int8)
        xd = rng.uniform(0.01, 0.1, k // 32).astype(np.float32)
        Ws = rng.uniform(0.5, 2.0, rows).astype(np.float32)
        _, P, _ = orc.matvec(orc.pack_q2(q), Ws, xq, xd, want_partials=True, bits=2)
        ref = np.einsum("rbj,bj->rb", q.astype(np.int64).reshape(rows, -1, 32),
                        xq.astype(np.int64).reshape(-1, 32))
        assert np.array_equal(P.astype(np.int64), ref), f"int2 partials {rows}x{k}"
    w = (rng.standard_normal((64, 6144)) * 0.02).astype(np.float32)
    Wq, Ws = orc.q2_quant(w)
    xq, xd = orc.q8_quant(rng.standard_normal(6144).astype(np.float32))
    y, _, _ = orc.matvec(Wq, Ws, xq, xd, bits=2)
    ref, absterm, _ = dot_ref64(Wq, Ws, xq, xd, bits=2)
    within_tol(y, ref, absterm, "int2 matvec")
    D, F, E, k, T = 256, 128, 6, 2, 5
    experts = {2: {}, 4: {}, 8: {}}
    for e in range(E + 1):
        mats = [rng.integers(-2, 2, size=shape).astype(np.int8) for shape in ((F, D), (F, D), (D, F))]
        sc = [rng.uniform(1e-3, 1e-2, m.shape[0]).astype(np.float32) for m in mats]
        experts[2][e] = Expert(*[a for m, s_ in zip(mats, sc) for a in (orc.pack_q2(m), s_)], bits=2)
        experts[4][e] = Expert(*[a for m, s_ in zip(mats, sc) for a in (orc.pack_q4(m), s_)], bits=4)
        experts[8][e] = Expert(*[a for m, s_ in zip(mats, sc) for a in (m, s_)], bits=8)
    xq, xd = orc.q8_quant(rng.standard_normal((T, D)).astype(np.float32))
    idx, wt = orc.route(rng.standard_normal((T, E)).astype(np.float32), np.zeros(E, np.float32), k)
    y = {b: orc.moe_layer(experts[b], E, 1, xq, xd, idx, wt)[0] for b in (2, 4, 8)}
    assert np.array_equal(y[2], y[8]) and np.array_equal(y[4], y[8]), "container identity"


ALL_PINS = [pin_nibble_codec, pin_rint_ties, pin_quant_closed_forms, pin_partials_bruteforce,
            pin_dot_fp64, pin_exp, pin_route, pin_expert_fp64, pin_moe_invariants, pin_rmsnorm,
            pin_dispatch, pin_router_logits, pin_int8_quant, pin_int8_container, pin_tier,
            pin_int2, pin_dropped_entries]
