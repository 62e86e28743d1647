"""Pins of the CPU oracle to facts fixed by the definitions, not by itself.

- hand-worked fixtures under tests/golden/ (values derived on paper);
- IEEE-754 bf16 rounding at hand-derived bit patterns, and PyTorch's own
  fp32 -> bf16 conversion on random and special values;
- brute force (bincount + stable argsort + route-side scatter) on many tiny
  random cases, including duplicates, bad ids, all-masked, T = 0, A = 1, E = 1
  and overflowing capacities;
- closed forms: identity experts give RNE(n_valid * x); power-of-two expert
  scales give RNE(sum_k c_k * x); weights summing to one give x within a
  derived bound;
- adjoint (VJP) identities in exact small-integer arithmetic;
- masked routes contribute nothing;
- planted mistakes are caught by the checkers used on the GPU outputs.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
import brute
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex(a):
    return np.array([[int(v, 16) for v in row] for row in a], dtype=np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build()


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def _f32(bits):
    return float(np.array([bits], np.uint32).view(np.float32)[0])


# (fp32 bits, bf16 bits) worked out from round-to-nearest-even on the top 16 bits
RNE_CASES = [
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # 1 + 2^-8: tie, even is 0x3F80
    (0x3F818000, 0x3F82),  # tie between 0x3F81 and 0x3F82 -> even 0x3F82
    (0x3F808001, 0x3F81),  # just above the tie
    (0x3F807FFF, 0x3F80),  # just below the tie
    (0xBF808001, 0xBF81),  # negative, rounds away in magnitude
    (0x7F7FFFFF, 0x7F80),  # max float rounds to +inf
    (0x7F7F7FFF, 0x7F7F),  # stays at max bf16
    (0xFF7FFFFF, 0xFF80),  # -> -inf
    (0x7F800000, 0x7F80),  # +inf
    (0xFF800000, 0xFF80),  # -inf
    (0x00000000, 0x0000),  # +0
    (0x80000000, 0x8000),  # -0
    (0x00010000, 0x0001),  # smallest bf16 subnormal, exact
    (0x00008000, 0x0000),  # half of it: tie to even 0
    (0x00018000, 0x0002),  # 1.5 x smallest subnormal: tie to even 2
    (0x00008001, 0x0001),  # above half: rounds up to the smallest subnormal
    (0x007FFFFF, 0x0080),  # largest fp32 subnormal rounds up to min normal
    (0x7FC00000, 0x7FC0),  # quiet NaN
    (0xFFC00001, 0x7FC0),  # negative NaN with payload -> canonical
    (0x7F800001, 0x7FC0),  # signalling NaN -> canonical quiet NaN
]


@pytest.mark.parametrize("f_bits,want", RNE_CASES)
def test_bf16_rne_hand_values(f_bits, want):
    assert oracle.f32_to_bf16(_f32(f_bits)) == want


def test_bf16_rne_matches_torch_on_random_and_specials():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x3F808000, 0x00008000, 0x7F7FFFFF, 0x80000000, 0x00018000],
                        np.uint32)
    bits = np.concatenate([bits, specials])
    vals = bits.view(np.float32)
    want = brute.f32_to_bf16_torch(vals)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in vals], np.uint16)
    nan = np.isnan(vals)
    # PyTorch also returns 0x7FC0 for every NaN
    assert np.array_equal(got[~nan], want[~nan])
    assert (got[nan] == 0x7FC0).all()


def test_bf16_widen_is_exact():
    for h in [0x0000, 0x8000, 0x0001, 0x3F80, 0xC0A0, 0x7F80, 0x7F7F]:
        want = np.array([h << 16], np.uint32).view(np.float32)[0]
        assert np.array_equal(np.float32(oracle.bf16_to_f32(h)), want)


# --------------------------------------------------------------------------
# hand-worked fixtures
# --------------------------------------------------------------------------

def test_golden_small_all_ops():
    g = json.load(open(os.path.join(GOLDEN, "prepare_dispatch_combine_small.json")))
    idx = np.array(g["topk_idx"], np.int64)
    p = oracle.prepare(idx, g["E"], g["A"], g["cap"])
    assert p.counts.tolist() == g["counts"]
    assert p.offsets.tolist() == g["offsets"]
    assert p.slot.tolist() == g["slot"]
    assert p.row_src[:p.live].tolist() == g["row_src"]
    assert p.status == g["status"]
    x = _hex(g["x"])
    w = np.array(g["topk_weights"], np.float32)
    canary = np.full((g["cap"], g["H"]), 0xABCD, np.uint16)
    recv, recv_w = oracle.dispatch(p, x, w, recv_init=canary,
                                   recv_w_init=np.full(g["cap"], -9.0, np.float32))
    live = p.live
    assert np.array_equal(recv[:live], _hex(g["recv"]))
    assert (recv[live:] == 0xABCD).all()
    assert recv_w[:live].tolist() == g["recv_w"]
    assert (recv_w[live:] == -9.0).all()
    out = oracle.combine(p, recv)
    assert np.array_equal(out, _hex(g["combine_identity"]))
    gb = oracle.combine_bwd(p, x, init=canary)
    assert np.array_equal(gb[:live], _hex(g["recv"]))
    _, gw = oracle.dispatch_bwd(p, recv, np.array(g["g_recv_w"], np.float32))
    assert gw.tolist() == g["grad_topk_weights"]
    _, gw0 = oracle.dispatch_bwd(p, recv, None)
    assert (gw0 == 0).all() and not np.signbit(gw0).any()


def test_golden_prepare_edge_cases():
    g = json.load(open(os.path.join(GOLDEN, "prepare_edge_cases.json")))
    for c in g["cases"]:
        idx = np.array(c["topk_idx"], np.int64).reshape(c["T"], c["K"])
        p = oracle.prepare(idx, c["E"], c["A"], c["cap"])
        assert p.counts.tolist() == c["counts"], c["name"]
        assert p.offsets.tolist() == c["offsets"], c["name"]
        assert p.slot.tolist() == c["slot"], c["name"]
        assert p.row_src[:p.live].tolist() == c["row_src"], c["name"]
        assert p.status == c["status"], c["name"]


def test_golden_combine_rounding():
    g = json.load(open(os.path.join(GOLDEN, "combine_rounding.json")))
    for c in g["cases"]:
        idx = np.array(c["topk_idx"], np.int64)
        p = oracle.prepare(idx, c["E"], c["A"], 64)
        rows = _hex(c["rows"])
        assert np.array_equal(oracle.combine(p, rows), _hex(c["combine"])), c["name"]
        gt, _ = oracle.dispatch_bwd(p, rows, None, want_grad_w=False)
        assert np.array_equal(gt, _hex(c["combine"])), c["name"]


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------

def _random_case(rng):
    T = int(rng.integers(0, 12))
    K = int(rng.integers(1, 5))
    E = int(rng.integers(1, 7))
    A = int(rng.choice([1, 2, 3, 4, 8]))
    H = int(rng.choice([1, 2, 3, 8]))
    kind = rng.integers(0, 4)
    if kind == 0:      # ids with duplicates and masks
        idx = rng.integers(-1, E, size=(T, K))
    elif kind == 1:    # all masked
        idx = np.full((T, K), -1)
    elif kind == 2:    # includes bad ids
        idx = rng.integers(-3, E + 3, size=(T, K))
    else:              # distinct where possible
        idx = np.stack([rng.permutation(max(E, K))[:K] for _ in range(T)]) if T else \
            np.zeros((0, K))
        idx = np.where(idx < E, idx, -1)
    worst = T * min(K, E) + E * (A - 1)
    cap = int(rng.choice([worst, worst + 3, max(0, worst // 2), 0]))
    return np.asarray(idx, np.int64).reshape(T, K), E, A, H, cap


def test_prepare_matches_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(1500):
        idx, E, A, H, cap = _random_case(rng)
        p = oracle.prepare(idx, E, A, cap)
        b = brute.prepare(idx, E, A, cap)
        assert p.counts.tolist() == b["counts"].tolist()
        assert p.offsets.tolist() == b["offsets"].tolist()
        assert p.slot.tolist() == b["slot"].tolist()
        assert p.row_src[:p.live].tolist() == b["row_src"].tolist()
        assert p.status == b["status"]
        assert not pins.check_prepare(idx, E, A, cap, p.counts, p.offsets, p.slot,
                                      p.row_src, p.status)


def test_payload_ops_match_brute_force():
    rng = np.random.default_rng(12)
    for _ in range(600):
        idx, E, A, H, cap = _random_case(rng)
        T, K = idx.shape
        p = oracle.prepare(idx, E, A, cap)
        b = brute.prepare(idx, E, A, cap)
        x = workloads.randn_bf16(rng, (T, H))
        w = rng.standard_normal((T, K)).astype(np.float32)
        recv, recv_w = oracle.dispatch(p, x, w)
        brecv, brecv_w = brute.dispatch(b, x, w, K, cap)
        assert np.array_equal(recv, brecv)
        assert np.array_equal(recv_w, brecv_w)
        rows = workloads.randn_bf16(rng, (max(cap, 1), H))
        assert np.array_equal(oracle.combine(p, rows), brute.combine(b, rows, T, K))
        g_w = rng.standard_normal(max(cap, 1)).astype(np.float32)
        gt, gw = oracle.dispatch_bwd(p, rows, g_w)
        assert np.array_equal(gt, brute.combine(b, rows, T, K))
        assert np.array_equal(gw, brute.dispatch_bwd_weights(b, g_w, T, K))
        g_res = workloads.randn_bf16(rng, (T, H))
        assert np.array_equal(oracle.combine_bwd(p, g_res), brute.dispatch(b, g_res, None, K,
                                                                           cap)[0])


def test_combine_special_values_match_brute_force():
    # Rows with +-0, +-inf, NaN, subnormals and extremes: brute force adds with
    # NumPy float32 and rounds with PyTorch, the oracle with its own C code.
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8001,
                         0x007F, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80, 0x0080], np.uint16)
    rng = np.random.default_rng(3)
    T, K, E, H = 64, 4, 4, 16
    idx = rng.integers(-1, E, size=(T, K))
    cap = T * K + E * 3
    p = oracle.prepare(idx, E, 4, cap)
    b = brute.prepare(idx, E, 4, cap)
    rows = rng.choice(specials, size=(cap, H))
    got = oracle.combine(p, rows)
    want = brute.combine(b, rows, T, K)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# invariants on the real routing generators
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_prepare_invariants_on_workloads(name):
    cfg = workloads.CONFIGS[name]
    r = workloads.make_routing(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    assert p.status == 0
    assert not pins.check_prepare(r.topk_idx, cfg.E, cfg.A, cap, p.counts, p.offsets,
                                  p.slot, p.row_src, p.status)
    assert not pins.check_pads_at_segment_end(p.offsets, p.counts, p.row_src, cap)
    valid = (r.topk_idx >= 0).sum()
    assert p.counts.sum() == valid
    if cfg.hot_fraction is not None:
        assert 0.45 < r.hot_share < 0.55   # one local expert holds about half the routes


def test_masked_slice_as_subset_of_global_experts():
    # The local slice [0,32) of 256 experts: prepare with E=32 and with E=256
    # places the same rows; the 224 extra experts have empty segments.
    cfg = workloads.scaled(workloads.CONFIGS["masked"], T=2048)
    r = workloads.make_routing(cfg)
    cap32 = oracle.recv_capacity_worst(cfg.T, cfg.K, 32, cfg.A)
    p32 = oracle.prepare(r.topk_idx, 32, cfg.A, cap32)
    p256 = oracle.prepare(r.topk_idx, 256, cfg.A, cap32 + 224 * 127)
    assert np.array_equal(p32.slot, p256.slot)
    assert (p256.counts[32:] == 0).all()
    assert (np.diff(p256.offsets[32:]) == 0).all()


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def _f32_of(bits):
    return brute.bf16_to_f32_np(bits)


def test_identity_experts_round_trip_is_n_valid_times_x():
    cfg = workloads.CONFIGS["tiny"]
    r = workloads.make_routing(cfg)
    x = workloads.make_tokens(cfg)
    idx = r.topk_idx.copy()
    idx[::7, 1] = -1           # some tokens lose a route
    idx[::13, :] = -1          # some lose all
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(idx, cfg.E, cfg.A, cap)
    recv, _ = oracle.dispatch(p, x, r.topk_weights)
    out = oracle.combine(p, recv)
    n = (idx >= 0).sum(axis=1).astype(np.float32)
    want = brute.f32_to_bf16_torch(_f32_of(x) * n[:, None])
    want[n == 0] = 0
    assert np.array_equal(out, want)


def test_power_of_two_expert_scales_closed_form():
    cfg = workloads.scaled(workloads.CONFIGS["mixtral"], T=512, H=256)
    r = workloads.make_routing(cfg)
    x = workloads.make_tokens(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    recv, _ = oracle.dispatch(p, x, r.topk_weights)
    scale = np.zeros(cap, np.float32)
    for e in range(cfg.E):
        scale[p.offsets[e]:p.offsets[e + 1]] = 2.0 ** (e - 3)
    expert_out = brute.f32_to_bf16_torch(_f32_of(recv) * scale[:, None])  # exact
    out = oracle.combine(p, expert_out)
    c = (2.0 ** (r.topk_idx.astype(np.float64) - 3)).sum(axis=1).astype(np.float32)
    want = brute.f32_to_bf16_torch(_f32_of(x) * c[:, None])
    assert np.array_equal(out, want)


def test_weights_summing_to_one_return_x_within_bound():
    # expert_out = bf16(recv * w) (one rounding, <= 2^-8 relative), an fp32 sum
    # of K terms and a final rounding (<= 2^-8): |out - x| <= (2^-7 + 2^-15)|x|
    # covers both roundings, their product and the fp32 slack of sum(w) and of
    # the K-term sum for K <= 8.
    cfg = workloads.scaled(workloads.CONFIGS["qwen3"], T=256, H=128)
    r = workloads.make_routing(cfg)
    x = workloads.make_tokens(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    recv, recv_w = oracle.dispatch(p, x, r.topk_weights)
    expert_out = brute.f32_to_bf16_torch(_f32_of(recv) * recv_w[:, None])
    out = _f32_of(oracle.combine(p, expert_out)).astype(np.float64)
    xf = _f32_of(x).astype(np.float64)
    assert (np.abs(out - xf) <= (2.0 ** -7 + 2.0 ** -15) * np.abs(xf)).all()


# --------------------------------------------------------------------------
# adjoints and masking
# --------------------------------------------------------------------------

def test_adjoint_identities_exact():
    # Small-integer bf16 values keep every fp32 sum exact, so the inner
    # products below are equal exactly (evaluated in fp64).
    cfg = workloads.scaled(workloads.CONFIGS["qwen3"], T=300, H=24)
    r = workloads.make_routing(cfg)
    idx = r.topk_idx.copy()
    idx[::5, 3] = -1
    rng = np.random.default_rng(9)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(idx, cfg.E, cfg.A, cap)
    x = workloads.small_int_bf16(rng, (cfg.T, cfg.H))
    w = rng.integers(-8, 9, size=(cfg.T, cfg.K)).astype(np.float32)
    G = workloads.small_int_bf16(rng, (cap, cfg.H))
    Gw = rng.integers(-8, 9, size=cap).astype(np.float32)
    recv, recv_w = oracle.dispatch(p, x, w)
    gt, gw = oracle.dispatch_bwd(p, G, Gw)
    lhs = pins.dot_f64(_f32_of(recv), _f32_of(G)) + pins.dot_f64(recv_w, Gw)
    rhs = pins.dot_f64(_f32_of(x), _f32_of(gt)) + pins.dot_f64(w, gw)
    assert lhs == rhs
    # combine and combine_bwd
    Y = workloads.small_int_bf16(rng, (cap, cfg.H))
    g = workloads.small_int_bf16(rng, (cfg.T, cfg.H))
    lhs = pins.dot_f64(_f32_of(oracle.combine(p, Y)), _f32_of(g))
    gy = oracle.combine_bwd(p, g)
    rhs = pins.dot_f64(_f32_of(Y[:p.live]), _f32_of(gy[:p.live]))
    assert lhs == rhs


def test_masked_routes_contribute_nothing():
    cfg = workloads.scaled(workloads.CONFIGS["masked"], T=1024, H=64)
    r = workloads.make_routing(cfg)
    rng = np.random.default_rng(4)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    x = workloads.make_tokens(cfg)
    w = r.topk_weights
    recv, recv_w = oracle.dispatch(p, x, w)
    dead = ~(r.topk_idx >= 0).any(axis=1)
    assert dead.any()
    x2 = x.copy()
    x2[dead] = workloads.randn_bf16(rng, (int(dead.sum()), cfg.H))
    w2 = w.copy()
    w2[r.topk_idx < 0] = 123.0
    recv2, recv_w2 = oracle.dispatch(p, x2, w2)
    assert np.array_equal(recv, recv2) and np.array_equal(recv_w, recv_w2)
    Y = workloads.randn_bf16(rng, (cap, cfg.H))
    assert (oracle.combine(p, Y)[dead] == 0).all()
    gt, gw = oracle.dispatch_bwd(p, Y, rng.standard_normal(cap).astype(np.float32))
    assert (gt[dead] == 0).all()
    assert (gw[r.topk_idx < 0] == 0).all()


# --------------------------------------------------------------------------
# planted mistakes are caught
# --------------------------------------------------------------------------

def test_checkers_catch_planted_mistakes():
    cfg = workloads.CONFIGS["tiny"]
    r = workloads.make_routing(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    args = (r.topk_idx, cfg.E, cfg.A, cap)
    ok = (p.counts, p.offsets, p.slot, p.row_src, p.status)
    assert not pins.check_prepare(*args, *ok)

    # 1. two routes of one expert swap rows (unstable order)
    slot = p.slot.copy()
    e0 = np.nonzero(r.topk_idx.reshape(-1) == 0)[0]
    slot[e0[0]], slot[e0[1]] = slot[e0[1]], slot[e0[0]]
    assert pins.check_prepare(*args, p.counts, p.offsets, slot, p.row_src, p.status)
    # 2. pads placed at the segment start
    rs = p.row_src.copy()
    lo, n = p.offsets[0], p.counts[0]
    pad = p.offsets[1] - lo - n
    if pad:
        rs[lo:lo + p.offsets[1] - lo] = np.concatenate([np.full(pad, -1), p.row_src[lo:lo + n]])
        assert pins.check_pads_at_segment_end(p.offsets, p.counts, rs, cap)
    # 3. offsets without the alignment
    off = np.concatenate([[0], np.cumsum(p.counts)]).astype(np.int32)
    assert pins.check_prepare(*args, p.counts, off, p.slot, p.row_src, p.status)
    # 4. an off-by-one count
    c = p.counts.copy()
    c[3] += 1
    assert pins.check_prepare(*args, c, p.offsets, p.slot, p.row_src, p.status)
    # 5. a missed status bit
    assert pins.check_prepare(*args, p.counts, p.offsets, p.slot, p.row_src, 2)


def test_reversed_accumulation_order_is_caught():
    # The k-order fixture distinguishes ascending from descending summation.
    g = json.load(open(os.path.join(GOLDEN, "combine_rounding.json")))
    c = g["cases"][0]
    rows = _f32_of(_hex(c["rows"])).reshape(-1)
    fwd = np.float32(np.float32(rows[0] + rows[1]) + rows[2])
    rev = np.float32(np.float32(rows[2] + rows[1]) + rows[0])
    assert brute.f32_to_bf16_torch(np.array([fwd]))[0] == int(c["combine"][0][0], 16)
    assert brute.f32_to_bf16_torch(np.array([rev]))[0] != int(c["combine"][0][0], 16)


# --------------------------------------------------------------------------
# weighted combine and its backward
# --------------------------------------------------------------------------

def _wbits(a):
    return np.array([int(v, 16) for v in a], np.uint32).view(np.float32)


def test_golden_combine_weighted():
    g = json.load(open(os.path.join(GOLDEN, "combine_weighted.json")))
    for c in g["forward_cases"]:
        p = oracle.prepare(np.array(c["topk_idx"], np.int64), c["E"], c["A"], 16)
        w = np.zeros(16, np.float32)
        w[:len(c["w_bits"])] = _wbits(c["w_bits"])
        rows = np.zeros((16, c["H"]), np.uint16)
        rows[:len(c["rows"])] = _hex(c["rows"])
        assert np.array_equal(oracle.combine_weighted(p, rows, w), _hex(c["combine_weighted"])), \
            c["name"]
    for c in g["backward_cases"]:
        p = oracle.prepare(np.array(c["topk_idx"], np.int64), c["E"], c["A"], 16)
        w = np.zeros(16, np.float32)
        w[:len(c["w_bits"])] = _wbits(c["w_bits"])
        gr, _, _ = oracle.combine_weighted_bwd(p, _hex(c["g"]), None, w)
        assert np.array_equal(gr[:p.live], _hex(c["grad_rows"])), c["name"]


def test_weighted_with_unit_and_power_of_two_weights():
    # w = 1: the weighted ops are the unweighted ones; w = 2^m: exact scaling,
    # so they equal the unweighted ops on exactly pre-scaled rows.
    cfg = workloads.scaled(workloads.CONFIGS["dsv3"], T=300, H=64)
    r = workloads.make_routing(cfg)
    idx = r.topk_idx.copy()
    idx[::9, 2] = -1
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(idx, cfg.E, cfg.A, cap)
    rng = np.random.default_rng(21)
    Y = workloads.randn_bf16(rng, (cap, cfg.H))
    g = workloads.randn_bf16(rng, (cfg.T, cfg.H))
    ones = np.ones(cap, np.float32)
    assert np.array_equal(oracle.combine_weighted(p, Y, ones), oracle.combine(p, Y))
    gr, _, _ = oracle.combine_weighted_bwd(p, g, None, ones)
    assert np.array_equal(gr[:p.live], oracle.combine_bwd(p, g)[:p.live])
    m = rng.integers(-3, 4, size=cap)
    w2 = (2.0 ** m).astype(np.float32)
    Ys = brute.f32_to_bf16_torch(brute.bf16_to_f32_np(Y) * w2[:, None])     # exact
    assert np.array_equal(oracle.combine_weighted(p, Y, w2), oracle.combine(p, Ys))
    gr2, _, _ = oracle.combine_weighted_bwd(p, g, None, w2)
    want = brute.f32_to_bf16_torch(brute.bf16_to_f32_np(oracle.combine_bwd(p, g)) *
                                   w2[:, None])
    live = p.live
    pad = p.row_src[:live] < 0
    assert np.array_equal(gr2[:live][~pad], want[:live][~pad])
    assert (gr2[:live][pad] == 0).all()


def test_weighted_adjoints_exact_small_ints():
    # For small-integer rows, gradients and weights every product and sum is
    # exact, so <combine_w(Y), g> = <Y, dY> = sum_r w_r dw_r exactly.
    cfg = workloads.scaled(workloads.CONFIGS["qwen3"], T=200, H=16)
    r = workloads.make_routing(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    rng = np.random.default_rng(8)
    Y = workloads.small_int_bf16(rng, (cap, cfg.H), 8)
    g = workloads.small_int_bf16(rng, (cfg.T, cfg.H), 8)
    w = rng.integers(-4, 5, size=cap).astype(np.float32)
    out = oracle.combine_weighted(p, Y, w)
    lhs = pins.dot_f64(_f32_of(out), _f32_of(g))
    gr, gw, _ = oracle.combine_weighted_bwd(p, g, Y, w)
    live = p.live
    assert lhs == pins.dot_f64(_f32_of(Y[:live]), _f32_of(gr[:live]))
    assert lhs == float(np.dot(w[:live].astype(np.float64), gw[:live]))
    # the weight gradient by an independent integer dot
    Yi = _f32_of(Y).astype(np.int64)
    gi = _f32_of(g).astype(np.int64)
    for rr in range(live):
        s = p.row_src[rr]
        want = 0 if s < 0 else int(np.dot(gi[s // cfg.K], Yi[rr]))
        assert gw[rr] == want


# --------------------------------------------------------------------------
# the tail policy and the capacity bound
# --------------------------------------------------------------------------

def test_zero_tail_makes_adjoints_hold_over_the_whole_buffer():
    # Combine never reads a row past the live total, so the gradient of such a
    # row is zero: with the tail policy, <combine(Y), g> = <Y, combine_bwd(g)>
    # over every row of the [cap,H] buffer even when that buffer started as
    # garbage; without it the stale rows break the identity (the check has
    # teeth). The same holds for dispatch and for the weighted pair.
    cfg = workloads.scaled(workloads.CONFIGS["qwen3"], T=150, H=16)
    r = workloads.make_routing(cfg)
    idx = r.topk_idx.copy()
    idx[::4, 2] = -1
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(idx, cfg.E, cfg.A, cap)
    assert p.live < cap
    rng = np.random.default_rng(21)
    Y = workloads.small_int_bf16(rng, (cap, cfg.H), 8)
    g = workloads.small_int_bf16(rng, (cfg.T, cfg.H), 8)
    garbage = workloads.small_int_bf16(rng, (cap, cfg.H), 8)
    lhs = pins.dot_f64(_f32_of(oracle.combine(p, Y)), _f32_of(g))
    gy = oracle.combine_bwd(p, g, init=garbage, zero_tail=True)
    assert (gy[p.live:] == 0).all()
    assert pins.dot_f64(_f32_of(Y), _f32_of(gy)) == lhs
    stale = oracle.combine_bwd(p, g, init=garbage, zero_tail=False)
    assert pins.dot_f64(_f32_of(Y), _f32_of(stale)) != lhs
    # dispatch: <D x, G> over the whole buffer equals <x, D^T G>
    x = workloads.small_int_bf16(rng, (cfg.T, cfg.H), 8)
    w = rng.integers(-4, 5, size=(cfg.T, cfg.K)).astype(np.float32)
    G = workloads.small_int_bf16(rng, (cap, cfg.H), 8)
    Gw = rng.integers(-4, 5, size=cap).astype(np.float32)
    recv, recv_w = oracle.dispatch(p, x, w, recv_init=garbage,
                                   recv_w_init=np.full(cap, 3.0, np.float32), zero_tail=True)
    assert (recv[p.live:] == 0).all() and (recv_w[p.live:] == 0).all()
    gt, gw = oracle.dispatch_bwd(p, G, Gw)
    assert (pins.dot_f64(_f32_of(recv), _f32_of(G)) + pins.dot_f64(recv_w, Gw) ==
            pins.dot_f64(_f32_of(x), _f32_of(gt)) + pins.dot_f64(w, gw))
    # weighted pair: <combine_w(Y), g> = <Y, dY> = <w, dw> over every row
    wr = rng.integers(-4, 5, size=cap).astype(np.float32)
    lhs_w = pins.dot_f64(_f32_of(oracle.combine_weighted(p, Y, wr)), _f32_of(g))
    gr, gw64, _ = oracle.combine_weighted_bwd(p, g, Y, wr, init=garbage, zero_tail=True)
    assert (gr[p.live:] == 0).all() and (gw64[p.live:] == 0).all()
    assert pins.dot_f64(_f32_of(Y), _f32_of(gr)) == lhs_w
    assert float(np.dot(wr.astype(np.float64), gw64)) == lhs_w


@pytest.mark.parametrize("T,K,E,A,want", [
    (4096, 8, 256, 128, 4096 * 8 + 256 * 127),
    (10, 8, 4, 1, 40),        # K > E: a token reaches at most E distinct experts
    (3, 5, 2, 3, 3 * 2 + 2 * 2),
    (7, 1, 1, 1, 7),          # A = 1: no pad row ever
    (0, 8, 32, 128, 32 * 127),
])
def test_capacity_bound_hand_values(T, K, E, A, want):
    assert oracle.recv_capacity_worst(T, K, E, A) == want


@pytest.mark.parametrize("T,K,E,A", [(4, 8, 4, 3), (7, 2, 5, 4), (5, 3, 3, 1), (1, 6, 6, 2)])
def test_capacity_bound_is_attained(T, K, E, A):
    # A routing that reaches the bound exactly: every token routes to min(K,E)
    # distinct experts (the rest masked), spread so that each expert's count
    # leaves it A-1 pad rows whenever T*min(K,E) allows. The bound is tight
    # from both sides: at the bound nothing overflows, and one row less
    # overflows whenever the routing fills it.
    m = min(K, E)
    idx = np.full((T, K), -1, np.int64)
    for t in range(T):
        for j in range(m):
            idx[t, j] = (t + j) % E
    cap = oracle.recv_capacity_worst(T, K, E, A)
    p = oracle.prepare(idx, E, A, cap)
    assert p.status == 0
    counts = np.bincount(idx[idx >= 0], minlength=E)
    total = int(((counts + A - 1) // A * A).sum())
    assert p.total == total <= cap
    if all(c % A == 1 % A for c in counts) and A > 1:
        assert total == cap
        assert oracle.prepare(idx, E, A, cap - 1).status & oracle.STATUS_OVERFLOW
