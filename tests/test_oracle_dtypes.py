"""Pins of the oracle's fp16 and fp32 payload paths and of the no-pad-fill
policy, against facts fixed outside the oracle:

- binary16 round-to-nearest-even at hand-derived bit patterns
  (tests/golden/payload_types.json), and NumPy's own binary32 <-> binary16
  conversions on every binary16 pattern and on random binary32 patterns;
- hand-worked combine cases (single rounding after an fp32 sum, subnormal and
  overflowing sums, ascending k in fp32, canonical NaN) and a weighted fp32
  case whose result differs between a fused and an unfused multiply-add;
- brute force (NumPy float32 column sums with NumPy's rounding) on random tiny
  cases with special values in every payload type;
- closed forms: identity experts give round(n_valid * x) in each type; exact
  small-integer adjoints of the weighted combine in fp16 and fp32;
- the no-pad-fill policy changes nothing but the pad rows, which keep their
  previous contents.
"""
import json
import os

import numpy as np
import pytest

import brute
import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FIXTURE = json.load(open(os.path.join(GOLDEN, "payload_types.json")))


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build()


def _f32(bits):
    return float(np.array([bits], np.uint32).view(np.float32)[0])


def _rows(hexrows, dtype):
    a = np.array([[int(v, 16) for v in row] for row in hexrows])
    if dtype == "fp32":
        return a.astype(np.uint32).view(np.float32)
    return a.astype(np.uint16)


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


# --------------------------------------------------------------------------
# binary16 conversions
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", FIXTURE["f32_to_f16"], ids=lambda c: c[0])
def test_f16_rne_hand_values(case):
    f_bits, want, _why = case
    assert oracle.f32_to_f16(_f32(int(f_bits, 16))) == int(want, 16)


def test_f16_widen_matches_numpy_on_every_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = brute.f16_to_f32_np(h)
    got = np.array([oracle.f16_to_f32(int(v)) for v in h], np.float32)
    nan = np.isnan(want)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()


def test_f16_rne_matches_numpy_on_random_patterns():
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    # concentrate a third of them on the binary16 range and its edges
    near = (rng.integers(0x33000000, 0x47800000, size=10000, dtype=np.uint64)
            .astype(np.uint32) | (rng.integers(0, 2, size=10000).astype(np.uint32) << 31))
    vals = np.concatenate([bits, near]).view(np.float32)
    want = brute.f32_to_f16_np(vals)
    got = np.array([oracle.f32_to_f16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)


def test_f16_round_trip_of_every_finite_pattern():
    # widening then rounding back returns the same binary16 pattern
    for h in range(0, 65536, 7):
        if (h & 0x7C00) == 0x7C00 and (h & 0x3FF):
            continue
        assert oracle.f32_to_f16(oracle.f16_to_f32(h)) == h


# --------------------------------------------------------------------------
# hand-worked cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("c", FIXTURE["combine_cases"], ids=lambda c: c["name"])
def test_golden_combine_payload_types(c):
    idx = np.array(c["topk_idx"], np.int64)
    dt = c["dtype"]
    p = oracle.prepare(idx, c["E"], c["A"], 16)
    rows = _rows(c["rows"], dt)
    pad = np.zeros((16 - rows.shape[0], c["H"]), rows.dtype)
    got = oracle.combine(p, np.concatenate([rows, pad]), dtype=dt)
    assert np.array_equal(_bits(got), _bits(_rows(c["combine"], dt))), c["derivation"]
    # dispatch_bwd's token part is the same sum
    gt, _ = oracle.dispatch_bwd(p, np.concatenate([rows, pad]), None, dtype=dt)
    assert np.array_equal(_bits(gt), _bits(got))


@pytest.mark.parametrize("c", FIXTURE["weighted_cases"], ids=lambda c: c["name"])
def test_golden_weighted_payload_types(c):
    idx = np.array(c["topk_idx"], np.int64)
    dt = c["dtype"]
    p = oracle.prepare(idx, c["E"], c["A"], 16)
    rows = np.zeros((16, c["H"]), np.float32 if dt == "fp32" else np.uint16)
    r = _rows(c["rows"], dt)
    rows[:r.shape[0]] = r
    w = np.zeros(16, np.float32)
    w[:len(c["w_bits"])] = np.array([int(v, 16) for v in c["w_bits"]],
                                    np.uint32).view(np.float32)
    got = oracle.combine_weighted(p, rows, w, dtype=dt)
    assert np.array_equal(_bits(got), _bits(_rows(c["combine_weighted"], dt))), c["derivation"]


def test_fused_case_differs_from_unfused():
    # the weighted fixture's two candidate answers, worked in NumPy float32
    c = FIXTURE["weighted_cases"][0]
    w = np.array([int(v, 16) for v in c["w_bits"]], np.uint32).view(np.float32)
    y = _rows(c["rows"], "fp32").reshape(-1)
    unfused = np.float32(w[0] * y[0]) + np.float32(w[1] * y[1])
    assert int(np.float32(unfused).view(np.uint32)) != int(c["combine_weighted"][0][0], 16)
    exact = float(w[0]) * float(y[0]) + float(w[1]) * float(y[1])   # exact in binary64
    assert np.float32(exact).view(np.uint32) == int(c["combine_weighted"][0][0], 16)


# --------------------------------------------------------------------------
# brute force with special values
# --------------------------------------------------------------------------

SPECIALS = {
    "fp16": np.array([0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E00, 0xFE01, 0x0001, 0x8001,
                      0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x3C00, 0xBC00, 0x3555, 0x6800],
                     np.uint16),
    "fp32": np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000,
                      0xFFA00001, 0x00000001, 0x80000001, 0x007FFFFF, 0x00800000,
                      0x7F7FFFFF, 0xFF7FFFFF, 0x3F800000, 0xBF800000, 0x33800000,
                      0x4B800000], np.uint32).view(np.float32),
}


def _random_payload(rng, dtype, shape):
    if dtype == "fp16":
        v = rng.standard_normal(shape).astype(np.float32) * 8
        out = v.astype(np.float16).view(np.uint16)
    else:
        out = rng.standard_normal(shape).astype(np.float32)
    mask = rng.random(shape) < 0.15
    out = out.copy()
    out[mask] = rng.choice(SPECIALS[dtype], size=int(mask.sum()))
    return out


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
def test_payload_types_match_brute_force(dtype):
    rng = np.random.default_rng(31 if dtype == "fp16" else 32)
    for _ in range(300):
        T = int(rng.integers(0, 10))
        K = int(rng.integers(1, 5))
        E = int(rng.integers(1, 6))
        A = int(rng.choice([1, 2, 4]))
        H = int(rng.choice([1, 3, 8]))
        idx = rng.integers(-1, E, size=(T, K)).astype(np.int64)
        cap = T * K + E * (A - 1)
        if rng.random() < 0.3:
            cap //= 2
        p = oracle.prepare(idx, E, A, cap)
        b = brute.prepare(idx, E, A, cap)
        x = _random_payload(rng, dtype, (T, H))
        w = rng.standard_normal((T, K)).astype(np.float32)
        recv, recv_w = oracle.dispatch(p, x, w, dtype=dtype)
        brecv, brecv_w = brute.dispatch(b, x, w, K, cap)
        assert np.array_equal(_bits(recv), _bits(brecv))
        assert np.array_equal(recv_w, brecv_w)
        rows = _random_payload(rng, dtype, (max(cap, 1), H))
        got = oracle.combine(p, rows, dtype=dtype)
        want = brute.combine(b, rows, T, K, dtype=dtype)
        assert np.array_equal(_bits(got), _bits(want))
        gt, _ = oracle.dispatch_bwd(p, rows, None, dtype=dtype)
        assert np.array_equal(_bits(gt), _bits(want))
        g = _random_payload(rng, dtype, (T, H))
        assert np.array_equal(_bits(oracle.combine_bwd(p, g, dtype=dtype)),
                              _bits(brute.dispatch(b, g, None, K, cap)[0]))


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
def test_identity_experts_give_n_valid_times_x(dtype):
    cfg = workloads.scaled(workloads.CONFIGS["qwen3"], T=300, H=32)
    r = workloads.make_routing(cfg)
    idx = r.topk_idx.copy()
    idx[::5, 1] = -1
    idx[::11, :] = -1
    rng = np.random.default_rng(40)
    widen, narrow = brute.CODECS[dtype]
    x = (narrow(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)) if dtype == "fp16"
         else rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(idx, cfg.E, cfg.A, cap)
    recv, _ = oracle.dispatch(p, x, None, dtype=dtype)
    out = oracle.combine(p, recv, dtype=dtype)
    n = (idx >= 0).sum(axis=1)
    # n * x for n <= 8 is at most 3 bits wider than x: exact in fp32 for fp16 x;
    # for fp32 x the ascending sum x + x + ... is the sequence of roundings of
    # 2x, 3x, ..., each exactly representable or rounded once, so compare with
    # the same ascending sum in NumPy float32.
    xf = widen(x)
    if dtype == "fp16":
        want = narrow(xf * n[:, None].astype(np.float32))
    else:
        acc = xf.copy()
        for m in range(2, 9):
            nxt = (acc + xf).astype(np.float32)
            acc = np.where((n >= m)[:, None], nxt, acc)
        want = narrow(acc)
    want[n == 0] = 0
    assert np.array_equal(_bits(out), _bits(want))


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
def test_weighted_adjoints_exact_small_ints(dtype):
    cfg = workloads.scaled(workloads.CONFIGS["dsv3"], T=150, H=16)
    r = workloads.make_routing(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    rng = np.random.default_rng(41)
    widen, narrow = brute.CODECS[dtype]
    Yi = rng.integers(-8, 9, size=(cap, cfg.H)).astype(np.float32)
    gi = rng.integers(-8, 9, size=(cfg.T, cfg.H)).astype(np.float32)
    Y, g = narrow(Yi), narrow(gi)
    w = rng.integers(-4, 5, size=cap).astype(np.float32)
    out = oracle.combine_weighted(p, Y, w, dtype=dtype)
    gr, gw, _ = oracle.combine_weighted_bwd(p, g, Y, w, dtype=dtype)
    live = p.live
    lhs = float(np.dot(widen(out).astype(np.float64).ravel(), gi.astype(np.float64).ravel()))
    assert lhs == float(np.dot(Yi[:live].astype(np.float64).ravel(),
                               widen(gr[:live]).astype(np.float64).ravel()))
    assert lhs == float(np.dot(w[:live].astype(np.float64), gw[:live]))
    for rr in range(live):
        s = p.row_src[rr]
        want = 0 if s < 0 else int(np.dot(gi[s // cfg.K].astype(np.int64),
                                          Yi[rr].astype(np.int64)))
        assert gw[rr] == want


# --------------------------------------------------------------------------
# no-pad-fill policy
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_no_pad_fill_changes_only_pad_rows(dtype):
    cfg = workloads.scaled(workloads.CONFIGS["dsv3"], T=200, H=24)
    r = workloads.make_routing(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    live = p.live
    pad = np.zeros(cap, bool)
    pad[:live] = p.row_src[:live] < 0
    assert pad.any()
    rng = np.random.default_rng(42)
    _, narrow = brute.CODECS[dtype]
    x = narrow(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
    g = narrow(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
    Y = narrow(rng.standard_normal((cap, cfg.H)).astype(np.float32))
    init = narrow(np.full((cap, cfg.H), 7.0, np.float32))
    init_w = np.full(cap, 7.0, np.float32)
    w = r.topk_weights
    rw = rng.standard_normal(cap).astype(np.float32)

    def check(fill, nofill):
        assert np.array_equal(_bits(nofill[~pad]), _bits(fill[~pad]))
        assert np.array_equal(_bits(nofill[pad]), _bits(init[pad] if nofill.ndim == 2
                                                        else init_w[pad]))
        assert (np.asarray(fill[pad]).astype(np.float64) == 0).all()

    a, aw = oracle.dispatch(p, x, w, recv_init=init, recv_w_init=init_w, dtype=dtype)
    b, bw = oracle.dispatch(p, x, w, recv_init=init, recv_w_init=init_w, dtype=dtype,
                            fill_pads=False)
    check(a, b)
    check(aw, bw)
    check(oracle.combine_bwd(p, g, init=init, dtype=dtype),
          oracle.combine_bwd(p, g, init=init, dtype=dtype, fill_pads=False))
    gr, gw, _ = oracle.combine_weighted_bwd(p, g, Y, rw, init=init, dtype=dtype)
    gr2, gw2, _ = oracle.combine_weighted_bwd(p, g, Y, rw, init=init, dtype=dtype,
                                              fill_pads=False)
    check(gr, gr2)
    assert np.array_equal(gw[~pad], gw2[~pad])


def test_thread_count_changes_no_bit():
    # the OpenMP build shares the row and token loops among threads; one
    # thread and every core must give the same bits for every op
    import zlib
    cfg = workloads.scaled(workloads.CONFIGS["qwen3"], T=700, H=256)
    r = workloads.make_routing(cfg)
    idx = r.topk_idx.copy()
    idx[::3, 1] = -1
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(idx, cfg.E, cfg.A, cap)
    rng = np.random.default_rng(zlib.crc32(b"threads"))
    x = workloads.randn_bf16(rng, (cfg.T, cfg.H))
    Y = workloads.randn_bf16(rng, (cap, cfg.H))
    g = workloads.randn_bf16(rng, (cfg.T, cfg.H))
    wr = rng.standard_normal(cap).astype(np.float32)
    Gw = rng.standard_normal(cap).astype(np.float32)

    def everything():
        recv, recv_w = oracle.dispatch(p, x, r.topk_weights, zero_tail=True)
        return [recv, recv_w.view(np.uint32), oracle.combine(p, Y),
                oracle.combine_bwd(p, g), *oracle.dispatch_bwd(p, Y, Gw),
                oracle.combine_weighted(p, Y, wr),
                *oracle.combine_weighted_bwd(p, g, Y, wr)[:2]]

    before = oracle.set_threads(0)
    try:
        assert oracle.set_threads(1) == 1
        one = everything()
        assert oracle.set_threads(max(2, os.cpu_count() or 2)) >= 2
        many = everything()
    finally:
        oracle.set_threads(before)
    for a, b in zip(one, many):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
