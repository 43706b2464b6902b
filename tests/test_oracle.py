"""CPU pins for the float64 oracle (no GPU).

Each test ties the oracle to something other than itself: the values printed
in the worked example of page "FlashAttention：为什么少搬数据，反而算得更快" §04,
closed forms, invariants, an independent brute-force spelling, and central
finite differences for the gradients.
"""

import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def hand_example_inputs():
    g = json.load(open(GOLDEN))
    e = np.array(g["exp_scores"], dtype=np.float64)
    # One query q = [1] and keys k_j = ln(e_j) give scores s_j = ln(e_j) at scale 1.
    q = np.array([[1.0]])
    k = np.log(e)[:, None]
    v = np.array(g["values"], dtype=np.float64)[:, None]
    return g, q, k, v


# ---------------------------------------------------------------- forward pins

def test_hand_example_one_block():
    g, q, k, v = hand_example_inputs()
    o, lse = oracle.head_forward(q, k, v, causal=False, scale=1.0)
    assert o[0, 0] == pytest.approx(g["output"], abs=1e-12)
    assert lse[0] == pytest.approx(math.log(10.0), abs=1e-12)
    # With one-hot values the output row is the weight row itself.
    o_w, _ = oracle.head_forward(q, k, np.eye(4), causal=False, scale=1.0)
    np.testing.assert_allclose(o_w[0], g["full_weights"], atol=1e-12)


def test_hand_example_two_blocks_state_by_state():
    g, q, k, v = hand_example_inputs()
    o, lse, trace = oracle.online_row(np.log(g["exp_scores"]), g["values"], block=g["block"])
    assert o == pytest.approx(g["output"], abs=1e-12)
    assert lse == pytest.approx(math.log(10.0), abs=1e-12)
    b1, b2 = g["blocks"]
    assert math.exp(trace[0]["m"]) == pytest.approx(b1["m_exp"], abs=1e-12)
    assert trace[0]["l"] == pytest.approx(b1["l"], abs=1e-12)
    assert trace[0]["U"] == pytest.approx(b1["U"], abs=1e-12)
    assert trace[1]["a"] == pytest.approx(b2["rescale"], abs=1e-12)
    assert trace[1]["l_rescaled"] == pytest.approx(b2["l_rescaled"], abs=1e-12)
    assert trace[1]["U_rescaled"] == pytest.approx(b2["U_rescaled"], abs=1e-12)
    assert math.exp(trace[1]["m"]) == pytest.approx(b2["m_exp"], abs=1e-12)
    assert trace[1]["l"] == pytest.approx(b2["l"], abs=1e-12)
    assert trace[1]["U"] == pytest.approx(b2["U"], abs=1e-12)
    assert trace[1]["U"] / trace[1]["l"] == pytest.approx(g["final"]["O"], abs=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nkv", [(9, 9), (5, 13), (13, 5), (1, 11)])
def test_rows_sum_to_one(causal, nq, nkv):
    q = rnd((nq, 4), 1)
    k = rnd((nkv, 4), 2)
    p, lse = oracle.head_forward(q, k, np.eye(nkv), causal, scale=0.7)
    vis = oracle.visible_mask(np.arange(nq), nq, nkv, causal)
    has = vis.any(axis=1)
    np.testing.assert_allclose(p[has].sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p >= 0)
    assert np.all(p[~vis] == 0)
    # Rows that see nothing: convention O = 0, LSE = -inf.
    assert np.all(p[~has] == 0) and np.all(np.isneginf(lse[~has]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 2, 3, 7, 64, 37])
def test_online_equals_full(causal, block):
    q, k, v = rnd((2, 4, 37, 8), 3), rnd((2, 2, 37, 8), 4), rnd((2, 2, 37, 8), 5)
    o, lse = oracle.attention_forward(q, k, v, causal, 0.3)
    o2, lse2 = oracle.online_forward(q, k, v, causal, 0.3, block)
    np.testing.assert_allclose(o2, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-12, rtol=0)


@settings(max_examples=40, deadline=None)
@given(nq=st.integers(1, 9), nkv=st.integers(1, 9), d=st.integers(1, 5),
       block=st.integers(1, 10), causal=st.booleans(), seed=st.integers(0, 10_000))
def test_online_equals_full_property(nq, nkv, d, block, causal, seed):
    q, k, v = rnd((1, 1, nq, d), seed), rnd((1, 1, nkv, d), seed + 1), rnd((1, 1, nkv, d), seed + 2)
    o, lse = oracle.attention_forward(q, k, v, causal, 1.3)
    o2, lse2 = oracle.online_forward(q, k, v, causal, 1.3, block)
    np.testing.assert_allclose(o2, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 5, 5, 3), (2, 4, 2, 3, 6, 4), (1, 3, 1, 6, 4, 2), (1, 2, 1, 1, 7, 3)])
def test_brute_force_matches(causal, shape):
    B, Hq, Hkv, nq, nkv, d = shape
    q, k, v = rnd((B, Hq, nq, d), 6), rnd((B, Hkv, nkv, d), 7), rnd((B, Hkv, nkv, d), 8)
    o, lse = oracle.attention_forward(q, k, v, causal, 0.45)
    ob, lb = oracle.brute_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.45)
    np.testing.assert_allclose(np.array(ob), o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.array(lb), lse, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_convexity(causal):
    q, k, v = rnd((11, 6), 9), rnd((11, 6), 10), rnd((11, 6), 11)
    o, _ = oracle.head_forward(q, k, v, causal, 1.0)
    for i in range(11):
        vis = v[: i + 1] if causal else v
        assert np.all(o[i] >= vis.min(axis=0) - 1e-12)
        assert np.all(o[i] <= vis.max(axis=0) + 1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nkv", [(8, 8), (3, 8), (8, 3)])
def test_uniform_attention_closed_form(causal, nq, nkv):
    # q = 0: every visible key has score 0, so O is the mean of the visible
    # value rows and LSE = ln(number visible).
    v = rnd((nkv, 5), 12)
    o, lse = oracle.head_forward(np.zeros((nq, 5)), rnd((nkv, 5), 13), v, causal, 0.9)
    for i in range(nq):
        last = min(nkv - 1, i + nkv - nq) if causal else nkv - 1
        if last < 0:
            assert np.all(o[i] == 0) and lse[i] == -np.inf
            continue
        np.testing.assert_allclose(o[i], v[: last + 1].mean(axis=0), atol=1e-12)
        assert lse[i] == pytest.approx(math.log(last + 1), abs=1e-12)


@pytest.mark.parametrize("scale", [1.0, 0.125, 2.5])
def test_single_key_closed_form(scale):
    q, k, v = rnd((6, 4), 14), rnd((1, 4), 15), rnd((1, 4), 16)
    o, lse = oracle.head_forward(q, k, v, False, scale)
    np.testing.assert_allclose(o, np.repeat(v, 6, axis=0), atol=1e-12)
    np.testing.assert_allclose(lse, scale * (q @ k[0]), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    q, k, v = rnd((7, 4), 17), rnd((9, 4), 18), rnd((9, 4), 19)
    c = rnd(4, 20)
    o, lse = oracle.head_forward(q, k, v, causal, 0.6)
    o2, lse2 = oracle.head_forward(q, k + c[None, :], v, causal, 0.6)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + 0.6 * (q @ c), atol=1e-12)


def test_permutation_invariance():
    q, k, v = rnd((5, 4), 21), rnd((12, 4), 22), rnd((12, 4), 23)
    perm = np.random.default_rng(24).permutation(12)
    o, lse = oracle.head_forward(q, k, v, False, 0.8)
    o2, lse2 = oracle.head_forward(q, k[perm], v[perm], False, 0.8)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


@pytest.mark.parametrize("nq,nkv", [(6, 6), (4, 9)])
def test_causal_row_is_prefix_attention(nq, nkv):
    q, k, v = rnd((nq, 3), 25), rnd((nkv, 3), 26), rnd((nkv, 3), 27)
    o, lse = oracle.head_forward(q, k, v, True, 1.1)
    for i in range(nq):
        last = i + nkv - nq
        oi, li = oracle.head_forward(q[i:i + 1], k[: last + 1], v[: last + 1], False, 1.1)
        np.testing.assert_allclose(o[i], oi[0], atol=1e-12)
        assert lse[i] == pytest.approx(li[0], abs=1e-12)
    if nq == nkv:
        np.testing.assert_allclose(o[0], v[0], atol=1e-12)


def test_sampled_rows_match_full():
    q, k, v = rnd((20, 4), 28), rnd((20, 4), 29), rnd((20, 4), 30)
    o, lse = oracle.head_forward(q, k, v, True, 0.5)
    rows = np.array([0, 7, 19])
    o2, lse2 = oracle.head_forward(q[rows], k, v, True, 0.5, row_index=rows, nq=20)
    np.testing.assert_allclose(o2, o[rows], atol=0)
    np.testing.assert_allclose(lse2, lse[rows], atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_mha(causal):
    q, k, v, do = rnd((2, 6, 5, 3), 31), rnd((2, 2, 7, 3), 32), rnd((2, 2, 7, 3), 33), rnd((2, 6, 5, 3), 34)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o, lse = oracle.attention_forward(q, k, v, causal, 0.5)
    o2, lse2 = oracle.attention_forward(q, kr, vr, causal, 0.5)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal, 0.5)
    dq2, dk2, dv2 = oracle.attention_backward(q, kr, vr, do, causal, 0.5)
    np.testing.assert_allclose(dq, dq2, atol=1e-12)
    np.testing.assert_allclose(dk, dk2.reshape(2, 2, 3, 7, 3).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(2, 2, 3, 7, 3).sum(axis=2), atol=1e-12)


# --------------------------------------------------------------- backward pins

def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.attention_forward(q, k, v, causal, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal,nq,nkv", [(False, 5, 7), (True, 5, 7), (True, 7, 4)])
def test_gradients_by_finite_differences(causal, nq, nkv):
    """Central differences of the forward's loss. The causal 7 x 4 case has
    query rows 0..2 that see no key: their O is the constant 0 of the no-key
    convention, so the differences give them zero gradient, and the
    backward must agree (dQ rows 0..2 are 0 and they add nothing to dK, dV)."""
    B, Hq, Hkv, d = 1, 2, 1, 3
    q, k, v, do = rnd((B, Hq, nq, d), 35), rnd((B, Hkv, nkv, d), 36), rnd((B, Hkv, nkv, d), 37), rnd((B, Hq, nq, d), 38)
    scale = 0.8
    grads = oracle.attention_backward(q, k, v, do, causal, scale)
    h = 1e-6
    for which, g in zip(range(3), grads):
        fd = np.zeros_like(g)
        base = [q, k, v]
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (_loss(*plus, do, causal, scale) - _loss(*minus, do, causal, scale)) / (2 * h)
        rel = np.linalg.norm(g - fd) / np.linalg.norm(fd)
        assert rel <= 1e-6, (which, rel)
        if which == 0 and causal and nq > nkv:
            assert np.all(g[:, :, : nq - nkv] == 0) and np.all(np.abs(fd[:, :, : nq - nkv]) < 1e-9)


@pytest.mark.parametrize("causal,nq,nkv", [(False, 6, 9), (True, 6, 9), (True, 9, 4), (True, 3, 0)])
def test_lse_is_scipy_logsumexp_of_the_visible_scores(causal, nq, nkv):
    """LSE_i is the log-sum-exp of row i's visible scaled scores, as
    scipy.special.logsumexp computes it (an independent routine); for a row
    that sees no key that is the log-sum-exp of an empty set, -inf."""
    from scipy.special import logsumexp

    q, k = rnd((nq, 5), 61), rnd((nkv, 5), 62)
    scale = 0.6
    _, lse = oracle.head_forward(q, k, rnd((nkv, 5), 63), causal, scale)
    vis = oracle.visible_mask(np.arange(nq), nq, nkv, causal)
    s = scale * (q @ k.T)
    for i in range(nq):
        want = logsumexp(s[i, vis[i]]) if vis[i].any() else logsumexp(np.array([]))
        if np.isneginf(want):
            assert np.isneginf(lse[i])
        else:
            assert lse[i] == pytest.approx(want, abs=1e-12)


def test_backward_hand_example_closed_form():
    # dO = 1 on the worked example: dV = P, dP_j = V_j, sum_k P_k dP_k = O = 29,
    # dS = P (V - 29) = [-1.9, -1.8, 0.4, 3.3]; dq = sum_j dS_j k_j; dk_j = dS_j q.
    g, q, k, v = hand_example_inputs()
    dq, dk, dv = oracle.head_backward(q, k, v, np.ones((1, 1)), causal=False, scale=1.0)
    np.testing.assert_allclose(dv[:, 0], g["full_weights"], atol=1e-12)
    ds = np.array([-1.9, -1.8, 0.4, 3.3])
    np.testing.assert_allclose(dk[:, 0], ds, atol=1e-12)
    expect_dq = float(np.sum(ds * np.log(g["exp_scores"])))
    assert dq[0, 0] == pytest.approx(expect_dq, abs=1e-12)
    assert dq[0, 0] == pytest.approx(2.93227337, abs=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    q, k, v, do = rnd((1, 4, 9, 5), 39), rnd((1, 2, 9, 5), 40), rnd((1, 2, 9, 5), 41), rnd((1, 4, 9, 5), 42)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal, 0.7)
    # Each softmax row's dS sums to zero, so the key gradients sum to zero.
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # Each P row sums to one, so summing dV over keys gives the sum of dO over
    # the queries (and heads) that read this kv head.
    np.testing.assert_allclose(dv.sum(axis=2), do.reshape(1, 2, 2, 9, 5).sum(axis=(2, 3)), atol=1e-12)


def test_backward_scale_dependence():
    # dQ and dK carry one factor of scale from S = scale * QK^T; with K = 0
    # all scores vanish, P is uniform, and dQ = scale * dS K = 0 exactly.
    q, v, do = rnd((4, 3), 43), rnd((6, 3), 44), rnd((4, 3), 45)
    dq, dk, dv = oracle.head_backward(q, np.zeros((6, 3)), v, do, False, 0.3)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, np.repeat(do.sum(axis=0, keepdims=True) / 6, 6, axis=0), atol=1e-12)


# ------------------------------------------------- planted mistakes are caught

def _catches(monkeypatch, patch_name, patched, tests):
    monkeypatch.setattr(ref, patch_name, patched)
    failures = 0
    for t in tests:
        try:
            t()
        except AssertionError:
            failures += 1
    return failures


def test_planted_causal_off_by_one_is_caught(monkeypatch):
    orig = ref.visible_mask

    def wrong(row_index, nq, nkv, causal):
        m = orig(row_index, nq, nkv, causal)
        if causal:
            rows = np.asarray(row_index)[:, None]
            m = np.arange(nkv)[None, :] < rows + (nkv - nq)
        return m

    n = _catches(monkeypatch, "visible_mask", wrong,
                 [lambda: test_uniform_attention_closed_form(True, 8, 8),
                  lambda: test_causal_row_is_prefix_attention(6, 6)])
    assert n >= 1


def test_planted_softmax_without_max_is_harmless_but_wrong_sum_is_caught(monkeypatch):
    def wrong(s):
        e = np.exp(s)
        return e / (np.sum(e, axis=1, keepdims=True) + 1.0), np.log(np.sum(e, axis=1))

    n = _catches(monkeypatch, "_softmax_rows", wrong,
                 [test_hand_example_one_block, lambda: test_rows_sum_to_one(False, 9, 9)])
    assert n >= 1


@pytest.mark.parametrize("page_size", [64, 128])
def test_paged_decode_equals_contiguous_decode(page_size):
    """Paged decode oracle against the definition on contiguous K/V: keys of
    each sequence scattered into a shuffled page pool must give the same
    O and LSE as the plain forward over that sequence's first len keys (the
    contiguous side slices the original arrays directly, not through the
    paging code)."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d = 3, 4, 2, 64
    lens = [1, 3 * page_size + 5, 2 * page_size]
    max_pages = 4
    n = max_pages * page_size
    k = rng.standard_normal((B, Hkv, n, d))
    v = rng.standard_normal((B, Hkv, n, d))
    q = rng.standard_normal((B, Hq, 1, d))
    num_pages = B * max_pages + 2
    order = rng.permutation(num_pages)
    table = order[: B * max_pages].reshape(B, max_pages)
    k_pages = rng.standard_normal((num_pages, Hkv, page_size, d))  # unused pages: noise
    v_pages = rng.standard_normal((num_pages, Hkv, page_size, d))
    for b in range(B):
        for p in range(max_pages):
            k_pages[table[b, p]] = k[b, :, p * page_size:(p + 1) * page_size]
            v_pages[table[b, p]] = v[b, :, p * page_size:(p + 1) * page_size]
    o, lse = oracle.paged_decode_forward(q, k_pages, v_pages, table, np.array(lens), 0.125)
    for b in range(B):
        ob, lb = oracle.attention_forward(q[b:b + 1], k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]],
                                          False, 0.125)
        np.testing.assert_allclose(o[b], ob[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], lb[0], rtol=0, atol=1e-12)


def test_paged_decode_out_of_range_entry_drops_its_keys():
    """A table entry outside [0, num_pages) names no page: the oracle's
    result is the definition over the sequence's keys with that page's keys
    removed (sliced out of the contiguous arrays directly)."""
    rng = np.random.default_rng(9)
    ps, max_pages, d = 64, 4, 32
    n = max_pages * ps
    k = rng.standard_normal((1, 2, n, d))
    v = rng.standard_normal((1, 2, n, d))
    q = rng.standard_normal((1, 4, 1, d))
    table = np.array([[2, 0, 3, 1]])
    k_pages = np.stack([k[0, :, table[0].tolist().index(p) * ps:][:, :ps] for p in range(4)])
    v_pages = np.stack([v[0, :, table[0].tolist().index(p) * ps:][:, :ps] for p in range(4)])
    for bad_entry in (7, -1):
        bad = table.copy()
        bad[0, 1] = bad_entry
        lens = np.array([3 * ps + 10])
        o, lse = oracle.paged_decode_forward(q, k_pages, v_pages, bad, lens, 0.2)
        keep = np.r_[0:ps, 2 * ps:3 * ps + 10]
        o_ref, l_ref = oracle.attention_forward(q, k[:, :, keep], v[:, :, keep], False, 0.2)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)
    bad = np.array([[9, 9, 9, 9]])
    o, lse = oracle.paged_decode_forward(q, k_pages, v_pages, bad, np.array([n]), 0.2)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_paged_decode_empty_sequence():
    """A sequence with no keys: O = 0, LSE = -inf (the no-key convention)."""
    rng = np.random.default_rng(8)
    k_pages = rng.standard_normal((2, 1, 64, 64))
    q = rng.standard_normal((1, 2, 1, 64))
    o, lse = oracle.paged_decode_forward(q, k_pages, k_pages, np.array([[1]]), np.array([0]), 0.1)
    assert (o == 0).all() and np.isneginf(lse).all()


# ------------------------------------------------------------------- dropout

from oracle import dropout as drop  # noqa: E402


def test_philox_matches_numpy_generator():
    """The oracle's Philox4x64-10 against numpy.random.Philox, an independent
    implementation of the same published generator. numpy advances its
    counter by one before producing the first 256-bit block."""
    rng = np.random.default_rng(11)
    counters = rng.integers(0, 2**63, size=(300, 4), dtype=np.uint64)
    keys = rng.integers(0, 2**64 - 1, size=(300, 2), dtype=np.uint64, endpoint=True)
    counters[:5] = 0
    keys[:5] = [[0, 0], [2**64 - 1, 2**64 - 1], [1, 0], [0, 1], [123456789, 987654321]]
    counters[5:10, 1:] = 2**64 - 1  # large words in every position but the incremented one
    for c, k in zip(counters, keys):
        expect = np.random.Philox(counter=c, key=k).random_raw(4)
        c1 = c.copy()
        c1[0] += np.uint64(1)
        got = drop.philox4x64(c1, k)
        assert np.array_equal(got, expect), (c, k)
    # Vectorised call over many counters equals the one-by-one results.
    c1 = counters.copy()
    c1[:, 0] += np.uint64(1)
    batch = drop.philox4x64(c1, keys)
    for i in range(0, 300, 37):
        assert np.array_equal(batch[i], np.random.Philox(counter=counters[i], key=keys[i]).random_raw(4))


def test_dropout_bytes_come_from_the_documented_counter():
    """Byte t of key group g of row i of head bh is byte t % 8 of word t // 8
    of philox((g, i, bh, offset), (seed, 0)) (checked on a few elements with
    direct generator calls)."""
    seed, offset, bh = 987, 4, 7
    u = drop.dropout_bytes(bh, np.arange(5), 100, seed, offset)
    for i, j in [(0, 0), (1, 31), (2, 32), (4, 99), (3, 70)]:
        w = drop.philox4x64(np.array([j // 32, i, bh, offset], dtype=np.uint64),
                            np.array([seed, 0], dtype=np.uint64))
        t = j % 32
        assert u[i, j] == (int(w[t // 8]) >> (8 * (t % 8))) & 0xFF


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_keep_rate(p):
    """Kept fraction within 5 standard deviations of 1 - theta / 256."""
    z = drop.keep_mask(3, np.arange(256), 512, p, seed=2024, offset=1)
    q = 1.0 - drop.threshold(p) / 256.0
    sd = math.sqrt(q * (1 - q) / z.size)
    assert abs(z.mean() - q) <= 5 * sd
    # No structure along rows or columns: per-column rates stay within 6 sd.
    col = z.mean(axis=0)
    assert np.max(np.abs(col - q)) <= 6 * math.sqrt(q * (1 - q) / z.shape[0])


def test_dropout_masks_differ_across_heads_seeds_offsets():
    base = drop.keep_mask(0, np.arange(64), 256, 0.5, 1, 0)
    for other in (drop.keep_mask(1, np.arange(64), 256, 0.5, 1, 0),
                  drop.keep_mask(0, np.arange(64), 256, 0.5, 2, 0),
                  drop.keep_mask(0, np.arange(64), 256, 0.5, 1, 1)):
        agree = np.mean(base == other)
        assert 0.45 < agree < 0.55  # independent masks agree about half the time


def test_dropout_threshold_and_scale():
    assert drop.threshold(0.0) == 0 and drop.keep_scale(0.0) == 1.0
    assert drop.threshold(0.25) == 64 and drop.keep_scale(0.25) == pytest.approx(256 / 192)
    assert drop.threshold(0.999) == 255
    with pytest.raises(ValueError):
        drop.threshold(1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_zero_probability_is_the_plain_definition(causal):
    q, k, v, do = rnd((2, 4, 7, 5), 60), rnd((2, 2, 9, 5), 61), rnd((2, 2, 9, 5), 62), rnd((2, 4, 7, 5), 63)
    o, lse = drop.attention_forward_dropout(q, k, v, causal, 0.6, 0.0, 5, 0)
    o_ref, lse_ref = oracle.attention_forward(q, k, v, causal, 0.6)
    np.testing.assert_allclose(o, o_ref, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-14)
    for g, g_ref in zip(drop.attention_backward_dropout(q, k, v, do, causal, 0.6, 0.0, 5, 0),
                        oracle.attention_backward(q, k, v, do, causal, 0.6)):
        np.testing.assert_allclose(g, g_ref, atol=1e-13)


def test_dropout_keeps_lse_and_scales_kept_terms():
    """LSE ignores the mask; with V = identity, row i of O is r P_i o Z_i."""
    q, k = rnd((6, 8), 64), rnd((8, 8), 65)
    z = drop.keep_mask(0, np.arange(6), 8, 0.3, 9, 0)
    r = drop.keep_scale(0.3)
    o, lse = drop.head_forward_dropout(q, k, np.eye(8), False, 0.5, z, r)
    o0, lse0 = oracle.head_forward(q, k, np.eye(8), False, 0.5)
    np.testing.assert_allclose(lse, lse0, atol=1e-14)
    np.testing.assert_allclose(o, r * o0 * z, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_gradients_by_finite_differences(causal):
    """With the mask fixed, O is a smooth function of q, k, v: central
    differences of sum(dO * O) match the analytic gradients."""
    rng = np.random.default_rng(66)
    nq, nkv, d = 5, 7, 3
    q, k, v, do = (rng.standard_normal(s) for s in [(nq, d), (nkv, d), (nkv, d), (nq, d)])
    z = rng.random((nq, nkv)) < 0.6
    r, scale = 1.7, 0.8
    grads = drop.head_backward_dropout(q, k, v, do, causal, scale, z, r)

    def loss(qq, kk, vv):
        return float(np.sum(do * drop.head_forward_dropout(qq, kk, vv, causal, scale, z, r)[0]))

    h = 1e-6
    for which, g in enumerate(grads):
        base = [q, k, v]
        fd = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.linalg.norm(g - fd) / np.linalg.norm(fd) <= 1e-6, which


def test_dropout_row_term_identity():
    """rowsum(P o dP) = rowsum(dO o O) still holds with dropout (what lets the
    backward use D = rowsum(dO o O))."""
    rng = np.random.default_rng(67)
    q, k, v, do = (rng.standard_normal(s) for s in [(6, 4), (9, 4), (9, 4), (6, 4)])
    z = rng.random((6, 9)) < 0.5
    r = 2.0
    o, _ = drop.head_forward_dropout(q, k, v, False, 0.9, z, r)
    s = 0.9 * (q @ k.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = r * z * (do @ v.T)
    np.testing.assert_allclose(np.sum(p * dp, axis=1), np.sum(do * o, axis=1), atol=1e-12)


# ---------------------------------------------------------------------- fp8

from oracle import fp8 as f8  # noqa: E402
import torch  # noqa: E402


def test_e4m3_table_matches_torch_float8():
    """The oracle's E4M3 decode (written from the format definition) against
    torch's float8_e4m3fn conversion, an independent implementation."""
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(f8.E4M3_TABLE))
    assert np.array_equal(t[~nan], f8.E4M3_TABLE[~nan])
    assert f8.e4m3_value(0x38) == 1.0 and f8.e4m3_value(0x7E) == 448.0
    assert f8.e4m3_value(0x01) == 2.0 ** -9 and f8.e4m3_value(0x08) == 2.0 ** -6
    assert np.isnan(f8.e4m3_value(0x7F)) and np.isnan(f8.e4m3_value(0xFF))


def test_fp8_forward_is_the_definition_on_decoded_inputs():
    rng = np.random.default_rng(90)
    q8, k8, v8 = (rng.integers(0, 256, size=s, dtype=np.uint8) for s in [(9, 16), (12, 16), (12, 16)])
    for a in (q8, k8, v8):
        a[(a & 0x7F) == 0x7F] = 0x30  # no NaN codes
    o, lse = f8.head_forward_fp8(q8, k8, v8, True, 0.25, 0.5, 0.125, 2.0)
    o_ref, lse_ref = oracle.head_forward(f8.decode(q8) * 0.5, f8.decode(k8) * 0.125,
                                         f8.decode(v8) * 2.0, True, 0.25)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_p_rounding_bound_holds_for_rounded_p(causal):
    """Rounding P (relative to the row maximum) to E4M3 with an independent
    rounder (torch) moves O by no more than p_rounding_bound."""
    rng = np.random.default_rng(91)
    nq, nkv, d = 40, 300, 32
    vals = torch.from_numpy(rng.standard_normal((nq + 2 * nkv, d))).to(torch.float8_e4m3fn)
    codes = vals.view(torch.uint8).numpy()
    q8, k8, v8 = codes[:nq], codes[nq:nq + nkv], codes[nq + nkv:]
    scale, dq, dk, dv = 0.3, 1.0, 1.0, 1.0
    q, k, v = f8.decode(q8), f8.decode(k8), f8.decode(v8)
    s = scale * (q @ k.T)
    vis = oracle.visible_mask(np.arange(nq), nq, nkv, causal)
    s = np.where(vis, s, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))          # values relative to the row max
    e8 = torch.from_numpy(e).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    o_rounded = (e8 @ v) / e.sum(axis=1, keepdims=True)
    o_exact, _ = f8.head_forward_fp8(q8, k8, v8, causal, scale, dq, dk, dv)
    bound = f8.p_rounding_bound(q8, k8, v8, causal, scale, dq, dk, dv)
    assert np.all(np.abs(o_rounded - o_exact) <= bound + 1e-12)
    assert np.max(np.abs(o_rounded - o_exact)) > 0  # the rounding is visible


# ------------------------------------------------- gradient error magnitudes

from oracle import bounds as gb  # noqa: E402


def test_gradient_magnitudes_hand_example_closed_form():
    """dO = 1 on the worked example of [KB] §04: P = [.1, .2, .4, .3],
    dP_j = V_j, O = D = 29 = Dabs, so A_j = P_j (V_j + 29) = [3.9, 9.8, 23.6,
    20.7]; Mk_j = A_j |q|, Mq = sum_j A_j |k_j|, Mv_j = P_j."""
    g, q, k, v = hand_example_inputs()
    mq, mk, mv, cq, ck, cv, rq, rk, rv, lq = gb.head_backward_magnitudes(q, k, v, np.ones((1, 1)),
                                                                         False, 1.0)
    a = np.array([3.9, 9.8, 23.6, 20.7])
    np.testing.assert_allclose(mk[:, 0], a, atol=1e-12)
    assert mq[0, 0] == pytest.approx(9.8 * math.log(2) + 23.6 * math.log(4) + 20.7 * math.log(3), abs=1e-12)
    np.testing.assert_allclose(mv[:, 0], g["full_weights"], atol=1e-12)
    w = np.array([10.0, 20.0, 30.0, 40.0]) + 29 + 1     # |dP_j| + Dabs + 1
    assert cq[0, 0] == pytest.approx(float(np.sum(w * np.abs(np.log(g["exp_scores"])))), abs=1e-12)
    np.testing.assert_allclose(ck[:, 0], w, atol=1e-12)
    np.testing.assert_allclose(cv[:, 0], 1.0)
    # One term per dK / dV element: root-sum-square = magnitude sum.
    np.testing.assert_allclose(rk, mk, atol=1e-12)
    np.testing.assert_allclose(rv, mv, atol=1e-12)
    rq_want = math.sqrt(sum((aj * math.log(ej)) ** 2 for aj, ej in zip(a, g["exp_scores"])))
    assert rq[0, 0] == pytest.approx(rq_want, abs=1e-12)
    # Common-mode D term of dQ: Dabs * sum_j P_j |k_j| = 29 * (.2 ln2 + .4 ln4 + .3 ln3).
    assert lq[0, 0] == pytest.approx(29 * (0.2 * math.log(2) + 0.4 * math.log(4) + 0.3 * math.log(3)),
                                     abs=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_magnitudes_dominate_gradients(causal):
    """Triangle inequality: |dV| <= Mv, |dK| <= Mk, |dQ| <= Mq element by
    element; with dO >= 0 the dV sum has no cancellation and Mv == dV."""
    q, k, v, do = rnd((13, 6), 60), rnd((17, 6), 61), rnd((17, 6), 62), rnd((13, 6), 63)
    dq, dk, dv = oracle.head_backward(q, k, v, do, causal, 0.6)
    mq, mk, mv, _, _, _, rq, rk, rv, _ = gb.head_backward_magnitudes(q, k, v, do, causal, 0.6)
    # sqrt(sum x^2) <= sum |x| <= sqrt(n) sqrt(sum x^2)
    for m, rr, n in ((mq, rq, 17), (mk, rk, 13), (mv, rv, 13)):
        assert np.all(rr <= m + 1e-12) and np.all(m <= np.sqrt(n) * rr + 1e-12)
    assert np.all(np.abs(dq) <= mq + 1e-12)
    assert np.all(np.abs(dk) <= mk + 1e-12)
    assert np.all(np.abs(dv) <= mv + 1e-12)
    _, _, dv_pos = oracle.head_backward(q, k, v, np.abs(do), causal, 0.6)
    mv_pos = gb.head_backward_magnitudes(q, k, v, np.abs(do), causal, 0.6)[2]
    np.testing.assert_allclose(mv_pos, dv_pos, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dtype,u", [(torch.bfloat16, 2.0 ** -8), (torch.float16, 2.0 ** -11)])
def test_gradient_bound_holds_for_rounded_p_and_ds(dtype, u):
    """A backward that rounds P (for dV), dS (for dK, dQ) and the output O
    (for D) to a 16-bit format with an independent rounder (torch) stays
    within u Mv, 2u Mk, 2u Mq of the exact gradients (+ the subnormal term for
    fp16), and the bound is not vacuous."""
    rng = np.random.default_rng(64)
    nq, nkv, d, scale = 48, 80, 16, 0.25
    q, k, v, do = (rng.standard_normal(s) for s in [(nq, d), (nkv, d), (nkv, d), (nq, d)])
    rd = lambda x: torch.from_numpy(x).to(dtype).to(torch.float64).numpy()  # noqa: E731
    s = np.where(oracle.visible_mask(np.arange(nq), nq, nkv, True), scale * (q @ k.T), -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o16 = rd(p @ v)
    dp = do @ v.T
    ds16 = rd(p * (dp - np.sum(do * o16, axis=1, keepdims=True)))
    got = (scale * (ds16 @ k), scale * (ds16.T @ q), rd(p).T @ do)
    ref = oracle.head_backward(q, k, v, do, True, scale)
    mq, mk, mv, cq, ck, cv, rq, rk, rv, lq = gb.head_backward_magnitudes(q, k, v, do, True, scale)
    sub = 2.0 ** -25 if dtype == torch.float16 else 0.0
    worst = 0.0
    rows = lambda x: np.linalg.norm(x, axis=1)  # noqa: E731
    for g, r, m, c, rr, lin, f in zip(got, ref, (mq, mk, mv), (cq, ck, cv), (rq, rk, rv),
                                      (lq, 0 * mk, 0 * mv), (2, 2, 1)):
        bound = f * u * m + sub * c
        assert np.all(np.abs(g - r) <= bound + 1e-15)
        worst = max(worst, float(np.max(np.abs(g - r) / (bound + 1e-300))))
        # Rows: independent roundings add up like a random walk (about
        # u R / sqrt(3) per element); 6 u R bounds them with room to spare.
        allow = 6 * u * rows(rr) + u * rows(lin) + sub * rows(c + 1)
        assert np.all(rows(g - r) <= allow + 1e-15)
        assert np.max(rows(g - r) / (allow + 1e-300)) < 0.5
    assert worst > 0.01


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_accumulation_bound_holds_for_perturbed_scores(causal):
    """accumulation_bound: moving every score by up to E_ij = eps8 scale
    sum_c |q_ic k_jc| (random and sign-aligned worst-case moves) and every
    P V term by up to eps8 of itself keeps O and LSE within the bound; the
    bound is not vacuous (a sign-aligned move uses a visible part of it)."""
    rng = np.random.default_rng(92)
    nq, nkv, d, scale, eps = 24, 90, 32, 0.4, 2.0 ** -6  # a large eps8 makes the effect visible
    vals = torch.from_numpy(rng.standard_normal((nq + 2 * nkv, d)) * 2).to(torch.float8_e4m3fn)
    codes = vals.view(torch.uint8).numpy()
    q8, k8, v8 = codes[:nq], codes[nq:nq + nkv], codes[nq + nkv:]
    q, k, v = f8.decode(q8), f8.decode(k8), f8.decode(v8)
    o_ref, lse_ref = f8.head_forward_fp8(q8, k8, v8, causal, scale, 1.0, 1.0, 1.0)
    o_b, lse_b = f8.accumulation_bound(q8, k8, v8, causal, scale, 1.0, 1.0, 1.0, eps8=eps)
    vis = oracle.visible_mask(np.arange(nq), nq, nkv, causal)
    e = eps * scale * (np.abs(q) @ np.abs(k).T)
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    worst = 0.0
    for trial in range(6):
        if trial < 3:
            delta = rng.uniform(-1, 1, e.shape) * e
        else:  # push the weight towards the keys whose V is largest in column `trial`
            c = trial - 3
            delta = np.sign(v[:, c] - o_ref[:, c:c + 1]) * e
        sp = s + delta
        m = sp.max(axis=1, keepdims=True)
        w = np.exp(sp - m)
        w_sum = w.sum(axis=1, keepdims=True)
        eta = rng.uniform(-1, 1, (nq, nkv, 1)) * eps
        o = ((w[:, :, None] * v[None, :, :]) * (1 + eta)).sum(axis=1) / w_sum
        lse = (m + np.log(w_sum))[:, 0]
        assert np.all(np.abs(o - o_ref) <= o_b + 1e-12)
        assert np.all(np.abs(lse - lse_ref) <= lse_b + 1e-12)
        worst = max(worst, float(np.max(np.abs(o - o_ref) / (o_b + 1e-300))))
    assert worst > 0.05
