"""Pins of the fp64 oracle against values and properties the pages and the
mathematics fix.  CPU only.

Each pin is chosen so that a plausible mistake in the oracle (a missing
rescale, a dropped term, a wrong sign, a transposed operand, a wrong scale
placement) fails at least one of them; the mutation tests at the bottom plant
such mistakes and check that they are caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import attention_ref as ar
from exact_attention_05_amd.inputs import worked_example_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# The 4-token worked example ([cnblogs] section 2)
# ---------------------------------------------------------------------------

def _worked_inputs(d=4):
    q, k, v = worked_example_qkv(d, torch.float32)
    return q.double().numpy(), k.double().numpy(), v.double().numpy()


def test_worked_example_scores_match_page():
    g = _golden("worked_example.json")
    q, k, _ = _worked_inputs()
    S = q[0, 0] @ k[0, 0].T
    assert np.array_equal(S[:2, :2], np.array(g["S11"], float))
    assert np.array_equal(S[:2, 2:], np.array(g["S12"], float))


def test_worked_example_blockwise_trace_matches_page():
    g = _golden("worked_example.json")
    q, k, v = _worked_inputs()
    B = g["block"]
    _, _, tr = ar.ref_blockwise_fwd(q, k, v, 1.0, False, B, B, trace=True)
    tr = tr[(0, 0)]
    m1, l1, a1 = tr[(0, 0)]
    m2, l2, a2 = tr[(0, 2)]
    assert np.array_equal(m1, np.array(g["m_after_block1"], float))
    # first non-empty block: the old contribution's coefficient is 0
    assert np.array_equal(a1, np.zeros(2))
    # after block 2 the running max is the max of the old max and the block max
    assert np.array_equal(m2, np.maximum(m1, np.array(g["blockmax_block2"], float)))
    # row 0 is rescaled by e^(20-30); row 1's max does not grow, so its factor is exactly 1
    assert a2[0] == pytest.approx(math.exp(g["row0_rescale_exponent"]), rel=1e-15)
    assert a2[1] == 1.0


def test_worked_example_closed_form():
    """Final probabilities by hand: row 0 scores [10, 20, 30, 5], row 1 [10, 10, 5, 5]."""
    q, k, v = _worked_inputs()
    O, LSE = ar.ref_fwd(q, k, v, 1.0, False)
    e5, e10, e20, e25 = (math.exp(-x) for x in (5, 10, 20, 25))
    z0 = 1.0 + e10 + e20 + e25  # factor out e^30
    row0 = np.array([e20, e10, 1.0, e25]) / z0
    lse0 = 30.0 + math.log(z0)
    z1 = 2.0 * (1.0 + e5)  # factor out e^10
    row1 = np.array([1.0, 1.0, e5, e5]) / z1
    lse1 = 10.0 + math.log(z1)
    for r in range(4):  # V = I, so O rows are the probability rows; rows 2, 3 repeat 0, 1
        want, wl = (row0, lse0) if r % 2 == 0 else (row1, lse1)
        np.testing.assert_allclose(O[0, 0, r], want, rtol=1e-13, atol=1e-300)
        assert LSE[0, 0, r] == pytest.approx(wl, rel=1e-15)


def test_worked_example_online_equals_one_shot():
    """[cnblogs] section 2 note: the online merge equals a one-shot softmax."""
    q, k, v = _worked_inputs()
    O1, L1 = ar.ref_fwd(q, k, v, 1.0, False)
    for Br in (1, 2, 4):
        for Bc in (1, 2, 3, 4):
            O2, L2 = ar.ref_blockwise_fwd(q, k, v, 1.0, False, Br, Bc)
            np.testing.assert_allclose(O2, O1, rtol=1e-13, atol=1e-300)
            np.testing.assert_allclose(L2, L1, rtol=1e-15)


# ---------------------------------------------------------------------------
# alpha pins ([Triton-ch8] exercise; [operatorworld] degeneration checks)
# ---------------------------------------------------------------------------

def test_alpha_exercise_value():
    g = _golden("alpha_exercise.json")
    n_before = g["blocks_before_jump"]
    Bc = 3
    # one query row; a key block's score max is set through q . k_j with q = e_0
    N = (n_before + 1) * Bc
    q = np.zeros((1, 1, 1, 2))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, 2))
    k[0, 0, :, 0] = -5.0
    for b in range(n_before):
        k[0, 0, b * Bc, 0] = g["m_old"]
    k[0, 0, n_before * Bc + 1, 0] = g["m_new"]
    v = _rand((1, 1, N, 2), 0)
    _, _, tr = ar.ref_blockwise_fwd(q, k, v, 1.0, False, 1, Bc, trace=True)
    tr = tr[(0, 0)]
    for b in range(1, n_before):
        m, _, a = tr[(0, b * Bc)]
        assert m[0] == g["m_old"] and a[0] == 1.0  # max unchanged: factor exactly 1
    m, _, a = tr[(0, n_before * Bc)]
    assert m[0] == g["m_new"]
    assert a[0] == pytest.approx(g["alpha"], rel=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_single_block_degenerates_to_softmax(causal):
    q, k, v = (_rand((2, 3, 7, 5), s) for s in (1, 2, 3))
    O1, L1 = ar.ref_fwd(q, k, v, 0.4, causal)
    O2, L2, tr = ar.ref_blockwise_fwd(q, k, v, 0.4, causal, 7, 7, trace=True)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L2, L1, rtol=1e-12)
    for h in tr:
        (_, _, a), = tr[h].values()
        assert np.all(a == 0.0)


# ---------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    q, k = _rand((2, 2, 9, 6), 4), _rand((2, 2, 9, 6), 5)
    v = np.ones((2, 2, 9, 3))
    O, LSE = ar.ref_fwd(q, k, v, 0.7, causal)
    assert np.max(np.abs(O - 1.0)) <= 1e-14
    S = 0.7 * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        S = np.where(np.tril(np.ones((9, 9), bool)), S, -np.inf)
    np.testing.assert_allclose(np.exp(S - LSE[..., None]).sum(-1), 1.0, rtol=1e-14)


def test_uniform_scores_noncausal():
    N = 11
    q = np.zeros((1, 2, N, 4))
    k, v = _rand((1, 2, N, 4), 6), _rand((1, 2, N, 5), 7)
    O, LSE = ar.ref_fwd(q, k, v, 0.5, False)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(LSE, math.log(N), rtol=1e-15)


def test_uniform_scores_causal():
    N = 10
    k = np.zeros((1, 1, N, 4))
    q, v = _rand((1, 1, N, 4), 8), _rand((1, 1, N, 3), 9)
    O, LSE = ar.ref_fwd(q, k, v, 1.3, True)
    for i in range(N):
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, : i + 1].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert LSE[0, 0, i] == pytest.approx(math.log(i + 1), abs=1e-15)


def test_uniform_scores_causal_backward():
    N = 8
    k = np.zeros((1, 1, N, 3))
    q, v, dO = (_rand((1, 1, N, 3), s) for s in (10, 11, 12))
    _, _, dV = ar.ref_bwd(q, k, v, dO, 0.9, True)
    for j in range(N):
        want = sum(dO[0, 0, i] / (i + 1) for i in range(j, N))
        np.testing.assert_allclose(dV[0, 0, j], want, rtol=1e-13, atol=1e-15)
    q0 = np.zeros_like(q)
    _, dK, _ = ar.ref_bwd(q0, _rand((1, 1, N, 3), 13), v, dO, 0.9, True)
    assert np.all(dK == 0.0)  # dK = scale dS^T Q vanishes with Q = 0


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    q, k, v = (_rand((1, 2, 8, 4), s) for s in (14, 15, 16))
    c = _rand((4,), 17)
    O1, L1 = ar.ref_fwd(q, k, v, 0.6, causal)
    O2, L2 = ar.ref_fwd(q, k + c, v, 0.6, causal)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L1 + 0.6 * (q @ c), rtol=1e-12, atol=1e-13)


def test_q_pos_subset_matches_full_rows():
    q, k, v = (_rand((1, 1, 12, 4), s) for s in (18, 19, 20))
    O, LSE = ar.ref_fwd(q, k, v, 0.5, True)
    rows = np.array([0, 5, 11])
    O2, L2 = ar.ref_fwd(q[:, :, rows], k, v, 0.5, True, q_pos=rows)
    np.testing.assert_allclose(O2, O[:, :, rows], rtol=1e-14)
    np.testing.assert_allclose(L2, LSE[:, :, rows], rtol=1e-14)


def test_fully_masked_row_reading():
    """A query that sees no key (reachable only through q_pos) gives O = 0, LSE = -inf."""
    q, k, v = (_rand((1, 1, 4, 3), s) for s in (21, 22, 23))
    O, LSE = ar.ref_fwd(q[:, :, :1], k[:, :, 2:], v[:, :, 2:], 1.0, True, q_pos=np.array([-1]))
    assert np.all(O == 0.0) and LSE[0, 0, 0] == -np.inf


# ---------------------------------------------------------------------------
# Brute force: blockwise online == global, every block shape on tiny N
# ---------------------------------------------------------------------------

@settings(max_examples=150, deadline=None)
@given(
    N=st.integers(1, 16),
    br=st.integers(1, 16),
    bc=st.integers(1, 16),
    causal=st.booleans(),
    seed=st.integers(0, 10_000),
)
def test_blockwise_equals_global(N, br, bc, causal, seed):
    Br, Bc = min(br, N), min(bc, N)
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((1, 1, N, 3)) * 3, rng.standard_normal((1, 1, N, 3)) * 3
    v = rng.standard_normal((1, 1, N, 2))
    O1, L1 = ar.ref_fwd(q, k, v, 0.8, causal)
    O2, L2 = ar.ref_blockwise_fwd(q, k, v, 0.8, causal, Br, Bc)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L1, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Independent implementations: scipy's softmax/logsumexp, torch SDPA in fp64
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_forward_against_scipy(causal):
    from scipy.special import logsumexp, softmax

    q, k, v = (_rand((2, 2, 13, 8), s) for s in (24, 25, 26))
    O, LSE = ar.ref_fwd(q, k, v, 0.35, causal)
    S = 0.35 * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        S = np.where(np.tril(np.ones((13, 13), bool)), S, -np.inf)
    np.testing.assert_allclose(O, softmax(S, axis=-1) @ v, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(LSE, logsumexp(S, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_backward_against_torch_autograd(causal):
    import torch.nn.functional as F

    q, k, v, dO = (_rand((2, 3, 10, 6), s) for s in (27, 28, 29, 30))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.45)
    out.backward(torch.tensor(dO))
    O, _ = ar.ref_fwd(q, k, v, 0.45, causal)
    dQ, dK, dV = ar.ref_bwd(q, k, v, dO, 0.45, causal)
    np.testing.assert_allclose(O, out.detach().numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Backward: central finite differences, and the rowsum invariants
# ---------------------------------------------------------------------------

def _loss(q, k, v, dO, scale, causal):
    O, _ = ar.ref_fwd(q, k, v, scale, causal)
    return float((O * dO).sum())


def _fd_grad(x, f, h=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 2), (5, 3), (6, 4)])
def test_backward_finite_differences(causal, N, d):
    q, k, v, dO = (_rand((1, 1, N, d), s) for s in (31, 32, 33, 34))
    s = 0.7
    dQ, dK, dV = ar.ref_bwd(q, k, v, dO, s, causal)
    gq = _fd_grad(q, lambda x: _loss(x, k, v, dO, s, causal))
    gk = _fd_grad(k, lambda x: _loss(q, x, v, dO, s, causal))
    gv = _fd_grad(v, lambda x: _loss(q, k, x, dO, s, causal))
    for got, want in ((dQ, gq), (dK, gk), (dV, gv)):
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    q, k, v, dO = (_rand((1, 2, 9, 5), s) for s in (35, 36, 37, 38))
    _, dK, _ = ar.ref_bwd(q, k, v, dO, 0.5, causal)
    # rowsum_j dS_ij = 0 for every i, hence sum_j dK_j = scale sum_i (sum_j dS_ij) Q_i = 0
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-13)
    # D_i = rowsum(P o dP) equals dO_i . O_i
    P = ar.ref_probs(q, k, 0.5, causal)
    O, _ = ar.ref_fwd(q, k, v, 0.5, causal)
    dP = dO @ np.swapaxes(v, -1, -2)
    np.testing.assert_allclose((P * dP).sum(-1), (dO * O).sum(-1), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Split-K decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S", [1, 2, 3, 7, 64, 97, 102])
def test_splitk_decode_equals_definition(S):
    L = 97
    q = _rand((2, 2, 1, 6), 39)
    k, v = _rand((2, 2, L, 6), 40), _rand((2, 2, L, 6), 41)
    O1, L1 = ar.ref_fwd(q, k, v, 0.4, False)
    O2, L2 = ar.ref_splitk_decode(q, k, v, 0.4, S)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L2, L1, rtol=1e-13)


def test_decode_chunk_bounds_cover_cache():
    for L, S in ((97, 7), (5, 8), (32768, 256), (1, 1)):
        b = ar.decode_chunk_bounds(L, S)
        assert b[0][0] == 0 and b[-1][1] == L
        assert all(b[i][1] == b[i + 1][0] for i in range(S - 1))
        assert all(hi - lo in (L // S, L // S + 1) for lo, hi in b)


def test_decode_partials_single_chunk_is_plain_softmax_state():
    """With one chunk the partial state is (sum e^(s-m) V, max s, sum e^(s-m))."""
    from scipy.special import logsumexp

    q, k, v = _rand((1, 1, 1, 4), 42), _rand((1, 1, 9, 4), 43), _rand((1, 1, 9, 4), 44)
    U, m, l = ar.ref_decode_partials(q, k, v, 0.5, 1)
    s = 0.5 * (k[0, 0] @ q[0, 0, 0])
    assert m[0, 0, 0] == s.max()
    assert m[0, 0, 0] + math.log(l[0, 0, 0]) == pytest.approx(logsumexp(s), rel=1e-15)


def test_decode_uniform_and_ones():
    L = 33
    q = np.zeros((1, 1, 1, 4))
    k, v = _rand((1, 1, L, 4), 45), _rand((1, 1, L, 4), 46)
    O, LSE = ar.ref_splitk_decode(q, k, v, 1.0, 5)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0].mean(axis=0), rtol=1e-13, atol=1e-15)
    assert LSE[0, 0, 0] == pytest.approx(math.log(L), rel=1e-15)
    O, _ = ar.ref_splitk_decode(_rand((1, 1, 1, 4), 47), k, np.ones((1, 1, L, 4)), 1.0, 40)
    assert np.max(np.abs(O - 1.0)) <= 1e-14


# ---------------------------------------------------------------------------
# Paged KV-cache decode ([FA1-vs-FA2] section 13 names the paged block table)
# ---------------------------------------------------------------------------

def _scatter_to_pool(k, bs, num_blocks, seed):
    """Cut a dense cache [B, H, L, d] into blocks of bs rows and place them at
    random distinct pool slots; returns (pool, table) with the unused slots
    filled with noise."""
    B, H, L, d = k.shape
    nb = -(-L // bs)
    rng = np.random.default_rng(seed)
    slots = rng.permutation(num_blocks)[:B * nb].reshape(B, nb)
    pool = rng.standard_normal((num_blocks, H, bs, d)) * 100.0
    for b in range(B):
        for j in range(nb):
            rows = k[b, :, j * bs:(j + 1) * bs]
            pool[slots[b, j], :, :rows.shape[1]] = rows
    return pool, slots


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_paged_decode_equals_dense_on_truncated_cache(bs):
    """Blocks scattered to random pool slots, ragged lengths: the result is the
    dense decode over each sequence's first seq_len keys."""
    B, H, L, d = 3, 2, 37, 5
    q = _rand((B, H, 1, d), 50)
    k, v = _rand((B, H, L, d), 51), _rand((B, H, L, d), 52)
    nblk = B * (-(-L // bs)) + 3
    kp, tab = _scatter_to_pool(k, bs, nblk, 53)
    vp = np.zeros_like(kp)
    for b in range(B):
        for j in range(tab.shape[1]):
            rows = v[b, :, j * bs:(j + 1) * bs]
            vp[tab[b, j], :, :rows.shape[1]] = rows
    lens = np.array([L, 1, 20])
    O, LSE = ar.ref_paged_decode(q, kp, vp, tab, lens, 0.6)
    for b in range(B):
        n = lens[b]
        O1, L1 = ar.ref_splitk_decode(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.6, 3)
        np.testing.assert_allclose(O[b], O1[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(LSE[b], L1[0], rtol=1e-13)


def test_paged_decode_brute_force_tiny():
    """One sequence of 5 tokens in blocks of 2 at pool slots (3, 0, 2): the
    weights written out term by term."""
    d = 2
    kp, vp = _rand((4, 1, 2, d), 54), _rand((4, 1, 2, d), 55)
    q = _rand((1, 1, 1, d), 56)
    table = np.array([[3, 0, 2]])
    keys = [kp[3, 0, 0], kp[3, 0, 1], kp[0, 0, 0], kp[0, 0, 1], kp[2, 0, 0]]
    vals = [vp[3, 0, 0], vp[3, 0, 1], vp[0, 0, 0], vp[0, 0, 1], vp[2, 0, 0]]
    s = [0.9 * (q[0, 0, 0, 0] * kk[0] + q[0, 0, 0, 1] * kk[1]) for kk in keys]
    w = [math.exp(x) for x in s]
    z = sum(w)
    want = [sum(w[i] * vals[i][c] for i in range(5)) / z for c in range(d)]
    O, LSE = ar.ref_paged_decode(q, kp, vp, table, np.array([5]), 0.9)
    np.testing.assert_allclose(O[0, 0, 0], want, rtol=1e-13)
    assert LSE[0, 0, 0] == pytest.approx(math.log(z), rel=1e-14)


def test_paged_decode_empty_sequence():
    kp = _rand((2, 1, 4, 3), 57)
    O, LSE = ar.ref_paged_decode(_rand((2, 1, 1, 3), 58), kp, kp, np.array([[0], [1]]), np.array([0, 3]), 1.0)
    assert np.all(O[0] == 0) and LSE[0, 0, 0] == -np.inf
    assert np.isfinite(LSE[1]).all()


def test_mutant_paged_row_index_fails_dense_pin(monkeypatch):
    """Swapping the block and the row index of a token must break the pin."""
    def bad_gather(pool, block_table, seq_len, h):
        pool = np.asarray(pool, dtype=np.float64)
        bs = pool.shape[2]
        rows = [pool[int(block_table[t % len(block_table)]), h, (t // len(block_table)) % bs] for t in range(seq_len)]
        return np.array(rows).reshape(seq_len, pool.shape[3])

    monkeypatch.setattr(ar, "gather_paged_rows", bad_gather)
    with pytest.raises(AssertionError):
        test_paged_decode_equals_dense_on_truncated_cache(4)


# ---------------------------------------------------------------------------
# FP8 (E4M3) quantisation and forward ([Triton-ch8] section 8.9)
# ---------------------------------------------------------------------------

def test_e4m3_round_matches_torch_cast():
    """torch's float8_e4m3fn cast is an independent implementation of the
    same rounding (nearest, ties to even) on [-448, 448]."""
    rng = np.random.default_rng(60)
    x = np.concatenate([
        rng.standard_normal(20000) * 30,
        np.exp2(rng.uniform(-14, 8.8, 20000)) * rng.choice([-1, 1], 20000),
        # every midpoint between neighbouring positive e4m3 values
        0.5 * (ar.e4m3_round(np.exp2(np.arange(-9, 8.8, 0.01))[:-1]) +
               ar.e4m3_round(np.exp2(np.arange(-9, 8.8, 0.01))[1:])),
    ])
    x = np.clip(x, -448, 448)
    ref = torch.tensor(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ar.e4m3_round(x), ref)


def test_e4m3_round_values_from_the_format():
    # representable values map to themselves; ties go to the even mantissa
    grid = [0.0, 2.0 ** -9, 3 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 1.75, 240.0, 448.0]
    assert list(ar.e4m3_round(np.array(grid))) == grid
    assert ar.e4m3_round(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 432.0])).tolist() == \
        [1.0, 1.25, 0.0, 2.0 ** -8, 448.0]
    assert ar.e4m3_round(np.array([-1.0625]))[0] == -1.0


def _fp32_bits_value(sign_exp, frac_bits):
    """An fp32 number written out from its fields: 2^sign_exp (1 + frac / 2^23)."""
    return math.ldexp(1.0 + frac_bits / 2.0 ** 23, sign_exp)


def test_fp8_block_scale_by_hand():
    """scale = max|x| / 448 in fp32 ([Triton-ch8] section 8.9.4).  3 / 448 =
    (12/7) 2^-8 and 12/7 = 1.101101101...b: the fraction's first 23 bits are
    10110110110110110110110b with 110b following, so it rounds up to
    ...110111b.  1 / 448 = 2^-9 (8/7) = 2^-9 1.001001001...b: the first 23
    fraction bits are 00100100100100100100100b and 100b follows, so it
    also rounds up."""
    assert ar.fp8_block_scale(3.0) == _fp32_bits_value(-8, 0b10110110110110110110111)
    assert ar.fp8_block_scale(1.0) == _fp32_bits_value(-9, 0b00100100100100100100101)
    assert ar.fp8_block_scale(448.0) == 1.0 and ar.fp8_block_scale(3.5) == 2.0 ** -7
    assert ar.fp8_block_scale(0.0) == 1.0


def test_quantize_fp8_blocks_known_block():
    """A block worked by hand: max|x| = 3, so x / scale is about 448 x / 3:
    1 -> 149.33 (neighbours 144, 160: 144), -3 -> -448, 2 -> 298.67 (288,
    320: 288), 0.5 -> 74.67 (72, 80: 72), 0 -> 0; none is near a midpoint,
    so the fp32 rounding of the scale does not matter.  A second block of
    row 2 alone has max 1.5 -> scale 1.5 / 448 and codes 448 and -149.33 ->
    -144."""
    x = np.array([[1.0, -3.0], [2.0, 0.5], [1.5, -0.5]])
    vals, scales = ar.quantize_fp8_blocks(x[None], 2)
    assert scales[0, 0] == ar.fp8_block_scale(3.0)
    assert scales[0, 1] == _fp32_bits_value(-9, 0b10110110110110110110111)  # 1.5 / 448 = (12/7) 2^-9
    assert vals[0].tolist() == [[144.0, -448.0], [288.0, 72.0], [448.0, -144.0]]


def test_quantize_fp8_blocks_error_bound():
    """Dequantised values are within half an e4m3 spacing of the input
    (2^-4 relative in the normal range, 2^-10 x scale below it, plus the
    fp32 quotient's own rounding), and every full block reaches 448."""
    x = np.random.default_rng(61).standard_normal((2, 300, 64)) * np.exp2(np.arange(300) % 7)[:, None]
    x = x.astype(np.float32).astype(np.float64)
    vals, scales = ar.quantize_fp8_blocks(x, 64)
    sr = np.repeat(scales, 64, axis=-1)[..., :300, None]
    deq = vals * sr
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sr) * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - x) <= bound)
    assert np.all(np.abs(vals) <= 448)
    blk_max = np.abs(vals).reshape(2, -1)[:, :4 * 64 * 64].reshape(2, 4, -1).max(-1)
    assert np.all(blk_max == 448)


def test_hadamard_rotation_is_orthogonal():
    from scipy.linalg import hadamard

    d = 64
    s = np.random.default_rng(62).choice([-1.0, 1.0], d)
    x, y = _rand((5, d), 63), _rand((7, d), 64)
    xr, yr = ar.hadamard_rotate(x, s), ar.hadamard_rotate(y, s)
    np.testing.assert_allclose(xr @ yr.T, x @ y.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(xr, (x * s) @ hadamard(d) / 8.0, rtol=1e-13, atol=1e-14)
    e = np.zeros(d)
    e[5] = 1.0
    assert np.allclose(np.abs(ar.hadamard_rotate(e, s)), 1.0 / 8.0)


def _fp8_inputs(N, d, seed, bm=32, bn=64, scale_rows=None):
    q, k, v = (_rand((1, 1, N, d), seed + i) for i in range(3))
    if scale_rows is not None:
        v = v * scale_rows[None, None, :, None]
    q8, sq = ar.quantize_fp8_blocks(q, bm)
    k8, sk = ar.quantize_fp8_blocks(k, bn)
    v8, sv = ar.quantize_fp8_blocks(v, bn)
    return q8, k8, v8, sq, sk, sv


def _dequant(x8, s, rows):
    """e4m3 values times their block's scale (written out here, not taken
    from the oracle, so the mutation test below changes one side only)."""
    return x8 * np.repeat(s, rows, axis=-1)[..., :x8.shape[-2], None]


def test_fp8_forward_worked_by_hand():
    """Four query rows in two blocks of two, four keys in two blocks of two,
    d = 1, scale = ln 2 (so p = 2^(score in units of ln 2 - running max)).
    K values k8 sk = [2, 1 | 3 x 0.5, -4 x 0.5] = [2, 1 | 1.5, -2], V values
    v8 = [1, 2 | 4, 7] with sv = [1 | 2], queries q8 = [1, -1 | 1, 0.5].

    Query block 0 (rows q = 1 and q = -1):
      key block 0: scores [2, 1] and [-2, -1]: m = 2 and -1, p = [1, 1/2] and
        [1/2, 1], max(p) = 1, so p / scale_p = 448 p = [448, 224], [224, 448]
        (exact); acc = (448 v0 + 224 v1) / 448 = 2 and (224 + 896) / 448 = 2.5.
      key block 1: scores [1.5, -2] (row 0: m stays 2, p = [2^-.5, 2^-4]) and
        [-1.5, 2] (row 1: m -> 2, alpha = 2^-3, p = [2^-3.5, 1]); max(p) = 1;
        448 p = [316.78 -> 320, 28] and [39.60 -> 40, 448];
        acc0 = 2 + (320*4 + 28*7) * 2/448 = 2 + 369/56,
        acc1 = 2.5/8 + (40*4 + 448*7) * 2/448 = 5/16 + 103/7.
      l0 = 3/2 + 2^-.5 + 2^-4,  l1 = 3/2 / 8 + 2^-3.5 + 1.
    Query block 1 (rows q = 1 and q = 0.5):
      key block 0: row 2 as row 0; row 3 scores [1, .5]: m = 1, p = [1,
        2^-.5]; max(p) = 1: 448 p = [448, 224] and [448, 316.78 -> 320];
        acc2 = 2, acc3 = (448 + 640) / 448 = 17/7.
      key block 1: row 2 p = [2^-.5, 2^-4]; row 3 scores [.75, -1], m stays 1,
        p = [2^-.25, 2^-2].  Now max(p) = 2^-.25 (row 3), below 1, so
        scale_p = 2^-.25 / 448 and p / scale_p = 448 p 2^.25:
        row 2 [376.71 -> 384, 33.30 -> 32], row 3 [448, 133.19 -> 128];
        acc2 += (384*4 + 32*7) * 2 * 2^-.25 / 448 = (55/7) 2^-.25,
        acc3 += (448*4 + 128*7) * 2 * 2^-.25 / 448 = 12 * 2^-.25.
      l2 = l0,  l3 = 1 + 2^-.5 + 2^-.25 + 1/4.
    The roundings 320, 40, 384, 32 and 128 are each at least 1.2 from a
    midpoint of their E4M3 neighbours.  LSE = (2, 2, 2, 1) ln 2 + ln l."""
    q8 = np.array([1.0, -1.0, 1.0, 0.5]).reshape(1, 1, 4, 1)
    k8 = np.array([2.0, 1.0, 3.0, -4.0]).reshape(1, 1, 4, 1)
    v8 = np.array([1.0, 2.0, 4.0, 7.0]).reshape(1, 1, 4, 1)
    sq, sk, sv = np.ones((1, 1, 2)), np.array([[[1.0, 0.5]]]), np.array([[[1.0, 2.0]]])
    O, LSE, Y, W = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, math.log(2.0), block_m=2, block_n=2, trace=True)
    r = 2.0 ** -0.5
    q = 2.0 ** -0.25
    want_codes = [[448, 224, 320, 28], [224, 448, 40, 448], [448, 224, 384, 32], [448, 320, 448, 128]]
    assert ar.e4m3_round(Y[0, 0]).tolist() == want_codes
    acc = [2 + 369 / 56, 5 / 16 + 103 / 7, 2 + 55 / 7 * q, 17 / 7 + 12 * q]
    l = [1.5 + r + 1 / 16, 1.5 / 8 + r / 8 + 1, 1.5 + r + 1 / 16, 1 + r + q + 0.25]
    m = [2, 2, 2, 1]
    for i in range(4):
        assert O[0, 0, i, 0] == pytest.approx(acc[i] / l[i], rel=1e-14), i
        assert LSE[0, 0, i] == pytest.approx((m[i] + math.log2(l[i])) * math.log(2.0), rel=1e-14), i
    # the trace reproduces O from the rounded values and their unit weights
    np.testing.assert_allclose((ar.e4m3_round(Y[0, 0]) * W[0, 0]) @ v8[0, 0], O[0, 0], rtol=1e-14)


def test_fp8_forward_uniform_scores_give_mean_of_v():
    """Q = 0: every p is 1, p / scale_p = 448 exactly, so O is the mean of
    the dequantised V and LSE = ln N."""
    N = 200
    q8, k8, v8, sq, sk, sv = _fp8_inputs(N, 64, 70)
    O, LSE = ar.ref_fwd_fp8(0 * q8, k8, v8, sq, sk, sv, 0.125)
    np.testing.assert_allclose(O[0, 0], _dequant(v8, sv, 64)[0, 0].mean(0)[None].repeat(N, 0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(LSE, math.log(N), rtol=1e-14)


def test_fp8_forward_single_key():
    """One key: p = 1, p / scale_p = 448, O = the dequantised v, LSE = the
    score."""
    q8, k8, v8, sq, sk, sv = _fp8_inputs(1, 64, 71)
    u = 0.125 * float(_dequant(q8, sq, 32)[0, 0, 0] @ _dequant(k8, sk, 64)[0, 0, 0])
    O, LSE = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125)
    np.testing.assert_allclose(O[0, 0, 0], _dequant(v8, sv, 64)[0, 0, 0], rtol=1e-14)
    assert LSE[0, 0, 0] == pytest.approx(u, rel=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bm,bn", [(32, 64), (7, 13), (150, 150)])
def test_fp8_forward_without_p_rounding_is_exact_attention(monkeypatch, causal, bm, bn):
    """With P left unrounded the method is exact attention of the dequantised
    inputs (section 8.9.3), for any block sizes, so every step other than
    P's rounding (scales, the online max and alpha, scale_p and the V scale
    of each block's product) is pinned to the plain definition."""
    q8, k8, v8, sq, sk, sv = _fp8_inputs(150, 64, 72, bm=bm, bn=bn)
    monkeypatch.setattr(ar, "e4m3_round", lambda x: np.asarray(x, dtype=np.float64))
    O, LSE = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125, causal, block_m=bm, block_n=bn)
    O2, L2 = ar.ref_fwd(_dequant(q8, sq, bm), _dequant(k8, sk, bn), _dequant(v8, sv, bn), 0.125, causal)
    np.testing.assert_allclose(O, O2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(LSE, L2, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_error_within_p_rounding_bound(causal):
    """O differs from exact attention of the dequantised inputs only by P's
    rounding: every p8 / (p / scale_p) is within half an E4M3 spacing, 2^-4
    relative (normal) or 2^-10 absolute (subnormal, with p / scale_p <= 448
    and scale_p p-relative), so |dO| <= 2^-4 max|v| + N 2^-10 max|v| / 448.
    V's rows vary in size so that a mix-up of V block scales breaks the
    bound."""
    N = 256
    q8, k8, v8, sq, sk, sv = _fp8_inputs(N, 64, 73, scale_rows=np.exp2(np.arange(N) // 64 * 3.0))
    O, _ = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125, causal)
    vd = _dequant(v8, sv, 64)
    O2, _ = ar.ref_fwd(_dequant(q8, sq, 32), _dequant(k8, sk, 64), vd, 0.125, causal)
    err = np.abs(O - O2)
    assert err.max() <= (2.0 ** -4 + N * 2.0 ** -10 / 448) * np.abs(vd).max()
    # and, on average, inside the per-key relative bound (errors of different keys partly cancel)
    assert np.sqrt((err ** 2).mean()) <= 2.0 ** -4 * np.sqrt((O2 ** 2).mean())


def test_fp8_forward_block_max_spans_the_rows():
    """The P scale is one per block of rows and keys: a row whose own largest
    p in a key block is below the block's largest p is rounded on a finer
    relative grid than alone.  Splitting the same inputs into one-row blocks
    changes those rows' results, and only by P rounding."""
    q8, k8, v8, sq, sk, sv = _fp8_inputs(256, 64, 78)
    O32, _ = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125, block_m=32)
    sq1 = np.repeat(sq, 32, axis=-1)
    O1, _ = ar.ref_fwd_fp8(q8, k8, v8, sq1, sk, sv, 0.125, block_m=1)
    assert np.any(O1 != O32)
    np.testing.assert_allclose(O1, O32, atol=2.0 ** -3 * np.abs(_dequant(v8, sv, 64)).max())


def test_hadamard_rotation_helps_outlier_features():
    """Incoherent processing ([Triton-ch8] section 8.9.5): with a few feature
    dimensions far larger than the rest, rotating Q and K before the block
    quantisation lowers the error of the scores."""
    rng = np.random.default_rng(75)
    N, d = 256, 64
    q, k = rng.standard_normal((1, 1, N, d)), rng.standard_normal((1, 1, N, d))
    q[..., 3] *= 40.0
    k[..., 3] *= 40.0
    s = rng.choice([-1.0, 1.0], d)
    S = q[0, 0] @ k[0, 0].T

    def score_err(signs):
        q8, sq = ar.quantize_fp8_blocks(q, 64, signs)
        k8, sk = ar.quantize_fp8_blocks(k, 64, signs)
        Sq = _dequant(q8, sq, 64)[0, 0] @ _dequant(k8, sk, 64)[0, 0].T
        return np.sqrt(((Sq - S) ** 2).mean())

    assert score_err(s) < 0.5 * score_err(None)


# ---------------------------------------------------------------------------
# Merging results over disjoint key sets ([FA1-vs-FA2] section 6)
# ---------------------------------------------------------------------------

def _fwd_on_keys(q, k, v, scale, keys):
    """Plain attention of every query over the key subset `keys` (no mask)."""
    return ar.ref_fwd(q, k[..., keys, :], v[..., keys, :], scale)


def test_merge_of_key_subsets_is_attention_over_their_union():
    q, k, v = _rand((2, 3, 9, 5), 90), _rand((2, 3, 13, 5), 91), _rand((2, 3, 13, 5), 92)
    perm = np.random.default_rng(93).permutation(13)
    A, Bk = perm[:6], perm[6:]
    Oa, La = _fwd_on_keys(q, k, v, 0.7, A)
    Ob, Lb = _fwd_on_keys(q, k, v, 0.7, Bk)
    O, L = ar.ref_merge_lse(Oa, La, Ob, Lb)
    O2, L2 = ar.ref_fwd(q, k, v, 0.7)
    np.testing.assert_allclose(O, O2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L, L2, rtol=1e-13)


def test_merge_ring_of_causal_shards_is_causal_attention():
    """G query/key shards of a causal problem: shard i of the queries sees
    the diagonal block causally and blocks j < i fully; merging those partial
    results in ring order gives causal attention over the whole sequence."""
    N, G, S = 24, 4, 6
    q, k, v = _rand((1, 2, N, 4), 94), _rand((1, 2, N, 4), 95), _rand((1, 2, N, 4), 96)
    O2, L2 = ar.ref_fwd(q, k, v, 0.5, causal=True)
    for i in range(G):
        rows = slice(i * S, (i + 1) * S)
        O, L = ar.ref_fwd(q[..., rows, :], k[..., rows, :], v[..., rows, :], 0.5, causal=True)
        for j in range(i - 1, -1, -1):
            cols = slice(j * S, (j + 1) * S)
            Oj, Lj = ar.ref_fwd(q[..., rows, :], k[..., cols, :], v[..., cols, :], 0.5)
            O, L = ar.ref_merge_lse(O, L, Oj, Lj)
        np.testing.assert_allclose(O, O2[..., rows, :], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(L, L2[..., rows], rtol=1e-13)


def test_merge_identity_and_symmetry():
    o, l = _rand((3, 4), 97), _rand((3,), 98)
    o2, l2 = _rand((3, 4), 99), _rand((3,), 100)
    empty_o, empty_l = np.zeros((3, 4)), np.full(3, -np.inf)
    O, L = ar.ref_merge_lse(o, l, empty_o, empty_l)
    assert np.array_equal(O, o) and np.array_equal(L, l)
    O, L = ar.ref_merge_lse(empty_o, empty_l, empty_o, empty_l)
    assert np.all(O == 0) and np.all(L == -np.inf)
    with np.errstate(invalid="ignore"):
        O, L = ar.ref_merge_lse(o, l, np.full((3, 4), np.nan), empty_l)  # an empty side's O is never read
    assert np.array_equal(O, o) and np.array_equal(L, l)
    Oab, Lab = ar.ref_merge_lse(o, l, o2, l2)
    Oba, Lba = ar.ref_merge_lse(o2, l2, o, l)
    np.testing.assert_allclose(Oab, Oba, rtol=1e-15)
    np.testing.assert_allclose(Lab, Lba, rtol=1e-15)
    # equal LSEs: the plain average, and LSE + ln 2
    O, L = ar.ref_merge_lse(o, l, o2, l)
    np.testing.assert_allclose(O, 0.5 * (o + o2), rtol=1e-15)
    np.testing.assert_allclose(L, l + np.log(2.0), rtol=1e-15)


# ---------------------------------------------------------------------------
# Mutation tests: plausible oracle mistakes must fail the pins above
# ---------------------------------------------------------------------------

_TRUE_STEP = ar.online_softmax_step


def _no_rescale_step(m_old, l_old, U_old, S_blk, V_blk):
    """The 'most common bug' of [operatorworld]: old U is not rescaled."""
    m_new, l_new, _, alpha = _TRUE_STEP(m_old, l_old, U_old, S_blk, V_blk)
    base = np.where(np.isfinite(m_new), m_new, 0.0)
    U_new = U_old + np.exp(S_blk - base[:, None]) @ V_blk
    return m_new, l_new, U_new, alpha


def test_mutant_no_rescale_fails_worked_example(monkeypatch):
    monkeypatch.setattr(ar, "online_softmax_step", _no_rescale_step)
    q, k, v = _worked_inputs()
    O_bad, _ = ar.ref_blockwise_fwd(q, k, v, 1.0, False, 2, 2)
    O, _ = ar.ref_fwd(q, k, v, 1.0, False)
    # row 0 weights key 1 at about e^-10 in truth, but at about 1 in the mutant
    assert O_bad[0, 0, 0, 1] > 0.4 and O[0, 0, 0, 1] < 1e-4


def _bwd_mutant(q, k, v, dO, scale, causal, kind):
    P = ar.ref_probs(q, k, scale, causal)[0, 0]
    q, k, v, dO = q[0, 0], k[0, 0], v[0, 0], dO[0, 0]
    dV = P.T @ dO
    dP = dO @ v.T
    D = (P * dP).sum(axis=1)
    if kind == "drop_D":
        D = 0 * D
    dS = P * (dP - D[:, None])
    if kind == "sign":
        dS = P * (D[:, None] - dP)
    dQ = scale * (dS @ k)
    dK = scale * (dS.T @ q)
    if kind == "transpose":
        dK = scale * (dS @ q)
    if kind == "no_scale":
        dQ = dS @ k
    if kind == "dV_no_transpose":
        dV = P @ dO
    return dQ, dK, dV


@pytest.mark.parametrize("kind", ["drop_D", "sign", "transpose", "no_scale", "dV_no_transpose"])
def test_mutant_backward_fails_finite_differences(kind):
    N, d, s = 5, 3, 0.7
    q, k, v, dO = (_rand((1, 1, N, d), x) for x in (31, 32, 33, 34))
    bad = _bwd_mutant(q, k, v, dO, s, True, kind)
    good = ar.ref_bwd(q, k, v, dO, s, True)
    gq = _fd_grad(q, lambda x: _loss(x, k, v, dO, s, True))
    gk = _fd_grad(k, lambda x: _loss(q, x, v, dO, s, True))
    gv = _fd_grad(v, lambda x: _loss(q, k, x, dO, s, True))
    fd = (gq[0, 0], gk[0, 0], gv[0, 0])
    err_bad = max(np.max(np.abs(b - f)) for b, f in zip(bad, fd))
    err_good = max(np.max(np.abs(g[0, 0] - f)) for g, f in zip(good, fd))
    assert err_good < 1e-7 and err_bad > 1e-3


def test_mutant_merge_without_weights_fails_decode_pin(monkeypatch):
    def bad_merge(a, b):
        m = max(a[1], b[1])
        return a[0] + b[0], m, a[2] + b[2]

    monkeypatch.setattr(ar, "merge_two", bad_merge)
    q = _rand((1, 1, 1, 6), 39)
    k, v = _rand((1, 1, 50, 6), 40) * 2, _rand((1, 1, 50, 6), 41)
    O1, _ = ar.ref_fwd(q, k, v, 1.0, False)
    O2, _ = ar.ref_splitk_decode(q, k, v, 1.0, 4)
    assert np.max(np.abs(O2 - O1)) > 1e-3


def test_mutant_fp8_v_scale_mixup_fails_bound(monkeypatch):
    """Scaling V by the Q block scales instead of its own must break the
    rounding bound pin."""
    true_rows = ar._rows_of_blocks

    def bad_rows(scales, block_rows, N):
        return true_rows(scales, block_rows, N)[..., ::-1].copy()  # rows take another block's scale

    monkeypatch.setattr(ar, "_rows_of_blocks", bad_rows)
    with pytest.raises(AssertionError):
        test_fp8_forward_error_within_p_rounding_bound(False)


@pytest.mark.parametrize("orig,mutated", [
    # the listing's last line taken literally: the whole accumulator times scale_p sv after each block
    ("acc = alpha[:, None] * acc + (p8 @ v8[h][j0:j1]) * f", "acc = (alpha[:, None] * acc + p8 @ v8[h][j0:j1]) * f"),
    # a P scale per row instead of one over the block's rows and keys
    ("lpmax = np.max(lp)", "lpmax = np.max(lp, axis=1, keepdims=True)"),
    # the block's product without its V scale
    ("f = scale_p * float(sv[h][jb])", "f = scale_p"),
])
def test_mutant_fp8_forward_fails_hand_worked_block(monkeypatch, orig, mutated):
    """Plausible misreadings of the FP8 method must break the hand-worked pin
    (a per-row P scale changes the trace's shapes, so it may fail there)."""
    src = open(ar.__file__).read()
    assert src.count(orig) == 1
    ns = {"__name__": "mutant"}
    exec(compile(src.replace(orig, mutated), ar.__file__, "exec"), ns)
    monkeypatch.setattr(ar, "ref_fwd_fp8", ns["ref_fwd_fp8"])
    with pytest.raises((AssertionError, ValueError)):
        test_fp8_forward_worked_by_hand()


def test_mutant_lse_merge_without_weights_fails_union_pin(monkeypatch):
    """Averaging the two partial outputs (ignoring their LSEs) must break the
    union pin."""
    monkeypatch.setattr(ar, "ref_merge_lse", lambda oa, la, ob, lb: (0.5 * (oa + ob), np.logaddexp(la, lb)))
    with pytest.raises(AssertionError):
        test_merge_of_key_subsets_is_attention_over_their_union()


def test_oracle_exports():
    for name in oracle.__all__ if hasattr(oracle, "__all__") else ():
        assert callable(getattr(oracle, name))
