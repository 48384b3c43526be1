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


def test_pow2_block_scale():
    for amax in (448.0, 449.0, 224.0, 224.5, 1.0, 3.5, 1e-3, 7e20):
        s = ar.pow2_block_scale(amax)
        assert math.log2(s) == int(math.log2(s))
        assert 224.0 < amax / s <= 448.0, (amax, s)
    assert ar.pow2_block_scale(0.0) == 1.0
    assert ar.pow2_block_scale(1e-40) == 2.0 ** -126


def test_quantize_fp8_blocks_known_block():
    x = np.array([[1.0, -2.0, 0.5], [0.25, 0.0, 1.5]])
    vals, scales = ar.quantize_fp8_blocks(x[None], 2)
    # amax 2: 448 2^-8 = 1.75 < 2 <= 3.5 = 448 2^-7, so the scale is 2^-7
    assert scales.tolist() == [[2.0 ** -7]]
    assert vals[0].tolist() == [[128.0, -256.0, 64.0], [32.0, 0.0, 192.0]]


def test_quantize_fp8_blocks_error_bound():
    """Dequantised values are within half an e4m3 spacing of the input:
    2^-4 relative in the normal range, 2^-10 x scale below it."""
    x = np.random.default_rng(61).standard_normal((2, 300, 64)) * np.exp2(np.arange(300) % 7)[:, None]
    vals, scales = ar.quantize_fp8_blocks(x, 64)
    sr = np.repeat(scales, 64, axis=-1)[..., :300, None]
    deq = vals * sr
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sr)
    assert np.all(np.abs(deq - x) <= bound)
    assert np.all(np.abs(vals) <= 448)
    blk_max = np.abs(vals[:, :256]).reshape(2, 4, 64 * 64).max(-1)  # the four full blocks
    assert np.all((blk_max >= 224) & (blk_max <= 448))


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


def _fp8_inputs(N, d, seed, bm=128, bn=64, scale_rows=None):
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


def test_fp8_forward_uniform_scores_give_mean_of_v():
    N = 200
    q8, k8, v8, sq, sk, sv = _fp8_inputs(N, 64, 70)
    O, LSE = ar.ref_fwd_fp8(0 * q8, k8, v8, sq, sk, sv, 0.125)
    np.testing.assert_allclose(O[0, 0], _dequant(v8, sv, 64)[0, 0].mean(0)[None].repeat(N, 0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(LSE, math.log(N), rtol=1e-14)


def test_fp8_forward_single_key():
    """One key: O = v^ e4m3(a) / a with a = 2^(u - ceil(u) + 3)."""
    q8, k8, v8, sq, sk, sv = _fp8_inputs(1, 64, 71)
    u = 0.125 * float(_dequant(q8, sq, 128)[0, 0, 0] @ _dequant(k8, sk, 64)[0, 0, 0]) * math.log2(math.e)
    a = 2.0 ** (u - math.ceil(u) + 3)
    O, LSE = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125)
    want = _dequant(v8, sv, 64)[0, 0, 0] * float(ar.e4m3_round(np.array([a]))[0]) / a
    np.testing.assert_allclose(O[0, 0, 0], want, rtol=1e-13)
    assert LSE[0, 0, 0] == pytest.approx(u * math.log(2), rel=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_without_p_rounding_is_exact_attention(monkeypatch, causal):
    """With P~ left unrounded the method is exact attention of the dequantised
    inputs (section 8.9.4), so every step other than P~'s rounding is pinned
    to the plain definition."""
    q8, k8, v8, sq, sk, sv = _fp8_inputs(150, 64, 72, bm=32)
    monkeypatch.setattr(ar, "e4m3_round", lambda x: np.asarray(x, dtype=np.float64))
    O, LSE = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125, causal, block_m=32)
    O2, L2 = ar.ref_fwd(_dequant(q8, sq, 32), _dequant(k8, sk, 64), _dequant(v8, sv, 64), 0.125, causal)
    np.testing.assert_allclose(O, O2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(LSE, L2, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_error_within_p_rounding_bound(causal):
    """O differs from exact attention of the dequantised inputs only by P~'s
    rounding: |dO| <= sum_j |e4m3(a_j) - a_j| |v_j| / l <= (2^-4 + 2^-7) max|v|
    (half a spacing: 2^-4 relative for normal a_j; subnormal a_j < 2^-6 are
    off by at most 2^-10 each, and l >= 4 since M < max u + 1).  V's rows
    vary in size so that a mix-up of V block scales breaks the bound."""
    N = 256
    q8, k8, v8, sq, sk, sv = _fp8_inputs(N, 64, 73, scale_rows=np.exp2(np.arange(N) // 64 * 3.0))
    O, _ = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125, causal)
    vd = _dequant(v8, sv, 64)
    O2, _ = ar.ref_fwd(_dequant(q8, sq, 128), _dequant(k8, sk, 64), vd, 0.125, causal)
    err = np.abs(O - O2)
    assert err.max() <= (2.0 ** -4 + N * 2.0 ** -12) * np.abs(vd).max()
    # and, on average, inside the per-key relative bound (errors of different keys partly cancel)
    assert np.sqrt((err ** 2).mean()) <= 2.0 ** -4 * np.sqrt((O2 ** 2).mean())


def test_fp8_forward_integer_reference_shift():
    """Every integer reference gives the same O while the a_j stay normal."""
    q8, k8, v8, sq, sk, sv = _fp8_inputs(120, 64, 74)
    O0, L0 = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.05)
    for shift in (1, 2, -3):
        O1, L1 = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.05, ref_shift=shift)
        np.testing.assert_allclose(O1, O0, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(L1, L0, rtol=1e-13)


def test_fp8_forward_rounding_slack():
    """The slack bounds how far O moves when every a_j is perturbed by a
    relative error below eps (as an fp32 evaluation would): the perturbed
    results, computed by rounding perturbed a_j, stay within it; with eps = 0
    and no subnormal a_j it is zero."""
    q8, k8, v8, sq, sk, sv = _fp8_inputs(60, 64, 76)
    eps = 2.0 ** -6  # large, so that the perturbations below do flip roundings
    O, _, R, _ = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125, tie_rel=eps)
    flipped = False
    rng = np.random.default_rng(77)
    true_round = ar.e4m3_round
    for _ in range(3):
        delta = rng.uniform(-eps, eps, 60)

        def jittered(x, _d=delta):
            x = np.asarray(x, dtype=np.float64)
            return true_round(np.minimum(x * (1 + _d[:x.shape[-1]]), 448.0)) if x.ndim == 1 and x.shape[0] == 60 \
                else true_round(x)

        ar.e4m3_round = jittered
        try:
            Oj, _ = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125)
        finally:
            ar.e4m3_round = true_round
        assert np.all(np.abs(Oj - O) <= R + 1e-15)
        flipped |= bool(np.any(Oj != O))
    assert flipped
    # uniform scores: every a_j is exactly 8, far from a tie and normal
    O0, _, R0, RL0 = ar.ref_fwd_fp8(0 * q8, k8, v8, sq, sk, sv, 0.125, tie_rel=eps)
    np.testing.assert_allclose(R0, np.abs(O0) * eps, rtol=1e-6)   # only l's own error remains
    np.testing.assert_allclose(RL0, np.log1p(eps), rtol=1e-12)
    # a score error bound widens every band, so the slack can only grow
    _, _, R1, RL1 = ar.ref_fwd_fp8(q8, k8, v8, sq, sk, sv, 0.125, tie_rel=eps, score_rel=2.0 ** -9)
    assert np.all(R1 >= R) and np.any(R1 > R) and np.all(RL1 > RL0[..., :1])


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


def test_mutant_lse_merge_without_weights_fails_union_pin(monkeypatch):
    """Averaging the two partial outputs (ignoring their LSEs) must break the
    union pin."""
    monkeypatch.setattr(ar, "ref_merge_lse", lambda oa, la, ob, lb: (0.5 * (oa + ob), np.logaddexp(la, lb)))
    with pytest.raises(AssertionError):
        test_merge_of_key_subsets_is_attention_over_their_union()


def test_oracle_exports():
    for name in oracle.__all__ if hasattr(oracle, "__all__") else ():
        assert callable(getattr(oracle, name))
