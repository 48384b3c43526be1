"""fp64 NumPy reference of exact attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the product path never does.

Conventions shared by every function:

* Tensors are NumPy arrays with any leading batch dimensions and the last two
  dimensions [sequence, head_dim]; they are widened to float64 on entry, so a
  bf16 or fp32 input is used at exactly the value the GPU reads.
* ``scale`` multiplies Q K^T before the max and the exponential
  ([xuesongtap] section 1; [Triton-ch8] section 8.1, where it is 1/sqrt(d)).
* ``causal`` masks key position j > query position i with -inf
  ([xuesongtap] section 2.2, last paragraph).  Query positions default to
  0..Nq-1 (square, top-left aligned); ``q_pos`` overrides them so a subset of
  query rows can be evaluated on its own.
* LSE is the natural-log log-sum-exp of the scaled scores, m + ln(l)
  ([xuesongtap] section 3; [Triton-ch8] section 8.8.2).
* A row that sees no key at all (only possible through ``q_pos`` or an empty
  key set) gets O = 0 and LSE = -inf; the pages leave this case open.
"""

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _visible(q_pos, k_pos, causal):
    """Boolean [Nq, Nk]: True where query q_pos[i] may attend key k_pos[j]."""
    if not causal:
        return np.ones((len(q_pos), len(k_pos)), dtype=bool)
    return k_pos[None, :] <= q_pos[:, None]


def _scores(q, k, scale, causal, q_pos):
    """S = scale * Q K^T with masked entries set to -inf ([xuesongtap] 1, 2.2)."""
    S = scale * (q @ k.T)
    vis = _visible(q_pos, np.arange(k.shape[0]), causal)
    return np.where(vis, S, NEG_INF)


def _softmax_rows(S):
    """Numerically stable softmax per row ([Triton-ch8] section 8.3.1).

    Returns (P, m, l): m is the row max, l = sum_j exp(S_ij - m_i) and
    P = exp(S - m) / l.  Rows that are all -inf give P = 0, m = -inf, l = 0.
    """
    m = S.max(axis=1, initial=NEG_INF)
    has_key = np.isfinite(m)
    E = np.zeros_like(S)
    E[has_key] = np.exp(S[has_key] - m[has_key, None])
    l = E.sum(axis=1)
    P = np.zeros_like(S)
    P[has_key] = E[has_key] / l[has_key, None]
    return P, m, l


def _heads(shape):
    return list(np.ndindex(*shape[:-2]))


def ref_probs(q, k, scale, causal=False, q_pos=None):
    """The attention probability matrix P = softmax(scale Q K^T) per head."""
    q, k = _f64(q), _f64(k)
    Nq = q.shape[-2]
    q_pos = np.arange(Nq) if q_pos is None else np.asarray(q_pos)
    P = np.zeros(q.shape[:-1] + (k.shape[-2],))
    for h in _heads(q.shape):
        P[h], _, _ = _softmax_rows(_scores(q[h], k[h], scale, causal, q_pos))
    return P


def ref_fwd(q, k, v, scale, causal=False, q_pos=None):
    """Naive three-step attention: S, then P = softmax(S), then O = P V.

    Follows the definition in [xuesongtap] section 1 and the naive
    implementation of [Triton-ch8] section 8.1, with the LSE of
    [xuesongtap] section 3.  Returns (O [..., Nq, dv], LSE [..., Nq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Nq = q.shape[-2]
    q_pos = np.arange(Nq) if q_pos is None else np.asarray(q_pos)
    O = np.zeros(q.shape[:-1] + (v.shape[-1],))
    LSE = np.full(q.shape[:-1], NEG_INF)
    for h in _heads(q.shape):
        P, m, l = _softmax_rows(_scores(q[h], k[h], scale, causal, q_pos))
        O[h] = P @ v[h]
        has_key = l > 0
        LSE[h][has_key] = m[has_key] + np.log(l[has_key])
    return O, LSE


def ref_bwd(q, k, v, dO, scale, causal=False, q_pos=None):
    """Gradients of O = softmax(scale Q K^T) V with respect to Q, K and V.

    P is rebuilt from Q and K (never from a saved LSE).  The formulas are
    those of [Triton-ch8] sections 8.8.1 and 8.8.3 and [operatorworld]
    (backward by recomputation):

        dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
        dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.

    The Greek letter multiplying dS K and dS^T Q on the tutorial page is the
    softmax scale (its kernel multiplies dq and dk by sm_scale in 8.8.4).
    Returns (dQ, dK, dV).
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    Nq = q.shape[-2]
    q_pos = np.arange(Nq) if q_pos is None else np.asarray(q_pos)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in _heads(q.shape):
        P, _, _ = _softmax_rows(_scores(q[h], k[h], scale, causal, q_pos))
        dV[h] = P.T @ dO[h]
        dP = dO[h] @ v[h].T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        dQ[h] = scale * (dS @ k[h])
        dK[h] = scale * (dS.T @ q[h])
    return dQ, dK, dV


def online_softmax_step(m_old, l_old, U_old, S_blk, V_blk):
    """One inner-loop update of the running state (m, l, U) for a key block.

    [xuesongtap] section 2.2 / [operatorworld] / [Triton-ch8] section 8.3.3:

        m_new = max(m_old, rowmax(S_blk))
        alpha = exp(m_old - m_new)         (0 while m_old is still -inf)
        P~    = exp(S_blk - m_new)
        l_new = alpha * l_old + rowsum(P~)
        U_new = alpha * U_old + P~ V_blk

    A row whose entries so far are all -inf keeps m = -inf, l = 0, U = 0
    (the invalid difference -inf - (-inf) is never formed).
    Returns (m_new, l_new, U_new, alpha).
    """
    m_new = np.maximum(m_old, S_blk.max(axis=1))
    alpha = np.zeros_like(m_old)
    seen = np.isfinite(m_old)
    alpha[seen] = np.exp(m_old[seen] - m_new[seen])
    base = np.where(np.isfinite(m_new), m_new, 0.0)
    P_blk = np.exp(S_blk - base[:, None])
    l_new = alpha * l_old + P_blk.sum(axis=1)
    U_new = alpha[:, None] * U_old + P_blk @ V_blk
    return m_new, l_new, U_new, alpha


def ref_blockwise_fwd(q, k, v, scale, causal, Br, Bc, trace=False):
    """FA-2 loop order: outer loop over Br-row query blocks, inner loop over
    Bc-row key/value blocks, unnormalised U divided by l once at the end
    ([xuesongtap] sections 2.1-2.2; [cnblogs] section 1 pseudocode).

    Returns (O, LSE) or, with ``trace``, (O, LSE, trace) where
    trace[head][(i0, j0)] = (m, l, alpha) after the block at rows i0 and
    keys j0.  It exists to pin the online algebra; ref_fwd is the authority.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Nq, Nk = q.shape[-2], k.shape[-2]
    O = np.zeros(q.shape[:-1] + (v.shape[-1],))
    LSE = np.full(q.shape[:-1], NEG_INF)
    traces = {}
    for h in _heads(q.shape):
        tr = {}
        for i0 in range(0, Nq, Br):
            rows = np.arange(i0, min(i0 + Br, Nq))
            Qi = q[h][rows]
            m = np.full(len(rows), NEG_INF)
            l = np.zeros(len(rows))
            U = np.zeros((len(rows), v.shape[-1]))
            for j0 in range(0, Nk, Bc):
                cols = np.arange(j0, min(j0 + Bc, Nk))
                S = scale * (Qi @ k[h][cols].T)
                if causal:
                    S = np.where(cols[None, :] <= rows[:, None], S, NEG_INF)
                m, l, U, alpha = online_softmax_step(m, l, U, S, v[h][cols])
                if trace:
                    tr[(i0, j0)] = (m.copy(), l.copy(), alpha.copy())
            has_key = l > 0
            O[h][rows[has_key]] = U[has_key] / l[has_key, None]
            LSE[h][rows[has_key]] = m[has_key] + np.log(l[has_key])
        traces[h] = tr
    if trace:
        return O, LSE, traces
    return O, LSE


def decode_chunk_bounds(L, num_splits):
    """Chunk c of a length-L cache covers keys [floor(cL/S), floor((c+1)L/S)).

    The pages split the cache into blocks without fixing the rule for
    L % S != 0; with S > L some chunks are empty.
    """
    return [((c * L) // num_splits, ((c + 1) * L) // num_splits) for c in range(num_splits)]


def ref_decode_partials(q, k, v, scale, num_splits):
    """Map step of FlashDecoding ([cnblogs] section 3 scenario B, step 2):
    for each chunk c of the cache, the unnormalised partial state
    ([FA1-vs-FA2] section 6)

        m_c = max_j s_j,  l_c = sum_j exp(s_j - m_c),
        U_c = sum_j exp(s_j - m_c) V_j,      s = scale K_c q.

    q: [..., 1, d]; k, v: [..., L, d].  Returns (U [..., S, dv], m [..., S],
    l [..., S]); an empty chunk gives U = 0, m = -inf, l = 0.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    L = k.shape[-2]
    bounds = decode_chunk_bounds(L, num_splits)
    lead = q.shape[:-2]
    U = np.zeros(lead + (num_splits, v.shape[-1]))
    m = np.full(lead + (num_splits,), NEG_INF)
    l = np.zeros(lead + (num_splits,))
    for h in np.ndindex(*lead):
        qv = q[h][0]
        for c, (lo, hi) in enumerate(bounds):
            if hi == lo:
                continue
            s = scale * (k[h][lo:hi] @ qv)
            m[h][c] = s.max()
            p = np.exp(s - m[h][c])
            l[h][c] = p.sum()
            U[h][c] = p @ v[h][lo:hi]
    return U, m, l


def merge_two(a, b):
    """Merge two partial states (U, m, l) into one ([FA1-vs-FA2] section 6):
    m = max(m_a, m_b), l = sum_w e^(m_w - m) l_w, U = sum_w e^(m_w - m) U_w.
    A state with m = -inf (an empty chunk) has weight 0."""
    Ua, ma, la = a
    Ub, mb, lb = b
    m = max(ma, mb)
    if m == NEG_INF:
        return np.zeros_like(Ua), NEG_INF, 0.0
    wa = 0.0 if ma == NEG_INF else np.exp(ma - m)
    wb = 0.0 if mb == NEG_INF else np.exp(mb - m)
    return wa * Ua + wb * Ub, m, wa * la + wb * lb


def merge_partials_tree(U, m, l):
    """Reduce step of FlashDecoding: merge the per-chunk states pairwise in a
    tree ([cnblogs] section 3 scenario B, step 3), then O = U / l and
    LSE = m + ln l.  U: [S, dv]; m, l: [S].  Returns (O [dv], LSE)."""
    states = [(U[c], m[c], l[c]) for c in range(len(m))]
    while len(states) > 1:
        nxt = [merge_two(states[i], states[i + 1]) for i in range(0, len(states) - 1, 2)]
        if len(states) % 2:
            nxt.append(states[-1])
        states = nxt
    Uf, mf, lf = states[0]
    if lf == 0:
        return np.zeros_like(Uf), NEG_INF
    return Uf / lf, mf + np.log(lf)


def ref_splitk_decode(q, k, v, scale, num_splits):
    """Split-K decode: per-chunk partials, then the pairwise merge.

    q: [..., 1, d]; k, v: [..., L, d].  Returns (O [..., 1, dv],
    LSE [..., 1]).  The definition it must equal is ref_fwd with one query
    row that sees every key.
    """
    U, m, l = ref_decode_partials(q, k, v, scale, num_splits)
    lead = U.shape[:-2]
    O = np.zeros(lead + (1, U.shape[-1]))
    LSE = np.full(lead + (1,), NEG_INF)
    for h in np.ndindex(*lead):
        O[h][0], LSE[h][0] = merge_partials_tree(U[h], m[h], l[h])
    return O, LSE


def gather_paged_rows(pool, block_table, seq_len, h):
    """Rows 0 .. seq_len-1 of head h of one sequence stored in a block pool.

    The pages name the paged block table as the KV-cache layout of decode
    kernels ([FA1-vs-FA2] section 13) without fixing it; the reading used
    here: the cache is a pool of fixed-size blocks, pool[blk, h, r, :] is row
    r of block blk for head h, and block_table[j] is the pool block holding
    the sequence's logical block j, so token t is row t % bs of block
    block_table[t // bs].  Returns [seq_len, d].
    """
    pool = _f64(pool)
    bs = pool.shape[2]
    rows = [pool[int(block_table[t // bs]), h, t % bs] for t in range(seq_len)]
    return np.array(rows).reshape(seq_len, pool.shape[3])


def ref_paged_decode(q, k_pool, v_pool, block_table, seq_lens, scale):
    """Decode of one query row per (b, h) against a paged KV cache.

    q: [B, H, 1, d]; k_pool, v_pool: [num_blocks, H, bs, d];
    block_table: [B, max_blocks]; seq_lens: [B].  For every (b, h) the
    sequence's keys and values are gathered through the block table and the
    result is plain attention of the single query over all of them (the
    query sees every key, as in the dense decode): (O [B, H, 1, d],
    LSE [B, H, 1]); a sequence of length 0 gives O = 0 and LSE = -inf.
    """
    q = _f64(q)
    B, H = q.shape[0], q.shape[1]
    O = np.zeros(q.shape[:-1] + (v_pool.shape[-1],))
    LSE = np.full(q.shape[:-1], NEG_INF)
    for b in range(B):
        n = int(seq_lens[b])
        for h in range(H):
            kb = gather_paged_rows(k_pool, block_table[b], n, h)
            vb = gather_paged_rows(v_pool, block_table[b], n, h)
            O[b, h], LSE[b, h] = ref_fwd(q[b, h], kb, vb, scale)
    return O, LSE



# ---------------------------------------------------------------------------
# FP8 (E4M3) forward ([Triton-ch8] section 8.9)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(x):
    """Round to the nearest FP8 E4M3 value, ties to even, for |x| <= 448.

    The format ([Triton-ch8] section 8.9.1: 4 exponent bits, 3 mantissa
    bits, largest finite value 448): exponent bias 7, normal values
    (1 + m/8) 2^(e-7) for e = 1..15, subnormals (m/8) 2^-6, so the spacing is
    2^(e-3) for a value in [2^e, 2^(e+1)) and 2^-9 below 2^-6.
    """
    x = _f64(x)
    a = np.abs(x)
    assert np.all(a <= E4M3_MAX), "e4m3_round expects clamped input"
    _, ex = np.frexp(a)                      # a = f 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # floor(log2 a), subnormal range at -6
    ulp = np.ldexp(1.0, e - 3)
    return np.sign(x) * np.round(a / ulp) * ulp   # a / ulp is exact; np.round ties to even


def hadamard_rotate(x, signs):
    """Incoherent processing ([Triton-ch8] section 8.9.5): x' = x D H / sqrt(d)
    with D = diag(signs) (random +-1, drawn by the caller) and H the Sylvester
    Hadamard matrix of order d (a power of two).  D H / sqrt(d) is
    orthogonal, so x' y'^T = x y^T."""
    x = _f64(x)
    d = x.shape[-1]
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == d, "d must be a power of two"
    return (x * _f64(signs)) @ H / np.sqrt(d)


def fp8_block_scale(amax):
    """A block's scale, max|x| / 448 ([Triton-ch8] section 8.9.4), evaluated
    in fp32 as the page's PyTorch code does (amax is an fp32 value; the
    quotient is IEEE fp32 division, correctly rounded).  An all-zero block,
    where the page's quotient would be 0 and x / scale undefined, gets 1 (any
    positive scale turns it into zero codes).  Returns a Python float holding
    the fp32 value."""
    a = np.float32(amax)
    if a == 0:
        return 1.0
    return float(a / np.float32(E4M3_MAX))


def quantize_fp8_blocks(x, block_rows, signs=None):
    """Per-block FP8 quantisation, the page's quantize_to_fp8 ([Triton-ch8]
    sections 8.9.3-8.9.4) with its block scales.

    x: [..., N, d] (values that fp32 holds exactly, e.g. bf16).  Rows are
    grouped into blocks of ``block_rows``; each block gets
    scale = fp8_block_scale(max|x|) and codes e4m3(clamp(x / scale, +-448)),
    x / scale divided in fp32 like the page's tensor code.  With ``signs``
    the rows are first rotated by hadamard_rotate and rounded to fp32 (the
    precision the values are held in before the division).  Returns
    (values [..., N, d] float64 -- the e4m3 values, exactly --,
    scales [..., ceil(N / block_rows)] -- fp32 values held in float64).
    """
    x = _f64(x)
    if signs is not None:
        x = hadamard_rotate(x, signs)
    x32 = x.astype(np.float32)
    N = x.shape[-2]
    nb = -(-N // block_rows)
    vals = np.zeros(x.shape)
    scales = np.zeros(x.shape[:-2] + (nb,))
    for idx in np.ndindex(*x.shape[:-2]):
        for b in range(nb):
            blk = x32[idx][b * block_rows:(b + 1) * block_rows]
            s = fp8_block_scale(np.max(np.abs(blk)))
            y = (blk / np.float32(s)).astype(np.float64)     # fp32 quotient
            vals[idx][b * block_rows:(b + 1) * block_rows] = e4m3_round(np.clip(y, -E4M3_MAX, E4M3_MAX))
            scales[idx][b] = s
    return vals, scales


def _rows_of_blocks(scales, block_rows, N):
    """Per-row copy of per-block scales: [..., nb] -> [..., N]."""
    return np.repeat(_f64(scales), block_rows, axis=-1)[..., :N]


def ref_fwd_fp8(q8, k8, v8, sq, sk, sv, scale, causal=False, block_m=32, block_n=64, trace=False):
    """FP8 attention forward, the method of [Triton-ch8] sections 8.9.3-8.9.4
    and the fa3_fp8_inner listing of section 8.9.6, in fp64.

    q8, k8, v8: [..., N, d] E4M3 values; sq: Q block scales [..., ceil(N /
    block_m)]; sk, sv: K and V block scales [..., ceil(N / block_n)]
    (dequantised value = E4M3 value x its block's scale).  Query rows are
    processed in blocks of block_m (the listing's BLOCK_M), keys in blocks of
    block_n (BLOCK_N), with the online state (m, l, acc) per row.  For each
    (query block, key block) that holds a visible pair:

        qk    = (q8 k8^T) sq sk scale               (masked to -inf if causal)
        m_new = max(m, rowmax(qk)),   alpha = e^(m - m_new)
        p     = e^(qk - m_new),       l = alpha l + rowsum(p)
        scale_p = max(p) / 448        (over the whole block: all its rows
                                       below N and all its keys)
        p8    = e4m3(p / scale_p)     (P requantised to FP8)
        acc   = alpha acc + (p8 v8) scale_p sv

    then O = acc / l and LSE = m + ln l.  The listing multiplies the whole
    accumulator by scale_p scale_v after adding the block's product; that is
    read as scaling the block's product only (the other reading mixes the
    scales of different blocks).  p / scale_p is evaluated as
    448 e^(qk - m_new - ln max(p)), which is the same number without the
    underflow of a block whose p are all far below the running max (such a
    block then adds scale_p ~ 0 times its product, as in fp32).  Blocks with
    no visible pair are skipped (their p would all be 0).

    Returns (O [..., N, dv], LSE [..., N]).  With ``trace`` it also returns
    Y, W [..., N, Nk]: Y the value each p8 was rounded from (p / scale_p;
    NaN where a key is masked or its block skipped) and W the weight of one
    unit of p8 in the final O, scale_p sv e^(m_new - m_final) / l_final, so
    that O = sum_j e4m3(Y_ij) W_ij v8_j.
    """
    q8, k8, v8 = _f64(q8), _f64(k8), _f64(v8)
    N, Nk = q8.shape[-2], k8.shape[-2]
    O = np.zeros(q8.shape[:-1] + (v8.shape[-1],))
    LSE = np.full(q8.shape[:-1], NEG_INF)
    Y = np.full(q8.shape[:-1] + (Nk,), np.nan) if trace else None
    W = np.zeros(q8.shape[:-1] + (Nk,)) if trace else None
    for h in _heads(q8.shape):
        sqr = _rows_of_blocks(sq[h], block_m, N)
        for i0 in range(0, N, block_m):
            i1 = min(i0 + block_m, N)
            rows = np.arange(i0, i1)
            m = np.full(i1 - i0, NEG_INF)
            l = np.zeros(i1 - i0)
            acc = np.zeros((i1 - i0, v8.shape[-1]))
            blocks = []  # (key range, Y, unit weight before the final rescale, m_new)
            for j0 in range(0, Nk, block_n):
                j1 = min(j0 + block_n, Nk)
                jb = j0 // block_n
                qk = (q8[h][i0:i1] @ k8[h][j0:j1].T) * sqr[i0:i1, None] * float(sk[h][jb]) * scale
                if causal:
                    qk = np.where(np.arange(j0, j1)[None, :] > rows[:, None], NEG_INF, qk)
                vis = np.isfinite(qk)
                if not vis.any():
                    continue
                m_new = np.maximum(m, np.max(qk, axis=1))
                alpha = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(m_new), m_new, 0.0)), 0.0)
                lp = np.where(vis, qk - np.where(np.isfinite(m_new), m_new, 0.0)[:, None], NEG_INF)  # ln p
                p = np.exp(lp)
                l = alpha * l + p.sum(axis=1)
                lpmax = np.max(lp)                      # ln max(p), finite: the block has a visible pair
                scale_p = np.exp(lpmax) / E4M3_MAX
                y = np.where(vis, E4M3_MAX * np.exp(lp - lpmax), 0.0)   # p / scale_p, in [0, 448]
                p8 = e4m3_round(y)
                f = scale_p * float(sv[h][jb])
                acc = alpha[:, None] * acc + (p8 @ v8[h][j0:j1]) * f
                m = m_new
                blocks.append((j0, j1, np.where(vis, y, np.nan), f, m_new.copy()))
            has = l > 0
            O[h][i0:i1] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
            LSE[h][i0:i1] = np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)
            if trace:
                for j0, j1, y, f, mb in blocks:
                    Y[h][i0:i1, j0:j1] = y
                    w = f * np.exp(np.where(np.isfinite(mb), mb - m, 0.0)) / np.where(has, l, 1.0)
                    W[h][i0:i1, j0:j1] = np.where(has & np.isfinite(mb), w, 0.0)[:, None]
    if trace:
        return O, LSE, Y, W
    return O, LSE


# ---------------------------------------------------------------------------
# Merging results over disjoint key sets (Ring Attention's per-step update)
# ---------------------------------------------------------------------------

def ref_merge_lse(o_a, lse_a, o_b, lse_b):
    """Attention over keys A u B from the results over A and over B alone.

    The partial-state merge of [FA1-vs-FA2] section 6 written for normalised
    outputs: with L = log(e^LSE_a + e^LSE_b), O = e^(LSE_a - L) O_a +
    e^(LSE_b - L) O_b and LSE = L.  This is the update each arriving K/V
    shard makes in Ring Attention ([xuesongtap] section 5; [cnblogs]
    section 3 scenario A).  A side with LSE = -inf (no keys) has weight 0
    and contributes nothing whatever its O holds; both empty give O = 0,
    LSE = -inf.  o: [..., N, d]; lse: [..., N].
    """
    o_a, o_b = _f64(o_a), _f64(o_b)
    la, lb = _f64(lse_a), _f64(lse_b)
    m = np.maximum(la, lb)
    base = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(la), np.exp(la - base), 0.0)
    wb = np.where(np.isfinite(lb), np.exp(lb - base), 0.0)
    tot = wa + wb
    safe = np.where(tot > 0, tot, 1.0)
    ta = np.where(wa[..., None] > 0, wa[..., None] * o_a, 0.0)
    tb = np.where(wb[..., None] > 0, wb[..., None] * o_b, 0.0)
    O = (ta + tb) / safe[..., None]
    L = np.where(tot > 0, base + np.log(safe), NEG_INF)
    return O, L
