"""CPU oracle for the GQA -> SAGA key-head merge (fp64 numpy).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module. The product path never does.

Source: "More Value per Key: Asymmetric Sparse Attention for Faster LLM
Decoding", §4 (merging key heads of a GQA teacher), Eqs. 11-18, Lemma 4.1
with its proof in App. A (Eqs. 19-27), Theorem 4.2, and the induced
permutations of App. B (Eqs. 28-34). Notation as there:
  X [L][D]       hidden states of L calibration tokens;
  W_K^r [D][d]   teacher key projection r, r = 0 .. h_kt - 1 (h_kt = 2 h_k^S);
  W_Q^j [D][d]   query projection j; Q^j = X W_Q^j are the realized queries;
  Q_r            the g = h_q / h_kt query heads j = r g .. r g + g - 1 that
                 share key head r (the blocks B_r of App. B);
  S_r            sum over j in Q_r of (Q^j)^T Q^j (Eq. 21);
  L_{a,b}(M)     sum over r in {a, b}, j in Q_r of
                 ||Q^j (X M)^T - Q^j (X W_K^r)^T||_F^2 (Eq. 13, the 1/sqrt(d)
                 factor dropped as there);
  M(a, b)        (W_K^a S_a + W_K^b S_b)(S_a + S_b)^+ (Eq. 15);
  w(a, b)        L_{a,b}(M(a, b)) (Eq. 16); the pairing is a minimum-weight
                 perfect matching of the complete graph on the h_kt heads
                 (Theorem 4.2).

Array layouts follow the usual linear-layer storage [out features][in
features]: Wq [h_q*d][D], Wk [h_kt*d][D], Wv [h_kt*d][D] (row block r is
(W^r)^T), Wo [D][h_q*d] (column block j is W_O,j^T). Inputs are float32 or
uint16 bf16 bit patterns, decoded exactly to fp64.

Readings where the pages leave a step open:
  - Moore-Penrose pseudo-inverse of the symmetric PSD matrix S_a + S_b from
    its eigen-decomposition, eigenvalues at or below PINV_REL * d * lambda_max
    counted as zero (PINV_REL = 2^-23: the statistics a production path
    accumulates in fp32 resolve no finer);
  - equal-weight matchings: the first in the order that pairs the lowest
    unmatched head first, with its lowest-numbered partner first;
  - sigma lists the matched pairs by their lower head, each as (lower,
    higher); merged head i is pair i.
"""
from __future__ import annotations

import numpy as np

PINV_REL = 2.0 ** -23


def f64(a):
    """float32 or bf16 bit patterns (uint16) -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def head_projection(W, r, d):
    """W^r as a [D][d] matrix from the [heads*d][D] storage."""
    return f64(W)[r * d:(r + 1) * d, :].T


def realized(X, W, heads, d):
    """[X W^h for each head h] ([L][d] each; Q^j = X W_Q^j for query heads)."""
    XW = f64(X) @ f64(W).T
    return [XW[:, h * d:(h + 1) * d] for h in range(heads)]


def query_stats(X, Wq, h_q, h_kt, d):
    """S [h_kt][d][d]: S_r = sum_{j in Q_r} (Q^j)^T Q^j (Eq. 21)."""
    g = h_q // h_kt
    Q = realized(X, Wq, h_q, d)
    return np.stack([sum(Q[j].T @ Q[j] for j in range(r * g, (r + 1) * g))
                     for r in range(h_kt)])


def key_gram(X, Wk):
    """(X W_K)^T (X W_K) over all teacher key heads, [h_kt*d][h_kt*d]: the Gram
    of the realized keys, in which the trace form of Eq. 23 is evaluated once
    X^T X is contracted with the key projections."""
    K = f64(X) @ f64(Wk).T
    return K.T @ K


def pinv_psd(P, d):
    """Moore-Penrose pseudo-inverse of a symmetric PSD matrix (eigenvalue cutoff
    PINV_REL * d * lambda_max)."""
    lam, V = np.linalg.eigh(P)
    cut = PINV_REL * d * max(float(lam.max()), 0.0)
    inv = np.where(lam > cut, 1.0 / np.where(lam > cut, lam, 1.0), 0.0)
    return (V * inv) @ V.T


def merged_projection(Wk, S, a, b, d):
    """Eq. 15: (W_K^a S_a + W_K^b S_b)(S_a + S_b)^+ as a [D][d] matrix."""
    Wa, Wb = head_projection(Wk, a, d), head_projection(Wk, b, d)
    return (Wa @ S[a] + Wb @ S[b]) @ pinv_psd(S[a] + S[b], d)


def pair_loss_trace(XtX, Wk, S, a, b, M, d):
    """Eq. 23: tr((M - W_a)^T X^T X (M - W_a) S_a) + (same for b)."""
    total = 0.0
    for r in (a, b):
        E = M - head_projection(Wk, r, d)
        total += float(np.trace(E.T @ XtX @ E @ S[r]))
    return total


def pair_loss_direct(X, Wq, Wk, h_q, h_kt, d, a, b, M):
    """Eq. 13 from its Frobenius norms of [L][L] logit differences (small L)."""
    g = h_q // h_kt
    X64 = f64(X)
    Q = realized(X, Wq, h_q, d)
    XM = X64 @ M
    total = 0.0
    for r in (a, b):
        XW = X64 @ head_projection(Wk, r, d)
        for j in range(r * g, (r + 1) * g):
            total += float(np.sum((Q[j] @ XM.T - Q[j] @ XW.T) ** 2))
    return total


def perfect_matchings(n):
    """Every perfect matching of heads 0 .. n-1 (n even) as a list of pairs
    (a, b), a < b: the lowest unmatched head is paired first, with its
    partners in increasing order."""
    def rec(rest):
        if not rest:
            yield []
            return
        a = rest[0]
        for i in range(1, len(rest)):
            for m in rec(rest[1:i] + rest[i + 1:]):
                yield [(a, rest[i])] + m
    return list(rec(list(range(n))))


def min_weight_matching(w):
    """Brute force over all perfect matchings: (pairs, total weight), the first
    minimum in perfect_matchings order (Theorem 4.2)."""
    best, best_w = None, None
    for m in perfect_matchings(w.shape[0]):
        tw = sum(w[a, b] for a, b in m)
        if best_w is None or tw < best_w:
            best, best_w = m, tw
    return best, best_w


def sigma_from_pairs(pairs):
    """sigma with consecutive entries the matched pairs (App. B)."""
    return [h for p in pairs for h in p]


def query_permutation(sigma, g):
    """pi_Q: the concatenation of the query blocks B_{sigma_1} .. (Eq. 30)."""
    return [s * g + t for s in sigma for t in range(g)]


def permute_heads(Wq, Wv, Wo, sigma, h_q, h_kt, d):
    """App. B, Eqs. 28-34: Wv's head blocks in sigma order, Wq's head blocks and
    Wo's column blocks in pi_Q order (storage layouts as in the module
    docstring; dtype kept)."""
    g = h_q // h_kt
    pq = query_permutation(sigma, g)
    Wq, Wv, Wo = np.asarray(Wq), np.asarray(Wv), np.asarray(Wo)
    wq = np.concatenate([Wq[j * d:(j + 1) * d] for j in pq], axis=0)
    wv = np.concatenate([Wv[r * d:(r + 1) * d] for r in sigma], axis=0)
    wo = np.concatenate([Wo[:, j * d:(j + 1) * d] for j in pq], axis=1)
    return wq, wv, wo


STRATEGIES = ("logit", "key", "sequential")


def key_weights(X, Wk, h_kt, d):
    """Eq. 35 (App. B.1, key matching): ||X W_K^a - X W_K^b||_F^2."""
    K = f64(X) @ f64(Wk).T
    w = np.zeros((h_kt, h_kt))
    for a in range(h_kt):
        for b in range(a + 1, h_kt):
            w[a, b] = w[b, a] = float(np.sum((K[:, a * d:(a + 1) * d] - K[:, b * d:(b + 1) * d]) ** 2))
    return w


def key_merge(X, Wq, Wk, h_q, h_kt, d, strategy="logit"):
    """The merge of §4 for one attention module, or one of the two other
    initialisations App. B.1 compares it with ("key": matching on Eq. 35 and
    the average of each pair; "sequential": heads (0, 1), (2, 3), .. averaged).
    Returns a dict:
      S          [h_kt][d][d]    query statistics (Eq. 21)
      H          [h_kt*d]^2      realized-key Gram
      w          [h_kt][h_kt]    the weights the matching ran on (Eq. 16 for
                                 "logit", Eq. 35 for "key", zeros for
                                 "sequential"), 0 on the diagonal
      pairs      matched pairs (a, b), a < b, by increasing a
      sigma      [h_kt]          consecutive matched pairs (App. B)
      objective  Eq. 14's objective for the pairs and merges returned (for
                 "logit" its minimum, Theorem 4.2)
      merged     [h_kt/2][d][D]  merged key projections in storage layout
                                 (M^T for pair i)"""
    assert h_kt % 2 == 0 and h_q % h_kt == 0 and strategy in STRATEGIES
    S = query_stats(X, Wq, h_q, h_kt, d)
    X64 = f64(X)
    XtX = X64.T @ X64
    w = np.zeros((h_kt, h_kt))
    Ms = {}
    for a in range(h_kt):
        for b in range(a + 1, h_kt):
            if strategy == "logit":
                Ms[(a, b)] = merged_projection(Wk, S, a, b, d)
                w[a, b] = w[b, a] = pair_loss_trace(XtX, Wk, S, a, b, Ms[(a, b)], d)
            else:
                Ms[(a, b)] = 0.5 * (head_projection(Wk, a, d) + head_projection(Wk, b, d))
    if strategy == "key":
        w = key_weights(X, Wk, h_kt, d)
    if strategy == "sequential":
        pairs = [(2 * i, 2 * i + 1) for i in range(h_kt // 2)]
    else:
        pairs, _ = min_weight_matching(w)
    objective = sum(pair_loss_trace(XtX, Wk, S, a, b, Ms[(a, b)], d) for a, b in pairs)
    return {"S": S, "H": key_gram(X, Wk), "w": w, "pairs": pairs,
            "sigma": sigma_from_pairs(pairs), "objective": objective,
            "merged": np.stack([Ms[p].T for p in pairs])}
