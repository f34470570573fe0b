"""CPU oracle for the rest of the Quant Experts calibration statistic: the frequency
partition of the important channels and the co-occurrence clustering of the
token-dependent ones.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark may import this module; the product
path (the HIP library and its Python binding) never does, and the two share no code.

Sources (the pages; cited by title and section):
  [DeepRead]   MCISLAB DeepRead summary "Quant Experts: Token-aware Adaptive Error
               Reconstruction with Mixture of Experts for Large Vision-Language Models
               Quantization", section "Method" (frequency partition: first k channels
               token-independent, the next N_r*k token-dependent; co-occurrence matrix of
               the token-dependent channels, NPMI similarity, spectral clustering on the
               normalized Laplacian, K-Means into N_r clusters).
  [PaperDaily] longzhangge PaperDaily post "西交大提出Quant Experts：token级量化补偿",
               section "核心设计：共享专家先保底，路由专家再补局部误差" (O_{t,i}: whether
               token t selects token-dependent channel i; the C x C co-occurrence counts;
               p(i), p(i,j) and the NPMI similarity in [-1, 1]; a threshold such as 0.2
               drops weak pairs).
  [listing]    thelatestinai.com listing of arXiv 2602.24059, Figure 6 (the similarity
               matrix S of the token-dependent channels and its clusters).

Precision: counts are exact integers; every floating-point step is float64.  A library
primitive serves for the symmetric eigendecomposition (numpy.linalg.eigh) and for the
integer product O^T O.

Readings of open points (each also listed in the design notes):
  * Frequency order: selection count descending, channel index ascending on ties.
  * p(i) = C_ii / T and p(i, j) = C_ij / T over the T calibration tokens.
  * NPMI(i, j) = ln(p(i,j) / (p(i) p(j))) / (-ln p(i,j)); -1 when p(i,j) = 0 (never
    together) and +1 when p(i,j) = 1 (always together, the limit of the formula).  The
    same formula on the diagonal gives +1 for a channel that occurs, -1 for one that never
    does.
  * Threshold: S_ij = NPMI(i,j) where NPMI(i,j) >= tau, else 0 (tau >= 0; default 0.2).
  * Spectral clustering follows the normalized-Laplacian algorithm of Ng, Jordan and
    Weiss (2001): d_i = sum_j S_ij, L = I - D^-1/2 S D^-1/2 (a row and column of zeros
    in D^-1/2 S D^-1/2 where d_i = 0), the eigenvectors of the n smallest eigenvalues of L
    as columns of U, each row of U scaled to unit length (zero rows stay zero).
  * K-Means (Lloyd) on the rows of U, seeded without randomness by farthest-point
    (maximin) selection starting from row 0 (the most frequent token-dependent channel);
    points go to the nearest centroid, the lower cluster on ties; a centroid is the mean
    of its points and an empty cluster keeps its centroid; iterate until no point moves.
    Labels are then renumbered in order of each cluster's lowest member.

Parity-pinned: every function is pinned by tests/test_oracle_calib.py (hand-worked
partitions and NPMI values, brute-force counting, spectral facts of disconnected and
connected graphs, planted partitions recovered exactly).
"""

from typing import Tuple

import numpy as np


def frequency_partition(hist: np.ndarray, k: int, n_r: int) -> Tuple[np.ndarray, np.ndarray]:
    """[DeepRead] "Method": order the channels by how often the calibration tokens select
    them; the first k are token-independent, the following n_r*k token-dependent.

    hist: selection counts per input channel.  Returns (indep int32 [k], dep int32 [n_r*k]).
    """
    h = np.asarray(hist, np.int64)
    d = h.shape[0]
    if k + n_r * k > d:
        raise ValueError("k + n_r*k exceeds the channel count")
    order = np.lexsort((np.arange(d), -h))
    return order[:k].astype(np.int32), order[k:k + n_r * k].astype(np.int32)


def occurrence(topk: np.ndarray, dep: np.ndarray, d_in: int) -> np.ndarray:
    """[PaperDaily] "核心设计": O[t, i] = 1 when token t's important channels include the
    i-th token-dependent channel, else 0.  topk: int [T, k] channel indices per token."""
    topk = np.asarray(topk, np.int64)
    T = topk.shape[0]
    C = len(dep)
    position = np.full(d_in, -1, np.int64)  # channel -> its index among the token-dependent ones
    position[np.asarray(dep, np.int64)] = np.arange(C)
    O = np.zeros((T, C), np.int64)
    p = position[topk]
    t_idx = np.broadcast_to(np.arange(T)[:, None], p.shape)
    sel = p >= 0
    O[t_idx[sel], p[sel]] = 1
    return O


def cooccurrence(topk: np.ndarray, dep: np.ndarray, d_in: int) -> np.ndarray:
    """[PaperDaily] "核心设计": C[i, j] = number of tokens whose important channels include
    both token-dependent channels i and j, i.e. C = O^T O.  int64 [C, C]."""
    O = occurrence(topk, dep, d_in)
    return O.T @ O


def npmi(cooc: np.ndarray, T: int) -> np.ndarray:
    """[PaperDaily] "核心设计": p(i) = C_ii/T, p(i,j) = C_ij/T and
    NPMI(i,j) = ln(p(i,j) / (p(i) p(j))) / (-ln p(i,j)), in [-1, 1];
    -1 where p(i,j) = 0, +1 where p(i,j) = 1.  float64 [C, C]."""
    Cm = np.asarray(cooc, np.float64)
    if T <= 0:
        raise ValueError("T must be positive")
    p = np.diag(Cm) / T
    out = np.empty_like(Cm)
    n = Cm.shape[0]
    for i in range(n):
        for j in range(n):
            pij = Cm[i, j] / T
            if Cm[i, j] == 0:
                out[i, j] = -1.0
            elif Cm[i, j] == T:
                out[i, j] = 1.0
            else:
                out[i, j] = np.log(pij / (p[i] * p[j])) / (-np.log(pij))
    return out


def similarity(cooc: np.ndarray, T: int, threshold: float = 0.2) -> np.ndarray:
    """[PaperDaily] "核心设计": the NPMI similarity with weak pairs (below the threshold)
    set to zero; [listing] Figure 6 (a) shows this matrix."""
    if threshold < 0:
        raise ValueError("threshold must be >= 0")
    S = npmi(cooc, T)
    return np.where(S >= threshold, S, 0.0)


def spectral_embedding(S: np.ndarray, n_clusters: int) -> Tuple[np.ndarray, np.ndarray]:
    """[DeepRead] "Method": spectral clustering on the normalized Laplacian.

    L = I - D^-1/2 S D^-1/2 with d_i = sum_j S_ij; U = eigenvectors of the n_clusters
    smallest eigenvalues of L, rows scaled to unit length.  Returns (U [C, n], the
    n_clusters smallest eigenvalues ascending)."""
    S = np.asarray(S, np.float64)
    n = S.shape[0]
    deg = S.sum(axis=1)
    inv_sqrt = np.zeros(n)
    pos = deg > 0
    inv_sqrt[pos] = 1.0 / np.sqrt(deg[pos])
    L = np.eye(n) - inv_sqrt[:, None] * S * inv_sqrt[None, :]
    w, V = np.linalg.eigh(L)  # ascending eigenvalues
    U = V[:, :n_clusters].copy()
    norms = np.sqrt((U * U).sum(axis=1))
    nz = norms > 0
    U[nz] /= norms[nz, None]
    return U, w[:n_clusters]


def kmeans(U: np.ndarray, n_clusters: int, max_iter: int = 300) -> np.ndarray:
    """[DeepRead] "Method": K-Means into n_clusters groups (Lloyd's iteration).

    Seeding: row 0, then repeatedly the row farthest (squared Euclidean) from the chosen
    centroids, the lowest row on ties.  Returns labels int32 [C], renumbered so that
    clusters appear in order of their lowest member."""
    U = np.asarray(U, np.float64)
    n = U.shape[0]
    if not 1 <= n_clusters <= n:
        raise ValueError("need 1 <= n_clusters <= rows")
    chosen = [0]
    dmin = ((U - U[0]) ** 2).sum(axis=1)
    while len(chosen) < n_clusters:
        nxt = int(np.argmax(dmin))  # first maximum: the lowest row on ties
        chosen.append(nxt)
        dmin = np.minimum(dmin, ((U - U[nxt]) ** 2).sum(axis=1))
    cent = U[chosen].copy()
    labels = np.full(n, -1, np.int64)
    for _ in range(max_iter):
        dist = ((U[:, None, :] - cent[None, :, :]) ** 2).sum(axis=2)
        new = np.argmin(dist, axis=1)  # first minimum: the lower cluster on ties
        if np.array_equal(new, labels):
            break
        labels = new
        for c in range(n_clusters):
            members = labels == c
            if members.any():
                cent[c] = U[members].mean(axis=0)
    return canonical_labels(labels)


def canonical_labels(labels: np.ndarray) -> np.ndarray:
    """Renumber cluster ids in order of first appearance (lowest member first)."""
    labels = np.asarray(labels)
    mapping = {}
    out = np.empty(labels.shape[0], np.int32)
    for i, l in enumerate(labels):
        if int(l) not in mapping:
            mapping[int(l)] = len(mapping)
        out[i] = mapping[int(l)]
    return out


def cluster_channels(cooc: np.ndarray, T: int, n_clusters: int, threshold: float = 0.2):
    """[DeepRead] "Method" + [PaperDaily] "核心设计": NPMI similarity -> normalized-Laplacian
    spectral embedding -> K-Means.  Returns (labels int32 [C], S, U, eigenvalues)."""
    S = similarity(cooc, T, threshold)
    U, w = spectral_embedding(S, n_clusters)
    return kmeans(U, n_clusters), S, U, w
