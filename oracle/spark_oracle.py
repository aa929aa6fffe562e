"""CPU oracle for SparK prefill pruning and decode attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it and
shares no code with it.

Plain NumPy, written for reading, not speed. Citations name the SparK
walkthrough page ("KV Cache 还能再砍一刀：SparK 在通道维度上做了一件被忽略多年的事",
ai-paper-analysis.pages.dev) by section and equation, and the AMD blog page
(bqwf.cn, "AAAI 2026 AMD论文Spark方法揭秘") by figure/table.

Precision: float64 everywhere except the two steps whose result decides an
integer (the channel mask). There the method's ranking is defined on fp32
values computed in a fixed order, so that a GPU can reproduce the mask bit for
bit:
  * channel energy A_j: a sequential fp32 sum of fl32(q^2) (exact squares of
    bf16 values) over the window rows, group head outer, window position inner;
  * saliency key: fl32(A_j * fl32(k^2)), one IEEE multiply.

Readings of points the pages leave open:
  * ||q^j||_2 is the L2 norm of channel j over the stacked window queries of
    all G query heads that share the KV head ("l2"); the walkthrough's
    mean-query proxy of section 3.2 is mode "mean" (A_j = m_j^2 with m_j the
    fp32 sum of the window queries; the 1/(GW)^2 factor does not change any
    ranking or recovery value and is omitted).
  * Ranking by w^2 = A_j k^2 instead of w = sqrt(A_j)|k|: same order in exact
    arithmetic, and needs no square root.
  * T = floor((1 - lambda) * D + 0.5) with lambda taken as an IEEE fp32 value.
  * Ties go to the lower channel index; kept values are packed in ascending
    channel order; mask word w bit b is channel 32w + b.
  * Recovery F default "mean_retained": per (batch, KV head, channel), the mean
    of the retained key values over all tokens (0 if none retained). The
    walkthrough's Degenerate F (section 3.3, F table) is "score_mean_pruned".
  * Decode: one new query per head attends to all S cached tokens (no causal
    mask), scale 1/sqrt(D), recovery only in the scores, V dense.
  * Cache growth (silent on the pages): generated keys are pruned with the
    prefill's A by the prefill's rule and appended; V dense; r fixed.
  * SparK-p (section 5.2): per token the fewest channels reaching p of the
    total saliency, decided in fp32 with a fixed pairwise summation tree;
    ties at the threshold kept together; ragged packed rows.
  * SparK-g (section 5.2): channel groups by channel energy rank (equal
    groups, most important first), per-group top-T_i by saliency key.
  * V-channel pruning (section 4.4, "norm-based"): per-token top-T_v of
    |v_tj|, ties to the lower channel, retained-mean recovery of V.
    Second reading of the same rule, the block mode: the channels fall into
    D/8 blocks of 8 consecutive channels, and per token the n_b blocks of
    largest squared L2 norm (fp32, summed in channel order) are kept, ties to
    the lower block; recovery as in the first reading.
  * Sampled F ("gaussian", "exponential", the other rows of the section 3.3 F
    table): mu and sigma are the mean and population standard deviation of
    the pruned saliency a_j |k_tj| per (batch, KV head); each pruned (t, j)
    draws its own w~ from a Philox4x32-10 stream keyed by a caller seed and
    counted by (t, j // 4, b * N_kv + h); Exp(1/mu) has mean mu.
    Parity unpinned against published generator test vectors (the pages hold
    none): the generator is pinned by its inverse, avalanche and uniformity,
    the transforms by their moments and the Box-Muller identity.
"""
from __future__ import annotations

import math

import numpy as np

QAGG_L2 = "l2"
QAGG_MEAN = "mean"

F_MEAN_RETAINED = "mean_retained"
F_ZERO = "zero"
F_CONST = "const"
F_SCORE_MEAN_PRUNED = "score_mean_pruned"
F_GAUSSIAN = "gaussian"
F_EXPONENTIAL = "exponential"
F_SAMPLED = (F_GAUSSIAN, F_EXPONENTIAL)


def num_kept(D: int, lam: float) -> int:
    """T = floor((1 - lambda) D + 0.5): channels kept per token.

    Walkthrough section 3.1 (the reduced objective keeps exactly T channels);
    lambda is the pruned fraction of key channels (AMD blog, Table 1 caption).
    lambda is rounded to fp32 first, as the C ABI receives it.
    """
    lam32 = float(np.float32(lam))
    if not (0.0 <= lam32 <= 1.0):
        raise ValueError("lambda must lie in [0, 1]")
    return int(math.floor((1.0 - lam32) * D + 0.5))


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def window_rows(q_win: np.ndarray, n_kv: int) -> np.ndarray:
    """Stack the window queries of each KV head's query group.

    q_win [B][N_q][W][D] -> [B][N_kv][G*W][D], row index g*W + w, where query
    head h*G + g reads KV head h.
    """
    B, Nq, W, D = q_win.shape
    G = Nq // n_kv
    return np.asarray(q_win).reshape(B, n_kv, G * W, D)


def chan_energy(q_win: np.ndarray, n_kv: int, qagg: str = QAGG_L2) -> np.ndarray:
    """A[b,h,j], the squared channel norm of the window queries (fp32, fixed order).

    Walkthrough section 3.1: saliency w = ||q^j||_2 ||k^j||_2; section 3.2 and
    its display equation: the queries of the last W positions stand in for
    the future queries.
    """
    rows = _f32(window_rows(q_win, n_kv))
    B, H, R, D = rows.shape
    acc = np.zeros((B, H, D), dtype=np.float32)
    if qagg == QAGG_L2:
        for i in range(R):            # sequential: row g*W + w in increasing order
            x = rows[:, :, i, :]
            acc = acc + x * x         # fp32: x*x exact for bf16 x, one rounding per add
        return acc
    if qagg == QAGG_MEAN:
        for i in range(R):
            acc = acc + rows[:, :, i, :]
        return acc * acc
    raise ValueError(qagg)


def saliency_keys(A: np.ndarray, k: np.ndarray) -> np.ndarray:
    """key[b,h,t,j] = fl32(A_j * fl32(k_tj^2)) = w^2 in fp32 (walkthrough section 3.1)."""
    k = _f32(k)
    return _f32(A)[:, :, None, :] * (k * k)


def select_top_t(keys: np.ndarray, T: int) -> np.ndarray:
    """Boolean mask of the T largest keys per token, ties to the lower channel.

    Walkthrough section 3.1: with the cross-channel terms dropped, the
    objective max sum_j w^j z^j subject to sum_j z^j = T is solved greedily
    by sorting the channels of each token.
    """
    order = np.argsort(-keys, axis=-1, kind="stable")
    mask = np.zeros(keys.shape, dtype=bool)
    np.put_along_axis(mask, order[..., :T], True, axis=-1)
    return mask


def mask_words(mask: np.ndarray) -> np.ndarray:
    """bool [..., D] -> uint32 [..., ceil(D/32)]; bit b of word w is channel 32w + b."""
    D = mask.shape[-1]
    nw = (D + 31) // 32
    if D != 32 * nw:
        mask = np.concatenate([mask, np.zeros(mask.shape[:-1] + (32 * nw - D,), bool)], axis=-1)
    m = mask.reshape(mask.shape[:-1] + (nw, 32)).astype(np.uint64)
    return (m << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)


def mask_from_words(words: np.ndarray, D: int) -> np.ndarray:
    """uint32 [..., ceil(D/32)] -> bool [..., D]."""
    w = np.asarray(words, dtype=np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
    return bits.reshape(w.shape[:-1] + (32 * w.shape[-1],))[..., :D].astype(bool)


def pack_kept(k: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Retained key values per token in ascending channel order: [..., T]."""
    T = int(mask[(0,) * (mask.ndim - 1)].sum()) if mask.size else 0
    kept = np.asarray(k)[mask]       # row-major: token by token, channel ascending
    return kept.reshape(mask.shape[:-1] + (T,))


def prune(q_win: np.ndarray, k: np.ndarray, n_kv: int, lam: float, qagg: str = QAGG_L2) -> dict:
    """Prefill pruning (walkthrough section 3.2, Fig. 3 prefill half).

    Returns A [B][N_kv][D] fp32, mask bool [B][N_kv][S][D], words uint32
    [B][N_kv][S][D/32] and packed [B][N_kv][S][T] (same dtype as k).
    """
    D = k.shape[-1]
    T = num_kept(D, lam)
    A = chan_energy(q_win, n_kv, qagg)
    mask = select_top_t(saliency_keys(A, k), T)
    return {"T": T, "A": A, "mask": mask, "words": mask_words(mask), "packed": pack_kept(k, mask)}


def stats(k: np.ndarray, mask: np.ndarray, A: np.ndarray, mode: str = F_MEAN_RETAINED,
          f_const: float = 0.01):
    """Recovery vector r [B][N_kv][D] (fp32) and retained count cnt (int32).

    Walkthrough section 3.3 step 1: prefill caches distribution statistics
    beside the pruned keys and the mask. ``k`` is the dense key tensor (only
    the retained entries are read, except by "score_mean_pruned", which needs
    the pruned ones).
      mean_retained:     r_j = mean of k_tj over tokens t that keep j (0 if none)
      zero / const:      the naive fills of section 3.3 (0 and a constant)
      score_mean_pruned: section 3.3 steps 1-4 with the Degenerate F:
                         mu = mean over pruned (t, j) of a_j |k_tj|, a_j = sqrt(A_j);
                         the back-solved key is mu / a_j (0 if a_j = 0).
      gaussian, exponential: the sampled F of the section 3.3 F table; the
                         statistics of step 1 are mu and sigma (population
                         standard deviation) of the pruned saliency a_j |k_tj|
                         per (batch, KV head), stored as r[..., 0] = mu,
                         r[..., 1] = sigma, the other entries 0. The samples
                         themselves are drawn at decode (decode_attn_sampled).
    """
    k64 = np.asarray(k, dtype=np.float64)
    cnt = mask.sum(axis=2).astype(np.int32)
    B, H, S, D = k64.shape
    if mode == F_MEAN_RETAINED:
        s = np.where(mask, k64, 0.0).sum(axis=2)
        r = np.where(cnt > 0, s / np.maximum(cnt, 1), 0.0)
    elif mode == F_ZERO:
        r = np.zeros((B, H, D))
    elif mode == F_CONST:
        r = np.full((B, H, D), float(np.float32(f_const)))
    elif mode == F_SCORE_MEAN_PRUNED:
        a = np.sqrt(np.asarray(A, dtype=np.float64))                    # [B][H][D]
        w = np.abs(k64) * a[:, :, None, :]
        npruned = (~mask).sum(axis=(2, 3))
        mu = np.where(npruned > 0, np.where(~mask, w, 0.0).sum(axis=(2, 3)) / np.maximum(npruned, 1), 0.0)
        r = np.where(a > 0, mu[:, :, None] / np.where(a > 0, a, 1.0), 0.0)
    elif mode in F_SAMPLED:
        a = np.sqrt(np.asarray(A, dtype=np.float64))
        w = np.abs(k64) * a[:, :, None, :]
        pr = ~mask
        npruned = pr.sum(axis=(2, 3))
        n1 = np.maximum(npruned, 1)
        mu = np.where(npruned > 0, np.where(pr, w, 0.0).sum(axis=(2, 3)) / n1, 0.0)
        m2 = np.where(npruned > 0, np.where(pr, w * w, 0.0).sum(axis=(2, 3)) / n1, 0.0)
        sigma = np.sqrt(np.maximum(m2 - mu * mu, 0.0))
        r = np.zeros((B, H, D))
        r[:, :, 0] = mu
        r[:, :, 1] = sigma
    else:
        raise ValueError(mode)
    return r.astype(np.float32), cnt


def expand_keys(packed: np.ndarray, mask: np.ndarray, r: np.ndarray) -> np.ndarray:
    """K_hat = mask ? stored value : r_j, in float64 (walkthrough section 3.3, Fig. 3 decode half)."""
    khat = np.broadcast_to(np.asarray(r, dtype=np.float64)[:, :, None, :], mask.shape).copy()
    khat[mask] = np.asarray(packed, dtype=np.float64).reshape(-1)
    return khat


def _attend(q: np.ndarray, keys: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query per head over all cached tokens, float64.

    q [B][N_q][D], keys/v [B][N_kv][S][D]; query head i reads KV head i // G.
    """
    q = np.asarray(q, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Nq, D = q.shape
    Nkv = keys.shape[1]
    G = Nq // Nkv
    out = np.empty((B, Nq, D), dtype=np.float64)
    for b in range(B):
        for i in range(Nq):
            h = i // G
            s = (keys[b, h] @ q[b, i]) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, i] = p @ v[b, h]
    return out


def decode_attn(q, packed, mask, v, r, scale: float | None = None) -> np.ndarray:
    """One decode step over the pruned cache: recover, then standard attention.

    Walkthrough section 3.3 and Fig. 3 (decode half); AMD blog Fig. 2.
    Returns out [B][N_q][D] in float64.
    """
    D = mask.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    return _attend(q, expand_keys(packed, mask, r), v, scale)


def dense_attn(q, k, v, scale: float | None = None) -> np.ndarray:
    """Unpruned attention (the full KV cache of walkthrough Fig. 2a), float64."""
    D = k.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    return _attend(q, np.asarray(k, dtype=np.float64), v, scale)


# ---------------------------------------------------------------- sampled recovery F
#
# Counter-based generator: Philox4x32 with 10 rounds, from its published
# definition (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
# random numbers: as easy as 1, 2, 3", SC 2011, section on the Philox
# family). One round maps the counter (c0, c1, c2, c3) under the round key
# (k0, k1) to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)),
# with 32 x 32 -> 64-bit products; the key is advanced by the Weyl constants
# between rounds.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_M32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of counters ctr = (c0, c1, c2, c3) (arrays, broadcast
    together) under key = (k0, k1) (ints): four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _M32 for x in ctr]
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = np.uint64(PHILOX_M0) * c0
        p1 = np.uint64(PHILOX_M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & _M32,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & _M32)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def uniform01(x) -> np.ndarray:
    """u = (x + 1/2) / 2^32 in (0, 1) for uint32 x, float64."""
    return (np.asarray(x, dtype=np.float64) + 0.5) * 2.0 ** -32


def recovery_samples(b: int, h: int, n_kv: int, S: int, D: int, mode: str, mu: float, sigma: float,
                     seed: int) -> np.ndarray:
    """Sampled saliency w~[t][j] for one (b, KV head), float64 (walkthrough
    section 3.3 step 2 and F table).

    Counter (t, j // 4, b * n_kv + h, 0), key (seed low 32 bits, seed high 32
    bits); the four outputs x0..x3 serve channels 4 (j // 4) + 0..3:
      exponential (mean mu):  w = -mu ln(u_i) for each output
      gaussian N(mu, sigma^2): Box-Muller on (u0, u1) and on (u2, u3):
                              R = sqrt(-2 ln u_even), theta = 2 pi u_odd,
                              z_even = R cos theta, z_odd = R sin theta,
                              w = mu + sigma z
    """
    t = np.arange(S, dtype=np.uint64)[:, None]
    jg = np.arange(D // 4, dtype=np.uint64)[None, :]
    x = philox4x32_10((t, jg, b * n_kv + h, 0), (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    u = [uniform01(xi) for xi in x]                                   # each [S][D/4]
    if mode == F_EXPONENTIAL:
        w = [-mu * np.log(ui) for ui in u]
    elif mode == F_GAUSSIAN:
        w = []
        for e in (0, 2):
            R = np.sqrt(-2.0 * np.log(u[e]))
            th = 2.0 * math.pi * u[e + 1]
            w += [mu + sigma * R * np.cos(th), mu + sigma * R * np.sin(th)]
    else:
        raise ValueError(mode)
    return np.stack(w, axis=-1).reshape(S, D)                        # channel 4 jg + i


def expand_keys_sampled(packed, mask, A, r, mode: str, seed: int) -> np.ndarray:
    """K_hat with sampled recovery, float64: mask ? stored value : w~_tj / a_j
    (0 if a_j = 0), a_j = sqrt(A_j), mu = r[..., 0], sigma = r[..., 1]
    (walkthrough section 3.3 steps 2-3)."""
    B, H, S, D = mask.shape
    a = np.sqrt(np.asarray(A, dtype=np.float64))
    r64 = np.asarray(r, dtype=np.float64)
    khat = np.zeros(mask.shape)
    for b in range(B):
        for h in range(H):
            w = recovery_samples(b, h, H, S, D, mode, float(r64[b, h, 0]), float(r64[b, h, 1]), seed)
            khat[b, h] = np.where(a[b, h] > 0, w / np.where(a[b, h] > 0, a[b, h], 1.0), 0.0)
    khat[mask] = np.asarray(packed, dtype=np.float64).reshape(-1)
    return khat


def decode_attn_sampled(q, packed, mask, v, A, r, mode: str, seed: int, scale: float | None = None) -> np.ndarray:
    """One decode step with a sampled recovery F: sample, back-solve, then
    standard attention (walkthrough section 3.3 steps 2-4 and F table).
    Returns out [B][N_q][D] in float64."""
    D = mask.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    return _attend(q, expand_keys_sampled(packed, mask, A, r, mode, seed), v, scale)


# ---------------------------------------------------------------- decode-time cache growth
#
# The pages prune only at prefill. Reading taken here: every generated
# token's key is pruned with the prefill's channel energy A by the prefill's
# own rule (top-T of fl32(A_j k^2), ties to the lower channel) and appended;
# its V row is appended dense; r stays as the prefill computed it.

def append_tokens(k_new: np.ndarray, A: np.ndarray, T: int) -> dict:
    """k_new [B][N_kv][n][D] -> mask [B][N_kv][n][D], words, packed [..., T]."""
    mask = select_top_t(saliency_keys(A, k_new), T)
    return {"mask": mask, "words": mask_words(mask), "packed": pack_kept(k_new, mask)}


def grow_cache(packed, mask, v, k_new, v_new, A, T: int):
    """The cache (packed, mask, v over S tokens) after appending the n tokens
    of k_new / v_new ([B][N_kv][n][D]) in order."""
    a = append_tokens(k_new, A, T)
    return (np.concatenate([packed, a["packed"]], axis=2), np.concatenate([mask, a["mask"]], axis=2),
            np.concatenate([np.asarray(v), np.asarray(v_new)], axis=2))


# ---------------------------------------------------------------- SparK-p (top-p)
#
# Walkthrough section 5.2: per token, the smallest channel set whose summed
# saliency is at least p = 99% of the token's total. Reading taken here, chosen
# so that the integer decision is made in one defined fp32 arithmetic:
#   w_tj = fl32(sqrt(key_tj)) (correctly rounded), the saliency a_j |k_tj|;
#   every sum over a token's channels is the pairwise tree that folds the
#   upper half onto the lower half (channel j with j + 64, then + 32, ...,
#   + 1), in fp32;
#   target = fl32(p * total), total the tree sum of all w;
#   sort the token's channels by key, largest first, and take prefixes of
#   that order, each one extended over the channels tied with its last key;
#   the token keeps the first (shortest) such prefix whose tree sum of w
#   reaches the target. Channels tied at the cut are kept together; a token
#   whose saliency is all zero has a zero target, which the empty set already
#   reaches, so it keeps none.
# The kept count T_t varies per token, so the packed store is ragged: token
# t's values sit at [row_off[t], row_off[t + 1]) of its head's region.

def tree_sum32(v: np.ndarray) -> np.ndarray:
    """fp32 pairwise sum over the last axis (length a power of two), folding
    the upper half onto the lower half at each level."""
    x = np.asarray(v, dtype=np.float32)
    n = x.shape[-1]
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    while n > 1:
        h = n // 2
        x = (x[..., :h] + x[..., h:n]).astype(np.float32)
        n = h
    return x[..., 0]


def select_top_p(keys: np.ndarray, p: float, chunk: int = 512) -> np.ndarray:
    """SparK-p kept set per token (see the section comment), in its plain form.

    The candidate sets are the prefixes of the token's channels in descending
    key order, each prefix extended over every channel tied with its last key
    (so a candidate is {key >= theta} for one of the token's key values
    theta), preceded by the empty set. The token keeps the first candidate,
    scanning from the empty set towards the whole row, whose fp32 tree sum of
    w reaches the target fl32(p * total). The empty set's sum is 0, so it is
    kept only when the target is 0 (an all-zero row).
    """
    k32 = _f32(keys)
    shape = k32.shape
    D = shape[-1]
    rows = k32.reshape(-1, D)
    out = np.zeros(rows.shape, dtype=bool)
    for lo in range(0, rows.shape[0], chunk):
        kk = rows[lo:lo + chunk]                                   # [n][D]
        w = np.sqrt(kk).astype(np.float32)
        target = (np.float32(p) * tree_sum32(w)).astype(np.float32)  # [n]
        theta = -np.sort(-kk, axis=-1)                             # key values, descending
        cand = kk[:, None, :] >= theta[:, :, None]                 # [n][candidate i][channel]: {key >= theta_i}
        sums = tree_sum32(np.where(cand, w[:, None, :], np.float32(0)))   # [n][D]
        reach = sums >= target[:, None]
        first = np.argmax(reach, axis=-1)                          # the total always reaches fl32(p * total)
        kept = np.take_along_axis(cand, first[:, None, None], axis=1)[:, 0, :]
        kept[target == 0] = False                                  # the empty set reaches a zero target
        out[lo:lo + chunk] = kept
    return out.reshape(shape)


def prune_topp(q_win: np.ndarray, k: np.ndarray, n_kv: int, p: float, qagg: str = QAGG_L2) -> dict:
    """SparK-p prefill pruning. Returns A, mask, words, counts [B][N_kv][S],
    row_off [B][N_kv][S + 1] (offsets within the head) and packed: all kept
    values in (b, head, token, channel) order, ragged."""
    A = chan_energy(q_win, n_kv, qagg)
    mask = select_top_p(saliency_keys(A, k), p)
    counts = mask.sum(axis=-1).astype(np.int32)
    row_off = np.zeros(counts.shape[:-1] + (counts.shape[-1] + 1,), dtype=np.int64)
    row_off[..., 1:] = np.cumsum(counts, axis=-1)
    return {"A": A, "mask": mask, "words": mask_words(mask), "counts": counts, "row_off": row_off,
            "packed": np.asarray(k)[mask]}


# ---------------------------------------------------------------- SparK-g (grouped ratios)
#
# Walkthrough section 5.2: channels are grouped by importance and each group
# is pruned at its own ratio, low-importance groups harder; with g = 4 the
# ratios are (0.25, 0.5, 0.75, 1.0). Reading taken here: per (batch, KV
# head), rank the channels by the channel energy A_j (descending, ties to the
# lower channel) and cut the ranking into g equal groups; group i (i = 0 the
# most important) gets the i-th ratio; every token keeps, in each group, the
# T_i = num_kept(D / g, ratio_i) members of largest saliency key (ties to the
# lower channel). Every token then keeps the same T = sum T_i channels.

def channel_groups(A: np.ndarray, g: int) -> np.ndarray:
    """Group index [B][N_kv][D] of each channel: rank by A descending (ties
    to the lower channel), cut into g equal groups."""
    A = _f32(A)
    D = A.shape[-1]
    if D % g:
        raise ValueError("g must divide D")
    order = np.argsort(-A, axis=-1, kind="stable")
    rank = np.empty_like(order)
    np.put_along_axis(rank, order, np.arange(D)[None, None, :].repeat(A.shape[0], 0).repeat(A.shape[1], 1), axis=-1)
    return rank // (D // g)


def grouped_num_kept(D: int, ratios) -> list:
    """T_i per group for group ratios (each group has D / g channels)."""
    g = len(ratios)
    return [num_kept(D // g, r) for r in ratios]


def select_grouped(keys: np.ndarray, groups: np.ndarray, Ts) -> np.ndarray:
    """Per token and group i, the T_i members of largest key (ties to the
    lower channel)."""
    mask = np.zeros(keys.shape, dtype=bool)
    gb = groups[:, :, None, :]
    for i, Ti in enumerate(Ts):
        member = np.broadcast_to(gb == i, keys.shape)
        # non-members rank below every member (keys are >= 0)
        k_i = np.where(member, keys.astype(np.float64), -1.0)
        mask |= select_top_t(k_i, Ti) & member
    return mask


def prune_grouped(q_win: np.ndarray, k: np.ndarray, n_kv: int, ratios, qagg: str = QAGG_L2) -> dict:
    """SparK-g prefill pruning: like prune() with the group-wise selection."""
    D = k.shape[-1]
    A = chan_energy(q_win, n_kv, qagg)
    groups = channel_groups(A, len(ratios))
    Ts = grouped_num_kept(D, ratios)
    mask = select_grouped(saliency_keys(A, k), groups, Ts)
    return {"T": int(sum(Ts)), "Ts": Ts, "A": A, "groups": groups, "mask": mask, "words": mask_words(mask),
            "packed": pack_kept(k, mask)}


# ---------------------------------------------------------------- V-channel pruning
#
# Walkthrough section 4.4 prunes the V cache too, by a norm-based rule that
# the page does not spell out. Reading taken here: per token, keep the
# T_v channels of largest |v_tj| (the norm of the single entry), ties to the
# lower channel, T_v = num_kept(D, lambda_v); a pruned entry is recovered by
# the channel's mean over the tokens that retain it (the retained-mean F of
# the keys), 0 if no token does.

def value_keys(v: np.ndarray) -> np.ndarray:
    """key = v^2 in fp32 (exact for bf16 v): ranks channels by |v_tj|."""
    v = _f32(v)
    return v * v


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Finite fp32 values to the nearest bfloat16 (8 significand bits, ties
    to even), returned as fp32: add half a bf16 unit (minus one, plus the
    kept part's lowest bit for the tie) to the bit pattern, then drop the low
    16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def prune_v(v: np.ndarray, lam_v: float) -> dict:
    """V-channel pruning of one cache: {"T", "mask", "words", "packed", "r",
    "cnt"} with r the retained-mean recovery of the pruned entries, rounded
    to bfloat16, the precision of the cached V entries it stands in for
    (walkthrough section 4.4 prunes V with K but does not spell the rule out;
    this is the reading taken)."""
    D = v.shape[-1]
    T = num_kept(D, lam_v)
    mask = select_top_t(value_keys(v), T)
    r, cnt = stats(v, mask, None, F_MEAN_RETAINED)
    return {"T": T, "mask": mask, "words": mask_words(mask), "packed": pack_kept(v, mask), "r": round_bf16(r),
            "cnt": cnt}


# Block reading of the same section's norm-based V rule: a token keeps whole
# blocks of 8 consecutive channels, the n_b = num_kept(D / 8, lambda_v) blocks
# whose V entries have the largest L2 norm, ties to the lower block. The norm
# is compared squared, as an fp32 sum of the block's 8 squares (exact for bf16
# v) added in channel order. Kept blocks are packed in ascending block order;
# a pruned entry is recovered as in prune_v.

V_BLOCK = 8


def value_block_keys(v: np.ndarray) -> np.ndarray:
    """Squared L2 norm of each block of V_BLOCK consecutive channels, fp32:
    [..., D] -> [..., D / V_BLOCK], the squares added one at a time in
    channel order, each sum rounded to fp32."""
    v = _f32(v)
    D = v.shape[-1]
    if D % V_BLOCK:
        raise ValueError("D must be a multiple of the block size")
    sq = (v * v).reshape(*v.shape[:-1], D // V_BLOCK, V_BLOCK)
    acc = np.zeros(sq.shape[:-1], dtype=np.float32)
    for c in range(V_BLOCK):
        acc = (acc + sq[..., c]).astype(np.float32)
    return acc


def prune_v_blocks(v: np.ndarray, lam_v: float) -> dict:
    """Block-mode V pruning of one cache: {"nb", "T", "block_mask", "mask",
    "packed", "r", "cnt"}. block_mask [..., S, D / 8] holds the kept blocks,
    mask the same per channel; packed holds each token's kept blocks back to
    back in ascending block order (T = 8 nb values); r is the retained-mean
    recovery rounded to bfloat16, as in prune_v."""
    D = v.shape[-1]
    nb = num_kept(D // V_BLOCK, lam_v)
    block_mask = select_top_t(value_block_keys(v), nb)
    mask = np.repeat(block_mask, V_BLOCK, axis=-1)
    r, cnt = stats(v, mask, None, F_MEAN_RETAINED)
    return {"nb": nb, "T": V_BLOCK * nb, "block_mask": block_mask, "mask": mask, "packed": pack_kept(v, mask),
            "r": round_bf16(r), "cnt": cnt}


def decode_attn_kv(q, k_packed, k_mask, r, v_packed, v_mask, rv, scale: float | None = None) -> np.ndarray:
    """Decode over a cache with both K and V channels pruned: K_hat as in
    decode_attn, V_hat = v_mask ? stored value : rv_j, then softmax attention
    (walkthrough sections 3.3 and 4.4). Returns out [B][N_q][D] in float64."""
    D = k_mask.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    return _attend(q, expand_keys(k_packed, k_mask, r), expand_keys(v_packed, v_mask, rv), scale)


def window_scores(q_win: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Window-summed causal softmax score per cached token, float64: [B][N_kv][S].

    The observation-window eviction that SparK is stacked on (walkthrough
    section 4.1; section 3.2 borrows its window). Query row (g, w) sits at
    position S - W + w and sees tokens t <= S - W + w; its softmax over those
    tokens is summed over the G heads of the group and the W window rows.
    """
    B, Nq, W, D = q_win.shape
    Nkv, S = k.shape[1], k.shape[2]
    rows = np.asarray(window_rows(q_win, Nkv), dtype=np.float64)    # [B][H][G*W][D]
    k64 = np.asarray(k, dtype=np.float64)
    pos = np.tile(np.arange(S - W, S), Nq // Nkv)                     # row position
    visible = np.arange(S)[None, :] <= pos[:, None]                   # [G*W][S]
    score = np.empty((B, Nkv, S), dtype=np.float64)
    for b in range(B):
        for h in range(Nkv):
            logit = (rows[b, h] @ k64[b, h].T) / math.sqrt(D)
            logit = np.where(visible, logit, -np.inf)
            p = np.exp(logit - logit.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            score[b, h] = p.sum(axis=0)
    return score


def snapkv_evict(q_win, k, v, keep: int):
    """Keep the `keep` highest-scoring tokens per (batch, KV head), ties to the lower t.

    Returns idx [B][N_kv][keep] (ascending), k_kept and v_kept [B][N_kv][keep][D].
    """
    score = window_scores(q_win, k)
    order = np.argsort(-score, axis=-1, kind="stable")[..., :keep]
    idx = np.sort(order, axis=-1)
    kk = np.take_along_axis(np.asarray(k), idx[..., None], axis=2)
    vv = np.take_along_axis(np.asarray(v), idx[..., None], axis=2)
    return idx.astype(np.int32), kk, vv
