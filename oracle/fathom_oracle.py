"""Fathom CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy implementation of what the Fathom
plane-prefix key scan computes.  Only the test-suite, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py`` may import this module; the product
path (the HIP library and its Python binding) never does, and the two share no
code.

Pages followed (cited by title and paragraph / sentence; the pages have no
numbered sections or equations):

* [Art] "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context
  Decoding" -- para 1 (top-k scan over all keys), para 2 (channel-major bit
  planes; a t-plane prefix is the t-bit quantized value), para 3 (per-query
  reverse water-filling under a total bit budget, closed form), limits para
  (GPU-resident scan is arithmetic-bound).
* [Abs] "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
  Caches", abstract: s1 (scan ranks all n keys for a top-k step), s2 (each
  query decides how many bits of each channel to read), s3 (4-bit K cache
  stored channel-major as bit planes; prefix = t-bit quantizer; budget spent
  by reverse water-filling over variance-weighted channel importance), s6
  (the store is the serving stack's 4-bit K copy).

Readings of what the pages leave open are marked READING(Zn); each one is
listed with its evidence in the design notes of this repository.

Precision: fp32 steps use float32 NumPy arrays (IEEE round-to-nearest, no FMA
contraction); variance and scores use float64, as stated per function.

Pins: every function here is checked by the ``-m "not gpu"`` tests against
something other than itself (hand-worked cases, an independent t-bit
quantizer, brute-force allocation search, exchange optimality, dense dot
products, closed forms).  No function is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

PLANES = 4                 # the store is a 4-bit K cache [Abs s3, s6]
LEVELS = 1 << PLANES       # 16 quantization bins
KEY_STEP = 1 << 24         # int32 ordering-key step per plane (a factor 4 in value)


# --------------------------------------------------------------------------
# Layout helper
# --------------------------------------------------------------------------

def plane_ldw(n: int) -> int:
    """Words per plane row: ceil(n / 32) rounded up to a multiple of 4.

    READING(Z4): word w of a plane row holds keys 32w .. 32w+31, key 32w+b at
    bit b; rows are padded to 16-byte multiples; padding bits are zero.
    """
    if n < 1:
        raise ValueError("n must be >= 1")
    words = (n + 31) // 32
    return (words + 3) // 4 * 4


# --------------------------------------------------------------------------
# Quantizer: per-(head, channel) asymmetric 4-bit codes  [Art para 2; Abs s3, s6]
# --------------------------------------------------------------------------

def key_range(keys: np.ndarray):
    """lo, hi per channel over all n keys of one head.

    READING(Z3): per-channel asymmetric quantization, range taken over the
    head's n keys.  keys: float32 [n, d] -> (lo, hi) float32 [d].
    """
    keys = np.asarray(keys, dtype=np.float32)
    assert keys.ndim == 2 and np.all(np.isfinite(keys)), "keys must be finite [n, d]"
    return keys.min(axis=0), keys.max(axis=0)


def quant_scale(lo: np.ndarray, hi: np.ndarray):
    """Bin width and inverse scale of the 16-bin quantizer.

    r = fl32(hi - lo); step = r / 16 (exact); inv = fl32(16 / r), a correctly
    rounded division, or 0 for a constant channel (READING(Z12)).
    Returns (step, inv) float32 [d].
    """
    lo = np.asarray(lo, dtype=np.float32)
    hi = np.asarray(hi, dtype=np.float32)
    r = (hi - lo).astype(np.float32)
    step = (r * np.float32(1.0 / LEVELS)).astype(np.float32)
    inv = np.zeros_like(r)
    pos = r > 0
    inv[pos] = np.float32(LEVELS) / r[pos]
    return step, inv.astype(np.float32)


def quantize(keys: np.ndarray, lo: np.ndarray, inv: np.ndarray) -> np.ndarray:
    """4-bit codes: code = min(15, floor(fl32(fl32(K - lo) * inv))).

    READING(Z1): a floor ("mid-rise") quantizer with 16 equal bins on
    [lo, hi].  Its t-bit truncations are themselves the t-bit floor
    quantizers of the same range, which is what makes a t-plane prefix
    exactly the channel's t-bit quantizer [Abs s3; Art para 2].
    keys float32 [n, d] -> codes uint8 [n, d].
    """
    keys = np.asarray(keys, dtype=np.float32)
    t = (keys - lo[None, :]).astype(np.float32)
    u = (t * inv[None, :]).astype(np.float32)
    code = np.minimum(np.floor(u), np.float32(LEVELS - 1))
    return code.astype(np.uint8)


def pack_planes(codes: np.ndarray, ldw: int) -> np.ndarray:
    """Channel-major MSB-first bit planes of one head [Art para 2; Abs s3].

    codes uint8 [n, d] -> planes uint32 [d, 4, ldw]; plane j holds bit (3 - j)
    of each code (j = 0 is the most significant), word w bit b is key 32w + b.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    n, d = codes.shape
    assert ldw * 32 >= n
    out = np.zeros((d, PLANES, ldw), dtype=np.uint32)
    for j in range(PLANES):
        bits = np.zeros((d, ldw * 32), dtype=np.uint8)
        bits[:, :n] = ((codes >> (PLANES - 1 - j)) & 1).T
        packed = np.packbits(bits, axis=1, bitorder="little")   # [d, ldw*4] bytes
        out[:, j, :] = packed.view("<u4")
    return out


def append_codes(keys_new: np.ndarray, lo: np.ndarray, step: np.ndarray) -> np.ndarray:
    """Codes of keys appended to a packed head at decode time.

    READING(Z18): a growing cache [Abs s1; Art para 1] keeps the quantizer
    fixed at packing: r = fl32(16 step) (exact, step being r / 16),
    inv = fl32(16 / r) (0 for r = 0), and the packer's code rule clamped to
    [0, 15], since a new key may fall outside the packed range:
        code = min(15, max(0, floor(fl32(fl32(K - lo) * inv)))).
    keys_new float32 [m, d] -> codes uint8 [m, d].
    """
    keys_new = np.asarray(keys_new, dtype=np.float32)
    assert keys_new.ndim == 2 and np.all(np.isfinite(keys_new)), "keys must be finite [m, d]"
    lo = np.asarray(lo, dtype=np.float32)
    r = (np.asarray(step, dtype=np.float32) * np.float32(LEVELS)).astype(np.float32)
    inv = np.zeros_like(r)
    pos = r > 0
    inv[pos] = np.float32(LEVELS) / r[pos]
    t = (keys_new - lo[None, :]).astype(np.float32)
    u = (t * inv[None, :]).astype(np.float32)
    code = np.clip(np.floor(u), 0.0, np.float32(LEVELS - 1))
    return code.astype(np.uint8)


def append_planes(planes: np.ndarray, n: int, codes_new: np.ndarray) -> np.ndarray:
    """The head's planes with the codes of keys n .. n + m - 1 written in
    (bits already there are replaced).  planes uint32 [d, 4, ldw]."""
    planes = np.array(planes, dtype=np.uint32, copy=True)
    codes_new = np.asarray(codes_new, dtype=np.uint8)
    m, d = codes_new.shape
    assert n + m <= planes.shape[2] * 32
    for t in range(m):
        w, b = divmod(n + t, 32)
        for c in range(d):
            for j in range(PLANES):
                bit = (int(codes_new[t, c]) >> (PLANES - 1 - j)) & 1
                planes[c, j, w] = (planes[c, j, w] & ~np.uint32(1 << b)) | np.uint32(bit << b)
    return planes


def unpack_plane_bits(planes: np.ndarray, n: int) -> np.ndarray:
    """Inverse view of ``pack_planes``: bits uint8 [d, 4, n]."""
    planes = np.ascontiguousarray(planes, dtype="<u4")
    d, p, ldw = planes.shape
    as_bytes = planes.view(np.uint8).reshape(d, p, ldw * 4)
    bits = np.unpackbits(as_bytes, axis=2, bitorder="little")
    return bits[:, :, :n]


def channel_variance(codes: np.ndarray, step: np.ndarray) -> np.ndarray:
    """Per-channel variance of the 4-bit reconstructions [Abs s3, "variance-
    weighted importance"].

    READING(Z5): the variance of lo + (code + 1/2) * step over the head's n
    keys, from exact integer moments S1 = sum(code), S2 = sum(code^2):
        var = fl32( fl64(S2*n - S1^2) / fl64(n^2) * (fl64(step) * fl64(step)) ).
    Order-independent and reproducible bit for bit.  float32 [d].
    """
    codes = np.asarray(codes)
    n = codes.shape[0]
    c64 = codes.astype(np.int64)
    s1 = c64.sum(axis=0)
    s2 = (c64 * c64).sum(axis=0)
    num = s2 * np.int64(n) - s1 * s1
    den = np.float64(n) * np.float64(n)
    st = np.asarray(step, dtype=np.float32).astype(np.float64)
    var = (num.astype(np.float64) / den) * (st * st)
    return var.astype(np.float32)


def pack_head(keys: np.ndarray, ldw: int | None = None):
    """All per-head store products: (planes, lo, step, var, codes).

    ldw: row length in words (default plane_ldw(n)); a longer row, as when
    heads of different lengths share one store, holds zero padding bits.
    READING(Z20): a head holding no key has no range: lo = step = var = 0 and
    all-zero planes.
    """
    keys = np.asarray(keys, dtype=np.float32)
    n, d = keys.shape
    if ldw is None:
        ldw = plane_ldw(n)
    if n == 0:
        z = np.zeros(d, np.float32)
        return np.zeros((d, PLANES, ldw), np.uint32), z, z.copy(), z.copy(), np.zeros((0, d), np.uint8)
    lo, hi = key_range(keys)
    step, inv = quant_scale(lo, hi)
    codes = quantize(keys, lo, inv)
    planes = pack_planes(codes, ldw)
    var = channel_variance(codes, step)
    return planes, lo, step, var, codes


# --------------------------------------------------------------------------
# Allocation: per-query reverse water-filling  [Art para 3; Abs s2, s3]
# --------------------------------------------------------------------------

def importance(q: np.ndarray, var: np.ndarray) -> np.ndarray:
    """w_c = fl32(fl32(q_c * q_c) * var_c), the variance-weighted importance.

    READING(Z6): the weight is q^2 sigma^2 on a 4^-j distortion ladder.
    var holds variances: finite and >= 0 (asserted).  A variance of -0 is the
    value 0, and so is the weight it gives: the result is normalised to +0 so
    that its bit pattern orders like its value (READING(Z19)).
    """
    q = np.asarray(q, dtype=np.float32)
    var = np.asarray(var, dtype=np.float32)
    assert np.all(np.isfinite(var)) and np.all(var >= 0), "var must hold finite variances >= 0"
    w = ((q * q).astype(np.float32) * var).astype(np.float32)
    return (w + np.float32(0.0)).astype(np.float32)


def ordering_keys(w: np.ndarray) -> np.ndarray:
    """int64 [d, 4]: K(c, j) = bits(w_c) - j * 2^24.

    For a normal w_c, K(c, j) orders candidates exactly as w_c * 4^-j
    (each plane divides the channel's distortion by 4, READING(Z7)).
    """
    bits = np.asarray(w, dtype=np.float32).view(np.int32).astype(np.int64)
    j = np.arange(PLANES, dtype=np.int64)
    return bits[:, None] - j[None, :] * KEY_STEP


def allocate(q: np.ndarray, var: np.ndarray, budget: int) -> np.ndarray:
    """Plane counts b_c in {0..4} with sum b_c = budget for one query.

    The budget goes to the candidates (c, j) in order of (K desc, c asc,
    j asc), READING(Z8, Z9): the exact integer minimiser of
    sum_c w_c 4^-b_c (greedy marginal allocation on a separable convex
    objective), the integer form of reverse water-filling.  uint8 [d].
    """
    w = importance(q, var)
    d = w.shape[0]
    if not 0 <= budget <= PLANES * d:
        raise ValueError("budget must be in [0, 4d]")
    K = ordering_keys(w).reshape(-1)
    c = np.repeat(np.arange(d), PLANES)
    j = np.tile(np.arange(PLANES), d)
    order = np.lexsort((j, c, -K))
    taken = order[:budget]
    return np.bincount(c[taken], minlength=d).astype(np.uint8)


def allocate_all(q: np.ndarray, var: np.ndarray, group: int, budget: int) -> np.ndarray:
    """Allocations for every query head; query q reads KV head q // group.

    q float32 [Q, d], var float32 [H, d] -> uint8 [Q, d].
    """
    q = np.asarray(q, dtype=np.float32)
    return np.stack([allocate(q[i], var[i // group], budget) for i in range(q.shape[0])])


def distortion(w: np.ndarray, b: np.ndarray) -> float:
    """Objective minimised by the allocation: sum_c w_c 4^-b_c (float64)."""
    return float(np.sum(np.asarray(w, np.float64) * np.power(4.0, -np.asarray(b, np.float64))))


# --------------------------------------------------------------------------
# Fixed-depth control reads  [Art findings bullets 1-2; Abs s4]
# --------------------------------------------------------------------------

CONTROL_UNIFORM = 0
CONTROL_TOP_CHANNELS = 1


def channel_order(q: np.ndarray) -> np.ndarray:
    """Channel indices by |q_c| descending (fp32 magnitudes), ties to the
    lower channel index."""
    a = np.abs(np.asarray(q, dtype=np.float32)).astype(np.float64)
    return np.lexsort((np.arange(a.shape[0]), -a))


def control_allocation(q: np.ndarray, budget: int, mode: int) -> np.ndarray:
    """Plane counts of a query-independent-depth read with the same budget.

    The pages compare Fathom with scans that read every key at a fixed width
    (136 and 68 bits).  READING(Z16): two such reads through the same scan:

    * CONTROL_UNIFORM: every channel reads floor(B/d) planes; the B mod d
      leftover planes go one each to the channels first in channel_order.
    * CONTROL_TOP_CHANNELS: the floor(B/4) channels first in channel_order
      read all 4 planes; the B mod 4 leftover planes go to the next one.

    uint8 [d], sum = budget.
    """
    q = np.asarray(q, dtype=np.float32)
    d = q.shape[0]
    if not 0 <= budget <= PLANES * d:
        raise ValueError("budget must be in [0, 4d]")
    rank = np.empty(d, dtype=np.int64)
    rank[channel_order(q)] = np.arange(d)
    if mode == CONTROL_UNIFORM:
        base, rem = divmod(budget, d)
        b = base + (rank < rem)
    elif mode == CONTROL_TOP_CHANNELS:
        r, rem = divmod(budget, PLANES)
        b = np.where(rank < r, PLANES, np.where(rank == r, rem, 0))
    else:
        raise ValueError("unknown control mode")
    return b.astype(np.uint8)


def control_allocation_all(q: np.ndarray, budget: int, mode: int) -> np.ndarray:
    """control_allocation for every query row: uint8 [Q, d]."""
    q = np.asarray(q, dtype=np.float32)
    return np.stack([control_allocation(q[i], budget, mode) for i in range(q.shape[0])])


# --------------------------------------------------------------------------
# Scores and top-k  [Art para 1, 2; Abs s1, s2]
# --------------------------------------------------------------------------

def scores_from_codes(codes: np.ndarray, lo, step, q, b) -> np.ndarray:
    """Partially dequantized dot product for the given keys (code form).

    Channel c contributes its b_c-bit truncation p = code >> (4 - b_c),
    reconstructed at its bin centre (READING(Z2)):
        khat_c = lo_c + (p + 1/2) * step_c * 2^(4 - b_c)
        s = sum_c q_c * khat_c                     (float64)
    codes uint8 [m, d] for any m keys -> float64 [m].
    """
    codes = np.asarray(codes)
    shift = (PLANES - np.asarray(b, dtype=np.int64))
    p = (codes.astype(np.int64) >> shift[None, :]).astype(np.float64)
    width = np.asarray(step, np.float32).astype(np.float64) * np.power(2.0, shift.astype(np.float64))
    khat = np.asarray(lo, np.float32).astype(np.float64)[None, :] + (p + 0.5) * width[None, :]
    return khat @ np.asarray(q, np.float32).astype(np.float64)


def score_offset(lo, step, q, b) -> float:
    """C_q = sum_c q_c (lo_c + step_c 2^(3 - b_c)), the score of an all-zero
    bit pattern (float64)."""
    b = np.asarray(b, dtype=np.float64)
    lo64 = np.asarray(lo, np.float32).astype(np.float64)
    st64 = np.asarray(step, np.float32).astype(np.float64)
    q64 = np.asarray(q, np.float32).astype(np.float64)
    return float(np.sum(q64 * (lo64 + st64 * np.power(2.0, 3.0 - b))))


def scores_from_planes(planes: np.ndarray, n: int, lo, step, q, b) -> np.ndarray:
    """Bit-plane form of the same scores: only plane prefixes are read.

        s(i) = C_q + sum_c sum_{j < b_c} q_c step_c 2^(3 - j) bit_{c,j}(i)
    planes uint32 [d, 4, ldw] -> float64 [n].
    """
    bits = unpack_plane_bits(planes, n).astype(np.float64)      # [d, 4, n]
    b = np.asarray(b, dtype=np.int64)
    q64 = np.asarray(q, np.float32).astype(np.float64)
    st64 = np.asarray(step, np.float32).astype(np.float64)
    s = np.full(n, score_offset(lo, step, q, b), dtype=np.float64)
    for c in range(planes.shape[0]):
        for j in range(int(b[c])):
            s += q64[c] * st64[c] * 2.0 ** (3 - j) * bits[c, j]
    return s


def topk(scores: np.ndarray, k: int):
    """Top-k by a full stable sort on (score desc, index asc) [Art para 1;
    Abs s1], READING(Z9, Z11).  Returns (idx int32 [k], score float32 [k])."""
    s = np.asarray(scores, dtype=np.float64)
    if not 1 <= k <= s.shape[0]:
        raise ValueError("k must be in [1, n]")
    idx = np.arange(s.shape[0])
    order = np.lexsort((idx, -s))[:k]
    return order.astype(np.int32), s[order].astype(np.float32)


def topk_padded(scores: np.ndarray, k: int):
    """``topk`` over a head that may hold fewer than k keys (ragged sessions).

    READING(Z20): the first min(k, n) ranks are the top-k of the n scores
    (score desc, index asc); ranks n .. k - 1 hold index -1 and score -inf.
    scores float [n], n >= 0 -> (idx int32 [k], score float32 [k]).
    """
    s = np.asarray(scores, dtype=np.float64)
    m = min(k, s.shape[0])
    idx = np.full(k, -1, np.int32)
    val = np.full(k, -np.inf, np.float32)
    if m > 0:
        idx[:m], val[:m] = topk(s, m)
    return idx, val


# --------------------------------------------------------------------------
# Whole step for small problems
# --------------------------------------------------------------------------

def decode_step(keys: np.ndarray, q: np.ndarray, group: int, budget: int, k: int):
    """Pack every head, allocate every query, score all keys, select top-k.

    keys float32 [H, n, d]; q float32 [Q, d] with Q = H * group.
    Returns a dict of per-head store products and per-query results.
    """
    keys = np.asarray(keys, dtype=np.float32)
    H, n, d = keys.shape
    assert q.shape[0] == H * group
    heads = [pack_head(keys[h]) for h in range(H)]
    var = np.stack([hd[3] for hd in heads])
    alloc = allocate_all(q, var, group, budget)
    scores = np.empty((q.shape[0], n), dtype=np.float64)
    idx = np.empty((q.shape[0], k), dtype=np.int32)
    val = np.empty((q.shape[0], k), dtype=np.float32)
    for i in range(q.shape[0]):
        planes, lo, step, _, codes = heads[i // group]
        scores[i] = scores_from_codes(codes, lo, step, q[i], alloc[i])
        idx[i], val[i] = topk(scores[i], k)
    return {
        "planes": np.stack([hd[0] for hd in heads]),
        "lo": np.stack([hd[1] for hd in heads]),
        "step": np.stack([hd[2] for hd in heads]),
        "var": var,
        "codes": np.stack([hd[4] for hd in heads]),
        "alloc": alloc,
        "scores": scores,
        "idx": idx,
        "val": val,
    }


# --------------------------------------------------------------------------
# Attention over the selected keys  [Abs title and s1; Art findings bullet 2]
# --------------------------------------------------------------------------

def attention(k_rows: np.ndarray, v_rows: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query over the given key/value rows.

    READING(Z17): the decode step that follows the top-k selection attends
    over the selected rows only, with the usual scaled dot-product softmax:
        p_i = exp(scale q.k_i - max_j scale q.k_j),  o = sum_i p_i v_i / sum_i p_i
    in float64 on the rows as stored.  k_rows, v_rows [m, d] (m >= 1) ->
    float64 [d].
    """
    K = np.asarray(k_rows).astype(np.float64)
    V = np.asarray(v_rows).astype(np.float64)
    if K.shape[0] < 1:
        raise ValueError("attention needs at least one row")
    z = scale * (K @ np.asarray(q, np.float32).astype(np.float64))
    p = np.exp(z - z.max())
    return (p @ V) / p.sum()


def sparse_attention(K: np.ndarray, V: np.ndarray, q: np.ndarray, idx: np.ndarray, scale: float) -> np.ndarray:
    """attention() over the rows idx of one head's K, V [n, d]."""
    idx = np.asarray(idx, dtype=np.int64)
    return attention(np.asarray(K)[idx], np.asarray(V)[idx], q, scale)


def attention_error(o_sparse: np.ndarray, o_dense: np.ndarray) -> float:
    """READING(Z17): relative L2 error of the sparse output against dense
    attention over all n keys."""
    o_dense = np.asarray(o_dense, np.float64)
    return float(np.linalg.norm(np.asarray(o_sparse, np.float64) - o_dense) / np.linalg.norm(o_dense))

