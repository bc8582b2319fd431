"""Helpers shared by the tests: cache sizing and numpy reference pieces that
are *not* the method (dense softmax attention, fp64 dequantised keys)."""
import numpy as np

D = 128
TIER_BITS = {0: (8, 8), 1: (4, 4), 2: (2, 3)}


def dense_attention(keys, values, q, scale):
    """Plain softmax attention in fp64: keys [n,128], values [n,128], q [128]."""
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    if keys.shape[0] == 0:
        return np.zeros(D), -np.inf
    lg = scale * (keys @ np.asarray(q, np.float64))
    m = lg.max()
    e = np.exp(lg - m)
    return (e[:, None] * values).sum(0) / e.sum(), m + np.log(e.sum())


def dequantize(r16, theta, s, tb, sb, half_split=False):
    """fp64 key from codes: pair j is (k[2j], k[2j+1]) (or (k[j], k[j+64])
    when half_split) = r s_j (cos th_j, sin th_j), th_c = -pi + c 2pi/2^tb,
    s = code/(2^sb - 1)."""
    r = np.asarray(r16, np.uint16).view(np.float16).astype(np.float64)
    N = 1 << tb
    L = (1 << sb) - 1
    th = -np.pi + np.asarray(theta, np.float64) * (2 * np.pi / N)
    sv = np.asarray(s, np.float64) / L
    k = np.zeros(np.shape(theta)[:-1] + (D,))
    xs, ys = (slice(0, 64), slice(64, 128)) if half_split else (slice(0, None, 2), slice(1, None, 2))
    k[..., xs] = r[..., None] * sv * np.cos(th)
    k[..., ys] = r[..., None] * sv * np.sin(th)
    return k


def upper_capacity(w, block16_max, extra_pages_per_row=3):
    """Generous cache dimensions for a workload: every row may hold
    ceil(ctx/P) + 3 pages (one partial page per tier)."""
    P = w["P"]
    rows = w["B"] * w["Hkv"]
    per_row = -(-int(w["stride"]) // P) + extra_pages_per_row
    pages = rows * per_row
    return per_row, pages, pages * block16_max


def kept_tokens(w, b, h):
    """positions and tiers of the kept tokens of (b, h), in page order
    (tier id ascending, then position ascending)."""
    t = w["tiers"][b, h, : int(w["ctx_len"][b])]
    out = []
    for tau in range(6):
        pos = np.nonzero(t == tau)[0]
        out.extend((int(p), tau) for p in pos)
    return out


def near_boundary_pairs(tb, per_boundary=2):
    """fp32 pairs whose angle lies extremely close to a rounding boundary of
    the tb-bit angle grid: for a boundary direction beta in the first octant,
    search integers M in [2^23, 2^24) for which M tan(beta) is nearly an
    integer Y; (M, Y) is then exactly representable.  The other octants
    follow by the exact maps (x,y)->(-y,x) and (x,y)->(y,x)."""
    N = 1 << tb
    M = np.arange(2 ** 23, 2 ** 24, dtype=np.float64)
    out = []
    for m in range(N):
        beta = -np.pi + (m + 0.5) * 2 * np.pi / N
        if not (0 < beta < np.pi / 4):
            continue
        y = M * np.tan(beta)
        frac = np.abs(y - np.round(y))
        best = np.argsort(frac)[:per_boundary]
        for i in best:
            out.append((float(M[i]), float(np.round(y[i]))))
    pairs = []
    for x, y in out:
        for (a, b) in [(x, y), (y, x)]:
            for _ in range(4):
                pairs.append((a, b))
                a, b = -b, a
    return pairs

