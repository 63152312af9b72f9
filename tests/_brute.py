"""Brute-force per-token definitions used to pin the oracle on tiny inputs.

Pure Python loops over tokens and channels: no blocking, no summaries, no matrix calls.
"""
import math


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def relu(a):
    return [x if x > 0 else 0.0 for x in a]


def block_tokens(j, n, b):
    return list(range(j * b, min((j + 1) * b, n)))


def pooled_mean(x, j, b):
    toks = block_tokens(j, len(x), b)
    d = len(x[0])
    return [sum(x[t][c] for t in toks) / len(toks) for c in range(d)]


def softmax_attention_row(q, keys, vals):
    d = len(q)
    if not keys:
        return [0.0] * len(vals[0]) if vals else [0.0] * d
    logits = [dot(q, k) / math.sqrt(d) for k in keys]
    m = max(logits)
    w = [math.exp(l - m) for l in logits]
    tot = sum(w)
    return [sum(w[t] * vals[t][c] for t in range(len(keys))) / tot for c in range(len(vals[0]))]


def linear_attention_row(q, keys, vals, eps=1e-6):
    fq = relu(q)
    num = [0.0] * len(vals[0]) if vals else []
    den = 0.0
    for k, v in zip(keys, vals):
        w = dot(fq, relu(k))
        den += w
        for c in range(len(v)):
            num[c] += w * v[c]
    return [x / (den + eps) for x in num]


# ----------------------------------------------------------------------------- E4M3 by search
def e4m3_table():
    """Every finite non-negative E4M3FN value with its code, enumerated from the format
    (OCP 8-bit floating point): exponent field 0 holds the subnormals m * 2^-9; fields 1..15
    hold (1 + m/8) * 2^(e - 7), except the NaN pattern e = 15, m = 7."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            out.append((m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7), (e << 3) | m))
    return out


def e4m3_nearest(x, table):
    """Nearest table value by search, ties to the even code, magnitudes clamped to 448."""
    a = min(abs(x), 448.0)
    v, _ = min(table, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return math.copysign(v, x) if v else 0.0


def pow2_block_exponent(amax):
    """Smallest integer e with 448 * 2^e >= amax, by counting up (0 for an all-zero block)."""
    if amax == 0:
        return 0
    e = -80
    while 448.0 * 2.0 ** e < amax:
        e += 1
    return e


def fp8_attention_row(q8, sq, tiles, table):
    """One query row of the quantised sparse branch in the power-of-two reading, token by
    token: per selected key tile (k8 rows, s_K, v8 rows, s_V) the base-2 logits
    y = s_Q s_K (q8 . k8) / sqrt(d) / ln 2, T = floor(max y), P8 = E4M3(2^(7 + y - T)), the
    tile weighs its P8 v8 sums by 2^(T - 7) s_V; the normaliser sums 2^y."""
    d = len(q8)
    if not tiles:
        return [0.0] * d
    ys = [[sq * sk * dot(q8, kr) / math.sqrt(d) / math.log(2.0) for kr in k8s]
          for k8s, sk, _, _ in tiles]
    Ts = [math.floor(max(y)) for y in ys]
    G = max(Ts)
    num = [0.0] * len(tiles[0][2][0])
    den = 0.0
    for (_, _, v8s, sv), y, T in zip(tiles, ys, Ts):
        w = 2.0 ** (T - 7 - G) * sv
        for yn, vr in zip(y, v8s):
            p8 = e4m3_nearest(2.0 ** (7 + yn - T), table)
            for c in range(len(vr)):
                num[c] += w * p8 * vr[c]
            den += 2.0 ** (yn - G)
    return [x / den for x in num]
