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
