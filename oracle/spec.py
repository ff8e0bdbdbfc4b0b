"""Speculative decoding's accept / resample step. TEST INFRASTRUCTURE ONLY.

Blog #54, interview question 3, and Part 8, "Thuật Toán Chấp Nhận & Từ Chối
Phỏng Đoán (Rejection Sampling)": the draft model proposes tokens x_1..x_K
with probabilities q_k(x_k); the target gives p_k over the same positions.
Token x_k is accepted with probability min(1, p_k(x_k) / q_k(x_k)); at the
first rejection the drafts after it are dropped and one token is drawn from
the residual max(0, p_k - q_k), renormalised. When every draft is accepted,
the target's pass over the drafts also yields the next token (Blog #54,
section 2.4 worked example: four drafts accepted, a fifth token produced),
drawn from p_{K+1}. The pages show that the resulting token has distribution
p exactly.

Readings taken where the pages leave the mechanics open (the kernel takes the
same decisions in the same arithmetic):
  * random numbers are inputs: one uniform u_k in [0, 1) (float32) per draft
    for the acceptance test, and one 32-bit integer U per sequence for the
    draw;
  * acceptance, in float32: accept iff p >= q, or u * q < p (u * q rounded
    once, to nearest even) -- u < p / q written without the division;
  * the draw is an inverse-CDF lookup in fixed point: each weight w(x) (the
    residual max(0, p - q) with p - q rounded once in float32, or p itself for
    the extra token) becomes the integer floor(w(x) * 2^32); with S the sum of
    those integers and T = floor(U * S / 2^32), the token drawn is the
    smallest x whose running sum exceeds T. Integer sums do not depend on
    their order, so the two sides agree bit for bit; the fixed point moves
    each probability by less than 2^-32 / S;
  * a residual whose integers are all zero (p and q equal to within 2^-32
    everywhere) draws from p instead.
"""
from __future__ import annotations

import numpy as np

FIXED_SHIFT = 32


def accept_draft(p_x: np.float32, q_x: np.float32, u: np.float32) -> bool:
    """The acceptance test for one drafted token (float32 arithmetic)."""
    p_x, q_x, u = np.float32(p_x), np.float32(q_x), np.float32(u)
    if p_x >= q_x:
        return True
    return bool(np.float32(u * q_x) < p_x)


def fixed_weights(w: np.ndarray) -> list:
    """floor(w * 2^32) for float32 weights in [0, 1], as Python integers."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)   # exact
    return [int(np.floor(x * 2.0 ** FIXED_SHIFT)) for x in w]


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """max(0, p - q) with the difference rounded once in float32."""
    d = np.asarray(p, dtype=np.float32) - np.asarray(q, dtype=np.float32)
    return np.maximum(d, np.float32(0.0))


def draw(weights: np.ndarray, U: int) -> int:
    """Inverse-CDF draw over fixed-point weights with a 32-bit uniform U."""
    ints = fixed_weights(weights)
    S = sum(ints)
    if S == 0:
        raise ValueError("all weights are zero")
    T = (int(U) * S) >> FIXED_SHIFT
    run = 0
    for x, v in enumerate(ints):
        run += v
        if run > T:
            return x
    raise AssertionError("unreachable: T < S")


def accept_sequence(p: np.ndarray, q: np.ndarray, draft, u_accept, U: int):
    """One sequence. p: [K+1][V], q: [K][V] float32 probabilities; draft: [K]
    token ids; u_accept: [K] float32; U: 32-bit integer.
    Returns (number of drafts accepted, tokens [K+1] with -1 past the end)."""
    K = len(draft)
    out = [-1] * (K + 1)
    for k in range(K):
        x = int(draft[k])
        if accept_draft(p[k][x], q[k][x], u_accept[k]):
            out[k] = x
            continue
        r = residual(p[k], q[k])
        if sum(fixed_weights(r)) == 0:
            r = np.asarray(p[k], dtype=np.float32)
        out[k] = draw(r, U)
        return k, out
    out[K] = draw(np.asarray(p[K], dtype=np.float32), U)
    return K, out


def accept_batch(p, q, draft, u_accept, U):
    """Batch: p [B][K+1][V], q [B][K][V], draft [B][K], u_accept [B][K], U [B]."""
    n = np.empty(len(draft), dtype=np.int32)
    toks = np.empty((len(draft), np.asarray(draft).shape[1] + 1), dtype=np.int32)
    for b in range(len(draft)):
        n[b], toks[b] = accept_sequence(p[b], q[b], draft[b], u_accept[b], int(U[b]))
    return n, toks
