"""Exact attention forward in fp64 on the CPU -- test infrastructure only.

What it computes (the definition, not an algorithm for computing it fast):

  O = softmax(scale * Q K^T + mask) V,   LSE_i = log sum_j exp(scale * q_i . k_j + mask_ij)

* The formula is the one stated at the top of "FlashAttention-3 Deep Dive"
  (mojostudio.in, introduction): softmax(Q K^T / sqrt(d_k)) V; ``scale``
  generalises 1/sqrt(d_k).  The pages call the method exact, so the oracle is
  the plain definition with the full score matrix materialised.
* The per-row log-sum-exp follows the softmax-statistics treatment listed in
  the Hopper tag page (l1-ca0.github.io, contents entry 4.6 "rescaling,
  correction, and LSE"); the section body is absent from the pages, so the
  reading is: natural log, including ``scale``, one fp32 value per query row.
* Causal: key j is masked for query i when j > i (top-left alignment; the
  configurations all have Sq == Sk where every convention agrees).
* GQA: query head h uses key/value head h // (Hq // Hkv) (consecutive groups;
  contents entry 9.5 of the Hopper tag page names GQA without a body).
* Varlen: cumulative offsets ``cu_seqlens`` cut the packed token axis into
  independent sequences ("FlashAttention-3 Deep Dive", FAQ on ragged
  batches); indices inside a sequence are local.
* A row that sees no key (empty sequence, Sk == 0) gets O = 0, LSE = -inf.

Rows are independent, so rows may be processed in chunks to bound memory, but
each row is computed completely (no streaming rescale).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Upcast the exact values the kernel consumes (torch or numpy) to fp64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", dtype=torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def head_probs(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
               rows: Optional[np.ndarray] = None, key_offset: int = 0, softcap: float = 0.0):
    """Softmax probabilities for one head.

    q [Sq, d], k [Sk, d] (fp64).  Returns (P [R, Sk], m [R], l [R]) for the
    selected query rows (all rows if ``rows`` is None), where
    P = exp(S - m) / l, S = scale * q k^T with -inf on masked entries,
    m = row max of S, l = sum_j exp(S_ij - m_i).  ``key_offset`` is the
    position of k's first row in the key sequence (for the causal mask).
    ``softcap`` > 0 caps the scores before the mask: S = softcap *
    tanh(scale q k^T / softcap) (attention softcapping, named in the API
    surface of "FlashAttention-3 Deep Dive" without a formula; this is the
    usual logit soft-capping).
    """
    Sq, Sk = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(Sq)
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)                      # [R, Sk]
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    if causal:
        j = key_offset + np.arange(Sk)[None, :]
        s = np.where(j > rows[:, None], -np.inf, s)
    m = s.max(axis=1) if Sk > 0 else np.full(len(rows), -np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m_safe[:, None])                  # exp(-inf) = 0 on masked entries
    l = p.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[:, None] > 0, p / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return p, m, l


def head_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                   rows: Optional[np.ndarray] = None, row_chunk: int = 1024, key_offset: int = 0,
                   softcap: float = 0.0):
    """Attention for one head: q [Sq, d], k/v [Sk, d] -> (O [R, d], LSE [R])."""
    Sq = q.shape[0]
    if rows is None:
        rows = np.arange(Sq)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    L = np.full(len(rows), -np.inf, dtype=np.float64)
    for c0 in range(0, len(rows), row_chunk):
        r = rows[c0:c0 + row_chunk]
        p, m, l = head_probs(q, k, scale, causal, r, key_offset, softcap)
        O[c0:c0 + len(r)] = p @ v
        with np.errstate(divide="ignore"):
            L[c0:c0 + len(r)] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, L


def attention(q, k, v, scale: float, causal: bool = False, cu_seqlens=None,
              heads: Optional[Sequence[int]] = None, rows: Optional[np.ndarray] = None,
              batches: Optional[Sequence[int]] = None, softcap: float = 0.0):
    """Exact attention forward in fp64 (``softcap`` as in ``head_probs``).

    Dense:  q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d]  ->  O [B, Sq, Hq, d], LSE [B, Hq, Sq]
    Varlen: q [T, Hq, d],     k/v [T, Hkv, d], cu_seqlens [nseq+1]
                                                    ->  O [T, Hq, d],    LSE [Hq, T]

    ``heads`` / ``batches`` / ``rows`` restrict the work to a subset (dense
    only); entries outside the subset are left as NaN so that a caller can
    compare only what was computed.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        T, Hq, d = q.shape
        O = np.zeros((T, Hq, d))
        L = np.full((Hq, T), -np.inf)
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            if b <= a:
                continue
            o_s, l_s = attention(q[None, a:b], k[None, a:b], v[None, a:b], scale, causal, softcap=softcap)
            O[a:b] = o_s[0]
            L[:, a:b] = l_s[0]
        return O, L
    B, Sq, Hq, d = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    hs = range(Hq) if heads is None else heads
    bs = range(B) if batches is None else batches
    partial = heads is not None or rows is not None or batches is not None
    O = np.full((B, Sq, Hq, v.shape[3]), np.nan if partial else 0.0)
    L = np.full((B, Hq, Sq), np.nan if partial else -np.inf)
    rsel = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    for b in bs:
        for h in hs:
            hk = h // group
            o, l = head_attention(q[b, :, h], k[b, :, hk], v[b, :, hk], scale, causal, rsel, softcap=softcap)
            O[b, rsel, h] = o
            L[b, h, rsel] = l
    return O, L


def partial_attention(q, k, v, scale: float, causal: bool, key_lo: int, key_hi: int):
    """Attention of every query over the keys [key_lo, key_hi) only: the
    partial state one split of the key axis produces in flash-decoding
    (Hopper tag page, contents 10 "Split-KV and the Combine Kernel", 10.2
    parallelisation over the KV sequence; the section bodies are absent from
    the pages, so this is the plain reading).  Dense layout as ``attention``;
    causal positions are absolute (key j hidden from query i when j > i).
    Returns (O_p [B, Sq, Hq, d], LSE_p [B, Hq, Sq]); a row that sees no key of
    the range gets O_p = 0 and LSE_p = -inf.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Sq, Hq, d = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    lo, hi = max(0, key_lo), min(k.shape[1], key_hi)
    O = np.zeros((B, Sq, Hq, v.shape[3]))
    L = np.full((B, Hq, Sq), -np.inf)
    if hi <= lo:
        return O, L
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            o, l = head_attention(q[b, :, h], k[b, lo:hi, hk], v[b, lo:hi, hk], scale, causal,
                                  key_offset=lo)
            O[b, :, h] = o
            L[b, h] = l
    return O, L


def combine(o_parts, lse_parts):
    """Merge attention results over disjoint key sets into the result over
    their union (the block-combine of two softmax states, Hopper tag page
    contents 3.2.1, used for the split-KV combine, contents 10.2.1):

        LSE = log sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) * O_p

    o_parts [P, B, Sq, Hq, d], lse_parts [P, B, Hq, Sq] (natural-log LSE, O_p
    normalised).  A part with LSE_p = -inf contributes nothing; a row whose
    parts are all -inf gets O = 0, LSE = -inf.
    """
    o_parts = _as_f64(o_parts)
    lse_parts = _as_f64(lse_parts)
    m = lse_parts.max(axis=0)                                   # [B, Hq, Sq]
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe[None])                        # [P, B, Hq, Sq]; 0 for -inf parts
    wsum = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(wsum > 0, m_safe + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    wn = np.where(wsum[None] > 0, w / np.where(wsum > 0, wsum, 1.0)[None], 0.0)
    wo = np.transpose(wn, (0, 1, 3, 2))[..., None]              # [P, B, Sq, Hq, 1]
    o_safe = np.where(wo > 0, o_parts, 0.0)
    return (wo * o_safe).sum(axis=0), lse


def attention_flops(Sq: int, Sk: int, d: int, causal: bool, B: int = 1, H: int = 1,
                    lengths: Optional[Sequence[int]] = None) -> float:
    """Algorithmic FLOPs: 4*d per unmasked (query, key) pair (two GEMMs,
    multiply + add each); masked pairs are not counted."""
    def pairs(sq, sk):
        if not causal:
            return sq * sk
        n = min(sq, sk)
        return n * (n + 1) // 2 + max(0, sq - sk) * sk
    if lengths is not None:
        return 4.0 * d * H * sum(pairs(n, n) for n in lengths)
    return 4.0 * d * B * H * pairs(Sq, Sk)


# ---------------------------------------------------------------- backward
def head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float, causal: bool,
                  dlse: Optional[np.ndarray] = None, row_chunk: int = 1024):
    """Gradients of one head's attention (fp64): q [Sq, d], k/v [Sk, d], the
    output gradient do [Sq, d] and optionally the gradient of the LSE output
    dlse [Sq]  ->  (dq [Sq, d], dk [Sk, d], dv [Sk, d]).

    Chain rule through the definition (the backward gradient math listed in
    the Hopper tag page, contents 7.1 -- 7.1.5; the section bodies are absent
    from the pages, so this is the textbook derivation):
      P = softmax(S), S = scale * q k^T (masked entries -inf, P = 0 there)
      dV = P^T dO,  dP = dO V^T,
      dS_ij = P_ij (dP_ij - D_i + dlse_i),  D_i = sum_j P_ij dP_ij = dO_i . O_i
        (the softmax Jacobian; dLSE_i / dS_ij = P_ij adds the dlse term),
      dQ = scale * dS K,  dK = scale * dS^T Q   (the scale is applied last).
    Rows are independent in P and dS, so they may be taken in chunks; dK and
    dV are sums over all rows.
    """
    Sq, d = q.shape
    Sk = k.shape[0]
    dq = np.zeros((Sq, d))
    dk = np.zeros((Sk, k.shape[1]))
    dv = np.zeros((Sk, v.shape[1]))
    for c0 in range(0, Sq, row_chunk):
        r = np.arange(c0, min(Sq, c0 + row_chunk))
        p, _, _ = head_probs(q, k, scale, causal, r)      # [R, Sk], rows of P
        o = p @ v
        dor = do[r]
        dv += p.T @ dor
        dp = dor @ v.T
        D = (dor * o).sum(axis=1)
        if dlse is not None:
            D = D - dlse[r]
        ds = p * (dp - D[:, None])
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv


def attention_backward(q, k, v, do, scale: float, causal: bool = False, dlse=None, cu_seqlens=None):
    """Gradients of exact attention in fp64 (see ``head_backward``).

    Dense:  q, do [B, Sq, Hq, d]; k, v [B, Sk, Hkv, d]; dlse [B, Hq, Sq] or None
            -> dq [B, Sq, Hq, d], dk, dv [B, Sk, Hkv, d]
    Varlen: q, do [T, Hq, d]; k, v [T, Hkv, d]; dlse [Hq, T] or None; cu_seqlens
            -> dq [T, Hq, d], dk, dv [T, Hkv, d]
    With GQA the gradient of a KV head is the sum over the query heads that
    read it.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    dl = None if dlse is None else _as_f64(dlse)
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            if b <= a:
                continue
            g = attention_backward(q[None, a:b], k[None, a:b], v[None, a:b], do[None, a:b], scale, causal,
                                   None if dl is None else dl[None, :, a:b])
            dq[a:b], dk[a:b], dv[a:b] = g[0][0], g[1][0], g[2][0]
        return dq, dk, dv
    B, Sq, Hq, d = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            gq, gk, gv = head_backward(q[b, :, h], k[b, :, hk], v[b, :, hk], do[b, :, h], scale, causal,
                                       None if dl is None else dl[b, h])
            dq[b, :, h] = gq
            dk[b, :, hk] += gk
            dv[b, :, hk] += gv
    return dq, dk, dv


def attention_backward_flops(Sq: int, Sk: int, d: int, causal: bool, B: int = 1, H: int = 1) -> float:
    """Algorithmic FLOP of the backward: five GEMMs of 2 d FLOP per unmasked
    (query, key) pair each (recomputed S, dV, dP, dQ, dK) = 10 d per pair,
    2.5 times the forward's 4 d."""
    return 2.5 * attention_flops(Sq, Sk, d, causal, B=B, H=H)
