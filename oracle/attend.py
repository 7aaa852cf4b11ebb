"""Plain fp64 CPU oracle for paged-KV POD attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. The product library never calls it and
shares no code with it.

What it computes is the plain definition of masked softmax attention, written
out per request and per query row, in float64 numpy. Sources (FlashInfer pages):

* POD article, www.dpshk.com/news/5405057
  - "plan 内部做了什么": per-request KV length from the page table
    (``get_seq_lens``): kv_len = (pages - 1) * page_size + last_page_len;
  - "plan/run 生命周期": num_qo_heads is a multiple of num_kv_heads, GQA otherwise;
  - "run 参数详解": sm_scale defaults to 1/sqrt(head_dim); outputs are one tensor
    per role, [rows, num_qo_heads, head_dim];
  - "批量 POD" example: NHD paged cache [pages, 2, page_size, num_kv_heads, head_dim].
* cuDNN backend article, www.gsyq.cn/news/452757
  - "Decode 能力矩阵与参数" table: rows of one request are consecutive; with
    q_len rows and kv_len keys, row i attends keys 0 .. kv_len - q_len + i
    (bottom-right causal); the left window keeps window_left keys strictly
    before the diagonal plus the diagonal itself; a sink is one extra softmax
    logit per qo head whose value row is zero;
  - "LSE 契约": lse is the base-2 log of the sum over valid keys of
    exp(scale * q . k).

Readings where the pages are silent (each listed with its reason in the design
notes of the repository):

* GQA mapping: qo head h reads kv head h // (num_qo_heads // num_kv_heads).
* Bottom-right causal alignment applies to every role (chunked prefill too).
* Window without causal: keys p - window_left .. kv_len - 1, p = kv_len - q_len + i.
* A sink is a raw natural-log logit (not multiplied by sm_scale); the returned
  lse excludes the sink while O includes it.
* A row with no valid key gives O = 0 and lse = -inf.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

LN2 = math.log(2.0)


class OracleInputError(ValueError):
    pass


def seq_lens(kv_indptr, last_page_len, page_size: int) -> np.ndarray:
    """KV length per request from the page table (POD article, "plan 内部做了什么")."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last_page_len = np.asarray(last_page_len, dtype=np.int64)
    pages = kv_indptr[1:] - kv_indptr[:-1]
    return (pages - 1) * page_size + last_page_len


def validate_role(qo_indptr, kv_indptr, last_page_len, page_size, num_qo_heads,
                  num_kv_heads, causal) -> None:
    """Input rules the pages state: heads divide, 1 <= last_page_len <= page_size,
    and causal rows need kv_len >= q_len (cuDNN article, decode parameter table)."""
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    lpl = np.asarray(last_page_len, dtype=np.int64)
    if num_qo_heads % num_kv_heads:
        raise OracleInputError("num_qo_heads must be a multiple of num_kv_heads")
    if qo_indptr[0] != 0 or kv_indptr[0] != 0:
        raise OracleInputError("indptr must start at 0")
    if np.any(np.diff(qo_indptr) < 0) or np.any(np.diff(kv_indptr) < 1):
        raise OracleInputError("qo_indptr non-decreasing; every request holds >= 1 page")
    if np.any(lpl < 1) or np.any(lpl > page_size):
        raise OracleInputError("1 <= last_page_len <= page_size")
    if causal:
        kv = seq_lens(kv_indptr, lpl, page_size)
        if np.any(kv < np.diff(qo_indptr)):
            raise OracleInputError("causal rows need kv_len >= q_len")


def logical_kv(k_pool, v_pool, kv_indptr, kv_indices, last_page_len, page_size: int,
               b: int, layout: str = "NHD") -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values of request b in logical order, float64 [kv_len, H_kv, D].

    Logical key j lives in physical page kv_indices[kv_indptr[b] + j // page_size],
    slot j % page_size (paged KV cache of the POD article, "批量 POD" example).
    """
    kv_len = int(seq_lens(kv_indptr[b:b + 2], last_page_len[b:b + 1], page_size)[0])
    j = np.arange(kv_len)
    pages = np.asarray(kv_indices)[kv_indptr[b] + j // page_size]
    slot = j % page_size
    if layout == "NHD":        # [P, page_size, H_kv, D]
        k = np.asarray(k_pool)[pages, slot]
        v = np.asarray(v_pool)[pages, slot]
    else:                      # HND: [P, H_kv, page_size, D]
        k = np.asarray(k_pool)[pages, :, slot]
        v = np.asarray(v_pool)[pages, :, slot]
    return k.astype(np.float64), v.astype(np.float64)


def valid_key_mask(qo_len: int, kv_len: int, causal: bool, window_left: int,
                   rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [n_rows, kv_len]: key j is visible to row i.

    Diagonal p_i = kv_len - qo_len + i (bottom-right). Causal keeps j <= p_i; a
    window keeps j >= p_i - window_left (cuDNN article, "Decode 能力矩阵与参数").
    """
    rows = np.arange(qo_len) if rows is None else np.asarray(rows)
    p = (kv_len - qo_len + rows)[:, None]
    j = np.arange(kv_len)[None, :]
    keep = np.ones((len(rows), kv_len), dtype=bool)
    if causal:
        keep &= j <= p
    if window_left >= 0:
        keep &= j >= p - window_left
    return keep


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray,
                sm_scale: float, sinks: Optional[np.ndarray] = None):
    """Masked softmax attention for a set of query rows of one request.

    q [n, H_qo, D]; k, v [kv_len, H_kv, D]; keep [n, kv_len].
    Returns O [n, H_qo, D] and lse [n, H_qo] (base 2, sink excluded), float64.
    """
    q = np.asarray(q, dtype=np.float64)
    n, hqo, d = q.shape
    hkv = k.shape[1]
    g = hqo // hkv
    o = np.zeros((n, hqo, d))
    lse = np.full((n, hqo), -np.inf)
    for h in range(hqo):
        kh = h // g
        s = sm_scale * (q[:, h, :] @ k[:, kh, :].T)          # [n, kv_len]
        s = np.where(keep, s, -np.inf)
        m = s.max(axis=1, initial=-np.inf)                   # [n]
        has = np.isfinite(m)
        msafe = np.where(has, m, 0.0)
        e = np.exp(s - msafe[:, None])                       # masked -> 0
        z = e.sum(axis=1)
        den = z.copy()
        if sinks is not None:
            den = den + np.exp(float(sinks[h]) - msafe)
        num = e @ v[:, kh, :]                                # [n, D]
        with np.errstate(invalid="ignore", divide="ignore"):
            o[:, h, :] = np.where(has[:, None], num / np.where(has, den, 1.0)[:, None], 0.0)
            lse[:, h] = np.where(has, (msafe + np.log(np.where(has, z, 1.0))) / LN2, -np.inf)
    return o, lse


def attend_role(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, last_page_len,
                page_size: int, num_qo_heads: int, num_kv_heads: int, causal: bool,
                window_left: int = -1, sm_scale: Optional[float] = None,
                sinks=None, layout: str = "NHD", requests=None, rows_of=None,
                validate: bool = True):
    """One role (prefill or decode) of a POD call, request by request.

    ``requests`` restricts the work to some request ids; ``rows_of`` maps a
    request id to the row indices (within the request) to compute. Returns
    dicts request -> (row ids, O, lse).
    """
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last_page_len = np.asarray(last_page_len, dtype=np.int64)
    if validate:
        validate_role(qo_indptr, kv_indptr, last_page_len, page_size, num_qo_heads,
                      num_kv_heads, causal)
    d = np.asarray(q).shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if kv_indices is None:
        kv_indices = np.arange(int(kv_indptr[-1]))
    kv_len = seq_lens(kv_indptr, last_page_len, page_size)
    sinks64 = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    res = {}
    reqs = range(len(qo_indptr) - 1) if requests is None else requests
    for b in reqs:
        qo_len = int(qo_indptr[b + 1] - qo_indptr[b])
        rows = np.arange(qo_len) if rows_of is None else np.asarray(rows_of(b))
        if len(rows) == 0:
            res[b] = (rows, np.zeros((0, num_qo_heads, d)), np.zeros((0, num_qo_heads)))
            continue
        k, v = logical_kv(k_pool, v_pool, kv_indptr, kv_indices, last_page_len, page_size,
                          b, layout)
        keep = valid_key_mask(qo_len, int(kv_len[b]), causal, window_left, rows)
        qb = np.asarray(q)[qo_indptr[b] + rows]
        o, lse = attend_rows(qb, k, v, keep, sm_scale, sinks64)
        res[b] = (rows, o, lse)
    return res


def attend_role_dense(*args, **kwargs):
    """attend_role over every request, stacked into [rows, H_qo, D] and [rows, H_qo]."""
    res = attend_role(*args, **kwargs)
    outs = [res[b][1] for b in sorted(res)]
    lses = [res[b][2] for b in sorted(res)]
    return np.concatenate(outs, axis=0), np.concatenate(lses, axis=0)


def merge_states(states):
    """Combine (O, lse) partial states over disjoint key sets (base-2 lse).

    L = log2 sum_k 2^lse_k and O = sum_k 2^(lse_k - L) O_k; a state with
    lse = -inf carries no keys and weighs 0. This is the cascade merge that
    the base-2 LSE contract of the cuDNN article feeds.
    """
    lses = np.stack([np.asarray(s[1], dtype=np.float64) for s in states])   # [S, ...]
    outs = np.stack([np.asarray(s[0], dtype=np.float64) for s in states])   # [S, ..., D]
    mx = lses.max(axis=0)
    has = np.isfinite(mx)
    msafe = np.where(has, mx, 0.0)
    w = np.exp2(lses - msafe)                                               # 0 where -inf
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.where(has, msafe + np.log2(np.where(has, tot, 1.0)), -np.inf)
        o = (w[..., None] * outs).sum(axis=0) / np.where(has, tot, 1.0)[..., None]
    o = np.where(has[..., None], o, 0.0)
    return o, L


def apply_sink(o, lse, sink):
    """Fold one per-head sink logit into a sink-free normalized state.

    O_sink = O / (1 + e^sink / 2^lse); the lse itself is unchanged.
    """
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    return o / (1.0 + np.exp(sink - lse * LN2))[..., None]


def e4m3_to_float(codes) -> np.ndarray:
    """Decode FP8 E4M3 bytes ("fn" variant: no infinities) to float64.

    Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
    Exponent field 0 holds the subnormals m/8 * 2^-6; every other field is
    (1 + m/8) * 2^(e - 7); only exponent 15 with mantissa 7 is NaN, so the
    largest finite magnitude is 1.75 * 2^8 = 448. This is the FP8 KV-cache
    element type whose calibration scales the POD article's run parameters
    (q_scale / k_scale / v_scale, "Decode 侧参数与'plan 覆盖'行为")
    describe.
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def attend_rows_fp8_scaled(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray,
                           sm_scale: float, q_scale: float, k_scale: float, v_scale: float,
                           sinks: Optional[np.ndarray] = None):
    """Decode attention over an FP8 KV cache with calibration scales (POD
    article, "Decode 侧参数与'plan 覆盖'行为": q_scale and k_scale multiply into the decode
    sm_scale; v_scale multiplies the decode output after the kernel).

    k, v hold the decoded FP8 values (float64). Returns O [n, H_qo, D] and the
    base-2 lse (sink excluded) of the scaled scores.
    """
    o, lse = attend_rows(q, k, v, keep, sm_scale * q_scale * k_scale, sinks)
    return o * v_scale, lse
