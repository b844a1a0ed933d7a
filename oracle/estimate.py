"""Estimator, softmax, value sum, top-k and recall (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The estimator takes an uncompressed full-precision query against a packed key
(hao.cnyes.com "TurboQuant", heading "1 bit 掃尾"; xujun.org note 189244,
"第二步：QJL") and returns the stage-1 approximation plus the residual
correction (suzuke blog, "第三步"):
    l = nu * ( <Pi q, c[idx]> + alpha * gamma * <S q, 2 bits - 1> ),
    alpha = sqrt(pi/2) / m.
Logits are raw inner-product estimates; attention scaling 1/sqrt(d) is applied
by the softmax (standard scaled dot-product attention; the pages give no
scale).
"""

import numpy as np

from .quant import unpack_bits, unpack_codes


def prep_query(p, q):
    """(q_rot, q_s) = (Pi q, S q) for queries q[..., d]."""
    q = np.asarray(q, np.float64)
    q_rot = q @ p.Pi.T
    q_s = q @ p.S.T if p.mode == "prod" else None
    return q_rot, q_s


def scores_one(p, q, code_rec, sign_rec, norm, rnorm):
    """Logit of one query against one packed key, written out term by term."""
    q = np.asarray(q, np.float64)
    idx = unpack_codes(p, code_rec[None, :])[0]
    approx = float(np.dot(p.Pi @ q, p.c[idx]))
    if p.mode != "prod":
        return float(norm) * approx
    s = 2.0 * unpack_bits(sign_rec[None, :], 1, p.m)[0] - 1.0
    corr = p.alpha * float(rnorm) * float(np.dot(p.S @ q, s))
    return float(norm) * (approx + corr)


def scores(p, Q, codes, signs, norms, rnorms):
    """Logits [nq, n] of queries Q[nq, d] against n packed keys."""
    q_rot, q_s = prep_query(p, Q)
    idx = unpack_codes(p, codes)
    approx = q_rot @ p.c[idx].T                      # [nq, n]
    nu = np.asarray(norms, np.float64)[None, :]
    if p.mode != "prod":
        return nu * approx
    s = 2.0 * unpack_bits(signs, 1, p.m).astype(np.float64) - 1.0
    gamma = np.asarray(rnorms, np.float64)[None, :]
    return nu * (approx + p.alpha * gamma * (q_s @ s.T))


def softmax(logits, scale):
    """Row softmax of scale * logits (float64)."""
    z = scale * np.asarray(logits, np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def attend(pk, pv, Q, kcodes, ksigns, knorms, krnorms, vcodes, vnorms, scale):
    """One decode step for one KV group: Q[qpg, d] against T packed keys/values.

    Returns (logits [qpg, T], probs [qpg, T], out [qpg, d]) where
    out = sum_t probs[:, t] * vhat_t and vhat_t is the MSE-stage dequantized
    value nu_t Pi_v^T c_v[idx_t] (the value cache kept by the same codebook
    stage, xujun.org note 189244, "KV 缓存"; values are never scored, so they
    need no QJL bit).
    """
    from .quant import dequant
    logits = scores(pk, Q, kcodes, ksigns, knorms, krnorms)
    probs = softmax(logits, scale)
    vhat = dequant(pv, vcodes, None, vnorms, None)
    return logits, probs, probs @ vhat


def topk(score_matrix, k):
    """Per row: ids of the k largest scores, ordered by (score desc, id asc)."""
    S = np.asarray(score_matrix, np.float64)
    nq, n = S.shape
    ids = np.empty((nq, k), np.int64)
    vals = np.empty((nq, k), np.float64)
    cols = np.arange(n)
    for i in range(nq):
        order = np.lexsort((cols, -S[i]))[:k]
        ids[i] = order
        vals[i] = S[i, order]
    return ids, vals


def exact_top1(Q, X, chunk=4096, db_chunk=65536):
    """Exact inner-product top-1 per query (float64 dots; ties -> lower id).

    The database is visited in chunks in increasing id order; a later chunk
    replaces the running best only with a strictly larger dot product, so
    ties keep the lower id exactly as one argmax over all ids would."""
    Q = np.asarray(Q, np.float64)
    X = np.asarray(X)
    best = np.zeros(Q.shape[0], np.int64)
    bestv = np.full(Q.shape[0], -np.inf)
    for s in range(0, Q.shape[0], chunk):
        q = Q[s:s + chunk]
        for c0 in range(0, X.shape[0], db_chunk):
            sc = q @ X[c0:c0 + db_chunk].astype(np.float64).T
            j = np.argmax(sc, axis=1)                # first maximum = lower id
            v = sc[np.arange(len(q)), j]
            up = v > bestv[s:s + chunk]
            best[s:s + chunk][up] = c0 + j[up]
            bestv[s:s + chunk][up] = v[up]
    return best


def recall_at_k(ids, top1, k):
    """Fraction of queries whose exact top-1 is within the first k returned ids
    (recall 1@k, xujun.org note 189244, "常见问题")."""
    ids = np.asarray(ids)[:, :k]
    return float(np.mean(np.any(ids == np.asarray(top1)[:, None], axis=1)))
