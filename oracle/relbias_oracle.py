"""Reference oracle for causal attention with a learned relative-position bias.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it shares no
code with that path.

What it computes (plain definition, float64, no tiling, no online softmax):

  For batch b, query head h (kv head g = floor(h / G)), query row i, key j:
    delta_ij = qpos[i] - kpos[j]
    visible_ij  <=>  delta_ij >= 0  and  (window == 0  or  delta_ij < window)
    beta(h, i, delta) = 0                          if mode == NONE or delta >= bias_range
                      = table[h, delta]            if mode == TABLE
                      = sum_f r[b,i,h,f] E[h,f,delta]   if mode == RPROJ
                      = sum_f r[b,i,h,f] E[f,delta]     if mode == RPROJ_SHARED
    s_ij = scale * <q[b,i,h,:], k[b,j,g,:]> + beta(h, i, delta_ij)
    optional temperature (temp_len > 0): s_ij <- tau(n_i) * s_ij, with n_i the
      number of keys query i sees and tau(n) = max(1, ln n / ln temp_len)
    o[b,i,h,:] = sum_{visible j} softmax_j(s_ij) v[b,j,g,:]
    lse[b,h,i] = log sum_{visible j} exp(s_ij)

Sources (pages on learned relative-position bias attention):
  * "Learned Relative-Position Bias" (codewithdark concepts page), section
    "Standard Relative Bias (T5-style)": scores are q.k / sqrt(d) plus a bias
    that depends on the distance i-j; section "Inkling's Input-Dependent
    Version (Conceptual)": local layers use the bias below a 512 distance,
    global layers below 1024 and a zero bias (content-only, NoPE) beyond.
  * "Thinking Machines dropped RoPE" (wpnews essay), the five numbered steps
    of the Inkling bias: per-token, per-head coefficients (step 1) weight a
    bank of learned distance functions (step 2); the curve is read at the
    query-key distance (step 3), forced to zero outside the hard-coded range
    and for keys ahead of the query (step 4), and added to the score before
    the softmax next to the causal mask (step 5).  The code listing on that
    page reads the curve of the *query* row at distance i-j and zeroes
    distances < 0 and >= the range.
  * Same essay, section "Option 3: position as a bias to the attention": the
    T5 form is a learned table indexed by distance, shared by all tokens.

Readings where the pages are silent or garbled (each is pinned by a test):
  * the bias is added after the content scale, not multiplied by it;
  * the window keeps keys with 0 <= delta < window (window keys including the
    query itself); window == 0 means no window (full causal);
  * the bias applies for 0 <= delta < bias_range and is exactly 0 at
    delta == bias_range;
  * the table is causal only (no negative-offset half, no buckets);
  * the bank E is per head ([Hq, R, bias_range]) in mode RPROJ; mode
    RPROJ_SHARED takes the essay's form, one bank [R, bias_range] that every
    head reads (step 2 of the same essay: the learned distance functions are
    common to all heads and tokens of the layer);
  * GQA: query head h reads kv head floor(h / G), G = Hq / Hkv.
  * context-length temperature ("Thinking Machines dropped RoPE", section "The
    temperature scale is dependent on context length"): global layers multiply
    the queries and the position bias by a factor of the number n of keys the
    query sees, flat up to 128k and growing logarithmically after; the page's
    formula is missing, and the plain log-n reading taken here is
    tau(n) = max(1, ln n / ln temp_len) with temp_len = 131072 for that page
    (an argument, so that small cases reach tau > 1).  It scales the whole
    logit, content term and bias alike.

Inputs are taken as stored (bf16 / fp32 values upcast to float64).

attention_backward / prefill_backward give the gradients of the same definition (chain rule
written out per batch and head); they are pinned against torch autograd through SDPA, central
finite differences and exact identities of the softmax gradient.
"""

from __future__ import annotations

import numpy as np

MODE_NONE = 0
MODE_TABLE = 1
MODE_RPROJ = 2
MODE_RPROJ_SHARED = 3

_MODES = {"none": MODE_NONE, "table": MODE_TABLE, "rproj": MODE_RPROJ,
          "rproj_shared": MODE_RPROJ_SHARED,
          MODE_NONE: MODE_NONE, MODE_TABLE: MODE_TABLE, MODE_RPROJ: MODE_RPROJ,
          MODE_RPROJ_SHARED: MODE_RPROJ_SHARED}


def _f64(x):
    """Upcast a numpy array or a torch tensor (any dtype, any device) to float64 numpy."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype, go through float64
        import torch  # local import: the oracle itself only needs numpy
        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def visible_mask(qpos, kpos, window):
    """Boolean [Sq, Sk]: key j visible to query i (causal, optional sliding window).

    Causal: keys ahead of the query are masked ("Thinking Machines dropped RoPE",
    step 4 and step 5).  Window: "Learned Relative-Position Bias", section
    "Hybrid Attention Interaction" (local layers use a 512 window); read here
    as 0 <= delta < window.
    """
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    delta = qpos[:, None] - kpos[None, :]
    vis = delta >= 0
    if window:
        vis &= delta < window
    return vis


def bias_matrix(mode, qpos, kpos, bias_range, h, *, table=None, r_rows=None, E=None):
    """Bias beta[i, j] for query head h, float64 [Sq, Sk].

    Only pairs at a distance d = qpos[i] - kpos[j] with 0 <= d < bias_range carry a bias; every
    other pair (keys ahead of the query, keys at or beyond the range) gets exactly 0 ("Thinking
    Machines dropped RoPE", step 4).  For an in-band pair:
      mode TABLE: table[h, d], the learned value of that distance ("Learned Relative-Position
        Bias", section "Standard Relative Bias (T5-style)", causal half only);
      mode RPROJ: sum_f r_rows[i, f] * E[h, f, d], the query token's coefficients weighting the
        bank of distance functions, each read at d ("Thinking Machines dropped RoPE", steps 1-3);
        r_rows is r[b, :, h, :] for the query rows, [Sq, R];
      mode RPROJ_SHARED: the same with one bank E [R, bias_range] for every head (same essay,
        step 2).
    """
    mode = _MODES[mode]
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    out = np.zeros((len(qpos), len(kpos)), dtype=np.float64)
    if mode == MODE_NONE:
        return out
    dist = qpos[:, None] - kpos[None, :]
    ii, jj = np.nonzero((dist >= 0) & (dist < bias_range))     # the in-band pairs
    d = dist[ii, jj]
    if mode == MODE_TABLE:
        out[ii, jj] = _f64(table)[h][d]
    else:
        bank = _f64(E) if mode == MODE_RPROJ_SHARED else _f64(E)[h]    # [R, bias_range]
        coef = _f64(r_rows)                                            # [Sq, R]
        # per pair: the query row's coefficients dotted with the bank column at the distance
        out[ii, jj] = np.einsum("pf,fp->p", coef[ii], bank[:, d])
    return out


def temperature(n_visible, temp_len):
    """Context-length temperature tau(n) = max(1, ln n / ln temp_len); 1 when temp_len == 0.

    "Thinking Machines dropped RoPE", section "The temperature scale is dependent
    on context length": flat until the threshold, logarithmic growth beyond.
    """
    n = np.asarray(n_visible, dtype=np.float64)
    if not temp_len:
        return np.ones_like(n)
    if temp_len < 2:
        raise ValueError("temp_len must be 0 or >= 2")
    return np.maximum(1.0, np.log(np.maximum(n, 1.0)) / np.log(float(temp_len)))


def attention(q, k, v, *, qpos, kpos, scale, window=0, bias_range=0, mode="none",
              table=None, r=None, E=None, rows=None, row_block=512, temp_len=0):
    """Plain definition of relative-position-bias attention, float64.

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D]; r [B, Sq, Hq, R] (RPROJ, RPROJ_SHARED);
    table [Hq, bias_range] (TABLE); E [Hq, R, bias_range] (RPROJ) or
    [R, bias_range] (RPROJ_SHARED).
    qpos [Sq], kpos [Sk]: integer token positions.
    rows: optional 1-D array of query-row indices to evaluate (others skipped).
    temp_len: context-length temperature threshold (0: none); the logit of a row
    that sees n keys is multiplied by temperature(n, temp_len).
    Returns (o [B, len(rows), Hq, D], lse [B, Hq, len(rows)]) in float64.

    Formula: "Learned Relative-Position Bias", section "Standard Relative Bias
    (T5-style)" (score = scaled content term + distance bias), with the bias of
    "Thinking Machines dropped RoPE", steps 1-5.  The softmax is the ordinary
    max-subtracted one over the visible keys of each row.
    """
    mode = _MODES[mode]
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q64.shape
    Hkv = k64.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    rproj = mode in (MODE_RPROJ, MODE_RPROJ_SHARED)
    r64 = _f64(r) if rproj else None
    tab64 = _f64(table) if mode == MODE_TABLE else None
    E64 = _f64(E) if rproj else None
    n = len(rows)
    o = np.zeros((B, n, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, n), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kk = k64[b, :, g, :]                   # [Sk, D]
            vv = v64[b, :, g, :]
            # keep one row block's [rows, keys] arrays near 8M elements
            step = max(1, min(row_block, (8 << 20) // max(1, kk.shape[0])))
            for s0 in range(0, n, step):
                rr = rows[s0:s0 + step]
                qq = q64[b, rr, h, :]              # [n_r, D]
                logits = scale * (qq @ kk.T)       # [n_r, Sk]
                beta = bias_matrix(mode, qpos[rr], kpos, bias_range, h, table=tab64,
                                   r_rows=None if r64 is None else r64[b, rr, h, :], E=E64)
                logits = logits + beta
                vis = visible_mask(qpos[rr], kpos, window)
                logits = logits * temperature(vis.sum(axis=1), temp_len)[:, None]
                logits = np.where(vis, logits, -np.inf)
                m = logits.max(axis=1, keepdims=True)
                if not np.all(np.isfinite(m)):
                    raise ValueError("a query row sees no key")
                p = np.exp(logits - m)
                l = p.sum(axis=1, keepdims=True)
                o[b, s0:s0 + len(rr), h, :] = (p @ vv) / l
                lse[b, h, s0:s0 + len(rr)] = (m + np.log(l))[:, 0]
    return o, lse


def prefill(q, k, v, *, scale, window=0, bias_range=0, mode="none", table=None, r=None,
            E=None, rows=None, row_block=512, temp_len=0):
    """Prefill: query i and key j sit at positions i and j (one sequence per batch row)."""
    S = q.shape[1]
    pos = np.arange(S, dtype=np.int64)
    return attention(q, k, v, qpos=pos, kpos=pos, scale=scale, window=window,
                     bias_range=bias_range, mode=mode, table=table, r=r, E=E, rows=rows,
                     row_block=row_block, temp_len=temp_len)


def decode(q, k_cache, v_cache, kv_len, *, scale, window=0, bias_range=0, mode="none",
           table=None, r=None, E=None, batch=None, temp_len=0):
    """Single-token decode against a KV cache.

    q [B, Hq, D] is the newest token, at position kv_len - 1; the cache already
    holds that token's own key/value at index kv_len - 1 (rows >= kv_len are
    ignored).  r [B, Hq, R] is that token's coefficients.  batch: optional list
    of batch indices to evaluate.  Returns (o [nb, Hq, D], lse [nb, Hq]).
    """
    bidx = range(q.shape[0]) if batch is None else list(batch)
    qpos = np.array([kv_len - 1], dtype=np.int64)
    kpos = np.arange(kv_len, dtype=np.int64)
    outs, lses = [], []
    for b in bidx:
        qb = q[b:b + 1][:, None]                    # [1, 1, Hq, D]
        kb = k_cache[b:b + 1, :kv_len]
        vb = v_cache[b:b + 1, :kv_len]
        rb = None if r is None else r[b:b + 1][:, None]
        o, l = attention(qb, kb, vb, qpos=qpos, kpos=kpos, scale=scale, window=window,
                         bias_range=bias_range, mode=mode, table=table, r=rb, E=E,
                         temp_len=temp_len)
        outs.append(o[0, 0])
        lses.append(l[0, :, 0])
    return np.stack(outs), np.stack(lses)



def attention_backward(q, k, v, dout, *, qpos, kpos, scale, window=0, bias_range=0,
                       mode="none", table=None, r=None, E=None, temp_len=0):
    """Gradients of attention() for an upstream gradient dout on o, float64.

    The bias is learned ("Thinking Machines dropped RoPE": the bank of distance functions
    and the coefficient projection are trained with the model; "Learned Relative-Position
    Bias", section "Standard Relative Bias (T5-style)": the table is a learned parameter),
    so the parameters that shape it get gradients too.  Plain chain rule of the definition,
    per (batch, head), no tiling:
      P = softmax of the masked logits s, o = P v
      dP = dout v^T,  dS = P * (dP - rowsum(dout * o))      (gradient on s)
      dZ = tau * dS      (gradient on scale * q.k + beta; tau = temperature, 1 if none)
      dq = scale * dZ k,  dk = scale * dZ^T q,  dv = P^T dout   (GQA: kv heads sum their
      query heads)
      beta's gradient is dZ at the in-band pairs (0 <= delta < bias_range):
        TABLE:  dtable[h, d] = sum of dZ over the pairs at distance d
        RPROJ:  with dC[i, d] = sum of dZ[i, j] over keys at distance d from query i,
                dr[b, i, h, :] = dC[i] @ E[h]^T  and  dE[h] += r[b, :, h, :]^T @ dC
        RPROJ_SHARED: the same with E [R, bias_range], dE summed over heads.

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D], dout like q.  Returns a dict with dq, dk, dv and
    dtable (TABLE) or dr and dE (RPROJ, RPROJ_SHARED).
    """
    mode = _MODES[mode]
    q64, k64, v64, do64 = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, D = q64.shape
    Hkv = k64.shape[2]
    G = Hq // Hkv
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    rproj = mode in (MODE_RPROJ, MODE_RPROJ_SHARED)
    r64 = _f64(r) if rproj else None
    E64 = _f64(E) if rproj else None
    tab64 = _f64(table) if mode == MODE_TABLE else None
    dq = np.zeros_like(q64)
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    out = {"dq": dq, "dk": dk, "dv": dv}
    if mode == MODE_TABLE:
        out["dtable"] = np.zeros_like(tab64)
    if rproj:
        out["dr"] = np.zeros_like(r64)
        out["dE"] = np.zeros_like(E64)
    delta = qpos[:, None] - kpos[None, :]
    vis = visible_mask(qpos, kpos, window)
    tau = temperature(vis.sum(axis=1), temp_len)[:, None]
    inband = vis & (delta >= 0) & (delta < bias_range) if mode != MODE_NONE else None
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qq, kk, vv, dd = q64[b, :, h, :], k64[b, :, g, :], v64[b, :, g, :], do64[b, :, h, :]
            beta = bias_matrix(mode, qpos, kpos, bias_range, h, table=tab64,
                               r_rows=None if r64 is None else r64[b, :, h, :], E=E64)
            s = np.where(vis, tau * (scale * (qq @ kk.T) + beta), -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ vv
            dp = dd @ vv.T
            ds = p * (dp - (dd * o).sum(axis=1, keepdims=True))
            dz = tau * ds
            dq[b, :, h, :] = scale * (dz @ kk)
            dk[b, :, g, :] += scale * (dz.T @ qq)
            dv[b, :, g, :] += p.T @ dd
            if mode == MODE_NONE:
                continue
            ii, jj = np.nonzero(inband)
            dist = delta[ii, jj]
            if mode == MODE_TABLE:
                np.add.at(out["dtable"][h], dist, dz[ii, jj])
            else:
                dC = np.zeros((Sq, bias_range))
                np.add.at(dC, (ii, dist), dz[ii, jj])
                bank = E64 if mode == MODE_RPROJ_SHARED else E64[h]    # [R, bias_range]
                out["dr"][b, :, h, :] = dC @ bank.T
                gE = r64[b, :, h, :].T @ dC                            # [R, bias_range]
                if mode == MODE_RPROJ_SHARED:
                    out["dE"] += gE
                else:
                    out["dE"][h] += gE
    return out


def prefill_backward(q, k, v, dout, *, scale, window=0, bias_range=0, mode="none", table=None,
                     r=None, E=None, temp_len=0):
    """attention_backward for a prefill (query i and key j at positions i and j)."""
    S = q.shape[1]
    pos = np.arange(S, dtype=np.int64)
    return attention_backward(q, k, v, dout, qpos=pos, kpos=pos, scale=scale, window=window,
                              bias_range=bias_range, mode=mode, table=table, r=r, E=E,
                              temp_len=temp_len)
