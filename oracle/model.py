"""Oracle: the math of one Orca iteration, written out plainly (numpy, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (pages and the part of each that is followed):
  [houmin]   garden.houmin.site/infra/orca, section 3.1.2 (selective batching):
             flatten all tokens of the batch into one [sum L, H] matrix for
             Linear/GeLU/LayerNorm/Add; a fused QKV Linear yields 3H columns
             (H of Q, H of K, H of V); split per request before attention,
             run attention per request, merge back to [sum L, H]; the phase of
             a request is known from whether the K/V manager holds a cache for
             it; each token's K/V cache entry is one [1, H] vector per layer.
  [0h-n0]    0h-n0.github.io paper digest of Orca, "Technical Details /
             Selective Batching": concat(X_1..X_n) in R^{(sum L_i) x H} for
             non-attention ops; split -> per request -> merge for attention.
  [arcsin2]  unpurerationalist.github.io notes on ORCA, section 3.2: the same
             split / merge around attention, the K/V manager appending each
             request's history.
  [estelledc] estelledc.github.io study notes, case 2: prompts of 128, 64 and
             256 tokens flatten into one 448-row matrix.

Readings where the pages leave a step open (each is listed in the design notes):
  * block structure: GPT-2/3 style pre-LayerNorm decoder block with a bias on
    all four Linear layers (the pages name LN, Linear, Add and GeLU only);
  * GeLU is the tanh approximation (Hendrycks & Gimpel 2016, eq. for GELU);
  * LayerNorm uses the population variance and eps inside the square root;
  * QKV columns are blocked [Q | K | V], heads contiguous inside each block;
  * scaled dot-product attention with scale 1/sqrt(d), d = H / heads; a query
    at absolute position p sees keys 0..p of its own request only;
  * "KV length" of a request is the number of entries cached BEFORE the
    iteration; its new K/V rows are appended at positions kv_len .. kv_len+q_len-1
    before attention, so an increment attends over kv_len + 1 keys;
  * Linear weights are stored [out, in] (row n produces output column n):
    y = a @ W.T + b.

Every function takes and returns numpy arrays; the dtype of the computation is
the dtype of the inputs (float64 by default in the tests).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

INITIATION = 0
INCREMENT = 1

LAYER_KEYS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
              "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2")


@dataclass(frozen=True)
class Req:
    """One request's slice of the flattened batch.

    q_offset, q_len: rows [q_offset, q_offset + q_len) of the [sum L, H] matrix
    kv_len:          cached K/V entries before this iteration
    [houmin] 3.1.2: a request with no cache yet is in the initiation phase.
    """
    q_offset: int
    q_len: int
    kv_len: int

    @property
    def phase(self) -> int:
        return INITIATION if self.kv_len == 0 else INCREMENT


# ---------------------------------------------------------------- elementwise

def layer_norm(z: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
               eps: float) -> np.ndarray:
    """Row-wise LayerNorm: (z - mean) / sqrt(var + eps) * gamma + beta.

    [0h-n0] Implementation notes: LayerNorm statistics and scaling are one
    fused operation.  Population variance (divide by H), eps inside the root.
    """
    mean = z.mean(axis=-1, keepdims=True)
    var = ((z - mean) ** 2).mean(axis=-1, keepdims=True)
    return (z - mean) / np.sqrt(var + eps) * gamma + beta


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GeLU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).

    [0h-n0] Implementation notes name a fused GeLU; the tanh form is the one
    the GPT family uses (Hendrycks & Gimpel 2016).
    """
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * z * (1.0 + np.tanh(c * (z + 0.044715 * z ** 3)))


def linear(a: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a @ W^T + b with W stored [out, in].  [houmin] 3.1.2: Linear runs on
    the flattened [sum L, H] matrix because it mixes no tokens."""
    return a @ w.T + b


# ------------------------------------------------------------------ attention

def request_attention(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray,
                      kv_len: int, heads: int) -> np.ndarray:
    """Attention of one request's q_len query rows over its own keys.

    q:      [q_len, H]  the request's query rows of this iteration
    k_all:  [kv_len + q_len, H]  cached keys followed by this iteration's keys
    v_all:  same shape, values
    Query j sits at absolute position p = kv_len + j and sees keys 0..p.
    Initiation (kv_len = 0) is causal attention over the prompt; increment
    (q_len = 1) is one query over the request's cache plus its own new key.
    [houmin] 3.1.2: attention runs separately for every request of the batch.
    """
    q_len, hidden = q.shape
    d = hidden // heads
    n_keys = k_all.shape[0]
    assert n_keys == kv_len + q_len
    out = np.zeros_like(q)
    pos = kv_len + np.arange(q_len)[:, None]          # [q_len, 1]
    key = np.arange(n_keys)[None, :]                  # [1, n_keys]
    visible = key <= pos                              # [q_len, n_keys]
    for h in range(heads):
        cols = slice(h * d, (h + 1) * d)
        s = q[:, cols] @ k_all[:, cols].T / math.sqrt(d)
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        out[:, cols] = p @ v_all[:, cols]
    return out


# ------------------------------------------------------- the selective iteration

def _check_batch(reqs: Sequence[Req], rows: int) -> None:
    off = 0
    for r in reqs:
        assert r.q_offset == off and r.q_len >= 1 and r.kv_len >= 0
        off += r.q_len
    assert off == rows


def selective_layer(p: dict, reqs: Sequence[Req], x: np.ndarray,
                    caches: Sequence[Tuple[np.ndarray, np.ndarray]],
                    heads: int, eps: float):
    """One decoder layer over the flattened batch, with selective batching.

    x:       [sum L, H] flattened rows of every request ([houmin] 3.1.2,
             [0h-n0] Selective Batching, [arcsin2] 3.2)
    caches:  per request (K, V), each [kv_len, H]: this layer's cache
    returns  (y [sum L, H], per-request (K_new, V_new) each [q_len, H])
    """
    hidden = x.shape[1]
    _check_batch(reqs, x.shape[0])
    a = layer_norm(x, p["ln1_g"], p["ln1_b"], eps)            # batched
    qkv = linear(a, p["w_qkv"], p["b_qkv"])                   # batched: [sum L, 3H]
    q = qkv[:, :hidden]
    k = qkv[:, hidden:2 * hidden]
    v = qkv[:, 2 * hidden:]
    o = np.zeros_like(x)
    appended = []
    for r, (kc, vc) in zip(reqs, caches):                      # split
        rows = slice(r.q_offset, r.q_offset + r.q_len)
        assert kc.shape == (r.kv_len, hidden) and vc.shape == (r.kv_len, hidden)
        k_all = np.concatenate([kc, k[rows]], axis=0)          # K/V manager append
        v_all = np.concatenate([vc, v[rows]], axis=0)
        o[rows] = request_attention(q[rows], k_all, v_all, r.kv_len, heads)
        appended.append((k[rows].copy(), v[rows].copy()))      # merge = same rows
    h1 = x + linear(o, p["w_o"], p["b_o"])                     # batched
    c = layer_norm(h1, p["ln2_g"], p["ln2_b"], eps)
    f = gelu_tanh(linear(c, p["w_1"], p["b_1"]))
    y = h1 + linear(f, p["w_2"], p["b_2"])
    return y, appended


def selective_iteration(params: Sequence[dict], reqs: Sequence[Req],
                        x: np.ndarray, caches, heads: int, eps: float):
    """One iteration of the whole model over an arbitrary mixed batch.

    params:  one dict per layer (keys LAYER_KEYS)
    caches:  caches[l][i] = (K, V) of request i at layer l, each [kv_len_i, H]
    returns  (y [sum L, H] after the last layer,
              appended[l][i] = (K_new, V_new), each [q_len_i, H])
    [houmin] 3.1.1/3.1.2: the engine runs exactly one iteration of the batch.
    """
    appended_all = []
    for l, p in enumerate(params):
        x, appended = selective_layer(p, reqs, x, caches[l], heads, eps)
        appended_all.append(appended)
    return x, appended_all


# ------------------------------------------------- reference formulations (C2)

def each_request_alone(params, reqs: Sequence[Req], x: np.ndarray, caches,
                       heads: int, eps: float):
    """Run every request as a batch of one and concatenate the results.

    The method claims selective batching computes exactly this
    ([houmin] 3.1.2: Linear does not mix tokens; attention is per request).
    """
    ys = []
    appended = [[] for _ in params]
    for i, r in enumerate(reqs):
        rows = slice(r.q_offset, r.q_offset + r.q_len)
        one = [Req(0, r.q_len, r.kv_len)]
        c1 = [[caches[l][i]] for l in range(len(params))]
        y, app = selective_iteration(params, one, x[rows], c1, heads, eps)
        ys.append(y)
        for l in range(len(params)):
            appended[l].append(app[l][0])
    return np.concatenate(ys, axis=0), appended


def padded_masked(params, reqs: Sequence[Req], x: np.ndarray, caches,
                  heads: int, eps: float):
    """The batched [B, L, H] formulation with padding and masking.

    [houmin] 3.1.2 ("problem"): without selective batching the layer takes one
    [B, L, H] tensor; irregular requests are padded and masked, which wastes
    compute.  Query j of request b may see key t iff t <= kv_len_b + j and
    j < q_len_b.  Padded query rows are computed and then dropped; padded
    keys are never visible.  Written independently of selective_layer.
    """
    n = len(reqs)
    hidden = x.shape[1]
    d = hidden // heads
    lq = max(r.q_len for r in reqs)
    lk = max(r.kv_len + r.q_len for r in reqs)
    xb = np.zeros((n, lq, hidden), dtype=x.dtype)
    for b, r in enumerate(reqs):
        xb[b, :r.q_len] = x[r.q_offset:r.q_offset + r.q_len]
    qlen = np.array([r.q_len for r in reqs])[:, None, None]
    kvl = np.array([r.kv_len for r in reqs])[:, None, None]
    j = np.arange(lq)[None, :, None]
    t = np.arange(lk)[None, None, :]
    real_q = j < qlen                                        # [n, lq, 1]
    visible = (t <= kvl + j) & real_q                        # [n, lq, lk]
    # padded query rows see key 0 only, to keep their softmax finite; dropped
    visible = visible | (~real_q & (t == 0))
    appended = []
    for l, p in enumerate(params):
        a = layer_norm(xb, p["ln1_g"], p["ln1_b"], eps)
        qkv = a @ p["w_qkv"].T + p["b_qkv"]                  # [n, lq, 3H]
        q = qkv[..., :hidden]
        kb = np.zeros((n, lk, hidden), dtype=x.dtype)
        vb = np.zeros((n, lk, hidden), dtype=x.dtype)
        app_l = []
        for b, r in enumerate(reqs):
            kc, vc = caches[l][b]
            kb[b, :r.kv_len] = kc
            vb[b, :r.kv_len] = vc
            kb[b, r.kv_len:r.kv_len + r.q_len] = qkv[b, :r.q_len, hidden:2 * hidden]
            vb[b, r.kv_len:r.kv_len + r.q_len] = qkv[b, :r.q_len, 2 * hidden:]
            app_l.append((kb[b, r.kv_len:r.kv_len + r.q_len].copy(),
                          vb[b, r.kv_len:r.kv_len + r.q_len].copy()))
        appended.append(app_l)
        qh = q.reshape(n, lq, heads, d).transpose(0, 2, 1, 3)     # [n, h, lq, d]
        kh = kb.reshape(n, lk, heads, d).transpose(0, 2, 1, 3)
        vh = vb.reshape(n, lk, heads, d).transpose(0, 2, 1, 3)
        s = qh @ kh.transpose(0, 1, 3, 2) / math.sqrt(d)          # [n, h, lq, lk]
        s = np.where(visible[:, None], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        pr = e / e.sum(axis=-1, keepdims=True)
        o = (pr @ vh).transpose(0, 2, 1, 3).reshape(n, lq, hidden)
        h1 = xb + o @ p["w_o"].T + p["b_o"]
        c = layer_norm(h1, p["ln2_g"], p["ln2_b"], eps)
        f = gelu_tanh(c @ p["w_1"].T + p["b_1"])
        xb = h1 + f @ p["w_2"].T + p["b_2"]
    y = np.concatenate([xb[b, :r.q_len] for b, r in enumerate(reqs)], axis=0)
    return y, appended
