"""Float64 CPU oracle of one MoE expert layer: routing, token dispatch, grouped
SwiGLU expert FFN, weighted combine, and the backward of each step.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the bench's CPU-baseline leg may use it.

What the pages fix and what is read into them
---------------------------------------------
* "Add MoE expert parallel training runtime" (Major changes) names
  the hot path: EP token dispatch followed by grouped expert compute. It gives
  no formulas.
* "Support combined expert and data parallelism in TrainerRank" (Desired
  behavior) asks for full source-order outputs, gradient accumulation, no
  padding by callers, and correct handling of uneven or empty work; its
  Acceptance section asks for an empty-work case, multiple microbatches and a
  comparison against a matched reference within stated tolerances.
* "Support pipeline parallelism in TrainerRank without exposing stage
  scheduling to callers" (Acceptance) adds accumulation across several
  forwards.

The layer itself is the conventional dropless top-k softmax MoE with SwiGLU
experts, which is the plainest reading of "token dispatch + grouped expert
compute" under the no-padding requirement:

  p      = softmax(logits[t, :])                     over all E experts
  ids    = the k largest logits, descending; equal logits go to the lower id
  w[t,j] = p[ids[t,j]]            (optionally divided by sum_j p[ids[t,j]])
  rows   = stable counting sort of the (token, slot) pairs by expert id
  H      = X_e @ W_gu[e].T        W_gu[e] = [W_gate; W_up], shape [2F, d]
  A      = silu(H[:, :F]) * H[:, F:]
  Y      = A @ W_down[e].T        W_down[e] shape [d, F]
  out[t] = sum_j w[t,j] * Y[row_of_slot[t,j]]

There is no capacity factor: every (token, expert) pair is computed, so an
expert may receive any number of rows including zero. Gradients are plain
sums (no averaging); the weight gradients of several microbatches add up.

Every function below stays in float64 from start to finish. Where the GPU
path rounds intermediates to the layer dtype (H, A, Y, dY, dH, dX_perm are
stored in bf16 for a bf16 layer; sums are rounded once), nothing on the pages
fixes those rounding points: agreement there is parity unpinned beyond the
stated tolerance.

Selection compares logits, not probabilities: exp() can merge distinct
logits into equal probabilities, comparing logits cannot. NaN ranks below
-inf; -0.0 and +0.0 are equal (a tie).
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "router_logits", "softmax", "route", "route_brute_force", "permute", "expert_ffn_fwd",
    "unpermute_combine", "unpermute_combine_bwd", "route_bwd", "router_bwd", "expert_ffn_bwd",
    "permute_bwd", "silu", "sigmoid", "swiglu_bwd", "layer_fwd", "layer_bwd", "dense_reference",
]


# ---------------------------------------------------------------------------
# elementary functions
# ---------------------------------------------------------------------------
def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-z)), evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z)."""
    return z * sigmoid(z)


def softmax(logits: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first. Entries equal to
    -inf get probability 0; each row needs at least one finite logit."""
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l, axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """logits[t, e] = <x[t], w_router[e]> + bias[e]  (w_router is [E, d])."""
    out = x @ w_router.T
    if bias is not None:
        out = out + bias[None, :]
    return out


def route(logits: np.ndarray, k: int, renorm: bool = False) -> Dict[str, np.ndarray]:
    """Top-k softmax routing plus the dispatch tables.

    Returns a dict with
      topk_idx    [T, k] int32  the k selected experts, descending logit,
                                ties to the lower id
      topk_w      [T, k] f64    softmax probability of each selected expert
                                (renormalised over the k when ``renorm``)
      counts      [E]    int32  rows per expert
      offsets     [E+1]  int32  exclusive prefix sum of counts
      row_of_slot [T, k] int32  row of the expert-contiguous buffer that
                                receives (t, j)
      src_of_row  [T*k]  int32  inverse map: the slot index t*k+j of each row

    Rows of one expert follow the source order (ascending t): this is a
    stable counting sort of the flattened slots by expert id, which keeps the
    dispatch deterministic and returns outputs to full source order.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    # Stable sort of -logit: descending logit, equal logits keep ascending id
    # order, NaN (sorted last by numpy) ranks below -inf.
    order = np.argsort(-logits, axis=1, kind="stable")
    topk_idx = order[:, :k].astype(np.int32)

    p = softmax(np.where(np.isnan(logits), -np.inf, logits)) if T else np.zeros((0, E))
    topk_w = np.take_along_axis(p, topk_idx.astype(np.int64), axis=1)
    if renorm and T:
        topk_w = topk_w / np.sum(topk_w, axis=1, keepdims=True)

    flat = topk_idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    src_of_row = np.argsort(flat, kind="stable").astype(np.int32)
    row_of_slot = np.empty(T * k, dtype=np.int32)
    row_of_slot[src_of_row] = np.arange(T * k, dtype=np.int32)
    return {
        "topk_idx": topk_idx,
        "topk_w": topk_w,
        "counts": counts,
        "offsets": offsets,
        "row_of_slot": row_of_slot.reshape(T, k),
        "src_of_row": src_of_row,
    }


def route_brute_force(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Selection by counting, for tiny inputs (pure Python loops).

    Expert a beats expert b when logit_a > logit_b, or they are equal and
    a < b (NaN loses to everything that is not NaN). An expert's rank is the
    number of experts that beat it; slot j holds the expert of rank j.
    Returns (topk_idx [T,k], mask [T,E] of selected experts).
    """
    T, E = logits.shape

    def beats(la, a, lb, b):
        na, nb = np.isnan(la), np.isnan(lb)
        if na or nb:
            if na and nb:
                return a < b
            return nb
        if la != lb:
            return la > lb
        return a < b

    idx = np.zeros((T, k), dtype=np.int32)
    mask = np.zeros((T, E), dtype=bool)
    for t in range(T):
        for e in range(E):
            rank = sum(1 for o in range(E) if o != e and beats(logits[t, o], o, logits[t, e], e))
            if rank < k:
                idx[t, rank] = e
                mask[t, e] = True
    return idx, mask


def permute(x: np.ndarray, row_of_slot: np.ndarray) -> np.ndarray:
    """Token dispatch: x_perm[row_of_slot[t, j]] = x[t]."""
    T, k = row_of_slot.shape
    x_perm = np.zeros((T * k, x.shape[1]), dtype=np.float64)
    for j in range(k):
        x_perm[row_of_slot[:, j]] = x
    return x_perm


def expert_ffn_fwd(x_perm: np.ndarray, w_gu: np.ndarray, w_down: np.ndarray,
                   offsets: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Grouped SwiGLU expert FFN over expert-contiguous rows.

    For each expert e with rows [offsets[e], offsets[e+1]):
      H = X_e @ W_gu[e].T            [M_e, 2F]
      A = silu(H[:, :F]) * H[:, F:]  [M_e, F]
      Y = A @ W_down[e].T            [M_e, d]
    Experts with no rows contribute nothing.
    """
    R, d = x_perm.shape
    E, twoF, _ = w_gu.shape
    F = twoF // 2
    h = np.zeros((R, twoF))
    a = np.zeros((R, F))
    y = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        he = x_perm[lo:hi] @ np.asarray(w_gu[e], dtype=np.float64).T
        ae = silu(he[:, :F]) * he[:, F:]
        h[lo:hi] = he
        a[lo:hi] = ae
        y[lo:hi] = ae @ np.asarray(w_down[e], dtype=np.float64).T
    return h, a, y


def unpermute_combine(y: np.ndarray, topk_w: np.ndarray, row_of_slot: np.ndarray) -> np.ndarray:
    """Weighted combine back to source order: out[t] = sum_j w[t,j] * Y[row_of_slot[t,j]]."""
    T, k = row_of_slot.shape
    out = np.zeros((T, y.shape[1]))
    for j in range(k):
        out += topk_w[:, j:j + 1] * y[row_of_slot[:, j]]
    return out


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def unpermute_combine_bwd(dout: np.ndarray, y: np.ndarray, topk_w: np.ndarray,
                          row_of_slot: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Backward of the combine.

    dY[row_of_slot[t,j]] = w[t,j] * dout[t]
    dw[t,j]              = <dout[t], Y[row_of_slot[t,j]]>
    """
    T, k = row_of_slot.shape
    dy = np.zeros_like(y, dtype=np.float64)
    dw = np.zeros((T, k))
    for j in range(k):
        rows = row_of_slot[:, j]
        dy[rows] = topk_w[:, j:j + 1] * dout
        dw[:, j] = np.sum(dout * y[rows], axis=1)
    return dy, dw


def route_bwd(dtopk_w: np.ndarray, logits: np.ndarray, topk_idx: np.ndarray,
              topk_w: np.ndarray, renorm: bool = False) -> np.ndarray:
    """Gradient of the routing weights with respect to the logits.

    The selection itself is piecewise constant, so only the weights carry a
    gradient. With g[t,j] = dL/dw[t,j]:
      no renorm: w_j = p_{e_j}; dp_i/dl_m = p_i (delta_im - p_m), so
                 dlogits[t,m] = p_m * (G_m - sum_j w_j g_j), where G_m = g_j
                 if m = e_j for some j, else 0.
      renorm:    w is a softmax over the selected logits only, so
                 dlogits[t,e_j] = w_j (g_j - sum_j' w_j' g_j'), zero elsewhere.
    """
    T, E = logits.shape
    dl = np.zeros((T, E))
    if T == 0:
        return dl
    s = np.sum(topk_w * dtopk_w, axis=1, keepdims=True)
    if renorm:
        np.put_along_axis(dl, topk_idx.astype(np.int64), topk_w * (dtopk_w - s), axis=1)
        return dl
    p = softmax(np.where(np.isnan(logits), -np.inf, logits))
    G = np.zeros((T, E))
    np.put_along_axis(G, topk_idx.astype(np.int64), dtopk_w, axis=1)
    return p * (G - s)


def router_bwd(dlogits: np.ndarray, x: np.ndarray, w_router: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Backward of logits = x @ w_router.T + b: dx_router = dlogits @ w_router,
    dw_router = dlogits.T @ x (the bias is not trained)."""
    return dlogits @ w_router, dlogits.T @ x


def swiglu_bwd(da: np.ndarray, hg: np.ndarray, hu: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Backward of A = silu(Hg) * Hu.

    d silu(z)/dz = sigmoid(z) * (1 + z * (1 - sigmoid(z))), hence
      dHg = dA * Hu * sigmoid(Hg) * (1 + Hg * (1 - sigmoid(Hg)))
      dHu = dA * silu(Hg)
    """
    sg = sigmoid(hg)
    return da * hu * sg * (1.0 + hg * (1.0 - sg)), da * hg * sg


def expert_ffn_bwd(dy: np.ndarray, x_perm: np.ndarray, h: np.ndarray, a: np.ndarray,
                   w_gu: np.ndarray, w_down: np.ndarray, offsets: np.ndarray):
    """Backward of the grouped SwiGLU FFN, expert by expert.

      dA      = dY_e @ W_down[e]
      dW_down = dY_e.T @ A_e
      dH      = swiglu_bwd(dA, H_gate, H_up)
      dX_e    = dH @ W_gu[e]
      dW_gu   = dH.T @ X_e
    Returns (dx_perm, dw_gu, dw_down, dh). Experts with no rows get zero
    weight gradients.
    """
    R, d = x_perm.shape
    E, twoF, _ = w_gu.shape
    F = twoF // 2
    dx = np.zeros((R, d))
    dh = np.zeros((R, twoF))
    dw_gu = np.zeros((E, twoF, d))
    dw_down = np.zeros((E, d, F))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wd = np.asarray(w_down[e], dtype=np.float64)
        wg = np.asarray(w_gu[e], dtype=np.float64)
        dye = dy[lo:hi]
        da = dye @ wd
        dw_down[e] = dye.T @ a[lo:hi]
        dhg, dhu = swiglu_bwd(da, h[lo:hi, :F], h[lo:hi, F:])
        dhe = np.concatenate([dhg, dhu], axis=1)
        dh[lo:hi] = dhe
        dx[lo:hi] = dhe @ wg
        dw_gu[e] = dhe.T @ x_perm[lo:hi]
    return dx, dw_gu, dw_down, dh


def permute_bwd(dx_perm: np.ndarray, row_of_slot: np.ndarray,
                dx_extra: Optional[np.ndarray] = None) -> np.ndarray:
    """Backward of the dispatch: dx[t] = sum_j dX_perm[row_of_slot[t,j]]
    (+ dx_extra[t], the router's contribution, when given)."""
    T, k = row_of_slot.shape
    dx = np.zeros((T, dx_perm.shape[1]))
    for j in range(k):
        dx += dx_perm[row_of_slot[:, j]]
    if dx_extra is not None:
        dx += dx_extra
    return dx


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------
def layer_fwd(x, w_gu, w_down, k, logits=None, w_router=None, bias=None, renorm=False):
    """Forward of the whole layer. Either ``logits`` are given, or they are
    computed by the router from ``x`` and ``w_router`` (+ ``bias``)."""
    if logits is None:
        logits = router_logits(x, w_router, bias)
    r = route(logits, k, renorm)
    x_perm = permute(x, r["row_of_slot"])
    h, a, y = expert_ffn_fwd(x_perm, w_gu, w_down, r["offsets"])
    out = unpermute_combine(y, r["topk_w"], r["row_of_slot"])
    saved = dict(r, logits=logits, x_perm=x_perm, h=h, a=a, y=y)
    return out, saved


def layer_bwd(dout, saved, w_gu, w_down, x=None, w_router=None, renorm=False):
    """Backward of the whole layer from the forward's saved tensors."""
    dy, dtopk_w = unpermute_combine_bwd(dout, saved["y"], saved["topk_w"], saved["row_of_slot"])
    dlogits = route_bwd(dtopk_w, saved["logits"], saved["topk_idx"], saved["topk_w"], renorm)
    dx_perm, dw_gu, dw_down, dh = expert_ffn_bwd(dy, saved["x_perm"], saved["h"], saved["a"],
                                                 w_gu, w_down, saved["offsets"])
    grads = dict(dy=dy, dtopk_w=dtopk_w, dlogits=dlogits, dx_perm=dx_perm, dw_gu=dw_gu,
                 dw_down=dw_down, dh=dh)
    dx_router = None
    if w_router is not None:
        dx_router, dw_router = router_bwd(dlogits, x, w_router)
        grads["dx_router"] = dx_router
        grads["dw_router"] = dw_router
    grads["dx"] = permute_bwd(dx_perm, saved["row_of_slot"], dx_router)
    return grads


def dense_reference(x, w_gu, w_down, logits, k, renorm=False):
    """Run every expert on every token, then mask: the result the dropless
    sparse layer must equal exactly (up to rounding order).

    The mask and weights are rebuilt here from their definitions (selection
    by counting, softmax of the full row), independently of ``route``.
    """
    T, E = logits.shape
    F = w_gu.shape[1] // 2
    _, mask = route_brute_force(logits, k)
    p = softmax(logits)
    w = np.where(mask, p, 0.0)
    if renorm:
        w = w / np.sum(w, axis=1, keepdims=True)
    out = np.zeros((T, x.shape[1]))
    for e in range(E):
        he = x @ w_gu[e].T
        ye = (silu(he[:, :F]) * he[:, F:]) @ w_down[e].T
        out += w[:, e:e + 1] * ye
    return out
