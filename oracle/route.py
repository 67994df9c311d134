"""Top-k softmax routing.

The router selects k of the E experts for every token ("Making Large MoE Models
Practical on a Single Machine", section 1; the txtmix article, section
"它在解一个什么问题": a layer stores E experts and each token goes to k << E of
them).  The pages leave the arithmetic open; this oracle takes the plain
reading:

  z[t, e] = sum_i x[t, i] * Wr[i, e]      every bf16*bf16 product is exact in
                                          fp64 and the sum is taken in fp64
  ids[t]  = the k experts with the largest z, ordered by z descending, ties
            to the lower expert index
  w[t, j] = exp(z[t, ids[t, j]]) / sum_j' exp(z[t, ids[t, j']])
            (softmax restricted to the chosen k, fp64, returned as fp32)
"""
import numpy as np

from .formats import bf16_to_f64


def logits(x_bf16, wr_bf16) -> np.ndarray:
    """fp64 router logits [T x E]."""
    return bf16_to_f64(x_bf16) @ bf16_to_f64(wr_bf16)


def topk_order(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row, z descending, ties to lower index."""
    T, E = z.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -z), axis=-1)   # primary key -z, secondary e
    return order[:, :k].astype(np.int32)


def softmax_chosen(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    zc = np.take_along_axis(z, ids.astype(np.int64), axis=1)
    ex = np.exp(zc - zc.max(axis=1, keepdims=True))
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def route(x_bf16, wr_bf16, k: int):
    """Return (ids [T x k] int32, w [T x k] fp32, min_gap).

    min_gap is the smallest relative gap between adjacent logits among the top
    k+1 of any token: a mismatch in ids against another implementation that
    also accumulates in fp64 is only possible where this gap is ~1e-15."""
    z = logits(x_bf16, wr_bf16)
    ids = topk_order(z, k)
    w = softmax_chosen(z, ids)
    kk = min(k + 1, z.shape[1])
    top = -np.sort(-z, axis=1)[:, :kk]
    if kk > 1:
        scale = np.maximum(np.abs(top[:, :1]), 1e-300)
        gap = float(np.min((top[:, :-1] - top[:, 1:]) / scale))
    else:
        gap = float("inf")
    return ids, w, gap
