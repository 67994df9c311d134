"""The expert FFN and the weighted top-k combine.

Every expert has a gate/up projection and a down projection, kept together in
one layer-expert record ("The Expert Cache That Follows the Router", section
"One logical expert, two physical levels of memory").  The pages do not name
the activation; the layer built here is SwiGLU:

  FFN_e(x) = (silu(x Wg_e) * (x Wu_e)) Wd_e,   silu(z) = z / (1 + exp(-z))

and the layer output is the gate-weighted sum of the routed experts' outputs,

  y[t] = sum_j w[t, j] * FFN_{id[t, j]}(x[t])     (j ascending).

Where an expert runs (hit, fill or host) does not change the result: the
partial sums of the GPU and the host branch merge exactly (METAL MEDIA summary,
Figure 2 caption; hyper.ai summary, section 方法).  Everything here is fp64 with
no intermediate rounding; inputs are the bf16 bits of x and decoded weights.
"""
import numpy as np

from .formats import bf16_to_f64


def silu(z):
    return z / (1.0 + np.exp(-z))


def ffn(x64: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """x64 [n x d] fp64 -> [n x d] fp64."""
    return (silu(x64 @ Wg) * (x64 @ Wu)) @ Wd


def expert_terms(x_bf16, ids, experts):
    """terms[t, j] = FFN_{ids[t, j]}(x[t]) as an fp64 array [T x k x d].

    `experts(e)` returns (Wg, Wu, Wd) of expert e of the current layer."""
    x64 = bf16_to_f64(x_bf16)
    T, k = ids.shape
    terms = np.zeros((T, k, x64.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        tt, jj = np.nonzero(ids == e)
        Wg, Wu, Wd = experts(int(e))
        terms[tt, jj] = ffn(x64[tt], Wg, Wu, Wd)
    return terms


def combine(terms: np.ndarray, w) -> np.ndarray:
    """y[t] = sum_j w[t, j] * terms[t, j], j ascending (fp64)."""
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    y = np.zeros((terms.shape[0], terms.shape[2]), dtype=np.float64)
    for j in range(terms.shape[1]):
        y += w64[:, j:j + 1] * terms[:, j]
    return y


def moe_layer(x_bf16, ids, w, experts) -> np.ndarray:
    """The routed-expert layer output [T x d] in fp64."""
    ids = np.asarray(ids)
    return combine(expert_terms(x_bf16, ids, experts), w)


def moe_layer_partitioned(x_bf16, ids, w, experts, on_host) -> np.ndarray:
    """The same layer evaluated as two partial sums, the way the cache splits it:
    G[t] over routes whose expert runs on the GPU (hit or fill), P[t] over
    routes whose expert runs on the host (`on_host(e)` true), then y = G + P."""
    ids = np.asarray(ids)
    terms = expert_terms(x_bf16, ids, experts)
    host = np.vectorize(lambda e: bool(on_host(int(e))))(ids) if ids.size else np.zeros(ids.shape, bool)
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    G = np.zeros((terms.shape[0], terms.shape[2]))
    P = np.zeros_like(G)
    for j in range(ids.shape[1]):
        g = ~host[:, j]
        G[g] += w64[g, j:j + 1] * terms[g, j]
        P[~g] += w64[~g, j:j + 1] * terms[~g, j]
    return G + P
