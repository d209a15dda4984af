"""The routed MoE FFN layer, oracle side (float64, plain numpy).

The layer (PocketLLM "Xing4.0-29B-A4B", section "Overview": a sigmoid-routed MoE with a
shared expert, 64 routed experts activated top-4 plus one shared; Red Lite "What we
learned", section "1. The idea": 512 experts of which a token uses 10; "DeepSeek-V4.1-Flash
... Xolotl", section "Why build an engine at all": a router picks 6 of 384 per token):

1. router logits   l = x W_r^T + b                                  (fp64)
2. selection       the k largest logits, descending, ties to the lower expert index;
                   NaN orders below every number
3. gating weights  sigmoid: s = 1/(1+e^-l), w_j = s_{id_j} / sum_j s_{id_j} (renormalised);
                   softmax: p = softmax(l) over all E, w_j = p_{id_j} (renormalised only
                   when asked)
4. sanitisation    an id outside [0, E) becomes expert 0 with weight 0 ("Running Qwen
                   Flash-Next NVFP4 in vLLM", B12x route validation)
5. permutation     route pairs (t, j) sorted stably by expert; offsets by histogram and
                   exclusive scan; inverse map; the shared expert's rows follow, token order
6. experts         SwiGLU: h = silu(W_g x) * (W_u x), o = W_d h, weights dequantised IQ4_NL
7. combine         y_t = sum_{j<k} w_tj o_(t,j) + o_shared,t, in that fixed order
                   (PocketLLM page, "Where the detail is": deterministic route reduction)

The grouped evaluation (step 5-6) is what the GPU computes; ``moe_layer_dense`` evaluates
every expert on every token and masks by the route table, the check PocketLLM's page
describes for its grouped MoE kernel (section "Without a server").
"""
from dataclasses import dataclass
import numpy as np

from . import iq4nl

SIGMOID = 0
SOFTMAX = 1


@dataclass(frozen=True)
class Desc:
    hidden: int
    ffn: int
    n_experts: int
    top_k: int
    n_shared: int = 1
    gating: int = SIGMOID
    renormalize: int = 1


# ---- expert bank -----------------------------------------------------------------------
# One buffer per layer; expert e (e == E: the shared expert) at byte offset e * stride;
# inside it: gate [F rows x H/32 blocks], then up [F x H/32], then down [H x F/32].

def expert_sizes(desc: Desc):
    g = iq4nl.matrix_bytes(desc.ffn, desc.hidden)
    d = iq4nl.matrix_bytes(desc.hidden, desc.ffn)
    return g, g, d


def expert_weights(bank: np.ndarray, stride: int, e: int, desc: Desc):
    """Dequantised (W_g [F,H], W_u [F,H], W_d [H,F]) of expert e, float64."""
    g, u, d = expert_sizes(desc)
    base = e * stride
    raw = np.asarray(bank, dtype=np.uint8)
    wg = iq4nl.dequantize_matrix(raw[base:base + g], desc.ffn, desc.hidden)
    wu = iq4nl.dequantize_matrix(raw[base + g:base + g + u], desc.ffn, desc.hidden)
    wd = iq4nl.dequantize_matrix(raw[base + g + u:base + g + u + d], desc.hidden, desc.ffn)
    return wg, wu, wd


def build_bank(mats, desc: Desc, stride: int = None) -> np.ndarray:
    """Quantise a list of (W_g, W_u, W_d) fp32 triples into one bank buffer."""
    g, u, d = expert_sizes(desc)
    stride = stride or (g + u + d)
    bank = np.zeros(stride * len(mats), dtype=np.uint8)
    for e, (wg, wu, wd) in enumerate(mats):
        b = e * stride
        bank[b:b + g] = iq4nl.quantize_matrix(wg)
        bank[b + g:b + g + u] = iq4nl.quantize_matrix(wu)
        bank[b + g + u:b + g + u + d] = iq4nl.quantize_matrix(wd)
    return bank


# ---- routing ---------------------------------------------------------------------------

def router_logits(x, w_router, bias=None):
    """l = x W_r^T (+ b), float64."""
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def select_topk(logits, k: int) -> np.ndarray:
    """ids[t, 0..k-1]: experts by (logit descending, index ascending); NaN lowest.

    -0.0 and +0.0 compare equal (IEEE), so they tie and the lower index wins.
    """
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    nan = np.isnan(l)
    val = np.where(nan, 0.0, l) + 0.0                  # +0.0 turns -0.0 into +0.0
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -val, nan), axis=-1)      # last key is primary
    return order[:, :k].astype(np.int32)


def gating_weights(logits, ids, gating: int, renormalize: int) -> np.ndarray:
    l = np.asarray(logits, np.float64)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    if gating == SIGMOID:
        w = 1.0 / (1.0 + np.exp(-sel))
    else:
        m = np.max(l, axis=1, keepdims=True)
        p = np.exp(l - m)
        p = p / np.sum(p, axis=1, keepdims=True)
        w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / np.sum(w, axis=1, keepdims=True)
    return w


def route(x, w_router, bias, desc: Desc):
    l = router_logits(x, w_router, bias)
    ids = select_topk(l, desc.top_k)
    return l, ids, gating_weights(l, ids, desc.gating, desc.renormalize)


def sanitize(ids, weights, n_experts: int):
    """Invalid ids (< 0 or >= E) -> id 0 with weight 0; valid routes keep both."""
    ids = np.asarray(ids)
    valid = (ids >= 0) & (ids < n_experts)
    return (np.where(valid, ids, 0).astype(np.int32),
            np.where(valid, weights, 0.0), int(np.count_nonzero(~valid)))


# ---- permutation -----------------------------------------------------------------------

def permute(ids, n_experts: int, n_shared: int):
    """Group route pairs by expert.

    Pair p = t*k + j.  Returns offsets [E+S+1] (routed slots of expert e are
    offsets[e] .. offsets[e+1]-1; the shared expert's T slots follow, token order),
    sorted_pairs [T*k] (pair id at each routed slot, stable in p) and pair_slot [T*k].
    """
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)[:n_experts]
    counts = np.concatenate([counts, np.full(n_shared, T)])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    pair_slot = np.empty(T * k, np.int32)
    pair_slot[sorted_pairs] = np.arange(T * k, dtype=np.int32)
    return offsets, sorted_pairs, pair_slot


def slot_tokens(sorted_pairs, T: int, k: int, n_shared: int) -> np.ndarray:
    """Token of every slot: routed slots from the pair id, then T shared slots per shared expert."""
    routed = np.asarray(sorted_pairs, np.int64) // k
    return np.concatenate([routed] + [np.arange(T)] * n_shared)


# ---- experts and combine ---------------------------------------------------------------

def silu(g):
    return g / (1.0 + np.exp(-g))


def expert_gate_up(wg, wu, x):
    """h = silu(W_g x) * (W_u x) for rows of x [m, H] -> [m, F]."""
    return silu(x @ wg.T) * (x @ wu.T)


def expert_down(wd, h):
    """o = W_d h for rows of h [m, F] -> [m, H]."""
    return h @ wd.T


def combine(o, pair_slot, weights, T: int, k: int, n_shared: int, residual=None):
    """y_t = sum_j w_tj o[slot(t, j)] + sum_s o[shared slot of t], fixed order."""
    o = np.asarray(o, np.float64)
    w = np.asarray(weights, np.float64)
    slot = np.asarray(pair_slot).reshape(T, k)
    y = np.zeros((T, o.shape[1]))
    for j in range(k):
        y += w[:, j:j + 1] * o[slot[:, j]]
    for s in range(n_shared):
        y += o[T * k + s * T + np.arange(T)]
    if residual is not None:
        y += np.asarray(residual, np.float64)
    return y


# ---- the layer -------------------------------------------------------------------------

def moe_layer(x, w_router, bias, bank, stride: int, desc: Desc, ids=None, weights=None,
              return_parts: bool = False):
    """One layer, grouped evaluation.  ``ids``/``weights`` override routing if given
    (they are sanitised first)."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    k, E, S = desc.top_k, desc.n_experts, desc.n_shared
    logits = None
    if ids is None:
        logits, ids, weights = route(x, w_router, bias, desc)
    ids, weights, n_invalid = sanitize(ids, weights, E)
    offsets, sorted_pairs, pair_slot = permute(ids, E, S)
    tok = slot_tokens(sorted_pairs, T, k, S)
    rows = T * k + S * T
    h = np.zeros((rows, desc.ffn))
    o = np.zeros((rows, desc.hidden))
    for e in range(E + S):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        wg, wu, wd = expert_weights(bank, stride, e, desc)
        h[a:b] = expert_gate_up(wg, wu, x[tok[a:b]])
        o[a:b] = expert_down(wd, h[a:b])
    y = combine(o, pair_slot, weights, T, k, S)
    if return_parts:
        return y, dict(logits=logits, ids=ids, weights=weights, offsets=offsets,
                       sorted_pairs=sorted_pairs, pair_slot=pair_slot, h=h, o=o,
                       n_invalid=n_invalid)
    return y


def moe_layer_dense(x, w_router, bias, bank, stride: int, desc: Desc):
    """Every expert on every token, masked by the route table (no permutation)."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    _, ids, w = route(x, w_router, bias, desc)
    y = np.zeros((T, desc.hidden))
    for e in range(desc.n_experts + desc.n_shared):
        wg, wu, wd = expert_weights(bank, stride, e, desc)
        out = expert_down(wd, expert_gate_up(wg, wu, x))
        if e < desc.n_experts:
            gate = np.sum(np.where(ids == e, w, 0.0), axis=1)
        else:
            gate = np.ones(T)
        y += gate[:, None] * out
    return y


def rmsnorm(x, eps: float = 1e-6):
    """Weight-free RMSNorm, x / sqrt(mean(x^2) + eps), the glue between chained layers."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)


def chain(x, layers, desc: Desc, eps: float = 1e-6):
    """x <- x + MoE_l(rmsnorm(x)) for each layer (w_router, bias, bank, stride)."""
    x = np.asarray(x, np.float64)
    for (w_router, bias, bank, stride) in layers:
        x = x + moe_layer(rmsnorm(x, eps), w_router, bias, bank, stride, desc)
    return x


def decode_bytes_per_token(desc: Desc, layers: int):
    """Expert bytes a decode token reads: (routed, shared), k routed + S shared experts a layer."""
    g, u, d = expert_sizes(desc)
    per = g + u + d
    return desc.top_k * per * layers, desc.n_shared * per * layers
