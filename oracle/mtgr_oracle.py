"""CPU oracle for the MTGR HSTU encoder forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this module.  The
product path (the HIP library and its binding) never imports it, and it imports nothing from the
product path.  It is plain numpy in float64, written from the pages' definitions, step by step,
with no blocking, fusion or reordering beyond what the definitions state.

Page keys used in citations:
  [P1] chenhuiyu blog "生成式推荐 18: MTGR" (Chinese)      [P2] the same blog post in English
  [P3] marovi.ai "MTGR: Industrial-Scale Generative Recommendation Framework in Meituan/zh"
  [P4] intelliparadigm article on MTGR hybrid modeling      [P5] fun-rec mdbook §7.3
       "MTGR: Hybrid Paradigm Modeling"

Definitions followed (all exact; the method has no approximation, heuristic or iteration):
  * sample layout D = [U, S, R, [C,I]_1..K], one sample per user      [P3 方法, eq. D; P5 7.3.1]
  * block: X~ = GroupLN(X); project X~ to Q, K, V, U;
           V~ = silu(K^T Q)/(N_U+N_S+N_R+N_I) masked by M, times V;
           X <- MLP(GroupLN(V~ (.) U)) + X                              [P3 方法, update equations]
  * mask M: rule 1 U and S keys visible to every query; rule 2 an R key is visible to a later
    R or C query (strictly earlier timestamp); rule 3 a candidate is visible only to itself
                                                    [P3 方法, mask paragraph; P5 7.3.4, Rules 1-3]
  * GroupLN: LayerNorm statistics of each token over its features, with affine parameters chosen
    by the token's group                                              [P5 7.3.3, GLN equation]
  * head: candidate hidden states -> MLP -> (CTR, CTCVR) logits      [P1/P2 token section; P5 7.3.1]

Readings where the pages are silent or garbled (the same numbering as the design notes):
  R1 the garbled silu(K^T Q) M V is read token-wise: v~_i = sum_j M[i,j] silu(q_i.k_j)/N v_j,
     with M applied elementwise.
  R2 N is the user's total token count (N_U+N_S+N_R+K), not the count of visible keys.
  R3 no scale and no relative bias inside silu.
  R4 R-key visibility uses strict '<' on float32 seconds; equal timestamps are invisible, except a
     token to itself.  R5: U and S queries never see R keys.  R6: candidates see only themselves
     among candidates; R, U and S queries never see C keys.
  R7 GroupLN statistics are per token (biased variance, eps=1e-5); gamma/beta per group.
  R8 Q, K, V, U projections are affine with no activation; heads split Q, K, V into contiguous
     d_h-wide slices; U gates the concatenated heads elementwise.
  R9 MLP is d -> h -> d with SiLU and biases.  R10: the head is d -> d/2 -> 2 with SiLU, raw logits.

parity pins: every function below is pinned by tests/test_oracle_pins.py (worked mask examples
from [P1] and [P5], GroupLN invariants and torch layer_norm, closed forms and library reductions
of the attention, silu against torch, a special case of the head, and permutation / independence /
isolation / temporal-replay invariants).  The readings R3, R8, R9 and R10 are parity unpinned with
respect to the paper: the pages never fix them, so they are pinned only by construction.
The block backward (the chain rule of the same equations) is pinned by central finite differences
of block_forward and by autograd of an independent torch formulation of the block.

R19 (bf16 storage, used only to set the tolerance of the bf16 block backward): the pages train in
bf16 mixed precision ([P3] 主要贡献 and 方法, training-framework paragraph) without saying where
values are rounded.  block_backward_bf16_storage reads "bf16 storage" as: arithmetic in float64,
and every tensor that is kept between two steps in the storage type -- plus the two per-pair
factors that enter a matrix product as bf16 operands (silu(S) and the masked dS) -- rounded to
the nearest bfloat16 (ties to even) where it is kept.  It is pinned by reducing exactly to
block_backward when the rounding is the identity, and by the rounding itself matching torch's
float32 -> bfloat16 conversion.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

G_U, G_S, G_R, G_C = 0, 1, 2, 3
NUM_GROUPS = 4


# ----------------------------------------------------------------------------------------------
# Mask  [P3 方法, mask paragraph; P5 7.3.4 Rules 1-3]
# ----------------------------------------------------------------------------------------------
MASK_MODES = ("dynamic", "causal", "full")


def mask(groups: np.ndarray, times: np.ndarray, mode: str = "dynamic") -> np.ndarray:
    """Mask of one user's tokens, by enumeration of every (query i, key j) pair.

    Returns uint8 [n, n]; rows are queries, columns keys; 1 = key visible to query.
    mode "dynamic": the three rules (token order is irrelevant: they look only at group ids and
    timestamps).  The ablation without the dynamic mask ([P1]/[P2] experiments; [P3] 结果) is read
    as the plain causal mask over the sequence order, which the pages name as what the three rules
    replace ([P3] 方法, mask paragraph; [P5] 7.3.4): mode "causal", key j visible iff j <= i.
    mode "full": every token of the user sees every other.
    """
    if mode == "causal":
        n = np.asarray(groups).shape[0]
        return np.tril(np.ones((n, n), dtype=np.uint8))
    if mode == "full":
        n = np.asarray(groups).shape[0]
        return np.ones((n, n), dtype=np.uint8)
    if mode != "dynamic":
        raise ValueError(mode)
    g = np.asarray(groups, dtype=np.int64)
    t = np.asarray(times, dtype=np.float32)
    n = g.shape[0]
    gi = g[:, None]            # query group, broadcast over keys
    gj = g[None, :]            # key group, broadcast over queries
    ti = t[:, None]
    tj = t[None, :]
    same = np.eye(n, dtype=bool)
    rule1_static = (gj == G_U) | (gj == G_S)                        # static keys: all queries
    rule2_causal = (gj == G_R) & ((gi == G_R) | (gi == G_C)) & (tj < ti)   # earlier R events
    rule3_self = same                                                # every token sees itself
    return (rule1_static | rule2_causal | rule3_self).astype(np.uint8)


def visible_pairs(groups: np.ndarray, times: np.ndarray) -> int:
    """Number of (query, key) pairs the mask lets through for one user."""
    return int(mask(groups, times).sum(dtype=np.int64))


# ----------------------------------------------------------------------------------------------
# Group-Layer Normalization  [P5 7.3.3, GLN equation; P3 方法, GLN paragraph]
# ----------------------------------------------------------------------------------------------
def group_layer_norm(x: np.ndarray, groups: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                     eps: float = 1e-5, shared: bool = False) -> np.ndarray:
    """x [n, d]; groups [n] in 0..3; gamma, beta [4, d].  Per-token mean and biased variance over
    the d features, then the affine parameters of the token's group.  shared=True is the
    ablation without GroupLN (one shared LayerNorm, [P3] 方法, GLN paragraph): every token takes
    the parameters of row 0."""
    x = np.asarray(x, dtype=np.float64)
    g = np.zeros(np.asarray(groups).shape[0], dtype=np.int64) if shared else np.asarray(groups, dtype=np.int64)
    d = x.shape[1]
    mu = x.sum(axis=1, keepdims=True) / d
    xc = x - mu
    var = (xc * xc).sum(axis=1, keepdims=True) / d
    xhat = xc / np.sqrt(var + eps)
    gam = np.asarray(gamma, dtype=np.float64)[g]
    bet = np.asarray(beta, dtype=np.float64)[g]
    return xhat * gam + bet


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), evaluated without overflow warnings."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """y = x W^T + b, W in [out, in] layout."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)
    return y


# ----------------------------------------------------------------------------------------------
# Masked SiLU attention with the U gate  [P3 方法, update equations]
# ----------------------------------------------------------------------------------------------
def hstu_attention(qkvu: np.ndarray, groups: np.ndarray, times: np.ndarray,
                   num_heads: int, mask_mode: str = "dynamic") -> np.ndarray:
    """One user's attention.  qkvu [n, 4d] = [Q | K | V | U]; returns V~ (.) U  [n, d].

    For head h (feature slice h*d_h:(h+1)*d_h of Q, K, V):
        V~_h = (silu(Q_h K_h^T) / N  *elementwise*  M) @ V_h,   N = n (the user's token count).
    """
    qkvu = np.asarray(qkvu, dtype=np.float64)
    n, four_d = qkvu.shape
    d = four_d // 4
    dh = d // num_heads
    if n == 0:
        return np.zeros((0, d))
    Q, K, V, U = qkvu[:, :d], qkvu[:, d:2 * d], qkvu[:, 2 * d:3 * d], qkvu[:, 3 * d:]
    M = mask(groups, times, mask_mode).astype(np.float64)
    N = float(n)
    vt = np.empty((n, d))
    for h in range(num_heads):
        sl = slice(h * dh, (h + 1) * dh)
        S = Q[:, sl] @ K[:, sl].T                    # S[i, j] = q_i . k_j
        A = silu(S) / N * M
        vt[:, sl] = A @ V[:, sl]
    return vt * U


# ----------------------------------------------------------------------------------------------
# HSTU block, encoder, head
# ----------------------------------------------------------------------------------------------
def block_forward(x: np.ndarray, groups: np.ndarray, times: np.ndarray, layer: Dict[str, np.ndarray],
                  num_heads: int, eps: float = 1e-5, return_parts: bool = False,
                  mask_mode: str = "dynamic", shared_norm: bool = False):
    """One HSTU block for one user [P3 方法, update equations]."""
    x = np.asarray(x, dtype=np.float64)
    xt = group_layer_norm(x, groups, layer["gln1_gamma"], layer["gln1_beta"], eps, shared_norm)
    qkvu = linear(xt, layer["w_qkvu"], layer.get("b_qkvu"))
    y = hstu_attention(qkvu, groups, times, num_heads, mask_mode)
    z = group_layer_norm(y, groups, layer["gln2_gamma"], layer["gln2_beta"], eps, shared_norm)
    hid = silu(linear(z, layer["w_mlp1"], layer.get("b_mlp1")))
    out = linear(hid, layer["w_mlp2"], layer.get("b_mlp2")) + x
    if return_parts:
        return out, dict(xt=xt, qkvu=qkvu, y=y, z=z, hid=hid)
    return out


def head_forward(x_cand: np.ndarray, head: Dict[str, np.ndarray]) -> np.ndarray:
    """Candidate readout: logits = W_h2 silu(W_h1 x + b_h1) + b_h2, columns (CTR, CTCVR)."""
    hid = silu(linear(x_cand, head["w_head1"], head.get("b_head1")))
    return linear(hid, head["w_head2"], head.get("b_head2"))


def encoder_forward(offsets: np.ndarray, groups: np.ndarray, times: np.ndarray, x: np.ndarray,
                    layers: Sequence[Dict[str, np.ndarray]], head: Optional[Dict[str, np.ndarray]],
                    num_heads: int, eps: float = 1e-5, mask_mode: str = "dynamic",
                    shared_norm: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """L blocks over every user of a packed batch, then the head at candidate tokens.

    Users are processed one at a time (no cross-user attention, [P1/P2] sequence packing).
    Returns (hidden [T, d], logits [C, 2]) with candidates in packed order.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    hidden = np.empty_like(x)
    for b in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        xb = x[lo:hi]
        for layer in layers:
            xb = block_forward(xb, groups[lo:hi], times[lo:hi], layer, num_heads, eps,
                               mask_mode=mask_mode, shared_norm=shared_norm)
        hidden[lo:hi] = xb
    cand = np.asarray(groups) == G_C
    logits = head_forward(hidden[cand], head) if head is not None else np.zeros((int(cand.sum()), 2))
    return hidden, logits


def params_layers(params) -> List[Dict[str, np.ndarray]]:
    """float64 copies of a generated parameter set's layers (values unchanged)."""
    return [{k: np.asarray(v, dtype=np.float64) for k, v in lay.items()} for lay in params.layers]


def params_head(params) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=np.float64) for k, v in params.head.items()}


# ----------------------------------------------------------------------------------------------
# Backward pass of one block (the training direction of the same update equations, [P3] 方法).
# Plain chain rule, float64, one user at a time; parameter gradients are sums over tokens.
# ----------------------------------------------------------------------------------------------
def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = sigma(z) (1 + z (1 - sigma(z)))."""
    z = np.asarray(z, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def linear_backward(x: np.ndarray, w: np.ndarray, dy: np.ndarray):
    """y = x W^T + b  ->  (dx = dy W, dW = dy^T x, db = sum_rows dy)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    return dy @ w, dy.T @ x, dy.sum(axis=0)


def group_layer_norm_backward(x: np.ndarray, groups: np.ndarray, gamma: np.ndarray, dy: np.ndarray,
                              eps: float = 1e-5, shared: bool = False):
    """Gradients of group_layer_norm: (dx [n, d], dgamma [4, d], dbeta [4, d]).

    With xhat = (x - mean) / s, s = sqrt(var + eps) (biased var over the d features):
        dxhat = dy * gamma[g];  dx = (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)) / s.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    n, d = x.shape
    g = np.zeros(n, dtype=np.int64) if shared else np.asarray(groups, dtype=np.int64)
    mean = x.mean(axis=1, keepdims=True)
    s = np.sqrt(((x - mean) ** 2).mean(axis=1, keepdims=True) + eps)
    xhat = (x - mean) / s
    dgamma = np.zeros((NUM_GROUPS, d))
    dbeta = np.zeros((NUM_GROUPS, d))
    for grp in range(NUM_GROUPS):
        sel = g == grp
        dgamma[grp] = (dy[sel] * xhat[sel]).sum(axis=0)
        dbeta[grp] = dy[sel].sum(axis=0)
    dxhat = dy * gamma[g]
    dx = (dxhat - dxhat.mean(axis=1, keepdims=True)
          - xhat * (dxhat * xhat).mean(axis=1, keepdims=True)) / s
    return dx, dgamma, dbeta


def hstu_attention_backward(qkvu: np.ndarray, groups: np.ndarray, times: np.ndarray,
                            num_heads: int, dy: np.ndarray, mask_mode: str = "dynamic") -> np.ndarray:
    """Gradient of hstu_attention w.r.t. qkvu [n, 4d] given dy = d loss / d (V~ (.) U).

    dV~ = dy (.) U and dU = dy (.) V~; per head, with A = silu(S) / N (.) M and S = Q K^T:
        dV = A^T dV~,  dA = dV~ V^T,  dS = dA (.) M / N (.) silu'(S),  dQ = dS K,  dK = dS^T Q.
    """
    qkvu = np.asarray(qkvu, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    n, four_d = qkvu.shape
    d = four_d // 4
    dh = d // num_heads
    dq = np.zeros((n, four_d))
    if n == 0:
        return dq
    Q, K, V, U = qkvu[:, :d], qkvu[:, d:2 * d], qkvu[:, 2 * d:3 * d], qkvu[:, 3 * d:]
    M = mask(groups, times, mask_mode).astype(np.float64)
    N = float(n)
    vt = np.empty((n, d))
    for h in range(num_heads):
        sl = slice(h * dh, (h + 1) * dh)
        S = Q[:, sl] @ K[:, sl].T
        A = silu(S) / N * M
        vt[:, sl] = A @ V[:, sl]
        dvt = dy[:, sl] * U[:, sl]
        dA = dvt @ V[:, sl].T
        dS = dA * M / N * silu_grad(S)
        dq[:, sl] = dS @ K[:, sl]
        dq[:, d + h * dh:d + (h + 1) * dh] = dS.T @ Q[:, sl]
        dq[:, 2 * d + h * dh:2 * d + (h + 1) * dh] = A.T @ dvt
    dq[:, 3 * d:] = dy * vt
    return dq


BLOCK_PARAM_NAMES = ("gln1_gamma", "gln1_beta", "w_qkvu", "b_qkvu", "gln2_gamma", "gln2_beta",
                     "w_mlp1", "b_mlp1", "w_mlp2", "b_mlp2")


def block_backward(x: np.ndarray, groups: np.ndarray, times: np.ndarray, layer: Dict[str, np.ndarray],
                   num_heads: int, dout: np.ndarray, eps: float = 1e-5, mask_mode: str = "dynamic",
                   shared_norm: bool = False):
    """Gradients of block_forward for one user given dout = d loss / d out.

    Returns (dx [n, d], grads) with grads[name] shaped like the parameter (biases included even
    when the layer has none).
    """
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    _, parts = block_forward(x, groups, times, layer, num_heads, eps, return_parts=True,
                             mask_mode=mask_mode, shared_norm=shared_norm)
    a = linear(parts["z"], layer["w_mlp1"], layer.get("b_mlp1"))     # MLP1 pre-activation
    grads = {}
    dhid, grads["w_mlp2"], grads["b_mlp2"] = linear_backward(parts["hid"], layer["w_mlp2"], dout)
    da = dhid * silu_grad(a)
    dz, grads["w_mlp1"], grads["b_mlp1"] = linear_backward(parts["z"], layer["w_mlp1"], da)
    dy, grads["gln2_gamma"], grads["gln2_beta"] = group_layer_norm_backward(
        parts["y"], groups, layer["gln2_gamma"], dz, eps, shared_norm)
    dqkvu = hstu_attention_backward(parts["qkvu"], groups, times, num_heads, dy, mask_mode)
    dxt, grads["w_qkvu"], grads["b_qkvu"] = linear_backward(parts["xt"], layer["w_qkvu"], dqkvu)
    dx1, grads["gln1_gamma"], grads["gln1_beta"] = group_layer_norm_backward(
        x, groups, layer["gln1_gamma"], dxt, eps, shared_norm)
    return dout + dx1, grads


def block_backward_batch(offsets: np.ndarray, groups: np.ndarray, times: np.ndarray, x: np.ndarray,
                         layer: Dict[str, np.ndarray], num_heads: int, dout: np.ndarray,
                         eps: float = 1e-5, mask_mode: str = "dynamic", shared_norm: bool = False):
    """block_backward over a packed batch: dx per token, parameter gradients summed over users."""
    offsets = np.asarray(offsets, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    dx = np.zeros_like(x)
    total = None
    for b in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        dxb, g = block_backward(x[lo:hi], groups[lo:hi], times[lo:hi], layer, num_heads, dout[lo:hi],
                                eps, mask_mode, shared_norm)
        dx[lo:hi] = dxb
        total = g if total is None else {k: total[k] + g[k] for k in g}
    if total is None:
        total = {k: np.zeros_like(np.asarray(layer[k] if layer.get(k) is not None else 0.0, dtype=np.float64))
                 for k in BLOCK_PARAM_NAMES if layer.get(k) is not None}
    return dx, total


# ----------------------------------------------------------------------------------------------
# The block backward under bf16 storage (reading R19): the same chain rule as block_backward,
# with the stored tensors rounded to bfloat16.  Test infrastructure for the bf16 tolerance only.
# ----------------------------------------------------------------------------------------------
def round_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each element (via float32; ties to even), returned as float64."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isfinite(f), out, f.astype(np.float64))


def block_backward_bf16_storage(x: np.ndarray, groups: np.ndarray, times: np.ndarray,
                                layer: Dict[str, np.ndarray], num_heads: int, dout: np.ndarray,
                                eps: float = 1e-5, mask_mode: str = "dynamic", shared_norm: bool = False,
                                store=round_bf16):
    """block_backward for one user with `store` applied wherever a bf16 tensor is kept (R19).

    Forward recompute: X~, QKVU, silu(S) as a product operand, the ungated V~ and the gated Y,
    Z, the MLP1 pre-activation a and then silu(a).  Backward: dout, da = dhid (.) silu'(a), dz,
    dy (the GLN2 input gradient), G = dy (.) U, the masked dS as a product operand, dQ/dK/dV/dU,
    and dX~.  The residual stream x, dx_in and every parameter gradient are sums in float64 of
    the stored values; db2 is the sum of the unrounded dout.  The factor 1/N is applied to the
    product's sum (silu(S) and dS are stored without it).  With store = identity this is
    block_backward step for step.
    """
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    n, d = x.shape
    dh = d // num_heads
    N = float(n)
    M = mask(groups, times, mask_mode).astype(np.float64)
    # forward recompute
    xt = store(group_layer_norm(x, groups, layer["gln1_gamma"], layer["gln1_beta"], eps, shared_norm))
    qkvu = store(linear(xt, layer["w_qkvu"], layer.get("b_qkvu")))
    Q, K, V, U = qkvu[:, :d], qkvu[:, d:2 * d], qkvu[:, 2 * d:3 * d], qkvu[:, 3 * d:]
    acc = np.empty((n, d))
    S_h, P_h = [], []
    for h in range(num_heads):
        sl = slice(h * dh, (h + 1) * dh)
        S = Q[:, sl] @ K[:, sl].T
        P = store(silu(S) * M)                         # a product operand
        acc[:, sl] = P @ V[:, sl] / N
        S_h.append(S)
        P_h.append(P)
    vt = store(acc)                                    # ungated V~
    y = store(acc * U)                                 # V~ (.) U
    z = store(group_layer_norm(y, groups, layer["gln2_gamma"], layer["gln2_beta"], eps, shared_norm))
    a = store(linear(z, layer["w_mlp1"], layer.get("b_mlp1")))
    hid = store(silu(a))
    # MLP2 and the SiLU
    grads = {}
    dout_s = store(dout)
    dhid = dout_s @ np.asarray(layer["w_mlp2"], dtype=np.float64)
    grads["w_mlp2"] = dout_s.T @ hid
    grads["b_mlp2"] = dout.sum(axis=0)
    da = store(dhid * silu_grad(a))
    # MLP1
    dz = store(da @ np.asarray(layer["w_mlp1"], dtype=np.float64))
    grads["w_mlp1"] = da.T @ z
    grads["b_mlp1"] = da.sum(axis=0)
    # GLN2
    dyg, grads["gln2_gamma"], grads["gln2_beta"] = group_layer_norm_backward(
        y, groups, layer["gln2_gamma"], dz, eps, shared_norm)
    dyg = store(dyg)
    # gate and attention
    G = store(dyg * U)
    dqkvu = np.zeros((n, 4 * d))
    for h in range(num_heads):
        sl = slice(h * dh, (h + 1) * dh)
        dP = G[:, sl] @ V[:, sl].T
        dS = store(dP * silu_grad(S_h[h]) * M)         # a product operand
        dqkvu[:, sl] = dS @ K[:, sl] / N
        dqkvu[:, d + h * dh:d + (h + 1) * dh] = dS.T @ Q[:, sl] / N
        dqkvu[:, 2 * d + h * dh:2 * d + (h + 1) * dh] = P_h[h].T @ G[:, sl] / N
    dqkvu[:, 3 * d:] = dyg * vt
    dqkvu = store(dqkvu)
    # QKVU and GLN1 with the residual path
    dxt = store(dqkvu @ np.asarray(layer["w_qkvu"], dtype=np.float64))
    grads["w_qkvu"] = dqkvu.T @ xt
    grads["b_qkvu"] = dqkvu.sum(axis=0)
    dx1, grads["gln1_gamma"], grads["gln1_beta"] = group_layer_norm_backward(
        x, groups, layer["gln1_gamma"], dxt, eps, shared_norm)
    return dout + dx1, grads


def block_backward_batch_bf16_storage(offsets: np.ndarray, groups: np.ndarray, times: np.ndarray,
                                      x: np.ndarray, layer: Dict[str, np.ndarray], num_heads: int,
                                      dout: np.ndarray, eps: float = 1e-5, mask_mode: str = "dynamic",
                                      shared_norm: bool = False, store=round_bf16):
    """block_backward_bf16_storage over a packed batch (dx per token, gradients summed over users)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    dx = np.zeros_like(x)
    total = None
    for b in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        dxb, g = block_backward_bf16_storage(x[lo:hi], groups[lo:hi], times[lo:hi], layer, num_heads,
                                             dout[lo:hi], eps, mask_mode, shared_norm, store)
        dx[lo:hi] = dxb
        total = g if total is None else {k: total[k] + g[k] for k in g}
    return dx, total
