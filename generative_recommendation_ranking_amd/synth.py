"""Seeded synthetic inputs and weights for the MTGR encoder forward.

This module draws random numbers and lays them out; it holds none of the method's arithmetic
(no normalisation, projection, mask or attention).  Both the GPU path and the CPU oracle consume
its arrays, so the two see bit-identical inputs.

Sample layout follows the user-level aggregation of the MTGR pages: one sample per user is the
token sequence D = [U, S, R, [C,I]_1..K] (marovi.ai page "MTGR: Industrial-Scale Generative
Recommendation Framework in Meituan", section 方法, the equation for D; fun-rec page "MTGR: Hybrid
Paradigm Modeling", section 7.3.1).  Users are packed back to back (sequence packing, chenhuiyu
blog "MTGR", section on the training system), described by offsets, a per-token group id
(0=U static user feature, 1=S long-term history, 2=R real-time event, 3=C candidate) and a
per-token timestamp in seconds (float32; -inf for U and S, which precede the aggregation window).

The pages measure on a proprietary Meituan dataset that is not available; these workloads stand
in for it with the pages' token groups and history caps.

Draw order (fixed, per workload seed = 250518654 + seed_offset, numpy PCG64):
  1. lengths: N_S for all users, then (large workload only) the long-tail users from one
     permutation, then N_R for all users, then K for all users (N_U is fixed);
  2. timestamps user by user: R = sort(uniform[0,3600)), C = uniform[0,3600) unsorted;
  3. embeddings N(0,1) [T,d] float32 in token order (rows in chunks of 65536, chunk c from the
     PCG64 state jumped c+1 times), times the group scale (U 1, S 0.5, R 2, C 4); bf16 workloads
     round them to bf16 (round to nearest even);
  4. parameters layer by layer: GLN1 gamma~U(0.5,1.5) [4,d], beta~U(-0.1,0.1) [4,d];
     W_qkvu [4d,d] Xavier-uniform per d x d block; GLN2 gamma, beta; W1 [h,d]; W2 [d,h]
     (Xavier-uniform); biases 0; then the head W_h1 [d/2,d], W_h2 [2,d/2] (Xavier-uniform,
     biases 0).  bf16 workloads round every parameter to bf16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

G_U, G_S, G_R, G_C = 0, 1, 2, 3
GROUP_SCALE = (1.0, 0.5, 2.0, 4.0)
SEED_BASE = 250518654

# Workloads: shapes of the MTGR model sizes on the pages (3 blocks d=512 small, 5 blocks d=768
# medium, 15 blocks d=768 large; marovi.ai page, section 结果) scaled to one GPU, and the pages'
# history caps (1000 long-term, 100 real-time events).
WORKLOADS: Dict[str, dict] = {
    "tiny-fp32": dict(seed_offset=0, L=1, d=64, H=2, h=128, B=4, n_u=8, n_s=(32, 32),
                      n_r=(8, 8), k=(8, 8), dtype="f32", tail=None),
    "small-bf16": dict(seed_offset=1, L=3, d=256, H=4, h=1024, B=256, n_u=16, n_s=(64, 1000),
                       n_r=(0, 100), k=(1, 64), dtype="bf16", tail=None),
    "medium-bf16": dict(seed_offset=2, L=5, d=512, H=4, h=2048, B=512, n_u=24, n_s=(200, 2000),
                        n_r=(10, 200), k=(8, 128), dtype="bf16", tail=None),
    "large-bf16": dict(seed_offset=3, L=8, d=768, H=6, h=3072, B=256, n_u=32, n_s=(1000, 3000),
                       n_r=(50, 300), k=(32, 256), dtype="bf16", tail=(0.1, 3000)),
    "inference-bf16": dict(seed_offset=4, L=5, d=512, H=4, h=2048, B=1024, n_u=24,
                           n_s=(1000, 1000), n_r=(0, 50), k=(512, 512), dtype="bf16", tail=None),
}


@dataclasses.dataclass
class Batch:
    """A packed jagged batch.  Tokens of user b are rows offsets[b]:offsets[b+1]."""
    offsets: np.ndarray      # int64 [B+1]
    group_ids: np.ndarray    # uint8 [T]
    timestamps: np.ndarray   # float32 [T]
    x: np.ndarray            # float32 [T, d]  (bf16-representable values for bf16 workloads)
    n_u: np.ndarray          # int64 [B]
    n_s: np.ndarray          # int64 [B]
    n_r: np.ndarray          # int64 [B]
    k: np.ndarray            # int64 [B]

    @property
    def num_users(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def num_tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def num_candidates(self) -> int:
        return int(self.k.sum())

    @property
    def d(self) -> int:
        return int(self.x.shape[1])


@dataclasses.dataclass
class Params:
    """Weights in torch Linear layout ([out, in], row-major), stored as float32 numpy arrays
    whose values are representable in `dtype` ("f32" or "bf16")."""
    dtype: str
    d: int
    H: int
    h: int
    layers: List[Dict[str, np.ndarray]]
    head: Dict[str, np.ndarray]
    ln_eps: float = 1e-5

    @property
    def num_layers(self) -> int:
        return len(self.layers)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even) -> float32; pure storage encoding (torch's RNE cast,
    multithreaded).  Returns a new array."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return round_to_bf16(a) if dtype == "bf16" else a


ROW_CHUNK = 65536


def _normal_rows(rng: np.random.Generator, T: int, d: int) -> np.ndarray:
    """N(0,1) float32 [T, d].  Rows come in chunks of ROW_CHUNK; chunk c is drawn from the
    caller's PCG64 state jumped c+1 times (independent streams, filled in parallel threads).
    The caller's own generator is not advanced."""
    import concurrent.futures
    x = np.empty((T, d), dtype=np.float32)
    chunks = [(c, s, min(s + ROW_CHUNK, T)) for c, s in enumerate(range(0, T, ROW_CHUNK))]

    def fill(job):
        c, lo, hi = job
        g = np.random.Generator(rng.bit_generator.jumped(c + 1))
        g.standard_normal((hi - lo, d), dtype=np.float32, out=x[lo:hi])

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, chunks))
    return x


def batch_from_lengths(n_u: Sequence[int], n_s: Sequence[int], n_r: Sequence[int],
                       k: Sequence[int], d: int, rng: np.random.Generator,
                       dtype: str = "f32") -> Batch:
    """Builds timestamps and embeddings for given per-user segment lengths (draw steps 2-3)."""
    n_u = np.asarray(n_u, dtype=np.int64)
    n_s = np.asarray(n_s, dtype=np.int64)
    n_r = np.asarray(n_r, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    n = n_u + n_s + n_r + k
    B = n.shape[0]
    offsets = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(n, out=offsets[1:])
    T = int(offsets[-1])
    group_ids = np.empty(T, dtype=np.uint8)
    timestamps = np.empty(T, dtype=np.float32)
    for b in range(B):
        o = int(offsets[b])
        segs = (int(n_u[b]), int(n_s[b]), int(n_r[b]), int(k[b]))
        p = o
        for g, cnt in enumerate(segs):
            group_ids[p:p + cnt] = g
            p += cnt
        s0 = o + segs[0] + segs[1]
        timestamps[o:s0] = -np.inf
        timestamps[s0:s0 + segs[2]] = np.sort(rng.uniform(0.0, 3600.0, segs[2])).astype(np.float32)
        timestamps[s0 + segs[2]:p] = rng.uniform(0.0, 3600.0, segs[3]).astype(np.float32)
    x = _normal_rows(rng, T, d)
    scale = np.asarray(GROUP_SCALE, dtype=np.float32)[group_ids]
    x *= scale[:, None]
    x = _encode(x, dtype)
    return Batch(offsets, group_ids, timestamps, x, n_u, n_s, n_r, k)


def _xavier(rng: np.random.Generator, fan_out: int, fan_in: int) -> np.ndarray:
    a = math.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-a, a, size=(fan_out, fan_in)).astype(np.float32)


def make_params(rng: np.random.Generator, L: int, d: int, H: int, h: int, dtype: str,
                head_hidden: Optional[int] = None) -> Params:
    """Draw step 4: per-layer parameters, then the candidate head."""
    layers = []
    for _ in range(L):
        lay = {}
        lay["gln1_gamma"] = rng.uniform(0.5, 1.5, size=(4, d)).astype(np.float32)
        lay["gln1_beta"] = rng.uniform(-0.1, 0.1, size=(4, d)).astype(np.float32)
        lay["w_qkvu"] = np.concatenate([_xavier(rng, d, d) for _ in range(4)], axis=0)
        lay["b_qkvu"] = np.zeros(4 * d, dtype=np.float32)
        lay["gln2_gamma"] = rng.uniform(0.5, 1.5, size=(4, d)).astype(np.float32)
        lay["gln2_beta"] = rng.uniform(-0.1, 0.1, size=(4, d)).astype(np.float32)
        lay["w_mlp1"] = _xavier(rng, h, d)
        lay["b_mlp1"] = np.zeros(h, dtype=np.float32)
        lay["w_mlp2"] = _xavier(rng, d, h)
        lay["b_mlp2"] = np.zeros(d, dtype=np.float32)
        layers.append({k_: _encode(v, dtype) for k_, v in lay.items()})
    hh = head_hidden if head_hidden is not None else d // 2
    head = {
        "w_head1": _xavier(rng, hh, d),
        "b_head1": np.zeros(hh, dtype=np.float32),
        "w_head2": _xavier(rng, 2, hh),
        "b_head2": np.zeros(2, dtype=np.float32),
    }
    head = {k_: _encode(v, dtype) for k_, v in head.items()}
    return Params(dtype=dtype, d=d, H=H, h=h, layers=layers, head=head)


def workload_lengths(name: str, rng: np.random.Generator):
    """Draw step 1 for a named workload."""
    w = WORKLOADS[name]
    B = w["B"]
    n_u = np.full(B, w["n_u"], dtype=np.int64)
    n_s = rng.integers(w["n_s"][0], w["n_s"][1], endpoint=True, size=B).astype(np.int64)
    if w["tail"] is not None:
        frac, val = w["tail"]
        idx = rng.permutation(B)[: int(round(frac * B))]
        n_s[idx] = val
    n_r = rng.integers(w["n_r"][0], w["n_r"][1], endpoint=True, size=B).astype(np.int64)
    k = rng.integers(w["k"][0], w["k"][1], endpoint=True, size=B).astype(np.int64)
    return n_u, n_s, n_r, k


def make_workload(name: str, with_params: bool = True):
    """Returns (Batch, Params) for a named workload, fully determined by its seed."""
    w = WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + w["seed_offset"]))
    n_u, n_s, n_r, k = workload_lengths(name, rng)
    batch = batch_from_lengths(n_u, n_s, n_r, k, w["d"], rng, w["dtype"])
    params = make_params(rng, w["L"], w["d"], w["H"], w["h"], w["dtype"]) if with_params else None
    return batch, params


def subset(batch: Batch, users: Sequence[int]) -> Batch:
    """Repacks the chosen users (in the given order) into a new batch."""
    users = [int(u) for u in users]
    rows = np.concatenate([np.arange(batch.offsets[u], batch.offsets[u + 1]) for u in users]) \
        if users else np.zeros(0, dtype=np.int64)
    n = np.asarray([batch.offsets[u + 1] - batch.offsets[u] for u in users], dtype=np.int64)
    offsets = np.zeros(len(users) + 1, dtype=np.int64)
    np.cumsum(n, out=offsets[1:])
    sel = np.asarray(users, dtype=np.int64)
    return Batch(offsets, batch.group_ids[rows].copy(), batch.timestamps[rows].copy(),
                 batch.x[rows].copy(), batch.n_u[sel].copy(), batch.n_s[sel].copy(),
                 batch.n_r[sel].copy(), batch.k[sel].copy())


def user_rows(batch: Batch, users: Sequence[int]) -> np.ndarray:
    """Token rows of the chosen users in the packed batch, in subset() order."""
    if len(users) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(batch.offsets[u], batch.offsets[u + 1]) for u in users])


def candidate_rows(batch: Batch, users: Sequence[int]) -> np.ndarray:
    """Rows of the logits matrix (candidates in packed order) that belong to the chosen users."""
    cand_off = np.zeros(batch.num_users + 1, dtype=np.int64)
    np.cumsum(batch.k, out=cand_off[1:])
    if len(users) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(cand_off[u], cand_off[u + 1]) for u in users])


# ---------------------------------------------------------------------------------------------
# Tokenizer inputs: field IDs per token, the per-group MLP weights, and the contents of the
# embedding store, as (table, id) pairs with their rows.  The field lists are this generator's
# choice (the pages name the kinds of fields, not their number): U tokens carry (feature slot,
# feature value); S and R items (item, category, brand, action) and (item, category, action,
# time bucket); candidates (item, category, brand, user x category cross bucket, hour-preference
# bucket, list position).  Item ids follow a Zipf law, so the batch repeats them across users.
# ---------------------------------------------------------------------------------------------
TOK_FIELD_TABLES = ([0, 1], [2, 3, 4, 5], [2, 3, 5, 6], [2, 3, 4, 7, 8, 9])
TOK_VOCAB = (32, 1000, 1_000_000, 1000, 10_000, 8, 64, 100, 24, 512)


@dataclasses.dataclass
class TokenizerSpec:
    d: int
    e: int
    field_tables: Sequence[Sequence[int]]
    mlps: List[Dict[str, np.ndarray]]      # per group: w1 [d][F_g e], b1 [d], w2 [d][d], b2 [d]

    @property
    def max_fields(self) -> int:
        return max(len(f) for f in self.field_tables)


def make_tokenizer_inputs(batch: Batch, rng: np.random.Generator, d: int, e: int = 64,
                          missing_frac: float = 0.05):
    """(spec, field_ids [T][F_max] int64, group_counts [4], store_tables, store_ids, store_values):
    the store holds every (table, id) pair the batch uses except about `missing_frac` of them,
    each with a N(0, 1) row rounded to bf16."""
    T = batch.num_tokens
    g = batch.group_ids.astype(np.int64)
    fmax = max(len(f) for f in TOK_FIELD_TABLES)
    ids = np.full((T, fmax), -1, dtype=np.int64)
    item = (rng.zipf(1.2, T) - 1) % TOK_VOCAB[2]
    for grp, tables in enumerate(TOK_FIELD_TABLES):
        rows = np.nonzero(g == grp)[0]
        for f, tab in enumerate(tables):
            if tab == 2:
                col = item[rows]
            elif tab == 3:
                col = item[rows] % TOK_VOCAB[3]
            elif tab == 4:
                col = (item[rows] * 7) % TOK_VOCAB[4]
            elif tab == 0 or tab == 9:       # slot of a U feature / list position of a candidate
                starts = np.concatenate([[0], np.nonzero(np.diff(rows) != 1)[0] + 1])
                run = np.zeros(len(rows), dtype=np.int64)
                for s0, s1 in zip(starts, np.concatenate([starts[1:], [len(rows)]])):
                    run[s0:s1] = np.arange(s1 - s0)
                col = run % TOK_VOCAB[tab]
            else:
                col = rng.integers(0, TOK_VOCAB[tab], len(rows))
            ids[rows, f] = col
    counts = np.bincount(g, minlength=4)[:4].astype(np.int64)
    mlps = []
    for tables in TOK_FIELD_TABLES:
        k = len(tables) * e
        mlps.append({"w1": round_to_bf16(_xavier(rng, d, k)),
                     "b1": round_to_bf16(rng.uniform(-0.1, 0.1, d).astype(np.float32)),
                     "w2": round_to_bf16(_xavier(rng, d, d)),
                     "b2": round_to_bf16(rng.uniform(-0.1, 0.1, d).astype(np.float32))})
    spec = TokenizerSpec(d=d, e=e, field_tables=TOK_FIELD_TABLES, mlps=mlps)
    pairs = set()
    for grp, tables in enumerate(TOK_FIELD_TABLES):
        rows = g == grp
        for f, tab in enumerate(tables):
            for i in np.unique(ids[rows, f]).tolist():
                pairs.add((tab, int(i)))
    pairs = sorted(pairs)
    keep = rng.random(len(pairs)) >= missing_frac
    tabs = np.array([p[0] for p in pairs], dtype=np.int64)[keep]
    pids = np.array([p[1] for p in pairs], dtype=np.int64)[keep]
    vals = round_to_bf16(rng.standard_normal((len(tabs), e)).astype(np.float32))
    return spec, ids, counts, tabs, pids, vals
