"""CPU oracle for MTGR's embedding front end -- TEST INFRASTRUCTURE ONLY.

Only the tests and the benchmark's CPU-baseline leg may import this module.  The product path
never imports it, and it imports nothing from the product path.  Plain Python dicts and numpy
float64, written from the pages' description, step by step.

What the pages say (page keys as in mtgr_oracle.py):
  * the embedding tables are hash-based and decoupled: a compact index from key to pointer plus a
    separate value structure, so sparse IDs can be inserted and evicted in real time without
    preallocating capacity                         [P3 方法, training-framework paragraph; P1/P2
                                                    training-system section]
  * embedding IDs are deduplicated (two stages, before the cross-device lookup) and tables are
    merged automatically to cut lookups            [P3 方法 and 主要贡献; P1/P2 training-system]
  * tokens: a scalar user feature becomes one token; a sequence item embeds its several fields,
    concatenates them and projects them to d_model with an MLP of its own domain; a candidate
    token is MLP(Concat(Emb(Item_i), Emb(Cross_i)))   [P1/P2 "Converting heterogeneous features
                                                    into tokens"; P5 7.3.2, candidate-token eq.]

Readings (the same numbering as the design notes):
  R15 every group (U, S, R, C) has its own fixed list of fields, each read from an embedding table
      of one common width e; the token's feature is the concatenation of its fields' embeddings in
      list order; the domain MLP is Linear(F_g e -> d) -> SiLU -> Linear(d -> d), with biases.
  R16 table merging: tables of the same width share one key space, key = (table << 40) | id, so one
      store and one dedup pass serve every field.  A key absent from the store embeds to zeros.
  R17 dedup: the batch's keys are reduced to their distinct values plus, for every occurrence, the
      index of its distinct key; each distinct key is looked up once.  On one device the second
      stage (at the key's owner, over the keys received from every device) sees a single sender
      and returns the first stage's result unchanged.
  R18 the store's observable behaviour is that of a map from key to value row: insert keeps an
      existing key's value, takes a free row for a new key and initialises it, fails when no row
      is free; lookup returns the value or reports the key missing; evict frees the key's row;
      evict_older evicts every key whose last use is older than a given step.

R15-R17 fill in what the pages leave open (how many fields, their widths, the MLP's depth) and are
parity unpinned with respect to the pages: the functions below are pinned to these readings, not
to anything the pages fix.

parity pins: tests/test_oracle_pins.py checks the store model against a brute-force list-of-pairs
model over random operation sequences and against its invariants, dedup against Python sets, and
the tokenizer against an independent torch formulation (nn.Embedding, cat, nn.Linear).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

KEY_TABLE_SHIFT = 40          # merged key = (table << 40) | id  (R16)
NUM_GROUPS = 4


def merged_key(table: int, ident: int) -> int:
    """R16: one key space for all tables of one width."""
    if not (0 <= ident < (1 << KEY_TABLE_SHIFT)):
        raise ValueError("id out of range")
    return (int(table) << KEY_TABLE_SHIFT) | int(ident)


# ----------------------------------------------------------------------------------------------
# The store: index (key -> row) plus a separate value arena with a free pool (R18).
# ----------------------------------------------------------------------------------------------
class EmbeddingStore:
    """Map model of the hash embedding store.  Rows are handed out from a free pool; which row a
    new key gets is not part of the behaviour (any free row is valid)."""

    def __init__(self, rows: int, dim: int):
        self.rows = int(rows)
        self.dim = int(dim)
        self.index: Dict[int, int] = {}
        self.values = np.zeros((self.rows, self.dim))
        self.last_seen = np.zeros(self.rows, dtype=np.int64)
        self.free: List[int] = list(range(self.rows - 1, -1, -1))   # pop() gives 0, 1, 2, ...
        self.failed = 0

    def insert(self, keys: Sequence[int], init: Optional[np.ndarray], step: int) -> List[int]:
        """Row of each key after the call, -1 where it could not be inserted.  A key already
        present keeps its value; a new key takes a free row initialised from its init row (zeros
        without init).  A key occurring twice in one call is inserted once."""
        out = []
        for i, k in enumerate(keys):
            k = int(k)
            if k < 0:
                self.failed += 1
                out.append(-1)
                continue
            if k in self.index:
                row = self.index[k]
            elif self.free:
                row = self.free.pop()
                self.index[k] = row
                self.values[row] = 0.0 if init is None else np.asarray(init[i], dtype=np.float64)
            else:
                self.failed += 1
                out.append(-1)
                continue
            self.last_seen[row] = step
            out.append(row)
        return out

    def lookup(self, keys: Sequence[int], step: int = -1) -> Tuple[np.ndarray, np.ndarray]:
        """(values [n][dim], found [n]); a missing key reads as zeros.  step >= 0 marks the found
        keys as used at that step."""
        vals = np.zeros((len(keys), self.dim))
        found = np.zeros(len(keys), dtype=bool)
        for i, k in enumerate(keys):
            row = self.index.get(int(k))
            if row is not None:
                vals[i] = self.values[row]
                found[i] = True
                if step >= 0:
                    self.last_seen[row] = step
        return vals, found

    def evict(self, keys: Sequence[int]) -> None:
        for k in keys:
            row = self.index.pop(int(k), None)
            if row is not None:
                self.free.append(row)

    def evict_older(self, threshold: int) -> None:
        stale = [k for k, row in self.index.items() if self.last_seen[row] < threshold]
        self.evict(stale)

    def live_keys(self) -> Dict[int, int]:
        return dict(self.index)

    def stats(self) -> Dict[str, int]:
        return {"live": len(self.index), "free_rows": len(self.free), "failed_inserts": self.failed}


# ----------------------------------------------------------------------------------------------
# Dedup (R17)
# ----------------------------------------------------------------------------------------------
def unique_with_inverse(keys: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Distinct keys (ascending) and, per occurrence, the index of its distinct key:
    keys == uniq[inverse]."""
    uniq, inv = np.unique(np.asarray(keys, dtype=np.int64), return_inverse=True)
    return uniq, inv.reshape(-1)


# ----------------------------------------------------------------------------------------------
# Tokenizer (R15-R17)
# ----------------------------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def token_features(field_ids: np.ndarray, groups: np.ndarray, field_tables: Sequence[Sequence[int]],
                   store: EmbeddingStore) -> List[np.ndarray]:
    """Per token, the concatenation of its fields' embeddings (R15): field f of group g reads table
    field_tables[g][f] at the token's id in column f of field_ids."""
    feats = []
    for t in range(field_ids.shape[0]):
        g = int(groups[t])
        parts = []
        for f, table in enumerate(field_tables[g]):
            key = merged_key(table, int(field_ids[t, f]))
            vals, _ = store.lookup([key])
            parts.append(vals[0])
        feats.append(np.concatenate(parts))
    return feats


def tokenize(field_ids: np.ndarray, groups: np.ndarray, field_tables: Sequence[Sequence[int]],
             store: EmbeddingStore, mlps: Sequence[Dict[str, np.ndarray]]) -> np.ndarray:
    """Encoder input x [T][d]: each token's domain MLP (mlps[g]: w1 [d][F_g e], b1 [d], w2 [d][d],
    b2 [d]) applied to its concatenated field embeddings."""
    feats = token_features(field_ids, groups, field_tables, store)
    d = np.asarray(mlps[0]["w2"]).shape[0]
    x = np.zeros((len(feats), d))
    for t, f in enumerate(feats):
        m = mlps[int(groups[t])]
        hid = silu(np.asarray(m["w1"], np.float64) @ f + np.asarray(m["b1"], np.float64))
        x[t] = np.asarray(m["w2"], np.float64) @ hid + np.asarray(m["b2"], np.float64)
    return x
