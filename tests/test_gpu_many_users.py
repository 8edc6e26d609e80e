"""GPU parity with more than 16,384 users in one batch.

Above that many users the attention work is queued in user-index order instead of longest first;
the host sizes the launch grid from the same rule, so every (user, head, q-tile) runs (packed users
are each computed in full: chenhuiyu blog "MTGR", training-system section).  Attention forward and
backward on ~2.2M tokens of short users (1-3 q-tiles each): every output row must be written
(outputs start as NaN) and sampled users -- the first and last in index order, the longest, and a
random few -- match the fp64 oracle at the single-kernel bf16 tolerance (1e-2 of the largest
magnitude per tensor; see test_gpu_parity.py).
"""
import numpy as np
import pytest
import torch

from generative_recommendation_ranking_amd import mtgr as M
from generative_recommendation_ranking_amd import synth
from oracle import mtgr_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 1e-2
B_USERS = 16_500


def rel_err(g, r):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)) if r.size else 0.0


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(16_500)
    n_u = np.full(B_USERS, 2)
    n_s = rng.integers(4, 201, B_USERS)
    n_r = rng.integers(0, 41, B_USERS)
    k = rng.integers(0, 17, B_USERS)
    b = synth.batch_from_lengths(n_u, n_s, n_r, k, 8, rng, "bf16")   # x unused here: 8 wide
    db = M.DeviceBatch(b)
    d, H = 256, 2
    g = torch.Generator(device=DEV)
    g.manual_seed(16_501)
    qkvu = torch.randn(b.num_tokens, 4 * d, device=DEV, generator=g)
    qkvu[:, :2 * d] *= 2.0 / np.sqrt(np.sqrt(d // H))   # scores with std ~4: the curved part of silu
    qkvu = qkvu.to(torch.bfloat16)
    n = np.diff(b.offsets)
    users = sorted(set([0, 1, 2, B_USERS - 5, B_USERS - 4, B_USERS - 3, B_USERS - 2, B_USERS - 1,
                        int(np.argmax(n))] + rng.choice(B_USERS, 6, replace=False).tolist()))
    assert b.num_users > 16_384 and int(n.max()) > 2 * 128
    return b, db, d, H, qkvu, users


def _host_rows(t, b, u):
    lo, hi = int(b.offsets[u]), int(b.offsets[u + 1])
    return t[lo:hi].float().cpu().numpy().astype(np.float64), lo, hi


def test_attention_fwd_more_than_16k_users(case):
    b, db, d, H, qkvu, users = case
    y = torch.full((b.num_tokens, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = M.workspace(M.mtgr_attention_workspace_size(db, d, H))
    M.mtgr_attention_fwd(db, d, H, M.MTGR_BF16, M.MTGR_MASK_DYNAMIC, qkvu, y, ws)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(y).any()), "rows of some users were never written"
    errs = []
    for u in users:
        q, lo, hi = _host_rows(qkvu, b, u)
        ref = O.hstu_attention(q, b.group_ids[lo:hi], b.timestamps[lo:hi], H)
        got = y[lo:hi].float().cpu().numpy()
        errs.append(rel_err(got, ref))
        assert errs[-1] < TOL, f"user {u}"
    print(f"attention fwd, {b.num_users} users, {b.num_tokens} tokens: max rel err {max(errs):.2e} "
          f"over users {users}")


def test_attention_bwd_more_than_16k_users(case):
    b, db, d, H, qkvu, users = case
    g = torch.Generator(device=DEV)
    g.manual_seed(16_502)
    vt = torch.randn(b.num_tokens, d, device=DEV, generator=g).to(torch.bfloat16)
    dy = torch.randn(b.num_tokens, d, device=DEV, generator=g).to(torch.bfloat16)
    dq = torch.full((b.num_tokens, 4 * d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = M.workspace(M.mtgr_attention_bwd_workspace_size(db, d, H, M.MTGR_BF16))
    M.mtgr_attention_bwd(db, d, H, M.MTGR_BF16, M.MTGR_MASK_DYNAMIC, qkvu, vt, dy, dq, ws)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(dq).any()), "rows of some users were never written"
    worst = 0.0
    for u in users:
        q, lo, hi = _host_rows(qkvu, b, u)
        dyu, _, _ = _host_rows(dy, b, u)
        vtu, _, _ = _host_rows(vt, b, u)
        ref = O.hstu_attention_backward(q, b.group_ids[lo:hi], b.timestamps[lo:hi], H, dyu)
        ref[:, 3 * d:] = dyu * vtu                      # dU from the V~ that was passed in
        got = dq[lo:hi].float().cpu().numpy()
        for blk, name in enumerate("QKVU"):
            sl = slice(blk * d, (blk + 1) * d)
            e = rel_err(got[:, sl], ref[:, sl])
            worst = max(worst, e)
            assert e < TOL, f"user {u} d{name}"
    print(f"attention bwd, {b.num_users} users: max rel err {worst:.2e}")
