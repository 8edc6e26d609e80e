"""Pins of the CPU oracle against things other than itself (runs without a GPU).

Each test checks the oracle against a fact the pages or the mathematics fix: hand-built masks for
the pages' worked examples, the block structure the pages describe, GroupLN invariants and torch's
layer_norm, closed forms and library reductions of the attention, and invariants the method must
satisfy (candidate permutation equivariance, candidate independence, user isolation, no temporal
leakage).  A plausible slip in the oracle (a wrong comparison, a transposed product, a dropped 1/N,
a wrong group index) fails at least one of them.
"""
import os

import numpy as np
import pytest
import torch

from oracle import mtgr_oracle as O
from generative_recommendation_ranking_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden_mask(name):
    rows, groups, times = [], None, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("groups"):
                groups = np.array([int(v) for v in line.split()[1:]], dtype=np.uint8)
            elif line.startswith("times"):
                times = np.array([float(v) for v in line.split()[1:]], dtype=np.float32)
            else:
                rows.append([int(v) for v in line.split()])
    return groups, times, np.array(rows, dtype=np.uint8)


# ------------------------------------------------------------------------------------------
# Mask: worked examples and block structure ([P1] eight-item example, [P5] 7.3.4)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["mask_toy8.txt", "mask_temporal_abc.txt"])
def test_mask_golden(name):
    g, t, expected = _read_golden_mask(name)
    assert expected.shape == (g.shape[0], g.shape[0])
    np.testing.assert_array_equal(O.mask(g, t), expected)


def test_mask_p5_layout_blocks():
    # [P5] 7.3.3 layout: [Age, Gender, City, Seq_1..100, RT_1..10, Cand_1..3]
    n_u, n_s, n_r, k = 3, 100, 10, 3
    g = np.array([0] * n_u + [1] * n_s + [2] * n_r + [3] * k, dtype=np.uint8)
    t_r = np.arange(n_r, dtype=np.float32) * 60.0            # distinct, increasing
    t_c = np.array([-1.0, 270.0, 10_000.0], dtype=np.float32)  # before all, mid, after all
    t = np.concatenate([np.full(n_u + n_s, -np.inf, np.float32), t_r, t_c])
    M = O.mask(g, t)
    s = n_u + n_s
    r0, r1 = s, s + n_r
    assert (M[:, :s] == 1).all()                       # rule 1: U/S columns all ones
    assert (M[:s, s:] == 0).all()                      # static rows see no R and no C
    np.testing.assert_array_equal(M[r0:r1, r0:r1], np.tril(np.ones((n_r, n_r), np.uint8)))  # rule 2
    np.testing.assert_array_equal(M[r1:, r1:], np.eye(k, dtype=np.uint8))  # rule 3: diagonal
    assert (M[r0:r1, r1:] == 0).all()                  # R rows never see candidates
    # candidate -> R by exposure time
    np.testing.assert_array_equal(M[r1 + 0, r0:r1], np.zeros(n_r, np.uint8))
    np.testing.assert_array_equal(M[r1 + 1, r0:r1], (t_r < 270.0).astype(np.uint8))
    np.testing.assert_array_equal(M[r1 + 2, r0:r1], np.ones(n_r, np.uint8))


def test_mask_ties_and_order_agnostic():
    rng = np.random.default_rng(7)
    # equal timestamps: invisible to each other (strict), visible to self
    g = np.array([0, 2, 2, 3], np.uint8)
    t = np.array([-np.inf, 5.0, 5.0, 5.0], np.float32)
    M = O.mask(g, t)
    np.testing.assert_array_equal(M, np.array([[1, 0, 0, 0], [1, 1, 0, 0], [1, 0, 1, 0], [1, 0, 0, 1]], np.uint8))
    # permuting the tokens permutes the mask (the rules are type-based, not position-based)
    g = np.array([0] * 3 + [1] * 5 + [2] * 6 + [3] * 4, np.uint8)
    t = np.concatenate([np.full(8, -np.inf), rng.uniform(0, 10, 10)]).astype(np.float32)
    perm = rng.permutation(g.shape[0])
    np.testing.assert_array_equal(O.mask(g[perm], t[perm]), O.mask(g, t)[np.ix_(perm, perm)])


def test_mask_empty_segments():
    # a user with only candidates, a user with only static tokens, an empty user
    np.testing.assert_array_equal(O.mask(np.array([3, 3, 3], np.uint8), np.array([1, 1, 1], np.float32)),
                                  np.eye(3, dtype=np.uint8))
    np.testing.assert_array_equal(O.mask(np.array([0, 1, 1], np.uint8), np.full(3, -np.inf, np.float32)),
                                  np.ones((3, 3), np.uint8))
    assert O.mask(np.zeros(0, np.uint8), np.zeros(0, np.float32)).shape == (0, 0)


def test_visible_pair_closed_form():
    # sorted distinct R: pairs = n*n_static + n_R(n_R+1)/2 + sum_c #{R: t_r < t_c} + K
    rng = np.random.default_rng(3)
    for _ in range(5):
        n_u, n_s, n_r, k = [int(v) for v in rng.integers(0, 20, 4)]
        t_r = np.sort(rng.permutation(1000)[:n_r].astype(np.float32))
        t_c = rng.uniform(0, 1000, k).astype(np.float32)
        g = np.array([0] * n_u + [1] * n_s + [2] * n_r + [3] * k, np.uint8)
        t = np.concatenate([np.full(n_u + n_s, -np.inf, np.float32), t_r, t_c])
        n = g.shape[0]
        expect = n * (n_u + n_s) + n_r * (n_r + 1) // 2 + sum(int((t_r < c).sum()) for c in t_c) + k
        assert O.visible_pairs(g, t) == expect


# ------------------------------------------------------------------------------------------
# GroupLN ([P5] 7.3.3): per-token statistics, per-group affine
# ------------------------------------------------------------------------------------------
def test_groupln_matches_layer_norm_per_group():
    rng = np.random.default_rng(11)
    n, d = 40, 48
    x = rng.standard_normal((n, d)) * rng.uniform(0.1, 5, (n, 1)) + rng.uniform(-3, 3, (n, 1))
    g = rng.integers(0, 4, n).astype(np.uint8)
    gamma = rng.uniform(0.5, 1.5, (4, d))
    beta = rng.uniform(-0.1, 0.1, (4, d))
    y = O.group_layer_norm(x, g, gamma, beta, 1e-5)
    for grp in range(4):
        rows = g == grp
        ref = torch.nn.functional.layer_norm(torch.from_numpy(x[rows]), (d,),
                                             torch.from_numpy(gamma[grp]), torch.from_numpy(beta[grp]), 1e-5)
        np.testing.assert_allclose(y[rows], ref.numpy(), rtol=0, atol=1e-12)


def test_groupln_invariants():
    rng = np.random.default_rng(12)
    n, d = 64, 32
    x = rng.standard_normal((n, d)) * 3.0 + 1.0
    g = np.repeat(np.arange(4, dtype=np.uint8), n // 4)
    ones, zeros = np.ones((4, d)), np.zeros((4, d))
    y = O.group_layer_norm(x, g, ones, zeros, 1e-5)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    # per-group pooled mean 0 / variance ~1 follows from the per-token statistics
    for grp in range(4):
        assert abs(y[g == grp].mean()) < 1e-12
        assert abs(y[g == grp].var() - 1.0) < 1e-5
    # invariant to a positive per-token scale (the groups' x1/x0.5/x2/x4 input scales), up to eps
    s = np.array([1.0, 0.5, 2.0, 4.0])[g][:, None]
    np.testing.assert_allclose(O.group_layer_norm(x * s, g, ones, zeros, 0.0),
                               O.group_layer_norm(x, g, ones, zeros, 0.0), atol=1e-12)


# ------------------------------------------------------------------------------------------
# Attention: library reductions and closed forms ([P3] update equation for V~)
# ------------------------------------------------------------------------------------------
def _qkvu(rng, n, d):
    return rng.standard_normal((n, 4 * d)) * 0.7


def _torch_silu_attention(q, k, v, u, maskmat, n):
    # dense silu attention with a given 0/1 mask, torch fp64
    q, k, v, u, m = (torch.from_numpy(a) for a in (q, k, v, u, maskmat))
    return ((torch.nn.functional.silu(q @ k.T) / n * m) @ v * u).numpy()


@pytest.mark.parametrize("H", [1, 2, 4])
def test_attention_all_static_is_dense_silu_attention(H):
    rng = np.random.default_rng(20 + H)
    n, d = 37, 32
    qkvu = _qkvu(rng, n, d)
    g = np.array([0] * 5 + [1] * (n - 5), np.uint8)
    t = np.full(n, -np.inf, np.float32)
    y = O.hstu_attention(qkvu, g, t, H)
    dh = d // H
    for h in range(H):
        sl = slice(h * dh, (h + 1) * dh)
        q, k, v = qkvu[:, sl], qkvu[:, d:2 * d][:, sl], qkvu[:, 2 * d:3 * d][:, sl]
        u = qkvu[:, 3 * d:][:, sl]
        ref = _torch_silu_attention(q, k, v, u, np.ones((n, n)), n)
        np.testing.assert_allclose(y[:, sl], ref, rtol=1e-12, atol=1e-14)


def test_attention_sorted_realtime_is_causal_tril():
    rng = np.random.default_rng(30)
    n, d = 29, 16
    qkvu = _qkvu(rng, n, d)
    g = np.full(n, 2, np.uint8)
    t = np.sort(rng.permutation(10_000)[:n]).astype(np.float32)   # strictly increasing
    y = O.hstu_attention(qkvu, g, t, 1)
    q, k, v, u = qkvu[:, :d], qkvu[:, d:2 * d], qkvu[:, 2 * d:3 * d], qkvu[:, 3 * d:]
    ref = _torch_silu_attention(q, k, v, u, torch.tril(torch.ones(n, n, dtype=torch.float64)).numpy(), n)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_attention_all_candidates_closed_form():
    rng = np.random.default_rng(31)
    K, d, H = 9, 24, 3
    qkvu = _qkvu(rng, K, d)
    g = np.full(K, 3, np.uint8)
    t = rng.uniform(0, 100, K).astype(np.float32)
    y = O.hstu_attention(qkvu, g, t, H)
    dh = d // H
    for i in range(K):
        for h in range(H):
            sl = slice(h * dh, (h + 1) * dh)
            q, k = qkvu[i, :d][sl], qkvu[i, d:2 * d][sl]
            v, u = qkvu[i, 2 * d:3 * d][sl], qkvu[i, 3 * d:][sl]
            s = float(q @ k)
            expect = s / (1.0 + np.exp(-s)) / K * v * u
            np.testing.assert_allclose(y[i, sl], expect, rtol=1e-12, atol=1e-15)


def test_attention_normaliser_is_total_token_count():
    # one static token and extra candidates: the static row's output scales as 1/N (N = all tokens)
    rng = np.random.default_rng(32)
    d = 8
    qkvu1 = _qkvu(rng, 1, d)
    g1 = np.array([0], np.uint8)
    y1 = O.hstu_attention(qkvu1, g1, np.array([-np.inf], np.float32), 1)
    extra = _qkvu(rng, 3, d)
    y4 = O.hstu_attention(np.concatenate([qkvu1, extra]), np.array([0, 3, 3, 3], np.uint8),
                          np.array([-np.inf, 1, 2, 3], np.float32), 1)
    np.testing.assert_allclose(y4[0], y1[0] / 4.0, rtol=1e-13)


# ------------------------------------------------------------------------------------------
# Block and encoder: closed forms and invariants
# ------------------------------------------------------------------------------------------
def _small_model(seed, L=2, d=32, H=2, h=64, scale_bias=0.0):
    rng = np.random.default_rng(seed)
    p = synth.make_params(rng, L, d, H, h, "f32")
    layers = O.params_layers(p)
    if scale_bias:
        for lay in layers:
            for key in ("b_qkvu", "b_mlp1", "b_mlp2"):
                lay[key] = rng.uniform(-scale_bias, scale_bias, lay[key].shape)
    head = O.params_head(p)
    return rng, layers, head


def _small_batch(rng, d, lengths):
    n_u, n_s, n_r, k = zip(*lengths)
    return synth.batch_from_lengths(n_u, n_s, n_r, k, d, rng, "f32")


def test_block_mlp_residual_closed_form():
    rng, layers, _ = _small_model(40, L=1, scale_bias=0.3)
    lay = dict(layers[0])
    lay["w_mlp1"] = np.zeros_like(lay["w_mlp1"])
    lay["b_mlp1"] = np.zeros_like(lay["b_mlp1"])
    b = _small_batch(rng, 32, [(2, 5, 4, 3)])
    out = O.block_forward(b.x, b.group_ids, b.timestamps, lay, 2)
    np.testing.assert_allclose(out, b.x.astype(np.float64) + lay["b_mlp2"], rtol=0, atol=1e-14)


def test_block_gate_closed_form():
    # U projection zero => gated attention is zero => GLN2 returns beta of the token's group
    rng, layers, _ = _small_model(41, L=1, scale_bias=0.3)
    lay = dict(layers[0])
    d = 32
    w = lay["w_qkvu"].copy()
    w[3 * d:] = 0.0
    bq = lay["b_qkvu"].copy()
    bq[3 * d:] = 0.0
    lay["w_qkvu"], lay["b_qkvu"] = w, bq
    b = _small_batch(rng, d, [(2, 5, 4, 3)])
    out = O.block_forward(b.x, b.group_ids, b.timestamps, lay, 2)
    z = lay["gln2_beta"][b.group_ids.astype(np.int64)]
    hid = O.silu(z @ lay["w_mlp1"].T + lay["b_mlp1"])
    np.testing.assert_allclose(out, b.x + hid @ lay["w_mlp2"].T + lay["b_mlp2"], rtol=1e-12, atol=1e-13)


def _encode(b, layers, head, H=2):
    return O.encoder_forward(b.offsets, b.group_ids, b.timestamps, b.x, layers, head, H)


def test_candidate_permutation_equivariance():
    rng, layers, head = _small_model(50)
    b = _small_batch(rng, 32, [(3, 6, 5, 7)])
    hid, logit = _encode(b, layers, head)
    c0 = 3 + 6 + 5
    perm = np.concatenate([np.arange(c0), c0 + rng.permutation(7)])
    b2 = synth.Batch(b.offsets, b.group_ids[perm], b.timestamps[perm], b.x[perm], b.n_u, b.n_s, b.n_r, b.k)
    hid2, logit2 = _encode(b2, layers, head)
    np.testing.assert_allclose(hid2, hid[perm], rtol=0, atol=1e-12)
    np.testing.assert_allclose(logit2, logit[perm[c0:] - c0], rtol=0, atol=1e-12)


def test_candidate_independence_and_duplicates():
    rng, layers, head = _small_model(51)
    b = _small_batch(rng, 32, [(3, 6, 5, 6)])
    c0 = 3 + 6 + 5
    b.x[c0 + 4] = b.x[c0 + 1]                  # candidates 1 and 4 identical (same features, time)
    b.timestamps[c0 + 4] = b.timestamps[c0 + 1]
    hid, logit = _encode(b, layers, head)
    np.testing.assert_allclose(logit[4], logit[1], rtol=0, atol=1e-13)
    x2 = b.x.copy()
    t2 = b.timestamps.copy()
    x2[c0 + 2] = rng.standard_normal(32) * 4
    t2[c0 + 2] = 1e6
    b2 = synth.Batch(b.offsets, b.group_ids, t2, x2, b.n_u, b.n_s, b.n_r, b.k)
    hid2, logit2 = _encode(b2, layers, head)
    others = np.array([i for i in range(b.num_tokens) if i != c0 + 2])
    np.testing.assert_allclose(hid2[others], hid[others], rtol=0, atol=1e-13)
    assert np.abs(hid2[c0 + 2] - hid[c0 + 2]).max() > 1e-3


def test_user_isolation_and_packing():
    rng, layers, head = _small_model(52)
    b = _small_batch(rng, 32, [(2, 4, 3, 2), (1, 9, 0, 5), (4, 0, 6, 0), (2, 3, 3, 3)])
    hid, logit = _encode(b, layers, head)
    for u in range(b.num_users):
        s = synth.subset(b, [u])
        hs, ls = _encode(s, layers, head)
        np.testing.assert_allclose(hs, hid[synth.user_rows(b, [u])], rtol=0, atol=1e-13)
        np.testing.assert_allclose(ls, logit[synth.candidate_rows(b, [u])], rtol=0, atol=1e-13)
    # perturbing user 1 leaves the other users unchanged
    x2 = b.x.copy()
    rows1 = synth.user_rows(b, [1])
    x2[rows1] = rng.standard_normal((rows1.shape[0], 32))
    b2 = synth.Batch(b.offsets, b.group_ids, b.timestamps, x2, b.n_u, b.n_s, b.n_r, b.k)
    hid2, _ = _encode(b2, layers, head)
    keep = synth.user_rows(b, [0, 2, 3])
    np.testing.assert_allclose(hid2[keep], hid[keep], rtol=0, atol=1e-13)


def test_temporal_replay_no_leak():
    # [P1] failure mode 3: an R event at time tau must not influence any token with t <= tau
    # (other than itself) nor any U/S token, through all layers.
    rng, layers, head = _small_model(53, L=3)
    b = _small_batch(rng, 32, [(2, 5, 12, 10)])
    hid, _ = _encode(b, layers, head)
    r0 = 2 + 5
    p = r0 + 6                                   # the 7th real-time event
    tau = b.timestamps[p]
    x2 = b.x.copy()
    x2[p] = rng.standard_normal(32) * 2.0     # (a constant shift would be removed by GroupLN)
    b2 = synth.Batch(b.offsets, b.group_ids, b.timestamps, x2, b.n_u, b.n_s, b.n_r, b.k)
    hid2, _ = _encode(b2, layers, head)
    unaffected = [i for i in range(b.num_tokens) if i != p and b.timestamps[i] <= tau]
    assert len(unaffected) > 7
    np.testing.assert_allclose(hid2[unaffected], hid[unaffected], rtol=0, atol=1e-13)
    later = [i for i in range(b.num_tokens) if b.timestamps[i] > tau]
    assert np.abs(hid2[later] - hid[later]).max() > 1e-6


# ------------------------------------------------------------------------------------------
# Generator
# ------------------------------------------------------------------------------------------
def test_round_to_bf16_is_round_to_nearest_even():
    # bit-level definition: add 0x7FFF plus the lowest kept bit, truncate the low 16 bits
    rng = np.random.default_rng(60)
    a = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    a[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 65504.0]  # exact ties
    u = a.view(np.uint32).astype(np.uint64)
    ref = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(synth.round_to_bf16(a), ref)
    assert synth.round_to_bf16(a[:2]).tolist() == [1.0, 1.0 + 4 * 2.0 ** -8]


def test_generator_deterministic_and_shapes():
    b1, p1 = synth.make_workload("tiny-fp32")
    b2, p2 = synth.make_workload("tiny-fp32")
    np.testing.assert_array_equal(b1.x, b2.x)
    np.testing.assert_array_equal(b1.timestamps, b2.timestamps)
    np.testing.assert_array_equal(p1.layers[0]["w_qkvu"], p2.layers[0]["w_qkvu"])
    assert b1.num_users == 4 and b1.num_tokens == 4 * 56
    assert p1.layers[0]["w_qkvu"].shape == (256, 64)
    # group order U, S, R, C within each user; R sorted; U/S at -inf
    for u in range(4):
        g = b1.group_ids[b1.offsets[u]:b1.offsets[u + 1]]
        assert (np.diff(g.astype(int)) >= 0).all()
        t = b1.timestamps[b1.offsets[u]:b1.offsets[u + 1]]
        assert np.isneginf(t[g < 2]).all()
        assert (np.diff(t[g == 2]) >= 0).all()


def test_silu_matches_torch_and_limits():
    z = np.concatenate([np.linspace(-50, 50, 2001), [-1000.0, 1000.0, 0.0]])
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(O.silu(z), ref, rtol=1e-15, atol=1e-300)
    assert O.silu(np.array([-1000.0]))[0] == 0.0 and O.silu(np.array([1000.0]))[0] == 1000.0


def test_head_special_case():
    # W_h1 picks features 0..3 of x, W_h2 sums the first two / the last two, biases shift:
    # logits = (silu(x0)+silu(x1)+b0, silu(x2)+silu(x3)+b1), computed with torch's silu
    rng = np.random.default_rng(70)
    x = rng.standard_normal((5, 8)) * 3
    w1 = np.zeros((4, 8)); w1[np.arange(4), np.arange(4)] = 1.0
    w2 = np.array([[1.0, 1.0, 0.0, 0.0], [0.0, 0.0, 1.0, 1.0]])
    head = {"w_head1": w1, "b_head1": np.zeros(4), "w_head2": w2, "b_head2": np.array([0.5, -0.25])}
    s = torch.nn.functional.silu(torch.from_numpy(x[:, :4])).numpy()
    expect = np.stack([s[:, 0] + s[:, 1] + 0.5, s[:, 2] + s[:, 3] - 0.25], axis=1)
    np.testing.assert_allclose(O.head_forward(x, head), expect, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------------------------------
# Ablation variants: shared LayerNorm, causal and full masks
# ------------------------------------------------------------------------------------------
def test_ablation_masks_are_library_patterns():
    g = np.array([0, 1, 1, 2, 2, 3, 3], np.uint8)
    t = np.array([-np.inf, -np.inf, -np.inf, 1, 2, 0, 5], np.float32)
    np.testing.assert_array_equal(O.mask(g, t, "causal"), torch.tril(torch.ones(7, 7, dtype=torch.uint8)).numpy())
    np.testing.assert_array_equal(O.mask(g, t, "full"), np.ones((7, 7), np.uint8))
    # the causal ablation is exactly the leak the dynamic rules remove: a later candidate sees an
    # earlier one and an R event that happened after it ([P5] 7.3.4)
    assert O.mask(g, t, "causal")[6, 5] == 1 and O.mask(g, t)[6, 5] == 0
    assert O.mask(g, t, "causal")[5, 3] == 1 and O.mask(g, t)[5, 3] == 0


def test_shared_layer_norm_is_torch_layer_norm():
    rng = np.random.default_rng(80)
    x = rng.standard_normal((30, 16)) * 2 + 0.5
    g = rng.integers(0, 4, 30).astype(np.uint8)
    gamma, beta = rng.uniform(0.5, 1.5, (4, 16)), rng.uniform(-0.1, 0.1, (4, 16))
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (16,), torch.from_numpy(gamma[0]),
                                         torch.from_numpy(beta[0]), 1e-5).numpy()
    np.testing.assert_allclose(O.group_layer_norm(x, g, gamma, beta, 1e-5, shared=True), ref, atol=1e-12)


def test_full_mask_attention_is_dense_and_causal_is_tril():
    rng = np.random.default_rng(81)
    n, d = 23, 16
    qkvu = rng.standard_normal((n, 4 * d)) * 0.7
    g = np.array([0] * 3 + [1] * 8 + [2] * 6 + [3] * 6, np.uint8)
    t = np.concatenate([np.full(11, -np.inf), rng.uniform(0, 9, 12)]).astype(np.float32)
    q, k, v, u = qkvu[:, :d], qkvu[:, d:2 * d], qkvu[:, 2 * d:3 * d], qkvu[:, 3 * d:]
    full = _torch_silu_attention(q, k, v, u, np.ones((n, n)), n)
    causal = _torch_silu_attention(q, k, v, u, np.tril(np.ones((n, n))), n)
    np.testing.assert_allclose(O.hstu_attention(qkvu, g, t, 1, "full"), full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(O.hstu_attention(qkvu, g, t, 1, "causal"), causal, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------------------
# Block backward: finite differences and autograd of an independent torch formulation
# ------------------------------------------------------------------------------------------
def _tiny_block(seed=90, d=16, H=2, h=24, with_bias=True):
    rng = np.random.default_rng(seed)
    g = np.array([0, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3], np.uint8)
    n = g.shape[0]
    t = np.concatenate([np.full(4, -np.inf), rng.uniform(0, 10, 4), rng.uniform(0, 10, 3)]).astype(np.float32)
    x = rng.standard_normal((n, d)) * np.array([1, .5, .5, .5, 2, 2, 2, 2, 4, 4, 4])[:, None]
    lay = {
        "gln1_gamma": rng.uniform(0.5, 1.5, (4, d)), "gln1_beta": rng.uniform(-0.1, 0.1, (4, d)),
        "w_qkvu": rng.standard_normal((4 * d, d)) / np.sqrt(d),
        "b_qkvu": rng.uniform(-0.2, 0.2, 4 * d) if with_bias else None,
        "gln2_gamma": rng.uniform(0.5, 1.5, (4, d)), "gln2_beta": rng.uniform(-0.1, 0.1, (4, d)),
        "w_mlp1": rng.standard_normal((h, d)) / np.sqrt(d),
        "b_mlp1": rng.uniform(-0.2, 0.2, h) if with_bias else None,
        "w_mlp2": rng.standard_normal((d, h)) / np.sqrt(h),
        "b_mlp2": rng.uniform(-0.2, 0.2, d) if with_bias else None,
    }
    lay["w_qkvu"][:2 * d] *= 2.0          # scores of order a few: the curved part of silu
    dout = rng.standard_normal((n, d))
    return g, t, x, lay, dout, H


@pytest.mark.parametrize("mask_mode,shared", [("dynamic", False), ("causal", True), ("full", False)])
def test_block_backward_matches_finite_differences(mask_mode, shared):
    g, t, x, lay, dout, H = _tiny_block()
    dx, grads = O.block_backward(x, g, t, lay, H, dout, mask_mode=mask_mode, shared_norm=shared)
    rng = np.random.default_rng(91)

    def loss(xx, ll):
        return float((O.block_forward(xx, g, t, ll, H, mask_mode=mask_mode, shared_norm=shared) * dout).sum())

    eps = 1e-6
    # directional derivative along a random direction, for the input and every parameter tensor
    for name in ("x",) + O.BLOCK_PARAM_NAMES:
        base = x if name == "x" else lay[name]
        v = rng.standard_normal(base.shape)
        if name == "x":
            fd = (loss(x + eps * v, lay) - loss(x - eps * v, lay)) / (2 * eps)
            an = float((dx * v).sum())
        else:
            lp, lm = dict(lay), dict(lay)
            lp[name], lm[name] = base + eps * v, base - eps * v
            fd = (loss(x, lp) - loss(x, lm)) / (2 * eps)
            an = float((grads[name] * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_block_backward_matches_torch_autograd():
    g, t, x, lay, dout, H = _tiny_block(seed=92)
    dx, grads = O.block_backward(x, g, t, lay, H, dout)
    # independent formulation: torch ops on the whole user, dense mask tensor built here from the
    # three rules, per-group affine by gather, autograd for every gradient
    T = torch.float64
    gt = torch.from_numpy(g.astype(np.int64))
    tt = torch.from_numpy(t.astype(np.float64))
    n, d = x.shape
    static_key = (gt == 0) | (gt == 1)
    rc_query = (gt == 2) | (gt == 3)
    r_key = gt == 2
    vis = static_key[None, :] | torch.eye(n, dtype=torch.bool) | (
        rc_query[:, None] & r_key[None, :] & (tt[None, :] < tt[:, None]))
    P = {k: torch.tensor(v, dtype=T, requires_grad=True) for k, v in lay.items() if v is not None}
    xt_ = torch.tensor(x, dtype=T, requires_grad=True)

    def gln(v, gamma, beta):
        return torch.nn.functional.layer_norm(v, (d,), eps=1e-5) * gamma[gt] + beta[gt]

    a1 = gln(xt_, P["gln1_gamma"], P["gln1_beta"])
    qkvu = a1 @ P["w_qkvu"].T + P["b_qkvu"]
    q, k, v, u = qkvu.split(d, dim=1)
    dh = d // H
    heads = []
    for hh in range(H):
        sl = slice(hh * dh, (hh + 1) * dh)
        s = q[:, sl] @ k[:, sl].T
        heads.append((torch.nn.functional.silu(s) * vis / n) @ v[:, sl])
    y = torch.cat(heads, dim=1) * u
    z = gln(y, P["gln2_gamma"], P["gln2_beta"])
    out = torch.nn.functional.silu(z @ P["w_mlp1"].T + P["b_mlp1"]) @ P["w_mlp2"].T + P["b_mlp2"] + xt_
    # P7(e): the block's forward itself, from this torch formulation with the dense mask
    np.testing.assert_allclose(O.block_forward(x, g, t, lay, H), out.detach().numpy(), rtol=1e-10, atol=1e-12)
    (out * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(dx, xt_.grad.numpy(), rtol=1e-10, atol=1e-12)
    for name, p in P.items():
        np.testing.assert_allclose(grads[name], p.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def _torch_block_forward(x, g, t, lay, H, eps=1e-5):
    """One HSTU block written independently with torch ops (marovi.ai MTGR page, 方法, the two
    update equations): a dense [n, n] mask tensor from the three rules (fun-rec 7.3.4), GroupLN as
    torch layer_norm plus a per-group gather of gamma/beta, F.silu, and matrix products."""
    T = torch.float64
    gt = torch.from_numpy(g.astype(np.int64))
    tt = torch.from_numpy(t.astype(np.float64))
    n, d = x.shape
    vis = ((gt == 0) | (gt == 1))[None, :] | torch.eye(n, dtype=torch.bool) | (
        ((gt == 2) | (gt == 3))[:, None] & (gt == 2)[None, :] & (tt[None, :] < tt[:, None]))
    P = {k: torch.tensor(v, dtype=T) for k, v in lay.items() if v is not None}
    zero = lambda m: torch.zeros(m, dtype=T)
    xt_ = torch.tensor(x, dtype=T)

    def gln(v, gamma, beta):
        return torch.nn.functional.layer_norm(v, (d,), eps=eps) * gamma[gt] + beta[gt]

    qkvu = gln(xt_, P["gln1_gamma"], P["gln1_beta"]) @ P["w_qkvu"].T + P.get("b_qkvu", zero(4 * d))
    q, k, v, u = qkvu.split(d, dim=1)
    dh = d // H
    heads = [(torch.nn.functional.silu(q[:, sl] @ k[:, sl].T) * vis / n) @ v[:, sl]
             for sl in (slice(i * dh, (i + 1) * dh) for i in range(H))]
    z = gln(torch.cat(heads, dim=1) * u, P["gln2_gamma"], P["gln2_beta"])
    hid = torch.nn.functional.silu(z @ P["w_mlp1"].T + P.get("b_mlp1", zero(P["w_mlp1"].shape[0])))
    return (hid @ P["w_mlp2"].T + P.get("b_mlp2", zero(d)) + xt_).numpy()


@pytest.mark.parametrize("seed,with_bias,shuffle_r", [(95, True, False), (96, False, True), (97, True, True)])
def test_block_forward_matches_torch_formulation(seed, with_bias, shuffle_r):
    """P7(e): the oracle's whole block equals an independent torch formulation with a dense mask,
    on users holding every group, unsorted R events, an R/C timestamp tie and zero or nonzero biases."""
    g, t, x, lay, _, H = _tiny_block(seed=seed, with_bias=with_bias)
    rng = np.random.default_rng(seed)
    if shuffle_r:
        t[4:8] = rng.permutation(t[4:8])
    t[9] = t[5]                                     # a candidate tied with an R event: not visible
    np.testing.assert_allclose(O.block_forward(x, g, t, lay, H), _torch_block_forward(x, g, t, lay, H),
                               rtol=1e-10, atol=1e-12)


def test_round_bf16_matches_torch_conversion():
    """R19's rounding is the nearest bfloat16, ties to even: torch's float32 -> bfloat16."""
    rng = np.random.default_rng(98)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.uniform(-30, 30, 4000),
                        [0.0, -0.0, 1.0, -1.5, 3.4e38, 1e-40, np.inf, -np.inf]]).astype(np.float32)
    # exact halfway cases: the 16 dropped bits are 0x8000, with an even and an odd kept bit
    ties = (rng.integers(0x3F000000, 0x47000000, 2000).astype(np.uint32) & 0xFFFF0000) | 0x8000
    v = np.concatenate([v, ties.view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(v), ref)


@pytest.mark.parametrize("mask_mode,shared", [("dynamic", False), ("causal", True), ("full", False)])
def test_bf16_storage_backward_reduces_to_exact(mask_mode, shared):
    """With the identity as the storage rounding, the R19 evaluation is the exact chain rule."""
    g, t, x, lay, dout, H = _tiny_block(seed=99)
    dx, grads = O.block_backward(x, g, t, lay, H, dout, mask_mode=mask_mode, shared_norm=shared)
    dx2, grads2 = O.block_backward_bf16_storage(x, g, t, lay, H, dout, mask_mode=mask_mode,
                                                shared_norm=shared, store=lambda a: a)
    np.testing.assert_allclose(dx2, dx, rtol=1e-12, atol=1e-13)
    for name in grads:
        np.testing.assert_allclose(grads2[name], grads[name], rtol=1e-12, atol=1e-13, err_msg=name)


def test_bf16_storage_backward_stays_near_exact():
    """With bf16 rounding (2^-9 relative per stored value) the result moves, but by a few percent
    at most of each tensor's largest magnitude."""
    g, t, x, lay, dout, H = _tiny_block(seed=100)
    lay = {k: (O.round_bf16(v) if v is not None else None) for k, v in lay.items()}
    x = O.round_bf16(x)
    dx, grads = O.block_backward(x, g, t, lay, H, dout)
    dx2, grads2 = O.block_backward_bf16_storage(x, g, t, lay, H, dout)
    rel = lambda a, b: float(np.abs(a - b).max() / np.abs(b).max())
    np.testing.assert_array_equal(grads2["b_mlp2"], grads["b_mlp2"])   # sums of the unrounded dout
    errs = [rel(dx2, dx)] + [rel(grads2[k], grads[k]) for k in grads if k != "b_mlp2"]
    assert 0.0 < min(errs) and max(errs) < 5e-2, errs


def test_block_backward_batch_sums_users_and_isolates_them():
    g, t, x, lay, dout, H = _tiny_block(seed=93)
    n = g.shape[0]
    offsets = np.array([0, n, 2 * n])
    x2 = np.concatenate([x, x[::-1].copy()])
    g2 = np.concatenate([g, g])
    t2 = np.concatenate([t, t])
    rng = np.random.default_rng(94)
    x2[n:] = rng.standard_normal((n, x.shape[1]))
    d2 = np.concatenate([dout, rng.standard_normal(dout.shape)])
    dx, grads = O.block_backward_batch(offsets, g2, t2, x2, lay, H, d2)
    dxa, ga = O.block_backward(x2[:n], g, t, lay, H, d2[:n])
    dxb, gb = O.block_backward(x2[n:], g, t, lay, H, d2[n:])
    np.testing.assert_array_equal(dx[:n], dxa)
    np.testing.assert_array_equal(dx[n:], dxb)
    for k in grads:
        np.testing.assert_allclose(grads[k], ga[k] + gb[k], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# embedding front end oracle (oracle/embedding_oracle.py)
# ---------------------------------------------------------------------------------------------
from oracle import embedding_oracle as EO


class _PairListStore:
    """Brute force: a plain list of [key, value, last_seen] entries and a count of free rows."""

    def __init__(self, rows, dim):
        self.entries, self.rows, self.dim, self.failed = [], rows, dim, 0

    def _find(self, k):
        for e in self.entries:
            if e[0] == k:
                return e
        return None

    def insert(self, keys, init, step):
        for i, k in enumerate(keys):
            e = self._find(int(k))
            if e is None:
                if int(k) < 0 or len(self.entries) >= self.rows:
                    self.failed += 1
                    continue
                e = [int(k), np.zeros(self.dim) if init is None else np.asarray(init[i], float), step]
                self.entries.append(e)
            e[2] = step

    def lookup(self, keys, step=-1):
        out, found = np.zeros((len(keys), self.dim)), np.zeros(len(keys), bool)
        for i, k in enumerate(keys):
            e = self._find(int(k))
            if e is not None:
                out[i], found[i] = e[1], True
                if step >= 0:
                    e[2] = step
        return out, found

    def evict(self, keys):
        ks = {int(k) for k in keys}
        self.entries = [e for e in self.entries if e[0] not in ks]

    def evict_older(self, threshold):
        self.entries = [e for e in self.entries if e[2] >= threshold]


def test_store_model_matches_brute_force_on_random_operations():
    rng = np.random.default_rng(5)
    rows, dim = 40, 3
    a, b = EO.EmbeddingStore(rows, dim), _PairListStore(rows, dim)
    for step in range(300):
        op = rng.integers(0, 4)
        keys = rng.integers(-1, 70, rng.integers(1, 9))
        if op == 0:
            init = rng.standard_normal((len(keys), dim))
            a.insert(keys, init, step)
            b.insert(keys, init, step)
        elif op == 1:
            st = step if rng.random() < 0.5 else -1
            va, fa = a.lookup(keys, st)
            vb, fb = b.lookup(keys, st)
            np.testing.assert_array_equal(fa, fb)
            np.testing.assert_array_equal(va, vb)
        elif op == 2:
            a.evict(keys)
            b.evict(keys)
        else:
            th = step - int(rng.integers(0, 40))
            a.evict_older(th)
            b.evict_older(th)
        assert sorted(a.index) == sorted(e[0] for e in b.entries)
        assert a.failed == b.failed
        # invariants: live + free = rows, live rows distinct
        assert len(a.index) + len(a.free) == rows
        assert len(set(a.index.values())) == len(a.index)


def test_store_model_insert_keeps_existing_value_and_fails_when_full():
    s = EO.EmbeddingStore(2, 2)
    r = s.insert([7, 7, 9], np.array([[1., 1.], [2., 2.], [3., 3.]]), step=0)
    assert r[0] == r[1] != r[2]
    v, f = s.lookup([7, 9, 11])
    np.testing.assert_array_equal(v, [[1, 1], [3, 3], [0, 0]])
    np.testing.assert_array_equal(f, [True, True, False])
    assert s.insert([12], None, step=1) == [-1] and s.stats()["failed_inserts"] == 1
    s.evict([7])
    assert s.insert([12], None, step=2)[0] >= 0              # the freed row is reused
    v, f = s.lookup([7, 12])
    np.testing.assert_array_equal(f, [False, True])
    np.testing.assert_array_equal(v[1], [0, 0])               # no init -> zeros


def test_store_model_evict_older_uses_last_use():
    s = EO.EmbeddingStore(8, 1)
    s.insert([1, 2, 3], None, step=0)
    s.lookup([2], step=5)
    s.insert([3], None, step=7)
    s.evict_older(5)
    assert sorted(s.index) == [2, 3]


def test_unique_with_inverse_against_sets():
    rng = np.random.default_rng(6)
    keys = rng.integers(0, 1 << 45, 500) // 1000 * 1000 + rng.integers(0, 3, 500)
    uniq, inv = EO.unique_with_inverse(keys)
    assert set(uniq.tolist()) == set(keys.tolist()) and len(uniq) == len(set(keys.tolist()))
    np.testing.assert_array_equal(uniq[inv], keys)
    assert np.all(np.diff(uniq) > 0)


def test_merged_key_separates_tables():
    assert EO.merged_key(0, 5) != EO.merged_key(1, 5)
    assert EO.merged_key(3, 0) == 3 << 40
    with pytest.raises(ValueError):
        EO.merged_key(1, 1 << 40)


def _tok_case(seed, e=4, d=6):
    rng = np.random.default_rng(seed)
    field_tables = [[0, 1], [2, 3, 4], [2, 3, 5], [2, 3, 6, 7]]      # item tables 2, 3 shared
    T = 40
    groups = np.sort(rng.integers(0, 4, T)).astype(np.int64)
    fmax = max(len(f) for f in field_tables)
    ids = rng.integers(0, 12, (T, fmax)).astype(np.int64)
    store = EO.EmbeddingStore(200, e)
    keys, vals = [], []
    for tab in range(8):
        for i in range(12):
            if (tab + i) % 5 != 0:                                   # some keys absent: zeros
                keys.append(EO.merged_key(tab, i))
                vals.append(rng.standard_normal(e))
    store.insert(keys, np.array(vals), step=0)
    mlps = [{"w1": rng.standard_normal((d, len(f) * e)), "b1": rng.standard_normal(d),
             "w2": rng.standard_normal((d, d)), "b2": rng.standard_normal(d)} for f in field_tables]
    return ids, groups, field_tables, store, mlps


def test_tokenizer_matches_torch_modules():
    ids, groups, field_tables, store, mlps = _tok_case(7)
    x = EO.tokenize(ids, groups, field_tables, store, mlps)
    # independent formulation: one nn.Embedding per table (absent keys -> zero rows), cat, two
    # nn.Linear layers with SiLU, per group
    e = store.dim
    embs = []
    for tab in range(8):
        w = torch.zeros(12, e, dtype=torch.float64)
        for i in range(12):
            k = EO.merged_key(tab, i)
            if k in store.index:
                w[i] = torch.from_numpy(store.values[store.index[k]])
        embs.append(torch.nn.Embedding.from_pretrained(w))
    for t in range(ids.shape[0]):
        g = int(groups[t])
        feat = torch.cat([embs[tab](torch.tensor(int(ids[t, f]))) for f, tab in enumerate(field_tables[g])])
        l1 = torch.nn.Linear(feat.numel(), mlps[g]["w1"].shape[0], dtype=torch.float64)
        l2 = torch.nn.Linear(mlps[g]["w2"].shape[1], mlps[g]["w2"].shape[0], dtype=torch.float64)
        with torch.no_grad():
            l1.weight.copy_(torch.from_numpy(mlps[g]["w1"])); l1.bias.copy_(torch.from_numpy(mlps[g]["b1"]))
            l2.weight.copy_(torch.from_numpy(mlps[g]["w2"])); l2.bias.copy_(torch.from_numpy(mlps[g]["b2"]))
            ref = l2(torch.nn.functional.silu(l1(feat)))
        np.testing.assert_allclose(x[t], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_tokenizer_is_per_token_and_ignores_unused_columns():
    ids, groups, field_tables, store, mlps = _tok_case(8)
    x = EO.tokenize(ids, groups, field_tables, store, mlps)
    perm = np.random.default_rng(9).permutation(len(groups))
    xp = EO.tokenize(ids[perm], groups[perm], field_tables, store, mlps)
    np.testing.assert_allclose(xp, x[perm], rtol=0, atol=0)
    ids2 = ids.copy()
    for t in range(len(groups)):
        ids2[t, len(field_tables[int(groups[t])]):] = 999999   # columns past the group's fields
    np.testing.assert_array_equal(EO.tokenize(ids2, groups, field_tables, store, mlps), x)
    for m in mlps:
        m["w2"] = np.zeros_like(m["w2"])
    x0 = EO.tokenize(ids, groups, field_tables, store, mlps)   # W2 = 0 -> x = b2 of the group
    np.testing.assert_array_equal(x0, np.stack([mlps[int(g)]["b2"] for g in groups]))
