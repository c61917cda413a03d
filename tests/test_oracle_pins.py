"""Pins of the fp64 oracle against facts that do not come from the oracle.

The oracle reconstructs K = U W, V = U' W' and runs two-pass softmax
attention (MILO summary, "4.4 MILO Workflow").  Each test below checks it
against something independent of that code: a library attention routine, an
evaluation in the absorbed order written as plain loops, closed forms and
invariants of softmax attention.
"""
import math

import numpy as np
import pytest
import torch

import oracle

rng = np.random.default_rng(1234)


def rand_blocks(rng, B, Hkv, d, toks, rks, rvs):
    """toks/rks/rvs: per sequence lists."""
    out = []
    for i in range(B):
        bl = []
        for T, r, rv in zip(toks[i], rks[i], rvs[i]):
            bl.append((rng.standard_normal((Hkv, T, r)), rng.standard_normal((Hkv, r, d)),
                       rng.standard_normal((Hkv, T, rv)), rng.standard_normal((Hkv, rv, d))))
        out.append(bl)
    return out


def run(q, blocks, kt, vt, tl, scale):
    return oracle.attend_logical(q, blocks, kt, vt, np.asarray(tl, np.int32), scale)


# --------------------------------------------------------------------------
# 1. full-rank identity reduces to a library attention routine
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Q,L_list", [(1, [4, 0, 7]), (3, [3, 5, 6]), (5, [5, 9, 5])])
def test_full_rank_identity_matches_sdpa(Q, L_list):
    B, Hq, Hkv, d = 3, 6, 2, 16
    G = Hq // Hkv
    scale = 0.37
    toks = [[5, 7, 3], [9], [4, 4]]
    eye = np.broadcast_to(np.eye(d), (Hkv, d, d))
    blocks = []
    for i in range(B):
        blocks.append([(rng.standard_normal((Hkv, T, d)), eye.copy(),
                        rng.standard_normal((Hkv, T, d)), eye.copy()) for T in toks[i]])
    cap = max(L_list)
    kt = rng.standard_normal((B, Hkv, cap, d))
    vt = rng.standard_normal((B, Hkv, cap, d))
    q = rng.standard_normal((B, Q, Hq, d))
    out, lse = run(q, blocks, kt, vt, L_list, scale)
    for i in range(B):
        L = L_list[i]
        Kb = np.concatenate([U for (U, _, _, _) in blocks[i]], 1)   # [Hkv][Nb][d]
        Vb = np.concatenate([Up for (_, _, Up, _) in blocks[i]], 1)
        K = np.concatenate([Kb, kt[i, :, :L]], 1)
        V = np.concatenate([Vb, vt[i, :, :L]], 1)
        Nb = Kb.shape[1]
        # blocks fully visible; tail bottom-right causal via torch.tril
        tail_mask = torch.ones(Q, L, dtype=torch.bool).tril(diagonal=L - Q)
        mask = torch.cat([torch.ones(Q, Nb, dtype=torch.bool), tail_mask], 1)
        qt = torch.from_numpy(q[i]).permute(1, 0, 2)[None]           # [1][Hq][Q][d]
        Kt = torch.from_numpy(K)[None]
        Vt = torch.from_numpy(V)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, Kt, Vt, attn_mask=mask, scale=scale, enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)
        # lse against torch.logsumexp of the same masked scores
        Kx = torch.from_numpy(K).repeat_interleave(G, 0)               # [Hq][N][d]
        sc = torch.einsum("hqd,hnd->hqn", qt[0], Kx) * scale
        sc = sc.masked_fill(~mask[None], float("-inf"))
        np.testing.assert_allclose(lse[i], torch.logsumexp(sc, -1).T.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# 2. absorbed evaluation order, written as plain loops on tiny inputs
# --------------------------------------------------------------------------
def absorbed_loops(qv, blocks_g, K_t, V_t, scale):
    """p = W q, s = scale * U p, softmax, z = a U', o = sum_b z_b W'_b."""
    d = len(qv)
    scores = []
    for (U, W, Up, Wp) in blocks_g:
        T, r = len(U), len(W)
        p = [sum(W[k][c] * qv[c] for c in range(d)) for k in range(r)]
        scores.append([scale * sum(U[t][k] * p[k] for k in range(r)) for t in range(T)])
    ts = [scale * sum(K_t[t][c] * qv[c] for c in range(d)) for t in range(len(K_t))]
    allv = [x for s in scores for x in s] + ts
    m = max(allv)
    Z = sum(math.exp(x - m) for x in allv)
    o = [0.0] * d
    for (U, W, Up, Wp), s in zip(blocks_g, scores):
        T, rv = len(Up), len(Wp)
        z = [sum(math.exp(s[t] - m) / Z * Up[t][k] for t in range(T)) for k in range(rv)]
        for c in range(d):
            o[c] += sum(z[k] * Wp[k][c] for k in range(rv))
    for t in range(len(K_t)):
        a = math.exp(ts[t] - m) / Z
        for c in range(d):
            o[c] += a * V_t[t][c]
    return o, m + math.log(Z)


def test_absorbed_order_plain_loops():
    B, Hq, Hkv, d = 2, 4, 2, 6
    toks = [[5, 3], [4]]
    rks = [[3, 1], [5]]
    rvs = [[2, 4], [0]]
    blocks = rand_blocks(rng, B, Hkv, d, toks, rks, rvs)
    L = [3, 2]
    kt = rng.standard_normal((B, Hkv, 3, d))
    vt = rng.standard_normal((B, Hkv, 3, d))
    q = rng.standard_normal((B, 1, Hq, d))
    out, lse = run(q, blocks, kt, vt, L, 0.45)
    for i in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            bg = [(U[g].tolist(), W[g].tolist(), Up[g].tolist(), Wp[g].tolist())
                  for (U, W, Up, Wp) in blocks[i]]
            o, l = absorbed_loops(q[i, 0, h].tolist(), bg, kt[i, g, :L[i]].tolist(),
                                  vt[i, g, :L[i]].tolist(), 0.45)
            np.testing.assert_allclose(out[i, 0, h], o, rtol=1e-12, atol=1e-13)
            assert abs(lse[i, 0, h] - l) < 1e-12


# --------------------------------------------------------------------------
# 3. normalisation and closed forms
# --------------------------------------------------------------------------
def test_weights_sum_to_one():
    """V rows all ones (U' = 1 column, W' = 1 row) => o == 1 for any scores."""
    B, Hq, Hkv, d = 2, 3, 1, 8
    blocks = []
    for i in range(B):
        bl = []
        for T in (6, 2, 5):
            r = 3
            bl.append((rng.standard_normal((Hkv, T, r)) * 3, rng.standard_normal((Hkv, r, d)),
                       np.ones((Hkv, T, 1)), np.ones((Hkv, 1, d))))
        blocks.append(bl)
    kt = rng.standard_normal((B, Hkv, 4, d)) * 2
    vt = np.ones((B, Hkv, 4, d))
    q = rng.standard_normal((B, 2, Hq, d))
    out, lse = run(q, blocks, kt, vt, [4, 3], 0.9)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_visible_rows():
    B, Hq, Hkv, d = 1, 2, 1, 5
    blocks = rand_blocks(rng, B, Hkv, d, [[4, 3]], [[2, 3]], [[3, 1]])
    kt = rng.standard_normal((B, Hkv, 5, d))
    vt = rng.standard_normal((B, Hkv, 5, d))
    q = np.zeros((B, 2, Hq, d))
    out, lse = run(q, blocks, kt, vt, [5], 1.0)
    (U1, W1, Up1, Wp1), (U2, W2, Up2, Wp2) = blocks[0]
    # mean of rows computed in factor space: (column sums of U') W'
    tot1 = Up1[0].sum(0) @ Wp1[0]
    tot2 = Up2[0].sum(0) @ Wp2[0]
    for j in range(2):
        vis = 5 - 2 + j + 1
        n = 4 + 3 + vis
        ref = (tot1 + tot2 + vt[0, 0, :vis].sum(0)) / n
        np.testing.assert_allclose(out[0, j, 0], ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[0, j, :], math.log(n), rtol=1e-13)


def test_single_visible_token():
    d = 7
    U = rng.standard_normal((1, 1, 3))
    W = rng.standard_normal((1, 3, d))
    Up = rng.standard_normal((1, 1, 2))
    Wp = rng.standard_normal((1, 2, d))
    q = rng.standard_normal((1, 1, 1, d))
    out, lse = run(q, [[(U, W, Up, Wp)]], np.zeros((1, 1, 0, d)), np.zeros((1, 1, 0, d)), [0], 0.3)
    v = sum(Up[0, 0, k] * Wp[0, k] for k in range(2))
    s = 0.3 * sum(sum(U[0, 0, k] * W[0, k, c] for k in range(3)) * q[0, 0, 0, c] for c in range(d))
    np.testing.assert_allclose(out[0, 0, 0], v, rtol=1e-13, atol=1e-14)
    assert abs(lse[0, 0, 0] - s) < 1e-13


def test_linear_in_value_projection():
    B, Hq, Hkv, d = 1, 2, 2, 8
    blocks = rand_blocks(rng, B, Hkv, d, [[6, 5]], [[2, 4]], [[3, 3]])
    kt = rng.standard_normal((B, Hkv, 2, d))
    vt = rng.standard_normal((B, Hkv, 2, d))
    q = rng.standard_normal((B, 1, Hq, d))
    o1, l1 = run(q, blocks, kt, vt, [2], 0.5)
    c = -2.5
    b2 = [[(U, W, Up, Wp * c) for (U, W, Up, Wp) in blocks[0]]]
    o2, l2 = run(q, b2, kt, vt * c, [2], 0.5)
    np.testing.assert_allclose(o2, c * o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-14)


def test_empty_context():
    d = 4
    out, lse = run(np.ones((2, 1, 1, d)), [[], []], np.zeros((2, 1, 3, d)),
                   np.zeros((2, 1, 3, d)), [0, 0], 1.0)
    assert np.all(out == 0.0)
    assert np.all(np.isneginf(lse))


def test_rank_zero_block_counts_in_normaliser():
    """A block with r = r' = 0 has T zero scores and zero values."""
    B, Hq, Hkv, d = 1, 1, 1, 6
    other = rand_blocks(rng, B, Hkv, d, [[5]], [[3]], [[2]])[0][0]
    T0 = 7
    zero = (np.zeros((1, T0, 0)), np.zeros((1, 0, d)), np.zeros((1, T0, 0)), np.zeros((1, 0, d)))
    q = rng.standard_normal((1, 1, 1, d))
    e = np.zeros((1, 1, 0, d))
    o_z, l_z = run(q, [[zero]], e, e, [0], 0.7)
    assert np.all(o_z == 0.0)
    assert abs(l_z[0, 0, 0] - math.log(T0)) < 1e-14
    o1, l1 = run(q, [[other]], e, e, [0], 0.7)
    o2, l2 = run(q, [[other, zero]], e, e, [0], 0.7)
    # softmax over a union: lse adds in log space, outputs reweight
    lt = np.logaddexp(l1, math.log(T0))
    np.testing.assert_allclose(l2, lt, rtol=1e-13)
    np.testing.assert_allclose(o2, o1 * np.exp(l1 - lt)[..., None], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# 4. block bookkeeping invariances
# --------------------------------------------------------------------------
def test_split_merge_permute_invariance():
    B, Hq, Hkv, d = 2, 4, 2, 8
    blocks = rand_blocks(rng, B, Hkv, d, [[9, 6, 4], [7, 5]], [[3, 5, 2], [4, 1]],
                         [[2, 6, 3], [5, 2]])
    kt = rng.standard_normal((B, Hkv, 3, d))
    vt = rng.standard_normal((B, Hkv, 3, d))
    q = rng.standard_normal((B, 1, Hq, d))
    base_o, base_l = run(q, blocks, kt, vt, [3, 2], 0.6)

    # split the first block of each sequence at token 3
    split = []
    for bl in blocks:
        U, W, Up, Wp = bl[0]
        split.append([(U[:, :3], W, Up[:, :3], Wp), (U[:, 3:], W, Up[:, 3:], Wp)] + bl[1:])
    o, l = run(q, split, kt, vt, [3, 2], 0.6)
    np.testing.assert_allclose(o, base_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, base_l, rtol=1e-13)

    # merge the first two blocks into one block-diagonal factorisation
    merged = []
    for bl in blocks:
        (U1, W1, Up1, Wp1), (U2, W2, Up2, Wp2) = bl[0], bl[1]
        H, T1, r1 = U1.shape
        T2, r2 = U2.shape[1], U2.shape[2]
        U = np.zeros((H, T1 + T2, r1 + r2)); U[:, :T1, :r1] = U1; U[:, T1:, r1:] = U2
        rv1, rv2 = Up1.shape[2], Up2.shape[2]
        Up = np.zeros((H, T1 + T2, rv1 + rv2)); Up[:, :T1, :rv1] = Up1; Up[:, T1:, rv1:] = Up2
        merged.append([(U, np.concatenate([W1, W2], 1), Up, np.concatenate([Wp1, Wp2], 1))] + bl[2:])
    o, l = run(q, merged, kt, vt, [3, 2], 0.6)
    np.testing.assert_allclose(o, base_o, rtol=1e-12, atol=1e-14)

    # permute block order
    perm = [list(reversed(bl)) for bl in blocks]
    o, l = run(q, perm, kt, vt, [3, 2], 0.6)
    np.testing.assert_allclose(o, base_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, base_l, rtol=1e-13)


# --------------------------------------------------------------------------
# 5. causal tail and GQA mapping probes
# --------------------------------------------------------------------------
def test_planted_future_token_is_masked():
    """Query j of a Q-row chunk sees tail tokens l <= L - Q + j only."""
    d, Q, L = 8, 4, 7
    q = np.zeros((1, Q, 1, d)); q[..., 0] = 1.0
    kt = np.zeros((1, 1, L, d)); vt = np.zeros((1, 1, L, d))
    lstar = 5
    kt[0, 0, lstar, 0] = 400.0         # huge score for the planted token
    vt[0, 0, lstar, :] = 1.0
    out, lse = run(q, [[]], kt, vt, [L], 1.0)
    for j in range(Q):
        sees = lstar <= L - Q + j
        if sees:
            np.testing.assert_allclose(out[0, j, 0], 1.0, atol=1e-12)
        else:
            np.testing.assert_allclose(out[0, j, 0], 0.0, atol=0)


def test_gqa_head_reads_group_h_over_G():
    Hq, Hkv, d = 6, 3, 4
    G = Hq // Hkv
    T = 5
    blocks = [[(rng.standard_normal((Hkv, T, 2)), rng.standard_normal((Hkv, 2, d)),
                np.ones((Hkv, T, 1)), np.array([[[10.0 * (g + 1)] * d] for g in range(Hkv)]))]]
    e = np.zeros((1, Hkv, 0, d))
    q = rng.standard_normal((1, 1, Hq, d))
    out, _ = run(q, blocks, e, e, [0], 1.0)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, 0, h], 10.0 * (h // G + 1), rtol=1e-14)


def test_selected_rows_match_full_run():
    B, Hq, Hkv, d, Q = 2, 4, 2, 8, 3
    blocks = rand_blocks(rng, B, Hkv, d, [[5, 4], [6]], [[2, 3], [4]], [[3, 2], [1]])
    kt = rng.standard_normal((B, Hkv, 4, d))
    vt = rng.standard_normal((B, Hkv, 4, d))
    q = rng.standard_normal((B, Q, Hq, d))
    full_o, full_l = run(q, blocks, kt, vt, [4, 3], 0.5)
    sel = [(1, 2, 3), (0, 0, 1)]
    o, l = oracle.attend_logical(q, blocks, kt, vt, np.array([4, 3], np.int32), 0.5, sel=sel)
    for (i, j, h) in sel:
        np.testing.assert_array_equal(o[i, j, h], full_o[i, j, h])
        assert l[i, j, h] == full_l[i, j, h]
    assert np.isnan(o[0, 1, 0]).all()


# --------------------------------------------------------------------------
# 6. stored output of the tiny workload (regression guard for the oracle)
# --------------------------------------------------------------------------
def test_oracle_matches_stored_tiny_output():
    import json
    import os
    import synth
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    ref = json.load(open(path))
    cfg = synth.get_config("tiny")
    for variant in ("base", "sharp"):
        out, lse = oracle.attend(synth.make_workload(cfg, variant=variant))
        np.testing.assert_allclose(out.ravel(), ref[variant]["out"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse.ravel(), ref[variant]["lse"], rtol=1e-12)
