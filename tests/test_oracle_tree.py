"""Oracle pins: tree build (AdaSpark Section 3.1 Proposition 1, Section 3.3 n-gram
fill) and greedy tree verification (Section 2.2)."""
import itertools

import numpy as np
import pytest

from oracle import oracle as O


def random_forest_inputs(rng, P, Kc, L, V=6):
    block = np.zeros((P, Kc), np.int32)
    for p in range(P):
        block[p] = rng.choice(V, Kc, replace=False)
    ng = np.full((P + 1, L), -1, np.int32)
    ngl = rng.integers(0, L + 1, P + 1).astype(np.int32)
    for s in range(P + 1):
        ng[s, :ngl[s]] = rng.integers(0, V, ngl[s])
    c_max = 1 + P * Kc + (P + 1) * L
    return block, ng, ngl, rng.standard_exponential(c_max).astype(np.float32), \
        rng.standard_exponential(c_max).astype(np.float32)


def parent_closed_best(parent, Q, k):
    """Max sum of Q over all parent-closed sets of k non-anchor nodes."""
    nodes = range(1, len(parent))
    best = -1.0
    for comb in itertools.combinations(nodes, k):
        s = set(comb) | {0}
        if all(parent[j] in s for j in comb):
            best = max(best, sum(Q[j] for j in comb))
    return best


def test_proposition1_best_first_prefix_is_optimal_tree():
    rng = np.random.Generator(np.random.Philox(31))
    checked = 0
    for trial in range(60):
        P, Kc, L = int(rng.integers(1, 4)), int(rng.integers(1, 3)), int(rng.integers(0, 3))
        block, ng, ngl, wn, wz = random_forest_inputs(rng, P, Kc, max(L, 1))
        full = O.tree_build(block, ng, ngl, wn, wz, rows_cap=64)
        cnt = full["count"]
        if cnt > 13:
            continue
        fpar, fQ = full["f_parent"], full["f_Q"]
        assert all(fpar[j] < j for j in range(1, cnt))          # parents precede children
        assert all(fQ[j] <= fQ[fpar[j]] for j in range(1, cnt))
        for rows in range(2, cnt + 1):
            t = O.tree_build(block, ng, ngl, wn, wz, rows_cap=rows)
            n = t["n_rows"]
            assert n == rows
            pr = t["parent_row"][:n]
            assert pr[0] == -1 and all(0 <= pr[i] < i for i in range(1, n))   # depth-first, a tree
            got = t["Q"][1:n].sum()
            assert got == pytest.approx(parent_closed_best(fpar, fQ, rows - 1), rel=1e-12)
            checked += 1
    assert checked > 100


def test_uniform_weights_give_equal_shares():
    # all weights 1: each of a parent's c children gets q = 1/(c+1) (the 'none'
    # outcome takes the same share), so Q is a product of such shares
    P, Kc, L = 3, 2, 4
    block = np.array([[1, 2], [3, 4], [5, 0]], np.int32)
    ng = np.full((P + 1, L), -1, np.int32)
    ngl = np.zeros(P + 1, np.int32)
    c_max = 1 + P * Kc + (P + 1) * L
    t = O.tree_build(block, ng, ngl, np.ones(c_max, np.float32), np.ones(c_max, np.float32), rows_cap=64)
    fQ = t["f_Q"]
    assert fQ[1] == pytest.approx(1 / 3) and fQ[2] == pytest.approx(1 / 3)       # position 1 under anchor
    assert fQ[3] == pytest.approx(1 / 9) and fQ[5] == pytest.approx(1 / 27)


def test_ngram_fill_agrees_and_branches():
    P, Kc, L = 3, 2, 6
    block = np.array([[10, 11], [20, 21], [30, 31]], np.int32)
    ng = np.full((P + 1, L), -1, np.int32)
    ngl = np.zeros(P + 1, np.int32)
    ng[0, :5] = [10, 20, 99, 98, 97]      # follows two picks, then branches below pick 2
    ngl[0] = 5
    ng[2, :2] = [31, 50]                  # from pick 2: agrees with a sibling at position 3, then new
    ngl[2] = 2
    c_max = 1 + P * Kc + (P + 1) * L
    t = O.tree_build(block, ng, ngl, np.ones(c_max, np.float32), np.ones(c_max, np.float32), rows_cap=64)
    tok, par, kind = t["f_token"], t["f_parent"], t["f_kind"]
    assert t["count"] == 1 + 6 + 3 + 1
    assert kind[1] & 4 and kind[3] & 4                 # picks 1, 2 agreed
    assert list(tok[7:10]) == [99, 98, 97] and par[7] == 3 and par[8] == 7 and par[9] == 8
    assert kind[6] & 4 and tok[10] == 50 and par[10] == 6   # sibling (30/31 rank 1) agreed, then new node
    # depth limit: nothing deeper than depth_max below the anchor
    t2 = O.tree_build(block, ng, ngl, np.ones(c_max, np.float32), np.ones(c_max, np.float32),
                      depth_max=3, rows_cap=64)
    assert t2["count"] == 1 + 6 + 1 + 0     # only 99 at depth 3 from the anchor chain; 50 would be depth 4


def path_forest(block, chains, depth_max, c_max):
    """The candidate forest from its definition (AdaSpark Section 3.3, n-gram
    fill): a node is a token path from the anchor.  The drafter block gives
    position p's candidates below pick p - 1 (a path through a token that
    several candidates hold goes through the lowest of them); chain s starts
    at the anchor (s = 0) or at pick s, and each of its tokens within the
    depth limit extends its path by one.  The first appearance of a path, in
    chain order and then token order, makes its node, numbered after the
    block; c_max drops the nodes past it (and every path below them).  A node
    that a chain reaches without making it is agreed."""
    P, Kc = block.shape
    index, info = {(): 0}, {0: ((), -1)}
    for p in range(1, P + 1):
        prefix = tuple(int(block[q, 0]) for q in range(p - 1))
        for k in range(Kc):
            j = 1 + (p - 1) * Kc + k
            path = prefix + (int(block[p - 1, k]),)
            index.setdefault(path, j)
            info[j] = (path, 0 if p == 1 else 1 + (p - 2) * Kc)
    n, agreed = 1 + P * Kc, set()
    for s_, chain in enumerate(chains):
        path = tuple(int(block[q, 0]) for q in range(s_))
        for i, tok in enumerate(chain):
            if len(path) + 1 > depth_max:
                break
            parent = index.get(path)
            path = path + (int(tok),)
            if path in index:
                agreed.add(index[path])
            elif parent is not None and n < c_max:
                index[path] = n
                info[n] = (path, parent)
                n += 1
    return n, index, info, agreed


@pytest.mark.parametrize("seed", range(6))
def test_forest_is_the_set_of_chain_paths(seed):
    """The oracle's chain walk (a descent per chain, then a new path) against
    the forest of distinct token paths: the node count, every node's token
    and parent, the order new nodes are made in and the agreed marks, on
    blocks whose picks follow a text and chains that continue it from each
    pick, with duplicate candidates, depth limits and c_max caps."""
    rng = np.random.default_rng(900 + seed)
    for _ in range(60):
        P, Kc, L, V = int(rng.integers(0, 7)), int(rng.integers(1, 4)), int(rng.integers(1, 9)), int(rng.integers(2, 5))
        text = rng.integers(0, V, P + L + 4)
        block = rng.integers(0, V, (P, Kc)).astype(np.int32)
        if P:
            block[:, 0] = np.where(rng.random(P) < 0.8, text[:P], block[:, 0])
        ng = np.full((P + 1, L), -1, np.int32)
        ngl = rng.integers(0, L + 1, P + 1).astype(np.int32)
        for s_ in range(P + 1):
            seq = text[s_:s_ + L] if rng.random() < 0.7 else rng.integers(0, V, L)
            ng[s_] = seq
        nd = 1 + P * Kc
        depth_max = int(rng.choice([64, int(rng.integers(1, 8))]))
        c_max = int(rng.choice([nd + (P + 1) * L, nd + int(rng.integers(0, 6))]))
        t = O.tree_build(block, ng, ngl, np.ones(c_max, np.float32), np.ones(c_max, np.float32),
                         depth_max=depth_max, rows_cap=8)
        chains = [ng[s_, :ngl[s_]] for s_ in range(P + 1)]
        n, index, info, agreed = path_forest(block, chains, depth_max, c_max)
        tok, par, kind = t["f_token"], t["f_parent"], t["f_kind"]
        assert t["count"] == n
        for j in range(1, n):
            path, parent = info[j]
            assert tok[j] == path[-1] and par[j] == parent, (j, path)
            assert bool(kind[j] & 4) == (j in agreed), j
            assert (kind[j] & 3) == (3 if j >= nd else (1 if (j - 1) % Kc == 0 else 2))


@pytest.mark.parametrize("rows_cap", [1, 2, 5, 16, 64])
def test_rows_are_the_depth_first_order_of_the_best_nodes(rows_cap):
    """The rows of the tree build from their definition (AdaSpark Section
    3.1): the rows_cap - 1 best candidates by Q (fp32, ties to the lower
    index), with the anchor, laid out depth first from the anchor with each
    node's children in index order, by a recursive walk."""
    rng = np.random.default_rng(31 + rows_cap)
    for _ in range(40):
        P, Kc, L = int(rng.integers(0, 6)), int(rng.integers(1, 4)), int(rng.integers(0, 8))
        block, ng, ngl, wn, wz = random_forest_inputs(rng, P, Kc, L, V=5)
        t = O.tree_build(block, ng, ngl, wn, wz, depth_max=int(rng.integers(1, 10)), rows_cap=rows_cap)
        cnt, tok, par, fq = t["count"], t["f_token"], t["f_parent"], t["f_Q"]
        order = sorted(range(1, cnt), key=lambda j: (-float(np.float32(fq[j])), j))
        chosen = {0} | set(order[:rows_cap - 1])
        rows = []
        def visit(u, prow):
            me = len(rows)
            rows.append((-1 if u == 0 else int(tok[u]), prow, float(fq[u])))
            for c in range(1, cnt):
                if c in chosen and par[c] == u:
                    visit(c, me)
        visit(0, -1)
        n = t["n_rows"]
        assert n == len(rows) == min(rows_cap, cnt)
        assert [(int(t["node_token"][i]), int(t["parent_row"][i]), float(t["Q"][i])) for i in range(n)] == rows
        assert all(t["node_token"][i] == -1 and t["parent_row"][i] == -1 for i in range(n, rows_cap))


def test_path_probabilities_from_the_weights():
    """Q of every node from its definition (AdaSpark Section 3.3, the
    Eq. (6) form with given weights): a node's share of its parent is its
    weight over the parent's 'none' weight plus all its children's weights
    (summed in index order), and Q is the product of the shares down the
    path, in fp64, on random forests and weights."""
    rng = np.random.default_rng(4242)
    for _ in range(80):
        P, Kc, L = int(rng.integers(0, 6)), int(rng.integers(1, 4)), int(rng.integers(0, 8))
        block, ng, ngl, wn, wz = random_forest_inputs(rng, P, Kc, L, V=5)
        t = O.tree_build(block, ng, ngl, wn, wz, depth_max=int(rng.integers(1, 10)), rows_cap=4)
        cnt, par, fq = t["count"], t["f_parent"], t["f_Q"]
        den = [float(wz[p]) for p in range(cnt)]
        for c in range(1, cnt):
            den[par[c]] += float(wn[c])
        q = [1.0] * cnt
        for j in range(1, cnt):
            q[j] = q[par[j]] * (float(wn[j]) / den[par[j]])
        assert list(map(float, fq)) == q


def chain_tree(tokens):
    n = len(tokens) + 1
    node_token = np.full(n, -1, np.int32)
    node_token[1:] = tokens
    parent = np.arange(-1, n - 1, dtype=np.int32)
    return node_token, parent


def test_chain_tree_equals_chain_verify_at_t0():
    rng = np.random.Generator(np.random.Philox(5))
    V, B, bs = 40, 6, 64
    z = rng.standard_normal((bs, B + 1, V)).astype(np.float32)
    am = np.argmax(z, -1)
    y = np.where(rng.random((bs, B)) < 0.7, am[:, :B], rng.integers(0, V, (bs, B))).astype(np.int32)
    ch = O.verify_chain(z.reshape(-1, V), np.arange(bs) * (B + 1), y, np.ones((bs, B), np.uint8),
                        np.full(bs, B, np.int32), np.zeros((bs, B), np.float32), np.zeros(bs, np.float32), 0.0)
    nt = np.zeros((bs, B + 1), np.int32)
    pr = np.zeros((bs, B + 1), np.int32)
    for r in range(bs):
        nt[r], pr[r] = chain_tree(y[r])
    tr = O.verify_tree(z.reshape(-1, V), np.arange(bs) * (B + 1), nt, pr, np.full(bs, B + 1, np.int32))
    assert np.array_equal(tr["out_num"], ch["out_num"])
    for r in range(bs):
        n = ch["out_num"][r]
        assert list(tr["out_tokens"][r, :n]) == list(ch["out_tokens"][r, :n])


def test_tree_walk_is_greedy_decode_of_markov_target():
    # rows are a Markov target p(.|token of the row's node); the committed
    # tokens are the greedy continuation for as long as the tree holds it
    rng = np.random.Generator(np.random.Philox(6))
    V = 5
    Z = rng.standard_normal((V, V)).astype(np.float32)
    g = [int(np.argmax(Z[0]))]
    for _ in range(8):
        g.append(int(np.argmax(Z[g[-1]])))
    # tree: anchor (token 0) -> greedy path of 4 nodes, plus wrong siblings
    node_token = [-1, g[0], (g[0] + 1) % V, g[1], g[2], (g[2] + 2) % V, g[3]]
    parent = [-1, 0, 0, 1, 3, 3, 4]
    rows = np.stack([Z[0 if i == 0 else node_token[i]] for i in range(len(node_token))])
    res = O.verify_tree(rows, np.array([0]), np.array([node_token], np.int32), np.array([parent], np.int32),
                        np.array([len(node_token)], np.int32))
    assert res["out_num"][0] == 5 and list(res["out_tokens"][0, :5]) == g[:5]
    assert list(res["out_path_rows"][0, :5]) == [0, 1, 3, 4, 6]
    # at most one child of an accepted node matches: a path
    assert len(set(res["out_path_rows"][0, :5])) == 5


# ---------------------------------------------------------------------------
# Eq. (6) scores and the S(n) curve (AdaSpark Section 3.3 "Form" and
# "Learning"; Section 3.1: a single walk down the best-first order yields S
# at every width)
# ---------------------------------------------------------------------------

def prior(**over):
    """The empty-store prior: pick ln 2 + logit h, sibling log r, every other
    coefficient and bucket weight 0."""
    coef = dict(a=[np.log(2.0), 1.0, 0.0, 0.0, 1.0, 0.0, 0.0], w_bucket=np.zeros(64), w_agreed=np.zeros((64, 2)),
                w_contra=np.zeros((8, 2)), psi_depth=np.zeros(16))
    coef.update(over)
    return coef


def scores(coef, P, Kc, h=None, sigma=None, r=None, psi_ctx=0.0, b_req=0.0, p_src=0.5, feat=None):
    return dict(coef=coef, h=np.full(P, 0.5) if h is None else h, sigma=np.full(P, 0.5) if sigma is None else sigma,
                r_share=np.full((P, Kc), 1.0 / max(1, Kc - 1)) if r is None else r, psi_ctx=psi_ctx, b_req=b_req,
                p_src=p_src, ng_feat=np.zeros((P + 1, 4), np.int32) if feat is None else feat)


def test_prior_gives_the_head_to_the_pick_and_shares_to_siblings():
    """With the prior and siblings' shares summing to 1, a pick's estimate is
    its confidence head h, each sibling gets its share of half the rest and
    'none' the other half: odds 2h/(1-h) and r against the none outcome's 1."""
    block = np.array([[10, 11, 12]], np.int32)
    ng = np.full((2, 3), -1, np.int32)
    t = O.tree_build(block, ng, np.zeros(2, np.int32), rows_cap=8, c_max=16,
                     scores=scores(prior(), 1, 3, h=np.array([0.7]), r=np.array([[0.0, 0.6, 0.4]])))
    fQ = t["f_Q"]
    assert fQ[1] == pytest.approx(0.7, rel=1e-12)
    assert fQ[2] == pytest.approx(0.6 * 0.15, rel=1e-12) and fQ[3] == pytest.approx(0.4 * 0.15, rel=1e-12)


def test_ngram_node_prior_and_bucket():
    """A lone n-gram node takes its source's precision at the prior; its
    bucket weight multiplies the odds.  The chain continues a 7-token copy
    (evidence class 2); the second node has one n-gram node above it, so its
    bucket is 4 * 2 + 1 = 9."""
    block = np.array([[10]], np.int32)
    ng = np.array([[20, 21, -1], [-1, -1, -1]], np.int32)        # anchor chain: 20 (not the pick), 21
    feat = np.array([[7, 1, 0, 100], [0, 0, 0, -1]], np.int32)
    wb = np.arange(64) * 0.01
    wb[9] = 0.5
    t = O.tree_build(block, ng, np.array([2, 0], np.int32), rows_cap=8, c_max=16,
                     scores=scores(prior(w_bucket=wb), 1, 1, h=np.array([0.6]), p_src=0.8, feat=feat))
    fp, fk, fQ, ft = t["f_parent"], t["f_kind"], t["f_Q"], t["f_token"]
    n1, n2 = 2, 3
    assert ft[n1] == 20 and ft[n2] == 21 and fp[n2] == n1 and (fk[n2] & 3) == 3
    odds1 = 0.8 / 0.2 * np.exp(wb[8])                 # bucket 4 * 2 + 0 under the anchor
    odds_pick = 2 * 0.6 / 0.4 * np.exp(-np.log(4.0))  # contradicted: minus max(0, logit 0.8)
    assert fQ[n1] == pytest.approx(odds1 / (1 + odds1 + odds_pick), rel=1e-12)
    assert fQ[1] == pytest.approx(odds_pick / (1 + odds1 + odds_pick), rel=1e-12)
    odds2 = 0.8 / 0.2 * np.exp(0.5)
    assert fQ[n2] == pytest.approx(fQ[n1] * odds2 / (1 + odds2), rel=1e-12)


def test_follower_node_bucket_and_agreement():
    """Tokens of the follower fallback are n-gram nodes of their own kind: a
    follower seen 5 times (evidence class 2) directly under the anchor has
    bucket 32 + 4 * 2 + 0 = 40, the follower after it (seen once, class 0,
    one n-gram node above) bucket 32 + 0 + 1 = 33; a follower token that
    agrees with the pick adds the agreed weight of its own bucket."""
    block = np.array([[10]], np.int32)
    ng = np.array([[20, 21, -1], [-1, -1, -1]], np.int32)
    fol = np.array([[5, 1, 0], [0, 0, 0]], np.int32)
    feat = np.array([[0, 0, 0, -1], [0, 0, 0, -1]], np.int32)   # no copy: the chain is all followers
    wb = np.zeros(64)
    wb[40], wb[33], wb[8] = 0.5, -0.25, 3.0                     # 8: the copy bucket a wrong kind would take
    t = O.tree_build(block, ng, np.array([2, 0], np.int32), rows_cap=8, c_max=16, ng_follow=fol,
                     scores=scores(prior(w_bucket=wb), 1, 1, h=np.array([0.6]), p_src=0.8, feat=feat))
    ft, fp, fQ = t["f_token"], t["f_parent"], t["f_Q"]
    n1, n2 = 2, 3
    assert ft[n1] == 20 and ft[n2] == 21 and fp[n2] == n1
    odds1 = 0.8 / 0.2 * np.exp(0.5)
    odds_pick = 2 * 0.6 / 0.4 * np.exp(-np.log(4.0))   # contradicted by the follower (its class 2)
    assert fQ[n1] == pytest.approx(odds1 / (1 + odds1 + odds_pick), rel=1e-12)
    odds2 = 0.8 / 0.2 * np.exp(-0.25)
    assert fQ[n2] == pytest.approx(fQ[n1] * odds2 / (1 + odds2), rel=1e-12)
    # agreement: the follower proposes the pick's own token
    ng2 = np.array([[10, -1, -1], [-1, -1, -1]], np.int32)
    fol2 = np.array([[9, 0, 0], [0, 0, 0]], np.int32)           # class 3: bucket 32 + 12 + 0 = 44
    wa = np.zeros((64, 2))
    wa[44, 0], wa[12, 0] = 0.375, 5.0
    t2 = O.tree_build(block, ng2, np.array([1, 0], np.int32), rows_cap=8, c_max=16, ng_follow=fol2,
                      scores=scores(prior(w_agreed=wa), 1, 1, h=np.array([0.6]), p_src=0.8, feat=feat))
    assert t2["count"] == 2 and (t2["f_kind"][1] & 4)
    odds = 2 * 0.6 / 0.4 * np.exp(np.log(4.0) + 0.375)
    assert t2["f_Q"][1] == pytest.approx(odds / (1 + odds), rel=1e-12)


def test_agreed_and_weak_sources():
    """An agreed pick adds max(0, logit p_src) plus its agreed-bucket weight;
    a source below 1/2 neither lifts the tokens it agrees with nor sinks the
    ones it contradicts."""
    block = np.array([[10], [11]], np.int32)
    ng = np.array([[10, 11], [-1, -1], [-1, -1]], np.int32)      # the anchor chain agrees with both picks
    feat = np.array([[40, 1, 0, 5], [0, 0, 0, -1], [0, 0, 0, -1]], np.int32)   # evidence class 5
    wa = np.zeros((64, 2))
    wa[20, 0], wa[21, 0] = 0.25, 0.125        # buckets 4 * 5 + 0 (position 1) and + 0 (position 2: no n-gram above)
    h = np.array([0.6, 0.7])
    for p_src, lift in ((0.9, np.log(9.0)), (0.3, 0.0)):
        t = O.tree_build(block, ng, np.array([2, 0, 0], np.int32), rows_cap=8, c_max=16,
                         scores=scores(prior(w_agreed=wa), 2, 1, h=h, p_src=p_src, feat=feat))
        assert t["count"] == 3 and (t["f_kind"][1] & 4) and (t["f_kind"][2] & 4)
        for node, hp, w in ((1, 0.6, 0.25), (2, 0.7, 0.25)):
            odds = 2 * hp / (1 - hp) * np.exp(lift + w)
            q = odds / (1 + odds)
            got = t["f_Q"][node] / (t["f_Q"][t["f_parent"][node]])
            assert got == pytest.approx(q, rel=1e-12), (p_src, node)


def test_s_curve_is_the_best_tree_of_every_width():
    """S(n) equals, for every width n, the largest sum of Q over parent-closed
    sets of n - 1 candidates (Proposition 1 applied at every width), with the
    Eq. (6) scores under random coefficients."""
    rng = np.random.Generator(np.random.Philox(77))
    checked = 0
    for trial in range(40):
        P, Kc, L = int(rng.integers(1, 4)), int(rng.integers(1, 3)), int(rng.integers(1, 3))
        block, ng, ngl, _, _ = random_forest_inputs(rng, P, Kc, L)
        coef = prior(a=rng.normal(0, 1, 7), w_bucket=rng.normal(0, 1, 64), w_agreed=rng.normal(0, 1, (64, 2)),
                     w_contra=rng.normal(0, 1, (8, 2)), psi_depth=rng.normal(0, 0.5, 16))
        feat = np.zeros((P + 1, 4), np.int32)
        feat[:, 0] = rng.integers(1, 20, P + 1)
        sc = scores(coef, P, Kc, h=rng.uniform(0.05, 0.95, P), sigma=rng.uniform(0.05, 0.95, P),
                    r=rng.uniform(0.05, 0.95, (P, Kc)), psi_ctx=rng.normal(), b_req=rng.normal(),
                    p_src=rng.uniform(0.05, 0.95), feat=feat)
        c_max = 1 + P * Kc + (P + 1) * L
        full = O.tree_build(block, ng, ngl, rows_cap=c_max, c_max=c_max, scores=sc)
        cnt = full["count"]
        if cnt > 12:
            continue
        # the estimates of a parent's children and its 'none' outcome are a distribution
        fpar, fQ = full["f_parent"], full["f_Q"]
        for par in range(cnt):
            kids = [j for j in range(1, cnt) if fpar[j] == par]
            if kids:
                assert sum(fQ[j] for j in kids) / fQ[par] < 1.0
        for n in range(1, cnt + 1):
            want = 0.0 if n == 1 else parent_closed_best(fpar, fQ, n - 1)
            assert full["S_curve"][n - 1] == pytest.approx(want, rel=1e-12, abs=1e-300)
            checked += 1
    assert checked > 100


# --- rows from a forest the caller built (AdaSpark Section 3.1) ---------------

def random_given_forest(rng, n, c_max, V=50, tie_q=False):
    """Parents below their children, tokens, acceptance estimates in [0, 1]."""
    token = np.full(c_max, -1, np.int32)
    parent = np.full(c_max, -1, np.int32)
    q = np.zeros(c_max, np.float32)
    for j in range(1, n):
        parent[j] = rng.integers(0, j)
        token[j] = rng.integers(0, V)
        q[j] = rng.choice([0.25, 0.5, 1.0]) if tie_q else rng.uniform(0.0, 1.0)
    return token, parent, q


def dfs_rows(parent, sel):
    """Pre-order of the selected nodes from node 0, children in index order."""
    rows, prow = [], []

    def visit(u, pr):
        rows.append(u)
        prow.append(pr)
        me = len(rows) - 1
        for c in range(1, len(parent)):
            if c in sel and parent[c] == u:
                visit(c, me)
    visit(0, -1)
    return rows, prow


def test_given_forest_hand_example():
    """Anchor with children 1 (q .9) and 2 (q .5); node 1 with children 3 (q .6)
    and 4 (q .95): Q = .9, .5, .54, .855; the best three are 1, 4, 3, laid out
    anchor, 1, 3, 4."""
    t = O.tree_forest([-1, 5, 6, 7, 8], [-1, 0, 0, 1, 1], [0, 0.9, 0.5, 0.6, 0.95], 5, rows_cap=4)
    assert t["n_rows"] == 4 and t["flag"] == 0
    assert list(t["node_token"]) == [-1, 5, 7, 8]
    assert list(t["parent_row"]) == [-1, 0, 1, 1]
    q = np.float32([0.9, 0.6, 0.95]).astype(np.float64)
    assert t["Q"][1:] == pytest.approx([q[0], q[0] * q[1], q[0] * q[2]], rel=0, abs=0)
    assert t["S_curve"] == pytest.approx([0.0, q[0], q[0] + q[0] * q[2], q[0] + q[0] * q[2] + q[0] * q[1]], rel=1e-15)
    # a cap above the forest keeps every node; a cap of one keeps the anchor
    assert O.tree_forest([-1, 5, 6, 7, 8], [-1, 0, 0, 1, 1], [0, 0.9, 0.5, 0.6, 0.95], 5, rows_cap=16)["n_rows"] == 5
    one = O.tree_forest([-1, 5, 6, 7, 8], [-1, 0, 0, 1, 1], [0, 0.9, 0.5, 0.6, 0.95], 5, rows_cap=1)
    assert one["n_rows"] == 1 and list(one["node_token"]) == [-1]


@pytest.mark.parametrize("tie_q", [False, True])
def test_given_forest_rows_are_the_best_tree_of_every_width(tie_q):
    """Proposition 1 on random forests: the rows hold the largest sum of Q over
    parent-closed sets of their size, S(n) is that sum at every width, Q is the
    product of q along the path, and the rows are the pre-order of the chosen
    set with children in index order."""
    rng = np.random.Generator(np.random.Philox(5150 + tie_q))
    checked = 0
    for trial in range(40):
        n = int(rng.integers(1, 12))
        token, parent, q = random_given_forest(rng, n, 12, tie_q=tie_q)
        full = O.tree_forest(token, parent, q, n, rows_cap=n)
        assert full["flag"] == 0 and full["count"] == n
        for j in range(1, n):   # the path product, root first
            path, u = [], j
            while u != 0:
                path.append(u)
                u = parent[u]
            want = 1.0
            for v in reversed(path):
                want *= float(q[v])
            assert full["f_Q"][j] == want
        for rows in range(1, n + 1):
            t = O.tree_forest(token, parent, q, n, rows_cap=rows)
            assert t["n_rows"] == rows
            best = 0.0 if rows == 1 else parent_closed_best(parent[:n], full["f_Q"], rows - 1)
            assert t["Q"][1:rows].sum() == pytest.approx(best, rel=1e-12, abs=1e-300)
            assert full["S_curve"][rows - 1] == pytest.approx(best, rel=1e-12, abs=1e-300)
            # the chosen set: fp32 Q descending, index ascending
            key = sorted(range(1, n), key=lambda j: (-np.float32(full["f_Q"][j]), j))
            sel = set(key[:rows - 1])
            order, prow = dfs_rows(parent[:n], sel)
            assert list(t["node_token"][:rows]) == [-1] + [int(token[u]) for u in order[1:]]
            assert list(t["parent_row"][:rows]) == prow
            checked += 1
    assert checked > 150


def test_given_forest_broken_rules_keep_the_anchor_alone():
    base_tok, base_par = [-1, 3, 4, 5], [-1, 0, 1, 1]
    good = [0.0, 0.5, 0.5, 0.5]
    assert O.tree_forest(base_tok, base_par, good, 4)["flag"] == 0
    for par, q in (([-1, 0, 2, 1], good),            # a parent not below its child
                   ([-1, 0, 1, 3], good),
                   ([-1, -1, 1, 1], good),           # a node without a parent
                   (base_par, [0.0, 0.5, 1.5, 0.5]),  # q above 1
                   (base_par, [0.0, -0.1, 0.5, 0.5]),  # q below 0
                   (base_par, [0.0, 0.5, float("nan"), 0.5])):
        t = O.tree_forest(base_tok, par, q, 4, rows_cap=4)
        assert t["flag"] == O.BAD_FOREST
        assert t["n_rows"] == 1 and list(t["node_token"]) == [-1, -1, -1, -1]
        assert list(t["S_curve"]) == [0.0, 0.0, 0.0, 0.0]
    # node counts outside [1, c_max] are clamped and flagged
    t = O.tree_forest(base_tok, base_par, good, 0, rows_cap=4)
    assert t["flag"] == O.BAD_LENGTH and t["n_rows"] == 1
    t = O.tree_forest(base_tok, base_par, good, 9, rows_cap=4)
    assert t["flag"] == O.BAD_LENGTH and t["n_rows"] == 4 and t["count"] == 4
    # q of exactly 0 and 1 are allowed: a zero-Q node is still a candidate
    t = O.tree_forest(base_tok, base_par, [0.0, 1.0, 0.0, 1.0], 4, rows_cap=4)
    assert t["flag"] == 0 and list(t["node_token"]) == [-1, 3, 4, 5] and list(t["Q"]) == [1.0, 1.0, 0.0, 1.0]
