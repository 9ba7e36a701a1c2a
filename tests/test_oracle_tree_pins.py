"""Pins of the coupled-Gumbel tree oracle (SPOT, Sec. 4.3 and App. A).

The checks use a "state-hashed" stand-in model: the logits of a block state
are a deterministic function of the state, which is exactly the setting of
SPOT's Propositions 1-2 (a target with a unique successor per state).
"""

import hashlib
import math

import numpy as np
import pytest
from scipy import stats

import oracle

M = -1  # mask symbol in a state tuple


def state_logits(state, V, scale=2.0, salt=0):
    """Deterministic logits [L, V] of a block state (tuple, M = masked)."""
    h = hashlib.sha256(repr((salt, tuple(state))).encode()).digest()
    rng = np.random.default_rng(int.from_bytes(h[:8], "little"))
    return rng.normal(0, scale, (len(state), V))


def masked_of(state):
    return [s for s, t in enumerate(state) if t == M]


def phi(state, G, T, V, salt=0):
    t = oracle.state_transition(state_logits(state, V, salt=salt), masked_of(state), G, T)
    return t["pos"], t["tok"]


def tree_tensors(root, nodes, V, salt=0):
    L = len(root)
    S = len(nodes)
    states = []
    for z, (par, pos, tok) in enumerate(nodes):
        if z == 0:
            states.append(tuple(root))
        else:
            st = list(states[par])
            assert st[pos] == M
            st[pos] = tok
            states.append(tuple(st))
    logits = np.stack([state_logits(s, V, salt=salt) for s in states])[None]
    masked = np.array([[t == M for t in s] for s in states])[None]
    parent = np.array([n[0] for n in nodes])[None]
    epos = np.array([max(n[1], 0) for n in nodes])[None]
    etok = np.array([max(n[2], 0) for n in nodes])[None]
    return logits, masked, parent, epos, etok, states


def orbit(root, G, T, V, depth, salt=0):
    st = list(root)
    out = []
    for _ in range(depth):
        if not masked_of(st):
            break
        s, v = phi(st, G, T, V, salt)
        out.append((s, v))
        st[s] = v
    return out


def gumbel(rng, L, V):
    u = rng.random((L, V))
    return -np.log(-np.log(np.clip(u, 2.0 ** -24, 1 - 2.0 ** -24)))


# ------------------------------------------------------ Gumbel-max law ---

@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_gumbel_draw_has_tempered_law(T):
    # SPOT App. A.3 Eq. 5-7: argmax_v[(1/T) log p(v) + G_v] ~ pi_T.
    rng = np.random.default_rng(20)
    V, N = 8, 20000
    x = rng.normal(0, 1.5, V)
    want = oracle.tempered_softmax(x, T)
    counts = np.zeros(V)
    for _ in range(N):
        g = gumbel(rng, 1, V)
        t = oracle.state_transition([x], [0], g, T)
        counts[t["tok"]] += 1
    assert stats.chisquare(counts, want * N).pvalue > 1e-4


def test_zero_temperature_limit_is_argmax():
    rng = np.random.default_rng(21)
    for _ in range(50):
        x = rng.normal(0, 3, 40)
        g = gumbel(rng, 1, 40)
        small = oracle.state_transition([x], [0], g, 1e-6)["tok"]
        greedy = oracle.state_transition([x], [0], None, 0.0)["tok"]
        assert small == greedy == int(np.argmax(x))


def test_position_selection_brute_force_and_ties():
    rng = np.random.default_rng(22)
    V, L = 16, 6
    for _ in range(50):
        rows = rng.normal(0, 2, (L, V))
        mpos = sorted(rng.choice(L, size=int(rng.integers(1, L + 1)), replace=False).tolist())
        conf = {s: float(np.max(np.exp(rows[s]) / np.exp(rows[s]).sum())) for s in mpos}
        best = max(mpos, key=lambda s: (conf[s], -s))
        assert oracle.state_transition(rows, mpos, None, 0.0)["pos"] == best
    rows = rng.normal(0, 2, (L, V))
    rows[4] = rows[1] + 0.0          # identical rows tie: lowest position wins
    rows[1, 0] = rows[4, 0] = 50.0
    assert oracle.state_transition(rows, [4, 1, 3], None, 0.0)["pos"] == 1


def test_coupling_bound():
    # SPOT Sec. 4.3: Pr[stale draw = fresh draw] >= (1 - d) / (1 + d),
    # d = TV(stale, fresh) of the tempered laws.
    rng = np.random.default_rng(23)
    V, N, T = 12, 4000, 1.0
    for sigma in (0.2, 0.6, 1.5):
        x = rng.normal(0, 2, V)
        xs = x + rng.normal(0, sigma, V)
        d = 0.5 * np.abs(oracle.tempered_softmax(x, T) - oracle.tempered_softmax(xs, T)).sum()
        agree = 0
        for _ in range(N):
            g = gumbel(rng, 1, V)
            a = oracle.state_transition([x], [0], g, T)["tok"]
            b = oracle.state_transition([xs], [0], g, T)["tok"]
            agree += a == b
        rate = agree / N
        assert rate >= (1 - d) / (1 + d) - 4 * math.sqrt(0.25 / N)


# ------------------------------------------------------------ tree walk ---

ROOT = [M, 3, M, M, 7, M, M, M]
V = 24


def _verify(root, nodes, G, T, salt=0):
    logits, masked, parent, epos, etok, states = tree_tensors(root, nodes, V, salt)
    r = oracle.verify_gumbel_tree(logits, masked, parent, epos, etok, None, G[None], T)
    return r, states


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_orbit_tree_is_accepted_to_full_depth(T):
    rng = np.random.default_rng(24)
    G = gumbel(rng, len(ROOT), V)
    orb = orbit(ROOT, G, T, V, 8)
    nodes = [(-1, -1, -1)]
    for k, (s, v) in enumerate(orb):
        nodes.append((k, s, v))
    r, states = _verify(ROOT, nodes, G, T)
    assert r["path_len"][0] == len(orb) == 6           # 6 masked positions
    assert list(r["path_nodes"][0, :7]) == list(range(7))
    assert r["num_commits"][0] == 6                    # last state terminal
    assert [(r["commit_pos"][0, k], r["commit_tok"][0, k]) for k in range(6)] == orb


def test_random_tree_commits_root_transition():
    rng = np.random.default_rng(25)
    G = gumbel(rng, len(ROOT), V)
    s0, v0 = phi(ROOT, G, 1.0, V)
    # positions/tokens chosen never to equal Phi of their parent
    logits_nodes = [(-1, -1, -1)]
    states = [tuple(ROOT)]
    for z in range(1, 10):
        par = int(rng.integers(0, z))
        st = list(states[par])
        mp = masked_of(st)
        ps, pv = phi(st, G, 1.0, V)
        s = mp[int(rng.integers(0, len(mp)))]
        v = int(rng.integers(0, V))
        if (s, v) == (ps, pv):
            v = (v + 1) % V
        logits_nodes.append((par, s, v))
        st[s] = v
        states.append(tuple(st))
    r, _ = _verify(ROOT, logits_nodes, G, 1.0)
    assert r["path_len"][0] == 0 and r["num_commits"][0] == 1
    assert (r["commit_pos"][0, 0], r["commit_tok"][0, 0]) == (s0, v0)


def test_drafter_invariance_prefix_of_same_orbit():
    # SPOT Prop. 2: for fixed G the committed trajectory is the orbit of
    # Phi_G whatever the tree; different trees commit prefixes of it.
    rng = np.random.default_rng(26)
    for trial in range(6):
        G = gumbel(rng, len(ROOT), V)
        orb = orbit(ROOT, G, 1.0, V, 8)
        for _ in range(4):
            nodes = [(-1, -1, -1)]
            states = [tuple(ROOT)]
            for z in range(1, 16):
                par = int(rng.integers(0, z))
                st = list(states[par])
                mp = masked_of(st)
                if not mp:
                    par, st, mp = 0, list(ROOT), masked_of(ROOT)
                if rng.random() < 0.6:
                    s, v = phi(st, G, 1.0, V)
                else:
                    s = mp[int(rng.integers(0, len(mp)))]
                    v = int(rng.integers(0, V))
                if any(nodes[k][0] == par and nodes[k][1:] == (s, v) for k in range(1, z)):
                    v = (v + 1) % V        # no duplicate children
                nodes.append((par, s, v))
                st[s] = v
                states.append(tuple(st))
            r, _ = _verify(ROOT, nodes, G, 1.0)
            k = r["num_commits"][0]
            got = [(r["commit_pos"][0, i], r["commit_tok"][0, i]) for i in range(k)]
            assert got == orb[:k]
            assert r["path_len"][0] + (1 if len(orb) > r["path_len"][0] else 0) == k


def test_chain_tree_reduces_to_chain_check():
    rng = np.random.default_rng(27)
    G = gumbel(rng, len(ROOT), V)
    orb = orbit(ROOT, G, 1.0, V, 8)
    for wrong_at in range(0, 5):
        nodes = [(-1, -1, -1)]
        for k in range(5):
            s, v = orb[k]
            if k == wrong_at:
                v = (v + 5) % V
            nodes.append((k, s, v))
        r, _ = _verify(ROOT, nodes, G, 1.0)
        assert r["path_len"][0] == wrong_at
        assert (r["commit_pos"][0, wrong_at], r["commit_tok"][0, wrong_at]) == orb[wrong_at]


def test_fixed_position_mode_matches_explicit_positions():
    rng = np.random.default_rng(28)
    G = gumbel(rng, len(ROOT), V)
    orb = orbit(ROOT, G, 1.0, V, 3)
    nodes = [(-1, -1, -1)] + [(k, s, v) for k, (s, v) in enumerate(orb)]
    logits, masked, parent, epos, etok, _ = tree_tensors(ROOT, nodes, V)
    nxt = np.array([[s for s, _ in orb] + [-1]])
    r = oracle.verify_gumbel_tree(logits, None, parent, epos, etok, None, G[None], 1.0,
                                  oracle.TREE_FIXED_POSITION, nxt)
    assert r["path_len"][0] == 3 and r["num_commits"][0] == 3


def test_tree_bad_input_status():
    rng = np.random.default_rng(29)
    G = gumbel(rng, len(ROOT), V)
    nodes = [(-1, -1, -1), (0, 0, 1), (1, 2, 3)]
    logits, masked, parent, epos, etok, _ = tree_tensors(ROOT, nodes, V)
    parent[0, 2] = 2                      # parent must precede the child
    r = oracle.verify_gumbel_tree(logits, masked, parent, epos, etok, None, G[None], 1.0)
    assert r["status"][0] == oracle.STATUS_BAD_INPUT and r["path_len"][0] == -1
