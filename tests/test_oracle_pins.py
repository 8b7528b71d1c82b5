"""Pins of the fp64 CPU oracle against closed forms, invariants, brute force
and the values the pages print.  CPU only.

Every test here checks the oracle against something other than itself:
  * closed forms of the gated delta rule (unit key with beta = 1 and no decay
    maps k to v; beta = 0 is pure decay; one token from a zero state gives
    y = beta (q.k) v);
  * the Comba error magnitudes the KBench spec prints for four wrong kernels;
  * special cases of the gate and L2-norm formulas;
  * brute force of the chunked WY algebra against the token recurrence.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import wy_chunkwise as wy
from gated_deltanet_linear_gdn_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_state(rng, *shape, scale=0.5):
    return scale * rng.standard_normal(shape)


def _unit(rng, *shape):
    z = rng.standard_normal(shape)
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


# ----------------------------------------------------------------- decode


@pytest.mark.parametrize("Dk,Dv", [(32, 32), (64, 48), (128, 128)])
def test_unit_key_beta_one_no_decay_maps_k_to_v(Dk, Dv):
    rng = np.random.default_rng(1)
    B, Hk, Hv = 2, 1, 2
    S = _rand_state(rng, B, Hv, Dv, Dk)
    q = rng.standard_normal((B, Hk, Dk))
    k = _unit(rng, B, Hk, Dk)
    v = rng.standard_normal((B, Hv, Dv))
    g = np.zeros((B, Hv))
    beta = np.ones((B, Hv))
    S1, _ = oracle.gdn_step(S, q, k, v, g, beta)
    for b in range(B):
        for h in range(Hv):
            # stored [Dv, Dk]: S1 @ k == v
            np.testing.assert_allclose(S1[b, h] @ k[b, 0], v[b, h], rtol=0, atol=1e-12)
            # a direction orthogonal to k reads the same before and after
            u = rng.standard_normal(Dk)
            u -= (u @ k[b, 0]) * k[b, 0]
            np.testing.assert_allclose(S1[b, h] @ u, S[b, h] @ u, rtol=0, atol=1e-12)


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(2)
    B, Hk, Hv, Dk, Dv = 3, 2, 4, 32, 16
    S = _rand_state(rng, B, Hv, Dv, Dk)
    q = rng.standard_normal((B, Hk, Dk))
    k = _unit(rng, B, Hk, Dk)
    v = rng.standard_normal((B, Hv, Dv))
    g = -rng.random((B, Hv))
    S1, y = oracle.gdn_step(S, q, k, v, g, np.zeros((B, Hv)))
    a = np.exp(g)[:, :, None, None]
    np.testing.assert_allclose(S1, a * S, rtol=1e-15, atol=0)
    hk = np.arange(Hv) // (Hv // Hk)
    y_ref = np.einsum("bhji,bhi->bhj", a * S, q[:, hk])
    np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-13)


def test_zero_state_single_token():
    rng = np.random.default_rng(3)
    B, Hk, Hv, Dk, Dv = 2, 2, 6, 64, 32
    q = rng.standard_normal((B, Hk, Dk))
    k = rng.standard_normal((B, Hk, Dk))   # any k: from zero the gate cannot matter
    v = rng.standard_normal((B, Hv, Dv))
    g = -rng.random((B, Hv))
    beta = rng.random((B, Hv))
    S1, y = oracle.gdn_step(np.zeros((B, Hv, Dv, Dk)), q, k, v, g, beta)
    hk = np.arange(Hv) // (Hv // Hk)
    qk = np.einsum("bhi,bhi->bh", q[:, hk], k[:, hk])
    np.testing.assert_allclose(y, beta[..., None] * qk[..., None] * v, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, beta[..., None, None] * v[..., :, None] * k[:, hk][..., None, :],
                               rtol=1e-15, atol=0)


def test_matrix_form_of_the_step():
    """S' = a (I - b k k^T) S + b k v^T in key-major form (stored as its transpose)."""
    rng = np.random.default_rng(4)
    B, Hk, Hv, Dk, Dv = 2, 1, 3, 32, 24
    S = _rand_state(rng, B, Hv, Dv, Dk)
    q = rng.standard_normal((B, Hk, Dk))
    k = _unit(rng, B, Hk, Dk)
    v = rng.standard_normal((B, Hv, Dv))
    g = -rng.random((B, Hv))
    beta = rng.random((B, Hv))
    S1, y = oracle.gdn_step(S, q, k, v, g, beta)
    for b in range(B):
        for h in range(Hv):
            kk = k[b, 0]
            Sm = S[b, h].T                      # Dk x Dv, math orientation
            Sn = np.exp(g[b, h]) * (np.eye(Dk) - beta[b, h] * np.outer(kk, kk)) @ Sm \
                + beta[b, h] * np.outer(kk, v[b, h])
            np.testing.assert_allclose(S1[b, h], Sn.T, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(y[b, h], Sn.T @ q[b, 0], rtol=1e-12, atol=1e-12)


def test_head_sharing_is_contiguous_groups():
    """Hv/Hk value heads in a row share one key head (hk = hv // (Hv/Hk))."""
    rng = np.random.default_rng(5)
    B, Hk, Hv, Dk, Dv = 2, 2, 6, 32, 32
    S = _rand_state(rng, B, Hv, Dv, Dk)
    tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv, act="f32")
    S1, y1 = oracle.gdn_step(S, tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"])
    rep = Hv // Hk
    qx = np.repeat(tok["q"], rep, axis=1)
    kx = np.repeat(tok["k"], rep, axis=1)
    S2, y2 = oracle.gdn_step(S, qx, kx, tok["v"], tok["g"], tok["beta"])
    assert np.array_equal(S1, S2) and np.array_equal(y1, y2)
    # the modulo mapping (hk = hv % Hk) is a different computation
    S3, _ = oracle.gdn_step(S, np.tile(tok["q"], (1, rep, 1)), np.tile(tok["k"], (1, rep, 1)),
                            tok["v"], tok["g"], tok["beta"])
    assert np.max(np.abs(S3 - S1)) > 1e-3


def test_oracle_rejects_bad_head_ratio():
    with pytest.raises(ValueError):
        oracle.gdn_step(np.zeros((1, 3, 4, 4)), np.zeros((1, 2, 4)), np.zeros((1, 2, 4)),
                        np.zeros((1, 3, 4)), np.zeros((1, 3)), np.zeros((1, 3)))


# ----------------------------------------------------------------- comba


def test_comba_zero_state_closed_form():
    rng = np.random.default_rng(6)
    B, H, K, V = 2, 3, 64, 32
    q = rng.standard_normal((B, H, K))
    k = _unit(rng, B, H, K)
    p = _unit(rng, B, H, K)
    v = rng.standard_normal((B, H, V))
    beta = rng.random((B, H))
    g = -rng.random((B, H))
    S1, o = oracle.comba_step(np.zeros((B, H, K, V)), q, k, v, p, beta, g)
    sc = K ** -0.5
    qk = np.einsum("bhi,bhi->bh", q, k)
    np.testing.assert_allclose(o, (beta * sc * qk)[..., None] * v, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, beta[..., None, None] * k[..., :, None] * v[..., None, :],
                               rtol=1e-15, atol=0)


def test_comba_with_p_equal_k_is_the_gated_delta_rule():
    """Reading with p = k makes Comba the GDN step on the transposed state with
    q pre-scaled (two independently written oracle functions agree)."""
    rng = np.random.default_rng(7)
    B, H, K, V = 2, 4, 32, 48
    S = _rand_state(rng, B, H, K, V)
    q = rng.standard_normal((B, H, K))
    k = _unit(rng, B, H, K)
    v = rng.standard_normal((B, H, V))
    beta = rng.random((B, H))
    g = -rng.random((B, H))
    sc = 0.37
    Sc, oc = oracle.comba_step(S, q, k, v, k, beta, g, scale=sc)
    Sg, yg = oracle.gdn_step(np.swapaxes(S, -1, -2), sc * q, k, v, g, beta)
    np.testing.assert_allclose(Sc, np.swapaxes(Sg, -1, -2), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oc, yg, rtol=1e-12, atol=1e-13)


def _relF(x, ref):
    return float(np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel()))


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split()
                vals[key] = float(val)
    return vals


def test_comba_wrong_kernels_land_where_the_spec_says():
    """Plant each mistake the KBench spec describes into the oracle's inputs or
    outputs and check the error lands near the printed magnitude (the worse
    of state_new and o, relative Frobenius)."""
    gold = _read_golden("comba_mutant_errors.txt")
    rng = np.random.default_rng(0)
    B, H, K, V = 32, 8, 128, 128
    S = np.zeros((B, H, K, V))
    for _ in range(synth.WARMUP_STEPS):
        t = synth.comba_token(rng, B, H, K, V)
        S, _ = oracle.comba_step(S, t["q"], t["k"], t["v"], t["p"], t["beta"], t["g"])
    S = S.astype(np.float32)                     # the state is handed over in fp32
    t = synth.comba_token(rng, B, H, K, V)
    args = (t["q"], t["k"], t["v"], t["p"], t["beta"], t["g"])
    Sr, orf = oracle.comba_step(S, *args)

    def worst(Sx, ox):
        return max(_relF(Sx, Sr), _relF(ox, orf))

    errs = {
        "bf16_state": worst(synth.round_bf16(Sr.astype(np.float32)), orf),
        "no_forget_gate": worst(*oracle.comba_step(S, t["q"], t["k"], t["v"], t["p"], t["beta"],
                                                   np.zeros_like(t["g"]))),
        "read_with_k": worst(*oracle.comba_step(S, t["q"], t["k"], t["v"], t["k"], t["beta"], t["g"])),
        "no_correction": worst(*oracle.comba_step(S, t["q"], t["k"], t["v"], np.zeros_like(t["p"]),
                                                  t["beta"], t["g"])),
    }
    band = {"bf16_state": 0.25, "no_forget_gate": 0.1, "read_with_k": 0.1, "no_correction": 0.1}
    for name, e in errs.items():
        assert abs(e / gold[name] - 1.0) < band[name], (name, e, gold[name])
    # a correct fp32 evaluation of the same step sits at the spec's ~1e-7
    S32, o32 = _comba_fp32_numpy(S, *args, scale=K ** -0.5)
    assert worst(S32, o32) < 10 * gold["correct_fp32"]


def _comba_fp32_numpy(S, q, k, v, p, beta, g, scale):
    """The Comba step in float32 numpy matrix form (spec_md), for calibration."""
    f = np.float32
    S = S.astype(f) * np.exp(g.astype(f))[..., None, None]
    u = (v.astype(f) - np.einsum("bhij,bhi->bhj", S, p.astype(f))) * beta.astype(f)[..., None]
    S = S + k.astype(f)[..., :, None] * u[..., None, :]
    o = np.einsum("bhij,bhi->bhj", S, (q.astype(f) * f(scale)))
    return S, o


# ----------------------------------------------------------------- gates


def test_gate_special_values():
    Hv = 4
    A_log = np.array([0.0, 0.5, 1.0, 2.7])
    dt = np.array([0.3, -0.2, 1.0, 0.0])
    a = np.tile(-dt, (3, 1))                      # a + dt_bias = 0 -> softplus = ln 2
    b = np.zeros((3, Hv))
    g, beta = oracle.gates(a, b, A_log, dt)
    np.testing.assert_allclose(g, np.tile(-np.exp(A_log) * np.log(2.0), (3, 1)), rtol=1e-15)
    np.testing.assert_allclose(beta, 0.5, rtol=0, atol=0)
    # A_log = 0: g = -softplus(x); large x: softplus(x) -> x; very negative: -> e^x
    x = np.array([[30.0, -30.0, 2.0, -1.0]])
    g, beta = oracle.gates(x, x, np.zeros(Hv), np.zeros(Hv))
    np.testing.assert_allclose(g[0, 0], -30.0, rtol=1e-13)
    np.testing.assert_allclose(g[0, 1], -np.exp(-30.0), rtol=1e-12)
    np.testing.assert_allclose(g[0, 2], -np.log1p(np.exp(2.0)), rtol=1e-15)
    np.testing.assert_allclose(beta[0], 1.0 / (1.0 + np.exp(-x[0])), rtol=1e-15)
    # symmetric pair: sigmoid(x) + sigmoid(-x) = 1, softplus(x) - softplus(-x) = x
    g1, b1 = oracle.gates(np.array([[1.7]]), np.array([[1.7]]), np.zeros(1), np.zeros(1))
    g2, b2 = oracle.gates(np.array([[-1.7]]), np.array([[-1.7]]), np.zeros(1), np.zeros(1))
    np.testing.assert_allclose(b1 + b2, 1.0, rtol=1e-15)
    np.testing.assert_allclose(-g1 + g2, 1.7, rtol=1e-14)


# ----------------------------------------------------------------- prefill


def _prefill_case(rng, lengths, Hk=2, Hv=4, Dk=16, Dv=8, pool=5):
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool, act="f32")
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    P0 = _rand_state(rng, pool, Hv, Dv, Dk)
    return inp, g, beta, P0


def test_l2norm_special_rows():
    """A unit key becomes k (1 + 1e-6)^-1/2; a zero row stays zero (no NaN)."""
    rng = np.random.default_rng(8)
    Dk, Dv = 16, 8
    k = _unit(rng, 1, 1, Dk)
    q = _unit(rng, 1, 1, Dk)
    v = rng.standard_normal((1, 1, Dv))
    P, y = oracle.gdn_prefill(q, k, v, np.zeros((1, 1)), np.ones((1, 1)), np.zeros((1, 1, Dv, Dk)),
                              [0], [0, 1], scale=1.0)
    c = (1 + 1e-6) ** -0.5
    np.testing.assert_allclose(P[0, 0], np.outer(v[0, 0], c * k[0, 0]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(y[0, 0], c * c * (q[0, 0] @ k[0, 0]) * v[0, 0], rtol=1e-13, atol=1e-15)
    P, y = oracle.gdn_prefill(np.zeros((1, 1, Dk)), np.zeros((1, 1, Dk)), v, np.zeros((1, 1)),
                              np.ones((1, 1)), np.zeros((1, 1, Dv, Dk)), [0], [0, 1])
    assert np.all(P == 0) and np.all(y == 0)


def test_prefill_is_the_decode_loop():
    """Prefill equals repeated decode steps on normalised, pre-scaled q/k."""
    rng = np.random.default_rng(9)
    lengths = [5, 0, 3]
    inp, g, beta, P0 = _prefill_case(rng, lengths)
    for name in ("q", "k", "v"):
        inp[name] = inp[name].astype(np.float64)
    P, y = oracle.gdn_prefill(inp["q"], inp["k"], inp["v"], g, beta, P0, inp["cache_indices"],
                              inp["cu_seqlens"])
    Dk = inp["q"].shape[-1]
    nrm = lambda x: x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)
    cu, ci = inp["cu_seqlens"], inp["cache_indices"]
    for s in range(len(lengths)):
        S = P0[ci[s]][None]
        for t in range(cu[s], cu[s + 1]):
            S, ys = oracle.gdn_step(S, (Dk ** -0.5) * nrm(inp["q"][t])[None], nrm(inp["k"][t])[None],
                                    inp["v"][t][None], g[t][None], beta[t][None])
            np.testing.assert_allclose(y[t], ys[0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(P[ci[s]], S[0], rtol=1e-13, atol=1e-14)


def test_prefill_decay_only():
    """beta = 0: S_T = exp(sum g) S_0 and y_t = exp(G_t) S_0 q^_t."""
    rng = np.random.default_rng(10)
    inp, g, beta, P0 = _prefill_case(rng, [7])
    P, y = oracle.gdn_prefill(inp["q"], inp["k"], inp["v"], g, np.zeros_like(beta), P0,
                              inp["cache_indices"], inp["cu_seqlens"])
    slot = inp["cache_indices"][0]
    G = np.cumsum(g, axis=0)                          # [T, Hv]
    np.testing.assert_allclose(P[slot], np.exp(G[-1])[:, None, None] * P0[slot], rtol=1e-13)
    Dk = inp["q"].shape[-1]
    q64 = inp["q"].astype(np.float64)
    qn = q64 / np.sqrt(np.sum(q64 ** 2, -1, keepdims=True) + 1e-6) * Dk ** -0.5
    hk = np.arange(4) // 2
    for t in range(7):
        ref = np.exp(G[t])[:, None] * np.einsum("hji,hi->hj", P0[slot], qn[t, hk])
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-13)


def test_prefill_orthonormal_keys_closed_form():
    """beta = 1, no decay, orthonormal keys, no L2 norm:
    S_T (key-major) = (I - sum k k^T) S_0 + sum k v^T."""
    rng = np.random.default_rng(11)
    Dk, Dv, T = 16, 8, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm[:, :T].T[:, None, :]                      # [T,1,Dk] orthonormal rows
    q = rng.standard_normal((T, 1, Dk))
    v = rng.standard_normal((T, 1, Dv))
    S0 = _rand_state(rng, 1, 1, Dv, Dk)
    P, _ = oracle.gdn_prefill(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), S0, [0], [0, T],
                              scale=1.0, l2norm=False)
    Kt = k[:, 0, :]
    ref = S0[0, 0].T
    ref = (np.eye(Dk) - Kt.T @ Kt) @ ref + Kt.T @ v[:, 0, :]
    np.testing.assert_allclose(P[0, 0], ref.T, rtol=1e-12, atol=1e-13)


def test_prefill_index_handling():
    """Unreferenced slots are bitwise untouched; zero-length sequences are no-ops;
    the order of sequences in the packed batch does not change any result."""
    rng = np.random.default_rng(12)
    lengths = [4, 0, 6]
    inp, g, beta, P0 = _prefill_case(rng, lengths, pool=6)
    ci, cu = inp["cache_indices"], inp["cu_seqlens"]
    P, y = oracle.gdn_prefill(inp["q"], inp["k"], inp["v"], g, beta, P0, ci, cu)
    untouched = [s for s in range(6) if s not in (ci[0], ci[2])]
    for s in untouched:
        assert np.array_equal(P[s], P0[s])
    # reverse the packed order of the three sequences
    order = [2, 1, 0]
    segs = [np.arange(cu[s], cu[s + 1]) for s in order]
    perm = np.concatenate(segs)
    cu2 = synth.cu_from_lengths([lengths[s] for s in order])
    P2, y2 = oracle.gdn_prefill(inp["q"][perm], inp["k"][perm], inp["v"][perm], g[perm], beta[perm],
                                P0, ci[order], cu2)
    assert np.array_equal(P2, P)
    assert np.array_equal(y2, y[perm])


def test_prefill_rejects_bad_indices():
    z = np.zeros
    with pytest.raises(ValueError):
        oracle.gdn_prefill(z((2, 1, 4)), z((2, 1, 4)), z((2, 1, 4)), z((2, 1)), z((2, 1)),
                           z((2, 1, 4, 4)), [2], [0, 2])
    with pytest.raises(ValueError):
        oracle.gdn_prefill(z((2, 1, 4)), z((2, 1, 4)), z((2, 1, 4)), z((2, 1)), z((2, 1)),
                           z((2, 1, 4, 4)), [0], [0, 3])


# ------------------------------------------------- chunked algebra, brute force


def _one_head_case(rng, T, Dk=8, Dv=5):
    Q = rng.standard_normal((T, Dk))
    K = _unit(rng, T, Dk)
    V = rng.standard_normal((T, Dv))
    g = np.log(rng.uniform(0.5, 1.0, size=T))
    beta = rng.uniform(0.1, 1.0, size=T)
    S0 = _rand_state(rng, Dv, Dk)
    return S0, Q, K, V, g, beta


def _token_head(S0, Q, K, V, g, beta):
    T, Dk = Q.shape
    P, y = oracle.gdn_prefill(Q[:, None], K[:, None], V[:, None], g[:, None], beta[:, None],
                              S0[None, None], [0], [0, T], scale=1.0, l2norm=False)
    return y[:, 0], P[0, 0]


@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("form", ["ratio", "page"])
def test_chunked_forms_match_the_token_recurrence(chunk, form):
    rng = np.random.default_rng(100 + chunk)
    S0, Q, K, V, g, beta = _one_head_case(rng, T=19)   # 19: a ragged last chunk
    y_ref, S_ref = _token_head(S0, Q, K, V, g, beta)
    O, S = wy.chunked_head(S0, Q, K, V, g, beta, chunk, form=form)
    np.testing.assert_allclose(O, y_ref, rtol=0, atol=1e-12 * np.abs(y_ref).max())
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12 * np.abs(S_ref).max())


def test_printed_w_recursion_fails_from_three_tokens():
    """Taken literally, the page's w line only agrees for chunks of <= 2 tokens."""
    rng = np.random.default_rng(200)
    S0, Q, K, V, g, beta = _one_head_case(rng, T=6)
    y_ref, S_ref = _token_head(S0, Q, K, V, g, beta)
    O2, S2 = wy.chunked_head(S0, Q, K, V, g, beta, 2, form="page", printed_w=True)
    assert np.max(np.abs(S2 - S_ref)) < 1e-12
    O6, S6 = wy.chunked_head(S0, Q, K, V, g, beta, 6, form="page", printed_w=True)
    assert np.max(np.abs(S6 - S_ref)) > 1e-3


# ---------------------------------------- layer prologue: conv1d (4 taps) + SiLU


def _silu(x):
    return x / (1.0 + np.exp(-x))


def test_conv_impulse_response_reads_taps_oldest_first():
    """A unit impulse at a sequence's first token, zero history: the
    pre-activation at token t is the weight of the tap t steps back, i.e.
    W[c][3 - t] (tap 3 = current token), and zero from t = 4 on."""
    rng = np.random.default_rng(3)
    T, C = 7, 5
    W = rng.standard_normal((C, 4))
    x = np.zeros((T, C))
    x[0, :] = 1.0
    out, hist = oracle.conv_silu(x, W, np.zeros((1, C, 3)), [0], [0, T])
    for t in range(4):
        np.testing.assert_allclose(out[t], _silu(W[:, 3 - t]), rtol=0, atol=1e-15)
    assert np.all(out[4:] == 0.0)
    assert np.all(hist[0] == 0.0)  # the impulse left the 3-token window


def test_conv_oldest_tap_reads_history_then_inputs():
    """W = (1, 0, 0, 0): out[t] = SiLU(x[t - 3]), the first three coming from
    the slot's history in order hist[0], hist[1], hist[2]."""
    rng = np.random.default_rng(4)
    T, C = 6, 3
    W = np.zeros((C, 4))
    W[:, 0] = 1.0
    x = rng.standard_normal((T, C))
    h0 = rng.standard_normal((2, C, 3))
    out, hist = oracle.conv_silu(x, W, h0, [1], [0, T])
    for t in range(3):
        np.testing.assert_allclose(out[t], _silu(h0[1, :, t]), rtol=1e-15)
    for t in range(3, T):
        np.testing.assert_allclose(out[t], _silu(x[t - 3]), rtol=1e-15)
    np.testing.assert_array_equal(hist[1], x[T - 3:].T)  # newest three inputs, oldest first
    np.testing.assert_array_equal(hist[0], h0[0])         # another slot: untouched


def test_conv_identity_tap_is_silu():
    rng = np.random.default_rng(5)
    T, C = 9, 4
    W = np.zeros((C, 4))
    W[:, 3] = 1.0
    x = 4.0 * rng.standard_normal((T, C))
    out, _ = oracle.conv_silu(x, W, rng.standard_normal((1, C, 3)), [0], [0, T])
    np.testing.assert_allclose(out, x * (1.0 / (1.0 + np.exp(-x))), rtol=1e-14)
    # SiLU special values
    o0, _ = oracle.conv_silu(np.zeros((1, 1)), np.array([[0, 0, 0, 1.0]]), np.zeros((1, 1, 3)), [0], [0, 1])
    assert o0[0, 0] == 0.0


@pytest.mark.parametrize("L", [0, 1, 2, 3, 5])
def test_conv_history_after_short_sequences(L):
    """The new history is the newest three of (old history, inputs)."""
    rng = np.random.default_rng(6 + L)
    C = 4
    W = rng.standard_normal((C, 4))
    x = rng.standard_normal((max(L, 1), C))[:L]
    h0 = rng.standard_normal((1, C, 3))
    _, hist = oracle.conv_silu(x.reshape(L, C), W, h0, [0], [0, L])
    expect = np.concatenate([h0[0], x.T], axis=1)[:, -3:]
    np.testing.assert_array_equal(hist[0], expect)


def test_conv_split_sequence_equals_whole():
    """Brute force: a sequence run in two calls, the history carried through
    the pool slot, gives the same outputs and final history as one call."""
    rng = np.random.default_rng(8)
    T, C = 11, 6
    W = rng.standard_normal((C, 4))
    x = rng.standard_normal((T, C))
    h0 = rng.standard_normal((3, C, 3))
    whole, hw = oracle.conv_silu(x, W, h0, [2], [0, T])
    for a in (1, 2, 3, 7):
        first, h1 = oracle.conv_silu(x[:a], W, h0, [2], [0, a])
        second, h2 = oracle.conv_silu(x[a:], W, h1, [2], [0, T - a])
        np.testing.assert_array_equal(np.concatenate([first, second]), whole)
        np.testing.assert_array_equal(h2, hw)


def test_conv_varlen_packing_matches_separate_calls():
    """Packed sequences with their own slots equal one call per sequence."""
    rng = np.random.default_rng(9)
    lens, slots, C = [4, 0, 1, 6], [3, 0, 1, 2], 5
    cu = np.concatenate([[0], np.cumsum(lens)])
    W = rng.standard_normal((C, 4))
    x = rng.standard_normal((cu[-1], C))
    h0 = rng.standard_normal((5, C, 3))
    out, hist = oracle.conv_silu(x, W, h0, slots, cu)
    ref_h = h0.copy()
    for s, L in enumerate(lens):
        o_s, h_s = oracle.conv_silu(x[cu[s]:cu[s + 1]], W, ref_h, [slots[s]], [0, L])
        np.testing.assert_array_equal(out[cu[s]:cu[s + 1]], o_s)
        ref_h = h_s
    np.testing.assert_array_equal(hist, ref_h)
    np.testing.assert_array_equal(hist[0], h0[0])  # zero-length sequence: slot untouched
    np.testing.assert_array_equal(hist[4], h0[4])  # slot nobody uses


# ---------------------------------------------- layer epilogue: gated RMS norm


def test_gated_rmsnorm_worked_example():
    """By hand: o = (3, 4) has mean square 12.5; with gamma = (1, 2) and
    z = (0, ln 3) (sigmoid 1/2 and 3/4), eps = 0:
    y = (3 * 0.5, 4 * 2 * 0.75) / sqrt(12.5)."""
    y = oracle.gated_rmsnorm(np.array([[[3.0, 4.0]]]), np.array([[[0.0, np.log(3.0)]]]),
                             np.array([1.0, 2.0]), eps=0.0)
    np.testing.assert_allclose(y[0, 0], [1.5 / np.sqrt(12.5), 6.0 / np.sqrt(12.5)], rtol=1e-15)


def test_gated_rmsnorm_unit_rms_and_scale_invariance():
    """With eps = 0, gamma = 1 and a saturated gate the output has unit RMS
    per (token, head) and is invariant to scaling o by c > 0 (odd in c)."""
    rng = np.random.default_rng(10)
    o = rng.standard_normal((3, 4, 32))
    z = np.full(o.shape, 60.0)  # sigmoid(60) = 1 in double
    y = oracle.gated_rmsnorm(o, z, np.ones(32), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * o, z, np.ones(32), eps=0.0), y, rtol=1e-14)
    np.testing.assert_allclose(oracle.gated_rmsnorm(-2.0 * o, z, np.ones(32), eps=0.0), -y, rtol=1e-14)


def test_gated_rmsnorm_gate_and_eps():
    """gamma and sigmoid(z) multiply column-wise; eps enters the mean square
    (a zero row stays zero)."""
    rng = np.random.default_rng(11)
    o = rng.standard_normal((2, 3, 16))
    z = rng.standard_normal(o.shape)
    gam = rng.standard_normal(16)
    eps = 0.25
    y = oracle.gated_rmsnorm(o, z, gam, eps=eps)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    np.testing.assert_allclose(y, o / np.sqrt(ms + eps) * gam / (1.0 + np.exp(-z)), rtol=1e-13)
    y0 = oracle.gated_rmsnorm(np.zeros((1, 1, 8)), np.zeros((1, 1, 8)), np.ones(8), eps=1e-6)
    assert np.all(y0 == 0.0)
    # eps inside the root, beside the mean square: a row of ones with eps = 3
    # gives 1 / sqrt(1 + 3) = 1/2 exactly
    y1 = oracle.gated_rmsnorm(np.ones((1, 1, 8)), np.full((1, 1, 8), 60.0), np.ones(8), eps=3.0)
    np.testing.assert_array_equal(y1, 0.5)


# ------------------------------------------------ multi-token decode windows


def _window_inputs(rng, B, T, Hk, Hv, Dk, Dv):
    toks = [synth.decode_token(rng, B, Hk, Hv, Dk, Dv, act="f32") for _ in range(T)]
    return {n: np.stack([t[n] for t in toks], axis=1) for n in toks[0]}


def test_window_verify_keeps_the_state_and_commit_prefixes():
    """A verify window (commit 0) returns the input state and the same
    outputs as a committed one; committing after k tokens gives the state of
    a k-token window; outputs are causal (a token's y is the same in every
    window that contains it)."""
    rng = np.random.default_rng(12)
    B, T, Hk, Hv, Dk, Dv = 2, 5, 1, 2, 32, 16
    S0 = 0.3 * rng.standard_normal((B, Hv, Dv, Dk))
    w = _window_inputs(rng, B, T, Hk, Hv, Dk, Dv)
    S_all, y_all = oracle.gdn_window(S0, w["q"], w["k"], w["v"], w["g"], w["beta"])
    S_ver, y_ver = oracle.gdn_window(S0, w["q"], w["k"], w["v"], w["g"], w["beta"], commit=0)
    np.testing.assert_array_equal(S_ver, S0)
    np.testing.assert_array_equal(y_ver, y_all)
    for kk in range(1, T + 1):
        S_k, y_k = oracle.gdn_window(S0, *(w[n][:, :kk] for n in ("q", "k", "v", "g", "beta")))
        S_c, _ = oracle.gdn_window(S0, w["q"], w["k"], w["v"], w["g"], w["beta"], commit=kk)
        np.testing.assert_array_equal(S_c, S_k)
        np.testing.assert_array_equal(y_k, y_all[:, :kk])
    assert not np.allclose(S_all, S0)


def test_window_closed_form_unit_keys():
    """beta = 1, log-gate 0 and orthonormal keys across the window: token t
    overwrites the state along k_t with v_t, so after the window S k_t = v_t
    for every t, and y_t = S_t q_t with S_t built the same way."""
    rng = np.random.default_rng(13)
    B, T, Hk, Hv, Dk, Dv = 1, 4, 1, 1, 16, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm[:, :T].T.reshape(B, T, Hk, Dk)
    v = rng.standard_normal((B, T, Hv, Dv))
    q = rng.standard_normal((B, T, Hk, Dk))
    S0 = rng.standard_normal((B, Hv, Dv, Dk))
    S, y = oracle.gdn_window(S0, q, k, v, np.zeros((B, T, Hv)), np.ones((B, T, Hv)))
    for t in range(T):
        np.testing.assert_allclose(S[0, 0] @ k[0, t, 0], v[0, t, 0], atol=1e-12)
    # the state after t tokens: S0 with its component along k_0..k_t replaced
    St = S0[0, 0].copy()
    for t in range(T):
        kt = k[0, t, 0]
        St = St - np.outer(St @ kt, kt) + np.outer(v[0, t, 0], kt)
        np.testing.assert_allclose(y[0, t, 0], St @ q[0, t, 0], atol=1e-12)


# ------------------------------------------------------------ comba prefill


def test_comba_prefill_with_p_equal_k_is_the_gdn_prefill():
    """Reading with p = k makes the Comba forward the (unnormalised) gated
    delta-rule prefill on the transposed pool with q pre-scaled: two
    independently written oracle functions, including their varlen plumbing."""
    rng = np.random.default_rng(61)
    lengths, H, K, V, P = [6, 0, 9, 1], 3, 16, 8, 6
    inp = synth.comba_prefill_inputs(rng, lengths, H, K, V, P, act="f32")
    P0 = _rand_state(rng, P, H, K, V)
    sc = 0.29
    Pc, oc = oracle.comba_prefill(inp["q"], inp["k"], inp["v"], inp["k"], inp["beta"], inp["g"], P0,
                                  inp["cache_indices"], inp["cu_seqlens"], scale=sc)
    Pg, yg = oracle.gdn_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                np.swapaxes(P0, -1, -2), inp["cache_indices"], inp["cu_seqlens"],
                                scale=sc, l2norm=False)
    np.testing.assert_allclose(Pc, np.swapaxes(Pg, -1, -2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oc, yg, rtol=1e-11, atol=1e-12)


def test_comba_prefill_one_hot_keys_closed_form():
    """Zero state, read key e0 then e1... worked by hand: token 1 writes row a1
    with u1 = beta1 v1; token 2 decays it by alpha2, reads row b2 and writes
    u2 = beta2 (v2 - [b2 == a1] alpha2 beta1 v1) into row a2.  The read and
    write roles are distinguishable: swapping p and k changes the result."""
    K, V, s = 4, 3, 0.5
    rng = np.random.default_rng(62)
    v = rng.standard_normal((2, 1, V))
    q = rng.standard_normal((2, 1, K))
    e = np.eye(K)
    k = np.stack([e[0], e[1]])[:, None, :]     # write rows 0 then 1
    p = np.stack([e[2], e[0]])[:, None, :]     # read row 2 (empty) then row 0
    beta = np.array([[0.8], [0.6]])
    g = np.array([[-0.3], [-0.7]])
    a1, a2 = np.exp(g[0, 0]), np.exp(g[1, 0])
    u1 = 0.8 * v[0, 0]
    row0 = a2 * u1
    u2 = 0.6 * (v[1, 0] - row0)
    ref = np.zeros((K, V))
    ref[0], ref[1] = row0, u2
    # an explicit query scale, and the spec's default K^-1/2 when none is given
    for arg, sc in ((s, s), (None, K ** -0.5)):
        P, o = oracle.comba_prefill(q, k, v, p, beta, g, np.zeros((1, 1, K, V)), [0], [0, 2], scale=arg)
        np.testing.assert_allclose(P[0, 0], ref, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(o[0, 0], sc * q[0, 0, 0] * u1, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(o[1, 0], sc * (q[1, 0, 0] * row0 + q[1, 0, 1] * u2), rtol=1e-14, atol=1e-15)
    Pswap, _ = oracle.comba_prefill(q, p, v, k, beta, g, np.zeros((1, 1, K, V)), [0], [0, 2], scale=s)
    assert not np.allclose(Pswap, ref)


def test_comba_prefill_split_and_index_handling():
    """Running a sequence in two calls equals one call; unnamed slots are
    bitwise untouched; zero-length sequences are no-ops."""
    rng = np.random.default_rng(63)
    H, K, V, P = 2, 8, 8, 5
    inp = synth.comba_prefill_inputs(rng, [7, 0, 3], H, K, V, P, act="f32")
    P0 = _rand_state(rng, P, H, K, V)
    ci, cu = inp["cache_indices"], inp["cu_seqlens"]
    args = [inp[n] for n in ("q", "k", "v", "p", "beta", "g")]
    Pw, ow = oracle.comba_prefill(*args, P0, ci, cu)
    for slot in set(range(P)) - {int(ci[0]), int(ci[2])}:
        assert np.array_equal(Pw[slot], P0[slot])
    # first sequence split after 4 tokens
    first = [a[:4] for a in args]
    rest = [np.concatenate([a[4:7], a[7:]]) for a in args]
    P1, o1 = oracle.comba_prefill(*first, P0, ci[:1], [0, 4])
    P2, o2 = oracle.comba_prefill(*rest, P1, ci, [0, 3, 3, 6])
    np.testing.assert_array_equal(P2, Pw)
    np.testing.assert_array_equal(np.concatenate([o1, o2]), ow)


def test_comba_prefill_rejects_bad_indices():
    z = np.zeros((2, 1, 4))
    zz = np.zeros((2, 1))
    with pytest.raises(ValueError):
        oracle.comba_prefill(z, z, z, z, zz, zz, np.zeros((2, 1, 4, 4)), [0, 0], [0, 1, 2])
    with pytest.raises(ValueError):
        oracle.comba_prefill(z, z, z, z, zz, zz, np.zeros((2, 1, 4, 4)), [2], [0, 2])
    with pytest.raises(ValueError):
        oracle.comba_prefill(z, z, z, z, zz, zz, np.zeros((2, 1, 4, 4)), [0], [0, 1])
