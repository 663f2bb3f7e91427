"""CPU tier: the fp64 oracle against pins that the pages and mathematics fix."""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rand_head(n, d, dv, seed, key_scale=1.0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, d))
    z /= np.linalg.norm(z, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv))
    aff = {k: (1.0 if k.startswith(("kappa", "eta")) else 0.0) + 0.3 * rng.standard_normal(d)
           for k in ("kappa_q", "nu_q", "kappa_k", "nu_k", "eta_q", "rho_q", "eta_k", "rho_k")}
    # make logits and memory keys O(1) so softmax is not flat
    for k in ("kappa_q", "kappa_k", "eta_q", "eta_k"):
        aff[k] = aff[k] * key_scale
    return z, v, aff


SHAPES = [(1, 1), (5, 1), (17, 3), (64, 16), (100, 16), (130, 64), (40, 40), (40, 80), (257, 64)]


@pytest.mark.parametrize("n,c", SHAPES)
def test_sca_matches_brute_force(n, c):
    z, v, a = rand_head(n, 8, 5, seed=n * 31 + c, key_scale=3.0)
    got = oracle.sca_head(z, v, a["kappa_q"], a["nu_q"], a["kappa_k"], a["nu_k"], c)
    q = z * a["kappa_q"] + a["nu_q"]
    k = z * a["kappa_k"] + a["nu_k"]
    want = pins.brute_sca(q, k, v, c)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,c", [(1, 1), (33, 33), (50, 64), (64, 1000)])
def test_sca_one_chunk_is_causal_attention(n, c):
    z, v, a = rand_head(n, 16, 7, seed=n + c, key_scale=4.0)
    got = oracle.sca_head(z, v, a["kappa_q"], a["nu_q"], a["kappa_k"], a["nu_k"], c)
    q = z * a["kappa_q"] + a["nu_q"]
    k = z * a["kappa_k"] + a["nu_k"]
    np.testing.assert_allclose(got, pins.causal_attention_torch(q, k, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,c", [(7, 1), (100, 16), (257, 64), (64, 64), (300, 7)])
def test_sca_equal_logits_give_window_mean(n, c):
    z, v, a = rand_head(n, 8, 6, seed=7 * n + c)
    zero = np.zeros(8)
    got = oracle.sca_head(z, v, zero, zero, a["kappa_k"], a["nu_k"], c)
    np.testing.assert_allclose(got, pins.window_mean(v, c), rtol=1e-12, atol=1e-13)


AWM_SHAPES = [(1, 1, 3, 2), (9, 1, 2, 3), (20, 3, 4, 5), (37, 4, 5, 3), (48, 16, 8, 12), (60, 7, 6, 6), (45, 5, 1, 2)]


@pytest.mark.parametrize("n,c,d,dv", AWM_SHAPES)
def test_awm_matches_unrolled_transition_products(n, c, d, dv):
    z, v, a = rand_head(n, d, dv, seed=n * 7 + c * 3 + d, key_scale=2.0)
    got = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c)
    qm = z * a["eta_q"] + a["rho_q"]
    km = z * a["eta_k"] + a["rho_k"]
    np.testing.assert_allclose(got, pins.awm_unrolled(qm, km, v, c), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("n,c,d,dv", AWM_SHAPES)
def test_awm_no_delta_is_online_softmax_linear_attention(n, c, d, dv):
    z, v, a = rand_head(n, d, dv, seed=n + 5 * c + d, key_scale=2.0)
    got = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c, no_delta=True)
    qm = z * a["eta_q"] + a["rho_q"]
    km = z * a["eta_k"] + a["rho_k"]
    np.testing.assert_allclose(got, pins.awm_no_delta_closed(qm, km, v, c), rtol=1e-11, atol=1e-12)


def test_awm_no_delta_constant_values_read_back_one():
    n, c, d = 90, 10, 6
    z, _, a = rand_head(n, d, 1, seed=3, key_scale=5.0)
    v = np.ones((n, 4))
    got = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c, no_delta=True)
    assert np.all(got[: 2 * c] == 0.0)
    np.testing.assert_allclose(got[2 * c:], 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,c", [(10, 1), (64, 8), (70, 8), (33, 5)])
def test_awm_constant_keys_closed_form(n, c):
    d, dv = 5, 4
    z, v, a = rand_head(n, d, dv, seed=n * c)
    zero = np.zeros(d)
    got = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], zero, a["rho_k"], c)
    np.testing.assert_allclose(got, pins.awm_const_key_closed(v, c), rtol=1e-11, atol=1e-12)


def test_online_softmax_normaliser_is_one():
    """tau^s = sum over all tokens up to chunk s of phi^s = 1 per feature, and
    psi(Q_m) tau = 1 for every query row."""
    n, c, d, dv = 53, 6, 7, 3
    z, v, a = rand_head(n, d, dv, seed=11, key_scale=3.0)
    trace = []
    oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c, trace=trace)
    km = z * a["eta_k"] + a["rho_k"]
    qm = z * a["eta_q"] + a["rho_q"]
    for t in trace:
        end = min(t["s"] * c, n)
        tau = (np.exp(km[:end]) / t["z"]).sum(axis=0)
        np.testing.assert_allclose(tau, 1.0, rtol=0, atol=1e-12)
        psi = oracle.feature_softmax(qm)
        np.testing.assert_allclose(psi @ tau, 1.0, rtol=0, atol=1e-12)
        # the phi the oracle used for chunk s is exp(K_s) / z^s
        a0 = (t["s"] - 1) * c
        np.testing.assert_allclose(t["phi"], np.exp(km[a0:end]) / t["z"], rtol=1e-14)


def test_memory_starts_empty():
    n, c = 50, 8
    z, v, a = rand_head(n, 4, 3, seed=1, key_scale=2.0)
    o = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c)
    assert np.all(o[: 2 * c] == 0.0)
    assert np.all(np.abs(o[2 * c:]).sum(axis=1) > 0)


def test_feature_softmax_reference():
    from scipy.special import softmax

    x = np.random.default_rng(0).standard_normal((9, 13)) * 30
    np.testing.assert_allclose(oracle.feature_softmax(x), softmax(x, axis=1), rtol=1e-13)


def test_chunk_ranges():
    assert oracle.chunk_ranges(10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert oracle.chunk_ranges(4, 4) == [(0, 4)]
    assert oracle.chunk_ranges(3, 10) == [(0, 3)]
    assert oracle.chunk_ranges(0, 3) == []


def test_forward_is_sum_of_parts():
    B, H, n, d, dv, c = 2, 3, 40, 4, 3, 7
    rng = np.random.default_rng(5)
    z = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, dv))
    p = {k: rng.standard_normal((H, d)) for k in
         ("kappa_q", "nu_q", "kappa_k", "nu_k", "eta_q", "rho_q", "eta_k", "rho_k")}
    r = oracle.forward(z, v, p, c)
    np.testing.assert_array_equal(r["o"], r["o_sca"] + r["o_m"])
    h = 2
    ref = oracle.sca_head(z[1, h], v[1, h], p["kappa_q"][h], p["nu_q"][h], p["kappa_k"][h], p["nu_k"][h], c)
    np.testing.assert_array_equal(r["o_sca"][1, h], ref)


# ---------------------------------------------------------------- golden

def _golden():
    with open(GOLDEN) as f:
        return {e["name"]: e for e in json.load(f)["examples"]}


def _frac(xs):
    return np.array([float(Fraction(x)) for x in xs])


def test_golden_sca_scalar_band():
    e = _golden()["sca_scalar_band"]
    k = np.log(np.array(e["exp_k"], float))[:, None]
    v = np.array(e["v"], float)[:, None]
    n = k.shape[0]
    one, zero = np.ones(1), np.zeros(1)
    # Q = 0*z + 1, K = 1*z + 0
    got = oracle.sca_head(k, v, zero, one * e["q_const"], one, zero, e["c"])
    np.testing.assert_allclose(got[:, 0], _frac(e["o_sca"]), rtol=1e-13)
    assert n == len(e["o_sca"])


def test_golden_awm_scalar():
    e = _golden()["awm_scalar_d1"]
    k = np.log(np.array(e["exp_k"], float))[:, None]
    v = np.array(e["v"], float)[:, None]
    one, zero = np.ones(1), np.zeros(1)
    got = oracle.awm_head(k, v, one, zero, one, zero, e["c"])
    np.testing.assert_allclose(got[:, 0], _frac(e["o_m"]), rtol=1e-13, atol=1e-15)
    got = oracle.awm_head(k, v, one, zero, one, zero, e["c"], no_delta=True)
    np.testing.assert_allclose(got[:, 0], _frac(e["o_m_no_delta"]), rtol=1e-13, atol=1e-15)


def test_golden_awm_d2():
    e = _golden()["awm_d2_rowwise"]
    z = np.log(np.array(e["exp_z"], float))
    v = np.array(e["v"], float)[:, None]
    one, zero = np.ones(2), np.zeros(2)
    got = oracle.awm_head(z, v, one, zero, one, zero, e["c"])
    np.testing.assert_allclose(got[:, 0], _frac(e["o_m"]), rtol=1e-13, atol=1e-15)


# ------------------------------------------------ planted mistakes are caught

def _mutant_awm(kind):
    """A copy of the memory recurrence with one plausible mistake planted."""

    def run(z, v, eta_q, rho_q, eta_k, rho_k, c):
        n, d = z.shape
        dv = v.shape[1]
        out = np.zeros((n, dv))
        zp = np.zeros(d)
        mprev = np.zeros((d, dv))
        mcur = np.zeros((d, dv))
        for s, (a, b) in enumerate(oracle.chunk_ranges(n, c), start=1):
            qm = oracle.affine(z[a:b], eta_q, rho_q)
            out[a:b] = oracle.feature_softmax(qm) @ (mcur if kind == "no_lag" else mprev)
            km = oracle.affine(z[a:b], eta_k, rho_k)
            ek = np.exp(km)
            zc = zp + ek.sum(axis=0)
            phi = ek / (zp if kind == "old_z" and s > 1 else zc)
            psi = oracle.feature_softmax(km)
            if kind == "psi_cols":
                psi = np.exp(km) / np.exp(km).sum(axis=0, keepdims=True)
            resid = v[a:b] - psi @ mcur
            if kind == "plus_delta":
                resid = v[a:b] + psi @ mcur
            ratio = (zp / zc)[:, None]
            if kind == "no_decay":
                ratio = 1.0
            mnext = ratio * mcur + phi.T @ resid
            mprev, mcur = mcur, mnext
            zp = zc
        return out

    return run


@pytest.mark.parametrize("kind", ["no_lag", "old_z", "psi_cols", "plus_delta", "no_decay"])
def test_pins_catch_planted_awm_mistakes(kind):
    n, c, d, dv = 40, 5, 4, 3
    z, v, a = rand_head(n, d, dv, seed=2, key_scale=2.0)
    args = (z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c)
    qm = z * a["eta_q"] + a["rho_q"]
    km = z * a["eta_k"] + a["rho_k"]
    want = pins.awm_unrolled(qm, km, v, c)
    np.testing.assert_allclose(_mutant_awm("none")(*args), want, rtol=1e-11, atol=1e-12)
    assert np.max(np.abs(_mutant_awm(kind)(*args) - want)) > 1e-3


@pytest.mark.parametrize("kind", ["two_prev", "no_prev", "strict_causal", "scaled"])
def test_pins_catch_planted_sca_mistakes(kind):
    n, c = 70, 8
    z, v, a = rand_head(n, 6, 4, seed=9, key_scale=3.0)
    q = z * a["kappa_q"] + a["nu_q"]
    k = z * a["kappa_k"] + a["nu_k"]
    out = np.zeros((n, 4))
    for s, (q0, q1) in enumerate(oracle.chunk_ranges(n, c)):
        k0 = {"two_prev": max(0, q0 - 2 * c), "no_prev": q0}.get(kind, max(0, q0 - c))
        qq = q[q0:q1] / (np.sqrt(6) if kind == "scaled" else 1.0)
        qp, kp = np.arange(q0, q1), np.arange(k0, q1)
        if kind == "strict_causal":
            qp = qp.copy()
            qp[1:] -= 1  # first row keeps itself so the row is not empty
        out[q0:q1] = oracle.sca_chunk(qq, k[k0:q1], v[k0:q1], qp, kp)
    assert np.max(np.abs(out - pins.brute_sca(q, k, v, c))) > 1e-3


def test_awm_readout_chunks_subset_matches_full():
    n, c = 70, 8
    z, v, a = rand_head(n, 5, 4, seed=4, key_scale=2.0)
    args = (z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c)
    full = oracle.awm_head(*args)
    part = oracle.awm_head(*args, readout_chunks=[0, 3, 8])
    assert sorted(part) == [0, 3, 8]
    for s, rows in part.items():
        np.testing.assert_array_equal(rows, full[s * c:min((s + 1) * c, n)])


STREAM_SPLITS = [
    (96, 16, [96]),                  # one segment
    (96, 16, [16, 16, 64]),          # one-chunk segments first
    (100, 16, [32, 48, 20]),         # ragged last segment
    (70, 7, [7] * 9 + [7]),          # every chunk its own segment
    (50, 10, [20, 30]),
    (41, 64, [41]),                  # one partial chunk
    (130, 64, [64, 64, 2]),          # last segment shorter than a chunk
]


def _stream(z, v, a, c, splits, no_delta=False):
    p = {k: np.asarray(x)[None, :] for k, x in a.items()}
    st = oracle.HeadStream(p, 0, c, no_delta=no_delta)
    parts, at = [], 0
    for m in splits:
        parts.append(st.push(z[at:at + m], v[at:at + m]))
        at += m
    assert at == len(z)
    return {k: np.concatenate([r[k] for r in parts]) for k in ("o_sca", "o_m", "o")}


@pytest.mark.parametrize("n,c,splits", STREAM_SPLITS)
def test_stream_matches_brute_force_and_unrolled_memory(n, c, splits):
    # the streamed rows against the independent formulations of both parts
    z, v, a = rand_head(n, 6, 5, seed=n + 11 * c + len(splits), key_scale=2.5)
    got = _stream(z, v, a, c, splits)
    q, k = z * a["kappa_q"] + a["nu_q"], z * a["kappa_k"] + a["nu_k"]
    qm, km = z * a["eta_q"] + a["rho_q"], z * a["eta_k"] + a["rho_k"]
    np.testing.assert_allclose(got["o_sca"], pins.brute_sca(q, k, v, c), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["o_m"], pins.awm_unrolled(qm, km, v, c), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("n,c,splits", STREAM_SPLITS[:4])
def test_stream_equals_one_call(n, c, splits):
    z, v, a = rand_head(n, 8, 4, seed=3 * n + c, key_scale=2.0)
    p = {k: np.asarray(x)[None, :] for k, x in a.items()}
    for no_delta in (False, True):
        want = oracle.forward_head(z, v, p, 0, c, no_delta=no_delta)
        got = _stream(z, v, a, c, splits, no_delta=no_delta)
        for key in ("o_sca", "o_m", "o"):
            np.testing.assert_allclose(got[key], want[key], rtol=1e-12, atol=1e-14)


def test_stream_rejects_a_push_after_a_partial_chunk():
    z, v, a = rand_head(40, 4, 3, seed=5)
    p = {k: np.asarray(x)[None, :] for k, x in a.items()}
    st = oracle.HeadStream(p, 0, 16)
    st.push(z[:20], v[:20])
    with pytest.raises(ValueError):
        st.push(z[20:], v[20:])


# chunk-wise variant: attention inside the chunk, memory read one chunk earlier

@pytest.mark.parametrize("n,c", SHAPES)
def test_chunkwise_sca_matches_brute_force(n, c):
    z, v, a = rand_head(n, 8, 5, seed=n * 13 + c, key_scale=3.0)
    got = oracle.sca_head(z, v, a["kappa_q"], a["nu_q"], a["kappa_k"], a["nu_k"], c, sliding=False)
    q = z * a["kappa_q"] + a["nu_q"]
    k = z * a["kappa_k"] + a["nu_k"]
    np.testing.assert_allclose(got, pins.brute_sca(q, k, v, c, prev=0), rtol=1e-12, atol=1e-12)
    zero = np.zeros(8)
    got = oracle.sca_head(z, v, zero, zero, a["kappa_k"], a["nu_k"], c, sliding=False)
    np.testing.assert_allclose(got, pins.window_mean(v, c, prev=0), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("n,c,d,dv", AWM_SHAPES)
def test_chunkwise_awm_matches_unrolled_and_no_delta_closed_form(n, c, d, dv):
    z, v, a = rand_head(n, d, dv, seed=n * 5 + c * 7 + d, key_scale=2.0)
    qm = z * a["eta_q"] + a["rho_q"]
    km = z * a["eta_k"] + a["rho_k"]
    got = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c, lag=1)
    np.testing.assert_allclose(got, pins.awm_unrolled(qm, km, v, c, lag=1), rtol=1e-11, atol=1e-12)
    got = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c, no_delta=True, lag=1)
    np.testing.assert_allclose(got, pins.awm_no_delta_closed(qm, km, v, c, lag=1), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("n,c", [(10, 1), (64, 8), (70, 8), (33, 5)])
def test_chunkwise_awm_constant_keys_closed_form(n, c):
    d, dv = 5, 4
    z, v, a = rand_head(n, d, dv, seed=n * c + 1)
    zero = np.zeros(d)
    got = oracle.awm_head(z, v, a["eta_q"], a["rho_q"], zero, a["rho_k"], c, lag=1)
    np.testing.assert_allclose(got, pins.awm_const_key_closed(v, c, lag=1), rtol=1e-11, atol=1e-12)
    # the first chunk reads nothing, the second reads the first chunk's mean
    assert np.all(got[:c] == 0.0)
    np.testing.assert_allclose(got[c:2 * c], np.broadcast_to(v[:c].mean(axis=0), got[c:2 * c].shape), rtol=1e-12)


def test_chunkwise_is_the_sliding_memory_one_chunk_earlier():
    # reading one chunk earlier: the variant's chunk s equals the sliding
    # form's chunk s + 1 readout when both use the same state (same queries)
    n, c, d, dv = 60, 6, 4, 3
    z, v, a = rand_head(n, d, dv, seed=21, key_scale=2.0)
    tr1, tr2 = [], []
    oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c, lag=1, trace=tr1)
    oracle.awm_head(z, v, a["eta_q"], a["rho_q"], a["eta_k"], a["rho_k"], c, lag=2, trace=tr2)
    for s in range(1, len(tr1)):
        np.testing.assert_array_equal(tr1[s - 1]["mem_read"], tr2[s]["mem_read"])


@pytest.mark.parametrize("splits", [[40], [8, 16, 16], [24, 8, 5]])
def test_const_key_stream_closed_form_matches_one_shot(splits):
    # the segment-by-segment closed forms (used at 16M tokens on the GPU) equal
    # the one-shot ones over the whole sequence
    c = 4
    v = np.random.default_rng(9).standard_normal((sum(splits), 3))
    want = pins.window_mean(v, c) + pins.awm_const_key_closed(v, c)
    ref = pins.ConstKeyStream(c)
    got, at = [], 0
    for m in splits:
        got += list(ref.push(v[at:at + m]))
        at += m
    np.testing.assert_allclose(np.concatenate(got), want, rtol=1e-12, atol=1e-13)
