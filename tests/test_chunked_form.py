"""CPU checks of the numpy model of the chunked (WY/UT) form.

In float64 the chunked recurrence must equal the token-sequential oracle up to
rounding ("MTP inference: review and commit structure", Verification and
limits: the chunk recurrence differs from the sequential one only in
rounding).  With the bf16 operand plan of the prefill kernels, a 4,096-token
prompt at the Qwen head size must stay well within the 2e-3 normwise bound;
rounding diag(s) U once instead of splitting it leaves no margin under that
bound (that is what the split buys).
"""
import numpy as np
import pytest

import chunked_form as cf
import oracle


def _sequential(q, k, v, g, beta, H0, scale):
    """One head through the oracle's token-sequential prefill."""
    T, dk = q.shape
    dv = v.shape[1]
    d = oracle.Dims(L=1, B=1, T=T, HV=1, HK=1, DK=dk, DV=dv, scale=scale)
    y = np.concatenate([q, k, v], axis=1)[None, None]
    st, o, err = oracle.prefill(d, y, g[None, None, :, None], beta[None, None, :, None],
                                H0[None, None, None])
    assert err == 0
    return st[0, 0, 0], o[0, 0, :, 0]


def _head(rng, T, dk, dv, state_std):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    g = -np.logaddexp(0.0, rng.standard_normal(T))          # -softplus
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))    # sigmoid
    H0 = state_std * rng.standard_normal((dk, dv))
    return q, k, v, g, beta, H0


@pytest.mark.parametrize("T,dk,dv,scale", [(1, 16, 16, 1.0), (64, 32, 16, 1.0), (150, 32, 48, 0.5),
                                           (200, 64, 32, 64 ** -0.5)])
def test_fp64_chunked_equals_sequential(T, dk, dv, scale):
    rng = np.random.default_rng(7000 + T)
    q, k, v, g, beta, H0 = _head(rng, T, dk, dv, 0.1)
    H_s, O_s = _sequential(q, k, v, g, beta, H0, scale)
    H_c, O_c = cf.chunked_head(q, k, v, g, beta, H0, scale=scale)
    assert np.abs(H_c - H_s).max() <= 1e-10 * np.abs(H_s).max()
    assert np.abs(O_c - O_s).max() <= 1e-10 * np.abs(O_s).max()


def test_chunk_size_does_not_change_the_result():
    rng = np.random.default_rng(7100)
    q, k, v, g, beta, H0 = _head(rng, 130, 32, 16, 0.1)
    H1, O1 = cf.chunked_head(q, k, v, g, beta, H0, chunk=64)
    H2, O2 = cf.chunked_head(q, k, v, g, beta, H0, chunk=16)
    assert np.abs(H1 - H2).max() <= 1e-12 * np.abs(H1).max()
    assert np.abs(O1 - O2).max() <= 1e-12 * np.abs(O1).max()


def _bf16_round(x):
    return cf._bf16(np.asarray(x, np.float32)).astype(np.float64)


def test_bf16_plan_at_qwen_size_and_why_diag_s_u_is_split():
    """One head of the 4,096-token workload (d = 128, q and k unit rows and v
    rounded to bf16 like the inputs, zero start state)."""
    rng = np.random.default_rng(7200)
    T, d = 4096, 128
    q, k, v, g, beta, _ = _head(rng, T, d, d, 0.0)
    q = _bf16_round(q / np.linalg.norm(q, axis=1, keepdims=True))
    k = _bf16_round(k / np.linalg.norm(k, axis=1, keepdims=True))
    v, g, beta = _bf16_round(v), _bf16_round(g), _bf16_round(beta)
    H0 = np.zeros((d, d))
    H_s, O_s = _sequential(q, k, v, g, beta, H0, 1.0)

    def err(plan):
        H, O = cf.chunked_head(q, k, v, g, beta, H0, bf16=True, plan=plan)
        return np.abs(O - O_s).max() / np.abs(O_s).max(), np.abs(H - H_s).max() / np.abs(H_s).max()

    e_o, e_s = err(None)
    assert e_o <= 5e-4 and e_s <= 5e-5, (e_o, e_s)
    e_o1, e_s1 = err(dict(ku=("x", "b")))
    assert e_s1 >= 1e-3 and e_s1 >= 100 * e_s, (e_s1, e_s)
