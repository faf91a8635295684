"""Pins of oracle.pipeline: reconstruction identity, the half-scale bound per
stage, the progressive infinity-norm bound, the zero-centroid (RTN) special case
and the smoothing gain on synthetic data."""
import numpy as np
import pytest

from oracle import pipeline, quant
from oracle.numerics import bf16_rne
from video_model_kv_amd import synth


@pytest.fixture(scope="module")
def tiny_k():
    wl = synth.workload(1)
    return synth.kv_chunk(wl, "K", 0)[:, 0]


def test_reconstruction_identity(tiny_k):
    res = pipeline.quantize_problem(tiny_k[:600], 16, 2, 64, iters=4)
    st = res.stages[0]
    lay = res.layout
    s = quant.expand_scales(st.scales, lay)
    rows = st.centroids_bf16[st.labels]
    # x_hat = S q + C (the dequantization of the QVG notes' overall framework)
    assert np.array_equal(st.y_hat, (s * st.q + rows).astype(np.float32))
    assert np.array_equal(res.x_hat, pipeline.dequantize_stages(res.stages, lay))
    # the stored centroid is the bf16 rounding of the k-means centroid
    assert np.array_equal(st.centroids_bf16, bf16_rne(st.centroids))
    r = (tiny_k[:600] - rows).astype(np.float64)
    assert np.all(np.abs(r - s * st.q) <= s * (0.5 + 2.0 ** -20))


def test_progressive_inf_norm_bound():
    wl = synth.workload(2, n_heads=1)
    x = synth.kv_tokens(wl, "V", 0, 1500)[:, 0]
    res = pipeline.quantize_problem(x, 32, 2, 32, n_stages=3, iters=5)
    slack = (1 + 2.0 ** -8) ** 2 * (1 + 2.0 ** -20)
    errs = []
    for st in res.stages:
        nxt = (st.y_in - st.y_hat).astype(np.float64)
        assert np.abs(nxt).max() <= np.abs(st.y_in.astype(np.float64)).max() * slack
        errs.append(np.linalg.norm(nxt))
    # the residual shrinks stage over stage on this data (reported, and checked)
    assert errs[0] > errs[1] > errs[2]
    assert np.array_equal(res.x_hat, pipeline.dequantize_stages(res.stages, res.layout))


def test_rtn_special_case_is_textbook_per_group_quantizer():
    """Zero centroids: the pipeline reduces to plain symmetric per-group RTN.
    Checked on a hand-worked token (two groups of four channels)."""
    x = np.array([[0.5, -3.0, 1.0, 2.0, 2.0, 1.0, -1.0, 0.5]], np.float32)
    x = np.repeat(x, 4, axis=0)
    res = pipeline.quantize_problem(x, 4, 2, 4, rtn=True)
    st = res.stages[0]
    assert np.all(st.centroids_bf16 == 0)
    assert st.q[0].tolist() == [0, -1, 0, 1, 1, 0, 0, 0]
    assert st.scales[0].tolist() == [3.0, 2.0]
    assert res.x_hat[0].tolist() == [0.0, -3.0, 0.0, 3.0, 2.0, 0.0, 0.0, 0.0]


def test_smoothing_beats_rtn_on_synthetic_keys(tiny_k):
    """Diagnostic (ratio is data-dependent, parity unpinned): clustering first
    must lower the key reconstruction error versus plain RTN."""
    sm = pipeline.quantize_problem(tiny_k, 64, 2, 64)
    rt = pipeline.quantize_problem(tiny_k, 64, 2, 64, rtn=True)
    e_sm = np.linalg.norm(tiny_k - sm.x_hat)
    e_rt = np.linalg.norm(tiny_k - rt.x_hat)
    assert e_rt / e_sm > 2.0


def test_mixed_precision_groups():
    wl = synth.workload(2, n_heads=1)
    x = synth.kv_tokens(wl, "K", 0, 800)[:, 0]
    perm = np.concatenate([np.arange(50, 76), np.arange(0, 50), np.arange(76, 128)])
    res = pipeline.quantize_problem(x, 16, 2, 32, iters=3, n_int4=26, perm=perm)
    st = res.stages[0]
    assert st.scales.shape == (800, 5)
    assert st.q[:, 50:76].min() >= -7 and st.q[:, 50:76].max() <= 7
    other = np.concatenate([np.arange(0, 50), np.arange(76, 128)])
    assert st.q[:, other].min() >= -1 and st.q[:, other].max() <= 1
    # int4 channels reconstruct better than int2 channels
    err = np.abs(x - res.x_hat)
    assert err[:, 50:76].mean() < err[:, other].mean()


@pytest.fixture(scope="module")
def two_stage_keys():
    wl = synth.workload(2, n_heads=1)
    x = synth.kv_tokens(wl, "K", 0, 700)[:, 0]
    return x


def test_psac_encode_uses_the_residual_after_all_stages(two_stage_keys):
    """PSAC encode (QuantWM summary, "QuantWM", second technique: the key error
    left after key quantization is projected on U).  With U = the first r unit
    vectors, coef[:, b] must be the bf16 rounding of x_b - x_hat_b, x_hat the
    sum of BOTH stages rebuilt from the stored fields.  The error of stage 1
    alone, the last stage's input, or the opposite sign all give other values,
    which the last asserts confirm on this input."""
    x = two_stage_keys
    r = 8
    u = np.eye(128)[:, :r]
    res = pipeline.quantize_problem(x, 16, 2, 32, n_stages=2, iters=4, u=u)
    x_hat = pipeline.dequantize_stages(res.stages, res.layout)
    e = x.astype(np.float64) - x_hat.astype(np.float64)     # exact: both bf16/fp32 grids fit fp64
    expect = bf16_rne(e[:, :r].astype(np.float32))          # e is fp32-exact here (one fp32 subtraction)
    assert np.array_equal(e[:, :r], (x - x_hat).astype(np.float32)[:, :r].astype(np.float64))
    assert res.coef.shape == (x.shape[0], r)
    assert np.array_equal(res.coef, expect)
    # the plausible mistakes are distinguishable on this input
    e1 = (x - res.stages[0].y_hat).astype(np.float32)[:, :r]
    y2 = res.stages[1].y_in[:, :r]
    assert not np.array_equal(bf16_rne(e1), expect)
    assert not np.array_equal(bf16_rne(y2), expect)
    assert not np.array_equal(bf16_rne(-e[:, :r].astype(np.float32)), expect)


def test_psac_full_rank_restores_exact_logits(two_stage_keys):
    """Full rank (U orthogonal, d x d): the corrected logits q.x_hat + (qU).coef
    equal q.x up to the bf16 rounding of the coefficients alone, i.e. within
    sum_b |(qU)_b| * 2^-8 |coef_b| (bf16's unit roundoff) per logit."""
    from oracle import attention
    x = two_stage_keys[:300]
    rng = np.random.default_rng(5)
    u, rm = np.linalg.qr(rng.standard_normal((128, 128)))
    u = u * np.sign(np.diag(rm))[None, :]
    res = pipeline.quantize_problem(x, 16, 2, 32, n_stages=2, iters=3, u=u)
    q = rng.standard_normal((40, 128)).astype(np.float32)
    s_corr = attention.logits(q, res.x_hat, res.coef, u, scale=1.0)
    s_true = q.astype(np.float64) @ x.astype(np.float64).T
    qu = q.astype(np.float64) @ u
    bound = np.abs(qu) @ np.abs(res.coef.astype(np.float64)).T * 2.0 ** -8 + 1e-9 * np.abs(s_true).max()
    assert np.all(np.abs(s_corr - s_true) <= bound)
    # without the correction the logits are far off (the bound is not vacuous)
    s_plain = attention.logits(q, res.x_hat, scale=1.0)
    assert np.max(np.abs(s_plain - s_true)) > 20 * np.max(bound)
