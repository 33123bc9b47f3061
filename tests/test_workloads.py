"""The seeded input generators: layout, determinism, rounding and recipes."""
import numpy as np
import pytest
from scipy import stats

import workloads as W


def test_bf16_rounding_is_single_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 5,
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 255.5,
                         1 + 2 ** -8 + 2 ** -40, 0.0, -0.0]])
    bits = W.round_to_bf16_bits(x)
    back = W.bf16_bits_to_f64(bits)
    # nearest: no bf16 value (8 significant bits) is closer
    m, e = np.frexp(x)
    ulp = np.ldexp(1.0, e - 8)
    assert (np.abs(back - x) <= ulp / 2).all()
    # ties go to the even mantissa
    assert W.bf16_bits_to_f64(W.round_to_bf16_bits(np.array([1 + 2 ** -8])))[0] == 1.0
    assert W.bf16_bits_to_f64(W.round_to_bf16_bits(np.array([1 + 3 * 2 ** -8])))[0] == 1 + 2 ** -6
    assert W.round_to_bf16_bits(np.array([-np.inf]))[0] == 0xFF80


def test_packed_layout_and_determinism():
    gam = [0, 3, 1, 0, 5]
    a = W.build("t", 9, gam, 300, W.BF16, 0.8, W.iid_normal_rows(2.0), 1.0)
    b = W.build("t", 9, gam, 300, W.BF16, 0.8, W.iid_normal_rows(2.0), 1.0,
                workers=1)
    for f in ("cu_draft", "target_logits", "draft_logits", "draft_tokens", "uniforms"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.cu_draft.tolist() == [0, 0, 3, 4, 4, 9]
    assert a.target_logits.shape == (9 + 5, 300) and a.draft_logits.shape == (9, 300)
    assert a.target_row(2, 1) == 3 + 2 + 1
    assert a.target_row(4, 5) == 4 + 4 + 5
    assert a.draft_row(4, 4) == 8
    u = a.uniforms.astype(np.float64) * 2 ** 24
    assert (u == np.floor(u)).all() and (a.uniforms >= 0).all() and (a.uniforms < 1).all()
    assert a.temperature == float(np.float32(0.8))


def test_draft_tokens_follow_q():
    """Gumbel-max draws follow softmax(l / T): chi-square on one fixed row."""
    rng = np.random.default_rng(4)
    l = rng.standard_normal(8) * 1.5
    T = 0.7
    counts = np.bincount([W.gumbel_max_token(l, T, rng) for _ in range(40000)],
                         minlength=8)
    q = np.exp(l / T - (l / T).max())
    q /= q.sum()
    assert stats.chisquare(counts, 40000 * q).pvalue > 1e-4


@pytest.mark.parametrize("idx", [1, 2])
def test_small_named_configs(idx):
    c = W.config(idx)
    s = W.CONFIG_SHAPES[idx]
    assert c.num_seqs == s["B"] and c.vocab == s["V"] and c.dtype == s["dtype"]
    assert (c.gammas == s["gamma"]).all()
    assert c.target_rows == s["B"] * (s["gamma"] + 1)
    assert ((c.draft_tokens >= 0) & (c.draft_tokens < c.vocab)).all()


def test_heavy_tail_recipe_reduced():
    c = W.config(3, num_seqs=2, vocab=4096)
    t = W.to_f64(c.target_logits, c.dtype)
    # the 50 largest per row sit about 6 above the N(0, 4) bulk
    top = np.sort(t, axis=1)[:, -50:]
    assert (top.mean(axis=1) > 10).all()
    c5 = W.config(5, num_seqs=4, vocab=512)
    for b in range(2):
        for i in range(4):
            np.testing.assert_array_equal(c5.draft_logits[c5.draft_row(b, i)],
                                          c5.target_logits[c5.target_row(b, i)])
    assert (c5.draft_logits[c5.draft_row(3, 0)] != c5.target_logits[c5.target_row(3, 0)]).any()
    c4 = W.config(4, num_seqs=64, vocab=256)
    assert set(np.unique(c4.gammas)) <= set(range(9)) and (c4.gammas == 0).any()
