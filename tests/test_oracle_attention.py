"""Pins for the oracle's attention over recalled tokens (oracle/attention.py).

* a hand-worked golden example of softmax(q K^T / sqrt(d)) V (§3.1);
* with every clustered token recalled, sparse decode equals full attention,
  checked against torch's float64 scaled_dot_product_attention (a library
  routine) on the tokens in their original order;
* a single attended row returns its value; q = 0 returns the mean value;
  the result is invariant to the order of the rows and to a common shift of
  the scores; an empty set returns zeros.
"""

import json
import os

import numpy as np
import torch

from oracle import attention, bf16, kmeans, pipeline
from synth import make_unit_inputs, make_init_indices


def test_golden_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attention_tiny.json")))
    out = attention.attend(np.array(g["q_heads"]), np.array(g["keys"], float),
                           np.array(g["values"], float))
    assert np.allclose(out, np.array(g["out"], float), rtol=0, atol=1e-12)


def test_full_budget_equals_sdpa():
    n, n_sink, k = 300, 16, 7
    kb, vb, cen = make_unit_inputs(5, 0, n, 8)
    init = make_init_indices(6, 1, n - n_sink, k)[0]
    st = pipeline.prefill_unit(kb, n, init, k, 3, n_sink=n_sink, v_bits=vb)
    rng = np.random.default_rng(0)
    q = bf16.round_rne(cen[rng.integers(0, 8, 4)] + rng.standard_normal((4, 128)))
    sel = pipeline.select_unit(q, st["cmean"], st["csize"], st["offsets"], st["k_clu_bits"], 10 ** 6)
    assert len(sel["positions"]) == n - n_sink
    out = pipeline.decode_unit(q, kb, vb, st["k_clu_bits"], st["v_clu_bits"], sel["positions"],
                               n_sink, n, n)
    Q = torch.from_numpy(bf16.widen(q))[None, :, None, :]          # [1, G, 1, d]
    K = torch.from_numpy(bf16.widen(kb[:n]))[None, None].expand(1, 4, n, 128)
    V = torch.from_numpy(bf16.widen(vb[:n]))[None, None].expand(1, 4, n, 128)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[0, :, 0].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((10, 16))
    V = rng.standard_normal((10, 16))
    q = rng.standard_normal((3, 16))
    assert np.allclose(attention.attend(q, K[:1], V[:1]), np.repeat(V[:1], 3, 0))
    assert np.allclose(attention.attend(np.zeros((2, 16)), K, V), np.repeat(V.mean(0, keepdims=True), 2, 0))
    p = rng.permutation(10)
    assert np.allclose(attention.attend(q, K[p], V[p]), attention.attend(q, K, V))
    w = rng.standard_normal(16)
    q1 = q[:1]
    # adding w to every key shifts q1's scores by the same constant q1.w
    assert np.allclose(attention.attend(q1, K + w, V), attention.attend(q1, K, V))
    assert np.array_equal(attention.attend(q, K[:0], V[:0]), np.zeros((3, 16)))


def test_attended_set_composition():
    k_tok = np.arange(10 * 2, dtype=float).reshape(10, 2)
    k_clu = -np.arange(8 * 2, dtype=float).reshape(8, 2)
    K, V = attention.attended_rows(k_tok, k_tok, k_clu, k_clu, [1, 5], 2, 7, 9)
    assert K.tolist() == [k_tok[0].tolist(), k_tok[1].tolist(), k_clu[1].tolist(),
                          k_clu[5].tolist(), k_tok[7].tolist(), k_tok[8].tolist()]
