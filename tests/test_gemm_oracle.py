"""Pins for the float64 flat-GEMM oracle (C = A . W^T of the decode linear layers).

FlashDecoding++ theory page, section 2 item 2 and section 4: the linear
layers of decoding multiply a flat activation matrix (M small) by fixed
weights.  Pinned by a plain triple loop, closed forms, and torch's bf16
decoder for the operand decoding.
"""
import numpy as np
import torch

import oracle
import synthetic


def test_triple_loop():
    a, w = synthetic.make_gemm(3, 5, 7, seed=1)
    A = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    W = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().numpy()
    ref = np.zeros((3, 5))
    for i in range(3):
        for j in range(5):
            acc = 0.0
            for t in range(7):
                acc += A[i, t] * W[j, t]
            ref[i, j] = acc
    np.testing.assert_allclose(oracle.flat_gemm(a, w), ref, rtol=1e-14, atol=1e-14)


def test_identity_and_one_hot_weights():
    a, _ = synthetic.make_gemm(4, 8, 8, seed=2)
    eye = synthetic.bf16_round(np.eye(8, dtype=np.float32))
    A = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.flat_gemm(a, eye), A)
    pick = synthetic.bf16_round(np.eye(8, dtype=np.float32)[[5, 0, 5]])
    np.testing.assert_array_equal(oracle.flat_gemm(a, pick), A[:, [5, 0, 5]])


def test_f32_operands_and_error_scale():
    a, w = synthetic.make_gemm(2, 6, 16, seed=3, dtype="f32")
    np.testing.assert_allclose(oracle.flat_gemm(a, w, a_dtype="f32", w_dtype="f32"),
                               a.astype(np.float64) @ w.astype(np.float64).T, rtol=1e-14)
    ab, wb = synthetic.make_gemm(2, 6, 16, seed=3)
    assert np.all(oracle.flat_gemm_abs(ab, wb) >= np.abs(oracle.flat_gemm(ab, wb)))


def test_error_scale_closed_forms():
    # |A| . |W|^T pinned from both sides: equal to the product itself when no
    # term can cancel (nonnegative operands), K for operands of +-1 whatever
    # the signs, and a scaled column of |A| for one-hot weight rows
    rng = np.random.default_rng(4)
    K = 64
    ab, wb = synthetic.make_gemm(3, 5, K, seed=4)
    pos_a = synthetic.bf16_round(np.abs(synthetic.bf16_to_f32(ab)))
    pos_w = synthetic.bf16_round(np.abs(synthetic.bf16_to_f32(wb)))
    np.testing.assert_array_equal(oracle.flat_gemm_abs(ab, wb), oracle.flat_gemm(pos_a, pos_w))
    signs_a = synthetic.bf16_round(rng.choice([-1.0, 1.0], size=(3, K)).astype(np.float32))
    signs_w = synthetic.bf16_round(rng.choice([-1.0, 1.0], size=(5, K)).astype(np.float32))
    np.testing.assert_array_equal(oracle.flat_gemm_abs(signs_a, signs_w), np.full((3, 5), float(K)))
    onehot = np.zeros((3, K), dtype=np.float32)
    onehot[0, 7], onehot[1, 0], onehot[2, K - 1] = -2.0, 0.5, -1.0
    got = oracle.flat_gemm_abs(ab, synthetic.bf16_round(onehot))
    A = np.abs(synthetic.bf16_to_f32(ab).astype(np.float64))
    np.testing.assert_array_equal(got, np.stack([2.0 * A[:, 7], 0.5 * A[:, 0], A[:, K - 1]], axis=1))
