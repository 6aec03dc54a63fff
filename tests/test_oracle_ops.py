"""Pins of the oracle's elementary operations against closed forms, brute force
and library routines (never against the oracle's own formula)."""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import depthwise_conv3, fuse_features, gqa_attention, rmsnorm, rope, silu

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_hand_values():
    # x = (3, 4): mean square 12.5, so the normalised vector is x / sqrt(12.5)
    out = rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), eps=0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(out, [3.0 / r, 2.0 * 4.0 / r], rtol=1e-15)


def test_rmsnorm_matches_torch_routine():
    x = RNG.standard_normal((7, 96)) * 3.0
    g = RNG.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(rmsnorm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-12)


def test_rmsnorm_scale_invariant_and_unit_rms():
    x = RNG.standard_normal((5, 64))
    g = np.ones(64)
    a = rmsnorm(x, g, 1e-12)
    np.testing.assert_allclose(rmsnorm(17.0 * x, g, 1e-12), a, rtol=1e-10)
    np.testing.assert_allclose(np.sqrt(np.mean(a * a, axis=-1)), 1.0, rtol=1e-10)


# ---------------------------------------------------------------- RoPE
def test_rope_hand_rotation_rotate_half_pairing():
    # D = 4: pairs are (0, 2) and (1, 3); pair j turns by pos * theta^(-2j/D)
    theta = 100.0
    z = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    out = rope(z, np.array([2]), theta)[0, 0]
    a0, a1 = 2.0 * 1.0, 2.0 * theta ** (-0.5)
    exp = [1.0 * math.cos(a0) - 3.0 * math.sin(a0), 2.0 * math.cos(a1) - 4.0 * math.sin(a1),
           1.0 * math.sin(a0) + 3.0 * math.cos(a0), 2.0 * math.sin(a1) + 4.0 * math.cos(a1)]
    np.testing.assert_allclose(out, exp, rtol=1e-14)


def test_rope_identity_norm_relative():
    q = RNG.standard_normal((1, 3, 64))
    k = RNG.standard_normal((1, 3, 64))
    np.testing.assert_array_equal(rope(q, np.array([0])), q)
    for p in (1, 77, 4095, 32768):
        np.testing.assert_allclose(np.linalg.norm(rope(q, np.array([p])), axis=-1),
                                   np.linalg.norm(q, axis=-1), rtol=1e-12)
    # score depends only on the position difference
    s1 = np.sum(rope(q, np.array([5]))[0] * rope(k, np.array([12]))[0], axis=-1)
    s2 = np.sum(rope(q, np.array([42]))[0] * rope(k, np.array([49]))[0], axis=-1)
    np.testing.assert_allclose(s1, s2, rtol=1e-9)


# ---------------------------------------------------------------- attention
def _brute_attention(q, k, v):
    nq, hq, d = q.shape
    nk, hkv, _ = k.shape
    grp = hq // hkv
    out = np.zeros_like(q)
    for i, h in itertools.product(range(nq), range(hq)):
        kv = h // grp
        s = [sum(q[i, h, t] * k[j, kv, t] for t in range(d)) / math.sqrt(d) for j in range(nk)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        for t in range(d):
            out[i, h, t] = sum(e[j] / z * v[j, kv, t] for j in range(nk))
    return out


def test_attention_brute_force_triple_loop():
    q = RNG.standard_normal((4, 4, 8))
    k = RNG.standard_normal((6, 2, 8))
    v = RNG.standard_normal((6, 2, 8))
    np.testing.assert_allclose(gqa_attention(q, k, v), _brute_attention(q, k, v), rtol=1e-10, atol=1e-12)


def test_attention_matches_torch_sdpa_noncausal_gqa():
    q = RNG.standard_normal((16, 8, 32))
    k = RNG.standard_normal((40, 2, 32))
    v = RNG.standard_normal((40, 2, 32))
    tq, tk, tv = (torch.from_numpy(a).transpose(0, 1) for a in (q, k, v))  # [heads, n, D]
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=False, enable_gqa=True)
    np.testing.assert_allclose(gqa_attention(q, k, v), ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_single_key_returns_value():
    q = RNG.standard_normal((1, 4, 8))
    k = RNG.standard_normal((1, 2, 8))
    v = RNG.standard_normal((1, 2, 8))
    out = gqa_attention(q, k, v)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[0, h // 2], rtol=1e-14)


def test_gqa_equals_mha_with_replicated_heads():
    q = RNG.standard_normal((5, 6, 8))
    k = RNG.standard_normal((9, 3, 8))
    v = RNG.standard_normal((9, 3, 8))
    k_rep = np.repeat(k, 2, axis=1)  # head h -> kv head h // 2
    v_rep = np.repeat(v, 2, axis=1)
    np.testing.assert_allclose(gqa_attention(q, k, v), gqa_attention(q, k_rep, v_rep), rtol=1e-14)


# ---------------------------------------------------------------- local conv
def test_conv_unit_taps():
    x = RNG.standard_normal((16, 8))
    one = lambda t: np.tile(np.eye(3)[t], (8, 1))  # noqa: E731
    np.testing.assert_array_equal(depthwise_conv3(x, one(1)), x)
    down = depthwise_conv3(x, one(0))  # y[i] = x[i-1]
    np.testing.assert_array_equal(down[1:], x[:-1])
    np.testing.assert_array_equal(down[0], 0.0)
    up = depthwise_conv3(x, one(2))  # y[i] = x[i+1]
    np.testing.assert_array_equal(up[:-1], x[1:])
    np.testing.assert_array_equal(up[-1], 0.0)


def test_conv_matches_library_correlation():
    x = RNG.standard_normal((16, 5))
    w = RNG.standard_normal((5, 3))
    ref = np.stack([np.correlate(np.pad(x[:, c], 1), w[c], mode="valid") for c in range(5)], axis=1)
    np.testing.assert_allclose(depthwise_conv3(x, w), ref, rtol=1e-13, atol=1e-14)
    # and torch's depthwise conv1d (cross-correlation, zero padding 1)
    t = F.conv1d(torch.from_numpy(x.T[None]), torch.from_numpy(w[:, None, :]), padding=1, groups=5)
    np.testing.assert_allclose(depthwise_conv3(x, w), t[0].numpy().T, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- fusion
def test_fuse_single_layer_identity_is_rmsnorm():
    h = RNG.standard_normal((9, 32)) * 4.0
    c = fuse_features([h], np.eye(32), np.ones(32), eps=0.0)
    np.testing.assert_allclose(c, h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True)), rtol=1e-13)
    np.testing.assert_allclose(np.sqrt(np.mean(c * c, axis=-1)), 1.0, rtol=1e-13)


def test_fuse_concat_order_follows_weight_blocks():
    h1, h2, h3 = (RNG.standard_normal((3, 16)) for _ in range(3))
    w = RNG.standard_normal((16, 48))
    g = RNG.standard_normal(16)
    a = fuse_features([h1, h2, h3], w, g)
    perm = np.concatenate([w[:, 32:48], w[:, 0:16], w[:, 16:32]], axis=1)
    np.testing.assert_allclose(fuse_features([h3, h1, h2], perm, g), a, rtol=1e-12)
    # the fused linear is x W^T: a single-row check against explicit sums
    y = np.array([sum(np.concatenate([h1, h2, h3], axis=1)[0, k] * w[n, k] for k in range(48))
                  for n in range(16)])
    np.testing.assert_allclose(a[0], y / np.sqrt(np.mean(y * y) + 1e-6) * g, rtol=1e-12)


def test_silu_closed_form():
    np.testing.assert_allclose(silu(np.array([0.0, 1.0, -2.0])),
                               [0.0, 1.0 / (1.0 + math.exp(-1.0)), -2.0 / (1.0 + math.exp(2.0))], rtol=1e-15)
    x = RNG.standard_normal(50)
    np.testing.assert_allclose(silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14)
