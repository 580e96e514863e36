"""Pins of the oracle's block-causal attention (CPU only)."""
import math

import numpy as np
import torch
import torch.nn.functional as Fn

import oracle


def _mask_by_enumeration(seg_len, T_q):
    """allowed[i][j] from the segment list, pair by pair."""
    owner = []
    for s, n in enumerate(seg_len):
        owner += [s] * n
    T_k = len(owner)
    return [[owner[j] <= owner[T_k - T_q + i] for j in range(T_k)] for i in range(T_q)]


def _brute_force(q, k, v, seg_len):
    T_q, H, d = q.shape
    T_k = k.shape[0]
    allowed = _mask_by_enumeration(seg_len, T_q)
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(T_q):
            scores = []
            for j in range(T_k):
                if allowed[i][j]:
                    scores.append((j, sum(q[i, h, c] * k[j, h, c] for c in range(d)) / math.sqrt(d)))
            m = max(s for _, s in scores)
            w = [(j, math.exp(s - m)) for j, s in scores]
            z = sum(e for _, e in w)
            for j, e in w:
                out[i, h] += (e / z) * v[j, h]
    return out


def test_mask_matches_enumeration():
    for seg_len, T_q in (([3, 4], 7), ([2, 3, 5], 10), ([2, 3, 5], 5), ([1, 1, 1, 1], 2), ([6], 6)):
        assert oracle.allowed_mask(seg_len, T_q).tolist() == _mask_by_enumeration(seg_len, T_q)


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(0)
    for seg_len, T_q in (([3, 5], 8), ([2, 3, 4], 9), ([2, 3, 4], 4), ([2, 3, 4], 1)):
        T_k = sum(seg_len)
        q = rng.standard_normal((T_q, 2, 8))
        k = rng.standard_normal((T_k, 2, 8))
        v = rng.standard_normal((T_k, 2, 8))
        assert np.allclose(oracle.attention(q, k, v, seg_len), _brute_force(q, k, v, seg_len),
                           rtol=1e-12, atol=1e-13)


def test_attention_vs_library_sdpa_with_mask():
    rng = np.random.default_rng(1)
    seg_len = [16, 40, 72]
    T_k = sum(seg_len)
    for T_q in (T_k, 72, 5):
        q = rng.standard_normal((T_q, 3, 128))
        k = rng.standard_normal((T_k, 3, 128))
        v = rng.standard_normal((T_k, 3, 128))
        mask = torch.tensor(_mask_by_enumeration(seg_len, T_q))
        ref = Fn.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(0, 1), torch.from_numpy(k).transpose(0, 1),
            torch.from_numpy(v).transpose(0, 1), attn_mask=mask).transpose(0, 1).numpy()
        assert np.allclose(oracle.attention(q, k, v, seg_len), ref, rtol=1e-11, atol=1e-12)
    # one segment is plain full attention
    q = rng.standard_normal((33, 2, 128))
    ref = Fn.scaled_dot_product_attention(torch.from_numpy(q).transpose(0, 1), torch.from_numpy(q).transpose(0, 1),
                                          torch.from_numpy(q).transpose(0, 1)).transpose(0, 1).numpy()
    assert np.allclose(oracle.attention(q, q, q, [33]), ref, rtol=1e-11, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    seg_len = [1, 4, 6]
    T = 11
    q = rng.standard_normal((T, 2, 128))
    k = rng.standard_normal((T, 2, 128))
    v = rng.standard_normal((T, 2, 128))
    o = oracle.attention(q, k, v, seg_len)
    assert np.allclose(o[0], v[0], atol=1e-14)               # one allowed key -> that value
    o0 = oracle.attention(np.zeros_like(q), k, v, seg_len)   # q = 0 -> mean of allowed values
    assert np.allclose(o0[3], v[:5].mean(axis=0), atol=1e-13)
    assert np.allclose(o0[10], v.mean(axis=0), atol=1e-13)
    vc = np.broadcast_to(rng.standard_normal((1, 2, 128)), v.shape)
    assert np.allclose(oracle.attention(q, k, vc, seg_len), vc[:T], atol=1e-13)


def test_online_softmax_agrees_with_two_pass():
    rng = np.random.default_rng(3)
    seg_len = [20, 44, 64]
    T = 128
    q = rng.standard_normal((T, 1, 128)) * 3
    k = rng.standard_normal((T, 1, 128)) * 3
    v = rng.standard_normal((T, 1, 128))
    allowed = oracle.allowed_mask(seg_len, T)
    out = np.zeros((T, 128))
    for i in range(T):
        m, l, acc = -np.inf, 0.0, np.zeros(128)
        for j0 in range(0, T, 32):             # streaming over key tiles
            js = [j for j in range(j0, j0 + 32) if allowed[i, j]]
            if not js:
                continue
            s = np.array([q[i, 0] @ k[j, 0] for j in js]) / math.sqrt(128)
            m_new = max(m, s.max())
            acc = acc * math.exp(m - m_new) + np.exp(s - m_new) @ v[js, 0]
            l = l * math.exp(m - m_new) + np.exp(s - m_new).sum()
            m = m_new
        out[i] = acc / l
    assert np.allclose(oracle.attention(q, k, v, seg_len)[:, 0], out, rtol=1e-11, atol=1e-12)


def test_later_segments_do_not_change_earlier_rows():
    rng = np.random.default_rng(4)
    seg_len = [5, 7, 9]
    T = 21
    q, k, v = (rng.standard_normal((T, 2, 128)) for _ in range(3))
    o1 = oracle.attention(q, k, v, seg_len)
    k2, v2 = k.copy(), v.copy()
    k2[12:] += 5.0
    v2[12:] -= 3.0
    o2 = oracle.attention(q, k2, v2, seg_len)
    assert np.array_equal(o1[:12], o2[:12])
    assert not np.allclose(o1[12:], o2[12:])
