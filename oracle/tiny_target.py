"""A tiny random causal target model, used only by the lossless-invariant test.

Test infrastructure only (see ``oracle/__init__.py``).  The pages treat the
target as an external model whose hidden states from several layers feed the
drafter and whose logits decide verification.  This stand-in is a float64
pre-norm causal transformer with random weights.

Every row goes through one shape-independent path (one matrix-vector product
per projection, attention of one query over the keys up to its own position),
so running a row alone (autoregressive decoding) or inside a block of rows
(verification) gives bit-identical logits; greedy speculative output can then
be compared with greedy autoregressive output exactly.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .draft import rmsnorm, rope, silu

F64 = np.float64


class TinyTarget:
    def __init__(self, vocab: int = 1024, hidden: int = 256, n_heads: int = 4, n_kv_heads: int = 2,
                 head_dim: int = 64, ffn: int = 512, n_layers: int = 4,
                 feature_layers: Sequence[int] = (1, 2, 3), seed: int = 7, max_len: int = 1024,
                 rope_theta: float = 1e6):
        rng = np.random.default_rng(seed)
        s = 1.0 / np.sqrt(hidden)
        self.vocab, self.hidden = vocab, hidden
        self.n_heads, self.n_kv_heads, self.head_dim = n_heads, n_kv_heads, head_dim
        self.n_layers = n_layers
        self.feature_layers = tuple(feature_layers)
        self.theta = rope_theta
        self.embed = rng.standard_normal((vocab, hidden))
        self.layers = []
        for _ in range(n_layers):
            self.layers.append(dict(
                wq=rng.standard_normal((n_heads * head_dim, hidden)) * s,
                wk=rng.standard_normal((n_kv_heads * head_dim, hidden)) * s,
                wv=rng.standard_normal((n_kv_heads * head_dim, hidden)) * s,
                wo=rng.standard_normal((hidden, n_heads * head_dim)) / np.sqrt(n_heads * head_dim),
                wg=rng.standard_normal((ffn, hidden)) * s,
                wu=rng.standard_normal((ffn, hidden)) * s,
                wd=rng.standard_normal((hidden, ffn)) / np.sqrt(ffn),
            ))
        # N(0,1)/sqrt(H) head: wide logit margins, so greedy choices are not near-ties
        self.w_lm = rng.standard_normal((vocab, hidden)) * s
        self.ones = np.ones(hidden)
        self.k = np.zeros((n_layers, max_len, n_kv_heads, head_dim))
        self.v = np.zeros((n_layers, max_len, n_kv_heads, head_dim))
        self.length = 0

    def reset(self) -> None:
        self.length = 0

    def truncate(self, length: int) -> None:
        """Roll the target's own cache back to `length` rows."""
        assert 0 <= length <= self.length
        self.length = length

    def _row(self, tok: int, pos: int) -> Tuple[np.ndarray, List[np.ndarray]]:
        group = self.n_heads // self.n_kv_heads
        x = self.embed[tok].copy()
        feats = []
        for l, w in enumerate(self.layers):
            u = rmsnorm(x, self.ones)
            q = (w["wq"] @ u).reshape(1, self.n_heads, self.head_dim)
            k = (w["wk"] @ u).reshape(1, self.n_kv_heads, self.head_dim)
            v = (w["wv"] @ u).reshape(1, self.n_kv_heads, self.head_dim)
            p = np.array([pos])
            q = rope(q, p, self.theta)[0]
            k = rope(k, p, self.theta)[0]
            self.k[l, pos] = k
            self.v[l, pos] = v[0]
            o = np.empty((self.n_heads, self.head_dim))
            for h in range(self.n_heads):
                kv = h // group
                s = self.k[l, : pos + 1, kv] @ q[h] / np.sqrt(self.head_dim)  # causal
                e = np.exp(s - s.max())
                o[h] = (e / e.sum()) @ self.v[l, : pos + 1, kv]
            x = x + w["wo"] @ o.reshape(-1)
            u = rmsnorm(x, self.ones)
            x = x + w["wd"] @ (silu(w["wg"] @ u) * (w["wu"] @ u))
            if l in self.feature_layers:
                feats.append(x.copy())
        logits = self.w_lm @ rmsnorm(x, self.ones)
        return logits, feats

    def forward(self, tokens: Sequence[int]) -> Tuple[np.ndarray, List[np.ndarray]]:
        """Run rows at positions length .. length+n-1 and append them.

        Returns logits [n, V] and the hidden states of the feature layers,
        a list of [n, H] arrays in the order of ``feature_layers``.
        """
        n = len(tokens)
        logits = np.empty((n, self.vocab))
        feats = [np.empty((n, self.hidden)) for _ in self.feature_layers]
        for i, t in enumerate(tokens):
            lg, fs = self._row(int(t), self.length + i)
            logits[i] = lg
            for j, f in enumerate(fs):
                feats[j][i] = f
        self.length += n
        return logits, feats
