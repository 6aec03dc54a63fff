"""Turn the shared seeded inputs (torch tensors) into oracle objects (float64 numpy)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import DraftState, DraftWeights, LayerWeights, OracleDims


def np64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def dims_of(wl) -> OracleDims:
    return OracleDims(hidden=wl.hidden, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                      head_dim=wl.head_dim, n_layers=wl.n_layers, ffn=wl.ffn, vocab=wl.vocab,
                      block=wl.block, n_target_layers=wl.n_target_layers, rms_eps=wl.rms_eps,
                      rope_theta=wl.rope_theta, conv_width=wl.conv_width, kv_int8=wl.kv == "int8")


def weights_of(w: dict, layers=None) -> DraftWeights:
    ls = []
    for lw in (w["layers"] if layers is None else [w["layers"][i] for i in layers]):
        ls.append(LayerWeights(
            w_q=np64(lw["w_q"]), w_k=np64(lw["w_k"]), w_v=np64(lw["w_v"]), w_o=np64(lw["w_o"]),
            w_gate=np64(lw["w_gate"]), w_up=np64(lw["w_up"]), w_down=np64(lw["w_down"]),
            g_in=np64(lw["g_in"]), g_post=np64(lw["g_post"]),
            conv=None if lw["conv"] is None else np64(lw["conv"])))
    return DraftWeights(embed=np64(w["embed"]), w_fc=np64(w["w_fc"]), g_fc=np64(w["g_fc"]),
                        g_final=np64(w["g_final"]), w_lm=np64(w["w_lm"]), layers=ls)


def state_of(ks, vs, ctx_lens, seqs=None) -> DraftState:
    """Oracle cache from the generator's K/V tensors (optionally a subset of sequences)."""
    sel = slice(None) if seqs is None else list(seqs)
    k = [np64(t[sel]) for t in ks]
    v = [np64(t[sel]) for t in vs]
    cl = np.asarray(ctx_lens, dtype=np.int64)
    cl = cl.copy() if seqs is None else cl[list(seqs)].copy()
    return DraftState(k=k, v=v, ctx_len=cl)
