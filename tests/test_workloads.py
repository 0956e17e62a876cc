"""The seeded input generators: the same seed gives the same tensors, another
seed different ones, and every tensor has the documented shape, dtype and
structure (K distinct experts per unmasked token, softmax weights, the
masking rate)."""
import numpy as np
import torch

import workloads as W


def _bytes(t):
    return t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.bfloat16 else \
        t.contiguous().view(torch.int16).numpy().tobytes()


def test_same_seed_same_tensors_other_seed_different():
    w = W.by_name("tiny").replace(mask_p=0.2)
    a = (W.make_x(w), *W.make_routing(w), W.make_y(w), W.make_rows(w, 7), W.make_expert_weights(w, 128))
    b = (W.make_x(w), *W.make_routing(w), W.make_y(w), W.make_rows(w, 7), W.make_expert_weights(w, 128))
    for u, v in zip(a, b):
        assert _bytes(u) == _bytes(v)
    w2 = w.replace(seed=w.seed + 1)
    c = (W.make_x(w2), *W.make_routing(w2), W.make_y(w2), W.make_rows(w2, 7), W.make_expert_weights(w2, 128))
    for u, v in zip(a, c):
        assert _bytes(u) != _bytes(v)


def test_shapes_and_routing_structure():
    for name in ("tiny", "mid", "skewed_masked"):
        w = W.by_name(name)
        if w.T * w.H > 10_000_000:
            w = w.replace(T=1024)
        x = W.make_x(w)
        idx, wt = W.make_routing(w)
        assert x.shape == (w.T, w.H) and x.dtype == torch.bfloat16
        assert idx.shape == (w.T, w.K) and idx.dtype == torch.int64
        assert wt.shape == (w.T, w.K) and wt.dtype == torch.float32
        ids = idx.numpy()
        assert ids.min() >= -1 and ids.max() < w.E
        for t in range(w.T):
            sel = ids[t][ids[t] >= 0]
            assert len(set(sel.tolist())) == len(sel)  # distinct experts
        # softmax over all K picks: each token's weights sum to 1
        assert np.allclose(wt.numpy().sum(axis=1), 1.0, atol=1e-5)
        if w.mask_p == 0 and w.full_mask_frac == 0:
            assert (ids >= 0).all()
        else:
            frac = float((ids < 0).mean())
            assert 0.5 * w.mask_p <= frac <= 2.0 * w.mask_p + w.full_mask_frac + 0.02
            if w.full_mask_frac:
                full = int((ids < 0).all(axis=1).sum())
                assert full >= round(w.full_mask_frac * w.T)


def test_small_int_generator_is_exact_integers():
    w = W.Workload("gi", T=4, H=64, K=2, E=4, seed=3)
    v = W.make_small_ints(w, (5, 64), lo=-2, hi=2)
    f = v.float().numpy()
    assert np.array_equal(f, np.round(f)) and f.min() >= -2 and f.max() <= 2
