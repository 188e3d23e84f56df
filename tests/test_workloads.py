"""The seeded input generators: reproducible, valid, and shaped as stated."""
import hashlib

import numpy as np
import torch

from moe_expert_load_ue_amd import workloads as W


def _digest(t):
    return hashlib.sha256(t.contiguous().numpy().tobytes()).hexdigest()


def _valid(r, E, k):
    a = r.reshape(-1, k).numpy()
    assert a.min() >= 0 and a.max() < E
    s = np.sort(a, axis=1)
    assert np.all(s[:, 1:] != s[:, :-1]), "experts distinct within a token"


def test_reproducible():
    for name in ("tiny", "pipeline", "large_ep", "dsv3"):
        a = W.make_routing(name, layers=2, tokens=2048)
        b = W.make_routing(name, layers=2, tokens=2048)
        assert _digest(a) == _digest(b)
    c = W.make_routing("tiny")
    assert c.shape == (1, 4096, 8) and c.dtype == torch.int32


def _spearman(x, y):
    rx = np.argsort(np.argsort(x)).astype(float)
    ry = np.argsort(np.argsort(y)).astype(float)
    return float(np.corrcoef(rx, ry)[0, 1])


def test_tiny_zipf_shape():
    cfg = W.CONFIGS["tiny"]
    r = W.make_routing(cfg)
    _valid(r, cfg.experts, cfg.topk)
    _, s, order, _ = W.layer_setup(cfg, 0)
    counts = np.bincount(r.numpy().ravel(), minlength=64)
    by_rank = counts[order.numpy()]            # Zipf rank 1, 2, ...
    assert _spearman(np.arange(64), by_rank) < -0.97
    # the top Zipf rank appears in nearly every token at s = 1.2, k = 8
    assert by_rank[0] > 0.9 * cfg.tokens


def test_large_ep_hot_share():
    cfg = W.CONFIGS["large_ep"]
    r = W.make_routing(cfg)
    _valid(r, cfg.experts, cfg.topk)
    _, s, order, hot = W.layer_setup(cfg, 0)
    counts = np.bincount(r.numpy().ravel(), minlength=cfg.experts)
    share = counts[hot.numpy()] / cfg.assignments
    # each hot expert appears in a token with p = 0.4: 5% of T*k
    sd = np.sqrt(cfg.tokens * 0.4 * 0.6) / cfg.assignments
    assert np.all(np.abs(share - 0.05) < 4 * sd), share
    assert _spearman(np.arange(252), counts[order.numpy()]) < -0.97
    # hot ids sit at random positions of the row
    pos = np.isin(r[0].numpy(), hot.numpy()).mean(axis=0)
    assert np.all(np.abs(pos - pos.mean()) < 0.01)


def test_dsv3_layers_nonstationary():
    cfg = W.CONFIGS["dsv3"]
    s = W.layer_exponents(cfg)
    assert len(s) == 58 and min(s) >= 0.6 and max(s) <= 1.4
    assert max(s) - min(s) > 0.5
    r = W.make_routing(cfg, layers=3, tokens=4096)
    _valid(r, cfg.experts, cfg.topk)
    tops = [int(np.argmax(np.bincount(r[i].numpy().ravel(), minlength=256)))
            for i in range(3)]
    assert len(set(tops)) > 1, "independent permutations per layer"


def test_later_step_same_distribution():
    """A later step redraws the tokens of each layer from the same
    distribution: different routing, the same expert order (the hottest
    experts agree), a close count profile."""
    for name in ("dsv3", "large_ep", "tiny"):
        cfg = W.CONFIGS[name]
        a = W.make_routing(cfg, layers=2, tokens=8192)
        b = W.make_routing(cfg, layers=2, tokens=8192, step=1)
        _valid(b, cfg.experts, cfg.topk)
        assert not torch.equal(a, b), name
        assert torch.equal(b, W.make_routing(cfg, layers=2, tokens=8192,
                                             step=1)), name
        for layer in range(2):
            ca = np.bincount(a[layer].numpy().ravel(), minlength=cfg.experts)
            cb = np.bincount(b[layer].numpy().ravel(), minlength=cfg.experts)
            assert np.argmax(ca) == np.argmax(cb), name
            tv = 0.5 * np.abs(ca / ca.sum() - cb / cb.sum()).sum()
            assert tv < 0.05, (name, tv)


def test_pipeline_drift():
    cfg = W.CONFIGS["pipeline"]
    s = W.layer_exponents(cfg)
    assert np.allclose(s, np.linspace(0.5, 1.5, 16))
    r = W.make_routing(cfg, layers=16, tokens=2048)
    _valid(r, cfg.experts, cfg.topk)
    top = [np.bincount(r[m].numpy().ravel(), minlength=128).max()
           for m in (0, 15)]
    assert top[1] > top[0], "skew grows with the exponent"


def test_stream_csr():
    rep_off, rep_buf, n = W.stream_csr()
    assert n == 64 and len(rep_off) == 33
    fan = np.diff(rep_off) - 1
    assert sorted(set(fan.tolist())) == [1, 2, 3, 4]
    used = [b for b in rep_buf if b >= 0]
    assert sorted(used) == list(range(64))
    sb = W.make_stream_buffers(elems=1000, n_mats=3)
    assert sb.master_w.dtype == torch.bfloat16 and sb.spare_g.shape == (64, 3, 1024)
    assert sb.mat("spare_g", 5, 2).shape == (1000,)
    assert torch.all(sb.spare_w.view(torch.int16) == -1)
    assert abs(float(sb.master_g[..., :1000].std()) - 0.02) < 0.002


def test_activations():
    x = W.make_activations(64, 128, 3)
    y = W.make_activations(64, 128, 3)
    z = W.make_activations(64, 128, 4)
    assert x.dtype == torch.bfloat16 and torch.equal(x, y) and not torch.equal(x, z)
