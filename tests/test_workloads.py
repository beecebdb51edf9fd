"""Seeded input generators: determinism, per-token regeneration, distributions
and the sizing of the expert-parallel share."""
import numpy as np
import torch

import workloads as W


def test_generator_is_deterministic_and_row_addressable():
    rows = torch.arange(0, 64, dtype=torch.int64)
    a = W.normal(7, W.S_X, rows, 33)
    b = W.normal(7, W.S_X, rows, 33)
    assert torch.equal(a, b)
    # any subset of rows regenerates to the same values
    sub = torch.tensor([5, 17, 63], dtype=torch.int64)
    assert torch.equal(W.normal(7, W.S_X, sub, 33), a[sub])
    # streams and seeds differ
    assert not torch.equal(a, W.normal(7, W.S_W1, rows, 33))
    assert not torch.equal(a, W.normal(8, W.S_X, rows, 33))


def test_normal_and_gumbel_moments():
    rows = torch.arange(0, 4096, dtype=torch.int64)
    z = W.normal(1, W.S_X, rows, 256).double()
    assert abs(z.mean().item()) < 0.01 and abs(z.std().item() - 1.0) < 0.01
    g = W.gumbel(1, W.S_LOGIT, rows, 256)
    # Gumbel(0,1): mean = Euler-Mascheroni constant, variance = pi^2 / 6
    assert abs(g.mean().item() - 0.5772156649) < 0.01
    assert abs(g.var().item() - np.pi ** 2 / 6) < 0.03
    u = W.uniform01(1, 0, rows, 256)
    assert u.min().item() > 0 and u.max().item() < 1


def test_tiny_workload_inputs():
    w = W.get("tiny_fp32")
    inp = W.make_inputs(w)
    assert inp["x"].shape == (256, 128) and inp["x"].dtype == torch.float32
    assert inp["logits"].shape == (256, 8) and inp["logits"].dtype == torch.float32
    assert inp["W1"].shape == (8, 256, 128) and inp["W2"].shape == (8, 128, 256)
    assert inp["dout"].shape == (256, 128)
    s = inp["W1"].double().std().item()
    assert abs(s - 0.02) < 0.001
    # logits are x . Wr
    ref = (inp["x"].double() @ inp["Wr"].double()).float()
    assert torch.equal(ref, inp["logits"])


def test_weights_are_per_expert_addressable():
    w = W.scaled("bf16_fwd", E=4, d=64, F=96, T=16)
    full = W.make_weights(w)
    part = W.make_weights(W.scaled("bf16_fwd", E=4, d=64, F=96, T=16, expert_begin=2, expert_end=4))
    assert torch.equal(full["W1"][2:], part["W1"]) and torch.equal(full["W2"][2:], part["W2"])


def test_ep_share_sizing_and_token_regeneration():
    w = W.get("ep_share")
    assert w.notes["perm_seed"] == W.EP_PERM_SEED
    n = W.local_pair_count(w)
    assert abs(n - 16384) <= 0.10 * 16384
    ids = W.ep_share_tokens(w)
    assert 14000 < ids.numel() < 16210
    assert bool((ids[1:] > ids[:-1]).all())
    # activations of a token depend only on its id
    x_all = W.normal(w.seed, W.S_X, ids[:50], 64)
    x_one = W.normal(w.seed, W.S_X, ids[7:8], 64)
    assert torch.equal(x_all[7:8], x_one)


def test_zipf_popularity():
    lp = W.zipf_log_popularity(128, 1.2, None).exp()
    assert abs(lp.sum().item() - 1.0) < 1e-12
    assert bool((lp[1:] < lp[:-1]).all())
    assert abs(lp[0].item() / lp[1].item() - 2 ** 1.2) < 1e-9
    lpp = W.zipf_log_popularity(256, 1.1, 34).exp()
    assert torch.allclose(torch.sort(lpp, descending=True).values, W.zipf_log_popularity(256, 1.1, None).exp())
