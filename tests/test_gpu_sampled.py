"""GPU parity of the sampled recovery F (Gaussian and Exponential rows of the
walkthrough's section 3.3 F table) through the C ABI, against the CPU oracle.

The statistics (mu, sigma) and every decode output must satisfy
|gpu - ref| <= 1e-3 + 2e-3 |ref| elementwise. Both sides draw the samples from
the same Philox4x32-10 counters, each implemented from the generator's
published definition; the GPU turns them into samples in fp32, the oracle in
float64.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops
from sparse_decode_attention_amd.configs import WORKLOADS

from test_gpu_parity import assert_tol, check_prefill, dev_bf16, host, run_prefill

pytestmark = pytest.mark.gpu

SAMPLED = ["gaussian", "exponential"]
SEED = 0x0123456789ABCDEF


def sampled_decode(g, x, lam, recovery, seed, step=0, splits=0):
    out = ops.decode_attn_sampled(dev_bf16(x["q_dec"][step]), g["k_packed"], g["mask"], dev_bf16(x["v"]),
                                  g["chan_energy"], g["r"], recovery, seed, lam, splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def sampled_case(w, seed, lam, recovery, rng_seed=SEED, splits=0, steps=1):
    x = gen.numpy_layer(w, seed=seed, steps=steps)
    g, ref, f = check_prefill(x, w.n_kv, lam, recovery=recovery)
    r_ref, _ = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    for s in range(steps):
        got = sampled_decode(g, x, lam, recovery, rng_seed, s, splits)
        want = oracle.decode_attn_sampled(f["q_dec"][s], ref["packed"], ref["mask"], f["v"], ref["A"], r_ref,
                                          recovery, rng_seed)
        assert_tol(got, want, f"{recovery} decode step {s}")
    return g, x, ref, f


@pytest.mark.parametrize("recovery", SAMPLED)
@pytest.mark.parametrize("qagg", ["l2", "mean"])
def test_sampled_prefill_stats(recovery, qagg):
    w = WORKLOADS["tiny_s1k"].with_(S=700)
    check_prefill(gen.numpy_layer(w, seed=21, steps=0), w.n_kv, 0.8, qagg, recovery)


@pytest.mark.parametrize("recovery", SAMPLED)
def test_sampled_stats_from_stored_cache(recovery):
    w = WORKLOADS["tiny_s1k"].with_(S=900)
    x = gen.numpy_layer(w, seed=22, steps=0)
    g, ref, f = check_prefill(x, w.n_kv, 0.5)
    r, cnt = ops.stats(g["k_packed"], g["mask"], g["chan_energy"], 0.5, recovery, k_dense=dev_bf16(x["k"]))
    torch.cuda.synchronize()
    r_ref, cnt_ref = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    np.testing.assert_array_equal(cnt.cpu().numpy(), cnt_ref)
    assert_tol(r.cpu().numpy(), r_ref, recovery)
    assert (r.cpu().numpy()[..., 2:] == 0).all()


@pytest.mark.parametrize("recovery", SAMPLED)
@pytest.mark.parametrize("lam", [0.5, 0.8, 0.3, 1.0])
def test_sampled_decode_tiny(recovery, lam):
    sampled_case(WORKLOADS["tiny_s1k"], 23, lam, recovery, steps=2)


@pytest.mark.parametrize("recovery", SAMPLED)
@pytest.mark.parametrize("B,S,n_q,n_kv,splits", [(1, 1, 32, 8, 0), (2, 63, 32, 8, 0), (1, 65, 8, 8, 2),
                                                 (2, 1000, 16, 8, 3), (1, 4097, 16, 2, 0), (1, 300, 8, 1, 5)])
def test_sampled_decode_ragged_and_groups(recovery, B, S, n_q, n_kv, splits):
    sampled_case(WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_q, n_kv=n_kv), 24, 0.7, recovery, splits=splits)


@pytest.mark.parametrize("recovery", SAMPLED)
def test_sampled_decode_seed(recovery):
    """Same seed: bitwise the same output. Seeds differing in either 32-bit
    half: different outputs, each matching the oracle for its own seed."""
    w = WORKLOADS["tiny_s1k"].with_(S=1500)
    g, x, ref, f = sampled_case(w, 25, 0.5, recovery, rng_seed=7)
    a = sampled_decode(g, x, 0.5, recovery, 7)
    np.testing.assert_array_equal(a, sampled_decode(g, x, 0.5, recovery, 7))
    r_ref, _ = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    for other in (8, 7 + (1 << 32)):
        b = sampled_decode(g, x, 0.5, recovery, other)
        assert np.abs(a - b).max() > 1e-4, other
        want = oracle.decode_attn_sampled(f["q_dec"][0], ref["packed"], ref["mask"], f["v"], ref["A"], r_ref,
                                          recovery, other)
        assert_tol(b, want, f"seed {other:#x}")


@pytest.mark.parametrize("recovery", SAMPLED)
def test_sampled_split_invariance(recovery):
    w = WORKLOADS["tiny_s1k"].with_(S=5000)
    x = gen.numpy_layer(w, seed=26, steps=1)
    g = run_prefill(x, w.n_kv, 0.5, recovery=recovery)
    outs = [sampled_decode(g, x, 0.5, recovery, SEED, splits=sp) for sp in (1, 2, 7, 0, 79)]
    for o in outs[1:]:
        assert_tol(o, outs[0], "split invariance")


@pytest.mark.parametrize("recovery", SAMPLED)
def test_sampled_lambda0_is_dense(recovery):
    w = WORKLOADS["tiny_s1k"].with_(S=2000)
    x = gen.numpy_layer(w, seed=27, steps=1)
    g = run_prefill(x, w.n_kv, 0.0, recovery=recovery)
    f = host(x)
    assert_tol(sampled_decode(g, x, 0.0, recovery, SEED), oracle.dense_attn(f["q_dec"][0], f["k"], f["v"]),
               "lambda=0 vs dense")


def test_sampled_gaussian_sigma0_is_the_degenerate_f():
    """With sigma forced to 0 every Gaussian sample is mu: the output is the
    Degenerate F's decode (r_j = mu / a_j) on the same cache."""
    w = WORKLOADS["tiny_s1k"].with_(S=1200)
    x = gen.numpy_layer(w, seed=28, steps=1)
    g = run_prefill(x, w.n_kv, 0.8, recovery="gaussian")
    deg = run_prefill(x, w.n_kv, 0.8, recovery="score_mean_pruned")
    g["r"][..., 1] = 0.0
    got = sampled_decode(g, x, 0.8, "gaussian", SEED)
    want = ops.decode_attn(dev_bf16(x["q_dec"][0]), deg["k_packed"], deg["mask"], dev_bf16(x["v"]), deg["r"], 0.8)
    torch.cuda.synchronize()
    assert_tol(got, want.cpu().numpy(), "sigma=0 vs degenerate")


@pytest.mark.parametrize("recovery", SAMPLED)
def test_sampled_full_size_s32k(recovery):
    """The benchmarked shape (LLaMA-3.1-8B layer, S=32768, lambda=0.5): the
    statistics and every decode output within tolerance."""
    w = WORKLOADS["llama8b_s32k_l05"]
    sampled_case(w, 0, w.lam, recovery)
