"""The allocation-free decode entry point (spark_decode_attn_noalloc, for
callers that cannot allocate device memory) through the C ABI: two calls in a
row, the second on a smaller problem, each equal bit for bit to
spark_decode_attn with the same split count and within tolerance of the CPU
oracle; a problem beyond the fixed scratch is rejected."""
import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops
from sparse_decode_attention_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

RTOL, ATOL = 2e-3, 1e-3
DEV = "cuda:0"


def assert_tol(got, ref, what):
    got = np.asarray(got, np.float64)
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    assert np.isfinite(got).all() and (excess <= 0).all(), f"{what}: worst excess {excess.max():.3e}"


def _case(w, seed, lam, splits):
    x = gen.numpy_layer(w, seed=seed, steps=1)
    d = {n: gen.to_torch_bf16(a, DEV) for n, a in x.items()}
    g = ops.prefill_prune(d["q_win"], d["k"], w.n_kv, lam)
    q, v = d["q_dec"][0], d["v"]
    ref_abi = ops.decode_attn(q, g["k_packed"], g["mask"], v, g["r"], lam, splits=splits)
    got = ops.decode_attn_noalloc(q, g["k_packed"], g["mask"], v, g["r"], lam, splits=splits)
    torch.cuda.synchronize()
    f = {n: gen.bf16_bits_to_f32(a) for n, a in x.items()}
    ref = oracle.prune(f["q_win"], f["k"], w.n_kv, lam)
    r_ref, _ = oracle.stats(f["k"], ref["mask"], ref["A"])
    want = oracle.decode_attn(f["q_dec"][0], ref["packed"], ref["mask"], f["v"], r_ref)
    return got.cpu().numpy(), ref_abi.cpu().numpy(), want


def test_noalloc_two_calls_second_smaller():
    cases = [(WORKLOADS["llama8b_s32k_l05"], 0, 0.5, 0),                     # the benchmarked shape
             (WORKLOADS["tiny_s1k"].with_(B=2, S=777, n_q=16, n_kv=4), 1, 0.8, 3)]   # smaller, ragged
    for w, seed, lam, splits in cases:
        print(f"case {w.name} B={w.B} S={w.S} lam={lam} splits={splits}", flush=True)
        got, ref_abi, want = _case(w, seed, lam, splits)
        np.testing.assert_array_equal(got, ref_abi)
        assert_tol(got, want, f"{w.name} S={w.S}")


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=DEV)
    S = 1 << 20
    assert ops.lib().spark_decode_workspace_bytes(64, S, 32, 8, 128, 64) > ops.NOALLOC_SCRATCH_BYTES
    st = ops.lib().spark_decode_attn_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                             64, S, 32, 8, 128, 0.5, 0.0, 64, q.data_ptr(), None)
    assert st == ops.ESCRATCH
