"""GPU parity: libspark (through the C ABI) against the CPU oracle.

Masks, packed values, channel energies and counts must match bit for bit;
recovery vectors and decode outputs must satisfy |gpu - ref| <= 1e-3 + 2e-3 |ref|
elementwise (fp32 arithmetic on bf16 inputs against the float64 oracle).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops
from sparse_decode_attention_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

RTOL, ATOL = 2e-3, 1e-3
DEV = "cuda:0"


def assert_tol(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    assert np.isfinite(got).all(), what
    assert (excess <= 0).all(), f"{what}: worst excess {excess.max():.3e} at {np.unravel_index(excess.argmax(), excess.shape)}"


def dev_bf16(bits):
    return gen.to_torch_bf16(bits, DEV)


def words_u32(mask_t):
    return mask_t.cpu().numpy().view(np.uint32)


def run_prefill(x, n_kv, lam, qagg="l2", recovery="mean_retained", f_const=0.01):
    out = ops.prefill_prune(dev_bf16(x["q_win"]), dev_bf16(x["k"]), n_kv, lam, qagg, recovery, f_const)
    torch.cuda.synchronize()
    return out


def host(x):
    return {n: gen.bf16_bits_to_f32(v) for n, v in x.items()}


def check_prefill(x, n_kv, lam, qagg="l2", recovery="mean_retained"):
    g = run_prefill(x, n_kv, lam, qagg, recovery)
    f = host(x)
    ref = oracle.prune(f["q_win"], f["k"], n_kv, lam, qagg)
    np.testing.assert_array_equal(g["chan_energy"].cpu().numpy(), ref["A"])
    np.testing.assert_array_equal(words_u32(g["mask"]), ref["words"])
    T = ref["T"]
    if T > 0:
        np.testing.assert_array_equal(g["k_packed"].view(torch.int16).cpu().numpy().view(np.uint16),
                                      gen.f32_to_bf16_bits(ref["packed"]))
    r_ref, cnt_ref = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    np.testing.assert_array_equal(g["cnt"].cpu().numpy(), cnt_ref)
    assert_tol(g["r"].cpu().numpy(), r_ref, f"r ({recovery})")
    return g, ref, f


# ------------------------------------------------------------------ prefill

@pytest.mark.parametrize("lam", [0.0, 0.5, 0.7, 0.8, 1.0])
def test_prefill_tiny(lam):
    w = WORKLOADS["tiny_s1k"]
    check_prefill(gen.numpy_layer(w, seed=0, steps=0), w.n_kv, lam)


@pytest.mark.parametrize("recovery", ["mean_retained", "zero", "const", "score_mean_pruned"])
@pytest.mark.parametrize("qagg", ["l2", "mean"])
def test_prefill_modes(recovery, qagg):
    w = WORKLOADS["tiny_s1k"].with_(S=700)
    check_prefill(gen.numpy_layer(w, seed=1, steps=0), w.n_kv, 0.8, qagg, recovery)


@pytest.mark.parametrize("recovery", ["zero", "const", "score_mean_pruned"])
@pytest.mark.parametrize("lam", [0.0, 1.0])
def test_prefill_modes_keep_all_or_none(recovery, lam):
    """lambda = 0 keeps every channel and lambda = 1 none: the select runs no
    bit search there, in every recovery mode."""
    w = WORKLOADS["tiny_s1k"].with_(S=300)
    check_prefill(gen.numpy_layer(w, seed=3, steps=0), w.n_kv, lam, recovery=recovery)


@pytest.mark.parametrize("B,S,n_q,n_kv", [(2, 1, 32, 8), (1, 63, 8, 8), (2, 65, 16, 8), (1, 257, 8, 4),
                                          (3, 1000, 16, 2), (1, 513, 8, 1)])
def test_prefill_ragged_and_groups(B, S, n_q, n_kv):
    w = WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_q, n_kv=n_kv, window=7)
    check_prefill(gen.numpy_layer(w, seed=2, steps=0), n_kv, 0.7)


def test_prefill_embedded_d8_brute_force():
    """D=8 problems with channels 8..127 zeroed: the GPU's kept set among the
    live channels equals exhaustive search of the reduced objective."""
    rng = np.random.default_rng(3)
    S = 300
    q = np.zeros((1, 1, 1, 128), np.float32)
    q[..., :8] = rng.choice([0.0, 0.5, 1.0, 2.0, 3.0], size=8)
    k = np.zeros((1, 1, S, 128), np.float32)
    k[..., :8] = rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 3.0, 0.5], size=(S, 8))
    x = {"q_win": gen.f32_to_bf16_bits(q), "k": gen.f32_to_bf16_bits(k)}
    for T in range(1, 9):
        lam = 1.0 - T / 128
        assert ops.num_kept(128, lam) == T
        g = run_prefill(x, 1, lam)
        words = words_u32(g["mask"])[0, 0]
        for t in range(S):
            w = [Fraction(abs(float(q[0, 0, 0, j]))) * Fraction(abs(float(k[0, 0, t, j]))) for j in range(8)]
            best, best_set = None, None
            for sub in itertools.combinations(range(8), T):
                v = sum((w[j] for j in sub), Fraction(0))
                if best is None or v > best:
                    best, best_set = v, sub
            got = tuple(j for j in range(128) if (int(words[t, j >> 5]) >> (j & 31)) & 1)
            assert got == best_set, (T, t)


@pytest.mark.parametrize("lam", [0.99, 0.985, 0.51, 0.5, 0.49, 0.012, 0.008])
def test_prefill_extreme_t_with_ties(lam):
    """T = 1, 2, 63, 64, 65, 126, 127 on keys with many exact ties: equal
    channel energies (every window row the same) and |k| from four values,
    plus all-zero tokens, whose kept set is the first T channels."""
    rng = np.random.default_rng(4)
    B, N_kv, S = 1, 2, 257
    q = np.ones((B, 2 * N_kv, 4, 128), np.float32)
    k = rng.choice([0.0, 1.0, -1.0, 2.0, -0.5, 0.5], size=(B, N_kv, S, 128)).astype(np.float32)
    k[:, :, ::17] = 0.0
    x = {"q_win": gen.f32_to_bf16_bits(q), "k": gen.f32_to_bf16_bits(k)}
    g, ref, _ = check_prefill(x, N_kv, lam)
    T = ops.num_kept(128, lam)
    zero = words_u32(g["mask"])[0, 0, 0]
    assert [(int(zero[j >> 5]) >> (j & 31)) & 1 for j in range(128)] == [1] * T + [0] * (128 - T)


def test_chan_energy_hand_cases_through_the_abi():
    """The oracle's hand cases for the window grouping and the fp32 order of
    A, embedded in D = 128 (other channels zero): query heads 0, 1 feed KV
    head 0 and heads 2, 3 feed KV head 1; squares 1, 1, 2^24, 1 in (head,
    row) order sum to 2^24 + 4 in sequential fp32."""
    q = np.zeros((1, 4, 1, 128), np.float32)
    for i in range(4):
        q[0, i, 0, i] = i + 1
    k = np.ones((1, 2, 3, 128), np.float32)
    for qagg in ("l2", "mean"):
        g = run_prefill({"q_win": gen.f32_to_bf16_bits(q), "k": gen.f32_to_bf16_bits(k)}, 2, 0.5, qagg)
        A = g["chan_energy"].cpu().numpy()
        np.testing.assert_array_equal(A[0, :, :4], [[1, 4, 0, 0], [0, 0, 9, 16]])
        assert not A[0, :, 4:].any()
    q2 = np.zeros((1, 2, 2, 128), np.float32)
    q2[0, :, :, 0] = [[1.0, 1.0], [4096.0, 1.0]]
    g = run_prefill({"q_win": gen.f32_to_bf16_bits(q2), "k": gen.f32_to_bf16_bits(k[:, :1])}, 1, 0.5)
    assert float(g["chan_energy"][0, 0, 0]) == 2.0 ** 24 + 4


def test_prefill_deterministic():
    w = WORKLOADS["tiny_s1k"].with_(S=2048)
    x = gen.numpy_layer(w, seed=4, steps=0)
    a = run_prefill(x, w.n_kv, 0.5)
    a = {n: (v.clone() if torch.is_tensor(v) else v) for n, v in a.items()}
    b = run_prefill(x, w.n_kv, 0.5)
    for n in ("mask", "k_packed", "r", "cnt", "chan_energy"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("recovery", ["mean_retained", "score_mean_pruned", "const"])
def test_stats_from_stored_cache(recovery):
    w = WORKLOADS["tiny_s1k"].with_(S=900)
    x = gen.numpy_layer(w, seed=5, steps=0)
    g, ref, f = check_prefill(x, w.n_kv, 0.5)
    r, cnt = ops.stats(g["k_packed"], g["mask"], g["chan_energy"], 0.5, recovery,
                       k_dense=dev_bf16(x["k"]))
    torch.cuda.synchronize()
    r_ref, cnt_ref = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    np.testing.assert_array_equal(cnt.cpu().numpy(), cnt_ref)
    assert_tol(r.cpu().numpy(), r_ref, recovery)


# ------------------------------------------------------------------ decode

def decode_case(w, seed, lam, splits=0, recovery="mean_retained", steps=1):
    x = gen.numpy_layer(w, seed=seed, steps=steps)
    g, ref, f = check_prefill(x, w.n_kv, lam, recovery=recovery)
    r_ref, _ = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    v = dev_bf16(x["v"])
    for s in range(steps):
        out = ops.decode_attn(dev_bf16(x["q_dec"][s]), g["k_packed"], g["mask"], v, g["r"], lam, splits=splits)
        torch.cuda.synchronize()
        want = oracle.decode_attn(f["q_dec"][s], ref["packed"], ref["mask"], f["v"], r_ref)
        assert_tol(out.cpu().numpy(), want, f"decode step {s}")
    return g, x


@pytest.mark.parametrize("lam", [0.5, 0.8, 0.7, 0.3])
def test_decode_tiny(lam):
    decode_case(WORKLOADS["tiny_s1k"], 0, lam, steps=2)


@pytest.mark.parametrize("recovery", ["zero", "const", "score_mean_pruned"])
def test_decode_recovery_modes(recovery):
    decode_case(WORKLOADS["tiny_s1k"].with_(S=777), 6, 0.8, recovery=recovery)


@pytest.mark.parametrize("B,S,n_q,n_kv,splits", [(1, 1, 32, 8, 0), (2, 63, 32, 8, 0), (1, 65, 8, 8, 2),
                                                 (2, 1000, 16, 8, 3), (1, 4097, 16, 2, 0), (1, 300, 8, 1, 5)])
def test_decode_ragged_and_groups(B, S, n_q, n_kv, splits):
    decode_case(WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_q, n_kv=n_kv), 7, 0.8, splits=splits)


def test_decode_lambda0_is_dense():
    w = WORKLOADS["tiny_s1k"].with_(S=2000)
    x = gen.numpy_layer(w, seed=8, steps=1)
    g = run_prefill(x, w.n_kv, 0.0)
    out = ops.decode_attn(dev_bf16(x["q_dec"][0]), g["k_packed"], g["mask"], dev_bf16(x["v"]), g["r"], 0.0)
    torch.cuda.synchronize()
    f = host(x)
    assert_tol(out.cpu().numpy(), oracle.dense_attn(f["q_dec"][0], f["k"], f["v"]), "lambda=0 vs dense")


def test_decode_lambda1_is_mean_v():
    w = WORKLOADS["tiny_s1k"].with_(S=1500)
    x = gen.numpy_layer(w, seed=9, steps=1)
    g = run_prefill(x, w.n_kv, 1.0)
    out = ops.decode_attn(dev_bf16(x["q_dec"][0]), None, g["mask"], dev_bf16(x["v"]), g["r"], 1.0)
    torch.cuda.synchronize()
    mean_v = host(x)["v"].astype(np.float64).mean(axis=2)
    assert_tol(out.cpu().numpy(), np.repeat(mean_v, w.G, axis=1), "lambda=1 vs mean V")


def test_decode_split_count_invariance_and_counter_reset():
    w = WORKLOADS["tiny_s1k"].with_(S=5000)
    x = gen.numpy_layer(w, seed=10, steps=1)
    g = run_prefill(x, w.n_kv, 0.5)
    q, v = dev_bf16(x["q_dec"][0]), dev_bf16(x["v"])
    outs = []
    for sp in (1, 2, 7, 0, 79, 79, 0):
        outs.append(ops.decode_attn(q, g["k_packed"], g["mask"], v, g["r"], 0.5, splits=sp).cpu().numpy())
    for o in outs[1:]:
        assert_tol(o, outs[0], "split invariance")
    np.testing.assert_array_equal(outs[4], outs[5])      # same split count: bitwise repeatable
    np.testing.assert_array_equal(outs[3], outs[6])


# ------------------------------------------------------------------ full-size workloads (bench launch config)

@pytest.mark.parametrize("name", ["llama8b_s32k_l05", "llama8b_s32k_l08"])
def test_full_size_s32k(name):
    """The benchmarked shape: all masks bitwise, all decode outputs within tolerance."""
    w = WORKLOADS[name]
    decode_case(w, 0, w.lam, steps=2)


def test_errors_on_device():
    w = WORKLOADS["tiny_s1k"]
    x = gen.numpy_layer(w, seed=0, steps=1)
    g = run_prefill(x, w.n_kv, 0.5)
    small = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    with pytest.raises(ops.SparkError) as e:
        ops.decode_attn(dev_bf16(x["q_dec"][0]), g["k_packed"], g["mask"], dev_bf16(x["v"]), g["r"], 0.5, ws=small)
    assert e.value.status == ops.ENOSPACE


def test_graph_replays_match_eager():
    """Prefill and decode captured in HIP graphs (no memset nodes: counters
    are reset by the kernel itself) give the eager results on every replay,
    with eager work and synchronisations between replays."""
    w = WORKLOADS["tiny_s1k"].with_(S=3000)
    x = gen.numpy_layer(w, seed=11, steps=3)
    q_win, k, v = dev_bf16(x["q_win"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    qs = [dev_bf16(x["q_dec"][s]) for s in range(3)]
    g = run_prefill(x, w.n_kv, 0.8)
    outs = [torch.empty((w.B, w.n_q, 128), dtype=torch.float32, device=DEV) for _ in range(3)]

    def work():
        ops.prefill_prune(q_win, k, w.n_kv, 0.8, out=g)
        for s in range(3):
            ops.decode_attn(qs[s], g["k_packed"], g["mask"], v, g["r"], 0.8, out=outs[s])

    work()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs] + [g["mask"].clone(), g["r"].clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g["mask"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs] + [g["mask"].clone(), g["r"].clone()]
        for a_, b_ in zip(got, eager):
            assert torch.equal(a_, b_), f"replay {rep}"
        work()          # eager work between replays
        torch.cuda.synchronize()


def test_decode_many_splits_s128k():
    """Auto and maximal split counts at S=131072 agree within tolerance."""
    w = WORKLOADS["llama8b_s128k_l08"].with_(n_q=8, n_kv=2)
    x = gen.numpy_layer(w, seed=12, steps=1)
    g = run_prefill(x, w.n_kv, w.lam)
    q, v = dev_bf16(x["q_dec"][0]), dev_bf16(x["v"])
    o_auto = ops.decode_attn(q, g["k_packed"], g["mask"], v, g["r"], w.lam).cpu().numpy()
    o_max = ops.decode_attn(q, g["k_packed"], g["mask"], v, g["r"], w.lam, splits=100000).cpu().numpy()
    o_one = ops.decode_attn(q, g["k_packed"], g["mask"], v, g["r"], w.lam, splits=1).cpu().numpy()
    assert_tol(o_max, o_auto, "max splits")
    assert_tol(o_one, o_auto, "one split")


def test_read_stream_diagnostic_reads_every_word():
    """The bandwidth-ceiling diagnostic folds every 32-bit word exactly once."""
    x = torch.randint(-2**31, 2**31 - 1, (3 * 1024 * 1024 + 4,), dtype=torch.int32, device=DEV)
    for blocks in (1, 7, 512):
        sink = torch.zeros(blocks, dtype=torch.int32, device=DEV)
        ops.read_stream(x, sink, blocks)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(x.cpu().numpy().view(np.uint32))
        assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want
