"""GPU parity of the window eviction stage (spark_window_evict) against the oracle.

Scores: |gpu - ref| <= 1e-6 + 2e-3 |ref| (fp32 logits and softmax on bf16
inputs against float64). Kept tokens: the selection is an integer decided by
floating point, so it is certified against the oracle's scores: every token
whose oracle score lies above the oracle's keep-th score by more than the
score tolerance must be kept, every token below it by more than that must
not be; tokens inside that band may go either way (when the band holds no
token, the kept set equals the oracle's exactly). The kept list must be
ascending, unique and of length keep; ties in fp32 go to the lower t.
Gathered rows are checked bit for bit against the inputs at the returned
indices.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops
from sparse_decode_attention_amd.configs import WORKLOADS, Workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
S_RTOL, S_ATOL = 2e-3, 1e-6


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def certify(idx, score_ref, keep, what):
    idx = np.asarray(idx)
    assert idx.shape == (keep,), what
    assert (np.diff(idx) > 0).all(), f"{what}: not ascending / unique"
    order = np.sort(score_ref)[::-1]
    thr = order[keep - 1]
    band = S_ATOL + S_RTOL * abs(thr)
    must = np.nonzero(score_ref > thr + band)[0]
    never = np.nonzero(score_ref < thr - band)[0]
    kept = np.zeros(score_ref.shape[0], dtype=bool)
    kept[idx] = True
    assert kept[must].all(), f"{what}: a clearly kept token is missing"
    assert not kept[never].any(), f"{what}: a clearly evicted token is kept"
    in_band = score_ref.shape[0] - must.size - never.size
    if in_band == 0 or must.size == keep:
        ref_idx = np.sort(np.argsort(-score_ref, kind="stable")[:keep])
        np.testing.assert_array_equal(idx, ref_idx)
    return in_band


def check_case(w: Workload, S: int, keep: int, seed: int = 0):
    x = gen.numpy_layer(w, seed=seed, steps=0, S=S)
    f = {n: gen.bf16_bits_to_f32(v) for n, v in x.items() if n != "q_dec"}
    got = ops.window_evict(gen.to_torch_bf16(x["q_win"], DEV), gen.to_torch_bf16(x["k"], DEV),
                           gen.to_torch_bf16(x["v"], DEV), w.n_kv, keep)
    torch.cuda.synchronize()
    ref_score = oracle.window_scores(f["q_win"], f["k"])
    sc = got["scores"].cpu().numpy().astype(np.float64)
    excess = np.abs(sc - ref_score) - (S_ATOL + S_RTOL * np.abs(ref_score))
    assert (excess <= 0).all(), f"scores: worst excess {excess.max():.3e}"
    idx = got["idx"].cpu().numpy()
    for b in range(w.B):
        for h in range(w.n_kv):
            certify(idx[b, h], ref_score[b, h], keep, f"b{b} h{h}")
            np.testing.assert_array_equal(bits(got["k"][b, h]), x["k"][b, h][idx[b, h]])
            np.testing.assert_array_equal(bits(got["v"][b, h]), x["v"][b, h][idx[b, h]])


def test_evict_tiny():
    w = WORKLOADS["snapkv_b8_s32k_keep4k_l07"]
    check_case(Workload("evict_tiny", w.cfg_id, 1, 1024, 32, 8, 128, 32, 0.7, 0, keep=128), 1024, 128)


@pytest.mark.parametrize("B,S,n_q,n_kv,W,keep", [
    (2, 700, 32, 8, 32, 70),       # ragged S (not a multiple of 16 or of a chunk)
    (1, 1500, 8, 8, 16, 1),        # G = 1, keep = 1
    (1, 600, 16, 2, 8, 600),       # G = 8, keep everything
    (1, 2048, 32, 8, 1, 300),      # one window row per head
])
def test_evict_shapes(B, S, n_q, n_kv, W, keep):
    check_case(Workload("evict_shape", 3, B, S, n_q, n_kv, 128, W, 0.7, 0, keep=keep), S, keep, seed=1)


def test_evict_exact_ties_go_to_lower_t():
    # identical keys: every token before the window gets the same fp32 score,
    # window tokens less (fewer rows see them); keep < S - W selects 0..keep-1
    B, n_q, n_kv, W, S, keep = 1, 32, 8, 32, 512, 100
    rng = np.random.default_rng(5)
    q = torch.from_numpy(rng.standard_normal((B, n_q, W, 128)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    row = torch.from_numpy(rng.standard_normal((1, 1, 1, 128)).astype(np.float32)).to(torch.bfloat16)
    k = row.expand(B, n_kv, S, 128).contiguous().to(DEV)
    v = torch.zeros_like(k)
    got = ops.window_evict(q, k, v, n_kv, keep)
    torch.cuda.synchronize()
    sc = got["scores"].cpu().numpy()
    assert (sc[..., : S - W + 1] == sc[..., :1]).all()
    np.testing.assert_array_equal(got["idx"].cpu().numpy(), np.broadcast_to(np.arange(keep), (B, n_kv, keep)))


def test_evict_full_size_sampled():
    """The stacked-eviction workload at full size (B=8, S=32768, keep 4096):
    scores, selection and gathered rows of sampled (b, KV head) pairs."""
    w = WORKLOADS["snapkv_b8_s32k_keep4k_l07"]
    x = gen.torch_layer(w, DEV, seed=0, steps=0)
    got = ops.window_evict(x["q_win"], x["k"], x["v"], w.n_kv, w.keep)
    torch.cuda.synchronize()
    G = w.n_q // w.n_kv
    for b, h in [(0, 0), (5, 3), (7, 7)]:
        qw = x["q_win"][b:b + 1, h * G:(h + 1) * G].float().cpu().numpy()
        kk = x["k"][b:b + 1, h:h + 1].float().cpu().numpy()
        ref = oracle.window_scores(qw, kk)[0, 0]
        sc = got["scores"][b, h].cpu().numpy().astype(np.float64)
        excess = np.abs(sc - ref) - (S_ATOL + S_RTOL * np.abs(ref))
        assert (excess <= 0).all(), f"b{b} h{h} scores: worst excess {excess.max():.3e}"
        idx = got["idx"][b, h].cpu().numpy()
        certify(idx, ref, w.keep, f"b{b} h{h}")
        sel = torch.from_numpy(idx.astype(np.int64)).to(DEV)
        assert torch.equal(got["k"][b, h], x["k"][b, h].index_select(0, sel))
        assert torch.equal(got["v"][b, h], x["v"][b, h].index_select(0, sel))


def test_evict_beyond_64k_tokens():
    """S = 70000 (more tokens per head than the register-held select takes),
    so the select that re-reads the scores runs: scores, the certified kept
    set and the gathered rows of both KV heads."""
    w = WORKLOADS["snapkv_b8_s32k_keep4k_l07"]
    check_case(Workload("evict_long", 4, 1, 70000, 8, 2, 128, 8, 0.7, 0, keep=5000), 70000, 5000, seed=2)
