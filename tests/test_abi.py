"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects invalid arguments with the documented status before
launching anything (no call here reaches a kernel launch)."""
import ctypes

import numpy as np
import pytest

import oracle
from sparse_decode_attention_amd import ops

FAKE = 0x10000          # 256-byte aligned, never dereferenced: every call below fails validation first
MIS = 0x10008           # 8-byte aligned only


def test_library_exports_every_declared_symbol():
    syms = ops.header_symbols()
    assert {"spark_prefill_prune", "spark_stats", "spark_decode_attn", "spark_num_kept"} <= set(syms)
    l = ops.lib()
    for s in syms:
        assert hasattr(l, s), s
        assert ctypes.cast(getattr(l, s), ctypes.c_void_p).value


def test_num_kept_matches_oracle_rule():
    lams = list(np.linspace(0, 1, 1001)) + [0.5, 0.7, 0.8, 0.2, 1 - 63.5 / 128, 1 - 25.5 / 128]
    for D in (8, 64, 128):
        for lam in lams:
            assert ops.num_kept(D, lam) == oracle.num_kept(D, lam), (D, lam)
    assert ops.num_kept(128, -0.1) == -1 and ops.num_kept(128, 1.5) == -1
    assert ops.num_kept(128, float("nan")) == -1 and ops.num_kept(0, 0.5) == -1


def test_strerror_names_every_status():
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert ops.strerror(st) and ops.strerror(st) != "unknown status"
    assert ops.strerror(7) == "unknown status"


def test_workspace_sizes():
    l = ops.lib()
    assert l.spark_prefill_workspace_bytes(1, 32768, 8, 128) > 0
    assert l.spark_prefill_workspace_bytes(0, 32768, 8, 128) == 0
    n_auto = l.spark_decode_workspace_bytes(1, 32768, 32, 8, 128, 0)
    n_one = l.spark_decode_workspace_bytes(1, 32768, 32, 8, 128, 1)
    assert n_auto > n_one >= ops.DECODE_COUNTER_BYTES
    assert l.spark_decode_workspace_bytes(1, 32768, 30, 8, 128, 0) == 0


def _prefill(**kw):
    a = dict(q_win=FAKE, k=FAKE, B=1, S=64, N_q=32, N_kv=8, D=128, lam=0.5, W=4, qagg=0, rec=0, fc=0.01,
             kp=FAKE, mask=FAKE, A=FAKE, r=FAKE, cnt=FAKE, ws=FAKE, nws=0, st=None)
    a.update(kw)
    return ops.lib().spark_prefill_prune(a["q_win"], a["k"], a["B"], a["S"], a["N_q"], a["N_kv"], a["D"],
                                         a["lam"], a["W"], a["qagg"], a["rec"], a["fc"], a["kp"], a["mask"],
                                         a["A"], a["r"], a["cnt"], a["ws"], a["nws"], a["st"])


def test_prefill_rejects_bad_arguments():
    assert _prefill(B=0) == ops.EINVAL
    assert _prefill(S=0) == ops.EINVAL
    assert _prefill(W=0) == ops.EINVAL
    assert _prefill(lam=1.2) == ops.EINVAL
    assert _prefill(lam=float("nan")) == ops.EINVAL
    assert _prefill(qagg=5) == ops.EINVAL
    assert _prefill(rec=9) == ops.EINVAL
    assert _prefill(N_q=30) == ops.EINVAL
    assert _prefill(N_q=24) == ops.EUNSUPPORTED          # G = 3
    assert _prefill(D=64) == ops.EUNSUPPORTED
    assert _prefill(k=None) == ops.EINVAL
    assert _prefill(mask=None) == ops.EINVAL
    assert _prefill(kp=None) == ops.EINVAL               # T > 0 needs the packed store
    assert _prefill(kp=MIS) == ops.EALIGN
    assert _prefill(ws=FAKE + 16) == ops.EALIGN
    assert _prefill(nws=16) == ops.ENOSPACE


def _decode(**kw):
    a = dict(q=FAKE, kp=FAKE, mask=FAKE, v=FAKE, r=FAKE, B=1, S=64, N_q=32, N_kv=8, D=128, lam=0.5,
             scale=0.0, splits=0, out=FAKE, ws=FAKE, nws=0, st=None)
    a.update(kw)
    return ops.lib().spark_decode_attn(a["q"], a["kp"], a["mask"], a["v"], a["r"], a["B"], a["S"], a["N_q"],
                                       a["N_kv"], a["D"], a["lam"], a["scale"], a["splits"], a["out"], a["ws"],
                                       a["nws"], a["st"])


def test_decode_rejects_bad_arguments():
    assert _decode(S=0) == ops.EINVAL
    assert _decode(splits=-1) == ops.EINVAL
    assert _decode(lam=-0.5) == ops.EINVAL
    assert _decode(scale=float("nan")) == ops.EINVAL
    assert _decode(N_kv=5) == ops.EINVAL
    assert _decode(N_q=16, N_kv=1) == ops.EUNSUPPORTED   # G = 16
    assert _decode(D=256) == ops.EUNSUPPORTED
    assert _decode(B=200, N_kv=8) == ops.ENOSPACE        # 1600 (b, kv head) pairs: counters enough, workspace not
    assert _decode(B=8193, N_kv=8) == ops.EUNSUPPORTED   # more (b, kv head) pairs than counters (65536)
    assert _decode(S=1 << 24) == ops.EUNSUPPORTED         # V rows addressed with 32-bit offsets per head
    assert _decode(v=None) == ops.EINVAL
    assert _decode(out=None) == ops.EINVAL
    assert _decode(q=MIS) == ops.EALIGN
    assert _decode(ws=FAKE + 64) == ops.EALIGN
    assert _decode(nws=ops.DECODE_COUNTER_BYTES) == ops.ENOSPACE


def _decode_sampled(**kw):
    a = dict(q=FAKE, kp=FAKE, mask=FAKE, v=FAKE, A=FAKE, r=FAKE, rec=4, seed=2**64 - 1, B=1, S=64, N_q=32,
             N_kv=8, D=128, lam=0.5, scale=0.0, splits=0, out=FAKE, ws=FAKE, nws=0, st=None)
    a.update(kw)
    return ops.lib().spark_decode_attn_sampled(a["q"], a["kp"], a["mask"], a["v"], a["A"], a["r"], a["rec"],
                                               a["seed"], a["B"], a["S"], a["N_q"], a["N_kv"], a["D"], a["lam"],
                                               a["scale"], a["splits"], a["out"], a["ws"], a["nws"], a["st"])


def test_decode_sampled_rejects_bad_arguments():
    for rec in (0, 1, 2, 3, 6, -1):
        assert _decode_sampled(rec=rec) == ops.EINVAL
    assert _decode_sampled(A=None) == ops.EINVAL
    assert _decode_sampled(A=MIS) == ops.EALIGN
    assert _decode_sampled(r=None) == ops.EINVAL
    assert _decode_sampled(S=0) == ops.EINVAL
    assert _decode_sampled(N_q=24) == ops.EUNSUPPORTED
    assert _decode_sampled(D=64) == ops.EUNSUPPORTED
    assert _decode_sampled(kp=None) == ops.EINVAL
    assert _decode_sampled(kp=None, lam=1.0, nws=0) == ops.ENOSPACE     # T = 0 needs no packed store
    assert _decode_sampled(rec=5) == ops.ENOSPACE
    assert _decode_sampled(nws=ops.DECODE_COUNTER_BYTES) == ops.ENOSPACE


def test_prefill_prune_v_rejects_bad_arguments():
    def call(**kw):
        a = dict(v=FAKE, B=1, S=64, N_kv=8, D=128, lam=0.5, vp=FAKE, vm=FAKE, rv=FAKE, cnt=None, ws=FAKE, nws=0)
        a.update(kw)
        return ops.lib().spark_prefill_prune_v(a["v"], a["B"], a["S"], a["N_kv"], a["D"], a["lam"], a["vp"], a["vm"],
                                               a["rv"], a["cnt"], a["ws"], a["nws"], None)
    assert call(S=0) == ops.EINVAL
    assert call(lam=1.5) == ops.EINVAL
    assert call(D=64) == ops.EUNSUPPORTED
    assert call(v=None) == ops.EINVAL
    assert call(vp=None) == ops.EINVAL                   # T_v > 0 needs the packed store
    assert call(vp=None, lam=1.0) == ops.ENOSPACE        # T_v = 0 does not
    assert call(rv=MIS) == ops.EALIGN
    assert call() == ops.ENOSPACE


def test_decode_kv_rejects_bad_arguments():
    def call(**kw):
        a = dict(q=FAKE, kp=FAKE, km=FAKE, r=FAKE, vp=FAKE, vm=FAKE, rv=FAKE, B=1, S=64, N_q=32, N_kv=8, D=128,
                 lam=0.5, lam_v=0.5, scale=0.0, splits=0, out=FAKE, ws=FAKE, nws=0)
        a.update(kw)
        return ops.lib().spark_decode_attn_kv(a["q"], a["kp"], a["km"], a["r"], a["vp"], a["vm"], a["rv"], a["B"],
                                              a["S"], a["N_q"], a["N_kv"], a["D"], a["lam"], a["lam_v"], a["scale"],
                                              a["splits"], a["out"], a["ws"], a["nws"], None)
    assert call(lam_v=-0.1) == ops.EINVAL
    assert call(vm=None) == ops.EINVAL
    assert call(rv=None) == ops.EINVAL
    assert call(vp=None) == ops.EINVAL
    assert call(vp=None, lam_v=1.0) == ops.ENOSPACE
    assert call(vp=MIS) == ops.EALIGN
    assert call(N_q=24) == ops.EUNSUPPORTED
    assert call() == ops.ENOSPACE


def test_num_kept_vblocks_and_mask_stride():
    assert ops.num_kept_vblocks(128, 0.5) == 8
    assert ops.num_kept_vblocks(128, 0.8) == 3          # floor(3.2 + 0.5)
    assert ops.num_kept_vblocks(128, 0.3) == 11         # floor(11.2 + 0.5)
    assert ops.num_kept_vblocks(128, 0.0) == 16 and ops.num_kept_vblocks(128, 1.0) == 0
    assert ops.num_kept_vblocks(132, 0.5) == -1         # not a multiple of 8
    assert ops.num_kept_vblocks(128, 1.5) == -1
    assert [ops.vblock_mask_stride(S) for S in (0, 1, 64, 65, 4096)] == [0, 64, 64, 128, 4096]


def test_prefill_prune_vblocks_rejects_bad_arguments():
    def call(**kw):
        a = dict(v=FAKE, B=1, S=64, N_kv=8, D=128, lam=0.5, vp=FAKE, vm=FAKE, rv=FAKE, cnt=None, ws=FAKE, nws=0)
        a.update(kw)
        return ops.lib().spark_prefill_prune_vblocks(a["v"], a["B"], a["S"], a["N_kv"], a["D"], a["lam"], a["vp"],
                                                     a["vm"], a["rv"], a["cnt"], a["ws"], a["nws"], None)
    assert call(S=0) == ops.EINVAL
    assert call(lam=1.5) == ops.EINVAL
    assert call(D=64) == ops.EUNSUPPORTED
    assert call(D=60) == ops.EINVAL                      # no whole blocks
    assert call(B=65536, N_kv=1) == ops.EUNSUPPORTED
    assert call(v=None) == ops.EINVAL
    assert call(vm=None) == ops.EINVAL
    assert call(vp=None) == ops.EINVAL                   # n_b > 0 needs the packed store
    assert call(vp=None, lam=1.0) == ops.ENOSPACE        # n_b = 0 does not
    assert call(vm=MIS) == ops.EALIGN
    assert call() == ops.ENOSPACE


def test_decode_kvb_rejects_bad_arguments():
    def call(**kw):
        a = dict(q=FAKE, kp=FAKE, km=FAKE, r=FAKE, vp=FAKE, vm=FAKE, rv=FAKE, B=1, S=64, N_q=32, N_kv=8, D=128,
                 lam=0.5, lam_v=0.5, scale=0.0, splits=0, out=FAKE, ws=FAKE, nws=0)
        a.update(kw)
        return ops.lib().spark_decode_attn_kvb(a["q"], a["kp"], a["km"], a["r"], a["vp"], a["vm"], a["rv"], a["B"],
                                               a["S"], a["N_q"], a["N_kv"], a["D"], a["lam"], a["lam_v"], a["scale"],
                                               a["splits"], a["out"], a["ws"], a["nws"], None)
    assert call(lam_v=-0.1) == ops.EINVAL
    assert call(vm=None) == ops.EINVAL
    assert call(rv=None) == ops.EINVAL
    assert call(vp=None) == ops.EINVAL
    assert call(vp=None, lam_v=1.0) == ops.ENOSPACE
    assert call(vm=MIS) == ops.EALIGN
    assert call(vp=MIS) == ops.EALIGN
    assert call(N_q=24) == ops.EUNSUPPORTED
    assert call(S=1 << 24) == ops.EUNSUPPORTED
    assert call() == ops.ENOSPACE


def test_num_kept_grouped():
    assert ops.num_kept_grouped(128, [0.25, 0.5, 0.75, 1.0]) == 48
    assert ops.num_kept_grouped(128, [0.5]) == ops.num_kept(128, 0.5)
    assert ops.num_kept_grouped(128, [0.0, 1.0]) == 64
    assert ops.num_kept_grouped(128, [0.5] * 8) == 64
    assert ops.num_kept_grouped(128, [0.5] * 3) == -1              # 3 does not divide 128
    assert ops.num_kept_grouped(128, [0.5] * 16) == -1             # more than 8 groups
    assert ops.num_kept_grouped(128, [0.5, 1.5]) == -1
    assert ops.lib().spark_num_kept_grouped(128, 4, None) == -1


def test_prefill_grouped_rejects_bad_arguments():
    def call(ratios=(0.25, 0.5, 0.75, 1.0), **kw):
        a = dict(q_win=FAKE, k=FAKE, B=1, S=64, N_q=32, N_kv=8, D=128, W=4, qagg=0, rec=0, fc=0.01,
                 kp=FAKE, mask=FAKE, A=FAKE, r=FAKE, cnt=FAKE, ws=FAKE, nws=0)
        a.update(kw)
        arr = ops._floats(ratios)
        return ops.lib().spark_prefill_prune_grouped(a["q_win"], a["k"], a["B"], a["S"], a["N_q"], a["N_kv"], a["D"],
                                                     len(ratios), arr, a["W"], a["qagg"], a["rec"], a["fc"], a["kp"],
                                                     a["mask"], a["A"], a["r"], a["cnt"], a["ws"], a["nws"], None)
    assert call(ratios=(0.5, 0.5, 0.5)) == ops.EINVAL
    assert call(ratios=(0.5, -1.0)) == ops.EINVAL
    assert call(rec=6) == ops.EINVAL
    assert call(N_q=24) == ops.EUNSUPPORTED
    assert call(kp=None) == ops.EINVAL
    assert call(kp=None, ratios=(1.0, 1.0)) == ops.ENOSPACE       # T = 0 needs no packed store
    assert call(mask=MIS) == ops.EALIGN
    assert call() == ops.ENOSPACE


def test_topp_entry_points_reject_bad_arguments():
    l = ops.lib()

    def pre(**kw):
        a = dict(q_win=FAKE, k=FAKE, B=1, S=64, N_q=32, N_kv=8, D=128, p=0.99, W=4, qagg=0, rec=0, fc=0.01,
                 kp=FAKE, ro=FAKE, mask=FAKE, A=FAKE, r=FAKE, cnt=None, ws=FAKE, nws=0)
        a.update(kw)
        return l.spark_prefill_prune_topp(a["q_win"], a["k"], a["B"], a["S"], a["N_q"], a["N_kv"], a["D"], a["p"],
                                          a["W"], a["qagg"], a["rec"], a["fc"], a["kp"], a["ro"], a["mask"], a["A"],
                                          a["r"], a["cnt"], a["ws"], a["nws"], None)
    assert pre(p=0.0) == ops.EINVAL
    assert pre(p=1.5) == ops.EINVAL
    assert pre(p=float("nan")) == ops.EINVAL
    assert pre(ro=None) == ops.EINVAL
    assert pre(kp=None) == ops.EINVAL
    assert pre(ro=FAKE + 2) == ops.EALIGN
    assert pre(D=64) == ops.EUNSUPPORTED
    assert pre() == ops.ENOSPACE

    def dec(**kw):
        a = dict(q=FAKE, kp=FAKE, ro=FAKE, mask=FAKE, v=FAKE, r=FAKE, B=1, S=64, N_q=32, N_kv=8, D=128, scale=0.0,
                 splits=0, out=FAKE, ws=FAKE, nws=0)
        a.update(kw)
        return l.spark_decode_attn_ragged(a["q"], a["kp"], a["ro"], a["mask"], a["v"], a["r"], a["B"], a["S"],
                                          a["N_q"], a["N_kv"], a["D"], a["scale"], a["splits"], a["out"], a["ws"],
                                          a["nws"], None)
    assert dec(ro=None) == ops.EINVAL
    assert dec(kp=None) == ops.EINVAL
    assert dec(ro=FAKE + 1) == ops.EALIGN
    assert dec(v=None) == ops.EINVAL
    assert dec(N_q=24) == ops.EUNSUPPORTED
    assert dec() == ops.ENOSPACE


def test_growth_entry_points_reject_bad_arguments():
    l = ops.lib()

    def app(**kw):
        a = dict(kn=FAKE, vn=FAKE, A=FAKE, B=1, N_kv=8, D=128, lam=0.5, pos=10, cap=64, kp=FAKE, mask=FAKE, v=FAKE)
        a.update(kw)
        return l.spark_append_token(a["kn"], a["vn"], a["A"], a["B"], a["N_kv"], a["D"], a["lam"], a["pos"],
                                    a["cap"], a["kp"], a["mask"], a["v"], None)
    assert app(pos=64) == ops.EINVAL
    assert app(pos=-1) == ops.EINVAL
    assert app(lam=2.0) == ops.EINVAL
    assert app(D=64) == ops.EUNSUPPORTED
    assert app(kp=None) == ops.EINVAL
    assert app(v=None) == ops.EINVAL
    assert app(mask=MIS) == ops.EALIGN

    def dec(**kw):
        a = dict(q=FAKE, kp=FAKE, mask=FAKE, v=FAKE, r=FAKE, B=1, S=64, cap=128, N_q=32, N_kv=8, D=128, lam=0.5,
                 scale=0.0, splits=0, out=FAKE, ws=FAKE, nws=0)
        a.update(kw)
        return l.spark_decode_attn_cap(a["q"], a["kp"], a["mask"], a["v"], a["r"], a["B"], a["S"], a["cap"], a["N_q"],
                                       a["N_kv"], a["D"], a["lam"], a["scale"], a["splits"], a["out"], a["ws"],
                                       a["nws"], None)
    assert dec(cap=32) == ops.EINVAL                     # S > S_cap
    assert dec(S=0) == ops.EINVAL
    assert dec(N_q=24) == ops.EUNSUPPORTED
    assert dec() == ops.ENOSPACE


def test_stats_rejects_bad_arguments():
    l = ops.lib()

    def call(**kw):
        a = dict(kp=FAKE, mask=FAKE, A=FAKE, kd=None, B=1, S=64, N_kv=8, D=128, lam=0.5, rec=0, fc=0.0,
                 r=FAKE, cnt=None, ws=FAKE, nws=0)
        a.update(kw)
        return l.spark_stats(a["kp"], a["mask"], a["A"], a["kd"], a["B"], a["S"], a["N_kv"], a["D"], a["lam"],
                             a["rec"], a["fc"], a["r"], a["cnt"], a["ws"], a["nws"], None)
    assert call(rec=3) == ops.EINVAL                     # pruned-score mean needs the dense keys
    assert call(rec=4) == ops.EINVAL                     # so do the sampled F
    assert call(rec=5) == ops.EINVAL
    assert call(kp=None) == ops.EINVAL
    assert call(rec=6, kd=FAKE) == ops.EINVAL
    assert call(D=96) == ops.EUNSUPPORTED
    assert call(mask=MIS) == ops.EALIGN
    assert call() == ops.ENOSPACE


def test_decode_ws_init_checks():
    l = ops.lib()
    assert l.spark_decode_ws_init(None, 4096, None) == ops.EINVAL
    assert l.spark_decode_ws_init(FAKE + 4, 4096, None) == ops.EALIGN
    assert l.spark_decode_ws_init(FAKE, 100, None) == ops.ENOSPACE


def test_read_stream_checks():
    l = ops.lib()
    assert l.spark_read_stream(None, 16, FAKE, 4, None) == ops.EINVAL
    assert l.spark_read_stream(FAKE, 16, FAKE, 0, None) == ops.EINVAL
    assert l.spark_read_stream(FAKE + 8, 16, FAKE, 4, None) == ops.EALIGN
    assert l.spark_read_stream(FAKE, 24, FAKE, 4, None) == ops.EALIGN


def test_window_evict_checks():
    l = ops.lib()
    assert l.spark_window_evict_workspace_bytes(8, 32768, 32, 8, 128, 32) > 0
    assert l.spark_window_evict_workspace_bytes(8, 32768, 30, 8, 128, 32) == 0

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, S=1024, N_q=32, N_kv=8, D=128, W=32, keep=128, idx=FAKE,
                 ko=FAKE, vo=FAKE, sc=None, ws=FAKE, nws=0)
        a.update(kw)
        return l.spark_window_evict(a["q"], a["k"], a["v"], a["B"], a["S"], a["N_q"], a["N_kv"], a["D"], a["W"],
                                    a["keep"], a["idx"], a["ko"], a["vo"], a["sc"], a["ws"], a["nws"], None)
    assert call(keep=0) == ops.EINVAL
    assert call(keep=1025) == ops.EINVAL
    assert call(W=0) == ops.EINVAL
    assert call(W=1025) == ops.EINVAL
    assert call(N_q=30) == ops.EINVAL
    assert call(D=64) == ops.EUNSUPPORTED
    assert call(N_q=64, W=64) == ops.EUNSUPPORTED          # G * W = 512 window rows
    assert call(S=(1 << 20) + 1) == ops.EUNSUPPORTED       # longer than the select takes
    assert call(S=(1 << 20)) == ops.ENOSPACE                # the longest cache passes the size checks
    assert call(ko=None) == ops.EINVAL                      # k_out and v_out go together
    assert call(idx=None) == ops.EINVAL
    assert call(k=MIS) == ops.EALIGN
    assert call(ws=FAKE + 16) == ops.EALIGN
    assert call() == ops.ENOSPACE


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    """The size check of the allocation-free decode runs before anything
    touches a device: a problem whose workspace would exceed the fixed
    scratch returns SPARK_ESCRATCH, invalid sizes SPARK_EINVAL."""
    l = ops.lib()
    B, S, N_q, N_kv = 64, 1 << 20, 32, 8
    assert l.spark_decode_workspace_bytes(B, S, N_q, N_kv, 128, 64) > ops.NOALLOC_SCRATCH_BYTES
    assert l.spark_decode_attn_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, B, S, N_q, N_kv, 128, 0.5, 0.0, 64, FAKE,
                                       None) == ops.ESCRATCH
    assert l.spark_decode_attn_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 30, 8, 128, 0.5, 0.0, 0, FAKE,
                                       None) == ops.EINVAL
