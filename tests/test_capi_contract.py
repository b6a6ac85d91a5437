"""C-ABI contract of libbasedla.so, checked without a GPU.

Loads the library, checks that every function include/based_la.h declares is
exported, and that invalid arguments are rejected with the documented status
before anything is launched (fake, never-dereferenced pointers are used).
"""
import ctypes

import pytest

from recurrent_lm_sequence_amd import based_la as bl

lib = bl.lib
A = 1 << 20  # fake, 16-byte aligned device addresses (never dereferenced: calls fail validation)


def P(x):
    return ctypes.c_void_p(x) if x else None


def test_every_declared_function_is_exported():
    names = bl.declared_functions()
    assert set(names) >= {"bla_feature_dim", "bla_status_string", "based_prefill",
                          "jrt_prefix_prefill", "based_decode_step"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in based_la.h but not exported"


def test_feature_dim():
    assert lib.bla_feature_dim(16) == 273
    assert lib.bla_feature_dim(1) == 3
    assert lib.bla_feature_dim(0) == -1


def test_status_strings():
    for s in range(4):
        assert lib.bla_status_string(s).startswith(b"BLA_")
    assert b"unknown" in lib.bla_status_string(99)


def prefill(B=2, H=2, N=100, d=16, dv=64, it=bl.BLA_BF16, ot=bl.BLA_F32, q=A, k=2 * A, v=3 * A,
            S0=0, z0=0, y=8 * A, S_out=0, z_out=0):
    return lib.based_prefill(B, H, N, d, dv, it, ot, 0.0, P(q), P(k), P(v), P(S0), P(z0), P(y),
                             P(S_out), P(z_out), None)


def jrt(M=10, ke=5 * A, ve=6 * A, **kw):
    B, H, N, d, dv = 2, 2, 100, 16, 64
    return lib.jrt_prefix_prefill(B, H, N, M, d, dv, bl.BLA_BF16, bl.BLA_F32, 0.0, P(A),
                                  P(2 * A), P(3 * A), P(ke), P(ve), None, None, P(8 * A), None,
                                  None, None)


@pytest.mark.parametrize("kw,want", [
    (dict(B=0), bl.BLA_ERR_INVALID),
    (dict(H=-1), bl.BLA_ERR_INVALID),
    (dict(N=-5), bl.BLA_ERR_INVALID),
    (dict(dv=0), bl.BLA_ERR_INVALID),
    (dict(it=7), bl.BLA_ERR_INVALID),
    (dict(ot=-1), bl.BLA_ERR_INVALID),
    (dict(d=8), bl.BLA_ERR_UNSUPPORTED),
    (dict(dv=48), bl.BLA_ERR_UNSUPPORTED),
    (dict(dv=128), bl.BLA_ERR_UNSUPPORTED),
    (dict(q=0), bl.BLA_ERR_INVALID),
    (dict(v=0), bl.BLA_ERR_INVALID),
    (dict(k=2 * A + 8), bl.BLA_ERR_INVALID),           # misaligned
    (dict(S0=9 * A), bl.BLA_ERR_INVALID),              # S0 without z0
    (dict(z0=9 * A), bl.BLA_ERR_INVALID),              # z0 without S0
    (dict(y=A + 64), bl.BLA_ERR_INVALID),              # y overlaps q
    (dict(S0=16 * A, z0=32 * A, S_out=16 * A + 256, z_out=40 * A), bl.BLA_ERR_INVALID),  # partial
    (dict(S_out=16 * A, z_out=16 * A + 1024), bl.BLA_ERR_INVALID),  # outputs overlap each other
])
def test_prefill_rejects_invalid(kw, want):
    assert prefill(**kw) == want


def test_prefill_nothing_to_produce_is_ok():
    # no y, no state outputs: nothing is launched and BLA_OK is returned
    assert prefill(y=0) == bl.BLA_OK


def test_jrt_rejects_missing_prefix_and_negative_m():
    assert jrt(ke=0) == bl.BLA_ERR_INVALID
    assert jrt(ve=0) == bl.BLA_ERR_INVALID
    assert jrt(M=-1) == bl.BLA_ERR_INVALID
    assert jrt(ke=5 * A + 4) == bl.BLA_ERR_INVALID


@pytest.mark.parametrize("args,want", [
    ((0, 16, 16, 64), bl.BLA_ERR_INVALID),
    ((4, 16, 12, 64), bl.BLA_ERR_UNSUPPORTED),
    ((4, 16, 16, 24), bl.BLA_ERR_UNSUPPORTED),
])
def test_decode_rejects_bad_dims(args, want):
    B, H, d, dv = args
    assert lib.based_decode_step(B, H, d, dv, bl.BLA_BF16, bl.BLA_F32, 0.0, P(A), P(2 * A),
                                 P(3 * A), P(16 * A), P(32 * A), P(8 * A), None) == want


def test_decode_rejects_null_state_and_aliasing():
    def call(S=16 * A, z=32 * A, y=8 * A, q=A):
        return lib.based_decode_step(4, 16, 16, 64, bl.BLA_BF16, bl.BLA_F32, 0.0, P(q),
                                     P(2 * A), P(3 * A), P(S), P(z), P(y), None)
    assert call(S=0) == bl.BLA_ERR_INVALID
    assert call(z=0) == bl.BLA_ERR_INVALID
    assert call(q=0) == bl.BLA_ERR_INVALID
    assert call(y=16 * A + 4096) == bl.BLA_ERR_INVALID   # y inside S
    assert call(z=16 * A + 64) == bl.BLA_ERR_INVALID     # z inside S


# ---------------- compact state layout entry points ----------------

def test_compact_dim():
    assert lib.bla_compact_dim(16) == 153
    assert lib.bla_compact_dim(1) == 3
    assert lib.bla_compact_dim(0) == -1
    assert {"bla_compact_dim", "based_prefill_compact", "jrt_prefix_prefill_compact",
            "based_decode_step_compact"} <= set(bl.declared_functions())


def prefill_c(S0=0, z0=0, S_out=0, z_out=0, y=8 * A, N=100, dv=64):
    return lib.based_prefill_compact(2, 2, N, 16, dv, bl.BLA_BF16, bl.BLA_F32, 0.0, P(A), P(2 * A),
                                     P(3 * A), P(S0), P(z0), P(y), P(S_out), P(z_out), None)


@pytest.mark.parametrize("kw", [
    dict(S0=16 * A),                                            # S0 without z0
    dict(S0=16 * A, z0=32 * A, S_out=16 * A + 256, z_out=40 * A),  # partial overlap with S0
    dict(S_out=16 * A, z_out=16 * A + 153 * 64 * 4 * 4 - 16),   # z_out inside the compact S_out
    dict(y=3 * A + 16),                                         # y overlaps v
])
def test_prefill_compact_rejects_invalid(kw):
    assert prefill_c(**kw) == bl.BLA_ERR_INVALID


def test_decode_compact_rejects_aliasing_within_compact_range():
    def call(S=16 * A, z=32 * A, y=8 * A):
        return lib.based_decode_step_compact(4, 16, 16, 64, bl.BLA_BF16, bl.BLA_F32, 0.0, P(A),
                                             P(2 * A), P(3 * A), P(S), P(z), P(y), None)
    # the compact S of 64 heads spans 64 * 153 * 64 * 4 bytes from S
    assert call(z=16 * A + 64 * 153 * 64 * 4 - 16) == bl.BLA_ERR_INVALID
    assert call(S=0) == bl.BLA_ERR_INVALID
    assert lib.based_decode_step_compact(4, 16, 12, 64, bl.BLA_BF16, bl.BLA_F32, 0.0, P(A),
                                         P(2 * A), P(3 * A), P(16 * A), P(32 * A), None,
                                         None) == bl.BLA_ERR_UNSUPPORTED


def test_jrt_ex_rejects_bad_layout_alignment_and_aliasing():
    def call(layout=0, plen=40 * A, y=8 * A):
        return lib.jrt_prefix_prefill_ex(2, 2, 100, 10, 16, 64, bl.BLA_BF16, bl.BLA_F32, 0.0,
                                         P(A), P(2 * A), P(3 * A), P(5 * A), P(6 * A), P(plen),
                                         None, None, P(y), None, None, layout, None)
    assert call(layout=2) == bl.BLA_ERR_INVALID
    assert call(layout=-1) == bl.BLA_ERR_INVALID
    assert call(plen=40 * A + 2) == bl.BLA_ERR_INVALID   # misaligned prefix lengths
    assert call(plen=8 * A + 4) == bl.BLA_ERR_INVALID    # prefix lengths inside y


# ---------------- sliding-window softmax attention ----------------

def swa_pf(B=2, H=2, N=100, d=64, dv=64, w=64, it=bl.BLA_BF16, ot=bl.BLA_F32, q=A, k=2 * A,
           v=3 * A, y=8 * A, kc=0, vc=0):
    return lib.swa_prefill(B, H, N, d, dv, w, it, ot, P(q), P(k), P(v), P(y), P(kc), P(vc), None)


@pytest.mark.parametrize("kw,want", [
    (dict(w=0), bl.BLA_ERR_INVALID),
    (dict(w=257), bl.BLA_ERR_UNSUPPORTED),
    (dict(d=32), bl.BLA_ERR_UNSUPPORTED),
    (dict(dv=128), bl.BLA_ERR_UNSUPPORTED),
    (dict(it=bl.BLA_F32), bl.BLA_ERR_UNSUPPORTED),
    (dict(kc=16 * A), bl.BLA_ERR_INVALID),              # k_cache without v_cache
    (dict(q=A + 8), bl.BLA_ERR_INVALID),                 # misaligned
    (dict(y=2 * A + 64), bl.BLA_ERR_INVALID),            # y overlaps k
    (dict(q=0), bl.BLA_ERR_INVALID),
])
def test_swa_prefill_rejects_invalid(kw, want):
    assert swa_pf(**kw) == want


def test_swa_decode_rejects_invalid():
    def call(pos=5, w=64, d=64, kc=16 * A, vc=32 * A, y=8 * A):
        return lib.swa_decode_step(2, 2, d, 64, w, pos, bl.BLA_BF16, bl.BLA_F32, P(A), P(2 * A),
                                   P(3 * A), P(kc), P(vc), P(y), None)
    assert call(pos=-1) == bl.BLA_ERR_INVALID
    assert call(kc=0) == bl.BLA_ERR_INVALID
    assert call(w=0) == bl.BLA_ERR_INVALID
    assert call(d=16) == bl.BLA_ERR_UNSUPPORTED
    assert call(y=16 * A + 64) == bl.BLA_ERR_INVALID     # y inside the key cache


def test_launches_beyond_the_work_item_limit_are_unsupported():
    # 2^23 heads (one workgroup each) exceed the 2^22-workgroup limit of one dispatch;
    # validation rejects them before anything is launched
    assert prefill(B=1 << 12, H=1 << 11, N=1) == bl.BLA_ERR_UNSUPPORTED
    assert lib.based_decode_step(1 << 12, 1 << 11, 16, 64, bl.BLA_BF16, bl.BLA_F32, 0.0, P(A),
                                 P(2 * A), P(3 * A), P(4 * A), P(8 * A), P(16 * A),
                                 None) == bl.BLA_ERR_UNSUPPORTED
    # sliding-window prefill: one workgroup per head and 128-query tile
    assert swa_pf(B=1 << 11, H=1 << 11, N=129) == bl.BLA_ERR_UNSUPPORTED


def test_1024_thread_prefill_heads_limit():
    # the bf16-input prefill (every d_v) and the fp32-input prefill at d_v <= 32 run
    # 1024 threads per head: 2^21 heads is the most one dispatch can carry, so
    # 2^21 + 1 heads is unsupported
    for kw in (dict(dv=32, it=bl.BLA_F32), dict(dv=16, it=bl.BLA_F32), dict(dv=64, it=bl.BLA_BF16),
               dict(dv=32, it=bl.BLA_BF16), dict(dv=16, it=bl.BLA_BF16)):
        assert prefill(B=(1 << 11) + 1, H=1 << 10, N=1, **kw) == bl.BLA_ERR_UNSUPPORTED
        # 2^21 heads pass validation (the call then fails on the overlapping fake
        # pointers, which proves the head count was accepted)
        assert prefill(B=1 << 11, H=1 << 10, N=1, **kw) == bl.BLA_ERR_INVALID
    # fp32 inputs at d_v = 64 run 512 threads per head
    assert prefill(B=(1 << 11) + 1, H=1 << 10, N=1, dv=64, it=bl.BLA_F32) == bl.BLA_ERR_INVALID


def test_per_head_length_limit():
    # a head's rows are addressed with 32-bit byte offsets: N * d_v * 4 (and M * d_v * 4)
    # must stay below 2^31.  The largest supported length passes validation (the call
    # then fails on the overlapping fake pointers); one token more is unsupported
    for dv in (16, 32, 64):
        n_max = ((1 << 31) - 1) // (dv * 4)
        assert prefill(B=1, H=1, N=n_max + 1, dv=dv) == bl.BLA_ERR_UNSUPPORTED
        assert prefill(B=1, H=1, N=n_max, dv=dv) == bl.BLA_ERR_INVALID
    n_max = ((1 << 31) - 1) // 256
    assert n_max == 8388607
    for M, want in ((n_max + 1, bl.BLA_ERR_UNSUPPORTED), (n_max, bl.BLA_ERR_INVALID)):
        assert lib.jrt_prefix_prefill(1, 1, 100, M, 16, 64, bl.BLA_BF16, bl.BLA_F32, 0.0, P(A),
                                      P(2 * A), P(3 * A), P(5 * A), P(6 * A), None, None,
                                      P(8 * A), None, None, None) == want
