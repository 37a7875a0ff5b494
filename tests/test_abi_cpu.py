"""C-ABI checks that need no GPU: the library loads, exports every function that
include/bsa.h declares, sizes its buffers as documented, and rejects bad
arguments on the host before anything is enqueued (no kernel is launched here:
every call below fails validation, so no device pointer is ever touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")
from block_sparse_attention_fractal_amd import _lib  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libbsa.so not built")
    return _lib.lib()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.bsa_version() == 520
    for code, name in [(0, "BSA_OK"), (1, "BSA_ERR_INVALID_ARG"), (2, "BSA_ERR_SHAPE"), (3, "BSA_ERR_DTYPE"),
                       (4, "BSA_ERR_UNSUPPORTED"), (5, "BSA_ERR_CAPACITY"), (6, "BSA_ERR_WORKSPACE"),
                       (7, "BSA_ERR_HIP")]:
        assert lib.bsa_status_str(code).decode() == name


def P(B=1, nh=8, T=8, H=32, W=32, D=128, Pp=8, N=64, dtype=1, layout=0):
    return _lib.Problem(B, nh, T, H, W, D, Pp, N, dtype, layout)


def sizes(lib, p):
    vals = [ctypes.c_int64() for _ in range(4)]
    st = lib.bsa_query_sizes(ctypes.byref(p), *[ctypes.byref(v) for v in vals])
    return st, [v.value for v in vals]


@pytest.mark.parametrize("B,nh,T,H,W", [(1, 8, 8, 32, 32), (1, 40, 21, 32, 48), (2, 24, 33, 48, 80), (1, 4, 4, 16, 16)])
def test_query_sizes(lib, B, nh, T, H, W):
    D = 128
    st, (rows, max_nnz, mws, fws) = sizes(lib, P(B, nh, T, H, W, D))
    assert st == 0
    S = T * H * W // 64
    assert rows == B * nh * S and max_nnz == rows * S
    # mask workspace: qp, kp (float64), logits (float64, SIP mode), counts, bitmap, scan chunk
    # sums, SIP row statistics (4 float64 per row); the screened cut's fp16 hi/lo operands of
    # queries and keys, query means, key (mean, exponent) pairs, query norms and exponents,
    # per-head statistics (3 x 8 bytes), the list of rows for the float64 path and its
    # length; each 256-aligned
    a = lambda x: (x + 255) // 256 * 256
    assert mws == (a(rows * D * 8) * 2 + a(rows * S * 8) + a(rows * 4) + a(rows * ((S + 31) // 32) * 4)
                   + a((rows + 1023) // 1024 * 4) + a(rows * 32)
                   + a(rows * 2 * D * 2) + a(B * nh * ((S + 15) // 16) * 16 * 2 * D * 2) + a(rows * 8) + a(rows * 16) + a(rows * 8) + a(rows * 4) + a(B * nh * 24)
                   + a(rows * 4) + a(4))
    # forward workspace: work counters and XCD bounds, per-item cost and order (one int32 each
    # per query-block pair), prepared V
    items = B * nh * ((S + 1) // 2)
    assert fws == 256 + 2 * a(items * 4) + a(B * nh * T * H * W * D * 2)
    assert mws % 256 == 0 and fws % 256 == 0
    aws = ctypes.c_int64()
    assert lib.bsa_query_attend_ws(ctypes.byref(P(B, nh, T, H, W, D)), ctypes.byref(aws)) == 0
    assert aws.value == 256 + 2 * a(items * 4)


def test_query_attend_ws(lib):
    aws = ctypes.c_int64()
    assert lib.bsa_query_attend_ws(ctypes.byref(P(dtype=0)), ctypes.byref(aws)) == 0
    assert aws.value == 256                     # float32: work counters only
    assert lib.bsa_query_attend_ws(ctypes.byref(P()), None) == 1
    assert lib.bsa_query_attend_ws(ctypes.byref(P(dtype=7)), ctypes.byref(aws)) == 3


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 3),                         # dtype
    (dict(layout=5), 1),                        # layout enum
    (dict(H=30), 2),                            # H % P
    (dict(W=20), 2),                            # W % P
    (dict(T=0), 2),                             # non-positive
    (dict(N=32), 4),                            # only N = 64
    (dict(Pp=4, N=64), 4),                      # original layout needs P*P == N
    (dict(D=96), 4),                            # bf16 D in {64, 128}
    (dict(dtype=0, D=96), 4),                   # f32 D in {64, 128}
    (dict(T=65, H=64, W=64), 4),                # S > 4096
    (dict(T=1, H=8, W=12, Pp=4, N=64, layout=1), 2),   # L % N
])
def test_query_sizes_rejects(lib, kw, code):
    st, _ = sizes(lib, P(**kw))
    assert st == code, lib.bsa_last_error().decode()
    assert lib.bsa_last_error().decode() != ""


def test_bf16_head_dim_64_limits(lib):
    """bf16 head_dim 64 is a valid problem (mask, permute, forward); the bf16 backward
    and the bf16 key-group path implement head_dim 128 only and say so on the host."""
    p = P(D=64)
    st, (rows, max_nnz, mws, fws) = sizes(lib, p)
    assert st == 0
    csr = _lib.CSR(FAKE, FAKE, max_nnz, None, None)
    bws = ctypes.c_int64()
    assert lib.bsa_query_backward_ws(ctypes.byref(p), ctypes.byref(bws)) == 0
    assert lib.bsa_backward(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, bws.value, None) == 4
    assert "head_dim" in lib.bsa_last_error().decode()
    vals = [ctypes.c_int64() for _ in range(3)]
    assert lib.bsa_query_group_sizes(ctypes.byref(p), 4, *[ctypes.byref(v) for v in vals]) == 4


def test_fractal_layout_allows_other_patch_sizes(lib):
    st, (rows, *_) = sizes(lib, P(T=2, H=16, W=16, Pp=4, N=64, layout=1))
    assert st == 0 and rows == 8 * 8


FAKE = 1 << 20          # never dereferenced: every call below fails validation first


def _mask_call(lib, p, thr=0.1, win=(-1, -1, -1), mode=0, cap=None, ws_bytes=None, q=FAKE, ws=FAKE, shift=None):
    st, (rows, max_nnz, mws, _) = sizes(lib, p)
    mp = _lib.MaskParams(thr, win[0], win[1], win[2], mode, 7)
    csr = _lib.CSR(FAKE, FAKE, max_nnz if cap is None else cap, None, shift)
    return lib.bsa_build_mask(ctypes.byref(p), ctypes.byref(mp), q, FAKE, ctypes.byref(csr), ws,
                              mws if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(thr=1.0), 1), (dict(thr=-0.1), 1), (dict(thr=float("nan")), 1), (dict(win=(1, -1, 1)), 1),
    (dict(mode=3), 1), (dict(mode=-1), 1), (dict(cap=10), 5), (dict(ws_bytes=1000), 6), (dict(q=None), 1),
    (dict(q=FAKE + 2), 1), (dict(ws=FAKE + 64), 6),
    (dict(mode=1), 1),                                   # SIP without a shift array
    (dict(mode=1, shift=FAKE + 2), 1),                   # misaligned shift array
])
def test_build_mask_rejects_before_launch(lib, kw, code):
    st = _mask_call(lib, P(), **kw)
    assert st == code, lib.bsa_last_error().decode()


def test_window_needs_square_patch_blocks(lib):
    st = _mask_call(lib, P(T=2, H=16, W=16, Pp=4, N=64, layout=1), win=(1, 1, 1))
    assert st == 4


def test_forward_rejects_before_launch(lib):
    p = P()
    st, (rows, max_nnz, mws, fws) = sizes(lib, p)
    csr = _lib.CSR(FAKE, FAKE, max_nnz, None, None)
    f = lib.bsa_forward
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE, fws - 1, None) == 6
    assert f(ctypes.byref(p), FAKE, None, FAKE, ctypes.byref(csr), FAKE, None, FAKE, fws, None) == 1
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, FAKE + 2, FAKE, fws, None) == 1
    bad = P(dtype=7)
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE, fws, None) == 3
    shifted = _lib.CSR(FAKE, FAKE, max_nnz, None, FAKE + 2)          # misaligned shift array
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(shifted), FAKE, None, FAKE, fws, None) == 1


def test_attend_rejects_a_small_workspace(lib):
    p = P()
    st, (rows, max_nnz, mws, fws) = sizes(lib, p)
    aws = ctypes.c_int64()
    assert lib.bsa_query_attend_ws(ctypes.byref(p), ctypes.byref(aws)) == 0
    csr = _lib.CSR(FAKE, FAKE, max_nnz, None, None)
    f = lib.bsa_attend
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE, aws.value - 1, None) == 6
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE + 64, aws.value, None) == 6
    assert f(ctypes.byref(p), FAKE, None, FAKE, ctypes.byref(csr), FAKE, None, FAKE, aws.value, None) == 1


def test_attend_static_rejects_before_touching_the_gpu(lib):
    """bsa_attend_static: null and misaligned pointers, and problems whose work order
    does not fit its 4 MiB static scratch, are rejected on the host."""
    p = P()
    st, (rows, max_nnz, mws, fws) = sizes(lib, p)
    csr = _lib.CSR(FAKE, FAKE, max_nnz, None, None)
    f = lib.bsa_attend_static
    assert f(ctypes.byref(p), FAKE, None, FAKE, ctypes.byref(csr), FAKE, None, None) == 1
    assert f(ctypes.byref(p), FAKE, FAKE + 8, FAKE, ctypes.byref(csr), FAKE, None, None) == 1
    big = P(B=10, nh=110, T=16, H=64, W=64)                  # 1100 heads x 512 query-block pairs
    aws = ctypes.c_int64()
    assert lib.bsa_query_attend_ws(ctypes.byref(big), ctypes.byref(aws)) == 0
    assert aws.value > 4 << 20
    assert f(ctypes.byref(big), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, None) == 6
    assert "static scratch" in lib.bsa_last_error().decode()


def test_training_pair_rejects_before_launch(lib):
    """bsa_attend_train / bsa_backward_train: missing output pair, float32 problems,
    shifted masks and the bf16 backward's head_dim limit are refused on the host."""
    p = P()
    st, (rows, max_nnz, mws, fws) = sizes(lib, p)
    aws, bws = ctypes.c_int64(), ctypes.c_int64()
    assert lib.bsa_query_attend_ws(ctypes.byref(p), ctypes.byref(aws)) == 0
    assert lib.bsa_query_backward_ws(ctypes.byref(p), ctypes.byref(bws)) == 0
    csr = _lib.CSR(FAKE, FAKE, max_nnz, None, None)
    shifted = _lib.CSR(FAKE, FAKE, max_nnz, None, FAKE)
    fa, fb = lib.bsa_attend_train, lib.bsa_backward_train
    assert fa(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE, FAKE, aws.value, None) == 1
    assert fa(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, FAKE, None, FAKE, aws.value, None) == 1
    assert fa(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, FAKE + 8, FAKE, FAKE, aws.value, None) == 1
    assert fa(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(shifted), FAKE, FAKE, FAKE, FAKE, aws.value, None) == 4
    pf = P(dtype=0)
    assert lib.bsa_query_attend_ws(ctypes.byref(pf), ctypes.byref(aws)) == 0
    assert fa(ctypes.byref(pf), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, FAKE, FAKE, FAKE, aws.value, None) == 4
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)   # o, o_lo, lse, dout, dq, dk, dv, ws
    assert fb(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), None, *args[1:], bws.value, None) == 1
    assert fb(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, *args[2:], bws.value, None) == 1
    assert fb(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(shifted), *args, bws.value, None) == 4
    assert lib.bsa_query_backward_ws(ctypes.byref(pf), ctypes.byref(bws)) == 0
    assert fb(ctypes.byref(pf), FAKE, FAKE, FAKE, ctypes.byref(csr), *args, bws.value, None) == 4
    p64 = P(D=64)
    assert lib.bsa_query_backward_ws(ctypes.byref(p64), ctypes.byref(bws)) == 0
    assert fb(ctypes.byref(p64), FAKE, FAKE, FAKE, ctypes.byref(csr), *args, bws.value, None) == 4
    assert "head_dim" in lib.bsa_last_error().decode()


def test_struct_layouts_match_the_header():
    # bsa_mask_params: double, 4 x int32, uint64 -> 32 bytes; bsa_csr: 5 pointer-sized fields
    assert ctypes.sizeof(_lib.MaskParams) == 32 and _lib.MaskParams.seed.offset == 24
    assert ctypes.sizeof(_lib.CSR) == 40 and _lib.CSR.shift.offset == 32


def test_permute_and_pool_reject_before_launch(lib):
    p = P()
    assert lib.bsa_permute(ctypes.byref(p), FAKE, FAKE, 0, None) == 1          # in place
    assert lib.bsa_permute(ctypes.byref(p), FAKE, FAKE + 8, 0, None) == 1      # misaligned
    assert lib.bsa_pool(ctypes.byref(p), FAKE, None, FAKE, FAKE, None) == 1
    assert lib.bsa_block_map(ctypes.byref(P(H=31)), FAKE, FAKE, FAKE, None) == 2


def group_sizes(lib, p, group=4):
    vals = [ctypes.c_int64() for _ in range(3)]
    st = lib.bsa_query_group_sizes(ctypes.byref(p), group, *[ctypes.byref(v) for v in vals])
    return st, [v.value for v in vals]


@pytest.mark.parametrize("B,nh,T,H,W", [(1, 8, 8, 32, 32), (1, 40, 21, 32, 48), (1, 24, 33, 48, 80)])
def test_query_group_sizes(lib, B, nh, T, H, W):
    D = 128
    st, (max_nnz, mws, fws) = group_sizes(lib, P(B, nh, T, H, W, D))
    assert st == 0, lib.bsa_last_error().decode()
    L = T * H * W
    S, SG = L // 64, L // 4
    rows = B * nh * S
    assert max_nnz == rows * SG
    # workspace: query-block means, a chunk of heads of screened group
    # logits (float32 rows of L/4 rounded up to 32 entries, as many heads as fit
    # 2 GiB, at least one), the screen operands (query fp16 hi/lo, whole 16-group
    # tiles of group fp16 hi/lo, query means, group (mean, exponent), query norms
    # and exponents, per-head statistics), the rows left to the float64 path and
    # their count, 256 float64 scratch rows of that path, the entries handed to the
    # exact ranking (count, (mass above, target), 64 (id, mass) pairs per row),
    # counts, bitmap, scan chunk sums
    a = lambda x: (x + 255) // 256 * 256
    pitch = (SG + 31) // 32 * 32
    per_head = S * pitch * 4
    chunk = max(1, min(B * nh, (1 << 31) // per_head))
    assert mws == (a(rows * D * 8) + a(chunk * per_head) + a(rows * 2 * D * 2)
                   + a(B * nh * ((SG + 15) // 16) * 16 * 2 * D * 2) + a(rows * 8) + a(B * nh * SG * 16)
                   + a(rows * 8) + a(rows * 4) + a(B * nh * 3 * 8) + a(rows * 4) + a(4) + a(256 * SG * 8)
                   + a(rows * 4) + a(rows * 16) + a(rows * 64 * 8) + a(rows * 4) + a(rows * ((SG + 31) // 32) * 4) + a((rows + 1023) // 1024 * 4))
    assert fws == 256 + 2 * a(rows * 4) + a(B * nh * L * D * 2)
    aws = ctypes.c_int64()
    assert lib.bsa_query_attend_groups_ws(ctypes.byref(P(B, nh, T, H, W, D)), 4, ctypes.byref(aws)) == 0
    assert aws.value == 256 + 2 * a(rows * 4)
    assert lib.bsa_query_attend_groups_ws(ctypes.byref(P(B, nh, T, H, W, D)), 4, None) == 1
    assert lib.bsa_query_attend_groups_ws(ctypes.byref(P(B, nh, T, H, W, D)), 8, ctypes.byref(aws)) == 4


def test_group_path_rejects_before_launch(lib):
    p = P()
    st, (max_nnz, mws, fws) = group_sizes(lib, p)
    assert st == 0
    assert group_sizes(lib, p, group=8)[0] == 4                       # only 4-token groups
    assert group_sizes(lib, P(B=2, nh=24, T=33, H=48, W=80))[0] == 4  # int32 CSR offsets: split by heads
    mp = _lib.MaskParams(0.1, -1, -1, -1, 0, 0)
    csr = _lib.CSR(FAKE, FAKE, max_nnz, None, None)
    g = lib.bsa_build_group_mask
    small = _lib.CSR(FAKE, FAKE, max_nnz - 1, None, None)
    assert g(ctypes.byref(p), 4, ctypes.byref(mp), FAKE, FAKE, ctypes.byref(small), FAKE, mws, None) == 5
    assert g(ctypes.byref(p), 4, ctypes.byref(mp), FAKE, FAKE, ctypes.byref(csr), FAKE, mws - 1, None) == 6
    sip = _lib.MaskParams(0.1, -1, -1, -1, 1, 0)
    assert g(ctypes.byref(p), 4, ctypes.byref(sip), FAKE, FAKE, ctypes.byref(csr), FAKE, mws, None) == 4
    bad_thr = _lib.MaskParams(1.5, -1, -1, -1, 0, 0)
    assert g(ctypes.byref(p), 4, ctypes.byref(bad_thr), FAKE, FAKE, ctypes.byref(csr), FAKE, mws, None) == 1
    wide = P(T=40, H=64, W=64, nh=1)                                   # L/4 = 40960 groups per head
    st, (mn, mw, _) = group_sizes(lib, wide)
    assert st == 0
    wcsr = _lib.CSR(FAKE, FAKE, mn, None, None)
    assert g(ctypes.byref(wide), 4, ctypes.byref(mp), FAKE, FAKE, ctypes.byref(wcsr), FAKE, mw, None) == 4
    f = lib.bsa_forward_groups
    assert f(ctypes.byref(p), 4, FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE, fws - 1, None) == 6
    assert f(ctypes.byref(p), 4, FAKE, None, FAKE, ctypes.byref(csr), FAKE, None, FAKE, fws, None) == 1
    shifted = _lib.CSR(FAKE, FAKE, max_nnz, None, FAKE)
    assert f(ctypes.byref(p), 4, FAKE, FAKE, FAKE, ctypes.byref(shifted), FAKE, None, FAKE, fws, None) == 4
    assert lib.bsa_attend_groups(ctypes.byref(p), 3, FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE, 256,
                                 None) == 4
    aws = ctypes.c_int64()
    assert lib.bsa_query_attend_groups_ws(ctypes.byref(p), 4, ctypes.byref(aws)) == 0
    assert 256 < aws.value < fws                  # work order, without the prepared V
    a = lib.bsa_attend_groups
    assert a(ctypes.byref(p), 4, FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE, aws.value - 1, None) == 6
    assert a(ctypes.byref(p), 4, FAKE, FAKE, FAKE, ctypes.byref(csr), FAKE, None, FAKE + 64, aws.value, None) == 6
    assert a(ctypes.byref(p), 4, FAKE, None, FAKE, ctypes.byref(csr), FAKE, None, FAKE, aws.value, None) == 1
    f32 = P(dtype=0, D=64)
    assert lib.bsa_prepare_v_groups(ctypes.byref(f32), 4, FAKE, FAKE + 256, None) == 4
