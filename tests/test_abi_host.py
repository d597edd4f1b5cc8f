"""CPU-only checks of libsra: it loads, exports every symbol sra.h declares,
its host-only functions agree with the oracle, and every invalid argument
is rejected with the documented status before any HIP call is made."""

import ctypes
import glob
import json
import os
import re

import numpy as np
import pytest
import torch

import oracle
import striped_ring_attention_amd as sra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, INVALID, UNSUPPORTED, HIPERR, WORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    return sra.load()


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(sra_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/*.h but not exported"
    # and the binding declares a prototype for each
    assert set(names) <= set(sra._PROTOS), set(names) - set(sra._PROTOS)


def test_abi_version_matches_header(lib):
    text = open(os.path.join(ROOT, "include", "sra.h")).read()
    v = int(re.search(r"#define SRA_ABI_VERSION (\d+)", text).group(1))
    assert lib.sra_abi_version() == v


def test_status_strings(lib):
    for code, name in ((0, b"SRA_OK"), (1, b"SRA_ERR_INVALID_ARG"), (2, b"SRA_ERR_UNSUPPORTED"),
                       (3, b"SRA_ERR_HIP"), (4, b"SRA_ERR_WORKSPACE")):
        assert lib.sra_status_str(code) == name


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.STRIPED])
@pytest.mark.parametrize("S,N", [(1, 1), (8, 1), (8, 8), (12, 3), (256, 4), (8192, 8), (1536, 16)])
def test_stripe_index_matches_oracle(S, N, layout):
    got = sra.stripe_index(S, N, layout).numpy()
    assert np.array_equal(got, oracle.stripe_index(S, N, layout))


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.STRIPED])
@pytest.mark.parametrize("S,N,tq,tk", [(256, 4, 64, 16), (256, 4, 16, 16), (60, 3, 7, 6), (96, 8, 5, 3),
                                       (1600, 8, 128, 64), (64, 64, 1, 1), (1024, 2, 128, 64)])
def test_tile_census_matches_oracle_enumeration(S, N, tq, tk, layout):
    got = sra.count_live_tiles(S, N, layout, tq, tk)
    want = oracle.live_tiles(S, N, layout, tq, tk)
    for g, w in zip(got, want):
        assert np.array_equal(g.numpy(), w)


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.STRIPED])
@pytest.mark.parametrize("S,N", [(64, 4), (60, 5), (96, 8), (1024, 8)])
def test_live_pairs_match_oracle(S, N, layout):
    assert np.array_equal(sra.count_live_pairs(S, N, layout).numpy(), oracle.live_pairs(S, N, layout))


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "tests", "golden", "census_*.json"))))
def test_census_golden(path):
    rec = json.load(open(path))
    for lname, layout in (("contiguous", oracle.CONTIGUOUS), ("striped", oracle.STRIPED)):
        live, full, part = sra.count_live_tiles(rec["seq"], rec["n_dev"], layout, rec["tile_q"], rec["tile_k"])
        assert live.tolist() == rec[lname]["live"]
        assert full.tolist() == rec[lname]["full"]
        assert part.tolist() == rec[lname]["partial"]
        assert sra.count_live_pairs(rec["seq"], rec["n_dev"], layout).tolist() == rec[lname]["pairs"]


def test_census_at_full_workload_sizes_closed_forms():
    """At the large workloads (too big for brute force) the census follows the
    mask algebra: striped rounds give every device T(T-1)/2 full + T partial
    square tiles; contiguous rounds r >= 1 are all-full or all-empty."""
    for S, N in ((65536, 8), (262144, 8), (786432, 16)):
        T = S // N // 128
        for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
            live, full, part = (t.numpy() for t in sra.count_live_tiles(S, N, layout, 128, 128))
            for r in range(N):
                for d in range(N):
                    src = (d - r) % N
                    if layout == oracle.STRIPED or src == d:
                        assert (full[r, d], part[r, d]) == (T * (T - 1) // 2, T)
                    else:
                        assert (full[r, d], part[r, d]) == ((T * T, 0) if src < d else (0, 0))
        pairs = sra.count_live_pairs(S, N, oracle.STRIPED).numpy()
        assert pairs.sum() == S * (S + 1) // 2


def test_kernel_tiles(lib):
    assert sra.kernel_tiles(torch.bfloat16, 128) == (256, 64)
    assert sra.kernel_tiles(torch.float32, 64) == (64, 16)
    d = sra.make_desc(1, 64, 1, 64, 4, 1, sra.DTYPE_BF16)
    a, b = ctypes.c_int32(), ctypes.c_int32()
    assert lib.sra_kernel_tiles(ctypes.byref(d), ctypes.byref(a), ctypes.byref(b)) == UNSUPPORTED


# --------------------------------------------------- argument validation ---

FAKE = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(1 << 30)


def desc(**kw):
    base = dict(batch=1, seq=64, heads=2, head_dim=128, n_dev=4, layout=1, dtype=sra.DTYPE_BF16, scale=0.0,
                schedule=0, order=0)
    base.update(kw)
    return sra.make_desc(base["batch"], base["seq"], base["heads"], base["head_dim"], base["n_dev"],
                         base["layout"], base["dtype"], base["scale"], base["schedule"], base["order"])


def rr(lib, d, rnd=0, dev=-1, q=FAKE, k=FAKE, v=FAKE, o=FAKE2, l=FAKE2):
    return lib.sra_ring_round_attn(ctypes.byref(d) if d is not None else None, rnd, dev, q, k, v, o, l, None, None)


def test_invalid_descriptors_rejected(lib):
    assert rr(lib, None) == INVALID
    assert rr(lib, desc(seq=63)) == INVALID              # not a multiple of n_dev
    assert rr(lib, desc(n_dev=0)) == INVALID
    assert rr(lib, desc(n_dev=128)) == INVALID           # more devices than tokens
    assert rr(lib, desc(layout=2)) == INVALID
    assert rr(lib, desc(dtype=7)) == INVALID
    assert rr(lib, desc(batch=0)) == INVALID
    assert rr(lib, desc(heads=0)) == INVALID
    assert rr(lib, desc(scale=-1.0)) == INVALID
    assert rr(lib, desc(scale=float("inf"))) == INVALID
    assert rr(lib, desc(schedule=5)) == INVALID
    assert rr(lib, desc(order=2)) == INVALID
    assert rr(lib, desc(order=-1)) == INVALID
    assert b"order" in lib.sra_last_error()
    # original order: one key tile must span < 2^31 bytes (devices x heads x head_dim)
    assert rr(lib, desc(order=1, seq=4096 * 512, n_dev=4096, heads=512)) == UNSUPPORTED
    assert rr(lib, desc(head_dim=64)) == UNSUPPORTED     # bf16 kernel is Dh=128 only
    assert rr(lib, desc(head_dim=96, dtype=sra.DTYPE_F32)) == UNSUPPORTED
    assert b"head_dim" in lib.sra_last_error()


def test_invalid_round_arguments_rejected(lib):
    d = desc()
    assert rr(lib, d, rnd=-1) == INVALID
    assert rr(lib, d, rnd=4) == INVALID
    assert rr(lib, d, dev=4) == INVALID
    assert rr(lib, d, dev=-2) == INVALID
    assert rr(lib, d, q=None) == INVALID
    assert rr(lib, d, l=None) == INVALID
    assert rr(lib, d, k=ctypes.c_void_p((1 << 20) + 2)) == INVALID    # misaligned


def test_invalid_fwd_arguments_rejected(lib):
    d = desc()
    need = lib.sra_fwd_workspace_bytes(ctypes.byref(d))
    assert need == 1 * 64 * 2 * 128 * 4
    fwd = lib.sra_ring_attn_fwd
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE2, FAKE2, None, 0, None, None, None) == WORKSPACE
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE2, FAKE2, ctypes.c_void_p(1 << 40), need - 1, None, None,
               None) == WORKSPACE
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE2, ctypes.c_void_p(1 << 40), need, None, None,
               None) == INVALID                                      # o aliases q
    assert fwd(ctypes.byref(desc(seq=63)), FAKE, FAKE, FAKE, FAKE2, FAKE2, None, 0, None, None, None) == INVALID
    # every written buffer (o, lse, workspace) must be disjoint from q, k, v and from each other
    O, LSE, WS = ctypes.c_void_p(1 << 32), ctypes.c_void_p(1 << 34), ctypes.c_void_p(1 << 36)
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, O, ctypes.c_void_p((1 << 20) + 64), WS, need, None, None,
               None) == INVALID                                      # lse inside q
    assert b"lse" in lib.sra_last_error()
    assert fwd(ctypes.byref(d), FAKE, FAKE2, FAKE, O, LSE, ctypes.c_void_p((1 << 30) + 4096), need, None, None,
               None) == INVALID                                      # workspace inside k
    assert b"workspace" in lib.sra_last_error()
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, O, ctypes.c_void_p((1 << 32) + 256), WS, need, None, None,
               None) == INVALID                                      # lse inside o
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, O, LSE, ctypes.c_void_p((1 << 34) + 16), need, None, None,
               None) == INVALID                                      # workspace overlaps lse
    assert b"overlap" in lib.sra_last_error()
    d1 = desc(n_dev=1)
    assert lib.sra_fwd_workspace_bytes(ctypes.byref(d1)) == 0
    df = desc(dtype=sra.DTYPE_F32, head_dim=64)
    assert lib.sra_fwd_workspace_bytes(ctypes.byref(df)) == 0


def test_invalid_bwd_arguments_rejected(lib):
    d = desc()
    need = lib.sra_bwd_workspace_bytes(ctypes.byref(d))
    assert need == 1 * 64 * 2 * 2 * 4
    bwd = lib.sra_ring_attn_bwd
    Q, K, V, O, LSE, DO = (ctypes.c_void_p(1 << s) for s in (20, 22, 24, 26, 28, 30))
    DQ, DK, DV, WS = (ctypes.c_void_p(1 << s) for s in (32, 34, 36, 38))

    def call(dd=d, **kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=LSE, do=DO, dq=DQ, dk=DK, dv=DV, ws=WS, n=need)
        a.update(kw)
        return bwd(ctypes.byref(dd), a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                   a["ws"], a["n"], None)

    assert call(dd=desc(dtype=sra.DTYPE_F32, head_dim=64)) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(n=need - 1) == WORKSPACE
    assert call(dq=None) == INVALID
    assert call(dk=ctypes.c_void_p((1 << 34) + 8)) == INVALID                  # misaligned
    assert call(dq=ctypes.c_void_p((1 << 20) + 4096)) == INVALID               # dq inside q
    assert call(ws=ctypes.c_void_p((1 << 26) + 64)) == INVALID                 # workspace inside o
    assert b"workspace" in lib.sra_last_error()
    assert call(ws=ctypes.c_void_p((1 << 28) + 16)) == INVALID                 # workspace inside lse
    assert call(dv=ctypes.c_void_p((1 << 28) + 16)) == INVALID                 # dv inside lse
    assert call(ws=ctypes.c_void_p((1 << 36) + 16)) == INVALID                 # workspace inside dv
    assert call(dk=DQ) == INVALID                                              # two gradients alias
    assert b"overlap" in lib.sra_last_error()


def test_noalloc_bwd_validation(lib):
    """The allocation-free backward validates like the workspace form and
    rejects problems larger than its library-held array before any HIP call."""
    nb = lib.sra_ring_attn_bwd_noalloc
    Q, K, V, O, LSE, DO = (ctypes.c_void_p(1 << s) for s in (20, 22, 24, 26, 28, 30))
    DQ, DK, DV = (ctypes.c_void_p(1 << s) for s in (32, 34, 36))
    big = desc(seq=1 << 25, heads=2, n_dev=1024)          # 67,108,864 rows > 33,554,432
    far = [ctypes.c_void_p((i + 1) << 38) for i in range(9)]   # 16 GiB tensors, disjoint
    assert nb(ctypes.byref(big), *far, None) == WORKSPACE
    assert b"allocation-free" in lib.sra_last_error()
    d = desc()
    assert nb(ctypes.byref(d), Q, K, V, O, LSE, DO, None, DK, DV, None) == INVALID
    assert nb(ctypes.byref(d), Q, K, V, O, LSE, DO, ctypes.c_void_p((1 << 20) + 256), DK, DV, None) == INVALID
    assert nb(ctypes.byref(desc(dtype=sra.DTYPE_F32, head_dim=64)), Q, K, V, O, LSE, DO, DQ, DK, DV,
              None) == UNSUPPORTED


def test_invalid_permute_and_merge_rejected(lib):
    P = lib.sra_stripe_permute
    assert P(FAKE, FAKE2, 1, 63, 256, 4, None) == INVALID          # seq % n_dev
    assert P(FAKE, FAKE2, 1, 64, 6, 4, None) == INVALID            # row_bytes % 4
    assert P(FAKE, FAKE2, 0, 64, 256, 4, None) == INVALID          # outer
    assert P(FAKE, FAKE2, 1, 64, (1 << 31) + 4, 4, None) == INVALID   # row too wide for 32-bit element offsets
    assert P(None, FAKE2, 1, 64, 256, 4, None) == INVALID
    assert P(FAKE, ctypes.c_void_p((1 << 20) + 100), 1, 64, 256, 4, None) == INVALID   # overlap
    assert lib.sra_unstripe(FAKE, FAKE2, 1, 64, 256, 0, None) == INVALID
    M = lib.sra_lse_merge
    assert M(FAKE, FAKE, FAKE2, FAKE2, 10, 96, None) == INVALID     # head_dim not a power of two
    assert M(FAKE, FAKE, FAKE2, FAKE2, -1, 128, None) == INVALID
    assert M(None, FAKE, FAKE2, FAKE2, 10, 128, None) == INVALID


def test_invalid_host_calls_rejected(lib):
    buf = (ctypes.c_int64 * 64)()
    assert lib.sra_stripe_index(63, 4, 1, buf) == INVALID
    assert lib.sra_stripe_index(64, 4, 3, buf) == INVALID
    assert lib.sra_stripe_index(64, 4, 1, None) == INVALID
    d = desc()
    assert lib.sra_count_live_tiles(ctypes.byref(d), 0, 16, buf, None, None) == INVALID
    assert lib.sra_count_live_tiles(ctypes.byref(d), 16, 16, None, None, None) == INVALID
    assert lib.sra_count_live_pairs(None, buf) == INVALID


def test_invalid_rope_arguments_rejected(lib):
    R = lib.sra_rope_permute

    def rope(d=None, x=FAKE, y=FAKE2, pos=None, base=10000.0):
        return R(ctypes.byref(d if d is not None else desc()), x, y, pos, base, None)

    assert R(None, FAKE, FAKE2, None, 10000.0, None) == INVALID
    assert rope(desc(seq=63)) == INVALID                   # seq % n_dev
    assert rope(desc(order=3)) == INVALID
    assert rope(desc(dtype=5)) == INVALID
    assert rope(desc(heads=0)) == INVALID
    assert rope(desc(head_dim=12)) == UNSUPPORTED          # not a multiple of 8
    assert rope(desc(head_dim=264)) == UNSUPPORTED         # beyond 256
    assert b"head_dim" in lib.sra_last_error()
    assert rope(base=1.0) == INVALID
    assert rope(base=float("inf")) == INVALID
    assert rope(base=float("nan")) == INVALID
    assert rope(x=None) == INVALID
    assert rope(y=ctypes.c_void_p((1 << 30) + 8)) == INVALID                 # misaligned
    assert rope(pos=ctypes.c_void_p((1 << 30) + 4)) == INVALID               # misaligned positions
    # striped device layout: rows move, so x and y must not overlap at all
    assert rope(desc(layout=oracle.STRIPED), y=FAKE) == INVALID
    assert rope(desc(layout=oracle.STRIPED), y=ctypes.c_void_p((1 << 20) + 4096)) == INVALID
    assert b"overlap" in lib.sra_last_error()
