"""CPU tests of the C ABI: the library loads and exports every declared
entry point; the host planner matches the oracle bit-exactly; every
argument error returns its status and writes nothing. No GPU calls."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


@pytest.fixture(scope="module")
def cp():
    import context_parallelism_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(cp_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(cp):
    names = declared_functions()
    assert "cp_attn_rank_fwd" in names and "cp_partition_index" in names
    lib = ctypes.CDLL(cp.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    bound = {s[0] for s in cp.SIGNATURES}
    assert set(names) == bound


def test_status_strings(cp):
    for code in (cp.CP_OK, cp.CP_EINVAL, cp.CP_ENOSPC, cp.CP_EUNSUPPORTED, cp.CP_EHIP):
        assert cp.cp_status_string(code) != "unknown status"
    assert cp.cp_status_string(12345) == "unknown status"


def test_partition_matches_oracle_on_workloads(cp):
    for w in workloads.WORKLOADS.values():
        cu = w.cu_seqlens
        for r in range(w.cp_size):
            a, acu = cp.partition_index(w.seq_len, w.n_img, cu, cp_size=w.cp_size, cp_rank=r)
            b, bcu = oracle.partition_index(w.seq_len, w.n_img, cu, w.cp_size, r)
            assert np.array_equal(a, b) and np.array_equal(acu, bcu)
            assert cp.pair_counts(w.seq_len, w.n_img, cu, cp_size=w.cp_size, cp_rank=r) == \
                oracle.pair_counts(w.seq_len, w.n_img, cu, w.cp_size, r)


def test_partition_matches_oracle_random(cp):
    rng = np.random.default_rng(1)
    for trial in range(300):
        n = int(rng.integers(1, 6))
        n_img, cu = workloads.random_meta(rng, n, 40, 200)
        T = int(cu[-1])
        P = int(rng.integers(1, 9))
        r = int(rng.integers(0, P))
        a, acu = cp.partition_index(T, n_img, cu, cp_size=P, cp_rank=r)
        b, bcu = oracle.partition_index(T, n_img, cu, P, r)
        assert np.array_equal(a, b) and np.array_equal(acu, bcu), (trial, n_img, cu, P, r)
        assert cp.pair_counts(T, n_img, cu, cp_size=P, cp_rank=r) == oracle.pair_counts(T, n_img, cu, P, r)


def test_contiguous_split_matches_oracle(cp):
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 5))
        n_img, cu = workloads.random_meta(rng, n, 40, 200)
        T = int(cu[-1])
        P = int(rng.integers(1, 9))
        r = int(rng.integers(0, P))
        a, acu = cp.partition_index(T, n_img, cu, cp_size=P, cp_rank=r, split="contiguous")
        b, bcu = oracle.partition_index(T, n_img, cu, P, r, split="contiguous")
        assert np.array_equal(a, b) and np.array_equal(acu, bcu), (trial, n_img, cu, P, r)
        assert cp.pair_counts(T, n_img, cu, cp_size=P, cp_rank=r, split="contiguous") == \
            oracle.pair_counts(T, n_img, cu, P, r, split="contiguous")
        H, Hkv = [(4, 4), (8, 2)][trial % 2]
        st = cp.plan_stats(T, n_img, cu, cp_size=P, cp_rank=r, heads=H, kv_heads=Hkv, head_dim=128,
                           dtype=trial % 2, split="contiguous")
        assert st["covered_pairs"] == oracle.pair_counts(T, n_img, cu, P, r, split="contiguous")[1]
    # ring steps of the plain split: rank r sees source ranks j <= r only
    L, P = 8192, 4
    c = L // (2 * P)
    for r in range(P):
        st = cp.plan_stats(L, cp_size=P, cp_rank=r, heads=4, kv_heads=4, head_dim=128, dtype=1,
                           split="contiguous")
        want = [0] * P
        for s in range(P):
            j = (r - s) % P
            want[s] = (2 * c) * (2 * c + 1) // 2 if j == r else (4 * c * c if j < r else 0)
        assert st["step_pairs"] == want, (r, st["step_pairs"], want)


def test_unknown_split_is_rejected(cp):
    idx = np.full(4, 77, np.int32)
    rows = ctypes.c_int64(-5)
    st = cp.cp_partition_index_ex(16, None, None, 1, 2, 0, 7, idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  4, ctypes.byref(rows), None)
    assert st == cp.CP_EUNSUPPORTED and rows.value == -5 and np.all(idx == 77)


def test_single_sample_null_meta(cp):
    a, _ = cp.partition_index(1000, cp_size=3, cp_rank=2)
    b, _ = oracle.partition_index(1000, None, None, 3, 2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", [0, 1])
def test_schedule_covers_every_visible_pair_once(cp, dtype):
    # the work list's spans expose exactly the rank's visible pairs, and by
    # ring step: step 0 holds 2c^2 + c (+ image terms), every other step 2c^2
    rng = np.random.default_rng(2)
    for trial in range(60):
        n = int(rng.integers(1, 4))
        n_img, cu = workloads.random_meta(rng, n, 70, 400)
        T = int(cu[-1])
        P = int(rng.integers(1, 7))
        r = int(rng.integers(0, P))
        H, Hkv = [(4, 4), (8, 2), (8, 4), (6, 3)][trial % 4]
        st = cp.plan_stats(T, n_img, cu, cp_size=P, cp_rank=r, heads=H, kv_heads=Hkv,
                           head_dim=128, dtype=dtype)
        assert st["covered_pairs"] == oracle.pair_counts(T, n_img, cu, P, r)[1]
        assert sum(st["step_pairs"]) == st["covered_pairs"]
    for w in workloads.WORKLOADS.values():
        if w.n_samples != 1 or any(w.n_img):
            continue
        c = w.seq_len // (2 * w.cp_size)
        for r in range(w.cp_size):
            st = cp.plan_stats(w.seq_len, cp_size=w.cp_size, cp_rank=r, heads=w.heads,
                               kv_heads=w.kv_heads, head_dim=w.head_dim, dtype=dtype)
            assert st["step_pairs"] == [2 * c * c + c] + [2 * c * c] * (w.cp_size - 1)
    w = workloads.get(3)
    n, c = w.n_img[0], w.text_len[0] // (2 * w.cp_size)
    st = cp.plan_stats(w.seq_len, w.n_img, None, cp_size=w.cp_size, cp_rank=w.rank, heads=w.heads,
                       kv_heads=w.kv_heads, head_dim=w.head_dim, dtype=1)
    assert st["step_pairs"][0] == 2 * c * c + c + n * (n + 1) // 2 + 2 * c * n
    assert st["step_pairs"][1:] == [2 * c * c] * (w.cp_size - 1)


def test_schedule_argument(cp):
    # CP_SCHED_*: the per-step schedule holds the step partials in the
    # workspace, the row-tile schedule only the plan; row tiles exist for
    # bf16 head_dim 128 only; unknown values are refused and write nothing
    kw = dict(cp_size=4, cp_rank=1, heads=8, kv_heads=2, head_dim=128)
    row = cp.workspace_size(5000, dtype=1, schedule="row_tile", **kw)
    step = cp.workspace_size(5000, dtype=1, schedule="per_step", **kw)
    auto = cp.workspace_size(5000, dtype=1, **kw)
    R, H, D, P = 2 * 625, 8, 128, 4
    assert step - row >= P * R * H * D * 4 + P * H * R * 4
    assert auto == step  # 10 row tiles x 4 head groups is below 512 workgroups
    for dtype, hd in ((0, 128), (1, 64), (0, 64)):
        with pytest.raises(cp.CpError) as e:
            cp.workspace_size(5000, dtype=dtype, schedule="row_tile", **dict(kw, head_dim=hd))
        assert e.value.status == cp.CP_EUNSUPPORTED
        assert cp.workspace_size(5000, dtype=dtype, schedule="per_step", **dict(kw, head_dim=hd)) == \
            cp.workspace_size(5000, dtype=dtype, **dict(kw, head_dim=hd))
    b = ctypes.c_size_t(12345)
    st = cp.cp_attn_rank_workspace_size_ex(5000, None, None, 1, 4, 1, 0, 3, 8, 2, 128, 1, ctypes.byref(b))
    assert st == cp.CP_EUNSUPPORTED and b.value == 12345
    fake = ctypes.c_void_p(4096)
    st = cp.cp_attn_rank_fwd_ex(fake, fake, fake, 1, 5000, None, None, 1, 4, 1, 0, 3, 8, 2, 128, fake, fake,
                                ctypes.c_void_p(1 << 20), 1 << 30, None, None)
    assert st == cp.CP_EUNSUPPORTED
    with pytest.raises(ValueError):
        cp.workspace_size(5000, dtype=1, schedule="rows", **kw)


def test_workspace_size_grows_with_problem(cp):
    a = cp.workspace_size(1000, cp_size=2, cp_rank=0, heads=4, kv_heads=4, head_dim=128, dtype=1)
    b = cp.workspace_size(2000, cp_size=2, cp_rank=0, heads=4, kv_heads=4, head_dim=128, dtype=1)
    c = cp.workspace_size(1000, cp_size=2, cp_rank=0, heads=4, kv_heads=4, head_dim=128, dtype=0)
    assert 0 < a < b and 0 < c and a % 256 == 0 and c % 256 == 0


# ------------------------------------------------------------------ errors

I32 = ctypes.POINTER(ctypes.c_int32)


def arr(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(I32)


def part(cp, seq_len, n_img, cu, n, P, r, cap=64):
    """Call cp_partition_index into a canary-filled buffer; returns (status, untouched)."""
    buf = np.full(cap, 7777, np.int32)
    rows = ctypes.c_int64(-5)
    img_a = None if n_img is None else arr(n_img)
    cu_a = None if cu is None else arr(cu)
    st = cp.cp_partition_index(seq_len, None if img_a is None else img_a[1],
                               None if cu_a is None else cu_a[1], n, P, r,
                               buf.ctypes.data_as(I32), cap, ctypes.byref(rows), None)
    return st, bool(np.all(buf == 7777)) and rows.value == -5


@pytest.mark.parametrize("args,code", [
    ((10, None, None, 1, 0, 0), "CP_EINVAL"),           # cp_size < 1
    ((10, None, None, 1, 2, 2), "CP_EINVAL"),           # rank out of range
    ((10, None, None, 1, 2, -1), "CP_EINVAL"),
    ((10, None, None, 1, 33, 0), "CP_EUNSUPPORTED"),    # cp_size above 32
    ((10, None, None, 2, 2, 0), "CP_EINVAL"),           # NULL cu_seqlens needs one sample
    ((0, None, None, 1, 2, 0), "CP_EINVAL"),            # empty single sample
    ((10, None, [1, 10], 1, 2, 0), "CP_EINVAL"),        # cu[0] != 0
    ((10, None, [0, 5, 5, 10], 3, 2, 0), "CP_EINVAL"),  # not strictly increasing
    ((10, None, [0, 4, 9], 2, 2, 0), "CP_EINVAL"),      # last != seq_len
    ((10, [11], None, 1, 2, 0), "CP_EINVAL"),           # image longer than sample
    ((10, [-1], None, 1, 2, 0), "CP_EINVAL"),           # negative image
    ((2 ** 31, None, None, 1, 2, 0), "CP_EUNSUPPORTED"),  # seq_len >= 2^31
    ((-1, None, None, 1, 2, 0), "CP_EINVAL"),
])
def test_partition_errors_write_nothing(cp, args, code):
    st, untouched = part(cp, *args)
    assert st == getattr(cp, code)
    assert untouched


def test_partition_capacity(cp):
    st, untouched = part(cp, 100, None, None, 1, 1, 0, cap=99)  # one rank: 100 rows
    assert st == cp.CP_ENOSPC and untouched
    st, _ = part(cp, 100, None, None, 1, 1, 0, cap=100)
    assert st == cp.CP_OK


def ws_status(cp, heads=4, kv_heads=4, head_dim=128, dtype=1, seq_len=100, P=2, r=0):
    b = ctypes.c_size_t(12345)
    st = cp.cp_attn_rank_workspace_size(seq_len, None, None, 1, P, r, heads, kv_heads, head_dim, dtype,
                                        ctypes.byref(b))
    return st, b.value


@pytest.mark.parametrize("kw,code", [
    (dict(heads=6, kv_heads=4), "CP_EINVAL"),
    (dict(heads=0), "CP_EINVAL"),
    (dict(kv_heads=0), "CP_EINVAL"),
    (dict(head_dim=96), "CP_EUNSUPPORTED"),
    (dict(head_dim=256), "CP_EUNSUPPORTED"),
    (dict(dtype=2), "CP_EUNSUPPORTED"),
    (dict(r=5), "CP_EINVAL"),
])
def test_workspace_size_errors(cp, kw, code):
    st, b = ws_status(cp, **kw)
    assert st == getattr(cp, code) and b == 12345


def test_fwd_argument_errors_before_any_device_work(cp):
    # argument checks run before any HIP call, so these are CPU-safe
    fake = ctypes.c_void_p(4096)  # never dereferenced: the call must fail first
    ok_ws = ws_status(cp)[1]

    def fwd(**kw):
        a = dict(q=fake, k=fake, v=fake, dtype=1, seq_len=100, n_img=None, cu=None, n=1, P=2, r=0,
                 H=4, Hkv=4, D=128, out=fake, lse=fake, ws=ctypes.c_void_p(1 << 20), wsb=ok_ws)
        a.update(kw)
        return cp.cp_attn_rank_fwd(a["q"], a["k"], a["v"], a["dtype"], a["seq_len"], a["n_img"],
                                   a["cu"], a["n"], a["P"], a["r"], a["H"], a["Hkv"], a["D"], a["out"],
                                   a["lse"], a["ws"], a["wsb"], None)
    assert fwd(q=None) == cp.CP_EINVAL
    assert fwd(out=None) == cp.CP_EINVAL
    assert fwd(ws=None) == cp.CP_EINVAL
    assert fwd(ws=ctypes.c_void_p((1 << 20) + 4)) == cp.CP_EINVAL  # workspace alignment
    assert fwd(q=ctypes.c_void_p(4098)) == cp.CP_EINVAL  # q alignment
    assert fwd(wsb=ok_ws - 1) == cp.CP_ENOSPC
    assert fwd(D=80) == cp.CP_EUNSUPPORTED
    assert fwd(dtype=7) == cp.CP_EUNSUPPORTED
    assert fwd(H=6) == cp.CP_EINVAL
    assert fwd(P=0) == cp.CP_EINVAL
    assert fwd(seq_len=2 ** 31) == cp.CP_EUNSUPPORTED


def test_gather_and_merge_argument_errors(cp):
    fake = ctypes.c_void_p(4096)
    assert cp.cp_gather_rows(fake, 5, 10, 64, fake, 4, fake, None) == cp.CP_EUNSUPPORTED
    assert cp.cp_gather_rows(fake, 1, 10, 4, fake, 4, fake, None) == cp.CP_EUNSUPPORTED  # 8-byte rows
    assert cp.cp_gather_rows(None, 1, 10, 64, fake, 4, fake, None) == cp.CP_EINVAL
    assert cp.cp_gather_rows(fake, 1, 10, 64, fake, 0, fake, None) == cp.CP_OK  # nothing to do
    assert cp.cp_lse_merge(fake, fake, fake, 0, 4, 2, 128, 1, fake, fake, None) == cp.CP_EINVAL
    assert cp.cp_lse_merge(fake, fake, fake, 33, 4, 2, 128, 1, fake, fake, None) == cp.CP_EUNSUPPORTED
    assert cp.cp_lse_merge(fake, fake, fake, 2, 4, 2, 96, 1, fake, fake, None) == cp.CP_EUNSUPPORTED
    assert cp.cp_lse_merge(None, fake, fake, 2, 4, 2, 128, 1, fake, fake, None) == cp.CP_EINVAL


def test_zero_row_problem(cp):
    a, cu_rows = cp.partition_index(0, None, np.array([0], np.int32), cp_size=4, cp_rank=1)
    assert a.size == 0 and list(cu_rows) == [0]
    assert cp.pair_counts(0, None, np.array([0], np.int32), cp_size=4, cp_rank=1) == (0, 0)


def bwd_ws_status(cp, heads=4, kv_heads=4, head_dim=128, dtype=1, seq_len=100, P=2, r=0, split=0):
    b = ctypes.c_size_t(12345)
    st = cp.cp_attn_rank_bwd_workspace_size(seq_len, None, None, 1, P, r, split, heads, kv_heads, head_dim,
                                            dtype, ctypes.byref(b))
    return st, b.value


@pytest.mark.parametrize("kw,code", [
    (dict(heads=6, kv_heads=4), "CP_EINVAL"),
    (dict(head_dim=96), "CP_EUNSUPPORTED"),
    (dict(head_dim=256), "CP_EUNSUPPORTED"),
    (dict(dtype=2), "CP_EUNSUPPORTED"),
    (dict(r=2), "CP_EINVAL"),
    (dict(P=0), "CP_EINVAL"),
    (dict(split=5), "CP_EUNSUPPORTED"),
])
def test_bwd_workspace_size_errors(cp, kw, code):
    st, b = bwd_ws_status(cp, **kw)
    assert st == getattr(cp, code) and b == 12345


def test_bwd_workspace_size_grows_with_problem(cp):
    st_a, a = bwd_ws_status(cp, seq_len=1000)
    st_b, b = bwd_ws_status(cp, seq_len=2000)
    assert st_a == st_b == cp.CP_OK and 0 < a < b
    # every forward dtype and head_dim has a backward; fp32 holds a wider Q copy
    st_c, c = bwd_ws_status(cp, seq_len=1000, dtype=0)
    st_d, d = bwd_ws_status(cp, seq_len=1000, head_dim=64)
    assert st_c == st_d == cp.CP_OK and c > a and 0 < d


def test_bwd_argument_errors_before_any_device_work(cp):
    # argument checks run before any HIP call, so these are CPU-safe
    fake = ctypes.c_void_p(4096)  # never dereferenced: the call must fail first
    ok_ws = bwd_ws_status(cp)[1]

    def bwd(**kw):
        a = dict(q=fake, k=fake, v=fake, out=fake, lse=fake, dout=fake, dtype=1, seq_len=100, cu=None, n=1,
                 P=2, r=0, H=4, Hkv=4, D=128, dq=fake, dk=fake, dv=fake, ws=ctypes.c_void_p(1 << 20), wsb=ok_ws)
        a.update(kw)
        return cp.cp_attn_rank_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dtype"],
                                   a["seq_len"], None, a["cu"], a["n"], a["P"], a["r"], 0, a["H"], a["Hkv"],
                                   a["D"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None)
    for name in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "ws"):
        assert bwd(**{name: None}) == cp.CP_EINVAL, name
    assert bwd(ws=ctypes.c_void_p((1 << 20) + 4)) == cp.CP_EINVAL  # workspace alignment
    assert bwd(dq=ctypes.c_void_p(4100)) == cp.CP_EINVAL  # 16-byte alignment of the gradients
    assert bwd(wsb=ok_ws - 1) == cp.CP_ENOSPC
    assert bwd(D=96) == cp.CP_EUNSUPPORTED
    assert bwd(dtype=3) == cp.CP_EUNSUPPORTED
    assert bwd(H=6) == cp.CP_EINVAL
    assert bwd(r=3) == cp.CP_EINVAL
    assert bwd(seq_len=2 ** 31) == cp.CP_EUNSUPPORTED
    # an empty packed batch (cu_seqlens = [0]) is a valid problem with nothing to do
    zero = np.array([0], np.int32)
    cu0 = zero.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert bwd(seq_len=0, cu=cu0, n=0, q=None, out=None, lse=None, dout=None, dq=None) == cp.CP_OK


def test_noalloc_refuses_a_plan_beyond_its_scratch_before_device_work(cp):
    # cp_attn_rank_fwd_noalloc: 3M rank rows need 24 MB of row index and step
    # masks, beyond its 16 MiB scratch; refused before any HIP call (the fake
    # pointers are never read), and argument errors as for cp_attn_rank_fwd
    fake = ctypes.c_void_p(4096)
    assert cp.CP_NOALLOC_SCRATCH_BYTES == 16 << 20
    st = cp.cp_attn_rank_fwd_noalloc(fake, fake, fake, 1, 3_000_000, None, None, 1, 1, 0, 2, 2, 128, fake,
                                     fake, None)
    assert st == cp.CP_ENOSPC
    assert cp.cp_attn_rank_fwd_noalloc(None, fake, fake, 1, 100, None, None, 1, 2, 0, 4, 4, 128, fake, fake,
                                       None) == cp.CP_EINVAL
    assert cp.cp_attn_rank_fwd_noalloc(fake, fake, fake, 1, 100, None, None, 1, 2, 0, 4, 4, 96, fake, fake,
                                       None) == cp.CP_EUNSUPPORTED
    assert cp.cp_attn_rank_fwd_noalloc(fake, fake, fake, 1, 100, None, None, 1, 2, 2, 4, 4, 128, fake, fake,
                                       None) == cp.CP_EINVAL
