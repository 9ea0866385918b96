"""Host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

``build()`` compiles the host-only sources of the library (planner,
workspace layout, host entry points, plan validator) with g++ -- no HIP,
no GPU code -- into ``_build/libcpattn_host_check.so``, with the plan
validator switched on (-DCPATTN_CHECK_PLANS): every plan the library
builds is checked record by record, and a bad one turns the call into
CP_EINVAL.

``python tests/sanitize_host.py run LIB`` (started by
tests/test_host_sanitized.py with the sanitizer runtime preloaded) drives
the host entry points through ctypes over the five workloads, random packed
metadata and the argument-error cases, and compares the partition and the
pair counts with a plain-Python owner rule (no numpy: nothing but this
script and the library runs under the sanitizer).
"""
from __future__ import annotations

import ctypes
import os
import random
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_parallelism_amd", "csrc")
LIB = os.path.join(ROOT, "_build", "libcpattn_host_check.so")
SOURCES = ["plan.cpp", "workspace.cpp", "capi_host.cpp", "plan_check.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build() -> str:
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-DCPATTN_CHECK_PLANS",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + SAN +
           [os.path.join(CSRC, s) for s in SOURCES] + ["-o", LIB])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer build failed:\n" + r.stdout + r.stderr)
    return LIB


def runtime_preload() -> str:
    """Path of g++'s ASan runtime, which must load before the library."""
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    return r.stdout.strip()


# ------------------------------------------------------------- the driver

I32 = ctypes.c_int32
I64 = ctypes.c_int64
P32 = ctypes.POINTER(I32)
P64 = ctypes.POINTER(I64)


def _arr(vals):
    a = (I32 * max(1, len(vals)))(*vals)
    return a, ctypes.cast(a, P32)


def owner_rows(cu, n_img, P, r, split):
    """Rank rows by the owner rule: text offset t is in chunk k = t // c;
    head-tail gives chunk k to rank min(k, 2P-1-k), the plain split to k // 2."""
    ids, padded, real = [], 0, 0
    for s in range(len(cu) - 1):
        a, b, n = cu[s], cu[s + 1], n_img[s]
        T = b - a - n
        c = -(-T // (2 * P))
        ids += list(range(a, a + n))
        padded += n * (n + 1) // 2
        real += n * (n + 1) // 2
        for t in range(2 * P * c):
            k = t // c
            own = min(k, 2 * P - 1 - k) if split == 0 else k // 2
            if own == r:
                ids.append(a + n + t if t < T else -1)
                padded += n + t + 1
                real += (n + t + 1) if t < T else 0
    return ids, padded, real


def drive(lib_path: str) -> int:
    lib = ctypes.CDLL(lib_path)
    lib.cp_partition_index_ex.argtypes = [I64, P32, P32, I32, I32, I32, I32, P32, I64, P64, P32]
    lib.cp_pair_counts_ex.argtypes = [I64, P32, P32, I32, I32, I32, I32, P64, P64]
    lib.cp_attn_rank_workspace_size_ex.argtypes = [I64, P32, P32, I32, I32, I32, I32, I32, I32, I32, I32,
                                                   I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.cp_attn_rank_plan_stats_ex.argtypes = [I64, P32, P32, I32, I32, I32, I32, I32, I32, I32, I32,
                                               P64, P64, P64, P64, P64]
    lib.cp_attn_rank_bwd_workspace_size.argtypes = [I64, P32, P32, I32, I32, I32, I32, I32, I32, I32, I32,
                                                    ctypes.POINTER(ctypes.c_size_t)]
    checked = 0

    def one(cu, n_img, P, r, split, shapes):
        nonlocal checked
        n = len(cu) - 1
        T = cu[-1]
        cu_a, cu_p = _arr(cu)
        im_a, im_p = _arr(n_img)
        rows = I64(0)
        assert lib.cp_partition_index_ex(T, im_p, cu_p, n, P, r, split, None, 0, ctypes.byref(rows), None) == 0
        idx = (I32 * max(1, rows.value))()
        cur = (I32 * (n + 1))()
        assert lib.cp_partition_index_ex(T, im_p, cu_p, n, P, r, split, ctypes.cast(idx, P32), rows.value,
                                         ctypes.byref(rows), ctypes.cast(cur, P32)) == 0
        want, padded, real = owner_rows(cu, n_img, P, r, split)
        assert list(idx[:rows.value]) == want, (cu, n_img, P, r, split)
        pp, rr = I64(0), I64(0)
        assert lib.cp_pair_counts_ex(T, im_p, cu_p, n, P, r, split, ctypes.byref(pp), ctypes.byref(rr)) == 0
        assert (pp.value, rr.value) == (padded, real), (cu, n_img, P, r, split)
        for H, Hkv, D, dtype in shapes:
            for sched in (0, 1, 2):
                b = ctypes.c_size_t(0)
                st = lib.cp_attn_rank_workspace_size_ex(T, im_p, cu_p, n, P, r, split, sched, H, Hkv, D, dtype,
                                                        ctypes.byref(b))
                row_tile_ok = dtype == 1 and D == 128
                assert st == (0 if (sched != 1 or row_tile_ok) else -3), (st, cu, P, r, H, Hkv, D, dtype, sched)
            vals = [I64(0) for _ in range(4)]
            steps = (I64 * P)()
            st = lib.cp_attn_rank_plan_stats_ex(T, im_p, cu_p, n, P, r, split, H, Hkv, D, dtype,
                                                *[ctypes.byref(x) for x in vals], ctypes.cast(steps, P64))
            assert st == 0 and vals[3].value == real, (st, cu, P, r)
            b = ctypes.c_size_t(0)
            assert lib.cp_attn_rank_bwd_workspace_size(T, im_p, cu_p, n, P, r, split, H, Hkv, D, dtype,
                                                       ctypes.byref(b)) == 0, (cu, P, r, H, Hkv, D, dtype)
        checked += 1

    # (64 MHA heads: one head per workgroup, 64 head groups per row tile)
    shapes = [(32, 8, 128, 1), (4, 4, 64, 1), (6, 2, 128, 0), (8, 2, 64, 1), (64, 64, 128, 1)]
    # the five workloads' metadata (rank shares only: plans are validated,
    # so the sizes are kept to what runs in seconds)
    workloads = [
        ([0, 256], [0], 2), ([0, 8192], [0], 4), ([0, 18688], [2304], 4), ([0, 65536], [0], 8),
        ([0, 3873, 13871, 19129, 26406, 35638, 44460, 48673, 55689],
         [1320, 2232, 1445, 1306, 2055, 773, 1169, 1916], 4),
    ]
    for cu, n_img, P in workloads:
        for r in range(P):
            one(cu, n_img, P, r, 0, shapes[:1])
    rng = random.Random(1234)
    for trial in range(300):
        n = rng.randint(1, 5)
        lens, imgs = [], []
        for _ in range(n):
            img = rng.randint(0, 70) if rng.random() < 0.6 else 0
            text = rng.randint(0, 400)
            if img + text == 0:
                text = 1
            lens.append(img + text)
            imgs.append(img)
        cu = [0]
        for x in lens:
            cu.append(cu[-1] + x)
        P = rng.randint(1, 9)
        one(cu, imgs, P, rng.randrange(P), trial % 2, shapes)
    # argument errors: statuses, nothing written
    rows = I64(-5)
    cu_a, cu_p = _arr([0, 5, 5, 10])
    assert lib.cp_partition_index_ex(10, None, cu_p, 3, 2, 0, 0, None, 0, ctypes.byref(rows), None) == -1
    assert lib.cp_partition_index_ex(10, None, None, 1, 33, 0, 0, None, 0, ctypes.byref(rows), None) == -3
    assert lib.cp_partition_index_ex(2 ** 31, None, None, 1, 2, 0, 0, None, 0, ctypes.byref(rows), None) == -3
    assert rows.value == -5
    print(f"host planner under the sanitizers: {checked} rank shares checked, plans valid", flush=True)
    return 0


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "run":
        sys.exit(drive(sys.argv[2]))
    print(build())
