"""The C ABI without a GPU: the library loads, it exports every function the
header declares, and muon_plan rejects bad arguments before any HIP call."""

import ctypes
import math
import os
import re

import pytest

from matrix_optimizer_step_muon_amd import muon

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(muon_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("muon_plan", "muon_step", "muon_plan_destroy", "muon_last_error",
                     "muon_plan_workspace_bytes", "muon_hparams_default"):
        assert required in names
    assert sorted(muon.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = muon.lib()
    for name in header_functions():
        assert hasattr(L, name), name


def test_hparams_default():
    hp = muon.hparams_default()
    assert hp.lr == pytest.approx(0.02) and hp.beta == pytest.approx(0.95)
    assert hp.eps == pytest.approx(1e-7)
    assert (hp.a, hp.b, hp.c) == pytest.approx((3.4445, -4.7750, 2.0315))
    assert hp.ns_steps == 5 and hp.nesterov == 1 and hp.dtype == muon.MUON_BF16
    assert muon.lib().muon_hparams_default(None) == -1


def test_struct_layout_matches_header():
    assert ctypes.sizeof(muon.muon_matrix) == 48
    assert ctypes.sizeof(muon.muon_hparams) == 36


# Fake, well-aligned device addresses. Validation rejects every case below
# before any HIP call, so nothing is dereferenced.
BASE = 0x7F0000000000


def desc(i, rows=64, cols=128, elem=2, w=True, delta=False):
    stride = 1 << 24
    b = BASE + i * 4 * stride
    return muon.muon_matrix(b if w else None, b + stride, b + 2 * stride,
                            b + 3 * stride if delta else None, rows, cols)


def plan_status(descs, hp=None, n=None):
    hp = hp or muon.make_hparams()
    arr = (muon.muon_matrix * max(len(descs), 1))(*descs)
    out = ctypes.c_void_p(123)
    st = muon.lib().muon_plan(arr, len(descs) if n is None else n, ctypes.byref(hp), ctypes.byref(out))
    return st, out.value, muon.last_error()


@pytest.mark.parametrize("case,status,msg", [
    ("n0", -1, "n must be"),
    ("rows0", -1, "rows and cols"),
    ("cols_neg", -1, "rows and cols"),
    ("g_null", -1, "g is NULL"),
    ("m_null", -1, "m is NULL"),
    ("w_delta_null", -1, "both NULL"),
    ("lr_nan", -1, "lr is not finite"),
    ("beta_one", -1, "beta must be"),
    ("beta_neg", -1, "beta must be"),
    ("eps_neg", -1, "eps must be"),
    ("eps_inf", -1, "eps is not finite"),
    ("steps_neg", -1, "ns_steps"),
    ("nesterov_2", -1, "nesterov"),
    ("dtype_7", -4, "dtype"),
    ("misaligned", -3, "16-byte aligned"),
    ("alias_within", -2, "overlaps"),
    ("alias_across", -2, "overlaps"),
    ("too_big", -1, "2^24"),
    ("too_big_f32", -1, "2^23"),
])
def test_plan_validation(case, status, msg):
    d = [desc(0), desc(1)]
    hp = muon.make_hparams()
    n = None
    if case == "n0":
        n = 0
    elif case == "rows0":
        d[0].rows = 0
    elif case == "cols_neg":
        d[1].cols = -3
    elif case == "g_null":
        d[0].g = None
    elif case == "m_null":
        d[1].m = None
    elif case == "w_delta_null":
        d[0].w = None
    elif case == "lr_nan":
        hp.lr = math.nan
    elif case == "beta_one":
        hp.beta = 1.0
    elif case == "beta_neg":
        hp.beta = -0.1
    elif case == "eps_neg":
        hp.eps = -1e-7
    elif case == "eps_inf":
        hp.eps = math.inf
    elif case == "steps_neg":
        hp.ns_steps = -1
    elif case == "nesterov_2":
        hp.nesterov = 2
    elif case == "dtype_7":
        hp.dtype = 7
    elif case == "misaligned":
        d[1].m = d[1].m + 8
    elif case == "alias_within":
        d[0].m = d[0].g + 64
    elif case == "alias_across":
        d[1].w = d[0].w + 128
    elif case == "too_big":
        d[0].cols = (1 << 24) + 1
    elif case == "too_big_f32":
        # fp32 tiles are 128 wide and tile coordinates 16 bits: 2^23 + 128
        # columns would need tile column 65536.
        hp.dtype = muon.MUON_F32
        d[0].rows, d[0].cols = 1, (1 << 23) + 128
    st, out, err = plan_status(d, hp, n)
    assert st == status, err
    assert msg in err
    assert out is None          # *out is cleared on error


def test_null_arguments():
    L = muon.lib()
    hp = muon.make_hparams()
    out = ctypes.c_void_p()
    assert L.muon_plan(None, 1, ctypes.byref(hp), ctypes.byref(out)) == -1
    arr = (muon.muon_matrix * 1)(desc(0))
    assert L.muon_plan(arr, 1, None, ctypes.byref(out)) == -1
    assert L.muon_plan(arr, 1, ctypes.byref(hp), None) == -1
    assert L.muon_step(None, None) == -1
    assert L.muon_plan_destroy(None) == 0           # NULL-safe
    assert L.muon_plan_workspace_bytes(None, None) == -1
    assert L.muon_plan_set_timing(None, 1) == -1
    assert L.muon_plan_kernel_times(None, None, None) == -1
    assert L.muon_plan_info(None, None, None) == -1


def test_adjacent_ranges_do_not_alias():
    # Back-to-back ranges [p, p + bytes) and [p + bytes, ...) are legal.
    rows, cols = 64, 128
    nbytes = rows * cols * 2
    b = BASE
    d = muon.muon_matrix(b, b + nbytes, b + 2 * nbytes, b + 3 * nbytes, rows, cols)
    st, out, err = plan_status([d])
    # Validation passes, so the next failure (if any) comes from HIP.
    assert st in (0, -5, -6), err
    if st == 0:
        muon.destroy_raw(out)


def test_no_gpu_valid_plan_reports_hip_error_not_crash():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    st, out, err = plan_status([desc(0)])
    assert st == -5 and out is None
    assert err.startswith("hip")


# ---- TP shard apply: validation (every case fails before any HIP call)

def shard(i, rows=64, cols=128, ldp=None, ldd=None):
    stride = 1 << 24
    b = BASE + (64 + i) * 2 * stride
    return muon.muon_shard(b, b + stride, rows, cols, ldp or cols, ldd or cols)


def apply_status(shards, dtype=muon.MUON_BF16, n=None):
    arr = (muon.muon_shard * max(len(shards), 1))(*shards)
    out = ctypes.c_void_p(123)
    st = muon.lib().muon_apply_plan(arr, len(shards) if n is None else n, dtype, ctypes.byref(out))
    return st, out.value, muon.last_error()


def test_shard_struct_layout_matches_header():
    assert ctypes.sizeof(muon.muon_shard) == 48


@pytest.mark.parametrize("case,status,msg", [
    ("n0", -1, "n must be"),
    ("p_null", -1, "NULL"),
    ("rows0", -1, "rows and cols"),
    ("too_big", -1, "2^24"),
    ("ldp_small", -1, "ldp and ldd"),
    ("ldd_small", -1, "ldp and ldd"),
    ("dtype_7", -4, "dtype"),
    ("misaligned", -3, "aligned"),
    ("p_over_p", -2, "overlaps"),
    ("p_over_d", -2, "overlaps"),
    ("p_is_d", -2, "overlaps"),
    ("column_blocks_overlap", -2, "overlaps"),
    ("other_stride_over_p", -2, "overlaps"),
])
def test_apply_plan_validation(case, status, msg):
    s = [shard(0), shard(1)]
    n, dtype = None, muon.MUON_BF16
    if case == "n0":
        n = 0
    elif case == "p_null":
        s[1].p = None
    elif case == "rows0":
        s[0].rows = 0
    elif case == "too_big":
        s[0].cols = (1 << 24) + 1
        s[0].ldp = s[0].ldd = s[0].cols
    elif case == "ldp_small":
        s[0].ldp = 100
    elif case == "ldd_small":
        s[1].ldd = 127
    elif case == "dtype_7":
        dtype = 7
    elif case == "misaligned":
        s[0].d = s[0].d + 1
    elif case == "p_over_p":
        s[1].p = s[0].p + 2 * 64 * 3          # inside shard 0's rows
    elif case == "p_over_d":
        s[1].d = s[0].p + 256
    elif case == "p_is_d":
        s[0].d = s[0].p
    elif case == "column_blocks_overlap":
        # two column blocks of one 64 x 256 matrix: columns [0, 128) and [100, 228)
        s[0].ldp = s[1].ldp = 256
        s[1].p = s[0].p + 2 * 100
    elif case == "other_stride_over_p":
        s[1].p = s[0].p + 2 * 1300           # a view with another stride, inside shard 0's range
        s[1].ldp = 200
    st, out, err = apply_status(s, dtype, n)
    assert st == status, err
    assert msg in err
    assert out is None


def test_disjoint_views_do_not_alias():
    """Column blocks of one matrix with its row stride, read-only views that
    share elements, and row blocks back to back all pass validation."""
    rows, cols, parts = 64, 256, 4
    b = BASE + (1 << 30)
    w = cols // parts
    s = [muon.muon_shard(b + 2 * r * w, b + (1 << 26), rows, w, cols, cols) for r in range(parts)]
    s.append(muon.muon_shard(b + (1 << 25), b + (1 << 26), rows, w, w, cols))   # d shared with the others
    st, out, err = apply_status(s)
    assert st in (0, -5, -6), err          # the next failure (if any) comes from HIP
    if st == 0:
        assert muon.lib().muon_apply_plan_destroy(out) == 0


def test_apply_null_arguments():
    L = muon.lib()
    out = ctypes.c_void_p()
    assert L.muon_apply_plan(None, 1, muon.MUON_BF16, ctypes.byref(out)) == -1
    arr = (muon.muon_shard * 1)(shard(0))
    assert L.muon_apply_plan(arr, 1, muon.MUON_BF16, None) == -1
    assert L.muon_apply(None, None) == -1
    assert L.muon_apply_plan_destroy(None) == 0


def test_no_gpu_valid_apply_plan_reports_hip_error_not_crash():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    st, out, err = apply_status([shard(0)])
    assert st == -5 and out is None
    assert err.startswith("hip")


# ---- fp32 master weights (MUON_BF16_F32_MASTER): validation with per-pointer sizes

def test_master_weights_ranges_use_fp32_sizes():
    """w, m and delta are fp32 and g bf16: a g placed right after half of an
    fp32 w overlaps it (it would not with a bf16 w)."""
    rows, cols = 64, 128
    b = BASE + (1 << 31)
    nb16 = rows * cols * 2
    hp = muon.make_hparams(dtype=muon.MUON_BF16_F32_MASTER)
    d = muon.muon_matrix(b, b + nb16, b + 8 * nb16, None, rows, cols)
    st, out, err = plan_status([d], hp)
    assert st == -2 and "overlaps" in err, err
    st_bf16, out_bf16, err_bf16 = plan_status([d], muon.make_hparams(dtype=muon.MUON_BF16))
    assert st_bf16 in (0, -5, -6), err_bf16       # back to back in bf16: no alias
    if st_bf16 == 0:
        muon.destroy_raw(out_bf16)
    d_ok = muon.muon_matrix(b, b + 2 * nb16, b + 3 * nb16, b + 5 * nb16, rows, cols)
    st, out, err = plan_status([d_ok], hp)
    assert st in (0, -5, -6), err
    if st == 0:
        muon.destroy_raw(out)


def test_master_weights_need_the_four_wave_engine(monkeypatch):
    monkeypatch.setenv("MUON_GEMM_VARIANT", "0")
    hp = muon.make_hparams(dtype=muon.MUON_BF16_F32_MASTER)
    st, out, err = plan_status([desc(0, elem=4)], hp)
    assert st == -4 and "four-wave" in err and out is None


# ---- muon_step_noalloc: validation before any HIP call

def noalloc_status(descs, hp=None):
    hp = hp or muon.make_hparams()
    arr = (muon.muon_matrix * max(len(descs), 1))(*descs)
    st = muon.lib().muon_step_noalloc(arr, len(descs), ctypes.byref(hp), None)
    return st, muon.last_error()


def test_noalloc_validates_like_muon_plan():
    d = [desc(0), desc(1)]
    d[1].w = d[0].w + 128
    st, err = noalloc_status(d)
    assert st == -2 and "overlaps" in err
    d = [desc(0)]
    d[0].rows = 0
    st, err = noalloc_status(d)
    assert st == -1 and "rows and cols" in err
    assert muon.lib().muon_step_noalloc(None, 1, None, None) == -1


def test_noalloc_rejects_a_workspace_beyond_the_scratch_before_any_hip_call():
    # 4096 x 4096 bf16 needs about 136 MB of workspace; the scratch holds 64 MiB.
    d = [desc(0, rows=4096, cols=4096)]
    d[0].g = d[0].w + (1 << 26)
    d[0].m = d[0].w + (2 << 26)
    st, err = noalloc_status(d)
    assert st == -1 and "static scratch" in err and str(64 << 20) in err


def test_no_gpu_noalloc_reports_hip_error_not_crash():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    st, err = noalloc_status([desc(0)])
    assert st == -5 and err.startswith("hip")
