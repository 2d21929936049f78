"""Host-side plan checks (bsa_plan_check_host), without a GPU.

Plan buffers are laid out here on the host, section by section as
bsa_plan_sections / bsa_plan_pair_sections / bsa_plan_cols_sections give,
from the oracle's plans (the GPU planner's output equals them bit for bit in
the GPU parity tests).  Unwritten parts hold garbage, as a device buffer
would.  Each consistent plan must pass; each planted inconsistency must be
reported as BSA_ERR_BAD_PLAN with a message that names it.
"""

import ctypes
import os

import numpy as np
import pytest

import block_sparse_attention_plan_amd as bsa
from oracle import bsa_oracle as O

OK, INVALID, TOO_SMALL, BAD_PLAN = 0, -1, -5, -7


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.library_path()):
        pytest.fail("libbsa.so is not built (python -m block_sparse_attention_plan_amd.build)")
    return bsa.load_library()


def _sections(fn, *dims):
    offs = (ctypes.c_size_t * 4)()
    assert fn(*dims, offs) == OK
    return [int(o) // 4 for o in offs]


def row_buffer(lib, lay):
    H, Mb, Nb = lay.shape
    n = lib.bsa_plan_buffer_bytes(H, Mb, Nb)
    o = _sections(lib.bsa_plan_sections, H, Mb, Nb) + _sections(lib.bsa_plan_pair_sections, H, Mb, Nb)
    buf = np.full(n // 4, -12345, np.int32)
    P, PP = O.plan(lay), O.plan_pairs(lay)
    for off, arr in ((o[0], P.row_ptr), (o[1], P.row_order), (o[2], [P.nnz_total]),
                     (o[3], P.col_idx), (o[4], PP.pair_ptr), (o[5], PP.pair_order),
                     (o[6], [PP.pair_total, PP.use_pairs]), (o[7], PP.pair_cols)):
        arr = np.asarray(arr, np.int32)
        buf[off:off + arr.size] = arr
    names = ["row_ptr", "row_order", "nnz", "col_idx", "pair_ptr", "pair_order", "pair_info",
             "pair_cols"]
    return buf, dict(zip(names, o))


def col_buffer(lib, lay, Hkv):
    H, Mb, Nb = lay.shape
    n = lib.bsa_plan_cols_buffer_bytes(H, Hkv, Mb, Nb)
    o = _sections(lib.bsa_plan_cols_sections, H, Hkv, Mb, Nb)
    buf = np.full(n // 4, -777, np.int32)
    C = O.plan_columns(lay, Hkv)
    for off, arr in ((o[0], C.col_ptr), (o[1], C.col_order), (o[2], [C.nnz_total]),
                     (o[3], C.row_idx)):
        arr = np.asarray(arr, np.int32)
        buf[off:off + arr.size] = arr
    return buf, dict(zip(["col_ptr", "col_order", "nnz", "row_idx"], o))


def check(lib, lay, rows=None, cols=None, Hkv=0):
    H, Mb, Nb = lay.shape
    st = lib.bsa_plan_check_host(
        rows.ctypes.data if rows is not None else None, 0 if rows is None else rows.nbytes,
        cols.ctypes.data if cols is not None else None, 0 if cols is None else cols.nbytes,
        H, Hkv, Mb, Nb)
    return st, lib.bsa_last_error().decode()


def layouts():
    rng = np.random.default_rng(7)
    yield "random", (rng.random((3, 9, 11)) < 0.35).astype(np.int32)
    yield "empty", np.zeros((2, 5, 4), np.int32)
    yield "full", np.ones((2, 6, 6), np.int32)
    win = np.zeros((4, 7, 7), np.int32)   # local window + global column, odd Mb
    for m in range(7):
        win[:, m, max(0, m - 2):m + 1] = 1
        win[:, m, 0] = 1
    yield "window_odd_rows", win
    yield "one_row", (rng.random((1, 1, 5)) < 0.6).astype(np.int32)


@pytest.mark.parametrize("name,lay", list(layouts()))
def test_consistent_plans_pass(lib, name, lay):
    rows, _ = row_buffer(lib, lay)
    assert check(lib, lay, rows=rows)[0] == OK
    H = lay.shape[0]
    for Hkv in sorted({1, H}):
        cols, _ = col_buffer(lib, lay, Hkv)
        assert check(lib, lay, cols=cols, Hkv=Hkv)[0] == OK
        st, msg = check(lib, lay, rows=rows, cols=cols, Hkv=Hkv)
        assert st == OK, msg


def _lay():
    rng = np.random.default_rng(11)
    lay = (rng.random((3, 9, 10)) < 0.4).astype(np.int32)
    lay[:, :, 0] = 1          # every row lists at least two columns
    lay[:, :, 9] = 1
    return lay


def _first_row_with(P, k):
    counts = np.diff(P.row_ptr)
    return int(np.nonzero(counts >= k)[0][0])


ROW_DAMAGE = {
    # name: (function(buf, off, P, PP, lay), substring of the message)
    "row_ptr_start": (lambda b, o, P, PP, lay: b.__setitem__(o["row_ptr"], 1), "row_ptr[0]"),
    "row_count_negative": (lambda b, o, P, PP, lay: b.__setitem__(o["row_ptr"] + 3, b[o["row_ptr"] + 5]),
                           "items"),
    "row_count_above_Nb": (lambda b, o, P, PP, lay: b.__setitem__(o["row_ptr"] + 1, lay.shape[2] + 1),
                           "items"),
    "nnz_total": (lambda b, o, P, PP, lay: b.__setitem__(o["nnz"], P.nnz_total - 1), "total"),
    "nnz_negative": (lambda b, o, P, PP, lay: b.__setitem__(o["nnz"], -3), "nnz_total"),
    "col_past_Nb": (lambda b, o, P, PP, lay: b.__setitem__(o["col_idx"] + P.nnz_total - 1, lay.shape[2]),
                    "outside"),
    "col_negative": (lambda b, o, P, PP, lay: b.__setitem__(o["col_idx"], -1), "outside"),
    "cols_swapped": (lambda b, o, P, PP, lay: _swap(b, o["col_idx"] + P.row_ptr[_first_row_with(P, 2)]),
                     "ascending"),
    "col_repeated": (lambda b, o, P, PP, lay: b.__setitem__(
        o["col_idx"] + P.row_ptr[_first_row_with(P, 2)] + 1, b[o["col_idx"] + P.row_ptr[_first_row_with(P, 2)]]),
        "ascending"),
    "row_order_repeat": (lambda b, o, P, PP, lay: b.__setitem__(o["row_order"] + 4, b[o["row_order"] + 2]),
                         "twice"),
    "row_order_range": (lambda b, o, P, PP, lay: b.__setitem__(o["row_order"], lay.shape[0] * lay.shape[1]),
                        "outside"),
    "use_flag": (lambda b, o, P, PP, lay: b.__setitem__(o["pair_info"] + 1, 2), "use flag"),
    "pair_total": (lambda b, o, P, PP, lay: b.__setitem__(o["pair_info"], PP.pair_total + 1), "total"),
    "pair_tag": (lambda b, o, P, PP, lay: b.__setitem__(o["pair_cols"] + 1, b[o["pair_cols"] + 1] ^ (3 << 24)),
                 "expected"),
    "pair_column": (lambda b, o, P, PP, lay: b.__setitem__(o["pair_cols"], b[o["pair_cols"]] + 1),
                    "expected"),
    "pair_order_repeat": (lambda b, o, P, PP, lay: b.__setitem__(o["pair_order"] + 1, b[o["pair_order"]]),
                          "twice"),
}


def _swap(b, i):
    b[i], b[i + 1] = b[i + 1], b[i]


@pytest.mark.parametrize("name", sorted(ROW_DAMAGE))
def test_damaged_plan_is_reported(lib, name):
    lay = _lay()
    rows, off = row_buffer(lib, lay)
    assert check(lib, lay, rows=rows)[0] == OK
    damage, text = ROW_DAMAGE[name]
    damage(rows, off, O.plan(lay), O.plan_pairs(lay), lay)
    st, msg = check(lib, lay, rows=rows)
    assert st == BAD_PLAN, (name, msg)
    assert text in msg, (name, msg)


def test_pair_missing_a_row_entry(lib):
    """A pair list that drops an entry while its count and the total stay
    consistent (the lists shift by one) fails the union comparison."""
    lay = _lay()
    rows, o = row_buffer(lib, lay)
    PP = O.plan_pairs(lay)
    Q = len(PP.pair_ptr) - 1
    base = o["pair_ptr"]
    rows[base + 1:base + Q + 1] -= 1         # pair 0 loses its last entry ...
    seg = rows[o["pair_cols"]:o["pair_cols"] + PP.pair_total].copy()
    last0 = PP.pair_ptr[1] - 1
    rows[o["pair_cols"]:o["pair_cols"] + PP.pair_total - 1] = np.delete(seg, last0)
    rows[o["pair_info"]] = PP.pair_total - 1  # ... and the total follows
    st, msg = check(lib, lay, rows=rows)
    assert st == BAD_PLAN and "missing column" in msg, msg


def test_last_pair_of_odd_rows_has_no_second_row(lib):
    lay = np.ones((2, 5, 3), np.int32)
    rows, o = row_buffer(lib, lay)
    PP = O.plan_pairs(lay)
    last = PP.pair_ptr[2] + 0   # head 0's last pair (rows 4 and the absent 5)
    assert PP.pair_cols[last] >> 24 == 1
    rows[o["pair_cols"] + last] |= 2 << 24
    st, msg = check(lib, lay, rows=rows)
    assert st == BAD_PLAN and "expected" in msg, msg


COL_DAMAGE = {
    "row_idx_past_Mb": (lambda b, o, C, lay: b.__setitem__(o["row_idx"] + C.nnz_total - 1, lay.shape[1]),
                        "outside"),
    "row_idx_order": (lambda b, o, C, lay: _swap(b, o["row_idx"] + C.col_ptr[
        int(np.nonzero(np.diff(C.col_ptr) >= 2)[0][0])]), "ascending"),
    "col_order_repeat": (lambda b, o, C, lay: b.__setitem__(o["col_order"] + 1, b[o["col_order"]]), "twice"),
    "col_ptr_start": (lambda b, o, C, lay: b.__setitem__(o["col_ptr"], 2), "col_ptr[0]"),
    "col_nnz": (lambda b, o, C, lay: b.__setitem__(o["nnz"], C.nnz_total + 1), "total"),
}


@pytest.mark.parametrize("name", sorted(COL_DAMAGE))
def test_damaged_column_plan_is_reported(lib, name):
    lay = _lay()
    cols, off = col_buffer(lib, lay, 3)
    assert check(lib, lay, cols=cols, Hkv=3)[0] == OK
    damage, text = COL_DAMAGE[name]
    damage(cols, off, O.plan_columns(lay, 3), lay)
    st, msg = check(lib, lay, cols=cols, Hkv=3)
    assert st == BAD_PLAN, (name, msg)
    assert text in msg, (name, msg)


def test_plans_of_different_layouts_disagree(lib):
    """Two consistent plans of same-shaped layouts with the same tile count
    but one tile moved: each passes alone, together they are reported."""
    lay = _lay()
    other = lay.copy()
    h, m = 1, 4
    live = np.nonzero(other[h, m])[0]
    dead = np.nonzero(other[h, m] == 0)[0]
    other[h, m, live[1]], other[h, m, dead[0]] = 0, 1
    rows, _ = row_buffer(lib, lay)
    cols, _ = col_buffer(lib, other, 3)
    assert check(lib, lay, rows=rows)[0] == OK and check(lib, lay, cols=cols, Hkv=3)[0] == OK
    st, msg = check(lib, lay, rows=rows, cols=cols, Hkv=3)
    assert st == BAD_PLAN and "missing from the column plan" in msg, msg
    cols2, _ = col_buffer(lib, other[:, :, ::-1].copy() * 0, 3)
    st, msg = check(lib, lay, rows=rows, cols=cols2, Hkv=3)
    assert st == BAD_PLAN and "live tiles" in msg, msg


def test_argument_errors(lib):
    lay = _lay()
    rows, _ = row_buffer(lib, lay)
    H, Mb, Nb = lay.shape
    assert lib.bsa_plan_check_host(None, 0, None, 0, H, 0, Mb, Nb) == INVALID
    assert lib.bsa_plan_check_host(rows.ctypes.data, rows.nbytes - 4, None, 0, H, 0, Mb, Nb) == TOO_SMALL
    assert lib.bsa_plan_check_host(rows.ctypes.data, rows.nbytes, None, 0, H, 2, Mb, Nb) == INVALID
    assert lib.bsa_plan_check_host(rows.ctypes.data, rows.nbytes, None, 0, 0, 0, Mb, Nb) == INVALID
    assert lib.bsa_plan_check(None, None, None) == INVALID


def test_debug_switch(lib):
    prev = lib.bsa_set_debug(1)
    try:
        assert lib.bsa_set_debug(1) == 1
        assert lib.bsa_set_debug(0) == 1
        assert lib.bsa_set_debug(0) == 0
    finally:
        lib.bsa_set_debug(prev)
