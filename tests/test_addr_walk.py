"""Host-side address walk of batch-1 megakernel plans (libmkcheck.so).

The walk replays every task of a plan's tape, at one decode position, through
the index helpers the kernels themselves use (csrc/mk_addr.h) and checks every
global index against the size of its buffer and every LDS index against the
plan's LDS regions.  It covers the Llama-8B shape that mk_load refuses (its
first GPU run faulted): every index of that plan is in bounds, so the walk
rules out an out-of-bounds index in the steady-state executors as the cause.
A negative slack tightens every limit by one element; the walk must then
report overruns, which shows that the accesses it checks reach the last
element of their buffers and that a one-element overrun would be caught."""

import ctypes
import os

import pytest

from persistent_megakernel_cu_amd import binding as mkb
from synth_inputs import LLAMA_1B, LLAMA_8B, TINY

CHECK_LIB = os.path.join(os.path.dirname(os.path.abspath(mkb.__file__)), "libmkcheck.so")


class Report(ctypes.Structure):
    _fields_ = [("checks", ctypes.c_longlong), ("violations", ctypes.c_longlong), ("first", ctypes.c_char * 256)]


@pytest.fixture(scope="module")
def walk():
    if not os.path.exists(CHECK_LIB):
        pytest.fail(f"{CHECK_LIB} is not built (run persistent_megakernel_cu_amd/build.py)")
    lib = ctypes.CDLL(CHECK_LIB)
    lib.mkcheck_walk.argtypes = [ctypes.POINTER(mkb.MkConfig), ctypes.c_int, ctypes.c_int, ctypes.c_longlong,
                                 ctypes.POINTER(Report)]
    lib.mkcheck_walk.restype = ctypes.c_int

    def run(shape, max_seq, pos, slack=0, num_wgs=256, **kw):
        cfg = mkb.make_config(shape, max_seq, **kw)
        rep = Report()
        rc = lib.mkcheck_walk(ctypes.byref(cfg), num_wgs, pos, slack, ctypes.byref(rep))
        return rc, rep

    return run


CASES = [
    (TINY, 48, [0, 1, 47]),
    (TINY.with_(n_kv_heads=4), 48, [0, 47]),                 # one query head per kv head
    (TINY.with_(tie_embeddings=False), 48, [5]),
    (LLAMA_1B, 256, [0, 128, 255]),                           # the benchmarked workload
    (LLAMA_1B, 8192, [0, 4096, 8191]),                        # 32 chunks, merged
    (LLAMA_1B.with_(n_heads=16), 1088, [1024, 1087]),         # two query heads per kv head
    (LLAMA_8B, 2112, [0, 2047, 2048, 2049, 2111]),            # head_dim 128, 9 chunks, untied LM head
    (LLAMA_8B, 8192, [8191]),
]


@pytest.mark.parametrize("shape,max_seq,positions", CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_every_index_in_bounds(walk, shape, max_seq, positions):
    for pos in positions:
        rc, rep = walk(shape, max_seq, pos)
        assert rc == mkb.MK_OK, rep.first.decode()
        assert rep.checks > 0
        assert rep.violations == 0, f"pos {pos}: {rep.first.decode()}"


@pytest.mark.parametrize("wgs", [2, 7, 64, 255])
def test_every_index_in_bounds_on_other_grids(walk, wgs):
    # fewer workgroups: more row items per wave, and the gate/up ranges'
    # one-workgroup offset wrapping around a grid that is not a multiple of 8
    for pos in (0, 47):
        rc, rep = walk(TINY, 48, pos, num_wgs=wgs)
        assert rc == mkb.MK_OK, rep.first.decode()
        assert rep.checks > 0
        assert rep.violations == 0, f"{wgs} workgroups, pos {pos}: {rep.first.decode()}"


@pytest.mark.parametrize("shape,max_seq,pos", [(TINY, 48, 47), (LLAMA_1B, 256, 255), (LLAMA_8B, 2112, 2049)],
                         ids=["tiny", "llama1b", "llama8b"])
def test_walk_catches_a_one_element_overrun(walk, shape, max_seq, pos):
    rc, rep = walk(shape, max_seq, pos, slack=-1)
    assert rc == mkb.MK_OK
    assert rep.violations > 0 and rep.first


def test_partial_input_plan_in_bounds(walk):
    for pos in (0, 255):
        rc, rep = walk(LLAMA_1B, 256, pos, partial_input=True)
        assert rc == mkb.MK_OK and rep.violations == 0, rep.first.decode()


def test_batched_plans_are_not_walked(walk):
    rc, rep = walk(TINY, 48, 0, batch=4)
    assert rc == mkb.MK_E_UNSUPPORTED
    assert b"batched" in rep.first
