"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic
work it prices the CFConv launches at, and which committed counter records
it takes."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cfconv_work_per_launch():
    """Forward: the two filter products, 2 D (Dr + D) flops per edge. Backward
    with source sums: both products and their tangents, 4 D (Dr + D); the
    first block (tangents of the second product only): 2 D (2 Dr + D); the
    launch price is the mean over the T blocks."""
    class M:
        D, Dr, T = 128, 50, 3
    fwd, bwd = bench.cf_flops(M, 1000.0)
    assert fwd == 2 * 128 * (50 + 128) * 1000
    with_q = 4 * 128 * (50 + 128) * 1000
    first = 2 * 128 * (2 * 50 + 128) * 1000
    assert bwd == (2 * with_q + first) / 3
    M.T = 1                      # one block: only the first block's kernel
    assert bench.cf_flops(M, 1000.0)[1] == first


def test_kernel_arguments_of_profiled_names():
    assert bench.kernel_args("void sn::k_cf_bwd<128, 64, 1, true>(sn::CfParams)", "bwd") == \
        ["128", "64", "1", "true"]
    assert bench.kernel_args("void sn::k_cf_fwd<64, 32, 0>(sn::CfParams)", "fwd") == \
        ["64", "32", "0"]
    assert bench.kernel_args("void sn::k_cf_fwd<64, 32, 0>(sn::CfParams)", "bwd") == []
    assert bench.kernel_args("void sn::k_atom<128, 128, 1, 3>(sn::AtomArgs)", "bwd") == []


def test_counter_records_of_the_current_kernels_are_taken():
    """Both CFConv kernels' committed records of the headline workload match
    the current kernel sources and are used; a record of other kernels is not."""
    from schnet_continuous_filter_amd import profiling
    c, m, *_ = bench.model_for("md1024", None)
    for kind in ("fwd", "bwd"):
        rec = bench.counter_record(kind, "md1024", m)
        assert rec is not None, kind
        assert rec["kernel_hash"] == profiling.kernel_hash()
        assert bench.utilisation_record(kind, "md1024", m) is not None
    c, m32, *_ = bench.model_for("md1024", "f32")   # no fp32 record of this workload
    assert bench.counter_record("bwd", "md1024", m32) is None
