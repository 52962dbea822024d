"""The committed profile summaries that bench.py reports from.

The headline's roofline.traffic comes from the FETCH_SIZE / WRITE_SIZE
counter summary under profiles/; bench.py only uses it while it was taken on
the current source of the headline kernel. A change to that kernel without
new counters turns the field null, which this test reports instead.
"""
import hashlib
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _fields(path):
    out = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def test_traffic_profile_matches_headline_source():
    f = _fields(bench.TRAFFIC_FILE)
    with open(bench.HEADLINE_SOURCE, "rb") as src:
        sha = hashlib.sha256(src.read()).hexdigest()
    assert f["kernel_source_sha256"] == sha, "headline kernel changed since its counters were taken"
    traffic = bench.measured_traffic()
    assert traffic is not None and traffic == float(f["traffic_bytes_per_dispatch"])


def test_traffic_profile_is_self_consistent():
    """read + write = traffic; each counter scaled by the copy calibration;
    the algorithmic bytes are X + F + Y of the headline layer."""
    f = _fields(bench.TRAFFIC_FILE)
    rd, wr = float(f["read_bytes_per_dispatch"]), float(f["write_bytes_per_dispatch"])
    assert abs(rd + wr - float(f["traffic_bytes_per_dispatch"])) <= 2
    assert abs(float(f["fetch_kib_per_dispatch"]) * 1024 * float(f["fetch_scale"]) - rd) <= 0.01 * rd
    assert abs(float(f["write_kib_per_dispatch"]) * 1024 * float(f["write_scale"]) - wr) <= 0.01 * wr
    x = 32 * 58 * 58 * 64 * 2
    w = 3 * 3 * 64 * 64 * 2
    y = 32 * 56 * 56 * 64 * 2
    assert int(f["algorithmic_bytes_per_dispatch"]) == x + w + y
    # no wasted re-reads: within 5 % of the algorithmic bytes
    assert 0.95 <= float(f["traffic_over_algorithmic"]) <= 1.05


def test_trace_summary_names_the_launched_headline_kernel():
    """The kernel-trace summary names the band kernel instantiation the
    launcher's defaults select, and bench's unprofiled time is consistent
    with the traced kernel duration."""
    with open(os.path.join(ROOT, "profiles", "kernel_trace_dense3x3_bf16.txt")) as fh:
        txt = fh.read()
    with open(bench.HEADLINE_SOURCE) as fh:
        src = fh.read()
    m = re.search(r"template <int KH, int KW, int CS, int NR, bool OB, bool GS = false, int SAUX = (\d+), "
                  r"int LS = (\d+), int LR = (\d+), int LT = (\d+)>", src)
    assert m, "launcher defaults not found"
    saux, ls, lr, lt = m.groups()
    assert f"kernel: dense_band_mfma<3, 3, 2, 9, {saux}, {ls}, true, {lr}, {lt}, false>" in txt
    # bench.py's per-launch time without the profiler (launch gaps included)
    # against the traced kernel mean: tracing lengthens the kernels, never
    # by more than a quarter here, and the gaps cannot make a launch shorter
    # than its kernel by more than that.
    ratio = float(re.search(r"unprofiled_over_trace_mean: ([0-9.]+)", txt).group(1))
    assert 0.75 <= ratio <= 1.1
