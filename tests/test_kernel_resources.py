"""The compiler's per-kernel resource report written by the build: every kernel of the
library runs without scratch memory (no register spills to memory), and the report
covers the hot-path kernels.  Skipped when the library has not been built here."""
import os

import pytest

REPORT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "selective_state_space_ssd_amd", "_build", "kernel_resources.txt")


def _rows():
    if not os.path.exists(REPORT):
        pytest.skip("no build report (run __graft_entry__.build() first)")
    with open(REPORT) as f:
        header = f.readline().rstrip("\n").split("\t")
        return [dict(zip(header, line.rstrip("\n").split("\t"))) for line in f if line.strip()]


def test_no_kernel_needs_scratch():
    rows = _rows()
    bad = [(r["kernel"], r["ScratchSize [bytes/lane]"]) for r in rows
           if r["ScratchSize [bytes/lane]"] != "0"]
    assert not bad, bad


def test_report_covers_the_hot_path_kernels():
    names = " ".join(r["kernel"] for r in _rows())
    for k in ("k_ssd_fused", "k_verify", "k_bwd_chain", "k_bwd_chunk_bf", "k_selective_scan",
              "k_seq_apply_bf"):
        assert k in names, k
