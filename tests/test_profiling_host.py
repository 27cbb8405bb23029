"""Host checks of the rocprofv3 summary code: counter scaling by the copy
calibration, kernel-name matching, and staleness by source digest."""
import csv
import os

from kv_cache_top_amd import profiling as PR

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_scaling(tmp_path, monkeypatch):
    col = "void pk::collide_kernel<4>(HIP_vector_type<unsigned int, 4u> const*, long)"
    cal = "pk::copy16_kernel(HIP_vector_type<unsigned int, 4u>*, unsigned long)"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # the counter reads half the calibration copy's 1 GiB for reads, all of it for writes
    _csv(f, "FETCH_SIZE", [(col, 1000.0), (col, 1002.0), (cal, 524288.0), (cal, 10.0)])
    _csv(w, "WRITE_SIZE", [(col, 300.0), (col, 300.0), (cal, 1048576.0)])
    out = tmp_path / "pmc_collide_x.md"
    r = PR.summarize_traffic(str(f), str(w), str(out), "collide", "x", 2_000_000, "cmd f", "cmd w")
    assert r["fetch_scale"] == 2.0 and r["write_scale"] == 1.0
    assert r["hbm_read_bytes_per_launch"] == int(1001.0 * 1024 * 2)
    assert r["hbm_write_bytes_per_launch"] == 300 * 1024
    assert r["kernel_symbol"] == "collide_kernel<4>" and r["dispatches"] == 2
    # load_traffic reads it back while the sources are unchanged, and not once they differ
    monkeypatch.setattr(PR, "PROFILES", str(tmp_path))
    assert PR.load_traffic("collide", "x") == r["hbm_bytes_per_launch"]
    assert PR.load_traffic("rerank", "x") is None
    monkeypatch.setattr(PR, "kernel_source_digest", lambda: "0000")
    assert PR.load_traffic("collide", "x") is None


def test_kernel_keys():
    assert PR.kernel_key("void pk::select_kernel<2>(unsigned int const*)") == "select"
    assert PR.kernel_key("pk::rerank_kernel(unsigned char const*)") == "rerank"
    assert PR.kernel_key("void pk::attend_kernel<unsigned short, float, float, 32>(x)") == "attend"


def test_committed_summaries_name_their_command():
    prof = os.path.join(PR.ROOT, "profiles")
    for name in os.listdir(prof):
        text = open(os.path.join(prof, name)).read()
        assert "rocprofv3" in text and "bench.py" in text, name


def test_kernel_keys_follow_pk_timing_names():
    from kv_cache_top_amd.profiling import kernel_key
    assert kernel_key("void pk::collide_kernel<4, 64>(HIP_vector_type<unsigned int, 4u> const*)") == "collide"
    assert kernel_key("void pk::select_sub_kernel<4, true, 16>(unsigned int const*)") == "select"
    assert kernel_key("void pk::append_qprep_kernel<unsigned short, unsigned short>(pk::QprepArgs)") == "qprep"
    assert kernel_key("void pk::rerank_topk_kernel<4, unsigned short, 2, true>(unsigned char const*)") == "rerank_topk"
