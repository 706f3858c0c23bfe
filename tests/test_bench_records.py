"""bench.py uses a committed rocprofv3 counter record only while the kernel's
sources and build flags are those it was taken on, by a digest of both.  The
digest must not depend on where the repository is checked out: GPU runs work
on a copy at another path."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_digest_independent_of_checkout_path(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    from linear_attention_recurrence_delta_amd import build_lib

    before = {k: bench.kernel_source_digest(k) for k in bench.KERNEL_SOURCES}
    other = "/elsewhere/checkout"

    def moved(flags):
        return [os.path.join(other, os.path.relpath(x, build_lib.ROOT)) if os.path.isabs(x) else x for x in flags]

    monkeypatch.setattr(build_lib, "COMMON", moved(build_lib.COMMON))
    monkeypatch.setattr(build_lib, "DEVICE", moved(build_lib.DEVICE))
    monkeypatch.setattr(build_lib, "PER_FILE", {k: moved(v) for k, v in build_lib.PER_FILE.items()})
    monkeypatch.setattr(build_lib, "ROOT", other)
    after = {k: bench.kernel_source_digest(k) for k in bench.KERNEL_SOURCES}
    assert before == after


def test_digest_follows_the_flags(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    from linear_attention_recurrence_delta_amd import build_lib

    before = bench.kernel_source_digest("kda_prefill_k3_dense_32k")
    monkeypatch.setattr(build_lib, "DEVICE", build_lib.DEVICE + ["-DSOMETHING_ELSE"])
    assert bench.kernel_source_digest("kda_prefill_k3_dense_32k") != before


def _csv(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w") as f:
        f.write(",".join('"%s"' % c for c in cols) + "\n")
        for i, (name, val) in enumerate(rows, 1):
            f.write('%d,"%s","%s",%f\n' % (i, name, counter, val))


def test_record_counters_from_pmc_csv(tmp_path):
    """--record-counters: the copy calibration (1 GiB copies issued before any
    library launch), the mean per dispatch of each kernel of a record, and the
    sum over the launches of a multi-kernel call."""
    sys.path.insert(0, ROOT)
    import json
    import bench

    copy = "__amd_rocclr_copyBuffer"
    dense = "void kda::kda_prefill_ws_kernel<2, 2, 8, false, false, false, false>(kda::PrefillParams)"
    fwd = "void kda::kda_prefill_ws_kernel<2, 2, 8, false, true, false, false>(kda::PrefillParams)"
    rev = "kda::(anonymous namespace)::kda_backward_kernel(kda::BackwardParams)"
    summ = "kda::(anonymous namespace)::kda_backward_sum_kernel(kda::BackwardParams)"
    # FETCH_SIZE counts half the bytes a copy reads, WRITE_SIZE all it writes (in KiB)
    half, full = (1 << 30) / 2048.0, (1 << 30) / 1024.0
    fetch = [(copy, half)] * 3 + [(dense, 100.0), (dense, 300.0), (fwd, 10.0), (rev, 20.0), (summ, 30.0),
                                  (copy, 5.0)]
    write = [(copy, full)] * 3 + [(dense, 50.0), (dense, 50.0), (fwd, 1.0), (rev, 2.0), (summ, 3.0), (copy, 5.0)]
    _csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "rec.json"
    bench.record_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), out_path=str(out))
    rec = json.load(open(out))
    d = rec["kda_prefill_k3_dense_32k"]
    assert d["fetch_kib"] == 200.0 and d["write_kib"] == 50.0
    assert d["hbm_bytes_per_launch"] == 1024 * (200 * 2 + 50)
    assert d["source_digest"] == bench.kernel_source_digest("kda_prefill_k3_dense_32k")
    b = rec["kda_backward_k3_dense_32k"]
    assert b["fetch_kib"] == 60.0 and b["write_kib"] == 6.0
    assert b["hbm_bytes_per_launch"] == 1024 * (60 * 2 + 6)
    assert "kda_decode_256x96" not in rec  # no dispatches: no record
