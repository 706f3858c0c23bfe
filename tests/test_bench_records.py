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
