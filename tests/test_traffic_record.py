"""bench.py reads a kernel's counter record (profiles/traffic_<stage>.txt) only while it still
describes that kernel: the same bytes of the listed sources and the same build options of the
kernel's file; otherwise it reports no traffic rather than a stale figure."""
import hashlib
import os

import bench


def _write_record(root, srcs, flags, beyond=1.25e11, clock=1.6):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    h = hashlib.sha256()
    for s in srcs:
        h.update(open(os.path.join(root, s), "rb").read())
    lines = ["# test record", "kernel: k", "source: " + ", ".join(srcs),
             "source_sha256: " + h.hexdigest(), "build_file: k_bwd_mfma.hip",
             "build_flags: " + flags, f"beyond_l2_bytes_per_launch: {beyond:.4e}",
             f"clock_ghz: {clock}"]
    with open(os.path.join(root, "profiles", "traffic_k.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def test_record_is_used_only_while_it_matches(tmp_path, monkeypatch):
    root = str(tmp_path)
    src = "kernel.hip"
    with open(os.path.join(root, src), "w") as f:
        f.write("// kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", root)
    flags = bench.kernel_build_flags("k_bwd_mfma.hip")
    _write_record(root, [src], flags)
    assert bench.profile_record("k") == {"beyond_l2_bytes_per_launch": 1.25e11, "clock_ghz": 1.6}
    _write_record(root, [src], flags + " -mllvm -some-other-option")   # other build options
    assert bench.profile_record("k") == {}
    _write_record(root, [src], flags)
    with open(os.path.join(root, src), "w") as f:                      # the kernel changed
        f.write("// kernel v2\n")
    assert bench.profile_record("k") == {}
    assert bench.profile_record("missing") == {}


def test_build_flags_leave_out_include_paths():
    flags = bench.kernel_build_flags("k_bwd_mfma.hip")
    assert "-I" not in flags.split() and "/" not in flags
    assert "--offload-arch=gfx950" in flags
