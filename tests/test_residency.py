"""The engine residency layer (include/dn_residency.h: host arrays canonical, fresh/ahead flags,
pull before host use, upload before a device step, pull after a failed step) driven through the
engine's cases against a host-only stand-in for the dn.h calls. CPU only."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "residency")


def test_residency_protocol(tmp_path):
    exe = tmp_path / "check_residency"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                           "-o", str(exe), os.path.join(HERE, "check_residency.c"), os.path.join(HERE, "fake_dn.c")])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "residency checks passed" in r.stdout


def test_residency_header_compiles_as_cxx(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text('#include "dn_residency.h"\nint main() { dn_resident r{}; return dnr_host_written(&r) == DN_E_INVAL ? 0 : 1; }\n')
    subprocess.check_call(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                           str(src)])
