"""The host-side C++ (the library's planner and the CPU oracle) built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, no GPU code) and run
over seeded call sequences: any out-of-bounds access, leak, use after free or
undefined behaviour aborts the driver."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-pthread"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build_and_run(tmp_path, name, sources):
    exe = os.path.join(str(tmp_path), name)
    subprocess.run(["g++", *FLAGS, *sources, "-o", exe], check=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ok" in r.stdout


def test_planner_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "plan_driver", [os.path.join(HERE, "plan_driver.cpp"),
                                             os.path.join(ROOT, "paged_kv_cache_gca_amd", "csrc", "gca_plan.cpp")])


def test_oracle_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "oracle_driver", [os.path.join(HERE, "oracle_driver.cpp"),
                                               os.path.join(ROOT, "oracle", "gca_oracle.cpp")])
