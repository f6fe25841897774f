"""CPU sanitizer leg: the library's host codec (df11_host.cpp) and the oracle
(df11_oracle.c) built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc/g++, host code only), linked into a plain C program that checks them
against each other byte for byte on seeded units and runs the oracle's pins
and the codec's argument checks."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc")
def test_host_codec_and_oracle_under_asan_and_ubsan(tmp_path):
    inc = os.path.join(ROOT, "include")
    objs = []
    for src, cc, std in ((os.path.join(ROOT, "entropy_decoding_amd", "csrc", "df11_host.cpp"), "g++", "-std=c++17"),
                         (os.path.join(ROOT, "oracle", "df11_oracle.c"), "gcc", "-std=c99"),
                         (os.path.join(ROOT, "tests", "sanitize", "df11_sanitize_check.c"), "gcc", "-std=c99")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call([cc, std, *SAN, "-Wall", "-I", inc, "-c", src, "-o", o])
        objs.append(o)
    exe = str(tmp_path / "df11_sanitize_check")
    subprocess.check_call(["g++", *SAN, *objs, "-pthread", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "sanitize ok" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc")
def test_host_length_limiter_equals_the_oracle_at_every_limit(tmp_path):
    """The host codec limits code lengths with boundary package-merge, the
    oracle with package-merge over stored lists; with the same tie rules they
    must give the same lengths at every limit (the 32-bit codebook limit is
    reached by the library only for Fibonacci-like histograms)."""
    inc = os.path.join(ROOT, "include")
    ora = str(tmp_path / "df11_oracle.o")
    subprocess.check_call(["gcc", "-std=c99", *SAN, "-I", inc, "-c",
                           os.path.join(ROOT, "oracle", "df11_oracle.c"), "-o", ora])
    exe = str(tmp_path / "package_merge_check")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-I", inc,
                           os.path.join(ROOT, "tests", "sanitize", "package_merge_check.cpp"), ora,
                           "-pthread", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "limiter ok" in r.stdout
