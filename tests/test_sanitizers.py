"""The host C code under AddressSanitizer and UndefinedBehaviorSanitizer: the
fp64 oracle (oracle/wanattn_oracle.c) and the seeded input generator
(seeded/seeded.c) are compiled with -fsanitize=address,undefined and the
oracle's pins (tests/test_oracle_pins.py) run against those builds, with the
sanitizer runtime preloaded and any report fatal.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = {
    "oracle": os.path.join(ROOT, "oracle", "wanattn_oracle.c"),
    "seeded": os.path.join(ROOT, "video_diffusion_transformer_wanattn_amd", "seeded", "seeded.c"),
}
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def run_pins(tmp_path, oracle_src=SOURCES["oracle"]):
    libs = {}
    for name, src in dict(SOURCES, oracle=oracle_src).items():
        libs[name] = str(tmp_path / f"lib{name}_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread", *SAN,
                               "-o", libs[name], src, "-lm"])
    env = dict(os.environ,
               WANATTN_ORACLE_LIB=libs["oracle"], WANATTN_SEEDED_LIB=libs["seeded"],
               LD_PRELOAD=runtime(),
               # reports go to files: pytest's capture of the child's stderr is
               # lost when a report ends the process
               ASAN_OPTIONS=f"detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan")
    # the library comparisons (torch's sdpa and layer_norm) are left out: they
    # check numbers, not the C code's memory use, and torch is slow to load
    # under the sanitizer runtime
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", "not library"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in sorted(os.listdir(tmp_path))
                      if f.startswith(("asan", "ubsan")))
    return r.returncode, r.stdout[-3000:] + r.stderr[-3000:] + reports[:6000]


@pytest.mark.skipif(runtime() is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    rc, out = run_pins(tmp_path)
    assert rc == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in out, out


@pytest.mark.skipif(runtime() is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_sanitizer_catches_a_planted_overread(tmp_path):
    # one key past the end of a row's score buffer: a heap read the numeric
    # pins need not notice, which the sanitized build must report
    src = open(SOURCES["oracle"]).read()
    old = "  for (int j = 0; j < nkeys; ++j) {\n    if (!allowed[j]) continue;\n    double s = 0.0;"
    assert src.count(old) == 1
    planted = tmp_path / "overread.c"
    planted.write_text(src.replace(old, old.replace("j < nkeys", "j <= nkeys")))
    rc, out = run_pins(tmp_path, str(planted))
    assert rc != 0 and "AddressSanitizer" in out, out
