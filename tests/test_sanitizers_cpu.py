"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

Three builds are made in a temporary directory and driven by the existing
CPU tests, each run in a child process with the sanitizer runtime preloaded
(Python itself is not instrumented):

- the oracle (sattn_oracle.c) and the input generator (sattn_testkit.c),
  built with gcc -fsanitize=address,undefined, under the oracle's pin tests
  (all but the 2^32-pattern encoder sweep and the 100 001-key case, which
  the instrumented build would take minutes over);
- the library's host code (argument validation, size and layout arithmetic,
  split choice, the host unpacker of api.cpp), built with hipcc and
  -Xarch_host -fsanitize=address,undefined (the device code is built as
  usual and never runs here), under the ABI tests.

Any sanitizer report aborts the child (-fno-sanitize-recover), so a run
passes only if every test passes with no report."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

ORACLE_TESTS = ["test_oracle_quant.py", "test_oracle_attention.py", "test_oracle_e4m3.py",
                "test_oracle_fp8qk.py", "test_oracle_lse.py", "test_oracle_qsmooth.py",
                "test_oracle_sparse.py", "test_testkit.py"]


def _clang_rt_dir() -> str:
    base = "/opt/rocm/lib/llvm/lib/clang"
    for ver in sorted(os.listdir(base), reverse=True):
        d = os.path.join(base, ver, "lib", "linux")
        if os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so")):
            return d
    pytest.skip("clang AddressSanitizer runtime not found")


def _run(env_extra, args, cwd=ROOT, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable] + args, cwd=cwd, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    return r.returncode, out


def _mapped(env_extra, importer: str, name: str) -> bool:
    """Whether a child process with env_extra maps a file whose path holds
    `name` after running `importer`."""
    code = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        {importer}
        print(any({name!r} in line for line in open("/proc/self/maps")))
    """)
    rc, out = _run(env_extra, ["-c", code])
    assert rc == 0, out
    return out.strip().splitlines()[-1] == "True"


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("sanitized"))
    from oracle import build as obuild
    from testkit import build as tbuild
    from precision_flash_attention_amd import build as pbuild
    paths = {
        "oracle": obuild.build(sanitize=True, out=os.path.join(d, "liboracle_san.so")),
        "testkit": tbuild.build(sanitize=True, out=os.path.join(d, "libtestkit_san.so")),
        "sattn": pbuild.build_host_sanitized(os.path.join(d, "libsattn_san.so")),
    }
    return paths


def test_oracle_pins_under_sanitizers(builds):
    gcc = lambda lib: subprocess.run(["gcc", f"-print-file-name={lib}"], capture_output=True,  # noqa: E731
                                     text=True, check=True).stdout.strip()
    env = {"LD_PRELOAD": f"{gcc('libasan.so')}:{gcc('libubsan.so')}",
           "SATTN_ORACLE_LIB": builds["oracle"], "SATTN_TESTKIT_LIB": builds["testkit"]}
    assert _mapped(env, "import oracle, testkit; oracle._load(); testkit._load()", "liboracle_san.so")
    assert _mapped(env, "import testkit; testkit._load()", "libtestkit_san.so")
    rc, out = _run(env, ["-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                         "-k", "not exhaustive_sweep and not flushes"]
                   + [os.path.join("tests", t) for t in ORACLE_TESTS])
    tail = "\n".join(out.splitlines()[-40:])
    assert rc == 0, tail
    assert "runtime error" not in out and "AddressSanitizer" not in out, tail
    assert " passed" in out, tail


def test_host_api_under_sanitizers(builds):
    rt = _clang_rt_dir()
    env = {"LD_PRELOAD": os.path.join(rt, "libclang_rt.asan-x86_64.so"),
           "LD_LIBRARY_PATH": rt + ":" + os.environ.get("LD_LIBRARY_PATH", ""),
           "SATTN_LIBRARY": builds["sattn"]}
    assert _mapped(env, "import precision_flash_attention_amd as s; s._load()", "libsattn_san.so")
    rc, out = _run(env, ["-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join("tests", "test_abi_cpu.py")])
    tail = "\n".join(out.splitlines()[-40:])
    assert rc == 0, tail
    assert "runtime error" not in out and "AddressSanitizer" not in out, tail
    assert " passed" in out, tail
