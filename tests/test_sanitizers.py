"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two child processes, each with its sanitizer runtime preloaded:
  - the oracle's test files against ``liboracle_q4q8_san.so`` (gcc's ASan
    and UBSan), so every oracle routine the pins exercise runs instrumented;
  - the C ABI tests (argument validation, group plans, status codes) against
    ``libq4q8_san.so``, whose host code is built with clang's ASan and UBSan.
A report from either sanitizer, or any failing test, fails the test here.
Both libraries are built by ``__graft_entry__.build()``; a missing one is
built here first."""
import importlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_TESTS = ["tests/test_oracle_fp16.py", "tests/test_oracle_quant.py", "tests/test_oracle_matmul.py",
                "tests/test_oracle_q8w.py", "tests/test_oracle_swiglu.py", "tests/test_independent_reading.py"]

# the child reports which library it loaded and whether the ASan runtime is mapped
PROBE = """
import sys
sys.path.insert(0, {root!r})
{load}
maps = open('/proc/self/maps').read()
print('LOADED', path, 'ASAN', 'asan' in maps)
"""


def _run(env_extra, args, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _check(res):
    text = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in text, text[-4000:]
    assert "runtime error:" not in text, text[-4000:]
    assert res.returncode == 0, text[-4000:]
    return text


def test_oracle_suite_under_asan_ubsan():
    ob = importlib.import_module("oracle.build")  # the module (the package re-exports its build())

    if not os.path.exists(ob.SAN_LIB_PATH):
        ob.build_sanitized()
    env = {"LD_PRELOAD": ob.asan_runtime(), "Q4Q8_ORACLE_LIB": ob.SAN_LIB_PATH}
    load = "import oracle; lib = oracle._load(); path = lib._name"
    text = _check(_run(env, ["-c", PROBE.format(root=ROOT, load=load)]))
    assert f"LOADED {ob.SAN_LIB_PATH} ASAN True" in text, text
    _check(_run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *ORACLE_TESTS]))


def test_abi_suite_under_asan_ubsan():
    bs = importlib.import_module("block_quantized_matmul_q8_amd.build_sanitized")

    if not os.path.exists(bs.SAN_LIB_PATH):
        bs.build_sanitized()
    env = {"LD_PRELOAD": bs.asan_runtime(), "Q4Q8_LIB": bs.SAN_LIB_PATH}
    load = "import block_quantized_matmul_q8_amd as q; lib = q.lib(); path = lib._name"
    text = _check(_run(env, ["-c", PROBE.format(root=ROOT, load=load)]))
    assert f"LOADED {bs.SAN_LIB_PATH} ASAN True" in text, text
    _check(_run(env, ["-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", "tests/test_abi.py"]))
