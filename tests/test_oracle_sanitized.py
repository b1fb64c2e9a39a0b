"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) passes every pin: no out-of-bounds access, use after
free or undefined behaviour on the pins' inputs. A planted one-element
overrun in a copy of the source must be reported, which shows the sanitized
build is live. The builds go to a temporary directory; the oracle the other
tests use is never modified."""
import os
import subprocess
import sys

import pytest

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
SAN = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def _runtime(name):
    path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")
pytestmark = pytest.mark.skipif(not (ASAN and UBSAN), reason="gcc sanitizer runtimes not found")


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    c.write_text(src_text)
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, *SAN, "-w", str(c), "-o", str(so), "-lm"])
    return str(so)


def _run(so, body):
    """Run `body` in a fresh interpreter with the sanitized oracle loaded
    (the sanitizer runtimes preloaded, since Python itself is not built
    with them)."""
    script = (f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
              f"import oracle\noracle._lib = oracle.load({so!r})\n" + body)
    env = dict(os.environ, LD_PRELOAD=f"{ASAN} {UBSAN}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    return subprocess.run([sys.executable, "-c", script], env=env, capture_output=True,
                          text=True, timeout=600)


def n_pins():
    sys.path.insert(0, TESTS)
    from oracle_pins import ALL_CHECKS
    return len(ALL_CHECKS)


@pytest.fixture(scope="module")
def src():
    with open(os.path.join(ROOT, "oracle", "oracle.c")) as f:
        return f.read()


def test_every_pin_passes_under_asan_and_ubsan(src, tmp_path):
    so = _build(src, tmp_path, "oracle_san")
    r = _run(so, "from oracle_pins import ALL_CHECKS\n"
                 "for c in ALL_CHECKS:\n    c()\n"
                 "print('pins', len(ALL_CHECKS))\n")
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip().endswith(f"pins {n_pins()}"), r.stdout


def test_planted_overrun_is_reported(src, tmp_path):
    """The pad fill of the flatten writes one element too many."""
    old = "memset(out + off * elem_size, 0, (size_t)((padded - off) * elem_size));"
    assert src.count(old) == 1
    bad = src.replace(old, "memset(out + off * elem_size, 0, (size_t)((padded - off + 1) * elem_size));")
    so = _build(bad, tmp_path, "oracle_overrun")
    r = _run(so, "import numpy as np\n"
                 "x = np.arange(1 << 20, dtype=np.float32)\n"
                 "oracle.flatten([x], (1 << 20) + 3)\n"
                 "print('not caught')\n")
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
