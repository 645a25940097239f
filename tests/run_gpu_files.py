"""Run every GPU test file in a pytest process of its own.

One process per file means that a fault or abort in one file (a bridge that
terminates the process, an unsupported configuration that aborts) cannot hide
the results of the files after it: each file reports on its own, and the
summary at the end lists every file with its exit status.

    python tests/run_gpu_files.py [--timeout SECONDS] [pytest args ...]

Files run in name order (test_zz_no_alloc.py last, as in a single pytest
run).  The exit status is 0 only if every file passed.
"""
import argparse
import glob
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def gpu_files():
    out = []
    for path in sorted(glob.glob(os.path.join(HERE, "test_*.py"))):
        with open(path) as f:
            if "pytest.mark.gpu" in f.read():
                out.append(path)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--timeout", type=int, default=900, help="seconds per file")
    args, extra = ap.parse_known_args()
    results = []
    for path in gpu_files():
        name = os.path.relpath(path, ROOT)
        print(f"[file] {name}", flush=True)
        t0 = time.time()
        cmd = [sys.executable, "-u", "-m", "pytest", "-q", "-m", "gpu", "--timeout", "300",
               "--timeout-method", "thread", "-p", "no:cacheprovider", name, *extra]
        try:
            rc = subprocess.run(cmd, cwd=ROOT, timeout=args.timeout).returncode
        except subprocess.TimeoutExpired:
            rc = "timeout"
        results.append((name, rc, time.time() - t0))
        print(f"[file] {name}: exit {rc} in {time.time() - t0:.0f}s", flush=True)
        if rc == "timeout" or rc < 0 or rc in (124, 134, 137, 139):
            # the process hung or died on a signal (a fault, an abort): start
            # nothing more on the GPU after it
            break
    print("\nsummary:")
    for name, rc, dt in results:
        print(f"  {'ok  ' if rc in (0, 5) else 'FAIL'} {name} (exit {rc}, {dt:.0f}s)")
    missing = [os.path.relpath(p, ROOT) for p in gpu_files()][len(results):]
    for name in missing:
        print(f"  skip {name} (not run after a process died)")
    sys.exit(0 if all(rc in (0, 5) for _, rc, _ in results) and not missing else 1)


if __name__ == "__main__":
    main()
