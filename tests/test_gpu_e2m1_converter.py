"""The library's E2M1 encoder on its own: the gfx950 converter
v_cvt_scalef32_pk_fp4_f32 with a unit scale (device helper bsfp::e2m1_pack2,
run by the test-support kernel in tests/hw) must implement the rule of
cvt.rn.satfinite.e2m1x2.f32 ("perf(cuda): enable hardware NVFP4/MXFP4
conversion on Blackwell builds", Problem / Background): nearest grid
magnitude, ties to the even code, |v| >= 6 (and infinity) to 6, the sign bit
of v kept (also for values that round to zero).

- every fp32 bit pattern except NaN, against the hand-derived decision
  boundaries of tests/golden/e2m1_thresholds.txt (the table the CPU pins
  check against the oracle over all bf16 values), evaluated with torch;
- 4 M random patterns and the neighbourhood of every boundary against the
  oracle's nearest-value encoder directly.
NaN inputs are outside the contract and not checked."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

from conftest import ROOT, read_golden

pytestmark = pytest.mark.gpu

PROBE = os.path.join(ROOT, "tests", "hw", "libe2m1_probe.so")


@pytest.fixture(scope="module")
def probe(bsfp):
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is missing: build it with tests/hw/build.py")
    L = C.CDLL(PROBE)
    L.e2m1_probe.restype = C.c_int
    L.e2m1_probe.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
    raw = getattr(torch._C, "_cuda_getCurrentRawStream")

    def run(f: torch.Tensor) -> torch.Tensor:
        assert f.dtype == torch.float32 and f.is_cuda and f.is_contiguous() and f.numel() % 2 == 0
        out = torch.empty(f.numel(), dtype=torch.uint8, device=f.device)
        rc = L.e2m1_probe(f.data_ptr(), f.numel(), out.data_ptr(), raw(f.device.index))
        assert rc == 0, rc
        return out
    return run


def table_codes(f: torch.Tensor) -> torch.Tensor:
    """E2M1 codes by the boundary table: the number of boundaries strictly
    below |v|, or the table's tie code on a boundary; sign bit of v."""
    rows = read_golden("e2m1_thresholds.txt")[:-1]  # the saturation row is implied
    a = f.abs()
    code = torch.zeros(f.shape, dtype=torch.uint8, device=f.device)
    for b, _below, _at, _above in rows:
        code += (a > float(b)).to(torch.uint8)
    for b, _below, at, _above in rows:
        code = torch.where(a == float(b), torch.full_like(code, int(at)), code)
    return code | (torch.signbit(f).to(torch.uint8) << 3)


def test_every_fp32_pattern(probe):
    chunk = 1 << 28
    bad = 0
    for start in range(0, 1 << 32, chunk):
        u = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        u = torch.where(u >= (1 << 31), u - (1 << 32), u).to(torch.int32)
        f = u.view(torch.float32)
        got = probe(f)
        want = table_codes(f)
        ok = (got == want) | torch.isnan(f)
        n_bad = int((~ok).sum().item())
        if n_bad and bad == 0:
            i = int((~ok).nonzero()[0].item())
            print(f"first mismatch: bits {int(u[i].item()) & 0xFFFFFFFF:#010x} "
                  f"got {int(got[i])} want {int(want[i])}")
        bad += n_bad
        del u, f, got, want, ok
    assert bad == 0


def test_boundaries_and_random_patterns_against_oracle(oracle_mod, probe):
    rng = np.random.default_rng(77)
    pats = [rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)]
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    bounds = [float(r[0]) for r in read_golden("e2m1_thresholds.txt")]
    for v in sorted(set(grid + bounds)):
        c = np.array([v], np.float32).view(np.uint32)[0].astype(np.int64)
        near = np.arange(c - 1024, c + 1025)
        near = near[near >= 0].astype(np.uint32)
        pats += [near, near | np.uint32(0x80000000)]
    pats.append(np.array([0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 1, 0x80000001],
                         np.uint32))
    u = np.concatenate(pats)
    if u.size % 2:
        u = np.concatenate([u, np.zeros(1, np.uint32)])
    f = u.view(np.float32)
    keep = ~np.isnan(f)
    got = probe(torch.from_numpy(f.copy()).cuda()).cpu().numpy()
    want = oracle_mod.e2m1_encode(f)
    assert np.array_equal(got[keep], want[keep])
