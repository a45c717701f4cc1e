"""Exhaustive sweep of the device cast: every fp32 bit pattern the quantizers can
be asked to cast with a unit scale goes through the HIP kernels, and every code
byte is compared with the oracle's saturating round-to-nearest-even encoder
("FP8 Formats for Deep Learning", review page, "Core claim": the E4M3 / E5M2
encodings; the standard rounding of its parameter ledger).

- MX path (mx_quantize, OCP floor rule): each 32-element block holds one planted
  value with floor(log2 |v|) equal to the element format's largest exponent, so
  the block scale is 2^0 and the other 31 elements are cast as they are.  The
  sweep covers every pattern with |x| < 2^(emax+1): the rounding range, the
  saturating range above the largest code, zeros, fp32 subnormals, both signs.
  The clamp counts are checked as well.
- Token path (fp8_quantize_token, round-up rule): each 128-element group holds a
  planted value equal to the largest code's value, so the scale is 2^0 and the
  other 127 elements -- every pattern with |x| <= fmax -- are cast unclamped.

The input patterns are generated on the device (a plain integer range viewed as
fp32); the expected codes come from oracle.encode_f32_range only."""
import threading

import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
from gpu_helpers import ORACLE_THREADS

pytestmark = pytest.mark.gpu

FMAX_BITS = {mx.E4M3: 0x43E00000, mx.E5M2: 0x47600000}  # fp32 patterns of 448 and 57344
EMAX_ELEM = {mx.E4M3: 8, mx.E5M2: 15}
CHUNK = 1 << 27  # sweep values per launch


def encode_range(fmt, start, n):
    """oracle.encode_f32_range over [start, start + n), split over host threads."""
    out = np.empty(n, np.uint8)
    step = -(-n // ORACLE_THREADS)

    def job(i0):
        out[i0:i0 + step] = oracle.encode_f32_range(fmt, start + i0, min(step, n - i0))
    ts = [threading.Thread(target=job, args=(i0,)) for i0 in range(0, n, step)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return out


def device_patterns(start, n, total):
    """fp32 values whose bit patterns are start .. start + n - 1, padded with +0.0 to
    `total` elements, generated on the GPU."""
    p = torch.zeros(total, dtype=torch.int64, device="cuda")
    p[:n] = torch.arange(start, start + n, dtype=torch.int64, device="cuda")
    p = torch.where(p >= 1 << 31, p - (1 << 32), p)
    return p.to(torch.int32).view(torch.float32)


def sweep_ranges(lo, hi):
    """(start, n) chunks of the positive patterns [lo, hi) and their negatives."""
    for sign in (0, 0x80000000):
        for s in range(lo, hi, CHUNK):
            yield sign + s, min(CHUNK, hi - s)


def first_mismatch(got, want, start):
    i = int(np.flatnonzero(got != want)[0])
    return "pattern 0x%08x: device 0x%02x, oracle 0x%02x" % (start + i, got[i], want[i])


@pytest.mark.parametrize("fmt", [mx.E4M3, mx.E5M2])
def test_mx_cast_every_pattern_below_twice_the_top_binade(fmt):
    per = 31
    hi = (127 + EMAX_ELEM[fmt] + 1) << 23          # patterns of |x| < 2^(emax+1)
    planted = float(2 ** EMAX_ELEM[fmt])           # floor(log2) = emax -> block exponent 0
    planted_code = int(oracle.encode(fmt, np.array([planted]))[0])
    fmax_bits = FMAX_BITS[fmt]
    checked = 0
    for start, n in sweep_ranges(0, hi):
        nblk = -(-n // per)
        vals = device_patterns(start, n, nblk * per).view(nblk, per)
        x = torch.empty((nblk, 32), dtype=torch.float32, device="cuda")
        x[:, 0] = planted
        x[:, 1:] = vals
        q, s, c = mx.quantize_mx(x, fmt, mx.RULE_FLOOR, counts=True)
        qh = q.cpu().numpy()
        sh = s.cpu().numpy()
        ch = c.cpu().numpy()
        assert np.all(sh == 127), "block scale not 2^0 in chunk at 0x%08x" % start
        assert np.all(qh[:, 0] == planted_code)
        got = qh[:, 1:].reshape(-1)[:n]
        want = encode_range(fmt, start, n)
        assert np.array_equal(got, want), first_mismatch(got, want, start)
        # patterns rise with the index within a chunk: element i clamps iff i >= t
        t = min(max(fmax_bits + 1 - (start & 0x7FFFFFFF), 0), n)
        lo = np.arange(nblk, dtype=np.int64) * per
        want_cnt = np.maximum(np.minimum(lo + per, n) - np.maximum(lo, t), 0)
        assert np.array_equal(ch.reshape(-1).astype(np.int64), want_cnt), "clamp counts in chunk at 0x%08x" % start
        checked += n
    assert checked == 2 * hi


@pytest.mark.parametrize("fmt", [mx.E4M3, mx.E5M2])
def test_token_cast_every_pattern_up_to_fmax(fmt):
    per = 127
    hi = FMAX_BITS[fmt] + 1                        # patterns of |x| <= fmax
    fmax = float(np.array([FMAX_BITS[fmt]], np.uint32).view(np.float32)[0])
    fmax_code = int(oracle.encode(fmt, np.array([fmax]))[0])
    checked = 0
    for start, n in sweep_ranges(0, hi):
        rows = -(-n // per)
        vals = device_patterns(start, n, rows * per).view(rows, per)
        x = torch.empty((rows, 128), dtype=torch.float32, device="cuda")
        x[:, 0] = fmax
        x[:, 1:] = vals
        q, s = mx.quantize_token(x, fmt, mx.ROW)
        qh = q.cpu().numpy()
        assert np.all(s.cpu().numpy() == 127), "group scale not 2^0 in chunk at 0x%08x" % start
        assert np.all(qh[:, 0] == fmax_code)
        got = qh[:, 1:].reshape(-1)[:n]
        want = encode_range(fmt, start, n)
        assert np.array_equal(got, want), first_mismatch(got, want, start)
        checked += n
    assert checked == 2 * hi
