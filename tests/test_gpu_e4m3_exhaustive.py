"""The device E4M3 conversion against the oracle's encoder, exhaustively.

Every E4M3 code of the library -- the V codes of the pre-pass and the P
operand of the fused kernel -- goes through one device helper (the hardware
convert v_cvt_pk_fp8_f32, packed as the fused kernel packs P).  The test
export sage_debug_e4m3_encode runs that helper on a range of FP32 bit
patterns; here every FP32 value of magnitude up to 480 (both signs, the
subnormals and zeros included) is converted and compared with the oracle's
OCP E4M3 encoder (round to nearest even, saturating), which is itself pinned
to the format definition and to torch's float8_e4m3fn conversion.

Above 464 -- the midpoint between the largest code 448 and the format's NaN
pattern -- the hardware convert (which has no saturating form on gfx950)
returns the NaN code, while the oracle saturates to 448.  No kernel converts
such a value:
* a V code converts x * fl(448 / a) with |x| <= a (the channel's absmax), at
  most 448 * (1 + 2^-23);
* the P operand converts 2^x with x = fma(S, c, log2 448 - m), m the rounded
  product of the row's largest S with c, so x exceeds log2 448 by at most the
  rounding of that product, |m| * 2^-24, and 2^x stays below 464 unless the
  scores reach 8.5e5 in log2 units.
The test therefore requires the oracle's codes for every pattern of magnitude
up to 464 (both signs, subnormals and zeros included) and records the NaN
code for the patterns from 464 to 480.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from tests import parity_util as pu

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26                      # patterns per device call
TOP = int(np.float32(480.0).view(np.uint32))       # 0x43f00000
MID = int(np.float32(464.0).view(np.uint32))       # 0x43e80000
NEG = 0x80000000


def _oracle_codes(orc, first, n, threads=16):
    bits = np.arange(first, first + n, dtype=np.uint32)
    x = bits.view(np.float32)
    cuts = np.linspace(0, n, threads + 1).astype(np.int64)
    out = np.empty(n, np.uint8)

    def one(i):
        a, b = cuts[i], cuts[i + 1]
        if b > a:
            out[a:b] = orc.e4m3_encode(x[a:b])

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(threads)))
    return out


@pytest.mark.parametrize("sign", ["positive", "negative"])
def test_every_pattern_up_to_480(orc, sign):
    base = 0 if sign == "positive" else NEG
    total = TOP + 1                  # bit patterns 0 .. bits(480) of this sign
    nan_code = 0x7F if sign == "positive" else 0xFF
    buf = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    mismatches = []
    beyond = 0
    for off in range(0, total, CHUNK):
        n = min(CHUNK, total - off)
        first = base + off
        pu.say(f"[e4m3 {sign}] patterns {first:#010x} .. {first + n - 1:#010x}")
        got = pu.qa.sage_debug_e4m3_encode(first, n, out=buf).cpu().numpy()
        want = _oracle_codes(orc, first, n)
        mag = np.arange(off, off + n, dtype=np.uint32)          # pattern without sign
        above = mag > MID
        beyond += int(above.sum())
        # above 464: the hardware's NaN code (the oracle saturates; no kernel gets here)
        assert np.all(got[above] == nan_code)
        bad = np.nonzero((got != want) & ~above)[0]
        if bad.size:
            vals = (np.uint32(first) + bad[:5].astype(np.uint32)).view(np.float32)
            mismatches.append((first, bad.size, list(zip(vals.tolist(), got[bad[:5]].tolist(),
                                                        want[bad[:5]].tolist()))))
    assert not mismatches, mismatches
    assert beyond == TOP - MID
