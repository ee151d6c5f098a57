"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/sage.h declares, and its host-side validation returns the documented
status for each bad argument without touching the GPU (fake, never
dereferenced device pointers are passed; every case fails before any HIP
call)."""
import ctypes
import os
import re

import pytest

import quantized_attention_03_amd as qa
from quantized_attention_03_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "sage.h")
FAKE = 0x10000          # aligned fake device address (never dereferenced)


def _declared():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"SAGE_API\s+[\w\s\*]*?\b(sage_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 14, names
    L = qa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_abi.EXPORTS)


def test_version_and_status_strings():
    L = qa.lib()
    assert L.sage_abi_version() == 3
    for code in range(14):
        assert L.sage_status_string(code)
    assert L.sage_status_string(999) == b"unknown status"


def _desc(**kw):
    d = _abi.Desc()
    qa.lib().sage_desc_init(ctypes.byref(d), kw.pop("dtype", 0), kw.pop("layout", 0),
                            kw.pop("batch", 2), kw.pop("hq", 8), kw.pop("hkv", 2),
                            kw.pop("nq", 100), kw.pop("nkv", 300), kw.pop("head_dim", 128))
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _fwd(d, q=FAKE, k=FAKE, v=FAKE, o=FAKE, ws=FAKE, ws_bytes=1 << 40):
    P = ctypes.c_void_p
    return qa.lib().sage_attn_fwd(ctypes.byref(d), P(q), P(k), P(v), P(o), None, P(ws),
                                  ws_bytes, None)


def _ws(d, cuq=None, cuk=None, n=0):
    out = ctypes.c_size_t(0)
    st = qa.lib().sage_workspace_size(ctypes.byref(d) if d is not None else None, cuq, cuk, n,
                                      ctypes.byref(out))
    return st, out.value


def test_desc_init_defaults():
    d = _desc()
    assert (d.smooth_k, d.smooth_q, d.smooth_v, d.is_causal, d.sm_scale) == (1, 0, 0, 0, 0.0)
    assert d.pv_mode == _abi.PV_FP8 and d.kv_split == 0 and d.qk_block == 0


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, "SAGE_ERR_DTYPE"),
    ("layout", 2, "SAGE_ERR_LAYOUT"),
    ("is_causal", 2, "SAGE_ERR_FLAGS"),
    ("smooth_v", -1, "SAGE_ERR_FLAGS"),
    ("head_dim", 80, "SAGE_ERR_HEAD_DIM"),
    ("head_dim", 256, "SAGE_ERR_HEAD_DIM"),
    ("hq", 0, "SAGE_ERR_SHAPE"),
    ("nq", -1, "SAGE_ERR_SHAPE"),
    ("batch", -3, "SAGE_ERR_SHAPE"),
    ("hq", 7, "SAGE_ERR_GQA"),
    ("pv_mode", 2, "SAGE_ERR_FLAGS"),
    ("pv_mode", -1, "SAGE_ERR_FLAGS"),
    ("kv_split", 100, "SAGE_ERR_FLAGS"),
    ("kv_split", -2, "SAGE_ERR_FLAGS"),
    ("qk_block", 16, "SAGE_ERR_FLAGS"),
    ("qk_block", 128, "SAGE_ERR_FLAGS"),
])
def test_descriptor_errors(field, value, status):
    d = _desc(**{field: value})
    assert _abi.STATUS_NAMES[_fwd(d)] == status
    assert _abi.STATUS_NAMES[_ws(d)[0]] == status


def test_nan_scale_rejected():
    d = _desc(sm_scale=float("nan"))
    assert _abi.STATUS_NAMES[_fwd(d)] == "SAGE_ERR_FLAGS"


def test_stride_errors():
    d = _desc()
    d.q_stride[0], d.q_stride[1], d.q_stride[2] = 100 * 128, 128, 12   # not a multiple of 8
    assert _abi.STATUS_NAMES[_fwd(d)] == "SAGE_ERR_STRIDE"
    d = _desc()
    d.k_stride[1] = -8
    assert _abi.STATUS_NAMES[_fwd(d)] == "SAGE_ERR_STRIDE"


def test_null_align_workspace_errors():
    d = _desc()
    assert _abi.STATUS_NAMES[qa.lib().sage_attn_fwd(None, None, None, None, None, None, None, 0,
                                                    None)] == "SAGE_ERR_NULL"
    assert _abi.STATUS_NAMES[_fwd(d, q=0)] == "SAGE_ERR_NULL"
    assert _abi.STATUS_NAMES[_fwd(d, ws=0)] == "SAGE_ERR_NULL"
    assert _abi.STATUS_NAMES[_fwd(d, k=FAKE + 4)] == "SAGE_ERR_ALIGN"
    assert _abi.STATUS_NAMES[_fwd(d, o=FAKE + 8)] == "SAGE_ERR_ALIGN"
    st, need = _ws(d)
    assert st == 0 and need > 0
    assert _abi.STATUS_NAMES[_fwd(d, ws_bytes=need - 1)] == "SAGE_ERR_WORKSPACE"


def test_varlen_seqlens_errors():
    d = _desc(batch=0, nq=0, nkv=0)
    I = ctypes.c_int32
    good_q, good_k = (I * 3)(0, 10, 30), (I * 3)(0, 50, 51)
    bad_start = (I * 3)(1, 10, 30)
    decreasing = (I * 3)(0, 10, 5)
    P = ctypes.c_void_p
    L = qa.lib()

    def run(cq, ck, n=2):
        return _abi.STATUS_NAMES[L.sage_attn_fwd_varlen(ctypes.byref(d), cq, ck, n, P(FAKE), P(FAKE),
                                                        P(FAKE), P(FAKE), None, P(FAKE), 1, None)]
    assert run(None, good_k) == "SAGE_ERR_NULL"
    assert run(bad_start, good_k) == "SAGE_ERR_SEQLENS"
    assert run(good_q, decreasing) == "SAGE_ERR_SEQLENS"
    assert run(good_q, good_k, n=-1) == "SAGE_ERR_SHAPE"
    assert run(good_q, good_k) == "SAGE_ERR_WORKSPACE"


def _pad(x, m):
    return (x + m - 1) // m * m


def test_quant_buf_sizes_follow_documented_layout():
    d = _desc(smooth_q=1, smooth_v=1)       # B=2, hq=8, hkv=2, nq=100, nkv=300, d=128
    s = qa.quant_buf_sizes(d)
    B, hq, hkv, dd = 2, 8, 2, 128
    npq, npk = _pad(100, 64), _pad(300, 128)
    assert s["q_codes"] == B * hq * npq * dd
    assert s["q_scale"] == B * hq * npq // 64 * 4
    assert s["k_codes"] == B * hkv * npk * dd == s["v_codes"]
    assert s["k_scale"] == B * hkv * npk // 64 * 4
    assert s["v_scale"] == B * hkv * dd * 4 == s["mu_k"] == s["mu_v"]
    assert s["mu_q"] == B * hq * dd * 4
    assert s["delta_s"] == B * hq * npk * 4
    d2 = _desc()
    assert qa.quant_buf_sizes(d2)["delta_s"] == 0 and qa.quant_buf_sizes(d2)["mu_q"] == 0
    # varlen: sum of per-sequence padded lengths
    I = ctypes.c_int32
    dv = _desc(batch=0, nq=0, nkv=0)
    cq, ck = (I * 4)(0, 1, 65, 65), (I * 4)(0, 129, 130, 130)
    z = _abi.QuantSizes()
    assert qa.lib().sage_quant_buf_sizes(ctypes.byref(dv), cq, ck, 3, ctypes.byref(z)) == 0
    assert z.q_codes == hq * (64 + 64 + 0) * dd          # lengths 1, 64, 0
    assert z.k_codes == hkv * (256 + 128 + 0) * dd      # lengths 129, 1, 0


def test_finer_qk_block_sizes():
    """32-token Q/K blocks: twice the Q and K scales, everything else equal
    (codes keep their 64-token row padding)."""
    a = qa.quant_buf_sizes(_desc(smooth_q=1))
    b = qa.quant_buf_sizes(_desc(smooth_q=1, qk_block=32))
    c = qa.quant_buf_sizes(_desc(smooth_q=1, qk_block=64))
    assert a == c
    assert b["q_scale"] == 2 * a["q_scale"] and b["k_scale"] == 2 * a["k_scale"]
    assert {k: v for k, v in b.items() if k not in ("q_scale", "k_scale")} == \
        {k: v for k, v in a.items() if k not in ("q_scale", "k_scale")}


def test_block_q_smoothing_sizes_and_flags():
    """smooth_q = SAGE_SMOOTH_Q_BLOCK adds the per-block means, deviation
    codes and scales (one per Q block, the index of q_scale), keeps everything
    else of smooth_q = 1, and is refused with 16-bit P.V or an unknown value."""
    hq, dd = 8, 128
    for qb in (64, 32):
        a = qa.quant_buf_sizes(_desc(smooth_q=1, qk_block=qb))
        b = qa.quant_buf_sizes(_desc(smooth_q=_abi.SMOOTH_Q_BLOCK, qk_block=qb))
        nqb = 2 * hq * _pad(100, 64) // qb                 # B = 2, nq = 100
        assert b["mu_qb"] == nqb * dd * 4 and b["mu_q_code"] == nqb * 2 * dd
        assert b["mu_q_cscale"] == nqb * 4 == b["q_scale"]
        assert a["mu_qb"] == a["mu_q_code"] == a["mu_q_cscale"] == 0
        assert {k: v for k, v in b.items() if not k.startswith("mu_q")} == \
            {k: v for k, v in a.items() if not k.startswith("mu_q")}
        assert b["mu_q"] == a["mu_q"]
    name = lambda st: _abi.STATUS_NAMES[st]
    assert name(_ws(_desc(smooth_q=_abi.SMOOTH_Q_BLOCK, pv_mode=_abi.PV_HALF))[0]) == "SAGE_ERR_FLAGS"
    assert name(_ws(_desc(smooth_q=3))[0]) == "SAGE_ERR_FLAGS"
    assert _ws(_desc(smooth_q=_abi.SMOOTH_Q_BLOCK))[0] == 0


def test_half_pv_sizes():
    """16-bit P.V operands: V is 2 bytes per element, no V scale, and the
    workspace (no V maxima) is not larger than the E4M3 one."""
    B, hkv, dd = 2, 2, 128
    npk = _pad(300, 128)
    for sv in (0, 1):
        f8 = qa.quant_buf_sizes(_desc(smooth_v=sv))
        h = qa.quant_buf_sizes(_desc(smooth_v=sv, pv_mode=_abi.PV_HALF))
        assert h["v_codes"] == 2 * f8["v_codes"] == 2 * B * hkv * npk * dd
        assert h["v_scale"] == 0 and f8["v_scale"] == B * hkv * dd * 4
        assert {k: v for k, v in h.items() if k not in ("v_codes", "v_scale")} == \
            {k: v for k, v in f8.items() if k not in ("v_codes", "v_scale")}
        st, wf8 = _ws(_desc(smooth_v=sv))
        st2, wh = _ws(_desc(smooth_v=sv, pv_mode=_abi.PV_HALF))
        assert st == st2 == 0 and wh <= wf8 + B * hkv * npk * dd


def _split(d, cuq=None, cuk=None, n=0):
    out = ctypes.c_int32(-7)
    st = qa.lib().sage_kv_split_size(ctypes.byref(d), cuq, cuk, n, ctypes.byref(out))
    return _abi.STATUS_NAMES[st], out.value


def test_kv_split_rule():
    """Explicit splits are used as given unless they cover the longest key
    range.  The automatic rule: decode shapes (GQA group x queries <= 32)
    aim at one round of one-wave units (256 compute units x 4 waves, or 3
    for 16-bit V at d = 128, whose LDS stages fit only three times) and at
    least two splits; other shapes split only grids below 256 workgroups,
    aiming at 512; at least 4 key tiles per split either way."""
    assert _split(_desc(nkv=1000, kv_split=256)) == ("SAGE_OK", 256)
    assert _split(_desc(nkv=1000, kv_split=1024)) == ("SAGE_OK", 0)
    assert _split(_desc(nkv=1000)) == ("SAGE_OK", 0)
    # decode: B=2, hkv=2, group 4, nq=1 -> 4 units, 1024 / 4 = 256 splits
    # wanted, at least 4 tiles each: 32768 keys = 256 tiles -> 512 keys
    assert _split(_desc(nq=1, nkv=32768, kv_split=-1)) == ("SAGE_OK", 512)
    # 16 tiles in all: max(4, ceil(16 / 256)) = 4 tiles
    assert _split(_desc(nq=1, nkv=2048, kv_split=-1)) == ("SAGE_OK", 512)
    # the decode workload: 8 x 8 = 64 units -> 1024 / 64 = 16 splits of
    # 256 / 16 = 16 tiles; with 16-bit V 768 / 64 = 12 -> ceil(256 / 12) = 22
    assert _split(_desc(batch=8, hq=32, hkv=8, nq=1, nkv=32768, kv_split=-1)) == ("SAGE_OK", 2048)
    assert _split(_desc(batch=8, hq=32, hkv=8, nq=1, nkv=32768, kv_split=-1, pv_mode=1)) == \
        ("SAGE_OK", 2816)
    # many units: still two splits (ceil(256 / 2) = 128 tiles)
    assert _split(_desc(batch=512, hq=32, hkv=8, nq=1, nkv=32768, kv_split=-1)) == \
        ("SAGE_OK", 16384)
    # group 4 x 9 queries = 36 rows: the fused kernel's rule, 2 * 2 workgroups
    # -> 128 splits wanted -> 4 tiles
    assert _split(_desc(nq=9, nkv=32768, kv_split=-1)) == ("SAGE_OK", 512)
    # a prefill grid (well over 256 workgroups) is not split
    assert _split(_desc(batch=4, hq=32, hkv=32, nq=4096, nkv=4096, kv_split=-1)) == ("SAGE_OK", 0)
    # keys that fit one split: no split
    assert _split(_desc(nq=1, nkv=300, kv_split=-1)) == ("SAGE_OK", 0)
    assert _split(_desc(kv_split=96))[0] == "SAGE_ERR_FLAGS"


def test_split_workspace_holds_the_partials():
    base = _ws(_desc(nq=4, nkv=4096))
    sp = _ws(_desc(nq=4, nkv=4096, kv_split=512))
    rows, nsplit, d = 2 * 8 * 4, 8, 128              # B*hq*nq rows, 4096/512 splits
    assert base[0] == sp[0] == 0
    assert sp[1] - base[1] >= nsplit * rows * (d + 2) * 4


def test_empty_problem_is_a_no_op():
    d = _desc(batch=0)
    # nothing to compute: returns OK after the argument checks (no device call
    # happens before the arch check, which an empty problem still performs)
    st = _fwd(d, q=0, k=0, v=0, o=0, ws=0, ws_bytes=0)
    assert _abi.STATUS_NAMES[st] in ("SAGE_OK", "SAGE_ERR_HIP", "SAGE_ERR_ARCH")


def test_e4m3_export_argument_errors():
    # each case fails before any HIP call
    L = qa.lib()
    u32 = ctypes.c_uint32
    name = lambda st: _abi.STATUS_NAMES[st]
    assert name(L.sage_debug_e4m3_encode(u32(0), u32(16), None, None)) == "SAGE_ERR_NULL"
    assert name(L.sage_debug_e4m3_encode(u32(0), u32(16), ctypes.c_void_p(FAKE + 4),
                                         None)) == "SAGE_ERR_ALIGN"
    assert name(L.sage_debug_e4m3_encode(u32(0xFFFFFFF0), u32(32), ctypes.c_void_p(FAKE),
                                         None)) == "SAGE_ERR_SHAPE"


def test_micro_rate_argument_errors():
    # each case fails before any HIP call
    L = qa.lib()
    name = lambda st: _abi.STATUS_NAMES[st]
    r = ctypes.c_double(0.0)
    assert name(L.sage_micro_rate(0, 16, None, None)) == "SAGE_ERR_NULL"
    assert name(L.sage_micro_rate(4, 16, ctypes.byref(r), None)) == "SAGE_ERR_FLAGS"
    assert name(L.sage_micro_rate(-1, 16, ctypes.byref(r), None)) == "SAGE_ERR_FLAGS"
    assert name(L.sage_micro_rate(0, 0, ctypes.byref(r), None)) == "SAGE_ERR_SHAPE"
    assert name(L.sage_micro_rate(1, (1 << 20) + 1, ctypes.byref(r), None)) == "SAGE_ERR_SHAPE"
    with pytest.raises(ValueError):
        qa.sage_micro_rate("bf16")


def test_noalloc_refuses_large_workspace_before_any_gpu_call():
    # B=2, H=32, N=4096, d=128: about 100 MB of workspace, beyond the 64 MiB array
    L = qa.lib()
    d = _abi.Desc()
    L.sage_desc_init(ctypes.byref(d), _abi.BF16, _abi.NHD, 2, 32, 32, 4096, 4096, 128)
    ws = ctypes.c_size_t(0)
    assert L.sage_workspace_size(ctypes.byref(d), None, None, 0, ctypes.byref(ws)) == 0
    assert ws.value > _abi.NOALLOC_WS_MAX
    f = ctypes.c_void_p(FAKE)
    assert _abi.STATUS_NAMES[L.sage_attn_fwd_noalloc(ctypes.byref(d), f, f, f, f, None, None)] \
        == "SAGE_ERR_WORKSPACE"
    # and the descriptor checks come first, as in sage_attn_fwd
    d.head_dim = 80
    assert _abi.STATUS_NAMES[L.sage_attn_fwd_noalloc(ctypes.byref(d), f, f, f, f, None, None)] \
        == "SAGE_ERR_HEAD_DIM"
