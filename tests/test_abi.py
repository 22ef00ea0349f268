"""The C ABI on the host: the library loads, exports every function that
include/*.h declares, and rejects bad arguments before any HIP call (these
checks run without a GPU; no call here reaches a kernel launch)."""
import ctypes
import glob
import os
import re

import pytest

from quantized_kv_cache_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000        # aligned, never dereferenced: validation fails first


def header_functions():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    return _lib.load()


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.qkv_abi_version() == 6


def _pack(**kw):
    d = dict(mode=_lib.QKV_AFFINE, bits=4, group_size=64, scale_dtype=_lib.QKV_F16, B=1, H=2,
             L_cap=64, D=128, codes=FAKE, scales=FAKE + 0x100000, biases=FAKE + 0x200000,
             stride_b=128, stride_h=64, stride_l=1)
    d.update(kw)
    return _lib.QkvPack(**d)


def _quant(L, pk, x=FAKE + 0x400000, dt=_lib.QKV_F16, strides=(16384, 8192, 128), n=64):
    st = L.qkv_quantize(ctypes.c_void_p(x) if x else None, dt, _lib.i64_array(strides), n,
                        ctypes.byref(pk), None)
    return st, L.qkv_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(bits=7), _lib.QKV_EUNSUPPORTED, "bits"),
    (dict(group_size=48), _lib.QKV_EUNSUPPORTED, "group_size"),
    (dict(D=160, group_size=32), _lib.QKV_EUNSUPPORTED, "head size"),
    (dict(mode=_lib.QKV_QSYM, bits=6, group_size=32, biases=None), _lib.QKV_EINVAL, "bits 4 or 5"),
    (dict(mode=_lib.QKV_QSYM, bits=4, group_size=32), _lib.QKV_EINVAL, "biases"),
    (dict(D=160, group_size=64), _lib.QKV_EINVAL, "multiple"),
    (dict(codes=FAKE + 4), _lib.QKV_EINVAL, "aligned"),
    (dict(scales=FAKE + 0x100001), _lib.QKV_EINVAL, "misaligned"),
    (dict(scales=FAKE + 0x100002), _lib.QKV_EINVAL, "misaligned"),     # a scale row is 4 bytes
    (dict(biases=FAKE + 0x200002), _lib.QKV_EINVAL, "misaligned"),
    (dict(biases=None), _lib.QKV_EINVAL, "biases"),
    (dict(codes=None), _lib.QKV_EINVAL, "null"),
    (dict(mode=_lib.QKV_Q8_0, bits=8, group_size=32), _lib.QKV_EINVAL, "biases"),
    (dict(mode=_lib.QKV_Q8_0, bits=8, group_size=32, biases=None, scale_dtype=_lib.QKV_F32),
     _lib.QKV_EINVAL, "fp16"),
    (dict(stride_l=-1), _lib.QKV_EINVAL, "stride"),
    (dict(mode=7), _lib.QKV_EINVAL, "mode"),
])
def test_quantize_rejects_bad_packs(L, kw, status, msg):
    st, err = _quant(L, _pack(**kw))
    assert st == status and msg in err, (st, err)


def test_quantize_rejects_bad_sources(L):
    assert _quant(L, _pack(), x=0)[0] == _lib.QKV_EINVAL
    assert _quant(L, _pack(), x=FAKE + 0x400008)[0] == _lib.QKV_EINVAL          # misaligned
    assert _quant(L, _pack(), strides=(16384, 8192, 100))[0] == _lib.QKV_EINVAL  # not /8
    assert _quant(L, _pack(), n=65)[0] == _lib.QKV_EINVAL                       # > L_cap
    assert _quant(L, _pack(), dt=_lib.QKV_F32)[0] == _lib.QKV_EUNSUPPORTED      # scale != src
    st, _ = _quant(L, _pack(), n=0)                                             # nothing to do
    assert st == _lib.QKV_OK
    # a source row stride of 2^27 bytes or more
    st, err = _quant(L, _pack(), strides=(16384, 8192, 1 << 26))
    assert st == _lib.QKV_EUNSUPPORTED and "2^27" in err, (st, err)


def _append(L, kp, vp, T=1, offset=0, k=FAKE + 0x400000, v=FAKE + 0x500000):
    return L.qkv_update_append(ctypes.c_void_p(k), ctypes.c_void_p(v), _lib.QKV_F16,
                               _lib.i64_array((256, 128, 128)), T, offset, ctypes.byref(kp),
                               ctypes.byref(vp), None)


def test_append_rejects(L):
    kp = _pack()
    vp = _pack(codes=FAKE + 0x800000, scales=FAKE + 0x900000, biases=FAKE + 0xa00000)
    assert _append(L, kp, vp, offset=64) == _lib.QKV_EINVAL          # past capacity
    assert _append(L, kp, vp, offset=-1) == _lib.QKV_EINVAL
    assert _append(L, kp, vp, T=0) == _lib.QKV_EINVAL
    assert _append(L, kp, kp) == _lib.QKV_EINVAL                      # K and V alias
    assert _append(L, kp, _pack(bits=8)) == _lib.QKV_EINVAL           # formats differ
    assert _append(L, kp, vp, T=2, offset=63) == _lib.QKV_EINVAL
    assert "capacity" in L.qkv_last_error().decode()


def _decode(L, q=FAKE + 0x1000000, out=FAKE + 0x2000000, kp=None, vp=None, Hq=4, Ln=64,
            mask=None, ms=None, ws=None, wsb=0, opts=None, qdt=_lib.QKV_F16):
    kp = kp or _pack()
    vp = vp or _pack(codes=FAKE + 0x800000, scales=FAKE + 0x900000, biases=FAKE + 0xa00000)
    return L.qsdpa_decode(ctypes.c_void_p(q) if q else None, qdt, 1, Hq, 128, ctypes.byref(kp),
                          ctypes.byref(vp), Ln, 1.0, ctypes.c_void_p(mask) if mask else None,
                          _lib.QKV_F32, _lib.i64_array(ms) if ms else None,
                          ctypes.c_void_p(out) if out else None,
                          ctypes.c_void_p(ws) if ws else None, wsb,
                          ctypes.byref(opts) if opts else None, None)


def test_decode_rejects(L):
    assert _decode(L, Hq=3) == _lib.QKV_EINVAL                        # Hq % Hk
    assert _decode(L, Ln=0) == _lib.QKV_EINVAL
    assert _decode(L, Ln=65) == _lib.QKV_EINVAL                       # > L_cap
    assert _decode(L, q=0) == _lib.QKV_EINVAL
    assert _decode(L, out=FAKE + 0x1000000) == _lib.QKV_EINVAL        # out aliases q
    assert _decode(L, out=FAKE + 0x100) == _lib.QKV_EINVAL            # out overlaps codes
    assert _decode(L, qdt=_lib.QKV_F32) == _lib.QKV_EUNSUPPORTED      # scale dtype != q
    assert _decode(L, vp=_pack(bits=8, codes=FAKE + 0x800000, scales=FAKE + 0x900000,
                               biases=FAKE + 0xa00000)) == _lib.QKV_EINVAL
    assert _decode(L, mask=FAKE + 0x3000000, ms=(0, 0, 0, -1)) == _lib.QKV_EINVAL
    # partitioned plans need a workspace
    opts = _lib.QkvAttnOpts(num_splits=4, algo=_lib.QKV_ALGO_GENERIC)
    assert _decode(L, opts=opts) == _lib.QKV_EWORKSPACE
    assert "workspace" in L.qkv_last_error().decode()
    assert _decode(L, opts=_lib.QkvAttnOpts(num_splits=-1, algo=0)) == _lib.QKV_EINVAL


def _decode_append(L, offset=63, kn=FAKE + 0x3000000, vn=FAKE + 0x3100000, strides=(256, 128, 128),
                   q=FAKE + 0x1000000, out=FAKE + 0x2000000, kp=None, vp=None, qdt=_lib.QKV_F16):
    kp = kp or _pack()
    vp = vp or _pack(codes=FAKE + 0x800000, scales=FAKE + 0x900000, biases=FAKE + 0xa00000)
    return L.qsdpa_decode_append(ctypes.c_void_p(q), qdt, 1, 4, 128, ctypes.c_void_p(kn) if kn else None,
                                 ctypes.c_void_p(vn) if vn else None, _lib.i64_array(strides), offset,
                                 ctypes.byref(kp), ctypes.byref(vp), 1.0, None, _lib.QKV_F32, None,
                                 ctypes.c_void_p(out), None, 0, None, None)


def test_decode_append_rejects(L):
    """qsdpa_decode_append checks the append (T = 1, the query dtype) and the
    decode over offset + 1 keys before it enqueues anything."""
    assert _decode_append(L, offset=64) == _lib.QKV_EINVAL               # row 64 beyond L_cap
    assert "capacity" in L.qkv_last_error().decode()
    assert _decode_append(L, offset=-1) == _lib.QKV_EINVAL
    assert _decode_append(L, kn=0) == _lib.QKV_EINVAL                    # null k_new
    assert _decode_append(L, vn=FAKE + 0x3100008) == _lib.QKV_EINVAL     # v_new not 16-byte aligned
    assert _decode_append(L, strides=(256, 128, 12)) == _lib.QKV_EINVAL  # stride not a multiple of 8
    assert _decode_append(L, qdt=_lib.QKV_F32) == _lib.QKV_EUNSUPPORTED  # scale dtype != new-token dtype
    assert _decode_append(L, out=FAKE + 0x100) == _lib.QKV_EINVAL        # out overlaps the K codes
    assert _decode_append(L, q=0) == _lib.QKV_EINVAL
    assert _decode_append(L, kn=FAKE + 0x2000000) == _lib.QKV_EINVAL     # k_new is out
    assert "new token" in L.qkv_last_error().decode()
    assert _decode_append(L, vn=FAKE + 0x900000) == _lib.QKV_EINVAL      # v_new inside V's scales


def test_workspace_bytes(L):
    kp = _pack()
    one = _lib.QkvAttnOpts(num_splits=1, algo=_lib.QKV_ALGO_GENERIC)
    four = _lib.QkvAttnOpts(num_splits=4, algo=_lib.QKV_ALGO_GENERIC)
    assert L.qsdpa_workspace_bytes(1, 4, 1, 128, 64, ctypes.byref(kp), _lib.QKV_F16,
                                   ctypes.byref(one)) == 0
    n = L.qsdpa_workspace_bytes(1, 4, 1, 128, 64, ctypes.byref(kp), _lib.QKV_F16,
                                ctypes.byref(four))
    # the fixed ticket header, then splits x 16 rows x (m, l, o[D]) floats per
    # (b, kv head, row tile)
    assert n == _lib.QKV_TICKET_BYTES + 2 * 2 * 16 * 130 * 4
    assert L.qsdpa_workspace_bytes(1, 3, 1, 128, 64, ctypes.byref(kp), _lib.QKV_F16, None) == 0


@pytest.mark.parametrize("shape, kernel", [
    # (B, Hq, Hk, Lq, D, L, q dtype, mode, bits, gs) -> kernel chosen by the plan
    ((1, 4, 1, 1, 64, 256, "f32", "affine", 8, 64), _lib.QKV_KERNEL_GENERIC),
    ((1, 32, 8, 1, 128, 65536, "f16", "affine", 4, 64), _lib.QKV_KERNEL_DECODE_NARROW),
    ((8, 32, 8, 1, 128, 16448, "f16", "affine", 8, 64), _lib.QKV_KERNEL_DECODE_NARROW),
    ((1, 32, 2, 1, 256, 20480, "f16", "q8_0", 8, 32), _lib.QKV_KERNEL_DECODE),
    ((1, 32, 2, 512, 256, 20480, "f16", "q8_0", 8, 32), _lib.QKV_KERNEL_PREFILL),
    ((1, 64, 2, 1, 128, 700, "f16", "affine", 4, 64), _lib.QKV_KERNEL_PREFILL),   # G = 32
    ((1, 8, 2, 1, 128, 700, "bf16", "affine", 4, 64), _lib.QKV_KERNEL_GENERIC),
    ((1, 32, 8, 1, 128, 65536, "f16", "affine", 3, 64), _lib.QKV_KERNEL_DECODE_STREAM),
    ((1, 32, 8, 1, 96, 16384, "f16", "affine", 4, 32), _lib.QKV_KERNEL_DECODE_STREAM),
    ((1, 32, 8, 1, 128, 65536, "f16", "qsym", 5, 32), _lib.QKV_KERNEL_DECODE_STREAM),
    ((1, 32, 4, 1, 128, 4096, "f16", "affine", 3, 64), _lib.QKV_KERNEL_GENERIC),   # G = 8
])
def test_plan_kernel_choice(L, shape, kernel):
    """The plan names the kernel each workload shape runs on (host logic only)."""
    B, Hq, Hk, Lq, D, Lk, qdt, mode, bits, gs = shape
    dt = {"f32": _lib.QKV_F32, "f16": _lib.QKV_F16, "bf16": _lib.QKV_BF16}[qdt]
    kp = _lib.QkvPack(mode={"affine": _lib.QKV_AFFINE, "q8_0": _lib.QKV_Q8_0, "qsym": _lib.QKV_QSYM}[mode],
                      bits=bits, group_size=gs, scale_dtype=dt if mode == "affine" else _lib.QKV_F16,
                      B=B, H=Hk, L_cap=Lk, D=D, codes=FAKE, scales=FAKE + 0x10000000,
                      biases=FAKE + 0x20000000 if mode == "affine" else None,
                      stride_b=Hk * Lk, stride_h=Lk, stride_l=1)
    pl = _lib.QkvAttnPlan()
    assert L.qsdpa_plan(B, Hq, Lq, D, Lk, ctypes.byref(kp), dt, None, ctypes.byref(pl)) == 0
    assert pl.kernel == kernel
    assert pl.algo == (_lib.QKV_ALGO_GENERIC if kernel in (_lib.QKV_KERNEL_GENERIC, _lib.QKV_KERNEL_DECODE_STREAM)
                       else _lib.QKV_ALGO_MATRIX)
    assert 1 <= pl.num_splits <= 256 and pl.num_splits * pl.keys_per_split >= Lk
    if kernel == _lib.QKV_KERNEL_PREFILL:
        # 128 GQA-packed rows per workgroup from 256 rows per (batch, kv head)
        assert pl.row_tile == (128 if (Hq // Hk) * Lq >= 256 else 64)


def test_plan_narrow_decode_tickets_fit_header(L):
    """The narrow decode merges its key splits in the kernel with one ticket
    per (batch, kv head) in the fixed ticket header: a call with more (batch,
    kv head) pairs than the header holds runs unsplit, even when splits are
    asked for."""
    words = _lib.QKV_TICKET_BYTES // 4
    for B, splits in ((words // 4, 8), (words // 4 + 1, 8), (words // 4 + 1, 0)):
        Hk, Hq, Lk, D = 4, 16, 4096, 128
        kp = _lib.QkvPack(mode=_lib.QKV_AFFINE, bits=4, group_size=64, scale_dtype=_lib.QKV_F16,
                          B=B, H=Hk, L_cap=Lk, D=D, codes=FAKE, scales=FAKE + 0x10000000,
                          biases=FAKE + 0x20000000, stride_b=Hk * Lk, stride_h=Lk, stride_l=1)
        opts = _lib.QkvAttnOpts(num_splits=splits)
        pl = _lib.QkvAttnPlan()
        assert L.qsdpa_plan(B, Hq, 1, D, Lk, ctypes.byref(kp), _lib.QKV_F16, ctypes.byref(opts),
                            ctypes.byref(pl)) == 0
        assert pl.kernel == _lib.QKV_KERNEL_DECODE_NARROW
        if B * Hk > words:
            assert pl.num_splits == 1
        else:
            assert pl.num_splits == splits


def test_plan_splits_do_not_collapse_past_a_granule(L):
    """The 16-row decode splits the keys in whole 256-key granules: one key
    more than 80 granules must not halve the splits (a chunk of 257 keys
    rounded up to 512), and an exact multiple keeps its plan."""
    for Lk, want in ((20480, 80), (20481, 81), (20700, 81)):
        kp = _lib.QkvPack(mode=_lib.QKV_Q8_0, bits=8, group_size=32, scale_dtype=_lib.QKV_F16,
                          B=1, H=2, L_cap=20736, D=256, codes=FAKE, scales=FAKE + 0x10000000, biases=None,
                          stride_b=2 * 20736, stride_h=20736, stride_l=1)
        pl = _lib.QkvAttnPlan()
        assert L.qsdpa_plan(1, 32, 1, 256, Lk, ctypes.byref(kp), _lib.QKV_F16, None, ctypes.byref(pl)) == 0
        assert pl.kernel == _lib.QKV_KERNEL_DECODE
        assert pl.num_splits == want and pl.keys_per_split == 256, (Lk, pl.num_splits, pl.keys_per_split)


@pytest.mark.parametrize("Lq,rows", [(15, 64), (16, 128), (100, 128)])
def test_prefill_row_tile(L, Lq, rows):
    """Prefill row tiles: 64 rows below 256 GQA-packed rows per (batch, kv
    head), 128 from there (host logic only)."""
    kp = _lib.QkvPack(mode=_lib.QKV_Q8_0, bits=8, group_size=32, scale_dtype=_lib.QKV_F16,
                      B=1, H=2, L_cap=4096, D=128, codes=FAKE, scales=FAKE + 0x10000000,
                      biases=None, stride_b=2 * 4096, stride_h=4096, stride_l=1)
    pl = _lib.QkvAttnPlan()
    assert L.qsdpa_plan(1, 32, Lq, 128, 4096, ctypes.byref(kp), _lib.QKV_F16, None,
                        ctypes.byref(pl)) == 0
    assert pl.kernel == _lib.QKV_KERNEL_PREFILL and pl.row_tile == rows


def test_measure_read_rejects_bad_arguments(L):
    sink = FAKE + 0x400000
    for buf, nbytes, wgs, snk in ((0, 4096, 64, sink), (FAKE, 4096, 64, 0), (FAKE, 0, 64, sink),
                                  (FAKE, 4100, 64, sink), (FAKE + 8, 4096, 64, sink),
                                  (FAKE, 4096, 0, sink), (FAKE, 4096, 8193, sink)):
        assert L.qkv_measure_read(buf, nbytes, wgs, snk, None) == _lib.QKV_EINVAL, (buf, nbytes, wgs)
        assert L.qkv_last_error()


def test_decode_rejects_workspace_overlapping_inputs(L):
    """The workspace is written by the call: it may not overlap q, either
    pack or the mask (nor out)."""
    opts = _lib.QkvAttnOpts(num_splits=4, algo=_lib.QKV_ALGO_GENERIC)
    need = L.qsdpa_workspace_bytes(1, 4, 1, 128, 64, ctypes.byref(_pack()), _lib.QKV_F16,
                                   ctypes.byref(opts))
    good = FAKE + 0x4000000
    assert need > _lib.QKV_TICKET_BYTES
    for ws, what in ((FAKE + 0x1000000 - 256 * 1024, "q"),          # runs into q
                     (FAKE + 0x800000 - 256 * 1024, "pack"),        # runs into V's codes
                     (FAKE + 0x100000, "pack"),                     # K's scales
                     (FAKE + 0x2000000, "out")):
        st = _decode(L, ws=ws, wsb=need, opts=opts)
        assert st == _lib.QKV_EINVAL and what in L.qkv_last_error().decode(), (hex(ws), what)
    st = _decode(L, ws=FAKE + 0x3000000 - 4096, wsb=need, opts=opts, mask=FAKE + 0x3000000,
                 ms=(0, 0, 0, 1))
    assert st == _lib.QKV_EINVAL and "mask" in L.qkv_last_error().decode()
    # out may not overlap the mask either
    st = _decode(L, mask=FAKE + 0x2000000, ms=(0, 0, 0, 1))
    assert st == _lib.QKV_EINVAL and "mask" in L.qkv_last_error().decode()
    assert good > 0


def test_workspace_reset_rejects(L):
    assert L.qsdpa_workspace_reset(None, _lib.QKV_TICKET_BYTES, None) == _lib.QKV_EINVAL
    assert L.qsdpa_workspace_reset(FAKE + 16, _lib.QKV_TICKET_BYTES, None) == _lib.QKV_EINVAL
    assert L.qsdpa_workspace_reset(FAKE, _lib.QKV_TICKET_BYTES - 256, None) == _lib.QKV_EINVAL
    assert "ticket header" in L.qkv_last_error().decode()


def test_measure_read_config_rejects_bad_arguments(L):
    sink = FAKE + 0x400000
    good = dict(buf=FAKE, nbytes=4096, wgs=64, threads=256, u=4, width=16, snk=sink)
    bad = [dict(buf=0), dict(snk=0), dict(width=2), dict(nbytes=4100), dict(buf=FAKE + 8),
           dict(threads=100), dict(threads=2048), dict(u=3), dict(u=32), dict(wgs=0),
           dict(wgs=8193), dict(nbytes=0)]
    for b in bad:
        a = dict(good, **b)
        st = L.qkv_measure_read_config(a["buf"], a["nbytes"], a["wgs"], a["threads"], a["u"],
                                       a["width"], a["snk"], None)
        assert st == _lib.QKV_EINVAL, b
        assert L.qkv_last_error()


def _dense(**kw):
    d = dict(mode=_lib.QKV_DENSE, bits=16, group_size=128, scale_dtype=_lib.QKV_F16, B=1, H=2,
             L_cap=64, D=128, codes=FAKE + 0x3000000, scales=None, biases=None,
             stride_b=128, stride_h=64, stride_l=1)
    d.update(kw)
    return _lib.QkvPack(**d)


@pytest.mark.parametrize("kw,msg", [(dict(bits=8), "fp16"), (dict(group_size=64), "fp16"),
                                    (dict(scale_dtype=_lib.QKV_F32), "fp16"),
                                    (dict(scales=FAKE), "no scales"), (dict(codes=FAKE + 8), "aligned")])
def test_dense_pack_rules(L, kw, msg):
    st = L.qkv_dequantize(ctypes.byref(_pack()), 8, ctypes.byref(_dense(**kw)), None)
    assert st == _lib.QKV_EINVAL and msg in L.qkv_last_error().decode(), L.qkv_last_error()


def test_dequantize_rejects(L):
    src, dst = _pack(), _dense()
    assert L.qkv_dequantize(ctypes.byref(dst), 8, ctypes.byref(dst), None) == _lib.QKV_EINVAL
    assert L.qkv_dequantize(ctypes.byref(src), 8, ctypes.byref(_pack(codes=FAKE + 0x3000000)),
                            None) == _lib.QKV_EINVAL                            # dst not dense
    assert L.qkv_dequantize(ctypes.byref(src), 65, ctypes.byref(dst), None) == _lib.QKV_EINVAL
    assert L.qkv_dequantize(ctypes.byref(src), 8, ctypes.byref(_dense(H=3)), None) == _lib.QKV_EINVAL
    assert L.qkv_dequantize(ctypes.byref(src), 8, ctypes.byref(_dense(codes=FAKE)), None) == \
        _lib.QKV_EINVAL                                                          # overlap
    assert L.qkv_dequantize(ctypes.byref(_pack(scale_dtype=_lib.QKV_F32)), 8, ctypes.byref(dst),
                            None) == _lib.QKV_EUNSUPPORTED
    assert L.qkv_dequantize(ctypes.byref(src), 0, ctypes.byref(dst), None) == _lib.QKV_OK


def test_dense_and_dequant_first_plans(L):
    dense = _dense(L_cap=4096, stride_b=8192, stride_h=4096)
    pl = _lib.QkvAttnPlan()
    assert L.qsdpa_plan(1, 8, 1, 128, 4096, ctypes.byref(dense), _lib.QKV_F16, None,
                        ctypes.byref(pl)) == 0
    assert pl.kernel == _lib.QKV_KERNEL_PREFILL
    q8 = _lib.QkvPack(mode=_lib.QKV_Q8_0, bits=8, group_size=32, scale_dtype=_lib.QKV_F16, B=1,
                      H=2, L_cap=4096, D=128, codes=FAKE, scales=FAKE + 0x10000000, biases=None,
                      stride_b=8192, stride_h=4096, stride_l=1)
    opts = _lib.QkvAttnOpts(num_splits=0, algo=_lib.QKV_ALGO_DEQUANT_F16)
    assert L.qsdpa_plan(1, 32, 64, 128, 4000, ctypes.byref(q8), _lib.QKV_F16, ctypes.byref(opts),
                        ctypes.byref(pl)) == 0
    assert pl.algo == _lib.QKV_ALGO_DEQUANT_F16 and pl.kernel == _lib.QKV_KERNEL_PREFILL
    # two dense fp16 copies of the 4000 attended rows come first in the workspace
    assert pl.workspace_bytes >= 2 * 2 * 4000 * 128 * 2
    # dense packs need fp16 queries
    st = L.qsdpa_decode(ctypes.c_void_p(FAKE + 0x1000000), _lib.QKV_F32, 1, 8, 128,
                        ctypes.byref(dense), ctypes.byref(_dense(codes=FAKE + 0x5000000, L_cap=4096,
                                                                 stride_b=8192, stride_h=4096)),
                        64, 1.0, None, 0, None, ctypes.c_void_p(FAKE + 0x2000000), None, 0, None, None)
    assert st == _lib.QKV_EUNSUPPORTED
