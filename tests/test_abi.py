"""CPU tests of the C-ABI library: it loads, exports every symbol that
include/wa.h declares, and rejects bad arguments on the host before any HIP
call (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wa.h")
DIAG_HEADER = os.path.join(ROOT, "include", "wa_diag.h")


@pytest.fixture(scope="module")
def wa():
    import whisper_attention_amd as wa
    return wa


def _declared(header=HEADER):
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(wa_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_three_operations():
    names = _declared()
    for n in ("wa_kv_quant_fp8", "wa_encoder_attn", "wa_decode_attn"):
        assert n in names


def test_library_exports_every_declared_symbol(wa):
    for name in _declared():
        assert hasattr(wa.lib, name), name
    assert set(wa.EXPORTED) == set(_declared())


def test_status_strings(wa):
    for s in range(5):
        assert wa.wa_status_string(s).startswith("WA_")
    assert "unknown" in wa.wa_status_string(99)


def test_workspace_sizes(wa):
    assert wa.wa_kv_quant_fp8_workspace_size(128, 20, "head") > 0
    assert wa.wa_kv_quant_fp8_workspace_size(128, 20, "tensor") > 0
    assert wa.wa_kv_quant_fp8_workspace_size(0, 20, "head") == 0
    # the counter plus at most 32 partials per sequence and scale group
    assert wa.wa_kv_quant_fp8_workspace_size(128, 20, "head") == 256 + 128 * 32 * 20 * 4
    assert wa.wa_kv_quant_fp8_workspace_size(3, 20, "tensor") == 768   # 256 + 3 * 32 * 4, rounded up to 256
    assert wa.lib.wa_kv_quant_fp8_workspace_size(3, 20, 7) == 0          # no such granularity
    assert wa.wa_decode_attn_workspace_size(1, 6, 1500) > 0      # split keys -> partials
    # 640 split counters (2560 bytes), then n_split * B * H partials of 68 floats
    n = wa.wa_decode_attn_workspace_size(1, 6, 1500)
    assert (n - 2560) % (6 * 68 * 4) == 0 and (n - 2560) // (6 * 68 * 4) > 1
    assert wa.wa_decode_attn_workspace_size(0, 6, 1500) == 0
    # a big batch needs no split, hence no workspace
    assert wa.wa_decode_attn_workspace_size(256, 20, 1500) == 0


FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation
MIS = 0x10002           # misaligned


def _S(wa, b=20 * 64 * 1500, t=20 * 64, h=64):
    return wa.Strides(b, t, h)


def _quant(wa, **kw):
    a = dict(x=FAKE, xs=_S(wa), B=2, H=20, T=1500, D=64, lens=None, dst=None, cache=FAKE,
             cs=wa.Strides(20 * 1500 * 64, 64, 1500 * 64), L=1500, scale=FAKE, gran=0, cs_=1,
             ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return wa.lib.wa_kv_quant_fp8(a["x"], a["xs"], a["B"], a["H"], a["T"], a["D"], a["lens"], a["dst"],
                                  a["cache"], a["cs"], a["L"], a["scale"], a["gran"], a["cs_"],
                                  a["ws"], a["wsb"], a["stream"])


def test_quant_validation(wa):
    assert _quant(wa, x=None) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, cache=None) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, scale=None) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, B=0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, H=-1) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, L=0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, gran=2) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, cs_=3) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, D=128) == wa.WA_ERR_UNSUPPORTED
    assert _quant(wa, x=MIS) == wa.WA_ERR_UNSUPPORTED
    assert _quant(wa, xs=_S(wa, t=20 * 64 + 4)) == wa.WA_ERR_UNSUPPORTED
    assert _quant(wa, cs=wa.Strides(20 * 1500 * 64, 8, 1500 * 64)) == wa.WA_ERR_UNSUPPORTED
    assert _quant(wa, ws=None) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant(wa, ws=MIS, wsb=1 << 20) == wa.WA_ERR_UNSUPPORTED
    assert _quant(wa, wsb=16) == wa.WA_ERR_WORKSPACE_TOO_SMALL


def _quant_fmt(wa, fmt, **kw):
    a = dict(x=FAKE, xs=_S(wa), B=2, H=20, T=1500, D=64, lens=None, dst=None, cache=FAKE,
             cs=wa.Strides(20 * 1500 * 64, 64, 1500 * 64), L=1500, scale=FAKE, gran=0, cs_=1,
             ws=FAKE, wsb=0)
    a.update(kw)
    return wa.lib.wa_kv_quant_fp8_fmt(a["x"], a["xs"], a["B"], a["H"], a["T"], a["D"], a["lens"],
                                      a["dst"], a["cache"], a["cs"], a["L"], a["scale"], a["gran"],
                                      fmt, a["cs_"], a["ws"], a["wsb"], None)


def test_quant_fmt_validation(wa):
    assert _quant_fmt(wa, 2) == wa.WA_ERR_INVALID_ARGUMENT
    assert _quant_fmt(wa, -1) == wa.WA_ERR_INVALID_ARGUMENT
    for fmt in (wa.WA_FP8_E4M3, wa.WA_FP8_E5M2):
        assert _quant_fmt(wa, fmt, x=None) == wa.WA_ERR_INVALID_ARGUMENT
        assert _quant_fmt(wa, fmt, D=128) == wa.WA_ERR_UNSUPPORTED
        assert _quant_fmt(wa, fmt, wsb=16) == wa.WA_ERR_WORKSPACE_TOO_SMALL


def test_quant_pair_validation(wa):
    S = _S(wa)
    cs = wa.Strides(20 * 1500 * 64, 64, 1500 * 64)

    def call(**kw):
        a = dict(k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, ksc=FAKE, vsc=FAKE, gran=0, fmt=0, wsb=0, D=64, vs=S)
        a.update(kw)
        return wa.lib.wa_kv_quant_fp8_kv(a["k"], S, a["v"], a["vs"], 2, 20, 1500, a["D"], None, None, a["kc"],
                                         a["vc"], cs, 1500, a["ksc"], a["vsc"], a["gran"], a["fmt"], 1, FAKE,
                                         a["wsb"], None)
    for name in ("k", "v", "kc", "vc", "ksc", "vsc"):
        assert call(**{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    assert call(fmt=2) == wa.WA_ERR_INVALID_ARGUMENT
    assert call(D=32) == wa.WA_ERR_UNSUPPORTED
    assert call(vs=_S(wa, t=20 * 64 + 4)) == wa.WA_ERR_UNSUPPORTED
    # the workspace holds two tensors' partials
    one = wa.wa_kv_quant_fp8_workspace_size(2, 20, "tensor")
    assert call(wsb=one) == wa.WA_ERR_WORKSPACE_TOO_SMALL


def _dequant(wa, **kw):
    a = dict(cache=FAKE, cs=wa.Strides(20 * 1500 * 64, 64, 1500 * 64), L=1500, scale=FAKE, gran=0,
             fmt=0, lens=None, B=2, H=20, T=1500, D=64, x=FAKE, xs=_S(wa))
    a.update(kw)
    return wa.lib.wa_kv_dequant_fp8(a["cache"], a["cs"], a["L"], a["scale"], a["gran"], a["fmt"],
                                    a["lens"], a["B"], a["H"], a["T"], a["D"], a["x"], a["xs"], None)


def test_dequant_validation(wa):
    for name in ("cache", "scale", "x"):
        assert _dequant(wa, **{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    for name in ("B", "H", "T", "L"):
        assert _dequant(wa, **{name: 0}) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dequant(wa, gran=2) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dequant(wa, fmt=3) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dequant(wa, D=32) == wa.WA_ERR_UNSUPPORTED
    assert _dequant(wa, B=65536) == wa.WA_ERR_UNSUPPORTED
    assert _dequant(wa, x=MIS) == wa.WA_ERR_UNSUPPORTED
    assert _dequant(wa, cache=MIS) == wa.WA_ERR_UNSUPPORTED
    assert _dequant(wa, xs=_S(wa, t=20 * 64 + 4)) == wa.WA_ERR_UNSUPPORTED
    assert _dequant(wa, cs=wa.Strides(20 * 1500 * 64, 8, 1500 * 64)) == wa.WA_ERR_UNSUPPORTED


def _enc(wa, **kw):
    s = _S(wa)
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, qs=s, ks=s, vs=s, os=s, B=2, H=20, T=1500, D=64,
             lens=None, causal=0, sc=0.125)
    a.update(kw)
    return wa.lib.wa_encoder_attn(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"],
                                  a["B"], a["H"], a["T"], a["D"], a["lens"], a["causal"], a["sc"], None)


def test_encoder_validation(wa):
    for name in ("q", "k", "v", "o"):
        assert _enc(wa, **{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc(wa, T=0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc(wa, causal=2) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc(wa, sc=0.0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc(wa, sc=float("nan")) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc(wa, D=80) == wa.WA_ERR_UNSUPPORTED
    assert _enc(wa, o=MIS) == wa.WA_ERR_UNSUPPORTED
    assert _enc(wa, ks=_S(wa, h=65)) == wa.WA_ERR_UNSUPPORTED
    # a position stride whose 64-row tile does not fit a 32-bit byte offset
    assert _enc(wa, vs=_S(wa, t=1 << 24)) == wa.WA_ERR_UNSUPPORTED
    assert _enc(wa, ks=_S(wa, t=1 << 24)) == wa.WA_ERR_UNSUPPORTED


def _cross(wa, **kw):
    s = _S(wa)
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, qs=s, ks=s, vs=s, os=s, B=2, H=20, Tq=224, Tk=1500, D=64,
             ql=None, kl=None, sc=0.125)
    a.update(kw)
    return wa.lib.wa_cross_attn(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"],
                                a["B"], a["H"], a["Tq"], a["Tk"], a["D"], a["ql"], a["kl"], a["sc"], None)


def test_cross_validation(wa):
    for name in ("q", "k", "v", "o"):
        assert _cross(wa, **{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    for name in ("B", "H", "Tq", "Tk"):
        assert _cross(wa, **{name: 0}) == wa.WA_ERR_INVALID_ARGUMENT
    assert _cross(wa, sc=float("inf")) == wa.WA_ERR_INVALID_ARGUMENT
    assert _cross(wa, sc=-0.125) == wa.WA_ERR_INVALID_ARGUMENT
    assert _cross(wa, D=32) == wa.WA_ERR_UNSUPPORTED
    for name in ("q", "k", "v", "o"):
        assert _cross(wa, **{name: MIS}) == wa.WA_ERR_UNSUPPORTED
    assert _cross(wa, qs=_S(wa, b=4)) == wa.WA_ERR_UNSUPPORTED
    assert _cross(wa, ks=_S(wa, t=1 << 24)) == wa.WA_ERR_UNSUPPORTED
    assert _cross(wa, vs=_S(wa, t=1 << 24)) == wa.WA_ERR_UNSUPPORTED


def _enc8(wa, **kw):
    s = _S(wa)
    a = dict(q=FAKE, qs=s, qsc=FAKE, k=FAKE, ks=s, ksc=FAKE, gran=0, v=FAKE, vs=s, o=FAKE, os=s, B=2, H=20,
             T=1500, D=64, lens=None, causal=0, sc=0.125)
    a.update(kw)
    return wa.lib.wa_encoder_attn_fp8qk(a["q"], a["qs"], a["qsc"], a["k"], a["ks"], a["ksc"], a["gran"],
                                        a["v"], a["vs"], a["o"], a["os"], a["B"], a["H"], a["T"], a["D"],
                                        a["lens"], a["causal"], a["sc"], None)


def test_encoder_fp8qk_validation(wa):
    for name in ("q", "k", "v", "o", "qsc", "ksc"):
        assert _enc8(wa, **{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc8(wa, gran=5) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc8(wa, causal=3) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc8(wa, sc=-1.0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _enc8(wa, D=128) == wa.WA_ERR_UNSUPPORTED
    assert _enc8(wa, q=MIS) == wa.WA_ERR_UNSUPPORTED
    # uint8 Q/K strides must be multiples of 16 bytes
    assert _enc8(wa, ks=_S(wa, t=20 * 64 + 8)) == wa.WA_ERR_UNSUPPORTED
    assert _enc8(wa, ks=_S(wa, t=1 << 25)) == wa.WA_ERR_UNSUPPORTED
    assert _enc8(wa, vs=_S(wa, t=1 << 24)) == wa.WA_ERR_UNSUPPORTED


def _dec(wa, **kw):
    cs = wa.Strides(20 * 1500 * 64, 64, 1500 * 64)
    a = dict(q=FAKE, qs=wa.Strides(20 * 64, 0, 64), kc=FAKE, vc=FAKE, cs=cs, L=1500, ks=FAKE, vs=FAKE,
             gran=0, lens=FAKE, B=1, H=6, D=64, sc=0.125, o=FAKE, os=wa.Strides(20 * 64, 0, 64),
             ws=FAKE, wsb=0)
    a.update(kw)
    return wa.lib.wa_decode_attn(a["q"], a["qs"], a["kc"], a["vc"], a["cs"], a["L"], a["ks"], a["vs"],
                                 a["gran"], a["lens"], a["B"], a["H"], a["D"], a["sc"], a["o"], a["os"],
                                 a["ws"], a["wsb"], None)


def test_decode_validation(wa):
    for name in ("q", "kc", "vc", "ks", "vs", "lens", "o"):
        assert _dec(wa, **{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dec(wa, L=0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dec(wa, gran=7) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dec(wa, sc=float("inf")) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dec(wa, D=32) == wa.WA_ERR_UNSUPPORTED
    assert _dec(wa, kc=MIS) == wa.WA_ERR_UNSUPPORTED
    assert _dec(wa, qs=wa.Strides(20 * 64, 0, 60)) == wa.WA_ERR_UNSUPPORTED
    # B*H = 6 splits the 1500 keys, so a workspace is required
    assert _dec(wa, ws=None) == wa.WA_ERR_INVALID_ARGUMENT
    assert _dec(wa, wsb=64) == wa.WA_ERR_WORKSPACE_TOO_SMALL


def test_valid_call_without_device_reports_hip_error(wa):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: a valid call with fake pointers would launch")
    assert _enc(wa) == wa.WA_ERR_HIP
    assert _cross(wa) == wa.WA_ERR_HIP


def _app(wa, **kw):
    cs = wa.Strides(20 * 1500 * 64, 64, 1500 * 64)
    ts = wa.Strides(20 * 64, 0, 64)
    a = dict(q=FAKE, qs=ts, kn=FAKE, vn=FAKE, ns=ts, kc=FAKE, vc=FAKE, cs=cs, L=1500, ks=FAKE, vs=FAKE,
             gran=0, lens=FAKE, B=1, H=6, D=64, sc=0.125, o=FAKE, os=ts, ws=FAKE, wsb=0)
    a.update(kw)
    return wa.lib.wa_decode_attn_append(a["q"], a["qs"], a["kn"], a["vn"], a["ns"], a["kc"], a["vc"],
                                        a["cs"], a["L"], a["ks"], a["vs"], a["gran"], a["lens"], a["B"],
                                        a["H"], a["D"], a["sc"], a["o"], a["os"], a["ws"], a["wsb"], None)


def test_decode_append_validation(wa):
    for name in ("q", "kn", "vn", "kc", "vc", "ks", "vs", "lens", "o"):
        assert _app(wa, **{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    assert _app(wa, B=0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _app(wa, D=128) == wa.WA_ERR_UNSUPPORTED
    assert _app(wa, kn=MIS) == wa.WA_ERR_UNSUPPORTED
    assert _app(wa, ns=wa.Strides(20 * 64, 0, 12)) == wa.WA_ERR_UNSUPPORTED
    assert _app(wa, ws=None) == wa.WA_ERR_INVALID_ARGUMENT
    assert _app(wa, wsb=64) == wa.WA_ERR_WORKSPACE_TOO_SMALL


def test_binding_refuses_host_tensors_and_bad_vectors(wa):
    """The binding passes only device pointers: host tensors are refused
    before any library call (the kernels would dereference them on the GPU)."""
    import torch
    q = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        wa.wa_encoder_attn(q, q, q, out=torch.empty_like(q))
    with pytest.raises(ValueError, match="GPU tensor"):
        wa.wa_cross_attn(q, q, q)
    with pytest.raises(ValueError, match="k and v"):
        wa.wa_cross_attn(q, q[:, :, :1], q)
    c = torch.zeros((1, 2, 4, 64), dtype=torch.uint8)
    s = torch.ones(1, dtype=torch.float32)
    with pytest.raises(ValueError):
        wa.wa_decode_attn(torch.zeros((1, 2, 64), dtype=torch.bfloat16), c, c, s, s,
                          torch.ones(1, dtype=torch.int32), "tensor", workspace=torch.zeros(16, dtype=torch.uint8))
    # a vector of the wrong dtype or length is refused whatever its device
    with pytest.raises(ValueError, match="lens"):
        wa._vec(torch.ones(3, dtype=torch.int64), torch.int32, 3, "lens")
    with pytest.raises(ValueError, match="scale"):
        wa._vec(torch.ones(2, dtype=torch.float32), torch.float32, 20, "scale")


def test_diag_library_exports_and_validates():
    """The measurement probes (libwa_diag.so, include/wa_diag.h) load, export
    what the header declares, and refuse bad arguments before any launch."""
    from whisper_attention_amd import diag
    names = _declared(DIAG_HEADER)
    assert set(diag.EXPORTED) == set(names)
    for n in names:
        assert hasattr(diag.lib, n), n
    assert diag.lib.wa_diag_mfma_ceiling(0, 512, 16, None, None) == 1
    assert diag.lib.wa_diag_mfma_ceiling(2, 512, 16, FAKE, None) == 1
    assert diag.lib.wa_diag_mfma_ceiling(0, 0, 16, FAKE, None) == 1
    assert diag.lib.wa_diag_mfma_ceiling(1, 512, (1 << 20) + 1, FAKE, None) == 1
    assert diag.lib.wa_diag_wall_clock_khz(None) == 1
    assert diag.lib.wa_diag_sclk_probe(8, 500, None, None) == 1
    assert diag.lib.wa_diag_sclk_probe(0, 500, FAKE, None) == 1
    assert diag.lib.wa_diag_sclk_probe(8, 0, FAKE, None) == 1
    assert diag.lib.wa_diag_sclk_probe(8, 100001, FAKE, None) == 1


@pytest.mark.parametrize("lang,std", [("c", "-std=c11"), ("c++", "-std=c++17")])
def test_headers_compile_as_plain_c_and_cpp(tmp_path, lang, std):
    """include/wa.h and include/wa_diag.h are a C ABI: a C (and a C++) file
    that includes both and takes the address of every declared function
    compiles with warnings as errors, against the ROCm runtime header only."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    names = _declared() + _declared(DIAG_HEADER)
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "wa.h"\n#include "wa_diag.h"\nint main(void) {\n' +
                   "".join(f"  (void)&{n};\n" for n in names) + "  return 0;\n}\n")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run([cc, std, "-fsyntax-only", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]


def test_binding_refuses_mismatched_shapes(wa):
    """Every size a kernel uses comes from one tensor, so the binding checks
    the others against it before any library call: a mismatch would be read
    or written out of bounds on the device.  (CPU tensors: the shape check
    comes first, so no pointer is ever taken.)"""
    import torch
    bf, u8, f32, i32 = torch.bfloat16, torch.uint8, torch.float32, torch.int32
    q = torch.zeros((2, 8, 3, 64), dtype=bf)
    short = torch.zeros((2, 7, 3, 64), dtype=bf)
    for kw in ({"k": short}, {"v": short}, {"out": short}):
        args = {"k": q, "v": q, "out": torch.empty_like(q)}
        args.update(kw)
        with pytest.raises(ValueError, match="expected shape"):
            wa.wa_encoder_attn(q, args["k"], args["v"], out=args["out"])
    with pytest.raises(ValueError, match="expected shape"):
        wa.wa_cross_attn(q, torch.zeros((2, 5, 3, 64), dtype=bf), torch.zeros((2, 5, 3, 64), dtype=bf),
                         out=short)
    qc = torch.zeros((2, 8, 3, 64), dtype=u8)
    s1 = torch.ones(1, dtype=f32)
    with pytest.raises(ValueError, match="expected shape"):
        wa.wa_encoder_attn_fp8qk(qc, s1, qc, s1, "tensor", q, out=short)
    # decode: caches [B][H][L][64] and out [B][H][64] against q [B][H][64]
    qd = torch.zeros((2, 3, 64), dtype=bf)
    lens = torch.ones(2, dtype=i32)
    ws = torch.zeros(16, dtype=u8)
    good = torch.zeros((2, 3, 10, 64), dtype=u8)
    for bad in (torch.zeros((1, 3, 10, 64), dtype=u8), torch.zeros((2, 4, 10, 64), dtype=u8),
                torch.zeros((2, 3, 10, 32), dtype=u8)):
        with pytest.raises(ValueError, match="expected shape"):
            wa.wa_decode_attn(qd, bad, bad, s1, s1, lens, "tensor", workspace=ws)
        with pytest.raises(ValueError, match="expected shape"):
            wa.wa_decode_attn_append(qd, qd, qd, bad, bad, s1, s1, lens, "tensor", workspace=ws)
    with pytest.raises(ValueError, match="expected shape"):
        wa.wa_decode_attn(qd, good, good, s1, s1, lens, "tensor", out=torch.zeros((2, 2, 64), dtype=bf),
                          workspace=ws)
    with pytest.raises(ValueError, match="expected shape"):
        wa.wa_decode_attn_append(qd, qd, qd, good, good, s1, s1, lens, "tensor",
                                 out=torch.zeros((1, 3, 64), dtype=bf), workspace=ws)
    # quantize: the cache [B][H][L][64] against x [B][T][H][64]
    x = torch.zeros((2, 8, 3, 64), dtype=bf)
    for bad in (torch.zeros((3, 3, 8, 64), dtype=u8), torch.zeros((2, 2, 8, 64), dtype=u8),
                torch.zeros((2, 3, 8, 16), dtype=u8)):
        with pytest.raises(ValueError, match="expected shape"):
            wa.wa_kv_quant_fp8(x, bad, s1, "tensor", workspace=ws)
        with pytest.raises(ValueError, match="expected shape"):
            wa.wa_kv_quant_fp8_kv(x, x, bad, bad, s1, s1, "tensor", workspace=ws)


def test_half_ulp_of_bf16_matches_the_format():
    """The parity bar's output-rounding term: half the distance from a bf16
    value to the next one up, checked against the bit patterns."""
    import numpy as np
    import torch
    from tests.gpu_helpers import half_ulp_bf16
    assert half_ulp_bf16(1.0) == 2.0 ** -8
    assert half_ulp_bf16(1.99) == 2.0 ** -8
    assert half_ulp_bf16(2.0) == 2.0 ** -7
    assert half_ulp_bf16(-0.75) == 2.0 ** -9
    assert half_ulp_bf16(64.0) == 0.25
    bits = np.arange(0x0080, 0x7F7F, 7, dtype=np.int32)          # positive normal bf16 patterns
    v = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    nxt = torch.from_numpy((bits + 1).astype(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(nxt - v, 2 * half_ulp_bf16(v))


def test_parity_bar_rejects_errors_beyond_the_bf16_bound():
    """assert_close applies the stated absolute bar where M <= 1 and the
    derived 2^-7 M + half-ulp bound everywhere."""
    import numpy as np
    import torch
    from tests.gpu_helpers import assert_close
    want = np.array([0.5, -0.25, 40.0, 70.0])
    mag = np.array([0.8, 0.9, 45.0, 70.0])
    got = torch.tensor(want, dtype=torch.float64)
    assert_close(got, want, "exact", mag=mag)
    # within the bound at large M: 0.3 < 2^-7 * 45 + 0.125
    assert_close(got + torch.tensor([0.0, 0.0, 0.3, 0.0], dtype=torch.float64), want, "large M", mag=mag)
    with pytest.raises(AssertionError, match="2\\^-7 M"):
        assert_close(got + torch.tensor([0.0, 0.0, 0.6, 0.0], dtype=torch.float64), want, "beyond", mag=mag)
    # M <= 1: 0.009 on one of 100 outputs is inside the stated max-abs and
    # mean-abs bars, but above 2^-7 * 0.8 + half-ulp
    w100, m100 = np.full(100, 0.5), np.full(100, 0.8)
    err = np.zeros(100)
    err[7] = 0.009
    with pytest.raises(AssertionError, match="2\\^-7 M"):
        assert_close(torch.from_numpy(w100 + err), w100, "small", mag=m100)
    # without M the stated bar applies to every output
    with pytest.raises(AssertionError, match="max-abs"):
        assert_close(got + torch.tensor([0.0, 0.0, 0.03, 0.0], dtype=torch.float64), want, "no M")


def _noalloc(wa, **kw):
    cs = wa.Strides(20 * 1500 * 64, 64, 1500 * 64)
    ts = wa.Strides(20 * 64, 0, 64)
    a = dict(q=FAKE, qs=ts, kc=FAKE, vc=FAKE, cs=cs, L=1500, ks=FAKE, vs=FAKE, gran=0, lens=FAKE, B=1, H=6,
             D=64, sc=0.125, o=FAKE, os=ts)
    a.update(kw)
    return wa.lib.wa_decode_attn_noalloc(a["q"], a["qs"], a["kc"], a["vc"], a["cs"], a["L"], a["ks"], a["vs"],
                                         a["gran"], a["lens"], a["B"], a["H"], a["D"], a["sc"], a["o"], a["os"],
                                         None)


def test_decode_noalloc_validation(wa):
    """The no-allocation decode entry point checks its arguments as
    wa_decode_attn does, on the host, before any HIP call."""
    for name in ("q", "kc", "vc", "ks", "vs", "lens", "o"):
        assert _noalloc(wa, **{name: None}) == wa.WA_ERR_INVALID_ARGUMENT
    assert _noalloc(wa, B=0) == wa.WA_ERR_INVALID_ARGUMENT
    assert _noalloc(wa, gran=3) == wa.WA_ERR_INVALID_ARGUMENT
    assert _noalloc(wa, D=128) == wa.WA_ERR_UNSUPPORTED
    assert _noalloc(wa, o=MIS) == wa.WA_ERR_UNSUPPORTED
    assert "scratch" in wa.wa_status_string(wa.WA_ERR_TOO_LARGE)


def test_decode_noalloc_scratch_covers_every_plan(wa):
    """The static scratch array holds the split-key partials of any call:
    the planner splits only below 640 (b, h) pairs, into at most
    ceil(1024 / (B*H)) chunks, so no shape reaches the WA_ERR_TOO_LARGE
    refusal (the check stays for a future planner)."""
    worst = 0
    for bh in list(range(1, 700)) + [1000, 5120, 65536]:
        for L in (1, 63, 64, 65, 255, 256, 257, 448, 1500, 4096, 65536, 1 << 20):
            worst = max(worst, wa.wa_decode_attn_workspace_size(1, bh, L))
    assert 0 < worst <= wa.WA_DECODE_NOALLOC_SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert "WA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)512 * 1024)" in hdr
    assert wa.WA_DECODE_NOALLOC_SCRATCH_BYTES == 512 * 1024


def test_decode_noalloc_without_device_reports_hip_error(wa):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: a valid call with fake pointers would launch")
    assert _noalloc(wa) == wa.WA_ERR_HIP
