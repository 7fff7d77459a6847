"""The C ABI without a GPU: the library loads, exports every function that
include/specverify.h declares, sizes workspaces, and rejects bad arguments on
the host before anything is launched.  No call here reaches the HIP runtime."""
import ctypes
import os
import re

import pytest
import torch

import draft_token_verification_spec_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sv.lib_path()), reason="libspecverify.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\s*\*)\s*(sv_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == {"sv_workspace_size", "sv_spec_verify", "sv_av_score", "sv_av_fit_step",
                          "sv_status_string", "sv_av_budget", "sv_av_calib_accumulate", "sv_av_calib_metrics",
                          "sv_tts_grad", "sv_filtered_workspace_size", "sv_spec_verify_filtered",
                          "sv_workspace_status", "sv_spec_verify_static"}
    lib = ctypes.CDLL(sv.lib_path())
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(sv.__all__)


def declared_prototypes():
    """name -> (return type, [parameter types]) from the header's prototypes
    (comments removed, each prototype up to its semicolon)."""
    text = re.sub(r"/\*.*?\*/", " ", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*(size_t|int|const char\s*\*)\s*(sv_\w+)\s*\(([^;]*)\)\s*;", text, re.M):
        params = [" ".join(q.split()) for q in m.group(3).split(",")]
        out[m.group(2)] = (" ".join(m.group(1).split()), params)
    return out


def ctype_of(decl: str):
    """The ctypes type a C parameter or return declaration passes as."""
    d = decl.replace("const ", "")
    if "*" in d:
        return ctypes.c_char_p if d.startswith("char") else ctypes.c_void_p
    base = d.split()[0]
    return {"int": ctypes.c_int, "size_t": ctypes.c_size_t, "int64_t": ctypes.c_int64,
            "float": ctypes.c_float}[base]


def test_binding_signatures_match_header_prototypes():
    # every entry point the binding calls passes exactly the header's
    # parameters, in the header's types (a mismatch would corrupt arguments
    # silently through ctypes)
    protos = declared_prototypes()
    assert set(protos) == set(declared_functions())
    for name, (res, args) in sv._SIGNATURES.items():
        ret, params = protos[name]
        assert res == ctype_of(ret), name
        assert len(args) == len(params), (name, len(args), len(params))
        for i, (a, p) in enumerate(zip(args, params)):
            assert a == ctype_of(p), (name, i, p)
    assert set(sv._SIGNATURES) == set(protos)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define SV_MAX_K (\d+)", text).group(1)) == sv.SV_MAX_K
    assert re.search(r"#define SV_MAX_V \(1 << (\d+)\)", text).group(1) == str(sv.SV_MAX_V.bit_length() - 1)
    assert re.search(r"#define SV_MAX_B \(1 << (\d+)\)", text).group(1) == str(sv.SV_MAX_B.bit_length() - 1)
    assert int(re.search(r"#define SV_BUDGET_MAX_ITEMS (\d+)", text).group(1)) == sv.SV_BUDGET_MAX_ITEMS
    assert int(re.search(r"#define SV_CALIB_AUC_BINS (\d+)", text).group(1)) == sv.SV_CALIB_AUC_BINS
    assert re.search(r"#define SV_CALIB_WORDS \(33 \+ 2 \* SV_CALIB_AUC_BINS\)", text)


def test_no_process_wide_settings_or_measurement_aids_exported():
    lib = ctypes.CDLL(sv.lib_path())
    for name in ("sv_set_verify_kernel", "sv_timing_enable", "sv_timing_read", "sv_read_probe"):
        assert not hasattr(lib, name), name


def test_workspace_status_rejections():
    lib = sv._load()
    assert lib.sv_workspace_status(None, FAKE, 16, FAKE, 1) == -3
    assert lib.sv_workspace_status(None, FAKE, 1 << 20, None, 1) == -1
    assert lib.sv_workspace_status(None, None, 0, None, 1) == -1


def test_static_scratch_constant_and_rejections():
    """sv_spec_verify_static: the scratch limit matches the binding, and bad
    arguments or shapes beyond the static scratch are refused on the host
    before the scratch is touched."""
    text = open(HEADER).read()
    assert re.search(r"#define SV_STATIC_SCRATCH_BYTES \(8u << 20\)", text)
    assert sv.SV_STATIC_SCRATCH_BYTES == 8 << 20
    lib = sv._load()
    V, K = 1024, 4
    ok = dict(stream=None, B=4, V=V, K=K, dt=0, draft=FAKE, dstart=FAKE, dstride=V, target=FAKE, tstart=FAKE,
              tstride=V, nd=FAKE, toks=FAKE, temp=FAKE, ua=FAKE, ur=FAKE, ub=FAKE, al=FAKE, ot=FAKE, lab=None,
              pd=None, pt=None, par=None, feat=None, score=None)
    call = lambda **kw: lib.sv_spec_verify_static(*{**ok, **kw}.values())
    assert call(B=-1) == -1 and call(V=0) == -1 and call(dt=5) == -1
    assert call(K=sv.SV_MAX_K + 1) == -2
    for k in ("target", "tstart", "nd", "temp", "ur", "ub", "al", "ot", "draft", "dstart", "toks", "ua"):
        assert call(**{k: None}) == -1, k
    assert call(tstride=V - 1) == -1
    assert call(score=FAKE) == -1  # a score needs the feature and the parameters
    assert call(B=0) == 0
    # the B = 256, K = 4, V = 128256 bf16 workspace fits the static scratch; a
    # batch of 2^16 requests of 16 drafts over 2^21 fp32 logits does not
    assert sv.sv_workspace_size(256, 128256, 4, 1) <= sv.SV_STATIC_SCRATCH_BYTES
    assert call(B=1 << 14, V=1 << 21, K=16, dt=0, dstride=1 << 21, tstride=1 << 21) == -2


def test_status_strings():
    assert sv.sv_status_string(0) == "ok"
    assert "argument" in sv.sv_status_string(-1)
    assert "unsupported" in sv.sv_status_string(-2)
    assert "workspace" in sv.sv_status_string(-3)
    assert "HIP" in sv.sv_status_string(-4)
    assert sv.sv_status_string(12345) == "unknown status"


def test_workspace_size():
    small = sv.sv_workspace_size(4, 1024, 4, sv.SV_F32)
    assert small > 0 and small % 256 == 0
    big = sv.sv_workspace_size(256, 128256, 4, sv.SV_BF16)
    assert big > small
    assert sv.sv_workspace_size(-1, 1024, 4, 0) == 0
    assert sv.sv_workspace_size(4, 0, 4, 0) == 0
    assert sv.sv_workspace_size(4, 1024, sv.SV_MAX_K + 1, 0) == 0
    assert sv.sv_workspace_size(4, sv.SV_MAX_V + 1, 4, 0) == 0
    assert sv.sv_workspace_size(4, 1024, 4, 9) == 0
    assert sv.sv_workspace_size(sv.SV_MAX_B + 1, 8, 1, 0) == 0
    assert sv.sv_workspace_size(sv.SV_MAX_B, 8, 1, 0) > 0


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails host checks first


def verify_call(**kw):
    args = dict(stream=None, B=4, V=1024, max_k=4, dtype=0, draft=FAKE, dstart=FAKE, dstride=1024, target=FAKE,
                tstart=FAKE, tstride=1024, num_draft=FAKE, tokens=FAKE, temp=FAKE, u_acc=FAKE, u_res=FAKE,
                u_bon=FAKE, accept_len=FAKE, out_tokens=FAKE, labels=None, p_d=None, p_t=None, params=None,
                feat=None, score=None, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    lib = sv._load()
    return lib.sv_spec_verify(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -1),
    (dict(V=0), -1),
    (dict(max_k=-1), -1),
    (dict(max_k=17), -2),
    (dict(V=sv.SV_MAX_V + 1, dstride=sv.SV_MAX_V + 1, tstride=sv.SV_MAX_V + 1), -2),
    (dict(dtype=5), -1),
    (dict(B=(1 << 18) + 1), -2),
    (dict(target=None), -1),
    (dict(tstart=None), -1),
    (dict(num_draft=None), -1),
    (dict(temp=None), -1),
    (dict(u_res=None), -1),
    (dict(u_bon=None), -1),
    (dict(accept_len=None), -1),
    (dict(out_tokens=None), -1),
    (dict(draft=None), -1),
    (dict(tokens=None), -1),
    (dict(u_acc=None), -1),
    (dict(tstride=1023), -1),
    (dict(dstride=100), -1),
    (dict(score=FAKE), -1),  # score needs feature and params
    (dict(score=FAKE, feat=FAKE), -1),
    (dict(ws=None), -3),
    (dict(ws_bytes=100), -3),
])
def test_spec_verify_rejects_before_launch(kw, status):
    assert verify_call(**kw) == status


def test_spec_verify_empty_batch_is_a_noop():
    assert verify_call(B=0, ws=None, ws_bytes=0, target=None) in (-1, 0)
    assert verify_call(B=0) == 0


def filtered_call(**kw):
    args = dict(stream=None, B=4, V=1024, max_k=4, dtype=0, draft=FAKE, dstart=FAKE, dstride=1024, target=FAKE,
                tstart=FAKE, tstride=1024, num_draft=FAKE, tokens=FAKE, temp=FAKE, top_k=FAKE, top_p=FAKE,
                u_acc=FAKE, u_res=FAKE, u_bon=FAKE, accept_len=FAKE, out_tokens=FAKE, labels=None, p_d=None,
                p_t=None, kept=None, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return sv._load().sv_spec_verify_filtered(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -1),
    (dict(max_k=17), -2),
    (dict(dtype=5), -1),
    (dict(top_k=None), -1),
    (dict(top_p=None), -1),
    (dict(target=None), -1),
    (dict(draft=None), -1),
    (dict(u_acc=None), -1),
    (dict(tstride=1023), -1),
    (dict(ws=None), -3),
    (dict(ws_bytes=100), -3),
])
def test_spec_verify_filtered_rejects_before_launch(kw, status):
    assert filtered_call(**kw) == status


def test_filtered_workspace_size():
    plain = sv.sv_workspace_size(256, 128256, 4, sv.SV_BF16)
    filt = sv.sv_filtered_workspace_size(256, 128256, 4, sv.SV_BF16)
    # the verification workspace, then 2 x 256 x 12 B of histograms per row
    # segment and 48 B of search state per row and search
    nseg = -(-128256 * 2 // 32768)
    assert filt >= plain + 256 * 9 * nseg * 2 * 256 * 12 + 256 * 9 * 2 * 48
    assert filt % 256 == 0
    assert sv.sv_filtered_workspace_size(4, 1024, sv.SV_MAX_K + 1, 0) == 0
    # one workspace one byte short is refused
    assert filtered_call(ws_bytes=sv.sv_filtered_workspace_size(4, 1024, 4, 0) - 1) == -3


def test_av_score_rejects_before_launch():
    lib = sv._load()
    base = [None, 4, 1024, 4, 0, FAKE, FAKE, 1024, FAKE, FAKE, FAKE, ctypes.c_float(0.3), FAKE, FAKE, FAKE, FAKE,
            1 << 30]
    def call(i, v):
        a = list(base)
        a[i] = v
        return lib.sv_av_score(*a)
    assert call(1, -1) == -1
    assert call(3, 17) == -2
    assert call(5, None) == -1   # draft logits
    assert call(7, 10) == -1     # stride < V
    assert call(10, None) == -1  # params
    assert call(12, None) == -1  # feature
    assert call(15, None) == -3  # workspace
    assert call(16, 8) == -3
    assert call(1, 0) == 0       # empty batch


def test_av_fit_rejects_before_launch():
    lib = sv._load()
    f = ctypes.c_float
    assert lib.sv_av_fit_step(None, -1, 4, FAKE, FAKE, FAKE, FAKE, f(10), f(1e-6), f(1.0), 0) == -1
    assert lib.sv_av_fit_step(None, 4, 17, FAKE, FAKE, FAKE, FAKE, f(10), f(1e-6), f(1.0), 0) == -2
    assert lib.sv_av_fit_step(None, 4, 4, None, FAKE, FAKE, FAKE, f(10), f(1e-6), f(1.0), 0) == -1
    assert lib.sv_av_fit_step(None, 4, 4, FAKE, FAKE, None, FAKE, f(10), f(1e-6), f(1.0), 0) == -1
    assert lib.sv_av_fit_step(None, 4, 4, FAKE, FAKE, FAKE, None, f(10), f(1e-6), f(1.0), 0) == -1
    assert lib.sv_av_fit_step(None, 4, 4, FAKE, FAKE, FAKE, FAKE, f(-1), f(1e-6), f(1.0), 0) == -1
    assert lib.sv_av_fit_step(None, 4, 4, FAKE, FAKE, FAKE, FAKE, f(10), f(float("nan")), f(1.0), 0) == -1
    for bad in (0.0, -1.0, float("nan")):
        assert lib.sv_av_fit_step(None, 4, 4, FAKE, FAKE, FAKE, FAKE, f(10), f(1e-6), f(bad), 0) == -1
    assert lib.sv_av_fit_step(None, 4, 0, None, None, None, None, f(10), f(1e-6), f(1.0), 0) == 0


def test_binding_refuses_host_tensors():
    """No CPU fallback: host tensors are rejected before any library call."""
    x = torch.zeros(2, 16)
    z = torch.zeros(1, dtype=torch.int64)
    with pytest.raises(ValueError):
        sv.sv_spec_verify(x, z, x, z, torch.zeros(1, dtype=torch.int32), torch.zeros(1, 1, dtype=torch.int32),
                          torch.ones(1), torch.zeros(1, 1), torch.zeros(1), torch.zeros(1), max_k=1)
    with pytest.raises(ValueError):
        sv.sv_av_score(x, z, torch.zeros(1, dtype=torch.int32), torch.ones(1), torch.zeros(2), max_k=1)


@pytest.mark.parametrize("B,max_k,nulls,status", [
    (-1, 4, (), -1), (4, -1, (), -1), (4, 17, (), -2), (1025, 4, (), -2), (257, 16, (), -2), (4097, 1, (), -2),
    (4, 4, ("num_draft",), -1), (4, 4, ("draft_cost",), -1), (4, 4, ("verify_cost",), -1),
    (4, 4, ("num_kept",), -1), (4, 4, ("budget",), -1), (4, 4, ("score",), -1),
    (0, 4, ("score", "num_draft", "draft_cost", "verify_cost", "num_kept", "budget"), 0),
])
def test_budget_rejects_before_launch(B, max_k, nulls, status):
    # every case is refused (or is empty) before anything reaches a device
    lib = ctypes.CDLL(sv.lib_path())
    fake = ctypes.c_void_p(16)
    args = {k: (None if k in nulls else fake)
            for k in ("score", "num_draft", "draft_cost", "verify_cost", "num_kept", "budget")}
    lib.sv_av_budget.restype = ctypes.c_int
    lib.sv_av_budget.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 6
    assert lib.sv_av_budget(None, B, max_k, args["score"], args["num_draft"], args["draft_cost"],
                            args["verify_cost"], args["num_kept"], args["budget"]) == status


def test_calib_rejects_before_launch():
    lib = ctypes.CDLL(sv.lib_path())
    fake = ctypes.c_void_p(16)
    lib.sv_av_calib_accumulate.restype = ctypes.c_int
    lib.sv_av_calib_accumulate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 3
    lib.sv_av_calib_metrics.restype = ctypes.c_int
    lib.sv_av_calib_metrics.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int]
    acc = lib.sv_av_calib_accumulate
    assert acc(None, -1, 4, fake, fake, fake) == -1
    assert acc(None, 4, 17, fake, fake, fake) == -2
    assert acc(None, 4, 4, fake, fake, None) == -1
    assert acc(None, 4, 4, None, fake, fake) == -1
    assert acc(None, 4, 4, fake, None, fake) == -1
    assert acc(None, 0, 4, None, None, fake) == 0  # nothing to add
    assert lib.sv_av_calib_metrics(None, None, fake, 0) == -1
    assert lib.sv_av_calib_metrics(None, fake, None, 1) == -1


def test_tts_grad_rejects_before_launch():
    lib = ctypes.CDLL(sv.lib_path())
    f = ctypes.c_void_p(16)
    fn = lib.sv_tts_grad
    fn.restype = ctypes.c_int
    fn.argtypes = ([ctypes.c_void_p] + [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64] * 3 +
                   [ctypes.c_void_p] * 3 + [ctypes.c_float] + [ctypes.c_void_p] * 3 + [ctypes.c_size_t])

    def call(B=4, V=64, K=4, dt=1, lam=0.0, stride=64, pstride=64, prev=None, pstart=None, ws=None, wsb=0,
             **nulls):
        a = dict(draft=f, dstart=f, target=f, tstart=f, nd=f, temp=f, w=f, grad=f, loss=f)
        a.update(nulls)
        return fn(None, B, V, K, dt, a["draft"], a["dstart"], stride, a["target"], a["tstart"], stride,
                  prev, pstart, pstride, a["nd"], a["temp"], a["w"], lam, a["grad"], a["loss"], ws, wsb)

    assert call(B=-1) == -1 and call(V=0) == -1 and call(dt=7) == -1 and call(lam=-1.0) == -1
    assert call(K=17) == -2 and call(V=(1 << 21) + 1, stride=(1 << 21) + 1) == -2
    for k in ("draft", "dstart", "target", "tstart", "nd", "temp", "w", "grad", "loss"):
        assert call(**{k: None}) == -1, k
    assert call(stride=63) == -1
    assert call(prev=f, pstart=None) == -1 and call(prev=f, pstart=f, pstride=10) == -1
    assert call(B=0) == 0 and call(K=0) == 0
    assert call(ws=f, wsb=sv.sv_workspace_size(4, 64, 4, 1) - 1) == -3  # too small a verification workspace


def test_read_probe_sizes_and_rejections():
    from draft_token_verification_spec_amd import measure

    assert measure.read_probe_sink_words(0) == 0
    assert measure.read_probe_sink_words(16) == 4  # one workgroup, four waves
    assert measure.read_probe_sink_words(32768) == 4
    assert measure.read_probe_sink_words(32768 + 16) == 8
    lib = measure._load()
    ok = dict(stream=None, data=FAKE, nbytes=1 << 20, sink=FAKE, words=1 << 20)
    call = lambda **kw: lib.svb_read_probe(*{**ok, **kw}.values())
    assert call(nbytes=0) == 0
    assert call(data=None) == -1
    assert call(sink=None) == -1
    assert call(nbytes=(1 << 20) + 8) == -1  # not a multiple of 16
    assert call(data=ctypes.c_void_p(0x10008)) == -1  # not 16-byte aligned
    assert call(words=measure.read_probe_sink_words(1 << 20) - 1) == -1
