"""The C-ABI library on the CPU: it loads, exports what the header declares, and
rejects bad arguments on the host before anything is enqueued.

No case here reaches a kernel launch: every call carries at least one argument
that validation rejects, so the fake (never dereferenced) device addresses are
safe even on a machine with a GPU.
"""
import ctypes
import json
import os
import re

import pytest

from mla_latent_kv_09_amd import build_lib, mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_kv.h")

OK, NULL, DIM, UNSUP, ALIGN, LAUNCH, DTYPE = 0, -1, -2, -3, -4, -5, -6
A = 0x10000          # fake 16-byte-aligned address (never dereferenced)
MIS = 0x10008        # fake misaligned address


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        build_lib.build()
    return mla.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("mla_absorb_q", "mla_decode_paged", "mla_combine", "mla_up_v"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(mla.EXPORTED) == set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (OK, NULL, DIM, UNSUP, ALIGN, LAUNCH, DTYPE, 12345):
        s = mla.status_string(code)
        assert isinstance(s, str) and s


def test_workspace_bytes(lib):
    bf16, fp32 = 0, 1
    # o_part rows in the storage type plus one float32 LSE per row.
    assert lib.mla_decode_workspace_bytes(16, 128, 1, 512, 16, bf16) == 16 * 128 * 16 * (512 * 2 + 4)
    assert lib.mla_decode_workspace_bytes(32, 128, 2, 512, 8, bf16) == 32 * 128 * 8 * (256 * 2 + 4)
    assert lib.mla_decode_workspace_bytes(16, 128, 1, 512, 16, fp32) == 16 * 128 * 16 * (512 * 4 + 4)
    assert lib.mla_decode_workspace_bytes(16, 128, 3, 512, 16, bf16) == 0  # 128 % 3 != 0
    assert lib.mla_decode_workspace_bytes(16, 128, 1, 512, 0, bf16) == 0
    assert lib.mla_decode_workspace_bytes(16, 128, 1, 512, 16, 7) == 0     # unknown dtype


# -------------------------------------------------------------- absorb / up_v

def _absorb(lib, q=A, w=A, o=A, T=16, H=128, G=1, d_hc=128, d_c=512, dt=0):
    return lib.mla_absorb_q(q, w, o, T, H, G, d_hc, d_c, dt, None)


def test_absorb_validation(lib):
    assert _absorb(lib, q=None) == NULL
    assert _absorb(lib, o=None) == NULL
    assert _absorb(lib, w=MIS) == ALIGN
    assert _absorb(lib, H=0) == DIM
    assert _absorb(lib, T=-1) == DIM
    assert _absorb(lib, H=128, G=3) == DIM
    assert _absorb(lib, d_c=511, G=2) == DIM
    assert _absorb(lib, dt=7) == DTYPE
    assert _absorb(lib, d_hc=4096, q=None) == UNSUP
    assert _absorb(lib, T=0, q=None) == OK        # nothing to do, nothing enqueued


def test_up_v_validation(lib):
    f = lambda o=A, w=A, out=A, T=16, H=128, G=1, d_hc=128, d_c=512, dt=0: lib.mla_up_v(
        o, w, out, T, H, G, d_hc, d_c, dt, None)
    assert f(out=None) == NULL
    assert f(o=MIS) == ALIGN
    assert f(d_hc=0) == DIM
    assert f(d_c=4096, o=None) == UNSUP
    assert f(dt=-1) == DTYPE
    assert f(T=0, w=None) == OK


def test_combine_validation(lib):
    f = lambda op=A, lp=A, ol=A, lo=None, T=16, H=128, G=1, d_c=512, S=16, dt=0: lib.mla_combine(
        op, lp, ol, lo, T, H, G, d_c, S, dt, None)
    assert f(op=None) == NULL
    assert f(lo=MIS, ol=A, op=A, lp=A, S=0) == DIM
    assert f(lo=MIS) == ALIGN
    assert f(S=257, op=None) == UNSUP
    assert f(dt=3) == DTYPE


def test_combine_up_v_fused_shapes(lib):
    """The fused merge + W_UV launch covers bf16, d_hc % 64 == 0, d_cg 512 with S <= 16 and
    d_cg 256 with S <= 32; everything else runs as the two calls."""
    fz = lambda H=128, G=1, d_hc=128, d_c=512, S=8, dt=0: lib.mla_combine_up_v_fused(H, G, d_hc, d_c, S, dt)
    assert fz() == 1 and fz(S=1) == 1 and fz(S=16) == 1
    assert fz(S=17) == 0 and fz(S=0) == 0
    assert fz(G=2, S=32) == 1 and fz(G=2, S=33) == 0       # d_cg 256
    assert fz(d_hc=96) == 0 and fz(d_hc=64) == 1
    assert fz(dt=1) == 0                                     # fp32
    assert fz(d_c=1024) == 0 and fz(G=4) == 0                # d_cg 1024, 128
    assert fz(H=100, G=3) == 0                               # heads not divisible by groups


def test_combine_up_v_validation(lib):
    f = lambda op=A, lp=A, w=A, ol=None, out=A, lo=None, T=16, H=128, G=1, d_hc=128, d_c=512, S=8, dt=0: \
        lib.mla_combine_up_v(op, lp, w, ol, out, lo, T, H, G, d_hc, d_c, S, dt, None)
    assert f(op=None) == NULL
    assert f(out=None) == NULL
    assert f(w=MIS) == ALIGN
    assert f(lo=MIS) == ALIGN
    assert f(ol=MIS) == ALIGN
    assert f(S=0) == DIM and f(d_hc=0) == DIM and f(T=-1) == DIM
    assert f(S=257) == UNSUP
    assert f(S=17) == UNSUP            # outside the fused kernel and no o_latent to go through
    assert f(S=17, ol=A, T=0) == OK    # ... accepted with one (nothing to do at T = 0)
    assert f(dt=3) == DTYPE
    assert f(T=0, op=None) == OK


def test_rope_table_validation(lib):
    assert lib.mla_rope_table(A, A, 0, 64, 10000.0, None) == DIM
    assert lib.mla_rope_table(A, A, 10, 63, 10000.0, None) == DIM
    assert lib.mla_rope_table(A, A, 10, 64, -1.0, None) == DIM
    assert lib.mla_rope_table(None, A, 10, 64, 10000.0, None) == NULL
    assert lib.mla_rope_table(A, MIS, 10, 64, 10000.0, None) == ALIGN


# -------------------------------------------------------------- decode

def _decode(lib, **kw):
    a = dict(q=A, qr=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, op=A, lp=A,
             B=16, T=16, maxp=64, pool=1024, H=128, G=1, d_hc=128, d_c=512, d_R=64, ps=64, S=16,
             pps=0, scale=0.0, causal=1, dt=0)
    a.update(kw)
    return lib.mla_decode_paged(a["q"], a["qr"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"],
                                a["sin"], a["rmp"], a["op"], a["lp"], a["B"], a["T"], a["maxp"],
                                a["pool"], a["H"], a["G"], a["d_hc"], a["d_c"], a["d_R"], a["ps"],
                                a["S"], a["pps"], a["scale"], a["causal"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=None), NULL), (dict(pt=None), NULL), (dict(op=None), NULL), (dict(cu=None), NULL),
    (dict(cos=A), NULL),                       # rope tables come in pairs
    (dict(kv=MIS), ALIGN), (dict(lp=MIS), ALIGN), (dict(cos=A, sin=MIS, rmp=10), ALIGN),
    (dict(d_R=63, kv=None), DIM), (dict(H=100, G=3, kv=None), DIM), (dict(S=0, kv=None), DIM),
    (dict(B=0, kv=None), DIM), (dict(maxp=0, kv=None), DIM), (dict(cos=A, sin=A, rmp=0), DIM),
    (dict(pps=-1, kv=None), DIM),
    (dict(maxp=(1 << 31) // 64 + 1, kv=None), UNSUP),   # max_pages * 64 past int32
    (dict(ps=16, kv=None), UNSUP), (dict(S=257, kv=None), UNSUP), (dict(d_c=4096, kv=None), UNSUP),
    (dict(dt=2), DTYPE),
    (dict(T=0, kv=None), OK),
])
def test_decode_validation(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(mla, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        mla.load(str(tmp_path / "missing.so"))


# -------------------------------------------------------------- append

def _append(lib, **kw):
    a = dict(c=A, k=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, B=16, T=16, maxp=64,
             pool=1024, d_c=512, d_R=64, ps=64, dt=0)
    a.update(kw)
    return lib.mla_append_kv(a["c"], a["k"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"], a["sin"],
                             a["rmp"], a["B"], a["T"], a["maxp"], a["pool"], a["d_c"], a["d_R"],
                             a["ps"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(c=None), NULL), (dict(k=None), NULL), (dict(kv=None), NULL), (dict(pt=None), NULL),
    (dict(sl=None), NULL), (dict(cu=None), NULL), (dict(sin=A), NULL),
    (dict(kv=MIS), ALIGN), (dict(k=MIS), ALIGN), (dict(cos=A, sin=MIS, rmp=10), ALIGN),
    (dict(d_R=63, kv=None), DIM), (dict(d_c=0, kv=None), DIM), (dict(B=0, kv=None), DIM),
    (dict(T=-1, kv=None), DIM), (dict(maxp=0, kv=None), DIM), (dict(pool=0, kv=None), DIM),
    (dict(cos=A, sin=A, rmp=0, kv=None), DIM),
    (dict(ps=16, kv=None), UNSUP), (dict(d_c=500, kv=None), UNSUP), (dict(d_R=6, kv=None), UNSUP),
    (dict(d_R=6, dt=1, kv=None), UNSUP),
    (dict(dt=5), DTYPE),
    (dict(T=0, kv=None), OK),
])
def test_append_validation(lib, kw, code):
    assert _append(lib, **kw) == code


# -------------------------------------------------------------- bench helpers (host only)

def test_bench_traffic_records_match_kernel_workload_splits_and_source():
    import bench
    recs = json.load(open(bench.TRAFFIC_FILE))["records"]
    assert recs, "the committed traffic file holds at least one record"
    for rec in recs:
        got = bench.measured_traffic(rec["kernel"], rec["workload"], rec["num_splits"])
        # a record is reported only while its kernel source is unchanged
        src = os.path.join(bench.CSRC, bench.KERNEL_SRC[rec["kernel"]])
        if bench.source_hash(src) == rec["kernel_source_sha256_16"]:
            assert got == rec["bytes_per_launch"]
        assert bench.measured_traffic(rec["kernel"], rec["workload"], rec["num_splits"] + 1) is None
        assert bench.measured_traffic(rec["kernel"], "no_such_workload", rec["num_splits"]) is None


def test_bench_decode_kernel_name_follows_the_library_rule(monkeypatch):
    import bench
    from mla_latent_kv_09_amd import workloads as wl
    monkeypatch.delenv("MLA_KV_DECODE_KERNEL", raising=False)
    c = wl.CONFIGS
    assert bench.decode_kernel_name(c["dsv3_b16_l4096"], 16, 8) == "decode_mfma_kernel"
    assert bench.decode_kernel_name(c["long_b16_l65536"], 16, 16) == "decode_m32_kernel"
    assert bench.decode_kernel_name(c["ragged_b64"], 96, 17) == "decode_m32_kernel"
    assert bench.decode_kernel_name(c["gla2_b32_l16384"], 32, 8) == "decode_mfma_kernel"
    assert bench.decode_kernel_name(c["tiny_fp32"], 1, 1) == "decode_generic_kernel"
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", "mfma128")
    assert bench.decode_kernel_name(c["long_b16_l65536"], 16, 16) == "decode_mfma_kernel"
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", "mfma32")
    assert bench.decode_kernel_name(c["dsv3_b16_l4096"], 16, 16) == "decode_m32_kernel"


# -------------------------------------------------------------- split planner (host only)

def _plan(lib, lens, qs, groups=1, cus=256):
    B = len(lens)
    L = (ctypes.c_int32 * max(B, 1))(*lens)
    Q = (ctypes.c_int32 * max(B, 1))(*qs)
    S, P = ctypes.c_int(-7), ctypes.c_int(-7)
    st = lib.mla_decode_plan(L, Q, B, groups, cus, ctypes.byref(S), ctypes.byref(P))
    return st, S.value, P.value


def test_plan_validation(lib):
    S = ctypes.c_int(0)
    L = (ctypes.c_int32 * 2)(100, 200)
    assert lib.mla_decode_plan(None, L, 2, 1, 256, ctypes.byref(S), ctypes.byref(S)) == NULL
    assert lib.mla_decode_plan(L, L, 2, 1, 256, None, ctypes.byref(S)) == NULL
    assert _plan(lib, [100, 200], [1, 1], cus=0)[0] == DIM
    assert _plan(lib, [100, 200], [1, 1], groups=0)[0] == DIM
    assert _plan(lib, [], [])[0] == DIM
    assert _plan(lib, [100, -1], [1, 1])[0] == DIM
    assert _plan(lib, [100, 200], [1, -1])[0] == DIM
    assert _plan(lib, [100, 200], [1, 1], cus=5000)[0] == UNSUP
    st, S, P = _plan(lib, [0], [1])
    assert st == OK and (S, P) == (1, 1)               # an empty sequence still has one page


# -------------------------------------------------------------- binding checks (host only)

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_rejects_wrong_output_buffers():
    """Caller-supplied outputs are checked for shape and dtype before anything reaches the
    library (CPU tensors: every case here fails on its shape or dtype first)."""
    import torch
    q_c, w = _t(4, 8, 16), _t(8, 16, 32)
    with pytest.raises(ValueError, match="q_abs must have shape"):
        mla.absorb_q(q_c, w, _t(4, 8, 16))
    with pytest.raises(TypeError, match="q_abs must be"):
        mla.absorb_q(q_c, w, _t(4, 8, 32, dtype=torch.float32))
    o_lat = _t(4, 8, 32)
    with pytest.raises(ValueError, match="out must have shape"):
        mla.up_v(o_lat, w, _t(4, 8, 32))
    with pytest.raises(TypeError, match="out must be"):
        mla.up_v(o_lat, w, _t(4, 8, 16, dtype=torch.float32))
    o_part, lse_part = _t(4, 8, 3, 32), _t(4, 8, 3, dtype=torch.float32)
    with pytest.raises(ValueError, match="o_latent must have shape"):
        mla.combine(o_part, lse_part, _t(4, 8, 16))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        mla.combine(o_part, lse_part, _t(4, 8, 32), lse_out=_t(4, 9, dtype=torch.float32))
    with pytest.raises(TypeError, match="lse_out must be"):
        mla.combine(o_part, lse_part, _t(4, 8, 32), lse_out=_t(4, 8))
    with pytest.raises(ValueError, match="lse_part must have shape"):
        mla.combine(o_part, _t(4, 8, 2, dtype=torch.float32), _t(4, 8, 32))


def test_binding_rejects_wrong_rope_tables():
    import torch
    T, H, d_cg, d_R = 2, 8, 32, 16
    args = (_t(T, H, d_cg), _t(T, H, d_R), _t(3, 64, d_cg + d_R),
            torch.zeros((1, 3), dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
            torch.zeros(2, dtype=torch.int32), _t(T, H, 2, d_cg), _t(T, H, 2, dtype=torch.float32))
    good = torch.zeros((100, d_R // 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="rope tables must be"):
        mla.decode_paged(*args, d_hc=16, rope=(torch.zeros((100, d_R)), good))
    with pytest.raises(TypeError, match="rope sin table must be"):
        mla.decode_paged(*args, d_hc=16, rope=(good, good.double()))
    with pytest.raises(TypeError, match="rope cos table must be"):
        mla.decode_paged(*args, d_hc=16, rope=(good.double(), good))
    with pytest.raises(ValueError, match="rope must be a"):
        mla.decode_paged(*args, d_hc=16, rope=(good, None))
    new_c, new_k = _t(T, d_cg), _t(T, d_R)
    with pytest.raises(ValueError, match="rope tables must be"):
        mla.append_kv(new_c, new_k, args[2], args[3], args[4], args[5],
                      rope=(torch.zeros((100, 3)), torch.zeros((100, 3))))


# -------------------------------------------------------------- no-allocation entry point

def _noalloc(lib, **kw):
    a = dict(q=A, qr=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, ol=A, lo=None,
             B=16, T=16, maxp=64, pool=1024, H=128, G=1, d_hc=128, d_c=512, d_R=64, ps=64, S=16,
             pps=0, scale=0.0, causal=1, dt=0)
    a.update(kw)
    return lib.mla_attend_noalloc(a["q"], a["qr"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"],
                                  a["sin"], a["rmp"], a["ol"], a["lo"], a["B"], a["T"], a["maxp"],
                                  a["pool"], a["H"], a["G"], a["d_hc"], a["d_c"], a["d_R"], a["ps"],
                                  a["S"], a["pps"], a["scale"], a["causal"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ol=None), NULL), (dict(ol=MIS), ALIGN), (dict(lo=MIS), ALIGN),
    # partials past the 64 MiB scratch: 96 tokens x 128 heads x 17 splits x 1028 B
    (dict(T=96, B=64, S=17), UNSUP),
    (dict(T=16, S=40), UNSUP),                   # 84 MB
    (dict(T=96, B=64, S=17, ol=None), NULL),     # pointers are checked before the capacity
    (dict(kv=None), NULL), (dict(d_R=63, kv=None), DIM), (dict(S=0, kv=None), DIM),
    (dict(dt=4), DTYPE), (dict(T=0, kv=None, ol=None), OK),
])
def test_noalloc_validation(lib, kw, code):
    """Every rejection happens on the host before any device call: the decode's own
    validation first, then the merge's output pointers, then the capacity."""
    assert _noalloc(lib, **kw) == code


# -------------------------------------------------------------- FP8 cache entry points

def test_fp8_page_bytes(lib):
    assert lib.mla_fp8_page_bytes(512, 64) == 64 * (512 + 128 + 4) == 41216
    assert lib.mla_fp8_page_bytes(64, 16) == 64 * (64 + 32 + 4)
    assert lib.mla_fp8_page_bytes(0, 64) == 0 and lib.mla_fp8_page_bytes(512, 63) == 0


def _decode8(lib, **kw):
    a = dict(q=A, qr=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, op=A, lp=A,
             B=16, T=16, maxp=64, pool=1024, H=128, G=1, d_hc=128, d_c=512, d_R=64, ps=64, S=16,
             pps=0, scale=0.0, causal=1)
    a.update(kw)
    return lib.mla_decode_paged_fp8(a["q"], a["qr"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"],
                                    a["sin"], a["rmp"], a["op"], a["lp"], a["B"], a["T"], a["maxp"],
                                    a["pool"], a["H"], a["G"], a["d_hc"], a["d_c"], a["d_R"],
                                    a["ps"], a["S"], a["pps"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=None), NULL), (dict(op=None), NULL), (dict(kv=MIS), ALIGN),
    (dict(d_R=63, kv=None), DIM), (dict(S=0, kv=None), DIM),
    (dict(ps=16, kv=None), UNSUP),
    # valid arguments but a shape the FP8 kernel does not implement
    (dict(H=64), UNSUP), (dict(G=2), UNSUP), (dict(d_c=256), UNSUP), (dict(d_R=32), UNSUP),
    (dict(T=0, kv=None), OK),
])
def test_fp8_decode_validation(lib, kw, code):
    assert _decode8(lib, **kw) == code


def _append8(lib, **kw):
    a = dict(c=A, k=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, B=16, T=16, maxp=64,
             pool=1024, d_c=512, d_R=64, ps=64)
    a.update(kw)
    return lib.mla_append_kv_fp8(a["c"], a["k"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"],
                                 a["sin"], a["rmp"], a["B"], a["T"], a["maxp"], a["pool"], a["d_c"],
                                 a["d_R"], a["ps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(c=None), NULL), (dict(kv=None), NULL), (dict(sin=A), NULL), (dict(kv=MIS), ALIGN),
    (dict(d_R=63, kv=None), DIM), (dict(B=0, kv=None), DIM),
    (dict(ps=16, kv=None), UNSUP), (dict(d_c=1024, kv=None), UNSUP), (dict(d_c=500, kv=None), UNSUP),
    (dict(d_R=12, kv=None), UNSUP), (dict(T=0, kv=None), OK),
])
def test_fp8_append_validation(lib, kw, code):
    assert _append8(lib, **kw) == code


def test_bench_names_the_fp8_kernel_and_counts_fp8_bytes():
    import bench
    from mla_latent_kv_09_amd import workloads as wl
    c = wl.CONFIGS["long_b16_l65536"]
    assert bench.decode_kernel_name(c, 16, 16, "fp8") == "decode_m32_kernel_fp8"
    assert bench.cache_row_bytes(c, "fp8") == 644 and bench.cache_row_bytes(c) == 1152
    att8, _, kv8, _ = bench.algorithmic_work(c, [65536] * 16, [1] * 16, "fp8")
    att, _, kv, _ = bench.algorithmic_work(c, [65536] * 16, [1] * 16)
    assert att8 == att and kv8 == 16 * 65536 * 644 and kv == 16 * 65536 * 1152


# -------------------------------------------------------------- MXFP4 cache entry points

def test_mxfp4_page_bytes(lib):
    assert lib.mla_mxfp4_page_bytes(512, 64) == 64 * (256 + 128 + 16) == 25600
    assert lib.mla_mxfp4_page_bytes(64, 16) == 64 * (32 + 32 + 2)
    assert lib.mla_mxfp4_page_bytes(0, 64) == 0 and lib.mla_mxfp4_page_bytes(512, 63) == 0
    assert lib.mla_mxfp4_page_bytes(48, 16) == 0          # d_c not a multiple of 32
    # never the size of an FP8 page of the same shape, so uint8 pools tell their format
    for d_c in range(32, 1025, 32):
        for d_R in (16, 32, 64, 128):
            assert lib.mla_mxfp4_page_bytes(d_c, d_R) != lib.mla_fp8_page_bytes(d_c, d_R)


def _decode4(lib, **kw):
    a = dict(q=A, qr=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, op=A, lp=A,
             B=16, T=16, maxp=64, pool=1024, H=128, G=1, d_hc=128, d_c=512, d_R=64, ps=64, S=16,
             pps=0, scale=0.0, causal=1)
    a.update(kw)
    return lib.mla_decode_paged_mxfp4(a["q"], a["qr"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"],
                                      a["sin"], a["rmp"], a["op"], a["lp"], a["B"], a["T"], a["maxp"],
                                      a["pool"], a["H"], a["G"], a["d_hc"], a["d_c"], a["d_R"],
                                      a["ps"], a["S"], a["pps"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=None), NULL), (dict(op=None), NULL), (dict(kv=MIS), ALIGN),
    (dict(d_R=63, kv=None), DIM), (dict(S=0, kv=None), DIM),
    (dict(ps=16, kv=None), UNSUP),
    (dict(H=64), UNSUP), (dict(G=2), UNSUP), (dict(d_c=256), UNSUP), (dict(d_R=32), UNSUP),
    (dict(T=0, kv=None), OK),
])
def test_mxfp4_decode_validation(lib, kw, code):
    assert _decode4(lib, **kw) == code


def _append4(lib, **kw):
    a = dict(c=A, k=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, B=16, T=16, maxp=64,
             pool=1024, d_c=512, d_R=64, ps=64)
    a.update(kw)
    return lib.mla_append_kv_mxfp4(a["c"], a["k"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"],
                                   a["sin"], a["rmp"], a["B"], a["T"], a["maxp"], a["pool"], a["d_c"],
                                   a["d_R"], a["ps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(c=None), NULL), (dict(kv=None), NULL), (dict(sin=A), NULL), (dict(kv=MIS), ALIGN),
    (dict(d_R=63, kv=None), DIM), (dict(B=0, kv=None), DIM),
    (dict(ps=16, kv=None), UNSUP), (dict(d_c=1024, kv=None), UNSUP), (dict(d_c=496, kv=None), UNSUP),
    (dict(d_c=8, kv=None), UNSUP), (dict(d_R=12, kv=None), UNSUP), (dict(T=0, kv=None), OK),
])
def test_mxfp4_append_validation(lib, kw, code):
    assert _append4(lib, **kw) == code


def test_bench_names_the_mxfp4_kernel_and_counts_mxfp4_bytes():
    import bench
    from mla_latent_kv_09_amd import workloads as wl
    c = wl.CONFIGS["long_b16_l65536"]
    assert bench.decode_kernel_name(c, 16, 16, "mxfp4") == "decode_m32_kernel_mxfp4"
    assert bench.cache_row_bytes(c, "mxfp4") == 256 + 128 + 16 == 400
    att4, _, kv4, _ = bench.algorithmic_work(c, [65536] * 16, [1] * 16, "mxfp4")
    att, _, _, _ = bench.algorithmic_work(c, [65536] * 16, [1] * 16)
    assert att4 == att and kv4 == 16 * 65536 * 400


# -------------------------------------------------------------- prefill dispatch (host only)

def test_branch_threshold(lib):
    assert mla.branch([1, 2, 1]) == mla.BRANCH_ABSORBED
    assert mla.branch([1, 255]) == mla.BRANCH_ABSORBED
    assert mla.branch([1, 256]) == mla.BRANCH_DECOMPRESSED
    assert mla.branch([4096] * 8) == mla.BRANCH_DECOMPRESSED
    assert mla.branch([300], threshold=512) == mla.BRANCH_ABSORBED
    L = (ctypes.c_int32 * 2)(1, 2)
    assert lib.mla_branch(None, 2, 256) == NULL
    assert lib.mla_branch(L, 0, 256) == DIM and lib.mla_branch(L, 2, 0) == DIM
    assert lib.mla_branch((ctypes.c_int32 * 1)(-1), 1, 256) == DIM


def test_prefill_workspace_bytes(lib):
    assert lib.mla_prefill_workspace_bytes(512, 128, 128, 0) == 2 * 512 * 64 * 128 * 128 * 2
    assert lib.mla_prefill_workspace_bytes(0, 128, 128, 0) == 0
    assert lib.mla_prefill_workspace_bytes(10, 128, 128, 1) == 0     # bf16 only


def _prefill(lib, **kw):
    a = dict(qc=A, qr=A, kv=A, pt=A, sl=A, cu=A, cos=None, sin=None, rmp=0, wk=A, wv=A, ws=A,
             out=A, lse=None, B=8, T=32768, maxp=64, pool=512, maxq=4096, H=128, G=1, d_hc=128,
             d_c=512, d_R=64, ps=64, scale=0.0, causal=1, dt=0)
    a.update(kw)
    return lib.mla_prefill_paged(a["qc"], a["qr"], a["kv"], a["pt"], a["sl"], a["cu"], a["cos"],
                                 a["sin"], a["rmp"], a["wk"], a["wv"], a["ws"], a["out"], a["lse"],
                                 a["B"], a["T"], a["maxp"], a["pool"], a["maxq"], a["H"], a["G"],
                                 a["d_hc"], a["d_c"], a["d_R"], a["ps"], a["scale"], a["causal"],
                                 a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ws=None), NULL), (dict(wk=None), NULL), (dict(out=None), NULL), (dict(cos=A), NULL),
    (dict(ws=MIS), ALIGN), (dict(lse=MIS), ALIGN),
    (dict(maxq=0, ws=None), DIM), (dict(d_R=63, ws=None), DIM), (dict(B=0, ws=None), DIM),
    (dict(H=128, G=3, ws=None), DIM),
    (dict(G=2, ws=None), UNSUP), (dict(d_hc=64, ws=None), UNSUP), (dict(ps=16, ws=None), UNSUP),
    (dict(dt=1, ws=None), UNSUP), (dict(dt=9), DTYPE),
    (dict(T=0, ws=None), OK),
])
def test_prefill_validation(lib, kw, code):
    assert _prefill(lib, **kw) == code
