"""C-ABI boundary checks that need no GPU: the library loads, exports every
symbol the header declares, and rejects every invalid argument before any
launch."""
import ctypes
import os
import re

import pytest

import w4a16_int4_grouped_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from w4a16_int4_grouped_moe_amd import build

        build.build()
    return moe.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_w4a16_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted([
        "moe_w4a16_align", "moe_w4a16_align_capacity", "moe_w4a16_align_scratch_size",
        "moe_w4a16_forward",
        "moe_w4a16_forward_block_m", "moe_w4a16_forward_scores", "moe_w4a16_forward_timed",
        "moe_w4a16_forward_split_max_pairs",
        "moe_w4a16_forward_noalloc", "moe_w4a16_noalloc_workspace_limit",
        "moe_w4a16_forward_prepacked", "moe_w4a16_forward_prepacked_timed",
        "moe_w4a16_prepack", "moe_w4a16_prepack_size",
        "moe_w4a16_route", "moe_w4a16_status_string", "moe_w4a16_workspace_size"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_probe_library_exports_its_entry_points():
    """The bench's streaming-read kernel lives in its own library (measurement
    only): it loads and exports its two calls; the pass size is whole grid
    steps of 512 MiB."""
    import os

    raw = ctypes.CDLL(os.path.join(os.path.dirname(moe.LIB_PATH), "libmoe_probe.so"))
    assert hasattr(raw, "moe_probe_stream_read")
    raw.moe_probe_stream_read_bytes.argtypes = [ctypes.c_int64]
    raw.moe_probe_stream_read_bytes.restype = ctypes.c_int64
    assert raw.moe_probe_stream_read_bytes(4 << 30) == 4 << 30
    assert raw.moe_probe_stream_read_bytes((1 << 29) - 1) == 0
    raw.moe_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]
    assert raw.moe_probe_stream_read(None, 1 << 30, None, None) != 0  # refused before any launch


def test_status_codes_match_header(lib):
    text = open(HEADER).read()
    for name in ["MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_ALIGNMENT",
                 "MOE_ERR_WORKSPACE", "MOE_ERR_UNSUPPORTED", "MOE_ERR_HIP"]:
        m = re.search(r"#define %s \(?(-?\d+)\)?" % name, text)
        assert m and int(m.group(1)) == getattr(moe, name), name
        assert moe.status_string(getattr(moe, name)).startswith(name)
    from w4a16_int4_grouped_moe_amd import _binding

    for name in ["MOE_MAX_EXPERTS", "MOE_MAX_SCORED"]:
        m = re.search(r"#define %s (\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(_binding, name), name


def P(**kw):
    base = dict(num_tokens=64, hidden=7168, inter=2048, num_experts=384, top_k=8,
                expert_base=0, group_size=32)
    base.update(kw)
    return moe.problem(**base)


def test_workspace_size_and_block_m(lib):
    p = P()
    assert moe.forward_block_m(p) == 4
    assert moe.forward_block_m(P(num_tokens=192)) == 4     # T k = 4 E
    assert moe.forward_block_m(P(num_tokens=193)) == 96
    assert moe.forward_block_m(P(num_tokens=512)) == 96
    assert moe.forward_block_m(P(num_tokens=4096)) == 96
    # the split bucketing: 96-row calls of fewer than 8192 pairs put experts
    # with at most 4 pairs in 4-row buckets
    assert moe.forward_split_max_pairs(P()) == 0                    # block_m 4
    assert moe.forward_split_max_pairs(P(num_tokens=193)) == 4
    assert moe.forward_split_max_pairs(P(num_tokens=1023)) == 4     # 8184 pairs
    assert moe.forward_split_max_pairs(P(num_tokens=1024)) == 0     # 8192 pairs
    assert moe.forward_split_max_pairs(P(num_tokens=4096)) == 0
    # widths that are not whole block tiles (7040 % 512 != 0, 1152 % 256 != 0)
    # take the same 96-row blocks, masked
    assert moe.forward_block_m(P(num_tokens=512, hidden=7040)) == 96
    assert moe.forward_block_m(P(num_tokens=4096, hidden=7040, inter=1152)) == 96
    # the 4-row kernel stages a work-group's group scales for the whole K in
    # its 64 KB of LDS (64 rows x 32 (odd number of 16-group units) bytes, plus
    # two 4 KB activation stages): hidden 12288 fits (58 KB), 14336 does not
    # (66 KB), and even one token then takes the 96-row blocks
    assert moe.forward_block_m(P(num_tokens=1, hidden=12288)) == 4
    assert moe.forward_block_m(P(num_tokens=1, hidden=14336)) == 96
    # one GPU's share of an 8-way tensor-parallel split (intermediate 256)
    assert moe.forward_block_m(P(inter=256)) == 4
    assert moe.forward_block_m(P(inter=256, num_tokens=4096)) == 96
    n = moe.workspace_size(p)
    T, H, I, k = 64, 7168, 2048, 8
    cap = T * k + min(384, T * k) * 3
    # at least: bucket arrays, h rows, per-pair y, shared h and s
    assert n >= 4 * cap + 2 * cap * I + 4 * T * k * H + 2 * T * I + 4 * T * H
    assert n < 1.2 * (4 * cap + 2 * cap * I + 4 * T * k * H + 2 * T * I + 4 * T * H) + 4096
    assert moe.workspace_size(P(num_tokens=0)) == 0
    assert moe.align_capacity(p, 4) == (cap, cap // 4)
    assert moe.align_capacity(P(num_tokens=1), 16) == (8 + 8 * 15, (8 + 8 * 15) // 16)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=7100), moe.MOE_ERR_SHAPE),
    (dict(hidden=96), moe.MOE_ERR_SHAPE),
    (dict(inter=2000), moe.MOE_ERR_SHAPE),
    (dict(top_k=0), moe.MOE_ERR_SHAPE),
    (dict(top_k=17), moe.MOE_ERR_SHAPE),
    (dict(num_experts=0), moe.MOE_ERR_SHAPE),
    (dict(num_experts=513), moe.MOE_ERR_UNSUPPORTED),
    (dict(group_size=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(group_size=128), moe.MOE_ERR_UNSUPPORTED),
    (dict(num_tokens=-1), moe.MOE_ERR_SHAPE),
    (dict(expert_base=-1), moe.MOE_ERR_SHAPE),
    (dict(num_tokens=1 << 28), moe.MOE_ERR_SHAPE),
])
def test_invalid_problem_rejected(lib, kw, status):
    p = P(**kw)
    n = ctypes.c_size_t(0)
    assert lib.moe_w4a16_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 9
    assert lib.moe_w4a16_forward(*args, ctypes.byref(p), fake, 1 << 40, None) == status


@pytest.mark.parametrize("T,status", [
    (60000, moe.MOE_OK),                 # bucketed h rows: 516,480 x 2048 x 2 B < 2 GiB
    (70000, moe.MOE_ERR_UNSUPPORTED),    # h rows past 2 GiB
    (150000, moe.MOE_ERR_UNSUPPORTED),   # x past 2 GiB as well
])
def test_arrays_past_2gib_rejected(lib, T, status):
    """The kernels address every array through 32-bit buffer resources whose
    out-of-range offset (2^31) must lie past the array: a problem that would
    need a larger array is refused before any launch."""
    p = P(num_tokens=T)
    n = ctypes.c_size_t(0)
    assert lib.moe_w4a16_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    if status != moe.MOE_OK:
        fake = ctypes.c_void_p(0x10000)
        assert lib.moe_w4a16_forward(*([fake] * 9), ctypes.byref(p), fake, 1 << 45,
                                     None) == status
    # a shared-expert or expert matrix past 2 GiB (2I x H bf16)
    p = P(num_tokens=1, hidden=16384, inter=32768)
    assert lib.moe_w4a16_workspace_size(ctypes.byref(p), ctypes.byref(n)) == \
        moe.MOE_ERR_UNSUPPORTED


def _fwd(lib, p, ptrs, ws_bytes=1 << 40):
    return lib.moe_w4a16_forward(*ptrs, ctypes.byref(p), ctypes.c_void_p(0x20000), ws_bytes,
                                 None)


def test_forward_argument_errors_before_launch(lib):
    p = P()
    good = [ctypes.c_void_p(0x10000 + 0x100 * i) for i in range(9)]
    assert lib.moe_w4a16_forward(*good, None, ctypes.c_void_p(0x20000), 1 << 40, None) == \
        moe.MOE_ERR_NULL
    for i in range(9):
        ptrs = list(good)
        ptrs[i] = None
        want = moe.MOE_OK if i == 7 else moe.MOE_ERR_NULL  # shared_w is optional
        if want == moe.MOE_OK:
            continue  # a valid call would launch; not on the CPU
        assert _fwd(lib, p, ptrs) == want, i
        ptrs[i] = ctypes.c_void_p(0x10008)  # 8-byte aligned only
        assert _fwd(lib, p, ptrs) == moe.MOE_ERR_ALIGNMENT, i
    assert lib.moe_w4a16_forward(*good, ctypes.byref(p), None, 1 << 40, None) == moe.MOE_ERR_NULL
    need = moe.workspace_size(p)
    assert _fwd(lib, p, good, need - 1) == moe.MOE_ERR_WORKSPACE
    # misaligned workspace
    assert lib.moe_w4a16_forward(*good, ctypes.byref(p), ctypes.c_void_p(0x20004), 1 << 40,
                                 None) == moe.MOE_ERR_ALIGNMENT


def test_zero_tokens_is_a_noop(lib):
    p = P(num_tokens=0)
    # no pointer is touched and nothing is launched
    assert lib.moe_w4a16_forward(*([None] * 9), ctypes.byref(p), None, 0, None) == moe.MOE_OK


def test_align_argument_errors(lib):
    p = P()
    cap_s, cap_b = moe.align_capacity(p, 16)
    f = ctypes.c_void_p
    ok = dict(ids=f(0x10000), sorted=f(0x20000), blocks=f(0x30000), npad=f(0x40000))

    def call(bm=16, cs=cap_s, cb=cap_b, scratch=None, nbytes=0, **over):
        a = dict(ok, **over)
        return lib.moe_w4a16_align(a["ids"], ctypes.byref(p), bm, a["sorted"], cs, a["blocks"],
                                   cb, a["npad"], scratch, nbytes, None)

    assert call(bm=0) == moe.MOE_ERR_SHAPE
    assert call(bm=2048) == moe.MOE_ERR_SHAPE
    assert call(cs=cap_s - 1) == moe.MOE_ERR_WORKSPACE
    assert call(cb=cap_b - 1) == moe.MOE_ERR_WORKSPACE
    assert call(ids=None) == moe.MOE_ERR_NULL
    assert call(npad=None) == moe.MOE_ERR_NULL
    assert call(sorted=f(0x20004)) == moe.MOE_ERR_ALIGNMENT
    need = moe.align_scratch_size(p)
    assert need == 4 * ((p.num_tokens * p.top_k + 255) // 256 + 1) * p.num_experts
    assert call(scratch=f(0x50000), nbytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(scratch=f(0x50008), nbytes=need) == moe.MOE_ERR_ALIGNMENT
    with pytest.raises(ValueError):
        moe.align_capacity(p, 0)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from w4a16_int4_grouped_moe_amd import _binding

    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _binding.library()


def test_route_argument_errors(lib):
    f = ctypes.c_void_p
    sc, ids, w = f(0x10000), f(0x20000), f(0x30000)

    def call(S=384, p=None, **over):
        a = dict(sc=sc, ids=ids, w=w)
        a.update(over)
        return lib.moe_w4a16_route(a["sc"], S, ctypes.byref(p or P()), a["ids"], a["w"], None)

    assert call(S=0) == moe.MOE_ERR_SHAPE
    assert call(S=1025) == moe.MOE_ERR_SHAPE
    assert call(S=7) == moe.MOE_ERR_SHAPE                      # top_k 8 > 7 scores
    assert call(S=383) == moe.MOE_ERR_SHAPE                    # local experts beyond the scores
    assert call(p=P(num_experts=48, expert_base=340)) == moe.MOE_ERR_SHAPE
    assert call(p=P(hidden=7100)) == moe.MOE_ERR_SHAPE          # the whole problem is checked
    assert call(sc=None) == moe.MOE_ERR_NULL
    assert call(ids=None) == moe.MOE_ERR_NULL
    assert call(w=f(0x30004)) == moe.MOE_ERR_ALIGNMENT
    assert call(p=P(num_tokens=0), sc=None, ids=None, w=None) == moe.MOE_OK  # no-op
    # the combined call checks the layer's arguments before its first launch
    good = [f(0x40000 + 0x100 * i) for i in range(7)]
    p = P()
    need = moe.workspace_size(p)
    args = [good[0], sc, 384] + good[1:7] + [ids, w, ctypes.byref(p), f(0x50000)]
    assert lib.moe_w4a16_forward_scores(*args, need - 1, None) == moe.MOE_ERR_WORKSPACE
    bad = list(args)
    bad[0] = None
    assert lib.moe_w4a16_forward_scores(*bad, need, None) == moe.MOE_ERR_NULL
    bad = list(args)
    bad[2] = 2000
    assert lib.moe_w4a16_forward_scores(*bad, need, None) == moe.MOE_ERR_SHAPE


def test_prepack_sizes_and_supported_widths(lib):
    # the full layer: the prepacked form is exactly as large as the four tensors
    per_expert = (2 * 2048 * 7168 // 2 + 2 * 2048 * 7168 // 32 * 2 +
                  7168 * 2048 // 2 + 7168 * 2048 // 32 * 2)
    assert moe.prepack_size(7168, 2048, 384) == 384 * per_expert
    # hidden 512, inter 768, 3 experts: W13 rows hold 16 scale groups (one
    # period of 16), W2 rows 24 (two periods, the second padded); regions are
    # 256-byte aligned
    rnd = lambda v: (v + 255) // 256 * 256
    codes13, scales13 = 3 * 1536 * 512 // 2, 3 * 1536 * 1 * 32
    codes2, scales2 = 3 * 512 * 768 // 2, 3 * 512 * 2 * 32
    assert moe.prepack_size(512, 768, 3) == (rnd(codes13) + rnd(scales13) + rnd(codes2) +
                                             rnd(scales2))
    # the tensor-parallel share (inter 256, the narrow down kernel) is served;
    # its W2 rows' 8 scale groups are padded to one period of 16
    assert moe.prepack_size(7168, 256, 384) == 384 * (2 * 256 * 7168 * 9 // 16 +
                                                      7168 * 256 // 2 + 7168 * 16 * 2)
    # widths the prefill tiles do not fit are not
    for hidden, inter in ((7168, 384), (640, 1024), (1024, 640), (7040, 2048)):
        n = ctypes.c_size_t()
        pp = P(hidden=hidden, inter=inter)
        assert lib.moe_w4a16_prepack_size(ctypes.byref(pp), ctypes.byref(n)) == \
            moe.MOE_ERR_UNSUPPORTED, (hidden, inter)


def test_prepack_argument_errors_before_launch(lib):
    p = P(num_experts=4)
    need = moe.prepack_size(7168, 2048, 4)
    w = [ctypes.c_void_p(0x10000 + 0x100 * i) for i in range(4)]
    buf = ctypes.c_void_p(0x90000)
    call = lambda ptrs, b=buf, n=need, pp=p: lib.moe_w4a16_prepack(*ptrs, ctypes.byref(pp), b, n,
                                                                   None)
    for i in range(4):
        ptrs = list(w)
        ptrs[i] = None
        assert call(ptrs) == moe.MOE_ERR_NULL, i
        ptrs[i] = ctypes.c_void_p(0x10008)
        assert call(ptrs) == moe.MOE_ERR_ALIGNMENT, i
    assert call(w, b=None) == moe.MOE_ERR_NULL
    assert call(w, b=ctypes.c_void_p(0x90004)) == moe.MOE_ERR_ALIGNMENT
    assert call(w, n=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(w, pp=P(num_experts=4, inter=384)) == moe.MOE_ERR_UNSUPPORTED


def test_forward_prepacked_argument_errors_before_launch(lib):
    p = P(num_experts=4)
    need = moe.prepack_size(7168, 2048, 4)
    ws = moe.workspace_size(p)
    x, ids, wts, sw, out = (ctypes.c_void_p(0x10000 + 0x100 * i) for i in range(5))
    buf = ctypes.c_void_p(0x90000)

    def call(b=buf, n=need, x=x, ids=ids, wts=wts, out=out, wsp=ctypes.c_void_p(0x20000),
             wsn=ws, pp=p):
        return lib.moe_w4a16_forward_prepacked(x, ids, wts, b, n, sw, out, ctypes.byref(pp), wsp,
                                               wsn, None)

    assert call(b=None) == moe.MOE_ERR_NULL
    assert call(b=ctypes.c_void_p(0x90008)) == moe.MOE_ERR_ALIGNMENT
    assert call(n=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(x=None) == moe.MOE_ERR_NULL
    assert call(out=ctypes.c_void_p(0x10004)) == moe.MOE_ERR_ALIGNMENT
    assert call(wsn=ws - 1) == moe.MOE_ERR_WORKSPACE
    assert call(pp=P(num_experts=4, inter=384)) == moe.MOE_ERR_UNSUPPORTED
    # zero tokens: a no-op that touches no pointer
    assert call(b=None, x=None, pp=P(num_tokens=0, num_experts=4)) == moe.MOE_OK


def test_noalloc_argument_errors_before_any_hip_call(lib):
    """The allocation-free variant checks its arguments (and its array's size
    limit) before resolving the array's address, so on a machine without a
    GPU every argument error still comes back as its own status."""
    good = [ctypes.c_void_p(0x10000 + 0x100 * i) for i in range(9)]
    call = lambda ptrs, p: lib.moe_w4a16_forward_noalloc(*ptrs, ctypes.byref(p), None)
    p = P(num_tokens=8)
    for i in range(9):
        if i == 7:
            continue  # shared_w is optional
        ptrs = list(good)
        ptrs[i] = None
        assert call(ptrs, p) == moe.MOE_ERR_NULL, i
        ptrs[i] = ctypes.c_void_p(0x10008)
        assert call(ptrs, p) == moe.MOE_ERR_ALIGNMENT, i
    assert lib.moe_w4a16_forward_noalloc(*good, None, None) == moe.MOE_ERR_NULL
    assert call(good, P(group_size=64)) == moe.MOE_ERR_UNSUPPORTED
    assert call(good, P(num_tokens=0)) == moe.MOE_OK
    # past the array: 193 Kimi-shape tokens take 96-row blocks (> 64 MiB)
    n = ctypes.c_size_t(0)
    assert lib.moe_w4a16_noalloc_workspace_limit(ctypes.byref(n)) == moe.MOE_OK
    assert n.value == 64 << 20
    assert moe.workspace_size(P(num_tokens=193)) > n.value
    assert call(good, P(num_tokens=193)) == moe.MOE_ERR_WORKSPACE
