"""The C ABI on the host: the library loads, exports what include/migemm.h
declares with the same struct layout, and rejects bad descriptions with the
documented status codes before touching a device."""
import os
import re
import subprocess
import tempfile

import pytest

from warp_specialized_pipelined_amd import migemm, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "migemm.h")


def have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gemm_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = migemm.load()
    names = header_functions()
    assert names == sorted(migemm.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", migemm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_library_shares_torchs_hip_runtime():
    """torch carries its own HIP runtime library; loading the binding first
    must still leave exactly one HIP runtime in the process (torch's), or the
    library could not use torch's device memory and streams."""
    import sys
    prog = ("import sys; sys.path.insert(0, %r)\n"
            "from warp_specialized_pipelined_amd import migemm\n"
            "migemm.load()\n"
            "import torch, os\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = sorted({os.path.realpath(l.split()[-1]) for l in maps if 'libamdhip64' in l})\n"
            "print(repr((libs, os.path.realpath(os.path.dirname(torch.__file__)))))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, check=True,
                         timeout=300).stdout
    libs, torch_dir = eval(out.strip().splitlines()[-1])
    assert len(libs) == 1, libs
    assert libs[0].startswith(torch_dir + os.sep), (libs, torch_dir)


def test_struct_layout_matches_c():
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "migemm.h"
#define F(s, f) printf(#s "." #f " %zu\n", offsetof(s, f))
int main(void) {
  printf("sizeof.desc %zu\n", sizeof(migemm_desc));
  printf("sizeof.info %zu\n", sizeof(migemm_plan_info));
  F(migemm_desc, M); F(migemm_desc, a_type); F(migemm_desc, a_rs); F(migemm_desc, d_cs);
  F(migemm_desc, device); F(migemm_desc, flags); F(migemm_desc, max_workgroups);
  F(migemm_desc, L); F(migemm_desc, d_bs); F(migemm_desc, debug_wait_ticks);
  F(migemm_desc, debug_force_wait); F(migemm_desc, reserved2);
  printf("sizeof.dbg %zu\n", sizeof(migemm_debug_info));
  F(migemm_debug_info, max_occupancy); F(migemm_debug_info, trace_offset);
  F(migemm_debug_info, trace_words);
  F(migemm_plan_info, grid); F(migemm_plan_info, tile_k); F(migemm_plan_info, handoff_slots);
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(line.rsplit(" ", 1) for line in out.strip().splitlines())
    import ctypes
    assert int(got["sizeof.desc"]) == ctypes.sizeof(migemm.migemm_desc)
    assert int(got["sizeof.info"]) == ctypes.sizeof(migemm.migemm_plan_info)
    assert int(got["sizeof.dbg"]) == ctypes.sizeof(migemm.migemm_debug_info)
    classes = {"migemm_desc": migemm.migemm_desc, "migemm_plan_info": migemm.migemm_plan_info,
               "migemm_debug_info": migemm.migemm_debug_info}
    for key, v in got.items():
        if key.startswith("sizeof"):
            continue
        s, f = key.split(".")
        cls = classes[s]
        assert getattr(cls, f).offset == int(v), key


def desc_for(w: synth.Workload, **over):
    a_rs, a_cs = synth.strides(w.a_layout, w.M, w.K)
    b_rs, b_cs = synth.strides(w.b_layout, w.K, w.N)
    t = migemm.MIGEMM_BF16 if w.dtype == synth.BF16 else migemm.MIGEMM_FP8_E4M3
    d = dict(M=w.M, N=w.N, K=w.K, a_type=t, b_type=t, a_rs=a_rs, a_cs=a_cs, b_rs=b_rs, b_cs=b_cs,
             c_rs=w.N, c_cs=1, d_rs=w.N, d_cs=1,
             flags=migemm.MIGEMM_F_TILE_CONSUMER if w.consumer else 0)
    d.update(over)
    return migemm.make_desc(**d)


@pytest.mark.parametrize("w", synth.WORKLOADS, ids=lambda w: w.name)
def test_every_workload_is_a_valid_description(w):
    assert migemm.gemm_desc_validate(desc_for(w)) == migemm.MIGEMM_OK


W = synth.WORKLOADS[2]  # 4000 x 3000 x 5000, row/row


@pytest.mark.parametrize("over,status", [
    (dict(M=-1), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(K=-5), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(a_type=7), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(a_type=migemm.MIGEMM_FP8_E4M3), migemm.MIGEMM_ERR_UNSUPPORTED),   # mixed A/B types
    (dict(d_type=migemm.MIGEMM_FP8_E4M3), migemm.MIGEMM_ERR_UNSUPPORTED),
    (dict(a_rs=4999), migemm.MIGEMM_ERR_INVALID_ARG),                       # stride < extent
    (dict(a_rs=5000, a_cs=2), migemm.MIGEMM_ERR_INVALID_ARG),               # no unit stride
    (dict(a_rs=5004), migemm.MIGEMM_ERR_MISALIGNED),                        # 10008-byte rows
    (dict(b_rs=3004), migemm.MIGEMM_ERR_MISALIGNED),
    (dict(d_rs=3001), migemm.MIGEMM_ERR_MISALIGNED),
    (dict(c_rs=1, c_cs=4000), migemm.MIGEMM_ERR_UNSUPPORTED),               # C col, D row
    (dict(flags=migemm.MIGEMM_F_TILE_CONSUMER, c_rs=1, c_cs=4000, d_rs=1, d_cs=4000),
     migemm.MIGEMM_ERR_UNSUPPORTED),                                        # consumer needs row D
    (dict(flags=0x100), migemm.MIGEMM_ERR_INVALID_ARG),                    # unknown flag
    (dict(flags=migemm.MIGEMM_F_TILE_M192), migemm.MIGEMM_OK),
    (dict(flags=migemm.MIGEMM_F_TILE_M256), migemm.MIGEMM_OK),
    (dict(flags=migemm.MIGEMM_F_TILE_M256 | migemm.MIGEMM_F_TILE_CONSUMER), migemm.MIGEMM_OK),
    (dict(flags=migemm.MIGEMM_F_TILE_M192 | migemm.MIGEMM_F_TILE_M256), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(flags=migemm.MIGEMM_F_TILE_M192 | migemm.MIGEMM_F_TILE_CONSUMER),
     migemm.MIGEMM_ERR_INVALID_ARG),                                        # 192 rows: no consumer
    (dict(flags=migemm.MIGEMM_F_TILE_M192 | migemm.MIGEMM_F_STREAM_K), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(flags=migemm.MIGEMM_F_TILE_M192 | migemm.MIGEMM_F_STREAM_K_FORCE),
     migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(flags=migemm.MIGEMM_F_TILE_M192, a_type=migemm.MIGEMM_FP8_E4M3, b_type=migemm.MIGEMM_FP8_E4M3),
     migemm.MIGEMM_ERR_UNSUPPORTED),                                        # 192 rows: bf16 only
    (dict(flags=migemm.MIGEMM_F_STREAM_K_FORCE), migemm.MIGEMM_OK),
    (dict(flags=migemm.MIGEMM_F_STREAM_K_FORCE | migemm.MIGEMM_F_TILE_CONSUMER),
     migemm.MIGEMM_ERR_UNSUPPORTED),
    (dict(flags=migemm.MIGEMM_F_STREAM_K), migemm.MIGEMM_OK),
    (dict(flags=migemm.MIGEMM_F_STREAM_K | migemm.MIGEMM_F_TILE_CONSUMER),
     migemm.MIGEMM_ERR_UNSUPPORTED),                                        # consumer: whole tiles
    (dict(flags=migemm.MIGEMM_F_CONSUMER_OVERLAP), migemm.MIGEMM_ERR_INVALID_ARG),  # no consumer
    (dict(flags=migemm.MIGEMM_F_CONSUMER_OVERLAP | migemm.MIGEMM_F_TILE_CONSUMER), migemm.MIGEMM_OK),
    (dict(flags=migemm.MIGEMM_F_CONSUMER_OVERLAP | migemm.MIGEMM_F_TILE_CONSUMER |
          migemm.MIGEMM_F_STREAM_K_FORCE), migemm.MIGEMM_ERR_UNSUPPORTED),
    (dict(max_workgroups=-1), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(flags=migemm.MIGEMM_F_HANDOFF_DEBUG), migemm.MIGEMM_ERR_INVALID_ARG),      # no consumer
    (dict(flags=migemm.MIGEMM_F_HANDOFF_DEBUG | migemm.MIGEMM_F_TILE_CONSUMER), migemm.MIGEMM_OK),
    (dict(flags=migemm.MIGEMM_F_HANDOFF_DEBUG | migemm.MIGEMM_F_TILE_CONSUMER,
          debug_wait_ticks=1000, debug_force_wait=1), migemm.MIGEMM_OK),
    (dict(debug_wait_ticks=1000), migemm.MIGEMM_ERR_INVALID_ARG),                   # needs the flag
    (dict(flags=migemm.MIGEMM_F_HANDOFF_DEBUG | migemm.MIGEMM_F_TILE_CONSUMER,
          debug_force_wait=-1), migemm.MIGEMM_ERR_INVALID_ARG),
    # strides whose products would wrap a 64-bit integer: each operand's span
    # (with its batches) is bounded at 2^47 bytes, exactly
    (dict(a_rs=1 << 62), migemm.MIGEMM_ERR_UNSUPPORTED),
    (dict(a_rs=1 << 59), migemm.MIGEMM_ERR_UNSUPPORTED),
    (dict(b_rs=1 << 61), migemm.MIGEMM_ERR_UNSUPPORTED),
    (dict(d_rs=1 << 60, c_rs=1 << 60), migemm.MIGEMM_ERR_UNSUPPORTED),
    # column-major A with a 2^24-byte leading stride (64 K rows span 2^30):
    # K = 2^23 puts it just below 2^47 bytes, K = 2^23 + 2 just past
    (dict(K=1 << 23, a_rs=1, a_cs=1 << 23), migemm.MIGEMM_OK),
    (dict(K=(1 << 23) + 2, a_rs=1, a_cs=1 << 23), migemm.MIGEMM_ERR_UNSUPPORTED),
    (dict(K=5001, a_rs=5008), migemm.MIGEMM_OK),                            # K-contiguous A, any K
    (dict(K=5001, a_rs=5001), migemm.MIGEMM_ERR_MISALIGNED),                # but 16-byte rows
])
def test_validation_status_codes(over, status):
    assert migemm.gemm_desc_validate(desc_for(W, **over)) == status


@pytest.mark.parametrize("over,status", [
    (dict(L=0), migemm.MIGEMM_OK),                                          # one product
    (dict(L=3, a_bs=0, b_bs=0, c_bs=0, d_bs=4000 * 3000), migemm.MIGEMM_OK),  # shared A, B, C
    (dict(L=-1), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(L=2, a_bs=-5000, d_bs=4000 * 3000), migemm.MIGEMM_ERR_INVALID_ARG),
    (dict(L=2, d_bs=4000 * 3000 - 8), migemm.MIGEMM_ERR_INVALID_ARG),        # D batches overlap
    (dict(L=2, a_bs=4, d_bs=4000 * 3000), migemm.MIGEMM_ERR_MISALIGNED),     # 8-byte batch step
    (dict(L=2, d_bs=4000 * 3000 + 4), migemm.MIGEMM_ERR_MISALIGNED),
    (dict(L=1 << 24, d_bs=4000 * 3000), migemm.MIGEMM_ERR_UNSUPPORTED),      # 2^31+ tiles
    (dict(L=3, a_bs=1 << 61, d_bs=4000 * 3000), migemm.MIGEMM_ERR_UNSUPPORTED),  # wrapping batch step
    (dict(L=2, a_bs=(1 << 46) // 2, d_bs=4000 * 3000), migemm.MIGEMM_OK),   # 64 TiB step: in range
])
def test_batch_validation(over, status):
    assert migemm.gemm_desc_validate(desc_for(W, **over)) == status


@pytest.mark.parametrize("t", [migemm.MIGEMM_BF16, migemm.MIGEMM_FP8_E4M3], ids=["bf16", "e4m3"])
def test_any_k_in_every_layout(t):
    """K needs no alignment in any layout; only the leading strides do."""
    align = 8 if t == migemm.MIGEMM_BF16 else 16
    for K in (1, 7, 9, 17, 5001):
        ldk = -(-K // align) * align                   # K rounded up to 16 bytes
        for a_rs, a_cs in ((ldk, 1), (1, 64)):         # A K- or M-contiguous
            for b_rs, b_cs in ((64, 1), (1, ldk)):     # B N- or K-contiguous
                d = migemm.make_desc(64, 64, K, t, t, a_rs, a_cs, b_rs, b_cs, 64, 1, 64, 1)
                assert migemm.gemm_desc_validate(d) == migemm.MIGEMM_OK, (K, a_rs, b_rs)
        d = migemm.make_desc(64, 64, K, t, t, K, 1, 64, 1, 64, 1, 64, 1)   # rows of K elements
        want = migemm.MIGEMM_OK if K % align == 0 else migemm.MIGEMM_ERR_MISALIGNED
        assert migemm.gemm_desc_validate(d) == want


@pytest.mark.parametrize("t", [migemm.MIGEMM_BF16, migemm.MIGEMM_FP8_E4M3], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("operand", ["A", "B"])
def test_stage_span_of_mn_contiguous_operands(t, operand):
    # One stage of an MN-contiguous operand is 128 bytes of K (64 bf16 or 128
    # e4m3 rows of ld elements), so it spans 128 * ld bytes whatever the
    # type; the loads address it with 32-bit offsets below 2^31.  With
    # ld = 2^24 a stage is 2^31 bytes: rejected.  (A check that assumed
    # 64-byte stages would have let it through.)
    for ld, status in [(2 ** 24, migemm.MIGEMM_ERR_UNSUPPORTED),
                       (2 ** 24 - 64, migemm.MIGEMM_OK)]:
        if operand == "A":   # column-major A: M-contiguous, ld between K columns
            d = migemm.make_desc(256, 256, 256, t, t, 1, ld, 1, 256, 256, 1, 256, 1)
        else:                # row-major B: N-contiguous, ld between K rows
            d = migemm.make_desc(256, 256, 256, t, t, 256, 1, ld, 1, 256, 1, 256, 1)
        assert migemm.gemm_desc_validate(d) == status, (ld, status)


def test_empty_and_degenerate_shapes_are_valid():
    for M, N, K in [(0, 0, 0), (0, 16, 16), (16, 0, 16), (16, 16, 0), (1, 1, 8)]:
        d = migemm.make_desc(M, N, K, 1, 1, max(K, 8), 1, max(N, 8), 1, max(N, 8), 1, max(N, 8), 1)
        assert migemm.gemm_desc_validate(d) == migemm.MIGEMM_OK, (M, N, K)


def test_column_major_d_is_valid():
    d = migemm.make_desc(100, 60, 64, 1, 1, 64, 1, 60 + 4, 1, 1, 104, 1, 104)
    assert migemm.gemm_desc_validate(d) == migemm.MIGEMM_OK


def test_status_strings():
    for st in range(-6, 1):
        s = migemm.gemm_status_string(st)
        assert s.startswith("MIGEMM_")
    assert "unknown" in migemm.gemm_status_string(-99)


def test_null_arguments_are_rejected_without_a_device():
    lib = migemm.load()
    assert lib.gemm_run(None, None, None, None, None, 1.0, 0.0, None, None) == migemm.MIGEMM_ERR_INVALID_ARG
    assert lib.gemm_plan_create(None, None) == migemm.MIGEMM_ERR_INVALID_ARG
    assert lib.gemm_plan_get_info(None, None) == migemm.MIGEMM_ERR_INVALID_ARG
    assert lib.gemm_plan_destroy(None) == migemm.MIGEMM_OK
    assert migemm.gemm_plan_workspace_size(None) == 0
    assert lib.gemm_workspace_init(None, None, None) == migemm.MIGEMM_ERR_INVALID_ARG


def test_pointers_that_are_not_live_plans_are_rejected_unread():
    # A host buffer that was never a plan, filled with bytes that would make
    # wild kernel arguments: every entry point must refuse it before reading
    # it (the library checks a plan against the plans alive in the process).
    import ctypes
    lib = migemm.load()
    junk = ctypes.create_string_buffer(b"\xff" * 4096)
    fake = ctypes.addressof(junk)
    bad = migemm.MIGEMM_ERR_INVALID_ARG
    assert lib.gemm_run(fake, None, None, None, None, 1.0, 0.0, None, None) == bad
    assert lib.gemm_run_with_tile_consumer(fake, None, None, None, None, 1.0, 0.0, None, None,
                                           None, None, None) == bad
    assert lib.gemm_run_no_alloc(fake, None, None, None, None, 1.0, 0.0, None) == bad
    assert lib.gemm_plan_get_info(fake, ctypes.byref(migemm.migemm_plan_info())) == bad
    assert lib.gemm_workspace_init(fake, fake, None) == bad
    assert lib.gemm_debug_read(fake, fake, None, ctypes.byref(migemm.migemm_debug_info())) == bad
    assert migemm.gemm_plan_workspace_size(fake) == 0
    assert lib.gemm_plan_destroy(fake) == bad          # nothing freed
    assert junk.raw == b"\xff" * 4096 + b"\x00"


@pytest.mark.skipif(have_gpu(), reason="checks the no-device path")
def test_plan_create_without_a_gpu_reports_device_error():
    with pytest.raises(migemm.MigemmError) as e:
        migemm.gemm_plan_create(desc_for(synth.WORKLOADS[0]))
    assert e.value.status == migemm.MIGEMM_ERR_DEVICE
    # validation errors are reported before the device query
    with pytest.raises(migemm.MigemmError) as e:
        migemm.gemm_plan_create(desc_for(W, M=-1))
    assert e.value.status == migemm.MIGEMM_ERR_INVALID_ARG


def test_header_constants_match_the_binding():
    # Every #define of the header has the same value in the Python binding.
    text = open(HEADER).read()
    defines = dict(re.findall(r"#define (MIGEMM_\w+) (0x[0-9a-fA-F]+|\d+)u?\b", text))
    assert "MIGEMM_F_CONSUMER_OVERLAP" in defines and len(defines) >= 6
    for name, value in defines.items():
        assert getattr(migemm, name) == int(value, 0), name


def test_validation_accepts_only_addressable_descriptions():
    """Property: for descriptions with sizes and strides anywhere in int64
    (hypothesis explores the extremes), gemm_desc_validate never crashes,
    and whatever it accepts keeps every operand -- with all its batches --
    within 2^47 bytes, its leading strides 16-byte aligned, and the 32-bit
    offsets of one tile band (256 rows, or one 128-byte stage of K rows)
    below 2^31.  The model uses Python's exact integers, not the library's
    arithmetic.  Leading strides are drawn as the contiguous extent plus an
    extra, rounded up to 16 bytes, so that most descriptions are valid and
    the bounds, not the alignment rule, decide."""
    from hypothesis import HealthCheck, given, settings, strategies as st

    size = st.one_of(st.integers(0, 3000), st.integers(0, 1 << 20),
                     st.sampled_from([0, 1, 255, 256, 257, 1 << 23, (1 << 23) + 2, 1 << 30, 1 << 40,
                                      (1 << 62) + 3, (1 << 63) - 1]))
    extra = st.one_of(st.just(0), st.integers(0, 1 << 16),
                      st.sampled_from([1 << 20, 1 << 23, 1 << 30, 1 << 40, 1 << 46, 1 << 47,
                                       1 << 59, 1 << 62]))
    layout = st.sampled_from(["row", "col"])
    accepted = []

    def up(x, a):
        return min(-(-x // a) * a, (1 << 63) - a)

    @settings(max_examples=3000, deadline=None, suppress_health_check=list(HealthCheck))
    @given(M=size, N=size, K=size, la=layout, lb=layout, xa=extra, xb=extra, xd=extra,
           fp8=st.booleans(), L=st.one_of(st.just(1), st.integers(2, 8), st.just(1 << 20)),
           xabs=extra, xbbs=extra, xdbs=extra)
    def check(M, N, K, la, lb, xa, xb, xd, fp8, L, xabs, xbbs, xdbs):
        t = migemm.MIGEMM_FP8_E4M3 if fp8 else migemm.MIGEMM_BF16
        es = 1 if fp8 else 2
        al = 16 // es
        lda = up((K if la == "row" else M) + xa, al)
        ldb = up((N if lb == "row" else K) + xb, al)
        ldd = up(N + xd, 8)
        a_rs, a_cs = (lda, 1) if la == "row" else (1, lda)
        b_rs, b_cs = (ldb, 1) if lb == "row" else (1, ldb)
        abs_ = up(M * K + xabs, al) if L > 1 else 0
        bbs = up(K * N + xbbs, al) if L > 1 else 0
        dbs = up(M * ldd + xdbs, 8) if L > 1 else 0
        d = migemm.make_desc(M, N, K, t, t, a_rs, a_cs, b_rs, b_cs, ldd, 1, ldd, 1, L=L,
                             a_bs=abs_, b_bs=bbs, c_bs=dbs, d_bs=dbs)
        if migemm.gemm_desc_validate(d) != migemm.MIGEMM_OK:
            return
        accepted.append((M, N, K))
        Lc = L if L > 1 else 1

        def span(rows, cols, rs, cs, e, bs):
            if rows <= 0 or cols <= 0:
                return 0
            return ((rows - 1) * rs + (cols - 1) * cs + 1) * e + (Lc - 1) * bs * e

        assert span(M, K, a_rs, a_cs, es, abs_) <= 1 << 47
        assert span(K, N, b_rs, b_cs, es, bbs) <= 1 << 47
        assert span(M, N, ldd, 1, 2, dbs) <= 1 << 47
        for rows_or_cols, ld, kmajor in ((M, lda, la == "row"), (N, ldb, lb == "col")):
            if rows_or_cols > 0 and K > 0:
                assert (ld * es) % 16 == 0
                assert (256 if kmajor else 128 // es) * ld * es < 1 << 31
        if M > 0 and N > 0:
            assert (ldd * 2) % 16 == 0 and 256 * ldd * 2 < 1 << 31

    check()
    assert len(accepted) > 500, len(accepted)   # the property was tested, not vacuous


def test_validation_under_host_sanitizers():
    """tests/c_validate_extremes.c runs gemm_desc_validate over ~375,000
    descriptions with sizes and strides from 0 to 2^63 - 1 (and the
    plan-taking entry points on pointers that are not plans) against the
    library built with the host address and undefined-behaviour sanitizers:
    any signed overflow, bad shift or out-of-bounds access aborts it with a
    report.  (The validation before its span bounds overflowed here.)"""
    exe = os.path.join(ROOT, "tests", "_build", "c_validate_extremes")
    asan_lib = os.path.join(ROOT, "warp_specialized_pipelined_amd", "_build", "libmigemm_asan.so")
    if not os.path.exists(exe):
        if not os.path.exists(asan_lib):
            pytest.skip("the sanitized library is built by __graft_entry__.build()")
        from warp_specialized_pipelined_amd import build
        build.build_c_client()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr[-2000:])
    tried, accepted = map(int, re.findall(r"tried (\d+) accepted (\d+)", r.stdout)[0])
    assert tried > 300000 and accepted > 1000, r.stdout
