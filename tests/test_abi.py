"""The C ABI loads, exports every symbol include/moe_route.h declares, and
rejects invalid arguments on the host before any HIP call (so these run
without a GPU). No test here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")

binding = pytest.importorskip("combine_moe_route_amd.binding")
lib = binding.lib

OK, EINVAL, ENOSPC, EALIGN, EHIP, ENULL = 0, -1, -2, -3, -4, -5
A = 0x100000      # fake device addresses: never dereferenced, validation fails first
B = 0x200000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 6
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert sorted(binding.EXPORTS) == names


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    for name, val in [("MOE_OK", OK), ("MOE_EINVAL", EINVAL), ("MOE_ENOSPC", ENOSPC),
                      ("MOE_EALIGN", EALIGN), ("MOE_EHIP", EHIP), ("MOE_ENULL", ENULL)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name
        assert getattr(binding, name) == val
    assert re.search(r"MOE_MAX_EXPERTS\s+1024", text)


def test_status_strings():
    for s in (OK, EINVAL, ENOSPC, EALIGN, EHIP, ENULL):
        assert binding.status_string(s) and binding.status_string(s) != "unknown status"
    assert binding.status_string(7) == "unknown status"


def test_max_rows_and_workspace():
    assert lib.moe_dispatch_max_rows(16384, 256, 8, 128) == 16384 * 8 + 256 * 127
    assert lib.moe_dispatch_max_rows(4096, 384, 8, 1) == 4096 * 8
    assert lib.moe_dispatch_max_rows(0, 4, 2, 1) == 0
    assert lib.moe_dispatch_max_rows(10, 4, 5, 1) == -1          # k > E
    assert lib.moe_dispatch_max_rows(10, 1025, 2, 1) == -1       # E too large
    assert lib.moe_dispatch_max_rows(10, 4, 2, 0) == -1          # row_align < 1
    assert lib.moe_dispatch_max_rows(10, 4, 2, 1025) == -1
    assert lib.moe_dispatch_max_rows(2 ** 28, 8, 8, 1) == -1     # rows overflow int32
    # each part 256-byte aligned: byte tile counts [tiles, E], int32 tile
    # prefixes [tiles, E], byte in-tile ranks [T, k]; tiles of 16 tokens up
    # to T = 1024, 32 up to 4096, else 64
    def ws(T, E, k):
        r = lambda n: (n + 255) // 256 * 256
        tt = 16 if T <= 1024 else 32 if T <= 4096 else 64
        tiles = (T + tt - 1) // tt
        return r(tiles * ((E + 3) // 4 * 4)) + r(4 * tiles * E) + r(T * k)
    assert lib.moe_dispatch_workspace_bytes(16384, 256, 8, 32) == 458752 == ws(16384, 256, 8)
    assert lib.moe_dispatch_workspace_bytes(4096, 384, 8, 1) == 278528 == ws(4096, 384, 8)
    assert lib.moe_dispatch_workspace_bytes(300, 8, 2, 1) == 1792 == ws(300, 8, 2)
    assert lib.moe_dispatch_workspace_bytes(0, 8, 2, 1) == 0 == ws(0, 8, 2)
    for T in (1, 16, 17, 1024, 1025, 4096, 4097, 100_000):
        assert lib.moe_dispatch_workspace_bytes(T, 96, 6, 3) == ws(T, 96, 6)
        assert lib.moe_dispatch_workspace_bytes(T, 65, 3, 5) == ws(T, 65, 3)   # rows padded to 68
    assert lib.moe_dispatch_workspace_bytes(300, 8, 2, 3) == 0   # E % groups != 0


def route(logits=A, T=16, E=8, k=2, idx=B, w=B + 4096):
    return lib.moe_route_topk(logits, T, E, k, idx, w, None)


def test_route_topk_validation():
    assert route(k=0) == EINVAL
    assert route(k=9) == EINVAL
    assert route(E=1025, k=2) == EINVAL
    assert route(T=-1) == EINVAL
    assert route(T=2 ** 31, k=2) == EINVAL
    assert route(T=2 ** 27, E=1024, k=8) == EINVAL       # one wave per token: 2^33 work-items
    assert route(T=2 ** 28, E=768, k=1) == EINVAL        # 16 lanes per token: 2^32 work-items
    assert route(logits=None) == ENULL
    assert route(idx=None) == ENULL
    assert route(logits=A + 2) == EALIGN
    assert route(T=0, logits=None, idx=None, w=None) == OK      # no-op


def test_route_variant_validation():
    sh = lambda logits=A, T=16, E=8, k=2, ns=1, idx=B, w=B + 4096: lib.moe_route_topk_shared(
        logits, T, E, k, ns, 1.0, idx, w, None)
    assert sh(ns=-1) == EINVAL
    assert sh(E=1020, ns=5) == EINVAL                   # E + n_shared > 1024
    assert sh(k=9) == EINVAL
    assert sh(logits=None) == ENULL
    assert sh(w=B + 2) == EALIGN
    assert sh(T=0, logits=None, idx=None, w=None) == OK
    rep = lambda idx=B, T=16, k=2, E=8, base=A: lib.moe_route_replicas(idx, T, k, E, base, None)
    assert rep(E=0) == EINVAL
    assert rep(k=0) == EINVAL
    assert rep(base=None) == ENULL
    assert rep(idx=B + 1) == EALIGN
    assert rep(T=0, idx=None, base=None) == OK


def dispatch(**kw):
    a = dict(x=A, idx=B, T=256, H=256, E=8, k=2, groups=1, row_align=1, dt=0, out=A + 2 ** 20,
             scales=A + 2 ** 21, counts=B + 2 ** 20, offsets=B + 2 ** 20 + 64,
             goff=B + 2 ** 20 + 128, row_src=B + 2 ** 21, dst_row=B + 2 ** 22,
             ws=B + 2 ** 23, wsb=1 << 20)
    a.update(kw)
    return lib.moe_dispatch(a["x"], a["idx"], a["T"], a["H"], a["E"], a["k"], a["groups"],
                            a["row_align"], a["dt"], a["out"], a["scales"], a["counts"],
                            a["offsets"], a["goff"], a["row_src"], a["dst_row"], a["ws"], a["wsb"],
                            None)


def test_dispatch_validation():
    assert dispatch(k=0) == EINVAL
    assert dispatch(k=9) == EINVAL
    assert dispatch(E=2000) == EINVAL
    assert dispatch(groups=3) == EINVAL                  # 8 % 3 != 0
    assert dispatch(groups=0) == EINVAL
    assert dispatch(groups=16) == EINVAL                 # more groups than experts
    assert dispatch(row_align=0) == EINVAL
    assert dispatch(row_align=2048) == EINVAL
    assert dispatch(dt=2) == EINVAL
    assert dispatch(H=12) == EINVAL                      # bf16 rows need H % 8 == 0
    assert dispatch(H=200, dt=1) == EINVAL               # FP8 rows need H % 128 == 0
    assert dispatch(H=0) == EINVAL
    assert dispatch(H=65544) == EINVAL
    assert dispatch(T=-5) == EINVAL
    assert dispatch(T=2 ** 29, k=8) == EINVAL            # rows overflow int32
    assert dispatch(T=2 ** 27, H=65536, k=1, E=1) == EINVAL   # launch grid too large
    # every kernel must fit a launch packet (blocks * threads < 2^32): bf16
    # rows of 7168 take 14 waves per token, so 5M tokens need 4.48G
    # work-items in the scatter; rejected before any launch, even with a
    # workspace too small (sizes are checked first)
    big = dict(T=5_000_000, H=7168, k=1, E=1, wsb=1 << 40)
    assert dispatch(**big) == EINVAL
    assert dispatch(**dict(big, wsb=16)) == EINVAL
    assert dispatch(**dict(big, T=4_000_000, wsb=16)) == ENOSPC   # 3.58G work-items fit
    assert dispatch(T=20_000_000, H=1024, k=1, E=1, dt=1, wsb=1 << 40) == EINVAL  # FP8: T blocks x 256
    assert dispatch(x=None) == ENULL
    assert dispatch(idx=None) == ENULL
    assert dispatch(out=None) == ENULL
    assert dispatch(row_src=None) == ENULL
    assert dispatch(dst_row=None) == ENULL
    assert dispatch(counts=None) == ENULL
    assert dispatch(offsets=None) == ENULL
    assert dispatch(dt=1, scales=None) == ENULL
    assert dispatch(ws=None) == ENULL
    assert dispatch(x=A + 8) == EALIGN                   # payloads need 16 bytes
    assert dispatch(out=A + 2 ** 20 + 4) == EALIGN
    assert dispatch(idx=B + 2) == EALIGN
    assert dispatch(dst_row=B + 2 ** 22 + 1) == EALIGN
    assert dispatch(wsb=7) == ENOSPC
    assert dispatch(wsb=lib.moe_dispatch_workspace_bytes(256, 8, 2, 1) - 4) == ENOSPC


def test_route_dispatch_validation():
    """moe_route_dispatch: the moe_dispatch checks plus the routing pointers;
    every case here is rejected before any launch."""
    def rd(**kw):
        a = dict(logits=A + 2 ** 24, x=A, T=256, H=256, E=8, k=2, groups=1, row_align=1, dt=0,
                 idx=B, w=B + 2 ** 19, out=A + 2 ** 20, scales=A + 2 ** 21, counts=B + 2 ** 20,
                 offsets=B + 2 ** 20 + 64, goff=B + 2 ** 20 + 128, row_src=B + 2 ** 21,
                 dst_row=B + 2 ** 22, ws=B + 2 ** 23, wsb=1 << 20)
        a.update(kw)
        return lib.moe_route_dispatch(a["logits"], a["x"], a["T"], a["H"], a["E"], a["k"],
                                      a["groups"], a["row_align"], a["dt"], a["idx"], a["w"],
                                      a["out"], a["scales"], a["counts"], a["offsets"], a["goff"],
                                      a["row_src"], a["dst_row"], a["ws"], a["wsb"], None)
    assert rd(k=0) == EINVAL
    assert rd(k=9, E=8) == EINVAL
    assert rd(groups=3) == EINVAL
    assert rd(H=200, dt=1) == EINVAL
    assert rd(logits=None, w=None) == ENULL
    assert rd(logits=None) == ENULL
    assert rd(w=None) == ENULL
    assert rd(idx=None) == ENULL
    assert rd(logits=A + 2 ** 24 + 2) == EALIGN
    assert rd(w=B + 2 ** 19 + 1) == EALIGN
    assert rd(wsb=16) == ENOSPC
    assert rd(ws=None, wsb=1 << 20) == ENULL
    assert rd(T=2 ** 29, k=8) == EINVAL                      # rows overflow int32


def test_dispatch_no_alloc_validation():
    """The no-alloc variant checks everything before any HIP call; a request
    needing more scratch than the library's array holds is MOE_ENOSPC."""
    cap = binding.MOE_NO_ALLOC_SCRATCH_BYTES
    assert cap == 16 << 20
    assert re.search(r"MOE_NO_ALLOC_SCRATCH_BYTES\s+\(16u << 20\)", open(HEADER).read())

    def na(**kw):
        a = dict(x=A, idx=B, T=256, H=256, E=8, k=2, groups=1, row_align=1, dt=0,
                 out=A + 2 ** 20, scales=A + 2 ** 21, counts=B + 2 ** 20,
                 offsets=B + 2 ** 20 + 64, goff=B + 2 ** 20 + 128, row_src=B + 2 ** 21,
                 dst_row=B + 2 ** 22)
        a.update(kw)
        return lib.moe_dispatch_no_alloc(a["x"], a["idx"], a["T"], a["H"], a["E"], a["k"],
                                         a["groups"], a["row_align"], a["dt"], a["out"],
                                         a["scales"], a["counts"], a["offsets"], a["goff"],
                                         a["row_src"], a["dst_row"], None)
    assert na(k=0) == EINVAL
    assert na(groups=3) == EINVAL
    assert na(H=12) == EINVAL
    assert na(x=None) == ENULL
    assert na(out=A + 2 ** 20 + 4) == EALIGN
    # workspace needed beyond the static scratch
    T_big = 2_000_000
    assert lib.moe_dispatch_workspace_bytes(T_big, 64, 8, 1) > cap
    assert na(T=T_big, E=64, k=8) == ENOSPC
    assert lib.moe_dispatch_workspace_bytes(16384, 256, 8, 32) <= cap


def test_combine_validation():
    c = lambda eo=A, dr=B, w=B + 4096, T=16, H=64, k=2, y=A + 2 ** 20: lib.moe_combine(
        eo, dr, w, T, H, k, y, None)
    assert c(H=60) == EINVAL
    assert c(H=0) == EINVAL
    assert c(k=0) == EINVAL
    assert c(k=1025) == EINVAL
    assert c(T=-1) == EINVAL
    assert c(T=2 ** 28, H=65536, k=1) == EINVAL          # launch grid too large
    assert c(T=5_000_000, H=7168, k=1) == EINVAL         # 4.48G work-items
    assert c(T=4_000_000, H=7168, k=1, y=None) == ENULL  # fits; fails later on the pointer
    assert c(eo=None) == ENULL
    assert c(y=None) == ENULL
    assert c(eo=A + 8) == EALIGN
    assert c(y=A + 2 ** 20 + 2) == EALIGN
    assert c(w=B + 4098) == EALIGN
    assert c(T=0, eo=None, dr=None, w=None, y=None) == OK


def test_grouped_gemm_workspace_bytes():
    # 256 bytes of header (tile count), then one int4 per possible 128-row
    # tile: ceil(max_rows / 128) + E (each segment adds at most one partial tile)
    assert lib.moe_grouped_gemm_workspace_bytes(147584, 256) == 256 + (1153 + 256) * 16
    assert lib.moe_grouped_gemm_workspace_bytes(1, 1) == 256 + 2 * 16
    assert lib.moe_grouped_gemm_workspace_bytes(0, 8) == 256 + 8 * 16
    assert lib.moe_grouped_gemm_workspace_bytes(-1, 8) == 0
    assert lib.moe_grouped_gemm_workspace_bytes(100, 0) == 0
    assert lib.moe_grouped_gemm_workspace_bytes(100, 1025) == 0


def test_grouped_gemm_validation():
    ws = lib.moe_grouped_gemm_workspace_bytes(1000, 8)

    def g(**kw):
        return lib.moe_grouped_gemm_fp8(
            kw.get("a", A), kw.get("asc", B), kw.get("off", B + 4096), kw.get("w", A + 2 ** 24),
            kw.get("wsc", B + 8192), kw.get("E", 8), kw.get("N", 512), kw.get("K", 256),
            kw.get("R", 1000), kw.get("y", A + 2 ** 26), kw.get("ws", B + 2 ** 20),
            kw.get("wsb", ws), None)
    assert g(N=384) == EINVAL                  # N % 256
    assert g(N=0) == EINVAL
    assert g(N=2 ** 21) == EINVAL
    assert g(K=200) == EINVAL                  # K % 128
    assert g(K=0) == EINVAL
    assert g(K=2 ** 21) == EINVAL
    assert g(E=0) == EINVAL
    assert g(E=1025) == EINVAL
    assert g(R=-1) == EINVAL
    assert g(R=2 ** 31) == EINVAL
    assert g(R=2 ** 31 - 1, N=2 ** 20) == EINVAL    # launch grid too large
    assert g(a=None) == ENULL
    assert g(wsc=None) == ENULL
    assert g(ws=None) == ENULL
    assert g(a=A + 8) == EALIGN
    assert g(w=A + 2 ** 24 + 4) == EALIGN
    assert g(y=A + 2 ** 26 + 4) == EALIGN
    assert g(asc=B + 2) == EALIGN
    assert g(ws=B + 2 ** 20 + 8) == EALIGN
    assert g(wsb=ws - 1) == ENOSPC
    assert g(R=0, a=None, asc=None, off=None, w=None, wsc=None, y=None, ws=None) == OK


def test_harness_validation():
    h = lambda **kw: lib.moe_harness_expert_scale(
        kw.get("disp", A), kw.get("sc", B), kw.get("rs", B + 4096), kw.get("idx", B + 8192),
        kw.get("off", B + 16384), kw.get("R", 100), kw.get("H", 256), kw.get("E", 8),
        kw.get("dt", 0), 0, kw.get("eo", A + 2 ** 20), None)
    assert h(H=100) == EINVAL
    assert h(dt=1, H=64) == EINVAL
    assert h(E=0) == EINVAL
    assert h(dt=3) == EINVAL
    assert h(off=None) == ENULL
    assert h(dt=1, sc=None) == ENULL
    assert h(disp=A + 4) == EALIGN


def test_binding_fails_loudly_without_library(tmp_path):
    """Any use of the API without the HIP library raises ImportError (no CPU
    fallback); the build module itself imports without it."""
    import subprocess
    import sys
    code = ("import os; os.environ['MOE_ROUTE_LIB']=%r\n"
            "import combine_moe_route_amd.build\n"
            "try:\n from combine_moe_route_amd import moe_dispatch\n"
            "except ImportError as e:\n print('IMPORTERROR', e)\n"
            % str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "IMPORTERROR" in r.stdout and "libmoeroute.so not found" in r.stdout, r.stderr
