"""The C ABI library: it loads, exports every entry point include/smla.h
declares, and rejects bad arguments before launching anything (no GPU needed:
argument checks run before the device is touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")


@pytest.fixture(scope="module")
def lib():
    from bwd_sparse_mla_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsmla.so is not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_pages_calls():
    names = declared_functions()
    assert "smla_fwd" in names and "smla_bwd" in names


def test_every_declared_symbol_is_exported(lib):
    from bwd_sparse_mla_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def test_version_and_workspace_queries(lib):
    assert lib.smla_version() == 1
    fwd = lib.smla_fwd_workspace_size(4096, 4096, 8, 2048)
    bwd = lib.smla_bwd_workspace_size(4096, 4096, 8, 2048, 0)
    assert 0 < fwd < bwd
    assert lib.smla_fwd_workspace_size(4096, 4096, 12, 2048) == 0     # unsupported heads
    assert lib.smla_fwd_workspace_size(4096, 4096, 256, 2048) == 0
    # 128 heads run as 64-head groups over two half-token rows per token
    assert lib.smla_fwd_workspace_size(300, 900, 128, 64) == lib.smla_fwd_workspace_size(600, 900, 64, 64) > 0
    for flags in (0, 2, 8):
        assert (lib.smla_bwd_workspace_size(300, 900, 128, 64, flags)
                == lib.smla_bwd_workspace_size(600, 900, 64, 64, flags) > 0)
    assert lib.smla_fwd_workspace_size(4096, 4096, 8, 0) == 0         # topk < 1
    assert lib.smla_bwd_workspace_size(16, 1 << 24, 8, 8, 0) == 0     # s_kv too large


def test_kv_group_workspace_queries(lib):
    # (token, kv group) pairs are rows of heads / G heads over s_kv * G flat kv rows;
    # below 64 heads per group the workspace also leads with a group-major copy of
    # lse (4 bytes per row)
    a256 = lambda x: (x + 255) // 256 * 256
    rows = 300 * 16
    stage = a256(rows * 4)
    assert (lib.smla_fwd_workspace_size_g(300, 900, 16, 2, 64)
            == lib.smla_fwd_workspace_size(600, 1800, 8, 64) + stage)
    assert (lib.smla_bwd_workspace_size_g(300, 900, 16, 2, 64, 8)
            == lib.smla_bwd_workspace_size(600, 1800, 8, 64, 8) + stage)
    assert lib.smla_fwd_workspace_size_g(300, 900, 8, 1, 64) == lib.smla_fwd_workspace_size(300, 900, 8, 64)
    for flags in (0, 2, 8):
        assert (lib.smla_bwd_workspace_size_g(100, 500, 256, 2, 64, flags)
                == lib.smla_bwd_workspace_size(200, 1000, 128, 64, flags) > 0)
    assert lib.smla_fwd_workspace_size_g(16, 16, 24, 2, 8) == 0          # 12 heads per group
    assert lib.smla_fwd_workspace_size_g(16, 16, 17, 2, 8) == 0          # heads not a multiple of G
    assert lib.smla_fwd_workspace_size_g(16, 16, 16, 0, 8) == 0          # G < 1
    assert lib.smla_fwd_workspace_size_g(16, 16, 8 * 65, 65, 8) == 0     # G > 64
    assert lib.smla_bwd_workspace_size_g(16, 1 << 21, 64, 8, 8, 0) == 0  # s_kv * G >= 2^24


FAKE = 0x100000  # 16-byte aligned, never dereferenced: the checks return first


def call_fwd(lib, q=FAKE, kv=FAKE, idx=FAKE, s_q=16, s_kv=16, heads=8, topk=4, out=FAKE,
             lse=FAKE, ws=FAKE, ws_bytes=None):
    P = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = lib.smla_fwd_workspace_size(s_q, s_kv, heads, topk) or 1
    return lib.smla_fwd(P(q), P(kv), P(idx), s_q, s_kv, heads, topk, 0.1, P(out), P(lse), P(ws),
                        ws_bytes, P(0))


def test_fwd_argument_errors(lib):
    from bwd_sparse_mla_amd import _lib
    assert call_fwd(lib, heads=12) == 2
    assert call_fwd(lib, topk=0) == 2
    assert call_fwd(lib, s_kv=0) == 2
    assert call_fwd(lib, s_q=-1) == 2
    assert call_fwd(lib, q=0) == 1
    assert call_fwd(lib, kv=0, s_q=0) == 1
    assert call_fwd(lib, lse=0) == 1
    assert call_fwd(lib, kv=FAKE + 2) == 3
    assert call_fwd(lib, ws=FAKE + 16) == 3
    assert call_fwd(lib, ws_bytes=10) == 4
    assert call_fwd(lib, ws=0) == 4
    assert b"workspace" in lib.smla_last_error()
    with pytest.raises(_lib.SmlaError):
        _lib.check(call_fwd(lib, heads=12))


def call_bwd(lib, flags=0, dkv=FAKE, dkv32=FAKE, dq=FAKE, heads=8, ws_bytes=None):
    P = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = lib.smla_bwd_workspace_size(16, 16, heads, 4, flags) or 1
    return lib.smla_bwd(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 16, 16, heads, 4,
                        0.1, P(dq), P(dkv), P(dkv32), flags, P(FAKE), ws_bytes, P(0))


def test_bwd_argument_errors(lib):
    assert call_bwd(lib, heads=7) == 2
    assert call_bwd(lib, dq=0) == 1
    assert call_bwd(lib, dkv=0, dkv32=0) == 1
    assert call_bwd(lib, flags=32) == 5
    assert call_bwd(lib, flags=1, dkv32=0) == 5
    assert call_bwd(lib, dkv32=FAKE + 4) == 3
    assert call_bwd(lib, ws_bytes=64) == 4
    # the atomic dkv mode needs its fp32 accumulator: a workspace sized for
    # the deterministic mode is too small for it
    det = lib.smla_bwd_workspace_size(16, 16, 8, 4, 0)
    atom = lib.smla_bwd_workspace_size(16, 16, 8, 4, 2)
    assert atom >= det + 64 * 576 * 4
    assert call_bwd(lib, flags=2, ws_bytes=det) == 4
    # the stored-P backward keeps P and dS of every union slot: 256 bytes per
    # (token, slot) bound on top of the plan
    stored = lib.smla_bwd_workspace_size(16, 16, 8, 4, 8)
    assert stored >= det + 16 * 4 * 256
    assert call_bwd(lib, flags=8, ws_bytes=det) == 4


def test_validate_argument_errors(lib):
    P = ctypes.c_void_p
    assert lib.smla_validate_indices(P(FAKE), 4, 4, 4, P(0), P(0)) == 1
    assert lib.smla_validate_indices(P(FAKE), 4, 0, 4, P(FAKE), P(0)) == 2
    assert lib.smla_validate_indices(P(FAKE), 4, 4, 4, P(FAKE + 4), P(0)) == 3


def test_no_cpu_fallback_in_product_package():
    """The product package never imports the oracle or computes on the CPU."""
    pkg = os.path.join(ROOT, "bwd_sparse_mla_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            text = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in text.replace("never imports the oracle", ""), fn


def test_plan_and_fwd_ex_argument_errors(lib):
    P = ctypes.c_void_p
    bws = lib.smla_bwd_workspace_size(16, 16, 8, 4, 0)
    fws = lib.smla_fwd_workspace_size(16, 16, 8, 4)
    assert bws > fws > 0
    assert lib.smla_plan(P(FAKE), 16, 16, 12, 4, P(FAKE), bws, P(0)) == 2      # heads
    assert lib.smla_plan(P(0), 16, 16, 8, 4, P(FAKE), bws, P(0)) == 1          # indices
    assert lib.smla_plan(P(FAKE), 16, 16, 8, 4, P(FAKE), fws, P(0)) == 4       # needs the bwd size
    assert lib.smla_plan(P(FAKE), 16, 16, 8, 4, P(FAKE + 16), bws, P(0)) == 3  # 256-byte alignment
    args = (P(FAKE), P(FAKE), P(FAKE), 16, 16, 8, 4, 0.1, P(FAKE), P(FAKE))
    assert lib.smla_fwd_ex(*args, 8, P(FAKE), fws, P(0)) == 5                  # unknown flag
    assert lib.smla_fwd_ex(*args, 4, P(FAKE), 64, P(0)) == 4                   # workspace
    assert call_bwd(lib, flags=16) == 5


def test_kv_group_call_argument_errors(lib):
    P = ctypes.c_void_p
    fws = lib.smla_fwd_workspace_size_g(16, 16, 16, 2, 4)
    bws = lib.smla_bwd_workspace_size_g(16, 16, 16, 2, 4, 0)
    assert bws > fws > 0
    assert lib.smla_plan_g(P(FAKE), 16, 16, 16, 3, 4, P(FAKE), bws, P(0)) == 2    # 16 % 3
    assert lib.smla_plan_g(P(FAKE), 16, 16, 16, 2, 4, P(FAKE), fws, P(0)) == 4    # workspace
    fargs = (P(FAKE), P(FAKE), P(FAKE), 16, 16)
    tail = (0.1, P(FAKE), P(FAKE), 0, P(FAKE), fws, P(0))
    assert lib.smla_fwd_g(*fargs, 16, 0, 4, *tail) == 2                          # G < 1
    assert lib.smla_fwd_g(*fargs, 48, 2, 4, *tail) == 2                          # 24 per group
    assert lib.smla_fwd_g(P(0), P(FAKE), P(FAKE), 16, 16, 16, 2, 4, *tail) == 1   # q
    assert lib.smla_fwd_g(*fargs, 16, 2, 4, 0.1, P(FAKE), P(FAKE), 0, P(FAKE), fws - 1,
                          P(0)) == 4
    bargs = (P(FAKE),) * 6 + (16, 16)
    btail = (0.1, P(FAKE), P(FAKE), P(0), 0, P(FAKE), bws, P(0))
    assert lib.smla_bwd_g(*bargs, 16, 5, 4, *btail) == 2                          # 16 % 5
    assert lib.smla_bwd_g(*bargs, 16, 2, 4, 0.1, P(FAKE), P(FAKE), P(0), 64, P(FAKE), bws,
                          P(0)) == 5                                               # unknown flag
    assert lib.smla_bwd_g(*bargs, 16, 2, 4, 0.1, P(FAKE), P(FAKE), P(0), 0, P(FAKE), bws - 1,
                          P(0)) == 4


def test_fp8_forward_argument_errors(lib):
    P = ctypes.c_void_p
    fws = lib.smla_fwd_workspace_size_g(16, 16, 8, 1, 4)
    tail = (0.1, P(FAKE), P(FAKE), 0, P(FAKE), fws, P(0))
    assert lib.smla_fwd_fp8(P(FAKE), P(0), P(FAKE), 16, 16, 8, 1, 4, *tail) == 1       # kv_fp8
    assert lib.smla_fwd_fp8(P(FAKE), P(FAKE), P(FAKE), 16, 16, 12, 1, 4, *tail) == 2   # heads
    assert lib.smla_fwd_fp8(P(FAKE), P(FAKE + 8), P(FAKE), 16, 16, 8, 1, 4, *tail) == 3
    assert lib.smla_fwd_fp8(P(FAKE), P(FAKE), P(FAKE), 16, 16, 8, 1, 4, 0.1, P(FAKE), P(FAKE),
                            0, P(FAKE), fws - 1, P(0)) == 4
    # SMLA_FP8_POW2_SCALES (16) is known to the fp8 forward only
    assert lib.smla_fwd_fp8(P(FAKE), P(FAKE), P(FAKE), 16, 16, 8, 1, 4, 0.1, P(FAKE), P(FAKE),
                            16, P(FAKE), fws - 1, P(0)) == 4
    assert lib.smla_fwd_fp8(P(FAKE), P(FAKE), P(FAKE), 16, 16, 8, 1, 4, 0.1, P(FAKE), P(FAKE),
                            32, P(FAKE), fws, P(0)) == 5
    assert lib.smla_fwd_g(P(FAKE), P(FAKE), P(FAKE), 16, 16, 8, 1, 4, 0.1, P(FAKE), P(FAKE),
                          16, P(FAKE), fws, P(0)) == 5


def test_nonfinite_argument_errors(lib):
    P = ctypes.c_void_p
    cnt = P(FAKE)
    assert lib.smla_nonfinite_count(P(FAKE), 2, 8, cnt, P(0)) == 2              # unknown dtype
    assert lib.smla_nonfinite_count(P(FAKE), 0, -1, cnt, P(0)) == 2             # negative size
    assert lib.smla_nonfinite_count(P(FAKE), 0, 8, P(0), P(0)) == 1             # null counter
    assert lib.smla_nonfinite_count(P(0), 1, 8, cnt, P(0)) == 1                 # null buffer
    assert lib.smla_nonfinite_count(P(FAKE + 8), 1, 8, cnt, P(0)) == 3          # 16-byte alignment
    assert lib.smla_nonfinite_count(P(FAKE), 1, 8, P(FAKE + 4), P(0)) == 3      # counter alignment
    assert lib.smla_nonfinite_replace(P(FAKE), P(FAKE + 8), 0, 8, cnt, P(0)) == 3
    # a reference that overlaps the buffer (other than the buffer itself) is refused
    assert lib.smla_nonfinite_replace(P(FAKE), P(FAKE + 16), 1, 64, cnt, P(0)) == 2
    assert b"overlaps" in lib.smla_last_error()


def test_fwd_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """smla_fwd_noalloc has a fixed per-device scratch buffer: a shape whose
    forward workspace exceeds it is refused before anything is launched (no
    GPU needed to see the refusal)."""
    from bwd_sparse_mla_amd import _lib
    cap = _lib.SMLA_NOALLOC_SCRATCH_BYTES
    assert lib.smla_fwd_workspace_size(4096, 4096, 8, 2048) <= cap      # the packed ragged batch fits
    assert lib.smla_fwd_workspace_size(8192, 8192, 16, 2048) > cap      # the recency workload does not
    P = ctypes.c_void_p
    st = lib.smla_fwd_noalloc(P(16), P(16), P(16), 8192, 8192, 16, 2048, 0.1, P(16), P(16), None)
    assert _lib.STATUS_NAMES[st] == "SMLA_ERR_WORKSPACE"
    msg = lib.smla_last_error().decode()
    assert "smla_fwd_noalloc" in msg and str(cap) in msg
    st = lib.smla_fwd_noalloc(P(16), P(16), P(16), 64, 64, 12, 64, 0.1, P(16), P(16), None)
    assert _lib.STATUS_NAMES[st] == "SMLA_ERR_SHAPE"      # unsupported head count
