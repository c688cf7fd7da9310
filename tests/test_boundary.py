"""Host-side checks of the C ABI library (CPU only: no kernel is launched).

Every rejected call returns its status before any HIP call, so these run on a
machine without a GPU.  Pointers passed here are never dereferenced.
"""

import ctypes
import os
import re

import pytest

import chunked_gated_delta_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails a host check


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(kda.exported_symbols)


def test_import_fails_loudly_without_the_library(tmp_path):
    """The binding has no fallback: a package copy without libkda.so refuses to import."""
    import shutil
    import subprocess
    import sys

    pkg = tmp_path / "chunked_gated_delta_amd"
    pkg.mkdir()
    src = os.path.join(ROOT, "chunked_gated_delta_amd")
    for name in os.listdir(src):
        if name.endswith(".py"):
            shutil.copy(os.path.join(src, name), pkg)
    r = subprocess.run([sys.executable, "-c", "import chunked_gated_delta_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "libkda.so is missing" in r.stderr


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kda.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_exports_are_c_abi():
    # extern "C": unmangled names in the dynamic symbol table
    import subprocess
    syms = subprocess.run(["nm", "-D", "--defined-only", kda.library_path], capture_output=True,
                          text=True, check=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", syms, re.M), name


def test_workspace_size():
    assert kda.kda_workspace_size(200, 2, 1) > 0
    assert kda.kda_workspace_size(32768, 96, 1) >= 256
    assert kda.kda_workspace_size(65536, 32, 16) >= kda.kda_workspace_size(65536, 32, 1)
    assert kda.kda_workspace_size(0, 2, 1) > 0          # an empty batch is legal
    assert kda.kda_workspace_size(10, 0, 1) == 0
    assert kda.kda_workspace_size(10, 2, 0) == 0
    # room for a processing order of all N sequences
    assert kda.kda_workspace_size(10 ** 6, 1, 10 ** 5) >= 4 * 10 ** 5
    # a long sequence with few heads runs on shards: room for their P, R, entering and
    # final states (16 shards x 8 heads x 4 x 64 KiB) beyond the chunk records
    records = (262144 // 64 + 1) * 8 * 90624
    assert kda.kda_workspace_size(262144, 8, 1) >= records + 16 * 8 * 4 * 65536


def test_is_supported():
    assert kda.kda_is_supported(128, 128, -5.0)
    assert kda.kda_is_supported(128, 128, 0.0)
    assert kda.kda_is_supported(128, 128, -2.5)
    for K, V in ((64, 64), (64, 128), (128, 64)):
        assert kda.kda_is_supported(K, V, -5.0)
    for K, V in ((128, 256), (256, 256), (32, 32), (96, 128), (128, 0), (0, 128)):
        assert not kda.kda_is_supported(K, V, -5.0)
    assert not kda.kda_is_supported(128, 128, -5.5)
    assert not kda.kda_is_supported(128, 128, 0.5)


def call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, scale=0.088, out=FAKE, ws=FAKE,
             ws_bytes=1 << 20, A_log=FAKE, dt=FAKE, lb=-5.0, init=None, fin=None, cu=None,
             B=1, T=200, H=2, K=128, V=128, N=1, stream=None)
    a.update(over)
    return kda.raw_call(a["q"], a["k"], a["v"], a["g"], a["b"], ctypes.c_float(a["scale"]),
                        a["out"], a["ws"], ctypes.c_size_t(a["ws_bytes"]), a["A_log"], a["dt"],
                        ctypes.c_float(a["lb"]), a["init"], a["fin"], a["cu"], a["B"], a["T"],
                        a["H"], a["K"], a["V"], a["N"], a["stream"])


INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "b", "out", "A_log", "dt"])
def test_null_required_pointer_is_invalid(field):
    assert call(**{field: None}) == INVALID


@pytest.mark.parametrize("over", [dict(B=0), dict(T=-1), dict(H=0), dict(N=0), dict(N=2),
                                  dict(B=2, N=2, cu=FAKE), dict(scale=float("nan"))])
def test_bad_sizes_are_invalid(over):
    assert call(**over) == INVALID


@pytest.mark.parametrize("over", [dict(K=32), dict(V=96), dict(K=256, V=256), dict(lb=-6.0),
                                  dict(lb=1.0)])
def test_unsupported_shapes(over):
    assert call(**over) == UNSUPPORTED


def test_workspace_checks():
    need = kda.kda_workspace_size(200, 2, 1)
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws_bytes=0) == WORKSPACE


def test_status_strings():
    lib = ctypes.CDLL(kda.library_path)
    lib.kda_status_string.restype = ctypes.c_char_p
    for code, name in kda.STATUS.items():
        assert lib.kda_status_string(code).decode() == name


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    v = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda.kda_fwd(x, x, v, x, torch.zeros(1, 4, 1, dtype=torch.bfloat16), 1.0, v.clone(),
                    torch.zeros(512, dtype=torch.uint8), torch.zeros(1), torch.zeros(1, 128), -5.0)


def shard_affine_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, ws=FAKE, ws_bytes=1 << 40, A_log=FAKE, dt=FAKE,
             lb=-5.0, P=FAKE, R=FAKE, cu=None, B=1, T=64, H=2, K=128, V=128, N=1)
    a.update(over)
    return kda._lib.kda_shard_affine(a["q"], a["k"], a["v"], a["g"], a["b"], a["ws"], a["ws_bytes"],
                                     a["A_log"], a["dt"], ctypes.c_float(a["lb"]), a["P"], a["R"], a["cu"],
                                     a["B"], a["T"], a["H"], a["K"], a["V"], a["N"], None)


def shard_scan_call(**over):
    a = dict(P=FAKE, R=FAKE, init=None, starts=FAKE, fin=None, n=2, H=2, K=128, V=128)
    a.update(over)
    return kda._lib.kda_shard_scan(a["P"], a["R"], a["init"], a["starts"], a["fin"], a["n"], a["H"],
                                   a["K"], a["V"], None)


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "b", "A_log", "dt", "P", "R"])
def test_shard_affine_null_pointer_is_invalid(field):
    assert shard_affine_call(**{field: None}) == INVALID


def test_shard_affine_checks():
    assert shard_affine_call(K=64, V=64) == UNSUPPORTED     # the forward's other head dims: not here
    assert shard_affine_call(K=128, V=64) == UNSUPPORTED
    assert shard_affine_call(lb=-6.0) == UNSUPPORTED
    assert shard_affine_call(B=2, N=1) == INVALID
    assert shard_affine_call(ws_bytes=16) == WORKSPACE
    assert shard_affine_call(ws=None) == WORKSPACE


def test_shard_scan_checks():
    for field in ("P", "R", "starts"):
        assert shard_scan_call(**{field: None}) == INVALID
    assert shard_scan_call(n=0) == INVALID
    assert shard_scan_call(H=0) == INVALID
    assert shard_scan_call(K=64) == UNSUPPORTED
    assert shard_scan_call(V=96) == UNSUPPORTED


def decode_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt=FAKE, lb=-5.0,
             init=None, fin=None, B=2, T=1, H=2, K=128, V=128)
    a.update(over)
    return kda._lib.kda_decode(a["q"], a["k"], a["v"], a["g"], a["b"], ctypes.c_float(a["scale"]), a["out"],
                               a["A_log"], a["dt"], ctypes.c_float(a["lb"]), a["init"], a["fin"], a["B"],
                               a["T"], a["H"], a["K"], a["V"], None)


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "b", "out", "A_log", "dt"])
def test_decode_null_pointer_is_invalid(field):
    assert decode_call(**{field: None}) == INVALID


def test_decode_checks():
    assert decode_call(B=0) == INVALID
    assert decode_call(H=0) == INVALID
    assert decode_call(T=-1) == INVALID
    assert decode_call(scale=float("nan")) == INVALID
    assert decode_call(K=32, V=32) == UNSUPPORTED
    assert decode_call(K=128, V=256) == UNSUPPORTED
    assert decode_call(lb=0.5) == UNSUPPORTED


def fwd_ex_call(flags, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, scale=0.088, out=FAKE, ws=FAKE, ws_bytes=1 << 40,
             A_log=FAKE, dt=FAKE, lb=-5.0, init=None, fin=None, cu=None, B=1, T=64, H=2, K=128, V=128, N=1)
    a.update(over)
    return kda._lib.kda_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["b"], ctypes.c_float(a["scale"]), a["out"],
                               a["ws"], a["ws_bytes"], a["A_log"], a["dt"], ctypes.c_float(a["lb"]), a["init"],
                               a["fin"], a["cu"], a["B"], a["T"], a["H"], a["K"], a["V"], a["N"], flags, None)


def test_fwd_ex_flag_checks():
    assert fwd_ex_call(128) == INVALID                    # unknown bit
    assert fwd_ex_call(1 << 31) == INVALID
    # the single-launch schedule is a known bit (ignored where the call does not qualify)
    assert fwd_ex_call(kda.FLAG_SINGLE_LAUNCH, ws_bytes=8) == WORKSPACE
    # keeping the records is a known bit
    assert fwd_ex_call(kda.FLAG_KEEP_RECORDS, ws_bytes=8) == WORKSPACE
    # reusing the workspace's records is a known bit: the call proceeds to the workspace check
    assert fwd_ex_call(kda.FLAG_REUSE_RECORDS, ws_bytes=8) == WORKSPACE
    assert fwd_ex_call(0, A_log=None) == INVALID          # gate parameters needed without GATE_GIVEN
    assert fwd_ex_call(kda.FLAG_BETA_GIVEN, dt=None) == INVALID
    assert fwd_ex_call(kda.FLAG_GATE_GIVEN, K=256, V=256, A_log=None, dt=None) == UNSUPPORTED
    assert fwd_ex_call(kda.FLAG_STATE_VK, ws_bytes=8) == WORKSPACE


def bwd_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, scale=0.088, dout=FAKE, dfin=None, dq=FAKE, dk=FAKE,
             dv=FAKE, dg=FAKE, db=FAKE, dA=FAKE, ddt=FAKE, dinit=None, ws=FAKE, ws_bytes=1 << 40, A_log=FAKE,
             dt=FAKE, lb=-5.0, init=None, cu=None, B=1, T=64, H=2, K=128, V=128, N=1)
    a.update(over)
    return kda._lib.kda_bwd(a["q"], a["k"], a["v"], a["g"], a["b"], ctypes.c_float(a["scale"]), a["dout"],
                            a["dfin"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dA"], a["ddt"], a["dinit"],
                            a["ws"], a["ws_bytes"], a["A_log"], a["dt"], ctypes.c_float(a["lb"]), a["init"],
                            a["cu"], a["B"], a["T"], a["H"], a["K"], a["V"], a["N"], None)


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "b", "dout", "dq", "dk", "dv", "dg", "db", "dA", "ddt",
                                   "A_log", "dt"])
def test_bwd_null_pointer_is_invalid(field):
    assert bwd_call(**{field: None}) == INVALID


def test_bwd_checks():
    assert bwd_call(B=0) == INVALID
    assert bwd_call(T=-1) == INVALID
    assert bwd_call(scale=float("nan")) == INVALID
    assert bwd_call(B=2, N=1) == INVALID                    # N must equal B without cu_seqlens
    assert bwd_call(K=32, V=32) == UNSUPPORTED              # head dims 64 and 128 only
    assert bwd_call(K=128, V=256) == UNSUPPORTED
    assert bwd_call(K=64, V=64, ws_bytes=8) == WORKSPACE     # 64: on to the workspace check
    assert bwd_call(K=64, V=128, ws_bytes=8) == WORKSPACE
    assert bwd_call(lb=-6.0) == UNSUPPORTED
    assert bwd_call(ws=None) == WORKSPACE
    need = kda.kda_bwd_workspace_size(64, 2, 1)
    assert bwd_call(ws_bytes=need - 1) == WORKSPACE
    assert need > kda.kda_workspace_size(64, 2, 1)


def test_bwd_workspace_size():
    assert kda.kda_bwd_workspace_size(0, 2, 1) > 0
    assert kda.kda_bwd_workspace_size(10, 0, 1) == 0
    assert kda.kda_bwd_workspace_size(10, 2, 0) == 0
    assert kda.kda_bwd_workspace_size(32768, 96, 1) > 20 * 10 ** 9 // 2


def bwd_ex_call(flags, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, scale=0.088, dout=FAKE, dfin=None, dq=FAKE, dk=FAKE,
             dv=FAKE, dg=FAKE, db=FAKE, dA=FAKE, ddt=FAKE, dinit=None, ws=FAKE, ws_bytes=8, A_log=FAKE,
             dt=FAKE, lb=-5.0, init=None, cu=None, B=1, T=64, H=2, K=128, V=128, N=1)
    a.update(over)
    return kda._lib.kda_bwd_ex(a["q"], a["k"], a["v"], a["g"], a["b"], ctypes.c_float(a["scale"]), a["dout"],
                               a["dfin"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dA"], a["ddt"],
                               a["dinit"], a["ws"], a["ws_bytes"], a["A_log"], a["dt"], ctypes.c_float(a["lb"]),
                               a["init"], a["cu"], a["B"], a["T"], a["H"], a["K"], a["V"], a["N"], flags, None)


def test_bwd_ex_flag_checks():
    assert bwd_ex_call(32) == INVALID                       # unknown bit (KEEP_RECORDS is forward-only)
    assert bwd_ex_call(64) == INVALID                       # so is SINGLE_LAUNCH
    assert bwd_ex_call(kda.FLAG_REUSE_RECORDS) == WORKSPACE  # a known bit: on to the workspace check
    assert bwd_ex_call(0, A_log=None) == INVALID            # gate parameters needed without GATE_GIVEN
    assert bwd_ex_call(0, dA=None) == INVALID
    # with the gate given they may be absent: the call then proceeds to the workspace check
    assert bwd_ex_call(kda.FLAG_GATE_GIVEN, A_log=None, dt=None, dA=None, ddt=None) == WORKSPACE
    assert bwd_ex_call(kda.FLAG_STATE_VK | kda.FLAG_NO_QK_NORM) == WORKSPACE


def test_fault_word_query_rejects_null_arguments():
    lib = ctypes.CDLL(kda.library_path)
    lib.kda_workspace_faults.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32), ctypes.c_void_p]
    word = ctypes.c_uint32(7)
    assert lib.kda_workspace_faults(None, ctypes.byref(word), None) == 1
    assert lib.kda_workspace_faults(FAKE, None, None) == 1
    assert word.value == 7  # untouched on rejection
    assert (kda.FAULT_WAIT_TIMEOUT, kda.FAULT_GATE_RANGE, kda.FAULT_QK_NORM, kda.FAULT_PLACEMENT) == (1, 2, 4, 8)


def test_workspace_sizes_grow_with_the_batch():
    """A size bought for an upper bound on the sequence count serves every smaller
    batch over the same tokens: the shard area of a call that splits (few chains)
    can exceed what more sequences need, so the reported size takes the maximum."""
    for T, H in ((65536, 1), (262144, 8), (20000, 2), (4096, 12)):
        fw = [kda.kda_workspace_size(T, H, n) for n in range(1, 41)]
        bw = [kda.kda_bwd_workspace_size(T, H, n) for n in range(1, 41)]
        assert all(a <= b for a, b in zip(fw, fw[1:])), (T, H, fw)
        assert all(a <= b for a, b in zip(bw, bw[1:])), (T, H, bw)


def test_noalloc_refuses_bad_and_oversized_calls_on_the_host():
    lib = ctypes.CDLL(kda.library_path)
    P, I64, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    lib.kda_fwd_noalloc.argtypes = [P, P, P, P, P, F, P, P, P, F, P, P, P, I64, I64, I64, I64, I64, I64, P]

    def call(B, T, H, N):
        return lib.kda_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, FAKE, -5.0, None, None, None,
                                   B, T, H, 128, 128, N, None)

    assert call(0, 64, 2, 1) == 1           # INVALID
    assert call(1, 64, 0, 1) == 1
    assert call(1, 32768, 96, 1) == 3       # WORKSPACE: 4.4 GB of records do not fit the scratch
    assert call(1, 1 << 20, 2, 1) == 3
    assert kda.NOALLOC_SCRATCH_BYTES == 160 << 20
