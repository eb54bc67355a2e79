"""The C ABI without a GPU: the library loads, exports every function the public header
declares, and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_06_amd as muir

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "muir.h")

# Fake, 256-byte aligned, non-overlapping "device" addresses. They are only ever
# passed in calls that fail validation, so nothing dereferences them.
BASE = 1 << 40
STRIDE = 1 << 32


def fake(i):
    return ctypes.c_void_p(BASE + i * STRIDE)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muir_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("muir_chunk_fwd", "muir_chunk_fwd_workspace_size", "muir_decode_step",
                     "muir_status_string", "muir_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = muir.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings():
    for code, name in muir.STATUS.items():
        assert muir.status_string(code) == name
    assert muir.status_string(99) == "MUIR_STATUS_UNKNOWN"
    assert muir.version() >= 10000


def test_workspace_size():
    ws = muir.chunk_fwd_workspace_size
    a = ws(2, 1000, 3, 64, 64, 64, muir.MUIR_BF16)
    b = ws(2, 1024, 3, 64, 64, 64, muir.MUIR_BF16)
    assert a == b > 0                      # ceil(T / chunk) slots
    assert ws(2, 1025, 3, 64, 64, 64, muir.MUIR_BF16) > b
    assert ws(1, 64, 1, 64, 64, 64, muir.MUIR_F32) > ws(1, 64, 1, 64, 64, 64, muir.MUIR_BF16)
    assert ws(1, 0, 1, 64, 64, 64, muir.MUIR_BF16) == 0
    for bad in [(0, 64, 1, 64, 64, 64), (1, 64, 1, 64, 128, 64), (1, 64, 1, 32, 32, 64),
                (1, 64, 1, 64, 64, 32), (1, -1, 1, 64, 64, 64)]:
        assert ws(*bad, muir.MUIR_BF16) == 0
    assert ws(1, 64, 1, 64, 64, 64, 7) == 0


def _chunk_call(**over):
    lib = muir.lib()
    args = dict(q=fake(0), k=fake(1), v=fake(2), a=fake(3), g=fake(4), e=fake(5), w=fake(6),
                r=fake(7), s0=fake(8), o=fake(9), s_out=fake(10), B=2, T=100, H=3, dk=64,
                dv=64, chunk=64, qkv=muir.MUIR_BF16, ws=fake(11),
                wsb=muir.chunk_fwd_workspace_size(2, 100, 3, 64, 64, 64, muir.MUIR_BF16),
                stream=None)
    args.update(over)
    st = lib.muir_chunk_fwd(args["q"], args["k"], args["v"], args["a"], args["g"], args["e"],
                            args["w"], args["r"], args["s0"], args["o"], args["s_out"],
                            args["B"], args["T"], args["H"], args["dk"], args["dv"],
                            args["chunk"], args["qkv"], args["ws"], args["wsb"], args["stream"])
    return st, muir.last_error()


@pytest.mark.parametrize("over,status", [
    (dict(B=0), 2), (dict(T=-1), 2), (dict(H=0), 2), (dict(dk=0), 2),
    (dict(dk=64, dv=128), 3), (dict(dk=32, dv=32), 3), (dict(chunk=32), 3),
    (dict(qkv=5), 3),
    (dict(q=None), 1), (dict(a=None), 1), (dict(o=None), 1), (dict(r=None), 1),
    (dict(ws=None), 4), (dict(wsb=1024), 4), (dict(ws=ctypes.c_void_p(BASE + 11 * STRIDE + 16)), 4),
    (dict(q=ctypes.c_void_p(BASE + 8)), 2),
    (dict(o=fake(2)), 5), (dict(s_out=fake(3)), 5),
    (dict(o=ctypes.c_void_p(BASE + 2 * STRIDE + 4096)), 5),
    (dict(s_out=ctypes.c_void_p(BASE + 8 * STRIDE + 256)), 5),
    (dict(o=fake(10)), 5), (dict(ws=fake(9)), 5),
])
def test_chunk_fwd_rejects_bad_arguments(over, status):
    st, msg = _chunk_call(**over)
    assert st == status, msg
    assert msg


def _gated_call(**over):
    lib = muir.lib()
    args = dict(q=fake(0), k=fake(1), v=fake(2), a=fake(3), g=fake(4), e=fake(5), w=fake(6),
                og=fake(12), r=fake(7), s0=fake(8), o=fake(9), s_out=fake(10), B=2, T=100, H=3,
                dk=64, dv=64, chunk=64, qkv=muir.MUIR_BF16, ws=fake(11),
                wsb=muir.chunk_fwd_workspace_size(2, 100, 3, 64, 64, 64, muir.MUIR_BF16),
                stream=None)
    args.update(over)
    st = lib.muir_chunk_fwd_gated(args["q"], args["k"], args["v"], args["a"], args["g"],
                                  args["e"], args["w"], args["og"], args["r"], args["s0"],
                                  args["o"], args["s_out"], args["B"], args["T"], args["H"],
                                  args["dk"], args["dv"], args["chunk"], args["qkv"], args["ws"],
                                  args["wsb"], args["stream"])
    return st, muir.last_error()


@pytest.mark.parametrize("over,status", [
    (dict(og=None), 1), (dict(og=ctypes.c_void_p(BASE + 12 * STRIDE + 8)), 2),
    (dict(o=fake(12)), 5), (dict(ws=fake(12)), 5), (dict(s_out=fake(12)), 5),
    (dict(chunk=48), 3), (dict(q=None), 1),
])
def test_chunk_fwd_gated_rejects_bad_arguments(over, status):
    st, msg = _gated_call(**over)
    assert st == status, msg
    assert msg


def _bwd_call(**over):
    lib = muir.lib()
    names = ["q", "k", "v", "a", "g", "e", "w", "r", "s0", "dout", "ds_out",
             "dq", "dk", "dv", "dla", "dg", "de", "dw", "dr", "ds0"]
    args = {n: fake(12 + i) for i, n in enumerate(names)}
    # Sizes are DK and DV here: dk and dv name gradient buffers.
    args.update(B=2, T=100, H=3, DK=64, DV=64, chunk=64, qkv=muir.MUIR_BF16, ws=fake(40),
                wsb=muir.chunk_bwd_workspace_size(2, 100, 3, 64, 64, 64, muir.MUIR_BF16),
                stream=None)
    args.update(over)
    st = lib.muir_chunk_bwd(*[args[n] for n in names], args["B"], args["T"], args["H"],
                            args["DK"], args["DV"], args["chunk"], args["qkv"], args["ws"],
                            args["wsb"], args["stream"])
    return st, muir.last_error()


def test_chunk_bwd_workspace_size():
    ws = muir.chunk_bwd_workspace_size
    assert ws(2, 100, 3, 64, 64, 64, muir.MUIR_BF16) > 0
    assert ws(2, 100, 3, 64, 64, 64, muir.MUIR_F32) > ws(2, 100, 3, 64, 64, 64, muir.MUIR_BF16)
    assert ws(2, 0, 3, 64, 64, 64, muir.MUIR_BF16) > 0  # the final-state adjoint still needs room
    for bad in [(2, 100, 3, 64, 64, 128), (2, 100, 3, 32, 32, 64), (2, 100, 3, 64, 128, 64),
                (0, 100, 3, 64, 64, 64), (2, -1, 3, 64, 64, 64)]:
        assert ws(*bad, muir.MUIR_BF16) == 0


@pytest.mark.parametrize("over,status", [
    (dict(B=0), 2), (dict(T=-1), 2), (dict(H=0), 2),
    (dict(chunk=128), 3), (dict(DK=32, DV=32), 3), (dict(DK=64, DV=128), 3), (dict(qkv=5), 3),
    (dict(q=None), 1), (dict(dout=None), 1), (dict(dq=None), 1), (dict(dla=None), 1),
    (dict(r=None), 1), (dict(dr=None), 1),
    (dict(ws=None), 4), (dict(wsb=1024), 4), (dict(ws=ctypes.c_void_p(BASE + 40 * STRIDE + 16)), 4),
    (dict(q=ctypes.c_void_p(BASE + 12 * STRIDE + 8)), 2),
    (dict(dq=fake(15)), 5), (dict(dq=fake(24)), 5), (dict(ds0=fake(20)), 5),
    (dict(ws=fake(23)), 5), (dict(dr=fake(19)), 5),
])
def test_chunk_bwd_rejects_bad_arguments(over, status):
    st, msg = _bwd_call(**over)
    assert st == status, msg
    assert msg


def test_scan_gated_requires_the_gate():
    lib = muir.lib()
    st = lib.muir_chunk_fwd_scan_gated(fake(2), fake(5), fake(6), None, None, fake(9), None, 2,
                                       100, 3, 64, 64, 64, muir.MUIR_BF16, fake(11),
                                       muir.chunk_fwd_workspace_size(2, 100, 3, 64, 64, 64,
                                                                     muir.MUIR_BF16), None)
    assert st == 1 and "og" in muir.last_error()


def _scalar_erase_call(**over):
    lib = muir.lib()
    args = dict(q=fake(0), k=fake(1), v=fake(2), a=fake(3), g=fake(4), e=fake(5), w=fake(6),
                r=fake(7), s0=fake(8), o=fake(9), s_out=fake(10), B=2, T=100, H=3, dk=64,
                dv=64, chunk=64, qkv=muir.MUIR_BF16, ws=fake(11),
                wsb=muir.chunk_fwd_scalar_erase_workspace_size(2, 100, 3, 64, 64, 64),
                stream=None)
    args.update(over)
    st = lib.muir_chunk_fwd_scalar_erase(args["q"], args["k"], args["v"], args["a"], args["g"],
                                         args["e"], args["w"], args["r"], args["s0"], args["o"],
                                         args["s_out"], args["B"], args["T"], args["H"],
                                         args["dk"], args["dv"], args["chunk"], args["qkv"],
                                         args["ws"], args["wsb"], args["stream"])
    return st, muir.last_error()


# e is [B, T, H] here: 2 * 100 * 3 * 4 = 2400 bytes, so an o starting 4 KiB past e's start
# does not overlap it, while one 1 KiB past does.
@pytest.mark.parametrize("over,status", [
    (dict(qkv=muir.MUIR_F32), 3), (dict(e=None), 1), (dict(w=None), 1), (dict(q=None), 1),
    (dict(chunk=32), 3), (dict(dk=64, dv=128), 3), (dict(ws=None), 4), (dict(wsb=64), 4),
    (dict(o=ctypes.c_void_p(BASE + 5 * STRIDE + 1024)), 5),
    (dict(e=ctypes.c_void_p(BASE + 5 * STRIDE + 8)), 2),
])
def test_scalar_erase_rejects_bad_arguments(over, status):
    st, msg = _scalar_erase_call(**over)
    assert st == status, msg
    assert msg


def test_scalar_erase_gate_is_one_value_per_token():
    """An o placed right after a [B, T, H] e does not alias it (a [B, T, H, dv] e would):
    the call then fails only for the next reason in line, a missing workspace."""
    st, msg = _scalar_erase_call(o=ctypes.c_void_p(BASE + 5 * STRIDE + 4096), ws=None)
    assert st == 4, msg


def test_scalar_erase_phases_reject_bad_arguments():
    lib = muir.lib()
    wsb = muir.chunk_fwd_scalar_erase_workspace_size(2, 100, 3, 64, 64, 64)
    assert wsb > muir.chunk_fwd_workspace_size(2, 100, 3, 64, 64, 64, muir.MUIR_BF16)
    solve = lambda v, e, qkv, ws, T=100, n=wsb: lib.muir_chunk_fwd_scalar_erase_solve(
        v, e, fake(6), 2, T, 3, 64, 64, qkv, ws, n, None)
    assert solve(fake(2), None, muir.MUIR_BF16, fake(11)) == 1
    assert solve(None, fake(5), muir.MUIR_BF16, fake(11)) == 1
    assert solve(fake(2), fake(5), muir.MUIR_F32, fake(11)) == 3
    assert solve(fake(2), fake(5), muir.MUIR_BF16, None) == 4
    assert solve(fake(2), fake(5), muir.MUIR_BF16, fake(11), n=wsb - 256) == 4
    assert solve(fake(2), fake(5), muir.MUIR_BF16, fake(11), T=-1) == 2
    scan = lambda o, qkv, ws: lib.muir_chunk_fwd_scalar_erase_scan(
        None, o, None, 2, 100, 3, 64, 64, 64, qkv, ws, wsb, None)
    assert scan(None, muir.MUIR_BF16, fake(11)) == 1
    assert scan(fake(9), muir.MUIR_F32, fake(11)) == 3
    assert scan(fake(9), muir.MUIR_BF16, None) == 4
    assert muir.chunk_fwd_scalar_erase_workspace_size(1, 64, 1, 64, 128, 64) == 0


@pytest.mark.parametrize("T", [1 << 21, 1 << 23])
def test_heads_past_32_bit_offsets_are_refused(T):
    """One head's tokens (T*H*dv*4 bytes) or workspace beyond 4 GiB: both forwards refuse
    the call instead of wrapping their 32-bit offsets."""
    wsb = muir.chunk_fwd_workspace_size(1, T, 16, 128, 128, 256, muir.MUIR_BF16)
    st, msg = _chunk_call(B=1, T=T, H=16, dk=128, dv=128, chunk=256, wsb=wsb)
    assert st == 3 and "4 GiB" in msg, msg
    wsb = muir.chunk_fwd_scalar_erase_workspace_size(1, T, 16, 128, 128, 256)
    st, msg = _scalar_erase_call(B=1, T=T, H=16, dk=128, dv=128, chunk=256, wsb=wsb)
    assert st == 3 and "4 GiB" in msg, msg


def _gates_call(**over):
    lib = muir.lib()
    args = dict(z=fake(0), Ua=fake(1), Ue=fake(2), Uw=fake(3), Ug=fake(4), ca=fake(5), ce=fake(6),
                cw=fake(7), cg=fake(8), a=fake(9), e=fake(10), w=fake(11), g=fake(12), B=2, T=100,
                H=3, d=64, stream=None)
    args.update(over)
    st = lib.muir_lowrank_gates(*[args[k] for k in ("z", "Ua", "Ue", "Uw", "Ug", "ca", "ce", "cw",
                                                  "cg", "a", "e", "w", "g", "B", "T", "H", "d",
                                                  "stream")])
    return st, muir.last_error()


@pytest.mark.parametrize("over,status", [
    (dict(B=0), 2), (dict(T=-1), 2), (dict(H=0), 2), (dict(d=32), 3),
    (dict(z=None), 1), (dict(Ua=None), 1), (dict(cg=None), 1),
    (dict(e=ctypes.c_void_p(BASE + 10 * STRIDE + 8)), 2),
    (dict(w=fake(0)), 5), (dict(g=fake(11)), 5), (dict(a=fake(5)), 5),
    (dict(T=1 << 24, H=64, d=128), 3),
])
def test_lowrank_gates_rejects_bad_arguments(over, status):
    st, msg = _gates_call(**over)
    assert st == status, msg
    assert msg


def test_lowrank_gates_skips_unrequested_gates():
    # No output requested: nothing to check or launch, even with the weights absent.
    st, msg = _gates_call(a=None, e=None, w=None, g=None, Ua=None, Ue=None, Uw=None, Ug=None,
                          ca=None, ce=None, cw=None, cg=None, z=None)
    assert st == 0, msg


def _lowrank_fwd_call(**over):
    lib = muir.lib()
    B, T, H, d, C = 2, 100, 3, 64, 64
    wsb = lib.muir_chunk_fwd_lowrank_workspace_size(B, T, H, d, d, C)
    args = dict(q=fake(0), k=fake(1), v=fake(2), z=fake(3), Ua=fake(4), Ue=fake(5), Uw=fake(6),
                Ug=fake(7), ca=fake(8), ce=fake(9), cw=fake(10), cg=fake(11), r=fake(12),
                s0=fake(13), o=fake(14), s_out=fake(15), B=B, T=T, H=H, dk=d, dv=d, chunk=C,
                qkv=muir.MUIR_BF16, ws=fake(16), wsb=wsb, stream=None)
    args.update(over)
    st = lib.muir_chunk_fwd_lowrank(*[args[k] for k in (
        "q", "k", "v", "z", "Ua", "Ue", "Uw", "Ug", "ca", "ce", "cw", "cg", "r", "s0", "o",
        "s_out", "B", "T", "H", "dk", "dv", "chunk", "qkv", "ws", "wsb", "stream")])
    return st, muir.last_error()


def test_lowrank_fwd_rejects_state_or_scale_in_the_gate_tail():
    """The low-rank call's workspace is the forward's plus a tail where the gate kernel writes
    e and w; an s0 or r placed in that tail must be refused, not overwritten."""
    lib = muir.lib()
    base = muir.chunk_fwd_workspace_size(2, 100, 3, 64, 64, 64, muir.MUIR_BF16)
    full = lib.muir_chunk_fwd_lowrank_workspace_size(2, 100, 3, 64, 64, 64)
    assert full > base
    tail = ctypes.c_void_p(BASE + 16 * STRIDE + ((base + 255) // 256) * 256)
    st, msg = _lowrank_fwd_call(s0=tail)
    assert st == 5 and "s0" in msg, msg
    st, msg = _lowrank_fwd_call(r=tail)
    assert st == 5 and "r" in msg, msg
    # The state updated in place (s0 == s_out) stays allowed.
    st, msg = _lowrank_fwd_call(s0=fake(15), wsb=1)
    assert st == 4, msg


def _decode_call(**over):
    lib = muir.lib()
    args = dict(q=fake(0), k=fake(1), v=fake(2), a=fake(3), g=fake(4), e=fake(5), w=fake(6),
                r=fake(7), state=fake(8), o=fake(9), B=4, H=2, dk=128, dv=128,
                qkv=muir.MUIR_BF16, stream=None)
    args.update(over)
    st = lib.muir_decode_step(args["q"], args["k"], args["v"], args["a"], args["g"], args["e"],
                              args["w"], args["r"], args["state"], args["o"], args["B"],
                              args["H"], args["dk"], args["dv"], args["qkv"], args["stream"])
    return st, muir.last_error()


@pytest.mark.parametrize("over,status", [
    (dict(B=0), 2), (dict(H=-1), 2), (dict(dk=96, dv=96), 3), (dict(dk=128, dv=64), 3),
    (dict(qkv=2), 3), (dict(state=None), 1), (dict(r=None), 1), (dict(v=None), 1),
    (dict(o=fake(1)), 5), (dict(state=fake(3)), 5), (dict(o=fake(8)), 5),
    (dict(e=ctypes.c_void_p(BASE + 5 * STRIDE + 4)), 2),
])
def test_decode_step_rejects_bad_arguments(over, status):
    st, msg = _decode_call(**over)
    assert st == status, msg
    assert msg


def test_python_binding_validates_before_calling():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(TypeError):
        muir.chunk_fwd(x.double(), x, x, x, x, x, x, torch.zeros(1, 64))
    # host tensors never reach the library
    with pytest.raises(ValueError):
        muir.chunk_fwd(x, x, x, x, x, x, x, torch.zeros(1, 64))
    with pytest.raises(ValueError):
        muir.decode_step(x[:, 0], x[:, 0], x[:, 0], x[:, 0], x[:, 0], x[:, 0], x[:, 0],
                         torch.zeros(1, 64), torch.zeros(1, 1, 64, 64))


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "muir.h"

int main(void) {
    /* Host-only calls: sizes, status text, and argument checks that fail before any launch. */
    const size_t ws = muir_chunk_fwd_workspace_size(1, 256, 2, 64, 64, 64, MUIR_F32);
    const muir_status_t st = muir_chunk_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                            NULL, NULL, 1, 256, 2, 64, 64, 64, MUIR_F32, NULL, 0,
                                            NULL);
    printf("%d %zu %d %s %s\n", muir_version(), ws, (int)st, muir_status_string(st),
           strlen(muir_last_error()) > 0 ? "detail" : "none");
    return st == MUIR_ERR_NULL && ws > 0 ? 0 : 1;
}
"""


def test_c_program_builds_and_calls_the_library(tmp_path):
    """The public header is plain C11 (and C++): a C caller compiles with warnings as errors,
    links against libmuir.so and gets sizes and argument errors back without a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = muir.lib()  # built, and loadable here
    libdir = os.path.dirname(muir.LIB_PATH)
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    inc = os.path.dirname(HEADER)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", f"-I{inc}", str(src), "-o", str(exe),
                    f"-L{libdir}", "-lmuir", f"-Wl,-rpath,{libdir}"], check=True)
    cxx = shutil.which("g++")
    if cxx is not None:
        subprocess.run([cxx, "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", f"-I{inc}", "-x", "c++",
                        str(src)], check=True)
    hip_inc = "/opt/rocm/include"
    if cxx is not None and os.path.exists(os.path.join(hip_inc, "hip", "hip_runtime_api.h")):
        # The stream parameter is HIP's own stream type: a hipStream_t passes without a cast.
        same = tmp_path / "stream_type.cpp"
        same.write_text('#include <type_traits>\n#include <hip/hip_runtime_api.h>\n#include "muir.h"\n'
                        "static_assert(std::is_same<muir_stream_t, hipStream_t>::value, \"stream\");\n")
        subprocess.run([cxx, "-std=c++17", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", f"-I{inc}",
                        f"-I{hip_inc}", str(same)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    version, ws, status, name, detail = out.stdout.split()
    assert int(version) == lib.muir_version()
    assert int(ws) == muir.chunk_fwd_workspace_size(1, 256, 2, 64, 64, 64, 0)
    assert name == "MUIR_ERR_NULL" and detail == "detail"


def test_noalloc_refuses_workspace_beyond_its_scratch():
    """muir_chunk_fwd_noalloc checks its sizes against the static scratch before touching the
    device: the long-context shape (712 MiB of workspace) is refused with WORKSPACE."""
    lib = muir.lib()
    limit = lib.muir_chunk_fwd_noalloc_max_workspace()
    assert limit == 128 << 20
    assert muir.chunk_fwd_workspace_size(1, 32768, 16, 128, 128, 256, muir.MUIR_BF16) > limit
    st = lib.muir_chunk_fwd_noalloc(*[fake(i) for i in range(11)], 1, 32768, 16, 128, 128, 256,
                                    muir.MUIR_BF16, None)
    assert st == 4 and "static scratch" in muir.last_error(), muir.last_error()


def test_state_bytes_of_the_24_layer_model():
    """Constant-memory inference (openai-hub news page, opening section; liuch.name summary,
    opening paragraph): the 24 layers of the 1.34B model, 16 heads of d = 128, keep about
    25 MB of fp32 state per sequence, exactly 24 x 16 x 128 x 128 x 4 = 25,165,824 bytes,
    whatever the sequence length (the size takes no T), while the chunk workspace grows
    with T. The decode step and the chunk forward take state buffers of exactly that size."""
    per_layer = muir.state_bytes(1, 16, 128, 128)
    assert 24 * per_layer == 25_165_824
    assert muir.state_bytes(8, 16, 128, 128) == 8 * per_layer
    assert muir.state_bytes(1, 16, 64, 64) == 16 * 64 * 64 * 4
    assert muir.state_bytes(0, 16, 128, 128) == 0 and muir.state_bytes(1, 16, 128, -1) == 0
    big = 2**31 - 1
    assert muir.state_bytes(big, big, big, big) == 0  # the product overflows
    ws = [muir.chunk_fwd_workspace_size(1, t, 16, 128, 128, 256, muir.MUIR_BF16)
          for t in (4096, 32768)]
    assert ws[1] == 8 * ws[0]
    # A state buffer of any other size is refused before anything is launched.
    import torch
    x = torch.zeros(1, 16, 128)
    with pytest.raises(ValueError):
        muir.decode_step(x, x, x, x, x, x, x, torch.zeros(16, 128), torch.zeros(1, 16, 128, 64))
