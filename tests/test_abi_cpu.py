"""The C-ABI library loads, exports every symbol include/hgrn2.h declares, and
rejects bad arguments before touching the GPU.  CPU only: no call here
reaches a kernel launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hgrn2.h")


@pytest.fixture(scope="module")
def lib():
    import linear_attention_hgrn2_amd as m
    return m.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hgrn[12]_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("hgrn2_fwd", "hgrn2_bwd", "hgrn2_decode_step", "hgrn2_fwd_chunk", "hgrn2_bwd_adjoint",
              "hgrn2_bwd_chunk", "hgrn2_fwd_tied", "hgrn2_bwd_tied", "hgrn2_fwd_chunk_tied",
              "hgrn2_bwd_chunk_tied", "hgrn2_decode_step_tied", "hgrn2_fwd_gate", "hgrn2_bwd_gate",
              "hgrn2_decode_step_gate", "hgrn2_bwd_gate_workspace_bytes", "hgrn1_fwd", "hgrn1_bwd",
              "hgrn1_states_bytes", "hgrn1_fwd_workspace_bytes", "hgrn1_bwd_workspace_bytes",
              "hgrn2_fwd_scalar", "hgrn2_bwd_scalar", "hgrn2_decode_step_scalar", "hgrn2_bwd_noalloc"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_strings(lib):
    assert lib.hgrn2_abi_version() == 9
    for s in range(5):
        assert lib.hgrn2_status_string(s).startswith(b"HGRN2_")


def test_sizes(lib):
    assert lib.hgrn2_num_chunks(4096, 64) == 64
    assert lib.hgrn2_num_chunks(250, 16) == 16
    assert lib.hgrn2_states_bytes(8, 4096, 16, 128, 128, 64, 0) == 8 * 16 * 65 * 128 * 128 * 4
    assert lib.hgrn2_states_bytes(8, 4096, 16, 128, 128, 64, 1) == 8 * 16 * 65 * 128 * 128 * 2
    assert lib.hgrn2_states_bytes(8, 4096, 16, 128, 128, 64, 5) == 0
    # the adjoint at each of the 7 chunk ends, plus the 8 chunk-boundary states when recomputed
    assert lib.hgrn2_bwd_workspace_bytes(1, 100, 1, 16, 16, 16, 0, 1) == 7 * 16 * 16 * 4
    assert lib.hgrn2_bwd_workspace_bytes(1, 100, 1, 16, 16, 16, 0, 0) == (7 + 8) * 16 * 16 * 4
    assert lib.hgrn2_bwd_workspace_bytes(1, 100, 1, 16, 16, 16, 1, 1) == 7 * 16 * 16 * 2
    assert lib.hgrn2_fwd_workspace_bytes(1, 100, 1, 16, 16, 16, 0, 1) == 0
    assert lib.hgrn2_fwd_workspace_bytes(1, 100, 1, 16, 16, 16, 0, 0) == 8 * 16 * 16 * 4
    # the forward without stored states (chunk 64, bf16, D 128, two walking workgroups per compute
    # unit): B1 H32 T32768 has 512 chunks, cut into P = 16 segments of 32 (512 workgroups);
    # summaries of (P + 1) states and P decay vectors
    assert lib.hgrn2_fwd_workspace_bytes(1, 32768, 32, 128, 128, 64, 1, 0) == 32 * (17 * 128 * 128 + 16 * 128) * 4
    # B4 H8 T2048: 512 workgroups would walk segments of 2 chunks, so 256 walk P = 8 segments of 4
    assert lib.hgrn2_fwd_workspace_bytes(4, 2048, 8, 128, 128, 64, 1, 0) == 32 * (9 * 128 * 128 + 8 * 128) * 4
    # B16 H16: P = 2
    assert lib.hgrn2_fwd_workspace_bytes(16, 4096, 16, 128, 128, 64, 1, 0) == 256 * (3 * 128 * 128 + 2 * 128) * 4
    # float32 at D 64 walks one workgroup per compute unit: P = 8 segments for 256 workgroups
    assert lib.hgrn2_fwd_workspace_bytes(1, 32768, 32, 64, 64, 64, 0, 0) == 32 * (9 * 64 * 64 + 8 * 64) * 4
    assert lib.hgrn2_supported(128, 64, 1) == 1
    assert lib.hgrn2_supported(48, 64, 1) == 0
    assert lib.hgrn2_supported(128, 128, 1) == 1     # chunk 128, bf16
    assert lib.hgrn2_supported(128, 128, 0) == 0     # float32 tiles at D 128, chunk 128 exceed the LDS
    assert lib.hgrn2_supported(64, 128, 0) == 1


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def _fwd(lib, **kw):
    a = dict(B=1, T=10, H=1, DK=16, DV=16, chunk=16, dt=0, q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000,
             lf=FAKE + 0x3000, h0=None, y=FAKE + 0x4000, ht=None, st=None, ws=None, wsb=0)
    a.update(kw)
    return lib.hgrn2_fwd(a["B"], a["T"], a["H"], a["DK"], a["DV"], a["chunk"], a["dt"], a["q"], a["k"],
                         a["v"], a["lf"], a["h0"], a["y"], a["ht"], a["st"], a["ws"], a["wsb"], None)


def test_fwd_rejections(lib):
    assert _fwd(lib, B=0) == 1
    assert _fwd(lib, T=-3) == 1
    assert _fwd(lib, q=None) == 1
    assert b"q is NULL" in lib.hgrn2_last_error()
    assert _fwd(lib, q=FAKE + 4) == 1                 # misaligned
    assert _fwd(lib, dt=7) == 1
    assert _fwd(lib, DK=48, DV=48) == 2
    assert _fwd(lib, DK=16, DV=32) == 2
    assert _fwd(lib, chunk=24) == 2
    assert _fwd(lib, chunk=256) == 2
    assert _fwd(lib, y=FAKE, st=FAKE + 0x8000) == 1    # y aliases q
    assert _fwd(lib) == 3                              # no states_out and no workspace
    assert _fwd(lib, ws=FAKE + 0x8000, wsb=100) == 3   # workspace too small
    assert _fwd(lib, st=FAKE + 0x2000) == 1            # states_out overlaps v


OUT_F32 = 0x100  # HGRN2_OUT_F32


def test_out_f32_flag(lib):
    """bfloat16 inputs with float32 token outputs: the same kernels exist, the
    sizes of states and workspaces do not change, other bits are rejected,
    and the aliasing checks size the outputs at 4 bytes per element."""
    assert lib.hgrn2_supported(128, 64, 1 | OUT_F32) == 1
    assert lib.hgrn2_supported(128, 128, 1 | OUT_F32) == 1
    assert lib.hgrn2_supported(128, 128, 0 | OUT_F32) == 0
    assert lib.hgrn2_states_bytes(8, 4096, 16, 128, 128, 64, 1 | OUT_F32) == 8 * 16 * 65 * 128 * 128 * 2
    for have in (0, 1):
        assert (lib.hgrn2_bwd_workspace_bytes(2, 300, 3, 64, 64, 64, 1 | OUT_F32, have)
                == lib.hgrn2_bwd_workspace_bytes(2, 300, 3, 64, 64, 64, 1, have))
        assert (lib.hgrn2_fwd_workspace_bytes(1, 32768, 32, 128, 128, 64, 1 | OUT_F32, have)
                == lib.hgrn2_fwd_workspace_bytes(1, 32768, 32, 128, 128, 64, 1, have))
    assert _fwd(lib, dt=1 | 0x200) == 1
    assert _fwd(lib, dt=2) == 1
    assert lib.hgrn2_states_bytes(8, 4096, 16, 128, 128, 64, 1 | 0x200) == 0
    # y ends 16 bytes into q when it holds float32 (10 tokens x 16 channels x 4 bytes), and
    # 304 bytes before q when it holds bfloat16; k (320 bytes) ends where q starts, inside y
    y = FAKE - (10 * 16 * 4 - 16)
    kw = dict(y=y, k=FAKE - 320, ws=FAKE + 0x8000, wsb=1 << 30)
    assert _fwd(lib, dt=1 | OUT_F32, **kw) == 1
    assert b"y overlaps input q" in lib.hgrn2_last_error()
    assert _fwd(lib, dt=1, **kw) == 1
    assert b"y overlaps input k" in lib.hgrn2_last_error()
    # decode: y [1, 1, 16] float32 reaching into q
    r = lib.hgrn2_decode_step(1, 1, 16, 16, 1 | OUT_F32, FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000,
                              FAKE + 0x4000, FAKE - 48, None)
    assert r == 1 and b"overlaps" in lib.hgrn2_last_error()


def test_bwd_rejections(lib):
    P = [FAKE + i * 0x100000 for i in range(12)]
    # no workspace (the adjoint states always need one)
    r = lib.hgrn2_bwd(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None,
                      P[5], P[6], P[7], P[8], None, None, 0, None)
    assert r == 3
    # states_in NULL: the workspace must also hold the recomputed states
    need = lib.hgrn2_bwd_workspace_bytes(1, 10, 1, 16, 16, 16, 0, 1)
    r = lib.hgrn2_bwd(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, None, P[4], None,
                      P[5], P[6], P[7], P[8], None, P[10], need, None)
    assert r == 3
    # dq aliases dy
    r = lib.hgrn2_bwd(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None,
                      P[4], P[6], P[7], P[8], None, P[10], need, None)
    assert r == 1
    # dq NULL
    r = lib.hgrn2_bwd(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None,
                      None, P[6], P[7], P[8], None, P[10], need, None)
    assert r == 1
    # workspace overlaps an output
    r = lib.hgrn2_bwd(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None,
                      P[5], P[6], P[7], P[8], None, P[8], need, None)
    assert r == 1


def test_staged_rejections(lib):
    P = [FAKE + i * 0x100000 for i in range(14)]
    # hgrn2_fwd_chunk: y aliases q; states NULL; unsupported D; good arguments never reach here
    assert lib.hgrn2_fwd_chunk(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], P[4], P[0], None) == 1
    assert lib.hgrn2_fwd_chunk(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[5], None) == 1
    assert lib.hgrn2_fwd_chunk(1, 10, 1, 48, 48, 16, 0, P[0], P[1], P[2], P[3], P[4], P[5], None) == 2
    assert lib.hgrn2_fwd_chunk(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], P[4] + 8, P[5], None) == 1
    # hgrn2_bwd_adjoint: adjoints NULL; adjoints overlap dy; dh0 overlaps adjoints
    assert lib.hgrn2_bwd_adjoint(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, None, None, None) == 1
    assert lib.hgrn2_bwd_adjoint(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, P[2], None, None) == 1
    assert lib.hgrn2_bwd_adjoint(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, P[3], P[3], None) == 1
    assert lib.hgrn2_bwd_adjoint(1, 10, 1, 16, 16, 24, 0, P[0], P[1], P[2], None, P[3], None, None) == 2
    # hgrn2_bwd_chunk: dv aliases the adjoints; dlog_f NULL
    assert lib.hgrn2_bwd_chunk(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7],
                               P[8], P[5], P[10], None) == 1
    assert lib.hgrn2_bwd_chunk(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7],
                               P[8], P[9], None, None) == 1
    assert lib.hgrn2_bwd_chunk(0, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7],
                               P[8], P[9], P[10], None) == 1


def test_tied_rejections(lib):
    P = [FAKE + i * 0x100000 for i in range(14)]
    # hgrn2_fwd_tied: q NULL; y aliases v; unsupported chunk; no states and no workspace
    assert lib.hgrn2_fwd_tied(1, 10, 1, 16, 16, 16, 0, None, P[1], P[2], None, P[3], None, P[4], None, 0,
                              None) == 1
    assert lib.hgrn2_fwd_tied(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, P[1], None, P[4], None, 0,
                              None) == 1
    assert lib.hgrn2_fwd_tied(1, 10, 1, 16, 16, 24, 0, P[0], P[1], P[2], None, P[3], None, P[4], None, 0,
                              None) == 2
    assert lib.hgrn2_fwd_tied(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, P[3], None, None, None, 0,
                              None) == 3
    # hgrn2_bwd_tied: no workspace; dlog_f aliases dy
    assert lib.hgrn2_bwd_tied(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, P[9], P[3], None, P[4], P[5],
                              P[6], None, None, 0, None) == 3
    need = lib.hgrn2_bwd_workspace_bytes(1, 10, 1, 16, 16, 16, 0, 1)
    assert lib.hgrn2_bwd_tied(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, P[9], P[3], None, P[4], P[5],
                              P[3], None, P[10], need, None) == 1
    # the staged tied launches and the tied decode step
    assert lib.hgrn2_fwd_chunk_tied(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], P[0], None) == 1
    assert lib.hgrn2_bwd_chunk_tied(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], P[4], P[5], P[6], None,
                                    P[8], None) == 1
    assert lib.hgrn2_decode_step_tied(1, 1, 24, 24, 0, P[0], P[1], P[2], P[3], P[4], None) == 2
    assert lib.hgrn2_decode_step_tied(1, 1, 16, 16, 0, P[0], P[1], P[2], P[3], P[0], None) == 1


def test_gate_rejections(lib):
    P = [FAKE + i * 0x100000 for i in range(16)]
    # hgrn2_fwd_gate: lower_bound NULL; lower_bound misaligned; y aliases z; lower_bound aliases y
    assert lib.hgrn2_fwd_gate(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], None, None, P[3], None, P[4], None, 0,
                              None) == 1
    assert lib.hgrn2_fwd_gate(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[5] + 2, None, P[3], None, P[4], None, 0,
                              None) == 1
    assert lib.hgrn2_fwd_gate(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[5], None, P[2], None, P[4], None, 0,
                              None) == 1
    assert lib.hgrn2_fwd_gate(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[3], None, P[4], None, 0,
                              None) == 1
    # the gate backward's workspace adds B*H*N*DK floats for the per-chunk dlb sums
    base = lib.hgrn2_bwd_workspace_bytes(2, 10, 3, 16, 16, 16, 0, 1)
    gate = lib.hgrn2_bwd_gate_workspace_bytes(2, 10, 3, 16, 16, 16, 0, 1)
    assert gate == base + 2 * 3 * 1 * 16 * 4
    assert lib.hgrn2_bwd_gate_workspace_bytes(0, 10, 3, 16, 16, 16, 0, 1) == 0
    args = lambda dlb, ws, wsb: (1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None,
                                 P[5], P[6], P[7], dlb, None, ws, wsb, None)
    need = lib.hgrn2_bwd_gate_workspace_bytes(1, 10, 1, 16, 16, 16, 0, 1)
    assert lib.hgrn2_bwd_gate(*args(None, P[10], need)) == 1                       # dlower_bound NULL
    assert lib.hgrn2_bwd_gate(*args(P[11], P[10], lib.hgrn2_bwd_workspace_bytes(1, 10, 1, 16, 16, 16, 0, 1))) == 3
    assert lib.hgrn2_bwd_gate(*args(P[7], P[10], need)) == 1                       # dlower_bound aliases dz
    assert lib.hgrn2_bwd_gate(*args(P[3], P[10], need)) == 1                       # dlower_bound aliases lower_bound
    # decode: lower_bound NULL, unsupported D
    assert lib.hgrn2_decode_step_gate(1, 1, 16, 16, 0, P[0], P[1], P[2], None, P[4], P[5], None) == 1
    assert lib.hgrn2_decode_step_gate(1, 1, 24, 24, 0, P[0], P[1], P[2], P[3], P[4], P[5], None) == 2


def test_scalar_rejections(lib):
    P = [FAKE + i * 0x100000 for i in range(16)]
    # hgrn2_fwd_scalar: k NULL (k is an input); y aliases log_a
    assert lib.hgrn2_fwd_scalar(1, 10, 1, 16, 16, 16, 0, P[0], None, P[2], P[3], None, P[4], None, P[5], None, 0,
                                None) == 1
    assert lib.hgrn2_fwd_scalar(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[3], None, P[5], None, 0,
                                None) == 1
    # hgrn2_bwd_scalar: dk NULL; dlog_a aliases dy
    need = lib.hgrn2_bwd_workspace_bytes(1, 10, 1, 16, 16, 16, 0, 1)
    assert lib.hgrn2_bwd_scalar(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None, P[5],
                                None, P[6], P[7], None, P[10], need, None) == 1
    assert lib.hgrn2_bwd_scalar(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None, P[5],
                                P[8], P[6], P[4], None, P[10], need, None) == 1
    assert lib.hgrn2_decode_step_scalar(1, 1, 24, 24, 0, P[0], P[1], P[2], P[3], P[4], P[5], None) == 2


def test_hgrn1_rejections(lib):
    P = [FAKE + i * 0x100000 for i in range(16)]
    S = lib.hgrn1_states_bytes(2, 70, 6)
    assert S == 2 * 3 * 6 * 4                      # 3 segments of 32 tokens
    G = 2 * 1 * 6 * 4                              # one group of segments
    assert lib.hgrn1_fwd_workspace_bytes(2, 70, 6, 1) == 2 * S + 3 * G
    assert lib.hgrn1_fwd_workspace_bytes(2, 70, 6, 0) == 2 * S + 3 * G
    assert lib.hgrn1_bwd_workspace_bytes(2, 70, 6, 1) == 2 * S + 3 * G
    assert lib.hgrn1_bwd_workspace_bytes(2, 70, 6, 0) == 2 * (2 * S + 3 * G)
    ws = 4 * S + 6 * G
    # hgrn1_fwd: odd C; tied must be 0/1; k NULL untied; y aliases v; small workspace
    assert lib.hgrn1_fwd(2, 70, 5, 0, 0, P[0], P[1], P[2], P[3], None, P[4], None, None, P[9], ws, None) == 2
    assert lib.hgrn1_fwd(2, 70, 6, 0, 2, P[0], P[1], P[2], P[3], None, P[4], None, None, P[9], ws, None) == 1
    assert lib.hgrn1_fwd(2, 70, 6, 0, 0, P[0], None, P[2], P[3], None, P[4], None, None, P[9], ws, None) == 1
    assert lib.hgrn1_fwd(2, 70, 6, 0, 1, P[0], None, P[2], P[3], None, P[2], None, None, P[9], ws, None) == 1
    assert lib.hgrn1_fwd(2, 70, 6, 0, 1, P[0], None, P[2], P[3], None, P[4], None, None, P[9], S, None) == 3
    assert lib.hgrn1_bwd(2, 70, 6, 0, 1, P[0], None, P[2], P[3], None, None, P[4], None, P[5], None, P[6],
                         P[7], None, P[9], 2 * S + 3 * G, None) == 3
    # hgrn1_bwd: dk NULL untied; dlog_f aliases dy
    assert lib.hgrn1_bwd(2, 70, 6, 0, 0, P[0], P[1], P[2], P[3], None, None, P[4], None, P[5], None, P[6],
                         P[7], None, P[9], ws, None) == 1
    assert lib.hgrn1_bwd(2, 70, 6, 0, 1, P[0], None, P[2], P[3], None, None, P[4], None, P[5], None, P[6],
                         P[4], None, P[9], ws, None) == 1


def test_noalloc_rejections(lib):
    """hgrn2_bwd_noalloc rejects a backward that needs more scratch than it has,
    and bad arguments, before any HIP call (this runs without a GPU)."""
    P = [FAKE + i * 0x100000 for i in range(12)]
    # B8 H16 T4096 d128 bf16 chunk 64 without states: adjoints + recomputed states > 256 MiB
    r = lib.hgrn2_bwd_noalloc(8, 4096, 16, 128, 128, 64, 1, P[0], P[1], P[2], P[3], None, None, P[4], None,
                              P[5], P[6], P[7], P[8], None, None)
    assert r == 3 and b"scratch" in lib.hgrn2_last_error()
    # invalid sizes win over the scratch size
    assert lib.hgrn2_bwd_noalloc(8, 4096, 16, 48, 48, 64, 1, P[0], P[1], P[2], P[3], None, None, P[4], None,
                                 P[5], P[6], P[7], P[8], None, None) == 2
    # dq NULL; dq misaligned
    assert lib.hgrn2_bwd_noalloc(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None,
                                 None, P[6], P[7], P[8], None, None) == 1
    assert lib.hgrn2_bwd_noalloc(1, 10, 1, 16, 16, 16, 0, P[0], P[1], P[2], P[3], None, P[9], P[4], None,
                                 P[5] + 4, P[6], P[7], P[8], None, None) == 1


def test_decode_rejections(lib):
    P = [FAKE + i * 0x100000 for i in range(8)]
    assert lib.hgrn2_decode_step(0, 1, 16, 16, 0, P[0], P[1], P[2], P[3], P[4], P[5], None) == 1
    assert lib.hgrn2_decode_step(1, 1, 24, 24, 0, P[0], P[1], P[2], P[3], P[4], P[5], None) == 2
    assert lib.hgrn2_decode_step(1, 1, 16, 16, 0, P[0], P[1], P[2], P[3], P[4], P[4], None) == 1


def test_product_path_does_not_import_the_oracle():
    import linear_attention_hgrn2_amd
    pkg = os.path.dirname(linear_attention_hgrn2_amd.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".h", ".hip", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.replace("oracle-free", ""), f


def test_size_limits(lib):
    """Sizes beyond the kernels' 32-bit offsets or grid are rejected before
    anything is launched: a sequence's chunk-boundary states (N + 1) D^2 E,
    a chunk's token rows chunk H D E, and one workgroup per chunk B H N."""
    big = dict(ws=FAKE + 0x10000000, wsb=1 << 62)
    # (N + 1) * 16 * 16 * 4 >= 2^32 at T = 2^26, chunk 16
    assert _fwd(lib, T=1 << 26, **big) == 1
    assert b"too large" in lib.hgrn2_last_error()
    # chunk * H * 16 * 4 >= 2^32 at H = 2^22
    assert _fwd(lib, H=1 << 22, **big) == 1
    assert b"too large" in lib.hgrn2_last_error()
    # B * H * N >= 2^31
    assert _fwd(lib, B=1 << 10, H=1 << 10, T=1 << 15, **big) == 1
    assert b"too large" in lib.hgrn2_last_error()
    # HGRN1: 32 * C * 4 >= 2^32
    P = [FAKE + i * 0x100000 for i in range(16)]
    assert lib.hgrn1_fwd(1, 1, 1 << 25, 0, 1, P[0], None, P[2], P[3], None, P[4], None, None, P[9], 1 << 62,
                         None) == 1
    assert b"too large" in lib.hgrn2_last_error()


def test_launch_work_items_fit_32_bits(lib):
    """Every launch's work-items (workgroups times their size) must fit the
    dispatch's 32-bit count; cases that pass the older per-dimension limits."""
    big = dict(ws=FAKE + 0x10000000, wsb=1 << 62)
    # chunk kernels: B*H*N = 2^24 < 2^31, but 2^24 workgroups of 4 * 64 work-items = 2^32
    assert _fwd(lib, B=1 << 10, H=1 << 7, T=128 * 64, chunk=64, **big) == 1
    assert b"too large" in lib.hgrn2_last_error()
    # 127/128 of it fits the size checks and stops at the next one (y overlaps q): no launch
    assert _fwd(lib, B=1 << 10, H=1 << 7, T=127 * 64, chunk=64, **big) == 1
    assert b"overlaps" in lib.hgrn2_last_error()
    # state scan: B*H = 2^24 (b, h) of 4 slices x 64 work-items (D = 128, chunk 16, float32) = 2^32,
    # while the chunk kernels (2^24 x 64) fit
    assert _fwd(lib, B=1 << 12, H=1 << 12, T=1, DK=128, DV=128, chunk=16, **big) == 1
    assert b"too large" in lib.hgrn2_last_error()
    # decode: 2^25 (b, h) of 256 work-items
    P = [FAKE + i * 0x100000 for i in range(8)]
    assert lib.hgrn2_decode_step(1 << 12, 1 << 13, 32, 32, 0, P[0], P[1], P[2], P[3], P[4], P[5], None) == 1
    assert b"too large" in lib.hgrn2_last_error()
    # HGRN1 segment pass: B * 8 segments * 32 workgroups of 256 = 2^32 (B = 2^16, C = 2^14, T = 256)
    P = [FAKE + i * 0x100000 for i in range(16)]
    assert lib.hgrn1_fwd(1 << 16, 256, 1 << 14, 0, 1, P[0], None, P[2], P[3], None, P[4], None, None, P[9],
                         1 << 62, None) == 1
    assert b"too large" in lib.hgrn2_last_error()
