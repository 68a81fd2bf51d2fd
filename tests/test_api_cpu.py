"""C ABI checks that need no GPU: symbols, status codes, validation, workspace sizes.

Only calls that fail validation are made (validation runs on the host before
any HIP call), so nothing here touches a device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infini.h")

binding = pytest.importorskip("compressive_linear_memory_amd.binding")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libinfini.so not built")
    return binding.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(infini_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    fns = header_functions()
    for f in ("infini_attn_fwd", "infini_attn_bwd", "infini_fwd_workspace_bytes",
              "infini_bwd_workspace_bytes", "infini_status_string", "infini_version"):
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    for f in header_functions():
        assert hasattr(L, f), f


def test_version_and_status_strings(L):
    assert L.infini_version() == 2
    for code in range(8):
        assert len(L.infini_status_string(code)) > 0
    assert L.infini_status_string(0) == b"ok"


def P(B=1, Hq=2, Hkv=2, N=64, d=32, L=16, dtype=0):
    return binding.Problem(B, Hq, Hkv, N, d, L, dtype)


FAKE = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(20)]   # never dereferenced


def fwd(L, p, ptrs=None, ws_bytes=1 << 40, null=()):
    a = list(ptrs or FAKE[:11])
    for i in null:
        a[i] = None
    # order: Q K V beta M0 z0 O M_S z_S lse ws
    return L.infini_attn_fwd(ctypes.byref(p), *a[:10], a[10], ws_bytes, None)


def test_workspace_sizes(L):
    assert L.infini_fwd_workspace_bytes(ctypes.byref(P())) > 0
    assert L.infini_bwd_workspace_bytes(ctypes.byref(P())) > 0
    assert L.infini_fwd_workspace_bytes(None) == 0
    assert L.infini_fwd_workspace_bytes(ctypes.byref(P(Hq=3, Hkv=2))) == 0
    assert L.infini_fwd_workspace_bytes(ctypes.byref(P(d=48))) == 0


def test_workspace_does_not_grow_with_sequence_length(L):
    """Bounded state: once a call has more segments than one chunk holds, the
    workspace stops growing with seq_len."""
    sizes_f = {L.infini_fwd_workspace_bytes(ctypes.byref(P(N=16 * s))) for s in (16, 32, 512, 4096)}
    sizes_b = {L.infini_bwd_workspace_bytes(ctypes.byref(P(N=16 * s))) for s in (16, 32, 512, 4096)}
    assert len(sizes_f) == 1 and len(sizes_b) == 1
    # and it never exceeds the 16-segment bound for short calls either
    big = L.infini_fwd_workspace_bytes(ctypes.byref(P(N=16 * 16)))
    for s in (1, 2, 7, 15):
        assert L.infini_fwd_workspace_bytes(ctypes.byref(P(N=16 * s))) <= big


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 6, 7, 8])
def test_fwd_null_required_pointer(L, idx):
    assert fwd(L, P(), null=(idx,)) == 1


def test_fwd_half_state_is_null_error(L):
    assert fwd(L, P(), null=(4,)) == 1     # M0 NULL but z0 not
    assert fwd(L, P(), null=(5,)) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(Hkv=0), 2), (dict(Hq=3, Hkv=2), 2), (dict(B=-1), 2), (dict(L=0), 2), (dict(N=-16), 2),
    (dict(d=48), 3), (dict(d=256), 3), (dict(dtype=7), 3),
    # per-call counts past 32 bits and element counts past the 64-bit index budget
    (dict(B=1 << 20, Hq=4096, Hkv=4096), 2), (dict(B=1 << 16, Hq=1 << 10, Hkv=1 << 10, N=1 << 20, d=128), 2),
])
def test_fwd_shape_errors(L, kw, code):
    assert fwd(L, P(**kw)) == code


def test_empty_batch_is_a_no_op(L):
    """batch = 0: every forward entry point validates and returns ok without
    issuing work (tensors of no elements may be NULL); decode needs a token."""
    p = P(B=0)
    assert L.infini_fwd_workspace_bytes(ctypes.byref(p)) == 0
    # Q K V beta M0 z0 O M_S z_S lse ws: only beta is non-empty
    assert fwd(L, p, [None, None, None, FAKE[3]] + [None] * 7, ws_bytes=0) == 0
    assert fwd(L, p, [None, None, None, None] + [None] * 7, ws_bytes=0) == 1   # beta is [q_heads]
    assert L.infini_fwd_memory(ctypes.byref(p), None, None, None, None, None, None, None, 0, None) == 0
    assert L.infini_fwd_attend(ctypes.byref(p), None, None, None, FAKE[3], None, None, None, 0, None) == 0
    one = (ctypes.c_void_p * 1)(None)
    assert L.infini_fwd_stream(ctypes.byref(p), 1, one, one, one, None, None, None, one, None, 0, 1, 1,
                               None, one, one) == 0
    a = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], None, None, FAKE[6], FAKE[7], FAKE[8]]
    for q in (P(B=0, N=1), P(N=0)):
        assert L.infini_decode(ctypes.byref(q), 0, *a, FAKE[10], 1 << 30, None) == 2
        assert L.infini_decode_workspace_bytes(ctypes.byref(q)) == 0


@pytest.mark.parametrize("dtype,d", [(0, 32), (0, 128), (1, 64), (1, 128)])
def test_empty_problem_size_queries(L, dtype, d):
    """Size queries of empty problems on every kernel path are well defined
    (no division by the zero segment or batch count)."""
    for kw in (dict(N=0), dict(B=0), dict(B=0, N=0), dict(N=0, L=2048)):
        p = P(Hq=32, Hkv=8, d=d, dtype=dtype, **kw)
        for f in (L.infini_fwd_workspace_bytes, L.infini_bwd_workspace_bytes):
            f(ctypes.byref(p))
        for g in (1, 4, 8):
            L.infini_fwd_stream_workspace_bytes(ctypes.byref(p), 2, g)
        assert L.infini_fwd_path(ctypes.byref(p)) is not None


def test_misaligned_tensor_pointers_are_refused(L):
    """Tensors move in 16-byte vectors: a tensor pointer off a 16-byte boundary
    is refused (3) before anything is issued; beta, dbeta and lse may sit
    anywhere (here the call then fails later, on its workspace)."""
    off = lambda i, k: ctypes.c_void_p(FAKE[i].value + k)
    for i in (0, 1, 2, 4, 6, 7, 10):              # Q K V M0 O M_S ws
        a = list(FAKE[:11])
        a[i] = off(i, 2)
        if i == 4:
            a[5] = off(5, 2)                       # M0 and z0 come together
        assert fwd(L, P(), a) == 3, i
    a = list(FAKE[:11])
    a[3] = off(3, 4)                               # beta
    a[9] = off(9, 4)                               # lse
    assert fwd(L, P(), a, ws_bytes=1) == 5
    p = P()
    b = list(FAKE[:17])
    b[10] = off(10, 8)                             # dQ
    assert L.infini_attn_bwd(ctypes.byref(p), *b[:16], b[16], 1 << 40, None) == 3
    b = list(FAKE[:17])
    b[13] = off(13, 4)                             # dbeta may sit anywhere: fails on the workspace
    assert L.infini_attn_bwd(ctypes.byref(p), *b[:16], b[16], 1, None) == 5
    assert L.infini_fwd_memory(ctypes.byref(p), FAKE[1], off(2, 6), None, None, FAKE[7], FAKE[8], FAKE[10],
                               1 << 40, None) == 3
    assert L.infini_fwd_attend(ctypes.byref(p), FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[6], None,
                               off(10, 1), 1 << 40, None) == 3
    d = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], off(4, 2), FAKE[5], None, None, FAKE[6], FAKE[7], FAKE[8]]
    assert L.infini_decode(ctypes.byref(P(N=3)), 0, *d, FAKE[10], 1 << 30, None) == 3   # Kcache


def test_fwd_workspace_too_small(L):
    need = L.infini_fwd_workspace_bytes(ctypes.byref(P()))
    assert fwd(L, P(), ws_bytes=need - 1) == 5
    assert fwd(L, P(), null=(10,)) == 5


def test_fwd_alias_output_overlaps_input(L):
    a = list(FAKE[:11])
    a[6] = ctypes.c_void_p(FAKE[0].value + 64)        # O inside Q
    assert fwd(L, P(), a) == 4
    a = list(FAKE[:11])
    a[7] = a[4]                                       # M_S == M0 (in-place state is refused)
    assert fwd(L, P(), a) == 4


def test_bwd_validation(L):
    p = P()
    a = list(FAKE[:17])
    # Q K V beta M0 z0 lse dO dM_S dz_S dQ dK dV dbeta dM0 dz0 ws
    def call(args, ws_bytes=1 << 40):
        return L.infini_attn_bwd(ctypes.byref(p), *args[:16], args[16], ws_bytes, None)
    b = list(a); b[7] = None
    assert call(b) == 1                               # dO missing
    b = list(a); b[14] = None
    assert call(b) == 1                               # dM0 without dz0
    b = list(a); b[10] = b[7]
    assert call(b) == 4                               # dQ aliases dO
    need = L.infini_bwd_workspace_bytes(ctypes.byref(p))
    assert call(a, need - 1) == 5


def test_ragged_final_segment_is_a_valid_shape(L):
    """A sequence that is not a multiple of seg_len ends in one shorter segment:
    accepted, and sized like the call with that segment full."""
    for N in (60, 49, 17, 1, 255):
        full = -(-N // 16) * 16
        for bwd in (False, True):
            f = L.infini_bwd_workspace_bytes if bwd else L.infini_fwd_workspace_bytes
            assert f(ctypes.byref(P(N=N))) == f(ctypes.byref(P(N=full))) > 0


def test_decode_validation(L):
    """Streaming decode: shape, pointer and workspace checks (no launch)."""
    P1 = P(N=3)                         # three new tokens, seg_len 16
    # Q K V beta Kcache Vcache M z O M_next z_next
    a = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], FAKE[5], None, None, FAKE[6], FAKE[7], FAKE[8]]

    def dec(p, pos, args, ws=FAKE[10], ws_bytes=1 << 30):
        return L.infini_decode(ctypes.byref(p), pos, *args, ws, ws_bytes, None)

    assert dec(P1, 14, a) == 2                               # 14 + 3 > 16
    assert dec(P1, -1, a) == 2
    b = list(a); b[0] = None
    assert dec(P1, 0, b) == 1                                # Q missing
    b = list(a); b[6] = FAKE[9]
    assert dec(P1, 0, b) == 1                                # M without z
    b = list(a); b[9] = None
    assert dec(P1, 13, b) == 1                               # completing call without M_next
    need = L.infini_decode_workspace_bytes(ctypes.byref(P1))
    assert need >= L.infini_fwd_workspace_bytes(ctypes.byref(P(N=16))) > 0
    assert dec(P1, 13, a, ws_bytes=need - 1) == 5
    assert dec(P1, 0, a, ws_bytes=need - 1) == 5            # key-split partials need it on every call
    assert dec(P1, 0, a, ws=None) == 5
    b = list(a); b[8] = FAKE[0]
    assert dec(P1, 0, b) == 4                                # O overlaps Q


def test_fwd_stream_validation(L):
    """Pipelined streaming forward: every argument is checked before any
    work is issued, so these calls touch no device (codes: 1 null, 2 shape,
    4 alias, 5 workspace)."""
    p = P(N=16)                                   # one 16-token segment per call
    n, npipe = 3, 2
    arr = lambda vals: (ctypes.c_void_p * len(vals))(*[v.value if v else None for v in vals])
    Q = arr(FAKE[0:3]); K = arr(FAKE[3:6]); V = arr(FAKE[6:9]); O = arr(FAKE[9:12])
    streams = arr([FAKE[15], FAKE[16]])
    events = arr([FAKE[17], FAKE[18], FAKE[19], FAKE[18]])
    need = L.infini_fwd_stream_workspace_bytes(ctypes.byref(p), npipe, 2)
    assert need >= 2 * npipe * L.infini_fwd_workspace_bytes(ctypes.byref(p)) > 0
    assert L.infini_fwd_stream_workspace_bytes(ctypes.byref(p), 0, 2) == 0
    assert L.infini_fwd_stream_workspace_bytes(ctypes.byref(p), npipe, 9) == 0

    def call(p=p, n=n, Q=Q, K=K, V=V, O=O, beta=FAKE[12], M=FAKE[13], z=FAKE[14], ws=ctypes.c_void_p(1 << 36),
             ws_bytes=need, npipe=npipe, group=2, streams=streams, events=events):
        return L.infini_fwd_stream(ctypes.byref(p), n, Q, K, V, beta, M, z, O, ws, ws_bytes, npipe, group, None,
                                   streams, events)

    assert call(n=0) == 2
    assert call(npipe=0) == 2
    assert call(group=0) == 2
    assert call(group=9) == 2
    assert call(streams=arr([FAKE[15], None])) == 1
    assert call(p=P(N=17 * 16)) == 2                            # more than 16 segments per call
    assert call(Q=None) == 1
    assert call(beta=None) == 1
    assert call(M=None) == 1
    assert call(events=arr([FAKE[17], None, FAKE[19], FAKE[18]])) == 1
    assert call(V=arr([FAKE[6], None, FAKE[8]])) == 1
    assert call(ws_bytes=need - 1) == 5
    assert call(O=arr([FAKE[9], ctypes.c_void_p(FAKE[4].value + 64), FAKE[11]])) == 4   # O[1] inside K[1]
    assert call(M=ctypes.c_void_p(FAKE[0].value + 64)) == 4                              # state inside Q[0]
    assert call(K=arr([FAKE[3], ctypes.c_void_p(FAKE[4].value + 2), FAKE[5]])) == 3     # K[1] misaligned


def test_decode_noalloc_refuses_problems_beyond_its_scratch(L):
    """The allocation-free decode checks its arguments like infini_decode and
    refuses a problem whose workspace would exceed the static scratch
    (INFINI_ERR_SCRATCH = 7) before touching any device."""
    arr = [FAKE[i] for i in range(12)]
    big = P(B=64, Hq=64, Hkv=64, N=64, d=128, L=4096, dtype=1)
    need = L.infini_decode_workspace_bytes(ctypes.byref(big))
    assert need > 32 << 20
    assert L.infini_decode_noalloc(ctypes.byref(big), 0, *arr[:11], None) == 7
    small = P(B=1, Hq=4, Hkv=2, N=3, d=64, L=16, dtype=1)
    a = list(arr)
    a[8] = a[0]                                   # O aliases Q
    assert L.infini_decode_noalloc(ctypes.byref(small), 0, *a[:11], None) == 4
    assert L.infini_decode_noalloc(ctypes.byref(small), 14, *arr[:11], None) == 2
    assert L.infini_decode_noalloc(None, 0, *arr[:11], None) == 1


def test_varlen_entry_points_validate_before_launch(L):
    """infini_attn_fwd_varlen / infini_attn_bwd_varlen: the length array must
    be 4-byte aligned (3) and must not overlap an output (4); the other
    checks are those of the uniform calls."""
    p = P(B=2, N=64, d=64, L=16, dtype=1)
    a = [FAKE[i] for i in range(20)]
    lens_bad = ctypes.c_void_p(FAKE[19].value + 2)
    # forward: Q K V beta M0 z0 O M_S z_S lse, then ws, ws_bytes, stream
    assert L.infini_attn_fwd_varlen(ctypes.byref(p), lens_bad, *a[:10], None, 0, None) == 3
    lens_in_O = ctypes.c_void_p(a[6].value + 16)          # inside O
    assert L.infini_attn_fwd_varlen(ctypes.byref(p), lens_in_O, *a[:10], None, 0, None) == 4
    # backward: Q K V beta M0 z0 lse dO dM_S dz_S dQ dK dV dbeta dM0 dz0, then ws, ws_bytes, stream
    assert L.infini_attn_bwd_varlen(ctypes.byref(p), lens_bad, *a[:16], None, 0, None) == 3
    lens_in_dQ = ctypes.c_void_p(a[10].value + 16)
    assert L.infini_attn_bwd_varlen(ctypes.byref(p), lens_in_dQ, *a[:16], FAKE[19], 1 << 30, None) == 4
    assert L.infini_attn_bwd_varlen(None, FAKE[19], *a[:16], None, 0, None) == 1


def test_taylor_feature_map_only_on_the_forward(L):
    """The Taylor feature map is taken by infini_attn_fwd(_varlen) only; the
    other entry points return INFINI_ERR_UNSUPPORTED (3) before any launch,
    and an unknown feature map is refused everywhere."""
    p = binding.Problem(1, 2, 2, 64, 32, 16, 0, 1)
    assert L.infini_fwd_path(ctypes.byref(p)) == b"generic_fp32_taylor2"
    assert L.infini_fwd_workspace_bytes(ctypes.byref(p)) > 0
    assert L.infini_bwd_workspace_bytes(ctypes.byref(p)) == 0
    assert L.infini_fwd_stream_workspace_bytes(ctypes.byref(p), 1, 1) == 0
    assert L.infini_decode_workspace_bytes(ctypes.byref(binding.Problem(1, 2, 2, 1, 32, 16, 0, 1))) == 0
    a = [FAKE[i] for i in range(20)]
    assert L.infini_attn_bwd(ctypes.byref(p), *a[:16], a[16], 1 << 30, None) == 3
    assert L.infini_fwd_memory(ctypes.byref(p), *a[:6], a[16], 1 << 30, None) == 3
    assert L.infini_fwd_attend(ctypes.byref(p), *a[:6], a[16], 1 << 30, None) == 3
    # bf16, head_dim 64/128: the matrix-core kernel form up to 16 D' tokens
    # (D' = 4161 at 64), the fp32 state sweep beyond
    assert L.infini_fwd_path(ctypes.byref(binding.Problem(1, 2, 2, 16 * 4161, 64, 64, 1, 1))) == b"mfma_bf16_taylor2"
    assert L.infini_fwd_path(ctypes.byref(binding.Problem(1, 2, 2, 16 * 4161 + 1, 64, 64, 1, 1))) == \
        b"generic_fp32_taylor2"
    assert L.infini_fwd_path(ctypes.byref(binding.Problem(1, 2, 2, 64, 32, 16, 1, 1))) == b"generic_fp32_taylor2"
    bad = binding.Problem(1, 2, 2, 64, 32, 16, 0, 7)
    assert L.infini_fwd_path(ctypes.byref(bad)) is None
    assert L.infini_attn_fwd(ctypes.byref(bad), *a[:10], a[16], 1 << 30, None) == 3


def test_taylor_matrix_core_workspace(L):
    """The matrix-core Taylor forward needs workspace only for a starting
    state: batch * q_heads * seq_len * (head_dim + 1) floats (rounded to 256
    bytes per part), which the size query covers; a call with M0 and no
    workspace is refused before any launch."""
    p = binding.Problem(1, 2, 1, 64, 64, 64, 1, 1)
    assert L.infini_fwd_path(ctypes.byref(p)) == b"mfma_bf16_taylor2"
    rows = 1 * 2 * 64
    need = -(-rows * 64 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    assert L.infini_fwd_workspace_bytes(ctypes.byref(p)) >= need
    a = [FAKE[i] for i in range(11)]
    a[10] = None                                              # no workspace
    assert L.infini_attn_fwd(ctypes.byref(p), *a[:10], None, 0, None) == 5
    assert L.infini_attn_fwd(ctypes.byref(p), *a[:10], FAKE[10], need - 1, None) == 5


def test_bwd_saved_validates_before_launch(L):
    """infini_attn_bwd_saved: M_S and z_S come as a pair (1), 16-byte aligned
    (3), and no output may overlap them (4); the other checks are those of
    infini_attn_bwd_varlen."""
    p = P(B=2, N=64, d=64, L=16, dtype=1)
    a = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(22)]   # never dereferenced
    # Q K V beta M0 z0 | M_S z_S | lse dO dM_S dz_S dQ dK dV dbeta dM0 dz0, then ws, ws_bytes, stream
    def call(ms, zs, rest=None, lens=None):
        r = list(rest or a[8:18])
        return L.infini_attn_bwd_saved(ctypes.byref(p), lens, *a[:6], ms, zs, *r, a[18], 1 << 40, None)
    assert call(a[6], None) == 1                           # z_S without M_S
    assert call(None, a[7]) == 1
    assert call(ctypes.c_void_p(a[6].value + 4), a[7]) == 3
    r = list(a[8:18]); r[4] = ctypes.c_void_p(a[6].value)  # dQ on M_S
    assert call(a[6], a[7], r) == 4
    r = list(a[8:18]); r[8] = a[7]                          # dM0 on z_S
    assert call(a[6], a[7], r) == 4
    assert L.infini_attn_bwd_saved(None, None, *a[:18], a[18], 1 << 40, None) == 1
