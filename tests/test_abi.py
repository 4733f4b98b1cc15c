"""Host-side checks of the C ABI (CPU only: no call here reaches the GPU).

The library loads, exports every function include/moe_decode.h declares, and
rejects bad arguments with the documented codes before any launch.  The
pointers passed are plain integers: every case returns during host-side
validation, which runs before any HIP call.
"""
import ctypes
import os
import re

import pytest

import moe_gate_up_amd as mg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_decode_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 9
    lib = ctypes.CDLL(mg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mg.EXPORTS)


def test_error_codes_match_header():
    src = open(HEADER).read()
    codes = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (MOE_(?:OK|ERR_\w+)) \(?(-?\d+)\)?", src)}
    for name, val in codes.items():
        assert getattr(mg, name) == val, name
    for val in codes.values():
        s = mg.strerror(val)
        assert s and s != "unknown error code"
    assert mg.strerror(12345) == "unknown error code"


A = 0x100000000000   # 16-byte aligned fake device addresses, never dereferenced,
S = 0x1000000000     # spaced 64 GiB apart so only the planted overlaps overlap


def gu(x=A, ids=A + 1 * S, wg=A + 2 * S, sg=A + 3 * S, wu=A + 4 * S, su=A + 5 * S, h=A + 6 * S,
       B=2, H=2048, I=768, E=128, k=8, rows=None, variant=0):
    L = mg.lib()
    args = [ctypes.c_void_p(p) for p in (x, ids, wg, sg, wu, su, h)] + [B, H, I, E, k]
    if rows is None:
        return L.moe_decode_gate_up(*args, None)
    return L.moe_decode_gate_up_ex(*args, variant, rows, None)


def dn(h=A, ids=A + 1 * S, tw=A + 2 * S, wd=A + 3 * S, sd=A + 4 * S, y=A + 5 * S,
       B=2, H=2048, I=768, E=128, k=8, rows=None, variant=0):
    L = mg.lib()
    args = [ctypes.c_void_p(p) for p in (h, ids, tw, wd, sd, y)] + [B, H, I, E, k]
    if rows is None:
        return L.moe_decode_down(*args, None)
    return L.moe_decode_down_ex(*args, variant, rows, None)


@pytest.mark.parametrize("fn", [gu, dn])
def test_shape_errors(fn):
    assert fn(B=-1) == mg.MOE_ERR_SHAPE
    assert fn(H=2047) == mg.MOE_ERR_SHAPE
    assert fn(I=100) == mg.MOE_ERR_SHAPE
    assert fn(k=0) == mg.MOE_ERR_SHAPE
    assert fn(k=129) == mg.MOE_ERR_SHAPE
    assert fn(E=0, k=1) == mg.MOE_ERR_SHAPE
    assert fn(H=8192 + 32) == mg.MOE_ERR_SHAPE       # beyond 4 blocks per lane
    assert fn(I=2048 + 32, k=8) == mg.MOE_ERR_SHAPE  # k*I beyond 8 blocks per lane


def test_empty_batch_is_a_noop():
    assert gu(B=0) == mg.MOE_OK
    assert dn(B=0) == mg.MOE_OK
    assert gu(B=0, x=0, h=0) == mg.MOE_OK            # no pointer is needed when B == 0


def test_null_pointer_errors():
    for name in ("x", "ids", "wg", "sg", "wu", "su", "h"):
        assert gu(**{name: 0}) == mg.MOE_ERR_NULL, name
    for name in ("h", "ids", "tw", "wd", "sd", "y"):
        assert dn(**{name: 0}) == mg.MOE_ERR_NULL, name


def test_alignment_errors():
    for name in ("x", "wg", "wu", "h"):
        assert gu(**{name: A + 8 * S + 8}) == mg.MOE_ERR_ALIGN, name
    # the matrix-core kernel copies 16-byte pieces of the scale tensors: asked for
    # explicitly it needs them 16-byte aligned
    for name in ("sg", "su"):
        assert gu(rows=0, variant=mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA, **{name: A + 8 * S + 4}) == mg.MOE_ERR_ALIGN, name
    assert gu(ids=A + 8 * S + 2) == mg.MOE_ERR_ALIGN
    for name in ("h", "wd"):
        assert dn(**{name: A + 8 * S + 8}) == mg.MOE_ERR_ALIGN, name
    assert dn(y=A + 8 * S + 1) == mg.MOE_ERR_ALIGN
    assert dn(tw=A + 8 * S + 2) == mg.MOE_ERR_ALIGN


def test_alias_errors():
    # h_out overlapping x / the gate weights
    assert gu(h=A + 16) == mg.MOE_ERR_ALIAS
    assert gu(wg=A + 6 * S - 4096) == mg.MOE_ERR_ALIAS
    # y overlapping h
    assert dn(y=A + 64) == mg.MOE_ERR_ALIAS


def test_bad_tuning_arguments():
    assert gu(rows=3) == mg.MOE_ERR_ARG
    assert gu(rows=-1) == mg.MOE_ERR_ARG
    assert gu(rows=16) == mg.MOE_ERR_ARG
    assert gu(H=8192, rows=4) == mg.MOE_ERR_ARG      # 8 passes x 4 rows exceeds the register budget
    assert gu(rows=1, variant=3) == mg.MOE_ERR_ARG
    assert gu(rows=1, variant=-1) == mg.MOE_ERR_ARG
    assert gu(rows=8, variant=mg.MOE_GATE_UP_EXPERT_GROUPED) == mg.MOE_ERR_ARG      # 2 passes x 8 rows > 8
    assert gu(B=129, rows=1, variant=mg.MOE_GATE_UP_EXPERT_GROUPED) == mg.MOE_ERR_ARG   # B*k > 1024
    assert gu(E=1025, rows=1, variant=mg.MOE_GATE_UP_EXPERT_GROUPED) == mg.MOE_ERR_ARG  # E > 1024
    assert dn(rows=5) == mg.MOE_ERR_ARG
    assert dn(I=1536, rows=8) == mg.MOE_ERR_ARG      # 12 passes x 8 rows exceeds the register budget
    assert dn(rows=1, variant=3) == mg.MOE_ERR_ARG
    assert dn(rows=1, variant=-1) == mg.MOE_ERR_ARG
    G = mg.MOE_DOWN_EXPERT_GROUPED
    assert dn(rows=4, variant=G) == mg.MOE_ERR_ARG                # the grouped kernel takes 8 rows
    assert dn(B=65, k=8, rows=8, variant=G) == mg.MOE_ERR_ARG     # B > 64
    assert dn(I=2080, k=2, rows=8, variant=G) == mg.MOE_ERR_ARG   # I beyond 2 passes
    assert dn(E=1025, rows=0, variant=G) == mg.MOE_ERR_ARG        # E > 1024


def cv(x=A, ids=A + 1 * S, tw=A + 2 * S, wg=A + 3 * S, sg=A + 4 * S, wu=A + 5 * S, su=A + 6 * S, wd=A + 7 * S,
       sd=A + 8 * S, y=A + 9 * S, ws=A + 10 * S, ws_bytes=1 << 30, B=2, H=2048, I=768, E=128, k=8):
    L = mg.lib()
    args = [ctypes.c_void_p(p) for p in (x, ids, tw, wg, sg, wu, su, wd, sd, y, ws)]
    return L.moe_decode_conventional(*args, ctypes.c_size_t(ws_bytes), B, H, I, E, k, None)


def test_conventional_path_arguments():
    need = mg.moe_decode_conventional_workspace(2, 2048, 768, 128, 8)
    assert 0 < need < (1 << 30)
    # grows with the batch: the padded rows are at most twice the slots
    assert mg.moe_decode_conventional_workspace(32, 2048, 768, 128, 8) > 8 * need
    assert cv(B=0) == mg.MOE_OK
    assert cv(ws=0) == mg.MOE_ERR_NULL
    assert cv(ws=A + 10 * S + 16) == mg.MOE_ERR_ALIGN          # workspace must be 256-byte aligned
    assert cv(ws_bytes=need - 1) == mg.MOE_ERR_ARG
    assert cv(B=129) == mg.MOE_ERR_SHAPE                       # B*k > 1024
    assert cv(H=16384, I=32) == mg.MOE_ERR_SHAPE               # H beyond 8192
    assert cv(y=A + 64) == mg.MOE_ERR_ALIAS                    # y overlapping x
    assert cv(ws=A + 9 * S) == mg.MOE_ERR_ALIAS                # workspace overlapping y
    assert cv(ws=A + 3 * S + 4096) == mg.MOE_ERR_ALIAS         # workspace overlapping the gate weights


def cvn(x=A, ids=A + 1 * S, tw=A + 2 * S, wg=A + 3 * S, sg=A + 4 * S, wu=A + 5 * S, su=A + 6 * S, wd=A + 7 * S,
        sd=A + 8 * S, y=A + 9 * S, B=2, H=2048, I=768, E=128, k=8):
    L = mg.lib()
    args = [ctypes.c_void_p(p) for p in (x, ids, tw, wg, sg, wu, su, wd, sd, y)]
    return L.moe_decode_conventional_noalloc(*args, B, H, I, E, k, None)


def test_conventional_noalloc_arguments():
    """The no-allocation form checks the same arguments before touching the
    device, and refuses shapes whose workspace exceeds its 32 MiB buffer."""
    assert cvn(B=0) == mg.MOE_OK
    assert cvn(x=0) == mg.MOE_ERR_NULL
    assert cvn(x=A + 8) == mg.MOE_ERR_ALIGN
    assert cvn(B=129) == mg.MOE_ERR_SHAPE                      # B*k > 1024
    assert cvn(y=A + 64) == mg.MOE_ERR_ALIAS                   # y overlapping x
    # 17 MB at 128 tokens of the H=2048 layer and at 64 tokens of the H=4096 one: accepted sizes
    assert mg.moe_decode_conventional_workspace(128, 2048, 768, 128, 8) <= 32 << 20
    assert mg.moe_decode_conventional_workspace(64, 4096, 1536, 128, 8) <= 32 << 20
    need = mg.moe_decode_conventional_workspace(128, 8192, 1536, 128, 8)
    assert need > 32 << 20
    assert cvn(B=128, H=8192, I=1536) == mg.MOE_ERR_SCRATCH


def test_plans():
    for B in (1, 8, 9, 10, 15, 16, 23, 24, 32, 42, 43, 64):
        v, r, g = mg.moe_decode_gate_up_plan(B, 2048, 768, 128, 8)
        if v == mg.MOE_GATE_UP_PER_SLOT:   # one wavefront per (tile, slot)
            assert r in (1, 2, 4, 8)
            assert g == -(-((768 + r - 1) // r) * B * 8 // 4)
        elif v == mg.MOE_GATE_UP_EXPERT_GROUPED:   # persistent: <= 2048 workgroups, <= the possible work items
            assert r in (1, 2, 4, 8)
            assert g == min(2048, -(-(B * 8 * -(-768 // (4 * r))) // 2))   # items taken in pairs
        else:   # matrix cores: one resident round; three workgroups per CU while units of 8 slots fit
            # three in LDS (B*k <= 341 slots here: the slot index grows with them), else two
            assert v == mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA and r == 16 and g == (768 if B <= 42 else 512)
        # on the matrix cores from 0.625 slots per expert on, per slot below
        assert (v == mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA) == (8 * B * 8 >= 5 * 128)
        assert (v == mg.MOE_GATE_UP_PER_SLOT) == (8 * B * 8 < 5 * 128)
    # H = 4096: the vector-unit grouped kernel from 5/16 of a slot per expert, the matrix cores from 7/4
    for B, v in ((4, mg.MOE_GATE_UP_PER_SLOT), (5, mg.MOE_GATE_UP_EXPERT_GROUPED), (8, mg.MOE_GATE_UP_EXPERT_GROUPED),
                 (27, mg.MOE_GATE_UP_EXPERT_GROUPED), (28, mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA),
                 (64, mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA)):
        assert mg.moe_decode_gate_up_plan(B, 4096, 1536, 128, 8)[0] == v, B
    # H = 6144 and 8192: the matrix cores from half a slot per expert on
    for H in (6144, 8192):
        assert mg.moe_decode_gate_up_plan(8, H, 1024, 128, 8)[0] == mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA
        assert mg.moe_decode_gate_up_plan(7, H, 1024, 128, 8)[0] == mg.MOE_GATE_UP_PER_SLOT
    # H not a multiple of 2048: never on the matrix cores; the vector-unit grouped kernel from one
    # slot per expert (half a slot from H = 4096)
    assert mg.moe_decode_gate_up_plan(16, 3072, 768, 128, 8)[0] == mg.MOE_GATE_UP_EXPERT_GROUPED
    assert mg.moe_decode_gate_up_plan(15, 3072, 768, 128, 8)[0] == mg.MOE_GATE_UP_PER_SLOT
    assert mg.moe_decode_gate_up_plan(8, 5120, 768, 128, 8)[0] == mg.MOE_GATE_UP_EXPERT_GROUPED
    assert mg.moe_decode_gate_up_plan(7, 5120, 768, 128, 8)[0] == mg.MOE_GATE_UP_PER_SLOT
    assert mg.moe_decode_gate_up_plan(1, 2048, 768, 128, 8)[0] == mg.MOE_GATE_UP_PER_SLOT
    assert mg.moe_decode_gate_up_plan(200, 2048, 768, 128, 8)[0] == mg.MOE_GATE_UP_PER_SLOT   # B*k > 1024
    for B in (1, 4, 5, 8, 11, 12, 16, 32, 64, 100):
        v, r, g = mg.moe_decode_down_plan(B, 2048, 768, 128, 8)
        if v == mg.MOE_DOWN_PER_TOKEN:     # one wavefront per (tile, token)
            assert r in (1, 2, 4, 8) and g == -(-((2048 + r - 1) // r) * B // 4)
        else:                              # one workgroup per 8 output dimensions
            assert v == mg.MOE_DOWN_EXPERT_GROUPED_MFMA and r == 8 and g == 2048 // 8
        # on the matrix cores from 5/16 of a slot per expert on
        assert (v == mg.MOE_DOWN_EXPERT_GROUPED_MFMA) == (16 * B * 8 >= 5 * 128)
    # the same at I = 1536
    assert mg.moe_decode_down_plan(5, 4096, 1536, 128, 8)[0] == mg.MOE_DOWN_EXPERT_GROUPED_MFMA
    assert mg.moe_decode_down_plan(4, 4096, 1536, 128, 8)[0] == mg.MOE_DOWN_PER_TOKEN
    # beyond the matrix-core kernel's limits (which include the vector-unit grouped kernel's): per token
    assert mg.moe_decode_down_plan(150, 2048, 768, 128, 8)[0] == mg.MOE_DOWN_PER_TOKEN    # B*k > 1024
    assert mg.moe_decode_down_plan(16, 2048, 768, 1100, 8)[0] == mg.MOE_DOWN_PER_TOKEN   # E > 1024
    with pytest.raises(mg.MoeDecodeError):
        mg.moe_decode_gate_up_plan(1, 100, 768, 128, 8)


def rt(lg=A, ids=A + 1 * S, tw=A + 2 * S, B=2, E=128, k=8):
    L = mg.lib()
    return L.moe_decode_route(*[ctypes.c_void_p(p) for p in (lg, ids, tw)], B, E, k, None)


def gr(x=A, lg=A + 1 * S, wg=A + 2 * S, sg=A + 3 * S, wu=A + 4 * S, su=A + 5 * S, h=A + 6 * S, ids=A + 7 * S,
       tw=A + 8 * S, B=2, H=2048, I=768, E=128, k=8, rows=None, variant=0):
    L = mg.lib()
    args = [ctypes.c_void_p(p) for p in (x, lg, wg, sg, wu, su, h, ids, tw)] + [B, H, I, E, k]
    if rows is None:
        return L.moe_decode_gate_up_routed(*args, None)
    return L.moe_decode_gate_up_routed_ex(*args, variant, rows, None)


def test_router_arguments():
    for fn in (rt, gr):
        assert fn(B=0) == mg.MOE_OK
        assert fn(B=-1) == mg.MOE_ERR_SHAPE
        assert fn(k=0) == mg.MOE_ERR_SHAPE
        assert fn(E=4, k=5) == mg.MOE_ERR_SHAPE                 # k > E
        assert fn(E=1056, k=8) == mg.MOE_ERR_SHAPE              # E beyond 16 logits per lane
        assert fn(E=256, k=65) == mg.MOE_ERR_SHAPE              # k beyond one selection per lane
        assert fn(lg=0) == mg.MOE_ERR_NULL
        assert fn(ids=0) == mg.MOE_ERR_NULL
        assert fn(tw=0) == mg.MOE_ERR_NULL
        assert fn(lg=A + 2) == mg.MOE_ERR_ALIGN
        assert fn(ids=A + 7 * S + 2 if fn is gr else A + S + 2) == mg.MOE_ERR_ALIGN
        assert fn(tw=A + 2 * S + 16, ids=A + 2 * S) == mg.MOE_ERR_ALIAS     # the two outputs overlap
        assert fn(ids=A + 256) == mg.MOE_ERR_ALIAS                          # ids over the logits
    assert rt(B=1 << 20, E=1024) == mg.MOE_ERR_SHAPE            # logits beyond 2^31 bytes
    assert gr(x=0) == mg.MOE_ERR_NULL
    assert gr(h=A + 8 * S + 16) == mg.MOE_ERR_ALIAS             # h over the router weights
    assert gr(h=A + 1 * S + 64) == mg.MOE_ERR_ALIAS             # h over the logits
    assert gr(ids=A + 2 * S + 64) == mg.MOE_ERR_ALIAS           # ids over the gate weights
    assert gr(H=2047) == mg.MOE_ERR_SHAPE
    assert gr(rows=3) == mg.MOE_ERR_ARG
    assert gr(rows=1, variant=3) == mg.MOE_ERR_ARG


def test_peak_argument_errors():
    L = mg.lib()
    v = ctypes.c_void_p
    assert L.moe_decode_copy_peak(v(A), v(A + 1 * S), 0, None) == mg.MOE_ERR_SHAPE
    assert L.moe_decode_copy_peak(v(A), v(A + 1 * S), 24, None) == mg.MOE_ERR_SHAPE
    assert L.moe_decode_copy_peak(v(A + 8), v(A + 1 * S), 32, None) == mg.MOE_ERR_ALIGN
    assert L.moe_decode_copy_peak(v(A), v(A + 16), 64, None) == mg.MOE_ERR_ALIAS
    assert L.moe_decode_copy_peak(None, v(A), 64, None) == mg.MOE_ERR_NULL
    assert L.moe_decode_read_peak(v(A), 0, v(A + 64), None) == mg.MOE_ERR_SHAPE
    assert L.moe_decode_read_peak(v(A), 64, None, None) == mg.MOE_ERR_NULL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 2048), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mg.moe_decode_gate_up(x, torch.zeros((1, 8), dtype=torch.int32), *(torch.zeros(1, dtype=torch.uint8),) * 4,
                              torch.zeros((1, 8, 768), dtype=torch.bfloat16), E=128, I=768)
