"""CPU tests of the C ABI: exports, host-side validation, split heuristic.

No test here launches GPU work: only entry points that return before any
HIP call (validation failures, host-only queries) are called.
"""
import ctypes
import os
import re

import pytest

import memory_efficient_tiled_amd as mta
from memory_efficient_tiled_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, EINVAL = binding.ATTN_OK, binding.ATTN_EINVAL
F16, BF16 = binding.ATTN_F16, binding.ATTN_BF16

# Fake, aligned, non-overlapping addresses: validation never dereferences.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(B=1, Hq=4, Hkv=2, Nq=100, Nkv=300, D=128, scale=0.088, causal=0,
            dtype=BF16)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(attn_\w+)\s*\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return mta.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "attn_fwd" in names and len(names) >= 7
    so = ctypes.CDLL(mta.lib_path())
    for n in names:
        assert hasattr(so, n), f"{n} declared in attn.h but not exported"


def check(**kw):
    a = dict(GOOD)
    a.update(kw)
    ptrs = dict(q=Q, k=K, v=V, out=O, lse=L)
    for p in ("q", "k", "v", "out", "lse"):
        if p in kw:
            ptrs[p] = kw[p]
    return binding.attn_fwd_check(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["out"],
                                  ptrs["lse"], a["B"], a["Hq"], a["Hkv"],
                                  a["Nq"], a["Nkv"], a["D"], a["scale"],
                                  a["causal"], a["dtype"])


def test_valid_arguments_pass():
    assert check() == OK
    assert check(D=64, dtype=F16, causal=1) == OK
    assert check(lse=None) == OK          # LSE output is optional
    assert check(scale=-0.5) == OK        # any finite scale
    assert check(scale=0.0) == OK
    assert check(D=256) == OK             # head dims 64, 96, 128 and 256
    assert check(D=96) == OK
    assert check(D=80) == OK
    assert check(causal=2) == OK          # bottom-right causal alignment


@pytest.mark.parametrize("kw", [
    dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Nq=0), dict(Nkv=-5),
    dict(Hq=6, Hkv=4),                     # Hq not a multiple of Hkv
    dict(D=72), dict(D=32), dict(D=512), dict(dtype=2), dict(causal=3), dict(causal=-1),
    dict(scale=float("inf")), dict(scale=float("nan")),
    dict(q=None), dict(k=None), dict(v=None), dict(out=None),
    dict(q=Q + 8), dict(out=O + 2), dict(lse=L + 2),       # misaligned
    dict(out=Q), dict(out=K + 64), dict(lse=O + 16),       # aliasing
    dict(B=70000, Hq=70000, Hkv=70000),                    # row count overflow
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_invalid_arguments_rejected(kw):
    assert check(**kw) == EINVAL


def test_attn_fwd_rejects_before_any_hip_call(lib):
    # null pointers are caught by validation; no device is touched
    rc = lib.attn_fwd(None, None, None, None, None, 1, 1, 1, 8, 8, 64,
                      0.125, 0, F16, None)
    assert rc == EINVAL
    rc = lib.attn_fwd_split(Q, K, V, O, L, 1, 1, 1, 8, 8, 64, 0.125, 0, F16,
                            -1, None)
    assert rc == EINVAL
    # the allocation-free variant validates the same way, before any HIP call
    rc = lib.attn_fwd_noalloc(None, None, None, None, None, 1, 1, 1, 8, 8, 64,
                              0.125, 0, F16, 0, None)
    assert rc == EINVAL
    rc = lib.attn_fwd_noalloc(Q, K, V, O, L, 1, 1, 1, 8, 8, 72, 0.125, 0, F16, 0, None)
    assert rc == EINVAL
    rc = lib.attn_fwd_noalloc(Q, K, V, O, L, 1, 1, 1, 8, 8, 64, 0.125, 0, F16, -1, None)
    assert rc == EINVAL


def plan(B, Hq, Hkv, Nq, Nkv, D, causal, dtype=BF16, num_splits=0):
    return binding.attn_fwd_plan(B, Hq, Hkv, Nq, Nkv, D, causal, dtype,
                                 num_splits, 256)


def test_split_heuristic():
    # the 17160-token video shape: 24 heads x 34 tiles of 512 rows (one per
    # CU) = 3 full rounds on 256 CUs + 48 tiles; only those 48 tiles (the
    # last 14 of head 22 and all 34 of head 23) are cut over their key range
    p = plan(1, 24, 24, 17160, 17160, 128, 0)
    assert p.tile_rows == 512 and p.num_splits >= 2
    assert p.split_rows == 13 * 512 + 264 + 17160
    assert p.workspace_bytes == p.num_splits * p.split_rows * 129 * 4
    assert binding.attn_fwd_num_splits(1, 24, 24, 17160, 17160, 128, 0, BF16) \
        == p.num_splits
    # 75600 tokens: 24 x 148 tiles = 13 rounds + 224 tiles, the last 224
    p = plan(1, 24, 24, 75600, 75600, 128, 0)
    assert p.num_splits >= 2 and p.split_rows == 75 * 512 + 336 + 75600
    # grids below one round of 512-row tiles use 256-row tiles
    assert plan(1, 26, 26, 2600, 2000, 128, 0).tile_rows == 256
    assert plan(1, 24, 24, 17160, 17160, 128, 1).tile_rows == 256
    # D = 256 has one tile: 8 waves of 32 rows
    assert plan(1, 16, 16, 8192, 8192, 256, 0).tile_rows == 256
    assert plan(1, 16, 8, 8192, 8192, 256, 1).tile_rows == 256
    assert plan(1, 32, 32, 8192, 8192, 96, 0).tile_rows == 128
    # a grid of whole rounds is never split
    p = plan(1, 32, 32, 2048, 2048, 128, 0)
    assert p.num_splits == 1 and p.split_rows == 0 and p.workspace_bytes == 0
    # causal grids that fill the device are balanced by launch order instead
    assert plan(1, 32, 8, 16384, 16384, 128, 1).num_splits == 1
    # one query row over a long key range: every row split over keys
    p = plan(1, 16, 16, 1, 65536, 128, 0)
    assert 2 <= p.num_splits <= 64 and p.split_rows == 16
    # short key ranges never split
    assert plan(1, 1, 1, 1, 64, 64, 0, F16).num_splits == 1
    assert binding.attn_fwd_num_splits(0, 1, 1, 1, 64, 64, 0, F16) == EINVAL
    # a forced count splits every row
    p = plan(1, 24, 24, 17160, 17160, 128, 0, num_splits=3)
    assert p.num_splits == 3 and p.split_rows == 24 * 17160
    with pytest.raises(binding.AttnError):
        plan(1, 3, 2, 10, 10, 64, 0)


def test_causal_split_choice():
    """A causal grid smaller than the device is cut over key ranges only when
    the pieces save more than the split path costs (values measured on
    MI355X: causal GQA 14/2 at 4096 tokens runs 54-58 us whole, 78-108 us
    in 2-8 pieces; one head of 16384 tokens at D = 128 358 us whole,
    126-135 us in 4 pieces; 4 heads x 2048 at D = 128 57 us whole, 38-45 us
    in 2-8; 16 heads x 1024 at D = 64 18 us whole, 38-44 us in 2-16)."""
    assert plan(1, 14, 2, 4096, 4096, 64, 1, F16).num_splits == 1
    assert plan(1, 16, 16, 1024, 1024, 64, 1, F16).num_splits == 1
    assert plan(1, 1, 1, 16384, 16384, 128, 1).num_splits == 4
    assert plan(1, 4, 4, 2048, 2048, 128, 1).num_splits == 8
    # grids that fill every slot are balanced by their longest-first order
    assert plan(1, 14, 2, 8192, 8192, 64, 1, F16).num_splits == 1


def test_small_grid_split_floor():
    """A non-causal grid smaller than the device that runs whole in less than
    an eager split call costs is not split (measured on MI355X: one head of
    1000 tokens at D = 64 18 us whole, 42-52 us in 2-8 pieces; four heads of
    1000 x 3000 32 us whole, 42-48 us in 2-16), while longer key ranges still
    are (two heads of 2048 at D = 128: 55 us whole, 41-46 us in 2-16)."""
    assert plan(1, 1, 1, 1000, 1000, 64, 0, F16).num_splits == 1
    assert plan(1, 4, 4, 1000, 3000, 64, 0, F16).num_splits == 1
    assert plan(1, 2, 2, 2048, 2048, 128, 0).num_splits >= 2
    assert plan(1, 8, 8, 512, 8192, 128, 0).num_splits >= 8


def test_gqa_packing_plans():
    """Short query ranges of a GQA group are packed into one row range of
    the KV head.  Decode over 64K keys with 16 query heads on 2 KV heads:
    2 tiles of 8 rows (the 128-row decode tile), cut into enough key ranges
    for two workgroups per CU; the 16 output rows are the ones merged."""
    p = plan(1, 16, 2, 1, 65536, 128, 0)
    assert p.tile_rows == 128 and p.split_rows == 16
    assert 2 * p.num_splits >= 2 * 256
    assert p.workspace_bytes == p.num_splits * 16 * 129 * 4
    # MHA decode is not packed: 16 one-row tiles
    m = plan(1, 16, 16, 1, 65536, 128, 0)
    assert m.tile_rows == 128 and 16 * m.num_splits >= 2 * 256
    # packed causal GQA with 100-row chunks (D = 64, 128-row tiles): aligned
    # bottom-right, each row sees about 4000 keys and the 700 packed rows of
    # each KV head are split; aligned top-left, no row sees more than 100
    # keys, and the pieces would cost more than they save
    g = plan(1, 14, 2, 100, 4096, 64, 2)
    assert g.tile_rows == 128 and g.num_splits >= 2 and g.split_rows == 1400
    assert plan(1, 14, 2, 100, 4096, 64, 1).num_splits == 1
    # a long query range is not packed and takes the 256-row tile
    assert plan(1, 14, 2, 4096, 4096, 128, 1).tile_rows == 256
    # the (192, 128) pair has one tile of 256 rows
    assert plan(1, 16, 2, 1, 65536, 192, 0).tile_rows == 256


@pytest.mark.parametrize("shape", [
    (1, 26, 26, 2600, 2000, 128), (1, 26, 13, 2600, 2000, 128),
    (1, 40, 8, 1700, 1000, 64), (2, 32, 8, 2100, 2000, 64),
    (1, 64, 8, 2100, 1000, 128)])
def test_tail_split_shapes(shape):
    """The shapes the GPU tests use for the last-round split: some, not all,
    rows are split, starting inside a head."""
    B, Hq, Hkv, Nq, Nkv, D = shape
    p = plan(B, Hq, Hkv, Nq, Nkv, D, 0, F16)
    assert p.num_splits >= 2
    assert 0 < p.split_rows < B * Hq * Nq
    assert p.split_rows % Nq != 0


def test_workspace_bytes():
    """attn_fwd_workspace_bytes(B, Hq, Nq, Nkv, D, causal): the bytes
    attn_fwd allocates on a 256-CU device, i.e. its plan's workspace."""
    ws = binding.attn_fwd_workspace_bytes
    for shape in [(1, 24, 17160, 17160, 128, 0), (1, 16, 1, 65536, 128, 0),
                  (1, 14, 4096, 4096, 64, 1), (2, 16, 10, 65536, 64, 2),
                  (1, 16, 8192, 8192, 192, 0), (1, 32, 2048, 2048, 128, 0)]:
        B, Hq, Nq, Nkv, D, causal = shape
        # the largest plan over every KV head count (GQA packing changes it)
        want = max(plan(B, Hq, Hkv, Nq, Nkv, D, causal).workspace_bytes
                   for Hkv in range(1, Hq + 1) if Hq % Hkv == 0)
        assert ws(B, Hq, Nq, Nkv, D, causal) == want, shape
    # one decode row over 64K keys is split; a grid of whole rounds is not
    assert ws(1, 16, 1, 65536, 128, 0) > 0
    assert ws(1, 32, 2048, 2048, 128, 0) == 0
    # invalid arguments give 0
    lib = binding.load_library()
    assert lib.attn_fwd_workspace_bytes(0, 16, 10, 100, 128, 0) == 0
    assert lib.attn_fwd_workspace_bytes(1, 16, 10, 100, 72, 0) == 0
    assert lib.attn_fwd_workspace_bytes(1, 16, 10, 100, 128, 3) == 0


def test_workspace_bytes_signature():
    """The header declares the query with the scope table's parameters."""
    import re
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    m = re.search(r"size_t\s+attn_fwd_workspace_bytes\(([^)]*)\)", text)
    assert m, "attn_fwd_workspace_bytes not declared"
    params = [p.split()[-1] for p in m.group(1).split(",")]
    assert params == ["B", "Hq", "Nq", "Nkv", "D", "causal"]


def test_strerror(lib):
    for code in (OK, EINVAL, binding.ATTN_EUNSUPPORTED, binding.ATTN_ENOMEM,
                 binding.ATTN_EHIP, binding.ATTN_ESCRATCH, 12345):
        assert lib.attn_strerror(code)
    assert b"scratch" in lib.attn_strerror(binding.ATTN_ESCRATCH)


def test_python_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="HIP device"):
        mta.attn_fwd(x, x, x)


def test_oracle_not_on_product_path():
    """The package never imports the oracle."""
    pkg = os.path.join(ROOT, "memory_efficient_tiled_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f


def mcheck(mask=0x60000000, mask_type=1, ms=(0, 0, 64), **kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=2, Hq=8, Hkv=2, Nq=64, Nkv=64, D=128,
             scale=0.088, causal=0, dtype=BF16)
    a.update(kw)
    lib = binding.load_library()
    null = ctypes.POINTER(ctypes.c_longlong)()
    st = (ctypes.c_longlong * 3)(*ms) if ms is not None else null
    return lib.attn_fwd_masked_check(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                     a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["D"],
                                     null, null, null, null, mask, mask_type, st,
                                     a["scale"], a["causal"], a["dtype"])


def test_masked_validation():
    assert mcheck() == OK
    assert mcheck(mask_type=2, ms=(8 * 64 * 64, 64 * 64, 64)) == OK
    assert mcheck(mask_type=0, mask=None) == OK          # no mask: the strided call
    assert mcheck(mask=None) == EINVAL
    assert mcheck(mask=0x60000004) == EINVAL              # not 8-byte aligned
    assert mcheck(mask_type=3) == EINVAL
    assert mcheck(ms=(0, 0, 66)) == EINVAL                # row stride not a multiple of 4
    assert mcheck(ms=(-4, 0, 64)) == EINVAL
    assert mcheck(ms=None) == EINVAL
    assert mcheck(mask=O) == EINVAL                       # overlaps the output


def test_masked_backward_validation():
    lib = binding.load_library()
    null = ctypes.POINTER(ctypes.c_longlong)()
    ms = (ctypes.c_longlong * 3)(0, 0, 64)
    args = (Q, K, V, O, 0x70000000, L, 0x80000000, 0x90000000, 0xA0000000, 2, 8, 2, 64, 64, 128)
    assert lib.attn_bwd_masked_check(*args, 0x60000000, 1, ms, 0.088, 0, BF16) == OK
    assert lib.attn_bwd_masked_check(*args, 0x60000000, 1, null, 0.088, 0, BF16) == EINVAL
    assert lib.attn_bwd_masked_check(*args, 0x60000002, 2, ms, 0.088, 0, BF16) == EINVAL
    assert lib.attn_bwd_masked_check(*args, 0x80000000, 1, ms, 0.088, 0, BF16) == EINVAL  # = dq
    assert lib.attn_bwd_masked_check(*args, None, 0, null, 0.088, 0, BF16) == OK


def dvcheck(D=192, Dv=128, vs=None, os_=None, mask=None, mask_type=0, ms=None, **kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=2, Hq=8, Hkv=2, Nq=64, Nkv=80,
             scale=0.072, causal=0, dtype=BF16)
    a.update(kw)
    lib = binding.load_library()
    null = ctypes.POINTER(ctypes.c_longlong)()
    arr = lambda t: (ctypes.c_longlong * 3)(*t) if t is not None else null  # noqa: E731
    return lib.attn_fwd_dv_check(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                 a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], D, Dv,
                                 null, null, arr(vs), arr(os_), mask, mask_type, arr(ms),
                                 a["scale"], a["causal"], a["dtype"])


def test_value_width_validation():
    """attn_fwd_dv: Dv == D for the supported D, or the (192, 128) pair; V and
    out take strides of Dv-element rows."""
    assert dvcheck() == OK
    assert dvcheck(D=128, Dv=128) == OK
    assert dvcheck(D=80, Dv=80, dtype=F16) == OK
    for D, Dv in [(192, 192), (128, 64), (192, 64), (64, 128), (128, 192), (192, 256)]:
        assert dvcheck(D=D, Dv=Dv) == EINVAL, (D, Dv)
    # V [2, 2, 80, 128]: a sequence stride of 128 is a whole row, 120 is not
    assert dvcheck(vs=(2 * 80 * 128, 80 * 128, 128)) == OK
    assert dvcheck(vs=(2 * 80 * 128, 80 * 128, 120)) == EINVAL
    # out [2, 8, 64, 128] viewed from [B, N, H, Dv] storage
    assert dvcheck(os_=(64 * 8 * 128, 128, 8 * 128)) == OK
    assert dvcheck(os_=(64 * 8 * 128, 64, 8 * 128)) == EINVAL     # rows of out overlap
    # the output ends 2*8*64*128*2 bytes after O: a V placed inside it overlaps
    assert dvcheck(v=O + 4096) == EINVAL
    assert dvcheck(mask=0x60000000, mask_type=1, ms=(0, 0, 80)) == OK
    assert dvcheck(mask=0x60000000, mask_type=1, ms=None) == EINVAL
    assert dvcheck(causal=2) == OK


def test_value_width_plan(lib):
    """The planning queries read D = 192 as the (192, 128) pair: partials of
    128 columns."""
    plan = binding.AttnPlan()
    assert lib.attn_fwd_plan(1, 16, 16, 8192, 8192, 192, 0, BF16, 4, 256,
                             ctypes.byref(plan)) == OK
    rows = plan.split_rows
    assert plan.num_splits == 4 and rows > 0
    assert plan.workspace_bytes == 4 * rows * (128 + 1) * 4
    assert lib.attn_fwd_num_splits(1, 16, 16, 8192, 8192, 192, 1, BF16, 256) >= 1
    assert lib.attn_fwd_num_splits(1, 16, 16, 8192, 8192, 160, 1, BF16, 256) == EINVAL


def test_value_width_backward_validation():
    """attn_bwd_dv: the (192, 128) pair; V, O, dO and dV sized by Dv."""
    lib = binding.load_library()
    null = ctypes.POINTER(ctypes.c_longlong)()
    # B=1 Hq=4 Hkv=2 Nq=64 Nkv=80: q/dq 64 KiB... placed 1 MiB apart
    base = [0x10000000 + i * 0x100000 for i in range(9)]
    q, k, v, o, do, lse, dq, dk, dv = base

    def chk(D=192, Dv=128, **kw):
        a = dict(q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv)
        a.update(kw)
        return lib.attn_bwd_dv_check(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                                     a["dq"], a["dk"], a["dv"], 1, 4, 2, 64, 80, D, Dv,
                                     None, 0, null, 0.072, 1, BF16)
    assert chk() == OK
    assert chk(D=128, Dv=128) == OK
    assert chk(D=192, Dv=192) == EINVAL and chk(D=128, Dv=64) == EINVAL
    # dv (2*80*128*2 = 40 KiB) placed so that it ends inside V's buffer
    assert chk(dv=v - 20 * 1024) == EINVAL
    assert chk(dv=v - 40 * 1024) == OK


def test_fp8_validation(lib):
    """attn_fwd_fp8: D = 128, positive finite descales, 16-bit output."""
    def chk(D=128, qd=0.01, kd=0.02, vd=0.03, out_dtype=BF16, causal=0, **kw):
        a = dict(q=Q, k=K, v=V, out=O, lse=L)
        a.update(kw)
        return lib.attn_fwd_fp8_check(a["q"], a["k"], a["v"], a["out"], a["lse"], 1, 4, 2, 100,
                                      300, D, qd, kd, vd, 0.088, causal, out_dtype)
    assert chk() == OK and chk(out_dtype=F16) == OK and chk(causal=2) == OK
    assert chk(D=64) == EINVAL and chk(D=256) == EINVAL
    assert chk(qd=0.0) == EINVAL and chk(kd=-1.0) == EINVAL and chk(vd=float("inf")) == EINVAL
    assert chk(out_dtype=7) == EINVAL
    assert chk(out=Q + 4096) == EINVAL          # output overlaps q
    assert chk(q=Q + 8) == EINVAL               # not 16-byte aligned


def test_workspace_pool_rejects_null(lib):
    # the argument check comes before any HIP call
    assert lib.attn_workspace_pool(None) == EINVAL
