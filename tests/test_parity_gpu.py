"""GPU parity: the HIP attention forward against the CPU oracle.

Every case draws seeded inputs, runs the library through its C ABI on the
GPU and compares with the float64 oracle element by element.  The named
workloads use the fixed tolerances (max |err| <= 4e-3, mean |err| <= 5e-4,
|lse err| <= 1e-3); at full size the oracle evaluates sampled query rows.
"""
import numpy as np
import pytest

from memory_efficient_tiled_amd import inputs
from tests.parity import (compare, gather_rows, log, oracle_rows, run_gpu,
                          to_device)

pytestmark = pytest.mark.gpu


def _case(device, B, Hq, Hkv, Nq, Nkv, D, dtype, causal, seed=0, scale=None,
          rows=None, num_splits=0, allowance=True, k_offset_std=None, Dv=None):
    log(f"case B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} Dv={Dv} {dtype} "
        f"causal={causal} seed={seed} splits={num_splits} scale={scale}")
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=seed,
                           k_offset_std=k_offset_std, sampled_rows=rows, Dv=Dv)
    o, l = run_gpu(x, scale, causal, device, num_splits=num_splits)
    r = None if rows is None else x.rows
    o_ref, l_ref = oracle_rows(x, scale, causal, rows=r)
    if r is not None:
        o, l = gather_rows(o, r), gather_rows(l, r)
    return compare(o, l, o_ref, l_ref, dtype, rounding_allowance=allowance,
                   what=f"N={Nq}x{Nkv} D={D} {dtype} causal={causal}")


# -- the named workloads -----------------------------------------------------

def _workload(device, name, rows=None, allowance=False):
    w = inputs.WORKLOADS[name]
    return _case(device, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.dtype, w.causal,
                 rows=rows, allowance=allowance, k_offset_std=w.k_offset_std, Dv=w.Dv)


def test_tiny_256(gpu_device):
    _workload(gpu_device, "tiny-256")


@pytest.mark.parametrize("n", [1024, 2048])
def test_sweep_full(gpu_device, n):
    _workload(gpu_device, f"sweep-{n}")


@pytest.mark.parametrize("n", [4096, 8192, 16384])
def test_sweep_sampled(gpu_device, n):
    _workload(gpu_device, f"sweep-{n}", rows=64)


@pytest.mark.parametrize("n", [4096, 8192, 16384])
def test_gqa_causal(gpu_device, n):
    _workload(gpu_device, f"gqa-causal-{n}", rows=96)


def test_dit_17160(gpu_device):
    _workload(gpu_device, "dit-17160", rows=96)


def test_dit_75600(gpu_device):
    # 256 sampled query rows per head, including rows 0 and Nq-1 (in the
    # ragged last query tile)
    _workload(gpu_device, "dit-75600", rows=256)


# -- edge shapes -------------------------------------------------------------

@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("D", [64, 80, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 7, 63, 65, 129, 1000])
def test_ragged_lengths(gpu_device, n, causal, D, dtype):
    _case(gpu_device, 2, 4, 2, n, n, D, dtype, causal, seed=n)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, "bottom_right"])
def test_causal_whole_grid_batches(gpu_device, D, causal):
    """One launch of whole causal tiles over 2 batches x 6 heads (a head
    count that is not a multiple of the 8 XCDs), tile index 0 of every
    (batch, head) first: every tile lands on its own rows."""
    nq, nkv = 1500, 1700 if causal == "bottom_right" else 1500
    log(f"causal whole grid D={D} {causal}")
    x = inputs.make_inputs(2, 6, 3, nq, nkv, D, inputs.F16, seed=D + len(str(causal)))
    o, l = run_gpu(x, None, causal, gpu_device, num_splits=1)
    o_ref, l_ref = oracle_rows(x, None, True, causal_offset=nkv - nq if causal == "bottom_right" else 0)
    compare(o, l, o_ref, l_ref, inputs.F16, rounding_allowance=True,
            what=f"causal whole grid D={D} {causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nkv", [(100, 300), (300, 100), (1, 777), (513, 64)])
def test_nq_ne_nkv(gpu_device, nq, nkv, causal):
    _case(gpu_device, 1, 4, 1, nq, nkv, 128, inputs.BF16, causal, seed=nq + nkv)


@pytest.mark.parametrize("G", [1, 2, 7, 8])
def test_gqa_groups(gpu_device, G):
    _case(gpu_device, 1, 2 * G, 2, 300, 300, 64, inputs.F16, True, seed=G)


@pytest.mark.parametrize("G", [1, 8])
def test_decode_long_keys(gpu_device, G):
    # one query row over 64K keys: the split-KV path
    _case(gpu_device, 1, 2 * G, 2, 1, 65536, 128, inputs.BF16, False, seed=40 + G)


# -- GQA head packing --------------------------------------------------------
# With G = Hq / Hkv > 1 query heads per KV head and a query range shorter
# than a tile, the G ranges are computed as one range of G * Nq rows (row r
# is head r / Nq, position r % Nq): causal masks take the position, tiles
# hold rows of several heads, and waves without rows skip the arithmetic.
# G = 1 (not packed) runs the same shapes through the decode tile alone.

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True, "bottom_right"])
@pytest.mark.parametrize("G", [1, 7, 8])
@pytest.mark.parametrize("nq", [1, 4, 16])
def test_gqa_packed_short_queries(gpu_device, nq, G, causal, D):
    dtype = inputs.BF16 if D == 128 else inputs.F16
    x = inputs.make_inputs(2, 2 * G, 2, nq, 1000, D, dtype, seed=nq * 31 + G)
    o, l = run_gpu(x, None, causal, gpu_device)
    o_ref, l_ref = oracle_rows(x, None, bool(causal),
                               causal_offset=1000 - nq if causal == "bottom_right" else 0)
    compare(o, l, o_ref, l_ref, dtype, rounding_allowance=True,
            what=f"packed G={G} Nq={nq} D={D} causal={causal}")


@pytest.mark.parametrize("nq,G,D", [(50, 7, 64), (100, 8, 128), (33, 3, 96), (60, 4, 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_packed_tiles_cross_heads(gpu_device, nq, G, D, causal):
    """Packed tiles whose rows span a head boundary (Nq not dividing the
    tile), ragged keys, forced and planned splits."""
    dtype = inputs.BF16 if D in (128, 256) else inputs.F16
    x = inputs.make_inputs(1, 2 * G, 2, nq, 777, D, dtype, seed=nq + G + D)
    for splits in (0, 3):
        o, l = run_gpu(x, None, causal, gpu_device, num_splits=splits)
        o_ref, l_ref = oracle_rows(x, None, causal)
        compare(o, l, o_ref, l_ref, dtype, rounding_allowance=True,
                what=f"packed G={G} Nq={nq} D={D} causal={causal} splits={splits}")


@pytest.mark.parametrize("nq", [1, 3])
def test_gqa_packed_strided(gpu_device, nq):
    """[B, N, H, D] storage viewed as [B, H, N, D]: one row per head packs
    (the head stride becomes the row stride); three rows per head cannot be
    re-indexed and run unpacked.  Both must give the same function."""
    import torch
    from memory_efficient_tiled_amd import attn_fwd
    x = inputs.make_inputs(2, 16, 2, nq, 900, 128, inputs.BF16, seed=70 + nq)
    q, k, v = (to_device(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), inputs.BF16,
                         gpu_device).transpose(1, 2) for a in (x.q, x.k, x.v))
    for causal in (False, "bottom_right"):
        out, lse = attn_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize(gpu_device)
        o_ref, l_ref = oracle_rows(x, None, bool(causal),
                                   causal_offset=900 - nq if causal else 0)
        compare(out.float().cpu().numpy().astype(np.float64),
                lse.cpu().numpy().astype(np.float64), o_ref, l_ref, inputs.BF16,
                rounding_allowance=True, what=f"packed strided Nq={nq} causal={causal}")


@pytest.mark.parametrize("D", [64, 80, 96, 128, 256])
@pytest.mark.parametrize("strided", [False, True])
def test_many_pieces_merge(gpu_device, D, strided):
    """Rows cut into more than 16 pieces are merged by a workgroup per row
    (40 forced pieces over 5000 keys; a few packed GQA rows); strided output
    rows ([B, N, H, D] storage) take the strided merge."""
    import torch
    from memory_efficient_tiled_amd import attn_fwd
    dtype = inputs.F16 if D == 80 else inputs.BF16
    x = inputs.make_inputs(2, 6, 2, 3, 5000, D, dtype, seed=500 + D)
    q, k, v = (to_device(a, dtype, gpu_device) for a in (x.q, x.k, x.v))
    out = None
    if strided:
        out = torch.empty((2, 3, 6, D), dtype=q.dtype, device=gpu_device).transpose(1, 2)
    o, l = attn_fwd(q, k, v, num_splits=40, out=out)
    torch.cuda.synchronize(gpu_device)
    o_ref, l_ref = oracle_rows(x, None, False)
    compare(o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
            o_ref, l_ref, dtype, rounding_allowance=True,
            what=f"40 pieces D={D} strided={strided}")


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_forced_splits(gpu_device, splits, causal):
    _case(gpu_device, 1, 3, 1, 200, 1500, 64, inputs.F16, causal, seed=7,
          num_splits=splits)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.5])
def test_scale_values(gpu_device, scale):
    _case(gpu_device, 1, 2, 2, 130, 190, 64, inputs.F16, True, seed=9,
          scale=scale)


# -- the 64-row tiles of D = 64 --------------------------------------------
# Chosen for non-causal D = 64 grids of at least two 256-row workgroups per
# CU (here 2 x 32 heads x 9 query tiles = 576 on 256 CUs): ragged query and
# key tails, GQA, Nq != Nkv, both dtypes, forced splits.

@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("nkv", [33, 700, 2100])
def test_wide_d64_tiles(gpu_device, nkv, dtype):
    _case(gpu_device, 2, 32, 8, 2100, nkv, 64, dtype, False, seed=nkv, rows=24)


@pytest.mark.parametrize("splits", [2, 5])
def test_wide_d64_tiles_split(gpu_device, splits):
    _case(gpu_device, 2, 32, 8, 2100, 2000, 64, inputs.F16, False, seed=11,
          rows=24, num_splits=splits)


# -- the 512-row tiles of D = 128 -------------------------------------------
# Chosen for non-causal D = 128 grids of at least one 512-row workgroup per
# CU (here 64 heads x 5 query tiles = 320 on 256 CUs, so the last 64 tiles
# are also split over keys): ragged query and key tails, GQA, both dtypes,
# forced splits, and keys that grow along the sequence so that the scores
# keep raising the running reference (the softmax's slow path).

@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("nkv", [33, 1000, 2047])
def test_wide_d128_tiles(gpu_device, nkv, dtype):
    from memory_efficient_tiled_amd import attn_fwd_plan
    assert attn_fwd_plan(1, 64, 8, 2100, nkv, 128, False, 0).tile_rows == 512
    _case(gpu_device, 1, 64, 8, 2100, nkv, 128, dtype, False, seed=nkv + 1,
          rows=24)


@pytest.mark.parametrize("splits", [1, 3])
def test_wide_d128_tiles_split(gpu_device, splits):
    _case(gpu_device, 1, 64, 64, 2100, 1500, 128, inputs.BF16, False, seed=12,
          rows=24, num_splits=splits)


def test_wide_d128_rising_scores(gpu_device):
    """Keys scaled up 8x along the sequence: the row maxima keep rising, so
    the running reference is raised (the softmax's slow path) on many key
    tiles, not only the first."""
    x = inputs.make_inputs(1, 64, 8, 2100, 2047, 128, inputs.F16, seed=13,
                           sampled_rows=24)
    ramp = np.linspace(1.0, 8.0, 2047, dtype=np.float32)[None, None, :, None]
    x.k = (x.k.astype(np.float32) * ramp).astype(np.float16)
    o, l = run_gpu(x, None, False, gpu_device)
    o_ref, l_ref = oracle_rows(x, None, False, rows=x.rows)
    compare(gather_rows(o, x.rows), gather_rows(l, x.rows), o_ref, l_ref,
            inputs.F16, rounding_allowance=True, what="rising scores")


# -- head dimension 256 --------------------------------------------------------
# One tile (8 waves x 32 rows, 32-key tiles, single-buffered pipeline, half of
# Q^T in LDS): the named shapes, split pieces, and rising scores.

@pytest.mark.parametrize("name", ["hd256-8192", "hd256-gqa-causal-8192"])
def test_hd256_workloads(gpu_device, name):
    # bf16 causal: the first rows see few keys, |o| is of order 1 and the
    # bf16 rounding of the output alone reaches 2^-9 |o|, so these shapes
    # (not among the pages' workloads) take the half-ulp allowance
    _workload(gpu_device, name, rows=64, allowance=True)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_d256_forced_splits(gpu_device, splits, causal):
    _case(gpu_device, 1, 4, 2, 333, 1500, 256, inputs.BF16, causal, seed=splits + 60,
          num_splits=splits)


def test_d256_decode_long_keys(gpu_device):
    _case(gpu_device, 1, 8, 2, 1, 40000, 256, inputs.F16, False, seed=66)


def test_d256_rising_scores(gpu_device):
    x = inputs.make_inputs(1, 8, 4, 700, 1999, 256, inputs.F16, seed=67)
    ramp = np.linspace(1.0, 8.0, 1999, dtype=np.float32)[None, None, :, None]
    x.k = (x.k.astype(np.float32) * ramp).astype(np.float16)
    o, l = run_gpu(x, None, False, gpu_device)
    o_ref, l_ref = oracle_rows(x, None, False)
    compare(o, l, o_ref, l_ref, inputs.F16, rounding_allowance=True,
            what="D=256 rising scores")


# -- head dimension 96 ---------------------------------------------------------

@pytest.mark.parametrize("name", ["hd96-8192", "hd96-causal-8192"])
def test_hd96_workloads(gpu_device, name):
    _workload(gpu_device, name, rows=64, allowance=True)


@pytest.mark.parametrize("splits", [3])
@pytest.mark.parametrize("causal", [False, True])
def test_d96_forced_splits_gqa(gpu_device, splits, causal):
    _case(gpu_device, 1, 6, 2, 333, 1500, 96, inputs.F16, causal, seed=splits + 70,
          num_splits=splits)


def test_d96_decode_long_keys(gpu_device):
    _case(gpu_device, 1, 8, 2, 1, 30000, 96, inputs.BF16, False, seed=73)


# -- head dimension 80 (computed as 96 with two zero chunks per row) ---------

def test_hd80_workload(gpu_device):
    _workload(gpu_device, "hd80-8192", rows=64, allowance=True)


@pytest.mark.parametrize("causal", [False, True])
def test_d80_forced_splits_gqa(gpu_device, causal):
    _case(gpu_device, 1, 6, 3, 250, 1300, 80, inputs.BF16, causal, seed=80, num_splits=4)


def test_d80_strided(gpu_device):
    """[B, N, H, 80] storage: rows of the sequence are H * 80 elements apart,
    so the zero chunks must not pick up the next head's values."""
    import torch
    from memory_efficient_tiled_amd import attn_fwd
    x = inputs.make_inputs(1, 4, 4, 300, 300, 80, inputs.F16, seed=81)
    q, k, v = (to_device(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), inputs.F16,
                         gpu_device).transpose(1, 2) for a in (x.q, x.k, x.v))
    out, lse = attn_fwd(q, k, v)
    torch.cuda.synchronize(gpu_device)
    o_ref, l_ref = oracle_rows(x, None, False)
    compare(out.float().cpu().numpy().astype(np.float64),
            lse.cpu().numpy().astype(np.float64), o_ref, l_ref, inputs.F16,
            rounding_allowance=True, what="D=80 strided")


# -- bottom-right causal alignment (keys j <= i + Nkv - Nq) ------------------

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("nq,nkv", [(100, 1000), (1, 777), (513, 600), (700, 90), (64, 64)])
def test_bottom_right(gpu_device, nq, nkv, D):
    """Queries after a cache of keys (Nq < Nkv) and more queries than keys
    (the first Nq - Nkv rows see no key: 0 and LSE -inf)."""
    x = inputs.make_inputs(1, 6, 2, nq, nkv, D, inputs.BF16, seed=nq + 3 * nkv)
    o, l = run_gpu(x, None, "bottom_right", gpu_device)
    o_ref, l_ref = oracle_rows(x, None, True, causal_offset=nkv - nq)
    compare(o, l, o_ref, l_ref, inputs.BF16, rounding_allowance=True,
            what=f"bottom-right {nq}x{nkv} D={D}")
    if nq > nkv:
        assert np.all(o[:, :, :nq - nkv] == 0.0)


@pytest.mark.parametrize("splits", [2, 5])
def test_bottom_right_forced_splits(gpu_device, splits):
    x = inputs.make_inputs(1, 4, 4, 300, 2000, 64, inputs.F16, seed=90 + splits)
    o, l = run_gpu(x, None, "bottom_right", gpu_device, num_splits=splits)
    o_ref, l_ref = oracle_rows(x, None, True, causal_offset=1700)
    compare(o, l, o_ref, l_ref, inputs.F16, rounding_allowance=True,
            what=f"bottom-right splits={splits}")


def test_bottom_right_d256_long_rows(gpu_device):
    x = inputs.make_inputs(1, 8, 4, 1000, 3000, 256, inputs.BF16, seed=93, sampled_rows=24)
    o, l = run_gpu(x, None, "bottom_right", gpu_device)
    o_ref, l_ref = oracle_rows(x, None, True, rows=x.rows, causal_offset=2000)
    compare(gather_rows(o, x.rows), gather_rows(l, x.rows), o_ref, l_ref, inputs.BF16,
            rounding_allowance=True, what="bottom-right D=256")


# -- attention masks (PyTorch SDPA attn_mask semantics) -----------------------

def _mask_case(device, B, Hq, Hkv, Nq, Nkv, D, dtype, kind, seed, causal=False, splits=0,
               mshape=None, Dv=None):
    """kind "bool": random keep mask (one row left with no key); "add": an
    additive mask in the inputs' dtype with -inf entries; "pad": key padding
    per batch (batch 1 keeps no key at all).  The mask is broadcast from
    ``mshape`` (default [B, 1, Nq, Nkv])."""
    import torch
    import oracle
    from memory_efficient_tiled_amd import attn_fwd
    log(f"mask case {kind} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} {dtype} "
        f"causal={causal} splits={splits}")
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=seed, Dv=Dv)
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    mshape = mshape or (B, 1, Nq, Nkv)
    if kind == "bool":
        keep = rng.random(mshape) < 0.7
        keep[(0,) * (len(mshape) - 2) + (min(3, mshape[-2] - 1),)] = False
        mt, bias = torch.from_numpy(keep).to(device), np.where(keep, 0.0, -np.inf)
    elif kind == "add":
        a = (2.0 * rng.standard_normal(mshape)).astype(np.float32)
        a[rng.random(mshape) < 0.2] = -np.inf
        st = inputs.to_storage(a, dtype)
        mt = to_device(st, dtype, device)
        bias = oracle.decode(st, dtype)
    else:  # key padding: batch b keeps its first n_b keys
        keep = np.zeros((B, 1, 1, Nkv), dtype=bool)
        for b in range(B):
            keep[b, ..., : (Nkv * 2) // 3 if b != 1 else 0] = True
        mt, bias = torch.from_numpy(keep).to(device), np.where(keep, 0.0, -np.inf)
    q, k, v = (to_device(a, dtype, device) for a in (x.q, x.k, x.v))
    o, l = attn_fwd(q, k, v, causal=causal, mask=mt, num_splits=splits)
    torch.cuda.synchronize(device)
    o = o.float().cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    sc = oracle.scale_value(None, D)
    off = Nkv - Nq if causal == "bottom_right" else 0
    o_ref, l_ref = oracle.attention(oracle.decode(x.q, dtype), oracle.decode(x.k, dtype),
                                    oracle.decode(x.v, dtype), sc, bool(causal),
                                    causal_offset=off,
                                    bias=np.broadcast_to(bias, (B, Hq, Nq, Nkv)))
    # A strong additive bias concentrates a row's weight on few keys, where
    # rounding P to the 16-bit MFMA operand (relative 2^-9 bf16, 2^-12 fp16)
    # moves o by up to that fraction of sum_j P_ij |v_j|: the oracle's
    # attention with |V| as the values gives that sum exactly.
    u = 2.0 ** -8 if dtype == inputs.BF16 else 2.0 ** -11
    pv, _ = oracle.attention(oracle.decode(x.q, dtype), oracle.decode(x.k, dtype),
                             np.abs(oracle.decode(x.v, dtype)), sc, bool(causal),
                             causal_offset=off, bias=np.broadcast_to(bias, (B, Hq, Nq, Nkv)))
    compare(o, l, o_ref, l_ref, dtype, rounding_allowance=True,
            what=f"mask {kind} {Nq}x{Nkv} D={D}", extra=u * pv)
    empty = np.isneginf(l_ref)
    assert np.all(o[empty] == 0.0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("kind", ["bool", "add", "pad"])
def test_masks(gpu_device, kind, dtype, D):
    # 301 keys: rows of the mask are padded to a multiple of 4 by the binding
    _mask_case(gpu_device, 2, 4, 2, 200, 301, D, dtype, kind, seed=D + len(kind))


@pytest.mark.parametrize("kind", ["bool", "add"])
def test_masks_per_head_causal_split(gpu_device, kind):
    _mask_case(gpu_device, 1, 6, 3, 130, 700, 64, inputs.BF16, kind, seed=95,
               causal="bottom_right", splits=3, mshape=(1, 6, 130, 700))


@pytest.mark.parametrize("D", [80, 96, 256])
def test_masks_other_head_dims(gpu_device, D):
    _mask_case(gpu_device, 1, 4, 4, 150, 260, D, inputs.F16, "add", seed=D)


@pytest.mark.parametrize("kind,nq,mshape", [
    ("bool", 4, (2, 8, 4, 300)),     # per-head mask: packs (head stride = Nq rows)
    ("pad", 1, None),                # key padding [B, 1, 1, Nkv]: packs
    ("add", 1, (2, 1, 1, 300)),      # one row per head, broadcast over heads: packs
    ("add", 3, (2, 1, 3, 300)),      # broadcast over heads with 3 rows: not packed
])
def test_masks_gqa_short_queries(gpu_device, kind, nq, mshape):
    _mask_case(gpu_device, 2, 8, 1, nq, 300, 64, inputs.BF16, kind, seed=97 + nq,
               mshape=mshape)


def test_mask_long_rows_sampled(gpu_device):
    """A 2-D boolean mask over 4096 keys, broadcast over batch and heads."""
    _mask_case(gpu_device, 1, 8, 8, 256, 4096, 128, inputs.BF16, "bool", seed=96,
               mshape=(256, 4096))


# -- split of the last partial round ---------------------------------------
# Grids that fill the device but end in a partial round of workgroups cut
# only that round's tiles over their key range (first split tile inside a
# head, ragged last query tile, GQA), for both tile widths.

@pytest.mark.parametrize("shape,dtype", [
    ((1, 26, 26, 2600, 2000, 128), inputs.BF16),
    ((1, 26, 13, 2600, 2000, 128), inputs.F16),
    ((1, 40, 8, 1700, 1000, 64), inputs.BF16),
])
def test_last_round_split(gpu_device, shape, dtype):
    from memory_efficient_tiled_amd import attn_fwd_plan
    B, Hq, Hkv, Nq, Nkv, D = shape
    p = attn_fwd_plan(B, Hq, Hkv, Nq, Nkv, D, False, 0)
    assert p.num_splits >= 2 and 0 < p.split_rows < B * Hq * Nq
    # 64 sampled rows per head (rows 0 and Nq-1 included) land on both sides
    # of the first split row
    _case(gpu_device, B, Hq, Hkv, Nq, Nkv, D, dtype, False, seed=Hq + D,
          rows=64)


# -- exact properties --------------------------------------------------------

def _dev(x, dtype, device):
    return to_device(x, dtype, device)


@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
def test_causal_row0_is_v0_exactly(gpu_device, dtype):
    import torch
    from memory_efficient_tiled_amd import attn_fwd
    x = inputs.make_inputs(1, 4, 2, 300, 300, 128, dtype, seed=3)
    out, lse = attn_fwd(_dev(x.q, dtype, gpu_device), _dev(x.k, dtype, gpu_device),
                        _dev(x.v, dtype, gpu_device), causal=True)
    torch.cuda.synchronize()
    v = _dev(x.v, dtype, gpu_device)
    for h in range(4):
        assert torch.equal(out[0, h, 0], v[0, h // 2, 0]), f"head {h}"


def test_constant_v(gpu_device):
    import torch
    from memory_efficient_tiled_amd import attn_fwd
    x = inputs.make_inputs(1, 2, 2, 200, 500, 64, inputs.F16, seed=4)
    c = np.linspace(-2, 2, 64).astype(np.float16)
    vc = np.broadcast_to(c, x.v.shape).copy()
    out, _ = attn_fwd(_dev(x.q, inputs.F16, gpu_device), _dev(x.k, inputs.F16, gpu_device),
                      _dev(vc, inputs.F16, gpu_device))
    torch.cuda.synchronize()
    err = np.abs(out.float().cpu().numpy() - c.astype(np.float32)).max()
    log(f"  constant V: max|err| {err:.3e}")
    assert err <= 4e-3


def test_deterministic(gpu_device):
    import torch
    from memory_efficient_tiled_amd import attn_fwd
    x = inputs.make_inputs(1, 4, 4, 1000, 3000, 128, inputs.BF16, seed=5)
    args = [_dev(a, inputs.BF16, gpu_device) for a in (x.q, x.k, x.v)]
    for splits in (1, 4):
        o1, l1 = attn_fwd(*args, num_splits=splits)
        o2, l2 = attn_fwd(*args, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_without_lse(gpu_device):
    x = inputs.make_inputs(1, 2, 2, 100, 100, 64, inputs.F16, seed=6)
    o, _ = run_gpu(x, None, False, gpu_device, return_lse=False)
    o_ref, _ = oracle_rows(x, None, False)
    compare(o, None, o_ref, None, inputs.F16, rounding_allowance=True,
            what="no lse")


def test_no_device_allocation_without_split(gpu_device):
    """A call that splits nothing allocates nothing: the library's plan has
    no workspace, and torch's allocator sees only the outputs."""
    import torch
    from memory_efficient_tiled_amd import attn_fwd, attn_fwd_plan
    assert attn_fwd_plan(1, 2, 2, 4096, 4096, 128, False, 1).workspace_bytes > 0
    x = inputs.make_inputs(1, 2, 2, 4096, 4096, 128, inputs.BF16, seed=8)
    args = [_dev(a, inputs.BF16, gpu_device) for a in (x.q, x.k, x.v)]
    out = torch.empty_like(args[0])
    lse = torch.empty(1, 2, 4096, dtype=torch.float32, device=gpu_device)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.max_memory_allocated()
    attn_fwd(*args, out=out, lse=lse, num_splits=1)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
    free0, _ = torch.cuda.mem_get_info()
    assert free0 > 0


@pytest.mark.parametrize("name,splits", [("decode-64k", 0), ("dit-17160", 0),
                                         ("gqa-causal-4096", 2), ("sweep-4096", 4)])
def test_split_path_memory_is_workspace_only(gpu_device, name, splits):
    """Peak device memory of a forward beyond its inputs and preallocated
    outputs: torch's allocator sees nothing, and the stream-ordered pool
    peaks at the plan's workspace (the split partials, O(rows x D)), far
    below one fp32 Nq x Nkv score matrix."""
    import torch
    from memory_efficient_tiled_amd import attn_fwd, attn_fwd_plan
    from tests.parity import PoolPeak
    w = inputs.WORKLOADS[name]
    dt = 1 if w.dtype == inputs.BF16 else 0
    plan = attn_fwd_plan(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.causal, dt, splits)
    ws = plan.workspace_bytes
    # the workspace is the split rows' fp32 partial outputs and LSE: linear in rows
    assert ws == plan.num_splits * plan.split_rows * (w.Dv + 1) * 4
    x = inputs.make_workload_inputs(w, seed=5, sampled_rows=None)
    q, k, v = (to_device(a, w.dtype, gpu_device) for a in (x.q, x.k, x.v))
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=gpu_device)
    attn_fwd(q, k, v, causal=w.causal, out=out, lse=lse, num_splits=splits)   # warm the pool
    torch.cuda.synchronize(gpu_device)
    pool = PoolPeak(gpu_device.index or 0)
    torch.cuda.reset_peak_memory_stats(gpu_device)
    before = torch.cuda.memory_allocated(gpu_device)
    pool.reset()
    attn_fwd(q, k, v, causal=w.causal, out=out, lse=lse, num_splits=splits)
    torch.cuda.synchronize(gpu_device)
    torch_delta = torch.cuda.max_memory_allocated(gpu_device) - before
    peak = pool.read()
    score = 4 * w.B * w.Hq * w.Nq * w.Nkv
    log(f"  {name}: workspace {ws} B, pool peak {peak} B, torch delta {torch_delta} B, "
        f"score matrix {score} B")
    assert torch_delta == 0
    assert ws > 0 and peak >= ws
    assert peak <= ws + (2 << 20)          # pool granularity
    if w.Nq >= 1024:
        assert peak * 15 < score


# -- value rows of another width: (D, Dv) = (192, 128) -----------------------
# 24-chunk K rows and 16-chunk V rows in one kernel (64-key tiles, part of
# Q^T in LDS): ragged query and key tails, GQA, Nq != Nkv, bottom-right
# alignment, forced splits (fp32 partials of Dv columns), strided views,
# masks, and sampled rows of the 8192-token workloads.

@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 63, 65, 1000])
def test_value_width_ragged(gpu_device, n, causal, dtype):
    _case(gpu_device, 2, 4, 2, n, n, 192, dtype, causal, seed=192 + n, Dv=128)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nkv", [(100, 300), (300, 100), (1, 777)])
def test_value_width_nq_ne_nkv(gpu_device, nq, nkv, causal):
    _case(gpu_device, 1, 6, 2, nq, nkv, 192, inputs.BF16, causal, seed=nq + nkv, Dv=128)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_value_width_forced_splits(gpu_device, splits, causal):
    _case(gpu_device, 1, 3, 1, 200, 1500, 192, inputs.BF16, causal, seed=splits,
          num_splits=splits, Dv=128)


@pytest.mark.parametrize("nq,nkv", [(100, 1000), (700, 90)])
def test_value_width_bottom_right(gpu_device, nq, nkv):
    x = inputs.make_inputs(1, 4, 2, nq, nkv, 192, inputs.BF16, seed=nq + 5 * nkv, Dv=128)
    o, l = run_gpu(x, None, "bottom_right", gpu_device)
    o_ref, l_ref = oracle_rows(x, None, True, causal_offset=nkv - nq)
    compare(o, l, o_ref, l_ref, inputs.BF16, rounding_allowance=True,
            what=f"bottom-right {nq}x{nkv} D=192 Dv=128")


def test_value_width_strided(gpu_device):
    """[B, N, H, E] storage for Q, K (E = 192) and V, out (E = 128), viewed
    as [B, H, N, E]: each tensor's sequence stride is H times its own row."""
    import torch
    from memory_efficient_tiled_amd import attn_fwd
    x = inputs.make_inputs(2, 4, 2, 300, 333, 192, inputs.F16, seed=193, Dv=128)
    q, k, v = (to_device(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), inputs.F16,
                         gpu_device).transpose(1, 2) for a in (x.q, x.k, x.v))
    out = torch.empty(2, 300, 4, 128, dtype=torch.float16, device=gpu_device).transpose(1, 2)
    _, lse = attn_fwd(q, k, v, causal=True, out=out)
    torch.cuda.synchronize(gpu_device)
    o_ref, l_ref = oracle_rows(x, None, True)
    compare(out.float().cpu().numpy().astype(np.float64),
            lse.cpu().numpy().astype(np.float64), o_ref, l_ref, inputs.F16,
            rounding_allowance=True, what="D=192 Dv=128 strided")


@pytest.mark.parametrize("kind", ["bool", "add"])
def test_value_width_masks(gpu_device, kind):
    _mask_case(gpu_device, 2, 4, 2, 150, 301, 192, inputs.BF16, kind, seed=194 + len(kind),
               Dv=128)


def test_value_width_mask_causal_split(gpu_device):
    _mask_case(gpu_device, 1, 4, 2, 130, 700, 192, inputs.F16, "add", seed=195,
               causal="bottom_right", splits=3, mshape=(1, 4, 130, 700), Dv=128)


@pytest.mark.parametrize("name", ["hd192v128-8192", "hd192v128-causal-8192"])
def test_value_width_workloads(gpu_device, name):
    _workload(gpu_device, name, rows=48)
