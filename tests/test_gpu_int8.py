"""GPU parity of the INT8 KV cache against the fp64 CPU oracle (needs an MI355X).

INT8 pools hold per-(block, KV head) tiles of codes followed by one fp32
scale per token.  The quantising cache write (separate and fused into the
decode launch) and block copies must match the oracle bit for bit: both
sides quantise in fp32 with correctly rounded division.  The attention
output over code * scale must match the oracle's fp64 result within 2e-2,
the 16-bit bound: the kernel widens codes exactly to the query type and
rounds only the weight * V-scale products, as the 16-bit path rounds the
weights.  Unused tail slots and unreferenced blocks carry NaN scales, so a
read past a context shows up as NaN.  Every call goes through the C ABI.
"""
import numpy as np
import pytest

from oracle import oracle
from paged_kv_cache_328_amd import pagedattn as pa
from paged_kv_cache_328_amd import workloads as wl
import tests._gpu as _g
from tests._gpu import (TOL, announce, check_attention, i8_scale_min, ints_to_dev, pool_dtype,
                        same_bits, tail_slots, to_dev, to_host)

pytestmark = pytest.mark.gpu

NAN32 = np.frombuffer(np.float32(np.nan).tobytes(), np.uint8)


def _sync():
    import torch
    torch.cuda.synchronize()


def poison_scales(kp, vp, slots, Hkv, D, BS):
    """NaN scales for the given slots (every KV head) of two host INT8 pools:
    a token whose scale is read turns its logit or its V contribution into NaN."""
    kflat, vflat = kp.reshape(-1), vp.reshape(-1)
    for slot in np.asarray(slots, np.int64).tolist():
        b, o = divmod(int(slot), BS)
        for h in range(Hkv):
            so = oracle.i8_offsets(b, h, o, 0, Hkv, D, BS)[2]
            kflat[so:so + 4] = NAN32
            vflat[so:so + 4] = NAN32


def run_i8_decode(case, label, partition_size=None, fused=False, r=0):
    """Decode over 8-bit pools (case.kv_dtype "i8" or "fp8").  Separate:
    pa_write_kv_i8 / pa_write_kv_fp8 of the step's tokens, pools compared with
    the oracle's write, then pa_decode.  Fused: the slot of position c - 1 is
    poisoned first and pa_decode appends the token itself; the touched blocks
    must equal the oracle's write."""
    import torch
    dtype, fmt = case.dtype, case.kv_dtype
    assert fmt in ("i8", "fp8")
    pt = pool_dtype(fmt)
    write = pa.pa_write_kv_fp8 if fmt == "fp8" else pa.pa_write_kv_i8
    tables = np.ascontiguousarray(case.block_tables[r])
    lens = case.context_lens
    kp, vp = case.k_cache, case.v_cache
    Hkv, D, BS = case.Hkv, case.D, case.BS
    poison_scales(kp, vp, tail_slots(tables, lens, BS), Hkv, D, BS)
    slots = np.ascontiguousarray(case.slot_mapping[r])
    live = slots >= 0
    if fused:
        poison_scales(kp, vp, slots[live], Hkv, D, BS)
    announce(f"{label}: upload {fmt} pools NB={case.NB} S={case.S} Hq={case.Hq} Hkv={Hkv} "
             f"D={D} BS={BS} q={dtype} max_ctx={case.max_context}")
    kd, vd = to_dev(kp, pt), to_dev(vp, pt)
    k_new, v_new = np.ascontiguousarray(case.new_k[r]), np.ascontiguousarray(case.new_v[r])
    kn, vn = to_dev(k_new, dtype), to_dev(v_new, dtype)
    oracle.write_kv_i8(k_new, v_new, dtype, kp, vp, slots, D, BS, fmt=fmt)
    if not fused:
        announce(f"{label}: {fmt} write T={case.S}")
        write(kn, vn, kd, vd, ints_to_dev(slots))
        _sync()
        assert same_bits(to_host(kd, pt), kp), f"{label}: K pool after the {fmt} write"
        assert same_bits(to_host(vd, pt), vp), f"{label}: V pool after the {fmt} write"
    q = np.ascontiguousarray(case.q[r])
    qd = to_dev(q, dtype)
    out = torch.empty_like(qd)
    P = case.partition_size if partition_size is None else partition_size
    announce(f"{label}: pa_decode {fmt} P={P} fused={fused}")
    extra = dict(k_new=kn, v_new=vn) if fused else {}
    pa.pa_decode(out, qd, kd, vd, ints_to_dev(tables), ints_to_dev(lens), case.scale,
                 case.max_context, partition_size=P, **extra)
    _sync()
    if fused:
        touched = np.unique(slots[live] // BS)
        idx = torch.from_numpy(touched.astype(np.int64)).to(_g.DEVICE)
        assert same_bits(to_host(kd.view(torch.uint8).index_select(0, idx), "u8"), kp[touched]), \
            f"{label}: K blocks"
        assert same_bits(to_host(vd.view(torch.uint8).index_select(0, idx), "u8"), vp[touched]), \
            f"{label}: V blocks"
    want = oracle.decode_i8(q, dtype, kp, vp, tables, lens, case.scale, D, BS, num_threads=16, bound=True,
                            fmt=fmt)
    return (check_attention(to_host(out, dtype), want, dtype, label, kv_scale_min=i8_scale_min(vp, D, BS)),
            to_host(out, dtype))


# ---------------------------------------------------------------------------- cache write / copy

@pytest.mark.parametrize("src", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D,BS", [(64, 16), (128, 16), (128, 32), (48, 8), (256, 16)])
def test_write_kv_i8_bit_exact(src, D, BS):
    """Quantising write: codes and scales equal the oracle's bit for bit.  The
    batch holds padding slots, a zero row (scale 0), rows of widely different
    magnitude and rows whose maximum sits in either sign."""
    rng = np.random.default_rng(2100 + D + BS)
    NB, Hkv, T = 24, 3, 40
    tile = wl.i8_tile_bytes(D, BS)
    kp = rng.integers(0, 256, size=(NB, Hkv, tile), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(NB, Hkv, tile), dtype=np.uint8)
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[[3, 17]] = -1
    mag = np.exp(rng.uniform(-6, 6, size=(T, Hkv, 1))).astype(np.float32)
    k32 = rng.standard_normal((T, Hkv, D), dtype=np.float32) * mag
    v32 = rng.standard_normal((T, Hkv, D), dtype=np.float32) * mag
    k32[5, 1] = 0.0
    v32[6, 2] = 0.0
    k32[7, 0, 3] = -50.0 * mag[7, 0, 0]
    kn, vn = wl.round_to_storage(k32, src), wl.round_to_storage(v32, src)
    kd, vd = to_dev(kp, "u8"), to_dev(vp, "u8")
    announce(f"pa_write_kv_i8 src={src} D={D} BS={BS} T={T}")
    pa.pa_write_kv_i8(to_dev(kn, src), to_dev(vn, src), kd, vd, ints_to_dev(slots))
    _sync()
    oracle.write_kv_i8(kn, vn, src, kp, vp, slots, D, BS)
    assert same_bits(to_host(kd, "u8"), kp)
    assert same_bits(to_host(vd, "u8"), vp)


def test_copy_blocks_i8_bit_exact():
    rng = np.random.default_rng(2200)
    NB, Hkv, D, BS = 40, 4, 128, 16
    tile = wl.i8_tile_bytes(D, BS)
    kp = rng.integers(0, 256, size=(NB, Hkv, tile), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(NB, Hkv, tile), dtype=np.uint8)
    perm = rng.permutation(NB)
    pairs = np.stack([perm[:10], perm[10:20]], axis=1).astype(np.int32)
    pairs = np.concatenate([pairs, np.array([[-1, 3], [2, NB]], np.int32)])  # skipped
    kd, vd = to_dev(kp, "u8"), to_dev(vp, "u8")
    announce(f"pa_copy_blocks INT8 pairs={pairs.shape[0]}")
    pa.pa_copy_blocks(kd, vd, ints_to_dev(pairs), head_dim=D)
    _sync()
    oracle.copy_blocks_i8(kp, vp, pairs[:-2], D, BS)  # the skipped pairs change nothing
    assert same_bits(to_host(kd, "u8"), kp)
    assert same_bits(to_host(vd, "u8"), vp)


# ---------------------------------------------------------------------------- decode, full size

def test_llama13b_f16_i8_full_size():
    run_i8_decode(wl.llama13b_f16(kv_dtype="i8"), "llama13b f16/i8")


def test_mixed_gqa_bf16_i8_full_size():
    run_i8_decode(wl.mixed_gqa_bf16(kv_dtype="i8"), "mixed_gqa bf16/i8")


def test_long_bf16_i8_full_size_p512():
    run_i8_decode(wl.long_bf16(kv_dtype="i8"), "long bf16/i8")


def test_fused_append_llama13b_f16_i8_full_size():
    run_i8_decode(wl.llama13b_f16(kv_dtype="i8"), "llama13b f16/i8 fused", fused=True)


def test_fused_append_mixed_gqa_bf16_i8_full_size():
    run_i8_decode(wl.mixed_gqa_bf16(kv_dtype="i8"), "mixed_gqa bf16/i8 fused", fused=True)


# ---------------------------------------------------------------------------- edge cases

EDGE_LENS = [0, 1, 2, 15, 16, 17, 32, 33, 64, 65, 100, 129, 257]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,BS", [(64, 16), (64, 32), (128, 16), (128, 32), (64, 8), (128, 8), (128, 64)])
@pytest.mark.parametrize("Hq,Hkv,P", [(4, 4, 0), (12, 4, 32), (40, 2, 64), (16, 2, 128)])
def test_i8_edge_shapes(fused, dtype, D, BS, Hq, Hkv, P):
    if P and P % BS:
        pytest.skip("partition size must be a multiple of the block size")
    case = wl.random_case(2300 + D + BS + Hq + P, len(EDGE_LENS), Hq, Hkv, D, BS, dtype, EDGE_LENS,
                          partition_size=P, kv_dtype="i8")
    run_i8_decode(case, f"i8 {dtype} D{D} BS{BS} {Hq}/{Hkv} P{P}", fused=fused)


@pytest.mark.parametrize("P", [0, 32, 128, 512, 2048])
def test_i8_partition_sizes(P):
    lens = [1, 31, 32, 33, 511, 512, 513, 1500, 3000]
    case = wl.random_case(2400, len(lens), 32, 8, 128, 16, "bf16", lens, partition_size=P,
                          kv_dtype="i8")
    run_i8_decode(case, f"i8 partition P={P}", fused=True)


@pytest.mark.parametrize("BS,P", [(16, 8192), (32, 16384), (8, 4096), (64, 16384)])
def test_i8_long_partitions(BS, P):
    """Partitions long enough that each wave reloads its block ids."""
    lens = [4095, 8193, 20000, 33000]
    case = wl.random_case(2450 + BS, len(lens), 8, 2, 128, BS, "f16", lens, partition_size=P,
                          kv_dtype="i8")
    run_i8_decode(case, f"i8 long partition BS={BS} P={P}", fused=True)


def test_i8_matches_16_bit_path_on_exactly_representable_values():
    """Where code * scale is exact in the query type (scales powers of two),
    the INT8 decode sees the same values as a 16-bit decode over the
    dequantised pool; the two outputs then differ only by the rounding of the
    weights, within the 16-bit tolerance of each other and of the oracle."""
    import torch
    lens = [7, 64, 300, 1000]
    case = wl.random_case(2500, len(lens), 16, 4, 128, 16, "bf16", lens, partition_size=256,
                          kv_dtype="i8")
    Hkv, D, BS = case.Hkv, case.D, case.BS
    tile = wl.i8_tile_bytes(D, BS)
    rng = np.random.default_rng(2501)
    for pool in (case.k_cache, case.v_cache):
        sc = (2.0 ** rng.integers(-7, -4, size=(case.NB, Hkv, BS))).astype(np.float32)
        pool[:, :, D * BS:] = sc.view(np.uint8).reshape(case.NB, Hkv, 4 * BS)
    tables = np.ascontiguousarray(case.block_tables[0])
    lens_a = case.context_lens
    # dequantised 16-bit pools: K codes [D/16][BS][16] regrouped into the
    # 16-bit K layout [D/8][BS][8]; V codes [D][BS] already in V's layout
    NB = case.NB
    kc = case.k_cache[:, :, :D * BS].view(np.int8).reshape(NB, Hkv, D // 16, BS, 2, 8)
    kc = kc.transpose(0, 1, 2, 4, 3, 5).reshape(NB, Hkv, D // 8, BS, 8).astype(np.float32)
    vc = case.v_cache[:, :, :D * BS].view(np.int8).reshape(NB, Hkv, D, BS).astype(np.float32)
    ks = case.k_cache[:, :, D * BS:].copy().view(np.float32)  # [NB, Hkv, BS]
    vs = case.v_cache[:, :, D * BS:].copy().view(np.float32)
    k16 = kc * ks[:, :, None, :, None]
    v16 = vc * vs[:, :, None, :]
    kf, vf = case.k_cache.reshape(-1), case.v_cache.reshape(-1)
    for b, h, o, d in [(0, 0, 0, 0), (3, 1, 5, 17), (NB - 1, Hkv - 1, BS - 1, D - 1), (7, 2, 9, 100)]:
        ko, vo, so = oracle.i8_offsets(b, h, o, d, Hkv, D, BS)
        s_k = np.frombuffer(kf[so:so + 4].tobytes(), np.float32)[0]
        s_v = np.frombuffer(vf[so:so + 4].tobytes(), np.float32)[0]
        assert k16[b, h, d // 8, o, d % 8] == np.float32(kf[ko:ko + 1].view(np.int8)[0]) * s_k
        assert v16[b, h, d, o] == np.float32(vf[vo:vo + 1].view(np.int8)[0]) * s_v
    k16 = wl.round_to_storage(k16, "bf16")
    v16 = wl.round_to_storage(v16, "bf16")
    q = np.ascontiguousarray(case.q[0])
    qd = to_dev(q, "bf16")
    o8, o16 = torch.empty_like(qd), torch.empty_like(qd)
    td, ld = ints_to_dev(tables), ints_to_dev(lens_a)
    announce("i8 vs 16-bit on exact values")
    pa.pa_decode(o8, qd, to_dev(case.k_cache, "u8"), to_dev(case.v_cache, "u8"), td, ld, case.scale,
                 case.max_context, partition_size=256)
    pa.pa_decode(o16, qd, to_dev(k16, "bf16"), to_dev(v16, "bf16"), td, ld, case.scale,
                 case.max_context, partition_size=256)
    _sync()
    want = oracle.decode_i8(q, "bf16", case.k_cache, case.v_cache, tables, lens_a, case.scale, D, BS,
                            num_threads=16, bound=True)
    want16 = oracle.decode(q, k16, v16, tables, lens_a, case.scale, "bf16", num_threads=16, bound=True)
    assert np.max(np.abs(want.out - want16.out)) < 1e-12  # the oracles agree on exact values
    check_attention(to_host(o8, "bf16"), want, "bf16", "i8 exact values",
                    kv_scale_min=i8_scale_min(case.v_cache, D, BS))
    check_attention(to_host(o16, "bf16"), want, "bf16", "16-bit over dequantised pool")
    a8 = wl.storage_to_f32(to_host(o8, "bf16"), "bf16")
    a16 = wl.storage_to_f32(to_host(o16, "bf16"), "bf16")
    assert float(np.max(np.abs(a8 - a16))) <= TOL["bf16"]
