"""GPU parity of the shared-prefix decode (pa_decode_prefix) against the fp64
CPU oracle (needs an MI355X).

Sequences of a group share their first blocks; pa_decode_prefix reads the
shared prefix once per group and merges it with each member's own tokens.
Its output must equal the oracle's plain decode within 2e-2; with the fused
append the touched pool bytes must equal the oracle's cache write.  NaN
fills unreferenced blocks and the unused tails.
"""
import numpy as np
import pytest

from oracle import oracle
from paged_kv_cache_328_amd import pagedattn as pa
from paged_kv_cache_328_amd import workloads as wl
import tests._gpu as _g
from tests._gpu import (announce, check_attention, i8_scale_min, ints_to_dev, poison_tails,
                        pool_dtype, same_bits, tail_slots, to_dev, to_host)
from tests.test_gpu_int8 import poison_scales

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def run_prefix_case(case, group_start, prefix_len, label, fused=False, partition_size=0,
                    min_prefix=False):
    import torch
    dtype, i8 = case.dtype, wl.is_q8(case.kv_dtype)  # i8: an 8-bit pool (INT8 or FP8)
    tables = np.ascontiguousarray(case.block_tables[0])
    lens = case.context_lens
    kc, vc = case.k_cache, case.v_cache
    if i8:
        poison_scales(kc, vc, tail_slots(tables, lens, case.BS), case.Hkv, case.D, case.BS)
    else:
        poison_tails(oracle, kc, vc, tables, lens, dtype)
    slots = np.ascontiguousarray(case.slot_mapping[0])
    pool_t = pool_dtype(case.kv_dtype) if i8 else dtype
    announce(f"{label}: upload NB={case.NB} S={case.S} groups={len(prefix_len)} Hq={case.Hq} "
             f"Hkv={case.Hkv} D={case.D} BS={case.BS} q={dtype} kv={case.kv_dtype} fused={fused}")
    kd, vd = to_dev(kc, pool_t), to_dev(vc, pool_t)
    k_new, v_new = np.ascontiguousarray(case.new_k[0]), np.ascontiguousarray(case.new_v[0])
    extra = {}
    if fused:
        extra = dict(k_new=to_dev(k_new, dtype), v_new=to_dev(v_new, dtype))
        if i8:
            oracle.write_kv_i8(k_new, v_new, dtype, kc, vc, slots, case.D, case.BS, fmt=case.kv_dtype)
        else:
            oracle.write_kv(k_new, v_new, kc, vc, slots, dtype)
    q = np.ascontiguousarray(case.q[0])
    qd = to_dev(q, dtype)
    out = torch.empty_like(qd)
    max_group = int(np.max(np.diff(group_start)))
    announce(f"{label}: pa_decode_prefix max_group={max_group} P={partition_size}")
    pa.pa_decode_prefix(out, qd, kd, vd, ints_to_dev(tables), ints_to_dev(lens), case.scale,
                        case.max_context, ints_to_dev(group_start), ints_to_dev(prefix_len),
                        max_group, int(np.max(prefix_len)), partition_size=partition_size,
                        min_prefix_len=int(np.min(prefix_len)) if min_prefix else 0, **extra)
    _sync()
    if fused:
        live = slots >= 0
        touched = np.unique(slots[live] // case.BS)
        idx = torch.from_numpy(touched.astype(np.int64)).to(_g.DEVICE)
        kb, vb = (kd.view(torch.uint8), vd.view(torch.uint8)) if i8 else (kd, vd)
        assert same_bits(to_host(kb.index_select(0, idx), pool_t), kc[touched]), f"{label}: K blocks"
        assert same_bits(to_host(vb.index_select(0, idx), pool_t), vc[touched]), f"{label}: V blocks"
    if i8:
        want = oracle.decode_i8(q, dtype, kc, vc, tables, lens, case.scale, case.D, case.BS,
                                num_threads=16, bound=True, fmt=case.kv_dtype)
    else:
        want = oracle.decode(q, kc, vc, tables, lens, case.scale, dtype, num_threads=16, bound=True)
    return (check_attention(to_host(out, dtype), want, dtype, label,
                            kv_scale_min=i8_scale_min(vc, case.D, case.BS) if i8 else None),
            to_host(out, dtype))


GROUPS = [(4, [3, 1, 40, 200]), (0, [7, 1]), (2, [1, 33]), (1, [1]), (6, [16, 17, 64, 1, 5, 9, 90, 2, 3, 4, 5,
                                                                      6, 7, 8, 9, 10, 11, 12])]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,BS", [(128, 16), (64, 32), (128, 8), (128, 64)])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 4), (32, 2)])
@pytest.mark.parametrize("fused", [False, True])
def test_prefix_groups_edge_shapes(dtype, D, BS, Hq, Hkv, fused):
    groups = [(max(1, (nb * 16) // BS) if nb else 0, sfx) for nb, sfx in GROUPS]
    case, gs, shared = wl.shared_prefix_case(4100 + D + BS + Hq, groups, Hq, Hkv, D, BS, dtype)
    run_prefix_case(case, gs, shared, f"prefix {dtype} D{D} BS{BS} {Hq}/{Hkv} fused={fused}", fused=fused)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("min_prefix", [False, True])
def test_prefix_groups_int8(kv, fused, min_prefix):
    case, gs, shared = wl.shared_prefix_case(4200, GROUPS, 32, 8, 128, 16, "bf16", kv_dtype=kv)
    run_prefix_case(case, gs, shared, f"prefix {kv} fused={fused} min_prefix={min_prefix}",
                    fused=fused, min_prefix=min_prefix)


def test_prefix_shorter_than_the_shared_blocks_and_zero():
    """prefix_len may be any count up to the shared tokens (here not a block
    multiple), or 0: the rest is attended per member."""
    case, gs, shared = wl.shared_prefix_case(4300, GROUPS, 16, 4, 128, 16, "f16")
    run_prefix_case(case, gs, np.maximum(shared - 5, 0).astype(np.int32), "prefix shorter by 5")
    case, gs, shared = wl.shared_prefix_case(4300, GROUPS, 16, 4, 128, 16, "f16")
    run_prefix_case(case, gs, np.zeros_like(shared), "prefix 0")


@pytest.mark.parametrize("P", [32, 256, 2048])
def test_prefix_with_partitions(P):
    """Long shared prefix (2048 tokens) and long private suffixes split into partitions."""
    case, gs, shared = wl.shared_prefix_case(4400, [(128, [1, 300, 1500, 2500]), (16, [700, 3])],
                                             32, 8, 128, 16, "bf16")
    run_prefix_case(case, gs, shared, f"prefix partitions P={P}", fused=True, partition_size=P)


def test_long_prefix_doubled_partitions():
    """Prefixes past 16,384 tokens take 512-token prefix partitions (at most
    64 prefix partials per row reach the merge): two groups sharing 17,600 and
    16,480 tokens."""
    case, gs, shared = wl.shared_prefix_case(4600, [(1100, [1, 40, 300]), (1030, [5, 64])],
                                             8, 2, 128, 16, "bf16")
    assert int(np.max(shared)) > 16384
    run_prefix_case(case, gs, shared, "long prefix", fused=True)


@pytest.mark.parametrize("fused", [False, True])
def test_min_prefix_len_bounds_the_grid(fused):
    """A host lower bound of the prefix lengths shrinks the grid of the
    members' own tokens; every unit that exists computes what it computed
    before, so the output is bit-identical to the call without the bound."""
    import torch
    groups = [(128, [1, 40, 300]), (64, [5, 700]), (70, [33])]
    outs = []
    for bound in (False, True):
        case, gs, shared = wl.shared_prefix_case(4700, groups, 16, 4, 128, 16, "bf16")
        tables = np.ascontiguousarray(case.block_tables[0])
        poison_tails(oracle, case.k_cache, case.v_cache, tables, case.context_lens, "bf16")
        kd, vd = to_dev(case.k_cache, "bf16"), to_dev(case.v_cache, "bf16")
        qd = to_dev(np.ascontiguousarray(case.q[0]), "bf16")
        extra = {}
        if fused:
            extra = dict(k_new=to_dev(np.ascontiguousarray(case.new_k[0]), "bf16"),
                         v_new=to_dev(np.ascontiguousarray(case.new_v[0]), "bf16"))
        out = torch.empty_like(qd)
        lo = int(np.min(shared)) if bound else 0
        announce(f"min prefix bound={lo} fused={fused}")
        pa.pa_decode_prefix(out, qd, kd, vd, ints_to_dev(tables), ints_to_dev(case.context_lens),
                            case.scale, case.max_context, ints_to_dev(gs), ints_to_dev(shared),
                            int(np.max(np.diff(gs))), int(np.max(shared)), min_prefix_len=lo,
                            **extra)
        _sync()
        outs.append(to_host(out, "bf16"))
    assert same_bits(outs[0], outs[1]), "the lower bound of the prefixes changed the output"
    if fused:
        oracle.write_kv(np.ascontiguousarray(case.new_k[0]), np.ascontiguousarray(case.new_v[0]),
                        case.k_cache, case.v_cache, np.ascontiguousarray(case.slot_mapping[0]), "bf16")
    want = oracle.decode(np.ascontiguousarray(case.q[0]), case.k_cache, case.v_cache, tables,
                         case.context_lens, case.scale, "bf16", num_threads=16, bound=True)
    check_attention(outs[1], want, "bf16", f"min prefix bound fused={fused}")


def test_cow_shaped_batch_matches_plain_decode():
    """32 sequences sharing a 2048-token prefix (block size 32) with private
    suffixes of 1..512 tokens: pa_decode_prefix and pa_decode agree."""
    import torch
    rng = np.random.default_rng(4500)
    suffix = rng.integers(1, 512, size=32, endpoint=True).tolist()
    case, gs, shared = wl.shared_prefix_case(4501, [(64, suffix)], 32, 8, 128, 32, "bf16")
    _, got = run_prefix_case(case, gs, shared, "cow-shaped prefix", fused=True)
    case2, _, _ = wl.shared_prefix_case(4501, [(64, suffix)], 32, 8, 128, 32, "bf16")
    tables = np.ascontiguousarray(case2.block_tables[0])
    poison_tails(oracle, case2.k_cache, case2.v_cache, tables, case2.context_lens, "bf16")
    kd, vd = to_dev(case2.k_cache, "bf16"), to_dev(case2.v_cache, "bf16")
    qd = to_dev(np.ascontiguousarray(case2.q[0]), "bf16")
    out = torch.empty_like(qd)
    announce("cow-shaped: pa_decode")
    pa.pa_decode(out, qd, kd, vd, ints_to_dev(tables), ints_to_dev(case2.context_lens), case2.scale,
                 case2.max_context, k_new=to_dev(case2.new_k[0], "bf16"),
                 v_new=to_dev(case2.new_v[0], "bf16"))
    _sync()
    a = wl.storage_to_f32(got, "bf16")
    b = wl.storage_to_f32(to_host(out, "bf16"), "bf16")
    assert float(np.max(np.abs(a - b))) <= 2e-2
