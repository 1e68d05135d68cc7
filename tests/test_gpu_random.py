"""A seeded sweep of pa_decode over randomly drawn configurations, each
checked against the fp64 oracle under the parity bound (and, with the fused
append, the stored token bit for bit).

Every case draws: batch size (1..70), KV heads (1..8) and query heads per KV
head (1, 2, 4, 8, 16 or 20), head_dim (64 or 128), block size (8..64),
f16 or bf16 queries, 16-bit or INT8 caches, context lengths (some empty,
some ragged, up to 3000 tokens), the partition size (the library's own or
an explicit multiple of the chunk and block sizes), whether the host copy of
the lengths is passed, whether the append is fused, and (with one query head
per KV head and 16-bit caches) which units compute the products.  So the
flat work list with and without the host's longest-first order, the
(head, partition, sequence) grid, the split and unsplit paths, both merges
and both decoders meet shapes none of the fixed tests spell out.  Unused
tail slots hold NaN (INT8: NaN scales)."""
import numpy as np
import pytest

from oracle import oracle
from paged_kv_cache_328_amd import pagedattn as pa
from paged_kv_cache_328_amd import workloads as wl
from tests import _gpu as _g
from tests._gpu import (announce, check_attention, i8_scale_min, ints_to_dev, poison_tails,
                        pool_dtype, same_bits, tail_slots, to_dev, to_host)
from tests.test_gpu_int8 import poison_scales

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng([2024, seed])
    S = int(rng.integers(1, 71))
    Hkv = int(rng.integers(1, 9))
    G = int(rng.choice([1, 2, 4, 8, 16, 20]))
    D = int(rng.choice([64, 128]))
    BS = int(rng.choice([8, 16, 32, 64]))
    dtype = str(rng.choice(["f16", "bf16"]))
    u = rng.random()
    kv = "i8" if u < 0.3 else "fp8" if u < 0.45 else None
    kind = rng.random()
    if kind < 0.2:
        lens = rng.integers(0, 40, size=S)
    elif kind < 0.6:
        lens = np.rint(np.exp(rng.uniform(0, np.log(3000), size=S))).astype(int)
    else:
        lens = rng.integers(0, 3001, size=S)
    lens[rng.random(S) < 0.05] = 0
    if lens.sum() * Hkv > 250_000:  # keep a case's pools and oracle run small
        lens = (lens * (250_000 / (lens.sum() * Hkv))).astype(int)
    step = max(32, BS)
    P = 0 if rng.random() < 0.5 else int(step * rng.integers(1, max(2, 1024 // step) + 1))
    host = bool(rng.random() < 0.7)
    fused = bool(rng.random() < 0.6)
    products = "auto"
    if G == 1 and kv is None and rng.random() < 0.5:
        products = str(rng.choice(["matrix", "valu"]))
    return dict(S=S, Hkv=Hkv, G=G, D=D, BS=BS, dtype=dtype, kv=kv, lens=[int(c) for c in lens], P=P,
                host=host, fused=fused, products=products)


@pytest.mark.parametrize("seed", range(160))
def test_random_configuration(seed):
    import torch
    c = draw(seed)
    S, Hkv, G, D, BS, dtype, kv = c["S"], c["Hkv"], c["G"], c["D"], c["BS"], c["dtype"], c["kv"]
    lens = c["lens"]
    fused = c["fused"] and max(lens) > 0
    case = wl.random_case(7000 + seed, S, G * Hkv, Hkv, D, BS, dtype, lens, kv_dtype=kv)
    i8 = wl.is_q8(kv)  # an 8-bit pool (INT8 or FP8)
    tables = np.ascontiguousarray(case.block_tables[0])
    lens_np = case.context_lens
    kc, vc = case.k_cache, case.v_cache
    slots = np.ascontiguousarray(case.slot_mapping[0])
    live = slots >= 0
    if i8:
        poison_scales(kc, vc, tail_slots(tables, lens_np, BS), Hkv, D, BS)
        if fused:
            poison_scales(kc, vc, slots[live], Hkv, D, BS)
    else:
        poison_tails(oracle, kc, vc, tables, lens_np, dtype)
        if fused:
            nan = np.full((int(live.sum()), Hkv, D), wl.nan_bits(dtype), wl.NP_STORAGE[dtype])
            oracle.write_kv(nan, nan.copy(), kc, vc, slots[live], dtype)
    label = (f"random seed {seed}: S={S} Hkv={Hkv} G={G} D={D} BS={BS} {dtype} kv={kv} "
             f"max_ctx={case.max_context} P={c['P']} host={c['host']} fused={fused} products={c['products']}")
    pool_t = pool_dtype(kv) if i8 else dtype
    announce(label + ": upload")
    kd, vd = to_dev(kc, pool_t), to_dev(vc, pool_t)
    q = np.ascontiguousarray(case.q[0])
    qd = to_dev(q, dtype)
    extra = {}
    if fused:
        k_new, v_new = np.ascontiguousarray(case.new_k[0]), np.ascontiguousarray(case.new_v[0])
        extra = dict(k_new=to_dev(k_new, dtype), v_new=to_dev(v_new, dtype))
    out = torch.empty_like(qd)
    announce(label + ": pa_decode")
    pa.pa_decode(out, qd, kd, vd, ints_to_dev(tables), ints_to_dev(lens_np), case.scale,
                 max(case.max_context, 1), partition_size=c["P"],
                 context_lens_host=lens_np if c["host"] else None, products=c["products"], **extra)
    torch.cuda.synchronize()
    got = to_host(out, dtype)
    if fused:
        touched = np.unique(slots[live] // BS)
        idx = torch.from_numpy(touched.astype(np.int64)).to(_g.DEVICE)
        if i8:
            oracle.write_kv_i8(k_new, v_new, dtype, kc, vc, slots, D, BS, fmt=kv)
        else:
            oracle.write_kv(k_new, v_new, kc, vc, slots, dtype)
        kb, vb = (kd.view(torch.uint8), vd.view(torch.uint8)) if i8 else (kd, vd)
        assert same_bits(to_host(kb.index_select(0, idx), pool_t), kc[touched]), label + ": K blocks"
        assert same_bits(to_host(vb.index_select(0, idx), pool_t), vc[touched]), label + ": V blocks"
    if i8:
        want = oracle.decode_i8(q, dtype, kc, vc, tables, lens_np, case.scale, D, BS, num_threads=16,
                                bound=True, fmt=kv)
    else:
        want = oracle.decode(q, kc, vc, tables, lens_np, case.scale, dtype, num_threads=16, bound=True)
    check_attention(got, want, dtype, label, kv_scale_min=i8_scale_min(vc, D, BS) if i8 else None)


def draw_prefill(seed):
    rng = np.random.default_rng([2025, seed])
    S = int(rng.integers(1, 71))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    D = int(rng.choice([64, 128]))
    BS = int(rng.choice([8, 16, 32, 64]))
    dtype = str(rng.choice(["f16", "bf16"]))
    u = rng.random()
    kv = "i8" if u < 0.35 else "fp8" if u < 0.5 else None
    priors = rng.integers(0, 400, size=S)
    chunks = rng.integers(0, 200, size=S)
    priors[rng.random(S) < 0.2] = 0
    tot = int((priors + chunks).sum()) * Hkv
    if tot > 120_000:  # keep a case's pools and oracle run small
        f = 120_000 / tot
        priors, chunks = (priors * f).astype(int), (chunks * f).astype(int)
    if chunks.sum() == 0:
        chunks[0] = 1
    return dict(S=S, Hkv=Hkv, G=G, D=D, BS=BS, dtype=dtype, kv=kv,
                priors=[int(x) for x in priors], chunks=[int(x) for x in chunks])


@pytest.mark.parametrize("seed", range(32))
def test_random_prefill_configuration(seed):
    """pa_prefill over drawn batches (1..70 sequences, so both the ranked and
    the unranked grid order), chunks of 0..199 rows on 0..399 earlier tokens,
    1..4 KV heads with 1..16 query heads each, both head_dims, every block
    size, f16/bf16, 16-bit or INT8 caches."""
    from tests.test_gpu_prefill import run_prefill
    c = draw_prefill(seed)
    case = wl.prefill_case(8000 + seed, c["priors"], c["chunks"], c["G"] * c["Hkv"], c["Hkv"], c["D"],
                           c["BS"], c["dtype"], kv_dtype=c["kv"])
    run_prefill(case, f"random prefill seed {seed}: S={c['S']} Hkv={c['Hkv']} G={c['G']} D={c['D']} "
                      f"BS={c['BS']} {c['dtype']} kv={c['kv']}")
