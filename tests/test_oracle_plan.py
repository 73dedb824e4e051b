"""Pins for oracle.plan: sharding, reassembly identity, slot sizes, footprint, digest."""
import os
import random

import numpy as np
import pytest

import synth
from oracle import plan as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([int(v) for v in line.split()])
    return rows


def _schema_specs(d):
    return [(n, dt, int(np.prod(s))) for n, dt, s in synth.block_schema(d)]


@pytest.mark.parametrize("row", _read_rows("slot_sizes.txt"))
def test_slot_sizes_match_hand_worked_values(row):
    d, k, n_bf, s_bf, n_f32, s_f32, f32_region, extent = row
    bp = op.plan_block(_schema_specs(d), k)
    g_bf, g_f32 = bp.groups
    assert (g_bf.dtype, g_f32.dtype) == ("bf16", "f32")
    assert (g_bf.numel, g_bf.shard, g_f32.numel, g_f32.shard) == (n_bf, s_bf, n_f32, s_f32)
    assert (g_bf.region, g_f32.region, bp.extent) == (0, f32_region, extent)


def test_page_example_shard_sizes():
    # "Distributed Layerwise Offload" (blog, 2026-07-30), "Overlap Analysis":
    # a 368 MB block has a 184 MB shard at DP2.
    bp = op.plan_block([("w", "bf16", 184_000_000)], 2)
    assert bp.shard_bytes(0) == 184_000_000
    # vLLM blog section 2: Cosmos3-Super DP4 keeps 124 GB / 4 = 31 GB per rank.
    bp = op.plan_block([("w", "bf16", 62_000_000_000)], 4)
    assert bp.shard_bytes(0) == 31_000_000_000


def test_workload_slot_bytes():
    # slot = the largest block; the irregular stack is sized by its d = 4096 blocks
    for name, want in [("tiny", 2379008), ("8blk", 37826816), ("nano", 339972352),
                       ("super", 944107776), ("irregular", 604291328)]:
        w = synth.WORKLOADS[name]
        plans, slot = op.plan_stack([_schema_specs(d) for d in w.block_widths()], w.k)
        assert slot == want, name


def test_param_offsets_follow_registration_order():
    d = 256
    bp = op.plan_block(_schema_specs(d), 2)
    names = [n for n, _, _ in synth.block_schema(d)]
    off = {n: bp.param_byte_offset(i) for i, n in enumerate(names)}
    # bf16 group: adaLN, qkv, out, fc1, fc2 back to back
    assert off["adaln.weight"] == 0
    assert off["attn.qkv.weight"] == 6 * d * d * 2
    assert off["attn.out.weight"] == 9 * d * d * 2
    assert off["mlp.fc1.weight"] == 10 * d * d * 2
    assert off["mlp.fc2.weight"] == 14 * d * d * 2
    # fp32 group after the padded bf16 region; eps buffers shift what follows by one element
    r = bp.groups[1].region
    assert off["adaln.bias"] == r
    assert off["norm1.weight"] == r + 6 * d * 4
    assert off["norm1.eps"] == r + 8 * d * 4
    assert off["attn.qkv.bias"] == r + (8 * d + 1) * 4
    assert off["mlp.fc2.bias"] == r + (18 * d + 2) * 4


def _random_params(rng, n_params):
    params = []
    for p in range(n_params):
        dt = rng.choice(["bf16", "f32", "fp8"])
        numel = rng.choice([0, 1, 2, 3, 5, 7, 31, 64, 257, rng.randint(0, 5000)])
        if dt == "bf16":
            a = np.array([rng.getrandbits(16) for _ in range(numel)], dtype=np.uint16)
        elif dt == "fp8":
            a = np.array([rng.getrandbits(8) for _ in range(numel)], dtype=np.uint8)
        else:
            a = np.array([rng.uniform(-1, 1) for _ in range(numel)], dtype=np.float32)
        params.append((f"p{p}", dt, a))
    return params


def test_reassembly_identity_randomised():
    """Concatenating the k shards and dropping the padding gives back every parameter's bytes."""
    rng = random.Random(1234)
    for trial in range(150):
        params = _random_params(rng, rng.randint(1, 6))
        k = rng.randint(1, 8)
        bp = op.plan_block(op.specs_of(params), k)
        shards = op.pack_block(params, bp)
        for g, gp in enumerate(bp.groups):
            assert all(s.size == gp.shard for s in shards[g])  # equal shards
            full = op.reassemble(shards[g])
            assert full.size == k * gp.shard >= gp.numel
            assert gp.shard * k - gp.numel < k  # at most k-1 pad elements
            assert not np.any(full[gp.numel:].view(np.uint8))  # padding is zero
            for p, off in zip(gp.members, gp.offsets):
                a = params[p][2].reshape(-1)
                got = full[off:off + a.size]
                assert got.tobytes() == a.tobytes()


def test_reassembly_edge_cases():
    a = np.arange(3, dtype=np.float32)
    # N < k: shards 0..2 hold one element each, the rest are pure padding
    bp = op.plan_block([("a", "f32", 3)], 5)
    sh = op.pack_block([("a", "f32", a)], bp)
    assert bp.groups[0].shard == 1 and [s.tolist() for s in sh[0]] == [[0.0], [1.0], [2.0], [0.0], [0.0]]
    # N = 0: empty shards and an empty region
    bp = op.plan_block([("a", "f32", 0)], 4)
    assert bp.groups[0].shard == 0 and bp.extent == 0
    # k = 1 (no all-gather: shard size forced to one shard per block)
    bp = op.plan_block([("a", "f32", 3)], 1)
    assert op.reassemble(op.pack_block([("a", "f32", a)], bp)[0]).tolist() == [0.0, 1.0, 2.0]


def test_footprint_is_two_largest_blocks_for_any_depth():
    w = synth.WORKLOADS["irregular"]
    for n in (1, 2, 3, 8, 72, 127, 128):
        specs = [_schema_specs(w.width(b)) for b in range(n)]
        plans, slot = op.plan_stack(specs, w.k)
        fp = op.weight_footprint(plans)
        assert fp == 2 * max(p.extent for p in plans) == 2 * slot
        if n >= 3:
            assert fp == 2 * 604291328
        # negative control: one buffer per block grows with depth and exceeds two slots
        per_block = sum(p.extent for p in plans)
        if n >= 8:
            assert per_block > fp


def test_digest_detects_changes_and_is_position_sensitive():
    rng = np.random.default_rng(0)
    buf = rng.integers(0, 256, size=4096 + 5, dtype=np.uint8)
    d0 = op.digest_regions([(0, buf)])
    b2 = buf.copy(); b2[4100] ^= 1
    assert op.digest_regions([(0, b2)]) != d0
    # swapping two words changes the digest (word position enters the mix)
    b3 = buf.copy(); b3[0:8], b3[8:16] = buf[8:16].copy(), buf[0:8].copy()
    assert op.digest_regions([(0, b3)]) != d0
    # the same bytes at another slot offset give another digest
    assert op.digest_regions([(256, buf)]) != d0
    # splitting one region in two at a word boundary does not change it
    assert op.digest_regions([(0, buf[:1024]), (1024, buf[1024:])]) == d0
