"""Oracle: per-block flattening, sharding, reassembly and slot sizing.

Follows [Aug] section 2 "Weight Sharding with AllGather Reconstruction" (the
``_shard_and_pin`` description: ceil-division shard size, zero padding so that
all shards are equal, one flat buffer per dtype) and [Jul] "How It Works /
Weight Sharding + AllGather" (parameters flattened by dtype, split into equal
shards, reassembled by ``all_gather_into_tensor``, whose output is the
rank-ordered concatenation of the shards).  Slot sizing follows [Aug] section 3
and [Jul] "Double-Buffer Memory Bound": two buffers, each sized to the largest
block.

Readings where the pages are silent:

* dtype groups are ordered by first appearance in the parameter list;
* inside a slot, group g's region starts at the previous region's end rounded
  up to ``align`` bytes (256); the block's extent is its last region's end
  rounded up the same way; bytes between regions are never written;
* a group with N_g = 0 has S_g = 0 and an empty region.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# element types of the block forms: bf16 and fp32 parameters, E4M3 ("fp8"),
# int8 ("i8") and E8M0 block scales ("e8m0") of the online-quantised forms
ELEMENT_BYTES = {"bf16": 2, "f32": 4, "fp8": 1, "i8": 1, "e8m0": 1}
NUMPY_DTYPE = {"bf16": np.uint16, "f32": np.float32, "fp8": np.uint8, "i8": np.int8, "e8m0": np.uint8}


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def align_up(v: int, a: int) -> int:
    return ceil_div(v, a) * a


@dataclass
class GroupPlan:
    dtype: str
    members: list          # parameter indices (registration order) in this group
    offsets: list          # element offset of each member inside the flat group buffer
    numel: int             # N_g
    shard: int             # S_g = ceil(N_g / k)
    region: int            # byte offset of the group's region inside the slot

    @property
    def elt(self) -> int:
        return ELEMENT_BYTES[self.dtype]


@dataclass
class BlockPlan:
    k: int
    groups: list           # list[GroupPlan] in first-appearance order
    extent: int            # bytes of the slot this block occupies (aligned)
    param_group: list      # param index -> group index
    param_offset: list     # param index -> element offset within its group

    def region_bytes(self, g: int) -> int:
        gp = self.groups[g]
        return self.k * gp.shard * gp.elt

    def shard_bytes(self, g: int) -> int:
        gp = self.groups[g]
        return gp.shard * gp.elt

    def param_byte_offset(self, p: int) -> int:
        """Byte offset of parameter p inside the slot (the zero-copy re-point)."""
        g = self.param_group[p]
        return self.groups[g].region + self.param_offset[p] * self.groups[g].elt


def plan_block(specs, k: int, align: int = 256) -> BlockPlan:
    """Plan one block.  ``specs`` = [(name, dtype, numel), ...] in registration order.

    [Aug] s.2: shard_size = ceil(total_numel / dp_size) per flat dtype buffer.
    """
    if k < 1:
        raise ValueError("k must be >= 1")
    order = []
    for _, dt, _ in specs:
        if dt not in ELEMENT_BYTES:
            raise ValueError(f"unknown dtype {dt}")
        if dt not in order:
            order.append(dt)
    groups = []
    param_group = [None] * len(specs)
    param_offset = [None] * len(specs)
    for gi, dt in enumerate(order):
        members, offs, run = [], [], 0
        for p, (_, pdt, numel) in enumerate(specs):
            if pdt != dt:
                continue
            if numel < 0:
                raise ValueError("negative numel")
            members.append(p)
            offs.append(run)
            param_group[p] = gi
            param_offset[p] = run
            run += int(numel)
        groups.append(GroupPlan(dt, members, offs, run, ceil_div(run, k), 0))
    cursor = 0
    for gp in groups:
        gp.region = cursor
        cursor = align_up(cursor + k * gp.shard * ELEMENT_BYTES[gp.dtype], align)
    return BlockPlan(k, groups, cursor, param_group, param_offset)


def plan_stack(blocks_specs, k: int, align: int = 256):
    """Plans for every block plus the slot size (= largest extent).

    [Aug] s.3: the two shared buffers are allocated once to the max block size.
    """
    plans = [plan_block(s, k, align) for s in blocks_specs]
    slot_bytes = max((p.extent for p in plans), default=0)
    return plans, slot_bytes


def specs_of(params):
    """[(name, dtype, ndarray)] -> [(name, dtype, numel)]."""
    return [(n, dt, int(a.size)) for n, dt, a in params]


def flat_group(params, bp: BlockPlan, g: int) -> np.ndarray:
    """The flat dtype buffer of group g: members concatenated in registration order."""
    gp = bp.groups[g]
    parts = [np.ascontiguousarray(params[p][2]).reshape(-1) for p in gp.members]
    dt = NUMPY_DTYPE[gp.dtype]
    if not parts:
        return np.zeros(0, dtype=dt)
    return np.concatenate([x.view(dt) for x in parts])


def pack_block(params, bp: BlockPlan):
    """Host shards of one block: shards[g][r] is an array of S_g elements.

    [Aug] s.2: shard r holds flat[r*S : (r+1)*S], zero where that range runs
    past N (ceil division + zero padding makes every shard equal-sized).
    """
    out = []
    for g, gp in enumerate(bp.groups):
        flat = flat_group(params, bp, g)
        rows = []
        for r in range(bp.k):
            shard = np.zeros(gp.shard, dtype=flat.dtype)
            lo, hi = r * gp.shard, min((r + 1) * gp.shard, gp.numel)
            if hi > lo:
                shard[: hi - lo] = flat[lo:hi]
            rows.append(shard)
        out.append(rows)
    return out


def reassemble(shards_g) -> np.ndarray:
    """all_gather_into_tensor output: the rank-ordered concatenation of the shards.

    [Jul] "Weight Sharding + AllGather", step 2.
    """
    if not shards_g:
        return np.zeros(0)
    return np.concatenate(shards_g)


def slot_regions(bp: BlockPlan, shards):
    """Expected bytes of each region of a slot holding this block: [(offset, bytes)]."""
    regs = []
    for g, gp in enumerate(bp.groups):
        buf = reassemble(shards[g]).view(np.uint8)
        regs.append((gp.region, buf))
    return regs


def weight_footprint(plans) -> int:
    """Peak device weight bytes of the double-buffer scheme: two slots of the largest block.

    [Jul] "Double-Buffer Memory Bound": exactly two blocks resident; HBM use
    depends only on the largest block, not on the block count.
    """
    return 2 * max((p.extent for p in plans), default=0)


# ---------------------------------------------------------------------------
# Slot digest: the race-detector definition (test instrumentation, not method)
# ---------------------------------------------------------------------------
#
# digest(slot, regions) = sum over regions, over 8-byte little-endian words w
# at byte offset o (relative to the slot base; the last partial word of a
# region is zero-extended), of mix(w + (o / 8) * 0x9E3779B97F4A7C15) mod 2^64,
# with mix the splitmix64 finaliser:
#   z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
#   z ^= z >> 31.
# Integer addition is associative, so any summation order gives one value.

_G = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def digest_regions(regions) -> int:
    """Digest of [(byte_offset, uint8 array)] regions; offsets must be multiples of 8."""
    total = np.uint64(0)
    with np.errstate(over="ignore"):
        for off, buf in regions:
            assert off % 8 == 0
            b = np.asarray(buf, dtype=np.uint8).reshape(-1)
            if b.size == 0:
                continue
            pad = (-b.size) % 8
            if pad:
                b = np.concatenate([b, np.zeros(pad, dtype=np.uint8)])
            w = b.view("<u8").astype(np.uint64)
            idx = np.arange(w.size, dtype=np.uint64) + np.uint64(off // 8)
            total = total + np.sum(_mix64(w + idx * _G), dtype=np.uint64)
    return int(total)
