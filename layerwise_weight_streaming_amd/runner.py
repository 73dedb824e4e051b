"""Device-memory plumbing around libdlo for one GPU, using PyTorch allocations.

PyTorch provides device memory (the two slots, x, cond, the workspace) and two
HIP streams; libdlo does all the work.  Nothing here computes any part of the
forward.
"""
from __future__ import annotations

import numpy as np

from . import HostStore, Plan, forward_stack, place_block


class StackRunner:
    """One streamed DiT stack on cuda:``device``.

    blocks: [(d_model, n_heads, [(name, dtype, numel)])] -- the plan's shapes.
    """

    def __init__(self, blocks, k, tokens, D, pinned=True, device=0, store_mode=None, pinned_limit=0, batch=1):
        import torch

        self.torch = torch
        self.dev = torch.device("cuda", device)
        self.plan = Plan(blocks, k)
        self.store = HostStore(self.plan, pinned=pinned, mode=store_mode, pinned_limit=pinned_limit)
        self.tokens, self.D, self.batch = tokens, D, batch
        self.n_blocks = len(blocks)
        sb = self.plan.slot_bytes
        # exactly two slots, each the size of the largest block
        before = torch.cuda.memory_allocated(self.dev)
        self.slots = [torch.empty(sb, dtype=torch.uint8, device=self.dev) for _ in range(2)]
        self.slot_alloc_bytes = torch.cuda.memory_allocated(self.dev) - before
        self.ws_bytes = self.plan.workspace_bytes(tokens)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.dev)
        self.x = torch.zeros((batch * tokens, D), dtype=torch.float32, device=self.dev)
        self.cond = torch.zeros((batch, D) if batch > 1 else (D,), dtype=torch.float32, device=self.dev)
        self.compute = torch.cuda.Stream(device=self.dev)
        self.copy = torch.cuda.Stream(device=self.dev)
        self.resident = None

    # -- inputs -----------------------------------------------------------------
    def pack(self, b_begin, blocks):
        self.store.pack(b_begin, blocks)

    def set_inputs(self, x, c):
        torch = self.torch
        self.x.copy_(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)))
        self.cond.copy_(torch.from_numpy(np.ascontiguousarray(c, dtype=np.float32)))
        torch.cuda.synchronize(self.dev)

    def make_resident(self, count=None):
        """Slot images of blocks 0 .. count-1 (all by default) in device buffers of their own."""
        torch = self.torch
        count = self.n_blocks if count is None else count
        self.resident = []
        for b in range(count):
            ext = self.plan.block_info(b)["extent"]
            buf = torch.empty(max(ext, 256), dtype=torch.uint8, device=self.dev)
            place_block(self.plan, self.store, b, buf.data_ptr(), buf.numel(), self.copy.cuda_stream)
            self.resident.append(buf)
        self.copy.synchronize()

    def free_resident(self):
        self.resident = None

    # -- runs -------------------------------------------------------------------
    def forward(self, passes, flags=0, resident=False, n_resident=0, want_run=True):
        """One dlo_forward_stack call.  resident=True: nothing streams; n_resident=R:
        blocks 0 .. R-1 resident, the rest streamed (resident images made on demand)."""
        from . import RESIDENT

        res_ptrs = None
        if resident or n_resident:
            need = self.n_blocks if resident else n_resident
            if self.resident is None or len(self.resident) < need:
                self.make_resident(need)
            if resident:
                flags |= RESIDENT
            res_ptrs = [b.data_ptr() for b in self.resident]
        return forward_stack(
            self.plan, None if resident else self.store,
            x=self.x.data_ptr(), x_row_stride=self.D, cond=self.cond.data_ptr(),
            workspace=self.ws.data_ptr(), workspace_bytes=self.ws_bytes,
            compute_stream=self.compute.cuda_stream, copy_stream=self.copy.cuda_stream,
            tokens=self.tokens, passes=passes,
            slots=(self.slots[0].data_ptr(), self.slots[1].data_ptr()),
            slot_bytes=self.plan.slot_bytes, flags=flags, resident_blocks=res_ptrs,
            n_resident=n_resident, want_run=want_run, batch=self.batch, cond_stride=self.D)

    def synchronize(self):
        self.compute.synchronize()
        self.copy.synchronize()

    def x_host(self):
        self.synchronize()
        return self.x.cpu().numpy()

    def slot_host(self, s):
        self.synchronize()
        return self.slots[s].cpu().numpy()

    def close(self):
        self.synchronize()
        self.resident = None
        self.store.close()
        self.plan.close()
