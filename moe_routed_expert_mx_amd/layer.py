"""Device buffers of one routed-experts layer, driven through the C ABI.

``MoeLayer`` uploads canonical FP4/E8M0 weights once, packs them with
``moe_pack_weights`` (the canonical copies are freed), owns the workspace and the
plan buffer, and runs one decode step, either as one moe_decode_run launch (B <= 8: the
experts kernel quantizes and routes the batch itself) or as the three ABI calls the
runtime page's PersistentExperts.run makes: plan (MXFP8 of x), units (moe_group),
experts.  torch only allocates memory and supplies the stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib


def _dev(a, device, dtype=None):
    t = torch.as_tensor(a) if isinstance(a, np.ndarray) else a
    return t.to(device=device, dtype=dtype) if dtype is not None else t.to(device)


class MoeLayer:
    def __init__(self, w13, s13, w2, s2, *, B_max: int, topk: int, device="cuda", replicas: int = 1):
        E, I2, Dh = w13.shape
        self.E, self.D, self.I = int(E), int(Dh) * 2, int(I2) // 2
        self.B_max, self.topk, self.device = int(B_max), int(topk), torch.device(device)
        sizes = _lib.moe_packed_weight_bytes(self.E, self.D, self.I)
        canon = [_dev(a, self.device, torch.uint8).contiguous() for a in (w13, s13, w2, s2)]
        self.packed = []
        for _ in range(max(1, replicas)):
            p = [torch.empty(n, dtype=torch.uint8, device=self.device) for n in sizes]
            _lib.moe_pack_weights(self.E, self.D, self.I, *canon, *p)
            self.packed.append(p)
        del canon
        self.structs = [_lib.moe_weights_t(self.E, self.D, self.I, *[t.data_ptr() for t in p]) for p in self.packed]
        ws_bytes = _lib.moe_workspace_bytes(self.E, self.D, self.I, self.B_max, self.topk)
        if ws_bytes == 0:
            raise ValueError("unsupported shape for the workspace")
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        _lib.moe_workspace_init(self.ws)
        self.plan = torch.empty(_lib.moe_plan_bytes(self.B_max, self.D), dtype=torch.uint8, device=self.device)
        self.units = torch.empty(_lib.moe_units_bytes(self.B_max, self.topk, self.E), dtype=torch.uint8,
                                 device=self.device)

    def prefetch_table(self, replica: int, experts) -> tuple:
        """The next-layer prefetch table (runtime page, run(..., ahead)) naming the packed
        weights of `experts` in replica `replica`: four rows per expert (FC1 codes and
        scales, FC2 codes and scales), each expert's slab being contiguous in the packed
        layout.  Pass it as ``ahead=`` to a decode-form forward() of another layer."""
        ranges = []
        for t in self.packed[replica]:
            per = t.numel() // self.E
            for e in experts:
                ranges.append((t.data_ptr() + int(e) * per, per))
        return _lib.prefetch_rows(ranges)

    def out_buffer(self, B: int) -> torch.Tensor:
        return torch.empty(B * self.topk, self.D, dtype=torch.bfloat16, device=self.device)

    DECODE_MAX = 8  # largest batch of the one-launch decode form
    AUTO_DECODE = True  # "auto" picks the decode form for B <= DECODE_MAX (faster at B = 1 and 8)

    def forward(self, x: torch.Tensor, ids: torch.Tensor, out: torch.Tensor | None = None, *, replica: int = 0,
                stream=None, path: str = "auto", **opts) -> torch.Tensor:
        """x: BF16 [B, D] (or its uint16 bits), ids: int32 [B, topk], both on the device.
        path: "decode" (one launch: for B <= 8 the decode kernel, for B > 8 the grouped kernel making its own
        plan and chunk table), "grouped" (plan and units in one launch, then experts) or "auto" (the decode form
        for B <= 8 when AUTO_DECODE is set, else grouped)."""
        B = x.shape[0]
        if B > self.B_max or ids.shape != (B, self.topk):
            raise ValueError("batch larger than B_max or ids of the wrong shape")
        if path not in ("auto", "decode", "grouped"):
            raise ValueError(f"unknown path {path!r}")
        if out is None:
            out = self.out_buffer(B)
        if path == "decode" or (path == "auto" and self.AUTO_DECODE and B <= self.DECODE_MAX):
            _lib.moe_decode_run(self.structs[replica], x, ids, self.ws, out, stream=stream, **opts)
            return out
        _lib.moe_plan_group(x, ids, self.E, self.plan, self.units, stream=stream)
        _lib.moe_experts_run(self.structs[replica], self.plan, self.units, B, self.topk, self.ws, out, stream=stream,
                             **opts)
        return out

    def kernel_name(self, B: int, path: str = "auto", exchange: int | None = None, col_tiles: int = 0,
                    grid: int = 0) -> str:
        """Name of the kernel that does a step's FC1/FC2 work (for reports).  The decode
        form runs decode_whole_kernel for batches within its limits (at most 128 distinct
        experts, B*topk <= 640, B*D/32 <= 2560, I <= 512) unless another exchange is asked
        for.  The grouped form runs grouped_kernel where the batch fits its tables (I <=
        384, at most 1024 chunks of 32 routes and 32 FC1 blocks per workgroup, with one
        workgroup per compute unit unless a grid is given) unless col_tiles is 1.  Everything
        else runs experts_kernel."""
        decode = path == "decode" or (path == "auto" and self.AUTO_DECODE and B <= self.DECODE_MAX)
        routes = B * self.topk
        if decode and B > self.DECODE_MAX:
            return "grouped_kernel (one launch)"
        if decode:
            whole = (min(self.E, routes) <= 128 and routes <= 640 and B * self.D // 32 <= 2560 and self.I <= 512)
            return "decode_whole_kernel" if exchange in (None, 0) and whole else "experts_kernel (decode form)"
        chunks = min(self.E, routes) + (routes + 31) // 32
        g = grid or min(torch.cuda.get_device_properties(self.device).multi_processor_count, 2048)
        fits = self.I <= 384 and chunks <= 1024 and (chunks * (self.I // 32) + g - 1) // g <= 32
        return "grouped_kernel" if col_tiles != 1 and fits else "experts_kernel"

    def experts(self, B: int, out: torch.Tensor, *, replica: int = 0, stream=None, **opts):
        """The experts kernel alone, on the plan and unit table of the last forward()."""
        _lib.moe_experts_run(self.structs[replica], self.plan, self.units, B, self.topk, self.ws, out, stream=stream,
                             **opts)

    def combine(self, rows: torch.Tensor, weights: torch.Tensor, y: torch.Tensor | None = None, *, stream=None):
        """Weighted top-k combine of the BF16 rows [B*topk, D] with FP32 weights [B, topk]
        into BF16 y [B, D]."""
        B = weights.shape[0]
        if y is None:
            y = torch.empty(B, self.D, dtype=torch.bfloat16, device=self.device)
        _lib.moe_combine(rows, weights, y, stream=stream)
        return y

    def unit_table(self, B: int):
        """The unit table moe_group left in the workspace: (header[4], unit_expert, unit_rows)."""
        U = B * self.topk
        hdr = torch.empty(4, dtype=torch.int32, device=self.device)
        ue = torch.empty(U, dtype=torch.int32, device=self.device)
        ur = torch.empty(U, 8, dtype=torch.int32, device=self.device)
        _lib.moe_units_export(self.units, B, self.topk, self.E, hdr, ue, ur)
        h = hdr.cpu().numpy()
        n = int(h[0])
        return h, ue[:n].cpu().numpy(), ur[:n].cpu().numpy()

    def plan_arrays(self, B: int):
        p = self.plan.cpu().numpy()
        codes = p[: B * self.D].reshape(B, self.D)
        scales = p[B * self.D: B * self.D + B * self.D // 32].reshape(B, self.D // 32)
        return codes, scales
