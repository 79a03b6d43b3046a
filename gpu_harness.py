"""Device-side harness: uploads a workloads.build() input dict and runs the
Compressor library on it through the Python binding.

Used by the GPU tests, the smoke check and the benchmark.  It moves data and
calls the library; it computes nothing of the operator itself.
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_kv_wkv_amd as cmp


def _bf16(a: np.ndarray, dev) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(dev).view(torch.bfloat16)


def _i32(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)


def _f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


class DeviceCase:
    """Device copies of one workload's inputs, packed weights and buffers."""

    def __init__(self, w: dict, device="cuda:0", x: torch.Tensor = None):
        self.w = w
        dev = torch.device(device)
        self.dev = dev
        self.shape = cmp.make_shape(w["ratio"], w["head_dim"], w["hidden"], w["rotate"],
                                    w["block_size"], w["num_blocks"], w["table_stride"],
                                    w["rope_dim"])
        self.x = x if x is not None else _bf16(w["x"], dev)
        self.wkv = _bf16(w["wkv"], dev)
        self.wgate = _bf16(w["wgate"], dev)
        self.w_packed = torch.empty((2 * w["coff"] * w["head_dim"], w["hidden"]),
                                    dtype=torch.bfloat16, device=dev)
        cmp.compressor_pack_weights(self.shape, self.wkv, self.wgate, self.w_packed)
        self.ape = _f32(w["ape"], dev)
        self.weight = _bf16(w["weight"], dev)
        self.hadamard = None if w["hadamard"] is None else _bf16(w["hadamard"], dev)
        self.cos = _bf16(w["cos"], dev)
        self.sin = _bf16(w["sin"], dev)
        self.start_pos = _i32(w["start_pos"], dev)
        self.cu_seqlens = _i32(w["cu_seqlens"], dev)
        self.seqused = _i32(w["seqused"], dev)
        self.kv_table = _i32(w["kv_block_table"], dev)
        self.st_table = _i32(w["state_block_table"], dev)
        self.kv_state0 = _f32(w["kv_state"], dev)
        self.score_state0 = _f32(w["score_state"], dev)
        self.kv_state = self.kv_state0.clone()
        self.score_state = self.score_state0.clone()
        self.out = torch.empty((w["out_rows"], w["head_dim"]), dtype=torch.bfloat16, device=dev)
        self.workspace = None

    def reset_state(self):
        self.kv_state.copy_(self.kv_state0)
        self.score_state.copy_(self.score_state0)

    def _args(self, decode: bool, **over):
        # a call without overrides reuses the arguments marshalled (and
        # size-checked) the first time: the tensors are allocated once and
        # only ever updated in place
        if not over and getattr(self, "_cached", None) and self._cached[0] == decode:
            return self._cached[1]
        B = self.w["batch"]
        if self.workspace is None or self.workspace_mode != decode:
            if decode:
                n = cmp.compressor_decode_workspace_size(self.shape, B, self.out.shape[0])
            else:
                n = cmp.compressor_prefill_workspace_size(self.shape, self.x.shape[0], B,
                                                          self.out.shape[0])
            self.workspace = torch.empty(n, dtype=torch.uint8, device=self.dev)
            self.workspace_mode = decode
            self._cached = None            # its arguments named the previous workspace
        kw = dict(x=self.x, batch=B, kv_state=self.kv_state, score_state=self.score_state,
                  state_block_table=self.st_table, w_packed=self.w_packed, ape=self.ape,
                  norm_weight=self.weight, sin=self.sin, cos=self.cos, out=self.out,
                  workspace=self.workspace, cu_seqlens=None if decode else self.cu_seqlens,
                  seqused=self.seqused, start_pos=self.start_pos, kv_block_table=self.kv_table,
                  hadamard=self.hadamard)
        kw.update(over)
        args = cmp.make_args(shape=self.shape, **kw)
        if not over:
            self._cached = (decode, args)
        return args

    def prefill(self, **over):
        cmp.compressor_prefill(self.shape, self._args(False, **over))

    def decode(self, **over):
        cmp.compressor_decode(self.shape, self._args(True, **over))

    def device_error(self) -> int:
        return cmp.compressor_last_device_error(self.workspace)

    # host copies ---------------------------------------------------------
    def out_bits(self) -> np.ndarray:
        return self.out.view(torch.int16).cpu().numpy().view(np.uint16)

    def states(self):
        return self.kv_state.cpu().numpy(), self.score_state.cpu().numpy()


class NsaCase:
    """One NSA compression call on the device (uploads a build_nsa dict)."""

    def __init__(self, w: dict, device="cuda:0"):
        self.w = w
        self.dev = torch.device(device)
        dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float16
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.dev).view(dt)
        self.input = up(w["input"])
        self.weight = up(w["weight"])
        self.out = up(w["output_cache"])
        self.slots = torch.from_numpy(w["slot_mapping"]).to(self.dev)
        self.lens = torch.from_numpy(w["act_seq_len"]).to(self.dev)
        self.table = (torch.from_numpy(w["block_table"]).to(self.dev)
                      if w["block_table"] is not None else None)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self.shape = cmp.make_nsa_shape(
            w["head_num"], w["head_dim"], w["cbs"], w["stride"], w["page"],
            cmp.NSA_F16 if w["dtype"] == "f16" else cmp.NSA_BF16,
            cmp.NSA_LAYOUT_PAGED if w["layout"] == "paged" else cmp.NSA_LAYOUT_TND)

    def run(self, **over):
        kw = dict(input=self.input, weight=self.weight, slot_mapping=self.slots,
                  act_seq_len=self.lens, output_cache=self.out, block_table=self.table,
                  device_error=self.err)
        kw.update(over)
        cmp.nsa_compress_with_cache(self.shape, **kw)

    def out_bits(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.out.view(torch.int16).cpu().numpy().view(np.uint16)

    def device_error(self) -> int:
        torch.cuda.synchronize()
        return int(self.err.item())
