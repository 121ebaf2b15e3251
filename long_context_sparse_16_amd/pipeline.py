"""One CSA (or HCA) attention step over a batch, driven through the C ABI.

``CSAStep`` holds device-resident inputs, outputs and workspaces for one
batch and exposes the hot-path stages as separate calls so that callers can
time them individually:

  compress()  new raw tokens -> appended compressed K/V entries
  index()     Lightning Indexer scores
  topk()      per-query top-k entry indices
  select()    decode at a block boundary: the block compression, indexer
              and top-k with the compression folded into the indexer launch
  attend()    attention over the selected entries + sliding window
              (HCA: dense attention over every visible entry + window)
  select_attend()  top-k selection and attention after index()
              (csa_select_attend)
  decode()    the whole step of a decode batch in one call (csa_decode:
              index() then select_attend(); at a block boundary the block
              compression inside the indexer launch)

Every stage is one library call; this module only allocates tensors and
passes them on.  Inputs are given in storage form: float32 arrays, or uint16
arrays holding bf16 codes.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (csa_attend, csa_attend_backward, csa_attend_backward_workspace_size,
               csa_compress, csa_compress_backward, csa_decode, csa_decode_index_topk,
               csa_decode_workspace_size, csa_index_scores, csa_quantize_fp8_rows,
               csa_quantize_mxfp4_rows, csa_select_attend, csa_topk,
               csa_topk_workspace_size, csa_attend_workspace_size, hca_attend,
               hca_attend_workspace_size, workspace)

# Query rows (B * T) up to which a CSA step runs as one csa_decode call.
DECODE_MAX_ROWS = 256


def to_device(a: np.ndarray, device, storage: str) -> torch.Tensor:
    """Upload a storage-form array (float32, int, or uint16 bf16 codes)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def bf16_codes_of(t: torch.Tensor) -> np.ndarray:
    """uint16 codes of a device bf16 tensor."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class CSAStep:
    def __init__(self, cfg, batch: dict, device="cuda:0", act: str = "relu"):
        self.cfg = cfg
        self.act = act
        self.device = torch.device(device)
        dev = self.device
        st = cfg.storage
        B, T, d = cfg.B, cfg.T, cfg.d
        n_cap = cfg.n_cap
        kv_dtype = torch.float32 if st == "f32" else torch.bfloat16
        self.kc = torch.zeros((B, n_cap, d), dtype=kv_dtype, device=dev)
        self.vc = torch.zeros((B, n_cap, d), dtype=kv_dtype, device=dev)
        if cfg.n_ctx_entries:
            self.kc[:, :cfg.n_ctx_entries] = to_device(batch["kc"], dev, st)
            self.vc[:, :cfg.n_ctx_entries] = to_device(batch["vc"], dev, st)
        self.kr = to_device(batch["kr"], dev, st)
        self.vr = to_device(batch["vr"], dev, st)
        self.z = to_device(batch["z"], dev, st) if cfg.n_new_tokens or cfg.block_end else None
        # a block-completing decode step with bf16 indexer keys folds the
        # compression into the indexer launch
        self.fused_select = (cfg.block_end and cfg.T == 1 and st == "bf16" and cfg.k > 0
                             and not (cfg.ki_fp8 or cfg.ki_mxfp4))
        self.q = to_device(batch["q"], dev, st)
        self.pos0 = torch.full((B,), cfg.pos0, dtype=torch.int64, device=dev)
        self.raw_pos0 = torch.full((B,), cfg.raw_pos0, dtype=torch.int64, device=dev)
        self.out = torch.empty((B, T, cfg.H, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, T, cfg.H), dtype=torch.float32, device=dev)
        if cfg.hca:
            self.att_ws = workspace(hca_attend_workspace_size(B, T, cfg.H, d, n_cap, cfg.W), dev)
            self.idx = None
            return
        if cfg.swa:
            self.att_ws = workspace(csa_attend_workspace_size(B, T, cfg.H, d, 0, cfg.W), dev)
            self.idx = None
            return
        self.qi = to_device(batch["qi"], dev, st)
        self.w = to_device(batch["w"], dev, "f32")
        self.qi_scale = None
        self.ki_codes = None
        self.ki_scale = None
        if cfg.ki_fp8:
            self.qi_codes, self.qi_scale = csa_quantize_fp8_rows(self.qi)
            self.ki_codes = torch.empty((B, n_cap, cfg.d_I), dtype=torch.uint8, device=dev)
            self.ki_scale = torch.ones((B, n_cap), dtype=torch.float32, device=dev)
            if cfg.n_ctx_entries:
                self.quantize_keys(0, cfg.n_ctx_entries)
        if cfg.ki_mxfp4:
            self.qi_codes, self.qi_scale = csa_quantize_mxfp4_rows(self.qi)
            # byte storage (torch cannot copy between FP4 / E8M0 tensors);
            # the indexer gets FP4 / E8M0 views of it
            self.ki_codes = torch.empty((B, n_cap, cfg.d_I // 2), dtype=torch.uint8, device=dev)
            self.ki_scale = torch.zeros((B, n_cap, cfg.d_I // 32), dtype=torch.uint8, device=dev)
            if cfg.n_ctx_entries:
                self.quantize_keys(0, cfg.n_ctx_entries)
        self.scores = torch.empty((B, T, n_cap), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, T, cfg.k), dtype=torch.int32, device=dev)
        self.topk_ws = workspace(csa_topk_workspace_size(B, T, n_cap, cfg.k), dev)
        self.att_ws = workspace(csa_attend_workspace_size(B, T, cfg.H, d, cfg.k, cfg.W), dev)
        # decode-shaped steps run as csa_decode (its own workspace)
        self.use_decode = B * T <= DECODE_MAX_ROWS
        self.dec_ws = (workspace(csa_decode_workspace_size(B, T, cfg.H, d, n_cap, cfg.k, cfg.W,
                                                           False), dev)
                       if self.use_decode else None)

    # ------------------------------------------------------------ stages
    def quantize_keys(self, first: int, last: int) -> None:
        """FP8 (codes + per-entry scale) or MXFP4 (codes + block scales) copy
        of compressed keys [first, last)."""
        if self.cfg.ki_mxfp4:
            codes, scales = csa_quantize_mxfp4_rows(self.kc[:, first:last].contiguous())
            self.ki_codes[:, first:last] = codes.view(torch.uint8)
            self.ki_scale[:, first:last] = scales.view(torch.uint8)
            return
        codes, scales = csa_quantize_fp8_rows(self.kc[:, first:last].contiguous())
        self.ki_codes[:, first:last] = codes
        self.ki_scale[:, first:last] = scales

    def compress(self) -> None:
        cfg = self.cfg
        if cfg.block_end:
            # the block ends at the query token: the last m raw rows
            r0 = cfg.R - cfg.m
            z = self.z[:, r0:].contiguous()
            csa_compress(self.kr[:, r0:].contiguous(), z, self.kc, cfg.m, cfg.n_ctx_entries)
            csa_compress(self.vr[:, r0:].contiguous(), z, self.vc, cfg.m, cfg.n_ctx_entries)
            if cfg.ki_fp8 or cfg.ki_mxfp4:
                self.quantize_keys(cfg.n_ctx_entries, cfg.n_cap)
            return
        if not cfg.n_new_tokens:
            return
        x_k = self.kr[:, cfg.raw_before:cfg.raw_before + cfg.n_new_tokens]
        x_v = self.vr[:, cfg.raw_before:cfg.raw_before + cfg.n_new_tokens]
        csa_compress(x_k, self.z, self.kc, cfg.m, cfg.n_ctx_entries)
        csa_compress(x_v, self.z, self.vc, cfg.m, cfg.n_ctx_entries)
        if cfg.ki_fp8 or cfg.ki_mxfp4:
            self.quantize_keys(cfg.n_ctx_entries, cfg.n_cap)

    def select(self) -> None:
        """Block compression + indexer + top-k of a block-completing decode
        step, the compression inside the indexer launch."""
        cfg = self.cfg
        csa_decode_index_topk(self.qi, self.w, self.kc, self.vc, self.kr, self.vr, self.z,
                              self.z, self.raw_pos0, self.pos0, cfg.m, cfg.k, act=self.act,
                              scores=self.scores, idx=self.idx, ws=self.topk_ws)

    def index_inputs(self):
        """(qi, ki, qi_scale, ki_scale) as the indexer takes them."""
        if self.cfg.ki_fp8:
            return self.qi_codes, self.ki_codes, self.qi_scale, self.ki_scale
        if self.cfg.ki_mxfp4:
            return (self.qi_codes, self.ki_codes.view(torch.float4_e2m1fn_x2), self.qi_scale,
                    self.ki_scale.view(torch.float8_e8m0fnu))
        return self.qi, self.kc, None, None

    def decode(self) -> None:
        """The whole decode step in one library call (csa_decode)."""
        cfg = self.cfg
        qi, ki, qs, ks = self.index_inputs()
        fuse = self.fused_select  # block compression inside the indexer launch
        csa_decode(qi, self.w, ki, self.q, self.kc, self.vc, self.kr, self.vr, self.raw_pos0,
                   self.pos0, cfg.m, cfg.k, cfg.W, cfg.scale, act=self.act, qi_scale=qs,
                   ki_scale=ks, zk=self.z if fuse else None, zv=self.z if fuse else None,
                   scores=self.scores, idx=self.idx, out=self.out, lse=self.lse, ws=self.dec_ws)

    def index(self) -> None:
        """Indexer scores; also builds the top-k histogram in the top-k
        workspace, which topk() then consumes."""
        cfg = self.cfg
        if cfg.ki_fp8:
            csa_index_scores(self.qi_codes, self.w, self.ki_codes, self.pos0, cfg.m, self.act,
                             qi_scale=self.qi_scale, ki_scale=self.ki_scale, scores=self.scores,
                             topk_ws=self.topk_ws, k=cfg.k)
        elif cfg.ki_mxfp4:
            csa_index_scores(self.qi_codes, self.w, self.ki_codes.view(torch.float4_e2m1fn_x2),
                             self.pos0, cfg.m, self.act, qi_scale=self.qi_scale,
                             ki_scale=self.ki_scale.view(torch.float8_e8m0fnu),
                             scores=self.scores, topk_ws=self.topk_ws, k=cfg.k)
        else:
            csa_index_scores(self.qi, self.w, self.kc, self.pos0, cfg.m, self.act,
                             scores=self.scores, topk_ws=self.topk_ws, k=cfg.k)

    def topk(self) -> None:
        csa_topk(self.scores, self.pos0, self.cfg.m, self.cfg.k, idx=self.idx, ws=self.topk_ws,
                 hist_ready=True)

    def select_attend(self) -> None:
        """Top-k selection and attention after index() (csa_select_attend:
        for few long rows the selection is made inside the attention
        launch)."""
        cfg = self.cfg
        csa_select_attend(self.scores, self.topk_ws, self.pos0, cfg.m, cfg.k, self.q, self.kc,
                          self.vc, self.kr, self.vr, self.raw_pos0, cfg.W, cfg.scale,
                          idx=self.idx, out=self.out, lse=self.lse, ws=self.att_ws)

    def attend(self) -> None:
        cfg = self.cfg
        if cfg.hca:
            hca_attend(self.q, self.kc, self.vc, cfg.m, self.kr, self.vr, self.raw_pos0,
                       self.pos0, cfg.W, cfg.scale, out=self.out, lse=self.lse, ws=self.att_ws)
        elif cfg.swa:
            csa_attend(self.q, self.kc, self.vc, None, self.kr, self.vr, self.raw_pos0,
                       self.pos0, cfg.W, cfg.scale, out=self.out, lse=self.lse, ws=self.att_ws)
        else:
            csa_attend(self.q, self.kc, self.vc, self.idx, self.kr, self.vr, self.raw_pos0,
                       self.pos0, cfg.W, cfg.scale, out=self.out, lse=self.lse, ws=self.att_ws)

    def stages(self) -> list:
        """The step as (name, call) pairs, in order (for per-stage timing)."""
        cfg = self.cfg
        if self.fused_select:
            return [("select", self.select), ("attend", self.attend)]
        out = []
        if cfg.n_new_tokens or cfg.block_end:
            out.append(("compress", self.compress))
        if cfg.k > 0 and self.use_decode:
            # the launches csa_decode makes
            return out + [("index", self.index), ("select_attend", self.select_attend)]
        if cfg.k > 0:
            out += [("index", self.index), ("topk", self.topk)]
        out.append(("attend", self.attend))
        return out

    def run(self) -> None:
        """The whole step: compress (if the step completes blocks), then
        indexer + top-k + attention (CSA), dense attention (HCA) or
        window-only attention (sliding-window layers).  Decode batches with
        a top-k run as one csa_decode call."""
        if self.cfg.k > 0 and self.use_decode and (self.fused_select or not self.cfg.block_end):
            if not self.fused_select:
                self.compress()
            self.decode()
            return
        if self.fused_select:
            self.select()
            self.attend()
            return
        self.compress()
        if self.cfg.k > 0:
            self.index()
            self.topk()
        self.attend()

    def backward(self, dout: torch.Tensor) -> dict:
        """Backward pass of the step's attention (and of its compression when
        the step appends entries) for the upstream gradient dout [B, T, H, d]
        fp32, after run().  Returns dq, dkc, dvc, dkr, dvr and, for a
        compressing step, dkr_c / dvr_c and dz_k / dz_v: the gradients that
        reach the chunk's raw K / V tokens and logits through the
        compressor (add dkr_c to dkr for the raw rows' total)."""
        cfg = self.cfg
        if getattr(self, "bwd_ws", None) is None:
            self.bwd_ws = workspace(csa_attend_backward_workspace_size(
                cfg.B, cfg.T, cfg.d, cfg.n_cap, cfg.k, cfg.W), self.device)
        g = csa_attend_backward(self.q, self.kc, self.vc, self.idx, self.kr, self.vr,
                                self.raw_pos0, self.pos0, cfg.W, cfg.scale, self.out, self.lse,
                                dout, ws=self.bwd_ws)
        if cfg.n_new_tokens:
            r0, r1 = cfg.raw_before, cfg.raw_before + cfg.n_new_tokens
            e0, e1 = cfg.n_ctx_entries, cfg.n_cap
            g["dkr_c"], g["dz_k"] = csa_compress_backward(self.kr[:, r0:r1], self.z,
                                                          g["dkc"][:, e0:e1].contiguous(), cfg.m)
            g["dvr_c"], g["dz_v"] = csa_compress_backward(self.vr[:, r0:r1], self.z,
                                                          g["dvc"][:, e0:e1].contiguous(), cfg.m)
        return g

    def run_unfused(self) -> None:
        """The same step with the block compression as separate launches."""
        self.compress()
        if self.cfg.k > 0:
            self.index()
            self.topk()
        self.attend()


class HybridStep:
    """One decode token through a stack of attention layers, each with its
    own caches and workspaces (layer kinds and shapes from
    ``workloads.layer_workloads``): the layers run one after another on the
    stream, as they would in the model."""

    def __init__(self, layer_cfgs, batches, device="cuda:0"):
        self.layers = [CSAStep(c, b, device) for c, b in zip(layer_cfgs, batches)]

    def run(self) -> None:
        for layer in self.layers:
            layer.run()
