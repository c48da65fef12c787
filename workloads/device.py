"""Device-side harness: uploads a workload's inputs and drives the five library calls.

Used by the GPU tests, ``bench.py`` and ``__graft_entry__.smoke``.  It only moves data
and calls the binding (every step of the path runs in librva's kernels).  The
projections that sit between the stages in a real model (QKV projection of the packed
hidden rows, LM head) are outside the path: their outputs -- q / k_new / v_new and the
target logits -- are generated per block position and packed into the ragged layout once
at set-up with the library's own packing call, exactly as the model's projections would
emit them for the scheduled rows.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from ragged_verify_acceptance_amd import rva

from .generate import Inputs, paged_cache

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


class DeviceStep:
    def __init__(self, inp: Inputs, mode: str = "compact", device="cuda", fill_unused=float("nan")):
        self.inp = inp
        wl = self.wl = inp.wl
        self.mode = rva.STATIC if mode == "static" else rva.COMPACT
        self.dev = device
        B, G1, gamma = inp.B, wl.G1, wl.gamma
        self.B = B
        dev = device
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        kv = _DT[wl.kv_dtype]
        lg = _DT[wl.logit_dtype]

        # ---- stage 1 inputs
        if wl.conf_from_head:
            self.hidden = inp.hidden().to(dev)
            self.head_w = torch.from_numpy(inp.head_w).to(dev)
            self.conf_in = None
        else:
            self.hidden = None
            self.head_w = None
            self.conf_in = torch.from_numpy(inp.conf()).to(dev)
        self.head_b = float(inp.head_b)
        bias, alpha, theta = inp.cost_tables()
        self.bias = float(bias)
        self.alpha = torch.from_numpy(alpha).to(dev)
        self.theta = torch.from_numpy(theta).to(dev)
        self.conf_out = torch.empty((B, G1), **f32)
        self.surv_out = torch.empty((B, G1), **f32)
        self.windows = torch.empty(B, **i32)
        self.windows_next = torch.empty(B, **i32)  # written by the overlapped scheduler
        self.K_out = torch.empty(1, **i32)
        self.ratio_out = torch.empty(1, dtype=torch.float64, device=dev)
        self.status = torch.zeros(1, **i32)

        # ---- stage 2
        self.tiers = list(wl.tiers)
        self.max_rows = self.tiers[-1]
        self.context_lens0 = torch.from_numpy(inp.context_lens).to(dev)
        self.context_lens = self.context_lens0.clone()
        self.pack_src = torch.stack([inp.request_pack_src(b) for b in range(B)]).to(dev)
        self.pack_dst = torch.empty((self.max_rows, wl.pack_hidden), dtype=torch.bfloat16, device=dev)
        self.cu = torch.empty(B + 1, **i32)
        self.row_req = torch.empty(self.max_rows, **i32)
        self.row_pos = torch.empty(self.max_rows, **i32)
        self.total_tier = torch.empty(2, **i32)

        # ---- stage 3
        qs, ks, vs = zip(*[inp.request_qkv(b) for b in range(B)])
        self.q_blk = torch.stack(qs).to(dev)      # [B, gamma, Hq, D]
        self.k_blk = torch.stack(ks).to(dev)
        self.v_blk = torch.stack(vs).to(dev)
        k_pool, v_pool = paged_cache(inp, fill_unused=fill_unused)
        self.k_cache = k_pool.to(dev)
        self.v_cache = v_pool.to(dev)
        self.block_table = torch.from_numpy(inp.block_table).to(dev)
        self.q = torch.zeros((self.max_rows, wl.Hq, wl.D), dtype=kv, device=dev)
        self.k_new = torch.zeros((self.max_rows, wl.Hkv, wl.D), dtype=kv, device=dev)
        self.v_new = torch.zeros((self.max_rows, wl.Hkv, wl.D), dtype=kv, device=dev)
        self.out = torch.empty((self.max_rows, wl.Hq, wl.D), dtype=kv, device=dev)
        self.scale = 1.0 / math.sqrt(wl.D)
        kvc = rva.BF16 if wl.kv_dtype == "bf16" else rva.F32
        ws = rva.verify_attention_workspace_size(B, gamma, wl.Hq, wl.Hkv, wl.D, wl.page,
                                                 inp.max_pages, kvc)
        self.attn_ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)

        # ---- stage 4-5
        tl, dl, toks = zip(*[inp.request_logits(b) for b in range(B)])
        self.target_blk = torch.stack(tl).to(dev)  # [B, gamma, V]
        self.draft_logits = torch.stack(dl).to(dev).contiguous()  # [B, gamma-1, V]
        self.draft_tokens = torch.from_numpy(np.stack(toks)).to(dev)
        ua, ur = inp.uniforms()
        self.u_accept = torch.from_numpy(ua).to(dev)
        self.u_resample = torch.from_numpy(ur).to(dev)
        self.target_logits = torch.zeros((self.max_rows, wl.V), dtype=lg, device=dev)
        self.accept_len = torch.empty(B, **i32)
        self.committed = torch.empty((B, gamma), **i32)
        self.pt_at = torch.empty((B, G1), **f32)
        self.pd_at = torch.empty((B, G1), **f32)
        self.labels = torch.empty((B, G1), **f32)
        self.accept_len_full = torch.empty(B, **i32)  # cap-accept mode
        self.cap_windows = torch.empty(B, **i32)
        self.acc_ws = torch.zeros(rva.accept_workspace_size(B, gamma, wl.V, self.max_rows),
                                  dtype=torch.uint8, device=dev)

    # ------------------------------------------------------------------ calls
    def schedule(self, windows=None):
        wl = self.wl
        rva.schedule_windows(self.B, wl.gamma, self.mode, self.hidden, wl.head_H, self.head_w,
                             self.head_b, self.conf_in, None, self.bias, self.alpha, self.theta,
                             self.conf_out, self.surv_out,
                             self.windows if windows is None else windows, self.K_out,
                             self.ratio_out, self.status)

    def pack(self, src=None, dst=None):
        src = self.pack_src if src is None else src
        dst = self.pack_dst if dst is None else dst
        rva.pack_ragged(self.B, self.wl.gamma, self.windows, self.context_lens, self.tiers, src,
                        dst, self.max_rows, self.cu, self.row_req, self.row_pos,
                        self.total_tier, self.status)

    def schedule_pack(self):
        """Stages 1 and 2 in one call (rva_schedule_and_pack): the same outputs as
        schedule() followed by pack()."""
        wl = self.wl
        rva.schedule_and_pack(self.B, wl.gamma, self.mode, self.hidden, wl.head_H, self.head_w,
                              self.head_b, self.conf_in, None, self.bias, self.alpha, self.theta,
                              self.conf_out, self.surv_out, self.windows, self.K_out,
                              self.ratio_out, self.context_lens, self.tiers, self.pack_src,
                              self.pack_dst, self.max_rows, self.cu, self.row_req, self.row_pos,
                              self.total_tier, self.status)

    def attention(self):
        wl, inp = self.wl, self.inp
        rva.verify_attention(self.B, wl.gamma, self.max_rows, wl.Hq, wl.Hkv, wl.D, wl.page,
                             inp.num_pages, inp.max_pages, self.q, self.k_new, self.v_new,
                             self.k_cache, self.v_cache, self.block_table, self.context_lens,
                             self.cu, self.total_tier, self.scale, self.out, self.attn_ws,
                             self.status)

    def accept(self, labels=True, probs=True):
        wl = self.wl
        rva.accept_and_commit(self.B, wl.gamma, wl.V, self.max_rows, self.target_logits,
                              self.draft_logits, self.draft_tokens, self.u_accept,
                              self.u_resample, self.cu, self.accept_len, self.committed,
                              self.context_lens, self.pt_at if probs else None,
                              self.pd_at if probs else None, self.labels if labels else None,
                              self.acc_ws, self.status)

    def accept_capped(self, caps=None, labels=True):
        """Cap-accept arm: the packed rows hold whole blocks; commits are capped at `caps`
        (host array), or at the device windows already in `cap_windows` when None."""
        wl = self.wl
        if caps is not None:
            self.cap_windows.copy_(torch.as_tensor(np.asarray(caps, np.int32)).to(self.dev))
        rva.accept_capped(self.B, wl.gamma, wl.V, self.max_rows, self.target_logits,
                          self.draft_logits, self.draft_tokens, self.u_accept, self.u_resample,
                          self.cu, self.cap_windows, self.accept_len, self.accept_len_full,
                          self.committed, self.context_lens, self.pt_at, self.pd_at,
                          self.labels if labels else None, self.acc_ws, self.status)

    def labels_only(self, out):
        wl = self.wl
        rva.confidence_labels(self.B, wl.gamma, wl.V, self.max_rows, self.target_logits,
                              self.draft_logits, self.cu, out, self.acc_ws, self.status)

    # ------------------------------------------------------------------ composition
    def prepare(self):
        """Schedule + pack once, then lay out the model-side inputs (q/k/v, target logits)
        in the packed order; afterwards every `step()` recomputes the same schedule."""
        self.schedule()
        self.pack()
        self.pack(self.q_blk, self.q)
        self.pack(self.k_blk, self.k_new)
        self.pack(self.v_blk, self.v_new)
        self.pack(self.target_blk, self.target_logits)

    def restore(self):
        self.context_lens.copy_(self.context_lens0)

    def step_capped(self, labels=True):
        """One cap-accept step: schedule (compact) -> the windows become the commit cap ->
        pack and verify whole blocks -> accept with the cap.  The packed inputs must be laid
        out for whole blocks (prepare_with_windows with gamma everywhere)."""
        self.schedule()
        self.cap_windows.copy_(self.windows)
        self.windows.fill_(self.wl.gamma)
        self.pack()
        self.attention()
        self.accept_capped(None, labels=labels)

    def step_overlapped(self, side, ev_attn, ev_sched, labels=True):
        """One step with the scheduling call off the critical path, as the SGLang integration
        runs it (the devpress.csdn.net article on DSpark in SGLang, section 4: the next
        step's scheduling overlaps the current forward on a separate stream; the confidences
        it reads are from an earlier step).  Pack, attention and acceptance use the windows
        scheduled during the previous step; the scheduling call for the next step runs on
        `side` once attention is done, beside the acceptance kernels.  Both buffers of
        windows alternate, so no call reads a buffer another stream is writing."""
        main = torch.cuda.current_stream()
        self.pack()
        self.attention()
        ev_attn.record(main)
        side.wait_event(ev_attn)
        with torch.cuda.stream(side):
            self.schedule(windows=self.windows_next)
            ev_sched.record(side)
        self.accept(labels=labels)
        main.wait_event(ev_sched)
        self.windows, self.windows_next = self.windows_next, self.windows

    def step(self, labels=True):
        """One pass of the whole path: stages 1 + 2 (one call), 3 and 4 (+5)."""
        self.schedule_pack()
        self.attention()
        self.accept(labels=labels)


def upload_windows(ds: DeviceStep, windows) -> None:
    """Overwrite the device windows (used by tests that feed a stage its inputs directly)."""
    w = torch.as_tensor(np.asarray(windows, np.int32))
    ds.windows[: w.numel()].copy_(w.to(ds.dev))


def prepare_with_windows(ds: DeviceStep, windows) -> None:
    """Pack with the given windows (instead of scheduling) and lay out q/k/v and the target
    logits in that packed order."""
    upload_windows(ds, windows)
    ds.pack()
    ds.pack(ds.q_blk, ds.q)
    ds.pack(ds.k_blk, ds.k_new)
    ds.pack(ds.v_blk, ds.v_new)
    ds.pack(ds.target_blk, ds.target_logits)
