"""One verification step as a fixed sequence of libsv calls on fixed-address buffers.

Host orchestration only (no arithmetic): torch allocates the device buffers
once, and every per-step value (seed, budget, temperatures, top-p, draft
tokens, survival estimates, offsets) lives at a fixed device address, in the
spirit of DScale's fixed-address workspaces ("DScale: Scaling Block-Diffusion
Speculative Decoding with Adaptive Verification", abstract).  A step is:

    dvl_alloc_pack            (when a verification budget is used)
    sv_topp_threshold         target rows: max, argmax, lse, top-p cut
    sv_softmax_stats          independent draft rows (dense proposal)
      or sv_mixture_q         latent-mixture proposal and category posterior
    sv_accept                 acceptance tests, first rejection
    sv_residual_sample        residual or bonus token
"""
from __future__ import annotations

import numpy as np
import torch

from . import (SV_BF16, SV_F32, SV_Q_DENSE, SV_Q_MIXTURE, dvl_alloc_pack, make_workspace, sv_accept, sv_mixture_q,
               sv_accept_sample, sv_residual_sample, sv_softmax_stats, sv_topp_threshold, sv_verify_rows,
               sv_verify_rows_dense)


def row_pitch(V: int, dtype: str) -> int:
    """Leading dimension (elements) that keeps every row 16-byte aligned."""
    per = 8 if dtype == "bf16" else 4
    return (V + per - 1) // per * per


def to_device_rows(arr: np.ndarray, ld: int, device="cuda", pad_bits: int | None = None) -> torch.Tensor:
    """Copy [..., V] logits (float32, or uint16 bf16 bits) to a [rows, ld] device tensor.
    Padding columns hold `pad_bits` (default: NaN) and are never read."""
    V = arr.shape[-1]
    flat = arr.reshape(-1, V)
    if arr.dtype == np.uint16:
        host = np.full((flat.shape[0], ld), 0x7FC0 if pad_bits is None else pad_bits, dtype=np.uint16)
        host[:, :V] = flat
        return torch.from_numpy(host.view(np.int16)).to(device).view(torch.bfloat16)
    host = np.full((flat.shape[0], ld), np.nan, dtype=np.float32)
    host[:, :V] = flat
    return torch.from_numpy(host).to(device)


class VerifyStep:
    def __init__(self, *, R: int, b: int, V: int, dtype: str, K: int = 0, max_pos: int | None = None,
                 device="cuda", diagnostics: bool = False, soft_branches: bool = False, ragged: bool = False):
        self.R, self.b, self.V, self.K = R, b, V, K
        self.dtype = dtype
        self.dt = SV_BF16 if dtype == "bf16" else SV_F32
        self.q_mode = SV_Q_MIXTURE if K > 0 else SV_Q_DENSE
        self.max_pos = R * b if max_pos is None else max_pos
        self.max_rows = self.max_pos + R
        self.device = device
        self.ws, self.ws_bytes = make_workspace(R, b, K, V, device)
        d = dict(device=device)
        i32, f32, f64 = torch.int32, torch.float32, torch.float64
        self.seed = torch.zeros(1, dtype=torch.int64, **d)
        self.budget = torch.zeros(1, dtype=i32, **d)
        self.a = torch.zeros(R * b, dtype=f32, **d)
        # per-request block length b_r <= b (None: every request drafted b positions)
        self.block_len = torch.full((R,), b, dtype=i32, **d) if ragged else None
        self._block_len_host = np.full(R, b, np.int32)
        self.s = torch.zeros(R * b, dtype=f32, **d)
        self.L = torch.zeros(R, dtype=i32, **d)
        self.pos_off = torch.zeros(R + 1, dtype=i32, **d)
        self.tgt_off = torch.zeros(R + 1, dtype=i32, **d)
        self.T = torch.zeros(R, dtype=f32, **d)
        self.top_p = torch.ones(R, dtype=f32, **d)
        self.x = torch.zeros(R * b, dtype=i32, **d)
        n = self.max_rows
        self.row_max = torch.zeros(n, dtype=f32, **d)
        self.row_argmax = torch.zeros(n, dtype=i32, **d)
        self.row_lse = torch.zeros(n, dtype=f64, **d)
        self.row_cut = torch.zeros(n, dtype=f32, **d)
        self.row_kept = torch.zeros(n, dtype=f64, **d)
        m = max(self.max_pos, 1)
        self.d_max = torch.zeros(m, dtype=f32, **d)
        self.d_argmax = torch.zeros(m, dtype=i32, **d)
        self.d_lse = torch.zeros(m, dtype=f64, **d)
        kk = max(K, 1)
        self.branch_tok = torch.zeros(R * kk * b, dtype=i32, **d)
        self.post_w = torch.zeros(R * b * kk, dtype=f64, **d)
        self.q_at_draft = torch.zeros(R * b, dtype=f64, **d)
        self.mix = torch.zeros(R * kk, dtype=f32, **d)
        # soft branches: the branch temperature T_b per request (0 keeps that request's branches greedy)
        self.soft = soft_branches
        self.branch_T = torch.zeros(R, dtype=f32, **d) if soft_branches else None
        self.n_acc = torch.zeros(R, dtype=i32, **d)
        self.token = torch.zeros(R, dtype=i32, **d)
        self.is_bonus = torch.zeros(R, dtype=i32, **d)
        self.diag = diagnostics
        self.p_out = torch.zeros(R * b, dtype=f64, **d) if diagnostics else None
        self.q_out = torch.zeros(R * b, dtype=f64, **d) if diagnostics else None
        self.u_out = torch.zeros(R * b, dtype=f32, **d) if diagnostics else None

    # ---------------------------------------------------------------- per-step inputs (host -> fixed addresses)
    def set_inputs(self, *, T, x, seed: int, top_p=None, mix=None, a=None, budget: int | None = None,
                   branch_T=None, block_len=None):
        self.T.copy_(torch.as_tensor(np.asarray(T, np.float32)))
        self.top_p.copy_(torch.as_tensor(np.ones(self.R, np.float32) if top_p is None else np.asarray(top_p, np.float32)))
        self.use_topp = top_p is not None
        self.x.copy_(torch.as_tensor(np.asarray(x, np.int32).reshape(-1)))
        self.seed.copy_(torch.tensor([np.int64(np.uint64(seed).view(np.int64))]))
        if mix is not None:
            self.mix.copy_(torch.as_tensor(np.asarray(mix, np.float32).reshape(-1)))
        if a is not None:
            self.a.copy_(torch.as_tensor(np.asarray(a, np.float32).reshape(-1)))
        if budget is not None:
            self.budget.fill_(int(budget))
        if block_len is not None:
            assert self.block_len is not None, "block lengths need ragged=True"
            self._block_len_host = np.asarray(block_len, np.int32).reshape(self.R).copy()
            self.block_len.copy_(torch.as_tensor(self._block_len_host))
        if branch_T is not None:
            assert self.soft, "branch temperatures need soft_branches=True"
            self.branch_T.copy_(torch.as_tensor(np.broadcast_to(np.asarray(branch_T, np.float32), (self.R,)).copy()))

    def set_full_verification(self):
        """Offsets for L_r = b_r (no DVL): the exclusive scans of b_r and b_r + 1."""
        L = self._block_len_host
        self.L.copy_(torch.as_tensor(L))
        self.pos_off.copy_(torch.as_tensor(np.concatenate([[0], np.cumsum(L)]).astype(np.int32)))
        self.tgt_off.copy_(torch.as_tensor(np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)))

    # ---------------------------------------------------------------- the calls
    def run_dvl(self, stream=None):
        dvl_alloc_pack(self.a, self.R, self.b, self.block_len, self.budget, self.s, self.L, self.pos_off,
                       self.tgt_off, self.ws, self.ws_bytes, stream)

    def run_rows(self, tgt, tgt_ld, stream=None):
        sv_topp_threshold(tgt, self.dt, tgt_ld, self.V, self.tgt_off, 0, self.R, self.max_rows, self.T,
                          self.top_p if self.use_topp else None, self.row_max, self.row_argmax, self.row_lse,
                          self.row_cut, self.row_kept, self.ws, self.ws_bytes, stream)

    def run_proposal(self, *, draft=None, draft_ld=0, comp=None, comp_ld=0, stream=None):
        if self.q_mode == SV_Q_DENSE:
            sv_softmax_stats(draft, self.dt, draft_ld, self.V, self.pos_off, self.b, self.R, self.max_pos, self.T,
                             self.d_max, self.d_argmax, self.d_lse, self.ws, self.ws_bytes, stream)
        else:
            sv_mixture_q(comp, self.dt, comp_ld, self.V, self.K, self.b, self.mix, self.pos_off, self.R,
                         self.max_pos, self.x, self.branch_tok, self.post_w, self.q_at_draft, self.ws,
                         self.ws_bytes, stream)

    def run_accept(self, tgt, tgt_ld, *, draft=None, draft_ld=0, stream=None):
        dense = self.q_mode == SV_Q_DENSE
        sv_accept(tgt, self.dt, tgt_ld, self.V, self.tgt_off, self.pos_off, self.R, self.b, self.T,
                  self.row_argmax, self.row_cut, self.row_kept, self.x, self.q_mode, draft if dense else None,
                  self.dt, draft_ld if dense else 0, self.d_argmax if dense else None,
                  self.d_lse if dense else None, None if dense else self.q_at_draft, self.seed, self.n_acc,
                  self.p_out, self.q_out, self.u_out, self.ws, self.ws_bytes, stream)
        sv_residual_sample(tgt, self.dt, tgt_ld, self.V, self.tgt_off, self.pos_off, self.R, self.b, self.T,
                           self.row_argmax, self.row_cut, self.row_kept, self.q_mode, draft if dense else None,
                           self.dt, draft_ld if dense else 0, self.d_argmax if dense else None,
                           self.d_lse if dense else None, self.K, None if dense else self.branch_tok,
                           None if dense else self.post_w, self.seed, self.n_acc, self.token, self.is_bonus,
                           self.ws, self.ws_bytes, stream)

    def run_rows_fused(self, tgt, tgt_ld, comp, comp_ld, stream=None):
        """Target rows and component rows (partial branch argmax, merged by
        sv_accept_sample) in one launch."""
        sv_verify_rows(tgt, self.dt, tgt_ld, self.V, self.tgt_off, self.R, self.max_rows, self.T,
                       self.top_p if self.use_topp else None, self.row_max, self.row_argmax, self.row_lse,
                       self.row_cut, self.row_kept, comp, comp_ld, self.K, self.b, self.pos_off, self.max_pos,
                       self.x, self.branch_T, self.ws, self.ws_bytes, stream)

    def run_rows_dense(self, tgt, tgt_ld, draft, draft_ld, stream=None):
        """Target rows and the dense draft's rows in one launch."""
        sv_verify_rows_dense(tgt, self.dt, tgt_ld, self.V, self.tgt_off, self.R, self.max_rows, self.T,
                             self.top_p if self.use_topp else None, self.row_max, self.row_argmax, self.row_lse,
                             self.row_cut, self.row_kept, draft, self.dt, draft_ld, self.b, self.pos_off,
                             self.max_pos, self.x, self.d_max, self.d_argmax, self.d_lse, self.ws, self.ws_bytes,
                             stream)

    def run_accept_sample(self, tgt, tgt_ld, *, draft=None, draft_ld=0, comp=None, comp_ld=0, stream=None):
        """Posterior (mixture), acceptance and the draw: two launches.  Soft
        branches read the component rows again (`comp`)."""
        dense = self.q_mode == SV_Q_DENSE
        sv_accept_sample(tgt, self.dt, tgt_ld, self.V, self.tgt_off, self.pos_off, self.R, self.b, self.T,
                         self.row_argmax, self.row_cut, self.row_kept, self.x, self.q_mode,
                         draft if dense else None, self.dt, draft_ld if dense else 0,
                         self.d_argmax if dense else None, self.d_lse if dense else None, self.K,
                         None if dense else self.mix, comp if self.soft else None, comp_ld if self.soft else 0,
                         self.branch_T, None if dense else self.branch_tok,
                         None if dense else self.post_w, None if dense else self.q_at_draft, self.seed, self.n_acc,
                         self.token, self.is_bonus, self.p_out, self.q_out, self.u_out, self.ws, self.ws_bytes,
                         stream)

    def run_verify(self, tgt, tgt_ld, *, draft=None, draft_ld=0, comp=None, comp_ld=0, side_stream=None,
                   fused=False):
        """The verification calls on torch's current stream.  With `side_stream`,
        the target-row statistics run there, concurrently with the proposal.
        With `fused`: sv_verify_rows (mixture) or sv_verify_rows_dense, then sv_accept_sample."""
        if fused:
            if self.q_mode == SV_Q_DENSE:
                self.run_rows_dense(tgt, tgt_ld, draft, draft_ld)
            else:
                self.run_rows_fused(tgt, tgt_ld, comp, comp_ld)
            self.run_accept_sample(tgt, tgt_ld, draft=draft, draft_ld=draft_ld, comp=comp, comp_ld=comp_ld)
            return
        if self.soft:
            raise ValueError("soft branches run on the fused calls (fused=True)")
        if side_stream is None:
            self.run_rows(tgt, tgt_ld)
            self.run_proposal(draft=draft, draft_ld=draft_ld, comp=comp, comp_ld=comp_ld)
        else:
            main = torch.cuda.current_stream()
            ev = torch.cuda.Event()
            ev.record(main)
            side_stream.wait_event(ev)
            self.run_rows(tgt, tgt_ld, side_stream)
            done = torch.cuda.Event()
            done.record(side_stream)
            self.run_proposal(draft=draft, draft_ld=draft_ld, comp=comp, comp_ld=comp_ld)
            main.wait_event(done)
        self.run_accept(tgt, tgt_ld, draft=draft, draft_ld=draft_ld)

    # ---------------------------------------------------------------- read-back (tests)
    def results(self) -> dict:
        torch.cuda.synchronize()
        g = lambda t: t.cpu().numpy()  # noqa: E731
        out = {"n_acc": g(self.n_acc), "token": g(self.token), "is_bonus": g(self.is_bonus), "L": g(self.L),
               "s": g(self.s), "pos_off": g(self.pos_off), "tgt_off": g(self.tgt_off),
               "row_max": g(self.row_max), "row_argmax": g(self.row_argmax), "row_lse": g(self.row_lse),
               "row_cut": g(self.row_cut), "row_kept": g(self.row_kept)}
        if self.q_mode == SV_Q_DENSE:
            out.update(d_max=g(self.d_max), d_argmax=g(self.d_argmax), d_lse=g(self.d_lse))
        else:
            out.update(branch_tok=g(self.branch_tok).reshape(self.R, self.K, self.b),
                       post_w=g(self.post_w).reshape(self.R, self.b, self.K),
                       q_at_draft=g(self.q_at_draft).reshape(self.R, self.b))
        if self.diag:
            out.update(p_x=g(self.p_out).reshape(self.R, self.b), q_x=g(self.q_out).reshape(self.R, self.b),
                       u_acc=g(self.u_out).reshape(self.R, self.b))
        return out


def pack_rows_device(full: torch.Tensor, L: np.ndarray, rows_per_req: int, out: torch.Tensor) -> torch.Tensor:
    """Stand-in for the target forward over the packed verification slots (not
    part of verification): request r contributes rows r*rows_per_req + j,
    j = 0..L[r], in request order, gathered into `out`."""
    idx = np.concatenate([r * rows_per_req + np.arange(int(L[r]) + 1) for r in range(len(L))]).astype(np.int64)
    n = len(idx)
    torch.index_select(full, 0, torch.from_numpy(idx).to(full.device), out=out[:n])
    return out


def pack_rows_by_offsets(full: torch.Tensor, tgt_off: torch.Tensor, rows_per_req: int, out: torch.Tensor,
                         slots: torch.Tensor) -> torch.Tensor:
    """Device-side stand-in for the target forward over the packed slots (not
    part of verification): slot k of `out` receives row r*rows_per_req + j of
    `full`, where r is the request whose range [tgt_off[r], tgt_off[r+1])
    holds k and j = k - tgt_off[r].  The offsets are read on the device only,
    so the copy can sit in a captured graph behind dvl_alloc_pack; slots past
    tgt_off[R] receive a copy of the last request's last row and are never
    read.  `slots` is arange(out.shape[0]) as int32 on the device."""
    R = tgt_off.numel() - 1
    r = torch.searchsorted(tgt_off[1:], slots, right=True).clamp_(max=R - 1)
    j = (slots.long() - tgt_off[r].long()).clamp_(0, rows_per_req - 1)
    torch.index_select(full, 0, r * rows_per_req + j, out=out)
    return out


def capture_graph(fn, warmup: int = 1) -> torch.cuda.CUDAGraph:
    """Record the launches `fn` makes on torch's current stream into a HIP graph.
    `fn` is run `warmup` times eagerly on a side stream first (torch's own lazy
    set-up must not happen under capture).  Every libsv call takes its per-step
    values (seed, budget, offsets, lengths, temperatures, top-p, tokens) from
    device memory, so one graph serves every step whose inputs are written to
    the same addresses before `replay()`.  The graph records raw addresses:
    `fn` (and so every buffer its closure holds) is kept alive as
    `graph.recorded_fn` for as long as the graph is."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.recorded_fn = fn
    return g
