"""Buffer set-up and call sequences for whole passes of the hot path.

Each class allocates the quantised operands, outputs and workspace of one
problem once (torch device memory), builds the ABI descriptors once, and then
issues the C-ABI calls of one pass in order on the current stream.  Nothing
here computes: all arithmetic happens inside libbqa's kernels.
"""
from __future__ import annotations

import torch

from . import (BQA_FP8E4M3, BQA_INT8, BQA_MXFP4, BQA_OP_FWD, BQA_OP_QUANTIZE_K, BQA_OP_QUANTIZE_KV,
               BQA_OP_QUANTIZE_NVFP4, BQA_OP_QUANTIZE_V, BQA_OP_BWD, BQA_PTQ_MXFP4, BQA_QAT_MXFP4, BQA_ROLE_K, BQA_ROLE_Q, BQA_ROLE_V,
               BQA_SAGE_I8_F16PV, BQA_SAGE_I8_F8PV, BQA_SAGE_I8_I8PV, BQA_THRIFT, bqa_attn_bwd, bqa_attn_fwd,
               bqa_attn_bwd_qknorm, bqa_attn_fwd_ptq, bqa_attn_fwd_thrift_nvfp4, bqa_quantize_blocks, bqa_quantize_nvfp4, bqa_quantize_kv, bqa_quantize_qknorm,
               bqa_select_blocks, bqa_workspace_size, dense, max_sel, problem, qtensor)


def sage_problem(B, Hq, Hkv, Nq, Nk, d, causal, mode, q_block=128, k_block=64, smooth_k=True, smooth_eps=0.0,
                 sm_scale=0.0):
    return problem(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, causal=int(causal), sm_scale=sm_scale, mode=mode,
                   q_block=q_block, k_block=k_block, smooth_k=int(smooth_k), smooth_eps=smooth_eps)


class SagePath:
    """SageAttention INT8 forward: quantise Q, K (smoothed), V, then attend.

    With fp8 P.V the attention kernel quantises Q itself (fuse_q, the
    default there): quantize() then handles K and V, and forward() writes the
    Q codes and scales to qc / qs only when keep_q_codes is set."""

    def __init__(self, p, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, fuse_q=None, keep_q_codes=True):
        dev = q.device
        self.p = p
        self.fuse_q = (p.mode == BQA_SAGE_I8_F8PV) if fuse_q is None else bool(fuse_q)
        self.keep_q_codes = keep_q_codes
        B, Hq, Hkv, Nq, Nk, d = p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d
        self.q, self.k, self.v = q, k, v
        self.qc = torch.empty((B, Hq, Nq, d), dtype=torch.int8, device=dev)
        self.qs = torch.empty((B, Hq, Nq // p.q_block), dtype=torch.float32, device=dev)
        self.kc = torch.empty((B, Hkv, Nk, d), dtype=torch.int8, device=dev)
        self.ks = torch.empty((B, Hkv, Nk // p.k_block), dtype=torch.float32, device=dev)
        self.mu = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
        self.qq = qtensor(BQA_INT8, 0, p.q_block, self.qc, self.qs)
        self.kq = qtensor(BQA_INT8, 0, p.k_block, self.kc, self.ks)
        self.vq = None
        if p.mode != BQA_SAGE_I8_F16PV:
            self.vc = torch.empty((B, Hkv, d, Nk), dtype=torch.uint8, device=dev)
            self.vs = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
            fmt = BQA_FP8E4M3 if p.mode == BQA_SAGE_I8_F8PV else BQA_INT8
            self.vq = qtensor(fmt, 1, Nk, self.vc, self.vs)
        # K and V go through one call in the fp8 / int8 P.V modes
        self.kv_joint = p.mode in (BQA_SAGE_I8_F8PV, BQA_SAGE_I8_I8PV)
        ws = max(bqa_workspace_size(p, BQA_OP_QUANTIZE_K), bqa_workspace_size(p, BQA_OP_QUANTIZE_V),
                 bqa_workspace_size(p, BQA_OP_QUANTIZE_KV), 16)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        odt = torch.float16 if p.mode == BQA_SAGE_I8_F16PV else torch.bfloat16
        self.o = torch.empty((B, Hq, Nq, d), dtype=odt, device=dev)
        self.lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
        self._qd, self._kd, self._vd, self._od = dense(q), dense(k), dense(v), dense(self.o)

    def quantize_q(self):
        bqa_quantize_blocks(self.p, BQA_ROLE_Q, self._qd, self.qq, workspace=self.ws)

    def quantize(self):
        if not self.fuse_q:
            self.quantize_q()
        if self.kv_joint:
            bqa_quantize_kv(self.p, self._kd, self._vd, self.kq, self.vq, k_mean=self.mu, workspace=self.ws)
            return
        bqa_quantize_blocks(self.p, BQA_ROLE_K, self._kd, self.kq, k_mean=self.mu, workspace=self.ws)
        if self.vq is not None:
            bqa_quantize_blocks(self.p, BQA_ROLE_V, self._vd, self.vq, workspace=self.ws)

    def forward(self):
        if self.p.mode == BQA_SAGE_I8_F16PV:
            bqa_attn_fwd(self.p, q=self.qq, k=self.kq, v_hi=self._vd, o=self._od, lse=self.lse)
        elif self.fuse_q:
            bqa_attn_fwd(self.p, q=self.qq if self.keep_q_codes else None, q_hi=self._qd, k=self.kq, v=self.vq,
                         o=self._od, lse=self.lse)
        else:
            bqa_attn_fwd(self.p, q=self.qq, k=self.kq, v=self.vq, o=self._od, lse=self.lse)

    def step(self):
        self.quantize()
        self.forward()
        return self.o


class SageTrainStep(SagePath):
    """SageBwd training step: the INT8 forward (per-channel INT8 V in P.V),
    then the backward from dO (delta from the stored O, INT8 dO, four INT8
    products and the bf16 dP = dO V^T)."""

    def __init__(self, p, q, k, v, d_o, int8_dp=False):
        super().__init__(p, q, k, v)
        dev = q.device
        self.d_o = d_o
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(v)
        self.ws_bwd = torch.empty(max(bqa_workspace_size(p, BQA_OP_BWD), 16), dtype=torch.uint8, device=dev)
        self._dod = dense(d_o)
        # the fully INT8 backward: V's INT8 codes per 64 tokens feed dP = dO V^T
        self.vq8 = None
        if int8_dp:
            self.vc8 = torch.empty((p.B, p.Hkv, p.Nk, p.d), dtype=torch.int8, device=dev)
            self.vs8 = torch.empty((p.B, p.Hkv, p.Nk // 64), dtype=torch.float32, device=dev)
            self.vq8 = qtensor(BQA_INT8, 0, 64, self.vc8, self.vs8)

    def quantize(self):
        super().quantize()
        if self.vq8 is not None:
            bqa_quantize_blocks(self.p, BQA_ROLE_V, self._vd, self.vq8)

    def backward(self):
        bqa_attn_bwd(self.p, q=self.qq, k=self.kq, v=self.vq8, v_hi=self._vd, o_for_delta=self._od, lse=self.lse,
                     d_o=self._dod, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws_bwd)

    def step(self):
        self.quantize()
        self.forward()
        self.backward()
        return self.dq, self.dk, self.dv


class SageQkNormTrainStep(SageTrainStep):
    """The SageBwd training step of the recommended recipe with QK-norm fused
    into it: q and k are the raw rows; the quantiser normalises them on the
    way in (keeping each row's inverse norm) and the backward returns the
    gradients of the raw rows."""

    def __init__(self, p, q_raw, k_raw, v, d_o):
        super().__init__(p, q_raw, k_raw, v, d_o)
        self.fuse_q = False
        dev = q_raw.device
        self.q_rn = torch.empty((p.B, p.Hq, p.Nq), dtype=torch.float32, device=dev)
        self.k_rn = torch.empty((p.B, p.Hkv, p.Nk), dtype=torch.float32, device=dev)

    def quantize(self):
        bqa_quantize_qknorm(self.p, BQA_ROLE_Q, self._qd, self.qq, inv_norm=self.q_rn)
        bqa_quantize_qknorm(self.p, BQA_ROLE_K, self._kd, self.kq, inv_norm=self.k_rn, k_mean=self.mu,
                            workspace=self.ws)
        bqa_quantize_blocks(self.p, BQA_ROLE_V, self._vd, self.vq, workspace=self.ws)

    def backward(self):
        bqa_attn_bwd_qknorm(self.p, q=self.qq, k=self.kq, v_hi=self._vd, o_for_delta=self._od, lse=self.lse,
                            d_o=self._dod, q_raw=self._qd, k_raw=self._kd, q_inv_norm=self.q_rn,
                            k_inv_norm=self.k_rn, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws_bwd)


def qat_problem(B, Hq, Hkv, Nq, Nk, d, sm_scale=0.0):
    return problem(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, causal=0, sm_scale=sm_scale, mode=BQA_QAT_MXFP4)


class QatPath:
    """Attn-QAT FP4 forward: MXFP4 Q, K (along d) and V (along tokens), then
    attend, emitting O and (with aux=True) the bf16 auxiliary output O'."""

    def __init__(self, p, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, aux: bool = True):
        dev = q.device
        self.p = p
        B, Hq, Hkv, Nq, Nk, d = p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d
        self.q, self.k, self.v = q, k, v
        u8 = torch.uint8
        self.qc = torch.empty((B, Hq, Nq, d // 2), dtype=u8, device=dev)
        self.qs = torch.empty((B, Hq, Nq, d // 32), dtype=u8, device=dev)
        self.kc = torch.empty((B, Hkv, Nk, d // 2), dtype=u8, device=dev)
        self.ks = torch.empty((B, Hkv, Nk, d // 32), dtype=u8, device=dev)
        self.vc = torch.empty((B, Hkv, d, Nk // 2), dtype=u8, device=dev)
        self.vs = torch.empty((B, Hkv, d, Nk // 32), dtype=u8, device=dev)
        self.qq = qtensor(BQA_MXFP4, 0, 32, self.qc, self.qs)
        self.kq = qtensor(BQA_MXFP4, 0, 32, self.kc, self.ks)
        self.vq = qtensor(BQA_MXFP4, 1, 32, self.vc, self.vs)
        self.o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
        self.oa = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev) if aux else None
        self.lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
        self.row_max = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(bqa_workspace_size(p, BQA_OP_FWD), 16) if aux else 16, dtype=u8, device=dev)
        self._qd, self._kd, self._vd = dense(q), dense(k), dense(v)
        self._od = dense(self.o)
        self._oad = dense(self.oa) if aux else None

    def quantize(self):
        bqa_quantize_blocks(self.p, BQA_ROLE_Q, self._qd, self.qq)
        bqa_quantize_blocks(self.p, BQA_ROLE_K, self._kd, self.kq)
        bqa_quantize_blocks(self.p, BQA_ROLE_V, self._vd, self.vq)

    def forward(self):
        bqa_attn_fwd(self.p, q=self.qq, k=self.kq, v=self.vq, o=self._od, o_aux=self._oad, lse=self.lse,
                     row_max=self.row_max, workspace=self.ws)

    def step(self):
        self.quantize()
        self.forward()
        return self.o


class QatTrainStep(QatPath):
    """Attn-QAT training step: the FP4 forward with O', then the backward
    (P recomputed from the same MXFP4 scores and fake-quantised for dV,
    delta' = rowsum(dO o O'), bf16 products against the FP4 operands)."""

    def __init__(self, p, q, k, v, d_o):
        super().__init__(p, q, k, v, aux=True)
        dev = q.device
        self.d_o = d_o
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(v)
        self.ws_bwd = torch.empty(max(bqa_workspace_size(p, BQA_OP_BWD), 16), dtype=torch.uint8, device=dev)
        self._dod = dense(d_o)

    def backward(self):
        bqa_attn_bwd(self.p, q=self.qq, k=self.kq, v=self.vq, o_for_delta=self._oad, lse=self.lse,
                     row_max=self.row_max, d_o=self._dod,
                     dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws_bwd)

    def step(self):
        self.quantize()
        self.forward()
        self.backward()
        return self.dq, self.dk, self.dv


def ptq_problem(B, Hq, Hkv, Nq, Nk, d, causal=False, smooth_k=True, sm_scale=0.0):
    return problem(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, causal=int(causal), sm_scale=sm_scale,
                   mode=BQA_PTQ_MXFP4, smooth_k=int(smooth_k), smooth_eps=0.0)


class PtqPath:
    """The post-training FP4 baseline: Q smoothed by its bf16 128-row block
    means and K by its token mean before MXFP4, V in MXFP4 along tokens, then
    attention with the means' score shifts and two-level P."""

    def __init__(self, p, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        dev = q.device
        self.p = p
        B, Hq, Hkv, Nq, Nk, d = p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d
        self.q, self.k, self.v = q, k, v
        u8 = torch.uint8
        self.qc = torch.empty((B, Hq, Nq, d // 2), dtype=u8, device=dev)
        self.qs = torch.empty((B, Hq, Nq, d // 32), dtype=u8, device=dev)
        self.kc = torch.empty((B, Hkv, Nk, d // 2), dtype=u8, device=dev)
        self.ks = torch.empty((B, Hkv, Nk, d // 32), dtype=u8, device=dev)
        self.vc = torch.empty((B, Hkv, d, Nk // 2), dtype=u8, device=dev)
        self.vs = torch.empty((B, Hkv, d, Nk // 32), dtype=u8, device=dev)
        self.qq = qtensor(BQA_MXFP4, 0, 32, self.qc, self.qs)
        self.kq = qtensor(BQA_MXFP4, 0, 32, self.kc, self.ks)
        self.vq = qtensor(BQA_MXFP4, 1, 32, self.vc, self.vs)
        self.qbar = torch.empty((B, Hq, (Nq + 127) // 128, d), dtype=torch.float32, device=dev)
        self.mu = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
        self.o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
        self.ws_k = torch.empty(max(bqa_workspace_size(p, BQA_OP_QUANTIZE_K), 16), dtype=u8, device=dev)
        self.ws = torch.empty(max(bqa_workspace_size(p, BQA_OP_FWD), 16), dtype=u8, device=dev)
        self._qd, self._kd, self._vd = dense(q), dense(k), dense(v)
        self._od = dense(self.o)

    def quantize(self):
        bqa_quantize_blocks(self.p, BQA_ROLE_Q, self._qd, self.qq, block_means=self.qbar)
        bqa_quantize_blocks(self.p, BQA_ROLE_K, self._kd, self.kq, k_mean=self.mu if self.p.smooth_k else None,
                            workspace=self.ws_k)
        bqa_quantize_blocks(self.p, BQA_ROLE_V, self._vd, self.vq)

    def forward(self):
        bqa_attn_fwd_ptq(self.p, q=self.qq, k=self.kq, v=self.vq, q_means=self.qbar, o=self._od, lse=self.lse,
                         workspace=self.ws)

    def step(self):
        self.quantize()
        self.forward()
        return self.o


def thrift_problem(B, Hq, Hkv, Nq, Nk, d, budget_ppm=50_000, causal=True, num_splits=0, sm_scale=0.0):
    return problem(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, causal=int(causal), sm_scale=sm_scale, mode=BQA_THRIFT,
                   sel_block=128, hp_budget_ppm=budget_ppm, num_splits=num_splits)


class ThriftPath:
    """ThriftAttention prefill: MXFP4 Q, K (with 128-token block means) and V,
    block selection, then the mixed-precision attention (FP4 for the
    unselected pairs, the bf16 inputs for the selected ones)."""

    def __init__(self, p, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        dev = q.device
        self.p = p
        B, Hq, Hkv, Nq, Nk, d = p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d
        self.q, self.k, self.v = q, k, v
        u8 = torch.uint8
        nqb, nkb = -(-Nq // 128), Nk // 128
        self.qc = torch.empty((B, Hq, Nq, d // 2), dtype=u8, device=dev)
        self.qs = torch.empty((B, Hq, Nq, d // 32), dtype=u8, device=dev)
        self.kc = torch.empty((B, Hkv, Nk, d // 2), dtype=u8, device=dev)
        self.ks = torch.empty((B, Hkv, Nk, d // 32), dtype=u8, device=dev)
        self.vc = torch.empty((B, Hkv, d, Nk // 2), dtype=u8, device=dev)
        self.vs = torch.empty((B, Hkv, d, Nk // 32), dtype=u8, device=dev)
        self.qm = torch.empty((B, Hq, nqb, d), dtype=torch.float32, device=dev)
        self.km = torch.empty((B, Hkv, nkb, d), dtype=torch.float32, device=dev)
        self.sel_idx = torch.empty((B, Hq, nqb, max_sel(p)), dtype=torch.int32, device=dev)
        self.sel_cnt = torch.empty((B, Hq, nqb), dtype=torch.int32, device=dev)
        self.qq = qtensor(BQA_MXFP4, 0, 32, self.qc, self.qs)
        self.kq = qtensor(BQA_MXFP4, 0, 32, self.kc, self.ks)
        self.vq = qtensor(BQA_MXFP4, 1, 32, self.vc, self.vs)
        self.o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
        self._qd, self._kd, self._vd, self._od = dense(q), dense(k), dense(v), dense(self.o)

    def quantize(self):
        bqa_quantize_blocks(self.p, BQA_ROLE_Q, self._qd, self.qq, block_means=self.qm)
        bqa_quantize_blocks(self.p, BQA_ROLE_K, self._kd, self.kq, block_means=self.km)
        bqa_quantize_blocks(self.p, BQA_ROLE_V, self._vd, self.vq)

    def select(self):
        bqa_select_blocks(self.p, self.qm, self.km, self.sel_idx, self.sel_cnt)

    def forward(self):
        bqa_attn_fwd(self.p, q=self.qq, k=self.kq, v=self.vq, q_hi=self._qd, k_hi=self._kd, v_hi=self._vd,
                     sel_idx=self.sel_idx, sel_cnt=self.sel_cnt, o=self._od, lse=self.lse)

    def step(self):
        self.quantize()
        self.select()
        self.forward()
        return self.o


class ThriftNvPath(ThriftPath):
    """ThriftAttention prefill with its FP4 path in NVFP4 emulation: the block
    means and selection as in ThriftPath; Q, K, V fake-quantised to NVFP4
    (dequantised bf16 values); the unselected pairs in bf16 instructions on
    those with two-level NVFP4 P, the selected pairs on the bf16 inputs."""

    def __init__(self, p, q, k, v):
        super().__init__(p, q, k, v)
        self.qn, self.kn, self.vn = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        self.ws_nv = torch.empty(max(bqa_workspace_size(p, BQA_OP_QUANTIZE_NVFP4), 16), dtype=torch.uint8,
                                 device=q.device)

    def quantize(self):
        super().quantize()
        for role, x, y in ((BQA_ROLE_Q, self._qd, self.qn), (BQA_ROLE_K, self._kd, self.kn),
                           (BQA_ROLE_V, self._vd, self.vn)):
            bqa_quantize_nvfp4(self.p, role, x, y, workspace=self.ws_nv)

    def forward(self):
        bqa_attn_fwd_thrift_nvfp4(self.p, q_nv=self.qn, k_nv=self.kn, v_nv=self.vn, q_hi=self._qd, k_hi=self._kd,
                                  v_hi=self._vd, sel_idx=self.sel_idx, sel_cnt=self.sel_cnt, o=self._od, lse=self.lse)


class ThriftDecodePath:
    """ThriftAttention decode: the double KV cache (MXFP4 codes with 128-token
    key means, next to the bf16 cache) is built once by `build_cache`; a
    step quantises the new query, selects each head's blocks and attends."""

    def __init__(self, p, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, v_tiled: bool = True):
        dev = q.device
        self.p = p
        B, Hq, Hkv, Nk, d = p.B, p.Hq, p.Hkv, p.Nk, p.d
        self.q, self.k, self.v = q, k, v
        u8 = torch.uint8
        self.qc = torch.empty((B, Hq, 1, d // 2), dtype=u8, device=dev)
        self.qs = torch.empty((B, Hq, 1, d // 32), dtype=u8, device=dev)
        self.kc = torch.empty((B, Hkv, Nk, d // 2), dtype=u8, device=dev)
        self.ks = torch.empty((B, Hkv, Nk, d // 32), dtype=u8, device=dev)
        # V codes of the cache blocked by 128 keys (one block's codes contiguous), or channel-major
        if v_tiled:
            self.vc = torch.empty((B, Hkv, Nk // 128, d, 64), dtype=u8, device=dev)
            self.vs = torch.empty((B, Hkv, Nk // 128, d, 4), dtype=u8, device=dev)
        else:
            self.vc = torch.empty((B, Hkv, d, Nk // 2), dtype=u8, device=dev)
            self.vs = torch.empty((B, Hkv, d, Nk // 32), dtype=u8, device=dev)
        self.qm = torch.empty((B, Hq, 1, d), dtype=torch.float32, device=dev)
        self.km = torch.empty((B, Hkv, Nk // 128, d), dtype=torch.float32, device=dev)
        self.sel_idx = torch.empty((B, Hq, 1, max_sel(p)), dtype=torch.int32, device=dev)
        self.sel_cnt = torch.empty((B, Hq, 1), dtype=torch.int32, device=dev)
        self.qq = qtensor(BQA_MXFP4, 0, 32, self.qc, self.qs)
        self.kq = qtensor(BQA_MXFP4, 0, 32, self.kc, self.ks)
        self.vq = qtensor(BQA_MXFP4, 2 if v_tiled else 1, 32, self.vc, self.vs)
        self.o = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(bqa_workspace_size(p, BQA_OP_FWD), 16), dtype=u8, device=dev)
        self._qd, self._kd, self._vd, self._od = dense(q), dense(k), dense(v), dense(self.o)

    def build_cache(self):
        bqa_quantize_blocks(self.p, BQA_ROLE_K, self._kd, self.kq, block_means=self.km)
        bqa_quantize_blocks(self.p, BQA_ROLE_V, self._vd, self.vq)

    def quantize(self):
        bqa_quantize_blocks(self.p, BQA_ROLE_Q, self._qd, self.qq, block_means=self.qm)
        bqa_select_blocks(self.p, self.qm, self.km, self.sel_idx, self.sel_cnt)

    def forward(self):
        bqa_attn_fwd(self.p, q=self.qq, k=self.kq, v=self.vq, q_hi=self._qd, k_hi=self._kd, v_hi=self._vd,
                     sel_idx=self.sel_idx, sel_cnt=self.sel_cnt, o=self._od, lse=self.lse, workspace=self.ws)

    def step(self):
        self.quantize()
        self.forward()
        return self.o


def attention_ops(p) -> float:
    """Effective operation count of one forward: 4 B Hq Nq Nk d, halved when causal."""
    ops = 4.0 * p.B * p.Hq * p.Nq * p.Nk * p.d
    return ops / 2 if p.causal else ops


def to_device(x, dtype: str, device="cuda") -> torch.Tensor:
    """fp32 NumPy array of bf16/fp16-exact values -> torch tensor of that dtype on the device."""
    t = torch.from_numpy(x)
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(device)

