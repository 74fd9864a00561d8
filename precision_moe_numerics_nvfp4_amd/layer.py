"""One pass of the expert layer's quantized hot path with preallocated buffers.

Forward ("Inkling 2 Small uses four-bit training ...", section "NVFP4
forward, MXFP8 backward"): NVFP4-quantize the activations per token and the
expert weights per expert, group the routed tokens by expert, run the NVFP4
grouped GEMM. Backward (section "Stochastic rounding across transposes"):
re-quantize the saved NVFP4 activations and weights to MXFP8 with stochastic
rounding through a float32 transpose, quantize dY to MXFP8 in both
orientations, run the dgrad and wgrad grouped GEMMs.

Every step is a library call on the current stream; buffers are allocated
once here (torch is the device allocator) so a step allocates nothing.
"""

import torch

from . import binding as B


class ExpertLayerStep:
    """Buffers and calls for T tokens of width K routed top-k to E local
    experts [e0, e0+E) with FFN width N (expert weight stored [E*N, K])."""

    def __init__(self, T, K, N, E, k, e0=0, x_dtype=torch.bfloat16, out_dtype=torch.float32,
                 seed=0x5EED0004, device="cuda"):
        self.T, self.K, self.N, self.E, self.k, self.e0 = T, K, N, E, k, e0
        self.seed = seed
        dev = torch.device(device)
        u8, f32, i64 = torch.uint8, torch.float32, torch.int64
        cap = T * k
        self.m_cap = cap
        # padded token width: sum_g pad32(M_g) <= M + 31 G, rounded to 32
        self.P = ((cap + 31 * E + 31) // 32) * 32
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)
        # forward
        self.xq = (e(T, K // 2), e(T, K // 16), e(T, dt=f32))
        self.wq = (e(E * N, K // 2), e(E * N, K // 16), e(E, dt=f32))
        self.perm = dict(offsets=e(E + 1, dt=i64), padded_offsets=e(E + 1, dt=i64),
                         row_token=e(cap, dt=torch.int32), row_slot=e(cap, dt=torch.int32),
                         codes=e(cap, K // 2), scales=e(cap, K // 16), outer=e(cap, dt=f32))
        self.ws = e(B.permute_workspace_size(T, k, E))
        self.y = e(cap, N, dt=out_dtype)
        # backward
        self.w_off = torch.arange(E + 1, dtype=i64, device=dev) * N
        self.xT = (e(K, self.P), e(K, self.P // 32))
        self.wT = (e(K, E * N), e(K, E * N // 32))
        self.dy8 = (e(cap, N), e(cap, N // 32))
        self.dyT = (e(N, self.P), e(N, self.P // 32))
        self.dx = e(cap, K, dt=out_dtype)
        self.dw = e(E, N, K, dt=f32)

    # --------------------------------------------------------------- steps
    def quantize_x(self, x):
        return B.nvfp4_quantize(x, None, *self.xq)

    def quantize_w(self, w):
        return B.nvfp4_quantize(w, self.N, *self.wq)

    def permute(self, topk_ids):
        return B.moe_permute(topk_ids, self.e0, self.E, *self.xq, workspace=self.ws, out=self.perm)

    def forward_gemm(self):
        p = self.perm
        return B.moe_fwd_grouped_gemm(p["codes"], p["scales"], p["outer"], *self.wq,
                                      p["offsets"], y=self.y)

    def requant_x(self):
        p = self.perm
        return B.mxfp8_requant_sr(p["codes"], p["scales"], p["outer"], p["offsets"],
                                  p["padded_offsets"], self.P, self.seed, 0,
                                  out=self.xT[0], out_e8=self.xT[1])

    def requant_w(self):
        return B.mxfp8_requant_sr(*self.wq, self.w_off, self.w_off, self.E * self.N, self.seed, 1,
                                  rows_per_group=self.N, out=self.wT[0], out_e8=self.wT[1])

    def quantize_dy(self, dy):
        """Both orientations in one pass (row-wise for the routed rows)."""
        p = self.perm
        B.mxfp8_quantize_dual(dy, p["offsets"], p["padded_offsets"], self.P, row_out=self.dy8,
                              col_out=self.dyT)

    def dgrad(self):
        return B.moe_bwd_dgrad(*self.dy8, *self.wT, self.perm["offsets"], self.N, self.K,
                               dx=self.dx)

    def wgrad(self):
        return B.moe_bwd_wgrad(*self.dyT, *self.xT, self.perm["padded_offsets"], self.N, self.K,
                               dw=self.dw)

    def step(self, x, w, topk_ids, dy):
        """The whole hot path once: forward then backward."""
        self.quantize_x(x)
        self.quantize_w(w)
        self.permute(topk_ids)
        self.forward_gemm()
        self.requant_x()
        self.requant_w()
        self.quantize_dy(dy)
        self.dgrad()
        self.wgrad()
