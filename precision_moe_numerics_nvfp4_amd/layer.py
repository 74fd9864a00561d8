"""One pass of the expert layer's quantized hot path with preallocated buffers.

Forward ("Inkling 2 Small uses four-bit training ...", section "NVFP4
forward, MXFP8 backward"): NVFP4-quantize the activations per token and the
expert weights per expert, group the routed tokens by expert, run the NVFP4
grouped GEMM. Backward (section "Stochastic rounding across transposes"):
re-quantize the saved NVFP4 activations and weights to MXFP8 with stochastic
rounding through a float32 transpose, quantize dY to MXFP8 in both
orientations, run the dgrad and wgrad grouped GEMMs.

Also here: the expert FFN around the layer (ExpertFFNStep: down-projection,
per-token re-quantization of the intermediate, weighted combine, backward
through both projections) and the NVFP4 backward (NVFP4BackwardStep), the
alternative the pages report as tried first and given up.

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
        self.wT = (e(E * K, N), e(E * K, N // 32))           # per expert [K, N]
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


class ExpertFFNStep:
    """The routed expert FFN around the layer: up-projection W1 [E, F, K],
    per-token NVFP4 re-quantization of the intermediate H, down-projection
    W2 [E, K, F], weighted combine back to token order; and the backward
    through both projections, the MXFP8 path of each. The nonlinearity
    between the projections is the caller's and is not applied here.

    Philox streams: tag 0 = X_perm, 1 = W1, 3 = H, 4 = W2. Stored precisions:
    H, Y2, dY2, dH, dX_perm, the output and dX are bfloat16; dW1, dW2 and the
    routing-weight gradient are float32."""

    def __init__(self, T, K, F, E, k, e0=0, seed=0x5EED0002, device="cuda"):
        self.T, self.K, self.F, self.E, self.k, self.e0 = T, K, F, E, k, e0
        self.seed = seed
        dev = torch.device(device)
        u8, f32, i64, bf = torch.uint8, torch.float32, torch.int64, torch.bfloat16
        cap = T * k
        self.m_cap = cap
        self.P = ((cap + 31 * E + 31) // 32) * 32
        P = self.P
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)
        nvfp4 = lambda r, c, n_outer: (e(r, c // 2), e(r, c // 16), e(n_outer, dt=f32))
        mx = lambda r, c: (e(r, c), e(r, c // 32))
        # forward
        self.xq = nvfp4(T, K, T)
        self.w1q = nvfp4(E * F, K, E)
        self.w2q = nvfp4(E * K, F, E)
        self.perm = dict(offsets=e(E + 1, dt=i64), padded_offsets=e(E + 1, dt=i64),
                         row_token=e(cap, dt=torch.int32), row_slot=e(cap, dt=torch.int32),
                         pair_row=e(T, k, dt=torch.int32),
                         codes=e(cap, K // 2), scales=e(cap, K // 16), outer=e(cap, dt=f32))
        self.ws = e(B.permute_workspace_size(T, k, E))
        self.h = e(cap, F, dt=bf)
        self.hq = nvfp4(cap, F, cap)
        self.y2 = e(cap, K, dt=bf)
        self.out = e(T, K, dt=bf)
        # backward
        self.w_off1 = torch.arange(E + 1, dtype=i64, device=dev) * F
        self.w_off2 = torch.arange(E + 1, dtype=i64, device=dev) * K
        self.dy2 = e(cap, K, dt=bf)
        self.dgate = torch.zeros((T, k), dtype=f32, device=dev)
        self.dy2_8, self.dy2T = mx(cap, K), mx(K, P)
        self.hT, self.w2T = mx(F, P), mx(E * F, K)          # weights: per expert blocks
        self.dh = e(cap, F, dt=bf)
        self.dh8, self.dhT = mx(cap, F), mx(F, P)
        self.xT, self.w1T = mx(K, P), mx(E * K, F)
        self.dxp = e(cap, K, dt=bf)
        self.dw1 = e(E, F, K, dt=f32)
        self.dw2 = e(E, K, F, dt=f32)
        self.dx = e(T, K, dt=bf)

    def quantize_weights(self, w1, w2):
        """w1 [E*F, K], w2 [E*K, F] (bf16|f32), one outer scale per expert."""
        B.nvfp4_quantize(w1, self.F, *self.w1q)
        B.nvfp4_quantize(w2, self.K, *self.w2q)

    def forward(self, x, topk_ids, gate):
        p = self.perm
        B.nvfp4_quantize(x, None, *self.xq)
        B.moe_permute(topk_ids, self.e0, self.E, *self.xq, workspace=self.ws, out=p)
        B.moe_fwd_grouped_gemm(p["codes"], p["scales"], p["outer"], *self.w1q, p["offsets"],
                               y=self.h)
        B.nvfp4_quantize_live(self.h, p["offsets"], *self.hq)
        B.moe_fwd_grouped_gemm(*self.hq, *self.w2q, p["offsets"], y=self.y2)
        B.moe_combine(self.y2, p["pair_row"], gate, out=self.out)
        return self.out

    def backward(self, dout, gate):
        p = self.perm
        off, poff, P, s = p["offsets"], p["padded_offsets"], self.P, self.seed
        B.moe_combine_bwd(dout, p["row_token"], p["row_slot"], off, self.k, gate=gate, y=self.y2,
                          dy=self.dy2, dgate=self.dgate)
        # down-projection
        B.mxfp8_quantize_dual(self.dy2, off, poff, P, row_out=self.dy2_8, col_out=self.dy2T)
        B.mxfp8_requant_sr(*self.hq, off, poff, P, s, 3, out=self.hT[0], out_e8=self.hT[1])
        B.mxfp8_requant_sr(*self.w2q, self.w_off2, self.w_off2, self.E * self.K, s, 4,
                           rows_per_group=self.K, out=self.w2T[0], out_e8=self.w2T[1])
        B.moe_bwd_dgrad(*self.dy2_8, *self.w2T, off, self.K, self.F, dx=self.dh)
        B.moe_bwd_wgrad(*self.dy2T, *self.hT, poff, self.K, self.F, dw=self.dw2)
        # up-projection
        B.mxfp8_quantize_dual(self.dh, off, poff, P, row_out=self.dh8, col_out=self.dhT)
        B.mxfp8_requant_sr(p["codes"], p["scales"], p["outer"], off, poff, P, s, 0,
                           out=self.xT[0], out_e8=self.xT[1])
        B.mxfp8_requant_sr(*self.w1q, self.w_off1, self.w_off1, self.E * self.F, s, 1,
                           rows_per_group=self.F, out=self.w1T[0], out_e8=self.w1T[1])
        B.moe_bwd_dgrad(*self.dh8, *self.w1T, off, self.F, self.K, dx=self.dxp)
        B.moe_bwd_wgrad(*self.dhT, *self.xT, poff, self.F, self.K, dw=self.dw1)
        B.moe_combine(self.dxp, p["pair_row"], None, out=self.dx)
        return self.dx

    def step(self, x, w1, w2, topk_ids, gate, dout):
        """Forward and backward once, weights quantized in the step."""
        self.quantize_weights(w1, w2)
        self.forward(x, topk_ids, gate)
        self.backward(dout, gate)


class NVFP4BackwardStep:
    """The layer's backward with NVFP4 gradient operands instead of MXFP8, on
    the saved forward state of an ExpertLayerStep: saved activations and
    weights re-quantized to NVFP4 through a float32 transpose, dY quantized to
    NVFP4 in both orientations, all with stochastic rounding; dgrad on the
    forward grouped GEMM (per-expert transposed weights), wgrad on its
    weight-gradient mode. Token groups of the transposed operands are padded
    to 128. Philox tags: 5 = activations, 6 = weights, 7 = dY row-wise,
    8 = dY transposed."""

    def __init__(self, layer, device="cuda"):
        self.L = layer
        T, K, N, E, k = layer.T, layer.K, layer.N, layer.E, layer.k
        dev = torch.device(device)
        u8, f32 = torch.uint8, torch.float32
        cap = T * k
        self.P = ((cap + 127 * E + 127) // 128) * 128
        P = self.P
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)
        nvfp4 = lambda r, c, n_outer: (e(r, c // 2), e(r, c // 16), e(n_outer, dt=f32))
        self.poff = e(E + 1, dt=torch.int64)
        self.xT = nvfp4(K, P, E)
        self.wT = nvfp4(E * K, N, E)
        self.dy = nvfp4(cap, N, cap)
        self.dyT = nvfp4(N, P, E)
        self.dx = e(cap, K, dt=layer.dx.dtype)
        self.dw = e(E, N, K, dt=f32)

    def requant(self):
        L, p = self.L, self.L.perm
        B.moe_padded_offsets(p["offsets"], 128, out=self.poff)
        B.nvfp4_requant_sr(p["codes"], p["scales"], p["outer"], p["offsets"], self.poff, self.P,
                           L.seed, 5, out=self.xT)
        B.nvfp4_requant_sr(*L.wq, L.w_off, L.w_off, L.E * L.N, L.seed, 6, rows_per_group=L.N,
                           per_group_layout=True, out=self.wT)

    def quantize_dy(self, dy):
        L, p = self.L, self.L.perm
        B.nvfp4_quantize_sr(dy, L.seed, 7, *self.dy)
        B.nvfp4_quantize_sr_colwise(dy, p["offsets"], self.poff, self.P, L.seed, 8, out=self.dyT)

    def dgrad(self):
        return B.moe_fwd_grouped_gemm(*self.dy, *self.wT, self.L.perm["offsets"], y=self.dx)

    def wgrad(self):
        return B.moe_bwd_wgrad_nvfp4(self.dyT, self.xT, self.poff, self.L.N, self.L.K, dw=self.dw)

    def backward(self, dy):
        self.requant()
        self.quantize_dy(dy)
        self.dgrad()
        self.wgrad()
