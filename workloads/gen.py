"""Seeded generators (see the package docstring for the workload recipes)."""

import numpy as np

__all__ = [
    "rng", "to_bf16_bits", "normal", "with_outliers", "route_uniform",
    "route_zipf", "zipf_placement", "philox_seed", "single_expert",
    "small_moe", "expert_share", "backward_dy", "decode", "streaming",
    "moe_case", "gates", "ffn_case",
]

N_EXPERTS = 384
EP_RANKS = 8
LOCAL_E0 = 144            # expert-parallel rank 3 of 8 owns experts 144..191
LOCAL_EXPERTS = 48


def rng(cfg, tid):
    return np.random.default_rng(np.random.SeedSequence([int(cfg), int(tid)]))


def philox_seed(cfg):
    return 0x5EED0000 + int(cfg)


def to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_u.shape[0], step):
        c = flat_u[i:i + step]
        flat_o[i:i + step] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
                              >> np.uint32(16)).astype(np.uint16)
    return out


def normal(cfg, tid, shape, std=1.0):
    x = rng(cfg, tid).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def with_outliers(x, cfg, tid, frac=0.001, factor=50.0):
    """Multiply a seeded fraction of entries by ``factor`` (in place)."""
    mask = rng(cfg, tid).random(size=x.shape) < frac
    x[mask] *= np.float32(factor)
    return x


def route_uniform(cfg, T, n_experts, k, tid=5):
    """k distinct experts per token, uniformly at random (argsort of keys)."""
    keys = rng(cfg, tid).random(size=(T, n_experts))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def zipf_placement(n_experts=N_EXPERTS, ranks=EP_RANKS):
    """Expert id of popularity rank r (1-based): popularity order dealt
    round-robin over the expert-parallel ranks, each owning a contiguous
    block of n_experts/ranks ids."""
    per = n_experts // ranks
    r = np.arange(1, n_experts + 1)
    return (per * ((r - 1) % ranks) + (r - 1) // ranks).astype(np.int32)


def route_zipf(cfg, T, k=8, s=1.1, n_experts=N_EXPERTS, tid=5):
    """Top-k distinct experts per token with Zipf(s) popularity via Gumbel-top-k
    over log p_r, p_r ~ r^-s; returned in descending score order."""
    r = np.arange(1, n_experts + 1, dtype=np.float64)
    logp = -s * np.log(r)
    logp -= np.log(np.exp(logp).sum())
    g = rng(cfg, tid).gumbel(size=(T, n_experts))
    score = logp[None, :] + g
    top = np.argpartition(-score, k - 1, axis=1)[:, :k]
    sc = np.take_along_axis(score, top, axis=1)
    order = np.argsort(-sc, axis=1, kind="stable")
    ranks = np.take_along_axis(top, order, axis=1)        # 0-based popularity rank
    return zipf_placement(n_experts)[ranks].astype(np.int32)


# ------------------------------------------------------------ the workloads

def single_expert():
    """Workload 1 (fp32, one expert, no routing)."""
    x = with_outliers(normal(1, 0, (64, 256)), 1, 6)
    w_math = with_outliers(normal(1, 1, (256, 512)), 1, 7)
    return dict(cfg=1, x=x, w=np.ascontiguousarray(w_math.T), dy=normal(1, 3, (64, 512)),
                topk=np.zeros((64, 1), np.int32), e0=0, n_local=1, E=1,
                T=64, K=256, N=512, k=1)


def small_moe(T=4096, K=1024, N=2048, E=8, k=2, cfg=2):
    """Workload 2 (bf16, 8 experts, top-2 uniform)."""
    x = to_bf16_bits(normal(cfg, 0, (T, K)))
    w = to_bf16_bits(normal(cfg, 1, (E * N, K), std=0.02))
    return dict(cfg=cfg, x=x, w=w, topk=route_uniform(cfg, T, E, k), e0=0, n_local=E,
                E=E, T=T, K=K, N=N, k=k)


def expert_share(T=32768, K=4096, F=1536, cfg=3):
    """Workload 3 (bf16, Zipf top-8 over 384, experts 144..191 local)."""
    topk = route_zipf(cfg, T, k=8)
    x = to_bf16_bits(normal(cfg, 0, (T, K)))
    w1 = to_bf16_bits(normal(cfg, 1, (LOCAL_EXPERTS * F, K), std=0.02))
    w2 = to_bf16_bits(normal(cfg, 2, (LOCAL_EXPERTS * K, F), std=0.02))
    return dict(cfg=cfg, x=x, w1=w1, w2=w2, topk=topk, e0=LOCAL_E0,
                n_local=LOCAL_EXPERTS, E=LOCAL_EXPERTS, T=T, K=K, N=F, k=8)


def expert_share_hidden(M, F=1536, cfg=3):
    """Workload 3's second-GEMM input H bf16 [M, F] ~ N(0,1)."""
    return to_bf16_bits(normal(cfg, 4, (M, F)))


def backward_dy(M, N, cfg=4, std=1e-3):
    """Workload 4 output gradient dY bf16 [M, N] ~ N(0, std^2)."""
    return to_bf16_bits(normal(cfg, 3, (M, N), std=std))


def decode(T=512, K=4096, F=1536, cfg=5):
    """Workload 5a (decode: top-8 uniform over 384, experts 144..191 local)."""
    topk = route_uniform(cfg, T, N_EXPERTS, 8)
    x = to_bf16_bits(normal(cfg, 0, (T, K)))
    w1 = to_bf16_bits(normal(cfg, 1, (LOCAL_EXPERTS * F, K), std=0.02))
    w2 = to_bf16_bits(normal(cfg, 2, (LOCAL_EXPERTS * K, F), std=0.02))
    return dict(cfg=cfg, x=x, w1=w1, w2=w2, topk=topk, e0=LOCAL_E0,
                n_local=LOCAL_EXPERTS, E=LOCAL_EXPERTS, T=T, K=K, N=F, k=8)


def streaming(rows=262144, cols=2048, cfg=5, tid=0):
    """Workload 5b: bf16 [rows, cols] ~ N(0,1) (1 GiB at the default size)."""
    return to_bf16_bits(normal(cfg, 10 + tid, (rows, cols)))


def moe_case(seed, T, K, N, E, k, routing="uniform", n_experts=None, e0=0,
             x_std=1.0, w_std=0.02, dy_std=1e-3, outliers=False, fp32=False):
    """A scaled-down expert layer for parity tests: same recipe as the
    workloads above at a size the oracle finishes in seconds.

    routing 'uniform': k distinct of n_experts (default E) uniformly;
    'zipf': Zipf(1.1) Gumbel-top-k over n_experts with the round-robin
    placement; local experts are [e0, e0+E).
    """
    n_experts = E if n_experts is None else n_experts
    x = normal(seed, 0, (T, K), std=x_std)
    w = normal(seed, 1, (E * N, K), std=w_std)
    dy = normal(seed, 3, (T * k, N), std=dy_std)
    if outliers:
        with_outliers(x, seed, 6)
        with_outliers(w, seed, 7)
    if routing == "uniform":
        topk = route_uniform(seed, T, n_experts, k)
    else:
        topk = route_zipf(seed, T, k=k, n_experts=n_experts)
    if not fp32:
        x, w, dy = to_bf16_bits(x), to_bf16_bits(w), to_bf16_bits(dy)
    return dict(cfg=seed, x=x, w=w, dy=dy, topk=topk, e0=e0, n_local=E, E=E,
                T=T, K=K, N=N, k=k)


def gates(cfg, T, k, tid=8):
    """Routing weights [T, k] float32: positive, each row summing to one (a
    softmax over the selected experts' scores; the scores are N(0, 1))."""
    s = rng(cfg, tid).standard_normal(size=(T, k))
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def ffn_case(seed, T, K, F, E, k, routing="uniform", n_experts=None, e0=0,
             x_std=1.0, w_std=0.02, dout_std=1e-3, fp32=False):
    """The routed expert FFN (up-projection K -> F, down-projection F -> K)
    at the same recipe as the workloads above: x [T, K], w1 [E, F, K],
    w2 [E, K, F], gate [T, k] float32, dout [T, K]."""
    n_experts = E if n_experts is None else n_experts
    x = normal(seed, 0, (T, K), std=x_std)
    w1 = normal(seed, 1, (E, F, K), std=w_std)
    w2 = normal(seed, 2, (E, K, F), std=w_std)
    dout = normal(seed, 3, (T, K), std=dout_std)
    if routing == "uniform":
        topk = route_uniform(seed, T, n_experts, k)
    else:
        topk = route_zipf(seed, T, k=k, n_experts=n_experts)
    g = gates(seed, T, k)
    if not fp32:
        x, w1, w2, dout = to_bf16_bits(x), to_bf16_bits(w1), to_bf16_bits(w2), to_bf16_bits(dout)
    return dict(cfg=seed, x=x, w1=w1, w2=w2, dout=dout, topk=topk, gate=g, e0=e0, n_local=E,
                E=E, T=T, K=K, F=F, k=k)
