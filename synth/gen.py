"""Seeded generators.  Every tensor gets its own generator whose seed is a
function of (config id, layer, expert, tensor id) only, so any single tensor of
any layer can be regenerated on its own (the 32-layer stack never has to be
held on the host).

Values depend on the device the generator runs on (torch's CPU and GPU streams
differ); a caller that feeds both the oracle and the GPU generates once and
copies.  Float16 tensors are drawn in float32 and rounded to nearest-even.
"""
import math

import numpy as np
import torch

_BASE = 250402658

# tensor ids
TID_X, TID_LOGITS, TID_ZIPF_PERM, TID_RANKS = 1, 2, 3, 4
TID_W1, TID_W3, TID_W2 = 10, 11, 12
TID_A1, TID_B1, TID_A3, TID_B3, TID_A2, TID_B2 = 20, 21, 22, 23, 24, 25
TID_W, TID_A, TID_B = 40, 41, 42


def tensor_seed(cfg_id: int, layer: int, expert: int, tid: int) -> int:
    ss = np.random.SeedSequence([_BASE, cfg_id, layer, expert, tid])
    a, b = ss.generate_state(2, dtype=np.uint32)
    return (int(a) << 31) ^ int(b)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, sigma, seed, device, dtype=torch.float32):
    g = _gen(seed, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(sigma)
    return t.to(dtype)


def gen_linear(cfg, device="cpu"):
    """C1-style single linear: returns dict of X (fp16 [M][K]), W (fp32 [N][K]),
    A (fp16 [K][r]), B (fp16 [r][N])."""
    c = cfg.cfg_id
    return {
        "X": _normal((cfg.M, cfg.K), cfg.x_sigma, tensor_seed(c, 0, 0, TID_X), device, torch.float16),
        "W": _normal((cfg.N, cfg.K), cfg.w_sigma, tensor_seed(c, 0, 0, TID_W), device),
        "A": _normal((cfg.K, cfg.rank), cfg.lr_sigma, tensor_seed(c, 0, 0, TID_A), device, torch.float16),
        "B": _normal((cfg.rank, cfg.N), cfg.lr_sigma, tensor_seed(c, 0, 0, TID_B), device, torch.float16),
    }


def gen_tokens(cfg, layer=0, device="cpu"):
    """Activations X fp16 [T][H] ~ N(0, x_sigma).  Every layer of a stack uses
    the same X (layer argument kept for completeness; callers pass 0)."""
    return _normal((cfg.T, cfg.H), cfg.x_sigma, tensor_seed(cfg.cfg_id, layer, 0, TID_X), device, torch.float16)


def gen_logits(cfg, layer=0, device="cpu"):
    """Router logits fp32 [T][E].  Plain N(0, sigma), or for a Zipf(alpha) skew
    N(0,1) + log p_{perm(e)} with p_i proportional to i^-alpha (i = 1..E) and a
    seeded permutation perm of the experts."""
    lg = _normal((cfg.T, cfg.E), cfg.logit_sigma, tensor_seed(cfg.cfg_id, layer, 0, TID_LOGITS), device)
    if cfg.zipf_alpha > 0:
        rng = np.random.default_rng(tensor_seed(cfg.cfg_id, layer, 0, TID_ZIPF_PERM))
        perm = rng.permutation(cfg.E)
        i = np.arange(1, cfg.E + 1, dtype=np.float64)
        p = i ** (-cfg.zipf_alpha)
        p /= p.sum()
        bias = np.log(p)[perm].astype(np.float32)
        lg = lg + torch.from_numpy(bias).to(device)
    return lg.contiguous()


def gen_ranks(cfg, layer=0):
    """Per-expert compensator ranks (host int list, E routed then S shared).
    Routed experts draw uniformly from cfg.ranks; shared experts get
    cfg.shared_rank."""
    rng = np.random.default_rng(tensor_seed(cfg.cfg_id, layer, 0, TID_RANKS))
    r = [int(x) for x in rng.choice(np.asarray(cfg.ranks), size=cfg.E)]
    return r + [int(cfg.shared_rank)] * cfg.S


def gen_expert(cfg, layer, expert, rank, device="cpu", which=("W1", "W3", "W2")):
    """One expert's weights: W1, W3 fp32 [F][H]; W2 fp32 [H][F]; compensators
    A1, A3 fp16 [H][r], B1, B3 fp16 [r][F], A2 fp16 [F][r], B2 fp16 [r][H]."""
    c, H, F = cfg.cfg_id, cfg.H, cfg.F
    out = {}
    spec = {
        "W1": ((F, H), cfg.w_sigma, TID_W1, torch.float32),
        "W3": ((F, H), cfg.w_sigma, TID_W3, torch.float32),
        "W2": ((H, F), cfg.w_sigma, TID_W2, torch.float32),
        "A1": ((H, rank), cfg.lr_sigma, TID_A1, torch.float16),
        "B1": ((rank, F), cfg.lr_sigma, TID_B1, torch.float16),
        "A3": ((H, rank), cfg.lr_sigma, TID_A3, torch.float16),
        "B3": ((rank, F), cfg.lr_sigma, TID_B3, torch.float16),
        "A2": ((F, rank), cfg.lr_sigma, TID_A2, torch.float16),
        "B2": ((rank, H), cfg.lr_sigma, TID_B2, torch.float16),
    }
    names = list(which)
    for w in which:
        names += {"W1": ["A1", "B1"], "W3": ["A3", "B3"], "W2": ["A2", "B2"]}.get(w, [])
    for n in names:
        shape, sig, tid, dt = spec[n]
        out[n] = _normal(shape, sig, tensor_seed(c, layer, expert, tid), device, dt)
    return out


def gen_moe_layer(cfg, layer=0, device="cpu"):
    """Everything one MoE layer needs, on `device`."""
    ranks = gen_ranks(cfg, layer)
    experts = [gen_expert(cfg, layer, e, ranks[e], device) for e in range(cfg.E + cfg.S)]
    return {
        "X": gen_tokens(cfg, 0, device),
        "logits": gen_logits(cfg, layer, device),
        "ranks": ranks,
        "experts": experts,
    }


def bytes_human(n: int) -> str:
    u = ["B", "KB", "MB", "GB", "TB"]
    i = max(0, min(len(u) - 1, int(math.log(max(n, 1), 1000))))
    return f"{n / 1000 ** i:.2f} {u[i]}"
