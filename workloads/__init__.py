"""Seeded synthetic inputs for the batch-1 decode MoE FFN stage.

This module serves both the CPU oracle and the HIP library (tests and
benchmark) and holds none of the stage's arithmetic: it draws random numbers
and packs them into the block formats the weights are stored in.  The
quantisers here only make weight bytes; both sides then read the same bytes.

Workloads (shapes of a Qwen3.6-35B-A3B MoE layer and smaller variants):
  tiny      H=512,  E=32,  k=4, F=128, shared 128, router rows duplicated in pairs
  layer     H=2048, E=256, k=8, F=512, shared 512 (one layer)
  stack     40 layers of `layer`, 128 tokens, fresh inputs per token
  e128      H=2048, E=128, k=8, F=768, no shared expert, 48 layers,
            router rows duplicated in groups of 4, 10% of tokens all-zero
  batch     `layer` shape at batch 8 and 32

Weight byte layouts (all little-endian):
  Q4_K 144 B: d f16 | dmin f16 | scales[12] | qs[128]
  Q5_K 176 B: d f16 | dmin f16 | scales[12] | qh[32] | qs[128]
  Q8_0  34 B: d f16 | q int8[32]
  Matrices are [rows][K/256 blocks] (K-quants) or [rows][K/32 blocks] (Q8_0);
  stacked expert matrices are [E][rows][...].
"""
from dataclasses import dataclass, field, replace

import numpy as np
import torch

Q8_0, Q8_1, Q4_K, Q5_K = 8, 9, 12, 13
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q8_0: 34, Q8_1: 36}
BLOCK_ELEMS = {Q4_K: 256, Q5_K: 256, Q8_0: 32, Q8_1: 32}
TYPE_NAMES = {Q4_K: "q4_k", Q5_K: "q5_k", Q8_0: "q8_0"}


@dataclass(frozen=True)
class Config:
    name: str
    H: int
    E: int
    k: int
    F: int
    Fs: int
    layers: int = 1
    tokens: int = 1
    batch: int = 1
    norm: bool = True            # False: the fp32 input is the router/FFN input directly
    three_input: bool = True     # residual + routed + shared (False: residual + routed)
    router_dup: int = 1          # router rows duplicated in groups of this size
    zero_token_frac: float = 0.0
    gate_up_type: int = Q4_K
    down_type: int = Q4_K
    shared_type: int = Q4_K
    eps: float = 1e-6
    weight_std: float = 0.02
    config_index: int = 0
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "tiny": Config("tiny", H=512, E=32, k=4, F=128, Fs=128, norm=False, router_dup=2, config_index=0),
    "layer": Config("layer", H=2048, E=256, k=8, F=512, Fs=512, tokens=128, config_index=1),
    "stack": Config("stack", H=2048, E=256, k=8, F=512, Fs=512, layers=40, tokens=128, config_index=2),
    "e128": Config("e128", H=2048, E=128, k=8, F=768, Fs=0, layers=48, tokens=128, three_input=False,
                   router_dup=4, zero_token_frac=0.10, config_index=3),
    "batch": Config("batch", H=2048, E=256, k=8, F=512, Fs=512, batch=32, config_index=4),
}


def variant(cfg, **kw):
    return replace(cfg, **kw)


def pad_k(typ, K):
    return (K + 255) // 256 * 256 if typ in (Q4_K, Q5_K) else (K + 31) // 32 * 32


def row_bytes(typ, K):
    assert K % BLOCK_ELEMS[typ] == 0
    return K // BLOCK_ELEMS[typ] * BLOCK_BYTES[typ]


# ------------------------------------------------------------------ seeds
# Tensor ids for the seed spawn key.
T_NORM, T_ROUTER, T_SGATE, T_GATE, T_UP, T_DOWN, T_SG, T_SU, T_SD, T_INPUT, T_RPREV, T_SPREV, T_ZERO, T_PAIR, T_STEER, \
    T_ATTN = range(16)


def seed_for(cfg_index, layer, tensor, expert=0, base=0):
    """64-bit seed from SeedSequence(base) with spawn key (config, layer, tensor, expert)."""
    ss = np.random.SeedSequence(base, spawn_key=(cfg_index, layer, tensor, expert))
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed, device="cpu", std=1.0):
    g = _gen(seed, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def rand_uniform(shape, seed, lo, hi, device="cpu"):
    g = _gen(seed, device)
    return lo + (hi - lo) * torch.rand(shape, generator=g, device=device, dtype=torch.float32)


# ------------------------------------------------------------------ encoders (data generation only)
def _f16_bytes(t):
    """fp16 tensor [..., n] -> uint8 [..., 2n] little-endian."""
    return t.to(torch.float16).contiguous().view(torch.uint8)


def pack_kquant_scales(sc, m):
    """sc, m: int tensors [..., 8] in 0..63 -> uint8 [..., 12].

    Sub-blocks 0..3 keep scale/min in the low 6 bits of bytes j and j+4;
    sub-blocks 4..7 keep their low 4 bits in the two nibbles of byte j+4 (for
    j = 4..7, i.e. bytes 8..11) and their top 2 bits in the top 2 bits of
    bytes j-4 (scale) and j (min)."""
    sc = sc.to(torch.int32)
    m = m.to(torch.int32)
    lo_sc, hi_sc = sc[..., :4], sc[..., 4:]
    lo_m, hi_m = m[..., :4], m[..., 4:]
    b0 = lo_sc | ((hi_sc >> 4) << 6)
    b1 = lo_m | ((hi_m >> 4) << 6)
    b2 = (hi_sc & 0xF) | ((hi_m & 0xF) << 4)
    return torch.cat([b0, b1, b2], dim=-1).to(torch.uint8)


def pack_nibbles(q):
    """q: int tensor [..., 256] in 0..15 -> uint8 [..., 128]: byte 32g+l holds
    element 64g+l (low nibble) and element 64g+32+l (high nibble)."""
    q = q.to(torch.int32).reshape(*q.shape[:-1], 4, 2, 32)
    b = q[..., 0, :] | (q[..., 1, :] << 4)
    return b.reshape(*q.shape[:-3], 128).to(torch.uint8)


def pack_high_bits(q5):
    """q5: int tensor [..., 256] in 0..31 -> qh uint8 [..., 32]: bit 2g of qh[l]
    is bit 4 of element 64g+l, bit 2g+1 that of element 64g+32+l."""
    hb = ((q5.to(torch.int32) >> 4) & 1).reshape(*q5.shape[:-1], 4, 2, 32)
    qh = torch.zeros(*q5.shape[:-1], 32, dtype=torch.int32, device=q5.device)
    for g in range(4):
        qh |= hb[..., g, 0, :] << (2 * g)
        qh |= hb[..., g, 1, :] << (2 * g + 1)
    return qh.to(torch.uint8)


def assemble_kquant(d, dmin, sc, m, q, typ):
    """Build K-quant blocks from fields: d, dmin fp tensors [...]; sc, m [..., 8]; q [..., 256]."""
    parts = [_f16_bytes(d.unsqueeze(-1)), _f16_bytes(dmin.unsqueeze(-1)), pack_kquant_scales(sc, m)]
    if typ == Q5_K:
        parts.append(pack_high_bits(q))
        parts.append(pack_nibbles(q & 0xF))
    else:
        parts.append(pack_nibbles(q))
    return torch.cat(parts, dim=-1)


def quantize_kquant(x, typ):
    """fp32 [..., K] -> K-quant bytes [..., K/256*bytes].  A simple min/max rule:
    per 32-element sub-block, step = (max - min(0, min)) / nmax and offset
    = -min(0, min); the block scales d, dmin are the largest step/offset over 63
    (rounded to fp16); the 6-bit sc, m round step/d and offset/dmin; codes
    round (x + dmin*m) / (d*sc) into 0..nmax."""
    nmax = 15 if typ == Q4_K else 31
    K = x.shape[-1]
    assert K % 256 == 0
    xb = x.reshape(*x.shape[:-1], K // 256, 8, 32).to(torch.float32)
    lo = torch.clamp(xb.amin(-1), max=0.0)
    hi = xb.amax(-1)
    step = (hi - lo) / nmax
    off = -lo
    d = (step.amax(-1) / 63.0).to(torch.float16).to(torch.float32)
    dmin = (off.amax(-1) / 63.0).to(torch.float16).to(torch.float32)
    sc = torch.where(d.unsqueeze(-1) > 0, torch.round(step / d.unsqueeze(-1).clamp_min(1e-30)), torch.zeros_like(step))
    m = torch.where(dmin.unsqueeze(-1) > 0, torch.round(off / dmin.unsqueeze(-1).clamp_min(1e-30)), torch.zeros_like(off))
    sc = sc.clamp(0, 63)
    m = m.clamp(0, 63)
    eff_step = (d.unsqueeze(-1) * sc).unsqueeze(-1)
    eff_off = (dmin.unsqueeze(-1) * m).unsqueeze(-1)
    q = torch.where(eff_step > 0, torch.round((xb + eff_off) / eff_step.clamp_min(1e-30)), torch.zeros_like(xb))
    q = q.clamp(0, nmax).to(torch.int32).reshape(*x.shape[:-1], K // 256, 256)
    blocks = assemble_kquant(d, dmin, sc.to(torch.int32), m.to(torch.int32), q, typ)
    return blocks.reshape(*x.shape[:-1], -1)


def quantize_q8_0(x):
    """fp32 [..., K] -> Q8_0 bytes [..., K/32*34]: d = fp16(amax/127), q = round(x/d)."""
    K = x.shape[-1]
    assert K % 32 == 0
    xb = x.reshape(*x.shape[:-1], K // 32, 32).to(torch.float32)
    d = (xb.abs().amax(-1) / 127.0).to(torch.float16).to(torch.float32)
    q = torch.where(d.unsqueeze(-1) > 0, torch.round(xb / d.unsqueeze(-1).clamp_min(1e-30)), torch.zeros_like(xb))
    q = q.clamp(-127, 127).to(torch.int8)
    out = torch.cat([_f16_bytes(d.unsqueeze(-1)), q.view(torch.uint8)], dim=-1)
    return out.reshape(*x.shape[:-1], -1)


def quantize(x, typ):
    return quantize_q8_0(x) if typ == Q8_0 else quantize_kquant(x, typ)


def quantize_padded(x, typ):
    """Zero-pad the last dim to a whole block of `typ`, then quantise."""
    K = x.shape[-1]
    Kp = pad_k(typ, K)
    if Kp != K:
        x = torch.nn.functional.pad(x, (0, Kp - K))
    return quantize(x, typ)


# ------------------------------------------------------------------ weights
def _router_rows(cfg, layer, device):
    """Router [E][H] fp32 ~N(0, std); rows duplicated in groups of router_dup."""
    distinct = cfg.E // cfg.router_dup
    base = randn((distinct, cfg.H), seed_for(cfg.config_index, layer, T_ROUTER), device, cfg.weight_std)
    return base.repeat_interleave(cfg.router_dup, dim=0).contiguous()


def _expert_matrix(cfg, layer, tensor, rows, K, typ, device, chunk_elems=1 << 27):
    """[E][rows][K] ~N(0, std) quantised to typ, generated one expert group at a time."""
    Kp = pad_k(typ, K)
    out = torch.empty((cfg.E, rows, row_bytes(typ, Kp)), dtype=torch.uint8, device=device)
    per = max(1, chunk_elems // (rows * K))
    for e0 in range(0, cfg.E, per):
        e1 = min(cfg.E, e0 + per)
        xs = [randn((rows, K), seed_for(cfg.config_index, layer, tensor, e), device, cfg.weight_std)
              for e in range(e0, e1)]
        x = torch.stack(xs)
        out[e0:e1] = quantize_padded(x, typ)
    return out


def layer_weights(cfg, layer=0, device="cpu", shared_type=None, down_type=None):
    """All weights of one layer as torch tensors on `device`."""
    shared_type = cfg.shared_type if shared_type is None else shared_type
    down_type = cfg.down_type if down_type is None else down_type
    w = {}
    w["norm_w"] = rand_uniform((cfg.H,), seed_for(cfg.config_index, layer, T_NORM), 0.5, 1.5, device)
    w["router_w"] = _router_rows(cfg, layer, device)
    w["gate"] = _expert_matrix(cfg, layer, T_GATE, cfg.F, cfg.H, cfg.gate_up_type, device)
    w["up"] = _expert_matrix(cfg, layer, T_UP, cfg.F, cfg.H, cfg.gate_up_type, device)
    w["down"] = _expert_matrix(cfg, layer, T_DOWN, cfg.H, cfg.F, down_type, device)
    if cfg.Fs > 0:
        w["shared_gate_w"] = randn((cfg.H,), seed_for(cfg.config_index, layer, T_SGATE), device, cfg.weight_std)
        sg = randn((cfg.Fs, cfg.H), seed_for(cfg.config_index, layer, T_SG), device, cfg.weight_std)
        su = randn((cfg.Fs, cfg.H), seed_for(cfg.config_index, layer, T_SU), device, cfg.weight_std)
        sd = randn((cfg.H, cfg.Fs), seed_for(cfg.config_index, layer, T_SD), device, cfg.weight_std)
        w["sgate"] = quantize_padded(sg, shared_type)
        w["sup"] = quantize_padded(su, shared_type)
        w["sdown"] = quantize_padded(sd, shared_type)
    w["_shared_type"] = shared_type
    w["_down_type"] = down_type
    return w


# ------------------------------------------------------------------ per-token inputs
def bf16_bits(t):
    """float tensor -> bf16 bit patterns (int16 viewed as uint16 numpy on host)."""
    return t.to(torch.bfloat16).view(torch.int16)


def token_inputs(cfg, token, device="cpu", layer=0):
    """Inputs of one token.
    norm=False: {'x': fp32 [H]}.
    norm=True:  {'residual', 'routed_prev', 'shared_prev'} bf16 [H] (shared_prev only
    for the 3-input form).  Tokens picked by zero_token_frac get an all-zero residual."""
    seed = seed_for(cfg.config_index, layer, T_INPUT, token)
    if not cfg.norm:
        return {"x": randn((cfg.H,), seed, device)}
    res = randn((cfg.H,), seed, device)
    if cfg.zero_token_frac > 0 and is_zero_token(cfg, token):
        res = torch.zeros_like(res)
    out = {"residual": res.to(torch.bfloat16)}
    return out


def attention_output(cfg, token, layer, device="cpu", std=1.0):
    """The attention block's output of one layer for one token: bf16 [H] drawn
    ~N(0, std) (a stand-in for the block the MoE stage follows; its own
    arithmetic is outside the stage)."""
    return randn((cfg.H,), seed_for(cfg.config_index, layer, T_ATTN, token), device, std).to(torch.bfloat16)


def prev_outputs(cfg, token, device="cpu", layer=0):
    """Independent bf16 N(0,1) draws for the previous layer's routed/shared outputs
    (used when one layer is run on its own)."""
    r = randn((cfg.H,), seed_for(cfg.config_index, layer, T_RPREV, token), device).to(torch.bfloat16)
    out = {"routed_prev": r}
    if cfg.three_input and cfg.Fs > 0:
        out["shared_prev"] = randn((cfg.H,), seed_for(cfg.config_index, layer, T_SPREV, token), device).to(torch.bfloat16)
    return out


def batch_pair(cfg, layer=0):
    """The two experts A < B that a quarter of a batch is steered to (seeded)."""
    rng = np.random.default_rng(seed_for(cfg.config_index, layer, T_PAIR))
    a, b = sorted(int(e) for e in rng.choice(cfg.E, size=2, replace=False))
    return a, b


def steered_tokens(cfg, n_tok, layer=0, frac=0.25):
    """Seeded choice of round(frac * n_tok) token indices of a batch."""
    rng = np.random.default_rng(seed_for(cfg.config_index, layer, T_STEER, n_tok))
    n = int(round(frac * n_tok))
    return sorted(int(t) for t in rng.choice(n_tok, size=n, replace=False))


def batch_inputs(cfg, n_tok, device="cpu", layer=0, lam=1.0):
    """Inputs of a batch of n_tok tokens (3-input norm form, bf16 [n_tok][H]).
    Every token draws residual, routed_prev and shared_prev ~N(0,1); the
    steered quarter instead gets residual = z + lam*sqrt(H)*unit(w * (R_A + R_B))
    (w the norm weight, R_A, R_B the two chosen router rows, z its own draw)
    and zero previous outputs, which pushes experts A and B to the top of its
    ranking.  Returns (inputs dict, steered token list, (A, B))."""
    res, rp, sp = [], [], []
    for t in range(n_tok):
        r = randn((cfg.H,), seed_for(cfg.config_index, layer, T_INPUT, t), device)
        res.append(r)
        rp.append(randn((cfg.H,), seed_for(cfg.config_index, layer, T_RPREV, t), device))
        sp.append(randn((cfg.H,), seed_for(cfg.config_index, layer, T_SPREV, t), device))
    a, b = batch_pair(cfg, layer)
    steer = steered_tokens(cfg, n_tok, layer)
    if steer:
        w = rand_uniform((cfg.H,), seed_for(cfg.config_index, layer, T_NORM), 0.5, 1.5, device)
        rows = _router_rows(cfg, layer, device)
        v = w * (rows[a] + rows[b])
        v = v / torch.linalg.vector_norm(v)
        for t in steer:
            res[t] = res[t] + lam * (cfg.H ** 0.5) * v
            rp[t] = torch.zeros_like(rp[t])
            sp[t] = torch.zeros_like(sp[t])
    out = {"residual": torch.stack(res).to(torch.bfloat16),
           "routed_prev": torch.stack(rp).to(torch.bfloat16),
           "shared_prev": torch.stack(sp).to(torch.bfloat16)}
    return out, steer, (a, b)


def zero_tokens(cfg, n_tokens):
    """Seeded choice of round(frac * n) token indices whose input is all zero."""
    n_zero = int(round(cfg.zero_token_frac * n_tokens))
    rng = np.random.default_rng(seed_for(cfg.config_index, 0, T_ZERO))
    return set(int(i) for i in rng.choice(n_tokens, size=n_zero, replace=False))


def is_zero_token(cfg, token, n_tokens=None):
    return token in zero_tokens(cfg, n_tokens or cfg.tokens)


def to_numpy_weights(w):
    """torch weight dict -> numpy dict (host) for the oracle."""
    out = {}
    for k, v in w.items():
        if k.startswith("_"):
            continue
        out[k] = v.detach().cpu().contiguous().numpy()
    return out


def u16(t):
    """bf16 torch tensor -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
