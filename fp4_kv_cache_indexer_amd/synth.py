"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module holds random-number generation and plain format casts only (the
casts to bfloat16 and to FP8 E4M3 are PyTorch's own round-to-nearest-even
conversions); none of the cache-write, indexer or attention arithmetic lives
here.

Streams: ``numpy.random.Generator(PCG64(SeedSequence([seed, cfg, tensor,
layer])))`` for host-side cases; large device-side cases use a seeded
``torch.Generator`` on the GPU with the same (seed, cfg, tensor, layer)
folded into its seed.
"""

from dataclasses import dataclass

import numpy as np
import torch

# tensor ids of the substreams
T_LATENT, T_GATE, T_QATTN, T_QIDX, T_WIDX, T_KEYS, T_SWA, T_OUTLIER, T_IDXPERM = range(9)

E4M3_CLIP = 448.0


def rng(seed, cfg, tensor, layer=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, tensor, layer])))


def torch_gen(seed, cfg, tensor, layer=0, device="cuda"):
    """Seeded torch generator; ``layer`` also serves as a per-sequence index
    when a large tensor is drawn one sequence at a time."""
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1_000_003 + cfg) * 1_000_033 + tensor) * 1_000_037 + layer)
    return g


def to_bf16_bits(a):
    """float array (numpy or torch) -> bfloat16 bit patterns (numpy uint16 or
    torch int16 view), round-to-nearest-even."""
    if isinstance(a, np.ndarray):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return a.to(torch.bfloat16)


def to_e4m3(a):
    """float array -> FP8 E4M3FN bytes (numpy uint8 or torch uint8), values
    first clipped to +-448 so the cast never produces NaN."""
    if isinstance(a, np.ndarray):
        t = torch.from_numpy(np.clip(np.ascontiguousarray(a, dtype=np.float32), -E4M3_CLIP, E4M3_CLIP))
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return a.clamp(-E4M3_CLIP, E4M3_CLIP).to(torch.float8_e4m3fn).view(torch.uint8)


def latent_np(g, shape, dist="normal", outlier_channels=None, outlier_gain=8.0):
    """Token latents: N(0,1) or Student-t (nu=3), with optional outlier
    channels multiplied by ``outlier_gain``."""
    if dist == "normal":
        x = g.standard_normal(shape, dtype=np.float32)
    elif dist == "t3":
        x = g.standard_t(3, size=shape).astype(np.float32)
    else:
        raise ValueError(dist)
    if outlier_channels is not None:
        x[..., outlier_channels] *= outlier_gain
    return x


def latent_dev(shape, gen, dist="normal", outlier_channels=None, outlier_gain=8.0, device="cuda"):
    """Device-side token latents (float32) with the distributions of
    ``latent_np``: N(0,1), or Student-t (nu=3) drawn as N / sqrt(chi2_3 / 3)."""
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if dist == "t3":
        c = torch.randn(tuple(shape) + (3,), generator=gen, device=device, dtype=torch.float32)
        x = x / torch.sqrt((c * c).sum(-1) / 3.0)
    elif dist != "normal":
        raise ValueError(dist)
    if outlier_channels is not None:
        x[..., torch.as_tensor(np.asarray(outlier_channels), device=device)] *= outlier_gain
    return x


def bf16_host_bits(t):
    """bfloat16 device tensor -> numpy uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def outlier_channels_np(seed, cfg, n=4, dim=512):
    return np.sort(rng(seed, cfg, T_OUTLIER).choice(dim, size=n, replace=False))


@dataclass
class DecodeCase:
    """Host-side inputs of a decode batch (numpy).  The FP4 main-KV cache is
    described by its bf16 token latents ``x_bits`` [S, T, 512] (and optional
    gate logits ``z_bits``); whoever needs the cache quantises them."""
    S: int
    N: int
    R: int
    H: int
    m: int
    top_k: int
    x_bits: np.ndarray          # [S, N*m, 512] uint16 (bf16)
    z_bits: object              # [S, N*m, 512] uint16 or None
    keys: np.ndarray            # [S, N, 128] uint8 (E4M3)
    q_idx: np.ndarray           # [R, 32, 128] uint8 (E4M3)
    w_idx: np.ndarray           # [R, 32] float32
    q: np.ndarray               # [R, H, 512] uint16 (bf16)
    swa: np.ndarray             # [S, cap, 512] uint8 (E4M3)
    swa_start: np.ndarray       # [R] int32
    swa_len: np.ndarray         # [R] int32
    row_seq: np.ndarray         # [R] int32
    n_valid: np.ndarray         # [R] int32


def make_decode_case(seed=0, cfg=0, S=1, N=4096, H=16, m=1, top_k=512, swa_cap=128,
                     swa_len=128, dist="normal", outliers=False, gate=False,
                     w_random=False, R=None, n_valid=None, layer=0):
    """Build a decode batch with one row per sequence (unless R is given, in
    which case rows cycle over the sequences)."""
    R = S if R is None else R
    och = outlier_channels_np(seed, cfg) if outliers else None
    x = latent_np(rng(seed, cfg, T_LATENT), (S, N * m, 512), dist, och)
    z = None
    if gate:
        z = to_bf16_bits(rng(seed, cfg, T_GATE).standard_normal((S, N * m, 512), dtype=np.float32))
    keys = to_e4m3(rng(seed, cfg, T_KEYS).standard_normal((S, N, 128), dtype=np.float32))
    q_idx = to_e4m3(rng(seed, cfg, T_QIDX, layer).standard_normal((R, 32, 128), dtype=np.float32))
    if w_random:
        w = rng(seed, cfg, T_WIDX, layer).uniform(0.25, 1.0, (R, 32)).astype(np.float32)
    else:
        w = np.ones((R, 32), dtype=np.float32)
    q = to_bf16_bits(rng(seed, cfg, T_QATTN, layer).standard_normal((R, H, 512), dtype=np.float32))
    swa = to_e4m3(latent_np(rng(seed, cfg, T_SWA, layer), (S, swa_cap, 512), dist, och))
    row_seq = (np.arange(R) % S).astype(np.int32)
    nv = np.full(R, N, dtype=np.int32) if n_valid is None else np.asarray(n_valid, dtype=np.int32)
    return DecodeCase(S=S, N=N, R=R, H=H, m=m, top_k=top_k, x_bits=to_bf16_bits(x), z_bits=z,
                      keys=keys, q_idx=q_idx, w_idx=w, q=q, swa=swa,
                      swa_start=np.zeros(R, dtype=np.int32),
                      swa_len=np.full(R, swa_len, dtype=np.int32),
                      row_seq=row_seq, n_valid=nv)
