"""Seeded synthetic inputs: BF16 KV pages and queries.

Shared by the tests, the benchmark and the smoke check on both sides of a parity comparison.
It holds no part of the method's arithmetic: only the value distribution of the workloads.

KV value model (per layer; sigma is per (K|V, KV head, dim) = channel):
  sigma_c = 2**u, u ~ U[-u_max, u_max];  x = sign * sigma_c * clamp(|z|, 2**-6, 8), z ~ N(0,1),
  sign = +-1 with equal odds; x is formed in fp32 and rounded to BF16 (nearest even).
  In a fraction `forced_frac` of the 512-value blocks (16 tokens x 32 dims of one page, K or V,
  KV head) one element, at a uniform position, is set to +-sigma_c * 2**forced_exp.
  Optional stress values, each element independently: exact +-0 (1%), a subnormal with
  mantissa uniform in 1..127 and random sign (0.5%), exponent 255 with mantissa uniform in
  0..127 and random sign, i.e. +-Inf or NaN (0.1%).
`sample` > 0 draws other values (z, signs, forced positions, stress) from the same per-channel
sigma - another sample of the same layer, as calibration data of one model would be.
Queries: q ~ N(0,1), rounded to BF16.
FP8 pages (fp8_kv_pages): the same values converted to E4M3 or E5M2 by torch.
"""
from __future__ import annotations

import torch


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 12345) % (2 ** 63))
    return g


def kv_pages(n_seq: int, n_pages: int, n_kv: int, *, seed: int, layer: int = 0,
             u_max: float = 3.0, forced_frac: float = 0.10, forced_exp: float = 12.0,
             stress: bool = False, sample: int = 0, device="cpu") -> torch.Tensor:
    """BF16 KV pages [n_seq, n_pages, 2 (K,V), n_kv, 16, 128] (natural token-major order)."""
    g = _gen(seed, 2 * layer, device)
    shape = (n_seq, n_pages, 2, n_kv, 16, 128)
    u = torch.rand((2, n_kv, 128), generator=g, device=device) * (2 * u_max) - u_max
    if sample:
        g = _gen(seed, 2 * layer + 1 + 2_000_000 * int(sample), device)
    sigma = torch.exp2(u)                                            # [2, Hkv, 128]
    x = torch.randn(shape, generator=g, device=device)
    x.abs_().clamp_(2.0 ** -6, 8.0)
    neg = torch.rand(shape, generator=g, device=device) < 0.5
    x[neg] *= -1.0
    del neg
    x *= sigma[None, None, :, :, None, :]
    kv = x.to(torch.bfloat16)
    del x

    if forced_frac > 0:
        bshape = (n_seq, n_pages, 2, n_kv, 4)
        pick = torch.rand(bshape, generator=g, device=device) < forced_frac
        pos_t = torch.randint(0, 16, bshape, generator=g, device=device)
        pos_d = torch.randint(0, 32, bshape, generator=g, device=device)
        fneg = torch.rand(bshape, generator=g, device=device) < 0.5
        s, p, c, h, j = pick.nonzero(as_tuple=True)
        t = pos_t[s, p, c, h, j]
        d = 32 * j + pos_d[s, p, c, h, j]
        val = sigma[c, h, d] * (2.0 ** forced_exp)
        val = torch.where(fneg[s, p, c, h, j], -val, val)
        kv[s, p, c, h, t, d] = val.to(torch.bfloat16)

    if stress:
        bits = kv.view(torch.int16)
        r = torch.rand(shape, generator=g, device=device)
        sgn = (torch.rand(shape, generator=g, device=device) < 0.5).to(torch.int32) << 15
        mant = torch.randint(0, 128, shape, generator=g, device=device, dtype=torch.int32)
        zero = r < 0.01
        sub = (r >= 0.01) & (r < 0.015)
        nonfin = (r >= 0.015) & (r < 0.016)
        del r
        w = bits.to(torch.int32) & 0xFFFF
        w = torch.where(zero, sgn, w)
        w = torch.where(sub, sgn | torch.clamp(mant, min=1), w)
        w = torch.where(nonfin, sgn | 0x7F80 | mant, w)
        kv = (((w + 32768) & 0xFFFF) - 32768).to(torch.int16).view(torch.bfloat16)
    return kv


FP8_DTYPES = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}   # KVZ_FP8_E4M3, KVZ_FP8_E5M2


def fp8_kv_pages(n_seq: int, n_pages: int, n_kv: int, *, seed: int, fmt: int, layer: int = 0,
                 u_max: float = 3.0, forced_frac: float = 0.05, forced_exp: float = 4.0,
                 stress: bool = False, sample: int = 0, device="cpu") -> torch.Tensor:
    """FP8 KV pages [n_seq, n_pages, 2, n_kv, 16, 128] as uint8 bytes: the BF16 value model
    above (forced elements at +-sigma_c * 2**forced_exp, which stays inside E4M3's range for
    u_max <= 3), converted to FP8 by torch (round to nearest even) - the initial FP8 conversion
    of a KV cache.  Stress values, each element independently: +-0 (1%), a subnormal (exponent
    field 0, nonzero fraction, 0.5%), an all-ones exponent field with any fraction and sign (NaN
    in E4M3 only for fraction 7; Inf or NaN in E5M2) (0.1%)."""
    kv = kv_pages(n_seq, n_pages, n_kv, seed=seed, layer=layer, u_max=u_max,
                  forced_frac=forced_frac, forced_exp=forced_exp, stress=False, sample=sample,
                  device=device)
    x = kv.float().to(FP8_DTYPES[fmt]).view(torch.uint8)
    del kv
    if stress:
        g = _gen(seed, 3_000_003 + 2 * layer + 7 * int(sample), device)
        shape = x.shape
        mw = 3 if fmt == 0 else 2
        r = torch.rand(shape, generator=g, device=device)
        sgn = (torch.rand(shape, generator=g, device=device) < 0.5).to(torch.int32) << 7
        frac = torch.randint(0, 1 << mw, shape, generator=g, device=device, dtype=torch.int32)
        w = x.to(torch.int32)
        w = torch.where(r < 0.01, sgn, w)
        w = torch.where((r >= 0.01) & (r < 0.015), sgn | torch.clamp(frac, min=1), w)
        top = (0x78 if fmt == 0 else 0x7C)
        w = torch.where((r >= 0.015) & (r < 0.016), sgn | top | frac, w)
        x = w.to(torch.uint8)
    return x.contiguous()


def queries(batch: int, num_q_heads: int, *, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, 1_000_001, device)
    return torch.randn((batch, num_q_heads, 128), generator=g, device=device).to(torch.bfloat16)


def bits(t: torch.Tensor):
    """BF16 tensor -> numpy uint16 bit patterns (on the host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
