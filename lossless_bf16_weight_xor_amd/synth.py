"""Seeded synthetic BF16 checkpoint pairs (workload generator).

This module draws random numbers and builds (old, new) weight pairs.  The
CPU oracle and the GPU path both consume its output.  It contains none of
the compression method: no XOR of checkpoints, no classification and no
packing.  Each mutation is built bitwise so that it belongs to a known
change class:

* mantissa-only: the 7-bit mantissa moves by k ulps, with a random sign and
  k ~ Geometric(1/2) on {1, 2, ...}; a draw that would leave [0, 127] is redrawn;
* exponent: the 8-bit exponent moves by +-1 and is kept inside [1, 254]
  (for normal values this is a scale by 2^+-1);
* sign: the sign bit is flipped.

The pages report roughly 2% (or 1%) of BF16 elements changing per step, most
of them mantissa-only and few exponent or sign changes ("Every byte counts:
ARCv3 and the case for cross-region RL", section "Deep dive into ARCv3";
"NeMo-DCR Cuts Trillion-Parameter Agentic RL Refits by About 35x", section
"Why refitting becomes a bottleneck").  They give no dataset, so every input
here is synthetic: weights ~ N(0, 0.02) rounded to bfloat16, and change
counts are fixed exactly as k = floor(rate * n + 1/2).

The module works on torch tensors on any device.  Large configurations are
generated on the GPU.  Bit patterns are handled as int32 values in
[0, 65535].
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Iterator

import torch

STD = 0.02
MIX_DEFAULT = (Fraction(95, 100), Fraction(45, 1000), Fraction(5, 1000))   # mant, exp, sign
MIX_ADVERSARIAL = (Fraction(60, 100), Fraction(30, 100), Fraction(10, 100))


# ---------------------------------------------------------------- basics ---

def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, gen: torch.Generator, device, std: float = STD) -> torch.Tensor:
    """Weights ~ N(0, std) drawn in fp32 and rounded to bfloat16 (nearest-even)."""
    return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std
            ).to(torch.bfloat16)


def exact_count(rate, n: int) -> int:
    """k = floor(rate * n + 1/2), computed with exact rationals."""
    r = Fraction(str(rate)) if not isinstance(rate, Fraction) else rate
    return int((r * n + Fraction(1, 2)).__floor__())


def class_counts(k: int, mix=MIX_DEFAULT) -> tuple[int, int, int]:
    """(n_mant, n_exp, n_sign) for k changes: the rarer two rounded, the rest mantissa."""
    _, f_exp, f_sign = mix
    n_sign = int((k * f_sign + Fraction(1, 2)).__floor__())
    n_exp = int((k * f_exp + Fraction(1, 2)).__floor__())
    return k - n_exp - n_sign, n_exp, n_sign


def bits(t: torch.Tensor) -> torch.Tensor:
    """bfloat16 tensor -> int32 tensor of its 16-bit patterns in [0, 65535]."""
    return t.contiguous().view(torch.int16).to(torch.int32) & 0xFFFF


def from_bits(v: torch.Tensor) -> torch.Tensor:
    """int32 patterns in [0, 65535] -> bfloat16 tensor."""
    return torch.where(v >= 32768, v - 65536, v).to(torch.int16).view(torch.bfloat16)


# ------------------------------------------------------------- mutations ---

def _mutate_mantissa(v: torch.Tensor, gen: torch.Generator) -> torch.Tensor:
    m = v & 0x7F
    out = torch.empty_like(m)
    todo = torch.arange(v.numel(), device=v.device)
    while todo.numel():
        sign = torch.randint(0, 2, (todo.numel(),), generator=gen, device=v.device,
                             dtype=torch.int32) * 2 - 1
        step = torch.empty(todo.numel(), device=v.device, dtype=torch.float32)
        step.geometric_(0.5, generator=gen)
        k = step.to(torch.int32)
        cand = m[todo] + sign * k
        # geometric_ can return 0 when its uniform draw is exactly 1; that is
        # outside the support {1, 2, ...} and is redrawn like a binade crossing
        ok = (k >= 1) & (cand >= 0) & (cand <= 127)
        out[todo[ok]] = cand[ok]
        todo = todo[~ok]
    return (v & 0xFF80) | out


def _mutate_exponent(v: torch.Tensor, gen: torch.Generator) -> torch.Tensor:
    e = (v >> 7) & 0xFF
    d = torch.randint(0, 2, v.shape, generator=gen, device=v.device, dtype=torch.int32) * 2 - 1
    d = torch.where(((e + d) < 1) | ((e + d) > 254), -d, d)
    return (v & 0x807F) | ((e + d) << 7)


def _mutate_sign(v: torch.Tensor) -> torch.Tensor:
    return v ^ 0x8000


def mutate(src: torch.Tensor, positions: torch.Tensor, counts, gen: torch.Generator
           ) -> torch.Tensor:
    """dst = src with positions[:n_mant] mantissa-nudged, the next n_exp exponent-shifted
    and the last n_sign sign-flipped.  `positions` must be distinct and in random order."""
    n_mant, n_exp, n_sign = counts
    assert positions.numel() == n_mant + n_exp + n_sign
    flat = bits(src.reshape(-1))
    out = flat.clone()
    pm = positions[:n_mant]
    pe = positions[n_mant:n_mant + n_exp]
    ps = positions[n_mant + n_exp:]
    if pm.numel():
        out[pm] = _mutate_mantissa(flat[pm], gen)
    if pe.numel():
        out[pe] = _mutate_exponent(flat[pe], gen)
    if ps.numel():
        out[ps] = _mutate_sign(flat[ps])
    return from_bits(out).reshape(src.shape)


# ------------------------------------------------------- position layouts ---

def uniform_positions(n: int, k: int, gen: torch.Generator, device) -> torch.Tensor:
    """k distinct positions, uniform without replacement, in random order."""
    if k == 0:
        return torch.empty(0, dtype=torch.int64, device=device)
    return torch.randperm(n, generator=gen, device=device)[:k]


def clustered_positions(rows: int, cols: int, k: int, gen: torch.Generator, device,
                        hot_row_frac=Fraction(1, 10), hot_share=Fraction(7, 10)
                        ) -> torch.Tensor:
    """70% of the k positions uniform among the elements of 10% of the rows (chosen at
    random), the rest uniform among the other rows; random order."""
    hot = int((rows * hot_row_frac + Fraction(1, 2)).__floor__())
    k_hot = int((k * hot_share + Fraction(1, 2)).__floor__())
    k_cold = k - k_hot
    row_perm = torch.randperm(rows, generator=gen, device=device)
    hot_rows, cold_rows = row_perm[:hot], row_perm[hot:]
    assert k_hot <= hot * cols and k_cold <= (rows - hot) * cols
    col = torch.arange(cols, device=device)

    def pick(row_set, kk):
        if kk == 0:
            return torch.empty(0, dtype=torch.int64, device=device)
        idx = torch.randperm(row_set.numel() * cols, generator=gen, device=device)[:kk]
        return row_set[idx // cols] * cols + col[idx % cols]

    pos = torch.cat([pick(hot_rows, k_hot), pick(cold_rows, k_cold)])
    return pos[torch.randperm(pos.numel(), generator=gen, device=device)]


def run_positions(n: int, k: int, gen: torch.Generator, device, max_run: int = 256
                  ) -> torch.Tensor:
    """k positions in contiguous runs of U{1..max_run} elements (the last run cut to
    fit), separated by a uniformly random composition of the n-k unchanged elements
    into gaps >= 0 (leading and trailing gaps included); random order."""
    if k == 0:
        return torch.empty(0, dtype=torch.int64, device=device)
    chunks = []
    total = 0
    while total < k:
        draw = torch.randint(1, max_run + 1, (2 * (k - total) // max_run + 64,),
                             generator=gen, device=device)
        chunks.append(draw)
        total += int(draw.sum())
    lens_t = torch.cat(chunks)
    ends = torch.cumsum(lens_t, 0)
    m = int(torch.searchsorted(ends, torch.tensor([k], device=device))[0]) + 1
    lens_t = lens_t[:m].clone()
    lens_t[-1] -= int(ends[m - 1]) - k          # cut the last run to fit exactly
    # stars and bars: m bar positions among (n - k + m) slots -> m + 1 gaps
    bars = torch.randperm(n - k + m, generator=gen, device=device)[:m].sort().values
    gaps = torch.diff(bars, prepend=torch.tensor([-1], device=device)) - 1
    starts = torch.cumsum(gaps, 0) + torch.cumsum(lens_t, 0) - lens_t
    run_id = torch.repeat_interleave(torch.arange(m, device=device), lens_t)
    offset = torch.arange(k, device=device) - torch.repeat_interleave(
        torch.cumsum(lens_t, 0) - lens_t, lens_t)
    pos = starts[run_id] + offset
    return pos[torch.randperm(k, generator=gen, device=device)]


# -------------------------------------------------------------- workloads ---

@dataclass
class TensorSpec:
    name: str
    shape: tuple


def seven_b_specs() -> list[TensorSpec]:
    """7B-shaped model: 32 layers, hidden 4096, FFN 11008, vocab 32000 (291 tensors)."""
    h, f, v = 4096, 11008, 32000
    specs = [TensorSpec("embed_tokens", (v, h))]
    for i in range(32):
        p = f"layers.{i}."
        specs += [TensorSpec(p + "q_proj", (h, h)), TensorSpec(p + "k_proj", (h, h)),
                  TensorSpec(p + "v_proj", (h, h)), TensorSpec(p + "o_proj", (h, h)),
                  TensorSpec(p + "gate_proj", (f, h)), TensorSpec(p + "up_proj", (f, h)),
                  TensorSpec(p + "down_proj", (h, f)),
                  TensorSpec(p + "input_layernorm", (h,)),
                  TensorSpec(p + "post_attention_layernorm", (h,))]
    specs += [TensorSpec("norm", (h,)), TensorSpec("lm_head", (v, h))]
    return specs


def seventy_b_half_specs() -> list[TensorSpec]:
    """40 of the 80 layers of a 70B-shaped model: hidden 8192, FFN 28672, GQA 64q/8kv
    heads of dim 128 (360 tensors, no embeddings)."""
    h, f, kv = 8192, 28672, 8 * 128
    specs = []
    for i in range(40):
        p = f"layers.{i}."
        specs += [TensorSpec(p + "q_proj", (h, h)), TensorSpec(p + "k_proj", (kv, h)),
                  TensorSpec(p + "v_proj", (kv, h)), TensorSpec(p + "o_proj", (h, h)),
                  TensorSpec(p + "gate_proj", (f, h)), TensorSpec(p + "up_proj", (f, h)),
                  TensorSpec(p + "down_proj", (h, f)),
                  TensorSpec(p + "input_layernorm", (h,)),
                  TensorSpec(p + "post_attention_layernorm", (h,))]
    return specs


def numel(shape) -> int:
    out = 1
    for s in shape:
        out *= s
    return out


def config_seed(config_index: int, item_index: int) -> int:
    return config_index * (1 << 20) + item_index


def make_pair(shape, rate, mix, seed: int, device, layout: str = "uniform"):
    """One (old, new) pair: old ~ N(0, 0.02) in bf16, new = old with exactly
    floor(rate*n + 1/2) mutated elements in the given class mix and layout."""
    gen = generator(seed, device)
    src = normal_bf16(shape, gen, device)
    n = numel(shape)
    k = exact_count(rate, n)
    counts = class_counts(k, mix)
    if layout == "clustered" and len(shape) == 2:
        pos = clustered_positions(shape[0], shape[1], k, gen, device)
    elif layout == "runs":
        pos = run_positions(n, k, gen, device)
    else:
        pos = uniform_positions(n, k, gen, device)
    return src, mutate(src, pos, counts, gen)


def config1(device):
    """Single 1024x1024 tensor, seed 0, 2% uniform changes, 95/4.5/0.5 mix."""
    return make_pair((1024, 1024), "0.02", MIX_DEFAULT, 0, device)


def config2(device, limit: int | None = None) -> Iterator[tuple[str, torch.Tensor, torch.Tensor]]:
    """7B-shaped checkpoint pair, 2% per tensor, clustered (70% of changes in 10% of
    rows) for 2-D tensors, uniform for the 1-D norms."""
    for i, spec in enumerate(seven_b_specs()[:limit]):
        layout = "clustered" if len(spec.shape) == 2 else "uniform"
        src, dst = make_pair(spec.shape, "0.02", MIX_DEFAULT, config_seed(2, i), device, layout)
        yield spec.name, src, dst


C3_RATES = ("0.00085", "0.01", "0.03", "0.05")


def config3(device, rate, n: int = 536_870_912):
    """One 1 GiB 1-D tensor at the given change rate, uniform, 95/4.5/0.5."""
    idx = C3_RATES.index(rate) if rate in C3_RATES else 99
    return make_pair((n,), rate, MIX_DEFAULT, config_seed(3, idx), device)


C4_CASES = ("A_uniform", "B_runs", "C_unchanged", "D_all_changed", "E_specials", "F_odd_length")

SPECIAL_PATTERNS = (0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0x0001, 0x007F)


def config4(device, case: str, n: int = 33_554_432):
    """Adversarial and edge cases on 64 MiB tensors (odd length for case F)."""
    idx = C4_CASES.index(case)
    seed = config_seed(4, idx)
    if case == "A_uniform":
        return make_pair((n,), "0.05", MIX_ADVERSARIAL, seed, device)
    if case == "B_runs":
        return make_pair((n,), "0.05", MIX_ADVERSARIAL, seed, device, layout="runs")
    if case == "C_unchanged":
        gen = generator(seed, device)
        src = normal_bf16((n,), gen, device)
        return src, src.clone()
    if case == "D_all_changed":
        return make_pair((n,), 1, MIX_ADVERSARIAL, seed, device)
    if case == "E_specials":
        return _specials_pair(n, seed, device)
    if case == "F_odd_length":
        return make_pair((n - 1,), "0.05", MIX_ADVERSARIAL, seed, device)
    raise ValueError(case)


def _specials_pair(n: int, seed: int, device):
    """1/16 of the elements replaced by +-0, +-inf, NaNs and subnormals, then 5% changed
    (60/30/10); a few positions are forced to the special transitions +0 -> -0,
    inf -> NaN, NaN payload change, subnormal mantissa change and exponent 0 -> 1."""
    gen = generator(seed, device)
    src_bits = bits(normal_bf16((n,), gen, device))
    n_spec = n // 16
    spec_pos = torch.randperm(n, generator=gen, device=device)[:n_spec]
    pats = torch.tensor(SPECIAL_PATTERNS, dtype=torch.int32, device=device)
    choice = torch.randint(0, len(SPECIAL_PATTERNS) + 1, (n_spec,), generator=gen, device=device)
    sub = torch.randint(1, 128, (n_spec,), generator=gen, device=device, dtype=torch.int32)
    sub = sub | (torch.randint(0, 2, (n_spec,), generator=gen, device=device,
                               dtype=torch.int32) << 15)                  # random subnormal
    vals = torch.where(choice < len(SPECIAL_PATTERNS),
                       pats[choice.clamp(max=len(SPECIAL_PATTERNS) - 1)], sub)
    src_bits[spec_pos] = vals
    src = from_bits(src_bits)
    k = exact_count("0.05", n)
    pos = uniform_positions(n, k, gen, device)
    dst_bits = bits(mutate(src, pos, class_counts(k, MIX_ADVERSARIAL), gen))
    # forced transitions at the first few elements (old -> new pattern pairs)
    forced = ((0x0000, 0x8000), (0x7F80, 0x7F81), (0x7FC0, 0x7FC1),
              (0x0001, 0x0002), (0x0001, 0x0081))
    for i, (a, b) in enumerate(forced):
        src_bits[i] = a
        dst_bits[i] = b
    return from_bits(src_bits), from_bits(dst_bits)


def config5_specs():
    return seventy_b_half_specs()


def config5(device, limit: int | None = None):
    """One-GPU share of a 70B-shaped model (40 of 80 layers), 1% uniform changes."""
    for i, spec in enumerate(seventy_b_half_specs()[:limit]):
        src, dst = make_pair(spec.shape, "0.01", MIX_DEFAULT, config_seed(5, i), device)
        yield spec.name, src, dst


def page_example(seed: int = 0):
    """The pages' API example on the CPU: src ~ randn(1024, 1024) in bf16 and
    dst = src + 1e-3 * randn, computed in bf16 ("Every byte counts: ARCv3 and the
    case for cross-region RL", section "Using ARCv3")."""
    gen = generator(seed, "cpu")
    src = torch.randn((1024, 1024), generator=gen, dtype=torch.bfloat16)
    noise = torch.randn((1024, 1024), generator=gen, dtype=torch.bfloat16)
    return src, src + 1e-3 * noise


# ------------------------------------------------------ the largest sizes ---

def huge_pair(n: int, seed: int, device):
    """A pair for the largest-size checks, built in chunks so no index
    permutation of n elements is needed: old ~ N(0, 0.02) in bf16, and every
    element of new differs from old.  Element i's change flips mantissa bits
    (a non-zero 7-bit pattern drawn per element); when i % 3 == 0 it also
    flips the lowest exponent bit, and when i % 97 == 0 the sign bit too.
    Returns (old, new) as flat bfloat16 tensors."""
    gen = generator(seed, device)
    old = torch.empty(n, dtype=torch.bfloat16, device=device)
    new = torch.empty(n, dtype=torch.bfloat16, device=device)
    step = 1 << 28
    for a in range(0, n, step):
        b = min(n, a + step)
        o = normal_bf16((b - a,), gen, device)
        idx = torch.arange(a, b, device=device, dtype=torch.int64)
        x = torch.randint(1, 128, (b - a,), generator=gen, device=device, dtype=torch.int32)
        x = x | torch.where(idx % 3 == 0, 0x0080, 0).to(torch.int32)
        x = x | torch.where(idx % 97 == 0, 0x8000, 0).to(torch.int32)
        ob = o.view(torch.int16).to(torch.int32) & 0xFFFF
        nb = (ob ^ x).to(torch.int16)
        old[a:b] = o
        new[a:b] = nb.view(torch.bfloat16)
        del o, idx, x, ob, nb
    return old, new
