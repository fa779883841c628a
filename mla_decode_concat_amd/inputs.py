"""Seeded synthetic inputs for the fused MLA decode epilogue.

This module is shared by the tests (which feed the same bytes to the CPU
oracle and to the GPU library) and by the benchmark.  It holds no arithmetic
of the epilogue itself: it only draws random tensors, picks slots and
positions, and builds the rotary table that the epilogue receives as an input
(the prhub summary of vLLM PR #54896, "implementation breakdown" item 2,
lists the rope table among the data the kernel reads).

Shapes follow the page's test (section "key source snippets"): ql_nope
[T, H, 512], q_pe [T, H, 64], kv_c [T, 512], k_pe [T, 64], a zero-filled paged
cache [num_blocks, block_size, 576] and int64 slots drawn as a prefix of a
random permutation of all cache slots.  The page seeds with 3; so do we.
"""
from __future__ import annotations

import dataclasses
import math

import torch

NOPE = 512
PE = 64
ROW = NOPE + PE
DEFAULT_SEED = 3
ROPE_THETA = 10000.0
ROPE_MAX_POSITION = 32768


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    heads: int
    num_blocks: int
    block_size: int = 64
    rope: bool = False
    q_fp8: bool = False
    kv_fp8: bool = False
    # slot recipe: "randint" (one draw in [0, num_slots)) or "randperm"
    # (first T of a permutation of all num_slots slots)
    slots: str = "randperm"
    # position recipe: "none", "uniform:<hi>" or "arange"
    positions: str = "none"
    q_scale: float = 0.05
    kv_scale: float = 0.05
    max_position: int = ROPE_MAX_POSITION
    dtype: str = "bf16"          # activations and unquantised outputs: bf16 | fp16
    rope_style: str = "neox"     # neox (i, i+32) | gptj (2i, 2i+1)
    table_dtype: str = "f32"     # rope table: f32 | bf16

    @property
    def num_slots(self) -> int:
        return self.num_blocks * self.block_size

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16

    def describe(self) -> str:
        bits = [] if self.dtype == "bf16" else [self.dtype]
        if self.rope:
            bits.append("rope" if self.rope_style == "neox" else "rope_gptj")
            if self.table_dtype != "f32":
                bits.append(f"table_{self.table_dtype}")
        if self.q_fp8:
            bits.append(f"q_e4m3(scale={self.q_scale})")
        if self.kv_fp8:
            bits.append(f"kv_e4m3(scale={self.kv_scale})")
        flags = "+".join(bits) if bits else "bf16-copy"
        return (f"T={self.tokens} H={self.heads} cache=[{self.num_blocks},"
                f"{self.block_size},576] {flags}")


# The five workloads: decode sizes around the row-split boundary, the
# full-head decode batch and the prefill-sized bandwidth case.
WORKLOADS = {
    "t1_h16_copy": Workload("t1_h16_copy", 1, 16, 1, slots="randint"),
    "t64_h16_rope_fp8": Workload("t64_h16_rope_fp8", 64, 16, 1, rope=True,
                                 q_fp8=True, kv_fp8=True, positions="uniform:4096"),
    "t65_h16_rope_fp8": Workload("t65_h16_rope_fp8", 65, 16, 2, rope=True,
                                 q_fp8=True, kv_fp8=True, positions="uniform:4096"),
    "t256_h128_rope_qfp8": Workload("t256_h128_rope_qfp8", 256, 128, 4096, rope=True,
                                    q_fp8=True, kv_fp8=False, positions="uniform:32768"),
    "t8192_h16_rope_kvfp8": Workload("t8192_h16_rope_kvfp8", 8192, 16, 4096, rope=True,
                                     q_fp8=False, kv_fp8=True, positions="arange"),
}
WORKLOAD_ORDER = list(WORKLOADS)


def rope_table(max_position: int = ROPE_MAX_POSITION, theta: float = ROPE_THETA,
               rot_dim: int = PE) -> torch.Tensor:
    """[max_position, 64] fp32 table: cos of the 32 angles, then their sin.

    Angle (p, i) = p * theta^(-2i/64), evaluated in float64 and rounded once
    to fp32.  This is the usual rotary frequency ladder; the epilogue takes
    the table as data, so its exact values never enter a parity comparison.
    """
    half = rot_dim // 2
    i = torch.arange(half, dtype=torch.float64)
    inv_freq = theta ** (-2.0 * i / rot_dim)
    p = torch.arange(max_position, dtype=torch.float64)
    ang = p[:, None] * inv_freq[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32).contiguous()


_TABLE_CACHE: dict = {}


def shared_rope_table(max_position: int = ROPE_MAX_POSITION) -> torch.Tensor:
    if max_position not in _TABLE_CACHE:
        _TABLE_CACHE[max_position] = rope_table(max_position)
    return _TABLE_CACHE[max_position]


def make_inputs(w: Workload, seed: int = DEFAULT_SEED) -> dict:
    """CPU tensors for one workload, drawn in a fixed order from one generator:
    ql_nope, q_pe, kv_c, k_pe (N(0,1) fp32 rounded to the activation type,
    bf16 or fp16), then slots, then positions.  The cache starts as zeros."""
    g = torch.Generator().manual_seed(seed)
    T, H = w.tokens, w.heads

    def randn_act(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32).to(w.torch_dtype)

    ql_nope = randn_act(T, H, NOPE)
    q_pe = randn_act(T, H, PE)
    kv_c = randn_act(T, NOPE)
    k_pe = randn_act(T, PE)
    out = dict(ql_nope=ql_nope, q_pe=q_pe, kv_c=kv_c, k_pe=k_pe)
    out.update(_slots_positions_cache(w, g))
    return out


UK_K = 128   # no-position width of a head's query before the W_UK product


def make_uk_inputs(w: Workload, seed: int = DEFAULT_SEED) -> dict:
    """CPU tensors for the epilogue fused into the W_UK product, drawn in a
    fixed order from one generator: the q projection's output q_b
    [T, H, 192] (N(0,1); q_nope is each head's first 128 columns, q_pe its
    last 64, both views of q_b as in a decode step), W_UK transposed per head
    w_uk_t [H, 512, 128] (N(0, 1/128), so that every latent column of the
    product has unit variance like ql_nope in make_inputs), kv_c, k_pe, then
    slots and positions as in make_inputs.  The cache starts as zeros."""
    g = torch.Generator().manual_seed(seed)
    T, H = w.tokens, w.heads

    def randn_act(*shape, scale=1.0):
        return (torch.randn(*shape, generator=g, dtype=torch.float32) * scale).to(w.torch_dtype)

    q_b = randn_act(T, H, UK_K + PE)
    w_uk_t = randn_act(H, NOPE, UK_K, scale=UK_K ** -0.5)
    kv_c = randn_act(T, NOPE)
    k_pe = randn_act(T, PE)
    out = dict(q_b=q_b, q_nope=q_b[..., :UK_K], q_pe=q_b[..., UK_K:], w_uk_t=w_uk_t, kv_c=kv_c,
               k_pe=k_pe)
    out.update(_slots_positions_cache(w, g))
    return out


def _slots_positions_cache(w: Workload, g: torch.Generator) -> dict:
    """Slots, positions (in that order from g), the zero cache, the rope
    table and the scales of a workload."""
    T = w.tokens
    S = w.num_slots
    if w.slots == "randint":
        slots = torch.randint(0, S, (T,), generator=g, dtype=torch.int64)
    elif w.slots == "randperm":
        if T > S:
            raise ValueError("more tokens than distinct slots")
        slots = torch.randperm(S, generator=g, dtype=torch.int64)[:T].contiguous()
    else:
        raise ValueError(w.slots)
    if w.positions == "none":
        positions = None
    elif w.positions == "arange":
        positions = torch.arange(T, dtype=torch.int64)
    elif w.positions.startswith("uniform:"):
        hi = int(w.positions.split(":")[1])
        positions = torch.randint(0, hi, (T,), generator=g, dtype=torch.int64)
    else:
        raise ValueError(w.positions)
    kv_dtype = torch.float8_e4m3fn if w.kv_fp8 else w.torch_dtype
    cache = torch.zeros(w.num_blocks, w.block_size, ROW, dtype=kv_dtype)
    table = None
    if w.rope:
        table = shared_rope_table(w.max_position)
        if w.table_dtype == "bf16":
            table = table.to(torch.bfloat16)
    return dict(cache=cache, slot_mapping=slots, positions=positions, rope_cos_sin=table,
                q_scale=torch.tensor([w.q_scale], dtype=torch.float32) if w.q_fp8 else None,
                kv_scale=torch.tensor([w.kv_scale], dtype=torch.float32) if w.kv_fp8 else None)


def custom(tokens: int, heads: int, num_blocks: int | None = None, block_size: int = 64,
           rope: bool = False, q_fp8: bool = False, kv_fp8: bool = False,
           positions: str | None = None, slots: str = "randperm", q_scale: float = 0.05,
           kv_scale: float = 0.05, max_position: int = ROPE_MAX_POSITION,
           name: str = "custom", dtype: str = "bf16", rope_style: str = "neox",
           table_dtype: str = "f32") -> Workload:
    """A workload with the same recipe at another size (ragged tests)."""
    if num_blocks is None:
        num_blocks = max(1, math.ceil(tokens / block_size))
    if positions is None:
        positions = f"uniform:{max_position}" if rope else "none"
    return Workload(name, tokens, heads, num_blocks, block_size, rope, q_fp8, kv_fp8,
                    slots, positions, q_scale, kv_scale, max_position, dtype, rope_style,
                    table_dtype)


# ---- inputs of the downstream decode attention --------------------------------

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """One decode step of MLA attention over the paged latent cache: B
    sequences with one query token each, H heads, seq_lens cached tokens."""
    name: str
    batch: int
    heads: int
    seq_lens: tuple            # one length per sequence
    block_size: int = 64
    q_fp8: bool = False
    kv_fp8: bool = False
    q_scale: float = 0.05
    kv_scale: float = 0.05
    sm_scale: float = 192 ** -0.5   # 1/sqrt(128 + 64): the head dims before absorption
    spare_blocks: int = 3           # pages not used by any sequence

    @property
    def max_blocks(self) -> int:
        return max(1, max((L + self.block_size - 1) // self.block_size for L in self.seq_lens))

    @property
    def num_blocks(self) -> int:
        used = sum((L + self.block_size - 1) // self.block_size for L in self.seq_lens)
        return used + self.spare_blocks

    def describe(self) -> str:
        Ls = self.seq_lens
        lens = f"L={Ls[0]}" if len(set(Ls)) == 1 else f"L={min(Ls)}..{max(Ls)}"
        bits = ["q_e4m3" if self.q_fp8 else "q_bf16", "kv_e4m3" if self.kv_fp8 else "kv_bf16"]
        return f"B={self.batch} H={self.heads} {lens} bs={self.block_size} " + "+".join(bits)


ATTN_WORKLOADS = {
    "attn_b64_l4096_h16_kvfp8": AttnWorkload("attn_b64_l4096_h16_kvfp8", 64, 16, (4096,) * 64,
                                             q_fp8=False, kv_fp8=True),
    "attn_b64_l4096_h16_bf16": AttnWorkload("attn_b64_l4096_h16_bf16", 64, 16, (4096,) * 64),
    "attn_b1_l1024_h16_kvfp8": AttnWorkload("attn_b1_l1024_h16_kvfp8", 1, 16, (1024,),
                                            q_fp8=False, kv_fp8=True),
    # one (sequence, head tile) per CU: no key split, no merge pass
    "attn_b256_l4096_h16_kvfp8": AttnWorkload("attn_b256_l4096_h16_kvfp8", 256, 16, (4096,) * 256,
                                              q_fp8=False, kv_fp8=True),
}


def make_attn_inputs(w: AttnWorkload, seed: int = DEFAULT_SEED) -> dict:
    """q [B,H,576] and a paged cache [num_blocks, bs, 576] drawn N(0,1) (bf16,
    or E4M3 codes of x / scale), a block table that hands each sequence a
    random set of pages, and the sequence lengths."""
    g = torch.Generator().manual_seed(seed)
    B, H = w.batch, w.heads

    def draw(shape, fp8, scale):
        x = torch.randn(*shape, generator=g, dtype=torch.float32)
        if fp8:
            return torch.clamp(x / scale, -448, 448).to(torch.float8_e4m3fn)
        return x.to(torch.bfloat16)

    q = draw((B, H, ROW), w.q_fp8, w.q_scale)
    cache = draw((w.num_blocks, w.block_size, ROW), w.kv_fp8, w.kv_scale)
    perm = torch.randperm(w.num_blocks, generator=g, dtype=torch.int64)
    block_table = torch.zeros(B, w.max_blocks, dtype=torch.int32)
    k = 0
    for b, L in enumerate(w.seq_lens):
        n = (L + w.block_size - 1) // w.block_size
        block_table[b, :n] = perm[k:k + n].to(torch.int32)
        k += n
    return dict(q=q, cache=cache, block_table=block_table,
                seq_lens=torch.tensor(w.seq_lens, dtype=torch.int32),
                q_scale=torch.tensor([w.q_scale], dtype=torch.float32) if w.q_fp8 else None,
                kv_scale=torch.tensor([w.kv_scale], dtype=torch.float32) if w.kv_fp8 else None)


def attn_custom(batch: int, heads: int, seq_lens, block_size: int = 64, q_fp8: bool = False,
                kv_fp8: bool = False, name: str = "attn_custom", **kw) -> AttnWorkload:
    if isinstance(seq_lens, int):
        seq_lens = (seq_lens,) * batch
    return AttnWorkload(name, batch, heads, tuple(int(x) for x in seq_lens), block_size, q_fp8,
                        kv_fp8, **kw)


def make_inputs_on_device(w: Workload, device: str, seed: int = DEFAULT_SEED,
                          chunk: int = 1 << 27, uk: bool = False) -> dict:
    """The same recipe as make_inputs, drawn on the device by torch's device
    generator (for sizes whose host copy would be impractical; the values
    differ from make_inputs' for the same seed).  Activations are N(0,1)
    fp32 rounded to the activation type, drawn ``chunk`` elements at a time;
    slots are a prefix of a random permutation of all cache slots; positions
    follow the workload's recipe.  The cache starts as zeros.  With ``uk``
    the recipe is make_uk_inputs' instead: q_b [T, H, 192] (q_nope and q_pe
    its views) and w_uk_t [H, 512, 128] with N(0, 1/128) entries in place of
    ql_nope and q_pe."""
    g = torch.Generator(device=device).manual_seed(seed)
    T, H = w.tokens, w.heads

    def randn_act(*shape, scale=1.0):
        out = torch.empty(*shape, dtype=w.torch_dtype, device=device)
        for part in out.view(-1).split(chunk):
            part.copy_(torch.randn(part.numel(), generator=g, dtype=torch.float32, device=device) * scale)
        return out

    extra = {}
    if uk:
        q_b = randn_act(T, H, UK_K + PE)
        w_uk_t = randn_act(H, NOPE, UK_K, scale=UK_K ** -0.5)
        extra = dict(q_b=q_b, q_nope=q_b[..., :UK_K], w_uk_t=w_uk_t)
        ql_nope, q_pe = None, q_b[..., UK_K:]
    else:
        ql_nope = randn_act(T, H, NOPE)
        q_pe = randn_act(T, H, PE)
    kv_c = randn_act(T, NOPE)
    k_pe = randn_act(T, PE)
    S = w.num_slots
    if w.slots != "randperm" or T > S:
        raise ValueError("device inputs take a prefix of a slot permutation")
    slots = torch.randperm(S, generator=g, dtype=torch.int64, device=device)[:T].contiguous()
    if w.positions == "none":
        positions = None
    elif w.positions == "arange":
        positions = torch.arange(T, dtype=torch.int64, device=device)
    elif w.positions.startswith("uniform:"):
        hi = int(w.positions.split(":")[1])
        positions = torch.randint(0, hi, (T,), generator=g, dtype=torch.int64, device=device)
    else:
        raise ValueError(w.positions)
    kv_dtype = torch.float8_e4m3fn if w.kv_fp8 else w.torch_dtype
    cache = torch.zeros(w.num_blocks, w.block_size, ROW, dtype=kv_dtype, device=device)
    table = None
    if w.rope:
        table = shared_rope_table(w.max_position)
        if w.table_dtype == "bf16":
            table = table.to(torch.bfloat16)
        table = table.to(device)
    out = dict(ql_nope=ql_nope, q_pe=q_pe, kv_c=kv_c, k_pe=k_pe, cache=cache,
               slot_mapping=slots, positions=positions, rope_cos_sin=table,
               q_scale=torch.tensor([w.q_scale], dtype=torch.float32, device=device) if w.q_fp8 else None,
               kv_scale=torch.tensor([w.kv_scale], dtype=torch.float32, device=device) if w.kv_fp8 else None)
    if uk:
        del out["ql_nope"]
        out.update(extra)
    return out
