"""Seeded synthetic inputs for the row-statistics sampler and top-K logprobs.

Shared by the tests, the smoke check and the benchmark. This module holds no
part of the method's arithmetic: it only draws logits, temperatures and keep
masks with torch generators, on CPU or on the GPU, from fixed seeds.

Workloads (rows x vocab, distribution, temperatures):

  C1  64 x 32768 (2 slots x canvas 32), N(0, 1), temps [1.0, 0.0], bf16 probs,
      data seed 1, noise seed 1234.
  C2  4096 x 262144 (16 x 256), N(0, 2.5^2), 512 rows get +15 on one token,
      slot temps a seeded shuffle of six 0.0, five 0.7, five 1.0, bf16 probs,
      data seed 2.
  C3  4096 x 262144, canvas 1 (one temperature per row), N(0, 2.5^2), temps
      U[0.1, 1.5], 205 adversarial rows (41 of each of five kinds), no probs,
      data seed 3.
  C4  4096 x 262144 (16 x 256), N(0, 3^2), K=20, 8 of 16 slots kept, slot
      temps eight 0.0 and eight 1.0 with both among kept slots, about ten of
      each row's top-40 values copied to random columns, and in half of the
      kept rows the K-th and (K+1)-th values made equal, data seed 4.
  C5  16384 x 262144 (32 x 512), row stride 262144 + 128, half N(0, 2^2)
      rows and half Zipf rows (logit of rank k is -1.1 ln k + N(0, 0.1^2)
      over a random permutation), 8 slots at T = 0 and 24 at U(0, 1.5],
      bf16 probs, data seed 5.

  S4  the stash over C4's logits: 16 requests (one per canvas of 256) with a
      permuted src, slots spread over a stash of 24, C4's kept half, valid
      200, 17 and 1 on three kept requests, two kept requests listing 5 and
      20 token ids, K = 20, width 24.

Every generator takes ``rows`` / ``vocab`` overrides so that the same recipe
runs at sizes a CPU oracle finishes in seconds.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

FLT_MAX = 3.4028234663852886e38
NOISE_SEED = 1234


@dataclass
class Workload:
    name: str
    logits: torch.Tensor          # [rows, vocab] fp32 view (row stride may exceed vocab)
    temps: torch.Tensor           # fp32 [slots]
    canvas_len: int
    seed: int = NOISE_SEED        # noise seed
    probs_dtype: torch.dtype | None = None
    keep_mask: torch.Tensor | None = None   # uint8 [slots], top-K workloads only
    K: int = 0
    special_rows: dict = field(default_factory=dict)  # kind -> LongTensor of rows

    @property
    def rows(self) -> int:
        return self.logits.shape[0]

    @property
    def vocab(self) -> int:
        return self.logits.shape[1]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, g, device, out=None):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _alloc(rows, vocab, ld, device):
    """A [rows, vocab] fp32 view with row stride ld (padding left at zero)."""
    if ld == vocab:
        return torch.empty(rows, vocab, dtype=torch.float32, device=device)
    base = torch.zeros(rows, ld, dtype=torch.float32, device=device)
    return base[:, :vocab]


def _fill_normal(x: torch.Tensor, std: float, g, chunk_rows=1024):
    rows = x.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x[r0:r1] = _randn((r1 - r0, x.shape[1]), std, g, x.device)


def _choice(n, k, g, device):
    """k distinct integers from [0, n), in increasing order."""
    perm = torch.randperm(n, generator=g, device=device)[:k]
    return torch.sort(perm).values


def c1(device="cpu", rows=64, vocab=32768, canvas_len=32) -> Workload:
    g = _gen(1, device)
    x = _alloc(rows, vocab, vocab, device)
    _fill_normal(x, 1.0, g)
    slots = (rows + canvas_len - 1) // canvas_len
    temps = torch.tensor(([1.0, 0.0] * slots)[:slots], dtype=torch.float32, device=device)
    return Workload("C1", x, temps, canvas_len, NOISE_SEED, torch.bfloat16)


def c2(device="cpu", rows=4096, vocab=262144, canvas_len=256) -> Workload:
    g = _gen(2, device)
    x = _alloc(rows, vocab, vocab, device)
    _fill_normal(x, 2.5, g)
    n_peak = rows // 8
    peak_rows = _choice(rows, n_peak, g, device)
    peak_cols = torch.randint(0, vocab, (n_peak,), generator=g, device=device)
    x[peak_rows, peak_cols] += 15.0
    slots = (rows + canvas_len - 1) // canvas_len
    # a 6/5/5 split of {0, 0.7, 1.0} over 16 slots, scaled to the slot count
    n0 = max(1, round(slots * 6 / 16)) if slots > 2 else 1
    n1 = max(1, (slots - n0) // 2) if slots > 1 else 0
    n2 = slots - n0 - n1
    base = torch.tensor([0.0] * n0 + [0.7] * n1 + [1.0] * n2, dtype=torch.float32)
    perm = torch.randperm(slots, generator=_gen(20, "cpu"))
    temps = base[perm].to(device)
    return Workload("C2", x, temps, canvas_len, NOISE_SEED, torch.bfloat16,
                    special_rows={"peaked": peak_rows})


ADVERSARIAL_KINDS = ("all_equal", "dup_max", "neg_inf_span", "huge", "subnormal")


def c3(device="cpu", rows=4096, vocab=262144, n_adv_per_kind=41,
       boundary=16384) -> Workload:
    """Stats-only read-bound workload with adversarial rows.

    ``boundary`` is a column period at which duplicated maxima and -inf spans
    are placed (slice edges of a split row); any value is a valid input.
    """
    g = _gen(3, device)
    x = _alloc(rows, vocab, vocab, device)
    _fill_normal(x, 2.5, g)
    temps = (0.1 + 1.4 * torch.rand(rows, generator=g, device=device)).to(torch.float32)
    n_adv = min(rows, n_adv_per_kind * len(ADVERSARIAL_KINDS))
    adv = _choice(rows, n_adv, g, device).cpu()
    per = max(1, n_adv // len(ADVERSARIAL_KINDS))
    special = {}
    gc = _gen(30, "cpu")  # structure decisions are drawn on the CPU
    for k, kind in enumerate(ADVERSARIAL_KINDS):
        rows_k = adv[k * per:(k + 1) * per]
        special[kind] = rows_k.to(device)
        for j, r in enumerate(rows_k.tolist()):
            t = float(temps[r])
            if kind == "all_equal":
                if j == 0:
                    # all +-0.0, signs mixed
                    signs = torch.randint(0, 2, (vocab,), generator=gc).bool()
                    row = torch.zeros(vocab, dtype=torch.float32)
                    row[signs] = -0.0
                    x[r] = row.to(device)
                else:
                    v = float(torch.randn(1, generator=gc)) * 3.0
                    x[r] = torch.full((vocab,), v, dtype=torch.float32, device=device)
            elif kind == "dup_max":
                ndup = int(torch.randint(2, 9, (1,), generator=gc))
                cand = []
                for b in range(boundary, vocab, boundary):
                    cand += [b - 1, b]
                cand = [c for c in cand if 0 <= c < vocab]
                pos = set()
                while len(pos) < min(ndup, vocab):
                    if cand and int(torch.randint(0, 2, (1,), generator=gc)) == 0:
                        pos.add(cand[int(torch.randint(0, len(cand), (1,), generator=gc))])
                    else:
                        pos.add(int(torch.randint(0, vocab, (1,), generator=gc)))
                v = float(x[r].max()) + 1.0 + float(torch.rand(1, generator=gc))
                idx = torch.tensor(sorted(pos), device=device)
                x[r, idx] = v
            elif kind == "neg_inf_span":
                frac = 0.10 + 0.89 * float(torch.rand(1, generator=gc))
                length = max(1, min(vocab - 1, int(frac * vocab)))
                if j % 3 == 0 and vocab > boundary:
                    start = boundary * int(torch.randint(0, max(1, (vocab - length) // boundary + 1), (1,), generator=gc))
                    start = min(start, vocab - length)
                else:
                    start = int(torch.randint(0, vocab - length + 1, (1,), generator=gc))
                x[r, start:start + length] = float("-inf")
            elif kind == "huge":
                # |x| in [0.5, 0.9] * FLT_MAX * min(T, 1): x / T stays finite
                mag = (0.5 + 0.4 * torch.rand(vocab, generator=gc, dtype=torch.float64))
                sign = torch.where(torch.rand(vocab, generator=gc) < 0.5, -1.0, 1.0).to(torch.float64)
                vals = (sign * mag * FLT_MAX * min(t, 1.0)).to(torch.float32)
                x[r] = vals.to(device)
            elif kind == "subnormal":
                # subnormal magnitudes 2^-149 .. 2^-127
                k_int = torch.randint(1, 1 << 22, (vocab,), generator=gc, dtype=torch.int64)
                sign = torch.where(torch.rand(vocab, generator=gc) < 0.5, -1, 1)
                sub = (sign * k_int).to(torch.float64) * 2.0 ** -149
                sub = sub.to(torch.float32)
                if j % 2 == 0:
                    x[r] = sub.to(device)
                else:
                    # sprinkle: 5% of a normal row replaced by subnormals
                    m = torch.rand(vocab, generator=gc) < 0.05
                    row = x[r].cpu()
                    row[m] = sub[m]
                    x[r] = row.to(device)
    return Workload("C3", x, temps, 1, NOISE_SEED, None, special_rows=special)


def c4(device="cpu", rows=4096, vocab=262144, canvas_len=256, K=20) -> Workload:
    g = _gen(4, device)
    x = _alloc(rows, vocab, vocab, device)
    _fill_normal(x, 3.0, g)
    slots = (rows + canvas_len - 1) // canvas_len
    gc = _gen(40, "cpu")
    # keep half of the slots; temps half 0.0 / half 1.0 with both among kept
    keep_idx = torch.randperm(slots, generator=gc)[: max(1, slots // 2)]
    keep = torch.zeros(slots, dtype=torch.uint8)
    keep[keep_idx] = 1
    temps = torch.ones(slots, dtype=torch.float32)
    kept = keep_idx.tolist()
    dropped = [s for s in range(slots) if s not in set(kept)]
    zero_slots = kept[: (len(kept) + 1) // 2] + dropped[: len(dropped) // 2]
    temps[zero_slots] = 0.0
    # copies of top values to random columns: forces index tie-breaks
    ntop = min(40, vocab)
    ncopy = min(10, ntop)
    chunk = 256
    tie_rows = []
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        top = torch.topk(x[r0:r1], ntop, dim=1)
        pick = torch.randint(0, ntop, (r1 - r0, ncopy), generator=g, device=device)
        vals = torch.gather(top.values, 1, pick)
        cols = torch.randint(0, vocab, (r1 - r0, ncopy), generator=g, device=device)
        x[r0:r1].scatter_(1, cols, vals)
    # in half of the kept rows, make the K-th and (K+1)-th largest values equal
    kept_rows = torch.cat([torch.arange(s * canvas_len, min(rows, (s + 1) * canvas_len))
                           for s in kept]) if kept else torch.zeros(0, dtype=torch.int64)
    if K + 1 <= vocab and len(kept_rows):
        sel = kept_rows[torch.randperm(len(kept_rows), generator=gc)[: len(kept_rows) // 2]]
        sel = torch.sort(sel).values.to(device)
        for r0 in range(0, len(sel), chunk):
            rr = sel[r0:r0 + chunk]
            top = torch.topk(x[rr], K + 1, dim=1)
            vk = top.values[:, K - 1]
            ck1 = top.indices[:, K]
            x[rr, ck1] = vk
        tie_rows = sel
    return Workload("C4", x, temps.to(device), canvas_len, NOISE_SEED, None,
                    keep_mask=keep.to(device), K=K,
                    special_rows={"kth_tie": torch.as_tensor(tie_rows, device=device)})


def c5(device="cpu", rows=16384, vocab=262144, canvas_len=512, pad=128) -> Workload:
    g = _gen(5, device)
    x = _alloc(rows, vocab, vocab + pad, device)
    gc = _gen(50, "cpu")
    zipf_mask = torch.zeros(rows, dtype=torch.bool)
    zipf_mask[torch.randperm(rows, generator=gc)[: rows // 2]] = True
    zipf_rows = torch.nonzero(zipf_mask).flatten()
    norm_rows = torch.nonzero(~zipf_mask).flatten()
    chunk = 256
    k = torch.arange(1, vocab + 1, dtype=torch.float32, device=device)
    base = -1.1 * torch.log(k)
    for r0 in range(0, len(norm_rows), chunk):
        rr = norm_rows[r0:r0 + chunk].to(device)
        x[rr] = _randn((len(rr), vocab), 2.0, g, device)
    for r0 in range(0, len(zipf_rows), chunk):
        rr = zipf_rows[r0:r0 + chunk].to(device)
        perm = torch.argsort(torch.rand(len(rr), vocab, generator=g, device=device), dim=1)
        vals = base.unsqueeze(0) + _randn((len(rr), vocab), 0.1, g, device)
        row_block = torch.empty(len(rr), vocab, dtype=torch.float32, device=device)
        row_block.scatter_(1, perm, vals)
        x[rr] = row_block
    slots = (rows + canvas_len - 1) // canvas_len
    n_zero = max(1, slots // 4)
    temps = 1.5 * (1.0 - torch.rand(slots, generator=gc, dtype=torch.float32))  # (0, 1.5]
    temps[torch.randperm(slots, generator=gc)[:n_zero]] = 0.0
    return Workload("C5", x, temps.to(device), canvas_len, NOISE_SEED, torch.bfloat16,
                    special_rows={"zipf": zipf_rows.to(device)})


def random_case(device="cpu", rows=8, vocab=100, canvas_len=3, seed=0, std=2.0,
                ld=None, t_choices=(0.0, 0.5, 1.0, 1.3), probs_dtype=torch.bfloat16,
                ties=False) -> Workload:
    """Small mixed case for edge sweeps: ragged shapes, padding, greedy slots."""
    g = _gen(1000 + seed, device)
    ld = vocab if ld is None else ld
    x = _alloc(rows, vocab, ld, device)
    _fill_normal(x, std, g)
    if ties:
        # quantise so exact duplicates (including of the maximum) are common
        x.copy_(torch.round(x * 2.0) / 2.0)
    slots = (rows + canvas_len - 1) // canvas_len
    gc = _gen(2000 + seed, "cpu")
    tc = torch.tensor(t_choices, dtype=torch.float32)
    temps = tc[torch.randint(0, len(tc), (slots,), generator=gc)]
    return Workload(f"random{seed}", x, temps.to(device), canvas_len, 777 + seed, probs_dtype)


@dataclass
class StashWorkload:
    """Arguments of one converged-logprob stash call (outputs excluded)."""
    name: str
    logits: torch.Tensor      # [canvases * canvas_len, vocab] fp32
    canvas_len: int
    src: torch.Tensor         # int32 [m]
    slots: torch.Tensor       # int32 [m], distinct
    keep: torch.Tensor        # uint8 [m]
    valid: torch.Tensor       # int32 [m]
    temps: torch.Tensor       # fp32 [m]
    K: int
    num_ids: torch.Tensor     # int32 [m]
    ids: torch.Tensor | None  # int32 [m, ids_stride]
    n_slots: int
    positions: int
    width: int
    logits_mode: bool = False

    @property
    def m(self) -> int:
        return self.slots.numel()

    @property
    def vocab(self) -> int:
        return self.logits.shape[1]


def stash_case(device="cpu", m=6, canvas_len=4, vocab=1000, K=5, seed=0, std=2.0, ld=None,
               with_ids=True, ties=False, width_pad=3, logits_mode=False,
               t_choices=(0.0, 0.5, 1.0, 1.3)) -> StashWorkload:
    """Small stash call: more canvases than requests, a permuted src, slots
    spread over a larger stash, valid counts from -1 to past the canvas,
    about two thirds of the requests kept, and (with_ids) some requests
    listing token ids, one of them out of order and repeated."""
    g = _gen(3000 + seed, device)
    gc = _gen(4000 + seed, "cpu")
    canvases = m + 2
    ld = vocab if ld is None else ld
    x = _alloc(canvases * canvas_len, vocab, ld, device)
    _fill_normal(x, std, g)
    if ties:
        x.copy_(torch.round(x * 2.0) / 2.0)
    src = torch.randperm(canvases, generator=gc)[:m].to(torch.int32)
    n_slots = m + 3
    slots = torch.randperm(n_slots, generator=gc)[:m].to(torch.int32)
    keep = (torch.rand(m, generator=gc) < 0.67).to(torch.uint8)
    keep[0] = 1
    valid = torch.randint(-1, canvas_len + 2, (m,), generator=gc, dtype=torch.int32)
    valid[0] = canvas_len
    tc = torch.tensor(t_choices, dtype=torch.float32)
    temps = tc[torch.randint(0, len(tc), (m,), generator=gc)]
    width = K + 1 + width_pad
    ids_stride = width + 2
    num_ids = torch.zeros(m, dtype=torch.int32)
    ids = None
    if with_ids:
        ids = torch.randint(0, vocab, (m, ids_stride), generator=gc, dtype=torch.int32)
        ids[:, 1] = ids[:, 0]  # a repeated id
        num_ids = torch.randint(0, ids_stride + 2, (m,), generator=gc, dtype=torch.int32)
        num_ids[torch.arange(m) % 2 == 0] = 0  # half the requests take the top-K
        ids = ids.to(device)
    return StashWorkload(f"stash{seed}", x, canvas_len, src.to(device), slots.to(device),
                         keep.to(device), valid.to(device), temps.to(device), K,
                         num_ids.to(device), ids, n_slots, canvas_len, width, logits_mode)


def stash_c4(device="cpu", K=20) -> StashWorkload:
    """The stash over the C4 logits (4096 x 262144 as 16 canvases of 256):
    16 requests with a permuted src, slots spread over a stash of 24, the
    kept half (C4's kept slots), three kept requests with valid below 256,
    and two kept requests listing 5 and 20 token ids; width K + 4."""
    w = c4(device, K=K)
    canvas_len = w.canvas_len
    m = w.rows // canvas_len
    gc = _gen(41, "cpu")
    src = torch.randperm(m, generator=gc).to(torch.int32)
    slots = torch.randperm(24, generator=gc)[:m].to(torch.int32)
    keep = w.keep_mask.cpu()[src.long()]
    temps = w.temps.cpu()[src.long()]
    valid = torch.full((m,), canvas_len, dtype=torch.int32)
    kept = torch.nonzero(keep).flatten().tolist()
    for j, v in zip(kept[:3], (200, 17, 1)):
        valid[j] = v
    width = K + 4
    ids_stride = 24
    ids = torch.randint(0, w.vocab, (m, ids_stride), generator=gc, dtype=torch.int32)
    num_ids = torch.zeros(m, dtype=torch.int32)
    for j, n in zip(kept[-2:], (5, 20)):
        num_ids[j] = n
    return StashWorkload("S4", w.logits, canvas_len, src.to(device), slots.to(device),
                         keep.to(device), valid.to(device), temps.to(device), K,
                         num_ids.to(device), ids.to(device), 24, canvas_len, width)


WORKLOADS = {"C1": c1, "C2": c2, "C3": c3, "C4": c4, "C5": c5}


def embedding(vocab: int, d: int, seed: int, device="cpu", ints: bool = False,
              dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """A seeded token-embedding table [vocab, d] for the self-conditioning
    product, in the model dtype (bfloat16 or float16): N(0, 1) values
    rounded to it, or (ints) integers in [-4, 4], which both hold exactly."""
    g = _gen(seed, device)
    if ints:
        e = torch.randint(-4, 5, (vocab, d), generator=g, device=device).to(torch.float32)
    else:
        e = torch.randn(vocab, d, generator=g, device=device, dtype=torch.float32)
    return e.to(dtype)


def probabilities(rows: int, vocab: int, seed: int, device="cpu",
                  dtype: torch.dtype = torch.bfloat16, ld: int | None = None) -> torch.Tensor:
    """Seeded probability-like rows [rows, vocab] in the model dtype, as input
    of the self-conditioning product of given probabilities: log-normal
    values exp(2.5 z), z ~ N(0, 1) (the spread of the C2 logits), divided by
    their expected row sum vocab * e^3.125, so rows sum to about 1 with a few
    large and many tiny entries (in fp16 most of a long row lies below the
    normal range); one column in 16 is exactly 0. With ld > vocab the rows are views into a
    wider [rows, ld] buffer (the padding holds NaN, which must never be read)."""
    g = _gen(seed, device)
    z = torch.randn(rows, vocab, generator=g, device=device, dtype=torch.float32)
    p = torch.exp(2.5 * z) / (vocab * 22.7599)
    zero = torch.randint(0, 16, (rows, vocab), generator=g, device=device) == 0
    p = torch.where(zero, torch.zeros_like(p), p).to(dtype)
    if ld is None or ld == vocab:
        return p
    buf = torch.full((rows, ld), float("nan"), dtype=dtype, device=device)
    buf[:, :vocab] = p
    return buf[:, :vocab]
