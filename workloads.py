"""Seeded synthetic inputs for the five workloads of the hot path.

This module holds input construction only -- random draws, bf16 rounding of
the draws, label/mask/index layouts -- and none of the log-softmax arithmetic.
It is the one module that both the HIP-path tests and the oracle tests take
their inputs from.

Recipes (numpy PCG64; fp32 draws, rounded to bf16 by round-to-nearest-even
where the workload is bf16).  Per-row parameters come from
``default_rng(seed)``; the logit matrix is drawn in blocks of BLOCK_ROWS rows,
block b from ``default_rng([seed, 1, b])``, so any block can be regenerated on
its own and blocks can be drawn in parallel.

  tiny   seed 0  64 x 4096 fp32, z = 2 N(0,1); labels uniform; 8 rows chosen by
                 permutation get -100; T = 1; g = 1.
                 (ms-swift PR #10337, the selective log-softmax semantics)
  chunk  seed 1  4096 x 32768 bf16, z = bf16(3 N(0,1)); labels uniform; T = 0.7;
                 top-K: 8 distinct uniform indices per row.
                 (ms-swift PR #10337, Experiment results table: 4096 x 32768)
  grpo   seed 2  8192 x 152064 bf16, z = bf16(3 N(0,1) + shift_r),
                 shift_r ~ U(-5, 5); labels uniform; exactly rows // 10 rows
                 masked out; g ~ N(0,1) fp32; T = 1.
                 (ms-swift PR #10337, Experiment results table: 8192 x 152064)
  sparse seed 3  2 sequences x 1024 tokens, suffix-cropped to 961 rows each
                 (1922 rows), V = 4096 fp32, z = 2 N(0,1); per sequence 4 spans
                 of 32 supervised rows at local rows 104, 344, 584, 824, labels
                 uniform there and -100 elsewhere; g = 1; T = 1.
                 (ms-swift PR #10353, Experiment results: 1922 kept rows,
                 256 supervised, vocabulary 4096)
  peaked seed 4  2048 x 151936; others N(0,1) (fp32, or their bf16 rounding);
                 labels uniform; margin per row uniform over
                 {5, 17, 20, 30, 50, 80}; z_t = dtype(max of the stored
                 others + margin); T in {1.0, 0.9}; g = 1.
                 (Liger PR #1555 page, unsloth-zoo #2080 Accuracy table:
                 margins 17/20/30/50 at V = 151936; Details: targets 5 to 40
                 above the rest)
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

IGNORE_INDEX = -100
BLOCK_ROWS = 256
PEAK_MARGINS = (5.0, 17.0, 20.0, 30.0, 50.0, 80.0)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return
    the 16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_values(logits: np.ndarray) -> np.ndarray:
    """The stored logits as float32 (exact for both fp32 and bf16 storage)."""
    return bf16_to_f32(logits) if logits.dtype == np.uint16 else logits


def _draw_matrix(seed, rows, vocab, fill, threads=8):
    """Draw [rows, vocab] block by block; fill(block_index, rng, r0, r1) returns
    the block's stored values."""
    nb = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    blocks = [None] * nb

    def one(b):
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        rng = np.random.default_rng([seed, 1, b])
        blocks[b] = fill(b, rng, r0, r1)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(nb)))
    return blocks


def _assemble(blocks, rows, vocab, dtype):
    out = np.empty((rows, vocab), dtype=dtype)
    r = 0
    for blk in blocks:
        out[r:r + blk.shape[0]] = blk
        r += blk.shape[0]
    return out


def tiny(rows=64, vocab=4096, n_ignored=8, seed=0):
    rng = np.random.default_rng(seed)
    labels = rng.integers(0, vocab, rows).astype(np.int64)
    labels[rng.permutation(rows)[:n_ignored]] = IGNORE_INDEX
    blocks = _draw_matrix(seed, rows, vocab,
                          lambda b, g, r0, r1: (2.0 * g.standard_normal((r1 - r0, vocab),
                                                                        dtype=np.float32)))
    logits = _assemble(blocks, rows, vocab, np.float32)
    return dict(name="tiny", logits=logits, labels=labels, row_mask=None, temperature=1.0,
                g=np.ones(rows, dtype=np.float32))


def chunk(rows=4096, vocab=32768, K=8, seed=1):
    rng = np.random.default_rng(seed)
    labels = rng.integers(0, vocab, rows).astype(np.int64)
    indices = np.stack([rng.choice(vocab, K, replace=False) for _ in range(rows)]).astype(np.int64)
    blocks = _draw_matrix(seed, rows, vocab,
                          lambda b, g, r0, r1: bf16_bits(3.0 * g.standard_normal(
                              (r1 - r0, vocab), dtype=np.float32)))
    logits = _assemble(blocks, rows, vocab, np.uint16)
    return dict(name="chunk", logits=logits, labels=labels, row_mask=None, temperature=0.7,
                indices=indices, g=np.ones(rows, dtype=np.float32))


def grpo_rows(rows=8192, vocab=152064, seed=2):
    """The per-row draws of grpo() (shift, labels, row mask, g) without the
    logit matrix."""
    rng = np.random.default_rng(seed)
    shift = rng.uniform(-5.0, 5.0, rows).astype(np.float32)
    labels = rng.integers(0, vocab, rows).astype(np.int64)
    row_mask = np.ones(rows, dtype=np.uint8)
    row_mask[rng.permutation(rows)[:rows // 10]] = 0
    g = rng.standard_normal(rows, dtype=np.float32)
    return shift, labels, row_mask, g


def grpo(rows=8192, vocab=152064, seed=2, temperature=1.0):
    shift, labels, row_mask, g = grpo_rows(rows, vocab, seed)

    def fill(b, gen, r0, r1):
        z = 3.0 * gen.standard_normal((r1 - r0, vocab), dtype=np.float32)
        z += shift[r0:r1, None]
        return bf16_bits(z)

    logits = _assemble(_draw_matrix(seed, rows, vocab, fill), rows, vocab, np.uint16)
    return dict(name="grpo", logits=logits, labels=labels, row_mask=row_mask,
                temperature=temperature, g=g)


def sparse(n_seq=2, seq_len=1024, kept=961, vocab=4096, span_starts=(104, 344, 584, 824),
           span_len=32, seed=3):
    rng = np.random.default_rng(seed)
    rows = n_seq * kept
    labels = np.full(rows, IGNORE_INDEX, dtype=np.int64)
    for s in range(n_seq):
        for a in span_starts:
            r0 = s * kept + a
            labels[r0:r0 + span_len] = rng.integers(0, vocab, span_len)
    blocks = _draw_matrix(seed, rows, vocab,
                          lambda b, g, r0, r1: (2.0 * g.standard_normal((r1 - r0, vocab),
                                                                        dtype=np.float32)))
    logits = _assemble(blocks, rows, vocab, np.float32)
    return dict(name="sparse", logits=logits, labels=labels, row_mask=None, temperature=1.0,
                g=np.ones(rows, dtype=np.float32), seq_shape=(n_seq, kept), seq_len=seq_len)


def peaked(dtype="f32", temperature=1.0, rows=2048, vocab=151936, seed=4):
    rng = np.random.default_rng(seed)
    labels = rng.integers(0, vocab, rows).astype(np.int64)
    margins = np.asarray(PEAK_MARGINS, dtype=np.float32)[rng.integers(0, len(PEAK_MARGINS), rows)]

    def fill(b, gen, r0, r1):
        z = gen.standard_normal((r1 - r0, vocab), dtype=np.float32)
        if dtype == "bf16":
            z = bf16_to_f32(bf16_bits(z))
        for i, r in enumerate(range(r0, r1)):
            t = labels[r]
            z[i, t] = -np.inf
            peak = np.float32(z[i].max() + margins[r])
            z[i, t] = peak
        return bf16_bits(z) if dtype == "bf16" else z

    store = np.uint16 if dtype == "bf16" else np.float32
    logits = _assemble(_draw_matrix(seed, rows, vocab, fill), rows, vocab, store)
    return dict(name=f"peaked_{dtype}_T{temperature:g}", logits=logits, labels=labels,
                row_mask=None, temperature=float(temperature), margins=margins,
                g=np.ones(rows, dtype=np.float32))


BUILDERS = dict(tiny=tiny, chunk=chunk, grpo=grpo, sparse=sparse, peaked=peaked)


LINEAR_MARGINS = (17.0, 20.0, 30.0, 50.0)


def linear(rows=8192, hidden=2560, vocab=151936, seed=5, peaked_frac=0.0, temperature=1.0):
    """Hidden states and a frozen head for the fused linear CE (unsloth-zoo
    #2080 Speed: 2560 x 151936 frozen head, 8192 and 2048 rows; Accuracy:
    margins 17 / 20 / 30 / 50).  bf16 bits.

    head W [vocab, hidden] ~ N(0, 1/hidden) so each row of W has norm ~1;
    hidden h [rows, hidden] ~ 3 N(0, 1), so a logit h . w_j is ~ N(0, 9);
    labels uniform; exactly rows // 10 rows masked; g ~ N(0, 1).  A fraction
    peaked_frac of the rows (chosen by permutation) is replaced by
    h = beta w_t + 0.05 N(0, 1) with beta = margin / |w_t|^2, so the target
    logit leads the others by about the margin (the oracle reads the exact
    logits of the stored values)."""
    rng = np.random.default_rng(seed)
    labels = rng.integers(0, vocab, rows).astype(np.int64)
    row_mask = np.ones(rows, dtype=np.uint8)
    row_mask[rng.permutation(rows)[:rows // 10]] = 0
    g = rng.standard_normal(rows, dtype=np.float32)
    n_peak = int(round(peaked_frac * rows))
    peak_rows = np.sort(rng.permutation(rows)[:n_peak])
    margins = np.asarray(LINEAR_MARGINS, np.float32)[rng.integers(0, len(LINEAR_MARGINS), n_peak)]
    scale = np.float32(1.0 / np.sqrt(hidden))
    w = _assemble(_draw_matrix(seed, vocab, hidden,
                               lambda b, gen, r0, r1: bf16_bits(
                                   scale * gen.standard_normal((r1 - r0, hidden),
                                                               dtype=np.float32))),
                  vocab, hidden, np.uint16)
    h = _assemble(_draw_matrix(seed + 1000, rows, hidden,
                               lambda b, gen, r0, r1: bf16_bits(
                                   3.0 * gen.standard_normal((r1 - r0, hidden),
                                                             dtype=np.float32))),
                  rows, hidden, np.uint16)
    prng = np.random.default_rng([seed, 2])
    for i, r in enumerate(peak_rows):
        wt = bf16_to_f32(w[labels[r]])
        beta = np.float32(margins[i] / float(np.dot(wt.astype(np.float64), wt)))
        h[r] = bf16_bits(beta * wt + np.float32(0.05) * prng.standard_normal(hidden,
                                                                              dtype=np.float32))
    return dict(name="linear", hidden=h, weight=w, labels=labels, row_mask=row_mask,
                temperature=temperature, g=g, peak_rows=peak_rows)


DISTILL_MARGINS = (20.0, 40.0, 60.0, 80.0)


def distill(rows=2048, vocab=151936, seed=6, dtype="bf16", temperature=1.0, peaked_frac=0.0):
    """Student and teacher logit rows for the generalized JSD (unsloth-zoo
    #2079 Numbers: 2048 rows, V = 151936, bf16; the peaked rows lead by 20 to
    80, the range its Summary names).

    student z_s = 3 N(0, 1) + shift_r with shift_r ~ U(-5, 5); teacher
    z_t = z_s + N(0, 1) (a teacher close to, but not equal to, the student);
    labels uniform with rows // 10 of them the ignore index (the label mask);
    rows // 20 rows masked by row_mask; g ~ U(0.5, 1.5).  A fraction
    peaked_frac of the rows is made peaked: the student's column a leads its
    other values by a margin from DISTILL_MARGINS, and the teacher leads by
    another margin either at the same column (even-numbered peaked rows) or
    at another one (odd-numbered), so both agreeing and disagreeing confident
    rows occur.  fp32 or bf16 (stored bit patterns)."""
    rng = np.random.default_rng(seed)
    shift = rng.uniform(-5.0, 5.0, rows).astype(np.float32)
    labels = rng.integers(0, vocab, rows).astype(np.int64)
    labels[rng.permutation(rows)[:rows // 10]] = IGNORE_INDEX
    row_mask = np.ones(rows, dtype=np.uint8)
    row_mask[rng.permutation(rows)[:rows // 20]] = 0
    g = rng.uniform(0.5, 1.5, rows).astype(np.float32)
    n_peak = int(round(peaked_frac * rows))
    peak_rows = np.sort(rng.permutation(rows)[:n_peak])
    ms = np.asarray(DISTILL_MARGINS, np.float32)[rng.integers(0, len(DISTILL_MARGINS), n_peak)]
    mt = np.asarray(DISTILL_MARGINS, np.float32)[rng.integers(0, len(DISTILL_MARGINS), n_peak)]
    cs = rng.integers(0, vocab, n_peak)
    ct = np.where(np.arange(n_peak) % 2 == 0, cs, (cs + 1 + rng.integers(0, vocab - 1, n_peak)) % vocab)
    peak_of = {int(r): i for i, r in enumerate(peak_rows)}

    def rnd(z):
        return bf16_to_f32(bf16_bits(z)) if dtype == "bf16" else z

    def fill(which):
        def f(b, gen, r0, r1):
            zs = rnd(3.0 * gen.standard_normal((r1 - r0, vocab), dtype=np.float32)
                     + shift[r0:r1, None])
            if which == "student":
                z = zs
            else:
                noise = np.random.default_rng([seed, 7, b]).standard_normal((r1 - r0, vocab),
                                                                             dtype=np.float32)
                z = rnd(zs + noise)
            for i, r in enumerate(range(r0, r1)):
                k = peak_of.get(r)
                if k is None:
                    continue
                col = cs[k] if which == "student" else ct[k]
                lead = ms[k] if which == "student" else mt[k]
                z[i, col] = -np.inf
                z[i, col] = np.asarray(rnd(np.float32(z[i].max() + lead))).reshape(-1)[0]
            return bf16_bits(z) if dtype == "bf16" else z
        return f

    store = np.uint16 if dtype == "bf16" else np.float32
    student = _assemble(_draw_matrix(seed, rows, vocab, fill("student")), rows, vocab, store)
    teacher = _assemble(_draw_matrix(seed, rows, vocab, fill("teacher")), rows, vocab, store)
    return dict(name=f"distill_{dtype}", student=student, teacher=teacher, labels=labels,
                row_mask=row_mask, temperature=float(temperature), g=g, peak_rows=peak_rows)
