"""Oracle of the pages' deployed key sketch and its exact shortlist
("Verify Before You Fetch", Appendix A.1 "Key Sketch", and section 5.1,
"2-bit sketch implementation"). Test infrastructure: only the tests, the
smoke entry and the benchmark's CPU baseline call it.

For each layer and KV head the sketch keeps the 16 RoPE channel pairs with
the largest mean key energy (32 of 128 channels). Each kept channel is stored
at 2 bits per token, uniformly between the minimum and the maximum of each
128-token group, with an fp16 zero point and scale. At decode time the sketch
scores every token that is not resident. Per KV head, the 128 tokens with the
largest score over the head's query rows form the shortlist: their keys are
read from host memory and scored exactly. The plan then uses exact weights on
the resident and shortlisted tokens and sketch weights on the rest of L.

Readings where the pages leave a step open (each is also listed in the
design notes):

* RoPE pairs are (j, j + d/2), the "rotate half" layout of the Qwen3- and
  Llama-family models the pages evaluate. A pair's energy is the sum over all
  tokens of k_j^2 + k_{j+d/2}^2 (a mean ranks the same). Ties go to the lower j.
* Kept channels are listed in increasing channel index. The 2-bit code of
  kept slot c sits in bits 2c and 2c+1 of the token's 64-bit word.
* Levels: zero z = fp16(min) and scale s = fp16(fp32(max - min) / 3), both
  saturated at the largest finite fp16. The code is
  clamp(rint(fp32(fp32(k - z) / s)), 0, 3), with rint rounding half to even,
  and 0 when s == 0. The dequantised value is fp32(z + code * s).
* Sketch logit: <q, k^_i> / sqrt(d) over the kept channels (the others count
  as 0), summed in float64 in increasing channel order. A bf16 query entry
  times an fp32 dequantised value is exact in float64, so only the additions
  round. The result is multiplied by the float64 value of 1/sqrt(d).
* Shortlist: the tokens of L outside S (those not resident), ranked by the
  largest sketch logit over the KV head's query heads, after rounding to
  fp32 (the precision in which the kernel ranks them); descending, then
  position ascending. Size min(n_short, |L minus S|).
* Plan: exact logits on S and on the shortlist, sketch logits on the rest of
  L. The shift m is the largest of the resident exact logits and the plan's
  logits on L.
* Host traffic: one bf16 key row (2 d bytes) per shortlisted token, on top
  of the 4 d bytes of each fetched row.
"""

import math

import numpy as np

N_PAIRS = 16        # RoPE channel pairs kept per KV head
GROUP = 128         # tokens per quantisation group
LEVELS = 3          # 2-bit codes: 0..3, three steps between min and max
FP16_MAX = 65504.0


def rope_pairs(d):
    """Channel pairs (j, j + d/2), j < d/2, that RoPE rotates together."""
    h = d // 2
    return np.stack([np.arange(h), np.arange(h) + h], axis=1)


def pair_energy(keys):
    """Energy of each RoPE pair over all tokens: sum_i k_ij^2 + k_i,j+d/2^2
    (float64). ``keys``: [n][d]."""
    k = np.asarray(keys, dtype=np.float64)
    pr = rope_pairs(k.shape[1])
    return (k[:, pr[:, 0]] ** 2).sum(axis=0) + (k[:, pr[:, 1]] ** 2).sum(axis=0)


def select_pairs(energy, n_pairs=N_PAIRS):
    """The n_pairs pairs of largest energy (ties: lower index), ascending."""
    order = sorted(range(len(energy)), key=lambda j: (-float(energy[j]), j))
    return np.array(sorted(order[:n_pairs]), dtype=np.int64)


def kept_channels(pairs, d):
    """The channels of the kept pairs, in increasing channel index."""
    pairs = np.asarray(pairs, dtype=np.int64)
    return np.sort(np.concatenate([pairs, pairs + d // 2]))


def _fp16_sat(x):
    """fp32 -> fp16 (round to nearest even), saturated at the largest
    finite fp16; returned as float32."""
    x = np.clip(np.asarray(x, dtype=np.float32), -FP16_MAX, FP16_MAX)
    return x.astype(np.float16).astype(np.float32)


def quantize_group(vals):
    """One 128-token group of the kept channels. ``vals``: [m][c] float32.
    Returns (zero [c], scale [c], codes [m][c] uint8); zero and scale are
    fp16 values held in float32."""
    v = np.asarray(vals, dtype=np.float32)
    mn = v.min(axis=0)
    mx = v.max(axis=0)
    zero = _fp16_sat(mn)
    scale = _fp16_sat((mx - mn).astype(np.float32) / np.float32(LEVELS))
    with np.errstate(divide="ignore", invalid="ignore"):
        x = (v - zero[None, :]).astype(np.float32) / scale[None, :]
    code = np.clip(np.rint(x), 0, LEVELS)
    code = np.where(scale[None, :] > 0, code, 0)
    return zero, scale, code.astype(np.uint8)


def build(keys, n_pairs=N_PAIRS):
    """The sketch of one (layer, KV head). ``keys``: [n][d] (bf16 values).

    Returns a dict: ``chan`` [2 n_pairs] kept channels, ascending; ``zero``
    and ``scale`` [ceil(n/128)][2 n_pairs] fp16 values (float32);
    ``codes`` [n][2 n_pairs] uint8 in 0..3; ``energy`` [d/2] pair energies.
    """
    k = np.asarray(keys, dtype=np.float32)
    n, d = k.shape
    energy = pair_energy(k)
    pairs = select_pairs(energy, n_pairs)
    chan = kept_channels(pairs, d)
    ng = (n + GROUP - 1) // GROUP
    zero = np.zeros((ng, chan.size), dtype=np.float32)
    scale = np.zeros((ng, chan.size), dtype=np.float32)
    codes = np.zeros((n, chan.size), dtype=np.uint8)
    for gi in range(ng):
        lo, hi = gi * GROUP, min(n, (gi + 1) * GROUP)
        zero[gi], scale[gi], codes[lo:hi] = quantize_group(k[lo:hi][:, chan])
    return dict(chan=chan, zero=zero, scale=scale, codes=codes, energy=energy,
                pairs=pairs)


def with_pairs(keys, pairs):
    """The sketch of ``keys`` built on the given pairs (used where two pair
    energies tie to within rounding and either choice is correct)."""
    k = np.asarray(keys, dtype=np.float32)
    sk = build(k)
    chan = kept_channels(pairs, k.shape[1])
    n = k.shape[0]
    for gi in range(sk["zero"].shape[0]):
        lo, hi = gi * GROUP, min(n, (gi + 1) * GROUP)
        sk["zero"][gi], sk["scale"][gi], sk["codes"][lo:hi] = \
            quantize_group(k[lo:hi][:, chan])
    sk["chan"] = chan
    sk["pairs"] = np.asarray(pairs, dtype=np.int64)
    return sk


def dequantize(sk):
    """k^ [n][c] float32: fp32(zero + code * scale) per token and kept
    channel (code * scale is exact in fp32)."""
    codes = np.asarray(sk["codes"])
    gi = np.arange(codes.shape[0]) // GROUP
    z = sk["zero"][gi]
    s = sk["scale"][gi]
    return (z + (codes.astype(np.float32) * s).astype(np.float32)).astype(np.float32)


def sketch_logits(qh, sk):
    """Sketch logits <q, k^_i> / sqrt(d) over the kept channels (float64,
    summed in increasing channel order). ``qh``: [d] (bf16 values)."""
    qh = np.asarray(qh, dtype=np.float64)
    kh = dequantize(sk)
    acc = np.zeros(kh.shape[0], dtype=np.float64)
    for c, ch in enumerate(sk["chan"]):
        acc = acc + qh[ch] * kh[:, c].astype(np.float64)
    return acc * (1.0 / math.sqrt(qh.size))


def shortlist(scores32, eligible, n_short):
    """Positions of the shortlist, ascending. ``scores32``: [grp][n] fp32
    sketch logits of the KV head's query heads; ``eligible``: [n] bool (the
    tokens of L outside S). Rank by the largest score over the heads,
    descending, then position ascending; keep min(n_short, #eligible)."""
    s = np.asarray(scores32, dtype=np.float32).max(axis=0)
    pos = np.nonzero(np.asarray(eligible))[0]
    if n_short <= 0 or pos.size == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((pos, -s[pos].astype(np.float64)))
    return np.sort(pos[order[:n_short]]).astype(np.int64)


def pack_codes(codes):
    """[n][32] codes -> [n] uint64 words, slot c in bits 2c, 2c+1."""
    codes = np.asarray(codes, dtype=np.uint64)
    words = np.zeros(codes.shape[0], dtype=np.uint64)
    for c in range(codes.shape[1]):
        words |= codes[:, c] << np.uint64(2 * c)
    return words


def unpack_codes(words, n_chan=2 * N_PAIRS):
    """Inverse of pack_codes."""
    words = np.asarray(words, dtype=np.uint64)
    return np.stack([((words >> np.uint64(2 * c)) & np.uint64(3)).astype(np.uint8)
                     for c in range(n_chan)], axis=1)


def storage_bytes(sk):
    """Bytes the sketch occupies as stored: 2 bits per kept channel and
    token, and an fp16 zero point and scale per kept channel and group."""
    n, c = np.asarray(sk["codes"]).shape
    return n * c * 2 // 8 + sk["zero"].size * 2 + sk["scale"].size * 2
