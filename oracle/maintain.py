"""Oracle of decode-time maintenance ("Verify Before You Fetch", section 3:
compression may be repeated during a request, sink and local tokens stay
resident; Appendix A.3.1: the per-(layer, head) list of resident positions
grows as tokens are generated, new tokens are written after the packed
region; Appendix A.3.2: the fetch reuses rows staged in earlier steps).
Test infrastructure: only the tests, the smoke entry and the benchmark's
CPU baseline call it.

Readings where the pages leave a step open:

* A generated token joins H (r = 1, resident) of every (request, KV head) at
  the next position; nothing else changes until the next compression.
* Its projected sketch row is bf16(P^T k) with P^T k summed in fp32 over
  increasing dimension (rounding each product and each partial sum); its
  2-bit code word is 0 and a group that starts at it gets zero points and
  scales 0 (the sketch of a token of H is never used while it stays in H).
* Repeated compression is PoissonComp over the context as it stands (fresh
  scores, the same seed rule), replacing r and the resident rows.
* Staging keeps the rows fetched by the previous step; a row fetched again
  in the next step comes from the staging instead of host memory. Host
  bytes saved per (request, KV head) = 2 d 2 bytes per row in both fetch
  unions.
"""

import numpy as np


def bf16_rne(x):
    """float32 -> bfloat16 bits, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def sketch_row(proj_g, k):
    """bf16(P_g^T k): fp32 products and partial sums in increasing
    dimension. proj_g [d][s] float32, k [d] float32."""
    proj_g = np.asarray(proj_g, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    acc = np.zeros(proj_g.shape[1], dtype=np.float32)
    for e in range(proj_g.shape[0]):
        acc = (acc + (proj_g[e] * k[e]).astype(np.float32)).astype(np.float32)
    return bf16_rne(acc)


def append_token(state, pos, k_new, v_new, proj=None):
    """One generated token at position ``pos`` joins H of every (request,
    KV head). ``state``: dict with host_kv [B][G][ns][2][d] uint16 (bf16
    bits), r [B][G][ns] float32, res_idx[b][g] int64 arrays (ascending),
    res_kv[b][g] [count][2][d] uint16, optional sketch [B][G][ns][s] uint16
    and codes [B][G][ns] uint64 / zs [B][G][ngroups][2][32] uint16.
    k_new, v_new: [B][G][d] uint16. Updated in place; returns state."""
    B, G = state["r"].shape[:2]
    state["host_kv"][:, :, pos, 0, :] = k_new
    state["host_kv"][:, :, pos, 1, :] = v_new
    state["r"][:, :, pos] = np.float32(1.0)
    for b in range(B):
        for g in range(G):
            idx = state["res_idx"][b][g]
            if idx.size and idx[-1] >= pos:
                raise ValueError("pos must follow every resident position")
            state["res_idx"][b][g] = np.append(idx, pos).astype(np.int64)
            row = np.stack([k_new[b, g], v_new[b, g]])[None]
            state["res_kv"][b][g] = np.concatenate([state["res_kv"][b][g], row])
            if proj is not None and state.get("sketch") is not None:
                kf = (k_new[b, g].astype(np.uint32) << 16).view(np.float32)
                state["sketch"][b, g, pos] = sketch_row(proj[g], kf)
    if state.get("codes") is not None:
        state["codes"][:, :, pos] = 0
        if pos % 128 == 0:
            state["zs"][:, :, pos // 128] = 0
    return state


def staged_hits(prev_union, union):
    """Rows of this step's fetch union that the previous step fetched (and
    staged): their sorted positions."""
    return np.intersect1d(np.asarray(prev_union, dtype=np.int64),
                          np.asarray(union, dtype=np.int64))
