"""Token permute into the masked-GEMM layout (oracle; test infrastructure only).

Follows the HALOps "GEMM" page, prefill_permute_to_masked_gemm section: every
(token, slot) pair of the top-k routing whose expert id is e sends the
token's row to the next free row of expert e's slot in the padded layout
[E, max_token_num, ...]; the per-expert counts are returned, a map records
the expert-local row each pair landed on, and the token's scale factors are
re-laid out at one byte per 32 elements.

Readings where the section leaves a step open (each one is also listed in
the design notes):
  * Order inside an expert: the section fixes none.  This oracle fills rows
    in row-major (token, slot) order.  Any other order is as correct; tests
    compare what is unique (counts, row contents, the map's consistency).
  * Ids outside [0, E) -- the section's -1 and anything else -- are
    unassigned: map -1, nothing written.
  * An expert named by more than max_token_num pairs: the section's kernel
    writes past the slot; here the pairs past max_token_num are dropped
    (map -1) and the count is the number of rows written.
  * Scale modes.  Broadcast: int32 [T, H/512], byte b (little-endian) of word
    w is the scale of the 128-group 4w + b; each 128-group scale becomes the
    scale of its four 32-groups.  Direct: uint8 [T, H/32], copied as is.
    The output is row-major [E, max_token_num, H/32] -- the scale layout the
    masked GEMM here takes -- instead of the SfAtom tiling.
  * The row payload (FP8 codes, BF16 values or packed FP4 codes) is opaque
    and copied bit for bit; its byte width need not be H.
"""

import numpy as np

BROADCAST, DIRECT = 0, 1


def expand_scales(scale, hidden, mode):
    """Per-32 scale bytes [T, hidden/32] of one scale tensor."""
    scale = np.asarray(scale)
    T = scale.shape[0]
    g32 = hidden // 32
    out = np.zeros((T, g32), np.uint8)
    if mode == DIRECT:
        out[:, :] = scale.astype(np.uint8)[:, :g32]
        return out
    words = scale.astype(np.int64) & 0xFFFFFFFF
    for g in range(g32):
        g128 = g // 4                       # the 128-group holding 32-group g
        w, b = g128 // 4, g128 % 4          # its word and byte
        out[:, g] = (words[:, w] >> (8 * b)) & 0xFF
    return out


def permute_to_masked(x_rows, scale, topk_ids, num_experts, max_tokens, hidden, mode):
    """Returns a dict:
      x       [E * max_tokens, RB] uint8, written rows filled (others 0)
      written [E * max_tokens] bool
      scale   [E, max_tokens, hidden/32] uint8 (written rows only, others 0)
      map     [T, topk] int32, expert-local row or -1
      counts  [E] int32, rows written per expert
    """
    x_rows = np.asarray(x_rows, np.uint8)
    T, RB = x_rows.shape
    ids = np.asarray(topk_ids, np.int64)
    ids = ids.reshape(T, -1) if ids.ndim != 2 else ids
    topk = ids.shape[1]
    E, M = int(num_experts), int(max_tokens)
    sf = expand_scales(scale, hidden, mode)
    out_x = np.zeros((E * M, RB), np.uint8)
    written = np.zeros(E * M, bool)
    out_s = np.zeros((E, M, hidden // 32), np.uint8)
    pmap = np.full((T, topk), -1, np.int32)
    counts = np.zeros(E, np.int64)
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if e < 0 or e >= E:
                continue
            p = int(counts[e])
            if p >= M:
                continue                    # dropped: the slot is full
            counts[e] = p + 1
            pmap[t, j] = p
            out_x[e * M + p] = x_rows[t]
            written[e * M + p] = True
            out_s[e, p] = sf[t]
    return {"x": out_x, "written": written, "scale": out_s, "map": pmap,
            "counts": counts.astype(np.int32)}
