"""Where mla_decode_paged puts each row's partials: the slot rule its C header
documents (include/mla.h, the num_splits argument of mla_decode_paged),
restated here from that text for the GPU tests.

The oracle carries no split plan: oracle.decode_split computes the partials of
whatever page ranges it is handed. The GPU tests hand it the ranges this rule
assigns, so that the kernel's o_part / lse_part can be compared slot by slot.
The rule is part of the interface (the layout of the caller's workspace), not
of the method: any page-aligned partition gives the same merged result (K3
study, "Inside the blocks").

Rule, for the rows r = b * s_q + i in order, row r having n_r visible pages,
P_r = n_0 + ... + n_(r-1) its first page in the concatenation and
P_tot = sum_r n_r:
  * 256 workgroups each scan one range of W consecutive pages of the
    concatenation: range k holds pages [k W, (k + 1) W);
  * num_splits S > 1: W = max(ceil(P_tot / 256), ceil((n_max - 1) / (S - 1)), 1);
    row r is cut at range borders, and its piece inside range k goes to slot
    k - floor(P_r / W);
  * S = 1: rows are not cut; each row is one piece, in slot 0.
Slots that receive no piece are empty.
"""
from __future__ import annotations

WORKGROUPS = 256  # ranges of the scan, as the header states


def header_pieces(row_pages, num_splits: int, workgroups: int = WORKGROUPS):
    """Per row, the list of (slot, first page, end page) the header's rule gives."""
    n = [int(x) for x in row_pages]
    total = sum(n)
    out = [[] for _ in n]
    if total == 0:
        return out
    S = int(num_splits)
    if S == 1:
        for r, nr in enumerate(n):
            if nr > 0:
                out[r] = [(0, 0, nr)]
        return out
    W = max(-(-total // workgroups), -(-(max(n) - 1) // (S - 1)), 1)
    start = 0
    for r, nr in enumerate(n):
        end = start + nr
        k = start // W
        while k * W < end:
            lo, hi = max(start, k * W), min(end, (k + 1) * W)
            out[r].append((k - start // W, lo - start, hi - start))
            k += 1
        start = end
    return out


def row_pages(seqlens, s_q: int, page: int = 64):
    """Visible pages of every row (b, i) in order: query i of an s_q-token
    chunk sees L_b - s_q + i + 1 keys."""
    pages = []
    for L in seqlens:
        for i in range(s_q):
            v = int(L) - s_q + i + 1
            pages.append(-(-v // page) if v > 0 else 0)
    return pages
