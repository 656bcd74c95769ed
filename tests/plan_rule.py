"""Host restatement of the load-balancing rule of the forward pass, used by the GPU tests
to check the plan the device writes (piece length, pieces, split sequences).

Chunks are cs tokens; n_slots chunk-kernel workgroups run at once.  A sequence of n
chunks is split when n > 9L/8: a first piece of L chunks, then ceil((n - L) / L) near-equal
later pieces (each run as two chains).  L is the smallest length >= max(4,
ceil(H S / n_slots)) with H (S + E(L)) <= n_slots L, where S is the total of chunks and E(L)
the chunks moved into later pieces, and with E(L) <= w_cap and the later pieces P(L) <=
np_cap (what the workspace holds); L then grows by 1/16 steps while the units longer
than L/2 outnumber the slots.
"""


def chunks(length, cs):
    return (length + cs - 1) // cs if length > 0 else 0


def split(n, L):
    return L > 0 and 8 * n > 9 * L


def later_pieces(n, L):
    R = n - L
    P = (R + L - 1) // L
    base, rem = divmod(R, P)
    return [base + (1 if i < rem else 0) for i in range(P)]


def plan(lengths, H, n_slots, cs, l_min=4, np_cap=None, w_cap=None):
    n_cu = n_slots
    n = [chunks(x, cs) for x in lengths]
    S, maxn = sum(n), max(n) if n else 0
    L0 = max(l_min, (H * S + n_cu - 1) // n_cu)
    L = 0
    if 8 * maxn > 9 * L0:
        lo, hi = L0, maxn
        while lo < hi:
            mid = lo + (hi - lo) // 2
            E = sum(x - mid for x in n if 8 * x > 9 * mid)
            P = sum((x - mid + mid - 1) // mid for x in n if 8 * x > 9 * mid)
            if H * (S + E) <= n_cu * mid and (w_cap is None or E <= w_cap) \
                    and (np_cap is None or P <= np_cap):
                hi = mid
            else:
                lo = mid + 1
        L = lo
        while L < maxn:
            big = 0
            for x in n:
                if split(x, L):
                    big += 1 + 2 * sum(1 for y in later_pieces(x, L) if 2 * y > L)
                elif 2 * x > L:
                    big += 1
            if H * big <= n_cu:
                break
            L = max(L + 1, L * 17 // 16)
        if not 8 * maxn > 9 * L:
            L = 0
    pieces = [later_pieces(x, L) for x in n if split(x, L)]
    return {"L": L, "n_split": len(pieces), "n_piece": sum(len(p) for p in pieces),
            "n_echunk": sum(sum(p) for p in pieces)}
