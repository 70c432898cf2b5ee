"""Expected region sizes of the sparse-step workspace (what the C ABI's
ckv_workspace_bytes must return, and where the fused step's published words
lie)."""


def workspace_regions(B, Hq, Hkv, D, max_blocks, budget):
    """Region sizes of the sparse-step workspace, each 256-byte aligned:
    control words, per-block scores, chunk partials, select candidates,
    gather partials, fused chunk headers, fused candidates, fused tagged
    weights, fused partials."""
    def up(x):
        return (x + 255) // 256 * 256
    G = Hq // Hkv
    bg = B * Hkv
    pst = D + 4
    n_chunks, n_slices = -(-max_blocks // 256), -(-max_blocks // 1024)
    kmax = min(max_blocks, budget // 16)
    kcap = max(kmax, 1)
    n_splits = min(64, max(1, min((kmax + 3) // 4, max(1, 256 // bg)), -(-kmax // 256)))
    return [up((64 + 8 * bg) * 4), up(B * Hq * max_blocks * 4), up(bg * n_chunks * G * pst * 4),
            up(bg * n_slices * kcap * 8), up(bg * n_splits * G * 2 * pst * 4),
            up(2 * bg * n_chunks * G * 8), up(2 * bg * n_chunks * kcap * 8),
            up(bg * n_chunks * G * 257 * 8), up(bg * 2 * n_chunks * G * (D + 2) * 8)]


# Fused chunk headers ([2][B*Hkv][n_chunks][G] words) and candidates
# ([2][B*Hkv][n_chunks][kcap] words): a call with tag t (the pair's epoch
# counter before the call, plus one) publishes into half t % 2 and clears the
# other half, so between calls half (epoch + 1) % 2 of every pair is zero.
PUBLISHED_REGIONS = (5, 6)


def published_row_words(Hq, Hkv, max_blocks, budget):
    """Words per (pair, half) of the header and candidate regions."""
    G = Hq // Hkv
    n_chunks = -(-max_blocks // 256)
    kcap = max(min(max_blocks, budget // 16), 1)
    return {5: n_chunks * G, 6: n_chunks * kcap}
