"""GPU parity of the heads' teacher-forced hit counts (medusa_head_hits) against
the oracle's loop: exact integers.  Cases span many blocks and the grid-stride
loop, heads past the 64 held in LDS, sequences too short for the far heads, and
the empty input."""
import numpy as np
import pytest

from oracle.calib import head_hit_counts

from _gpu import say

pytestmark = pytest.mark.gpu


def _case(seed, N, H, K, vocab, n_tokens):
    rng = np.random.default_rng(seed)
    tokens = rng.integers(0, vocab, n_tokens).astype(np.int32)
    topk = rng.integers(0, vocab, (N, H, K)).astype(np.int32)
    # plant hits at a few ranks so every bin sees some
    for t in range(N):
        for k in range(H):
            j = t + k + 2
            if j < n_tokens and rng.random() < 0.4:
                topk[t, k, rng.integers(0, K)] = tokens[j]
    return topk, tokens


@pytest.mark.parametrize("seed,N,H,K,vocab,n_tokens", [
    (0, 3000, 4, 10, 50, 3005),     # 47 blocks; the last heads lose their targets at the end
    (1, 1500, 5, 8, 7, 1200),       # tokens shorter than the positions: many without a target
    (2, 40, 70, 2, 5, 100),         # heads past the 64 LDS position bins
    (3, 100000, 3, 4, 30, 100010),  # 1172 blocks of pairs on a 1024-block grid: grid-stride loop
])
def test_head_hits_match_oracle(dev, seed, N, H, K, vocab, n_tokens):
    import torch
    from speculative_decoding_heads_amd import api
    say("head hits", N, H, K, n_tokens)
    topk, tokens = _case(seed, N, H, K, vocab, n_tokens)
    counts, positions = api.head_hits(torch.from_numpy(topk).to(dev), torch.from_numpy(tokens).to(dev))
    torch.cuda.synchronize()
    if N <= 3000:
        rc, rp = head_hit_counts(topk, tokens)
    else:
        # the oracle's loop on a slice of positions, and the per-head totals of
        # the rest by the same definition written as array compares
        rc, rp = head_hit_counts(topk[:2000], tokens[:2000 + H + 1])
        for k in range(H):
            t = np.arange(2000, N)
            t = t[t + k + 2 < n_tokens]
            rp[k] += len(t)
            rc[k] += (topk[t, k, :] == tokens[t + k + 2][:, None]).sum(0)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(positions.cpu().numpy(), rp)


def test_head_hits_accumulate_and_empty(dev):
    import torch
    from speculative_decoding_heads_amd import api
    say("head hits accumulate")
    topk, tokens = _case(5, 500, 4, 10, 20, 510)
    tk, tt = torch.from_numpy(topk).to(dev), torch.from_numpy(tokens).to(dev)
    c, p = api.head_hits(tk, tt)
    api.head_hits(tk, tt, c, p)
    api.head_hits(tk[:0], tt, c, p)  # N = 0: nothing added
    torch.cuda.synchronize()
    rc, rp = head_hit_counts(topk, tokens)
    np.testing.assert_array_equal(c.cpu().numpy(), 2 * rc)
    np.testing.assert_array_equal(p.cpu().numpy(), 2 * rp)
