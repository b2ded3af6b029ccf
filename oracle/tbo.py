"""CPU oracle for the two-batch-overlap split (test infrastructure: only the
test suite may import it; it shares no code with the library).

"Large-scale EP: DeepEP, EPLB and two-batch overlap", section "TBO: hiding
communication behind computation" and its split-point exercise: a prefill
batch is cut at the sequence boundary whose cumulative token count is closest
to half, never inside a sequence; a decode batch in half by request count.
Reading: both micro-batches non-empty (cut after 1 .. n-1 sequences), ties to
the earlier cut; fewer than two sequences: no cut (0).
"""


def split(seq_lens, decode=False):
    n = len(seq_lens)
    if any(v < 0 for v in seq_lens):
        raise ValueError("negative sequence length")
    if n < 2:
        return 0
    if decode:
        return n // 2
    total = sum(seq_lens)
    gaps = [abs(2 * sum(seq_lens[:i]) - total) for i in range(1, n)]
    return 1 + gaps.index(min(gaps))
