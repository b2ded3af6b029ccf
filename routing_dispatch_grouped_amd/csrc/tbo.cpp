// Two-batch overlap: where a batch is cut into two micro-batches.  Host code.
//
// "Large-scale EP: DeepEP, EPLB and two-batch overlap", section "TBO: hiding
// communication behind computation", and its exercise on the split point: a
// prefill batch is cut at the sequence boundary whose cumulative token count
// is closest to half the batch, never inside a sequence (so the halves are
// usually not equal); a decode batch is cut in half by request count.
#include <cstdint>

#include "rdg.h"

extern "C" int rdg_tbo_split(const int32_t* seq_lens, int n_seqs, int decode) {
    if (n_seqs < 0 || (n_seqs > 0 && !seq_lens)) return RDG_EINVAL;
    if (n_seqs < 2) return 0;  // nothing to cut: one micro-batch
    if (decode) return n_seqs / 2;
    int64_t total = 0;
    for (int i = 0; i < n_seqs; ++i) {
        if (seq_lens[i] < 0) return RDG_EINVAL;
        total += seq_lens[i];
    }
    // cut after sequence i-1, i in [1, n_seqs - 1]: |2 * prefix - total| smallest, ties to the lower i
    int best = 1;
    int64_t best_gap = -1, prefix = 0;
    for (int i = 1; i < n_seqs; ++i) {
        prefix += seq_lens[i - 1];
        const int64_t gap = 2 * prefix > total ? 2 * prefix - total : total - 2 * prefix;
        if (best_gap < 0 || gap < best_gap) {
            best_gap = gap;
            best = i;
        }
    }
    return best;
}
