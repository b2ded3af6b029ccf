// Expert-parallel load balancer: placement of logical experts (with
// redundant copies) onto GPUs from measured per-expert loads.  Host code; it
// runs off the hot path (between rebalances) and produces the table that the
// remap kernel reads.
//
// What it computes ("Large-scale EP: DeepEP, EPLB and two-batch overlap",
// section "EPLB: redundant experts and rebalancing"; H100 deployment article,
// section "Expert-parallel load balancer"): a hierarchical assignment --
// expert groups are spread over nodes first, then each node's experts get
// its slots -- in which the most loaded experts get extra copies and rarely
// used experts share a GPU with busier ones, for any GPU count.
//
// The rules, the plainest reading of that description:
//   1. groups to nodes (when the group count is a multiple of the node
//      count, else the machine is one node): group load = sum of its
//      experts' loads; groups by decreasing load (ties: lower id) each go to
//      the least-loaded node that still takes groups (ties: lower node);
//   2. every expert of a node starts with one copy; each remaining slot of
//      the node goes to the expert with the largest load per copy (ties:
//      lower id);
//   3. copies (load / copy count each) by decreasing load (ties: lower
//      expert id, then lower copy index) each go to the node's least-loaded
//      GPU with a free slot (ties: lower GPU), taking its next slot;
//      physical id = GPU * slots per GPU + slot.
// Loads are doubles and every sum is formed in the order above, so the
// result is exactly reproducible.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "rdg.h"

namespace {

struct Copy {
    double load;
    int expert, replica;
};

// Least-loaded pack with room among packs [0, n) (ties: lower index).
int least_loaded(const std::vector<double>& load, const std::vector<int>& used, int base, int n, int cap) {
    int best = -1;
    for (int p = base; p < base + n; ++p) {
        if (used[p] >= cap) continue;
        if (best < 0 || load[p] < load[best]) best = p;
    }
    return best;
}

}  // namespace

extern "C" int rdg_eplb_place(const double* load, int n_logical, int n_groups, int n_nodes, int n_gpus,
                              int n_physical, int r_max, int32_t* phy2log, int32_t* log2phy, int32_t* n_replica,
                              double* gpu_load) {
    const int N = n_logical;
    if (!load || !phy2log || !log2phy || !n_replica || N <= 0 || n_groups <= 0 || N % n_groups || n_nodes <= 0 ||
        n_gpus <= 0 || n_gpus % n_nodes || n_physical <= 0 || n_physical % n_gpus || n_physical < N || r_max <= 0)
        return RDG_EINVAL;
    for (int e = 0; e < N; ++e)
        if (!std::isfinite(load[e]) || load[e] < 0.0) return RDG_EINVAL;

    const bool hier = n_nodes > 1 && n_groups % n_nodes == 0;
    const int nodes = hier ? n_nodes : 1;
    const int gpn = n_gpus / nodes, spg = n_physical / n_gpus, per_group = N / n_groups;
    const int slots_per_node = n_physical / nodes;

    // 1. groups to nodes
    std::vector<int> node_of_group(n_groups, 0);
    if (hier) {
        std::vector<double> gload(n_groups, 0.0);
        for (int g = 0; g < n_groups; ++g)
            for (int e = g * per_group; e < (g + 1) * per_group; ++e) gload[g] += load[e];
        std::vector<int> order(n_groups);
        for (int g = 0; g < n_groups; ++g) order[g] = g;
        std::sort(order.begin(), order.end(), [&](int a, int b) { return gload[a] != gload[b] ? gload[a] > gload[b] : a < b; });
        std::vector<double> nload(nodes, 0.0);
        std::vector<int> nused(nodes, 0);
        for (int g : order) {
            const int nd = least_loaded(nload, nused, 0, nodes, n_groups / nodes);
            node_of_group[g] = nd;
            nused[nd] += 1;
            nload[nd] += gload[g];
        }
    }

    std::vector<double> gl(n_gpus, 0.0);
    std::vector<int> gused(n_gpus, 0);
    std::vector<int> cnt(N, 1);
    std::vector<int> experts;
    std::vector<Copy> copies;
    for (int nd = 0; nd < nodes; ++nd) {
        experts.clear();
        for (int e = 0; e < N; ++e)
            if (node_of_group[e / per_group] == nd) experts.push_back(e);
        if ((int)experts.size() > slots_per_node) return RDG_EINVAL;
        // 2. copies of the most loaded experts (per copy)
        for (int extra = slots_per_node - (int)experts.size(); extra > 0; --extra) {
            int best = experts[0];
            for (size_t i = 1; i < experts.size(); ++i) {
                const int e = experts[i];
                if (load[e] / cnt[e] > load[best] / cnt[best]) best = e;
            }
            cnt[best] += 1;
        }
        for (int e : experts)
            if (cnt[e] > r_max) return RDG_ECAPACITY;
        // 3. copies to the node's GPUs
        copies.clear();
        for (int e : experts)
            for (int r = 0; r < cnt[e]; ++r) copies.push_back({load[e] / cnt[e], e, r});
        std::sort(copies.begin(), copies.end(), [](const Copy& a, const Copy& b) {
            if (a.load != b.load) return a.load > b.load;
            if (a.expert != b.expert) return a.expert < b.expert;
            return a.replica < b.replica;
        });
        for (const Copy& c : copies) {
            const int gpu = least_loaded(gl, gused, nd * gpn, gpn, spg);
            const int p = gpu * spg + gused[gpu];
            gused[gpu] += 1;
            gl[gpu] += c.load;
            phy2log[p] = c.expert;
            log2phy[(size_t)c.expert * r_max + c.replica] = p;
        }
    }
    for (int e = 0; e < N; ++e) {
        n_replica[e] = cnt[e];
        for (int r = cnt[e]; r < r_max; ++r) log2phy[(size_t)e * r_max + r] = -1;
    }
    if (gpu_load)
        for (int g = 0; g < n_gpus; ++g) gpu_load[g] = gl[g];
    return RDG_OK;
}
