"""CPU oracle for the expert-parallel load balancer's placement (test
infrastructure: only the test suite may import it; the product path never
touches it, and it shares no code with the library).

What it computes follows the pages' description of the balancer:

* "Large-scale EP: DeepEP, EPLB and two-batch overlap", section "EPLB:
  redundant experts and rebalancing": the measured per-expert token counts
  are turned into a new expert-to-GPU mapping; the assignment is
  hierarchical -- expert groups are first spread over nodes, and the
  experts of a node are then assigned inside it, so that one node's
  experts come from the same group where possible; redundant slots
  (256 logical experts in 288 physical ones) hold extra copies of the
  popular experts.
* "SGLang open-sources the first DeepSeek-V3/R1 H100 deployment ...",
  section "Expert-parallel load balancer": the most used experts get more
  copies, the rarely used ones share a GPU with medium ones; any GPU count
  (not only powers of two); balance = mean over maximum of the GPUs' loads.

The pages name the steps but not their rules; the plainest reading, used
here and written out in the design notes:

1. Groups to nodes (only when the group count is a multiple of the node
   count; otherwise the whole machine is treated as one node): each group's
   load is the sum of its experts' loads; groups in decreasing load (ties:
   lower group id) each go to the node with the least load so far among
   nodes that still take groups (each node takes groups / nodes of them;
   ties: lower node id).
2. Replicas inside a node: every expert of the node starts with one copy;
   each remaining slot of the node goes, one at a time, to the expert with
   the largest load per copy (ties: lower expert id).
3. Copies to GPUs inside a node: every copy carries its expert's load
   divided by the expert's copy count; copies in decreasing load (ties:
   lower expert id, then lower copy index) each go to the node's GPU with
   the least load so far among GPUs with a free slot (ties: lower GPU id);
   a copy takes the GPU's next slot.  Physical id = GPU * slots per GPU +
   slot.

Plain Python loops over lists; loads are Python floats (IEEE doubles), and
every sum is formed in the order stated above.
"""


def _balanced_pack(items, n_packs, cap, pack_base=0):
    """items: list of (load, key...) already in processing order.  Returns
    (assignment list of (pack, slot) per item, pack loads)."""
    loads = [0.0] * n_packs
    used = [0] * n_packs
    out = []
    for it in items:
        best = -1
        for p in range(n_packs):
            if used[p] >= cap:
                continue
            if best < 0 or loads[p] < loads[best]:
                best = p
        out.append((pack_base + best, used[best]))
        used[best] += 1
        loads[best] += it[0]
    return out, loads


def place(load, n_groups, n_nodes, n_gpus, n_physical):
    """Returns dict(phy2log [n_physical], log2phy (list of lists of physical
    ids per logical expert), n_replica [N], gpu_load [n_gpus], hierarchical)."""
    load = [float(v) for v in load]
    N = len(load)
    if (N == 0 or n_groups <= 0 or N % n_groups or n_nodes <= 0 or n_gpus <= 0 or n_gpus % n_nodes
            or n_physical % n_gpus or n_physical < N):
        raise ValueError("invalid EPLB shape")
    hier = n_groups % n_nodes == 0 and n_nodes > 1
    nodes = n_nodes if hier else 1
    gpn = n_gpus // nodes               # GPUs per node
    spg = n_physical // n_gpus          # slots per GPU
    per_group = N // n_groups

    # 1. groups to nodes
    if hier:
        gload = []
        for g in range(n_groups):
            s = 0.0
            for e in range(g * per_group, (g + 1) * per_group):
                s += load[e]
            gload.append(s)
        order = sorted(range(n_groups), key=lambda g: (-gload[g], g))
        assign, _ = _balanced_pack([(gload[g], g) for g in order], nodes, n_groups // nodes)
        node_of_group = [0] * n_groups
        for g, (nd, _slot) in zip(order, assign):
            node_of_group[g] = nd
    else:
        node_of_group = [0] * n_groups

    phy2log = [-1] * n_physical
    log2phy = [[] for _ in range(N)]
    n_rep = [0] * N
    gpu_load = [0.0] * n_gpus
    slots_per_node = n_physical // nodes
    for nd in range(nodes):
        experts = [e for e in range(N) if node_of_group[e // per_group] == nd]
        if slots_per_node < len(experts):
            raise ValueError("fewer slots than experts on a node")
        # 2. replicas
        cnt = {e: 1 for e in experts}
        for _ in range(slots_per_node - len(experts)):
            best = experts[0]
            for e in experts[1:]:
                if load[e] / cnt[e] > load[best] / cnt[best]:
                    best = e
            cnt[best] += 1
        # 3. copies to the node's GPUs
        copies = [(load[e] / cnt[e], e, r) for e in experts for r in range(cnt[e])]
        copies.sort(key=lambda c: (-c[0], c[1], c[2]))
        assign, loads = _balanced_pack(copies, gpn, spg, pack_base=nd * gpn)
        for (ld, e, r), (gpu, slot) in zip(copies, assign):
            p = gpu * spg + slot
            phy2log[p] = e
        for e in experts:
            n_rep[e] = cnt[e]
            log2phy[e] = [0] * cnt[e]
        for (ld, e, r), (gpu, slot) in zip(copies, assign):
            log2phy[e][r] = gpu * spg + slot
        for i in range(gpn):
            gpu_load[nd * gpn + i] = loads[i]
    return dict(phy2log=phy2log, log2phy=log2phy, n_replica=n_rep, gpu_load=gpu_load, hierarchical=hier)


def balance(gpu_load):
    """Mean over maximum of the GPUs' loads (1.0 = perfectly balanced)."""
    m = max(gpu_load)
    return 1.0 if m == 0 else (sum(gpu_load) / len(gpu_load)) / m
