// Host-side planning code of the library, plain C++ with no HIP dependency (so
// that it can also be built and checked under the address and undefined-
// behaviour sanitizers on its own):
//
// * eplb_place -- EPLB placement of logical experts, with redundant replicas,
//   on GPUs (page "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠",
//   anrans.github.io, section "EPLB 与路由约束"). Hierarchical strategy: pack
//   the expert groups onto the nodes, balanced by load with the same number
//   of groups per node; inside each node give the hottest experts extra
//   replicas; pack each node's physical experts onto its GPUs, balanced, the
//   same number per GPU. Global strategy: the same over all experts and GPUs
//   at once. Balanced packing takes items heaviest first (equal weights:
//   lower index first) into the lightest pack that still has room (equal
//   totals: lower pack); replication repeatedly adds a replica to the expert
//   with the highest load per replica (equal: the expert listed first). Sums
//   are float64 in placement order.
// * expert_capacity -- C = ceil(c * T * k / E) with c = num / den, in exact
//   integer arithmetic (ch15 section 4.3, capacity factor).
#include "host_plan.h"

#include <algorithm>
#include <vector>

namespace moe {

namespace {

std::vector<std::vector<int>> balanced_pack(const std::vector<double>& w, int n_packs) {
  const int n = (int)w.size();
  const int room = n / n_packs;
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a] > w[b]; });
  std::vector<std::vector<int>> packs(n_packs);
  std::vector<double> total(n_packs, 0.0);
  for (int item : order) {
    int target = -1;
    for (int p = 0; p < n_packs; ++p)
      if ((int)packs[p].size() < room && (target < 0 || total[p] < total[target])) target = p;
    packs[target].push_back(item);
    total[target] += w[item];
  }
  return packs;
}

}  // namespace

int eplb_place(const double* load, int E, int num_groups, int num_nodes, int num_gpus, int num_physical,
               bool hierarchical, int* phys_to_logical, int* replica_offsets, int* replica_slots) {
  const int G = E / num_groups;
  std::vector<std::vector<int>> node_experts;
  if (hierarchical) {
    std::vector<double> group_load(num_groups, 0.0);
    for (int g = 0; g < num_groups; ++g)
      for (int e = g * G; e < (g + 1) * G; ++e) group_load[g] += load[e];
    for (const auto& groups : balanced_pack(group_load, num_nodes)) {
      std::vector<int> experts;
      for (int g : groups)
        for (int e = g * G; e < (g + 1) * G; ++e) experts.push_back(e);
      node_experts.push_back(experts);
    }
  } else {
    std::vector<int> all(E);
    for (int e = 0; e < E; ++e) all[e] = e;
    node_experts.push_back(all);
  }
  std::vector<int> count(E, 0);
  int slot = 0;
  for (const auto& experts : node_experts) {
    const int n = (int)experts.size();
    const int n_phys = (int)((long)num_physical * n / E);
    const int n_gpus = (int)((long)num_gpus * n / E);
    for (int e : experts) count[e] = 1;
    for (int r = n; r < n_phys; ++r) {
      int best = experts[0];
      for (int i = 1; i < n; ++i) {
        const int e = experts[i];
        if (load[e] / count[e] > load[best] / count[best]) best = e;
      }
      ++count[best];
    }
    std::vector<int> physical;
    std::vector<double> weight;
    for (int e : experts)
      for (int c = 0; c < count[e]; ++c) {
        physical.push_back(e);
        weight.push_back(load[e] / count[e]);
      }
    for (const auto& pack : balanced_pack(weight, n_gpus))
      for (int i : pack) phys_to_logical[slot++] = physical[i];
  }
  // replica table: slots of each expert in ascending order (a counting sort)
  for (int e = 0; e <= E; ++e) replica_offsets[e] = 0;
  for (int s = 0; s < num_physical; ++s) ++replica_offsets[phys_to_logical[s] + 1];
  for (int e = 0; e < E; ++e) replica_offsets[e + 1] += replica_offsets[e];
  std::vector<int> fill(replica_offsets, replica_offsets + E);
  for (int s = 0; s < num_physical; ++s) replica_slots[fill[phys_to_logical[s]]++] = s;
  return slot;
}

int64_t expert_capacity(int64_t tokens_times_k, int64_t factor_num, int64_t factor_den, int64_t num_experts) {
  // every factor is below 2^31, so the 128-bit product and quotient are exact
  const __int128 q = (__int128)factor_num * tokens_times_k;
  const __int128 den = (__int128)factor_den * num_experts;
  const __int128 c = (q + den - 1) / den;
  return c > (__int128)INT64_MAX ? INT64_MAX : (int64_t)c;
}

}  // namespace moe
