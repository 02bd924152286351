// Host-side planning functions of the library (plain C++, no HIP): the EPLB
// placement planner and the exact capacity of the capacity factor.
#pragma once

#include <stdint.h>

namespace moe {

// Placement of num_physical slots (see moe_eplb_place in include/moe.h);
// returns the number of slots written (num_physical on success).
int eplb_place(const double* load, int num_experts, int num_groups, int num_nodes, int num_gpus,
               int num_physical, bool hierarchical, int* phys_to_logical, int* replica_offsets,
               int* replica_slots);

// ceil(factor_num * tokens_times_k / (factor_den * num_experts)), exact for
// factors below 2^31; INT64_MAX if the result does not fit.
int64_t expert_capacity(int64_t tokens_times_k, int64_t factor_num, int64_t factor_den, int64_t num_experts);

}  // namespace moe
