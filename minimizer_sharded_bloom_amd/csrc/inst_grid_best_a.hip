// Specialized kernel sets of the lowest-FPR block of the (s, m) grid at H = 4.
#include "sbf_spec.hpp"
#include "sbf_spec_list.hpp"

namespace sbf {
#define SBF_ENTRY(K, M, S, H) {0u, K, M, S, H, &spec_set<K, M, S, H>},
static const SpecEntry table[] = {SBF_GRID_BEST_A(SBF_ENTRY)};
const SpecEntry* spec_table_grid_best_a(size_t* n)
{
    *n = sizeof(table) / sizeof(table[0]);
    return table;
}
}  // namespace sbf
