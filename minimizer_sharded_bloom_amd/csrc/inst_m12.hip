// Specialized kernel sets of the k = 31 sweep with m = 12.
#include "sbf_spec.hpp"
#include "sbf_spec_list.hpp"

namespace sbf {
#define SBF_ENTRY(K, M, S, H) {0u, K, M, S, H, &spec_set<K, M, S, H>},
static const SpecEntry table[] = {SBF_SWEEP_M(SBF_ENTRY, 12)};
const SpecEntry* spec_table_m12(size_t* n)
{
    *n = sizeof(table) / sizeof(table[0]);
    return table;
}
}  // namespace sbf
