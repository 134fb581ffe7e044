// Specialized kernel sets of one slice of the wider (s, m, H) grid.
#include "sbf_spec.hpp"
#include "sbf_spec_list.hpp"

namespace sbf {
#define SBF_ENTRY(K, M, S, H) {0u, K, M, S, H, &spec_set<K, M, S, H>},
static const SpecEntry table[] = {SBF_SLICE_M_A(SBF_ENTRY)};
const SpecEntry* spec_table_slice_m_a(size_t* n)
{
    *n = sizeof(table) / sizeof(table[0]);
    return table;
}
}  // namespace sbf
