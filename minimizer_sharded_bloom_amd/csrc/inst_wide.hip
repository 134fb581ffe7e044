// Specialized kernel sets of the wide-block variant.
#include "sbf_spec_list.hpp"
#include "sbf_wide.hpp"

namespace sbf {
#define SBF_ENTRY_WIDE(K, M, S, H) {2u, K, M, S, H, &wide_set<K, M, S, H>},
static const SpecEntry table[] = {SBF_WIDE(SBF_ENTRY_WIDE)};
const SpecEntry* spec_table_wide(size_t* n)
{
    *n = sizeof(table) / sizeof(table[0]);
    return table;
}
}  // namespace sbf
