// tactics_table.hpp -- the measured per-(N, K, batch) tactic table.
#pragma once

#include "../../include/tp1_proj.h"

namespace tp1 {

// Exact (N, K, bin) lookup in the table measured on MI355X.  Returns false
// when the shape/bin was not measured.
bool lookup_measured_tactic(int N, int K, int bin, proj_tactic_t *out);

}  // namespace tp1
