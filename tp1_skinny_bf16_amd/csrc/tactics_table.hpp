// tactics_table.hpp -- the measured per-(N, K, batch) tactic table.
#pragma once

#include "../../include/tp1_proj.h"

namespace tp1 {

// Lookup in the table measured on MI355X: the tactic of the smallest
// measured bin >= bin for (N, K).  Returns false when the shape was not
// measured or every measured bin is below `bin`.
bool lookup_measured_tactic(int N, int K, int bin, proj_tactic_t *out);

// For a shape the table has not measured: the tactics of measured shapes
// within a factor of two (|ln(N/N')| + |ln(K/K')| <= ln 2), nearest first,
// each that shape's tactic for the smallest measured bin >= bin; at most
// max_out of them.  Returns how many were written.
int nearby_measured_tactics(int N, int K, int bin, proj_tactic_t *out, int max_out);

}  // namespace tp1
