// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches) and keeping the median
// fastest; ties within 1% go to fewer launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc}}.
#include "tactics_table.hpp"

namespace tp1 {

namespace {
struct Entry {
    int N, K, bin;
    proj_tactic_t t;
};

const Entry kTable[] = {
    {0, 0, 0, {0, 0, 0, 0, 0, 0}},  // sentinel (no measured rows yet)
};
}  // namespace

bool lookup_measured_tactic(int N, int K, int bin, proj_tactic_t *out) {
    for (const Entry &e : kTable) {
        if (e.N == N && e.K == K && e.bin == bin && e.t.kernel != 0) {
            *out = e.t;
            return true;
        }
    }
    return false;
}

}  // namespace tp1
