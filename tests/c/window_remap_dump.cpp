// Host-side dump of the paged first step's window-relink rule (window_remap
// in the library's internal header) for the H2O schedule with a proportional
// budget, so a CPU test can check its invariants.  Reads lines
// "t n_att e n_sink budget_num budget_den" and prints
// "ok front src m" (ok 0: plain compaction; the other fields are then 0).
#include <cstdio>

#include "h2o_internal.h"

int main()
{
    int t, n_att, e, n_sink, num, den;
    while (std::scanf("%d %d %d %d %d %d", &t, &n_att, &e, &n_sink, &num, &den) == 6) {
        h2o::Sched s{};
        s.selector = h2o::kSelH2O;
        s.n_sink = n_sink;
        s.budget_num = num;
        s.budget_den = den;
        h2o::WindowRemap r{};
        const bool ok = h2o::window_remap(s, t, n_att, e, r);
        std::printf("%d %d %d %d\n", ok ? 1 : 0, ok ? r.front : 0, ok ? r.src : 0, ok ? r.m : 0);
    }
    return 0;
}
