// Host-side check of the read-ahead template (int8_dequant_dot_amd/csrc/pipeline.hpp),
// compiled with the host compiler: the scheduling fence is defined away and the
// device qualifiers become plain inline.  For every depth, both drain forms and
// every loop length up to 4 * DEPTH + 5 it checks the contract the kernels rely on
// ("Tune loop unrolling and pipelining", §Separate depth from unrolling;
// "Functions and structured control flow", §Pipeline reads ahead of ordered
// computation):
//   - load() and consume() are each called exactly n times, in order, and
//     consume(i) receives the value load i returned;
//   - an empty loop issues no load;
//   - a loop shorter than DEPTH - 1 (or DEPTH <= 1) runs serially: load i is
//     issued only after consume(i - 1), so one record is in flight;
//   - otherwise exactly min(n, i + DEPTH) loads have been issued when
//     consume(i) runs: DEPTH - 1 records read ahead of the consumer in the
//     startup and steady phases, never more, and the drain issues the missing
//     loads without running further ahead.
// Prints "ok <cases>" on success, or the first violation and exits 1.
#include <cstdio>
#include <cstdlib>

#define LOOM_PIPELINE_INLINE inline
#define LOOM_SCHED_FENCE() ((void)0)
#include "pipeline.hpp"

namespace {

struct Record {
    long index;
    long check;  // a second field, so that the ring moves whole structs
};

int failures = 0;

void fail(const char *what, int depth, bool straight, long n, long i, long issued) {
    if (failures++ < 10)
        std::printf("FAIL %s: DEPTH=%d straight=%d n=%ld consume=%ld issued=%ld\n", what, depth, (int)straight, n,
                    i, issued);
}

template <int DEPTH, bool STRAIGHT>
void check(long n) {
    long issued = 0, consumed = 0;
    const bool serial = DEPTH <= 1 || n < DEPTH - 1;
    loom::pipelined<DEPTH, Record, STRAIGHT>(
        n,
        [&]() {
            Record r{issued, 1000003 * issued + 7};
            ++issued;
            return r;
        },
        [&](const Record &r) {
            const long i = consumed;
            if (r.index != i || r.check != 1000003 * i + 7) fail("out of order or wrong value", DEPTH, STRAIGHT, n, i, issued);
            const long want = serial ? i + 1 : (n < i + DEPTH ? n : i + DEPTH);
            if (issued != want) fail("read-ahead", DEPTH, STRAIGHT, n, i, issued);
            ++consumed;
        });
    if (issued != n) fail("load count", DEPTH, STRAIGHT, n, consumed, issued);
    if (consumed != n) fail("consume count", DEPTH, STRAIGHT, n, consumed, issued);
}

template <int DEPTH>
int check_depth() {
    int cases = 0;
    for (long n = 0; n <= 4 * DEPTH + 5; ++n) {
        check<DEPTH, false>(n);
        check<DEPTH, true>(n);
        cases += 2;
    }
    return cases;
}

}  // namespace

int main() {
    int cases = 0;
    cases += check_depth<1>();
    cases += check_depth<2>();
    cases += check_depth<3>();
    cases += check_depth<4>();
    cases += check_depth<5>();
    cases += check_depth<6>();
    cases += check_depth<7>();
    cases += check_depth<8>();
    cases += check_depth<16>();
    cases += check_depth<32>();
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("ok %d\n", cases);
    return 0;
}
