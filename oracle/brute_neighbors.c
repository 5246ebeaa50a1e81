/*
 * Brute-force O(N^2) neighbour search in fp64 -- part of the oracle.
 *
 * TEST INFRASTRUCTURE ONLY: linked by oracle/layer.py through ctypes; nothing
 * in the product path loads it.
 *
 * Definition (E2Former-V2 explainer, section 5.2 asks that the neighbour list
 * be verified; section 3.2 caps it with masked padding): for a target i, the
 * neighbour set is every j != i with d2 < rc2, where
 *     dx = (double)x_j - (double)x_i   (likewise dy, dz)
 *     d2 = (dx*dx + dy*dy) + dz*dz
 * evaluated left to right with every product and sum rounded separately.
 * Build with -ffp-contract=off so no fused multiply-add changes a rounding.
 *
 * Two passes: count for a list of targets, then fill rows at caller-given
 * offsets (unsorted; the caller sorts and applies any cap).
 */
#include <stdint.h>

static double pair_d2(const float *pos, int64_t i, int64_t j)
{
    double dx = (double)pos[3 * j + 0] - (double)pos[3 * i + 0];
    double dy = (double)pos[3 * j + 1] - (double)pos[3 * i + 1];
    double dz = (double)pos[3 * j + 2] - (double)pos[3 * i + 2];
    double xx = dx * dx;
    double yy = dy * dy;
    double zz = dz * dz;
    double s = xx + yy;
    return s + zz;
}

/* counts[t] = |N(targets[t])| (uncapped); returns the total. */
int64_t oracle_nbr_count(const float *pos, int32_t n, const int32_t *targets, int32_t nt,
                         double rc2, int64_t *counts)
{
    int64_t total = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : total)
    for (int32_t t = 0; t < nt; ++t) {
        int64_t i = targets[t];
        int64_t c = 0;
        for (int64_t j = 0; j < n; ++j) {
            if (j == i)
                continue;
            if (pair_d2(pos, i, j) < rc2)
                ++c;
        }
        counts[t] = c;
        total += c;
    }
    return total;
}

/* Row t is written at idx[offsets[t] ..] in increasing j, with its d2 values. */
void oracle_nbr_fill(const float *pos, int32_t n, const int32_t *targets, int32_t nt,
                     double rc2, const int64_t *offsets, int32_t *idx, double *d2)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int32_t t = 0; t < nt; ++t) {
        int64_t i = targets[t];
        int64_t o = offsets[t];
        for (int64_t j = 0; j < n; ++j) {
            if (j == i)
                continue;
            double v = pair_d2(pos, i, j);
            if (v < rc2) {
                idx[o] = (int32_t)j;
                d2[o] = v;
                ++o;
            }
        }
    }
}
