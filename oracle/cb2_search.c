/* Brute-force CB2 codebook search for the fp64 oracle.
 *
 * TEST INFRASTRUCTURE ONLY: built into oracle/_cb2_search.so and called by
 * oracle/qmoe_oracle.py; never linked into the product library.
 *
 * For each group g of 8 weights, the error of codebook entry e is
 *   err(e) = sum over j = 0..7 (in that order) of (|w_j| - s_g * mag[e][j])^2
 * with mag = |T| / 4, every step rounded in fp64 (built with
 * -ffp-contract=off so no fused multiply-add changes a rounding).  The chosen
 * entry is the lowest e with the smallest error.  This is the same loop as
 * cb2_search_numpy, written out in C so that full-size matrices finish in
 * seconds instead of minutes.
 */
#include <stdint.h>

void cb2_search(int64_t n_groups, const double* absw, const double* scale,
                const double* mag, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < n_groups; ++g) {
    const double* a = absw + g * 8;
    const double s = scale[g];
    double best = 0.0;
    int best_e = 0;
    for (int e = 0; e < 256; ++e) {
      double err = 0.0;
      for (int j = 0; j < 8; ++j) {
        double d = a[j] - s * mag[e * 8 + j];
        err = err + d * d;
      }
      if (e == 0 || err < best) {
        best = err;
        best_e = e;
      }
    }
    out[g] = (uint8_t)best_e;
  }
}
