// Helpers shared by the oracle's translation units (oracle only).
#ifndef DSPARK_ORACLE_INTERNAL_H
#define DSPARK_ORACLE_INTERNAL_H
#include <stdint.h>
#include <vector>

double orc_internal_widen(int dt, const void *src, int64_t i);
const void *orc_internal_row(int dt, const void *base, int64_t row, int64_t len);
std::vector<double> orc_internal_softmax(const std::vector<double> &z);
void orc_internal_stats(const std::vector<double> &z, double *m, double *S);
std::vector<double> orc_internal_scaled_row(int V, int dt, double temp, const void *row);

// Draft logits of one position: z_v = (U_k(v) + sum_i W1[prev, i] W2[i, v]) / T.
std::vector<double> orc_internal_draft_logits(int V, int r, int dt, double temp,
                                              const void *U_row, const void *W1,
                                              const void *W2, int prev);
#endif
