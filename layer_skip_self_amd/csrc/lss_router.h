// DyTC router of the CAS-Spec cascade, host side.
//   - EMA acceptance predictor a <- 0.2 r + 0.8 a (CAS-Spec blog, section 3.1),
//     initial value 0.65 (section 4.1 gives 0.6-0.7);
//   - latency model b0 + b1 seq_len + b2 executed_layers (section 3.2);
//   - routing / draft-length assignment from those two heuristics (CAS-Spec
//     abstract): the plan maximizes expected tokens per predicted second.
#pragma once
#include <stdint.h>

namespace router {

constexpr double kAlpha = 0.2;
constexpr double kAInit = 0.65;

double predict(const double* beta, int seq_len, int depth);
// k per level (0 = fastest), total <= k_max; see lss_router_plan in lss.h.
void plan(const double* a, const double* t_hat, int n_levels, double t_verify, int k_max, int32_t* out);
void update(double* a, int n_levels, const int32_t* slot_levels, int k, int n);
bool fit(const double* samples, int n, double* beta);
// tree routing: width and k per level of the next tree round (see
// lss_router_plan_tree in lss.h); row_cost[r - 1] scales a pass over r rows
// (nullptr: 1)
void plan_tree(const double* a, const double* t_hat, int n_levels, double t_verify, const double* row_cost,
               int k_max, int b_max, int nodes_max, int32_t* width_out, int32_t* out);
void update_tree(double* a, int n_levels, const int32_t* depth_levels, int D, int n, int branch);

}  // namespace router
