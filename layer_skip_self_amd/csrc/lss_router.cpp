// DyTC router (host): plan enumeration, EMA update, least-squares latency fit.
#include "lss_router.h"

#include <algorithm>
#include <cmath>
#include <vector>

namespace router {

double predict(const double* beta, int seq_len, int depth) {
  return beta[0] + beta[1] * (double)seq_len + beta[2] * (double)depth;
}

namespace {

// Expected accepted length of a window ordered most precise level first,
// each slot accepted independently with its level's rate.
double expected(const double* a, const int32_t* k, int nl) {
  double e = 0.0, prod = 1.0;
  for (int v = nl - 1; v >= 0; --v)
    for (int i = 0; i < k[v]; ++i) {
      prod *= a[v];
      e += prod;
    }
  return e;
}

double cost(const double* t_hat, double t_verify, const int32_t* k, int nl) {
  double c = t_verify;
  for (int v = nl - 1; v >= 0; --v) c += k[v] * t_hat[v];
  return c;
}

// key order: score, then smaller total, then larger k of the most precise level, ...
bool better(double s, int tot, const int32_t* k, double bs, int btot, const int32_t* bk, int nl) {
  if (s != bs) return s > bs;
  if (tot != btot) return tot < btot;
  for (int v = nl - 1; v >= 0; --v)
    if (k[v] != bk[v]) return k[v] > bk[v];
  return false;
}

}  // namespace

void plan(const double* a, const double* t_hat, int nl, double t_verify, int k_max, int32_t* out) {
  int32_t k[8] = {0}, best[8] = {0};
  double bs = -1.0;
  int btot = 0;
  bool have = false;
  // enumerate every (k[nl-1], ..., k[0]) >= 0 with total <= k_max
  struct Rec {
    static void go(int v, int used, int nl, int k_max, int32_t* k, const double* a, const double* t_hat,
                   double t_verify, int32_t* best, double& bs, int& btot, bool& have) {
      if (v < 0) {
        const double s = (expected(a, k, nl) + 1.0) / cost(t_hat, t_verify, k, nl);
        if (!have || better(s, used, k, bs, btot, best, nl)) {
          for (int i = 0; i < nl; ++i) best[i] = k[i];
          bs = s;
          btot = used;
          have = true;
        }
        return;
      }
      for (int x = 0; x <= k_max - used; ++x) {
        k[v] = x;
        go(v - 1, used + x, nl, k_max, k, a, t_hat, t_verify, best, bs, btot, have);
      }
      k[v] = 0;
    }
  };
  Rec::go(nl - 1, 0, nl, k_max, k, a, t_hat, t_verify, best, bs, btot, have);
  for (int i = 0; i < nl; ++i) out[i] = best[i];
}

void update(double* a, int nl, const int32_t* lev, int k, int n) {
  const int reached = n + 1 < k ? n + 1 : k;
  for (int v = 0; v < nl; ++v) {
    int rc = 0, ac = 0;
    for (int i = 0; i < reached; ++i) rc += lev[i] == v;
    for (int i = 0; i < n; ++i) ac += lev[i] == v;
    if (rc > 0) {
      const double r = (double)ac / (double)rc;
      a[v] = kAlpha * r + (1.0 - kAlpha) * a[v];
    }
  }
}

// ---- tree routing: the levels drafting the depths of a width-B token tree
namespace {

// first depth hit by one of B independent tries at rate a (a itself for one)
double first_hit(double a, int B) { return B == 1 ? a : 1.0 - std::pow(1.0 - a, (double)B); }

double expected_tree(const double* a, int B, const int32_t* k, int nl) {
  double e = 0.0, prod = 1.0;
  bool first = true;
  for (int v = nl - 1; v >= 0; --v)
    for (int i = 0; i < k[v]; ++i) {
      prod = first ? first_hit(a[v], B) : prod * a[v];
      first = false;
      e += prod;
    }
  return e;
}

double rc(const double* row_cost, int r) { return row_cost ? row_cost[r - 1] : 1.0; }

// verify of 1 + B D rows, the first depth's pass 1 row, later depths B rows
// (per level in window order, as the chain's cost)
double tree_cost(const double* t_hat, double t_verify, const double* row_cost, int B, const int32_t* k, int nl) {
  int D = 0;
  for (int v = 0; v < nl; ++v) D += k[v];
  double c = t_verify * rc(row_cost, 1 + B * D);
  bool first = true;
  for (int v = nl - 1; v >= 0; --v) {
    if (k[v] == 0) continue;
    const int f = first ? 1 : 0;
    first = false;
    const double w = (double)f * rc(row_cost, 1) + (double)(k[v] - f) * rc(row_cost, B);
    c += w * t_hat[v];
  }
  return c;
}

}  // namespace

void plan_tree(const double* a, const double* t_hat, int nl, double t_verify, const double* row_cost, int k_max,
               int b_max, int nodes_max, int32_t* width_out, int32_t* out) {
  int32_t k[8] = {0}, best[8] = {0};
  double bs = -1.0;
  int btot = 0, bB = 1;
  bool have = false;
  for (int B = 1; B <= b_max; ++B) {
    const int dmax = std::min(k_max, nodes_max / B);
    // enumerate (k[nl-1], ..., k[0]) >= 0 with total <= dmax; key: score,
    // fewer nodes, smaller width, then the chain's order
    struct Rec {
      static void go(int v, int used, int nl, int dmax, int B, int32_t* k, const double* a, const double* t_hat,
                     double t_verify, const double* row_cost, int32_t* best, double& bs, int& btot, int& bB,
                     bool& have) {
        if (v < 0) {
          const double s = (expected_tree(a, B, k, nl) + 1.0) / tree_cost(t_hat, t_verify, row_cost, B, k, nl);
          bool take = !have;
          if (!take) {
            if (s != bs) take = s > bs;
            else if (B * used != bB * btot) take = B * used < bB * btot;
            else if (B != bB) take = B < bB;
            else
              for (int i = nl - 1; i >= 0; --i)
                if (k[i] != best[i]) {
                  take = k[i] > best[i];
                  break;
                }
          }
          if (take) {
            for (int i = 0; i < nl; ++i) best[i] = k[i];
            bs = s;
            btot = used;
            bB = B;
            have = true;
          }
          return;
        }
        for (int x = 0; x <= dmax - used; ++x) {
          k[v] = x;
          go(v - 1, used + x, nl, dmax, B, k, a, t_hat, t_verify, row_cost, best, bs, btot, bB, have);
        }
        k[v] = 0;
      }
    };
    Rec::go(nl - 1, 0, nl, dmax, B, k, a, t_hat, t_verify, row_cost, best, bs, btot, bB, have);
  }
  for (int i = 0; i < nl; ++i) out[i] = best[i];
  *width_out = bB;
}

void update_tree(double* a, int nl, const int32_t* lev, int D, int n, int branch) {
  const bool top1 = n >= 1 && branch == 0;
  const int reached = n + 1 < D ? n + 1 : D;
  const int acc = n < D ? n : D;
  for (int v = 0; v < nl; ++v) {
    int rcnt = 0, acnt = 0;
    for (int i = 0; i < reached; ++i) rcnt += lev[i] == v;
    for (int i = 0; i < acc; ++i) acnt += lev[i] == v && (i > 0 || top1);
    if (rcnt > 0) {
      const double r = (double)acnt / (double)rcnt;
      a[v] = kAlpha * r + (1.0 - kAlpha) * a[v];
    }
  }
}

bool fit(const double* s, int n, double* beta) {
  // normal equations (A^T A) b = A^T y with rows (1, seq_len, depth)
  double m[3][4] = {{0}};
  for (int i = 0; i < n; ++i) {
    const double x[3] = {1.0, s[i * 3 + 0], s[i * 3 + 1]};
    const double y = s[i * 3 + 2];
    for (int r = 0; r < 3; ++r) {
      for (int c = 0; c < 3; ++c) m[r][c] += x[r] * x[c];
      m[r][3] += x[r] * y;
    }
  }
  // Gaussian elimination with partial pivoting
  for (int c = 0; c < 3; ++c) {
    int p = c;
    for (int r = c + 1; r < 3; ++r)
      if (std::fabs(m[r][c]) > std::fabs(m[p][c])) p = r;
    if (std::fabs(m[p][c]) < 1e-300) return false;
    if (p != c)
      for (int j = 0; j < 4; ++j) std::swap(m[p][j], m[c][j]);
    for (int r = 0; r < 3; ++r) {
      if (r == c) continue;
      const double f = m[r][c] / m[c][c];
      for (int j = c; j < 4; ++j) m[r][j] -= f * m[c][j];
    }
  }
  for (int c = 0; c < 3; ++c) beta[c] = m[c][3] / m[c][c];
  return true;
}

}  // namespace router
