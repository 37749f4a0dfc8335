// Draft-length controller of the C ABI (host only): per lane, the
// acceptance statistics of the most recent batches decide whether the next
// batch drafts one token more or one less.  Rule: page
// www.2kiu.com/news/5895634 section 4.4 (window of 100 batches, above 0.8
// lengthen, below 0.6 shorten, K within [2, 10]); the general policy is page
// www.cf-1.com/news/5155685 section 2.4.
#include "specverify.h"

#include <cstdint>
#include <new>
#include <vector>

namespace {

// One lane: a ring of the last `window` observations (accepted, drafted)
// with their exact integer totals.
struct Lane {
  std::vector<int64_t> acc, dr;  // ring storage, size window
  int64_t sum_acc = 0, sum_dr = 0;
  int32_t head = 0;   // slot of the oldest observation
  int32_t count = 0;  // observations held
  int32_t k = 0;

  void clear() {
    sum_acc = sum_dr = 0;
    head = count = 0;
  }
  void push(int64_t a, int64_t d, int32_t window) {
    if (count == window) {  // drop the oldest
      sum_acc -= acc[head];
      sum_dr -= dr[head];
      head = head + 1 == window ? 0 : head + 1;
      --count;
    }
    int32_t slot = head + count;
    if (slot >= window) slot -= window;
    acc[slot] = a;
    dr[slot] = d;
    sum_acc += a;
    sum_dr += d;
    ++count;
  }
};

}  // namespace

struct sv_dynk {
  int32_t window;
  double hi, lo;
  int32_t k_min, k_max;
  std::vector<Lane> lanes;
};

extern "C" {

sv_dynk* sv_dynk_create(int32_t lanes, int32_t window, double raise_above, double lower_below, int32_t k_min,
                        int32_t k_max, int32_t k_init) {
  if (lanes < 1 || window < 1 || k_min < 0 || k_max < k_min || k_init < k_min || k_init > k_max) return nullptr;
  if (!(0.0 <= lower_below && lower_below <= raise_above && raise_above <= 1.0)) return nullptr;
  sv_dynk* c = new (std::nothrow) sv_dynk;
  if (!c) return nullptr;
  try {
    c->window = window;
    c->hi = raise_above;
    c->lo = lower_below;
    c->k_min = k_min;
    c->k_max = k_max;
    c->lanes.resize((size_t)lanes);
    for (Lane& l : c->lanes) {
      l.acc.assign((size_t)window, 0);
      l.dr.assign((size_t)window, 0);
      l.k = k_init;
    }
  } catch (...) {
    delete c;
    return nullptr;
  }
  return c;
}

int sv_dynk_observe(sv_dynk* c, const int64_t* accepted, const int64_t* drafted, int32_t* k_next) {
  if (!c || !accepted || !drafted) return SV_ERR_NULL;
  const size_t n = c->lanes.size();
  for (size_t i = 0; i < n; ++i)
    if (!(accepted[i] >= 0 && accepted[i] <= drafted[i])) return SV_ERR_PARAM;
  for (size_t i = 0; i < n; ++i) {
    Lane& l = c->lanes[i];
    if (drafted[i] > 0) {
      l.push(accepted[i], drafted[i], c->window);
      if (l.count == c->window) {
        const double rate = (double)l.sum_acc / (double)l.sum_dr;
        if (rate > c->hi && l.k < c->k_max) {
          ++l.k;
          l.clear();
        } else if (rate < c->lo && l.k > c->k_min) {
          --l.k;
          l.clear();
        }
      }
    }
    if (k_next) k_next[i] = l.k;
  }
  return SV_OK;
}

int32_t sv_dynk_k(const sv_dynk* c, int32_t lane) {
  if (!c || lane < 0 || (size_t)lane >= c->lanes.size()) return -1;
  return c->lanes[(size_t)lane].k;
}

void sv_dynk_destroy(sv_dynk* c) { delete c; }

}  // extern "C"
