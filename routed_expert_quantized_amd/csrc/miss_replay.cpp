// miss_replay.cpp — replay of the expert-cache miss policies over a sequence of
// routings (host code; the per-layer cache state of a streaming MoE engine).
//
// "Which Expert Misses Are Worth Waiting For? Substitution and Caching for
// Mixture-of-Experts Inference on a Consumer GPU" (gist.science): section 手法
// (method) defines the substituted gate mass m, the fetch-all, 0.15-rule and
// first-choice policies and background admission at an accumulated substituted
// mass; section 主な貢献と知見 (findings), item 5, pairs them with frequency-based
// eviction and beta = 0.5. Where the page is silent: one cache of `capacity`
// slots, initially empty; frequency counts every selection of an expert, counted
// for a token's k selections before its slots are decided; an admission into a
// full cache evicts the lowest frequency (lower id on ties) among the experts the
// current token did not select; slots are decided in slot order, a synchronous
// fetch is resident at once, background admissions follow in slot order, and any
// admission resets the expert's accumulator.
#include <cstdint>
#include <set>
#include <utility>
#include <vector>

#include "moe.h"

namespace moe {

namespace {

class ExpertCache {
 public:
  ExpertCache(int E, int capacity) : resident_(E, 0), freq_(E, 0), acc_(E, 0.0), capacity_(capacity) {}

  bool resident(int e) const { return resident_[e] != 0; }

  void count(int e) {
    if (resident_[e]) by_freq_.erase({freq_[e], e});
    ++freq_[e];
    if (resident_[e]) by_freq_.insert({freq_[e], e});
  }

  // admit e, evicting the lowest-frequency resident not in chosen[0..k)
  void admit(int e, const int32_t* chosen, int k) {
    if ((int)by_freq_.size() >= capacity_) {
      for (auto it = by_freq_.begin(); it != by_freq_.end(); ++it) {
        bool busy = false;
        for (int j = 0; j < k; ++j) busy |= chosen[j] == it->second;
        if (!busy) {
          resident_[it->second] = 0;
          by_freq_.erase(it);
          break;
        }
      }
    }
    resident_[e] = 1;
    by_freq_.insert({freq_[e], e});
    acc_[e] = 0.0;
  }

  // background admission: add g to e's substituted mass; admit at >= beta
  bool accumulate(int e, double g, double beta, const int32_t* chosen, int k) {
    acc_[e] += g;
    if (acc_[e] < beta) return false;
    admit(e, chosen, k);
    return true;
  }

  const std::vector<uint8_t>& flags() const { return resident_; }

 private:
  std::vector<uint8_t> resident_;
  std::vector<int64_t> freq_;
  std::vector<double> acc_;
  std::set<std::pair<int64_t, int>> by_freq_;  // residents by (frequency, id)
  int capacity_;
};

}  // namespace

void miss_replay(const int32_t* idx, const float* gate, int T, int k, int E, int capacity, int policy,
                 float threshold, float beta, float* m, int32_t* sync, int32_t* bg, uint8_t* resident) {
  ExpertCache cache(E, capacity);
  std::vector<std::pair<int, double>> substituted;
  substituted.reserve(k);
  for (int t = 0; t < T; ++t) {
    const int32_t* id = idx + (int64_t)t * k;
    const float* g = gate + (int64_t)t * k;
    for (int s = 0; s < k; ++s) cache.count(id[s]);
    double mass = 0.0;
    int fetched = 0, admitted = 0;
    substituted.clear();
    for (int s = 0; s < k; ++s) {
      const int e = id[s];
      if (cache.resident(e)) continue;
      const bool fetch = policy == MOE_MISS_FETCH_ALL ||
                         (policy == MOE_MISS_RULE && (s == 0 || (double)g[s] >= (double)threshold)) ||
                         (policy == MOE_MISS_FIRST_CHOICE && s == 0);
      if (fetch) {
        cache.admit(e, id, k);
        ++fetched;
      } else {
        mass += (double)g[s];
        substituted.push_back({e, (double)g[s]});
      }
    }
    if (beta > 0.0f)
      for (const auto& sg : substituted) admitted += cache.accumulate(sg.first, sg.second, (double)beta, id, k);
    m[t] = (float)mass;
    sync[t] = fetched;
    bg[t] = admitted;
  }
  if (resident)
    for (int e = 0; e < E; ++e) resident[e] = cache.flags()[e];
}

}  // namespace moe
