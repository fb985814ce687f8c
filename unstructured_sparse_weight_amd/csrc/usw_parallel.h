// Host-side fork-join helper shared by the encoders: f(lo, hi) over an even
// split of [0, n) on up to 16 threads.
#pragma once

#include <algorithm>
#include <cstdint>
#include <thread>
#include <vector>

namespace usw {

inline int worker_count(int64_t items) {
  unsigned hw = std::thread::hardware_concurrency();
  int n = static_cast<int>(hw ? std::min(hw, 16u) : 4u);
  if (items < n) n = static_cast<int>(std::max<int64_t>(items, 1));
  return n;
}

template <class F>
void parallel_for(int64_t n, F&& f) {
  const int nt = worker_count(n);
  if (nt <= 1) {
    f(static_cast<int64_t>(0), n);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(nt);
  for (int t = 0; t < nt; ++t) {
    const int64_t lo = n * t / nt, hi = n * (t + 1) / nt;
    th.emplace_back([&f, lo, hi] { f(lo, hi); });
  }
  for (auto& x : th) x.join();
}

}  // namespace usw
