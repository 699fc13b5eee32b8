// Host check of the workgroup placement map (test infrastructure): for every grid size up to
// 6000 and a few large ones, placed_index must be a bijection of [0, n), give each XCD
// (ids congruent mod 8) a contiguous range, and give the workgroups of each CU (local indices
// congruent mod kCUsPerXCD within an XCD) a contiguous sub-range.  Exit status 0 means it holds.
#include <cstdio>
#include <vector>
#include <algorithm>

#include "mamba_common.h"

static bool contiguous(std::vector<int64_t>& v) {
  std::sort(v.begin(), v.end());
  for (size_t i = 1; i < v.size(); ++i)
    if (v[i] != v[i - 1] + 1) return false;
  return true;
}

int main() {
  std::vector<uint32_t> sizes;
  for (uint32_t n = 1; n <= 6000; ++n) sizes.push_back(n);
  for (uint32_t n : {48u * 26, 48u * 25, 1280u * 64, 1u << 20, (1u << 20) + 13, 2147483647u / 64})
    sizes.push_back(n);
  for (uint32_t n : sizes) {
    std::vector<char> seen(n, 0);
    std::vector<std::vector<int64_t>> xcd(8), cu(8 * mamba::kCUsPerXCD);
    for (uint32_t id = 0; id < n; ++id) {
      const int64_t j = mamba::placed_index(id, n);
      if (j < 0 || j >= (int64_t)n || seen[j]) {
        std::printf("n=%u: id %u maps to %lld (out of range or taken)\n", n, id, (long long)j);
        return 1;
      }
      seen[j] = 1;
      if (n <= 6000) {
        xcd[id & 7].push_back(j);
        cu[(id & 7) * mamba::kCUsPerXCD + (id >> 3) % mamba::kCUsPerXCD].push_back(j);
      }
    }
    for (auto& v : xcd)
      if (!contiguous(v)) { std::printf("n=%u: an XCD range is not contiguous\n", n); return 1; }
    for (auto& v : cu)
      if (!contiguous(v)) { std::printf("n=%u: a CU range is not contiguous\n", n); return 1; }
  }
  std::printf("placement map: bijective and contiguous for %zu grid sizes\n", sizes.size());
  return 0;
}
