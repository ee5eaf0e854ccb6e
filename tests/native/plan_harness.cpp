// Test harness for the host planner built on its own (with the address and
// undefined-behaviour sanitizers by tests/test_host_sanitizers.py): reads
// one case per line, "num_cus batch kv_indptr[0] ... kv_indptr[batch]", and
// prints the plan words, the workspace bytes the plan needs and the
// workspace bound for its sizes, or the planner's error.
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "mla_internal.h"

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    if (line.empty()) continue;
    std::istringstream in(line);
    long long cus = 0, batch = 0;
    in >> cus >> batch;
    std::vector<int32_t> ind;
    long long v;
    while (in >> v) ind.push_back((int32_t)v);
    if ((long long)ind.size() != batch + 1) {
      std::printf("bad-case\n");
      continue;
    }
    mla::PlanResult p;
    std::string err;
    const int st = mla::build_plan(ind.data(), (int32_t)batch, (int32_t)cus, &p, &err);
    if (st != MLA_OK) {
      std::printf("error %d\n", st);
      continue;
    }
    const size_t bound = mla::workspace_bound((int32_t)batch, (int64_t)ind[batch] - ind[0], (int32_t)cus);
    std::printf("need %zu bound %zu words", p.workspace_bytes, bound);
    for (int32_t w : p.words) std::printf(" %d", (int)w);
    std::printf("\n");
  }
  return 0;
}
