// Test driver for the library's host planning code (host_plan.cpp), built on
// its own so that it can run under the address and undefined-behaviour
// sanitizers. Reads cases from stdin, one per line:
//   P E G nodes gpus phys hier load_0 .. load_{E-1}   -> "P n p2l... | offsets... | slots..."
//   C tk num den E                                     -> "C value"
#include <cstdio>
#include <vector>

#include "host_plan.h"

int main() {
  char kind;
  while (std::scanf(" %c", &kind) == 1) {
    if (kind == 'P') {
      int E, G, nodes, gpus, phys, hier;
      if (std::scanf("%d %d %d %d %d %d", &E, &G, &nodes, &gpus, &phys, &hier) != 6) return 2;
      std::vector<double> load(E);
      for (int e = 0; e < E; ++e)
        if (std::scanf("%lf", &load[e]) != 1) return 2;
      std::vector<int> p2l(phys, -1), offs(E + 1, -1), slots(phys, -1);
      const int n = moe::eplb_place(load.data(), E, G, nodes, gpus, phys, hier != 0, p2l.data(), offs.data(),
                                    slots.data());
      std::printf("P %d", n);
      for (int v : p2l) std::printf(" %d", v);
      std::printf(" |");
      for (int v : offs) std::printf(" %d", v);
      std::printf(" |");
      for (int v : slots) std::printf(" %d", v);
      std::printf("\n");
    } else if (kind == 'C') {
      long long tk, num, den, E;
      if (std::scanf("%lld %lld %lld %lld", &tk, &num, &den, &E) != 4) return 2;
      std::printf("C %lld\n", (long long)moe::expert_capacity(tk, num, den, E));
    } else {
      return 2;
    }
  }
  return 0;
}
