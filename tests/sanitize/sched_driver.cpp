// Randomised driver of the step planner's C ABI (include/pa_sched.h), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sched_sanitizers.py: requests of random prompts (some sharing
// prefixes) arrive, steps are planned and their inputs fetched, sampled
// tokens are fed back, requests finish early, pools run dry. Any memory or
// undefined-behaviour error ends the run with a report.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "pa_sched.h"

// The library's error recording lives in its GPU host layer; the planner
// alone needs only these two.
namespace pa {
int record_error(int code, const char*, ...) { return code; }
void clear_error() {}
}  // namespace pa

int main() {
  for (int seed = 1; seed <= 12; ++seed) {
    std::mt19937 rng(seed);
    const int NB = 20 + rng() % 80;
    pa_sched* s = pa_sched_create(NB, 16, 8 + rng() % 200, 1 + rng() % 16, (int)(rng() % 3) * 16, rng() % 2);
    std::vector<std::vector<int>> pref(3);
    for (auto& p : pref) for (int i = 0, n = 16 * (1 + rng() % 4); i < n; ++i) p.push_back(rng() % 1000);
    int added = 0, live = 0;
    for (int step = 0; step < 1500; ++step) {
      if (added < 60 && rng() % 3 == 0) {
        std::vector<int> p;
        if (rng() % 2) p = pref[rng() % 3];
        for (int i = 0, n = 1 + rng() % 50; i < n; ++i) p.push_back(rng() % 1000);
        if (pa_sched_add_request(s, added, p.data(), (int)p.size(), 1 + rng() % 20) == 0) { ++added; ++live; }
      }
      int S, T, MB;
      if (pa_sched_schedule(s, &S, &T, &MB)) { fprintf(stderr, "schedule failed seed %d step %d\n", seed, step); return 1; }
      std::vector<int64_t> ids(S), slots(T);
      std::vector<int> qsl(S + 1), lens(S), table((size_t)S * (MB + 1)), toks(T), pos(T), sampled(S);
      if (pa_sched_step_inputs(s, ids.data(), qsl.data(), lens.data(), table.data(), MB + 1, slots.data(), toks.data(), pos.data())) { fprintf(stderr, "inputs failed seed %d step %d\n", seed, step); return 1; }
      for (int i = 0; i < S; ++i) sampled[i] = rng() % 1000;
      if (S) pa_sched_update(s, sampled.data());
      if (rng() % 50 == 0 && added) pa_sched_finish_request(s, rng() % added);
      pa_sched_stats st; pa_sched_get_stats(s, &st);
      if (st.num_free_blocks > NB) { fprintf(stderr, "bad free count\n"); return 1; }
      if (!S && st.num_waiting == 0 && st.num_running == 0 && added >= 60) break;
    }
    pa_sched_destroy(s);
  }
  printf("planner driver ok\n");
  return 0;
}
