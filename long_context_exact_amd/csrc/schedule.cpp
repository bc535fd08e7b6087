// Chunk-pair schedules of P workers over P contiguous token chunks
// ([DistFlashAttn §3.1]: worker w holds chunk w).  Host-only, no HIP.
//
// Unbalanced (§3.2; App. B, Fig. 5): at step t every worker w >= t attends
// its own queries to chunk w - t; workers w < t idle.  P steps.
//
// Token-level load balanced (§1, §3.2 and Fig. 3; App. B, Fig. 6): the
// workers that the unbalanced ring leaves idle take the latest tokens'
// work.  Step 0: diagonal pairs (w, w).  Step t in 1..P/2: worker w >= t
// does (w, w - t) for itself; worker h < t does (h + P - t, h) — the pair
// of owner h + P - t against the helper's own key/value chunk — and
// returns the partial (O, LSE) to that owner, except when P - t == t (that
// pair is already an owner pair of this step).  Every causal pair appears
// once, in 1 + floor(P/2) steps.
#include <stdint.h>

#include <string>

#include "dfa.h"
#include "errors.hpp"

extern "C" dfa_status dfa_balanced_schedule(int32_t num_workers, int32_t balanced,
                                            dfa_work_item* items, int64_t capacity,
                                            int64_t* num_items, int32_t* num_steps) {
  using dfa::fail;
  if (num_items == nullptr || num_steps == nullptr)
    return fail(DFA_ERR_INVALID, "dfa_balanced_schedule: num_items and num_steps must be non-null");
  if (num_workers < 1 || num_workers > 65536)
    return fail(DFA_ERR_INVALID, "dfa_balanced_schedule: num_workers must be in [1, 65536], got " +
                                     std::to_string(num_workers));
  if (balanced != 0 && balanced != 1)
    return fail(DFA_ERR_INVALID, "dfa_balanced_schedule: balanced must be 0 or 1");
  if (capacity < 0 || (items == nullptr && capacity > 0))
    return fail(DFA_ERR_INVALID, "dfa_balanced_schedule: bad capacity / items");
  const int64_t p = num_workers;
  const int64_t total = p * (p + 1) / 2;
  const int32_t steps = balanced ? int32_t(1 + p / 2) : int32_t(p);
  *num_items = total;
  *num_steps = steps;
  if (capacity < total)
    return fail(DFA_ERR_CAPACITY, "dfa_balanced_schedule: capacity " + std::to_string(capacity) +
                                      " < required " + std::to_string(total));
  int64_t n = 0;
  for (int32_t t = 0; t < steps; ++t) {
    for (int32_t w = 0; w < num_workers; ++w) {
      dfa_work_item it{};
      if (t == 0) {
        it = {0, w, w, w, 0, w};
      } else if (w >= t) {
        it = {t, w, w, w - t, 1, w};
      } else if (balanced && num_workers - t > t) {
        const int32_t owner = w + num_workers - t;
        it = {t, w, owner, w, 1, owner};
      } else {
        continue;  // idle slot
      }
      items[n++] = it;
    }
  }
  return n == total ? DFA_OK : fail(DFA_ERR_INVALID, "dfa_balanced_schedule: internal count");
}

// Local sliding window (App. F, discussion of sparse attention): a query
// sees only the `window` tokens ending at itself, so the work per worker is
// already nearly even; each worker keeps its query chunk and loops only over
// the key/value chunks that hold keys inside some window of its queries.
// The pair (w, w - t), t >= 1, has its closest tokens (t - 1) * C + 1 apart
// and its farthest (t + 1) * C - 1 apart.
extern "C" dfa_status dfa_window_schedule(int32_t num_workers, int64_t chunk_len, int64_t window,
                                          dfa_work_item* items, int64_t capacity,
                                          int64_t* num_items, int32_t* num_steps) {
  using dfa::fail;
  const std::string fn = "dfa_window_schedule";
  if (num_items == nullptr || num_steps == nullptr)
    return fail(DFA_ERR_INVALID, fn + ": num_items and num_steps must be non-null");
  if (num_workers < 1 || num_workers > 65536)
    return fail(DFA_ERR_INVALID, fn + ": num_workers must be in [1, 65536], got " +
                                     std::to_string(num_workers));
  if (chunk_len < 1 || window < 1)
    return fail(DFA_ERR_INVALID, fn + ": chunk_len and window must be >= 1");
  if (capacity < 0 || (items == nullptr && capacity > 0))
    return fail(DFA_ERR_INVALID, fn + ": bad capacity / items");
  const int64_t p = num_workers;
  // steps: t = 0 plus every t >= 1 with (t - 1) * C + 1 < window, t < P
  int64_t steps = 1;
  while (steps < p && (steps - 1) * chunk_len + 1 < window) ++steps;
  int64_t total = 0;
  for (int64_t t = 0; t < steps; ++t) total += p - t;
  *num_items = total;
  *num_steps = int32_t(steps);
  if (capacity < total)
    return fail(DFA_ERR_CAPACITY, fn + ": capacity " + std::to_string(capacity) +
                                      " < required " + std::to_string(total));
  int64_t n = 0;
  for (int64_t t = 0; t < steps; ++t) {
    // farthest pair (t + 1) * C - 1 apart: inside the window -> full pair
    const int32_t kind = t == 0 ? 0 : ((t + 1) * chunk_len - 1 < window ? 1 : 2);
    for (int64_t w = t; w < p; ++w)
      items[n++] = {int32_t(t), int32_t(w), int32_t(w), int32_t(w - t), kind, int32_t(w)};
  }
  return DFA_OK;
}

extern "C" dfa_status dfa_global_window_schedule(int32_t num_workers, int64_t chunk_len,
                                                 int64_t window, int64_t n_global,
                                                 dfa_work_item* items, int64_t capacity,
                                                 int64_t* num_items, int32_t* num_steps) {
  using dfa::fail;
  const std::string fn = "dfa_global_window_schedule";
  if (num_items == nullptr || num_steps == nullptr)
    return fail(DFA_ERR_INVALID, fn + ": num_items and num_steps must be non-null");
  if (num_workers < 1 || num_workers > 65536)
    return fail(DFA_ERR_INVALID, fn + ": num_workers must be in [1, 65536], got " +
                                     std::to_string(num_workers));
  if (chunk_len < 1 || window < 1)
    return fail(DFA_ERR_INVALID, fn + ": chunk_len and window must be >= 1");
  if (n_global < 1 || n_global > chunk_len)
    return fail(DFA_ERR_INVALID, fn + ": n_global must be in [1, chunk_len], got " +
                                     std::to_string(n_global));
  if (capacity < 0 || (items == nullptr && capacity > 0))
    return fail(DFA_ERR_INVALID, fn + ": bad capacity / items");
  const int64_t p = num_workers;
  int64_t steps = 1;  // as in the window schedule
  while (steps < p && (steps - 1) * chunk_len + 1 < window) ++steps;
  // a pair over chunk 0 keeps keys n_global..C-1; none is left when n_global = C
  const bool drop0 = n_global == chunk_len;
  int64_t total = p;  // one global item per worker
  for (int64_t t = 0; t < steps; ++t) total += (p - t) - (drop0 ? 1 : 0);
  *num_items = total;
  *num_steps = int32_t(steps);
  if (capacity < total)
    return fail(DFA_ERR_CAPACITY, fn + ": capacity " + std::to_string(capacity) +
                                      " < required " + std::to_string(total));
  int64_t n = 0;
  for (int64_t t = 0; t < steps; ++t) {
    const int32_t kind = t == 0 ? 0 : ((t + 1) * chunk_len - 1 < window ? 1 : 2);
    for (int64_t w = t; w < p; ++w) {
      if (t == 0)  // the worker's global item comes first (kv chunk -1)
        items[n++] = {0, int32_t(w), int32_t(w), -1, 3, int32_t(w)};
      if (drop0 && w - t == 0) continue;
      items[n++] = {int32_t(t), int32_t(w), int32_t(w), int32_t(w - t), kind, int32_t(w)};
    }
  }
  return DFA_OK;
}
