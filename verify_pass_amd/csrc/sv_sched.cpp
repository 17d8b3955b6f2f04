// Iteration-level batching of a swarm of sequences (host only).
//
// "Why Static Batching Wastes an RX 9070 XT Agent Swarm and Continuous
// Batching Wins It Back": a step over B sequences pays one shared weight
// stream, so lanes that finished but still ride the step ("What a draining
// batch actually costs") waste it; iteration-level scheduling ("Continuous
// batching refills the slot instead of freezing it") decides membership every
// step and gives a finished sequence's slot to a waiting one on the very next
// step.  The scheduler only decides which requests occupy which lanes; the
// verify pass itself is unchanged.
//
// Requests are served in submission order.  Policies:
//   static      a batch takes the next `slots` waiting requests when every
//               lane is free and keeps all its lanes (finished ones as
//               padding) until every member is done;
//   shrink      the same batches, a finished member leaving at once;
//   continuous  every step, each free lane takes the next waiting request.
#include <cstdint>
#include <new>
#include <vector>

#include "../../include/sv.h"

struct sv_sched {
  int slots = 0, policy = 0;
  std::vector<int> lane;    // request per lane, -1 empty
  std::vector<long long> left;  // tokens the lane's request still needs
  std::vector<long long> queue; // tokens of every submitted request
  size_t next = 0;          // next waiting request
  bool stepped = false;     // next() called since the last commit()
};

extern "C" sv_status sv_sched_create(int32_t slots, int32_t policy, sv_sched **out) {
  if (!out || slots <= 0 || policy < SV_SCHED_STATIC || policy > SV_SCHED_CONTINUOUS) return SV_ERR_INVALID_ARG;
  sv_sched *s = new (std::nothrow) sv_sched;
  if (!s) return SV_ERR_INVALID_ARG;
  s->slots = slots;
  s->policy = policy;
  s->lane.assign(slots, -1);
  s->left.assign(slots, 0);
  *out = s;
  return SV_OK;
}

extern "C" sv_status sv_sched_destroy(sv_sched *s) {
  delete s;
  return SV_OK;
}

extern "C" sv_status sv_sched_submit(sv_sched *s, int32_t tokens, int32_t *request_out) {
  if (!s || tokens <= 0 || s->queue.size() >= 0x7FFFFFFF) return SV_ERR_INVALID_ARG;
  if (request_out) *request_out = (int32_t)s->queue.size();
  s->queue.push_back(tokens);
  return SV_OK;
}

extern "C" sv_status sv_sched_next(sv_sched *s, int32_t *slot_request, int32_t *live, int32_t *width) {
  if (!s || !slot_request || !live || !width) return SV_ERR_INVALID_ARG;
  const int n = s->slots;
  auto take = [&](int k) {
    s->lane[k] = (int)s->next;
    s->left[k] = s->queue[s->next];
    ++s->next;
  };
  if (s->policy == SV_SCHED_CONTINUOUS) {
    for (int k = 0; k < n; ++k) {
      const bool free_lane = s->lane[k] < 0 || s->left[k] == 0;
      if (free_lane && s->next < s->queue.size()) take(k);
      else if (free_lane) s->lane[k] = -1;
    }
  } else {
    bool all_done = true;
    for (int k = 0; k < n; ++k)
      if (s->lane[k] >= 0 && s->left[k] > 0) all_done = false;
    if (all_done) {
      for (int k = 0; k < n; ++k) {
        s->lane[k] = -1;
        s->left[k] = 0;
        if (s->next < s->queue.size()) take(k);
      }
    }
    if (s->policy == SV_SCHED_SHRINK)
      for (int k = 0; k < n; ++k)
        if (s->lane[k] >= 0 && s->left[k] == 0) s->lane[k] = -1;
  }
  int w = 0, any = 0;
  for (int k = 0; k < n; ++k) {
    slot_request[k] = s->lane[k];
    live[k] = (s->lane[k] >= 0 && s->left[k] > 0) ? 1 : 0;
    any |= live[k];
    w += s->lane[k] >= 0 ? 1 : 0;
  }
  *width = any ? w : 0;
  s->stepped = any != 0;
  return SV_OK;
}

extern "C" sv_status sv_sched_commit(sv_sched *s, const int32_t *emitted, int32_t *useful_out) {
  if (!s || !emitted) return SV_ERR_INVALID_ARG;
  if (!s->stepped) return SV_ERR_INVALID_ARG;  // commit follows a step with live lanes
  long long useful = 0;
  for (int k = 0; k < s->slots; ++k) {
    if (s->lane[k] < 0 || s->left[k] == 0) continue;
    if (emitted[k] < 0) return SV_ERR_INVALID_ARG;
    const long long t = emitted[k] < s->left[k] ? emitted[k] : s->left[k];
    s->left[k] -= t;
    useful += t;
  }
  if (useful_out) *useful_out = (int32_t)useful;
  s->stepped = false;
  return SV_OK;
}
