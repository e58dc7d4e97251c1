// Goodput step selection (xLLM docs, "Adaptive speculative inference",
// section "Adaptive draft step (MTP)" and its policy options): host code
// that turns completed verification results into the step count of the
// next decode batch. Before a batch is submitted one step count s is chosen
// for the whole batch, the one maximising B * (1 + sum of the first s
// per-position prefix acceptances) / cost_ms(s); the acceptances are counted
// over a window of completed batches, the candidates are re-scored every
// update_interval batches, and the step changes only when the predicted
// relative gain is strictly above switch_min_gain.
//
// Rules the page leaves open: candidates are 1 .. max_steps and the
// controller starts at max_steps; prefix acceptance j is the share, among
// the window's requests that verified at least j + 1 drafts, of those that
// accepted at least j + 1; a position no request in the window verified
// keeps its last estimate (0 before any); estimates are refreshed after
// every observed batch; equal scores go to the smaller step count.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "vspec_verify.h"

namespace {

double score(const double* est, const double* cost, int s, int32_t B) {
  double total = 1.0;
  for (int j = 0; j < s; ++j) total += est[j];
  return static_cast<double>(B) * total / cost[s - 1];
}

int32_t select_step(const double* est, const double* cost, int32_t S, int32_t B, int32_t current, double min_gain) {
  int32_t best = 1;
  double best_score = score(est, cost, 1, B);
  for (int s = 2; s <= S; ++s) {
    const double v = score(est, cost, s, B);
    if (v > best_score) {
      best = s;
      best_score = v;
    }
  }
  if (best != current && best_score > (1.0 + min_gain) * score(est, cost, current, B)) return best;
  return current;
}

bool costs_ok(const double* cost, int32_t S) {
  if (!cost) return false;
  for (int s = 0; s < S; ++s)
    if (!(cost[s] > 0.0) || !isfinite(cost[s])) return false;
  return true;
}

}  // namespace

extern "C" {

vsv_status vsv_goodput_init(vsv_goodput* g, int32_t max_steps, int32_t window_size, int32_t update_interval,
                            double switch_min_gain) {
  if (!g || max_steps < 1 || max_steps > VSV_GOODPUT_MAX_STEPS || window_size < 1 ||
      window_size > VSV_GOODPUT_MAX_WINDOW || update_interval < 1 || !isfinite(switch_min_gain))
    return VSV_EINVAL;
  memset(g, 0, sizeof(*g));
  g->max_steps = max_steps;
  g->window_size = window_size;
  g->update_interval = update_interval;
  g->switch_min_gain = switch_min_gain;
  g->current = max_steps;
  return VSV_OK;
}

vsv_status vsv_goodput_observe(vsv_goodput* g, const int32_t* accepted_len, const int32_t* verify_len,
                               int32_t num_requests) {
  if (!g || g->max_steps < 1 || g->max_steps > VSV_GOODPUT_MAX_STEPS || g->window_size < 1 ||
      g->window_size > VSV_GOODPUT_MAX_WINDOW || num_requests < 0)
    return VSV_EINVAL;
  if (num_requests > 0 && (!accepted_len || !verify_len)) return VSV_EINVAL;
  for (int32_t i = 0; i < num_requests; ++i)
    if (verify_len[i] < 0 || accepted_len[i] < 0 || accepted_len[i] > verify_len[i]) return VSV_EINVAL;
  const int S = g->max_steps;
  int32_t* reached = g->reached[g->head];
  int32_t* accepted = g->accepted[g->head];
  for (int j = 0; j < S; ++j) reached[j] = accepted[j] = 0;
  for (int32_t i = 0; i < num_requests; ++i) {
    const int k = verify_len[i] < S ? verify_len[i] : S;
    const int a = accepted_len[i] < S ? accepted_len[i] : S;
    for (int j = 0; j < k; ++j) ++reached[j];
    for (int j = 0; j < a; ++j) ++accepted[j];
  }
  g->head = (g->head + 1) % g->window_size;
  if (g->filled < g->window_size) ++g->filled;
  for (int j = 0; j < S; ++j) {
    int64_t r = 0, acc = 0;
    for (int b = 0; b < g->filled; ++b) {
      r += g->reached[b][j];
      acc += g->accepted[b][j];
    }
    if (r > 0) g->estimate[j] = static_cast<double>(acc) / static_cast<double>(r);
  }
  ++g->since;
  return VSV_OK;
}

vsv_status vsv_goodput_step(vsv_goodput* g, const double* cost_ms, int32_t batch_size, int32_t* step) {
  if (!g || !step || g->max_steps < 1 || g->max_steps > VSV_GOODPUT_MAX_STEPS || batch_size < 0 ||
      g->current < 1 || g->current > g->max_steps)
    return VSV_EINVAL;
  if (!costs_ok(cost_ms, g->max_steps)) return VSV_EINVAL;
  if (g->since >= g->update_interval) {
    g->current = select_step(g->estimate, cost_ms, g->max_steps, batch_size, g->current, g->switch_min_gain);
    g->since = 0;
  }
  *step = g->current;
  return VSV_OK;
}

int32_t vsv_goodput_select(const double* prefix_acceptance, const double* cost_ms, int32_t max_steps,
                           int32_t batch_size, int32_t current, double switch_min_gain) {
  if (!prefix_acceptance || max_steps < 1 || current < 1 || current > max_steps || batch_size < 0 ||
      !costs_ok(cost_ms, max_steps) || !isfinite(switch_min_gain))
    return -1;
  return select_step(prefix_acceptance, cost_ms, max_steps, batch_size, current, switch_min_gain);
}

}  // extern "C"
