// Active-window schedule of pipelined decoding (host code; the rules and the
// passages they follow are stated with the declarations in d2f.h).
#include <cmath>
#include <cstring>

#include "d2f_internal.h"

namespace d2f {
namespace {

bool passes(int32_t committed, float tau, int32_t block_size) {
  return (double)committed > (double)tau * (double)block_size;
}

d2f_status_t check_params(const d2f_window_params_t* p) {
  if (p == nullptr) return fail(D2F_ERR_INVALID_ARG, "window params are NULL");
  if (p->block_size < 1 || p->total_blocks < 1 || p->max_win_blocks < 1 ||
      p->max_win_blocks > D2F_MAX_WINDOW)
    return fail(D2F_ERR_INVALID_ARG, "window params out of range (block %d, window %d, total %d)",
                p->block_size, p->max_win_blocks, p->total_blocks);
  if (std::isnan(p->tau_add) || std::isnan(p->tau_act))
    return fail(D2F_ERR_INVALID_ARG, "window thresholds are NaN");
  return D2F_OK;
}

}  // namespace
}  // namespace d2f

using namespace d2f;

extern "C" {

d2f_status_t d2f_window_init(const d2f_window_params_t* params, d2f_window_t* state) {
  d2f_status_t st = check_params(params);
  if (st != D2F_OK) return st;
  if (state == nullptr) return fail(D2F_ERR_INVALID_ARG, "window state is NULL");
  std::memset(state, 0, sizeof(*state));
  state->n_win = 1;
  state->started = 1;
  state->phase[0] = D2F_AGGRESSIVE;
  return D2F_OK;
}

d2f_status_t d2f_window_after_commit(const d2f_window_params_t* params, d2f_window_t* state,
                                     const int32_t* n_committed, int32_t* persisted_out,
                                     int32_t* appended_out) {
  d2f_status_t st = check_params(params);
  if (st != D2F_OK) return st;
  if (state == nullptr || persisted_out == nullptr || appended_out == nullptr)
    return fail(D2F_ERR_INVALID_ARG, "window state or outputs are NULL");
  const int32_t B = params->block_size;
  if (state->persisted >= params->total_blocks)
    return fail(D2F_ERR_INVALID_ARG, "every block was already persisted");
  if (state->n_win < 1 || state->n_win > params->max_win_blocks)
    return fail(D2F_ERR_INVALID_ARG, "window state holds %d blocks", state->n_win);
  if (n_committed == nullptr) return fail(D2F_ERR_INVALID_ARG, "n_committed is NULL");
  for (int k = 0; k < state->n_win; ++k) {
    const int64_t c = (int64_t)state->committed[k] + n_committed[k];
    if (n_committed[k] < 0 || c > B)
      return fail(D2F_ERR_INVALID_ARG, "block %d: %d committed + %d > block size %d", k,
                  state->committed[k], n_committed[k], B);
  }
  d2f_window_t w = *state;
  // 1. counts
  for (int k = 0; k < w.n_win; ++k) w.committed[k] += n_committed[k];
  // 2. persist complete blocks from the front
  int persisted = 0;
  while (persisted < w.n_win && w.committed[persisted] == B) ++persisted;
  if (persisted > 0) {
    const int left = w.n_win - persisted;
    std::memmove(w.committed, w.committed + persisted, sizeof(int32_t) * left);
    std::memmove(w.phase, w.phase + persisted, left);
    w.n_win = left;
    w.first += persisted;
    w.persisted += persisted;
  }
  // 3. append
  int appended = 0;
  if (w.started < params->total_blocks && w.n_win < params->max_win_blocks &&
      (w.n_win == 0 || passes(w.committed[w.n_win - 1], params->tau_add, B))) {
    w.committed[w.n_win] = 0;
    w.phase[w.n_win] = D2F_CONSERVATIVE;
    ++w.n_win;
    ++w.started;
    appended = 1;
  }
  // 4. phases for the next pass
  for (int k = 0; k < w.n_win; ++k)
    if (k == 0 || passes(w.committed[k - 1], params->tau_act, B)) w.phase[k] = D2F_AGGRESSIVE;
  for (int k = w.n_win; k < D2F_MAX_WINDOW; ++k) {
    w.committed[k] = 0;
    w.phase[k] = 0;
  }
  *state = w;
  *persisted_out = persisted;
  *appended_out = appended;
  return D2F_OK;
}

}  // extern "C"
