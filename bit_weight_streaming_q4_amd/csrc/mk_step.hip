// mk_step.hip — persistent single-launch decode step (layer loop, lm_head,
// verification and Gated DeltaNet commit in one cooperative launch).
#include <hip/hip_runtime.h>

#include "mk.h"
#include "mk_internal.h"

struct mk_stack {
  int dummy;
};

extern "C" {
int mk_stack_create(const mk_stack_desc* desc, mk_stack** out) {
  (void)desc;
  if (out) *out = nullptr;
  return MK_ERR_ARG;
}
void mk_stack_destroy(mk_stack* st) { (void)st; }
size_t mk_decode_step_workspace(const mk_stack* st, int32_t T) {
  (void)st;
  (void)T;
  return 0;
}
int mk_decode_step(mk_stack* st, float* x, int32_t T, const int32_t* h_group_start, int32_t G,
                   const int32_t* drafts, const float* gdn_q, const float* gdn_k, const float* gdn_v,
                   const float* gdn_g, const float* gdn_beta, float* gdn_o, int32_t* h_tokens, int32_t* h_n_acc,
                   int32_t* d_argmax, float* trace, void* ws, size_t ws_bytes, void* stream) {
  return MK_ERR_ARG;
}
}
