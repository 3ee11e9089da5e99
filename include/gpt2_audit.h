/*
 * gpt2_audit.h -- host-only replay of the training step's launches against
 * the buffer layout, for testing on a machine without a GPU.
 *
 * gpt2_audit_step lays out the buffers for (cfg, B, T) at stand-in
 * addresses (never dereferenced) and runs gpt2_build, a logits-only
 * gpt2_forward, gpt2_forward with targets, gpt2_zero_grad, gpt2_backward,
 * gpt2_update, three gpt2_decode_step calls (first, middle and last
 * position) and a forward and backward with bfloat16 products, with the
 * launch audit on: every launcher declares the element
 * ranges its kernels would read or write (from the kernels' index formulas,
 * grids and leading dimensions) instead of launching, and each range is
 * checked against the named tensors of the layout (the 16 parameter tensors
 * of params, grads, adam_m and adam_v, the activation tensors, the work
 * regions at their exact sizes, the id buffers; stacked tensors cut per
 * layer).  A range must stay inside the tensor it starts in, or cover a run
 * of adjacent whole tensors exactly.  Nothing runs on a GPU and no device
 * memory is touched.
 *
 * shrink_region (may be NULL or "") names one tensor of that table, e.g.
 * "work:splitk_dw" or "acts:qkv[3]", whose size the check takes as
 * shrink_floats smaller: a test of the check itself.  *n_ranges gets the
 * number of ranges declared, *n_violations the number outside their tensor;
 * report (report_len bytes, may be NULL) the first violations as text.
 * Returns GPT2_EINVAL for a configuration gpt2_query_sizes rejects, or the
 * status of a step call that refused to run.
 */
#ifndef GPT2_MI_AUDIT_H
#define GPT2_MI_AUDIT_H

#include <stddef.h>

#include "gpt2.h"

#ifdef __cplusplus
extern "C" {
#endif

gpt2_status gpt2_audit_step(const gpt2_config *cfg, int B, int T, const char *shrink_region, size_t shrink_floats,
                            char *report, size_t report_len, long long *n_ranges, long long *n_violations);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_MI_AUDIT_H */
