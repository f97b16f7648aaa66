/*
 * cautious_adam.h - C ABI of the library's optimizer for the non-matrix parameters: one
 * cautious-Adam step over a list of tensors, in one fused elementwise pass on the GPU.
 *
 * Source: the RecursiveFromBest record analysis at lqnn.cn (news/184262), section 3.3
 * "bigram 与 value-embedding 银行上的 C-Optim / 谨慎 Adam". The record trains the embedding-
 * like parameters (token embedding / LM head, value-embedding banks, bigram table, scalars)
 * with Adam whose weight decay is cautious: decay acts on an element only where the Adam
 * update and the parameter have the same sign (a mask update * p > 0, then the masked decay
 * term added to the update). The section's parameter table gives each tensor a decay
 * multiplier (150 for embed and lm_head, 0 for scalars). The hidden matrices take the Muon
 * step of muon.h; this is the other half of that table.
 *
 * What one call computes for every element of every tensor (t = cfg->step, counting from 1):
 *   m <- beta1 m + (1 - beta1) g                      (textbook Adam moments, fp32 buffers)
 *   v <- beta2 v + (1 - beta2) g^2
 *   u  = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *   u <- u + weight_decay * wd_mul * p   where u and p are both > 0 or both < 0
 *   p <- p - lr u
 * The page prints neither Adam's moments nor the effective decay: the moments are textbook
 * Adam, the effective decay is the base decay times the tensor's multiplier, and the decay
 * is decoupled (it never enters m or v), so with the mask all set the step is AdamW's and
 * with it all clear, Adam's.
 *
 * Arithmetic is fp32 (parameters and gradients stored in bf16 are widened exactly; a bf16
 * parameter is rounded to nearest even once, after the update). 1 - beta^t is formed in
 * double on the host.
 *
 * Conventions are those of muon.h: device buffers on the current HIP device, contiguous,
 * 16-byte aligned base addresses, owned by the caller; work enqueued on `stream` without
 * synchronising; arguments validated on the host before anything is enqueued (an error
 * return has enqueued nothing and muon_last_error() describes it); NaN and Inf propagated.
 * The call allocates nothing and needs no workspace.
 */
#ifndef CAUTIOUS_ADAM_H
#define CAUTIOUS_ADAM_H

#include "muon.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One tensor of the step, viewed as numel contiguous elements (any shape).
 *   param       param_dtype, updated in place
 *   grad        grad_dtype, read only; may be shared between tensors
 *   exp_avg     fp32 first moment m, updated in place; zero-fill it before step 1
 *   exp_avg_sq  fp32 second moment v, updated in place; zero-fill it before step 1
 *   numel       in [0, 2^40]; a tensor with numel 0 is skipped and its pointers may be NULL
 *   wd_mul      finite multiplier of cfg->weight_decay for this tensor
 * No written buffer may overlap any other buffer of the call. */
typedef struct {
  void *param;
  const void *grad;
  float *exp_avg;
  float *exp_avg_sq;
  int64_t numel;
  muon_dtype param_dtype;
  muon_dtype grad_dtype;
  float wd_mul;
} muon_adam_tensor;

/* Hyper-parameters of one step, shared by every tensor of the call. lr, eps and
 * weight_decay are finite with eps >= 0; beta1 and beta2 are in [0, 1); step >= 1 is the
 * index t of this step in the bias corrections (the caller counts steps). */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  int64_t step;
} muon_adam_config;

/* Fills cfg with the textbook Adam defaults (the page prints no values): lr 1e-3,
 * beta1 0.9, beta2 0.999, eps 1e-8, weight_decay 0, step 1. A NULL cfg is ignored. */
void muon_adam_config_default(muon_adam_config *cfg);

/* One cautious-Adam step over tensors[0..n-1] (n >= 0; n = 0 is a no-op). Tensors of one
 * dtype pair share launches; each launch covers up to 32 tensors. */
int muon_cautious_adam_step(const muon_adam_tensor *tensors, int64_t n,
                            const muon_adam_config *cfg, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CAUTIOUS_ADAM_H */
