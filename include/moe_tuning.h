/*
 * moe_tuning.h -- process-wide overrides of the MoE layer's kernel-selection rules, for tests and
 * benchmarks.
 *
 * By default every entry point of moe.h and moe_block.h picks its GEMM kernel, the spread of GEMM blocks
 * over the chip and any split of the reduction dimension from the sizes alone. A test that wants to run
 * every kernel on the same inputs, or compare two block orders bit for bit, sets a knob here first. Every
 * setting computes the same layer: block orders and grids give bitwise identical results; another GEMM
 * kernel or a K split changes only the fp32 summation order.
 *
 * Knobs are plain process-wide integers (atomic: reading or setting one from any thread is safe). A value
 * applies to every call that starts after it is set, from any thread and on any device, until it is set
 * again; 0 restores the size-based rule. Production callers leave them at 0. Nothing else in the library
 * reads the environment or any other global setting.
 */
#ifndef SIGMOID_ROUTED_MIXTURE_MOE_TUNING_H
#define SIGMOID_ROUTED_MIXTURE_MOE_TUNING_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_tune_knob {
    /* GEMM kernel of every grouped and dense GEMM: 0 by size; 1 the 128-token register-streaming kernel,
       2 its 256-token form, 3 the LDS-copy kernel (where every operand fits its 32-bit offsets; else the
       size rule's fallback), 4 the 16-token weight-streaming kernel. */
    MOE_TUNE_GEMM_PATH = 0,
    /* Split of the LDS-copy kernel's grouped blocks over the 8 XCDs: 0 by size (the work-balanced split for
       the down GEMM), 1 equal block counts for both GEMMs. */
    MOE_TUNE_XCD_SPLIT = 1,
    /* 0 by size (persistent routed GEMMs above the decode sizes), 1 one workgroup per block everywhere. */
    MOE_TUNE_PERSIST = 2,
    /* K split of decode-sized grouped GEMMs: 0 by the live block count, 1 never split, 2 always split in two,
       3 the largest split each GEMM allows (gate/up 4 where four ranges are whole steps of the copy ring,
       else 2; down up to 4 ranges at up to 16 tokens). */
    MOE_TUNE_KSPLIT = 3,
    /* Block order of the persistent routed GEMMs: 0 by size (experts in index order, each cut into chunks
       of up to 16 token tiles, contiguous XCD ranges); 1 the same with chunks of up to 128 tiles; dealt
       orders, the chunks dealt over the XCDs in turn: 2 largest experts first, 3 in index order, 4 largest
       first alternating with the smallest within each XCD. */
    MOE_TUNE_ORDER = 4,
    /* Shared expert above the decode sizes, when it has the routed width and no stream of its own: 0 by size
       (one more group of the persistent routed GEMMs), 1 a dense MLP on the main stream before them. */
    MOE_TUNE_SHARED = 5,
    /* Copy ring of the LDS-copy kernel at up to 32 tokens: 0 by size (three K steps of weights in flight; one
       workgroup per CU running its blocks back to back where the launch allows it and few blocks per CU are
       expected, else one workgroup per block), 1 the two-step ring of larger batches, 2 the three-step ring
       with one workgroup per block, 3 the three-step ring streamed wherever the launch allows it. */
    MOE_TUNE_RING = 6,
    /* Router top-k and permutation of the mixture at up to 16 tokens: 0 by size (one launch: the workgroup
       that routes the last token permutes them all), 1 two launches, as above 16 tokens. */
    MOE_TUNE_ROUTE_PERMUTE = 7,
    /* Stream-K in the streamed decode GEMMs (one workgroup per CU, each taking one contiguous share of all
       blocks' K steps, where the launch has at least as many blocks as CUs and no split is forced): 0 by size
       (the down GEMM), 1 never (whole blocks or the K split's equal ranges), 2 the down and the gate/up GEMM. */
    MOE_TUNE_STREAMK = 8,
    MOE_TUNE_KNOBS = 9 /* number of knobs */
} moe_tune_knob;

/* Sets a knob. MOE_ERR_INVALID_ARG for an unknown knob or a value outside the knob's range (nothing
   changes then). */
moe_status moe_set_tuning(int knob, int value);

/* The knob's current value, or -1 for an unknown knob. */
int moe_get_tuning(int knob);

#ifdef __cplusplus
}
#endif

#endif /* SIGMOID_ROUTED_MIXTURE_MOE_TUNING_H */
