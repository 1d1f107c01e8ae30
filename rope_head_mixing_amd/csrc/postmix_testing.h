// postmix_testing.h -- a test hook of libpostmix.so, not part of its public
// interface (include/postmix.h) and not installed.
//
// By default a shape runs the tiled kernels when its channels split into
// 128- or 256-channel parts that hold the whole pe range, and the general
// (persistent, one wave per workgroup) kernels otherwise.  The parity tests
// run both families on the same inputs and compare them, so they need a way
// to force the general kernels on shapes the tiled ones would take.
#pragma once

#ifdef __cplusplus
extern "C" {
#endif

// enable != 0: the calls that THIS THREAD makes afterwards route every shape
// through the general kernels (postmix_bwd then runs its two separate
// computations); other threads are unaffected.  Y and dO agree with the
// tiled kernels up to fp32 summation order; dW of either family is bitwise
// repeatable, but the two sum in different orders.  Returns the calling
// thread's previous setting.
int pm_testing_set_general_kernels(int enable);

#ifdef __cplusplus
}
#endif
