// sbf_spec_list.hpp -- parameter sets (k, m, s, H) compiled as specialized
// kernel sets ([cuSBF] §IV-A / §IV-G: parameters are compile-time constants
// so every hash, window and s-mer loop unrolls).  Any other valid parameters
// run on the generic kernels.
//
// The (s, m, H) grid at k = 31 is the parameter sweep: s in {24,26,28,30},
// m in {12,16,20}, H in {2,3,4,6}; (31,16,28,4) is the paper's operating
// point ([cuSBF] §V-B).
#pragma once

#define SBF_SWEEP_M(X, M)                                                                        \
    X(31, M, 24, 2) X(31, M, 24, 3) X(31, M, 24, 4) X(31, M, 24, 6) X(31, M, 26, 2) X(31, M, 26, 3) \
    X(31, M, 26, 4) X(31, M, 26, 6) X(31, M, 28, 2) X(31, M, 28, 3) X(31, M, 28, 4) X(31, M, 28, 6) \
    X(31, M, 30, 2) X(31, M, 30, 3) X(31, M, 30, 4) X(31, M, 30, 6)

// Extra shapes that exercise the compile-time paths: the worked example of
// Fig. 2 (k=9, m=5, s=6), s = m = k (one m-mer, one s-mer), k = 32 (a full
// 64-bit k-mer), a wide halo (w - 1 = 20), and the salted bit address (H > 10).
#define SBF_EXTRA(X) X(9, 5, 6, 3) X(31, 31, 31, 4) X(32, 16, 28, 4) X(21, 1, 19, 5) X(31, 16, 28, 12)
