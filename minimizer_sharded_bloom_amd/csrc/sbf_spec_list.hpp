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

// Slices of the wider grid of [cuSBF] §V-B / Fig. 4 through the operating
// point (31,16,28,4): s = 16..31 at (m, H) = (16, 4), m = 8..31 at
// (s, H) = (28, 4), and H in {1, 5, 8, 16} at (m, s) = (16, 28) (H = 12 is in
// SBF_EXTRA; the sweep above holds the rest).  Split for parallel builds.
#define SBF_SLICE_S_A(X) X(31, 16, 16, 4) X(31, 16, 17, 4) X(31, 16, 18, 4) X(31, 16, 19, 4) X(31, 16, 20, 4) X(31, 16, 21, 4)
#define SBF_SLICE_S_B(X) X(31, 16, 22, 4) X(31, 16, 23, 4) X(31, 16, 25, 4) X(31, 16, 27, 4) X(31, 16, 29, 4) X(31, 16, 31, 4)
#define SBF_SLICE_M_A(X) X(31, 8, 28, 4) X(31, 9, 28, 4) X(31, 10, 28, 4) X(31, 11, 28, 4) X(31, 13, 28, 4) X(31, 14, 28, 4) X(31, 15, 28, 4)
#define SBF_SLICE_M_B(X) X(31, 17, 28, 4) X(31, 18, 28, 4) X(31, 19, 28, 4) X(31, 21, 28, 4) X(31, 22, 28, 4) X(31, 23, 28, 4) X(31, 24, 28, 4)
#define SBF_SLICE_M_C(X) X(31, 25, 28, 4) X(31, 26, 28, 4) X(31, 27, 28, 4) X(31, 28, 28, 4) X(31, 29, 28, 4) X(31, 30, 28, 4) X(31, 31, 28, 4)
#define SBF_SLICE_H(X) X(31, 16, 28, 1) X(31, 16, 28, 5) X(31, 16, 28, 8) X(31, 16, 28, 16)

// The lowest-FPR block of the two-dimensional (s, m) grid at H = 4 on
// genome-like input (s = 23..26, m = 21..23; the grid's map puts its
// minimum there, several times below (28, 16, 4)), split in two for
// parallel builds.
#define SBF_GRID_BEST_A(X) X(31, 21, 23, 4) X(31, 22, 23, 4) X(31, 23, 23, 4) X(31, 21, 24, 4) X(31, 22, 24, 4) X(31, 23, 24, 4)
#define SBF_GRID_BEST_B(X) X(31, 21, 25, 4) X(31, 22, 25, 4) X(31, 23, 25, 4) X(31, 21, 26, 4) X(31, 22, 26, 4) X(31, 23, 26, 4)

// Wide-block variant (512-bit blocks, whole-block addressing): the operating
// point and its neighbours in s, H and m.
#define SBF_WIDE(X)                                                                                               \
    X(31, 16, 28, 4) X(31, 16, 24, 4) X(31, 16, 26, 4) X(31, 16, 30, 4) X(31, 16, 28, 2) X(31, 16, 28, 3)          \
    X(31, 16, 28, 6) X(31, 16, 28, 8) X(31, 12, 28, 4) X(31, 20, 28, 4) X(31, 16, 24, 2) X(31, 12, 30, 6)          \
    X(21, 11, 19, 3) X(32, 16, 28, 4) X(9, 5, 6, 12) X(31, 8, 28, 4) X(31, 31, 28, 4)
