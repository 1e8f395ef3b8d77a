// rmm_select.h -- the select + gather launch (host side), shared by
// rmm_select.hip and the C entry points.  Not part of the public ABI.
#pragma once
#include "rmm_internal.h"

namespace rmm {

// Rows of A the fused select + gather kernel stages: `slices` workgroups per
// group, `rows` consecutive rows each (the last slices of a short group may
// have fewer or none).  A is bf16 with leading dimension lda; Ap the panel.
struct SelectGather {
    const uint16_t *A;
    int64_t M, lda, gr;
    int slices;
    int64_t rows;
    uint16_t *Ap;
    int64_t ldp;
};

// Chooses slices and rows per slice for a linear selection of M x K (bf16 A,
// group_rows rows per group) and the LDS staging size nrb (1 KiB blocks per
// wave).  False when the fused kernel does not cover the shape (fp32 A,
// K > 8192, 512 or more groups, rows that do not fit 96 KiB): the caller then
// runs the selection and the gather as two launches.
bool select_gather_plan(int dt, int64_t M, int64_t K, int64_t lda, int64_t group_rows, SelectGather &ga,
                        int &nrb);
hipError_t launch_select_gather(const float *scores, const SelectShape &sh, int32_t *idx, int64_t ldidx,
                                float *thresh, double *bound, const SelectGather &ga, int nrb, hipStream_t s);

}  // namespace rmm
