// Matrix-core path of the grouped dgrad (kernel in tile.hip, next to the
// forward tile kernel whose fp16 decode it shares).
#pragma once

#include "gnf4_internal.h"

namespace gnf4 {

// dx = dy . dequant(W[expert]) for every group of at least `rows_min` rows.
// `row_exp` holds one power-of-two exponent per dy row, as launch_row_exp
// writes them for an [M, N] matrix.  Requires N % 8 == 0 and 16-byte
// aligned dy (rows are read in 16-byte chunks).
hipError_t launch_dgrad_tile(const DgradArgs& a, const int32_t* row_exp, int rows_min,
                             hipStream_t stream);

}  // namespace gnf4
