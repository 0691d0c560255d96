// Matrix-core path of the grouped dgrad (kernel in tile.hip, next to the
// forward tile kernel whose fp16 decode it shares).
#pragma once

#include "gnf4_internal.h"

namespace gnf4 {

// dx = dy . dequant(W[expert]) for every group of at least `rows_min` rows.
// dy is read as launch_stage_x staged it for an [M, N] matrix (natural
// order): `dyh` [M + 1, ld] fp16 rows, row M all zeros, and `row_exp`
// [M + 1] their power-of-two exponents.
hipError_t launch_dgrad_tile(const DgradArgs& a, const int32_t* row_exp, const uint16_t* dyh,
                             int ld, int rows_min, hipStream_t stream);

}  // namespace gnf4
