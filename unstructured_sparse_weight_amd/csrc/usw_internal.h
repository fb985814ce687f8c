// Internal declarations shared by the host and device halves of libusw.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "usw.h"

namespace usw {

struct Geometry {
  int64_t M, K, gt_m, gt_k;
  int64_t Gr, Gc, ngt;   // GroupTile rows, columns, count
  int64_t Tr, Tc;        // TCTiles per GroupTile side
  int64_t bt_per_gt;     // BitmapTiles per GroupTile
  int64_t nbt;           // BitmapTiles in the matrix
};

usw_status make_geometry(int64_t M, int64_t K, int64_t gt_m, int64_t gt_k, Geometry* g);
size_t values_alloc_bytes(int32_t val_type, int64_t nnz);
double f16_to_f64(uint16_t h);
uint16_t f64_to_f16_rne(double x);

}  // namespace usw
