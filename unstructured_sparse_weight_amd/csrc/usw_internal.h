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

// IE-BME: local tiles of lt_m x lt_k cut into r_a x c_a areas of am x ak.
struct UnionGeometry {
  int64_t M, K, lt_m, lt_k, r_a, c_a;
  int64_t Q;          // areas per LT
  int64_t am, ak;     // area shape = union-mask shape of an LT
  int64_t lr, lc;     // LT rows and columns of the matrix
  int64_t nlt;        // LTs
  int64_t nw;         // union words per LT
};

// Tiled-CBC: GTiles of 256 x 16, columns of 256 x 1 with 4 bitmap words.
constexpr int kCbcTM = 256;
constexpr int kCbcTK = 16;
constexpr int kCbcWpc = kCbcTM / 64;

struct CbcGeometry {
  int64_t M, K;
  int64_t gr, gc;   // GTile rows and columns
  int64_t ngt;
};

usw_status make_cbc_geometry(int64_t M, int64_t K, CbcGeometry* g);

usw_status make_union_geometry(int64_t M, int64_t K, int64_t lt_m, int64_t lt_k, int64_t r_a, int64_t c_a,
                               UnionGeometry* g);
size_t values_alloc_bytes(int32_t val_type, int64_t nnz);

// Prefill (MFMA) kernel for fp16 values and N > 32: launch shape and split-K
// factor, workspace size, launch.
struct PrefillPlan {
  int waves;    // 8: the 512-token kernel, 4: the 256-token kernel
  int ntiles;   // token tiles of 64 * waves
  int splits;   // workgroups per (strip, token tile)
  int wgs;      // > 0: stream-K over this many workgroups (512-token tiles only)
};
// tiles512 = false keeps N > 256 on the 256-token kernel, which needs no
// workspace at splits = 1 (the 512-token kernel reads a copy of X there).
PrefillPlan prefill_plan(const Geometry& g, int N, int splits_req, bool tiles512 = true);
size_t prefill_counter_bytes(const Geometry& g, const PrefillPlan& p);
size_t prefill_workspace_bytes(const Geometry& g, int N, const PrefillPlan& p);
// counters: the plan's per-tile counters (prefill_counter_bytes, zero at the
// start of the launch); part: the rest of the workspace (prefill_workspace_bytes
// minus the counter bytes): partial sums, then for the 512-token kernel the
// fragment-ordered copy of X.  Unused when the workspace size is 0.
usw_status prefill_launch(const usw_fmt* f, const Geometry& g, const uint16_t* X, void* Y, bool f16out, int N,
                          uint32_t* counters, float* part, const PrefillPlan& p, void* stream);

}  // namespace usw
