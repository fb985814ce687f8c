// Host half of the usw library: status strings, encoding sizes, the TCA-BME
// encoder (fp16 and INT4 values) and the format validator.
//
// Format: blog "SpInfer: How bitmaps make sparse LLMs actually fast", section
// "How TCA-BME addresses the indexing overhead" (three-level tiling, Bitmap /
// Values / GroupTile-offset arrays, storage equation).  The orders inside each
// level are the row-major readings stated in include/usw.h.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "usw.h"
#include "usw_internal.h"
#include "usw_parallel.h"
#include "usw_quant.h"

namespace usw {

usw_status make_geometry(int64_t M, int64_t K, int64_t gt_m, int64_t gt_k, Geometry* g) {
  if (gt_m <= 0 || gt_k <= 0 || gt_m % 16 || gt_k % 16) return USW_ERR_BAD_SHAPE;
  if (M <= 0 || K <= 0 || M % gt_m || K % gt_k) return USW_ERR_BAD_SHAPE;
  if (M > (1 << 30) || K > (1 << 30)) return USW_ERR_BAD_SHAPE;
  g->M = M;
  g->K = K;
  g->gt_m = gt_m;
  g->gt_k = gt_k;
  g->Gr = M / gt_m;
  g->Gc = K / gt_k;
  g->ngt = g->Gr * g->Gc;
  g->Tr = gt_m / 16;
  g->Tc = gt_k / 16;
  g->bt_per_gt = g->Tr * g->Tc * 4;
  g->nbt = M * K / 64;
  return USW_OK;
}

usw_status make_union_geometry(int64_t M, int64_t K, int64_t lt_m, int64_t lt_k, int64_t r_a, int64_t c_a,
                               UnionGeometry* g) {
  if (M <= 0 || K <= 0 || lt_m <= 0 || lt_k <= 0 || r_a <= 0 || c_a <= 0) return USW_ERR_BAD_SHAPE;
  if (M % lt_m || K % lt_k || lt_m % r_a || lt_k % c_a) return USW_ERR_BAD_SHAPE;
  if (M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 31) - 1) return USW_ERR_BAD_SHAPE;
  const int64_t am = lt_m / r_a, ak = lt_k / c_a;
  if ((am * ak) % 64) return USW_ERR_BAD_SHAPE;
  g->M = M;
  g->K = K;
  g->lt_m = lt_m;
  g->lt_k = lt_k;
  g->r_a = r_a;
  g->c_a = c_a;
  g->Q = r_a * c_a;
  g->am = am;
  g->ak = ak;
  g->lr = M / lt_m;
  g->lc = K / lt_k;
  g->nlt = g->lr * g->lc;
  g->nw = am * ak / 64;
  return USW_OK;
}

usw_status make_cbc_geometry(int64_t M, int64_t K, CbcGeometry* g) {
  if (M <= 0 || K <= 0 || M % kCbcTM || K % kCbcTK) return USW_ERR_BAD_SHAPE;
  if (M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 31) - 1) return USW_ERR_BAD_SHAPE;
  g->M = M;
  g->K = K;
  g->gr = M / kCbcTM;
  g->gc = K / kCbcTK;
  g->ngt = g->gr * g->gc;
  return USW_OK;
}

namespace {

inline bool is_kept(const uint16_t* W, const uint8_t* mask, int64_t idx) {
  if (mask) return mask[idx] != 0;
  return (W[idx] & 0x7FFFu) != 0;  // +0 and -0 dropped; NaN and Inf kept
}

// Visit the elements of GroupTile g in storage order: f(bt_index_in_matrix,
// position, linear_index_in_W).
template <class F>
inline void for_each_in_group(const Geometry& g, int64_t gid, F&& f) {
  const int64_t gi = gid / g.Gc, gj = gid % g.Gc;
  for (int64_t t = 0; t < g.Tr * g.Tc; ++t) {
    const int64_t ti = t / g.Tc, tj = t % g.Tc;
    for (int b = 0; b < 4; ++b) {
      const int64_t r0 = gi * g.gt_m + 16 * ti + 8 * (b >> 1);
      const int64_t c0 = gj * g.gt_k + 16 * tj + 8 * (b & 1);
      const int64_t bt = gid * g.bt_per_gt + 4 * t + b;
      for (int p = 0; p < 64; ++p) f(bt, p, (r0 + (p >> 3)) * g.K + c0 + (p & 7));
    }
  }
}

usw_status count_groups(const Geometry& g, const uint16_t* W, const uint8_t* mask, std::vector<int64_t>* off) {
  off->assign(g.ngt + 1, 0);
  int64_t* o = off->data();
  parallel_for(g.Gr, [&](int64_t lo, int64_t hi) {
    for (int64_t gi = lo; gi < hi; ++gi)
      for (int64_t gj = 0; gj < g.Gc; ++gj) {
        int64_t c = 0;
        for (int64_t r = gi * g.gt_m; r < (gi + 1) * g.gt_m; ++r)
          for (int64_t k = gj * g.gt_k; k < (gj + 1) * g.gt_k; ++k) c += is_kept(W, mask, r * g.K + k);
        o[gi * g.Gc + gj + 1] = c;
      }
  });
  for (int64_t i = 0; i < g.ngt; ++i) o[i + 1] += o[i];
  if (o[g.ngt] >= (int64_t(1) << 32)) return USW_ERR_CAPACITY;
  return USW_OK;
}

size_t values_logical_bytes(int32_t val_type, int64_t nnz) {
  if (val_type == USW_VAL_F16) return static_cast<size_t>(2 * nnz);
  if (val_type == USW_VAL_I2) return static_cast<size_t>((nnz + 3) / 4);
  return static_cast<size_t>((nnz + 1) / 2);
}

// Largest positive code of a quantised value type (INT4 7, 2-bit 1).
int code_max(int32_t val_type) { return val_type == USW_VAL_I2 ? 1 : 7; }

// b-bit row scales over the kept entries (largest kept magnitude as
// sign-cleared fp16 bits, then int_scale_bits): writes the fp16 bits and
// returns their values.
std::vector<double> row_scales(const uint16_t* W, const uint8_t* mask, int64_t M, int64_t K, uint16_t* scales,
                               int qmax = 7) {
  std::vector<double> rscale(static_cast<size_t>(M), 0.0);
  parallel_for(M, [&](int64_t lo, int64_t hi) {
    for (int64_t m = lo; m < hi; ++m) {
      uint16_t amax = 0;
      for (int64_t k = 0; k < K; ++k) {
        const uint16_t a = W[m * K + k] & 0x7FFFu;
        if (a > amax && is_kept(W, mask, m * K + k)) amax = a;
      }
      const uint16_t s = int_scale_bits(amax, qmax);
      scales[m] = s;
      rscale[m] = f16_to_f64(s);
    }
  });
  return rscale;
}

// Packs INT4 codes two per byte, element 2i in the low nibble of byte i.
void pack_i4(const std::vector<int8_t>& q, int64_t n, uint8_t* vb) {
  parallel_for((n + 1) / 2, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
      const uint8_t a = static_cast<uint8_t>(q[2 * i]) & 0xF;
      const uint8_t b = (2 * i + 1 < n) ? (static_cast<uint8_t>(q[2 * i + 1]) & 0xF) : 0;
      vb[i] = static_cast<uint8_t>(a | (b << 4));
    }
  });
}

// Packs 2-bit codes four per byte, element 4i + j in bits 2j, 2j+1 of byte i.
void pack_i2(const std::vector<int8_t>& q, int64_t n, uint8_t* vb) {
  parallel_for((n + 3) / 4, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
      uint8_t b = 0;
      for (int j = 0; j < 4; ++j)
        if (4 * i + j < n) b |= static_cast<uint8_t>((static_cast<uint8_t>(q[4 * i + j]) & 0x3) << (2 * j));
      vb[i] = b;
    }
  });
}

// Linear index in W of position p = i * ak + j of area q of LT t.  perm
// (NULL: rows in order) rearranges each LT's rows: stored row s of LT t is
// the LT's row perm[t * lt_m + s] of W.
inline int64_t union_elem(const UnionGeometry& g, const int32_t* perm, int64_t t, int64_t q, int64_t p) {
  const int64_t ti = t / g.lc, tj = t % g.lc;
  const int64_t ar = q / g.c_a, ac = q % g.c_a;
  const int64_t i = p / g.ak, j = p % g.ak;
  const int64_t s = ar * g.am + i;
  const int64_t r = perm ? perm[t * g.lt_m + s] : s;
  return (ti * g.lt_m + r) * g.K + tj * g.lt_k + ac * g.ak + j;
}

// Union bit of position p of LT t: any of the Q area weights kept.
inline bool union_on(const UnionGeometry& g, const int32_t* perm, const uint16_t* W, const uint8_t* mask, int64_t t,
                     int64_t p) {
  for (int64_t q = 0; q < g.Q; ++q)
    if (is_kept(W, mask, union_elem(g, perm, t, q, p))) return true;
  return false;
}

// Every LT's row order a permutation of its rows.
bool valid_row_orders(const UnionGeometry& g, const int32_t* perm) {
  std::vector<uint8_t> seen(static_cast<size_t>(g.lt_m));
  for (int64_t t = 0; t < g.nlt; ++t) {
    std::fill(seen.begin(), seen.end(), uint8_t(0));
    for (int64_t s = 0; s < g.lt_m; ++s) {
      const int32_t r = perm[t * g.lt_m + s];
      if (r < 0 || r >= g.lt_m || seen[static_cast<size_t>(r)]) return false;
      seen[static_cast<size_t>(r)] = 1;
    }
  }
  return true;
}

// Kept count of every column tile (GTile t, column c at t * 16 + c), their
// total and the total of the runs padded to 8.
void count_cbc(const CbcGeometry& g, const uint16_t* W, const uint8_t* mask, std::vector<int64_t>* cnt,
               int64_t* total, int64_t* padded) {
  cnt->assign(static_cast<size_t>(g.ngt * kCbcTK), 0);
  int64_t* c = cnt->data();
  parallel_for(g.ngt, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      const int64_t ti = t / g.gc, tj = t % g.gc;
      for (int k = 0; k < kCbcTK; ++k) {
        int64_t n = 0;
        for (int r = 0; r < kCbcTM; ++r) n += is_kept(W, mask, (ti * kCbcTM + r) * g.K + tj * kCbcTK + k);
        c[t * kCbcTK + k] = n;
      }
    }
  });
  *total = 0;
  *padded = 0;
  for (int64_t i = 0; i < g.ngt * kCbcTK; ++i) {
    *total += c[i];
    *padded += (c[i] + 7) / 8 * 8;
  }
}

// offsets[t] = payload elements before LT t (Q times the active positions).
usw_status count_union(const UnionGeometry& g, const int32_t* perm, const uint16_t* W, const uint8_t* mask,
                       std::vector<int64_t>* off) {
  off->assign(g.nlt + 1, 0);
  int64_t* o = off->data();
  parallel_for(g.nlt, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      int64_t c = 0;
      for (int64_t p = 0; p < g.am * g.ak; ++p) c += union_on(g, perm, W, mask, t, p);
      o[t + 1] = g.Q * c;
    }
  });
  for (int64_t i = 0; i < g.nlt; ++i) o[i + 1] += o[i];
  if (o[g.nlt] >= (int64_t(1) << 32)) return USW_ERR_CAPACITY;
  return USW_OK;
}

}  // namespace

// The kernels read whole 16-byte chunks starting at the chunk that holds a
// GroupTile's first value, even for an empty GroupTile at the very end, so
// the allocation extends to the next 16-byte boundary strictly past the data.
size_t values_alloc_bytes(int32_t val_type, int64_t nnz) {
  return (values_logical_bytes(val_type, nnz) & ~size_t(15)) + 16;
}

}  // namespace usw

using namespace usw;

namespace {

usw_status union_query_impl(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m, int32_t lt_k,
                            int32_t r_a, int32_t c_a, int32_t val_type, const int32_t* perm, int64_t* payload,
                            size_t* bytes_bitmaps, size_t* bytes_offsets, size_t* bytes_values,
                            size_t* bytes_values_alloc, size_t* bytes_scales) {
  if (!W && !mask) return USW_ERR_NULL_ARG;
  UnionGeometry g;
  usw_status st = make_union_geometry(M, K, lt_m, lt_k, r_a, c_a, &g);
  if (st) return st;
  if (val_type != USW_VAL_F16 && val_type != USW_VAL_I4 && val_type != USW_VAL_I2) return USW_ERR_BAD_DTYPE;
  if (perm && (g.lt_m > 256 || !valid_row_orders(g, perm))) return USW_ERR_BAD_SHAPE;
  std::vector<int64_t> off;
  st = count_union(g, perm, W, mask, &off);
  if (st) return st;
  const int64_t n = off[g.nlt];
  if (payload) *payload = n;
  if (bytes_bitmaps) *bytes_bitmaps = static_cast<size_t>(8 * g.nlt * g.nw);
  if (bytes_offsets) *bytes_offsets = static_cast<size_t>(4 * (g.nlt + 1));
  if (bytes_values) *bytes_values = values_logical_bytes(val_type, n);
  if (bytes_values_alloc) *bytes_values_alloc = values_alloc_bytes(val_type, n);
  if (bytes_scales) *bytes_scales = val_type != USW_VAL_F16 ? static_cast<size_t>(2 * M) : 0;
  return USW_OK;
}

usw_status union_encode_impl(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                             int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type, const int32_t* perm,
                             uint64_t* bitmaps, uint32_t* offsets, void* values, size_t values_capacity,
                             uint16_t* scales, uint8_t* rowmap) {
  if (!W || !bitmaps || !offsets || !values) return USW_ERR_NULL_ARG;
  UnionGeometry g;
  usw_status st = make_union_geometry(M, K, lt_m, lt_k, r_a, c_a, &g);
  if (st) return st;
  if (val_type != USW_VAL_F16 && val_type != USW_VAL_I4 && val_type != USW_VAL_I2) return USW_ERR_BAD_DTYPE;
  const bool quant = val_type != USW_VAL_F16;
  if (quant && !scales) return USW_ERR_NULL_ARG;
  if (perm && (g.lt_m > 256 || !valid_row_orders(g, perm))) return USW_ERR_BAD_SHAPE;
  std::vector<int64_t> off;
  st = count_union(g, perm, W, mask, &off);
  if (st) return st;
  const int64_t total = off[g.nlt];
  const size_t logical = values_logical_bytes(val_type, total);
  if (values_capacity < logical) return USW_ERR_CAPACITY;
  for (int64_t i = 0; i <= g.nlt; ++i) offsets[i] = static_cast<uint32_t>(off[i]);
  if (perm)
    for (int64_t t = 0; t < g.nlt; ++t)
      for (int64_t s = 0; s < g.lt_m; ++s) rowmap[t * g.lt_m + perm[t * g.lt_m + s]] = static_cast<uint8_t>(s);

  // INT4 / 2-bit: scales and codes of the rows of W, whatever LT row they
  // are stored in.
  const int qmax = code_max(val_type);
  std::vector<double> rscale;
  if (quant) rscale = row_scales(W, mask, M, K, scales, qmax);
  std::vector<int8_t> q;
  if (quant) q.assign(static_cast<size_t>(total), 0);
  uint16_t* v16 = static_cast<uint16_t*>(values);

  // Per LT: the union words, then the Q area streams, each holding the area's
  // weight (0 where pruned) at every active position in row-major order.
  parallel_for(g.nlt, [&](int64_t lo, int64_t hi) {
    std::vector<int64_t> active;
    for (int64_t t = lo; t < hi; ++t) {
      active.clear();
      uint64_t* words = bitmaps + t * g.nw;
      for (int64_t w = 0; w < g.nw; ++w) words[w] = 0;
      for (int64_t p = 0; p < g.am * g.ak; ++p)
        if (union_on(g, perm, W, mask, t, p)) {
          words[p >> 6] |= 1ull << (p & 63);
          active.push_back(p);
        }
      const int64_t P = static_cast<int64_t>(active.size());
      for (int64_t qa = 0; qa < g.Q; ++qa)
        for (int64_t r = 0; r < P; ++r) {
          const int64_t lin = union_elem(g, perm, t, qa, active[static_cast<size_t>(r)]);
          const int64_t idx = off[t] + qa * P + r;
          const bool kept = is_kept(W, mask, lin);
          if (val_type == USW_VAL_F16)
            v16[idx] = kept ? W[lin] : uint16_t(0);
          else
            q[static_cast<size_t>(idx)] = kept ? int_code(W[lin], rscale[lin / g.K], qmax) : int8_t(0);
        }
    }
  });

  uint8_t* vb = static_cast<uint8_t*>(values);
  if (val_type == USW_VAL_I4) pack_i4(q, total, vb);
  if (val_type == USW_VAL_I2) pack_i2(q, total, vb);
  if (values_capacity > logical) std::memset(vb + logical, 0, values_capacity - logical);
  return USW_OK;
}

}  // namespace

extern "C" {

int32_t usw_abi_version(void) { return USW_ABI_VERSION; }

const char* usw_status_str(usw_status s) {
  switch (s) {
    case USW_OK: return "ok";
    case USW_ERR_NULL_ARG: return "a required pointer is NULL";
    case USW_ERR_BAD_SHAPE: return "M, K must be positive multiples of gt_m, gt_k; gt_m, gt_k multiples of 16";
    case USW_ERR_BAD_DTYPE: return "unknown value type or output type";
    case USW_ERR_BAD_N: return "N must be at least 1";
    case USW_ERR_UNSUPPORTED: return "no kernel for this request";
    case USW_ERR_MISALIGNED: return "a device pointer is not 16-byte aligned";
    case USW_ERR_WORKSPACE: return "workspace missing or too small";
    case USW_ERR_CORRUPT: return "encoding is corrupt: offsets disagree with bitmaps";
    case USW_ERR_HIP: return "HIP call failed";
    case USW_ERR_CAPACITY: return "output buffer too small or NNZ does not fit 32 bits";
    default: return "unknown status";
  }
}

usw_status usw_encode_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t gt_m,
                            int32_t gt_k, int32_t val_type, int64_t* nnz, size_t* bytes_bitmaps,
                            size_t* bytes_offsets, size_t* bytes_values, size_t* bytes_values_alloc,
                            size_t* bytes_scales) {
  if (!W && !mask) return USW_ERR_NULL_ARG;
  Geometry g;
  usw_status st = make_geometry(M, K, gt_m, gt_k, &g);
  if (st) return st;
  if (val_type != USW_VAL_F16 && val_type != USW_VAL_I4) return USW_ERR_BAD_DTYPE;
  std::vector<int64_t> off;
  st = count_groups(g, W, mask, &off);
  if (st) return st;
  const int64_t n = off[g.ngt];
  if (nnz) *nnz = n;
  if (bytes_bitmaps) *bytes_bitmaps = static_cast<size_t>(8 * g.nbt);
  if (bytes_offsets) *bytes_offsets = static_cast<size_t>(4 * (g.ngt + 1));
  if (bytes_values) *bytes_values = val_type == USW_VAL_F16 ? static_cast<size_t>(2 * n) : static_cast<size_t>((n + 1) / 2);
  if (bytes_values_alloc) *bytes_values_alloc = values_alloc_bytes(val_type, n);
  if (bytes_scales) *bytes_scales = val_type == USW_VAL_I4 ? static_cast<size_t>(2 * M) : 0;
  return USW_OK;
}

usw_status usw_encode(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t gt_m, int32_t gt_k,
                      int32_t val_type, uint64_t* bitmaps, uint32_t* offsets, void* values, size_t values_capacity,
                      uint16_t* scales) {
  if (!W || !bitmaps || !offsets || !values) return USW_ERR_NULL_ARG;
  Geometry g;
  usw_status st = make_geometry(M, K, gt_m, gt_k, &g);
  if (st) return st;
  if (val_type != USW_VAL_F16 && val_type != USW_VAL_I4) return USW_ERR_BAD_DTYPE;
  if (val_type == USW_VAL_I4 && !scales) return USW_ERR_NULL_ARG;
  std::vector<int64_t> off;
  st = count_groups(g, W, mask, &off);
  if (st) return st;
  const int64_t nnz = off[g.ngt];
  const size_t logical = val_type == USW_VAL_F16 ? static_cast<size_t>(2 * nnz) : static_cast<size_t>((nnz + 1) / 2);
  if (values_capacity < logical) return USW_ERR_CAPACITY;

  for (int64_t i = 0; i <= g.ngt; ++i) offsets[i] = static_cast<uint32_t>(off[i]);

  // INT4: per-row scale over the kept entries, in fp64.
  std::vector<double> rscale;
  if (val_type == USW_VAL_I4) rscale = row_scales(W, mask, M, K, scales);

  std::vector<int8_t> q;  // INT4 codes in storage order, packed afterwards
  if (val_type == USW_VAL_I4) q.assign(static_cast<size_t>(nnz), 0);
  uint16_t* v16 = static_cast<uint16_t*>(values);

  parallel_for(g.ngt, [&](int64_t lo, int64_t hi) {
    for (int64_t gid = lo; gid < hi; ++gid) {
      int64_t idx = off[gid];
      uint64_t bm = 0;
      int64_t cur_bt = -1;
      for_each_in_group(g, gid, [&](int64_t bt, int p, int64_t lin) {
        if (bt != cur_bt) {
          if (cur_bt >= 0) bitmaps[cur_bt] = bm;
          cur_bt = bt;
          bm = 0;
        }
        if (!is_kept(W, mask, lin)) return;
        bm |= 1ull << p;
        if (val_type == USW_VAL_F16) {
          v16[idx] = W[lin];
        } else {
          q[static_cast<size_t>(idx)] = i4_code(W[lin], rscale[lin / g.K]);
        }
        ++idx;
      });
      if (cur_bt >= 0) bitmaps[cur_bt] = bm;
    }
  });

  uint8_t* vb = static_cast<uint8_t*>(values);
  if (val_type == USW_VAL_I4) pack_i4(q, nnz, vb);
  if (values_capacity > logical) std::memset(vb + logical, 0, values_capacity - logical);
  return USW_OK;
}

usw_status usw_validate(const usw_fmt* f) {
  if (!f) return USW_ERR_NULL_ARG;
  Geometry g;
  usw_status st = make_geometry(f->M, f->K, f->gt_m, f->gt_k, &g);
  if (st) return st;
  if (f->val_type != USW_VAL_F16 && f->val_type != USW_VAL_I4) return USW_ERR_BAD_DTYPE;
  if (!f->bitmaps || !f->offsets) return USW_ERR_NULL_ARG;
  if (f->nnz > 0 && !f->values) return USW_ERR_NULL_ARG;
  if (f->val_type == USW_VAL_I4 && !f->scales) return USW_ERR_NULL_ARG;
  if (f->reserved != 0) return USW_ERR_BAD_SHAPE;
  if (f->nnz < 0 || f->nnz >= (int64_t(1) << 32)) return USW_ERR_CORRUPT;
  if (f->offsets[0] != 0 || static_cast<int64_t>(f->offsets[g.ngt]) != f->nnz) return USW_ERR_CORRUPT;
  for (int64_t gid = 0; gid < g.ngt; ++gid) {
    if (f->offsets[gid + 1] < f->offsets[gid]) return USW_ERR_CORRUPT;
    int64_t c = 0;
    for (int64_t b = 0; b < g.bt_per_gt; ++b) c += __builtin_popcountll(f->bitmaps[gid * g.bt_per_gt + b]);
    if (c != static_cast<int64_t>(f->offsets[gid + 1] - f->offsets[gid])) return USW_ERR_CORRUPT;
  }
  return USW_OK;
}

usw_status usw_cbc_encode_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int64_t* nnz,
                                int64_t* nnz_padded, size_t* bytes_bitmaps, size_t* bytes_tile_offsets,
                                size_t* bytes_colinfo, size_t* bytes_values) {
  if (!W && !mask) return USW_ERR_NULL_ARG;
  CbcGeometry g;
  usw_status st = make_cbc_geometry(M, K, &g);
  if (st) return st;
  std::vector<int64_t> cnt;
  int64_t total = 0, padded = 0;
  count_cbc(g, W, mask, &cnt, &total, &padded);
  if (padded >= (int64_t(1) << 32)) return USW_ERR_CAPACITY;
  if (nnz) *nnz = total;
  if (nnz_padded) *nnz_padded = padded;
  if (bytes_bitmaps) *bytes_bitmaps = static_cast<size_t>(8 * g.ngt * kCbcTK * kCbcWpc);
  if (bytes_tile_offsets) *bytes_tile_offsets = static_cast<size_t>(4 * (g.ngt + 1));
  if (bytes_colinfo) *bytes_colinfo = static_cast<size_t>(4 * g.ngt * kCbcTK);
  if (bytes_values) *bytes_values = static_cast<size_t>(2 * padded);
  return USW_OK;
}

usw_status usw_cbc_encode(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, uint64_t* bitmaps,
                          uint32_t* tile_offsets, uint32_t* colinfo, uint16_t* values, size_t values_capacity) {
  if (!W || !bitmaps || !tile_offsets || !colinfo || (!values && values_capacity)) return USW_ERR_NULL_ARG;
  CbcGeometry g;
  usw_status st = make_cbc_geometry(M, K, &g);
  if (st) return st;
  std::vector<int64_t> cnt;
  int64_t total = 0, padded = 0;
  count_cbc(g, W, mask, &cnt, &total, &padded);
  if (padded >= (int64_t(1) << 32)) return USW_ERR_CAPACITY;
  if (values_capacity < static_cast<size_t>(2 * padded)) return USW_ERR_CAPACITY;
  // Tile offsets: prefix of the padded runs of each GTile's columns.
  int64_t acc = 0;
  for (int64_t t = 0; t < g.ngt; ++t) {
    tile_offsets[t] = static_cast<uint32_t>(acc);
    for (int c = 0; c < kCbcTK; ++c) acc += (cnt[static_cast<size_t>(t * kCbcTK + c)] + 7) / 8 * 8;
  }
  tile_offsets[g.ngt] = static_cast<uint32_t>(acc);
  parallel_for(g.ngt, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      const int64_t ti = t / g.gc, tj = t % g.gc;
      int64_t idx = tile_offsets[t], run = 0;
      for (int c = 0; c < kCbcTK; ++c) {
        const int64_t col = tj * kCbcTK + c;
        uint64_t* words = bitmaps + (t * kCbcTK + c) * kCbcWpc;
        for (int j = 0; j < kCbcWpc; ++j) words[j] = 0;
        int64_t n = 0;
        for (int r = 0; r < kCbcTM; ++r) {
          const int64_t lin = (ti * kCbcTM + r) * g.K + col;
          if (!is_kept(W, mask, lin)) continue;
          words[r >> 6] |= 1ull << (r & 63);
          values[idx + n] = W[lin];
          ++n;
        }
        const int64_t np = (n + 7) / 8 * 8;
        for (int64_t i = n; i < np; ++i) values[idx + i] = 0;
        colinfo[t * kCbcTK + c] = static_cast<uint32_t>((run << 16) | n);
        idx += np;
        run += np;
      }
    }
  });
  for (size_t i = static_cast<size_t>(padded); i < values_capacity / 2; ++i) values[i] = 0;
  return USW_OK;
}

usw_status usw_cbc_validate(const usw_cbc_fmt* f) {
  if (!f) return USW_ERR_NULL_ARG;
  CbcGeometry g;
  usw_status st = make_cbc_geometry(f->M, f->K, &g);
  if (st) return st;
  if (f->tile_m != kCbcTM || f->tile_k != kCbcTK || f->reserved != 0) return USW_ERR_BAD_SHAPE;
  if (f->val_type != USW_VAL_F16) return USW_ERR_BAD_DTYPE;
  if (!f->bitmaps || !f->tile_offsets || !f->colinfo || (f->nnz_padded > 0 && !f->values)) return USW_ERR_NULL_ARG;
  if (f->nnz_padded < 0 || f->nnz_padded >= (int64_t(1) << 32)) return USW_ERR_CORRUPT;
  if (f->tile_offsets[0] != 0 || static_cast<int64_t>(f->tile_offsets[g.ngt]) != f->nnz_padded) return USW_ERR_CORRUPT;
  for (int64_t t = 0; t < g.ngt; ++t) {
    int64_t run = 0;
    for (int c = 0; c < kCbcTK; ++c) {
      int64_t n = 0;
      for (int j = 0; j < kCbcWpc; ++j) n += __builtin_popcountll(f->bitmaps[(t * kCbcTK + c) * kCbcWpc + j]);
      const uint32_t ci = f->colinfo[t * kCbcTK + c];
      if (static_cast<int64_t>(ci >> 16) != run || static_cast<int64_t>(ci & 0xFFFFu) != n) return USW_ERR_CORRUPT;
      run += (n + 7) / 8 * 8;
    }
    if (f->tile_offsets[t + 1] < f->tile_offsets[t] ||
        static_cast<int64_t>(f->tile_offsets[t + 1] - f->tile_offsets[t]) != run)
      return USW_ERR_CORRUPT;
  }
  return USW_OK;
}

usw_status usw_union_encode_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                                  int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type, int64_t* payload,
                                  size_t* bytes_bitmaps, size_t* bytes_offsets, size_t* bytes_values,
                                  size_t* bytes_values_alloc, size_t* bytes_scales) {
  return union_query_impl(W, mask, M, K, lt_m, lt_k, r_a, c_a, val_type, nullptr, payload, bytes_bitmaps,
                          bytes_offsets, bytes_values, bytes_values_alloc, bytes_scales);
}

usw_status usw_union_encode(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                            int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type, uint64_t* bitmaps,
                            uint32_t* offsets, void* values, size_t values_capacity, uint16_t* scales) {
  return union_encode_impl(W, mask, M, K, lt_m, lt_k, r_a, c_a, val_type, nullptr, bitmaps, offsets, values,
                           values_capacity, scales, nullptr);
}

usw_status usw_union_encode_reordered_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K,
                                            int32_t lt_m, int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type,
                                            const int32_t* perm, int64_t* payload, size_t* bytes_values,
                                            size_t* bytes_values_alloc) {
  if (!perm) return USW_ERR_NULL_ARG;
  return union_query_impl(W, mask, M, K, lt_m, lt_k, r_a, c_a, val_type, perm, payload, nullptr, nullptr,
                          bytes_values, bytes_values_alloc, nullptr);
}

usw_status usw_union_encode_reordered(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                                      int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type, const int32_t* perm,
                                      uint64_t* bitmaps, uint32_t* offsets, void* values, size_t values_capacity,
                                      uint16_t* scales, uint8_t* rowmap) {
  if (!perm || !rowmap) return USW_ERR_NULL_ARG;
  return union_encode_impl(W, mask, M, K, lt_m, lt_k, r_a, c_a, val_type, perm, bitmaps, offsets, values,
                           values_capacity, scales, rowmap);
}

usw_status usw_union_validate(const usw_union_fmt* f) {
  if (!f) return USW_ERR_NULL_ARG;
  UnionGeometry g;
  usw_status st = make_union_geometry(f->M, f->K, f->lt_m, f->lt_k, f->r_a, f->c_a, &g);
  if (st) return st;
  if (f->val_type != USW_VAL_F16 && f->val_type != USW_VAL_I4 && f->val_type != USW_VAL_I2) return USW_ERR_BAD_DTYPE;
  if (!f->bitmaps || !f->offsets) return USW_ERR_NULL_ARG;
  if (f->payload > 0 && !f->values) return USW_ERR_NULL_ARG;
  if (f->val_type != USW_VAL_F16 && !f->scales) return USW_ERR_NULL_ARG;
  if (f->reserved != 0) return USW_ERR_BAD_SHAPE;
  if (f->payload < 0 || f->payload >= (int64_t(1) << 32)) return USW_ERR_CORRUPT;
  if (f->offsets[0] != 0 || static_cast<int64_t>(f->offsets[g.nlt]) != f->payload) return USW_ERR_CORRUPT;
  for (int64_t t = 0; t < g.nlt; ++t) {
    if (f->offsets[t + 1] < f->offsets[t]) return USW_ERR_CORRUPT;
    int64_t c = 0;
    for (int64_t w = 0; w < g.nw; ++w) c += __builtin_popcountll(f->bitmaps[t * g.nw + w]);
    if (g.Q * c != static_cast<int64_t>(f->offsets[t + 1] - f->offsets[t])) return USW_ERR_CORRUPT;
  }
  if (f->rowmap) {
    if (g.lt_m > 256) return USW_ERR_BAD_SHAPE;
    std::vector<uint8_t> seen(static_cast<size_t>(g.lt_m));
    for (int64_t t = 0; t < g.nlt; ++t) {
      std::fill(seen.begin(), seen.end(), uint8_t(0));
      for (int64_t r = 0; r < g.lt_m; ++r) {
        const uint8_t s = f->rowmap[t * g.lt_m + r];
        if (s >= g.lt_m || seen[s]) return USW_ERR_CORRUPT;
        seen[s] = 1;
      }
    }
  }
  return USW_OK;
}

}  // extern "C"
