// Consistency checks of plans held in host memory (the debug mode of the C
// ABI copies a plan there before the call that uses it).
//
// A row plan stores, per (head, block row), the ascending list of live
// column blocks (the CSR form of the next.gr "Block Sparse Attention
// Techniques" tutorial, section 3.2), an order of the rows, and the same
// lists for pairs of neighbouring rows (their union, each entry tagged with
// the rows that list it).  A column plan stores the transposed lists.  The
// kernels trust these arrays for their memory accesses: an out-of-range
// count, column or order entry would send them outside their buffers.  Each
// check below states one property the kernels rely on; the first violation
// found is described in `msg`.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "bsa_internal.h"

namespace bsa {
namespace {

bool bad(char *msg, size_t n, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, n, fmt, ap);
  va_end(ap);
  return false;
}

const int32_t *section(const void *buf, size_t off) {
  return reinterpret_cast<const int32_t *>(static_cast<const char *>(buf) + off);
}

// ptr[0] = 0, every count in [0, max_count], ptr[n] = total.
bool check_ptr(const int32_t *ptr, int64_t n, int32_t max_count, int64_t total, const char *what,
               char *msg, size_t mlen) {
  if (ptr[0] != 0) return bad(msg, mlen, "%s[0] = %d, not 0", what, ptr[0]);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t c = (int64_t)ptr[i + 1] - ptr[i];
    if (c < 0 || c > max_count)
      return bad(msg, mlen, "%s: entry %lld holds %lld items (allowed 0..%d)", what, (long long)i,
                 (long long)c, max_count);
  }
  if (ptr[n] != total)
    return bad(msg, mlen, "%s[%lld] = %d, but the total is %lld", what, (long long)n, ptr[n],
               (long long)total);
  return true;
}

// order holds every value of [0, n) exactly once.
bool check_perm(const int32_t *order, int64_t n, const char *what, char *msg, size_t mlen) {
  std::vector<char> seen((size_t)n, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t x = order[i];
    if (x < 0 || x >= n)
      return bad(msg, mlen, "%s[%lld] = %d is outside [0, %lld)", what, (long long)i, x,
                 (long long)n);
    if (seen[(size_t)x])
      return bad(msg, mlen, "%s lists %d twice (at %lld)", what, x, (long long)i);
    seen[(size_t)x] = 1;
  }
  return true;
}

// Every list strictly ascending, every value in [0, limit).
bool check_lists(const int32_t *ptr, const int32_t *val, int64_t n, int32_t limit,
                 const char *what, char *msg, size_t mlen) {
  for (int64_t i = 0; i < n; ++i) {
    for (int32_t t = ptr[i]; t < ptr[i + 1]; ++t) {
      const int32_t x = val[t];
      if (x < 0 || x >= limit)
        return bad(msg, mlen, "%s: list %lld holds %d, outside [0, %d)", what, (long long)i, x,
                   limit);
      if (t > ptr[i] && x <= val[t - 1])
        return bad(msg, mlen, "%s: list %lld is not strictly ascending (%d after %d)", what,
                   (long long)i, x, val[t - 1]);
    }
  }
  return true;
}

}  // namespace

bool check_plan_host(const void *buf, size_t bytes, int32_t H, int32_t Mb, int32_t Nb, char *msg,
                     size_t mlen) {
  PlanGeometry g;
  if (!plan_geometry(H, Mb, Nb, &g)) return bad(msg, mlen, "invalid dimensions");
  if (bytes < g.total) return bad(msg, mlen, "%zu bytes given, the plan spans %zu", bytes, g.total);
  const int64_t R = (int64_t)H * Mb;
  const int32_t Mp = (Mb + 1) / 2;
  const int64_t Q = (int64_t)H * Mp;
  const int32_t *row_ptr = section(buf, g.off_row_ptr);
  const int32_t *row_order = section(buf, g.off_row_order);
  const int32_t nnz = *section(buf, g.off_nnz);
  const int32_t *col_idx = section(buf, g.off_col_idx);
  if (nnz < 0 || (int64_t)nnz > R * Nb)
    return bad(msg, mlen, "nnz_total = %d is outside [0, %lld]", nnz, (long long)(R * Nb));
  if (!check_ptr(row_ptr, R, Nb, nnz, "row_ptr", msg, mlen)) return false;
  if (!check_lists(row_ptr, col_idx, R, Nb, "col_idx", msg, mlen)) return false;
  if (!check_perm(row_order, R, "row_order", msg, mlen)) return false;

  // Pairs: the union of rows 2p and 2p + 1 of each head, tagged per row.
  const int32_t *pair_ptr = section(buf, g.off_pair_ptr);
  const int32_t *pair_order = section(buf, g.off_pair_order);
  const int32_t *pair_info = section(buf, g.off_pair_info);
  const int32_t *pair_cols = section(buf, g.off_pair_cols);
  if (pair_info[1] != 0 && pair_info[1] != 1)
    return bad(msg, mlen, "pair_info[1] (use flag) = %d, not 0 or 1", pair_info[1]);
  if (pair_info[0] < 0 || (int64_t)pair_info[0] > Q * Nb)
    return bad(msg, mlen, "pair_total = %d is outside [0, %lld]", pair_info[0],
               (long long)(Q * Nb));
  if (!check_ptr(pair_ptr, Q, Nb, pair_info[0], "pair_ptr", msg, mlen)) return false;
  if (!check_perm(pair_order, Q, "pair_order", msg, mlen)) return false;
  for (int32_t h = 0; h < H; ++h) {
    for (int32_t p = 0; p < Mp; ++p) {
      const int64_t pi = (int64_t)h * Mp + p;
      const int64_t r0 = (int64_t)h * Mb + 2 * p;
      const bool two = 2 * p + 1 < Mb;
      // Merge the two rows' lists (already checked ascending) and compare.
      int32_t a = row_ptr[r0], ae = row_ptr[r0 + 1];
      int32_t b = two ? row_ptr[r0 + 1] : 0, be = two ? row_ptr[r0 + 2] : 0;
      int32_t t = pair_ptr[pi];
      const int32_t te = pair_ptr[pi + 1];
      while (a < ae || b < be) {
        int32_t n, tag = 0;
        if (b >= be || (a < ae && col_idx[a] < col_idx[b])) {
          n = col_idx[a++];
          tag = 1;
        } else if (a >= ae || col_idx[b] < col_idx[a]) {
          n = col_idx[b++];
          tag = 2;
        } else {
          n = col_idx[a++];
          ++b;
          tag = 3;
        }
        if (t >= te)
          return bad(msg, mlen, "pair %lld (head %d, rows %d, %d) is missing column %d", (long long)pi,
                     h, 2 * p, 2 * p + 1, n);
        const int32_t want = n | (tag << 24);
        if (pair_cols[t] != want)
          return bad(msg, mlen,
                     "pair %lld (head %d, rows %d, %d), entry %d: 0x%08x, expected column %d "
                     "with row tags %d",
                     (long long)pi, h, 2 * p, 2 * p + 1, t - pair_ptr[pi], (unsigned)pair_cols[t],
                     n, tag);
        ++t;
      }
      if (t != te)
        return bad(msg, mlen, "pair %lld (head %d) lists %d entries beyond its rows' union",
                   (long long)pi, h, te - t);
    }
  }
  return true;
}

bool check_plan_cols_host(const void *buf, size_t bytes, int32_t H, int32_t Hkv, int32_t Mb,
                          int32_t Nb, char *msg, size_t mlen) {
  PlanColsGeometry g;
  if (!plan_cols_geometry(H, Hkv, Mb, Nb, &g)) return bad(msg, mlen, "invalid dimensions");
  if (bytes < g.total) return bad(msg, mlen, "%zu bytes given, the plan spans %zu", bytes, g.total);
  const int64_t C = (int64_t)H * Nb;
  const int32_t *col_ptr = section(buf, g.off_col_ptr);
  const int32_t *col_order = section(buf, g.off_col_order);
  const int32_t nnz = *section(buf, g.off_nnz);
  const int32_t *row_idx = section(buf, g.off_row_idx);
  if (nnz < 0 || (int64_t)nnz > C * Mb)
    return bad(msg, mlen, "nnz_total = %d is outside [0, %lld]", nnz, (long long)(C * Mb));
  if (!check_ptr(col_ptr, C, Mb, nnz, "col_ptr", msg, mlen)) return false;
  if (!check_lists(col_ptr, row_idx, C, Mb, "row_idx", msg, mlen)) return false;
  return check_perm(col_order, (int64_t)Hkv * Nb, "col_order", msg, mlen);
}

bool check_transpose_host(const void *rows, const void *cols, int32_t H, int32_t Hkv, int32_t Mb,
                          int32_t Nb, char *msg, size_t mlen) {
  PlanGeometry g;
  PlanColsGeometry gc;
  if (!plan_geometry(H, Mb, Nb, &g) || !plan_cols_geometry(H, Hkv, Mb, Nb, &gc))
    return bad(msg, mlen, "invalid dimensions");
  const int32_t *row_ptr = section(rows, g.off_row_ptr);
  const int32_t *col_idx = section(rows, g.off_col_idx);
  const int32_t *col_ptr = section(cols, gc.off_col_ptr);
  const int32_t *row_idx = section(cols, gc.off_row_idx);
  if (*section(rows, g.off_nnz) != *section(cols, gc.off_nnz))
    return bad(msg, mlen, "the plans hold %d and %d live tiles", *section(rows, g.off_nnz),
               *section(cols, gc.off_nnz));
  // Both lists are ascending and checked, so walking the rows in order and
  // each column's list with a cursor visits every tile of the layout once.
  std::vector<int32_t> cursor((size_t)H * Nb);
  for (int64_t c = 0; c < (int64_t)H * Nb; ++c) cursor[(size_t)c] = col_ptr[c];
  for (int32_t h = 0; h < H; ++h)
    for (int32_t m = 0; m < Mb; ++m) {
      const int64_t r = (int64_t)h * Mb + m;
      for (int32_t t = row_ptr[r]; t < row_ptr[r + 1]; ++t) {
        const int64_t c = (int64_t)h * Nb + col_idx[t];
        int32_t &u = cursor[(size_t)c];
        if (u >= col_ptr[c + 1] || row_idx[u] != m)
          return bad(msg, mlen, "tile (head %d, row %d, column %d) is missing from the column plan",
                     h, m, col_idx[t]);
        ++u;
      }
    }
  return true;
}

}  // namespace bsa
