// The device-side preconditions of the paged decode, as one predicate shared
// by the host check (mla_validate_paged_host) and the device check run under
// MLA_VALIDATE=1.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define MLA_HD __host__ __device__
#else
#define MLA_HD
#endif

namespace mla {

// Sequence b is usable by the decode when 0 <= len <= max_seqlen, its tokens
// fit its row of the block table (len <= max_pages * page), and every page it
// uses, block_table[b, k] for k < ceil(len / page), names a page of the pool
// [0, num_pages).  Table entries past the pages a sequence uses are never
// read and may hold anything.
MLA_HD inline bool sequence_ok(const int32_t* bt_row, int32_t len, int32_t max_seqlen,
                               int32_t max_pages, int32_t page, int32_t num_pages) {
  if (len < 0 || len > max_seqlen || (int64_t)len > (int64_t)max_pages * page) return false;
  const int32_t used = (int32_t)(((int64_t)len + page - 1) / page);
  for (int32_t k = 0; k < used; ++k) {
    const int32_t p = bt_row[k];
    if (p < 0 || p >= num_pages) return false;
  }
  return true;
}

}  // namespace mla
