// Row-statistics pass: its workgroup size, argument block and launchers.
// The row kernels (sv_rows.hip) see only this header and sv_device.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kRowThreads = 256;    // row-statistics workgroup
constexpr int kTreeMaxNodes = 256;  // token-tree nodes

// Rows of one launch of the row-statistics pass, listed explicitly: every
// sequence reads the same R rows, row[j] = (1 << 15 if it is a draft row) |
// its position in the sequence's target (or draft) rows.  Only the rows a
// call needs are listed (a token tree's leaf draft rows are not), so the grid
// holds no workgroup that would exit at once.  Workgroup (b, j, seg) =
// blockIdx (b * R + j) * S + seg reduces segment seg of that row and writes
// part[(b * R_out + slot) * S + seg], slot = i for target row i and
// d_slot0 + i for draft row i.  The kernel reads its row from this list
// (a load from the argument block); that measured 1.6% faster on the 1.1 GB
// window pass than deriving the row from the index, for a reason not
// established (delaying each workgroup's start by the same time does not
// reproduce it).
constexpr int kMaxLaunchRows = 2 * kTreeMaxNodes;
constexpr uint16_t kDraftRow = 0x8000;

struct RowSet {
  const char *t;
  int64_t t_stride_bytes;
  const char *d;
  int64_t d_stride_bytes;
  const int32_t *window_len;      // window calls: rows past the window are skipped
  const int32_t *status;          // early exit: only sequences still verifying
  int32_t *arrive;                // zeroed per sequence by its first workgroup (split draw)
  int32_t B, R;                   // sequences, listed rows per sequence
  int32_t R_out, d_slot0;         // row results per sequence, slot of draft row 0
  int32_t gamma;
  int32_t V, S, seg_len;
  uint16_t row[kMaxLaunchRows];

  void add_target(int lo, int hi) {
    for (int i = lo; i < hi; ++i) row[R++] = static_cast<uint16_t>(i);
  }
  void add_draft(int lo, int hi) {
    for (int i = lo; i < hi; ++i) row[R++] = static_cast<uint16_t>(kDraftRow | i);
  }
};

// Per-sequence state of the early-exit window (workspace): verifying, or done.
constexpr int32_t kSeqVerifying = -2;

// Grid: B * R * S workgroups, formed from rs.
void launch_row_stats(int dtype, bool argmax, const RowSet &rs, float2 *part, hipStream_t st);
int probe_blocks(size_t bytes);
void launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st);

}  // namespace sv
