// Row-statistics pass: its workgroup size, argument block and launchers.
// The row kernels (sv_rows.hip) see only this header and sv_device.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kRowThreads = 256;    // row-statistics workgroup
constexpr int kTreeMaxNodes = 256;  // token-tree nodes; the draft-row mask below has one bit per node

// Rows of one launch of the row-statistics pass.  Sequence b owns rows_t
// target rows (t0, t0+1, ...) then rows_d draft rows (d0, d0+1, ...);
// workgroup (b, j, seg) reduces segment seg of row j of its sequence and
// writes part[(b * R_out + slot) * S + seg], slot = t_slot0 + j for target
// rows and d_slot0 + (j - rows_t) for draft rows.
struct RowSet {
  const char *t;
  int64_t t_stride_bytes;
  const char *d;
  int64_t d_stride_bytes;
  int32_t rows_t, rows_d;
  int32_t t0, d0;                 // first target / draft row of the launch
  int32_t R_out, t_slot0, d_slot0;
  const int32_t *window_len;      // window calls: rows past the window are skipped
  const int32_t *status;          // early exit: only sequences still verifying
  int32_t gamma;
  int32_t V, S, seg_len;
  uint64_t dmask[kTreeMaxNodes / 64];  // draft row i read iff bit i is set
};

// Per-sequence state of the early-exit window (workspace): verifying, or done.
constexpr int32_t kSeqVerifying = -2;

void launch_row_stats(int dtype, bool argmax, const RowSet &rs, int64_t blocks, float2 *part, hipStream_t st);
int probe_blocks(size_t bytes);
void launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st);

}  // namespace sv
