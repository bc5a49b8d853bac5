// Checked mode: device-side validation of the index inputs that the paged kernels take on
// trust (page ids, sequence lengths, selected page lists). Kernels of the hot path read
// through these indices without bounds checks; a caller that wants them verified runs
// ubs_check_paged on the same stream first, and ubs_check_status reports the first
// violation recorded.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace ubs {

// Record the violation (kind, b, index, value, head) unless one is already recorded.
__device__ __forceinline__ void report(int32_t* st, int kind, int b, int idx, int value, int g) {
  if (atomicCAS(&st[0], 0, kind) == 0) {
    st[1] = b;
    st[2] = idx;
    st[3] = value;
    st[4] = g;
  }
}

// Sequence length of b from seq_lens or cu_seqlens; reports and returns -1 if invalid.
__device__ __forceinline__ int seq_len(const CheckArgs& a, int b, bool report_it) {
  int L;
  if (a.cu_seqlens) {
    const int lo = a.cu_seqlens[b], hi = a.cu_seqlens[b + 1];
    if ((b == 0 && lo != 0) || hi < lo) {
      if (report_it) report(a.status, kCheckCuSeqlens, b, b + 1, hi, -1);
      return -1;
    }
    L = hi - lo;
  } else {
    L = a.seq_lens[b];
  }
  if (L < 0 || (int64_t)L > (int64_t)a.max_pages * a.P) {
    if (report_it) report(a.status, kCheckSeqLen, b, 0, L, -1);
    return -1;
  }
  return L;
}

// Thread per (b, j) page-table entry, then per (b, dense g, slot) selected entry.
__global__ __launch_bounds__(256) void check_kernel(const CheckArgs a) {
  const int64_t n_pt = (int64_t)a.B * a.max_pages;
  const int64_t n_sel = a.selected ? (int64_t)a.B * a.dense.n * a.max_selected : 0;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n_pt + n_sel; x += (int64_t)gridDim.x * 256) {
    if (x < n_pt) {
      const int b = (int)(x / a.max_pages), j = (int)(x % a.max_pages);
      const int L = seq_len(a, b, j == 0);
      if (L < 0) continue;
      if ((int64_t)j * a.P >= L) continue;   // past the sequence: never read
      const int p = a.page_table[x];
      if (p < 0 || p >= a.num_pages) report(a.status, kCheckPageId, b, j, p, -1);
    } else {
      const int64_t y = x - n_pt;
      const int slot = (int)(y % a.max_selected);
      const int64_t bd = y / a.max_selected;
      const int b = (int)(bd / a.dense.n), g = a.dense.h[bd % a.dense.n];
      const int L = seq_len(a, b, false);
      if (L < 0) continue;
      const int n_pages = (L + a.P - 1) / a.P;
      const int64_t bg = (int64_t)b * a.Hkv + g;
      const int n = a.num_selected[bg];
      if (n < 0 || n > a.max_selected || n > n_pages) {
        if (slot == 0) report(a.status, kCheckNumSelected, b, 0, n, g);
        continue;
      }
      if (slot >= n) continue;
      const int32_t* row = a.selected + bg * a.max_selected;
      const int s = row[slot];
      if (s < 0 || s >= n_pages) report(a.status, kCheckSelected, b, slot, s, g);
      else if (slot > 0 && row[slot - 1] >= s) report(a.status, kCheckSelectedOrder, b, slot, s, g);
    }
  }
}

hipError_t launch_check(const CheckArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.max_pages + (a.selected ? (int64_t)a.B * a.dense.n * a.max_selected : 0);
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ubs
