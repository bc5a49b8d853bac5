// append_kv: write the K/V rows of newly decoded (or prefilled) tokens into the paged
// cache (the step beside decode in the LServe serving loop; the paged layout of the
// blog's "LServe -- Decode Phase": token t of sequence b at row t % P of physical page
// page_table[b][t / P]). One thread per 16-byte piece of a row: loads and stores are
// coalesced within each D-element row. The page summaries of the touched sub-pages are
// refreshed afterwards by the bounds kernel in its update form.
#include "common.h"
#include "launch.h"

namespace ubs {

template <int D>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  constexpr int CPR = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.n_new * a.Hkv * CPR;
  if (idx >= total) return;
  const int c = (int)(idx % CPR);
  int64_t rest = idx / CPR;
  const int g = (int)(rest % a.Hkv);
  rest /= a.Hkv;
  const int x = (int)(rest % a.n_new);
  const int b = (int)(rest / a.n_new);
  const int t = a.seq_lens[b] + x;
  const int page = a.page_table[(int64_t)b * a.max_pages + t / a.P];
  const int64_t src = (((int64_t)b * a.n_new + x) * a.Hkv + g) * D + c * 8;
  const int64_t dst = (((int64_t)page * a.Hkv + g) * a.P + t % a.P) * D + c * 8;
  st16(a.k_cache + dst, ld16(a.k_new + src));
  st16(a.v_cache + dst, ld16(a.v_new + src));
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.n_new * a.Hkv * (a.D / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
#define UBS_APPEND(DD)                                                                   \
  if (a.D == DD) {                                                                       \
    hipLaunchKernelGGL((append_kernel<DD>), dim3((unsigned)blocks), dim3(256), 0, s, a); \
    return hipGetLastError();                                                            \
  }
  UBS_APPEND(64) UBS_APPEND(128)
#undef UBS_APPEND
  return hipErrorInvalidValue;
}

}  // namespace ubs
