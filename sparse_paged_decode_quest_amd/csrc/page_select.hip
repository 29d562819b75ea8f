// Page lists from page scores: one kSelThreads-thread workgroup per (request, KV head) row.
// The selection rules and their sources are described in select_row.h.
#include "select_row.h"

namespace spd {

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void page_select_kernel(SelectArgs a) {
  __shared__ SelectSmem sm;
  const int b = blockIdx.x / a.num_kv_heads;
  const int h = blockIdx.x % a.num_kv_heads;
  const size_t row = (size_t)b * a.num_kv_heads + h;
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const bool streaming = (a.streaming_mask >> h) & 1ull;
  select_row<KPT>(a, a.scores + row * a.max_pages, n, row, streaming, sm);
}

int launch_page_select(const SelectArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.batch * a.num_kv_heads)), block(kSelThreads);
  switch (select_kpt(a.max_pages)) {
    case 8: hipLaunchKernelGGL(page_select_kernel<8>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(page_select_kernel<32>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(page_select_kernel<0>, grid, block, 0, stream, a); break;
  }
  return 0;
}

}  // namespace spd
