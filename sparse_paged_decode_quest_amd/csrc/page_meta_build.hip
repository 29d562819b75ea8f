// Bulk statistics (every page of every request, at prefill), the pages [first_page, first_page
// + span) of each request, or its last `span` pages (the page the newest token is in, during
// decode): key min / max (page meta) or key mean / variance (page summaries).  Pages here are
// 16-token logical pages, also when physical pages hold several (hierarchical paging).
#include "meta_build.h"

namespace spd {

template <int D, int KVD, bool STATS>
__global__ __launch_bounds__(256) void page_meta_build_kernel(MetaArgs a) {
  const int wave = threadIdx.x / kWave;
  const int b = blockIdx.x / a.blocks_per_req;
  const int item = (blockIdx.x % a.blocks_per_req) * 4 + wave;  // (page offset, head) pair
  if (b >= a.batch) return;
  const int p_off = item / a.num_kv_heads;
  const int h = item % a.num_kv_heads;
  const int len = a.seq_lens[b];
  const int n = row_logical_pages(len, a.max_pages, a.lgs);  // logical pages (hierarchical paging)
  int start = 0, end = n;
  if (a.first_page) {
    start = a.first_page[b];
    if (start < 0) start = 0;
    end = start + a.span < n ? start + a.span : n;
  } else if (a.span < (a.max_pages << a.lgs)) {  // the last `span` pages of the request
    start = n - a.span > 0 ? n - a.span : 0;
  }
  const int p = start + p_off;
  if (p >= end) return;
  if constexpr (STATS) build_page_stats<D, KVD>(a, b, p, h, len);
  else build_page_meta<D, KVD>(a, b, p, h, len);
}

int launch_page_meta_build(const MetaArgs& a, int head_dim, int kv_dtype, hipStream_t stream) {
  dim3 grid((unsigned)(a.batch * a.blocks_per_req)), block(256);
#define SPD_META_CASE(D, K)                                                          \
  if (head_dim == D && kv_dtype == K) {                                              \
    if (a.stats) hipLaunchKernelGGL((page_meta_build_kernel<D, K, true>), grid, block, 0, stream, a);  \
    else hipLaunchKernelGGL((page_meta_build_kernel<D, K, false>), grid, block, 0, stream, a);     \
    return 0;                                                                        \
  }
  SPD_META_CASE(64, SPD_DTYPE_F32)
  SPD_META_CASE(128, SPD_DTYPE_F32)
  SPD_META_CASE(64, SPD_DTYPE_F16)
  SPD_META_CASE(128, SPD_DTYPE_F16)
  SPD_META_CASE(64, SPD_DTYPE_FP8_E4M3FN)
  SPD_META_CASE(128, SPD_DTYPE_FP8_E4M3FN)
#undef SPD_META_CASE
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
