// Page copies for copy-on-write: a sequence about to write into a page that
// another sequence still holds gets a fresh page, and this kernel copies the
// shared page's contents there first (the snapshot of libmir-metal
// src/engine/kv/paged/mod.rs shares pages by reference counts; the copy on a
// later write into a shared, partly filled page is the step it implies).
//
// A page of one layer is contiguous in both page arrays (K [P][Hkv][bs][D],
// V [P][Hkv][D][bs]: Hkv slabs back to back), and so are its int8 scales, so
// each (pair, layer) is two or four plain block copies.  One workgroup per
// (pair, layer); 16-byte accesses when the block size allows.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <typename T>
__device__ __forceinline__ void block_copy(const char* src, char* dst, int64_t bytes) {
  const T* s = reinterpret_cast<const T*>(src);
  T* d = reinterpret_cast<T*>(dst);
  const int64_t n = bytes / (int64_t)sizeof(T);
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

__global__ __launch_bounds__(256) void copy_pages_kernel(CopyArgs a) {
  const int pair = blockIdx.x, layer = blockIdx.y;
  const int src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
  if (src < 0 || src >= a.n_pages || dst < 0 || dst >= a.n_pages) {
    if (threadIdx.x == 0 && layer == 0) report(a.status, PKV_DEV_WRITE_PAGE);
    return;
  }
  const int64_t s0 = (int64_t)layer * a.n_pages + src, d0 = (int64_t)layer * a.n_pages + dst;
  const int64_t pb = a.page_bytes;
  const char* k = static_cast<const char*>(a.k_pages);
  const char* v = static_cast<const char*>(a.v_pages);
  char* kw = static_cast<char*>(a.k_pages);
  char* vw = static_cast<char*>(a.v_pages);
  if (pb % 16 == 0) {
    block_copy<uint4>(k + s0 * pb, kw + d0 * pb, pb);
    block_copy<uint4>(v + s0 * pb, vw + d0 * pb, pb);
  } else {
    block_copy<uint32_t>(k + s0 * pb, kw + d0 * pb, pb);
    block_copy<uint32_t>(v + s0 * pb, vw + d0 * pb, pb);
  }
  if (a.k_scales) {
    const int64_t sb = a.scale_bytes;
    block_copy<uint32_t>(reinterpret_cast<const char*>(a.k_scales) + s0 * sb,
                         reinterpret_cast<char*>(a.k_scales) + d0 * sb, sb);
    block_copy<uint32_t>(reinterpret_cast<const char*>(a.v_scales) + s0 * sb,
                         reinterpret_cast<char*>(a.v_scales) + d0 * sb, sb);
  }
}

}  // namespace

hipError_t launch_copy_pages(const CopyArgs& a, const Launch& l) {
  if (a.n_pairs <= 0) return hipSuccess;
  return launch1(copy_pages_kernel, dim3(a.n_pairs, a.n_layers), dim3(256), 0, l, a);
}

}  // namespace pkv
