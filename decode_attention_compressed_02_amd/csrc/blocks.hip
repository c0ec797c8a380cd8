// blocks.hip -- whole-block copies in a paged sparse pool: the device half of
// copy-on-write ("Reuse, Evict, or Limit Earlier Context" section 1.3: before
// a sequence writes into a block other sequences still reference, the block
// is copied to a fresh one that the writer then owns).
//
// One workgroup of 256 threads per (copy, plane) streams the block's bytes
// with 16-byte accesses; a block of a plane is H_kv x block_size x k_stride
// entries (k_stride bytes per row for the index planes, k_stride times the
// value width for the value planes), always a multiple of 16 bytes.
#include "swan_internal.h"

namespace swan {

typedef uint32_t cpy_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_copy_blocks(CopyBlocksArgs a)
{
    const int i = blockIdx.x, plane = blockIdx.y;
    const int src = a.src[i], dst = a.dst[i];
    // ids outside the pool are a caller error: the pair is skipped
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst) return;
    uint8_t *base = plane == 0 ? a.kidx : plane == 1 ? a.vidx : plane == 2 ? a.kval : a.vval;
    const int64_t idx_bytes = (plane & 1) ? a.block_bytes_vidx : a.block_bytes_kidx; // planes 0, 2 keys; 1, 3 values
    const int64_t bytes = plane < 2 ? idx_bytes : a.vbytes * idx_bytes;
    const cpy_u32x4 *s = (const cpy_u32x4 *)(base + (int64_t)src * bytes);
    cpy_u32x4 *d = (cpy_u32x4 *)(base + (int64_t)dst * bytes);
    for (int64_t j = threadIdx.x; j < bytes / 16; j += 256) d[j] = s[j];
}

hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_copy_blocks, dim3(a.count, 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
