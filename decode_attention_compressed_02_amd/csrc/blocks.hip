// blocks.hip -- whole-block copies in a paged sparse pool: the device half of
// copy-on-write ("Reuse, Evict, or Limit Earlier Context" section 1.3: before
// a sequence writes into a block other sequences still reference, the block
// is copied to a fresh one that the writer then owns).
//
// One workgroup of 256 threads per (copy, plane) streams the block's bytes
// with 16-byte accesses; a block of a plane is H_kv x block_size x k_stride
// entries (k_stride bytes per row for the index planes, k_stride times the
// value width for the value planes), always a multiple of 16 bytes.
//
// k_paged_update does the same copies, and the block-table writes of a step,
// from pairs carried in its launch arguments: the host's bookkeeping reaches
// the device without a host-to-device copy, whose completion the next kernel
// would otherwise have to wait for.
#include "swan_internal.h"

namespace swan {

typedef uint32_t cpy_u32x4 __attribute__((ext_vector_type(4)));

// plane 0 / 1: key / value indices, 2 / 3: key / value values
__device__ __forceinline__ void copy_block_plane(const uint8_t *const base[4], int64_t bytes_kidx, int64_t bytes_vidx,
                                                 int vbytes, int plane, int src, int dst)
{
    const int64_t idx_bytes = (plane & 1) ? bytes_vidx : bytes_kidx;
    const int64_t bytes = plane < 2 ? idx_bytes : vbytes * idx_bytes;
    const cpy_u32x4 *s = (const cpy_u32x4 *)(base[plane] + (int64_t)src * bytes);
    cpy_u32x4 *d = (cpy_u32x4 *)(const_cast<uint8_t *>(base[plane]) + (int64_t)dst * bytes);
    for (int64_t j = threadIdx.x; j < bytes / 16; j += 256) d[j] = s[j];
}

__global__ __launch_bounds__(256) void k_copy_blocks(CopyBlocksArgs a)
{
    const int i = blockIdx.x, plane = blockIdx.y;
    const int src = a.src[i], dst = a.dst[i];
    // ids outside the pool are a caller error: the pair is skipped
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst) return;
    const uint8_t *const base[4] = {a.kidx, a.vidx, a.kval, a.vval};
    copy_block_plane(base, a.block_bytes_kidx, a.block_bytes_vidx, a.vbytes, plane, src, dst);
}

// the entries and pairs were checked on the host
__global__ __launch_bounds__(256) void k_paged_update(PagedUpdateArgs a)
{
    if (blockIdx.x == 0) {
        for (int t = threadIdx.x; t < a.n_entries; t += 256) a.table[a.entry[t][0]] = a.entry[t][1];
        return;
    }
    const int i = (blockIdx.x - 1) / 4, plane = (blockIdx.x - 1) % 4;
    const uint8_t *const base[4] = {a.kidx, a.vidx, a.kval, a.vval};
    copy_block_plane(base, a.block_bytes_kidx, a.block_bytes_vidx, a.vbytes, plane, a.copy[i][0], a.copy[i][1]);
}

hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_copy_blocks, dim3(a.count, 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_paged_update(const PagedUpdateArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_paged_update, dim3(1 + 4 * a.n_copies), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace swan
