// abi.hip -- the extern "C" entry points declared in swan.h: host-side
// validation (before anything is enqueued), split planning and dispatch.
#include <stdarg.h>
#include <stdio.h>

#include "swan_internal.h"

#include <mutex>
#include <vector>

namespace {

thread_local char g_err[512] = "";

swan_status fail(swan_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

swan_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return SWAN_OK;
    return fail(SWAN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int32_t row_stride(int32_t k)
{
    int32_t s = 8;
    while (s < k) s *= 2;
    return s;
}

swan_status check_dims(const swan_dims *d)
{
    if (!d) return fail(SWAN_ERR_INVALID_ARG, "dims is NULL");
    if (d->d_h != swan::kD) return fail(SWAN_ERR_UNSUPPORTED, "d_h = %d, only 128 is supported", d->d_h);
    if (d->B < 1 || d->N_h < 1 || d->H_kv < 1)
        return fail(SWAN_ERR_INVALID_ARG, "B, N_h, H_kv must be >= 1 (got %d, %d, %d)", d->B, d->N_h, d->H_kv);
    if (d->B > 65535 || d->H_kv > 65535) return fail(SWAN_ERR_INVALID_ARG, "B and H_kv must be <= 65535");
    if (d->N_h % d->H_kv) return fail(SWAN_ERR_INVALID_ARG, "N_h = %d is not a multiple of H_kv = %d", d->N_h, d->H_kv);
    const int g = d->N_h / d->H_kv;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(SWAN_ERR_UNSUPPORTED, "GQA group g = %d, supported: 1, 2, 4, 8", g);
    if (d->k < 1 || d->k > d->d_h) return fail(SWAN_ERR_INVALID_ARG, "k = %d outside 1..%d", d->k, d->d_h);
    if (d->R < 0) return fail(SWAN_ERR_INVALID_ARG, "R = %d < 0", d->R);
    if (d->block_size < 0) return fail(SWAN_ERR_INVALID_ARG, "block_size < 0");
    if (d->block_size > 0) {
        if (d->max_blocks < 1 || d->num_blocks < 1)
            return fail(SWAN_ERR_INVALID_ARG, "paged layout needs max_blocks >= 1 and num_blocks >= 1");
        // table slots (b * max_blocks + j) travel as int32 and a sequence's
        // sparse rows are counted in int32 (positions are int32)
        if ((int64_t)d->B * d->max_blocks > INT32_MAX)
            return fail(SWAN_ERR_UNSUPPORTED, "B * max_blocks = %lld block-table slots, at most %d are supported",
                        (long long)d->B * d->max_blocks, INT32_MAX);
        if ((int64_t)d->max_blocks * d->block_size > INT32_MAX)
            return fail(SWAN_ERR_UNSUPPORTED, "max_blocks * block_size = %lld sparse rows a sequence, at most %d are "
                                              "supported", (long long)d->max_blocks * d->block_size, INT32_MAX);
    } else if (d->n_cap < 0) {
        return fail(SWAN_ERR_INVALID_ARG, "n_cap < 0");
    }
    if (d->split_tokens < 0 || d->split_tokens % 64)
        return fail(SWAN_ERR_INVALID_ARG, "split_tokens = %d must be 0 or a positive multiple of 64", d->split_tokens);
    if (d->value_format != SWAN_VALUES_FP16 && d->value_format != SWAN_VALUES_FP8_E4M3)
        return fail(SWAN_ERR_UNSUPPORTED, "value_format = %d, supported: 0 (fp16), 1 (fp8 E4M3)", d->value_format);
    if (d->k_v < 0 || d->k_v > d->d_h) return fail(SWAN_ERR_INVALID_ARG, "k_v = %d outside 0..%d", d->k_v, d->d_h);
    if (d->k_v > 0) {
        const int ks = row_stride(d->k), ksv = row_stride(d->k_v);
        if (ksv != ks && ksv != 2 * ks && 2 * ksv != ks)
            return fail(SWAN_ERR_UNSUPPORTED, "k = %d and k_v = %d: stored row widths %d and %d, supported when equal "
                                              "or one twice the other", d->k, d->k_v, ks, ksv);
    }
    if (d->layers < 0 || (d->layers > 1 && d->B % d->layers))
        return fail(SWAN_ERR_INVALID_ARG, "layers = %d: must be 0 or 1 (one layer) or divide B = %d", d->layers, d->B);
    if (d->block_size == 0) {
        // the decode reads a unit's rows of each plane through one buffer
        // resource, whose byte range is 32-bit
        const int ks = row_stride(d->k), ksv = row_stride(d->k_v > 0 ? d->k_v : d->k);
        const int64_t unit_plane = (int64_t)d->n_cap * (ks > ksv ? ks : ksv) *
                                   (d->value_format == SWAN_VALUES_FP8_E4M3 ? 1 : 2);
        if (unit_plane >= ((int64_t)1 << 32))
            return fail(SWAN_ERR_UNSUPPORTED, "n_cap = %d: %lld bytes of one (sequence, kv head) value plane, below "
                                              "2^32 are supported", d->n_cap, (long long)unit_plane);
    }
    return SWAN_OK;
}

int value_bytes(const swan_dims *d) { return d->value_format == SWAN_VALUES_FP8_E4M3 ? 1 : 2; }
// sequences of one layer: the batch holds `layers` layers' sequences, layer-major
int layer_seqs(const swan_dims *d) { return d->layers > 1 ? d->B / d->layers : d->B; }
// kept value coordinates (k unless keys and values keep different counts)
int kept_v(const swan_dims *d) { return d->k_v > 0 ? d->k_v : d->k; }
int row_bytes(const swan_dims *d)
{
    return swan::sparse_row_bytes(row_stride(d->k), row_stride(kept_v(d)), value_bytes(d));
}

int64_t row_cap(const swan_dims *d)
{
    return d->block_size > 0 ? (int64_t)d->max_blocks * d->block_size : (int64_t)d->n_cap;
}

swan_status check_cache(const swan_dims *d, const swan_cache *c, bool need_buf)
{
    if (!c) return fail(SWAN_ERR_INVALID_ARG, "cache is NULL");
    if (!c->k_idx || !c->k_val || !c->v_idx || !c->v_val) return fail(SWAN_ERR_INVALID_ARG, "sparse plane is NULL");
    if (need_buf && d->R > 0 && (!c->k_buf || !c->v_buf)) return fail(SWAN_ERR_INVALID_ARG, "dense buffer is NULL");
    if (d->block_size > 0 && !c->block_table) return fail(SWAN_ERR_INVALID_ARG, "paged layout needs block_table");
    return SWAN_OK;
}

swan::SparseGeom geom(const swan_dims *d, const swan_cache *c)
{
    swan::SparseGeom g;
    g.H = d->H_kv;
    g.ks = row_stride(d->k);
    g.ks_v = row_stride(kept_v(d));
    g.n_cap = d->n_cap;
    g.bs = d->block_size;
    g.max_blocks = d->max_blocks;
    g.num_blocks = d->num_blocks;
    g.vbytes = value_bytes(d);
    g.bt = d->block_size > 0 ? c->block_table : nullptr;
    return g;
}

struct Plan {
    int W; // waves of the split pass
};

// The split pass runs W waves over nearly equal ranges of the batch's work
// rows (unit_work: sparse rows plus buffered tokens weighted by their bytes);
// max_pos bounds every unit, and the kernels use active_waves() <= W of them
// for the batch at hand.  The automatic plan launches one wave per
// resident-wave slot of the chip (the split kernel's LDS footprint and
// register budget decide how many fit on a CU), fewer when the longest batch
// max_pos allows has under kMinWaveRows work rows per wave; split_tokens sets
// the rows per wave instead.
Plan plan(const swan_dims *d, int32_t max_pos)
{
    const int g = d->N_h / d->H_kv, ks = row_stride(d->k), ksv = row_stride(kept_v(d));
    const int64_t total_max = (int64_t)d->B * d->H_kv * swan::unit_work(max_pos, d->R, row_cap(d), row_bytes(d)).len;
    int slots = INT32_MAX;
    if (d->split_tokens == 0) {
        slots = swan::kCUs * swan::split_waves_per_cu(g, ks > ksv ? ks : ksv);
    }
    Plan p;
    p.W = (int)swan::active_waves(total_max, slots, d->split_tokens);
    return p;
}

// partials: one per (piece, query head of the group); a piece is a wave's
// share of one unit, and there are at most W + B H_kv of them
size_t partial_count(const swan_dims *d, const Plan &p)
{
    return ((size_t)p.W + (size_t)d->B * d->H_kv) * (size_t)(d->N_h / d->H_kv);
}

size_t workspace_bytes(const swan_dims *d, const Plan &p)
{
    return partial_count(d, p) * (swan::kD + 2) * sizeof(float);
}

// the checks of a decode call other than its workspace's, and its plan
swan_status check_decode_plan(const swan_dims *d, const swan_cache *c, const int32_t *pos, int32_t max_pos, Plan *out)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if (c && (st = check_cache(d, c, true))) return st;
    if (!pos) return fail(SWAN_ERR_INVALID_ARG, "pos is NULL");
    const int64_t n_max = (int64_t)max_pos + 1 - d->R;
    if (n_max > row_cap(d))
        return fail(SWAN_ERR_CAPACITY, "max_pos = %d needs %lld sparse rows, capacity is %lld", max_pos,
                    (long long)n_max, (long long)row_cap(d));
    *out = plan(d, max_pos);
    if (out->W > swan::kMaxWaves)
        return fail(SWAN_ERR_INVALID_ARG, "split_tokens = %d gives %d waves, at most %d are supported", d->split_tokens,
                    out->W, swan::kMaxWaves);
    return SWAN_OK;
}

swan_status check_decode(const swan_dims *d, const swan_cache *c, const int32_t *pos, int32_t max_pos,
                         const void *ws, size_t ws_bytes, Plan *out)
{
    swan_status st = check_decode_plan(d, c, pos, max_pos, out);
    if (st) return st;
    if (!ws) return fail(SWAN_ERR_INVALID_ARG, "workspace is NULL");
    if (ws_bytes < workspace_bytes(d, *out))
        return fail(SWAN_ERR_INVALID_ARG, "workspace of %zu bytes, need %zu", ws_bytes, workspace_bytes(d, *out));
    return SWAN_OK;
}

// The partials of swan_decode_attn_noalloc: a file-scope device array, one
// copy on every GPU the library runs on, held until the process ends.  Host
// code never uses its name as an address (on the host the name stands for a
// host-side shadow): the address on each device comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kScratchBytes = SWAN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices]; // address of `scratch` per device, null until looked up

// the scratch array of the device `stream` runs on, which must be the
// current device (the symbol's address is looked up on the current device)
swan_status scratch_for(hipStream_t stream, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (stream) {
        hipDevice_t sdev = -1;
        if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return hip_status(e, "hipStreamGetDevice");
        if ((int)sdev != dev)
            return fail(SWAN_ERR_INVALID_ARG, "stream belongs to device %d, the current device is %d", (int)sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SWAN_ERR_UNSUPPORTED, "device %d: the no-allocation scratch serves devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
            return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SWAN_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SWAN_OK;
}

} // namespace

namespace swan {
hipError_t launch_mfma_f64(double x, int waves, int iters, double *sink, hipStream_t s); // measure.hip
}

extern "C" {

const char *swan_status_str(swan_status s)
{
    switch (s) {
    case SWAN_OK: return "SWAN_OK";
    case SWAN_ERR_INVALID_ARG: return "SWAN_ERR_INVALID_ARG";
    case SWAN_ERR_UNSUPPORTED: return "SWAN_ERR_UNSUPPORTED";
    case SWAN_ERR_CAPACITY: return "SWAN_ERR_CAPACITY";
    case SWAN_ERR_HIP: return "SWAN_ERR_HIP";
    }
    return "SWAN_ERR_UNKNOWN";
}

const char *swan_last_error(void) { return g_err; }

int32_t swan_row_stride(int32_t k) { return row_stride(k); }

swan_status swan_cache_bytes(const swan_dims *d, size_t out[5])
{
    swan_status st = check_dims(d);
    if (st) return st;
    if (!out) return fail(SWAN_ERR_INVALID_ARG, "out is NULL");
    const size_t ks = (size_t)row_stride(d->k), ksv = (size_t)row_stride(kept_v(d));
    const size_t rows = d->block_size > 0 ? (size_t)d->num_blocks * d->H_kv * d->block_size
                                          : (size_t)d->B * d->H_kv * d->n_cap;
    out[0] = rows * ks;
    out[1] = rows * ks * (size_t)value_bytes(d);
    out[2] = rows * ksv;
    out[3] = rows * ksv * (size_t)value_bytes(d);
    out[4] = (size_t)d->B * d->H_kv * d->R * swan::kD * 2;
    return SWAN_OK;
}

swan_status swan_project_qk(const swan_dims *d, const float *q, const float *k, const int32_t *pos,
                            const float *P_qk, float rope_base, float *q_hat, uint16_t *k_hat, void *stream)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if (!q || !k || !pos || !P_qk || !q_hat || !k_hat) return fail(SWAN_ERR_INVALID_ARG, "NULL array argument");
    if (!(rope_base > 1.0f)) return fail(SWAN_ERR_INVALID_ARG, "rope_base must be > 1");
    swan::ProjectArgs a{d->B, d->N_h, d->H_kv, q, k, pos, P_qk, rope_base, q_hat, k_hat, layer_seqs(d)};
    return hip_status(swan::launch_project(a, (hipStream_t)stream), "swan_project_qk launch");
}

swan_status swan_append_evict(const swan_dims *d, const swan_cache *c, const int32_t *pos, int32_t max_pos,
                              const uint16_t *k_hat, const float *v_hat, void *stream)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if ((st = check_cache(d, c, true))) return st;
    if (!pos || !k_hat || !v_hat) return fail(SWAN_ERR_INVALID_ARG, "NULL array argument");
    const int64_t row = d->R > 0 ? (int64_t)max_pos - d->R : (int64_t)max_pos; // newest row written
    if (row >= row_cap(d))
        return fail(SWAN_ERR_CAPACITY, "max_pos = %d writes sparse row %lld, capacity is %lld", max_pos,
                    (long long)row, (long long)row_cap(d));
    swan::AppendArgs a;
    a.B = d->B;
    a.H = d->H_kv;
    a.R = d->R;
    a.k = d->k;
    a.k_v = kept_v(d);
    a.geom = geom(d, c);
    a.kidx = c->k_idx;
    a.vidx = c->v_idx;
    a.kval = (uint8_t *)c->k_val;
    a.vval = (uint8_t *)c->v_val;
    a.kbuf = c->k_buf;
    a.vbuf = c->v_buf;
    a.pos = pos;
    a.k_hat = k_hat;
    a.v_hat = v_hat;
    return hip_status(swan::launch_append(a, (hipStream_t)stream), "swan_append_evict launch");
}

swan_status swan_project_append(const swan_dims *d, const swan_cache *c, const float *q, const float *k,
                                const float *v_hat, const int32_t *pos, int32_t max_pos, const float *P_qk,
                                float rope_base, float *q_hat, uint16_t *k_hat, void *stream)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if ((st = check_cache(d, c, true))) return st;
    if (!q || !k || !v_hat || !pos || !P_qk || !q_hat || !k_hat) return fail(SWAN_ERR_INVALID_ARG, "NULL array argument");
    if (!(rope_base > 1.0f)) return fail(SWAN_ERR_INVALID_ARG, "rope_base must be > 1");
    const int64_t row = d->R > 0 ? (int64_t)max_pos - d->R : (int64_t)max_pos;
    if (row >= row_cap(d))
        return fail(SWAN_ERR_CAPACITY, "max_pos = %d writes sparse row %lld, capacity is %lld", max_pos,
                    (long long)row, (long long)row_cap(d));
    swan::ProjectArgs p{d->B, d->N_h, d->H_kv, q, k, pos, P_qk, rope_base, q_hat, k_hat, layer_seqs(d)};
    swan::AppendArgs a;
    a.B = d->B;
    a.H = d->H_kv;
    a.R = d->R;
    a.k = d->k;
    a.k_v = kept_v(d);
    a.geom = geom(d, c);
    a.kidx = c->k_idx;
    a.vidx = c->v_idx;
    a.kval = (uint8_t *)c->k_val;
    a.vval = (uint8_t *)c->v_val;
    a.kbuf = c->k_buf;
    a.vbuf = c->v_buf;
    a.pos = pos;
    a.k_hat = k_hat;
    a.v_hat = v_hat;
    return hip_status(swan::launch_project_append(p, a, (hipStream_t)stream), "swan_project_append launch");
}

swan_status swan_project_append_paged(const swan_dims *d, const swan_cache *c, const float *q, const float *k,
                                      const float *v_hat, const int32_t *pos, int32_t max_pos, const float *P_qk,
                                      float rope_base, float *q_hat, uint16_t *k_hat, int32_t *block_table,
                                      const int32_t *entries, int32_t n_entries, const int32_t *copies,
                                      int32_t n_copies, void *stream)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if (d->block_size <= 0)
        return fail(SWAN_ERR_INVALID_ARG, "swan_project_append_paged needs the paged layout (block_size > 0)");
    if ((st = check_cache(d, c, true))) return st;
    if (!block_table || block_table != c->block_table)
        return fail(SWAN_ERR_INVALID_ARG, "block_table must be the table cache->block_table points at");
    if (n_entries < 0 || n_copies < 0) return fail(SWAN_ERR_INVALID_ARG, "negative count");
    if ((n_entries > 0 && !entries) || (n_copies > 0 && !copies)) return fail(SWAN_ERR_INVALID_ARG, "NULL pair array");
    const int64_t n_slots = (int64_t)d->B * d->max_blocks;
    for (int32_t i = 0; i < n_entries; ++i) {
        const int32_t at = entries[2 * i], id = entries[2 * i + 1];
        if (at < 0 || at >= n_slots || id < -1 || id >= d->num_blocks)
            return fail(SWAN_ERR_INVALID_ARG, "entry %d = (%d, %d): slot outside [0, %lld) or block outside [-1, %d)", i,
                        at, id, (long long)n_slots, d->num_blocks);
        // the one-launch path reads each append's block from these entries: at
        // most one may set a slot (checked where that path is taken)
        if (n_entries <= swan::kFusedEntries)
            for (int32_t j = 0; j < i; ++j)
                if (entries[2 * j] == at)
                    return fail(SWAN_ERR_INVALID_ARG, "entries %d and %d write the same slot %d", j, i, at);
    }
    for (int32_t i = 0; i < n_copies; ++i) {
        const int32_t src = copies[3 * i], dst = copies[3 * i + 1], skip = copies[3 * i + 2];
        if (src < 0 || src >= d->num_blocks || dst < 0 || dst >= d->num_blocks || src == dst)
            return fail(SWAN_ERR_INVALID_ARG, "copy %d = (%d, %d): ids outside [0, %d) or equal", i, src, dst,
                        d->num_blocks);
        if (skip < -1 || skip >= d->block_size)
            return fail(SWAN_ERR_INVALID_ARG, "copy %d: skip row %d outside [-1, %d)", i, skip, d->block_size);
    }
    if (!q || !k || !v_hat || !pos || !P_qk || !q_hat || !k_hat) return fail(SWAN_ERR_INVALID_ARG, "NULL array argument");
    if (!(rope_base > 1.0f)) return fail(SWAN_ERR_INVALID_ARG, "rope_base must be > 1");
    const int64_t row = d->R > 0 ? (int64_t)max_pos - d->R : (int64_t)max_pos;
    if (row >= row_cap(d))
        return fail(SWAN_ERR_CAPACITY, "max_pos = %d writes sparse row %lld, capacity is %lld", max_pos,
                    (long long)row, (long long)row_cap(d));
    if (n_entries > swan::kFusedEntries || n_copies > swan::kFusedCopies) {
        // more than one launch carries: the table update first, then the step's
        // projection and append (same results, one more launch).  Every check
        // of swan_project_append has passed above, so once the update (which
        // validates before it enqueues) has launched, the append cannot fail
        // validation.
        std::vector<int32_t> pairs((size_t)2 * n_copies);
        for (int32_t i = 0; i < n_copies; ++i) {
            pairs[2 * i] = copies[3 * i];
            pairs[2 * i + 1] = copies[3 * i + 1];
        }
        if ((st = swan_paged_update(d, c, block_table, entries, n_entries, pairs.data(), n_copies, stream))) return st;
        return swan_project_append(d, c, q, k, v_hat, pos, max_pos, P_qk, rope_base, q_hat, k_hat, stream);
    }
    swan::ProjectArgs p{d->B, d->N_h, d->H_kv, q, k, pos, P_qk, rope_base, q_hat, k_hat, layer_seqs(d)};
    swan::AppendArgs a;
    a.B = d->B;
    a.H = d->H_kv;
    a.R = d->R;
    a.k = d->k;
    a.k_v = kept_v(d);
    a.geom = geom(d, c);
    a.kidx = c->k_idx;
    a.vidx = c->v_idx;
    a.kval = (uint8_t *)c->k_val;
    a.vval = (uint8_t *)c->v_val;
    a.kbuf = c->k_buf;
    a.vbuf = c->v_buf;
    a.pos = pos;
    a.k_hat = k_hat;
    a.v_hat = v_hat;
    swan::StepUpdateArgs u;
    u.n_entries = n_entries;
    u.n_copies = n_copies;
    u.table = block_table;
    for (int32_t i = 0; i < n_entries; ++i) {
        u.entry[i][0] = entries[2 * i];
        u.entry[i][1] = entries[2 * i + 1];
    }
    for (int32_t i = 0; i < n_copies; ++i)
        for (int t = 0; t < 3; ++t) u.copy[i][t] = copies[3 * i + t];
    return hip_status(swan::launch_project_append_paged(p, a, u, (hipStream_t)stream),
                      "swan_project_append_paged launch");
}

size_t swan_decode_workspace_bytes(const swan_dims *d, int32_t max_pos)
{
    if (check_dims(d)) return 0;
    return workspace_bytes(d, plan(d, max_pos));
}

int32_t swan_decode_num_splits(const swan_dims *d, int32_t max_pos)
{
    if (check_dims(d)) return -1;
    return plan(d, max_pos).W;
}

static swan::SplitArgs split_args(const swan_dims *d, const swan_cache *c, const Plan &p, const int32_t *pos,
                                  const float *q_hat, void *ws)
{
    swan::SplitArgs a;
    a.B = d->B;
    a.N_h = d->N_h;
    a.H = d->H_kv;
    a.R = d->R;
    a.W = p.W;
    a.split_tokens = d->split_tokens;
    a.k = d->k;
    a.k_v = kept_v(d);
    a.row_cap = (int)row_cap(d);
    a.geom = geom(d, c);
    a.pos = pos;
    a.q_hat = q_hat;
    a.kidx = c->k_idx;
    a.vidx = c->v_idx;
    a.kval = (uint8_t *)c->k_val;
    a.vval = (uint8_t *)c->v_val;
    a.kbuf = c->k_buf;
    a.vbuf = c->v_buf;
    a.part_o = (float *)ws;
    a.part_ml = (float *)ws + partial_count(d, p) * swan::kD;
    return a;
}

swan_status swan_decode_split(const swan_dims *d, const swan_cache *c, const int32_t *pos, int32_t max_pos,
                              const float *q_hat, void *ws, size_t ws_bytes, void *stream)
{
    Plan p;
    swan_status st = check_decode(d, c, pos, max_pos, ws, ws_bytes, &p);
    if (st) return st;
    if (!c) return fail(SWAN_ERR_INVALID_ARG, "cache is NULL");
    if (!q_hat) return fail(SWAN_ERR_INVALID_ARG, "q_hat is NULL");
    const swan::SplitArgs a = split_args(d, c, p, pos, q_hat, ws);
    return hip_status(swan::launch_split(a, d->N_h / d->H_kv, (hipStream_t)stream), "swan_decode_split launch");
}

swan_status swan_decode_reduce(const swan_dims *d, const int32_t *pos, int32_t max_pos, const void *ws,
                               size_t ws_bytes, float *o_hat, void *stream)
{
    Plan p;
    swan_status st = check_decode(d, nullptr, pos, max_pos, ws, ws_bytes, &p);
    if (st) return st;
    if (!o_hat) return fail(SWAN_ERR_INVALID_ARG, "o_hat is NULL");
    swan::ReduceArgs r;
    r.B = d->B;
    r.N_h = d->N_h;
    r.H = d->H_kv;
    r.R = d->R;
    r.W = p.W;
    r.split_tokens = d->split_tokens;
    r.row_bytes = row_bytes(d);
    r.row_cap = (int)row_cap(d);
    r.pos = pos;
    r.part_o = (const float *)ws;
    r.part_ml = (const float *)ws + partial_count(d, p) * swan::kD;
    r.o_hat = o_hat;
    return hip_status(swan::launch_reduce(r, (hipStream_t)stream), "swan_decode_reduce launch");
}

swan_status swan_decode_attn(const swan_dims *d, const swan_cache *c, const int32_t *pos, int32_t max_pos,
                             const float *q_hat, float *o_hat, void *ws, size_t ws_bytes, void *stream)
{
    Plan p;
    swan_status st = check_decode(d, c, pos, max_pos, ws, ws_bytes, &p);
    if (st) return st;
    if (!c) return fail(SWAN_ERR_INVALID_ARG, "cache is NULL");
    if (!q_hat || !o_hat) return fail(SWAN_ERR_INVALID_ARG, "NULL array argument");
    if ((st = swan_decode_split(d, c, pos, max_pos, q_hat, ws, ws_bytes, stream))) return st;
    return swan_decode_reduce(d, pos, max_pos, ws, ws_bytes, o_hat, stream);
}

swan_status swan_decode_attn_noalloc(const swan_dims *d, const swan_cache *c, const int32_t *pos, int32_t max_pos,
                                     const float *q_hat, float *o_hat, void *stream)
{
    Plan p;
    swan_status st = check_decode_plan(d, c, pos, max_pos, &p);
    if (st) return st;
    if (!c) return fail(SWAN_ERR_INVALID_ARG, "cache is NULL");
    if (!q_hat || !o_hat) return fail(SWAN_ERR_INVALID_ARG, "NULL array argument");
    const size_t need = workspace_bytes(d, p);
    if (need > kScratchBytes)
        return fail(SWAN_ERR_CAPACITY, "the split pass needs %zu bytes of partials, the no-allocation scratch holds "
                                       "%zu (swan_decode_attn takes a workspace of any size)", need, kScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_for((hipStream_t)stream, &ws))) return st;
    // the same two launches as swan_decode_attn, over the scratch array; the
    // split pass writes every partial the reduce pass reads, so nothing is
    // cleared between calls
    if ((st = swan_decode_split(d, c, pos, max_pos, q_hat, ws, kScratchBytes, stream))) return st;
    return swan_decode_reduce(d, pos, max_pos, ws, kScratchBytes, o_hat, stream);
}

swan_status swan_prefill_convert(const swan_dims *d, const swan_cache *c, const int32_t *len, int32_t max_len,
                                 int64_t T_stride, const float *k_raw, const float *v_hat, const float *P_qk,
                                 float rope_base, void *stream)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if ((st = check_cache(d, c, true))) return st;
    if (!len || !k_raw || !v_hat || !P_qk) return fail(SWAN_ERR_INVALID_ARG, "NULL array argument");
    if (max_len < 0 || T_stride < max_len)
        return fail(SWAN_ERR_INVALID_ARG, "need 0 <= max_len <= T_stride (got %d, %lld)", max_len, (long long)T_stride);
    if (!(rope_base > 1.0f)) return fail(SWAN_ERR_INVALID_ARG, "rope_base must be > 1");
    if ((int64_t)max_len - d->R > row_cap(d))
        return fail(SWAN_ERR_CAPACITY, "max_len = %d needs %lld sparse rows, capacity is %lld", max_len,
                    (long long)((int64_t)max_len - d->R), (long long)row_cap(d));
    if (max_len == 0) return SWAN_OK;
    swan::PrefillArgs a;
    a.B = d->B;
    a.H = d->H_kv;
    a.R = d->R;
    a.k = d->k;
    a.k_v = kept_v(d);
    a.T_stride = T_stride;
    a.max_len = max_len;
    a.geom = geom(d, c);
    a.kidx = c->k_idx;
    a.vidx = c->v_idx;
    a.kval = (uint8_t *)c->k_val;
    a.vval = (uint8_t *)c->v_val;
    a.kbuf = c->k_buf;
    a.vbuf = c->v_buf;
    a.len = len;
    a.k_raw = k_raw;
    a.v_hat = v_hat;
    a.P = P_qk;
    a.Bl = layer_seqs(d);
    a.base = rope_base;
    return hip_status(swan::launch_prefill(a, (hipStream_t)stream), "swan_prefill_convert launch");
}

swan_status swan_copy_blocks(const swan_dims *d, const swan_cache *c, const int32_t *src, const int32_t *dst,
                             int32_t count, void *stream)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if (d->block_size <= 0) return fail(SWAN_ERR_INVALID_ARG, "swan_copy_blocks needs the paged layout (block_size > 0)");
    if ((st = check_cache(d, c, false))) return st;
    if (count < 0) return fail(SWAN_ERR_INVALID_ARG, "count = %d < 0", count);
    if (count == 0) return SWAN_OK;
    if (!src || !dst) return fail(SWAN_ERR_INVALID_ARG, "NULL block id array");
    if (count > 65535) return fail(SWAN_ERR_INVALID_ARG, "count = %d > 65535", count);
    if (((int64_t)d->H_kv * d->block_size * row_stride(d->k)) % 16 ||
        ((int64_t)d->H_kv * d->block_size * row_stride(kept_v(d))) % 16)
        return fail(SWAN_ERR_UNSUPPORTED, "a block of an index plane (H_kv * block_size * k_stride bytes) must be a "
                                          "multiple of 16 bytes");
    swan::CopyBlocksArgs a;
    a.count = count;
    a.num_blocks = d->num_blocks;
    a.block_bytes_kidx = (int64_t)d->H_kv * d->block_size * row_stride(d->k);
    a.block_bytes_vidx = (int64_t)d->H_kv * d->block_size * row_stride(kept_v(d));
    a.vbytes = value_bytes(d);
    a.kidx = c->k_idx;
    a.vidx = c->v_idx;
    a.kval = (uint8_t *)c->k_val;
    a.vval = (uint8_t *)c->v_val;
    a.src = src;
    a.dst = dst;
    return hip_status(swan::launch_copy_blocks(a, (hipStream_t)stream), "swan_copy_blocks launch");
}

swan_status swan_paged_update(const swan_dims *d, const swan_cache *c, int32_t *block_table, const int32_t *entries,
                              int32_t n_entries, const int32_t *copies, int32_t n_copies, void *stream)
{
    swan_status st = check_dims(d);
    if (st) return st;
    if (d->block_size <= 0) return fail(SWAN_ERR_INVALID_ARG, "swan_paged_update needs the paged layout (block_size > 0)");
    if ((st = check_cache(d, c, false))) return st;
    if (!block_table || block_table != c->block_table)
        return fail(SWAN_ERR_INVALID_ARG, "block_table must be the table cache->block_table points at");
    if (n_entries < 0 || n_copies < 0) return fail(SWAN_ERR_INVALID_ARG, "negative count");
    if ((n_entries > 0 && !entries) || (n_copies > 0 && !copies)) return fail(SWAN_ERR_INVALID_ARG, "NULL pair array");
    const int64_t n_slots = (int64_t)d->B * d->max_blocks;
    for (int32_t i = 0; i < n_entries; ++i) {
        const int32_t at = entries[2 * i], id = entries[2 * i + 1];
        if (at < 0 || at >= n_slots || id < -1 || id >= d->num_blocks)
            return fail(SWAN_ERR_INVALID_ARG, "entry %d = (%d, %d): slot outside [0, %lld) or block outside [-1, %d)", i,
                        at, id, (long long)n_slots, d->num_blocks);
    }
    for (int32_t i = 0; i < n_copies; ++i) {
        const int32_t src = copies[2 * i], dst = copies[2 * i + 1];
        if (src < 0 || src >= d->num_blocks || dst < 0 || dst >= d->num_blocks || src == dst)
            return fail(SWAN_ERR_INVALID_ARG, "copy %d = (%d, %d): ids outside [0, %d) or equal", i, src, dst,
                        d->num_blocks);
    }
    if (n_copies > 0 && (((int64_t)d->H_kv * d->block_size * row_stride(d->k)) % 16 ||
                         ((int64_t)d->H_kv * d->block_size * row_stride(kept_v(d))) % 16))
        return fail(SWAN_ERR_UNSUPPORTED, "a block of an index plane (H_kv * block_size * k_stride bytes) must be a "
                                          "multiple of 16 bytes");
    swan::PagedUpdateArgs a;
    a.num_blocks = d->num_blocks;
    a.block_bytes_kidx = (int64_t)d->H_kv * d->block_size * row_stride(d->k);
    a.block_bytes_vidx = (int64_t)d->H_kv * d->block_size * row_stride(kept_v(d));
    a.vbytes = value_bytes(d);
    a.kidx = c->k_idx;
    a.vidx = c->v_idx;
    a.kval = (uint8_t *)c->k_val;
    a.vval = (uint8_t *)c->v_val;
    a.table = block_table;
    // as many launches as the pairs need; each carries its share by value
    int32_t e = 0, k = 0;
    while (e < n_entries || k < n_copies) {
        a.n_entries = n_entries - e < swan::kUpdateEntries ? n_entries - e : swan::kUpdateEntries;
        a.n_copies = n_copies - k < swan::kUpdateCopies ? n_copies - k : swan::kUpdateCopies;
        for (int i = 0; i < a.n_entries; ++i) {
            a.entry[i][0] = entries[2 * (e + i)];
            a.entry[i][1] = entries[2 * (e + i) + 1];
        }
        for (int i = 0; i < a.n_copies; ++i) {
            a.copy[i][0] = copies[2 * (k + i)];
            a.copy[i][1] = copies[2 * (k + i) + 1];
        }
        if ((st = hip_status(swan::launch_paged_update(a, (hipStream_t)stream), "swan_paged_update launch"))) return st;
        e += a.n_entries;
        k += a.n_copies;
    }
    return SWAN_OK;
}

swan_status swan_measure_stream_read(const void *buf, size_t bytes, int32_t waves, uint32_t *sink, void *stream)
{
    if (!buf || !sink) return fail(SWAN_ERR_INVALID_ARG, "NULL buffer or sink");
    if ((uintptr_t)buf % 16) return fail(SWAN_ERR_INVALID_ARG, "buffer is not 16-byte aligned");
    if (bytes == 0 || bytes % 16 || bytes > ((size_t)1 << 40))
        return fail(SWAN_ERR_INVALID_ARG, "bytes = %zu: must be a positive multiple of 16, at most 2^40", bytes);
    if (waves < 1 || waves > swan::kMaxWaves)
        return fail(SWAN_ERR_INVALID_ARG, "waves = %d outside 1..%d", waves, swan::kMaxWaves);
    return hip_status(swan::launch_stream_read(buf, (int64_t)bytes, waves, sink, (hipStream_t)stream),
                      "swan_measure_stream_read launch");
}

swan_status swan_measure_mfma_f64(double x, int32_t waves, int32_t iters, double *sink, void *stream)
{
    if (!sink) return fail(SWAN_ERR_INVALID_ARG, "NULL sink");
    if (waves < 1 || waves > swan::kMaxWaves)
        return fail(SWAN_ERR_INVALID_ARG, "waves = %d outside 1..%d", waves, swan::kMaxWaves);
    if (iters < 4 || iters > (1 << 20) || iters % 4)
        return fail(SWAN_ERR_INVALID_ARG, "iters = %d: must be a multiple of 4 in 4..1048576", iters);
    return hip_status(swan::launch_mfma_f64(x, waves, iters, sink, (hipStream_t)stream), "swan_measure_mfma_f64 launch");
}

} // extern "C"
