// ssd_api.cpp -- the extern "C" entry points declared in include/ssd_replay.h:
// host-side argument checks (all of them before any HIP call, so a rejected
// call launches nothing) and the translation into kernel argument blocks.
#include "ssd_replay.h"

#include <algorithm>
#include <limits>
#include <vector>

#include "ssd_internal.hpp"

namespace {

using ssd::Dims;

bool pow2_in(int v, int lo, int hi) {
    if (v < lo || v > hi)
        return false;
    return (v & (v - 1)) == 0;
}

// bf16_state: the recurrent update also takes a bf16 state; everything that
// touches the replay cache requires fp32 ([RFC] section 4).
int check_shape(const ssd_shape *sh, Dims *d, bool bf16_state = false) {
    if (!sh)
        return SSD_ERR_NULL;
    if (sh->state_dtype != SSD_F32 && !(bf16_state && sh->state_dtype == SSD_BF16))
        return SSD_ERR_STATE_NOT_FP32;
    if ((sh->io_dtype != SSD_F32 && sh->io_dtype != SSD_BF16) ||
        (sh->dt_dtype != SSD_F32 && sh->dt_dtype != SSD_BF16))
        return SSD_ERR_DTYPE;
    if (sh->H <= 0 || sh->G <= 0 || sh->H % sh->G != 0)
        return SSD_ERR_SHAPE;
    if (!pow2_in(sh->chunk_size, 16, 256) || !pow2_in(sh->P, 16, 128) ||
        !pow2_in(sh->N, 16, 128) || sh->H > 65535)
        return SSD_ERR_UNSUPPORTED;
    d->H = sh->H;
    d->G = sh->G;
    d->P = sh->P;
    d->N = sh->N;
    d->Q = sh->chunk_size;
    d->io_bf16 = sh->io_dtype == SSD_BF16;
    d->dt_bf16 = sh->dt_dtype == SSD_BF16;
    d->softplus = sh->dt_softplus != 0;
    return SSD_OK;
}

// cu_seqlens_host: cu[0] == 0, non-decreasing, cu[S] == T, and the grid
// (S * H workgroups) fits a 1D launch.
int check_seqs(const Dims &d, int32_t S, int64_t T, const int32_t *cu_host, const int32_t *cu) {
    if (S < 0 || T < 0 || T > std::numeric_limits<int32_t>::max())
        return SSD_ERR_SHAPE;
    if (S == 0)
        return T == 0 ? SSD_OK : SSD_ERR_SHAPE;
    if (!cu_host || !cu)
        return SSD_ERR_NULL;
    if (cu_host[0] != 0 || cu_host[S] != T)
        return SSD_ERR_SHAPE;
    for (int32_t s = 0; s < S; ++s)
        if (cu_host[s + 1] < cu_host[s])
            return SSD_ERR_SHAPE;
    if ((int64_t)S * d.H > std::numeric_limits<int32_t>::max())
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Arrays the kernels move in 16-byte pieces (NULL passes).
bool a16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

template <class... T>
bool all_a16(const T *...p) {
    return (a16(p) && ...);
}

// need_work = false: the call does not use the cache's work array (the
// decode entry point that brings its own)
int check_cache(const ssd_shape *sh, const ssd_replay_cache *c, bool need_work = true) {
    if (!c)
        return SSD_ERR_NULL;
    if (c->state_dtype != SSD_F32)
        return SSD_ERR_STATE_NOT_FP32;
    if (c->chunk_size != sh->chunk_size)
        return SSD_ERR_CHUNK_MISMATCH;
    if (!c->state || !c->state_bf || !c->buf_x || !c->buf_dt || !c->buf_B || !c->buf_len ||
        !c->boundary_pos || (need_work && !c->work))
        return SSD_ERR_NULL;
    if (c->num_slots <= 0)
        return SSD_ERR_SHAPE;
    if (c->buf_pages) {
        const int pt = c->page_tokens;
        if (pt < 16 || pt > c->chunk_size || (pt & (pt - 1)) != 0 || c->num_pages <= 0)
            return SSD_ERR_SHAPE;
    }
    if (!all_a16(c->state, c->state_bf, c->buf_x, c->buf_B, c->buf_C))
        return SSD_ERR_ALIGN;
    return SSD_OK;
}

// Buffer addressing of a checked cache.
ssd::BufMap buf_map(const ssd_replay_cache *c) {
    ssd::BufMap m = {};
    if (c->buf_pages) {
        m.pages = c->buf_pages;
        int sh = 0;
        while ((1 << sh) < c->page_tokens)
            ++sh;
        m.shift = sh;
        m.npp = c->chunk_size >> sh;
        m.num_pages = c->num_pages;
    }
    return m;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

// Debug builds (SSD_DEBUG_CHECKS) also check that the slot_idx entries of a
// call that lie in [0, num_slots) are distinct: every kernel reads and writes
// a slot from one place per call, so a repeated slot is undefined behaviour
// the release build does not look for (it would need the device array on
// the host, a synchronising copy). Entries outside the range are the
// skipped positions some calls allow. Returns SSD_ERR_SHAPE on a repeat.
#ifdef SSD_DEBUG_CHECKS
int check_slots_distinct(const int32_t *slot_idx, int32_t n, int32_t num_slots) {
    if (!slot_idx || n <= 0 || num_slots <= 0)
        return SSD_OK;
    std::vector<int32_t> h((size_t)n);
    if (ssd::copy_to_host(h.data(), slot_idx, sizeof(int32_t) * (size_t)n) != hipSuccess)
        return SSD_ERR_HIP;
    std::vector<char> seen((size_t)num_slots, 0);
    for (int32_t v : h) {
        if (v < 0 || v >= num_slots)
            continue;
        if (seen[(size_t)v])
            return SSD_ERR_SHAPE;
        seen[(size_t)v] = 1;
    }
    return SSD_OK;
}
#else
int check_slots_distinct(const int32_t *, int32_t, int32_t) { return SSD_OK; }
#endif

// One engine per shape, so prefill and decode of a shape always share the
// same chunk arithmetic.
hipError_t launch_scan_any(const ssd::ScanArgs &a, hipStream_t stream) {
    return ssd::mfma_supported(a.d) ? ssd::launch_scan_mfma(a, stream)
                                    : ssd::launch_scan(a, stream);
}

size_t dtype_bytes(int dt) { return dt == SSD_BF16 ? 2 : 4; }

}  // namespace

namespace {

// Replay-mode scan shared by prefill (mode 0), speculative verification
// (mode 1: outputs only) and acceptance (mode 2: chunk states and buffer
// append of the first take[s] tokens, no outputs).
int replay_scan(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t S, int64_t T,
                const int32_t *cu_host, const int32_t *cu, const int32_t *slot_idx,
                const void *x, const void *dt, const void *B, const void *C, const float *A,
                const float *D, const float *dt_bias, void *y, int mode, const int32_t *take,
                hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if ((st = check_cache(sh, cache)) != SSD_OK)
        return st;
    if ((st = check_seqs(d, S, T, cu_host, cu)) != SSD_OK)
        return st;
    if (!slot_idx && S > cache->num_slots)
        return SSD_ERR_SHAPE;
    if (S == 0)
        return SSD_OK;
    if (!A || (mode == 2 && !take))
        return SSD_ERR_NULL;
    if (T > 0 && (!x || !dt || !B))
        return SSD_ERR_NULL;
    if (T > 0 && mode != 2 && (!C || !y))
        return SSD_ERR_NULL;
    if (T > 0 && mode == 2 && cache->buf_C && !C)
        return SSD_ERR_NULL;
    if (!all_a16(x, B, C, y))
        return SSD_ERR_ALIGN;
    if ((st = check_slots_distinct(slot_idx, S, cache->num_slots)) != SSD_OK)
        return st;
    ssd::ScanArgs a = {};
    a.d = d;
    a.S = S;
    a.cu = cu;
    a.slot_idx = slot_idx;
    a.x = x; a.dt = dt; a.B = B; a.C = C;
    a.A = A; a.D = D; a.dt_bias = dt_bias;
    a.y = mode == 2 ? nullptr : y;
    a.replay = 1;
    a.num_slots = cache->num_slots;
    a.cache_state = cache->state;
    a.cache_state_bf = cache->state_bf;
    a.buf_x = cache->buf_x; a.buf_dt = cache->buf_dt; a.buf_B = cache->buf_B;
    a.buf_len = cache->buf_len;
    a.bm = buf_map(cache);
    a.dry = mode == 1;
    a.no_y = mode == 2;
    a.take = mode == 2 ? take : nullptr;
    // the sweeps of verification and acceptance list their sequences in the
    // work array (distinct slots: S <= num_slots, the list's room)
    a.work = mode != 0 ? cache->work : nullptr;
    for (int32_t s = 0; s < S; ++s)
        a.max_len = std::max(a.max_len, cu_host[s + 1] - cu_host[s]);
    if (mode == 1)   // verification writes only y
        return hip_status(ssd::mfma_supported(d) ? ssd::launch_verify_mfma(a, (hipStream_t)stream)
                                                 : ssd::launch_scan(a, (hipStream_t)stream));
    hipError_t e = launch_scan_any(a, (hipStream_t)stream);
    if (e != hipSuccess)
        return SSD_ERR_HIP;
    ssd::CommitArgs c = {};
    c.d = d;
    c.S = S;
    c.cu = cu;
    c.slot_idx = slot_idx;
    c.x = x; c.dt = dt; c.B = B; c.C = C;
    c.fresh = 0;
    c.num_slots = cache->num_slots;
    c.state_src = nullptr;
    c.cache_state = cache->state;
    c.cache_state_bf = cache->state_bf;
    c.buf_x = cache->buf_x; c.buf_dt = cache->buf_dt;
    c.buf_B = cache->buf_B; c.buf_C = cache->buf_C;
    c.buf_len = cache->buf_len;
    c.boundary_pos = cache->boundary_pos;
    c.bm = a.bm;
    c.take = a.take;
    return hip_status(ssd::launch_commit(c, (hipStream_t)stream));
}

}  // namespace

extern "C" {

const char *ssd_status_string(int status) {
    switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: inconsistent sizes";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown dtype";
    case SSD_ERR_STATE_NOT_FP32: return "SSD_ERR_STATE_NOT_FP32: the SSM state must be fp32";
    case SSD_ERR_CHUNK_MISMATCH: return "SSD_ERR_CHUNK_MISMATCH: cache and call chunk sizes differ";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape outside the built set";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: HIP launch or runtime error";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: an array is not 16-byte aligned";
    default: return "unknown ssd_status";
    }
}

size_t ssd_replay_cache_bytes(const ssd_shape *sh, int32_t num_slots, int32_t with_C) {
    Dims d;
    if (check_shape(sh, &d) != SSD_OK || num_slots < 0)
        return 0;
    const size_t io = dtype_bytes(sh->io_dtype), dtb = dtype_bytes(sh->dt_dtype);
    const size_t state = (size_t)d.H * d.P * d.N * (sizeof(float) + sizeof(uint16_t));
    const size_t per_tok = (size_t)d.H * d.P * io + (size_t)d.H * dtb +
                           (with_C ? 2 : 1) * (size_t)d.G * d.N * io;
    const size_t per_slot =
        state + (size_t)d.Q * per_tok + 3 * sizeof(int32_t) + sizeof(int64_t);
    return per_slot * (size_t)num_slots + 34 * sizeof(int32_t);
}

size_t ssd_replay_page_bytes(const ssd_shape *sh, int32_t page_tokens, int32_t with_C) {
    Dims d;
    if (check_shape(sh, &d) != SSD_OK || page_tokens < 16 || page_tokens > d.Q ||
        (page_tokens & (page_tokens - 1)) != 0)
        return 0;
    const size_t io = dtype_bytes(sh->io_dtype), dtb = dtype_bytes(sh->dt_dtype);
    const size_t per_tok = (size_t)d.H * d.P * io + (size_t)d.H * dtb +
                           (with_C ? 2 : 1) * (size_t)d.G * d.N * io;
    return per_tok * (size_t)page_tokens;
}

int ssd_replay_cache_refresh(const ssd_shape *sh, const ssd_replay_cache *cache,
                             hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if ((st = check_cache(sh, cache)) != SSD_OK)
        return st;
    return hip_status(ssd::launch_refresh_state_bf(cache->state, cache->state_bf,
                                                   (int64_t)cache->num_slots * d.H, d.P, d.N,
                                                   (hipStream_t)stream));
}

size_t ssd_prefill_workspace_bytes(const ssd_shape *sh, int32_t num_seqs, int64_t total_tokens) {
    (void)sh;
    (void)num_seqs;
    (void)total_tokens;
    return 0;
}

int ssd_prefill_varlen(const ssd_shape *sh, int32_t S, int64_t T, const int32_t *cu_host,
                       const int32_t *cu, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const float *dt_bias,
                       const float *init_state, void *y, float *final_state,
                       float *boundary_state, float *chunk_states, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if ((st = check_seqs(d, S, T, cu_host, cu)) != SSD_OK)
        return st;
    if (workspace_bytes < ssd_prefill_workspace_bytes(sh, S, T) ||
        (ssd_prefill_workspace_bytes(sh, S, T) > 0 && !workspace))
        return SSD_ERR_WORKSPACE;
    if (S == 0)
        return SSD_OK;
    if (!A || (T > 0 && (!x || !dt || !B || !C || !y)))
        return SSD_ERR_NULL;
    if (!all_a16(x, B, C, y, init_state, final_state, boundary_state, chunk_states))
        return SSD_ERR_ALIGN;
    ssd::ScanArgs a = {};
    a.d = d;
    a.S = S;
    a.cu = cu;
    a.slot_idx = nullptr;
    a.x = x; a.dt = dt; a.B = B; a.C = C;
    a.A = A; a.D = D; a.dt_bias = dt_bias;
    a.y = y;
    a.init_state = init_state;
    a.final_state = final_state;
    a.boundary_state = boundary_state;
    a.chunk_states = chunk_states;
    a.replay = 0;
    return hip_status(launch_scan_any(a, (hipStream_t)stream));
}

int64_t ssd_prefill_chunk_count(int32_t S, const int32_t *cu_host, int32_t Q) {
    if (!cu_host || S < 0 || Q < 1)
        return -1;
    int64_t n = 0;
    for (int32_t s = 0; s < S; ++s) {
        if (cu_host[s + 1] < cu_host[s])
            return -1;
        n += (cu_host[s + 1] - cu_host[s]) / Q;
    }
    return n;
}

int ssd_commit_boundary(const ssd_shape *sh, int32_t S, int64_t T, const int32_t *cu_host,
                        const int32_t *cu, const int32_t *slot_idx, const void *x,
                        const void *dt, const void *B, const void *C,
                        const float *boundary_state, const ssd_replay_cache *cache,
                        hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if ((st = check_cache(sh, cache)) != SSD_OK)
        return st;
    if ((st = check_seqs(d, S, T, cu_host, cu)) != SSD_OK)
        return st;
    if (!slot_idx && S > cache->num_slots)
        return SSD_ERR_SHAPE;
    if (S == 0)
        return SSD_OK;
    if (!boundary_state || (T > 0 && (!x || !dt || !B || (cache->buf_C && !C))))
        return SSD_ERR_NULL;
    if (!all_a16(x, B, C, boundary_state))
        return SSD_ERR_ALIGN;
    if ((st = check_slots_distinct(slot_idx, S, cache->num_slots)) != SSD_OK)
        return st;
    ssd::CommitArgs a = {};
    a.d = d;
    a.S = S;
    a.cu = cu;
    a.slot_idx = slot_idx;
    a.x = x; a.dt = dt; a.B = B; a.C = C;
    a.fresh = 1;
    a.num_slots = cache->num_slots;
    a.state_src = boundary_state;
    a.cache_state = cache->state;
    a.cache_state_bf = cache->state_bf;
    a.buf_x = cache->buf_x; a.buf_dt = cache->buf_dt;
    a.buf_B = cache->buf_B; a.buf_C = cache->buf_C;
    a.buf_len = cache->buf_len;
    a.boundary_pos = cache->boundary_pos;
    a.bm = buf_map(cache);
    return hip_status(ssd::launch_commit(a, (hipStream_t)stream));
}

int ssd_replay_prefill(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t S, int64_t T,
                       const int32_t *cu_host, const int32_t *cu, const int32_t *slot_idx,
                       const void *x, const void *dt, const void *B, const void *C,
                       const float *A, const float *D, const float *dt_bias, void *y,
                       hipStream_t stream) {
    return replay_scan(sh, cache, S, T, cu_host, cu, slot_idx, x, dt, B, C, A, D, dt_bias, y, 0,
                       nullptr, stream);
}

int ssd_replay_verify(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t S, int64_t T,
                      const int32_t *cu_host, const int32_t *cu, const int32_t *slot_idx,
                      const void *x, const void *dt, const void *B, const void *C,
                      const float *A, const float *D, const float *dt_bias, void *y,
                      hipStream_t stream) {
    return replay_scan(sh, cache, S, T, cu_host, cu, slot_idx, x, dt, B, C, A, D, dt_bias, y, 1,
                       nullptr, stream);
}

int ssd_replay_accept(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t S, int64_t T,
                      const int32_t *cu_host, const int32_t *cu, const int32_t *slot_idx,
                      const int32_t *accepted, const void *x, const void *dt, const void *B,
                      const void *C, const float *A, const float *dt_bias, hipStream_t stream) {
    return replay_scan(sh, cache, S, T, cu_host, cu, slot_idx, x, dt, B, C, A, nullptr, dt_bias,
                       nullptr, 2, accepted, stream);
}

}  // extern "C"

namespace {

// The conv before the scan, for a decode step that takes it in the same
// launch (conv.xBC non-null; the other fields as in ssd_conv1d_update).
struct DecodeConv {
    const void *xBC = nullptr;
    const float *weight = nullptr, *bias = nullptr;
    void *state = nullptr;
    int32_t width = 0, act = 0;
};

// One decode step; own_work: the library's static bookkeeping array takes
// the place of cache->work (which may then be NULL).
int replay_decode(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t batch,
                  const int32_t *slot_idx, const void *x, const void *dt, const void *B,
                  const void *C, const float *A, const float *D, const float *dt_bias, void *y,
                  bool own_work, hipStream_t stream, const DecodeConv &conv = DecodeConv()) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if ((st = check_cache(sh, cache, !own_work)) != SSD_OK)
        return st;
    if (own_work && cache->num_slots > ssd::kStaticMaxSlots)
        return SSD_ERR_WORKSPACE;
    if (batch < 0 || (!slot_idx && batch > cache->num_slots) ||
        (int64_t)batch * d.H > std::numeric_limits<int32_t>::max())
        return SSD_ERR_SHAPE;
    if (batch == 0)
        return SSD_OK;
    if (!x || !dt || !B || !C || !A || !y)
        return SSD_ERR_NULL;
    if (!all_a16(x, B, C, y))
        return SSD_ERR_ALIGN;
    if ((st = check_slots_distinct(slot_idx, batch, cache->num_slots)) != SSD_OK)
        return st;
    ssd::DecodeArgs a = {};
    a.d = d;
    a.batch = batch;
    a.slot_idx = slot_idx;
    a.x = x; a.dt = dt; a.B = B; a.C = C;
    a.A = A; a.D = D; a.dt_bias = dt_bias;
    a.y = y;
    a.num_slots = cache->num_slots;
    a.cache_state = cache->state;
    a.cache_state_bf = cache->state_bf;
    a.buf_x = cache->buf_x; a.buf_dt = cache->buf_dt;
    a.buf_B = cache->buf_B; a.buf_C = cache->buf_C;
    a.buf_len = cache->buf_len;
    a.boundary_pos = cache->boundary_pos;
    a.work = cache->work;
    if (own_work && ssd::static_work(&a.work, (hipStream_t)stream) != hipSuccess)
        return SSD_ERR_HIP;
    a.bm = buf_map(cache);
    if (conv.xBC) {
        // one launch when the matrix-core engine runs the step with each
        // workgroup's heads in one B/C group (bf16 I/O); otherwise the conv
        // update and the step as two launches (the same bits either way:
        // one conv_point, the same inputs)
        if (ssd::mfma_supported(d) && d.io_bf16 && (d.H / d.G) % 4 == 0) {
            a.xBC = conv.xBC;
            a.cw = conv.weight;
            a.cb = conv.bias;
            a.cstate = conv.state;
            a.cW = conv.width;
            a.cact = conv.act != 0;
            return hip_status(ssd::launch_decode_mfma(a, (hipStream_t)stream));
        }
        ssd::ConvArgs c = {};
        c.d = d;
        c.W = conv.width;
        c.act = conv.act != 0;
        c.S = batch;
        c.slot_idx = slot_idx;
        c.num_slots = cache->num_slots;
        c.xBC = conv.xBC; c.weight = conv.weight; c.bias = conv.bias;
        c.state = conv.state;
        c.x = const_cast<void *>(x); c.B = const_cast<void *>(B); c.C = const_cast<void *>(C);
        const hipError_t e = ssd::launch_conv_update(c, (hipStream_t)stream);
        if (e != hipSuccess)
            return hip_status(e);
    }
    return hip_status(ssd::mfma_supported(d) ? ssd::launch_decode_mfma(a, (hipStream_t)stream)
                                             : ssd::launch_decode(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int ssd_replay_decode(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t batch,
                      const int32_t *slot_idx, const void *x, const void *dt, const void *B,
                      const void *C, const float *A, const float *D, const float *dt_bias,
                      void *y, hipStream_t stream) {
    return replay_decode(sh, cache, batch, slot_idx, x, dt, B, C, A, D, dt_bias, y, false,
                         stream);
}

int ssd_replay_decode_static(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t batch,
                             const int32_t *slot_idx, const void *x, const void *dt,
                             const void *B, const void *C, const float *A, const float *D,
                             const float *dt_bias, void *y, hipStream_t stream) {
    return replay_decode(sh, cache, batch, slot_idx, x, dt, B, C, A, D, dt_bias, y, true,
                         stream);
}

int ssd_replay_decode_conv(const ssd_shape *sh, const ssd_replay_cache *cache, int32_t batch,
                           const int32_t *slot_idx, int32_t width, int32_t activation,
                           const void *xBC, const float *weight, const float *bias,
                           void *conv_state, void *x, void *B, void *C, const void *dt,
                           const float *A, const float *D, const float *dt_bias, void *y,
                           hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if (width < 2 || width > 4)
        return SSD_ERR_UNSUPPORTED;
    if (batch > 65535)
        return SSD_ERR_SHAPE;
    if (batch > 0 && (!xBC || !weight || !conv_state))
        return SSD_ERR_NULL;
    if (!all_a16(xBC, conv_state) || !all_a16(weight, bias))
        return SSD_ERR_ALIGN;
    DecodeConv conv;
    conv.xBC = xBC;
    conv.weight = weight;
    conv.bias = bias;
    conv.state = conv_state;
    conv.width = width;
    conv.act = activation;
    return replay_decode(sh, cache, batch, slot_idx, x, dt, B, C, A, D, dt_bias, y, false,
                         stream, conv);
}

int ssd_conv1d_varlen(const ssd_shape *sh, int32_t W, int32_t act, int32_t S, int64_t T,
                      const int32_t *cu_host, const int32_t *cu, const int32_t *slot_idx,
                      int32_t num_slots, const void *xBC, const float *weight, const float *bias,
                      void *conv_state, void *x, void *B, void *C, hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if (W < 2 || W > 4)
        return SSD_ERR_UNSUPPORTED;
    if ((st = check_seqs(d, S, T, cu_host, cu)) != SSD_OK)
        return st;
    if (S > 65535 || (conv_state && (num_slots <= 0 || (!slot_idx && S > num_slots))))
        return SSD_ERR_SHAPE;
    if (S == 0)
        return SSD_OK;
    if (!weight || (T > 0 && (!xBC || !x || !B || !C)))
        return SSD_ERR_NULL;
    if (!all_a16(xBC, conv_state, x, B, C) || !all_a16(weight, bias))
        return SSD_ERR_ALIGN;
    if (conv_state && (st = check_slots_distinct(slot_idx, S, num_slots)) != SSD_OK)
        return st;
    int32_t maxlen = 0;
    for (int32_t s = 0; s < S; ++s)
        maxlen = std::max(maxlen, cu_host[s + 1] - cu_host[s]);
    ssd::ConvArgs a = {};
    a.d = d;
    a.W = W;
    a.act = act != 0;
    a.S = S;
    a.cu = cu;
    a.maxlen = maxlen;
    a.slot_idx = conv_state ? slot_idx : nullptr;
    a.num_slots = conv_state ? num_slots : S;
    a.xBC = xBC; a.weight = weight; a.bias = bias;
    a.state = conv_state;
    a.x = x; a.B = B; a.C = C;
    return hip_status(ssd::launch_conv_fwd(a, (hipStream_t)stream));
}

int ssd_conv1d_update(const ssd_shape *sh, int32_t W, int32_t act, int32_t batch,
                      const int32_t *slot_idx, int32_t num_slots, const void *xBC,
                      const float *weight, const float *bias, void *conv_state, void *x, void *B,
                      void *C, hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d);
    if (st != SSD_OK)
        return st;
    if (W < 2 || W > 4)
        return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || batch > 65535 || num_slots < 0 || (!slot_idx && batch > num_slots))
        return SSD_ERR_SHAPE;
    if (batch == 0)
        return SSD_OK;
    if (!weight || !xBC || !conv_state || !x || !B || !C)
        return SSD_ERR_NULL;
    if (!all_a16(xBC, conv_state, x, B, C) || !all_a16(weight, bias))
        return SSD_ERR_ALIGN;
    if ((st = check_slots_distinct(slot_idx, batch, num_slots)) != SSD_OK)
        return st;
    ssd::ConvArgs a = {};
    a.d = d;
    a.W = W;
    a.act = act != 0;
    a.S = batch;
    a.slot_idx = slot_idx;
    a.num_slots = num_slots;
    a.xBC = xBC; a.weight = weight; a.bias = bias;
    a.state = conv_state;
    a.x = x; a.B = B; a.C = C;
    return hip_status(ssd::launch_conv_update(a, (hipStream_t)stream));
}

int ssm_state_update(const ssd_shape *sh, int32_t batch, int32_t num_slots,
                     const int32_t *slot_idx, void *state, const void *x, const void *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const float *dt_bias, void *y, hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d, true);
    if (st != SSD_OK)
        return st;
    if (batch < 0 || num_slots < 0 || (!slot_idx && batch > num_slots) ||
        (int64_t)batch * d.H > std::numeric_limits<int32_t>::max())
        return SSD_ERR_SHAPE;
    if (batch == 0)
        return SSD_OK;
    if (!state || !x || !dt || !A || !B || !C || !y)
        return SSD_ERR_NULL;
    if (!all_a16(state, x, B, C, y))
        return SSD_ERR_ALIGN;
    if ((st = check_slots_distinct(slot_idx, batch, num_slots)) != SSD_OK)
        return st;
    ssd::SsuArgs a = {};
    a.d = d;
    a.batch = batch;
    a.slot_idx = slot_idx;
    a.num_slots = num_slots;
    a.state = state;
    a.state_bf16 = sh->state_dtype == SSD_BF16;
    a.x = x; a.dt = dt; a.B = B; a.C = C;
    a.A = A; a.D = D; a.dt_bias = dt_bias;
    a.y = y;
    return hip_status(ssd::launch_ssu(a, (hipStream_t)stream));
}

int ssm_state_update_varlen(const ssd_shape *sh, int32_t S, int64_t T, const int32_t *cu_host,
                            const int32_t *cu, const int32_t *slot_idx, int32_t num_slots,
                            void *state, const void *x, const void *dt, const float *A,
                            const void *B, const void *C, const float *D, const float *dt_bias,
                            void *y, hipStream_t stream) {
    Dims d;
    int st = check_shape(sh, &d, true);
    if (st != SSD_OK)
        return st;
    if ((st = check_seqs(d, S, T, cu_host, cu)) != SSD_OK)
        return st;
    if (num_slots < 0 || (!slot_idx && S > num_slots))
        return SSD_ERR_SHAPE;
    if (S == 0)
        return SSD_OK;
    if (!state || !A || (T > 0 && (!x || !dt || !B || !C || !y)))
        return SSD_ERR_NULL;
    if (!all_a16(state, x, B, C, y))
        return SSD_ERR_ALIGN;
    if ((st = check_slots_distinct(slot_idx, S, num_slots)) != SSD_OK)
        return st;
    ssd::SsuArgs a = {};
    a.d = d;
    a.batch = S;
    a.slot_idx = slot_idx;
    a.num_slots = num_slots;
    a.state = state;
    a.state_bf16 = sh->state_dtype == SSD_BF16;
    a.cu = cu;
    a.x = x; a.dt = dt; a.B = B; a.C = C;
    a.A = A; a.D = D; a.dt_bias = dt_bias;
    a.y = y;
    return hip_status(ssd::launch_ssu(a, (hipStream_t)stream));
}

}  // extern "C"
