// abi_host_check.cpp -- the C ABI layer (csrc/ssd_api.cpp) on the CPU, built
// with AddressSanitizer and UndefinedBehaviorSanitizer and with the
// debug-build checks (SSD_DEBUG_CHECKS), against stand-ins for the kernel
// launchers: every entry point is called with valid arguments, with each
// kind of bad argument, and at its edges (empty packs, NULL optionals), and
// the stand-ins check the argument block each accepted call hands over.
// "Device" arrays here are host allocations of the right size, so the
// debug-build slot check (which copies slot_idx back) reads real memory.
//
// Exit status 0 when every expectation holds; a sanitizer report aborts.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ssd_internal.hpp"
#include "ssd_replay.h"

namespace {

int g_fail = 0;
int g_launches = 0;

#define EXPECT(cond)                                                           \
    do {                                                                       \
        if (!(cond)) {                                                         \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,  \
                         __LINE__, #cond);                                     \
            ++g_fail;                                                          \
        }                                                                      \
    } while (0)

// Argument blocks that reach a launcher must be complete.
void seen(bool ok) {
    ++g_launches;
    EXPECT(ok);
}

}  // namespace

namespace ssd {
hipError_t launch_scan(const ScanArgs &a, hipStream_t) {
    seen(a.cu && a.A && a.d.H > 0 && (a.replay ? a.cache_state != nullptr : true));
    return hipSuccess;
}
const int32_t *g_last_work = nullptr;
hipError_t launch_decode(const DecodeArgs &a, hipStream_t) {
    seen(a.x && a.y && a.work && a.batch > 0);
    g_last_work = a.work;
    return hipSuccess;
}
bool mfma_supported(const Dims &) { return false; }
hipError_t launch_scan_mfma(const ScanArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_mfma(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_verify_mfma(const ScanArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_conv_fwd(const ConvArgs &a, hipStream_t) {
    seen(a.weight && a.W >= 2 && a.W <= 4 && a.maxlen >= 0);
    return hipSuccess;
}
hipError_t launch_conv_update(const ConvArgs &a, hipStream_t) {
    seen(a.state && a.S > 0);
    return hipSuccess;
}
hipError_t launch_decode_advance(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_commit(const CommitArgs &a, hipStream_t) {
    seen(a.cache_state && a.buf_len && a.boundary_pos);
    return hipSuccess;
}
hipError_t launch_ssu(const SsuArgs &a, hipStream_t) {
    seen(a.state && a.batch > 0);
    return hipSuccess;
}
hipError_t launch_refresh_state_bf(const float *, void *, int64_t heads, int, int, hipStream_t) {
    seen(heads > 0);
    return hipSuccess;
}
int32_t g_static_work[2 * kStaticMaxSlots + 34];
hipError_t static_work(int32_t **out, hipStream_t) {
    *out = g_static_work;
    return hipSuccess;
}
hipError_t copy_to_host(void *dst, const void *src, size_t bytes) {
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}
}  // namespace ssd

namespace {

// 16-byte aligned, zeroed host memory standing in for a device array
struct Arena {
    std::vector<void *> blocks;
    void *get(size_t bytes) {
        bytes = (bytes + 15) / 16 * 16;
        void *p = std::aligned_alloc(16, bytes ? bytes : 16);
        std::memset(p, 0, bytes ? bytes : 16);
        blocks.push_back(p);
        return p;
    }
    ~Arena() {
        for (void *p : blocks)
            std::free(p);
    }
};

ssd_shape shape(int H, int G, int P, int N, int Q) {
    ssd_shape s = {H, G, P, N, Q, SSD_BF16, SSD_BF16, SSD_F32, 1};
    return s;
}

}  // namespace

int main() {
    Arena ar;
    const int H = 4, G = 2, P = 16, N = 16, Q = 16, slots = 6;
    ssd_shape sh = shape(H, G, P, N, Q);
    const int32_t cu[] = {0, 5, 5, 40};   // three sequences, one empty
    const int S = 3, T = 40;
    int32_t *dcu = static_cast<int32_t *>(ar.get(sizeof(cu)));
    std::memcpy(dcu, cu, sizeof(cu));
    void *x = ar.get((size_t)T * H * P * 2), *dt = ar.get((size_t)T * H * 2);
    void *B = ar.get((size_t)T * G * N * 2), *C = ar.get((size_t)T * G * N * 2);
    void *y = ar.get((size_t)T * H * P * 2);
    float *A = static_cast<float *>(ar.get(H * 4)), *D = static_cast<float *>(ar.get(H * 4));
    float *st = static_cast<float *>(ar.get((size_t)S * H * P * N * 4));
    float *fin = static_cast<float *>(ar.get((size_t)S * H * P * N * 4));
    float *bnd = static_cast<float *>(ar.get((size_t)S * H * P * N * 4));
    const int64_t F = ssd_prefill_chunk_count(S, cu, Q);
    EXPECT(F == 0 + 0 + 2);
    float *cs = static_cast<float *>(ar.get((size_t)F * H * P * N * 4));

    // ---- prefill
    EXPECT(ssd_prefill_varlen(&sh, S, T, cu, dcu, x, dt, A, B, C, D, nullptr, nullptr, y, fin,
                              bnd, cs, nullptr, 0, nullptr) == SSD_OK);
    EXPECT(ssd_prefill_varlen(&sh, S, T, cu, dcu, x, dt, A, B, C, nullptr, nullptr, st, y,
                              nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SSD_OK);
    EXPECT(ssd_prefill_varlen(&sh, 0, 0, cu, dcu, nullptr, nullptr, A, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                              nullptr) == SSD_OK);
    EXPECT(ssd_prefill_varlen(&sh, S, T - 1, cu, dcu, x, dt, A, B, C, D, nullptr, nullptr, y,
                              nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SSD_ERR_SHAPE);
    EXPECT(ssd_prefill_varlen(&sh, S, T, cu, dcu, x, dt, A, B, C, D, nullptr, nullptr, y, nullptr,
                              nullptr, (float *)((char *)cs + 4), nullptr, 0,
                              nullptr) == SSD_ERR_ALIGN);
    EXPECT(ssd_prefill_varlen(nullptr, S, T, cu, dcu, x, dt, A, B, C, D, nullptr, nullptr, y,
                              nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SSD_ERR_NULL);
    {
        const int32_t bad[] = {0, 7, 3, 40};
        EXPECT(ssd_prefill_varlen(&sh, S, T, bad, dcu, x, dt, A, B, C, D, nullptr, nullptr, y,
                                  nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SSD_ERR_SHAPE);
        EXPECT(ssd_prefill_chunk_count(S, bad, Q) == -1);
    }
    EXPECT(ssd_prefill_chunk_count(S, nullptr, Q) == -1);
    EXPECT(ssd_prefill_chunk_count(S, cu, 0) == -1);
    for (int q : {8, 24, 512}) {
        ssd_shape b = shape(H, G, P, N, q);
        EXPECT(ssd_prefill_varlen(&b, S, T, cu, dcu, x, dt, A, B, C, D, nullptr, nullptr, y,
                                  nullptr, nullptr, nullptr, nullptr, 0,
                                  nullptr) == SSD_ERR_UNSUPPORTED);
    }
    {
        ssd_shape b = sh;
        b.state_dtype = SSD_BF16;
        EXPECT(ssd_prefill_varlen(&b, S, T, cu, dcu, x, dt, A, B, C, D, nullptr, nullptr, y,
                                  nullptr, nullptr, nullptr, nullptr, 0,
                                  nullptr) == SSD_ERR_STATE_NOT_FP32);
    }

    // ---- replay cache
    const size_t cbytes = ssd_replay_cache_bytes(&sh, slots, 1);
    EXPECT(cbytes > 0);
    EXPECT(ssd_replay_cache_bytes(&sh, -1, 1) == 0);
    ssd_replay_cache c = {};
    c.state = static_cast<float *>(ar.get((size_t)slots * H * P * N * 4));
    c.state_bf = ar.get((size_t)slots * H * P * N * 2);
    c.buf_x = ar.get((size_t)slots * Q * H * P * 2);
    c.buf_dt = ar.get((size_t)slots * Q * H * 2);
    c.buf_B = ar.get((size_t)slots * Q * G * N * 2);
    c.buf_C = ar.get((size_t)slots * Q * G * N * 2);
    c.buf_len = static_cast<int32_t *>(ar.get(slots * 4));
    c.boundary_pos = static_cast<int64_t *>(ar.get(slots * 8));
    c.work = static_cast<int32_t *>(ar.get((2 * slots + 34) * 4));
    c.num_slots = slots;
    c.chunk_size = Q;
    c.state_dtype = SSD_F32;

    int32_t *sl = static_cast<int32_t *>(ar.get(16 * 4));
    auto set_slots = [&](std::initializer_list<int32_t> v) {
        int i = 0;
        for (int32_t e : v)
            sl[i++] = e;
    };
    set_slots({4, 0, 2});
    EXPECT(ssd_commit_boundary(&sh, S, T, cu, dcu, sl, x, dt, B, C, bnd, &c, nullptr) == SSD_OK);
    EXPECT(ssd_replay_prefill(&sh, &c, S, T, cu, dcu, sl, x, dt, B, C, A, D, nullptr, y,
                              nullptr) == SSD_OK);
    EXPECT(ssd_replay_verify(&sh, &c, S, T, cu, dcu, sl, x, dt, B, C, A, D, nullptr, y,
                             nullptr) == SSD_OK);
    int32_t *acc = static_cast<int32_t *>(ar.get(S * 4));
    EXPECT(ssd_replay_accept(&sh, &c, S, T, cu, dcu, sl, acc, x, dt, B, C, A, nullptr,
                             nullptr) == SSD_OK);
    EXPECT(ssd_replay_accept(&sh, &c, S, T, cu, dcu, sl, nullptr, x, dt, B, C, A, nullptr,
                             nullptr) == SSD_ERR_NULL);
    // debug build: a repeated slot is refused before anything is launched
    set_slots({4, 0, 4});
    const int before = g_launches;
    EXPECT(ssd_commit_boundary(&sh, S, T, cu, dcu, sl, x, dt, B, C, bnd, &c, nullptr) ==
           SSD_ERR_SHAPE);
    EXPECT(ssd_replay_prefill(&sh, &c, S, T, cu, dcu, sl, x, dt, B, C, A, D, nullptr, y,
                              nullptr) == SSD_ERR_SHAPE);
    EXPECT(ssd_replay_decode(&sh, &c, 3, sl, x, dt, B, C, A, D, nullptr, y, nullptr) ==
           SSD_ERR_SHAPE);
    EXPECT(g_launches == before);
    // repeated entries outside the slot range are skipped positions, not repeats
    set_slots({-1, 2, -1, 99, 99, 5});
    EXPECT(ssd_replay_decode(&sh, &c, 6, sl, x, dt, B, C, A, D, nullptr, y, nullptr) == SSD_OK);
    set_slots({5, 4, 3, 2, 1, 0});
    EXPECT(ssd_replay_decode(&sh, &c, 6, sl, x, dt, B, C, A, D, nullptr, y, nullptr) == SSD_OK);
    EXPECT(ssd_replay_decode(&sh, &c, 0, sl, x, dt, B, C, A, D, nullptr, y, nullptr) == SSD_OK);
    EXPECT(ssd_replay_decode(&sh, &c, slots + 1, nullptr, x, dt, B, C, A, D, nullptr, y,
                             nullptr) == SSD_ERR_SHAPE);
    {
        ssd_replay_cache b = c;
        b.chunk_size = 32;
        EXPECT(ssd_replay_decode(&sh, &b, 2, nullptr, x, dt, B, C, A, D, nullptr, y, nullptr) ==
               SSD_ERR_CHUNK_MISMATCH);
        b = c;
        b.state_dtype = SSD_BF16;
        EXPECT(ssd_replay_decode(&sh, &b, 2, nullptr, x, dt, B, C, A, D, nullptr, y, nullptr) ==
               SSD_ERR_STATE_NOT_FP32);
        b = c;
        b.work = nullptr;
        EXPECT(ssd_replay_decode(&sh, &b, 2, nullptr, x, dt, B, C, A, D, nullptr, y, nullptr) ==
               SSD_ERR_NULL);
        b = c;
        b.buf_pages = static_cast<int32_t *>(ar.get(slots * 4 * 4));
        b.page_tokens = 8;   // below 16
        b.num_pages = 4;
        EXPECT(ssd_replay_decode(&sh, &b, 2, nullptr, x, dt, B, C, A, D, nullptr, y, nullptr) ==
               SSD_ERR_SHAPE);
        b.page_tokens = 16;
        EXPECT(ssd_replay_decode(&sh, &b, 2, nullptr, x, dt, B, C, A, D, nullptr, y, nullptr) ==
               SSD_OK);
    }
    // the allocation-free decode: the library's array replaces cache->work
    {
        ssd_replay_cache b = c;
        b.work = nullptr;
        set_slots({0, 1});
        EXPECT(ssd_replay_decode_static(&sh, &b, 2, sl, x, dt, B, C, A, D, nullptr, y,
                                        nullptr) == SSD_OK);
        EXPECT(ssd::g_last_work == ssd::g_static_work);
        EXPECT(ssd_replay_decode(&sh, &c, 2, sl, x, dt, B, C, A, D, nullptr, y, nullptr) ==
               SSD_OK);
        EXPECT(ssd::g_last_work == c.work);
        EXPECT(ssd_replay_decode(&sh, &b, 2, sl, x, dt, B, C, A, D, nullptr, y, nullptr) ==
               SSD_ERR_NULL);
        b.num_slots = ssd::kStaticMaxSlots + 1;
        EXPECT(ssd_replay_decode_static(&sh, &b, 2, sl, x, dt, B, C, A, D, nullptr, y,
                                        nullptr) == SSD_ERR_WORKSPACE);
    }
    EXPECT(ssd_replay_cache_refresh(&sh, &c, nullptr) == SSD_OK);
    EXPECT(ssd_replay_page_bytes(&sh, 16, 1) > 0 && ssd_replay_page_bytes(&sh, 12, 1) == 0);

    // ---- recurrent update, one token and varlen
    {
        ssd_shape b = sh;
        b.state_dtype = SSD_BF16;
        void *bst = ar.get((size_t)slots * H * P * N * 2);
        set_slots({1, 3});
        EXPECT(ssm_state_update(&b, 2, slots, sl, bst, x, dt, A, B, C, D, nullptr, y, nullptr) ==
               SSD_OK);
        set_slots({3, 3});
        EXPECT(ssm_state_update(&b, 2, slots, sl, bst, x, dt, A, B, C, D, nullptr, y, nullptr) ==
               SSD_ERR_SHAPE);
        set_slots({0, 1, 2});
        EXPECT(ssm_state_update_varlen(&sh, S, T, cu, dcu, sl, slots, c.state, x, dt, A, B, C, D,
                                       nullptr, y, nullptr) == SSD_OK);
        EXPECT(ssm_state_update_varlen(&sh, S, T, cu, dcu, nullptr, 2, c.state, x, dt, A, B, C, D,
                                       nullptr, y, nullptr) == SSD_ERR_SHAPE);
    }

    // ---- conv pair
    {
        const int cd = H * P + 2 * G * N;
        void *xbc = ar.get((size_t)T * cd * 2);
        float *w = static_cast<float *>(ar.get((size_t)cd * 4 * 4));
        void *cst = ar.get((size_t)slots * cd * 3 * 2);
        set_slots({2, 5, 1});
        EXPECT(ssd_conv1d_varlen(&sh, 4, 1, S, T, cu, dcu, sl, slots, xbc, w, nullptr, cst, x, B,
                                 C, nullptr) == SSD_OK);
        EXPECT(ssd_conv1d_varlen(&sh, 5, 1, S, T, cu, dcu, sl, slots, xbc, w, nullptr, cst, x, B,
                                 C, nullptr) == SSD_ERR_UNSUPPORTED);
        set_slots({2, 5, 2});
        EXPECT(ssd_conv1d_varlen(&sh, 4, 1, S, T, cu, dcu, sl, slots, xbc, w, nullptr, cst, x, B,
                                 C, nullptr) == SSD_ERR_SHAPE);
        EXPECT(ssd_conv1d_update(&sh, 3, 0, 3, sl, slots, xbc, w, nullptr, cst, x, B, C,
                                 nullptr) == SSD_ERR_SHAPE);
        set_slots({0, 1, 2});
        EXPECT(ssd_conv1d_update(&sh, 3, 0, 3, sl, slots, xbc, w, nullptr, cst, x, B, C,
                                 nullptr) == SSD_OK);
        EXPECT(ssd_conv1d_update(&sh, 3, 0, 3, sl, slots, xbc, w, nullptr, nullptr, x, B, C,
                                 nullptr) == SSD_ERR_NULL);
    }

    for (int code = 0; code >= -12; --code)
        EXPECT(ssd_status_string(code) != nullptr);

    std::printf("abi host check: %d launches accepted, %d failed expectations\n", g_launches,
                g_fail);
    return g_fail == 0 ? 0 : 1;
}
