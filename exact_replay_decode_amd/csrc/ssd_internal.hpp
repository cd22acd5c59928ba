// ssd_internal.hpp -- argument blocks passed from the C ABI layer to the
// kernel launchers. Host-side only types; every pointer is a device pointer.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace ssd {

struct Dims {
    int32_t H, G, P, N, Q;
    int32_t io_bf16;   // 1: x/B/C/y are bf16, 0: fp32
    int32_t dt_bf16;   // 1: dt is bf16, 0: fp32
    int32_t softplus;
};

// Where buffered position j of a slot lives in the buffer arrays: row
// slot * Q + j (contiguous), or row page * page_tokens + j % page_tokens
// with page = pages[slot * npp + j / page_tokens] (paged pool).
struct BufMap {
    const int32_t *pages;     // [slots, npp] or null = contiguous
    int32_t shift;            // log2(page_tokens)
    int32_t npp;              // pages per slot, Q / page_tokens
    int32_t num_pages;        // pages in the pool
};

// One chunked-scan launch over S sequences, plain or replay.
struct ScanArgs {
    Dims d;
    int32_t S;
    const int32_t *cu;        // [S+1]
    const int32_t *slot_idx;  // [S] or null (replay mode)
    const void *x, *dt, *B, *C;
    const float *A, *D, *dt_bias;
    void *y;
    // plain mode
    const float *init_state;  // [S,H,P,N] or null
    float *final_state;       // [S,H,P,N] or null
    float *boundary_state;    // [S,H,P,N] or null
    float *chunk_states;      // [full chunks,H,P,N] or null: state after each full chunk
    // replay mode (replay != 0): resume from the slot's boundary + buffer
    int32_t replay;
    int32_t num_slots;
    float *cache_state;       // [slots,H,P,N]
    void *cache_state_bf;     // [slots,H,P,N] bf16 copy of cache_state
    const void *buf_x, *buf_dt, *buf_B;
    const int32_t *buf_len;   // [slots]
    BufMap bm;
    // speculative drafts (replay mode): dry = outputs only, the cache is not
    // written (verification); no_y = no outputs, only the chunk states of
    // chunks that fill (acceptance); take[s] (device, or null) caps sequence
    // s's token count
    int32_t dry, no_y;
    const int32_t *take;
    int32_t only_cross;       // dry replay of the sequences whose drafts cross the chunk end
    // plain prefill with each head's P columns in two halves, one workgroup
    // each (launched with the half width; d.P stays the full width); 0 or 1:
    // one workgroup per head
    int32_t psplit;
    // verification: the most drafts any sequence has (host-side count)
    int32_t max_len;
    // the cache's work array (or null): the sweeps of verification and
    // acceptance take their sequences from a list kept in it
    int32_t *work;
};

// Write the trailing partial chunk of each sequence into the slot buffers
// and advance buf_len / boundary_pos; optionally copy a boundary state in.
struct CommitArgs {
    Dims d;
    int32_t S;
    const int32_t *cu;
    const int32_t *slot_idx;  // or null
    const void *x, *dt, *B, *C;
    int32_t fresh;            // 1: slot starts empty (after a plain prefill)
    int32_t num_slots;
    const float *state_src;   // [S,H,P,N] copied to the slot state, or null
    float *cache_state;
    void *cache_state_bf;     // bf16 copy, written with cache_state
    void *buf_x, *buf_dt, *buf_B, *buf_C;  // buf_C may be null
    int32_t *buf_len;
    int64_t *boundary_pos;
    BufMap bm;
    const int32_t *take;      // [S] caps each sequence's token count, or null
};

struct DecodeArgs {
    Dims d;
    int32_t batch;
    const int32_t *slot_idx;  // or null
    const void *x, *dt, *B, *C;  // new token [batch,...]
    const float *A, *D, *dt_bias;
    void *y;
    int32_t num_slots;
    float *cache_state;
    void *cache_state_bf;     // bf16 copy of cache_state
    void *buf_x, *buf_dt, *buf_B, *buf_C;
    int32_t *buf_len;
    int64_t *boundary_pos;
    int32_t *work;            // [2*slots+34]: arrival counters [slots], commit-list
                              // count and done counters [34], commit list [slots]
    BufMap bm;
    const int32_t *order;     // or null: batch positions by rank, heaviest first
    // with the conv before the scan in the same launch (xBC non-null): the
    // token's x | B | C are the causal conv of xBC [batch, conv_dim] (width
    // cW, taps cw [conv_dim, cW], bias cb, SiLU if cact) over the slot's conv
    // state cstate [slots, conv_dim, cW - 1], written to x, B, C, which the
    // step then reads as its inputs
    const void *xBC;
    const float *cw, *cb;
    void *cstate;
    int32_t cW, cact;
};

// Causal depthwise conv1d before the scan: prefill (S sequences of a varlen
// pack) or decode (S = batch rows of one token).
struct ConvArgs {
    Dims d;                   // H, G, P, N, io dtype (conv_dim = H*P + 2*G*N)
    int32_t W;                // kernel width, 2..4
    int32_t act;              // 1: SiLU after the conv
    int32_t S;
    const int32_t *cu;        // [S+1] (prefill)
    int32_t maxlen;           // longest sequence (prefill)
    const int32_t *slot_idx;  // [S] or null
    int32_t num_slots;
    const void *xBC;          // [T, conv_dim]
    const float *weight;      // [conv_dim, W]
    const float *bias;        // [conv_dim] or null
    void *state;              // [slots, conv_dim, W-1] or null (prefill)
    void *x, *B, *C;          // outputs [T,H,P], [T,G,N], [T,G,N]
};

// Recurrent update: batch rows of one token each, or (cu given) batch
// sequences of a varlen pack, each a run of tokens.
struct SsuArgs {
    Dims d;
    int32_t batch;
    const int32_t *slot_idx;
    int32_t num_slots;
    void *state;              // [slots,H,P,N] fp32, or bf16 when state_bf16
    int32_t state_bf16;
    const int32_t *cu;        // [batch+1] or null
    const void *x, *dt, *B, *C;
    const float *A, *D, *dt_bias;
    void *y;
};

// fp32-FMA engine (any supported shape; the only engine for fp32 x/B/C)
hipError_t launch_scan(const ScanArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// matrix-core engine (bf16 x/B/C/y, P in {32, 64}, N in {32, 64, 128})
bool mfma_supported(const Dims &d);
hipError_t launch_scan_mfma(const ScanArgs &a, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_verify_mfma(const ScanArgs &a, hipStream_t stream);   // dry replay of drafts
// causal conv1d (ssd_conv.hip)
hipError_t launch_conv_fwd(const ConvArgs &a, hipStream_t stream);
hipError_t launch_conv_update(const ConvArgs &a, hipStream_t stream);
// shared by both engines
hipError_t launch_decode_advance(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_commit(const CommitArgs &a, hipStream_t stream);
hipError_t launch_ssu(const SsuArgs &a, hipStream_t stream);
// the library's own decode bookkeeping array (ssd_scratch.hip): caches of
// at most kStaticMaxSlots slots; *out = this device's copy (all zero
// between calls), cleared on the stream at its first use on the device
constexpr int32_t kStaticMaxSlots = 32768;
hipError_t static_work(int32_t **out, hipStream_t stream);
// synchronous device -> host copy (debug-build argument checks only)
hipError_t copy_to_host(void *dst, const void *src, size_t bytes);
// bf16 copy of `heads` fp32 [P][N] states (the cache's read-out operand)
hipError_t launch_refresh_state_bf(const float *state, void *state_bf, int64_t heads, int P, int N,
                                   hipStream_t stream);

}  // namespace ssd
