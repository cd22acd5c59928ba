/*
 * ssd_replay.h -- C ABI of the MI355X (gfx950) Mamba2 SSD scan with
 * exact-replay decode.
 *
 * Sources (web pages; the code cites them by title and section):
 *  [RFC]  vLLM RFC "Mamba2: exact-replay decode so that prefill, chunked
 *         prefill and decode produce identical bits".
 *  [RSSM] ReplaySSM reproduction README, "Cache SSM inputs instead of
 *         writing back state for every token".
 *
 * The scan (per head h, group g = h / (H/G), token t):
 *   delta_t = softplus(dt_t + dt_bias[h])      (dt_softplus = 1)
 *           = dt_t + dt_bias[h]                (dt_softplus = 0)
 *   state   = exp(delta_t A[h]) state + delta_t x_t (outer) B_t   [P x N]
 *   y_t     = state . C_t + D[h] x_t                               [P]
 * computed chunk by chunk ([RFC] section 1 names the chunked scan; [RSSM]
 * "Core equations" give the per-chunk closed form) on a chunk grid anchored
 * at each sequence's boundary position.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless their name ends in _host. Arrays are
 *    row-major and contiguous with the layouts given below. x, B, C, y, every
 *    state array and the x/B/C buffers must be 16-byte aligned (the kernels
 *    move them in 16-byte pieces); other arrays need their natural alignment.
 *  - T = packed token count, S = number of sequences, Q = chunk_size.
 *    x, y: [T,H,P]; dt: [T,H] (raw dt); B, C: [T,G,N]; A, D, dt_bias: [H]
 *    fp32; states: [.,H,P,N] fp32; cu_seqlens: [S+1] int32, cu[0] = 0,
 *    non-decreasing, cu[S] = T.
 *  - Every call is asynchronous on `stream`, allocates no device memory and
 *    returns SSD_OK (0) or a negative ssd_status. All argument checks run on
 *    the host before anything is launched, so a failed check launches
 *    nothing. Launch failures map to SSD_ERR_HIP. No exception crosses the
 *    ABI.
 *  - The caller owns every buffer; the library frees nothing and keeps no
 *    per-call state. Outputs must not alias inputs unless stated.
 *  - Results are deterministic: fixed tile shapes, fixed reduction orders,
 *    no atomics in arithmetic.
 */
#ifndef SSD_REPLAY_H
#define SSD_REPLAY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,            /* a required pointer is NULL */
    SSD_ERR_SHAPE = -2,           /* sizes inconsistent (H % G, cu_seqlens, counts) */
    SSD_ERR_DTYPE = -3,           /* unknown dtype code */
    SSD_ERR_STATE_NOT_FP32 = -4,  /* [RFC] section 4: fp32 state is required */
    SSD_ERR_CHUNK_MISMATCH = -5,  /* [RFC] section 4: one chunk size for prefill and decode */
    SSD_ERR_WORKSPACE = -6,       /* workspace missing or too small */
    SSD_ERR_UNSUPPORTED = -7,     /* P, N or chunk_size outside the built set */
    SSD_ERR_HIP = -8,             /* a HIP launch or runtime call failed */
    SSD_ERR_ALIGN = -9            /* a token, state or buffer array is not 16-byte aligned */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Problem shape shared by all calls.
 * Supported: chunk_size in {16,32,64,128,256}; P and N in {16,32,64,128};
 * H % G == 0; io_dtype (x, B, C, y) and dt_dtype in {SSD_F32, SSD_BF16};
 * state_dtype must be SSD_F32, except that the recurrent update
 * (ssm_state_update, ssm_state_update_varlen) also takes SSD_BF16. */
typedef struct {
    int32_t H, G, P, N, chunk_size;
    int32_t io_dtype;
    int32_t dt_dtype;
    int32_t state_dtype;
    int32_t dt_softplus;
} ssd_shape;

/* Exact-replay cache for num_slots sequences ([RFC] section 3, "State
 * representation"): the fp32 state at the last multiple of the chunk size
 * plus a token-major buffer of the inputs received since then.
 *   state         [num_slots,H,P,N] fp32   boundary state
 *   state_bf      [num_slots,H,N/16,P,16]  the boundary state rounded to bf16
 *                 bf16                     (nearest even), element (p, n) of a
 *                                          head at (n/16)*16P + 16p + n%16: the
 *                                          operand of the state read-out, which
 *                                          rounds the state to bf16 in prefill
 *                                          too. Written by the library whenever
 *                                          it writes state; decode reads it
 *                                          instead of the fp32 state (half the
 *                                          bytes). A caller that writes state
 *                                          itself calls ssd_replay_cache_refresh.
 *   buf_x         [num_slots,Q,H,P] io     buffered x
 *   buf_dt        [num_slots,Q,H]   dt     buffered raw dt ([RFC] section 3:
 *                                          raw dt, not softplus(dt + bias))
 *   buf_B, buf_C  [num_slots,Q,G,N] io     buffered B and C; buf_C may be NULL
 *                                          (the scan never reads buffered C)
 *   buf_len       [num_slots] int32        tokens buffered, in [0, Q)
 *   boundary_pos  [num_slots] int64        sequence position of the boundary,
 *                                          a multiple of Q
 *   work          [2*num_slots+34] int32   bookkeeping: per-slot arrival
 *                                          counters (the last workgroup of
 *                                          a slot advances buf_len), done
 *                                          counters, and a list area: a
 *                                          large decode batch's ranking
 *                                          (positions, heaviest first), the
 *                                          slots whose chunk filled in this
 *                                          step, or the sequences the
 *                                          verification / acceptance sweep
 *                                          replays; zero before first use,
 *                                          and every call leaves it zero
 * A fresh slot is all zeros. The struct itself is a host object; the
 * pointers in it are device pointers.
 *
 * Paged buffers ([RFC] section 6, implementation notes: the buffers live in
 * the paged mamba cache, so slot and position are indexed separately). With
 * buf_pages == NULL the buffers are contiguous per slot as above. Otherwise
 * buf_x, buf_dt, buf_B and buf_C are pools of num_pages pages of page_tokens
 * rows each ([num_pages,page_tokens,H,P] and so on), and buffered position
 * j of a slot is row j % page_tokens of page buf_pages[slot][j / page_tokens]:
 *   buf_pages     [num_slots,Q/page_tokens] int32, on the device
 *   page_tokens   a power of two with 16 <= page_tokens <= Q
 *   num_pages     pages in each pool (> 0)
 * The state, its bf16 copy, buf_len and boundary_pos stay indexed by slot.
 * Only the entries of the positions a call reads or writes need to be
 * pages (positions 0..buf_len for a decode step; up to the larger of the
 * buffered and the trailing tokens for a prefill or commit), so pages can
 * be handed out as a slot's buffer grows and returned when its chunk
 * completes. If such an entry is outside [0, num_pages), that sequence is
 * skipped: nothing of its slot and none of its outputs are written. Entries
 * in use must not share a page. */
typedef struct {
    float *state;
    void *state_bf;
    void *buf_x;
    void *buf_dt;
    void *buf_B;
    void *buf_C;
    int32_t *buf_len;
    int64_t *boundary_pos;
    int32_t *work;
    int32_t num_slots;
    int32_t chunk_size;
    int32_t state_dtype;
    const int32_t *buf_pages;
    int32_t page_tokens;
    int32_t num_pages;
} ssd_replay_cache;

/* Rebuild the bf16 state copy (state_bf) of every slot from the fp32 state,
 * for a caller that wrote cache->state itself. */
int ssd_replay_cache_refresh(const ssd_shape *shape, const ssd_replay_cache *cache,
                             hipStream_t stream);

/* Human-readable name of a status code. Never NULL. */
const char *ssd_status_string(int status);

/* Bytes of device memory one exact-replay cache of num_slots slots needs
 * (state, its bf16 copy, buffers and metadata), with or without the C
 * buffer; 0 for a bad shape. [RFC] section 4 sizes the buffer at about
 * 1.16 MiB and the fp32 state at 1 MiB per layer and sequence for H=32, G=1,
 * P=64, N=128, Q=256; the bf16 copy adds 0.5 MiB. */
size_t ssd_replay_cache_bytes(const ssd_shape *shape, int32_t num_slots,
                              int32_t with_C);

/* Bytes of one buffer page of page_tokens rows (x, raw dt, B and, with
 * with_C, C) for a paged cache; 0 for a bad shape or page size. */
size_t ssd_replay_page_bytes(const ssd_shape *shape, int32_t page_tokens,
                             int32_t with_C);

/* Workspace bytes ssd_prefill_varlen needs (currently 0: the prefill kernel
 * carries the inter-chunk state on chip). */
size_t ssd_prefill_workspace_bytes(const ssd_shape *shape, int32_t num_seqs,
                                   int64_t total_tokens);

/* Chunked scan over a varlen pack ([RFC] section 1: the prefill kernel;
 * section 2, item 3: prefix- and packing-invariant; item 4: fp32 carry
 * between chunks).
 * Each sequence s starts from init_state[s] (NULL = zeros) on a chunk grid
 * anchored at its first token; chunks never straddle sequences.
 *   y              [T,H,P]   all rows written
 *   final_state    [S,H,P,N] state after the last token (NULL = not stored)
 *   boundary_state [S,H,P,N] state after the last full chunk, i.e. after
 *                  len - len % Q tokens; init_state when len < Q (NULL = not
 *                  stored)
 *   chunk_states   [F,H,P,N] the intermediate states ([RFC] section 3,
 *                  prefill bullet: the boundary is taken from the state at
 *                  the end of the last full chunk, as prefix caching takes
 *                  its block states): row off(s) + c holds the state after
 *                  (c + 1) * Q tokens of sequence s, for every full chunk
 *                  c < len_s / Q, where off(s) = sum over s' < s of
 *                  floor(len_s' / Q) and F = off(S)
 *                  (ssd_prefill_chunk_count). Bit-identical to the state the
 *                  same tokens leave in boundary_state. NULL = not stored.
 * cu_seqlens_host is read synchronously for the checks; cu_seqlens is the
 * same array on the device. */
int ssd_prefill_varlen(const ssd_shape *shape, int32_t num_seqs,
                       int64_t total_tokens, const int32_t *cu_seqlens_host,
                       const int32_t *cu_seqlens, const void *x, const void *dt,
                       const float *A, const void *B, const void *C,
                       const float *D, const float *dt_bias,
                       const float *init_state, void *y, float *final_state,
                       float *boundary_state, float *chunk_states,
                       void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Rows F of ssd_prefill_varlen's chunk_states for a pack: the number of full
 * chunks, sum over sequences of floor(len_s / chunk_size), from the host
 * copy of cu_seqlens (cu[0] = 0, non-decreasing). -1 for a NULL array, a
 * negative count, a decreasing cu_seqlens or a chunk_size < 1. */
int64_t ssd_prefill_chunk_count(int32_t num_seqs, const int32_t *cu_seqlens_host,
                                int32_t chunk_size);

/* Store a fresh prefill into replay-cache slots ([RFC] section 3, "Prefill
 * / chunked prefill / recompute": the boundary state comes from the last
 * full chunk and the trailing partial chunk's inputs go to the buffer).
 * For sequence s of the pack (its x/dt/B/C as passed to ssd_prefill_varlen,
 * its boundary_state[s] as that call returned it) and slot = slot_idx[s]
 * (NULL = s): state <- boundary_state[s]; buffer <- the last len % Q
 * tokens; buf_len <- len % Q; boundary_pos <- len - len % Q.
 * slot_idx entries must be distinct and < cache->num_slots. */
int ssd_commit_boundary(const ssd_shape *shape, int32_t num_seqs,
                        int64_t total_tokens, const int32_t *cu_seqlens_host,
                        const int32_t *cu_seqlens, const int32_t *slot_idx,
                        const void *x, const void *dt, const void *B,
                        const void *C, const float *boundary_state,
                        const ssd_replay_cache *cache, hipStream_t stream);

/* Exact-replay prefill, chunked prefill or recompute ([RFC] section 3,
 * second bullet): every sequence resumes at its slot's boundary. The
 * buffered tokens are put in front of the new ones, their outputs are not
 * written, the chunk grid is the slot's, and afterwards the slot holds the
 * state after the last full chunk and the trailing partial chunk.
 * Sequence s has new tokens cu[s]..cu[s+1]-1 and uses slot slot_idx[s]
 * (NULL = s); y[T,H,P] receives the new tokens' outputs. Zero-length
 * sequences leave their slot untouched. Slots must be distinct. */
int ssd_replay_prefill(const ssd_shape *shape, const ssd_replay_cache *cache,
                       int32_t num_seqs, int64_t total_tokens,
                       const int32_t *cu_seqlens_host, const int32_t *cu_seqlens,
                       const int32_t *slot_idx, const void *x, const void *dt,
                       const void *B, const void *C, const float *A,
                       const float *D, const float *dt_bias, void *y,
                       hipStream_t stream);

/* Exact-replay decode step ([RFC] section 3, first bullet): one new token
 * per sequence. For slot = slot_idx[b] (NULL = b) holding k = buf_len
 * tokens, the chunk made of the k buffered tokens plus the new token is
 * replayed from the boundary state through the prefill's chunk arithmetic,
 * and the new token's output row goes to y[b]. The token is appended to the
 * buffer; when it fills the chunk (k + 1 == Q) the chunk's end state becomes
 * the boundary state, buf_len returns to 0 and boundary_pos advances by Q.
 * y[b] is bit-identical to the row a single ssd_prefill_varlen over the
 * whole sequence produces. Inputs x[batch,H,P], dt[batch,H],
 * B/C[batch,G,N]; y[batch,H,P]. Slots must be distinct; a position whose
 * slot_idx entry is outside [0, num_slots) is skipped (its y row is not
 * written). One launch, or two for a batch with more workgroups than the
 * device runs at once (a ranking of the positions, heaviest first, goes
 * ahead of the step); no host synchronisation either way. */
int ssd_replay_decode(const ssd_shape *shape, const ssd_replay_cache *cache,
                      int32_t batch, const int32_t *slot_idx, const void *x,
                      const void *dt, const void *B, const void *C,
                      const float *A, const float *D, const float *dt_bias,
                      void *y, hipStream_t stream);

/* ssd_replay_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same step, bit for bit, but the decode bookkeeping lives
 * in the library's own per-GPU array instead of cache->work, which is not
 * read and may be NULL. Nothing is allocated on any call. Limits and
 * sharing:
 *  - cache->num_slots <= 32768 (the array holds 2 * 32768 + 34 int32 words
 *    per GPU, kept until the process ends); larger caches get
 *    SSD_ERR_WORKSPACE and nothing is launched;
 *  - every call on one GPU uses that GPU's one array: calls that overlap in
 *    time on one GPU (streams without an ordering between them) race and
 *    give undefined results; calls ordered on one stream are fine;
 *  - each call leaves the array zero; the first call on a device clears it
 *    with a small kernel on `stream` before the step.
 * Returns what ssd_replay_decode returns, plus SSD_ERR_HIP when the array's
 * address cannot be looked up. */
int ssd_replay_decode_static(const ssd_shape *shape, const ssd_replay_cache *cache,
                             int32_t batch, const int32_t *slot_idx, const void *x,
                             const void *dt, const void *B, const void *C,
                             const float *A, const float *D, const float *dt_bias,
                             void *y, hipStream_t stream);

/* Decode step with the causal conv before the scan in the same launch
 * ([RFC] section 2, item 6: the conv's decode form, before the SSM decode):
 * ssd_conv1d_update(shape, width, activation, batch, slot_idx,
 * cache->num_slots, xBC, weight, bias, conv_state, x, B, C) followed by
 * ssd_replay_decode(shape, cache, batch, slot_idx, x, dt, B, C, A, D,
 * dt_bias, y), bit for bit, as one launch (plus the ranking launch that
 * ssd_replay_decode may put ahead) when the matrix-core engine runs the
 * shape with bf16 I/O and (H / G) % 4 == 0, else as those two calls.
 * x [batch,H,P] and B/C [batch,G,N] are outputs here (the conv's, which the
 * step then reads); conv_state [num_slots, conv_dim, width - 1] is indexed
 * by the cache's slots and updated in place. Arguments and errors as for
 * the two calls; a position the step skips (slot out of range) gets no
 * conv either. */
int ssd_replay_decode_conv(const ssd_shape *shape, const ssd_replay_cache *cache,
                           int32_t batch, const int32_t *slot_idx, int32_t width,
                           int32_t activation, const void *xBC, const float *weight,
                           const float *bias, void *conv_state, void *x, void *B, void *C,
                           const void *dt, const float *A, const float *D,
                           const float *dt_bias, void *y, hipStream_t stream);

/* Speculative verification, output only ([RSSM] "Motivation and method":
 * drafts are verified with an output-only form instead of materialising a
 * state per draft; the acceptance length then advances only the committed
 * input pointer, and rejected drafts never enter the recurrence).
 * Sequence s has draft tokens cu[s]..cu[s+1]-1 (x/dt/B/C as in prefill) and
 * slot slot_idx[s] (NULL = s). The drafts are replayed after the slot's
 * committed tokens through the prefill's chunk arithmetic, crossing chunk
 * boundaries on chip, and y[T,H,P] receives every draft's output. Nothing in
 * the cache is written. Draft j's output is bit-identical to the one a
 * decode step would give it after drafts 0..j-1 were accepted. Paged
 * caches need pages for the committed positions only. Slots distinct. */
int ssd_replay_verify(const ssd_shape *shape, const ssd_replay_cache *cache,
                      int32_t num_seqs, int64_t total_tokens,
                      const int32_t *cu_seqlens_host, const int32_t *cu_seqlens,
                      const int32_t *slot_idx, const void *x, const void *dt,
                      const void *B, const void *C, const float *A,
                      const float *D, const float *dt_bias, void *y,
                      hipStream_t stream);

/* Acceptance after ssd_replay_verify: commit the first accepted[s] drafts
 * of each sequence (accepted: device int32 [S], clamped to [0, drafts]) as
 * if they had been decoded one by one: they are appended to the slot's
 * buffer, and each chunk they fill becomes the new boundary state (the
 * prefill's chunk-state update); buf_len and boundary_pos advance. The
 * drafts are passed again exactly as to the verification; the rejected ones
 * are never read. No outputs are computed (D is not needed); C is read only
 * when the cache buffers C. Slots distinct. */
int ssd_replay_accept(const ssd_shape *shape, const ssd_replay_cache *cache,
                      int32_t num_seqs, int64_t total_tokens,
                      const int32_t *cu_seqlens_host, const int32_t *cu_seqlens,
                      const int32_t *slot_idx, const int32_t *accepted,
                      const void *x, const void *dt, const void *B, const void *C,
                      const float *A, const float *dt_bias, hipStream_t stream);

/* Recurrent selective-state update, the conventional decode path the RFC
 * compares against ([RFC] section 1; [RSSM] "Motivation and method": it
 * reads and writes the full state every token). For slot = slot_idx[b]
 * (NULL = b): h = exp(delta A) state[slot] + delta x (outer) B in fp32;
 * y[b] <- h . C + D x; state[slot] <- h stored in the cache dtype.
 * shape->state_dtype selects that dtype: SSD_F32, or SSD_BF16 (rounded to
 * nearest even; the RFC's default cache). state is [num_slots,H,P,N],
 * updated in place; x[batch,H,P], dt[batch,H], B/C[batch,G,N],
 * y[batch,H,P]. Slots must be distinct. */
int ssm_state_update(const ssd_shape *shape, int32_t batch, int32_t num_slots,
                     const int32_t *slot_idx, void *state, const void *x,
                     const void *dt, const float *A, const void *B,
                     const void *C, const float *D, const float *dt_bias,
                     void *y, hipStream_t stream);

/* Multi-token recurrent update over a varlen pack, for packed-history
 * recovery ([RFC] section 3b: generated history is replayed with a
 * multi-token recurrent update that rounds the state to the cache dtype
 * after every token, so the recovered state continues exactly like an
 * uninterrupted decode). Sequence s (tokens cu[s]..cu[s+1]-1) advances
 * state[slot_idx[s]] (NULL = s) token by token with the arithmetic and the
 * per-token rounding of ssm_state_update, so the outputs y[T,H,P] and the
 * final state are bit-identical to one ssm_state_update call per token. The
 * state stays on chip between tokens. Slots must be distinct. */
int ssm_state_update_varlen(const ssd_shape *shape, int32_t num_seqs,
                            int64_t total_tokens, const int32_t *cu_seqlens_host,
                            const int32_t *cu_seqlens, const int32_t *slot_idx,
                            int32_t num_slots, void *state, const void *x,
                            const void *dt, const float *A, const void *B,
                            const void *C, const float *D, const float *dt_bias,
                            void *y, hipStream_t stream);

/* Causal depthwise conv1d, the step before the scan ([RFC] section 2, item
 * 6: its prefill form and its decode form give the same bits; bf16 operands
 * are promoted to fp32 before the accumulation). The channels are the
 * concatenated projection xBC = [x (H*P) | B (G*N) | C (G*N)], conv_dim =
 * H*P + 2*G*N, and for channel c, kernel width W in {2,3,4}:
 *   out_t[c] = act(bias[c] + sum_{i<W} weight[c][i] * in_{t-W+1+i}[c])
 * in fp32, as an fmaf chain from the bias over i = 0..W-1, with act(v) =
 * v / (1 + exp(-v)) (SiLU) when activation != 0, else the identity. Inputs
 * before a sequence come from its conv state: the W-1 previous inputs,
 * oldest first. Outputs go straight to the scan's inputs x [T,H,P],
 * B [T,G,N], C [T,G,N] (io_dtype; bf16 rounds to nearest even).
 *   xBC         [T, conv_dim]               io_dtype
 *   weight      [conv_dim, W]               fp32
 *   bias        [conv_dim] fp32 or NULL (zeros)
 *   conv_state  [num_slots, conv_dim, W-1]  io_dtype, channel-major
 * Both forms evaluate every output with the same device routine on the same
 * W inputs, so decoding token by token reproduces the prefill's bits, and a
 * prefill split at any point reproduces the unsplit one. Pointers,
 * weight and bias included, are 16-byte aligned (SSD_ERR_ALIGN).
 * shape->chunk_size and dt_dtype are not used (any valid value). */

/* Prefill form over a varlen pack. Sequence s (tokens cu[s]..cu[s+1]-1)
 * starts from conv_state[slot_idx[s]] (slot_idx NULL = s) and leaves there
 * its last W-1 inputs (for a sequence shorter than W-1, the newer rows of
 * the old state followed by its inputs). The state is read before it is
 * written, so in-place use is the normal case; a fresh slot must be zero.
 * conv_state NULL: zero history, nothing stored (slot_idx and num_slots
 * ignored). Slots must be distinct. S <= 65535. */
int ssd_conv1d_varlen(const ssd_shape *shape, int32_t width, int32_t activation,
                      int32_t num_seqs, int64_t total_tokens,
                      const int32_t *cu_seqlens_host, const int32_t *cu_seqlens,
                      const int32_t *slot_idx, int32_t num_slots, const void *xBC,
                      const float *weight, const float *bias, void *conv_state,
                      void *x, void *B, void *C, hipStream_t stream);

/* Decode form: one token per row b (xBC [batch, conv_dim]); slot =
 * slot_idx[b] (NULL = b); conv_state[slot] is updated in place; outputs x
 * [batch,H,P], B/C [batch,G,N]. Slots must be distinct. batch <= 65535. */
int ssd_conv1d_update(const ssd_shape *shape, int32_t width, int32_t activation,
                      int32_t batch, const int32_t *slot_idx, int32_t num_slots,
                      const void *xBC, const float *weight, const float *bias,
                      void *conv_state, void *x, void *B, void *C, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_REPLAY_H */
