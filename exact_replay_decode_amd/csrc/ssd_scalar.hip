// ssd_scalar.hip -- chunked scan, exact-replay decode, boundary commit and
// the recurrent state update, computed with fp32 FMAs in fixed orders.
//
// The chunk arithmetic is the per-chunk closed form of the ReplaySSM
// reproduction page ("Core equations"), per head h and chunk of Q tokens
// starting from state S0 (lam = in-chunk inclusive cumulative sum of
// delta*A):
//   y_i   = exp(lam_i) (C_i . S0) + sum_{j<=i} (C_i . B_j) exp(lam_i - lam_j)
//           delta_j x_j + D x_i
//   S_end = exp(lam_last) S0 + sum_j exp(lam_last - lam_j) delta_j x_j B_j^T
// The vLLM RFC "Mamba2: exact-replay decode ..." (section 3) replays a
// partial chunk from the fp32 boundary state through this same arithmetic
// to decode. Bit identity between the two follows from three facts that the
// code below keeps:
//  * every output entry (row i, column p) and every state entry (p, n) is a
//    sequential fmaf chain over a fixed index order (n ascending, j
//    ascending) that reads only tokens 0..i of the chunk;
//  * the in-chunk scan is prefix-consistent (ssd_device.hpp);
//  * the decode kernel calls the very same device functions (emit_rows,
//    chunk_state_update) with a chunk view whose first k positions read the
//    slot buffer.
#include <algorithm>

#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kRows = 16;  // output rows per tile
constexpr int kJB = 32;    // tokens per staged block
constexpr int kMaxE = kRows * 128 / kBlock;  // output entries per thread
constexpr int kMaxS = 128 * 128 / kBlock;    // state entries per thread

// Offsets (in floats) of the scan kernels' LDS regions.
struct LdsLayout {
    int S, Ct, Bb, xb, Mb, lam, dlt, wb, tot, total;
    __host__ __device__ LdsLayout(int P, int N) {
        int o = 0;
        S = o;   o += P * (N + 1);
        Ct = o;  o += kRows * (N + 1);
        Bb = o;  o += kJB * (N + 1);
        xb = o;  o += kJB * P;
        Mb = o;  o += kRows * kJB;
        lam = o; o += kMaxQ;
        dlt = o; o += kMaxQ;
        wb = o;  o += kJB;
        tot = o; o += 8;
        total = o;
    }
};

// Buffer row of buffered position j of a slot: slot * Q + j, or through the
// slot's page-table entry when the buffers are paged.
__device__ __forceinline__ int64_t buf_row(const BufMap &m, int slot, int Q, int j) {
    if (!m.pages)
        return (int64_t)slot * Q + j;
    return ((int64_t)m.pages[(int64_t)slot * m.npp + (j >> m.shift)] << m.shift) +
           (j & ((1 << m.shift) - 1));
}

// Whether the page-table entries of the slot's positions [0, npos) are pages
// of the pool (always true for contiguous buffers).
__device__ bool buf_pages_ok(const BufMap &m, int slot, int npos) {
    if (!m.pages)
        return true;
    const int n = (npos + (1 << m.shift) - 1) >> m.shift;
    for (int i = 0; i < n; ++i) {
        const int pg = m.pages[(int64_t)slot * m.npp + i];
        if (pg < 0 || pg >= m.num_pages)
            return false;
    }
    return true;
}

// Where chunk position j of the current chunk lives: positions [0, nb) in
// the slot buffer, positions [nb, n_valid) in the packed input starting at
// token tok_base. Positions >= n_valid do not exist.
template <class IO, class DT>
struct ChunkView {
    using T = typename IO::T;
    using TD = typename DT::T;
    const T *x, *B, *C;
    const TD *dt;
    const T *bx, *bB;      // buffer arrays (whole pool)
    const TD *bdt;
    BufMap bm;
    int slot, Q;
    int64_t tok_base;
    int nb, n_valid;
    int h, g, H, G, P, N;

    __device__ int64_t brw(int j) const { return buf_row(bm, slot, Q, j); }
    __device__ const T *xrow(int j) const {
        return j < nb ? bx + (brw(j) * H + h) * P
                      : x + ((tok_base + (j - nb)) * H + h) * P;
    }
    __device__ float dtv(int j) const {
        return j < nb ? DT::ld(bdt, brw(j) * H + h)
                      : DT::ld(dt, (tok_base + (j - nb)) * H + h);
    }
    __device__ const T *brow(int j) const {
        return j < nb ? bB + (brw(j) * G + g) * N
                      : B + ((tok_base + (j - nb)) * G + g) * N;
    }
    // C is only read for rows whose output is produced (never buffered rows)
    __device__ const T *crow(int j) const { return C + ((tok_base + (j - nb)) * G + g) * N; }
    __device__ int64_t token(int j) const { return tok_base + (j - nb); }
};

// delta and lam for the chunk; lanes past n_valid contribute zero.
template <class IO, class DT>
__device__ void prepare_chunk(const ChunkView<IO, DT> &v, float A_h, float bias,
                              int softplus, float *lds, const LdsLayout &L) {
    const int j = threadIdx.x;
    float d = 0.0f, a = 0.0f;
    if (j < v.n_valid) {
        d = delta_of(v.dtv(j), bias, softplus);
        a = d * A_h;
    }
    const float l = block_scan_inclusive(a, lds + L.tot);
    lds[L.lam + j] = l;
    lds[L.dlt + j] = d;
    __syncthreads();
}

// Outputs of chunk rows [r0, r1) (r1 - r0 <= kRows) from the state S held in
// LDS. y row i goes to packed token v.token(i).
template <class IO, class DT>
__device__ void emit_rows(const ChunkView<IO, DT> &v, int r0, int r1, float D_h,
                          typename IO::T *y, float *lds, const LdsLayout &L) {
    const int tid = threadIdx.x;
    const int P = v.P, N = v.N, N1 = N + 1;
    const int nr = r1 - r0;
    float *S = lds + L.S, *Ct = lds + L.Ct, *Bb = lds + L.Bb, *xb = lds + L.xb;
    float *Mb = lds + L.Mb;
    const float *lam = lds + L.lam, *dlt = lds + L.dlt;

    for (int e = tid; e < nr * N; e += kBlock) {
        const int r = e / N, n = e % N;
        Ct[r * N1 + n] = IO::ld(v.crow(r0 + r), n);
    }
    float acc_in[kMaxE];
#pragma unroll
    for (int k = 0; k < kMaxE; ++k)
        acc_in[k] = 0.0f;
    __syncthreads();

    for (int jb = 0; jb < r1; jb += kJB) {
        const int nj = min(kJB, r1 - jb);
        for (int e = tid; e < nj * N; e += kBlock) {
            const int jj = e / N, n = e % N;
            Bb[jj * N1 + n] = IO::ld(v.brow(jb + jj), n);
        }
        for (int e = tid; e < nj * P; e += kBlock) {
            const int jj = e / P, p = e % P;
            xb[jj * P + p] = IO::ld(v.xrow(jb + jj), p);
        }
        __syncthreads();
        for (int e = tid; e < nr * kJB; e += kBlock) {
            const int r = e / kJB, jj = e % kJB;
            const int i = r0 + r, j = jb + jj;
            float m = 0.0f;
            if (jj < nj && j <= i) {
                float cb = 0.0f;
                for (int n = 0; n < N; ++n)
                    cb = fmaf(Ct[r * N1 + n], Bb[jj * N1 + n], cb);
                m = intra_weight(cb, lam[i], lam[j], dlt[j]);
            }
            Mb[r * kJB + jj] = m;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxE; ++k) {
            const int e = tid + kBlock * k;
            if (e < nr * P) {
                const int r = e / P, p = e % P;
                const int jmax = min(nj, r0 + r - jb + 1);
                float acc = acc_in[k];
                for (int jj = 0; jj < jmax; ++jj)
                    acc = fmaf(Mb[r * kJB + jj], xb[jj * P + p], acc);
                acc_in[k] = acc;
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int k = 0; k < kMaxE; ++k) {
        const int e = tid + kBlock * k;
        if (e < nr * P) {
            const int r = e / P, p = e % P, i = r0 + r;
            float acc_off = 0.0f;
            for (int n = 0; n < N; ++n)
                acc_off = fmaf(Ct[r * N1 + n], S[p * N1 + n], acc_off);
            const float xv = IO::ld(v.xrow(i), p);
            float yv = fmaf(decay_exp(lam[i]), acc_off, acc_in[k]);
            yv = fmaf(D_h, xv, yv);
            yv = yv + 0.0f;  // -0 -> +0
            y[(v.token(i) * v.H + v.h) * P + p] = IO::cvt(yv);
        }
    }
    __syncthreads();
}

// S <- exp(lam_last) S + sum_{j < n_valid} exp(lam_last - lam_j) delta_j x_j B_j^T
// with lam_last = lam[n_valid - 1]; S in LDS.
template <class IO, class DT>
__device__ void chunk_state_update(const ChunkView<IO, DT> &v, float *lds, const LdsLayout &L) {
    const int tid = threadIdx.x;
    const int P = v.P, N = v.N, N1 = N + 1;
    const int ne = P * N / kBlock;
    float *S = lds + L.S, *Bb = lds + L.Bb, *xb = lds + L.xb, *wb = lds + L.wb;
    const float *lam = lds + L.lam, *dlt = lds + L.dlt;
    const float lam_last = lam[v.n_valid - 1];

    float acc[kMaxS];
#pragma unroll
    for (int k = 0; k < kMaxS; ++k)
        acc[k] = 0.0f;

    for (int jb = 0; jb < v.n_valid; jb += kJB) {
        const int nj = min(kJB, v.n_valid - jb);
        for (int e = tid; e < nj * N; e += kBlock) {
            const int jj = e / N, n = e % N;
            Bb[jj * N1 + n] = IO::ld(v.brow(jb + jj), n);
        }
        for (int e = tid; e < nj * P; e += kBlock) {
            const int jj = e / P, p = e % P;
            xb[jj * P + p] = IO::ld(v.xrow(jb + jj), p);
        }
        if (tid < nj)
            wb[tid] = state_weight(lam_last, lam[jb + tid], dlt[jb + tid]);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxS; ++k) {
            if (k < ne) {
                const int e = tid + kBlock * k;
                const int p = e / N, n = e % N;
                float a = acc[k];
                for (int jj = 0; jj < nj; ++jj)
                    a = fmaf(wb[jj] * xb[jj * P + p], Bb[jj * N1 + n], a);
                acc[k] = a;
            }
        }
        __syncthreads();
    }
    const float dec = decay_exp(lam_last);
#pragma unroll
    for (int k = 0; k < kMaxS; ++k) {
        if (k < ne) {
            const int e = tid + kBlock * k;
            const int p = e / N, n = e % N;
            S[p * N1 + n] = fmaf(dec, S[p * N1 + n], acc[k]);
        }
    }
    __syncthreads();
}

__device__ void state_load(float *S, const float *src, int P, int N) {
    const int N1 = N + 1;
    for (int e = threadIdx.x; e < P * N; e += kBlock) {
        const int p = e / N, n = e % N;
        S[p * N1 + n] = src ? src[e] : 0.0f;
    }
    __syncthreads();
}

// fp32 state out of LDS; with dst_bf, also its bf16 copy (nearest even)
__device__ void state_store(float *dst, const float *S, int P, int N,
                            uint16_t *dst_bf = nullptr) {
    const int N1 = N + 1;
    for (int e = threadIdx.x; e < P * N; e += kBlock) {
        const int p = e / N, n = e % N;
        const float v = S[p * N1 + n];
        dst[e] = v;
        if (dst_bf)
            dst_bf[state_bf_index(p, n, P)] = bf16_rne(v);
    }
}

// One workgroup per (head, sequence); chunks in order, the fp32 state stays
// in LDS from one chunk to the next.
template <class IO, class DT>
__global__ __launch_bounds__(kBlock) void k_scan(ScanArgs a) {
    extern __shared__ float lds[];
    using T = typename IO::T;
    using TD = typename DT::T;
    const Dims d = a.d;
    const int H = d.H, G = d.G, P = d.P, N = d.N, Q = d.Q;
    const int s = blockIdx.x / H, h = blockIdx.x % H;
    const int g = h / (H / G);
    const int64_t PN = (int64_t)P * N;
    const LdsLayout L(P, N);

    const int64_t t0 = a.cu[s];
    const int len = seq_len(a.cu, a.take, s);
    const int slot = a.replay ? (a.slot_idx ? a.slot_idx[s] : s) : s;
    if (a.replay && (len == 0 || slot < 0 || slot >= a.num_slots))
        return;
    const int nbuf = a.replay ? a.buf_len[slot] : 0;
    if (nbuf < 0 || nbuf >= Q)  // corrupt slot metadata: leave the slot alone
        return;
    // acceptance without a chunk that fills: only the commit kernel's append
    if (a.no_y && nbuf + len < Q)
        return;
    if (a.replay && !buf_pages_ok(a.bm, slot, a.dry ? nbuf : replay_npos(nbuf, len, Q)))
        return;

    const float *init = a.replay ? a.cache_state + ((int64_t)slot * H + h) * PN
                                 : (a.init_state ? a.init_state + ((int64_t)s * H + h) * PN
                                                 : nullptr);
    state_load(lds + L.S, init, P, N);

    ChunkView<IO, DT> v;
    v.x = static_cast<const T *>(a.x);
    v.B = static_cast<const T *>(a.B);
    v.C = static_cast<const T *>(a.C);
    v.dt = static_cast<const TD *>(a.dt);
    v.bx = static_cast<const T *>(a.buf_x);
    v.bB = static_cast<const T *>(a.buf_B);
    v.bdt = static_cast<const TD *>(a.buf_dt);
    v.bm = a.bm; v.slot = slot; v.Q = Q;
    v.h = h; v.g = g; v.H = H; v.G = G; v.P = P; v.N = N;

    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.0f;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const int total = nbuf + len;
    const int nfull = total / Q;
    // without outputs only the chunks that fill are processed
    const int nchunks = a.no_y ? nfull : (total + Q - 1) / Q;
    float *bnd = a.replay ? a.cache_state + ((int64_t)slot * H + h) * PN
                          : (a.boundary_state ? a.boundary_state + ((int64_t)s * H + h) * PN
                                              : nullptr);
    uint16_t *bnd_bf = a.replay ? static_cast<uint16_t *>(a.cache_state_bf) +
                                      ((int64_t)slot * H + h) * PN
                                : nullptr;
    const bool write_bnd = bnd && (!a.replay || nfull > 0) && !a.dry;
    T *y = static_cast<T *>(a.y);
    // chunk-end states of the full chunks (plain prefill)
    float *cst = nullptr;
    if (!a.replay && a.chunk_states)
        cst = a.chunk_states +
              ((int64_t)full_chunks_before(a.cu, s, Q, reinterpret_cast<int *>(lds + L.tot)) * H +
               h) * PN;

    for (int c = 0; c < nchunks; ++c) {
        if (c == nfull && write_bnd)
            state_store(bnd, lds + L.S, P, N, bnd_bf);
        if (cst && c >= 1 && c <= nfull)   // the state after full chunk c - 1
            state_store(cst + (int64_t)(c - 1) * H * PN, lds + L.S, P, N);
        v.nb = (c == 0) ? nbuf : 0;
        v.n_valid = min(Q, total - c * Q);
        v.tok_base = t0 + (int64_t)c * Q + v.nb - nbuf;
        prepare_chunk(v, A_h, bias, d.softplus, lds, L);
        for (int rt = (v.nb / kRows) * kRows; !a.no_y && rt < v.n_valid; rt += kRows)
            emit_rows(v, max(rt, v.nb), min(rt + kRows, v.n_valid), D_h, y, lds, L);
        if (v.n_valid == Q || (!a.replay && a.final_state))
            chunk_state_update(v, lds, L);
    }
    if (cst && nfull == nchunks && nfull > 0)
        state_store(cst + (int64_t)(nfull - 1) * H * PN, lds + L.S, P, N);
    if (nfull == nchunks && write_bnd)
        state_store(bnd, lds + L.S, P, N, bnd_bf);
    if (!a.replay && a.final_state)
        state_store(a.final_state + ((int64_t)s * H + h) * PN, lds + L.S, P, N);
}

// One workgroup per (head, batch row): replay the slot's buffered tokens
// plus the new token, emit the new row, append the token, and commit the
// chunk-end state when the chunk fills.
template <class IO, class DT>
__global__ __launch_bounds__(kBlock) void k_decode(DecodeArgs a) {
    extern __shared__ float lds[];
    using T = typename IO::T;
    using TD = typename DT::T;
    const Dims d = a.d;
    const int H = d.H, G = d.G, P = d.P, N = d.N, Q = d.Q;
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int hpg = H / G, g = h / hpg;
    const int64_t PN = (int64_t)P * N;
    const LdsLayout L(P, N);
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0 || slot >= a.num_slots)
        return;
    const int k = a.buf_len[slot];
    if (k < 0 || k >= Q || !buf_pages_ok(a.bm, slot, k + 1))
        return;
    float *st = a.cache_state + ((int64_t)slot * H + h) * PN;
    state_load(lds + L.S, st, P, N);

    T *bx = static_cast<T *>(a.buf_x);   // buffer arrays (whole pool)
    T *bB = static_cast<T *>(a.buf_B);
    TD *bdt = static_cast<TD *>(a.buf_dt);
    const int64_t rk = buf_row(a.bm, slot, Q, k);   // buffer row of position k

    ChunkView<IO, DT> v;
    v.x = static_cast<const T *>(a.x);
    v.B = static_cast<const T *>(a.B);
    v.C = static_cast<const T *>(a.C);
    v.dt = static_cast<const TD *>(a.dt);
    v.bx = bx; v.bB = bB; v.bdt = bdt;
    v.bm = a.bm; v.slot = slot; v.Q = Q;
    v.h = h; v.g = g; v.H = H; v.G = G; v.P = P; v.N = N;
    v.tok_base = b;
    v.nb = k;
    v.n_valid = k + 1;

    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    prepare_chunk(v, a.A[h], bias, d.softplus, lds, L);
    emit_rows(v, k, k + 1, a.D ? a.D[h] : 0.0f, static_cast<T *>(a.y), lds, L);

    // append the new token at buffer position k (reads above touch only
    // positions < k of the buffer)
    const int tid = threadIdx.x;
    const T *xin = static_cast<const T *>(a.x) + ((int64_t)b * H + h) * P;
    for (int p = tid; p < P; p += kBlock)
        bx[(rk * H + h) * P + p] = xin[p];
    if (tid == 0)
        bdt[rk * H + h] = static_cast<const TD *>(a.dt)[(int64_t)b * H + h];
    if (h % hpg == 0) {
        const T *bin = static_cast<const T *>(a.B) + ((int64_t)b * G + g) * N;
        for (int n = tid; n < N; n += kBlock)
            bB[(rk * G + g) * N + n] = bin[n];
        if (a.buf_C) {
            T *bC = static_cast<T *>(a.buf_C);
            const T *cin = static_cast<const T *>(a.C) + ((int64_t)b * G + g) * N;
            for (int n = tid; n < N; n += kBlock)
                bC[(rk * G + g) * N + n] = cin[n];
        }
    }
    if (k + 1 == Q) {
        chunk_state_update(v, lds, L);
        state_store(st, lds + L.S, P, N,
                    static_cast<uint16_t *>(a.cache_state_bf) + ((int64_t)slot * H + h) * PN);
    }
}

// buf_len / boundary_pos advance after a decode step (separate launch: every
// head's workgroup of a slot reads buf_len first).
// Slots the decode kernel skipped (a missing page) are not advanced.
__global__ void k_decode_advance(int batch, const int32_t *slot_idx, int32_t *buf_len,
                                 int64_t *boundary_pos, int Q, int num_slots, BufMap bm) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch)
        return;
    const int slot = slot_idx ? slot_idx[b] : b;
    if (slot < 0 || slot >= num_slots)
        return;
    const int k = buf_len[slot];
    if (k < 0 || k >= Q || !buf_pages_ok(bm, slot, k + 1))
        return;
    if (k + 1 == Q) {
        buf_len[slot] = 0;
        boundary_pos[slot] += Q;
    } else {
        buf_len[slot] = k + 1;
    }
}

// Trailing partial chunk -> slot buffers; buf_len / boundary_pos update;
// optional boundary-state copy. Workgroup (s, 0) handles sequence s's buffer
// and metadata; workgroup (s, 1 + h) copies head h of its boundary state
// (and writes the bf16 copy) when state_src is given.
// Rows [row0, row0 + ntok) of a token-major array (per elements of type E
// per row) to buffer positions dst0.. of a slot, kCopyBatch elements per
// thread loaded before any is stored (loads of a batch are in flight
// together). Whole workgroup.
constexpr int kCopyBatch = 8;

template <class E, bool PAGED>
__device__ __forceinline__ void copy_rows_batched(const BufMap &bm, int slot, int Q, int dst0,
                                                  E *d, const E *s, int n, int per, int tid) {
    for (int e0 = 0; e0 < n; e0 += kCopyBatch * kBlock) {
        E v[kCopyBatch];
#pragma unroll
        for (int i = 0; i < kCopyBatch; ++i) {
            const int e = e0 + tid + i * kBlock;
            v[i] = s[e < n ? e : n - 1];
        }
#pragma unroll
        for (int i = 0; i < kCopyBatch; ++i) {
            const int e = e0 + tid + i * kBlock;
            const int j = dst0 + (e < n ? e : n - 1) / per;
            const int64_t row = PAGED ? ((int64_t)bm.pages[(int64_t)slot * bm.npp + (j >> bm.shift)]
                                         << bm.shift) + (j & ((1 << bm.shift) - 1))
                                      : (int64_t)slot * Q + j;
            if (e < n)
                d[row * per + e % per] = v[i];
        }
    }
}

template <class E>
__device__ __forceinline__ void copy_to_buffer(const BufMap &bm, int slot, int Q, int dst0,
                                               void *dst, const void *src, int64_t row0,
                                               int ntok, int per, int tid) {
    // (32-bit element indices: at most Q rows of at most H*P elements)
    const E *s = static_cast<const E *>(src) + row0 * per;
    E *d = static_cast<E *>(dst);
    const int n = ntok * per;
    if (bm.pages)
        copy_rows_batched<E, true>(bm, slot, Q, dst0, d, s, n, per, tid);
    else
        copy_rows_batched<E, false>(bm, slot, Q, dst0, d, s, n, per, tid);
}

template <class IO, class DT>
__global__ __launch_bounds__(kBlock) void k_commit(CommitArgs a) {
    using T = typename IO::T;
    using TD = typename DT::T;
    const Dims d = a.d;
    const int s = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
    const int H = d.H, G = d.G, P = d.P, N = d.N, Q = d.Q;
    const int slot = a.slot_idx ? a.slot_idx[s] : s;
    const int64_t t0 = a.cu[s];
    const int len = seq_len(a.cu, a.take, s);
    if ((!a.fresh && len == 0) || slot < 0 || slot >= a.num_slots)
        return;
    if (part > 0) {
        // (state_src comes with fresh slots only: buf_len is not read here,
        // workgroup (s, 0) writes it)
        if (!a.state_src || !buf_pages_ok(a.bm, slot, replay_npos(0, len, Q)))
            return;
        const int h = part - 1;
        const int64_t PN = (int64_t)P * N;
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 *src =
            reinterpret_cast<const f32x4 *>(a.state_src + ((int64_t)s * H + h) * PN);
        f32x4 *dst = reinterpret_cast<f32x4 *>(a.cache_state + ((int64_t)slot * H + h) * PN);
        uint16_t *dbf = static_cast<uint16_t *>(a.cache_state_bf) + ((int64_t)slot * H + h) * PN;
        const int n4 = (int)(PN / 4);
        // kCopyBatch pieces per thread loaded before any is stored
        for (int e0 = 0; e0 < n4; e0 += kCopyBatch * kBlock) {
            f32x4 v[kCopyBatch];
#pragma unroll
            for (int i = 0; i < kCopyBatch; ++i) {
                const int e = e0 + tid + i * kBlock;
                v[i] = src[e < n4 ? e : n4 - 1];
            }
#pragma unroll
            for (int i = 0; i < kCopyBatch; ++i) {
                const int e = e0 + tid + i * kBlock;
                if (e < n4) {
                    dst[e] = v[i];
                    const int p = 4 * e / N, n = 4 * e % N;
                    *reinterpret_cast<uint2 *>(dbf + state_bf_index(p, n, P)) = make_uint2(
                        bf16_rne(v[i].x) | ((uint32_t)bf16_rne(v[i].y) << 16),
                        bf16_rne(v[i].z) | ((uint32_t)bf16_rne(v[i].w) << 16));
                }
            }
        }
        return;
    }
    const int nbuf = a.fresh ? 0 : a.buf_len[slot];
    if (nbuf < 0 || nbuf >= Q || !buf_pages_ok(a.bm, slot, replay_npos(nbuf, len, Q)))
        return;
    const int total = nbuf + len;
    const int nfull = total / Q, tail = total % Q;
    // new tokens [src0, len) go to buffer positions dst0..
    const int src0 = nfull == 0 ? 0 : len - tail;
    const int dst0 = nfull == 0 ? nbuf : 0;
    const int ntok = len - src0;

    const T *x = static_cast<const T *>(a.x);
    const T *B = static_cast<const T *>(a.B);
    const T *C = static_cast<const T *>(a.C);
    const TD *dt = static_cast<const TD *>(a.dt);
    const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N;
    // token rows in 16-byte pieces (a row of x or B is a multiple of 32
    // bytes), each to the buffer row of its position
    const int64_t src_row0 = t0 + src0;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    copy_to_buffer<u32x4>(a.bm, slot, Q, dst0, a.buf_x, x, src_row0, ntok,
                          (int)(HP * (int64_t)sizeof(T) / 16), tid);
    copy_to_buffer<u32x4>(a.bm, slot, Q, dst0, a.buf_B, B, src_row0, ntok,
                          (int)(GN * (int64_t)sizeof(T) / 16), tid);
    if (a.buf_C)
        copy_to_buffer<u32x4>(a.bm, slot, Q, dst0, a.buf_C, C, src_row0, ntok,
                              (int)(GN * (int64_t)sizeof(T) / 16), tid);
    copy_to_buffer<TD>(a.bm, slot, Q, dst0, a.buf_dt, dt, src_row0, ntok, H, tid);
    __syncthreads();
    if (tid == 0) {
        a.buf_len[slot] = nfull == 0 ? total : tail;
        a.boundary_pos[slot] = (a.fresh ? 0 : a.boundary_pos[slot]) + (int64_t)nfull * Q;
    }
}

// bf16 copy of the whole cache state (one workgroup per slot and head).
__global__ __launch_bounds__(kBlock) void k_refresh_state_bf(const float *state, uint16_t *state_bf,
                                                             int P, int N) {
    const int64_t PN = (int64_t)P * N;
    const float4 *src = reinterpret_cast<const float4 *>(state + blockIdx.x * PN);
    uint16_t *dst = state_bf + blockIdx.x * PN;
    for (int64_t e = threadIdx.x; e < PN / 4; e += kBlock) {
        const float4 v = src[e];
        const int p = (int)((4 * e) / N), n = (int)((4 * e) % N);
        *reinterpret_cast<uint2 *>(dst + state_bf_index(p, n, P)) =
            make_uint2(bf16_rne(v.x) | ((uint32_t)bf16_rne(v.y) << 16),
                       bf16_rne(v.z) | ((uint32_t)bf16_rne(v.w) << 16));
    }
}

// ---- recurrent update ------------------------------------------------------
//
// Layout: a state row spans L = N / 16 consecutive lanes; lane c of the row
// owns the 16 columns 4(c + L k) + e (k, e < 4): four pieces of 4 columns,
// so the row's lanes read consecutive pieces (coalesced). A workgroup
// covers 256 / L rows per pass and a thread holds NR rows (a template
// parameter). The row's output is the thread's 16 products in order, then a
// lane tree over the L lanes. The one-token and the multi-token kernels
// share this layout and every line of arithmetic (ssu_seg, ssu_row_out), so
// their bits agree.

// 4 consecutive values of an array of storage type IO.
template <class IO>
struct Piece4;
template <>
struct Piece4<IoBF16> {
    uint2 u;
    __device__ __forceinline__ void load(const uint16_t *p) { u = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ void get(float *f) const {
        f[0] = __uint_as_float(u.x << 16);
        f[1] = __uint_as_float(u.x & 0xffff0000u);
        f[2] = __uint_as_float(u.y << 16);
        f[3] = __uint_as_float(u.y & 0xffff0000u);
    }
};
template <>
struct Piece4<IoF32> {
    uint4 u;
    __device__ __forceinline__ void load(const float *p) { u = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void get(float *f) const {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
};

// A lane's 16 values of a row: pieces at element offsets 4 L k from p
// (p = the row's column 4c).
template <class IO>
struct Seg16 {
    Piece4<IO> pc[4];
    __device__ __forceinline__ void load(const typename IO::T *p, int L) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            pc[k].load(p + 4 * L * k);
    }
    __device__ __forceinline__ void get(float (&f)[16]) const {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            pc[k].get(f + 4 * k);
    }
};

// State storage: fp32, or bf16 (rounded to nearest even on every store,
// the cache-dtype rounding of each token).
struct StF32 {
    using T = float;
    using IO = IoF32;
    __device__ static __forceinline__ void store16(T *p, int L, const float (&v)[16]) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<float4 *>(p + 4 * L * k) =
                make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    }
    // the value the store keeps (fp32: the value itself)
    __device__ static __forceinline__ float round(float v) { return v; }
};

struct StBF16 {
    using T = uint16_t;
    using IO = IoBF16;
    __device__ static __forceinline__ void store16(T *p, int L, const float (&v)[16]) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<uint2 *>(p + 4 * L * k) =
                make_uint2(bf16_rne(v[4 * k]) | ((uint32_t)bf16_rne(v[4 * k + 1]) << 16),
                           bf16_rne(v[4 * k + 2]) | ((uint32_t)bf16_rne(v[4 * k + 3]) << 16));
    }
    __device__ static __forceinline__ float round(float v) {
        return __uint_as_float((uint32_t)bf16_rne(v) << 16);
    }
};

// One token on one row segment: s = alpha s + (delta x_p) B_n, then the
// segment's share of y_p = sum_n s C_n (products in column order).
__device__ __forceinline__ float ssu_seg(float (&sv)[16], float alpha, float dx,
                                         const float (&bv)[16], const float (&cv)[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
        sv[j] = fmaf(alpha, sv[j], dx * bv[j]);
    float part = sv[0] * cv[0];
#pragma unroll
    for (int j = 1; j < 16; ++j)
        part = fmaf(sv[j], cv[j], part);
    return part;
}

// Row sum over the L = N/16 lanes of a row (L in {1, 2, 4, 8}, consecutive
// and aligned), then y_p; complete in the row's last lane. A fixed DPP
// tree, no LDS traffic: lane pairs 1 apart, 2 apart (quad permutes), then
// the two quads of each 8-lane half row (half mirror). The lanes of a row
// are active or inactive together.
__device__ __forceinline__ float ssu_row_out(float part, int L, float D_h, float xv) {
    if (L >= 2)
        part = part + dpp_from<0xb1, 0xf>(part);      // quad_perm [1,0,3,2]
    if (L >= 4)
        part = part + dpp_from<0x4e, 0xf>(part);      // quad_perm [2,3,0,1]
    if (L >= 8)
        part = part + dpp_from<0x141, 0xf>(part);     // row_half_mirror
    return fmaf(D_h, xv, part) + 0.0f;   // -0 -> +0
}

// Recurrent update, one workgroup per (head, batch row): the state is read,
// updated in fp32 and stored in its cache dtype.
template <class IO, class DT, class ST, int NR>
__global__ __launch_bounds__(kBlock) void k_ssu(SsuArgs a) {
    using T = typename IO::T;
    using TD = typename DT::T;
    const Dims d = a.d;
    const int H = d.H, G = d.G, P = d.P, N = d.N;
    const int b = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x;
    const int g = h / (H / G);
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0 || slot >= a.num_slots)
        return;
    const int L = N / 16, c = tid % L, rr = tid / L, RP = kBlock / L;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float dl = delta_of(DT::ld(static_cast<const TD *>(a.dt), (int64_t)b * H + h), bias,
                              d.softplus);
    const float alpha = decay_exp(dl * a.A[h]);
    const float D_h = a.D ? a.D[h] : 0.0f;
    Seg16<IO> bs, cs;
    bs.load(static_cast<const T *>(a.B) + ((int64_t)b * G + g) * N + 4 * c, L);
    cs.load(static_cast<const T *>(a.C) + ((int64_t)b * G + g) * N + 4 * c, L);
    float bv[16], cv[16];
    bs.get(bv);
    cs.get(cv);
    const T *xt = static_cast<const T *>(a.x) + ((int64_t)b * H + h) * P;
    typename ST::T *st = static_cast<typename ST::T *>(a.state) + ((int64_t)slot * H + h) * P * N;
    T *y = static_cast<T *>(a.y) + ((int64_t)b * H + h) * P;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int p = rr + RP * i;
        if (p < P) {   // uniform over the L lanes of a row
            typename ST::T *row = st + (int64_t)p * N + 4 * c;
            Seg16<typename ST::IO> ss;
            ss.load(row, L);
            float sv[16];
            ss.get(sv);
            const float xv = IO::ld(xt, p);
            const float part = ssu_seg(sv, alpha, dl * xv, bv, cv);
            ST::store16(row, L, sv);
            const float yv = ssu_row_out(part, L, D_h, xv);
            if (c == L - 1)
                y[p] = IO::cvt(yv);
        }
    }
}

// Multi-token recurrent update over a varlen pack (packed-history recovery:
// vLLM RFC "Mamba2: exact-replay decode ...", section 3b, replays generated
// history with a multi-token update that rounds the state to the cache
// dtype after every token). One workgroup per (sequence, head); the state
// stays in registers across the sequence's tokens, rounded to the cache
// dtype after each one exactly as a store and reload would, so the result
// is bit-identical to one k_ssu launch per token. Outputs for every token.
template <class IO, class DT, class ST, int NR>
__global__ __launch_bounds__(kBlock) void k_ssu_varlen(SsuArgs a) {
    using T = typename IO::T;
    using TD = typename DT::T;
    const Dims d = a.d;
    const int H = d.H, G = d.G, P = d.P, N = d.N;
    const int s = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x;
    const int g = h / (H / G);
    const int slot = a.slot_idx ? a.slot_idx[s] : s;
    const int64_t t0 = a.cu[s];
    const int len = a.cu[s + 1] - a.cu[s];
    if (slot < 0 || slot >= a.num_slots || len == 0)
        return;
    const int L = N / 16, c = tid % L, rr = tid / L, RP = kBlock / L;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float A_h = a.A[h];
    const float D_h = a.D ? a.D[h] : 0.0f;
    typename ST::T *st = static_cast<typename ST::T *>(a.state) + ((int64_t)slot * H + h) * P * N;
    float sr[NR][16];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int p = min(rr + RP * i, P - 1);   // rows past P are never stored
        Seg16<typename ST::IO> ss;
        ss.load(st + (int64_t)p * N + 4 * c, L);
        ss.get(sr[i]);
    }
    const T *xs = static_cast<const T *>(a.x);
    const TD *dts = static_cast<const TD *>(a.dt);
    const T *Bs = static_cast<const T *>(a.B);
    const T *Cs = static_cast<const T *>(a.C);
    T *ys = static_cast<T *>(a.y);
    // one token's inputs as stored (converted where used), loaded one token
    // ahead so that their latency overlaps the current token's arithmetic
    struct TokIn {
        Seg16<IO> b, c;
        T x[NR];
    };
    auto load_tok = [&](int64_t tok, TokIn &in) {
        in.b.load(Bs + (tok * G + g) * N + 4 * c, L);
        in.c.load(Cs + (tok * G + g) * N + 4 * c, L);
#pragma unroll
        for (int i = 0; i < NR; ++i)
            in.x[i] = xs[(tok * H + h) * P + min(rr + RP * i, P - 1)];
    };
    // delta and decay depend on the token and head only: the workgroup
    // computes them for kBlock tokens at a time, one token per thread (the
    // same routines, so the same values as the one-token kernel), into LDS
    __shared__ float s_dl[kBlock], s_al[kBlock];
    TokIn nxt;
    load_tok(t0, nxt);
    for (int t = 0; t < len; ++t) {
        const int64_t tok = t0 + t;
        if (t % kBlock == 0) {
            __syncthreads();   // the previous tokens' reads are done
            if (t + tid < len) {
                const float v = delta_of(DT::val(dts[(tok + tid) * H + h]), bias, d.softplus);
                s_dl[tid] = v;
                s_al[tid] = decay_exp(v * A_h);
            }
            __syncthreads();
        }
        const TokIn cur = nxt;
        const float dl = s_dl[t % kBlock], alpha = s_al[t % kBlock];
        if (t + 1 < len)
            load_tok(tok + 1, nxt);
        float bv[16], cv[16];
        cur.b.get(bv);
        cur.c.get(cv);
        T *y = ys + (tok * H + h) * P;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int p = rr + RP * i;
            if (p < P) {   // uniform over the L lanes of a row
                const float xv = IO::val(cur.x[i]);
                const float part = ssu_seg(sr[i], alpha, dl * xv, bv, cv);
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    sr[i][j] = ST::round(sr[i][j]);
                const float yv = ssu_row_out(part, L, D_h, xv);
                if (c == L - 1)
                    y[p] = IO::cvt(yv);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int p = rr + RP * i;
        if (p < P)
            ST::store16(st + (int64_t)p * N + 4 * c, L, sr[i]);
    }
}

// Rows per thread: P * (N/16) / 256, at least 1 (at most 8: P, N <= 128).
template <class IO, class DT, class ST>
void launch_ssu_kernels(const SsuArgs &a, hipStream_t stream) {
    const dim3 grid(a.d.H * a.batch), block(kBlock);
    const int nr = std::max(1, a.d.P * (a.d.N / 16) / kBlock);
#define SSU_CASE(R)                                                   \
    case R:                                                           \
        if (a.cu)                                                     \
            k_ssu_varlen<IO, DT, ST, R><<<grid, block, 0, stream>>>(a); \
        else                                                          \
            k_ssu<IO, DT, ST, R><<<grid, block, 0, stream>>>(a);        \
        break;
    switch (nr) {
        SSU_CASE(1)
        SSU_CASE(2)
        SSU_CASE(4)
    default:
        SSU_CASE(8)
    }
#undef SSU_CASE
}

template <class K>
hipError_t prep_lds(K kernel, size_t bytes) {
    if (bytes > 64 * 1024)
        return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    return hipSuccess;
}

template <class IO, class DT>
hipError_t scan_impl(const ScanArgs &a, hipStream_t stream) {
    const LdsLayout L(a.d.P, a.d.N);
    const size_t bytes = sizeof(float) * L.total;
    hipError_t e = prep_lds(k_scan<IO, DT>, bytes);
    if (e != hipSuccess)
        return e;
    k_scan<IO, DT><<<dim3(a.d.H * a.S), dim3(kBlock), bytes, stream>>>(a);
    return hipGetLastError();
}

template <class IO, class DT>
hipError_t decode_impl(const DecodeArgs &a, hipStream_t stream) {
    const LdsLayout L(a.d.P, a.d.N);
    const size_t bytes = sizeof(float) * L.total;
    hipError_t e = prep_lds(k_decode<IO, DT>, bytes);
    if (e != hipSuccess)
        return e;
    k_decode<IO, DT><<<dim3(a.d.H * a.batch), dim3(kBlock), bytes, stream>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_decode_advance(a, stream);
}

template <class IO, class DT>
hipError_t commit_impl(const CommitArgs &a, hipStream_t stream) {
    k_commit<IO, DT><<<dim3(a.S, a.state_src ? 1 + a.d.H : 1), dim3(kBlock), 0, stream>>>(a);
    return hipGetLastError();
}

template <class IO, class DT>
hipError_t ssu_impl(const SsuArgs &a, hipStream_t stream) {
    // batch rows (one token each), or sequences of a varlen pack (cu given)
    if (a.state_bf16)
        launch_ssu_kernels<IO, DT, StBF16>(a, stream);
    else
        launch_ssu_kernels<IO, DT, StF32>(a, stream);
    return hipGetLastError();
}

template <template <class, class> class F, class Args>
hipError_t dispatch(const Args &a, hipStream_t stream) {
    if (a.d.io_bf16)
        return a.d.dt_bf16 ? F<IoBF16, IoBF16>::run(a, stream) : F<IoBF16, IoF32>::run(a, stream);
    return a.d.dt_bf16 ? F<IoF32, IoBF16>::run(a, stream) : F<IoF32, IoF32>::run(a, stream);
}

template <class IO, class DT> struct ScanF { static hipError_t run(const ScanArgs &a, hipStream_t s) { return scan_impl<IO, DT>(a, s); } };
template <class IO, class DT> struct DecodeF { static hipError_t run(const DecodeArgs &a, hipStream_t s) { return decode_impl<IO, DT>(a, s); } };
template <class IO, class DT> struct CommitF { static hipError_t run(const CommitArgs &a, hipStream_t s) { return commit_impl<IO, DT>(a, s); } };
template <class IO, class DT> struct SsuF { static hipError_t run(const SsuArgs &a, hipStream_t s) { return ssu_impl<IO, DT>(a, s); } };

}  // namespace

hipError_t launch_scan(const ScanArgs &a, hipStream_t stream) { return dispatch<ScanF>(a, stream); }
hipError_t launch_decode_advance(const DecodeArgs &a, hipStream_t stream) {
    k_decode_advance<<<dim3((a.batch + 255) / 256), dim3(256), 0, stream>>>(
        a.batch, a.slot_idx, a.buf_len, a.boundary_pos, a.d.Q, a.num_slots, a.bm);
    return hipGetLastError();
}
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) { return dispatch<DecodeF>(a, stream); }
hipError_t launch_commit(const CommitArgs &a, hipStream_t stream) { return dispatch<CommitF>(a, stream); }
hipError_t launch_ssu(const SsuArgs &a, hipStream_t stream) { return dispatch<SsuF>(a, stream); }
hipError_t copy_to_host(void *dst, const void *src, size_t bytes) {
    return hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
}
hipError_t launch_refresh_state_bf(const float *state, void *state_bf, int64_t heads, int P, int N,
                                   hipStream_t stream) {
    if (heads <= 0)
        return hipSuccess;
    k_refresh_state_bf<<<dim3((unsigned)heads), dim3(kBlock), 0, stream>>>(
        state, static_cast<uint16_t *>(state_bf), P, N);
    return hipGetLastError();
}

}  // namespace ssd
