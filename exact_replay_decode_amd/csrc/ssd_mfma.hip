// ssd_mfma.hip -- the chunked scan and exact-replay decode on gfx950 matrix
// cores (bf16 inputs, fp32 accumulation, fp32 state).
//
// Per chunk of Q tokens (ReplaySSM reproduction page, "Core equations"; the
// vLLM RFC "Mamba2: exact-replay decode ...", section 3, replays the same
// chunk arithmetic for decode), for one head with state S (P x N):
//   G^T[s][t]  = B_s . C_t                                  (MFMA, K = N)
//   M[t][s]    = bf16( G[t][s] exp(lam_t - lam_s) delta_s ),  s <= t, else 0
//                evaluated as G 2^(l_t - u_s), l = lam log2(e) and
//                u_s = l_s - log2(delta_s), both precomputed per token; off the
//                diagonal block as (G 2^(l_t - c)) 2^(c - u_s), c = l at the end
//                of the 32-token block of s (both factors <= 1, no overflow)
//   Y^T[p][t]  = exp(lam_t) (S_bf . C_t)[p] + (X^T M^T)[p][t] (MFMA, K = N, s)
//   y[t][p]    = fmaf(D, x[t][p], Y^T[p][t])
//   S^T[n][p]  = exp(lam_last) S^T[n][p] + sum_s B_s[n] (w_s x_s[p]),
//                w_s = exp(lam_last - lam_s) delta_s: the decayed state is the
//                MFMA accumulator the chunk's inputs are added into
//                (16x16x32 MFMA tiles, K = s ascending in steps of 32; w x
//                split into bf16 hi + lo)
// S_bf is S rounded to bf16 for the read-out contraction; C.B^T operands are
// exact bf16; the state path keeps about 16 mantissa bits through the hi/lo
// split and is never rounded between chunks.
//
// Bit identity between prefill and decode: a 32-row block of chunk rows
// ("t-block") is always computed by tblock_part() with the same MFMA
// shapes and the same K order; decode calls it for the t-block holding the
// new token with the rows after it zero-filled. Each output element of an
// MFMA depends only on its own row and column operands, masked weights are
// selected to +0 (never multiplied), so the rows after the new token cannot
// change it. The chunk-end state is computed tile by tile with
// state_kstep() in both paths.
//
// LDS tiles are row-major with 16 bytes of padding per row; operands that
// contract over tokens are fetched transposed with ds_read_b64_tr_b16.
#include <algorithm>

#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kPad = 8;  // bf16 elements of padding per LDS row

__device__ __forceinline__ uint16_t bf16_bits(float f) { return bf16_rne(f); }
__device__ __forceinline__ float bf16_float(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
__device__ __forceinline__ float fexp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float flog2(float v) { return __builtin_amdgcn_logf(v); }

// two floats -> packed bf16 pair (round to nearest even), low half = a
__device__ __forceinline__ uint32_t bf16_pack(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS layout, in bytes, for a chunk of Qp rows (Qp = max(Q, 32)).
struct MLayout {
    int XS, BS, SS;                 // row strides in bf16 elements
    int X, B, S, sbb, lam, u, el, w, beta, scb, tot, bytes;
    __host__ __device__ MLayout(int Qp, int P, int N) {
        XS = P + kPad;
        BS = N + kPad;
        SS = N + kPad;
        int o = 0;
        X = o;   o += Qp * XS * 2;
        B = o;   o += Qp * BS * 2;
        S = o;   o += P * SS * 2;
        sbb = o - S;               // a second S_bf follows (the prefill alternates)
        o += sbb;
        lam = o; o += kMaxQ * 4;   // in-chunk cumulative sum, log2 units
        u = o;   o += kMaxQ * 4;   // lam - log2(delta)
        el = o;  o += kMaxQ * 4;
        w = o;   o += kMaxQ * 4;
        beta = o; o += kMaxQ * 4;  // 2^(c - u_s), c = l at the end of s's 32-block
        scb = o - lam;             // a second set of the five per-row arrays follows
        o += scb;
        tot = o; o += 64;     // one float per wave
        bytes = o;
    }
    // the layout of one prefill chunk: per-row arrays and S_bf of set b (the
    // prefill computes the next chunk's set while this chunk reads its own),
    // x and B tile rows from row r0 on
    __host__ __device__ MLayout chunk(int b, int r0) const {
        MLayout r = buf(b);
        r.S += b * sbb;
        r.X += r0 * XS * 2;
        r.B += r0 * BS * 2;
        return r;
    }
    // the layout whose per-row arrays are set b (0 or 1)
    __host__ __device__ MLayout buf(int b) const {
        MLayout r = *this;
        const int d = b * scb;
        r.lam += d;
        r.u += d;
        r.el += d;
        r.w += d;
        r.beta += d;
        return r;
    }
};

// The lane index, produced afresh at each use: the compiler can neither
// hoist nor merge it, so lane-derived addresses are recomputed where they are
// used instead of being kept live (or spilled) across the chunk loops.
__device__ __forceinline__ int lane_id() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

__device__ __forceinline__ bf16x8 lds_b128(const char *lds, int byte_off) {
    return *reinterpret_cast<const bf16x8 *>(lds + byte_off);
}

// Transposed fetch of an MFMA operand from a row-major bf16 tile (row
// stride `stride` elements): each 16-lane group reads a 4-row x 16-column
// block, lane l of the group supplying row l / 4, columns 4 (l % 4) .. +3,
// and receives rows 0..3 of one column. tr_lane is that per-lane byte
// offset; lds_tr8 fetches the blocks at byte addresses a and a + d (plus
// the lane offset `la`, which may include further per-lane terms), giving
// the lane 8 k-values of its column. Returned as raw bf16 bit patterns.
__device__ __forceinline__ int tr_lane(int lane, int stride) {
    const int l = lane & 15;
    return ((l >> 2) * stride + 4 * (l & 3)) * 2;
}

__device__ __forceinline__ i16x8 lds_tr8(const char *lds, int la, int a, int d) {
    const lds_char *p = (const lds_char *)lds + la;
    i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + a));
    i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + a + d));
    i16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const i16x8 &v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------
// The pieces of a t-block's output arithmetic. Prefill and decode build the
// same operands and call these in the same order, so each output element is
// produced by the same MFMA sequence in both.

// C . S_bf for one 32-wide p-tile: K = n ascending in steps of 16 (then
// readout_scale multiplies column t by exp(lam_t)). sa(k) returns the A
// operand S_bf[p][16k + 8g .. +7].
template <int N, class F>
__device__ __forceinline__ f32x16 readout_raw(F sa, const bf16x8 *cf) {
    f32x16 a = {};
#pragma unroll
    for (int k = 0; k < N / 16; ++k)
        a = mfma(sa(k), cf[k], a);
    return a;
}

__device__ __forceinline__ f32x16 readout_scale(f32x16 a, float el_t) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
        a[r] = a[r] * el_t;
    return a;
}

// G^T for one 32-row s-block: K = n ascending. ba(k) returns the A operand
// B[s][16k + 8g .. +7] for s = 32 sg + lane % 32.
template <int N, class F>
__device__ __forceinline__ f32x16 gram_block(F ba, const bf16x8 *cf) {
    f32x16 gt = {};
#pragma unroll
    for (int k = 0; k < N / 16; ++k)
        gt = mfma(ba(k), cf[k], gt);
    return gt;
}

// A lane's per-row values of one s-block: v[q] = a[s_base + 8q + 4g .. +3]
// (g = lane / 32), the rows s of its accumulator elements gt[4q .. 4q + 3].
__device__ __forceinline__ void srows(const float *a, int s_base, float4 (&v)[4], int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        v[q] = *reinterpret_cast<const float4 *>(a + s_base + 8 * q + 4 * g);
}

// Weights of the diagonal s-block, packed to bf16 pairs: gt[4q + e] =
// G[t][s] for s = s_base + 8q + 4g + e; m = G 2^(l_t - u_s) for s <= t and +0
// otherwise (selected, never multiplied). u4: the rows' u (srows).
__device__ __forceinline__ void m_diag_rows(const f32x16 &gt, float lam_t, const float4 (&u4)[4],
                                            int s_base, int t, uint32_t (&mb)[8], int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int s0 = s_base + 8 * q + 4 * g;
        const float us[4] = {u4[q].x, u4[q].y, u4[q].z, u4[q].w};
        float m[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[e] = gt[4 * q + e] * fexp2(lam_t - us[e]);
            m[e] = (s0 + e <= t) ? m[e] : 0.0f;
        }
        mb[2 * q] = bf16_pack(m[0], m[1]);
        mb[2 * q + 1] = bf16_pack(m[2], m[3]);
    }
}

__device__ __forceinline__ void m_diag(const f32x16 &gt, float lam_t, const float *uu, int s_base,
                                       int t, uint32_t (&mb)[8], int lane) {
    float4 u4[4];
    srows(uu, s_base, u4, lane);
    m_diag_rows(gt, lam_t, u4, s_base, t, mb, lane);
}

// Weights of an earlier s-block: (G alpha) beta_s with alpha = 2^(l_t - c)
// and beta_s = 2^(c - u_s), c = l at the end of the s-block. b4: the rows'
// beta (srows).
__device__ __forceinline__ void m_off_rows(const f32x16 &gt, float alpha, const float4 (&b4)[4],
                                           uint32_t (&mb)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        mb[2 * q] = bf16_pack((gt[4 * q] * alpha) * b4[q].x, (gt[4 * q + 1] * alpha) * b4[q].y);
        mb[2 * q + 1] =
            bf16_pack((gt[4 * q + 2] * alpha) * b4[q].z, (gt[4 * q + 3] * alpha) * b4[q].w);
    }
}

__device__ __forceinline__ void m_off(const f32x16 &gt, float alpha, const float *bt, int s_base,
                                      uint32_t (&mb)[8], int lane) {
    float4 b4[4];
    srows(bt, s_base, b4, lane);
    m_off_rows(gt, alpha, b4, mb);
}

// Y^T[p][t] += sum_s X^T[p][s] M^T[s][t] over one s-block, K = 16 rows per
// MFMA: rows r0 = 16 half + 4g .. +3 and r0 + 8 .. +11 of the block, read
// transposed from the row-major LDS tile (xbase, row stride xs, block row 0
// at xrow0); mb[4 half .. 4 half + 3] holds the matching M^T rows. mx_load
// fetches the X^T operands (xo[half][pt - PT0]) so that a caller can issue
// them ahead of the weights; mx_apply runs the MFMAs, half by half.
template <int PT0, int PT1>
__device__ __forceinline__ void mx_load(const char *lds, int xbase, int xs, int xrow0,
                                        bf16x8 (&xo)[2][PT1 - PT0], int lane) {
    const int g = lane >> 5;
    // lane terms: the k-group's rows 4g.., the 16-column half of the p-tile
    const int la = tr_lane(lane, xs) + (4 * g * xs + 16 * ((lane >> 4) & 1)) * 2;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int pt = PT0; pt < PT1; ++pt) {
            const int a = xbase + ((xrow0 + 16 * half) * xs + 32 * pt) * 2;
            xo[half][pt - PT0] = as_bf16x8(lds_tr8(lds, la, a, 8 * xs * 2));
        }
}

template <int PT0, int PT1>
__device__ __forceinline__ void mx_apply(const uint32_t (&mb)[8], const bf16x8 (&xo)[2][PT1 - PT0],
                                         f32x16 *acc) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 bv = {mb[4 * half], mb[4 * half + 1], mb[4 * half + 2], mb[4 * half + 3]};
        const bf16x8 bop = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
        for (int pt = PT0; pt < PT1; ++pt)
            acc[pt] = mfma(xo[half][pt - PT0], bop, acc[pt]);
    }
}

template <int PT0, int PT1>
__device__ __forceinline__ void mx_accumulate(const uint32_t (&mb)[8], const char *lds, int xbase,
                                              int xs, int xrow0, f32x16 *acc, int lane) {
    bf16x8 xo[2][PT1 - PT0];
    mx_load<PT0, PT1>(lds, xbase, xs, xrow0, xo, lane);
    mx_apply<PT0, PT1>(mb, xo, acc);
}

// Output of one 32-row t-block in prefill: p-tiles [PT0, PT1) of Y^T for
// chunk rows t = 32 tau + (lane % 32). cf[k] holds C[t][16k + 8g .. +7]
// (g = lane/32) for output rows (other rows' columns are not used). acc[pt] receives
// Y^T[p][t] (without the D x term) for p = 32 pt + 8 (r/4) + 4 g + r % 4.
// tblock_part takes the s-blocks [sg0, sg1] (sg1 <= tau) after the read-out
// when sg0 == 0 (which initialises acc): the prefill runs a t-block's
// s-blocks in two parts around its half-chunk barrier, accumulating in the
// same order.
template <int P, int N, int PT0, int PT1>
__device__ __forceinline__ void tblock_part(int tau, int sg0, int sg1, const bf16x8 *cf,
                                            const char *lds, const MLayout &L, f32x16 *acc) {
    const int lane = lane_id();
    const int g = lane >> 5, c = lane & 31;
    const float *lam = reinterpret_cast<const float *>(lds + L.lam);
    const float *uu = reinterpret_cast<const float *>(lds + L.u);
    const float *bt = reinterpret_cast<const float *>(lds + L.beta);
    const float *el = reinterpret_cast<const float *>(lds + L.el);
    const int t = 32 * tau + c;

    if (sg0 == 0) {
        // read-out (each chain K-ascending, as readout_raw); the operands of
        // one K step are loaded at a time, so they do not all stay live
#pragma unroll
        for (int pt = PT0; pt < PT1; ++pt)
            acc[pt] = f32x16{};
#pragma unroll
        for (int k = 0; k < N / 16; ++k) {
#pragma unroll
            for (int pt = PT0; pt < PT1; ++pt)
                acc[pt] = mfma(lds_b128(lds, L.S + ((32 * pt + c) * L.SS + 16 * k + 8 * g) * 2),
                               cf[k], acc[pt]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int pt = PT0; pt < PT1; ++pt)
            acc[pt] = readout_scale(acc[pt], el[t]);
    }

    const float lam_t = lam[t];
    // per s-block: all eight B operands of C.B^T are fetched before its
    // first MFMA (one LDS round trip instead of eight), and the per-row
    // values of the weights and the X^T operands of M.X while its MFMAs run
    for (int sg = sg0; sg <= sg1; ++sg) {
        bf16x8 bo[N / 16];
#pragma unroll
        for (int k = 0; k < N / 16; ++k)
            bo[k] = lds_b128(lds, L.B + ((32 * sg + c) * L.BS + 16 * k + 8 * g) * 2);
        __builtin_amdgcn_sched_barrier(0);
        const f32x16 gt = gram_block<N>([&](int k) { return bo[k]; }, cf);
        float4 rv[4];
        srows(sg == tau ? uu : bt, 32 * sg, rv, lane);
        const float c_end = lam[32 * sg + 31];
        bf16x8 xo[2][PT1 - PT0];
        mx_load<PT0, PT1>(lds, L.X, L.XS, 32 * sg, xo, lane);
        uint32_t mb[8];
        if (sg == tau)
            m_diag_rows(gt, lam_t, rv, 32 * sg, t, mb, lane);
        else
            m_off_rows(gt, fexp2(lam_t - c_end), rv, mb);
        mx_apply<PT0, PT1>(mb, xo, acc);
    }
}

// ---------------------------------------------------------------------------
// The chunk-state update. The state S (P x N, fp32) is held as 16 x 16 tiles
// of S^T (rows n, columns p) in the accumulator layout of the 16x16x32 MFMA:
// lane l holds p = 16 ps + l % 16 and n = 16 nt + 4 (l / 16) + r, r = 0..3
// (ps: the tile's 16-row p-slab, nt: its n-tile). Each tile is first
// multiplied by exp(lam_last), then takes, per K = 32 step of chunk rows
// (steps ascending), S^T += B^T (w x) with the token operand w x split into
// bf16 hi + lo, hi first. A tile's arithmetic does not depend on which wave
// computes it or next to which other tile: the prefill's four state waves
// take one p-slab each (so every element of w x is split once), the decode
// walks its head's slabs one after another.

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kStateWaves = 4;

// The prefill's state waves sw = 0..3: wave sw owns p-slab sw % (P / 16) and
// NT n-tiles from nt0 (with P = 32 each of the two slabs is shared by two
// waves, one n-half each).
template <int P, int N>
struct Slab {
    static constexpr int NPS = P / 16;
    static constexpr int NPART = kStateWaves / NPS;
    static constexpr int NT = (N / 16) / NPART;
    static_assert(NPS * NPART == kStateWaves && NT >= 1, "state tiles per wave");
    __device__ static __forceinline__ void own(int sw, int &ps, int &nt0) {
        ps = sw % NPS;
        nt0 = (sw / NPS) * NT;
    }
};

// bf16 hi + lo split of the chunk-state token operand w_s x_s[p] for the 8
// rows s a lane holds (xv: raw bf16 x, ws: the rows' state weights).
__device__ __forceinline__ void split_wx(const i16x8 &xv, const float (&ws)[8], bf16x8 &bhi,
                                         bf16x8 &blo) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = bf16_float((uint16_t)xv[j]) * ws[j];
    u32x4 hv, lv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t h2 = bf16_pack(v[2 * j], v[2 * j + 1]);
        hv[j] = h2;
        const float lo0 = v[2 * j] - bf16_float(h2 & 0xffff);
        const float lo1 = v[2 * j + 1] - bf16_float(h2 >> 16);
        lv[j] = bf16_pack(lo0, lo1);
    }
    bhi = __builtin_bit_cast(bf16x8, hv);
    blo = __builtin_bit_cast(bf16x8, lv);
}

// A state K step's arithmetic from its operands: xv (the lane's 8 raw x values),
// ws (their state weights) and bop(i), the B^T operand of n-tile nt0 + i.
template <int NT, class F>
__device__ __forceinline__ void state_kstep_ops(const i16x8 &xv, const float (&ws)[8], F bop,
                                                f32x4 (&acc)[NT]) {
    bf16x8 bhi, blo;
    split_wx(xv, ws, bhi, blo);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const bf16x8 a = bop(i);
        acc[i] = mfma16(a, bhi, acc[i]);
        acc[i] = mfma16(a, blo, acc[i]);
    }
}

// One K = 32 step for NT n-tiles (from nt0) of a p-slab: rows row0 ..
// row0 + 31 of the row-major x tile (byte base xb, row stride xs elements,
// the slab's first column xc) and of the B tile (bb, bs); wk points at the
// state weights of those rows. Lane group q = (lane % 64) / 16 supplies rows
// 8q .. 8q + 7 of the step: k index j of both operands is row 8q + j.
template <int NT>
__device__ __forceinline__ void state_kstep(const char *lds, int xb, int xs, int xc, int bb,
                                            int bs, int row0, int nt0, const float *wk,
                                            f32x4 (&acc)[NT]) {
    const int lane = lane_id();
    const int q = lane >> 4;
    const i16x8 xv = lds_tr8(lds, tr_lane(lane, xs) + 8 * q * xs * 2, xb + (row0 * xs + xc) * 2,
                             4 * xs * 2);
    const float4 w0 = *reinterpret_cast<const float4 *>(wk + 8 * q);
    const float4 w1 = *reinterpret_cast<const float4 *>(wk + 8 * q + 4);
    const float ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const int lab = tr_lane(lane, bs) + 8 * q * bs * 2;
    state_kstep_ops<NT>(
        xv, ws,
        [&](int i) {
            return as_bf16x8(lds_tr8(lds, lab, bb + (row0 * bs + 16 * (nt0 + i)) * 2, 4 * bs * 2));
        },
        acc);
}

// The prefill's form of the step, for waves that have direct global-to-LDS
// loads in flight into other rows of the same tiles. The compiler cannot
// tell those rows apart and would wait for every load before each LDS read;
// here each fetch is an asm statement that waits for its own reads
// (lgkmcnt) only. XS and BS are the x and B row strides in elements.
__device__ __forceinline__ uint32_t lds_off(const void *p) {
    return (uint32_t)(uintptr_t)(const lds_char *)p;
}

template <int D>
__device__ __forceinline__ i16x8 lds_tr8_own(uint32_t a) {
    i16x4 x, y;
    asm volatile("ds_read_b64_tr_b16 %0, %2\n\t"
                 "ds_read_b64_tr_b16 %1, %2 offset:%3\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(x), "=&v"(y)
                 : "v"(a), "i"(D));
    const i16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return v;
}

__device__ __forceinline__ void lds_f32x8_own(uint32_t a, f32x4 &w0, f32x4 &w1) {
    asm volatile("ds_read_b128 %0, %2\n\t"
                 "ds_read_b128 %1, %2 offset:16\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(w0), "=&v"(w1)
                 : "v"(a));
}

// Four n-tiles' B^T operands in one asm statement (one LDS round trip):
// tiles at byte addresses a, a + 32, a + 64, a + 96, each two transposed
// fetches D bytes apart.
template <int D>
__device__ __forceinline__ void lds_tr8x4_own(uint32_t a, bf16x8 (&o)[4]) {
    i16x4 r[8];
    asm volatile("ds_read_b64_tr_b16 %0, %8\n\t"
                 "ds_read_b64_tr_b16 %1, %8 offset:%9\n\t"
                 "ds_read_b64_tr_b16 %2, %8 offset:32\n\t"
                 "ds_read_b64_tr_b16 %3, %8 offset:%10\n\t"
                 "ds_read_b64_tr_b16 %4, %8 offset:64\n\t"
                 "ds_read_b64_tr_b16 %5, %8 offset:%11\n\t"
                 "ds_read_b64_tr_b16 %6, %8 offset:96\n\t"
                 "ds_read_b64_tr_b16 %7, %8 offset:%12\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                   "=&v"(r[6]), "=&v"(r[7])
                 : "v"(a), "i"(D), "i"(32 + D), "i"(64 + D), "i"(96 + D));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const i16x8 v = {r[2 * i][0],     r[2 * i][1],     r[2 * i][2],     r[2 * i][3],
                         r[2 * i + 1][0], r[2 * i + 1][1], r[2 * i + 1][2], r[2 * i + 1][3]};
        o[i] = as_bf16x8(v);
    }
}

template <int NT, int XS, int BS>
__device__ __forceinline__ void state_kstep_own(const char *lds, int xb, int xc, int bb, int row0,
                                                int nt0, const float *wk, f32x4 (&acc)[NT]) {
    const int lane = lane_id();
    const int q = lane >> 4;
    const uint32_t l0 = lds_off(lds);
    const i16x8 xv = lds_tr8_own<4 * XS * 2>(l0 + tr_lane(lane, XS) + 8 * q * XS * 2 + xb +
                                             (row0 * XS + xc) * 2);
    f32x4 w0, w1;
    lds_f32x8_own(lds_off(wk + 8 * q), w0, w1);
    const float ws[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    const uint32_t lab = l0 + tr_lane(lane, BS) + 8 * q * BS * 2 + bb + (row0 * BS + 16 * nt0) * 2;
    if constexpr (NT % 4 == 0) {
        // the B^T operands four tiles per LDS round trip
        bf16x8 bo[NT];
#pragma unroll
        for (int i = 0; i < NT; i += 4)
            lds_tr8x4_own<4 * BS * 2>(lab + 32 * i, *reinterpret_cast<bf16x8(*)[4]>(bo + i));
        state_kstep_ops<NT>(xv, ws, [&](int i) { return bo[i]; }, acc);
    } else {
        state_kstep_ops<NT>(
            xv, ws, [&](int i) { return as_bf16x8(lds_tr8_own<4 * BS * 2>(lab + 32 * i)); }, acc);
    }
}

// Tiles nt0 .. nt0 + NT - 1 of p-slab ps <-> a [P][N] fp32 state in global
// memory (one float4 per lane and tile); a null source loads zeros.
template <int P, int N, int NT, bool LOAD>
__device__ __forceinline__ void slab_io(float *g, int ps, int nt0, f32x4 (&S)[NT]) {
    const int lane = lane_id();
    const int p = 16 * ps + (lane & 15), q = lane >> 4;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t e = (int64_t)p * N + 16 * (nt0 + i) + 4 * q;
        if (LOAD) {
            const float4 v = g ? *reinterpret_cast<const float4 *>(g + e)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
            S[i][0] = v.x;
            S[i][1] = v.y;
            S[i][2] = v.z;
            S[i][3] = v.w;
        } else {
            *reinterpret_cast<float4 *>(g + e) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
        }
    }
}

// bf16 (nearest even) of the tiles: into the row-major S_bf tile in LDS
// (byte base sb, row stride ss; sb < 0: not stored) and into a [N/16][gP][16]
// bf16 copy in global memory (gbf, or null), the tiles' rows from row gp0 of
// it (a workgroup holding columns gp0 .. gp0 + P - 1 of a head of width gP).
template <int P, int NT>
__device__ __forceinline__ void slab_bf16(const f32x4 (&S)[NT], int ps, int nt0, char *lds, int sb,
                                          int ss, uint16_t *gbf, int gP = P, int gp0 = 0) {
    const int lane = lane_id();
    const int p = 16 * ps + (lane & 15), q = lane >> 4;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int n = 16 * (nt0 + i) + 4 * q;
        const uint2 v = make_uint2(bf16_pack(S[i][0], S[i][1]), bf16_pack(S[i][2], S[i][3]));
        if (sb >= 0)
            *reinterpret_cast<uint2 *>(lds + sb + (p * ss + n) * 2) = v;
        if (gbf)
            *reinterpret_cast<uint2 *>(gbf + state_bf_index(gp0 + p, n, gP)) = v;
    }
}

template <int NT>
__device__ __forceinline__ void slab_scale(f32x4 (&S)[NT], float dec) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[i][r] = S[i][r] * dec;
}

// Buffer row of buffered position j of one slot, for one wave.
// Contiguous buffers: row slot * Q + j. Paged buffers: lane i holds the
// slot's page-table entry i (entries repeat across the wave) and a lookup
// is one lane shuffle, so no lookup waits on memory; every lane of the wave
// must take part in a lookup.
template <bool PG>
struct SlotRows;

template <>
struct SlotRows<false> {
    int64_t base;
    SlotRows() = default;
    __device__ SlotRows(const BufMap &, int slot, int Q) : base((int64_t)slot * Q) {}
    __device__ bool ok(const BufMap &, int) const { return true; }
    __device__ int64_t operator()(int j) const { return base + j; }
};

template <>
struct SlotRows<true> {
    int ent, shift;
    SlotRows() = default;
    __device__ SlotRows(const BufMap &m, int slot, int) : shift(m.shift) {
        ent = m.pages[(int64_t)slot * m.npp + (lane_id() & (m.npp - 1))];
    }
    // the entries of positions [0, npos) are pages of the pool (same answer
    // in every lane)
    __device__ bool ok(const BufMap &m, int npos) const {
        const int n = (npos + (1 << shift) - 1) >> shift;
        const bool bad = lane_id() < n && (ent < 0 || ent >= m.num_pages);
        return __ballot(bad) == 0;
    }
    __device__ int64_t operator()(int j) const {
        return ((int64_t)__shfl(ent, j >> shift, 64) << shift) + (j & ((1 << shift) - 1));
    }
};

// Chunk positions: [0, nb) from the slot buffer, [nb, n_valid) from the
// packed input starting at token tok_base; later rows are zero.
template <class DT, bool PG = false>
struct MView {
    using TD = typename DT::T;
    const uint16_t *x, *B, *C;
    const TD *dt;
    const uint16_t *bx, *bB;   // buffer arrays (whole pool), rows through `rows`
    const TD *bdt;
    SlotRows<PG> rows;
    int64_t tok_base;
    int nb, n_valid;
    int h, g, H, G;
    // input x and output y rows: elements per token (H times the full head
    // width) and the first column of this workgroup's part of the head
    int64_t xrow;
    int xoff;
    __device__ int64_t token(int j) const { return tok_base + (j - nb); }
};

__device__ __forceinline__ uint4 keep_if(bool ok, const uint4 &u) {
    return make_uint4(ok ? u.x : 0u, ok ? u.y : 0u, ok ? u.z : 0u, ok ? u.w : 0u);
}

// Chunk rows [r0, r0 + kSlab) of x and B straight from global memory into
// LDS tile rows [h0, h0 + kSlab), with no registers in between (gfx950's
// direct loads to LDS: a wave's 64 lanes fill 1 KB of LDS, 16 bytes each,
// in lane order). The x and B regions of the slab are whole 1 KB pieces;
// wave wv of the NWV waves that stage takes pieces wv, wv + NWV, .... Lanes
// whose 16 bytes fall in a row's padding or in a row past n_valid load
// nothing; the rows past n_valid are zeroed by the same waves. The loads
// count in vmcnt: the staging waves wait (wait_vmcnt<0>) before the barrier
// that publishes the rows. Buffered rows (below nb) come from the slot
// buffer, the others from the input.
constexpr int kSlab = 128;

typedef __attribute__((address_space(3))) void lds_void;

// One stream (x or B) of a slab: K pieces of 1 KB, of which this wave takes
// k0, k0 + NWV, ...; a piece covers bytes [1024 k, 1024 k + 1024) of the
// LDS tile rows (RB bytes each, VB of them data). A lane's (row, byte)
// advances by a constant step from piece to piece.
template <int VB, int RB, int K, int NWV>
__device__ __forceinline__ void stage_stream(const char *gbase, int gstride, int r0, int n_valid,
                                             int k0, char *ldst) {
    constexpr int DR = NWV * 1024 / RB, DC = NWV * 1024 % RB;
    const int o = k0 * 1024 + 16 * lane_id();
    int row = o / RB, cb = o - (o / RB) * RB;
    for (int k = k0; k < K; k += NWV) {
        const int j = r0 + row;
        if (cb < VB && j < n_valid)
            __builtin_amdgcn_global_load_lds(gbase + (uint32_t)(j * gstride + cb),
                                             (lds_void *)(ldst + k * 1024), 16, 0, 0);
        row += DR;
        cb += DC;
        if (cb >= RB) {
            cb -= RB;
            ++row;
        }
    }
}

// The same with rows below nb from a contiguous slot buffer (row j at
// gbuf + j * gstride) and the others from the input (row j at
// gin + (j - nb) * gstride).
template <int VB, int RB, int K, int NWV>
__device__ __forceinline__ void stage_stream_split(const char *gbuf, const char *gin, int gstride,
                                                   int nb, int r0, int n_valid, int k0,
                                                   char *ldst) {
    constexpr int DR = NWV * 1024 / RB, DC = NWV * 1024 % RB;
    const int o = k0 * 1024 + 16 * lane_id();
    int row = o / RB, cb = o - (o / RB) * RB;
    for (int k = k0; k < K; k += NWV) {
        const int j = r0 + row;
        if (cb < VB && j < n_valid) {
            const char *src = j < nb ? gbuf + (uint32_t)(j * gstride + cb)
                                     : gin + (uint32_t)((j - nb) * gstride + cb);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(ldst + k * 1024), 16, 0, 0);
        }
        row += DR;
        cb += DC;
        if (cb >= RB) {
            cb -= RB;
            ++row;
        }
    }
}

template <int P, int N, int NWV, class DT, bool PG>
__device__ __forceinline__ void stage_slab(const MView<DT, PG> &v, int r0, int h0, int wv,
                                           char *lds, const MLayout &L) {
    constexpr int XRB = (P + kPad) * 2, BRB = (N + kPad) * 2;   // row strides, bytes
    constexpr int XK = kSlab * XRB / 1024, BK = kSlab * BRB / 1024;
    static_assert(XK * 1024 == kSlab * XRB && BK * 1024 == kSlab * BRB, "1 KB pieces");
    const int lane = lane_id();
    if (v.nb == 0) {
        // every row is an input token: row j at base + j * stride; the
        // pieces are dealt to the waves as one sequence, x then B
        const char *xb = reinterpret_cast<const char *>(v.x + v.token(0) * v.xrow + v.xoff);
        const char *bb = reinterpret_cast<const char *>(v.B + (v.token(0) * v.G + v.g) * N);
        stage_stream<P * 2, XRB, XK, NWV>(xb, (int)v.xrow * 2, r0, v.n_valid, wv,
                                          lds + L.X + h0 * XRB);
        stage_stream<N * 2, BRB, BK, NWV>(bb, v.G * N * 2, r0, v.n_valid,
                                          ((wv - XK) % NWV + NWV) % NWV, lds + L.B + h0 * BRB);
    } else if constexpr (!PG) {
        // buffered rows from the slot's contiguous buffer rows (row j at slot
        // row rows(0) + j), the others from the input (row nb is token
        // tok_base)
        const int64_t b0 = v.rows(0);
        const char *xbuf = reinterpret_cast<const char *>(v.bx + b0 * v.xrow + v.xoff);
        const char *bbuf = reinterpret_cast<const char *>(v.bB + (b0 * v.G + v.g) * N);
        const char *xin = reinterpret_cast<const char *>(v.x + v.tok_base * v.xrow + v.xoff);
        const char *bin = reinterpret_cast<const char *>(v.B + (v.tok_base * v.G + v.g) * N);
        stage_stream_split<P * 2, XRB, XK, NWV>(xbuf, xin, (int)v.xrow * 2, v.nb, r0, v.n_valid,
                                                wv, lds + L.X + h0 * XRB);
        stage_stream_split<N * 2, BRB, BK, NWV>(bbuf, bin, v.G * N * 2, v.nb, r0, v.n_valid,
                                                ((wv - XK) % NWV + NWV) % NWV,
                                                lds + L.B + h0 * BRB);
    } else {
        for (int k = wv; k < XK + BK; k += NWV) {
            const bool isx = k < XK;
            const int kk = isx ? k : k - XK;
            const int o = kk * 1024 + 16 * lane;
            const int row = isx ? o / XRB : o / BRB, cb = isx ? o % XRB : o % BRB;
            const int j = r0 + row;
            const bool ok = cb < (isx ? P * 2 : N * 2) && j < v.n_valid;
            const int jj = ok ? j : 0;
            const int64_t br = v.rows(jj);   // (paged: every lane takes part)
            const bool buf = jj < v.nb;
            const uint16_t *src =
                isx ? (buf ? v.bx + br * v.xrow + v.xoff : v.x + v.token(jj) * v.xrow + v.xoff)
                    : (buf ? v.bB + (br * v.G + v.g) * N : v.B + (v.token(jj) * v.G + v.g) * N);
            char *dst = lds + (isx ? L.X + h0 * XRB : L.B + h0 * BRB) + kk * 1024;
            if (ok)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const char *>(src) + cb,
                                                 (lds_void *)dst, 16, 0, 0);
        }
    }
    // rows of the slab past n_valid: zeros (16-byte pieces, x then B)
    const int v0 = min(max(v.n_valid - r0, 0), kSlab);
    const int nz = (kSlab - v0) * (P / 8 + N / 8);
    for (int e = lane + 64 * wv; e < nz; e += 64 * NWV) {
        const int row = v0 + e / (P / 8 + N / 8), q = e % (P / 8 + N / 8);
        char *dst = q < P / 8 ? lds + L.X + ((h0 + row) * (P + kPad) + 8 * q) * 2
                              : lds + L.B + ((h0 + row) * (N + kPad) + 8 * (q - P / 8)) * 2;
        *reinterpret_cast<uint4 *>(dst) = make_uint4(0, 0, 0, 0);
    }
}

// Raw dt of chunk rows lane + 64 i (one wave; rows past the chunk load row 0).
template <class DT, bool PG>
__device__ __forceinline__ void load_dt(const MView<DT, PG> &v, typename DT::T (&raw)[4]) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        const int jd = j < v.n_valid ? j : 0;
        const int64_t br = v.rows(jd);
        raw[i] = jd < v.nb ? v.bdt[br * v.H + v.h] : v.dt[v.token(jd) * v.H + v.h];
    }
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maximum, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// Per-row quantities of a chunk, computed by the whole workgroup (one row per
// thread; rows past n_valid have delta 0): lam (in-chunk cumulative sum of
// delta A, log2 units), u = lam - log2(delta), 2^lam, beta = 2^(c - u) with c
// the lam at the end of the row's 32-row block, and, with `weights`, the
// state weights w = 2^(lam_last - lam) delta.
__device__ __forceinline__ void chunk_scalars(float dt_raw, int n_valid, float A2_h, float bias,
                                              int softplus, bool weights, char *lds,
                                              const MLayout &L) {
    float *lam = reinterpret_cast<float *>(lds + L.lam);
    float *uu = reinterpret_cast<float *>(lds + L.u);
    float *el = reinterpret_cast<float *>(lds + L.el);
    float *w = reinterpret_cast<float *>(lds + L.w);
    const int j = threadIdx.x;
    float d = 0.0f, a = 0.0f;
    if (j < n_valid) {
        d = delta_of(dt_raw, bias, softplus);
        a = d * A2_h;
    }
    const float l = block_scan_inclusive(a, reinterpret_cast<float *>(lds + L.tot));
    if (j < kMaxQ) {
        lam[j] = l;
        uu[j] = l - flog2(d);
        el[j] = fexp2(l);
    }
    __syncthreads();
    if (j < kMaxQ) {
        reinterpret_cast<float *>(lds + L.beta)[j] = fexp2(lam[j | 31] - uu[j]);
        if (weights)
            w[j] = fexp2(lam[n_valid - 1] - l) * d;
    }
}

// The same per-row quantities computed by one wave for rows j = lane + 64 i
// (wave_scan_segments evaluates the block scan's tree), into the per-row
// arrays of layout L; the state weights always.
template <class DT>
__device__ __forceinline__ void chunk_scalars_wave(const typename DT::T (&raw)[4], int n_valid,
                                                   float A2_h, float bias, int softplus,
                                                   char *lds, const MLayout &L) {
    const int lane = lane_id();
    float *lam = reinterpret_cast<float *>(lds + L.lam);
    float *uu = reinterpret_cast<float *>(lds + L.u);
    float *el = reinterpret_cast<float *>(lds + L.el);
    float *w = reinterpret_cast<float *>(lds + L.w);
    float *bt = reinterpret_cast<float *>(lds + L.beta);
    float dv[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        float dd = 0.0f, aa = 0.0f;
        if (j < n_valid) {
            dd = delta_of(DT::val(raw[i]), bias, softplus);
            aa = dd * A2_h;
        }
        dv[i] = dd;
        lv[i] = aa;
    }
    wave_scan_segments(lv, 4);
    // lam of the chunk's last row
    const int jl = n_valid - 1;
    float last = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float t = __shfl(lv[i], jl & 63, 64);
        last = (jl >> 6) == i ? t : last;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        const float l = lv[i];
        const float u = l - flog2(dv[i]);
        lam[j] = l;
        uu[j] = u;
        el[j] = fexp2(l);
        bt[j] = fexp2(__shfl(l, lane | 31, 64) - u);
        w[j] = fexp2(last - l) * dv[i];
    }
}

// Rows [0, rows) of the chunk's x (CX 16-byte pieces per row) and B (CB
// pieces per row) into the padded LDS tiles; chunk row j is global row
// rmap(j) of xs / bs (strides in elements); rows past n_valid are zero.
// Both streams share one index space so that eight pieces per thread are in
// flight at a time.
template <int CX, int CB, class RM>
__device__ __forceinline__ void stage_rows(const RM &rmap, const uint16_t *xs, int64_t xstride,
                                           const uint16_t *bs, int64_t bstride, int rows,
                                           int n_valid, char *xdst, int XS, char *bdst, int BS) {
    const int nthr = blockDim.x, tid = threadIdx.x;
    const int nx = rows * CX, total = nx + rows * CB;
    for (int e0 = 0; e0 < total; e0 += 8 * nthr) {
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = e0 + tid + i * nthr;
            const bool isx = e < nx;
            const int f = isx ? e : e - nx, C = isx ? CX : CB;
            const int j = f / C, q = f % C;
            const int jj = (e < total && j < n_valid) ? j : 0;
            const int64_t gr = rmap(jj);
            v[i] = isx ? *reinterpret_cast<const uint4 *>(xs + gr * xstride + 8 * q)
                       : *reinterpret_cast<const uint4 *>(bs + gr * bstride + 8 * q);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = e0 + tid + i * nthr;
            const bool isx = e < nx;
            const int f = isx ? e : e - nx, C = isx ? CX : CB;
            const int j = f / C, q = f % C;
            if (e < total)
                *reinterpret_cast<uint4 *>((isx ? xdst : bdst) + (j * (isx ? XS : BS) + 8 * q) * 2) =
                    keep_if(j < n_valid, v[i]);
        }
    }
}

// C fragments of t-block tau: lane gets C[t][16k + 8g .. +7] for rows t that
// produce output (t in [row_lo, n_valid)), zeros otherwise. When every row
// of the t-block is an output row the loaded values are used as they are,
// so nothing waits for the loads before the first MFMA that reads them.
template <int N, class DT, bool PG>
__device__ __forceinline__ void load_cfrag(const MView<DT, PG> &v, int tau, int row_lo,
                                           bf16x8 (&cf)[N / 16]) {
    // rows outside [row_lo, n_valid) load row row_lo and are zeroed after
    const int lane = lane_id();
    const int g = lane >> 5, t = 32 * tau + (lane & 31);
    const bool ok = t >= row_lo && t < v.n_valid && t >= v.nb;
    const bool all = row_lo <= 32 * tau && 32 * tau + 32 <= v.n_valid && v.nb <= 32 * tau;
    const int tt = ok ? t : row_lo;
    const uint16_t *src = v.C + (v.token(tt) * v.G + v.g) * N;
    uint4 raw[N / 16];
#pragma unroll
    for (int k = 0; k < N / 16; ++k)
        raw[k] = *reinterpret_cast<const uint4 *>(src + 16 * k + 8 * g);
    if (all) {
#pragma unroll
        for (int k = 0; k < N / 16; ++k)
            cf[k] = __builtin_bit_cast(bf16x8, raw[k]);
    } else {
#pragma unroll
        for (int k = 0; k < N / 16; ++k)
            cf[k] = __builtin_bit_cast(bf16x8, keep_if(ok, raw[k]));
    }
}

// The prefill's form: rows that produce no output keep the row they loaded
// (row row_lo, an input token) instead of zeros. Column t of the read-out,
// C.B^T and M.X tiles depends on lane column t of cf alone, and columns of
// rows that are not outputs are never stored, so every stored element is
// the same; leaving out the select lets the fragments be loaded straight
// into the registers the MFMAs read.
template <int N, class DT, bool PG>
__device__ __forceinline__ void load_cfrag_raw(const MView<DT, PG> &v, int tau, int row_lo,
                                               bf16x8 (&cf)[N / 16]) {
    const int lane = lane_id();
    const int g = lane >> 5, t = 32 * tau + (lane & 31);
    const bool ok = t >= row_lo && t < v.n_valid && t >= v.nb;
    const uint16_t *src = v.C + (v.token(ok ? t : row_lo) * v.G + v.g) * N;
#pragma unroll
    for (int k = 0; k < N / 16; ++k)
        cf[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src + 16 * k + 8 * g));
}

// y rows [row_lo, row_hi) of t-block tau: y = fmaf(D, x, acc), -0 -> +0.
template <int P, int PT0, int PT1, class V>
__device__ __forceinline__ void emit_tblock(const V &v, int tau, int row_lo, int row_hi,
                                            float D_h, const char *lds, const MLayout &L,
                                            const f32x16 *acc, uint16_t *y) {
    const int lane = lane_id();
    const int g = lane >> 5, c = lane & 31;
    const int t = 32 * tau + c;
    if (t < row_lo || t >= row_hi)
        return;
    uint16_t *yrow = y + v.token(t) * v.xrow + v.xoff;
    const char *xrow = lds + L.X + t * L.XS * 2;
    // four outputs at a time (bf16 pairs rounded to nearest even, as one
    // conversion each), so that few of them are live at once
#pragma unroll
    for (int pt = PT0; pt < PT1; ++pt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int p = 32 * pt + 8 * q + 4 * g;
            const uint2 xr = *reinterpret_cast<const uint2 *>(xrow + 2 * p);
            float yv[4];
            yv[0] = fmaf(D_h, bf16_float(xr.x & 0xffff), acc[pt][4 * q]);
            yv[1] = fmaf(D_h, bf16_float(xr.x >> 16), acc[pt][4 * q + 1]);
            yv[2] = fmaf(D_h, bf16_float(xr.y & 0xffff), acc[pt][4 * q + 2]);
            yv[3] = fmaf(D_h, bf16_float(xr.y >> 16), acc[pt][4 * q + 3]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                yv[e] = yv[e] + 0.0f;  // -0 -> +0
            *reinterpret_cast<uint2 *>(yrow + p) =
                make_uint2(bf16_pack(yv[0], yv[1]), bf16_pack(yv[2], yv[3]));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Renumber them so that consecutive work items (the heads of one
// sequence, which share its B and C rows) run on the same XCD.
__device__ __forceinline__ int xcd_local_index(int bid, int nblocks) {
    constexpr int kXcds = 8;
    if (nblocks % kXcds != 0)
        return bid;
    return (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
}

// Prefill workgroups have 12 waves (three per SIMD; wave w runs on SIMD
// w % 4). Waves 0..3 are the state waves: each owns a quarter of the fp32
// state in registers and updates it over the chunk, and they stage the
// chunk rows into LDS. Waves 4..11 each compute the outputs of one 32-row
// t-block: with 8 t-blocks wave 4 + k takes k and wave 8 + k takes 7 - k, so
// every SIMD has the same causal work. t-blocks 0..3 finish (and store their
// outputs) in the first half of the chunk, on the older waves, which a SIMD
// issues first; in the second half they are idle and t-blocks 4..7 have the
// SIMDs to themselves. One t-block wave also computes the next chunk's
// per-row quantities (into the other set of per-row arrays) once its own
// t-block is done: with two slabs t-block 3's (idle in the second half, next
// to t-block 4, the lightest there), with one slab an idle wave.
constexpr int kPrefillWaves = 12;

__device__ __forceinline__ int wave_tblock(int nT, int wave) {
    const int i = wave - kStateWaves;
    if (i < 0)
        return -1;
    if (nT == 8)
        return i < 4 ? i : 11 - i;
    return i < nT ? i : -1;
}

template <int P, int N, class DT, bool PG, bool RP>
__device__ __forceinline__ void scan_one(const ScanArgs &a, int s, int h, char *lds,
                                         int part = 0) {
    using TD = typename DT::T;
    using SL = Slab<P, N>;
    const Dims d = a.d;
    const int H = d.H, G = d.G, Q = d.Q;
    const int Qp = Q < 32 ? 32 : Q;
    const int g = h / (H / G);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool swave = wave < kStateWaves;
    // this workgroup's columns of the head: P of the head's d.P (all of them,
    // or half with psplit), from column p0; a head's state is [d.P][N]
    const int p0 = part * P;
    const int64_t HS = (int64_t)d.P * N, p0N = (int64_t)p0 * N;
    const MLayout L(kMaxQ, P, N);
    // replay calls (RP) read the slot cache and buffer; plain prefill does not
    constexpr bool replay = RP;

    const int64_t t0 = a.cu[s];
    const int len = seq_len(a.cu, a.take, s);
    const int slot = replay ? (a.slot_idx ? a.slot_idx[s] : s) : s;
    if (replay && (len == 0 || slot < 0 || slot >= a.num_slots))
        return;
    const int nbuf = replay ? a.buf_len[slot] : 0;
    if (nbuf < 0 || nbuf >= Q)
        return;
    // acceptance without a chunk that fills has no work here (the buffer
    // append is the commit kernel's); with only_cross, verification handles
    // just the sequences whose drafts run past the chunk end
    if (((RP && a.no_y) && nbuf + len < Q) || ((RP && a.only_cross) && nbuf + len <= Q))
        return;
    const SlotRows<PG> rows(a.bm, slot, Q);
    if (!rows.ok(a.bm, (RP && a.dry) ? nbuf : replay_npos(nbuf, len, Q)))
        return;

    float *init = replay ? a.cache_state + ((int64_t)slot * H + h) * HS + p0N
                           : (a.init_state ? const_cast<float *>(a.init_state) +
                                                 ((int64_t)s * H + h) * HS + p0N
                                           : nullptr);
    // the state waves' tiles of the state, and its bf16 read-out copy in LDS
    int ps, nt0;
    SL::own(swave ? wave : 0, ps, nt0);
    f32x4 S[SL::NT];
    if (swave)
        slab_io<P, N, SL::NT, true>(init, ps, nt0, S);

    MView<DT, PG> v;
    v.x = static_cast<const uint16_t *>(a.x);
    v.B = static_cast<const uint16_t *>(a.B);
    v.C = static_cast<const uint16_t *>(a.C);
    v.dt = static_cast<const TD *>(a.dt);
    v.bx = replay ? static_cast<const uint16_t *>(a.buf_x) : nullptr;
    v.bB = replay ? static_cast<const uint16_t *>(a.buf_B) : nullptr;
    v.bdt = replay ? static_cast<const TD *>(a.buf_dt) : nullptr;
    v.rows = rows;
    v.h = h; v.g = g; v.H = H; v.G = G;
    v.xrow = (int64_t)H * d.P;
    v.xoff = h * d.P + p0;

    const float A2_h = a.A[h] * kLog2e;
    const float D_h = a.D ? a.D[h] : 0.0f;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const int total = nbuf + len;
    const int nfull = total / Q;
    // without outputs only the chunks that fill are processed
    const int nchunks = (RP && a.no_y) ? nfull : (total + Q - 1) / Q;
    float *bnd = replay ? a.cache_state + ((int64_t)slot * H + h) * HS + p0N
                          : (a.boundary_state ? a.boundary_state + ((int64_t)s * H + h) * HS + p0N
                                              : nullptr);
    uint16_t *bnd_bf = replay ? static_cast<uint16_t *>(a.cache_state_bf) +
                                      ((int64_t)slot * H + h) * HS
                                : nullptr;
    const bool write_bnd = bnd && (!replay || nfull > 0) && !(RP && a.dry);
    uint16_t *y = static_cast<uint16_t *>(a.y);
    // chunk-end states of the full chunks (plain prefill): rows from
    // full_chunks_before(s) on
    float *cst = nullptr;
    if (!replay && a.chunk_states)
        cst = a.chunk_states +
              ((int64_t)full_chunks_before(a.cu, s, Q, reinterpret_cast<int *>(lds + L.tot)) * H +
               h) * HS + p0N;
    const int tau = wave_tblock(Qp / 32, wave);
    auto set_chunk = [&](int c) {
        v.nb = (c == 0) ? nbuf : 0;
        v.n_valid = min(Q, total - c * Q);
        v.tok_base = t0 + (int64_t)c * Q + v.nb - nbuf;
    };

    // The chunk rows pass through LDS in slabs of 128 rows, double-buffered
    // in the two halves of the x and B tiles, by direct loads (no registers),
    // all staged by the state waves:
    //  - chunk size 256: rows 0..127 (slab A) in half 0, 128..255 (slab B)
    //    in half 1. Phase 1: every t-block takes its s-blocks 0..3 (t-blocks
    //    0..3 finish), the state waves stage slab B and take their K steps
    //    0..3. Phase 2: t-blocks 4..7 take s-blocks 4.., the state waves
    //    stage the next chunk's slab A and take their K steps 4..7. Two
    //    barriers per chunk.
    //  - chunk size <= 128: chunk c in half c % 2, the next chunk staged in
    //    the other half during this one. One barrier.
    // S_bf and the per-row arrays alternate between two sets, so the state
    // waves write the next chunk's while this chunk reads its own.
    const bool two = Qp > kSlab;
    auto lay = [&](int c) { return L.chunk(c & 1, two ? 0 : kSlab * (c & 1)); };
    if (nchunks > 0) {
        set_chunk(0);
        if (swave) {
            slab_bf16<P, SL::NT>(S, ps, nt0, lds, L.S, L.SS, nullptr);
            stage_slab<P, N, kStateWaves>(v, 0, 0, wave, lds, L);
            if (wave == 0) {
                TD rawdt[4];
                load_dt<DT>(v, rawdt);
                chunk_scalars_wave<DT>(rawdt, v.n_valid, A2_h, bias, d.softplus, lds,
                                       L.buf(0));
            }
            wait_vmcnt<0>();
        }
        __syncthreads();
    }
    // The two roles run separate copies of the chunk loop (so that neither
    // keeps the other's registers live), meeting at the same barriers.
    if (swave) {
        for (int c = 0; c < nchunks; ++c) {
            const MLayout Lc = lay(c);
            // S is the state after c chunks
            if (c == nfull && write_bnd) {
                slab_io<P, N, SL::NT, false>(bnd, ps, nt0, S);
                if (bnd_bf)
                    slab_bf16<P, SL::NT>(S, ps, nt0, lds, -1, 0, bnd_bf, d.P, p0);
            }
            if (cst && c >= 1 && c <= nfull)
                slab_io<P, N, SL::NT, false>(cst + (int64_t)(c - 1) * H * HS, ps, nt0, S);
            set_chunk(c);
            const int n_valid = v.n_valid;
            const bool upd = n_valid == Q || (!replay && a.final_state);
            const bool more = c + 1 < nchunks;
            const MView<DT, PG> vc = v;
            if (more)
                set_chunk(c + 1);
            const int nk = Qp / 32, nk1 = two ? kSlab / 32 : nk;
            // K steps [k0, k1) of this chunk, through tile pointer t
            auto ksteps = [&](char *t, int k0, int k1) {
                const float *w = reinterpret_cast<const float *>(t + Lc.w);
                for (int kk = k0; kk < k1; ++kk)
                    state_kstep_own<SL::NT, P + kPad, N + kPad>(t, Lc.X, 16 * ps, Lc.B, 32 * kk,
                                                                nt0, w + 32 * kk, S);
            };
            // Phase 1 (or the only phase): staging this chunk's slab B (two
            // slabs) or the next chunk into the other half, then the K steps
            // over the rows that are in
            if (two) {
                stage_slab<P, N, kStateWaves>(vc, kSlab, kSlab, wave, lds, L);
            } else if (more) {
                stage_slab<P, N, kStateWaves>(v, 0, kSlab * ((c + 1) & 1), wave, lds, L);
            }
            if (upd) {
                slab_scale<SL::NT>(
                    S, fexp2(reinterpret_cast<const float *>(lds + Lc.lam)[n_valid - 1]));
                ksteps(lds, 0, nk1);
            }
            if (!two && upd && more)
                slab_bf16<P, SL::NT>(S, ps, nt0, lds, L.chunk((c + 1) & 1, 0).S, L.SS, nullptr);
            if (two) {
                wait_vmcnt<0>();
                __syncthreads();   // phase 2: slab B is in, slab A is free
                // staging the next chunk's slab A, the remaining K steps and
                // the next chunk's read-out copy
                if (more)
                    stage_slab<P, N, kStateWaves>(v, 0, 0, wave, lds, L);
                if (upd)
                    ksteps(lds, nk1, nk);
                if (upd && more)
                    slab_bf16<P, SL::NT>(S, ps, nt0, lds, L.chunk((c + 1) & 1, 0).S, L.SS,
                                         nullptr);
            }
            wait_vmcnt<0>();
            __syncthreads();   // end of chunk c
        }
        if (cst && nfull == nchunks && nfull > 0)
            slab_io<P, N, SL::NT, false>(cst + (int64_t)(nfull - 1) * H * HS, ps, nt0, S);
        if (nfull == nchunks && write_bnd) {
            slab_io<P, N, SL::NT, false>(bnd, ps, nt0, S);
            if (bnd_bf)
                slab_bf16<P, SL::NT>(S, ps, nt0, lds, -1, 0, bnd_bf, d.P, p0);
        }
        if (!replay && a.final_state)
            slab_io<P, N, SL::NT, false>(a.final_state + ((int64_t)s * H + h) * HS + p0N, ps, nt0,
                                         S);
    } else {
        // t-block waves. The C rows of the t-block's next chunk go out right
        // after its outputs; a t-block without output rows loads the chunk's
        // last row (n_valid - 1 >= nb is an input token).
        bf16x8 cf[N / 16];
        auto load_c = [&](const MView<DT, PG> &vv) {
            const int lo = max(32 * tau, vv.nb), hi = min(32 * tau + 32, vv.n_valid);
            load_cfrag_raw<N, DT>(vv, tau, lo < hi ? lo : vv.n_valid - 1, cf);
        };
        if (nchunks > 0 && tau >= 0) {
            set_chunk(0);
            load_c(v);
        }
        const int sgA = kSlab / 32 - 1;   // last s-block of slab A
        for (int c = 0; c < nchunks; ++c) {
            const MLayout Lc = lay(c);
            set_chunk(c);
            const MView<DT, PG> vc = v;
            const bool more = c + 1 < nchunks;
            if (more)
                set_chunk(c + 1);
            const int lo = max(32 * tau, vc.nb), hi = min(32 * tau + 32, vc.n_valid);
            const bool out = tau >= 0 && lo < hi && !(RP && a.no_y);
            f32x16 acc[P / 32];
            // t-block 3 (four s-blocks, outputs and C loads, all in phase 1) is
            // the longest path of phase 1: its wave goes first on its SIMD
            // until the phase barrier
            if (two && tau == sgA)
                __builtin_amdgcn_s_setprio(1);
            // s-blocks of slab A (all of them with one slab)
            if (out)
                tblock_part<P, N, 0, P / 32>(tau, 0, two ? min(tau, sgA) : tau, cf, lds, Lc, acc);
            if (!two || tau <= sgA) {
                if (out)
                    emit_tblock<P, 0, P / 32>(vc, tau, lo, hi, D_h, lds, Lc, acc, y);
                if (tau >= 0 && more)
                    load_c(v);
            }
            if (two) {
                if (tau == sgA)
                    __builtin_amdgcn_s_setprio(0);
                __syncthreads();   // phase 2: slab B is in
                if (tau > sgA) {
                    if (out) {
                        tblock_part<P, N, 0, P / 32>(tau, sgA + 1, tau, cf, lds, Lc, acc);
                        emit_tblock<P, 0, P / 32>(vc, tau, lo, hi, D_h, lds, Lc, acc, y);
                    }
                    if (more)
                        load_c(v);
                }
            }
            // the next chunk's per-row arrays (the scalar wave has no phase-2
            // t-block work, so the dt load's latency is not in its way)
            if (wave == (two ? kStateWaves + 3 : kStateWaves + 7) && more) {
                TD rawdt[4];
                load_dt<DT>(v, rawdt);
                chunk_scalars_wave<DT>(rawdt, v.n_valid, A2_h, bias, d.softplus, lds,
                                       L.buf((c + 1) & 1));
            }
            __syncthreads();   // end of chunk c
        }
    }
}

// One workgroup per (sequence, head).
template <int P, int N, class DT, bool PG, bool RP>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void k_scan_mfma(ScanArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int wid = xcd_local_index(blockIdx.x, gridDim.x);
    if (a.psplit == 2) {
        // both halves of a head's columns next to each other
        const int hp = wid % (2 * a.d.H);
        scan_one<P, N, DT, PG, RP>(a, wid / (2 * a.d.H), hp >> 1, lds, hp & 1);
    } else {
        scan_one<P, N, DT, PG, RP>(a, wid / a.d.H, wid % a.d.H, lds);
    }
}

// The work array after the per-slot arrival counters: [0] number of entries
// on the list, [1] finished groups, [2, 2 + kDoneGroups) finished
// workgroups per group, then the list itself (slots whose chunk-state update
// is pending, a decode batch's ranking, or the sequences a sweep replays).
// Every call leaves it zero.
constexpr int kDoneGroups = 32;
constexpr int kListHead = 2 + kDoneGroups;

// End of a launch that read the list: every workgroup counts itself out (in
// kDoneGroups groups by blockIdx, then once per group, so that no counter
// takes many atomics); the last one zeroes entries [0, nclear) of the list,
// and its count when `count` is set. Every workgroup has read what it needs
// from the list before counting out.
__device__ __forceinline__ void work_list_done(int32_t *list, int nclear, bool count) {
    __shared__ int is_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        int last = 0;
        const int W = gridDim.x;
        const int grp = blockIdx.x % kDoneGroups;
        const int members = (W - grp + kDoneGroups - 1) / kDoneGroups;
        int32_t *sub = list + 2 + grp;
        if (__hip_atomic_fetch_add(sub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            members - 1) {
            __hip_atomic_store(sub, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int groups = W < kDoneGroups ? W : kDoneGroups;
            if (__hip_atomic_fetch_add(list + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                groups - 1) {
                __hip_atomic_store(list + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last = 1;
            }
        }
        is_last = last;
    }
    __syncthreads();
    if (is_last) {
        for (int i = threadIdx.x; i < nclear; i += blockDim.x)
            list[kListHead + i] = 0;
        if (count && threadIdx.x == 0)
            list[0] = 0;
    }
}

// Whether sequence s has work in a sweep: drafts that run past the chunk end
// (verification), or accepted drafts that fill the chunk (acceptance).
__device__ __forceinline__ bool sweep_has_work(const ScanArgs &a, int s) {
    const int slot = a.slot_idx ? a.slot_idx[s] : s;
    const int len = seq_len(a.cu, a.take, s);
    if (len <= 0 || slot < 0 || slot >= a.num_slots)
        return false;
    const int k = a.buf_len[slot];
    return k >= 0 && k < a.d.Q && (a.no_y ? k + len >= a.d.Q : k + len > a.d.Q);
}

// The acceptance sweep's list: the sequences whose accepted drafts fill the
// chunk (one workgroup; list order does not matter).
__global__ __launch_bounds__(1024) void k_sweep_list(ScanArgs a) {
    int32_t *list = a.work + a.num_slots;
    for (int s = threadIdx.x; s < a.S; s += blockDim.x)
        if (sweep_has_work(a, s))
            list[kListHead + atomicAdd(list, 1)] = s;
}

// Replay calls where few sequences have work: verification of drafts that
// run past the chunk end (dry replay, only_cross), and acceptance (no_y),
// where only the sequences whose accepted drafts fill a chunk have any.
// One round of workgroups (at most one per compute unit), so the pairs with
// nothing to do cost no dispatch of a large-LDS workgroup.
// The sequences come from the list that the verification kernel or
// k_sweep_list put in the work array: the pairs (listed sequence, head) are
// dealt to the workgroups in turn, so no workgroup has more than one pair
// more than another, and the last workgroup empties the list.
template <int P, int N, class DT, bool PG>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void k_scan_cross(ScanArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int H = a.d.H;
    int32_t *wl = a.work + a.num_slots;
    const int n = wl[0];
    for (int j = blockIdx.x; j < n * H; j += gridDim.x) {
        const int s = wl[kListHead + j / H];
        __syncthreads();   // the previous pair's LDS use is over
        scan_one<P, N, DT, PG, true>(a, s, j % H, lds);
    }
    work_list_done(wl, n, true);
}

// ---------------------------------------------------------------------------
// Exact-replay decode. A workgroup of kDecodeWaves waves serves that many
// heads of one slot, one wave per head. Each wave computes the single output
// row k = buf_len of the t-block holding it, with the prefill's operands and
// MFMA order:
//   - the read-out operand S_bf comes from the cache's bf16 state copy, the
//     rounding the prefill applies to the same fp32 state;
//   - C . B^T and the weights are built for column k % 32 only (the other
//     columns of C are zero and their weights are selected to zero): an MFMA
//     output element depends only on its own row and column;
//   - when the workgroup's heads share a B/C group, each wave computes C . B^T
//     for a quarter of the s-blocks and hands column k % 32 over in LDS;
//   - the X rows of each s-block pass through a small per-wave LDS tile for
//     the transposed read (rows after k are zero), loaded one block ahead;
//   - the in-chunk scan is the prefill's block scan, one 64-row segment at a
//     time (wave_scan_segments).
// The last workgroup of a slot to arrive advances buf_len / boundary_pos
// (per-slot arrival counter). When the token filled the chunk, the
// chunk-state update with the prefill's own chunk arithmetic follows in the
// same kernel (FUSED, each wave its head: decode_commit). A batch with more
// workgroups than run at once is ranked first (k_decode_order: filling
// slots, then the longest buffers), and its workgroups are dispatched in
// rank order, so the heaviest start first rather than forming the launch's
// tail. Only a batch longer than the slot count (positions outside the slot
// range) takes the unfused form, where the last workgroup puts the slot on a
// list and a second kernel (k_decode_commit) updates the listed slots.
constexpr int kDecodeWaves = 4;

// Workgroups of the chunk-commit kernel: as many as fit on the device at
// once (compute units x workgroups per unit that the LDS allows, at most 4)
// and at most one per (sequence, head) of the batch, each handling one head
// of a full chunk at a time; when no chunk filled they return at once, in
// one dispatch round.
constexpr int kLdsBytesPerCu = 160 * 1024;

// Per-wave LDS of the decode kernel, in bytes.
struct DLayout {
    int XS, cXS, cBS;
    int lam, u, beta, gc, X, cX, cB, w, bytes;
    __host__ __device__ DLayout(int Qp, int P, int N, bool fused) {
        XS = P + kPad;
        int o = 0;
        lam = o;  o += Qp * 4;
        u = o;    o += Qp * 4;
        beta = o; o += Qp * 4;
        gc = o;   o += (kMaxQ / 32) * 32 * 4;   // C.B^T column k % 32 per s-block
        X = o;    o += 32 * XS * 2;              // padded 32-row x tile
        // with the chunk-state update in the same launch: its 32-row blocks
        // (x: the 32 columns of two p-slabs, B: all N) over the arrays above
        // once the output is written, and the state weights of the
        // chunk-filling step
        cXS = 32 + kPad;
        cBS = N + kPad;
        cX = 0;
        cB = cX + 32 * cXS * 2;
        w = o;
        if (fused) {
            const int cend = cB + 32 * cBS * 2;
            o = o > cend ? o : cend;
            w = o;
            o += Qp * 4;
        }
        bytes = (o + 15) & ~15;
    }
};

// Registers a decode wave carries from the first phase to the second.
template <int P, class DT>
struct DecodeCarry {
    f32x16 acc[P / 32];          // read-out, scaled: the Y^T accumulators
    float lam_k;
    uint4 xa[P / 16], xb[P / 16];   // x tiles of s-blocks 0 and 1 (in flight)
};

// Rows 32 sg .. +31 of the head's x (buffer below k, the token at k; rows
// after k are loaded from the token and zeroed when stored), as 16-byte
// pieces lane + 64 i of the row-major tile.
template <int P, bool PG>
__device__ __forceinline__ void load_x_tile(const uint16_t *bx, const SlotRows<PG> &rows,
                                            const uint16_t *xin, int H, int h, int k, int sg,
                                            uint4 (&xr)[P / 16]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < P / 16; ++i) {
        const int e = lane + 64 * i, r = e / (P / 8), q = e % (P / 8);
        const int row = 32 * sg + r;
        const int64_t br = rows(row);
        const uint16_t *src = row < k ? bx + (br * H + h) * P : xin;
        xr[i] = *reinterpret_cast<const uint4 *>(src + 8 * q);
    }
}

// Phase 1: the wave's loads, the read-out, the append of the token, the
// in-chunk scan and the C.B^T columns of the s-blocks this wave owns.
template <int P, int N, class DT, bool PG, bool FUSED>
__device__ __forceinline__ void decode_front(const DecodeArgs &a, const SlotRows<PG> &rows, int b,
                                             int slot, int h, int k, int wave, bool gshare,
                                             char *lds, const DLayout &L, DecodeCarry<P, DT> &cy) {
    using TD = typename DT::T;
    constexpr int NPT = P / 32, NK = N / 16;
    const Dims d = a.d;
    const int H = d.H, G = d.G, Q = d.Q;
    const int Qp = Q < 32 ? 32 : Q;
    const int g = h / (H / G);
    const int lane = threadIdx.x & 63, gl = lane >> 5, c = lane & 31;
    const int tau = k >> 5;
    const bool col = c == (k & 31);   // lanes of output column k % 32
    const int64_t PN = (int64_t)P * N;
    const uint16_t *sbf = static_cast<const uint16_t *>(a.cache_state_bf) +
                          ((int64_t)slot * H + h) * PN;
    const uint16_t *xin = static_cast<const uint16_t *>(a.x) + ((int64_t)b * H + h) * P;
    const uint16_t *Bin = static_cast<const uint16_t *>(a.B) + ((int64_t)b * G + g) * N;
    const uint16_t *Cin = static_cast<const uint16_t *>(a.C) + ((int64_t)b * G + g) * N;
    const TD *dtin = static_cast<const TD *>(a.dt) + (int64_t)b * H + h;
    // buffer arrays (whole pool); position j is row rows(j)
    const uint16_t *bB = static_cast<const uint16_t *>(a.buf_B);
    const TD *bdt = static_cast<const TD *>(a.buf_dt);
    // s-blocks whose C.B^T column this wave computes
    const int sg0 = gshare ? wave : 0, sgs = gshare ? kDecodeWaves : 1;

    // every load that does not depend on earlier results goes out first
    const float A2 = a.A[h] * kLog2e;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    TD rawdt[4];   // raw dt of rows lane + 64 i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        const int64_t br = rows(j);
        rawdt[i] = j < k ? bdt[br * H + h] : dtin[0];
    }
    uint4 xtok = make_uint4(0, 0, 0, 0), btok = make_uint4(0, 0, 0, 0);
    if (lane < P / 8)
        xtok = *reinterpret_cast<const uint4 *>(xin + 8 * lane);
    if (lane < N / 8)
        btok = *reinterpret_cast<const uint4 *>(Bin + 8 * lane);
    bf16x8 cf[NK];
    {
        uint4 raw[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            raw[kk] = *reinterpret_cast<const uint4 *>(Cin + 16 * kk + 8 * gl);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            cf[kk] = __builtin_bit_cast(bf16x8, keep_if(col, raw[kk]));
    }
    auto load_brows = [&](int sg, uint4 (&br)[NK]) {
        const int s = 32 * sg + c;
        const int64_t rs = rows(s);
        const uint16_t *brow = s < k ? bB + (rs * G + g) * N : Bin;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            br[kk] = *reinterpret_cast<const uint4 *>(brow + 16 * kk + 8 * gl);
    };
    // read-out C . S_bf (operand (pt, kk) is 1 KiB contiguous in the copy);
    // all operand loads are in flight before the first MFMA waits on one
    bf16x8 sa[NPT][NK];
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            sa[pt][kk] = *reinterpret_cast<const bf16x8 *>(
                sbf + ((int64_t)kk * P + 32 * pt + c) * 16 + 8 * gl);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
        cy.acc[pt] = readout_raw<N>([&](int kk) { return sa[pt][kk]; }, cf);

    // append the token at buffer position k now: this step reads only
    // positions < k of the buffer (the token itself comes from the input)
    {
        const int64_t rk = rows(k);
        uint16_t *bx = static_cast<uint16_t *>(a.buf_x);
        uint16_t *bBw = static_cast<uint16_t *>(a.buf_B);
        TD *bdtw = static_cast<TD *>(a.buf_dt);
        if (lane < P / 8)
            *reinterpret_cast<uint4 *>(bx + (rk * H + h) * P + 8 * lane) = xtok;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == k)
                bdtw[rk * H + h] = rawdt[i];
        if (h % (H / G) == 0 && lane < N / 8) {
            *reinterpret_cast<uint4 *>(bBw + (rk * G + g) * N + 8 * lane) = btok;
            if (a.buf_C) {
                uint16_t *bC = static_cast<uint16_t *>(a.buf_C);
                *reinterpret_cast<uint4 *>(bC + (rk * G + g) * N + 8 * lane) =
                    *reinterpret_cast<const uint4 *>(Cin + 8 * lane);
            }
        }
    }

    // B rows of the first owned s-block and the first two x tiles (in flight
    // during the scan)
    uint4 braw[NK];
    if (sg0 <= tau)
        load_brows(sg0, braw);
    {
        const uint16_t *bxr = static_cast<const uint16_t *>(a.buf_x);
        load_x_tile<P>(bxr, rows, xin, H, h, k, 0, cy.xa);
        if (tau >= 1)
            load_x_tile<P>(bxr, rows, xin, H, h, k, 1, cy.xb);
    }

    // delta and the in-chunk cumulative sum (log2 units) over rows j = lane + 64 i
    const int nseg = (32 * (tau + 1) + 63) >> 6;
    float dv[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        float dd = 0.0f, aa = 0.0f;
        if (i < nseg && j <= k) {
            dd = delta_of(DT::val(rawdt[i]), bias, d.softplus);
            aa = dd * A2;
        }
        dv[i] = dd;
        lv[i] = aa;
    }
    wave_scan_segments(lv, nseg);
    float *lam = reinterpret_cast<float *>(lds + L.lam);
    float *uu = reinterpret_cast<float *>(lds + L.u);
    float *bt = reinterpret_cast<float *>(lds + L.beta);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        const float lend = __shfl(lv[i], lane | 31, 64);   // lam[j | 31]
        if (i < nseg && j < Qp) {
            const float l = lv[i];
            const float u = l - flog2(dv[i]);  // +inf where delta is 0
            lam[j] = l;
            uu[j] = u;
            bt[j] = fexp2(lend - u);
        }
    }
    cy.lam_k = lam[k];
    if (FUSED && k + 1 == Q) {
        // the token fills the chunk: state weights 2^(lam_last - lam_j) delta_j
        // for the chunk-state update (zero past row k)
        float *w = reinterpret_cast<float *>(lds + L.w);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = lane + 64 * i;
            if (i < nseg && j < Qp)
                w[j] = fexp2(cy.lam_k - lv[i]) * dv[i];
        }
    }
    const float el_k = fexp2(cy.lam_k);
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
        cy.acc[pt] = readout_scale(cy.acc[pt], el_k);

    // C.B^T of the owned s-blocks; column k % 32 to LDS
    float *gcol = reinterpret_cast<float *>(lds + L.gc);
    for (int sg = sg0; sg <= tau; sg += sgs) {
        const bool more = sg + sgs <= tau;
        const bool srow = 32 * sg + c <= k;   // rows after k are zero
        const f32x16 gt = gram_block<N>(
            [&](int kk) { return __builtin_bit_cast(bf16x8, keep_if(srow, braw[kk])); }, cf);
        if (col) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4 *>(gcol + 32 * sg + 8 * q + 4 * gl) =
                    make_float4(gt[4 * q], gt[4 * q + 1], gt[4 * q + 2], gt[4 * q + 3]);
        }
        if (more)
            load_brows(sg + sgs, braw);
    }
}

// Phase 2: weights and M.X over the s-blocks, and the output row.
template <int P, int N, class DT, bool PG>
__device__ __forceinline__ void decode_back(const DecodeArgs &a, const SlotRows<PG> &rows, int b,
                                            int h, int k, int wave, bool gshare, char *lds_all,
                                            const DLayout &L, DecodeCarry<P, DT> &cy) {
    constexpr int NPT = P / 32;
    const Dims d = a.d;
    const int H = d.H;
    const int lane = threadIdx.x & 63, gl = lane >> 5, c = lane & 31;
    const int tau = k >> 5;
    const bool col = c == (k & 31);
    char *lds = lds_all + wave * L.bytes;
    const uint16_t *xin = static_cast<const uint16_t *>(a.x) + ((int64_t)b * H + h) * P;
    const uint16_t *bx = static_cast<const uint16_t *>(a.buf_x);   // whole pool
    const float *lam = reinterpret_cast<const float *>(lds + L.lam);
    const float *uu = reinterpret_cast<const float *>(lds + L.u);
    const float *bt = reinterpret_cast<const float *>(lds + L.beta);

    // x tile of each s-block: 32 rows x P through registers into the padded
    // LDS tile, the next two blocks' rows in flight during this block's work
    // (tiles 0 and 1 were issued in phase 1)
    constexpr int XPL = P / 16;  // 16-byte pieces of a tile per lane
    uint4 (&xa)[XPL] = cy.xa;
    uint4 (&xb)[XPL] = cy.xb;
    for (int sg = 0; sg <= tau; ++sg) {
        // C.B^T column of this s-block, back in the MFMA output layout
        const int owner = gshare ? sg % kDecodeWaves : wave;
        const float *gcol = reinterpret_cast<const float *>(lds_all + owner * L.bytes + L.gc);
        f32x16 gt;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(gcol + 32 * sg + 8 * q + 4 * gl);
            gt[4 * q] = v.x;
            gt[4 * q + 1] = v.y;
            gt[4 * q + 2] = v.z;
            gt[4 * q + 3] = v.w;
        }
        uint32_t mb[8];
        if (sg == tau)
            m_diag(gt, cy.lam_k, uu, 32 * sg, k, mb, lane);
        else
            m_off(gt, fexp2(cy.lam_k - lam[32 * sg + 31]), bt, 32 * sg, mb, lane);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            mb[q] = col ? mb[q] : 0u;
#pragma unroll
        for (int i = 0; i < XPL; ++i) {
            const int e = lane + 64 * i, r = e / (P / 8), q = e % (P / 8);
            *reinterpret_cast<uint4 *>(lds + L.X + (r * L.XS + 8 * q) * 2) =
                keep_if(32 * sg + r <= k, xa[i]);   // rows after k are zero
        }
        if (sg + 1 <= tau) {
#pragma unroll
            for (int i = 0; i < XPL; ++i)
                xa[i] = xb[i];
        }
        if (sg + 2 <= tau)
            load_x_tile<P>(bx, rows, xin, H, h, k, sg + 2, xb);
        mx_accumulate<0, NPT>(mb, lds, L.X, L.XS, 0, cy.acc, lane);
    }

    // y row k: fmaf(D, x, Y^T) -> bf16, -0 -> +0 (lanes of column k % 32);
    // x_k is row k - 32 tau of the last x tile
    if (col) {
        const float D_h = a.D ? a.D[h] : 0.0f;
        uint16_t *yrow = static_cast<uint16_t *>(a.y) + ((int64_t)b * H + h) * P;
        const char *xk = lds + L.X + (k - 32 * tau) * L.XS * 2;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = 32 * pt + 8 * q + 4 * gl;
                const uint2 xv = *reinterpret_cast<const uint2 *>(xk + 2 * p);
                const float xs[4] = {bf16_float(xv.x & 0xffff), bf16_float(xv.x >> 16),
                                     bf16_float(xv.y & 0xffff), bf16_float(xv.y >> 16)};
                uint16_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float yv = fmaf(D_h, xs[e], cy.acc[pt][4 * q + e]);
                    yv = yv + 0.0f;
                    o[e] = bf16_bits(yv);
                }
                *reinterpret_cast<uint2 *>(yrow + p) =
                    make_uint2(o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16));
            }
        }
    }
}

// Phase 3, only when the token fills the chunk: the chunk-state update of
// the wave's head, S <- 2^lam_last S + sum_j B_j (w_j x_j), with the
// prefill's tile arithmetic (state_kstep: K = 32 rows per step, hi then lo),
// so the new boundary state has the bits a prefill of the same tokens
// leaves. The weights w_j were put in LDS by phase 1. The head's p-slabs are
// taken two at a time (all n-tiles of both live); per step, rows
// 32 kk .. +31 of x (the two slabs' 32 columns) and of B (all N) pass
// through LDS for the transposed reads, the next step's rows in flight
// during this step's MFMAs; rows below k come from the slot buffer, row k
// from the step's input (the buffer row written by this step is not read
// back), rows after k are zero.
template <int P, int N, class DT, bool PG>
__device__ __forceinline__ void decode_commit(const DecodeArgs &a, const SlotRows<PG> &rows, int b,
                                              int slot, int h, int k, char *lds, const DLayout &L,
                                              float lam_last) {
    constexpr int NPS = P / 16, NT = N / 16;
    constexpr int SP = 2;         // p-slabs per pass
    static_assert(NPS % SP == 0, "slab pairs");
    constexpr int BPL = N / 16;   // 16-byte pieces of a 32-row B block per lane
    constexpr int XPL = 32 * 16 * SP / 8 / 64;   // ... of a 32-row x block (SP slabs)
    const Dims d = a.d;
    const int H = d.H, G = d.G, Q = d.Q;
    const int Qp = Q < 32 ? 32 : Q;
    const int g = h / (H / G);
    const int64_t PN = (int64_t)P * N;
    const uint16_t *bx = static_cast<const uint16_t *>(a.buf_x);   // whole pools
    const uint16_t *bB = static_cast<const uint16_t *>(a.buf_B);
    const uint16_t *xin = static_cast<const uint16_t *>(a.x) + ((int64_t)b * H + h) * P;
    const uint16_t *Bin = static_cast<const uint16_t *>(a.B) + ((int64_t)b * G + g) * N;
    float *st = a.cache_state + ((int64_t)slot * H + h) * PN;
    uint16_t *sbf = static_cast<uint16_t *>(a.cache_state_bf) + ((int64_t)slot * H + h) * PN;
    const float *w = reinterpret_cast<const float *>(lds + L.w);
    const float dec = fexp2(lam_last);
    const int nkk = Qp / 32;

    // x piece i of lane: row e / (2 SP), 8 columns from 16 p0 + 8 (e % (2 SP))
    auto load_block = [&](int p0, int kk, uint4 (&xr)[XPL], uint4 (&br)[BPL]) {
        const int lane = lane_id();
#pragma unroll
        for (int i = 0; i < XPL; ++i) {
            const int e = lane + 64 * i, j = 32 * kk + e / (2 * SP);
            const int64_t rj = rows(j < k ? j : 0);
            const uint16_t *src = j < k ? bx + (rj * H + h) * P : xin;
            xr[i] = *reinterpret_cast<const uint4 *>(src + 16 * p0 + 8 * (e % (2 * SP)));
        }
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            const int e = lane + 64 * i, j = 32 * kk + e / (N / 8);
            const int64_t rj = rows(j < k ? j : 0);
            const uint16_t *src = j < k ? bB + (rj * G + g) * N : Bin;
            br[i] = *reinterpret_cast<const uint4 *>(src + 8 * (e % (N / 8)));
        }
    };
    auto store_block = [&](int kk, const uint4 (&xr)[XPL], const uint4 (&br)[BPL]) {
        const int lane = lane_id();
#pragma unroll
        for (int i = 0; i < XPL; ++i) {
            const int e = lane + 64 * i, r = e / (2 * SP);
            *reinterpret_cast<uint4 *>(lds + L.cX + (r * L.cXS + 8 * (e % (2 * SP))) * 2) =
                keep_if(32 * kk + r <= k, xr[i]);
        }
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            const int e = lane + 64 * i, r = e / (N / 8);
            *reinterpret_cast<uint4 *>(lds + L.cB + (r * L.cBS + 8 * (e % (N / 8))) * 2) =
                keep_if(32 * kk + r <= k, br[i]);
        }
    };

#pragma unroll 1
    for (int p0 = 0; p0 < NPS; p0 += SP) {
        uint4 xa[XPL], ba[BPL];
        load_block(p0, 0, xa, ba);
        // the slabs' old tiles, decayed to the chunk end
        f32x4 acc[SP][NT];
#pragma unroll
        for (int q = 0; q < SP; ++q) {
            slab_io<P, N, NT, true>(st, p0 + q, 0, acc[q]);
            slab_scale<NT>(acc[q], dec);
        }
        for (int kk = 0; kk < nkk; ++kk) {
            store_block(kk, xa, ba);
            if (kk + 1 < nkk)
                load_block(p0, kk + 1, xa, ba);
#pragma unroll
            for (int q = 0; q < SP; ++q)
                state_kstep<NT>(lds, L.cX, L.cXS, 16 * q, L.cB, L.cBS, 0, 0, w + 32 * kk, acc[q]);
        }
        // the new tiles of the fp32 state and of its bf16 copy
#pragma unroll
        for (int q = 0; q < SP; ++q) {
            slab_io<P, N, NT, false>(st, p0 + q, 0, acc[q]);
            slab_bf16<P, NT>(acc[q], p0 + q, 0, lds, -1, 0, sbf);
        }
    }
}

// The conv before the scan, for one workgroup's part of a decode step with
// the conv in the same launch (xBC non-null): the x channels of heads
// h0 .. h0 + kDecodeWaves - 1 and the B | C channels of their group g, one
// channel per thread, from the slot's conv state (the W - 1 previous
// inputs) and the token's xBC row, with the conv's own conv_point; the
// outputs go to the step's input rows x[b], B[b], C[b] (bf16, nearest
// even), and the x channels' state, which this workgroup alone reads, is
// shifted in place. The B | C channels are read by every workgroup of the
// slot; the slot's last workgroup shifts them (conv_shift_bc).
template <int P, int N, int W>
__device__ __forceinline__ void conv_token(const DecodeArgs &a, int b, int slot, int h0, int g) {
    const int H = a.d.H, G = a.d.G;
    const int cd = H * P + 2 * G * N;
    const int t = threadIdx.x;
    const uint16_t *in = static_cast<const uint16_t *>(a.xBC) + (int64_t)b * cd;
    uint16_t *st = static_cast<uint16_t *>(a.cstate) + (int64_t)slot * cd * (W - 1);
    auto point = [&](int c, uint16_t (&raw)[W]) {
        float v[W], w[W];
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
            raw[i] = st[(int64_t)c * (W - 1) + i];
        raw[W - 1] = in[c];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            v[i] = IoBF16::val(raw[i]);
            w[i] = a.cw[(int64_t)c * W + i];
        }
        return IoBF16::cvt(conv_point<W>(w, v, a.cb ? a.cb[c] : 0.0f, a.cact != 0));
    };
    if (t < kDecodeWaves * P && h0 + t / P < H) {
        const int c = (h0 + t / P) * P + t % P;
        uint16_t raw[W];
        const uint16_t o = point(c, raw);
        static_cast<uint16_t *>(const_cast<void *>(a.x))[(int64_t)b * H * P + c] = o;
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
            st[(int64_t)c * (W - 1) + i] = raw[i + 1];
    }
    if (t < 2 * N) {
        const bool isB = t < N;
        const int n = isB ? t : t - N;
        const int c = H * P + (isB ? 0 : G * N) + g * N + n;
        uint16_t raw[W];
        const uint16_t o = point(c, raw);
        uint16_t *dst = static_cast<uint16_t *>(const_cast<void *>(isB ? a.B : a.C));
        dst[((int64_t)b * G + g) * N + n] = o;
    }
}

// The slot's B | C conv state (every group's 2N channels) shifted by one
// input, by one wave of the slot's last workgroup.
template <int P, int N, int W>
__device__ __forceinline__ void conv_shift_bc(const DecodeArgs &a, int b, int slot) {
    const int H = a.d.H, G = a.d.G;
    const int cd = H * P + 2 * G * N;
    const uint16_t *in = static_cast<const uint16_t *>(a.xBC) + (int64_t)b * cd;
    uint16_t *st = static_cast<uint16_t *>(a.cstate) + (int64_t)slot * cd * (W - 1);
    for (int c = H * P + (threadIdx.x & 63); c < cd; c += 64) {
        uint16_t raw[W];
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
            raw[i] = st[(int64_t)c * (W - 1) + i];
        raw[W - 1] = in[c];
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
            st[(int64_t)c * (W - 1) + i] = raw[i + 1];
    }
}

template <int P, int N>
__device__ __forceinline__ void conv_token_w(const DecodeArgs &a, int b, int slot, int h0, int g) {
    switch (a.cW) {
    case 2: conv_token<P, N, 2>(a, b, slot, h0, g); break;
    case 3: conv_token<P, N, 3>(a, b, slot, h0, g); break;
    default: conv_token<P, N, 4>(a, b, slot, h0, g); break;
    }
}

template <int P, int N>
__device__ __forceinline__ void conv_shift_bc_w(const DecodeArgs &a, int b, int slot) {
    switch (a.cW) {
    case 2: conv_shift_bc<P, N, 2>(a, b, slot); break;
    case 3: conv_shift_bc<P, N, 3>(a, b, slot); break;
    default: conv_shift_bc<P, N, 4>(a, b, slot); break;
    }
}

// Ranking of a large batch before its decode launch: batch positions whose
// token fills the chunk first (their workgroups also run the chunk-state
// update), then by the number of 32-row s-blocks the replay walks, most
// first; positions the decode skips last. A counting sort in one workgroup;
// positions of one bin in any order (what a workgroup computes does not
// depend on when it runs). The ranking goes to the commit-list area of the
// work array (batch <= num_slots entries), which the decode launch then
// reads and leaves zero.
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void k_decode_order(DecodeArgs a) {
    constexpr int kBins = kMaxQ / 32 + 2;
    constexpr int kHeld = 4;   // positions per thread whose bins stay in registers
    __shared__ int count[kBins];
    const int Q = a.d.Q;
    int32_t *order = a.work + a.num_slots + kListHead;
    auto bin_of = [&](int b) {
        const int slot = a.slot_idx ? a.slot_idx[b] : b;
        if (slot < 0 || slot >= a.num_slots)
            return kBins - 1;
        const int k = a.buf_len[slot];
        if (k < 0 || k >= Q)
            return kBins - 1;
        return k + 1 == Q ? 0 : kMaxQ / 32 - (k >> 5);
    };
    if (threadIdx.x < kBins)
        count[threadIdx.x] = 0;
    int held[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i) {
        const int b = threadIdx.x + kOrderThreads * i;
        held[i] = b < a.batch ? bin_of(b) : -1;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kHeld; ++i)
        if (held[i] >= 0)
            atomicAdd(&count[held[i]], 1);
    for (int b = threadIdx.x + kOrderThreads * kHeld; b < a.batch; b += kOrderThreads)
        atomicAdd(&count[bin_of(b)], 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        int at = 0;
        for (int i = 0; i < kBins; ++i) {
            const int n = count[i];
            count[i] = at;   // first rank of bin i
            at += n;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kHeld; ++i)
        if (held[i] >= 0)
            order[atomicAdd(&count[held[i]], 1)] = threadIdx.x + kOrderThreads * i;
    for (int b = threadIdx.x + kOrderThreads * kHeld; b < a.batch; b += kOrderThreads)
        order[atomicAdd(&count[bin_of(b)], 1)] = b;
}

// End of a ranked decode launch: the last workgroup zeroes the ranking.
__device__ __forceinline__ void decode_order_done(const DecodeArgs &a) {
    work_list_done(a.work + a.num_slots, a.batch, false);
}

template <int P, int N, class DT, bool PG, bool FUSED>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(3, 3)))
void k_decode_mfma(DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds_all[];
    const int H = a.d.H, G = a.d.G, Q = a.d.Q;
    const int Qp = Q < 32 ? 32 : Q;
    const int HQ = (H + kDecodeWaves - 1) / kDecodeWaves;
    // Workgroup -> (rank r, head quarter hq). Without a ranking, rank r is
    // batch position r and the workgroups are renumbered so that those of
    // one slot run on one XCD (they share its B rows). With one, they are
    // taken in dispatch order: workgroup i runs on XCD i % 8 as that XCD's
    // (i / 8)-th, so each XCD takes every eighth rank, in rank order, with a
    // rank's workgroups together (rank i / HQ when the batch is not a
    // multiple of 8).
    int r, hq;
    if (!a.order) {
        const int wid = xcd_local_index(blockIdx.x, gridDim.x);
        r = wid / HQ;
        hq = wid % HQ;
    } else if (a.batch % 8 == 0) {
        const int j = blockIdx.x / 8;
        r = (j / HQ) * 8 + blockIdx.x % 8;
        hq = j % HQ;
    } else {
        r = blockIdx.x / HQ;
        hq = blockIdx.x % HQ;
    }
    const int b = a.order ? a.order[r] : r;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int h = hq * kDecodeWaves + wave;
    const DLayout L(Qp, P, N, FUSED);
    // nothing is done for a position outside the batch, or a slot, buffer
    // length or page entry out of range (the same for the whole workgroup);
    // a ranked launch still counts the workgroup out
    const int slot = b < 0 || b >= a.batch ? -1 : a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0 || slot >= a.num_slots) {
        if (a.order)
            decode_order_done(a);
        return;
    }
    const int k = a.buf_len[slot];
    if (k < 0 || k >= Q) {
        if (a.order)
            decode_order_done(a);
        return;
    }
    // positions 0..k of the buffer are read or written
    const SlotRows<PG> rows(a.bm, slot, Q);
    if (!rows.ok(a.bm, k + 1)) {
        if (a.order)
            decode_order_done(a);
        return;
    }
    // the workgroup's heads share one B/C group: C.B^T is split between them
    const bool gshare = (H / G) % kDecodeWaves == 0;
    if (a.xBC) {
        // the token's x | B | C from the conv before the scan (the host
        // takes this path only when the workgroup's heads share one group)
        conv_token_w<P, N>(a, b, slot, hq * kDecodeWaves, (hq * kDecodeWaves) / (H / G));
        __syncthreads();   // the conv outputs are the step's inputs
    }
    DecodeCarry<P, DT> cy;
    if (h < H)
        decode_front<P, N, DT, PG, FUSED>(a, rows, b, slot, h, k, wave, gshare,
                                          lds_all + wave * L.bytes, L, cy);
    __syncthreads();  // C.B^T columns of every wave are in LDS
    // Every wave of this workgroup has read buf_len (and used it) by now,
    // so the workgroup counts itself in; the slot's last workgroup to
    // arrive advances buf_len when it is done. The counter needs only
    // atomicity, no ordering: no workgroup reads what the last one writes
    // during this launch, and the launch boundary publishes the writes.
    // (An acquire/release atomic here would write back and invalidate the
    // L2 in every workgroup.)
    int prev = 0;
    if (threadIdx.x == 0)
        prev = __hip_atomic_fetch_add(a.work + slot, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    if (h < H)
        decode_back<P, N, DT>(a, rows, b, h, k, wave, gshare, lds_all, L, cy);
    if (FUSED && k + 1 == Q) {
        __syncthreads();  // every wave is done with the C.B^T columns in LDS
        if (h < H)
            decode_commit<P, N, DT>(a, rows, b, slot, h, k, lds_all + wave * L.bytes, L,
                                    cy.lam_k);
    }
    if (threadIdx.x == 0 && prev == HQ - 1) {
        __hip_atomic_store(a.work + slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.buf_len[slot] = k + 1 == Q ? 0 : k + 1;
        if (k + 1 == Q) {
            a.boundary_pos[slot] += Q;
        }
        if (!FUSED && k + 1 == Q) {
            // the chunk is full: its state update runs in k_decode_commit
            int32_t *list = a.work + a.num_slots;
            const int at = __hip_atomic_fetch_add(list, 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
            list[kListHead + at] = slot;
        }
    }
    // the slot's last workgroup: every workgroup of the slot has read the
    // B | C conv state (before counting itself in), so it can be shifted
    if (a.xBC && wave == 0 && __shfl(prev, 0, 64) == HQ - 1)
        conv_shift_bc_w<P, N>(a, b, slot);
    if (a.order)
        decode_order_done(a);
    (void)G;
}

// Chunk-state update of the slots whose chunk the decode step filled (the
// list k_decode_commit finds in the cache's work array): one head of one
// slot per workgroup at a time, with the prefill's chunk arithmetic (the
// per-row quantities of chunk_scalars, the state tiles of state_kstep with
// the prefill's four-wave split),
// on the chunk's Q tokens, all in the slot buffer now. Writes the new fp32
// boundary state and its bf16 copy. The last workgroup to finish empties the
// list.
constexpr int kCommitWaves = 4;

template <int P, int N, class DT, bool PG>
__global__ __launch_bounds__(64 * kCommitWaves) void k_decode_commit(DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    using TD = typename DT::T;
    static_assert(kCommitWaves == kStateWaves, "the commit's waves are the state tiles' owners");
    const Dims d = a.d;
    const int H = d.H, G = d.G, Q = d.Q;
    const int Qp = Q < 32 ? 32 : Q;
    const MLayout L(Qp, P, N);
    int32_t *list = a.work + a.num_slots;   // count, done counters, slots
    const int raw = list[0];
    if (raw == 0)
        return;
    // (a count outside [0, num_slots] means the work array was not zeroed:
    // nothing is processed and the counters are cleared)
    const int count = raw > 0 && raw <= a.num_slots ? raw : 0;
    if (count == 0) {
        if (blockIdx.x == 0 && threadIdx.x < kListHead)
            list[threadIdx.x] = 0;
        return;
    }
    const int64_t PN = (int64_t)P * N;
    for (int e = blockIdx.x; e < count * H; e += gridDim.x) {
        const int slot = list[kListHead + e / H], h = e % H, g = h / (H / G);
        if (slot < 0 || slot >= a.num_slots)
            continue;
        // (the decode step checked the same entries before listing the slot)
        const SlotRows<PG> rows(a.bm, slot, Q);
        if (!rows.ok(a.bm, Q))
            continue;
        const uint16_t *bx = static_cast<const uint16_t *>(a.buf_x);   // whole pool
        const uint16_t *bB = static_cast<const uint16_t *>(a.buf_B);
        const TD *bdt = static_cast<const TD *>(a.buf_dt);
        float *st = a.cache_state + ((int64_t)slot * H + h) * PN;
        using SL = Slab<P, N>;
        int ps, nt0;
        SL::own(threadIdx.x >> 6, ps, nt0);
        f32x4 S[SL::NT];
        slab_io<P, N, SL::NT, true>(st, ps, nt0, S);
        const int64_t rd = rows(threadIdx.x < Q ? threadIdx.x : 0);
        const float dt_raw = DT::ld(bdt, rd * H + h);
        __syncthreads();  // the previous entry's LDS reads are done
        stage_rows<P / 8, N / 8>(rows, bx + h * P, (int64_t)H * P, bB + g * N, (int64_t)G * N, Qp,
                                 Q, lds + L.X, L.XS, lds + L.B, L.BS);
        chunk_scalars(dt_raw, Q, a.A[h] * kLog2e, a.dt_bias ? a.dt_bias[h] : 0.0f, d.softplus,
                      true, lds, L);
        __syncthreads();
        slab_scale<SL::NT>(S, fexp2(reinterpret_cast<const float *>(lds + L.lam)[Q - 1]));
        for (int kk = 0; kk < Qp / 32; ++kk)
            state_kstep<SL::NT>(lds, L.X, L.XS, 16 * ps, L.B, L.BS, 32 * kk, nt0,
                                reinterpret_cast<const float *>(lds + L.w) + 32 * kk, S);
        slab_io<P, N, SL::NT, false>(st, ps, nt0, S);
        slab_bf16<P, SL::NT>(S, ps, nt0, lds, -1, 0,
                             static_cast<uint16_t *>(a.cache_state_bf) + ((int64_t)slot * H + h) * PN);
    }
    // The workgroups that had entries ([0, W)) count themselves out, in 32
    // groups (blockIdx % 32) and then once per group, so that no counter
    // takes many atomics; the last one empties the list. Workgroups past W
    // touch nothing (a late one may find the list already empty).
    const int W = count * H < (int)gridDim.x ? count * H : (int)gridDim.x;
    if (blockIdx.x >= W)
        return;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int grp = blockIdx.x % kDoneGroups;
        const int members = (W - grp + kDoneGroups - 1) / kDoneGroups;
        int32_t *sub = list + 2 + grp;
        if (__hip_atomic_fetch_add(sub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            members - 1) {
            __hip_atomic_store(sub, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int groups = W < kDoneGroups ? W : kDoneGroups;
            if (__hip_atomic_fetch_add(list + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                groups - 1) {
                for (int i = 0; i < count; ++i)
                    list[kListHead + i] = 0;
                __hip_atomic_store(list + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(list, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Speculative verification, many rows at once. A workgroup of kDecodeWaves
// waves serves that many heads of one sequence, one wave per head (no
// barriers: each wave has its own LDS). The wave computes the outputs of
// the sequence's T draft rows k .. k+T-1 of the chunk (k = buf_len), t-block
// by t-block, with the prefill's operands and MFMA order: the read-out from
// the cache's bf16 state copy, the same in-chunk scan (one wave emulating
// the block scan), C.B^T blocks, decay weights and X.M accumulation. An
// output row depends only on its own columns of C and M, so each draft's
// output has the bits decode would give it. Operands come from global
// memory: committed rows from the slot buffer, drafts from the inputs, rows
// after the last draft are zero. When the workgroup's heads share a B/C
// group, the C.B^T blocks are computed once per workgroup (each wave a
// quarter of the s-blocks) and read by all four from LDS; the workgroup then
// meets at two barriers per t-block. Nothing but y is written. Sequences whose
// drafts run past the chunk end are left to the prefill kernel's dry replay.
struct VLayout {
    int XS;
    int lam, u, beta, X, bytes;
    __host__ __device__ VLayout(int Qp, int P) {
        XS = P + kPad;
        int o = 0;
        lam = o;  o += Qp * 4;
        u = o;    o += Qp * 4;
        beta = o; o += Qp * 4;
        X = o;    o += 32 * XS * 2;
        bytes = (o + 15) & ~15;
    }
};

template <int P, int N, class DT, bool PG, bool GSHARE>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(GSHARE ? 3 : 1)))
void k_verify_mfma(ScanArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds_all[];
    using TD = typename DT::T;
    constexpr int NPT = P / 32, NK = N / 16;
    const Dims d = a.d;
    const int H = d.H, G = d.G, Q = d.Q;
    const int Qp = Q < 32 ? 32 : Q;
    const int HQ = (H + kDecodeWaves - 1) / kDecodeWaves;
    const int wid = xcd_local_index(blockIdx.x, gridDim.x);
    const int sq = wid / HQ;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = (wid % HQ) * kDecodeWaves + wave;
    const VLayout L(Qp, P);
    char *lds = lds_all + wave * L.bytes;
    // GSHARE: the launcher's choice when the workgroup's heads share a B/C
    // group ((H / G) % 4 == 0); every head of the workgroup exists then and
    // the returns below are the same for all four waves
    constexpr bool gshare = GSHARE;
    float *gsh = reinterpret_cast<float *>(lds_all + kDecodeWaves * L.bytes);
    const int64_t t0 = a.cu[sq];
    const int T = a.cu[sq + 1] - a.cu[sq];
    const int slot = a.slot_idx ? a.slot_idx[sq] : sq;
    if (T <= 0 || h >= H || slot < 0 || slot >= a.num_slots)
        return;
    const int k = a.buf_len[slot];
    // drafts that run past the chunk end are the sweep's: the sequence's
    // first workgroup puts it on the sweep's list
    if (k >= 0 && k < Q && k + T > Q && wid % HQ == 0 && threadIdx.x == 0) {
        int32_t *wl = a.work + a.num_slots;
        wl[kListHead + atomicAdd(wl, 1)] = sq;
    }
    if (k < 0 || k >= Q || k + T > Q)
        return;
    const SlotRows<PG> rows(a.bm, slot, Q);
    if (!rows.ok(a.bm, k))
        return;
    const int g = h / (H / G);
    const int lane = threadIdx.x & 63, gl = lane >> 5, c = lane & 31;
    const int last = k + T - 1;
    const int tau0 = k >> 5, tau1 = last >> 5;
    const int64_t PN = (int64_t)P * N;
    const uint16_t *bx = static_cast<const uint16_t *>(a.buf_x);   // whole pools
    const uint16_t *bB = static_cast<const uint16_t *>(a.buf_B);
    const TD *bdt = static_cast<const TD *>(a.buf_dt);
    const uint16_t *xin = static_cast<const uint16_t *>(a.x);
    const uint16_t *Bin = static_cast<const uint16_t *>(a.B);
    const uint16_t *Cin = static_cast<const uint16_t *>(a.C);
    const TD *din = static_cast<const TD *>(a.dt);
    // draft index of chunk row j (clamped: rows outside the drafts load a
    // draft row whose value is never used)
    auto dj = [&](int j) { return t0 + min(max(j - k, 0), T - 1); };

    const float A2 = a.A[h] * kLog2e;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float D_h = a.D ? a.D[h] : 0.0f;
    TD rawdt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        const int64_t br = rows(j);
        rawdt[i] = j < k ? bdt[br * H + h] : din[dj(j) * H + h];
    }
    const uint16_t *sbf = static_cast<const uint16_t *>(a.cache_state_bf) +
                          ((int64_t)slot * H + h) * PN;

    // delta and the in-chunk cumulative sum (log2 units) over rows 0..last
    const int nseg = (32 * (tau1 + 1) + 63) >> 6;
    float dv[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        float dd = 0.0f, aa = 0.0f;
        if (i < nseg && j <= last) {
            dd = delta_of(DT::val(rawdt[i]), bias, d.softplus);
            aa = dd * A2;
        }
        dv[i] = dd;
        lv[i] = aa;
    }
    wave_scan_segments(lv, nseg);
    float *lam = reinterpret_cast<float *>(lds + L.lam);
    float *uu = reinterpret_cast<float *>(lds + L.u);
    float *bt = reinterpret_cast<float *>(lds + L.beta);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        const float lend = __shfl(lv[i], lane | 31, 64);   // lam[j | 31]
        if (i < nseg && j < Qp) {
            const float l = lv[i];
            const float u = l - flog2(dv[i]);  // +inf where delta is 0
            lam[j] = l;
            uu[j] = u;
            bt[j] = fexp2(lend - u);
        }
    }

    for (int tau = tau0; tau <= tau1; ++tau) {
        const int t = 32 * tau + c;                    // this lane's output row
        const bool outc = t >= k && t <= last;
        bf16x8 cf[NK];
        {
            const uint16_t *crow = Cin + (dj(t) * G + g) * N;
            uint4 raw[NK];
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
                raw[kk] = *reinterpret_cast<const uint4 *>(crow + 16 * kk + 8 * gl);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
                cf[kk] = __builtin_bit_cast(bf16x8, keep_if(outc, raw[kk]));
        }
        const float lam_t = lam[t];
        // read-out from the bf16 state copy (operand (pt, kk) is 1 KiB
        // contiguous); it starts the accumulators, before any s-block
        f32x16 acc[NPT];
        auto readout = [&]() {
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt)
                acc[pt] = readout_scale(
                    readout_raw<N>(
                        [&](int kk) {
                            return *reinterpret_cast<const bf16x8 *>(
                                sbf + ((int64_t)kk * P + 32 * pt + c) * 16 + 8 * gl);
                        },
                        cf),
                    fexp2(lam_t));
        };
        // B rows and x rows of s-block sg (committed rows from the buffer,
        // drafts from the inputs)
        constexpr int XPL = P / 16;
        auto load_b = [&](int sg, uint4 (&braw)[NK]) {
            const int srow = 32 * sg + c;
            const int64_t rs = rows(srow);
            const uint16_t *brow =
                srow < k ? bB + (rs * G + g) * N : Bin + (dj(srow) * G + g) * N;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
                braw[kk] = *reinterpret_cast<const uint4 *>(brow + 16 * kk + 8 * gl);
        };
        auto load_x = [&](int sg, uint4 (&xr)[XPL]) {
#pragma unroll
            for (int i = 0; i < XPL; ++i) {
                const int e = lane + 64 * i, r = e / (P / 8), q = e % (P / 8);
                const int row = 32 * sg + r;
                const int64_t br = rows(row);
                const uint16_t *src =
                    row < k ? bx + (br * H + h) * P : xin + (dj(row) * H + h) * P;
                xr[i] = *reinterpret_cast<const uint4 *>(src + 8 * q);
            }
        };
        auto gram_of = [&](int sg, const uint4 (&braw)[NK]) {
            const bool sok = 32 * sg + c <= last;
            return gram_block<N>(
                [&](int kk) { return __builtin_bit_cast(bf16x8, keep_if(sok, braw[kk])); }, cf);
        };
        // weights of s-block sg from its C.B^T block, the x rows through the
        // wave's LDS tile, Y^T += X^T M^T
        auto accumulate = [&](int sg, const f32x16 &gt, const uint4 (&xr)[XPL]) {
            uint32_t mb[8];
            if (sg == tau)
                m_diag(gt, lam_t, uu, 32 * sg, t, mb, lane);
            else
                m_off(gt, fexp2(lam_t - lam[32 * sg + 31]), bt, 32 * sg, mb, lane);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                mb[q] = outc ? mb[q] : 0u;
#pragma unroll
            for (int i = 0; i < XPL; ++i) {
                const int e = lane + 64 * i, r = e / (P / 8), q = e % (P / 8);
                *reinterpret_cast<uint4 *>(lds + L.X + (r * L.XS + 8 * q) * 2) =
                    keep_if(32 * sg + r <= last, xr[i]);
            }
            mx_accumulate<0, NPT>(mb, lds, L.X, L.XS, 0, acc, lane);
        };
        if constexpr (gshare) {
            // The C.B^T blocks of this t-block, split between the waves
            // (s-blocks wave, wave + 4, ...) and handed over in LDS: only the
            // columns of the t-block's drafts (chunk rows c_lo .. c_lo + gcols
            // - 1 of it; the others' weights are zeroed anyway), column t at
            // floats (t - c_lo) * 32 + s. The read-out follows the hand-over
            // and each block's B rows are loaded just before its MFMAs, so
            // that the wave holds no more than three waves per SIMD allow.
            const int gcols = min(a.max_len, 32);
            const int c_lo = max(k, 32 * tau) - 32 * tau;
            const bool gcol = c >= c_lo && c < c_lo + gcols;
            uint4 nx_[XPL];
            load_x(0, nx_);
            if (tau > tau0)
                __syncthreads();   // the previous t-block's blocks are read
            for (int sg = wave; sg <= tau; sg += kDecodeWaves) {
                uint4 braw[NK];
                load_b(sg, braw);
                const f32x16 gt = gram_of(sg, braw);
                if (gcol) {
                    float *dst = gsh + (sg * gcols + c - c_lo) * 32 + 4 * gl;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<float4 *>(dst + 8 * q) =
                            make_float4(gt[4 * q], gt[4 * q + 1], gt[4 * q + 2], gt[4 * q + 3]);
                }
            }
            __syncthreads();
            readout();
            for (int sg = 0; sg <= tau; ++sg) {
                uint4 xr[XPL];
#pragma unroll
                for (int i = 0; i < XPL; ++i)
                    xr[i] = nx_[i];
                if (sg < tau)
                    load_x(sg + 1, nx_);
                f32x16 gt = {};
                if (gcol) {
                    const float *src = gsh + (sg * gcols + c - c_lo) * 32 + 4 * gl;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 v = *reinterpret_cast<const float4 *>(src + 8 * q);
                        gt[4 * q] = v.x;
                        gt[4 * q + 1] = v.y;
                        gt[4 * q + 2] = v.z;
                        gt[4 * q + 3] = v.w;
                    }
                }
                accumulate(sg, gt, xr);
            }
        } else {
            readout();
            // one block ahead of their use
            uint4 nb_[NK], nx_[XPL];
            load_b(0, nb_);
            load_x(0, nx_);
            for (int sg = 0; sg <= tau; ++sg) {
                uint4 braw[NK], xr[XPL];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk)
                    braw[kk] = nb_[kk];
#pragma unroll
                for (int i = 0; i < XPL; ++i)
                    xr[i] = nx_[i];
                if (sg < tau) {
                    load_b(sg + 1, nb_);
                    load_x(sg + 1, nx_);
                }
                accumulate(sg, gram_of(sg, braw), xr);
            }
        }
        // y for the draft rows of this t-block: fmaf(D, x, Y^T) -> bf16,
        // -0 -> +0; x_t is row t - 32 tau of the last x tile
        if (outc) {
            uint16_t *yrow = static_cast<uint16_t *>(a.y) + (dj(t) * H + h) * P;
            const char *xt = lds + L.X + c * L.XS * 2;
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int p = 32 * pt + 8 * q + 4 * gl;
                    const uint2 xv = *reinterpret_cast<const uint2 *>(xt + 2 * p);
                    const float xs[4] = {bf16_float(xv.x & 0xffff), bf16_float(xv.x >> 16),
                                         bf16_float(xv.y & 0xffff), bf16_float(xv.y >> 16)};
                    uint16_t o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float yv = fmaf(D_h, xs[e], acc[pt][4 * q + e]);
                        yv = yv + 0.0f;
                        o[e] = bf16_bits(yv);
                    }
                    *reinterpret_cast<uint2 *>(yrow + p) =
                        make_uint2(o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16));
                }
            }
        }
    }
}

template <class K>
hipError_t set_lds(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int P, int N, class DT, bool PG>
hipError_t scan_mfma(const ScanArgs &a, hipStream_t stream) {
    const MLayout L(kMaxQ, P, N);   // scan_one's layout: full-height tiles for every chunk size
    hipError_t e;
    if (a.only_cross || a.no_y) {
        if (!a.work)
            return hipErrorInvalidValue;   // the sweeps take their sequences from it
        if ((e = set_lds(k_scan_cross<P, N, DT, PG>, L.bytes)) != hipSuccess)
            return e;
        int dev = 0, cus = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess ||
            (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
                hipSuccess)
            return e;
        const int grid = std::max(1, std::min(a.d.H * a.S, cus));
        if (a.no_y) {
            k_sweep_list<<<dim3(1), dim3(1024), 0, stream>>>(a);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
        k_scan_cross<P, N, DT, PG><<<dim3(grid), dim3(64 * kPrefillWaves), L.bytes, stream>>>(a);
        return hipGetLastError();
    }
    if constexpr (P == 64) {
        // Few (sequence, head) pairs (a batch-1 prompt or prompt chunk): each
        // head's columns in two halves, one workgroup each. The halves share
        // nothing but the per-row quantities and C.B^T, which each computes
        // identically, so every output and state element has the bits of the
        // one-workgroup form, on twice as many compute units.
        int dev = 0, cus = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess ||
            (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
                hipSuccess)
            return e;
        if ((int64_t)a.d.H * a.S * 2 <= cus) {
            const MLayout Lh(kMaxQ, P / 2, N);
            if (PG && !a.replay)
                return hipErrorInvalidValue;   // paged buffers belong to replay calls
            void (*kern)(ScanArgs);
            if constexpr (PG)
                kern = k_scan_mfma<P / 2, N, DT, true, true>;
            else
                kern = a.replay ? k_scan_mfma<P / 2, N, DT, false, true>
                                : k_scan_mfma<P / 2, N, DT, false, false>;
            if ((e = set_lds(kern, Lh.bytes)) != hipSuccess)
                return e;
            ScanArgs h = a;
            h.psplit = 2;
            kern<<<dim3(2 * a.d.H * a.S), dim3(64 * kPrefillWaves), Lh.bytes, stream>>>(h);
            return hipGetLastError();
        }
    }
    if (a.replay) {
        if ((e = set_lds(k_scan_mfma<P, N, DT, PG, true>, L.bytes)) != hipSuccess)
            return e;
        k_scan_mfma<P, N, DT, PG, true>
            <<<dim3(a.d.H * a.S), dim3(64 * kPrefillWaves), L.bytes, stream>>>(a);
        return hipGetLastError();
    }
    if (PG)
        return hipErrorInvalidValue;   // paged buffers belong to replay calls
    if ((e = set_lds(k_scan_mfma<P, N, DT, false, false>, L.bytes)) != hipSuccess)
        return e;
    k_scan_mfma<P, N, DT, false, false>
        <<<dim3(a.d.H * a.S), dim3(64 * kPrefillWaves), L.bytes, stream>>>(a);
    return hipGetLastError();
}

template <int P, int N, class DT>
hipError_t scan_mfma(const ScanArgs &a, hipStream_t stream) {
    return a.replay && a.bm.pages ? scan_mfma<P, N, DT, true>(a, stream)
                                  : scan_mfma<P, N, DT, false>(a, stream);
}

template <int P, int N, class DT, bool PG>
hipError_t decode_mfma(const DecodeArgs &a, hipStream_t stream) {
    const int Qp = a.d.Q < 32 ? 32 : a.d.Q;
    const int HQ = (a.d.H + kDecodeWaves - 1) / kDecodeWaves;
    hipError_t e;
    int dev = 0, cus = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return e;
    // A batch whose workgroups all run at once (three per compute unit) does
    // the chunk-state updates inside the decode launch: one launch per step,
    // and no workgroup waits behind an updating one.
    //
    // A larger batch (with at most num_slots positions, the room the ranking
    // has) is ranked first, heaviest workgroups first, and does the updates
    // in the same launch too: the updating workgroups start first instead of
    // becoming the launch's tail. Beyond that (only with positions outside
    // the slot range) the updates are left to k_decode_commit.
    const bool fits = (int64_t)HQ * a.batch <= (int64_t)std::max(1, cus) * 3;
    if (fits || a.batch <= a.num_slots) {
        DecodeArgs o = a;
        if (!fits) {
            k_decode_order<<<dim3(1), dim3(kOrderThreads), 0, stream>>>(a);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
            o.order = a.work + a.num_slots + kListHead;
        }
        const size_t bytes = (size_t)DLayout(Qp, P, N, true).bytes * kDecodeWaves;
        if ((e = set_lds(k_decode_mfma<P, N, DT, PG, true>, bytes)) != hipSuccess)
            return e;
        k_decode_mfma<P, N, DT, PG, true>
            <<<dim3(HQ * a.batch), dim3(64 * kDecodeWaves), bytes, stream>>>(o);
        return hipGetLastError();
    }
    const size_t bytes = (size_t)DLayout(Qp, P, N, false).bytes * kDecodeWaves;
    if ((e = set_lds(k_decode_mfma<P, N, DT, PG, false>, bytes)) != hipSuccess)
        return e;
    k_decode_mfma<P, N, DT, PG, false>
        <<<dim3(HQ * a.batch), dim3(64 * kDecodeWaves), bytes, stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const MLayout LC(Qp, P, N);
    if ((e = set_lds(k_decode_commit<P, N, DT, PG>, LC.bytes)) != hipSuccess)
        return e;
    // at most one workgroup per (sequence, head) that could commit: a small
    // batch launches a small grid
    const int per_cu = std::max(1, std::min(4, kLdsBytesPerCu / (int)LC.bytes));
    const int64_t items = (int64_t)a.batch * a.d.H;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)std::max(1, cus) * per_cu,
                                                                  items));
    k_decode_commit<P, N, DT, PG><<<dim3(grid), dim3(64 * kCommitWaves), LC.bytes, stream>>>(a);
    return hipGetLastError();
}

template <int P, int N, class DT>
hipError_t decode_mfma(const DecodeArgs &a, hipStream_t stream) {
    return a.bm.pages ? decode_mfma<P, N, DT, true>(a, stream)
                      : decode_mfma<P, N, DT, false>(a, stream);
}

// Verification: the multi-row kernel for sequences whose drafts stay in the
// chunk, then the prefill kernel's dry replay for those that run past its
// end (it skips the others).
template <int P, int N, class DT, bool PG>
hipError_t verify_mfma(const ScanArgs &a, hipStream_t stream) {
    const int Qp = a.d.Q < 32 ? 32 : a.d.Q;
    // per-wave areas, then the shared C.B^T blocks (32 x 32 fp32 each)
    const bool gshare = (a.d.H / a.d.G) % kDecodeWaves == 0;
    // (the shared blocks keep only the drafts' columns: at most 32 of each)
    const size_t bytes = (size_t)VLayout(Qp, P).bytes * kDecodeWaves +
                         (gshare ? (size_t)(Qp / 32) * 32 * std::min(a.max_len, 32) * 4 : 0);
    const auto kern = gshare ? k_verify_mfma<P, N, DT, PG, true> : k_verify_mfma<P, N, DT, PG, false>;
    hipError_t e = set_lds(kern, bytes);
    if (e != hipSuccess)
        return e;
    const int HQ = (a.d.H + kDecodeWaves - 1) / kDecodeWaves;
    kern<<<dim3(HQ * a.S), dim3(64 * kDecodeWaves), bytes, stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    ScanArgs c = a;
    c.only_cross = 1;
    return scan_mfma<P, N, DT, PG>(c, stream);
}

template <int P, int N>
hipError_t verify_pn(const ScanArgs &a, hipStream_t s) {
    if (a.bm.pages)
        return a.d.dt_bf16 ? verify_mfma<P, N, IoBF16, true>(a, s)
                           : verify_mfma<P, N, IoF32, true>(a, s);
    return a.d.dt_bf16 ? verify_mfma<P, N, IoBF16, false>(a, s)
                       : verify_mfma<P, N, IoF32, false>(a, s);
}

template <int P, int N>
hipError_t scan_pn(const ScanArgs &a, hipStream_t s) {
    return a.d.dt_bf16 ? scan_mfma<P, N, IoBF16>(a, s) : scan_mfma<P, N, IoF32>(a, s);
}
template <int P, int N>
hipError_t decode_pn(const DecodeArgs &a, hipStream_t s) {
    return a.d.dt_bf16 ? decode_mfma<P, N, IoBF16>(a, s) : decode_mfma<P, N, IoF32>(a, s);
}

#define SSD_PN_SWITCH(FN, A, S)                                   \
    switch (A.d.P * 1000 + A.d.N) {                               \
    case 32032: return FN<32, 32>(A, S);                          \
    case 32064: return FN<32, 64>(A, S);                          \
    case 32128: return FN<32, 128>(A, S);                         \
    case 64032: return FN<64, 32>(A, S);                          \
    case 64064: return FN<64, 64>(A, S);                          \
    case 64128: return FN<64, 128>(A, S);                         \
    default: return hipErrorInvalidValue;                         \
    }

}  // namespace

bool mfma_supported(const Dims &d) {
    return d.io_bf16 && (d.P == 32 || d.P == 64) && (d.N == 32 || d.N == 64 || d.N == 128);
}

hipError_t launch_scan_mfma(const ScanArgs &a, hipStream_t stream) { SSD_PN_SWITCH(scan_pn, a, stream) }

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream) {
    SSD_PN_SWITCH(decode_pn, a, stream)
}

hipError_t launch_verify_mfma(const ScanArgs &a, hipStream_t stream) {
    SSD_PN_SWITCH(verify_pn, a, stream)
}

}  // namespace ssd
