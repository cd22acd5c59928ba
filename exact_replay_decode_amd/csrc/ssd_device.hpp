// ssd_device.hpp -- device helpers shared by every scan kernel.
//
// Everything that decides a rounding lives here, so the prefill kernel and
// the replay-decode kernel round identically: softplus, the decay exponent,
// the dtype conversions, and the prefix-consistent in-chunk scan.
// The library is built with -ffp-contract=off; every fused multiply-add is
// written as fmaf on purpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kBlock = 256;       // threads per workgroup of the scan kernels
constexpr int kMaxQ = 256;        // largest chunk size
constexpr float kLog2e = 1.4426950408889634f;

// ---- storage types --------------------------------------------------------

struct IoF32 {
    using T = float;
    __device__ static __forceinline__ float ld(const T *p, int64_t i) { return p[i]; }
    __device__ static __forceinline__ float val(T v) { return v; }
    __device__ static __forceinline__ T cvt(float v) { return v; }
};

struct IoBF16 {
    using T = uint16_t;
    __device__ static __forceinline__ float ld(const T *p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
    __device__ static __forceinline__ float val(T v) {
        return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }
    // round to nearest even; NaN stays NaN
    __device__ static __forceinline__ T cvt(float v) {
        uint32_t u = __float_as_uint(v);
        if ((u & 0x7fffffffu) > 0x7f800000u)
            return static_cast<T>((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return static_cast<T>(u >> 16);
    }
};

// fp32 -> bf16 bits, round to nearest even (the hardware conversion). Every
// bf16 copy of the state, and the read-out operand made from it, uses this.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Position of state element (p, n) of one head in the cache's bf16 state
// copy, laid out [N/16][P][16]: the 16-wide n-blocks of all rows in turn, so
// that the read-out operand of 32 rows x 16 columns is 1 KiB contiguous.
__host__ __device__ __forceinline__ int64_t state_bf_index(int p, int n, int P) {
    return (int64_t)(n >> 4) * 16 * P + 16 * p + (n & 15);
}

// Buffer positions a replay prefill or commit of len new tokens touches in
// a slot holding nbuf: it reads [0, nbuf) and writes the trailing partial
// chunk.
__host__ __device__ __forceinline__ int replay_npos(int nbuf, int len, int Q) {
    const int total = nbuf + len;
    const int tail = total % Q;
    return total < Q ? total : (nbuf > tail ? nbuf : tail);
}

// Token count of sequence s: its cu_seqlens span, capped by take[s] when
// given (accepted draft counts; negative counts as 0).
__device__ __forceinline__ int seq_len(const int32_t *cu, const int32_t *take, int s) {
    const int len = cu[s + 1] - cu[s];
    if (!take)
        return len;
    const int t = take[s];
    return t < 0 ? 0 : (t < len ? t : len);
}

// Row of sequence s's first full chunk in a packed array of chunk-end
// states: the full chunks (floor(len / Q)) of sequences 0..s-1. Every thread
// of the workgroup calls it (blockDim.x a multiple of 64); red is one int of
// LDS per wave, free on entry and on return.
__device__ __forceinline__ int full_chunks_before(const int32_t *cu, int s, int Q, int *red) {
    int v = 0;
    for (int i = threadIdx.x; i < s; i += blockDim.x)
        v += (cu[i + 1] - cu[i]) / Q;
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    const int nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    int tot = 0;
    for (int w = 0; w < nw; ++w)
        tot += red[w];
    __syncthreads();
    return tot;
}

// ---- scalar functions that fix the rounding ------------------------------

// delta = softplus(dt + bias) = max(u, 0) + log1p(exp(-|u|)): log1p(exp(u))
// for u <= 0 (plus +0, which changes no value here) and u + log1p(exp(-u))
// otherwise, with one exp/log1p evaluation for both signs; or dt + bias
// when softplus is off.
__device__ __forceinline__ float delta_of(float dt_raw, float bias, int softplus) {
    const float u = dt_raw + bias;
    if (!softplus)
        return u;
    return fmaxf(u, 0.0f) + log1pf(expf(-fabsf(u)));
}

// exp(v) for the decay factors, v <= 0 up to rounding: one v_exp_f32 (2^x)
// of v * log2(e).
__device__ __forceinline__ float decay_exp(float v) {
    return __builtin_amdgcn_exp2f(v * kLog2e);
}

// weight of token j in row i of the intra-chunk product:
// (C_i . B_j) * exp(lam_i - lam_j) * delta_j
__device__ __forceinline__ float intra_weight(float cb, float lam_i, float lam_j, float dlt_j) {
    return (cb * decay_exp(lam_i - lam_j)) * dlt_j;
}

// weight of token j in the chunk-end state: exp(lam_last - lam_j) * delta_j
__device__ __forceinline__ float state_weight(float lam_last, float lam_j, float dlt_j) {
    return decay_exp(lam_last - lam_j) * dlt_j;
}

// ---- prefix-consistent inclusive scan -------------------------------------
// Lane t's result depends only on the values of lanes 0..t and on a fixed
// combination tree: a DPP scan inside each 64-lane wave, then the totals of
// the earlier waves added in ascending order.

// v from lane (DPP control CTRL) of the rows enabled in ROW_MASK; 0 where
// the source lane is outside the row or the row is not enabled.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_from(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Within each 16-lane row: add the value 1, 2, 4, 8 lanes below (row_shr);
// then rows 1 and 3 add lane 15 of the row below (row_bcast:15) and rows 2
// and 3 add lane 31 (row_bcast:31). Lane t reads only lanes below t. (Adding
// the 0 of a lane without a source leaves the value unchanged: the summands
// are finite and never -0.)
__device__ __forceinline__ float wave_scan_inclusive(float v) {
    v = v + dpp_from<0x111, 0xf>(v);
    v = v + dpp_from<0x112, 0xf>(v);
    v = v + dpp_from<0x114, 0xf>(v);
    v = v + dpp_from<0x118, 0xf>(v);
    v = v + dpp_from<0x142, 0xa>(v);
    v = v + dpp_from<0x143, 0xc>(v);
    return v;
}

// Over a whole workgroup (any number of waves up to 8). `tot` is 8 floats of
// LDS. Every thread of the block must call it.
__device__ __forceinline__ float block_scan_inclusive(float v, float *tot) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    v = wave_scan_inclusive(v);
    if (lane == 63)
        tot[wave] = v;
    __syncthreads();
    float r = v;
    if (wave > 0) {
        float pre = tot[0];
        for (int w = 1; w < wave; ++w)
            pre = pre + tot[w];
        r = pre + v;
    }
    __syncthreads();
    return r;
}

// The same sums computed by a single wave that holds rows lane + 64 i in
// v[i], i < nseg <= 4: segment i takes the place of the block's wave i.
__device__ __forceinline__ void wave_scan_segments(float (&v)[4], int nseg) {
    float tot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < nseg) {
            v[i] = wave_scan_inclusive(v[i]);
            tot[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
        }
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        if (i < nseg) {
            float pre = tot[0];
            for (int w = 1; w < i; ++w)
                pre = pre + tot[w];
            v[i] = pre + v[i];
        }
    }
}

// One output point of the causal conv before the scan: bias, then the W
// taps in order (fmaf), then SiLU v / (1 + exp(-v)) with the hardware exp2
// and reciprocal (a few ulps, far below the bf16 storage rounding). Every
// form of the conv (prefill, decode, and the decode step with the conv in
// the same launch) calls only this, so they produce the same bits.
template <int W>
__device__ __forceinline__ float conv_point(const float *w, const float (&v)[W], float bias,
                                            bool act) {
    float acc = bias;
#pragma unroll
    for (int i = 0; i < W; ++i)
        acc = fmaf(w[i], v[i], acc);
    return act ? __fdividef(acc, 1.0f + __expf(-acc)) : acc;
}

}  // namespace ssd
