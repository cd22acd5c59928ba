// ssd_conv.hip -- causal depthwise conv1d of the Mamba2 mixer, the step
// before the scan, in its prefill form (varlen pack, any number of tokens)
// and its decode form (one token per sequence).
//
// vLLM RFC "Mamba2: exact-replay decode ...", section 2, item 6: the prefill
// and decode forms of this conv produce the same bits; bf16 operands are
// promoted to fp32 before the accumulation. Here both forms evaluate every
// output point with one device function (conv_point) on the same W inputs
// in the same order, so the pair is bit-identical by construction:
//   out[c] = act(bias[c] + sum_{i<W} w[c][i] * in_{t-W+1+i}[c]),
// the sum as an fmaf chain from the bias, taps in order, act = SiLU.
// Inputs before a sequence come from its conv state, the W-1 previous inputs
// (oldest first), stored channel-major [conv_dim, W-1] per slot.
//
// Memory: every thread owns 16 bytes of channels (8 bf16 or 4 fp32) and a
// run of tokens, keeps the last W-1 inputs in registers and writes straight
// into the scan's x / B / C arrays (the channel split costs nothing). The
// prefill is a pure stream: each input byte is read once (plus W-1 rows of
// halo per run) and each output byte written once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
namespace {

template <class IO>
struct Lanes;
template <>
struct Lanes<IoBF16> {
    static constexpr int CG = 8;   // channels per 16 bytes
    __device__ static __forceinline__ void unpack(const uint4 &u, float (&f)[8]) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(w[k] << 16);
            f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ uint4 pack(const float (&f)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = IoBF16::cvt(f[2 * k]) | ((uint32_t)IoBF16::cvt(f[2 * k + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <>
struct Lanes<IoF32> {
    static constexpr int CG = 4;
    __device__ static __forceinline__ void unpack(const uint4 &u, float (&f)[4]) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ static __forceinline__ uint4 pack(const float (&f)[4]) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

// The thread's CG channels starting at c0: taps and bias, read as 16-byte
// pieces (the CG * W taps are contiguous and c0 * W * 4 bytes is a
// multiple of 16 because CG * W * 4 is).
template <int W, int CG>
struct Taps {
    float w[CG][W];
    float b[CG];
    __device__ Taps(const float *weight, const float *bias, int c0) {
        float f[CG * W];
        const float4 *wp = reinterpret_cast<const float4 *>(weight + (int64_t)c0 * W);
#pragma unroll
        for (int k = 0; k < CG * W / 4; ++k) {
            const float4 v = wp[k];
            f[4 * k] = v.x;
            f[4 * k + 1] = v.y;
            f[4 * k + 2] = v.z;
            f[4 * k + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < CG; ++j) {
#pragma unroll
            for (int i = 0; i < W; ++i)
                w[j][i] = f[j * W + i];
        }
        if (bias) {
            const float4 *bp = reinterpret_cast<const float4 *>(bias + c0);
#pragma unroll
            for (int k = 0; k < CG / 4; ++k) {
                const float4 v = bp[k];
                b[4 * k] = v.x;
                b[4 * k + 1] = v.y;
                b[4 * k + 2] = v.z;
                b[4 * k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < CG; ++j)
                b[j] = 0.0f;
        }
    }
};

// Where channel c0's 16-byte group of token t goes: x, B or C.
template <class T>
__device__ __forceinline__ T *out_ptr(const ConvArgs &a, int64_t t, int c0) {
    const int HP = a.d.H * a.d.P, GN = a.d.G * a.d.N;
    if (c0 < HP)
        return static_cast<T *>(a.x) + t * HP + c0;
    if (c0 < HP + GN)
        return static_cast<T *>(a.B) + t * GN + (c0 - HP);
    return static_cast<T *>(a.C) + t * GN + (c0 - HP - GN);
}

// The conv state of one slot's CG channels from c0: CG x (W-1) values,
// channel-major, 16 * (W-1) contiguous bytes.
template <class IO, int W>
__device__ __forceinline__ void load_state(const typename IO::T *st, float (&h)[Lanes<IO>::CG][W]) {
    constexpr int CG = Lanes<IO>::CG;
    uint4 raw[W - 1];
#pragma unroll
    for (int k = 0; k < W - 1; ++k)
        raw[k] = reinterpret_cast<const uint4 *>(st)[k];
    float f[W - 1][CG];
#pragma unroll
    for (int k = 0; k < W - 1; ++k)
        Lanes<IO>::unpack(raw[k], f[k]);
    // element e of the chunk is channel e / (W-1), history slot e % (W-1)
#pragma unroll
    for (int e = 0; e < CG * (W - 1); ++e)
        h[e / (W - 1)][e % (W - 1)] = f[e / CG][e % CG];
}

template <class IO, int W>
__device__ __forceinline__ void store_state(typename IO::T *st, const float (&h)[Lanes<IO>::CG][W]) {
    constexpr int CG = Lanes<IO>::CG;
    float f[W - 1][CG];
#pragma unroll
    for (int e = 0; e < CG * (W - 1); ++e)
        f[e / CG][e % CG] = h[e / (W - 1)][e % (W - 1)];
#pragma unroll
    for (int k = 0; k < W - 1; ++k)
        reinterpret_cast<uint4 *>(st)[k] = Lanes<IO>::pack(f[k]);
}

// Prefill: workgroup = kConvGroups channel groups x kConvRuns runs of
// kConvRun tokens of one sequence; grid (token tiles, channel blocks,
// sequences). Tiles past a sequence's end return at once.
constexpr int kConvGroups = 32;
constexpr int kConvRuns = 8;
constexpr int kConvRun = 32;
constexpr int kConvTile = kConvRuns * kConvRun;
constexpr int kConvBatch = 4;

template <class IO, int W>
__global__ __launch_bounds__(kConvGroups * kConvRuns) void k_conv_fwd(ConvArgs a) {
    using T = typename IO::T;
    constexpr int CG = Lanes<IO>::CG;
    const int s = blockIdx.z;
    const int64_t t0 = a.cu[s];
    const int len = a.cu[s + 1] - a.cu[s];
    const int p0 = blockIdx.x * kConvTile + (threadIdx.x / kConvGroups) * kConvRun;
    const int cg = blockIdx.y * kConvGroups + threadIdx.x % kConvGroups;
    const int conv_dim = a.d.H * a.d.P + 2 * a.d.G * a.d.N;
    if (p0 >= len || cg * CG >= conv_dim)
        return;
    const int c0 = cg * CG;
    const int slot = a.slot_idx ? a.slot_idx[s] : s;
    if (a.state && (slot < 0 || slot >= a.num_slots))
        return;
    const Taps<W, CG> tp(a.weight, a.bias, c0);
    const T *in = static_cast<const T *>(a.xBC);

    // window: h[j][0..W-2] = inputs p0-W+1 .. p0-1 of channel c0 + j
    float h[CG][W];
    if (p0 >= W - 1) {
#pragma unroll
        for (int k = 0; k < W - 1; ++k) {
            float f[CG];
            Lanes<IO>::unpack(*reinterpret_cast<const uint4 *>(
                                  in + (t0 + p0 - (W - 1) + k) * conv_dim + c0), f);
#pragma unroll
            for (int j = 0; j < CG; ++j)
                h[j][k] = f[j];
        }
    } else {
        float st[CG][W];
        if (a.state)
            load_state<IO, W>(static_cast<const T *>(a.state) +
                                  ((int64_t)slot * conv_dim + c0) * (W - 1), st);
        else
#pragma unroll
            for (int j = 0; j < CG; ++j)
#pragma unroll
                for (int k = 0; k < W - 1; ++k)
                    st[j][k] = 0.0f;
        // sequence position q = p0 - (W-1) + k; state slot q + W - 1 when q < 0
#pragma unroll
        for (int k = 0; k < W - 1; ++k) {
            const int q = p0 - (W - 1) + k;
            if (q >= 0) {
                float f[CG];
                Lanes<IO>::unpack(*reinterpret_cast<const uint4 *>(in + (t0 + q) * conv_dim + c0),
                                  f);
#pragma unroll
                for (int j = 0; j < CG; ++j)
                    h[j][k] = f[j];
            } else {
#pragma unroll
                for (int j = 0; j < CG; ++j)
                    h[j][k] = st[j][q + W - 1];
            }
        }
    }

    // tokens in batches of kConvBatch, all of a batch's loads in flight
    // before its arithmetic (rows past the run reload the last row)
    const int pend = min(p0 + kConvRun, len);
    for (int p = p0; p < pend; p += kConvBatch) {
        uint4 r[kConvBatch];
#pragma unroll
        for (int u = 0; u < kConvBatch; ++u)
            r[u] = *reinterpret_cast<const uint4 *>(in + (t0 + min(p + u, pend - 1)) * conv_dim +
                                                    c0);
#pragma unroll
        for (int u = 0; u < kConvBatch; ++u) {
            if (p + u >= pend)
                break;
            float f[CG], o[CG];
            Lanes<IO>::unpack(r[u], f);
#pragma unroll
            for (int j = 0; j < CG; ++j) {
                h[j][W - 1] = f[j];
                o[j] = conv_point<W>(tp.w[j], h[j], tp.b[j], a.act);
#pragma unroll
                for (int k = 0; k < W - 1; ++k)
                    h[j][k] = h[j][k + 1];
            }
            *reinterpret_cast<uint4 *>(out_ptr<T>(a, t0 + p + u, c0)) = Lanes<IO>::pack(o);
        }
    }
}

// Final conv state of each sequence: its last W-1 inputs, or for a sequence
// shorter than W-1 the newer rows of the old state followed by its inputs.
// One thread per (sequence, channel group); it reads everything it needs
// before writing, so the state may be updated in place (k_conv_fwd, which
// reads the old state, runs before).
template <class IO, int W>
__global__ __launch_bounds__(256) void k_conv_state(ConvArgs a) {
    using T = typename IO::T;
    constexpr int CG = Lanes<IO>::CG;
    const int conv_dim = a.d.H * a.d.P + 2 * a.d.G * a.d.N;
    const int cg = blockIdx.x * blockDim.x + threadIdx.x, s = blockIdx.y;
    if (cg * CG >= conv_dim)
        return;
    const int c0 = cg * CG;
    const int slot = a.slot_idx ? a.slot_idx[s] : s;
    const int64_t t0 = a.cu[s];
    const int len = a.cu[s + 1] - a.cu[s];
    if (slot < 0 || slot >= a.num_slots || len == 0)
        return;
    T *st = static_cast<T *>(a.state) + ((int64_t)slot * conv_dim + c0) * (W - 1);
    const T *in = static_cast<const T *>(a.xBC);
    float old[CG][W] = {}, nw[CG][W];
    if (len < W - 1)
        load_state<IO, W>(st, old);
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int q = len - (W - 1) + k;   // sequence position of new slot k
        if (q >= 0) {
            float f[CG];
            Lanes<IO>::unpack(*reinterpret_cast<const uint4 *>(in + (t0 + q) * conv_dim + c0), f);
#pragma unroll
            for (int j = 0; j < CG; ++j)
                nw[j][k] = f[j];
        } else {
#pragma unroll
            for (int j = 0; j < CG; ++j)
                nw[j][k] = old[j][q + W - 1];
        }
    }
    store_state<IO, W>(st, nw);
}

// Decode: one token per batch row; thread = (row, channel group). Reads the
// slot's state and the token, writes the outputs and the shifted state.
template <class IO, int W>
__global__ __launch_bounds__(256) void k_conv_update(ConvArgs a) {
    using T = typename IO::T;
    constexpr int CG = Lanes<IO>::CG;
    const int conv_dim = a.d.H * a.d.P + 2 * a.d.G * a.d.N;
    const int groups = conv_dim / CG;
    // one thread per (row, channel group), rows back to back
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)a.S * groups)
        return;
    const int b = (int)(idx / groups), cg = (int)(idx % groups);
    const int c0 = cg * CG;
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0 || slot >= a.num_slots)
        return;
    T *st = static_cast<T *>(a.state) + ((int64_t)slot * conv_dim + c0) * (W - 1);
    const Taps<W, CG> tp(a.weight, a.bias, c0);
    float h[CG][W], f[CG], o[CG];
    load_state<IO, W>(st, h);
    Lanes<IO>::unpack(*reinterpret_cast<const uint4 *>(static_cast<const T *>(a.xBC) +
                                                       (int64_t)b * conv_dim + c0),
                      f);
#pragma unroll
    for (int j = 0; j < CG; ++j) {
        h[j][W - 1] = f[j];
        o[j] = conv_point<W>(tp.w[j], h[j], tp.b[j], a.act);
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
            h[j][k] = h[j][k + 1];
    }
    *reinterpret_cast<uint4 *>(out_ptr<T>(a, b, c0)) = Lanes<IO>::pack(o);
    store_state<IO, W>(st, h);
}

template <class IO, int W>
hipError_t conv_fwd(const ConvArgs &a, hipStream_t stream) {
    constexpr int CG = Lanes<IO>::CG;
    const int conv_dim = a.d.H * a.d.P + 2 * a.d.G * a.d.N;
    const int groups = conv_dim / CG;
    if (a.maxlen > 0) {
        const dim3 grid((a.maxlen + kConvTile - 1) / kConvTile,
                        (groups + kConvGroups - 1) / kConvGroups, a.S);
        k_conv_fwd<IO, W><<<grid, dim3(kConvGroups * kConvRuns), 0, stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (!a.state)
        return hipSuccess;
    k_conv_state<IO, W><<<dim3((groups + 255) / 256, a.S), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

template <class IO, int W>
hipError_t conv_update(const ConvArgs &a, hipStream_t stream) {
    constexpr int CG = Lanes<IO>::CG;
    const int groups = (a.d.H * a.d.P + 2 * a.d.G * a.d.N) / CG;
    const int64_t threads = (int64_t)a.S * groups;
    k_conv_update<IO, W><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

template <class IO>
hipError_t conv_fwd_w(const ConvArgs &a, hipStream_t s) {
    switch (a.W) {
    case 2: return conv_fwd<IO, 2>(a, s);
    case 3: return conv_fwd<IO, 3>(a, s);
    default: return conv_fwd<IO, 4>(a, s);
    }
}
template <class IO>
hipError_t conv_update_w(const ConvArgs &a, hipStream_t s) {
    switch (a.W) {
    case 2: return conv_update<IO, 2>(a, s);
    case 3: return conv_update<IO, 3>(a, s);
    default: return conv_update<IO, 4>(a, s);
    }
}

}  // namespace

hipError_t launch_conv_fwd(const ConvArgs &a, hipStream_t stream) {
    return a.d.io_bf16 ? conv_fwd_w<IoBF16>(a, stream) : conv_fwd_w<IoF32>(a, stream);
}

hipError_t launch_conv_update(const ConvArgs &a, hipStream_t stream) {
    return a.d.io_bf16 ? conv_update_w<IoBF16>(a, stream) : conv_update_w<IoF32>(a, stream);
}

}  // namespace ssd
