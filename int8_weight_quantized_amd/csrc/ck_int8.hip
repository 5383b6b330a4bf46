// ck_int8.hip -- INT8 linear layer for MI355X (gfx950, CDNA4): kernels and
// the C ABI declared in include/ck_int8.h.
//
// Three steps, as the comfy-kitchen pages describe the layer:
//   quantise   bf16 x -> int8 codes + fp32 scale, per row or per tensor
//              (issue #278, "Two separate problems", item 2; issue #280,
//              Summary);
//   product    int8 x int8 with an exact int32 accumulator over K, here on
//              the CDNA4 matrix cores (v_mfma_i32_32x32x32_i8) (issue #280,
//              "Kernel used", "Exactness");
//   epilogue   acc * x_scale[m] * w_scale[n] (+ bias[n]) in fp32, left to
//              right, then bf16, straight from the accumulator registers
//              (issue #280, "Kernel used", "Exactness").
// Every row/column/tile offset is 64-bit (issue #136, "Suggested fix").
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off (no fused
// multiply-add anywhere: the epilogue is one rounding per operation).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <set>
#include <thread>
#include <tuple>

#include "ck_int8.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// ===========================================================================
// Step 1: quantisation
// ===========================================================================
//
// One wavefront per row.  A lane reads 16 bytes (8 bf16) at a time, so a
// wave moves 1 KiB per load instruction, fully coalesced.  Rows of up to
// kQzRegChunks * 512 elements stay in registers between the absmax pass and
// the code pass, so x is read from HBM once; longer rows are re-read (the
// second read hits L2).
//
// absmax works on the bf16 bit patterns: for finite values |x| is the
// pattern with the sign bit cleared, and unsigned order of those patterns is
// the order of the magnitudes, so the integer max is exactly max |x|.

constexpr int kQzWaves = 4;        // rows per 256-thread block
constexpr int kQzRegChunks = 16;   // 16 x 512 elements = rows up to 8192
#ifndef AMAX_WAVES
#define AMAX_WAVES 8       // waves (rows at a time) per block of the tensor-wide amax pass
#endif
#ifndef ROT_AMAX_BLOCKS
#define ROT_AMAX_BLOCKS 1024u // largest grid of the rotated amax pass (a multiple of 8)
#endif
static_assert(ROT_AMAX_BLOCKS % 8 == 0, "rotated amax grid by XCD");
#ifndef AMAX_BLOCKS
#define AMAX_BLOCKS 256    // largest grid of that pass (a multiple of 8)
#endif
static_assert(AMAX_BLOCKS % 8 == 0, "amax grid by XCD");

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b)
{
    return __uint_as_float(b << 16);
}

// Running max of |x| over bf16 bit patterns, two 16-bit maxima per word
// (one v_pk_max_u16 per 32-bit word); absmax_fold gives the larger half.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t absmax_pk(uint32_t m2, const v4i v)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        m2 = __builtin_bit_cast(uint32_t,
                                __builtin_elementwise_max(__builtin_bit_cast(u16x2, m2),
                                                          __builtin_bit_cast(u16x2, (uint32_t)v[i] & 0x7fff7fffu)));
    return m2;
}

__device__ __forceinline__ uint32_t absmax_fold(uint32_t m2) { return max(m2 & 0xffffu, m2 >> 16); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

// q = clamp(rint(x / s), -127, 127); the division is the correctly rounded
// IEEE one (no fast-math), rint rounds half to even.  s == 0 only for an
// all-zero row or tensor, whose codes are 0.
__device__ __forceinline__ int quant_code(float x, float s)
{
    if (s == 0.0f) return 0;
    float t = __builtin_rintf(x / s);
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    return (int)t;
}

__device__ __forceinline__ uint2 quant8(const v4i v, float s)
{
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = (uint32_t)v[i];
        const uint32_t c0 = (uint32_t)(quant_code(bf16_bits_to_f32(w & 0xffffu), s) & 0xff);
        const uint32_t c1 = (uint32_t)(quant_code(bf16_bits_to_f32(w >> 16), s) & 0xff);
        const uint32_t pair = c0 | (c1 << 8);
        if (i < 2) lo |= pair << (16 * i);
        else       hi |= pair << (16 * (i - 2));
    }
    return make_uint2(lo, hi);
}

// The same codes without a division per element.  With r = fl(1/s) a
// normal float, each value v (an exact bf16 x, or an fp32 rotated value)
// is converted twice, as a = fl(v r + 128 - d) and b = fl(v r + 128 + d),
// d = 2^-14, each one fused multiply-add (one rounding, <= 2^-17 at these
// magnitudes), by v_cvt_pk_u8_f32, which rounds to the nearest integer,
// ties to even, into a byte (saturating to [0, 255]).  v r lies within
// |v/s| 2^-24 <= 2^-17 of v/s (|v/s| <= 127 (1 + 2^-23)) and fl(v/s)
// within 2^-18 of v/s.  When the two bytes agree, rounding is constant on
// an interval of half-width > 3 * 2^-16 around v r + 128, which holds
// fl(v/s) + 128 strictly inside, so the byte is rint(fl(v/s)) + 128 (128 is
// even, so ties to even are kept) and byte ^ 0x80 is the code the
// division gives; the clamp to +-127 is never active there.  Returns
// false when any pair disagrees (a few values in 10^4): the caller then
// takes the correctly rounded division for the chunk.
__device__ __forceinline__ bool codes8_pk(const float (&v)[8], float r, uint2& out)
{
    constexpr float kLo = 128.0f - 6.103515625e-05f, kHi = 128.0f + 6.103515625e-05f;
    uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(v[e], r, kLo), e & 3, lo[e >> 2]);
        hi[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(v[e], r, kHi), e & 3, hi[e >> 2]);
    }
    out = make_uint2(lo[0] ^ 0x80808080u, lo[1] ^ 0x80808080u);
    return lo[0] == hi[0] && lo[1] == hi[1];
}

// Eight codes of one 16-byte chunk of bf16 x: through codes8_pk when r =
// fl(1/s) is a normal float, else (or for a chunk codes8_pk declines) the
// correctly rounded division of quant8, so the codes are exactly quant8's.
__device__ __forceinline__ uint2 quant8_fast(const v4i v, float s, float r, bool recip)
{
    if (recip) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = (uint32_t)v[i];
            f[2 * i] = __uint_as_float(w << 16);
            f[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
        }
        uint2 o;
        if (codes8_pk(f, r, o)) return o;
    }
    return quant8(v, s);
}

// 8 codes, stored non-temporally.  x is read once and q is consumed by the
// GEMM from HBM (or not at all by this kernel), so the quantisation streams
// both past the caches: 80666 x 5376 went from 273 to 244 us standalone,
// with the quantise + GEMM step unchanged within noise.
__device__ __forceinline__ void store8_stream(int8_t* p, uint2 v)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}

// PER_ROW: compute each row's scale.  Otherwise the tensor-wide scale is
// amax / 127 from amax_cell (the fp32 bits of the amax, written by
// tensor_amax_kernel), and row 0 stores it in scale[0]; or, with no cell,
// the scale the preceding kernels left in scale[0].  NC 16-byte chunks per
// lane stay in registers (rows up to NC * 512 elements); the host picks the
// smallest NC that holds the row, so short rows keep the register count,
// and with it the number of resident waves, low.  REST: the row may be
// longer than NC * 512 elements (the rest is read again for the codes) or
// k may not be a multiple of 8 (the last k % 8 elements go one per lane);
// without it neither loop is compiled, which frees the registers they hold
// (80666 x 5376: 70 instead of 84 VGPRs, seven waves per SIMD instead of
// five).
template <bool PER_ROW, int NC, bool REST>
__global__ __launch_bounds__(64 * kQzWaves) void quantize_rows_kernel(
    const uint16_t* __restrict__ x, int64_t m, int64_t k, int64_t ldx,
    int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale,
    const uint32_t* __restrict__ amax_cell)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kQzWaves + (threadIdx.x >> 6);
    if (row >= m) return;
    const uint16_t* xr = x + row * ldx;
    int8_t* qr = q + row * ldq;
    const int64_t nvec = k >> 3;                  // whole 8-element chunks

    // Every chunk slot is loaded (a slot past the row re-reads the row's
    // last chunk and is left out below), so all NC loads of a lane go out
    // before the first wait.  With each load under its own `v < nvec` test
    // the compiler waited for each in turn: eleven round trips per row at
    // k = 5376 (one row: 8.2 us).
    v4i buf[NC];
    if (nvec > 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t v = min((int64_t)c * 64 + lane, nvec - 1);
            buf[c] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(xr + v * 8));
        }
    }
    float s;
    if (PER_ROW) {
        uint32_t m2 = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if ((int64_t)c * 64 + lane < nvec) m2 = absmax_pk(m2, buf[c]);
        if (REST)
            for (int64_t v = (int64_t)NC * 64 + lane; v < nvec; v += 64)
                m2 = absmax_pk(m2, *reinterpret_cast<const v4i*>(xr + v * 8));
        uint32_t mb = absmax_fold(m2);
        if (REST)
            for (int64_t j = nvec * 8 + lane; j < k; j += 64)
                mb = max(mb, (uint32_t)xr[j] & 0x7fffu);
        mb = wave_max_u32(mb);
        s = bf16_bits_to_f32(mb) / 127.0f;
        if (lane == 0) scale[row] = s;
    } else {
        if (amax_cell) {
            s = __uint_as_float(*amax_cell) / 127.0f;
            if (row == 0 && lane == 0) scale[0] = s;
        } else {
            s = scale[0];
        }
    }

    // 1/s is used when it is a normal float (s of 2^-126 .. 2^126); for a
    // zero or subnormal scale every code takes the division.
    const float r = 1.0f / s;
    const bool recip = s > 0.0f && r < 8.5070592e+37f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t v = (int64_t)c * 64 + lane;
        if (v < nvec) store8_stream(qr + v * 8, quant8_fast(buf[c], s, r, recip));
    }
    if (!REST) return;
    for (int64_t v = (int64_t)NC * 64 + lane; v < nvec; v += 64) {
        const v4i x8 = *reinterpret_cast<const v4i*>(xr + v * 8);
        *reinterpret_cast<uint2*>(qr + v * 8) = quant8_fast(x8, s, r, recip);
    }
    for (int64_t j = nvec * 8 + lane; j < k; j += 64)
        qr[j] = (int8_t)quant_code(bf16_bits_to_f32(xr[j]), s);
}

// ---------------------------------------------------------------------------
// Step 0 + step 1 for ConvRot checkpoints: online rotation, then quantisation
// ---------------------------------------------------------------------------
// x_rot = x H with H block diagonal: K/b copies of the Sylvester-Hadamard
// matrix of order b (a power of two, b <= 512) scaled by r = fl(1/sqrt(b))
// (#278 "int8_linear silently falls back ...", "Suggested fix": the weight
// is stored as W H^T and the activation is rotated online).  A 512-element
// chunk of a row sits in one wave as 8 consecutive values per lane, so a
// block never leaves its chunk: butterflies with h < 8 stay inside a lane,
// h = 8d pairs lane L with lane L ^ d.  Blocks of 16 to 256 take a
// 1024-element segment as 16 consecutive values per lane instead, so h = 8
// also stays inside the lane and h = 16d pairs lanes L and L ^ d: one
// cross-lane stage fewer, each of which costs two or three instructions
// per value against one.  Stages run in the order h = 1, 2, 4, ..., b/2;
// in each pair the lower element becomes u + v and the upper u - v, every
// operation one fp32 rounding; then each value is multiplied by r.  The
// layout changes which lane does the work, not the arithmetic.  The codes follow from the fp32 results with the same formula as
// the unrotated kernels.

enum { ROT_ROW = 0, ROT_TENSOR_AMAX = 1, ROT_TENSOR_CODES = 2 };

typedef float f32x8 __attribute__((ext_vector_type(8)));

// The value of lane L ^ D, D in {1, 2, ..., 32}, without going through the
// LDS unit: DPP lane moves inside rows of 16 (x ^ 7 reverses 8 lanes, x ^ 15
// reverses 16, quad permutations give x ^ 1, 2, 3), and the gfx950
// permlane swaps for 16 and 32 (each exchanges half-row or half-wave blocks
// of two registers; with both operands v, result [0] holds the partner in
// the upper block, [1] in the lower one).
template <int D>
__device__ __forceinline__ float lane_xor(float v, int lane)
{
    const int x = __float_as_int(v);
    if constexpr (D == 1) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    } else if constexpr (D == 2) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    } else if constexpr (D == 4) {                 // (x ^ 7) ^ 3
        const int t = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
        return __int_as_float(__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, false));
    } else if constexpr (D == 8) {                 // (x ^ 15) ^ 7
        const int t = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);
        return __int_as_float(__builtin_amdgcn_update_dpp(0, t, 0x141, 0xF, 0xF, false));
    } else if constexpr (D == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
        return __uint_as_float((lane & 16) ? p[0] : p[1]);
    } else {
        static_assert(D == 32, "lane distance");
        const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
        return __uint_as_float((lane & 32) ? p[0] : p[1]);
    }
}

template <int D, int B>
__device__ __forceinline__ void lane_stage(f32x8& v, int lane)
{
    if constexpr (8 * D < B) {
        const float sg = (lane & D) ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = lane_xor<D>(v[e], lane) + sg * v[e];
    }
}

template <int LB>              // block b = 2^LB
__device__ __forceinline__ void rotate_chunk(f32x8& v, int lane, float r)
{
    constexpr int B = 1 << LB;
#pragma unroll
    for (int h = 1; h < 8 && h < B; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!(e & h)) {
                const float u = v[e], w = v[e + h];
                v[e] = u + w;
                v[e + h] = u - w;
            }
    // Lane pair (L, L ^ d): the lower lane forms u + v, the upper u - v,
    // written as other + (+-1 * own): the product is exact and x - y is
    // x + (-y) in IEEE arithmetic, so each is the one rounding of the pair.
    lane_stage<1, B>(v, lane);
    lane_stage<2, B>(v, lane);
    lane_stage<4, B>(v, lane);
    lane_stage<8, B>(v, lane);
    lane_stage<16, B>(v, lane);
    lane_stage<32, B>(v, lane);
    if constexpr (LB > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * r;
    }
}

// The same rotation for blocks of 16 and more with 16 consecutive values
// per lane (lo = the first 8, hi = the next 8): stages h = 1, 2, 4 inside
// each half, h = 8 between the halves, then h = 16 d between lanes L and
// L ^ d, in the same order and with the same operations as rotate_chunk.
template <int D, int B>
__device__ __forceinline__ void lane_stage16(f32x8& lo, f32x8& hi, int lane)
{
    if constexpr (16 * D < B) {
        const float sg = (lane & D) ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = lane_xor<D>(lo[e], lane) + sg * lo[e];
#pragma unroll
        for (int e = 0; e < 8; ++e) hi[e] = lane_xor<D>(hi[e], lane) + sg * hi[e];
    }
}

template <int LB>
__device__ __forceinline__ void rotate_pair(f32x8& lo, f32x8& hi, int lane, float r)
{
    static_assert(LB >= 4, "blocks of 16 and more");
    constexpr int B = 1 << LB;
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!(e & h)) {
                float u = lo[e], w = lo[e + h];
                lo[e] = u + w;
                lo[e + h] = u - w;
                u = hi[e]; w = hi[e + h];
                hi[e] = u + w;
                hi[e + h] = u - w;
            }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float u = lo[e], w = hi[e];
        lo[e] = u + w;
        hi[e] = u - w;
    }
    lane_stage16<1, B>(lo, hi, lane);
    lane_stage16<2, B>(lo, hi, lane);
    lane_stage16<4, B>(lo, hi, lane);
    lane_stage16<8, B>(lo, hi, lane);
    lane_stage16<16, B>(lo, hi, lane);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = lo[e] * r;
        hi[e] = hi[e] * r;
    }
}

// Eight codes from fp32 values t: through codes8_pk with rs = fl(1/s) a
// normal float (the bound there holds for any |t/s| <= 127);
// other chunks, and every chunk when rs is not usable, take the correctly
// rounded division.
__device__ __forceinline__ uint2 quant8_f32(const f32x8 t, float s, float rs, bool recip)
{
    if (recip) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = t[e];
        uint2 o;
        if (codes8_pk(y, rs, o)) return o;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t b = (uint32_t)(quant_code(t[e], s) & 0xff);
        if (e < 4) lo |= b << (8 * e);
        else       hi |= b << (8 * (e - 4));
    }
    return make_uint2(lo, hi);
}

// One wave per row; NC chunks of the row stay in registers, chunks past
// them are read again for the code pass.  MODE: per-row scales; the
// tensor-wide amax pass (an fp32 atomic max, as bits, into the cell that
// `scale` points to; block 0 also zeroes `clear` when given, as in
// tensor_amax_kernel); or the tensor-wide code pass, with the scale
// amax / 127 from amax_cell (row 0 stores it in scale[0]) or, with no cell,
// in scale[0].  k % 8 == 0, k % b == 0 and 16-byte aligned rows (checked on
// the host).
template <int MODE, int NC, int LB>
__global__ __launch_bounds__(64 * kQzWaves) void quantize_rot_kernel(
    const uint16_t* __restrict__ x, int64_t m, int64_t k, int64_t ldx,
    int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale, float r,
    uint32_t* __restrict__ clear, const uint32_t* __restrict__ amax_cell)
{
    const int lane = threadIdx.x & 63;
    if (MODE == ROT_TENSOR_AMAX && clear && blockIdx.x == 0 && threadIdx.x == 0) *clear = 0u;
    // The amax pass runs at most ROT_AMAX_BLOCKS blocks: block b takes the
    // row groups b, b + G, b + 2G, ... (G = gridDim.x, a multiple of 8 when
    // it is smaller than the group count, so each row is read on the XCD
    // where the code pass reads it again) and folds its rows' maxima into one
    // atomic.  The other modes run one block per group.
    uint32_t amax_rows = 0u;
    for (int64_t grp = blockIdx.x; grp * kQzWaves < m; grp += gridDim.x) {
    const int64_t row = grp * kQzWaves + (threadIdx.x >> 6);
    const bool live = row < m;                    // dead waves still join the block reduction
    const uint16_t* xr = x + (live ? row : 0) * ldx;
    int8_t* qr = q + (live ? row : 0) * ldq;
    const int64_t nvec = live ? k >> 3 : 0;

    // Blocks of 16 to 256 (k % 16 == 0) hold 16 consecutive values per
    // lane: chunk slot c is half c % 2 of segment c / 2, 1024 elements a
    // segment, lane L holding elements 16 L .. 16 L + 15 of it, so the
    // h = 8 stage stays inside the lane.  Other blocks hold 8 per lane,
    // chunk c covering elements 512 c .. 512 c + 511 (for 512 the paired
    // form needs more registers than three waves per SIMD leave).
    constexpr bool PAIR = LB >= 4 && LB <= 8;
    auto vec_of = [&](int64_t c) -> int64_t {
        return PAIR ? (c >> 1) * 128 + 2 * lane + (c & 1) : c * 64 + lane;
    };
    const int64_t nchunk = PAIR ? 2 * ((nvec + 127) / 128) : (nvec + 63) / 64;
    auto to_f32 = [&](int64_t c, v4i raw) {
        if (vec_of(c) >= nvec) raw = v4i{0, 0, 0, 0};
        f32x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32((uint32_t)raw[i] & 0xffffu);
            v[2 * i + 1] = bf16_bits_to_f32((uint32_t)raw[i] >> 16);
        }
        return v;
    };
    auto load_raw = [&](int64_t c) {
        const int64_t vi = vec_of(c);
        v4i raw = {0, 0, 0, 0};
        if (vi < nvec) raw = *reinterpret_cast<const v4i*>(xr + vi * 8);
        return raw;
    };
    // rotated chunk slots c and c + 1 (c even) past the register-held ones
    auto load_rot2 = [&](int64_t c, f32x8& v0, f32x8& v1) {
        v0 = to_f32(c, load_raw(c));
        v1 = to_f32(c + 1, load_raw(c + 1));
        if constexpr (PAIR) {
            rotate_pair<LB>(v0, v1, lane, r);
        } else {
            rotate_chunk<LB>(v0, lane, r);
            rotate_chunk<LB>(v1, lane, r);
        }
    };

    // The register-held chunks are loaded four at a time, all four before
    // the first is used (a slot past the row re-reads its last chunk and is
    // zeroed), so a row costs a quarter of the round trips it would one
    // chunk at a time, for 16 more registers.
    constexpr int G = 4;
    static_assert(NC % G == 0, "chunk groups");
    f32x8 buf[NC];
    float amax = 0.0f;
#pragma unroll
    for (int c0 = 0; c0 < NC; c0 += G) {
        if (c0 < nchunk) {
            v4i raw[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t vi = min(vec_of(c0 + g), nvec - 1);
                raw[g] = *reinterpret_cast<const v4i*>(xr + vi * 8);
            }
#pragma unroll
            for (int g = 0; g < G; g += 2) {
                const int c = c0 + g;
                if (c < nchunk) {
                    buf[c] = to_f32(c, raw[g]);
                    buf[c + 1] = to_f32(c + 1, raw[g + 1]);
                    if constexpr (PAIR) {
                        rotate_pair<LB>(buf[c], buf[c + 1], lane, r);
                    } else {
                        rotate_chunk<LB>(buf[c], lane, r);
                        rotate_chunk<LB>(buf[c + 1], lane, r);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fmaxf(fabsf(buf[c][e]), fabsf(buf[c + 1][e])));
                }
            }
        }
    }
    // Only the 16-chunk kernel takes rows longer than its registers hold:
    // the host picks 4, 8 or 12 chunks only for rows that fit, and the
    // paired count 2 ceil(nvec / 128) is the smallest even number at or
    // above ceil(nvec / 64), so it fits an even NC too.
    constexpr bool LONG = NC >= 16;
    if (MODE != ROT_TENSOR_CODES) {
        for (int64_t c = NC; LONG && c < nchunk; c += 2) {
            f32x8 v0, v1;
            load_rot2(c, v0, v1);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fmaxf(fabsf(v0[e]), fabsf(v1[e])));
        }
        amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
    }
    if (MODE == ROT_TENSOR_AMAX) {
        amax_rows = max(amax_rows, __float_as_uint(amax));
        continue;
    }
    if (!live) return;
    float s;
    if (MODE == ROT_ROW) {
        s = amax / 127.0f;
        if (lane == 0) scale[row] = s;
    } else if (amax_cell) {
        s = __uint_as_float(*amax_cell) / 127.0f;
        if (row == 0 && lane == 0) scale[0] = s;
    } else {
        s = scale[0];
    }
    const float rs = 1.0f / s;
    const bool recip = s > 0.0f && rs < 8.5070592e+37f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t vi = vec_of(c);
        if (c < nchunk && vi < nvec)
            *reinterpret_cast<uint2*>(qr + vi * 8) = quant8_f32(buf[c], s, rs, recip);
    }
    for (int64_t c = NC; LONG && c < nchunk; c += 2) {
        f32x8 v0, v1;
        load_rot2(c, v0, v1);
        const int64_t v0i = vec_of(c), v1i = vec_of(c + 1);
        if (v0i < nvec) *reinterpret_cast<uint2*>(qr + v0i * 8) = quant8_f32(v0, s, rs, recip);
        if (v1i < nvec) *reinterpret_cast<uint2*>(qr + v1i * 8) = quant8_f32(v1, s, rs, recip);
    }
    if (MODE != ROT_TENSOR_AMAX) break;           // one group: no loop is compiled
    }   // row groups
    if (MODE == ROT_TENSOR_AMAX) {
        __shared__ uint32_t red[kQzWaves];
        if (lane == 0) red[threadIdx.x >> 6] = amax_rows;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t mb = 0;
#pragma unroll
            for (int w = 0; w < kQzWaves; ++w) mb = max(mb, red[w]);
            if (mb != 0u) atomicMax(reinterpret_cast<uint32_t*>(scale), mb);
        }
    }
}

// Rows that are not 16-byte aligned (ldx % 8 != 0, or q rows not 8-byte
// aligned): one wave per row, one element per lane and step, the same
// arithmetic as the aligned kernel's division path; the tensor-wide scale
// as in quantize_rows_kernel.
template <bool PER_ROW>
__global__ __launch_bounds__(64 * kQzWaves) void quantize_rows_any_kernel(
    const uint16_t* __restrict__ x, int64_t m, int64_t k, int64_t ldx,
    int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale,
    const uint32_t* __restrict__ amax_cell)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kQzWaves + (threadIdx.x >> 6);
    if (row >= m) return;
    const uint16_t* xr = x + row * ldx;
    int8_t* qr = q + row * ldq;
    float s;
    if (PER_ROW) {
        uint32_t mb = 0;
        for (int64_t j = lane; j < k; j += 64) mb = max(mb, (uint32_t)xr[j] & 0x7fffu);
        mb = wave_max_u32(mb);
        s = bf16_bits_to_f32(mb) / 127.0f;
        if (lane == 0) scale[row] = s;
    } else if (amax_cell) {
        s = __uint_as_float(*amax_cell) / 127.0f;
        if (row == 0 && lane == 0) scale[0] = s;
    } else {
        s = scale[0];
    }
    for (int64_t j = lane; j < k; j += 64) qr[j] = (int8_t)quant_code(bf16_bits_to_f32(xr[j]), s);
}

// Tensor-wide scale.  tensor_amax folds the absmax of every wave's rows
// into a cell holding zero, with an unsigned atomic max of the fp32 bit
// pattern (non-negative floats order like their patterns).  With a cell of
// the stream's counter block, the code kernel then reads the amax from it
// and stores the scale, and the same amax launch clears the stream's other
// cell for its next call (two launches).  Otherwise the cell is scale[0]
// itself, in four launches:
//   tensor_amax_zero : the cell scale[0] := 0 (as bits);
//   tensor_amax      : the atomic max into scale[0];
//   tensor_amax_final: scale[0] := amax / 127;
//   the code kernel reads scale[0].
__global__ void tensor_amax_zero_kernel(uint32_t* cell) { *cell = 0u; }

// Rows at any alignment: one element per lane and step.
__global__ __launch_bounds__(256) void tensor_amax_kernel(
    const uint16_t* __restrict__ x, int64_t m, int64_t k, int64_t ldx,
    uint32_t* cell, uint32_t* clear)
{
    if (clear && blockIdx.x == 0 && threadIdx.x == 0) *clear = 0u;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    uint32_t mb = 0;
    for (int64_t row = wave; row < m; row += nwaves) {
        const uint16_t* xr = x + row * ldx;
        for (int64_t j = lane; j < k; j += 64)
            mb = max(mb, (uint32_t)xr[j] & 0x7fffu);
    }
    // one atomic per block: many blocks updating one cell serialise in L2
    __shared__ uint32_t red[4];
    mb = wave_max_u32(mb);
    if (lane == 0) red[threadIdx.x >> 6] = mb;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t b = max(max(red[0], red[1]), max(red[2], red[3]));
        if (b != 0u) atomicMax(cell, b << 16);
    }
}

// 16-byte aligned rows, one wave per row as in quantize_rows_kernel: a row
// goes in passes of NC chunks per lane, all NC loads of a pass out before
// the first wait (a slot past the row re-reads the row's last chunk and is
// left out of the max), so a row of up to NC * 512 elements costs one round
// trip to memory.  TAIL: k % 8 != 0, the last k % 8 elements one per lane.
// Blocks of AMAX_WAVES waves, one atomic per block: the atomics of all
// blocks meet on one cell at the end and run one at a time (at 4096 x 4096,
// 1024 blocks of one row per wave took 5 us longer than 512 of two), so the
// host sizes the grid for two rows per wave.  4096 x 4096, 8 waves, 256
// blocks: 6.7 us against 9.2 us for 512 blocks of 4 waves walking their
// rows four loads at a time; the code kernel after it 5.8 us.
//
// Row placement follows the code kernel that runs next: its block c takes
// rows 4c .. 4c + 3 and runs on XCD c % 8, reading x again, so each row is
// read here on that same XCD and the second read finds it in that XCD's
// L2 (4096 x 4096: code kernel 5.6 us this way, 10.2 us when the rows land
// on other XCDs).  Blocks go to the XCDs in turn, block b to XCD b % 8;
// with a grid of 8 G blocks, block b = 8 j + x and wave w = 4 t + r take
// row 4 (x + 8 (T j + t)) + r (T = AMAX_WAVES / 4), which covers rows
// 0 .. AMAX_WAVES * 8 G - 1 once, and then the same plus multiples of that
// count.  Another grid takes the rows in order (still each once, its own
// XCD order aside).
template <int NC, bool TAIL>
__global__ __launch_bounds__(64 * AMAX_WAVES) void tensor_amax_rows_kernel(
    const uint16_t* __restrict__ x, int64_t m, int64_t k, int64_t ldx,
    uint32_t* cell, uint32_t* clear)
{
    static_assert(AMAX_WAVES % 4 == 0, "whole code-kernel blocks per amax block");
    constexpr int T = AMAX_WAVES / 4;
    if (clear && blockIdx.x == 0 && threadIdx.x == 0) *clear = 0u;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t nwaves = (int64_t)gridDim.x * AMAX_WAVES;
    const int64_t nvec = k >> 3;
    const int64_t cb = (gridDim.x & 7) == 0
        ? (int64_t)(blockIdx.x & 7) + 8 * ((int64_t)(blockIdx.x >> 3) * T + (w >> 2))
        : (int64_t)blockIdx.x * T + (w >> 2);
    uint32_t mb = 0, m2 = 0;
    for (int64_t row = 4 * cb + (w & 3); row < m; row += nwaves) {
        const uint16_t* xr = x + row * ldx;
        for (int64_t base = lane; base < nvec + lane; base += (int64_t)NC * 64) {
            v4i buf[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int64_t v = min(base + c * 64, nvec - 1);
                buf[c] = *reinterpret_cast<const v4i*>(xr + v * 8);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (base + c * 64 < nvec) m2 = absmax_pk(m2, buf[c]);
        }
        if (TAIL)
            for (int64_t j = nvec * 8 + lane; j < k; j += 64)
                mb = max(mb, (uint32_t)xr[j] & 0x7fffu);
    }
    mb = max(mb, absmax_fold(m2));
    __shared__ uint32_t red[AMAX_WAVES];
    mb = wave_max_u32(mb);
    if (lane == 0) red[w] = mb;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = red[0];
#pragma unroll
        for (int i = 1; i < AMAX_WAVES; ++i) b = max(b, red[i]);
        if (b != 0u) atomicMax(cell, b << 16);
    }
}

__global__ void tensor_amax_final_kernel(float* scale)
{
    scale[0] = scale[0] / 127.0f;
}

// ---------------------------------------------------------------------------
// Measurement aid: the quantisation's memory traffic without its arithmetic
// ---------------------------------------------------------------------------
// Reads `chunks` 16-byte chunks (8 bf16) and writes one 8-byte word per
// chunk (8 codes' worth), both streamed past the caches as the quantisation
// does, with U independent loads in flight per lane over a grid-stride
// loop.  The written word is the xor of the chunk's halves, so every loaded
// byte is used.  Its rate is the ceiling the quantisation is measured
// against: the same bytes in the same 2 : 1 read : write mix, nothing else.
template <int U>
__global__ __launch_bounds__(256) void hbm_stream_kernel(const v4i* __restrict__ src,
                                                         uint2* __restrict__ dst, int64_t chunks)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (U - 1) * stride < chunks; i += U * stride) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u)
            __builtin_nontemporal_store(u32x2{(unsigned)(v[u][0] ^ v[u][2]), (unsigned)(v[u][1] ^ v[u][3])},
                                        reinterpret_cast<u32x2*>(dst + i + u * stride));
    }
    for (; i < chunks; i += stride) {
        const v4i v = __builtin_nontemporal_load(src + i);
        __builtin_nontemporal_store(u32x2{(unsigned)(v[0] ^ v[2]), (unsigned)(v[1] ^ v[3])},
                                    reinterpret_cast<u32x2*>(dst + i));
    }
}

// ---------------------------------------------------------------------------
// Measurement aid: the int8 matrix cores with nothing else to do
// ---------------------------------------------------------------------------
// 8 waves per block (two per SIMD, the GEMM's occupancy), one block per CU.
// Every wave keeps 8 accumulator tiles of 32 x 32 (128 registers, as the
// GEMM's waves do) and per iteration runs two half-steps of 8 independent
// v_mfma_i32_32x32x32_i8 products, each half-step with its own set of
// 4 + 2 random operand fragments (16 bytes per lane each):
//   mode 0: the two sets stay in registers, so the loop is products only;
//   mode 1: the sets come from LDS, from 8 rotating 6 KiB slices of one
//           48 KiB table, read every half-step as a GEMM main loop reads
//           its fragments.
// The operand table is word i = lowbias32(i + 12288 * seed), the 32-bit
// integer hash published by C. Wellons ("Prospecting for hash functions",
// 2018); set h of mode 0 is slice h.  Each lane stores the xor of its
// accumulators.  The rates bound what the GEMM's matrix cores can deliver
// under the board's power limit, without (mode 0) and with (mode 1) the
// LDS traffic of operand reads, and no global memory traffic.
__device__ __forceinline__ uint32_t lowbias32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

constexpr int kCeilSlices = 8, kCeilFrags = 6;   // fragments per set: 4 A + 2 B

__device__ __forceinline__ void ceiling_products(v16i (&acc)[8], const v4i (&f)[kCeilFrags])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i * 2 + j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[4 + j], f[i], acc[i * 2 + j], 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(int64_t iters, int32_t* __restrict__ out,
                                                           uint32_t seed)
{
    __shared__ v4i table[kCeilSlices * kCeilFrags * 64];      // 48 KiB
    const int lane = threadIdx.x & 63;
    uint32_t* tw = reinterpret_cast<uint32_t*>(table);
    for (int i = threadIdx.x; i < kCeilSlices * kCeilFrags * 64 * 4; i += 512)
        tw[i] = lowbias32((uint32_t)i + 12288u * seed);
    __syncthreads();
    v16i acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0;
    if constexpr (MODE == 0) {
        v4i f0[kCeilFrags], f1[kCeilFrags];
#pragma unroll
        for (int f = 0; f < kCeilFrags; ++f) {
            f0[f] = table[f * 64 + lane];
            f1[f] = table[(kCeilFrags + f) * 64 + lane];
        }
        for (int64_t it = 0; it < iters; ++it) {
            ceiling_products(acc, f0);
            ceiling_products(acc, f1);
        }
    } else {
        // half-step q multiplies slice q % 8; the compiler interleaves each
        // slice's reads with the products (two waves per SIMD cover the waits)
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int sl = (int)((2 * it + h) & (kCeilSlices - 1));
                v4i f[kCeilFrags];
#pragma unroll
                for (int k = 0; k < kCeilFrags; ++k) f[k] = table[(sl * kCeilFrags + k) * 64 + lane];
                ceiling_products(acc, f);
            }
        }
    }
    int x = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) x ^= acc[t][r];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// ===========================================================================
// Steps 2 + 3: the int8 GEMM with the fused epilogue
// ===========================================================================
//
// Block tile BM x BN, K in stages of 64 bytes.  WM x WN waves; each wave
// owns a (BM/WM) x (BN/WN) sub-tile made of 32 x 32 v_mfma_i32_32x32x32_i8
// tiles whose int32 accumulators live in registers from the first K stage
// to the epilogue.
//
// Two main loops feed the matrix cores:
//   gemm_dma_kernel  (k % 64 == 0): global_load_lds_dwordx4 copies each
//     stage straight from global memory into one of S LDS buffers, S-1
//     stages ahead of the stage being multiplied, with no register staging.
//     One barrier per stage: it publishes stage t and frees the buffer of
//     stage t-1, which the same iteration then refills with stage t+S-1.
//   gemm_kernel (any k % 16 == 0): loads go through registers, two stages
//     ahead, into two LDS buffers; a final partial stage is zero-filled.
//
// Rows past m (or n) are read from row m-1 (n-1) instead, so the hot loop's
// loads carry no per-lane condition; those rows' results are never stored.
//
// The weight fragment is the instruction's first operand and the activation
// fragment its second, so the 32 x 32 result D holds out[m, n] at
// D[n_local][m_local].  With the CDNA accumulator layout (lane L, register
// r: row 8*(r/4) + 4*(L/32) + r%4, column L%32), lane L then holds row
// m_local = L%32 and, per group g = r/4, four consecutive columns
// n_local = 8g + 4*(L/32) + 0..3: the epilogue packs those four bf16
// values into one 8-byte store.
//
// The K order inside an instruction does not matter: both fragments are
// loaded with the same lane -> byte -> k assignment and integer sums are
// exact in any order.
//
// LDS layout of a stage: row r (of BM or BN), 16-byte chunk c of the 64
// bytes at r*64 + 16*(c ^ f(r)), f(r) = (r >> 2) & 3.  gfx950 serves a
// 128-bit LDS read 16 lanes at a time from a 256-byte window of banks; a
// fragment read puts 16 consecutive lanes on 16 consecutive rows at one
// chunk, and with f those rows' chunks fill the 16 slots of the window
// exactly once (measured: as fast as a sequential read; without the
// swizzle, twice as slow).  Stores of 4 rows x 4 chunks by 16 consecutive
// lanes are conflict-free for the same reason.  A DMA load
// writes 64 lanes x 16 bytes contiguously, i.e. 16 whole rows; lane L takes
// row 16*blk + L/4 and physical chunk L%4, so it fetches logical chunk
// (L%4) ^ f(row) from global memory.
//
// Launch order: block ids are dealt round-robin to the 8 XCDs, so block b
// runs on XCD b % 8.  The first floor(grid/8)*8 ids are renumbered so that
// each XCD receives a contiguous range of tiles; within the range, tiles go
// column-major over groups of group_m row tiles, so blocks resident at the
// same time on one XCD share A rows and B columns in that XCD's L2.

constexpr int kBK = 64;

struct GemmArgs {
    const int8_t* q;
    const int8_t* w;
    const float* xs;
    const float* ws;
    const void* bias;    // [n] of the output's type (fp32 for fp32 output), or NULL
    void* out;
    int64_t ldq, ldw, ldo;
    int64_t m, n, k;
    int tiles_m, tiles_n, group_m;
    int xs_stride;   // 1: per-row x scale, 0: tensor-wide
    int ws_stride;   // 1: per-column w scale, 0: tensor-wide
    int vec_store;   // out rows allow 16-byte (2) or 8-byte (1) stores, or neither (0)
    int stream_out;  // non-temporal output stores (launches of more than one wave of blocks)
    unsigned* sched; // persistent kernel: tile counters (see gemm_persist_kernel), zero between launches
};

// What the epilogue writes: bf16, the raw int32 accumulators, fp16 or fp32.
enum { EPI_BF16 = 0, EPI_I32 = 1, EPI_F16 = 2, EPI_F32 = 3 };
constexpr int kNumEpi = 4;

__device__ __forceinline__ int lds_swz(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ int lds_off(int row, int chunk)
{
    return row * kBK + ((chunk ^ lds_swz(row)) << 4);
}

// fp32 epilogue of one accumulator: one rounding per operation.
__device__ __forceinline__ float epilogue_value(int a, float xs, float ws,
                                                float b, bool has_bias)
{
#pragma clang fp contract(off)
    float t = (float)a;
    t = t * xs;
    t = t * ws;
    if (has_bias) t = t + b;
    return t;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f)
{
    const __bf16 h = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Two values rounded to bf16 (nearest, ties to even) in one conversion;
// `lo` lands in bits 0..15.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne_bits(float lo, float hi)
{
    const bf16x2 h = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f16x2_rne_bits(float lo, float hi)
{
    const f16x2 h = __builtin_convertvector(f32x2{lo, hi}, f16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// Two epilogue values rounded to the 16-bit output type, `lo` in bits 0..15.
template <int EPI>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (EPI == EPI_F16) return f16x2_rne_bits(lo, hi);
    else return bf16x2_rne_bits(lo, hi);
}

// bias[c] widened to fp32 (exact for every output type).
template <int EPI>
__device__ __forceinline__ float bias_at(const void* bias, int64_t c)
{
    if constexpr (EPI == EPI_F32) {
        return static_cast<const float*>(bias)[c];
    } else if constexpr (EPI == EPI_F16) {
        return (float)__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(bias)[c]);
    } else {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(bias)[c]);
    }
}

// v with its bytes from `valid` on (0 < valid < 16) cleared: a 16-byte chunk
// that straddles the end of K contributes only its first `valid` bytes.
__device__ __forceinline__ v4i keep_bytes(v4i v, int valid)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int nb = min(max(valid - 4 * d, 0), 4);
        const uint32_t m = nb == 4 ? 0xffffffffu : (1u << (8 * nb)) - 1u;
        v[d] = (int)((uint32_t)v[d] & m);
    }
    return v;
}

template <bool B> struct BoolTag { static constexpr bool value = B; };

// s_waitcnt immediate that waits for the vector-memory counter only.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most N vector-memory operations of this wave are pending.
// The empty asm keeps the compiler from moving memory accesses across the
// wait: it does not know what the direct-to-LDS loads write.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
    asm volatile("" : : : "memory");
}

// 32-bit LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane, global -> LDS: lane L's bytes land at m0 + 16*L.
// The LDS write is invisible to the compiler, so callers wait on the
// vector-memory counter (and a barrier) before reading the data.
__device__ __forceinline__ void dma16(const int8_t* base, uint32_t voff, uint32_t lds)
{
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Origin of tile pid in the grouped order: groups of group_m row tiles,
// walked column by column inside a group, so that tiles close in the order
// share A and B panels.
template <int BM, int BN>
__device__ __forceinline__ void grouped_origin(const GemmArgs& a, int pid, int64_t& m0, int64_t& n0)
{
    const int per_group = a.group_m * a.tiles_n;
    const int gid = pid / per_group;
    const int first_m = gid * a.group_m;
    const int gsz = min(a.tiles_m - first_m, a.group_m);
    const int in_g = pid - gid * per_group;
    m0 = (int64_t)(first_m + in_g % gsz) * BM;
    n0 = (int64_t)(in_g / gsz) * BN;
}

// Origin of the tile of launch-order block pid out of num: blocks go to the
// XCDs round robin (block b to XCD b % 8), so XCD x gets the grouped-order
// range [x * num / 8, (x + 1) * num / 8) (the last num % 8 blocks keep their
// own ids) and its L2 sees neighbouring tiles.
template <int BM, int BN>
__device__ __forceinline__ void tile_origin_at(const GemmArgs& a, int pid, int num, int64_t& m0,
                                               int64_t& n0)
{
    const int full = num & ~7;
    if (pid < full) pid = (pid & 7) * (full >> 3) + (pid >> 3);
    grouped_origin<BM, BN>(a, pid, m0, n0);
}

template <int BM, int BN>
__device__ __forceinline__ void tile_origin(const GemmArgs& a, int64_t& m0, int64_t& n0)
{
    tile_origin_at<BM, BN>(a, blockIdx.x, gridDim.x, m0, n0);
}

// One 64-byte K stage of a wave's sub-tile, out of LDS.
template <int FM, int FN, int TM, int TN>
__device__ __forceinline__ void mma_stage(const int8_t* la, const int8_t* lb, int wm, int wn,
                                          int lane, v16i (&acc)[FM][FN])
{
    const int frag_row = lane & 31;
    const int frag_half = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int chunk = kk * 2 + frag_half;
        v4i fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[i] = *reinterpret_cast<const v4i*>(&la[lds_off(wm * TM + i * 32 + frag_row, chunk)]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[j] = *reinterpret_cast<const v4i*>(&lb[lds_off(wn * TN + j * 32 + frag_row, chunk)]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
}

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(v16i (&acc)[FM][FN])
{
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
}

// LDS layout for stages of BKB bytes of K per row (64 or 128): chunk c of
// row r at r*BKB + 16*(c ^ swz(r)).  For 64-byte rows swz(r) = (r>>2)&3 (four
// rows per 256-byte bank window); for 128-byte rows swz(r) = (r>>1)&7 (two
// rows per window).  Either way the 16 consecutive rows read by 16
// consecutive lanes at one logical chunk land on 16 distinct 16-byte slots.
template <int BKB>
__device__ __forceinline__ int swz_b(int row)
{
    static_assert(BKB == 64 || BKB == 128, "stage width");
    return BKB == 64 ? (row >> 2) & 3 : (row >> 1) & 7;
}

template <int BKB>
__device__ __forceinline__ int lds_off_b(int row, int chunk)
{
    return row * BKB + ((chunk ^ swz_b<BKB>(row)) << 4);
}

// One K step (32 bytes) of fragments, and the 32 x 32 products it feeds.
template <int FM, int FN>
struct Frags {
    v4i a[FM];
    v4i b[FN];
};

template <int FM, int FN, int TM, int TN, int BKB = kBK>
__device__ __forceinline__ void load_frags(Frags<FM, FN>& f, const int8_t* la, const int8_t* lb,
                                           int wm, int wn, int lane, int kk)
{
    const int frag_row = lane & 31;
    const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i)
        f.a[i] = *reinterpret_cast<const v4i*>(&la[lds_off_b<BKB>(wm * TM + i * 32 + frag_row, chunk)]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
        f.b[j] = *reinterpret_cast<const v4i*>(&lb[lds_off_b<BKB>(wn * TN + j * 32 + frag_row, chunk)]);
}

template <int FM, int FN>
__device__ __forceinline__ void mfma_frags(const Frags<FM, FN>& f, v16i (&acc)[FM][FN])
{
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Epilogue straight from the accumulators: each lane writes, per 32 x 32
// tile and group g, four consecutive columns of one row.
template <int FM, int FN, int TM, int TN, int EPI>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const v16i (&acc)[FM][FN],
                                           int64_t m0, int64_t n0, int wm, int wn, int lane)
{
    const int frag_row = lane & 31;
    const int col_off = 4 * (lane >> 5);
    if constexpr (EPI == EPI_I32) {
        int32_t* out = reinterpret_cast<int32_t*>(a.out);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t gm = m0 + wm * TM + i * 32 + frag_row;
            if (gm >= a.m) continue;
            int32_t* orow = out + gm * a.ldo;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t gn = n0 + wn * TN + j * 32 + g * 8 + col_off;
                    if (a.vec_store && gn + 3 < a.n) {
                        v4i v = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                                 acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                        *reinterpret_cast<v4i*>(orow + gn) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (gn + e < a.n) orow[gn + e] = acc[i][j][4 * g + e];
                    }
                }
        }
        return;
    } else {
        const bool has_bias = a.bias != nullptr;
        float xsv[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t gm = m0 + wm * TM + i * 32 + frag_row;
            xsv[i] = a.xs[(gm < a.m ? gm : 0) * a.xs_stride];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t gn = n0 + wn * TN + j * 32 + g * 8 + col_off;
                float wsv[4], bv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t c = gn + e < a.n ? gn + e : 0;
                    wsv[e] = a.ws[c * a.ws_stride];
                    bv[e] = has_bias ? bias_at<EPI>(a.bias, c) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int64_t gm = m0 + wm * TM + i * 32 + frag_row;
                    if (gm >= a.m || gn >= a.n) continue;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = epilogue_value(acc[i][j][4 * g + e], xsv[i], wsv[e], bv[e], has_bias);
                    if constexpr (EPI == EPI_F32) {
                        float* orow = reinterpret_cast<float*>(a.out) + gm * a.ldo;
                        if (a.vec_store && gn + 3 < a.n) {
                            *reinterpret_cast<float4*>(orow + gn) = make_float4(v[0], v[1], v[2], v[3]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (gn + e < a.n) orow[gn + e] = v[e];
                        }
                    } else {
                        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + gm * a.ldo;
                        const uint32_t p0 = pack2<EPI>(v[0], v[1]), p1 = pack2<EPI>(v[2], v[3]);
                        if (a.vec_store && gn + 3 < a.n) {
                            *reinterpret_cast<uint2*>(orow + gn) = make_uint2(p0, p1);
                        } else {
                            const uint32_t h[4] = {p0 & 0xffffu, p0 >> 16, p1 & 0xffffu, p1 >> 16};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (gn + e < a.n) orow[gn + e] = (uint16_t)h[e];
                        }
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS pipeline, S stages in flight (k % 64 == 0)
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int EPI, int S, bool IL, int BKB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(GemmArgs a)
{
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int KS = BKB / 32;                              // 32-byte K steps per stage
    constexpr int CPR = BKB / 16;                             // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                             // rows per 1-KiB DMA load
    // With two stage buffers and 8 waves, only the first wave of each SIMD
    // issues the stage loads (twice as many); the second keeps the matrix
    // core fed while the first waits on the memory pipeline.
    constexpr int DW = (NW == 8 && S == 2) ? 4 : NW;            // waves that issue loads
    constexpr int A_LD = BM / RPI / DW, B_LD = BN / RPI / DW;   // loads per such wave and stage
    constexpr int L = A_LD + B_LD;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(A_LD * DW * RPI == BM && B_LD * DW * RPI == BN, "DMA split");
    static_assert(S >= 2 && (S - 2) * L <= 63 && (S - 1) * L <= 63, "stages");
    static_assert(KS % 2 == 0, "fragment sets alternate within a stage");

    static_assert(BM <= 64 * NW && BN <= 64 * NW, "one scale per thread");
    static_assert(NW * TM * TN * 2 <= S * (BM + BN) * BKB, "output transpose fits the stages");

    // Stage buffers (A then B); after the main loop the same bytes hold the
    // bf16 output sub-tiles of the waves.  The scale area holds x_scale,
    // w_scale and bias (as fp32) of the tile's rows and columns.
    __shared__ __attribute__((aligned(1024))) int8_t smem[S * (BM + BN) * BKB];
    __shared__ __attribute__((aligned(16))) float scl[BM + 2 * BN];
    int8_t* const lds_a = smem;
    int8_t* const lds_b = smem + S * BM * BKB;

    int64_t m0, n0;
    tile_origin<BM, BN>(a, m0, n0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // This thread's row scale, column scale and bias, fetched now so that
    // their latency hides under the main loop.
    const int t = threadIdx.x;
    constexpr bool LDS_EPI = EPI == EPI_BF16 || EPI == EPI_F16;   // 16-bit output via LDS
    float t_xs = 0.0f, t_ws = 0.0f, t_b = 0.0f;
    if constexpr (LDS_EPI) {
        if (t < BM) t_xs = a.xs[min<int64_t>(m0 + t, a.m - 1) * a.xs_stride];
        if (t < BN) {
            const int64_t c = min<int64_t>(n0 + t, a.n - 1);
            t_ws = a.ws[c * a.ws_stride];
            if (a.bias) t_b = bias_at<EPI>(a.bias, c);
        }
    }

    // Per-lane byte offsets (from the tile's first row) and per-wave LDS
    // block addresses of the stage-0 buffers.
    const int8_t* a_base = a.q + m0 * a.ldq;
    const int8_t* b_base = a.w + n0 * a.ldw;
    const int a_rows = (int)min<int64_t>(BM, a.m - m0);
    const int b_rows = (int)min<int64_t>(BN, a.n - n0);
    uint32_t a_off[A_LD], a_dst[A_LD], b_off[B_LD], b_dst[B_LD];
    const uint32_t la0 = lds_addr(lds_a), lb0 = lds_addr(lds_b);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int blk = i * DW + wave % DW;
        const int row = blk * RPI + lane / CPR;
        const int chunk = (lane % CPR) ^ swz_b<BKB>(row);
        a_off[i] = (uint32_t)(min(row, a_rows - 1) * a.ldq + chunk * 16);
        a_dst[i] = la0 + blk * 1024;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int blk = i * DW + wave % DW;
        const int row = blk * RPI + lane / CPR;
        const int chunk = (lane % CPR) ^ swz_b<BKB>(row);
        b_off[i] = (uint32_t)(min(row, b_rows - 1) * a.ldw + chunk * 16);
        b_dst[i] = lb0 + blk * 1024;
    }
    const bool loader = wave < DW;
    auto issue_one = [&](int d, int buf, int64_t stage) {
        if (!loader) return;
        const uint32_t k0 = (uint32_t)(stage * BKB);
        if (d < A_LD) dma16(a_base, a_off[d] + k0, a_dst[d] + buf * (BM * BKB));
        else dma16(b_base, b_off[d - A_LD] + k0, b_dst[d - A_LD] + buf * (BN * BKB));
    };
    auto issue = [&](int buf, int64_t stage) {
#pragma unroll
        for (int d = 0; d < L; ++d) issue_one(d, buf, stage);
    };

    v16i acc[FM][FN];
    zero_acc(acc);

    // Software pipeline over K steps of 32 bytes (KS per stage), with two
    // fragment register sets used alternately: the fragments of the next
    // step are read while the current step's products run.  Before the last
    // step's products of stage j come the barrier that publishes stage j+1,
    // the DMA refill of stage j's buffer and the reads of (stage j+1,
    // step 0), so those products cover their latency.  The scheduling
    // barriers keep the compiler from regrouping the phases.
    const int64_t nk = a.k / BKB;
    if (nk > 0) {
        // Stages 0 .. S-1 in flight; loads past the last stage re-read it
        // (never used), so every stage issues exactly L loads per lane.
#pragma unroll
        for (int s = 0; s < S; ++s) issue(s, min<int64_t>(s, nk - 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * L));        // stage 0 landed
        __syncthreads();
        Frags<FM, FN> f[2];
        load_frags<FM, FN, TM, TN, BKB>(f[0], lds_a, lds_b, wm, wn, lane, 0);
        for (int64_t kt = 0; kt < nk; kt += S) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int64_t j = kt + s;
                if (j < nk) {
                    const int8_t* la = lds_a + s * (BM * BKB);
                    const int8_t* lb = lds_b + s * (BN * BKB);
                    const int nb = (s + 1) % S;
#pragma unroll
                    for (int kk = 0; kk < KS - 1; ++kk) {
                        load_frags<FM, FN, TM, TN, BKB>(f[(kk + 1) & 1], la, lb, wm, wn, lane, kk + 1);
                        __builtin_amdgcn_sched_barrier(0);
                        mfma_frags(f[kk & 1], acc);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * L));   // stage j+1 landed
                    __syncthreads();
                    const int64_t refill = min<int64_t>(j + S, nk - 1);
                    if (!IL) issue(s, refill);
                    load_frags<FM, FN, TM, TN, BKB>(f[0], lds_a + nb * (BM * BKB),
                                                    lds_b + nb * (BN * BKB), wm, wn, lane, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    const Frags<FM, FN>& fl = f[(KS - 1) & 1];
                    if (!IL) {
                        mfma_frags(fl, acc);
                    } else {
                        // one refill load after every STRIDE products, so a
                        // busy memory pipeline never holds up many of them
                        constexpr int NP = FM * FN, STRIDE = NP / L > 0 ? NP / L : 1;
                        constexpr int PER = L > NP ? (L + NP - 1) / NP : 1;   // loads per product
                        int d = 0;
#pragma unroll
                        for (int p = 0; p < NP; ++p) {
                            const int i = p / FN, jj = p % FN;
                            acc[i][jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fl.b[jj], fl.a[i],
                                                                              acc[i][jj], 0, 0, 0);
                            __builtin_amdgcn_sched_barrier(0);
                            if (p % STRIDE == STRIDE - 1) {
#pragma unroll
                                for (int e = 0; e < PER; ++e)
                                    if (d < L) {
                                        issue_one(d, s, refill);
                                        ++d;
                                    }
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
#pragma unroll
                        for (; d < L; ++d) issue_one(d, s, refill);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }

    // K tail (k % BKB bytes): one more stage, loaded through registers into
    // buffer 0 with every byte at or past k replaced by zero (exact: those
    // products are 0).  Rows are 16-byte aligned and at least k rounded up
    // to 16 bytes long, so the chunk that straddles k is readable.
    const int rem = (int)(a.k - nk * BKB);
    if (rem > 0) {
        __syncthreads();                      // every wave is done with the stages
        const int64_t kb = nk * BKB;
        constexpr int CA = BM * CPR, CB = BN * CPR;
        for (int c = t; c < CA + CB; c += 64 * NW) {
            const bool is_a = c < CA;
            const int cc = is_a ? c : c - CA;
            const int row = cc / CPR, ch = cc % CPR;
            const int start = ch * 16;
            v4i v = {0, 0, 0, 0};
            if (start < rem) {
                const int8_t* src = is_a ? a_base + (int64_t)min(row, a_rows - 1) * a.ldq
                                         : b_base + (int64_t)min(row, b_rows - 1) * a.ldw;
                v = *reinterpret_cast<const v4i*>(src + kb + start);
                if (rem - start < 16) v = keep_bytes(v, rem - start);
            }
            *reinterpret_cast<v4i*>((is_a ? lds_a : lds_b) + lds_off_b<BKB>(row, ch)) = v;
        }
        __syncthreads();
        const int steps = (rem + 31) / 32;
        for (int kk = 0; kk < steps; ++kk) {
            Frags<FM, FN> ft;
            load_frags<FM, FN, TM, TN, BKB>(ft, lds_a, lds_b, wm, wn, lane, kk);
            mfma_frags(ft, acc);
        }
    }

    if constexpr (!LDS_EPI) {
        store_tile<FM, FN, TM, TN, EPI>(a, acc, m0, n0, wm, wn, lane);
        return;
    }

    // ---- epilogue: fp32 math in registers, bf16 sub-tile through LDS, then
    // row segments of TN*2 contiguous bytes to global memory.
    __syncthreads();                          // every wave is done with the stages
    if (t < BM) scl[t] = t_xs;
    if (t < BN) {
        scl[BM + t] = t_ws;
        scl[BM + BN + t] = t_b;
    }
    __syncthreads();

    // Wave sub-tile layout: TM rows of RB = TN*2 bytes.  A 256-byte bank
    // window holds RPW rows; (row, 16-byte chunk, 8-byte half) of a value
    // written by lane L is permuted so that 32 lanes writing 8 bytes each on
    // 32 consecutive rows hit 32 distinct 8-byte slots of one window, and 16
    // lanes reading 16 consecutive chunks hit 16 distinct 16-byte slots.
    constexpr int RB = TN * 2, CH = RB / 16, RPW = 256 / RB;
    static_assert(RPW * CH == 16, "window geometry");
    int8_t* const wt = smem + wave * (TM * RB);
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    // The lane's scale operands leave LDS in one batch ahead of the
    // arithmetic: rows i*32 + frag_row, columns j*32 + g*8 + 4*half + e.
    float xsr[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) xsr[i] = scl[wm * TM + i * 32 + frag_row];
    auto convert = [&](auto bias_tag) {
        constexpr bool HB = decltype(bias_tag)::value;
        v4i wsr[FN][4], bsr[FN][4];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = wn * TN + j * 32 + g * 8 + 4 * half;
                wsr[j][g] = *reinterpret_cast<const v4i*>(&scl[BM + c0]);
                if constexpr (HB) bsr[j][g] = *reinterpret_cast<const v4i*>(&scl[BM + BN + c0]);
            }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = i * 32 + frag_row;
            const int cx = (r / RPW) % CH;
            const int hx = (r / (RPW * CH)) & 1;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float b = 0.0f;
                        if constexpr (HB) b = __int_as_float(bsr[j][g][e]);
                        v[e] = epilogue_value(acc[i][j][4 * g + e], xsr[i],
                                              __int_as_float(wsr[j][g][e]), b, HB);
                    }
                    const int cc = (j * 32 + g * 8 + 4 * half) >> 3;
                    const int off = r * RB + ((cc ^ cx) << 4) + ((half ^ hx) << 3);
                    *reinterpret_cast<uint2*>(wt + off) =
                        make_uint2(pack2<EPI>(v[0], v[1]), pack2<EPI>(v[2], v[3]));
                }
        }
    };
    if (a.bias) convert(BoolTag<true>{});
    else convert(BoolTag<false>{});
    // Each wave reads back only its own sub-tile: LDS operations of one wave
    // complete in order, so no barrier is needed here.  All reads go out
    // before the first store.
    uint16_t* const out = reinterpret_cast<uint16_t*>(a.out);
    const int64_t row0 = m0 + wm * TM, col0 = n0 + wn * TN;
    const bool full = row0 + TM <= a.m && col0 + TN <= a.n && a.vec_store == 2;
    constexpr int NV = TM * CH / 64;                          // 16-byte chunks per lane
    static_assert((TM * CH) % 64 == 0, "chunks per lane");
    v4i ov[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int c = u * 64 + lane;
        const int r = c / CH, cc = c % CH;
        v4i v = *reinterpret_cast<const v4i*>(wt + r * RB + ((cc ^ ((r / RPW) % CH)) << 4));
        if ((r / (RPW * CH)) & 1) v = v4i{v[2], v[3], v[0], v[1]};
        ov[u] = v;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int c = u * 64 + lane;
        const int r = c / CH, cc = c % CH;
        const int64_t gm = row0 + r, gn = col0 + cc * 8;
        uint16_t* dst = out + gm * a.ldo + gn;
        const v4i v = ov[u];
        // Streaming (non-temporal) stores when the launch has several waves
        // of blocks: the output is not read again by this kernel, and
        // keeping it out of the way of the A and B panels in L2 measured 3-4 %
        // faster on 80666x28672x5376 and 99900x21504x5376 (and 1 % slower on
        // the single-wave 4096^3).
        auto put = [&](uint16_t* p, v4i v) {
            if (a.stream_out) __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(p));
            else *reinterpret_cast<v4i*>(p) = v;
        };
        if (full) {
            put(dst, v);
        } else if (gm < a.m) {
            if (a.vec_store == 2 && gn + 8 <= a.n) {
                put(dst, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (gn + e < a.n) dst[e] = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Persistent variant of tile 12 (k a positive multiple of 128, bf16 / fp16
// output)
// ---------------------------------------------------------------------------
// One block per CU claims tiles one after another (claim_start /
// claim_finish).  What this saves over one block per tile: the wait for a
// tile's first K stages, which load while the previous tile's epilogue
// runs; the gap between blocks on a CU; and the idling of fast XCDs, which
// take over tiles of slow ones.
//   - The row and column scales and the bias of a tile are copied straight
//     into LDS (two buffers, so the next tile's copy never meets the
//     current one); nothing is held in registers across the main loop.
//   - The main loop reads and loads nothing past the tile's last K stage,
//     so once every wave has passed its last barrier both stage buffers
//     are free.
//   - In the epilogue every wave converts its accumulators one 32 x 32
//     fragment at a time through a private 2 KiB LDS region and writes them
//     out, while the loaders (waves 0-3, as in tile 12) spread the loads of
//     the next tile's scales and K stages 0 and 1 over that work.
// Loads and stores of a wave complete in order, so at the start of a tile
// the loaders wait until at most the operations issued after stage 0 are
// pending.
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds)
{
    asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Each lane's 16-bit value lands in the low half of its own 4-byte LDS slot.
__device__ __forceinline__ void dma2(const void* base, uint32_t voff, uint32_t lds)
{
    asm volatile("global_load_lds_ushort %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Tile claiming of the persistent kernels.  The grouped tile order is cut
// into 8 equal ranges, one per XCD (block b runs on XCD b % 8), plus the
// last num % 8 tiles.  sched[x] counts the tiles of range x handed out,
// sched[8] those of the rest, sched[9] the blocks that have finished.  A
// block takes tiles of its own XCD's range first, so that the XCD's L2 sees
// neighbouring tiles, then tiles left in the other ranges and the rest: an
// XCD that runs faster than the others helps them finish instead of
// idling.  A claim is split in two: claim_start issues the atomic on the
// block's own range, claim_finish (later, when its result has arrived)
// turns it into a tile id or, once the own range is empty, looks for tiles
// elsewhere.  Called by one lane of the block.
struct Claims {
    bool own_done;
    unsigned emptied;                          // other ranges seen exhausted
};

__device__ __forceinline__ unsigned claim_start(unsigned* sched, const Claims& c)
{
    if (c.own_done) return ~0u;
    // The address as a per-lane value in the global address space: the
    // compiler then issues this one atomic as is (a global, not a flat,
    // atomic, so that waits on LDS operations never wait for it), instead
    // of its wave-wide form whose result it reads back, and so waits for,
    // right away.
    uint64_t addr = (uint64_t)(uintptr_t)(sched + (blockIdx.x & 7));
    asm volatile("" : "+v"(addr));
    auto* p = (__attribute__((address_space(1))) unsigned*)addr;
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int claim_finish(unsigned* sched, int num, unsigned t, Claims& c)
{
    const unsigned per = (unsigned)num >> 3, rest = (unsigned)num & 7;
    const int x = blockIdx.x & 7;
    if (!c.own_done) {
        if (t < per) return (int)(x * per + t);
        c.own_done = true;
    }
    for (int d = 1; d < 8; ++d) {
        const int y = (x + d) & 7;
        if (c.emptied & (1u << y)) continue;
        if (__hip_atomic_load(sched + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < per) {
            const unsigned u = atomicAdd(sched + y, 1u);
            if (u < per) return (int)(y * per + u);
        }
        c.emptied |= 1u << y;
    }
    const unsigned u = atomicAdd(sched + 8, 1u);
    return u < rest ? (int)(8 * per + u) : -1;
}

// After the block's last claim: the last block to get here clears the
// counters for the next launch on the stream.
__device__ __forceinline__ void claims_done(unsigned* sched)
{
    __threadfence();
    if (atomicAdd(sched + 9, 1u) == gridDim.x - 1) {
        __threadfence();
        for (int q = 0; q < 10; ++q)
            __hip_atomic_store(sched + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int EPI>
__device__ __forceinline__ float bias_from_bits(uint32_t bits)
{
    if constexpr (EPI == EPI_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    else return __uint_as_float(bits << 16);
}

template <int BM, int BN, int WM, int WN, int EPI, bool HB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_persist_kernel(GemmArgs a)
{
    // HB: the launch has a bias (without one the add, one fp32 operation of
    // five per output, is left out of the epilogue)
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int S = 2, BKB = 128, KS = BKB / 32, CPR = BKB / 16, RPI = 64 / CPR;
    constexpr int DW = NW / 2;                                  // loader waves
    constexpr int A_LD = BM / RPI / DW, B_LD = BN / RPI / DW, L = A_LD + B_LD;
    constexpr int SCL = BM + 2 * BN;                            // floats per scale buffer
    constexpr int G0 = 6, G1 = 5, G2 = L - G0 - G1;             // refill loads per step, see the main loop
    static_assert(G0 <= FM * FN && G1 <= FM * FN && G2 >= 0 && G2 <= FM * FN && KS >= 3, "refill groups");
    // Output staging: one 32 x 32 fragment (2 KiB of 16-bit values) per wave.
    constexpr int RB = 64, CH = RB / 16, RPW = 256 / RB;        // region row bytes, chunks, rows per window
    constexpr int REG = 32 * RB;                                // bytes of a wave's region
    constexpr int NV = 32 * CH / 64;                            // 16-byte chunks per lane and region
    constexpr int NF = FM * FN;                                 // fragments per wave
    static_assert(NW == 8 && DW * 2 == NW && DW * 64 == BM && BM == BN, "roles");
    static_assert(A_LD * DW * RPI == BM && B_LD * DW * RPI == BN, "load split");
    // At most 3 + 2*L loads and NF*NV stores per tile go out between waits.
    static_assert(3 + 2 * L + NF * NV <= 63, "wait count");
    // The epilogue issues one load after each group of four outputs and a
    // fragment's stores after the next fragment's loads; after a full tile,
    // the stores of the fragment before the one that carries the last
    // stage-0 load and of every later one, and all of stage 1, follow
    // stage 0.
    constexpr int PEND_FULL = L + NV * (NF - (L - 1) / 4 + 1);
    static_assert((L - 1) / 4 >= 1 && (L - 1) / 4 < NF, "stage 0 ends inside the epilogue");
    static_assert(RPW * CH == 16 && (32 * CH) % 64 == 0, "region geometry");
    static_assert(2 * L <= NF * 4, "epilogue loads fit the output groups");
    // EPI_I32 (the raw accumulators, for checking them) runs the same tile
    // walk and main loop; its epilogue stores straight from the registers
    // and it loads no scales.
    constexpr bool I32 = EPI == EPI_I32;
    static_assert(EPI == EPI_BF16 || EPI == EPI_F16 || (I32 && !HB), "16-bit or int32 outputs");

    __shared__ __attribute__((aligned(1024))) int8_t smem[S * (BM + BN) * BKB];
    __shared__ __attribute__((aligned(16))) float scl[2 * SCL];
    __shared__ __attribute__((aligned(16))) int8_t ostage[NW * REG];
    __shared__ int tile_ids[2];                                 // ids of the next two tiles
    int8_t* const lds_a = smem;
    int8_t* const lds_b = smem + S * BM * BKB;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const bool loader = wave < DW;
    const int num_tiles = a.tiles_m * a.tiles_n;
    const int64_t nk = a.k / BKB;
    // The lane id as an opaque value, so that per-lane address arithmetic of
    // the once-per-tile code is done where it is used instead of being
    // hoisted out of the tile loop and held (spilled) across the main loop.
    auto lane_now = [&]() {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };

    uint32_t a_dst[A_LD], b_dst[B_LD];
    const uint32_t la0 = lds_addr(lds_a), lb0 = lds_addr(lds_b);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) a_dst[i] = la0 + (i * DW + wave % DW) * 1024;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) b_dst[i] = lb0 + (i * DW + wave % DW) * 1024;

    // Per-tile state: origin, operand bases and per-lane offsets.
    int64_t m0 = 0, n0 = 0;
    int a_rows = 1, b_rows = 1;
    const int8_t* a_base = a.q;
    const int8_t* b_base = a.w;
    uint32_t a_off[A_LD], b_off[B_LD];
    // The per-lane offsets depend on the tile only through the clamping of
    // rows past the edge, so they are recomputed only for edge tiles and
    // for the first tile after one.
    bool clamped = true;
    auto setup = [&](int id) {
        grouped_origin<BM, BN>(a, id, m0, n0);
        a_base = a.q + m0 * a.ldq;
        b_base = a.w + n0 * a.ldw;
        a_rows = (int)min<int64_t>(BM, a.m - m0);
        b_rows = (int)min<int64_t>(BN, a.n - n0);
        const bool edge = a_rows < BM || b_rows < BN;
        if (!edge && !clamped) return;
        clamped = edge;
        const int ln = lane_now();
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int row = (i * DW + wave % DW) * RPI + ln / CPR;
            const int chunk = (ln % CPR) ^ swz_b<BKB>(row);
            a_off[i] = (uint32_t)(min(row, a_rows - 1) * a.ldq + chunk * 16);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int row = (i * DW + wave % DW) * RPI + ln / CPR;
            const int chunk = (ln % CPR) ^ swz_b<BKB>(row);
            b_off[i] = (uint32_t)(min(row, b_rows - 1) * a.ldw + chunk * 16);
        }
    };
    // Three loads per loader lane: x scale of row 64*wave + lane, w scale
    // and bias of that column (rows and columns past the edge repeat the
    // last one).  Without a bias the third load repeats the w scale, so the
    // count never changes.
    auto issue_scales = [&](int buf) {
        if (I32 || !loader) return;
        const uint32_t sb = lds_addr(scl + buf * SCL) + wave * 256;
        const int ln = lane_now();
        const int r = min(wave * 64 + ln, a_rows - 1);
        const int c = min(wave * 64 + ln, b_rows - 1);
        const float* ws = a.ws + n0 * a.ws_stride;
        dma4(a.xs + m0 * a.xs_stride, (uint32_t)(r * a.xs_stride * 4), sb);
        dma4(ws, (uint32_t)(c * a.ws_stride * 4), sb + BM * 4);
        if constexpr (HB) dma2(static_cast<const uint16_t*>(a.bias) + n0, (uint32_t)(c * 2), sb + (BM + BN) * 4);
        else dma4(ws, (uint32_t)(c * a.ws_stride * 4), sb + (BM + BN) * 4);
    };
    auto issue_one = [&](int d, int buf, int64_t stage) {
        if (!loader) return;
        const uint32_t k0 = (uint32_t)(stage * BKB);
        if (d < A_LD) dma16(a_base, a_off[d] + k0, a_dst[d] + buf * (BM * BKB));
        else dma16(b_base, b_off[d - A_LD] + k0, b_dst[d - A_LD] + buf * (BN * BKB));
    };
    auto issue = [&](int buf, int64_t stage) {
#pragma unroll
        for (int d = 0; d < L; ++d) issue_one(d, buf, stage);
    };

    // Tile claiming (claim_start / claim_finish): one lane claims the ids
    // two tiles ahead; the atomic goes out at the top of a tile and its
    // result is used at the start of the epilogue, so its latency hides
    // under the main loop.
    const bool sched_lane = wave == DW && threadIdx.x == 64 * DW;
    Claims claims{false, 0u};
    if (sched_lane) {
        const int t0 = claim_finish(a.sched, num_tiles, claim_start(a.sched, claims), claims);
        tile_ids[0] = t0;
        tile_ids[1] = t0 >= 0 ? claim_finish(a.sched, num_tiles, claim_start(a.sched, claims), claims)
                              : -1;
    }
    __syncthreads();
    int tile = __builtin_amdgcn_readfirstlane(tile_ids[0]), cur = 0, it = 0;
    unsigned pending = 0;                                       // sched lane: claim_start's result
    bool stores_pending = false;     // the wave's last epilogue issued exactly NF*NV stores
    if (tile < 0) {                  // (tile is the same for the whole block)
        if (sched_lane) claims_done(a.sched);
        return;
    }
    setup(tile);
    issue_scales(0);
    issue(0, 0);
    issue(1, min<int64_t>(1, nk - 1));

    uint16_t* const out = reinterpret_cast<uint16_t*>(a.out);
    v16i acc[FM][FN];
    for (;; ++it) {
        zero_acc(acc);
        // scales + stage 0 landed (loads and stores complete in order, so
        // only what was issued after stage 0 may still be pending: stage 1
        // and, after a full tile, the output stores counted in PEND_FULL)
        if (loader) {
            if (I32) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));     // every store and load done
            else if (stores_pending) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PEND_FULL));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));
        }
        __syncthreads();
        // The bias slots become fp32 in place, so that the epilogue adds a
        // float with no conversion.
        if constexpr (HB) {
            if (loader) {
                float* bs = scl + cur * SCL + BM + BN + wave * 64 + lane_now();
                *bs = bias_from_bits<EPI>(__float_as_uint(*bs));
            }
        }
        if (sched_lane && tile_ids[(it + 1) & 1] >= 0) pending = claim_start(a.sched, claims);
        Frags<FM, FN> f[2];
        load_frags<FM, FN, TM, TN, BKB>(f[0], lds_a, lds_b, wm, wn, lane, 0);
        for (int64_t kt = 0; kt < nk; kt += S) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int64_t j = kt + s;
                if (j < nk) {
                    const int8_t* la = lds_a + s * (BM * BKB);
                    const int8_t* lb = lds_b + s * (BN * BKB);
                    const int nb = s ^ 1;
                    // The L loads that refill a stage buffer go out one after
                    // each product, in three groups: G0 in the last step of
                    // stage j (once the barrier has freed the buffer), G1 and
                    // G2 in the first two steps of stage j+1.  A wave whose
                    // load waits on the memory pipeline holds back its next
                    // product; spread out, the loads measured 2-2.5 % faster
                    // than all L in one step.  Here the rest of stage j+1's
                    // loads (issued from stage j-1) go out.
                    const bool rest = j > 0 && j + 1 < nk;
#pragma unroll
                    for (int kk = 0; kk < KS - 1; ++kk) {
                        load_frags<FM, FN, TM, TN, BKB>(f[(kk + 1) & 1], la, lb, wm, wn, lane, kk + 1);
                        __builtin_amdgcn_sched_barrier(0);
                        const Frags<FM, FN>& fk = f[kk & 1];
                        const int first = kk == 0 ? G0 : G0 + G1;
                        const int count = kk == 0 ? G1 : kk == 1 ? G2 : 0;
#pragma unroll
                        for (int p = 0; p < FM * FN; ++p) {
                            const int i = p / FN, jj = p % FN;
                            acc[i][jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fk.b[jj], fk.a[i],
                                                                              acc[i][jj], 0, 0, 0);
                            __builtin_amdgcn_sched_barrier(0);
                            if (p < count && rest) issue_one(first + p, s ^ 1, j + 1);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    if (loader) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // stage j+1 landed
                    __syncthreads();
                    // Past the last stage nothing is read or loaded, so once
                    // every wave is through this barrier the stage buffers
                    // are free for the next tile.
                    const int64_t refill = j + S;
                    const bool more_k = refill < nk;
                    if (j + 1 < nk)
                        load_frags<FM, FN, TM, TN, BKB>(f[0], lds_a + nb * (BM * BKB),
                                                        lds_b + nb * (BN * BKB), wm, wn, lane, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    const Frags<FM, FN>& fl = f[(KS - 1) & 1];
                    constexpr int NP = FM * FN;
                    int d = 0;
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        const int i = p / FN, jj = p % FN;
                        acc[i][jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fl.b[jj], fl.a[i],
                                                                          acc[i][jj], 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        if (d < G0) {
                            if (more_k) issue_one(d, s, refill);
                            ++d;
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        if (loader) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

        // ---- epilogue of this tile, prologue of the next
        const int next = __builtin_amdgcn_readfirstlane(tile_ids[(it + 1) & 1]);
        const bool more = next >= 0;
        // the slot of this tile's id takes the id two tiles ahead (read after
        // the next tile's barriers)
        if (sched_lane)
            tile_ids[it & 1] = next >= 0 ? claim_finish(a.sched, num_tiles, pending, claims) : -1;
        const int64_t cm0 = m0, cn0 = n0;
        const float* const sc = scl + cur * SCL;
        if (more) {
            setup(next);
            issue_scales(cur ^ 1);
        }
        if constexpr (I32) {
            // The raw accumulators, stored straight from the registers: lane
            // L holds row L % 32 of each 32 x 32 fragment and, per group g,
            // the four columns 8g + 4 (L / 32) + 0..3 (16 bytes).  The
            // loaders issue the next tile's stages 0 and 1 at the cadence of
            // the 16-bit epilogue, one load per group of four outputs.
            int32_t* const oi = reinterpret_cast<int32_t*>(a.out);
            const int ln = lane_now();
            const int r = ln & 31, half = ln >> 5;
            const int64_t stage1 = min<int64_t>(1, nk - 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jn = 0; jn < FN; ++jn)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int e = (i * FN + jn) * 4 + g;
                        if (more && e < 2 * L) {
                            if (e < L) issue_one(e, 0, 0);
                            else issue_one(e - L, 1, stage1);
                        }
                        const int64_t gm = cm0 + wm * TM + i * 32 + r;
                        const int64_t gn = cn0 + wn * TN + jn * 32 + g * 8 + 4 * half;
                        if (gm >= a.m) continue;
                        int32_t* dst = oi + gm * a.ldo + gn;
                        const v4i v = {acc[i][jn][4 * g + 0], acc[i][jn][4 * g + 1],
                                       acc[i][jn][4 * g + 2], acc[i][jn][4 * g + 3]};
                        if (a.vec_store && gn + 3 < a.n) {
                            *reinterpret_cast<v4i*>(dst) = v;
                        } else {
#pragma unroll
                            for (int c = 0; c < 4; ++c)
                                if (gn + c < a.n) dst[c] = v[c];
                        }
                    }
        } else {
            // Each wave converts its sub-tile one 32 x 32 fragment at a time
            // through its own region and writes it out as 32 row segments of 64
            // bytes.  A wave reads back only what it wrote, and LDS operations
            // of one wave complete in order, so no barrier is needed.  Meanwhile
            // the loaders issue the next tile's K stages 0 and 1, one load per
            // group of four outputs.
            int8_t* const reg = ostage + wave * REG;
            const int ln = lane_now();
            const int r = ln & 31;                                  // row within the fragment
            const int half = ln >> 5;
            const int cx = (r / RPW) % CH;
            const int hx = (r / (RPW * CH)) & 1;
            const bool full = cm0 + wm * TM + TM <= a.m && cn0 + wn * TN + TN <= a.n && a.vec_store == 2;
            const int64_t stage1 = min<int64_t>(1, nk - 1);
            v4i wsr[FN][4], bsr[FN][4];
    #pragma unroll
            for (int jn = 0; jn < FN; ++jn)
    #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c0 = wn * TN + jn * 32 + g * 8 + 4 * half;
                    wsr[jn][g] = *reinterpret_cast<const v4i*>(&sc[BM + c0]);
                    if constexpr (HB) bsr[jn][g] = *reinterpret_cast<const v4i*>(&sc[BM + BN + c0]);
                }
            // A fragment's row segments go out after the next fragment is
            // converted, so that the LDS latency of reading it back is hidden.
            auto store_frag = [&](const v4i (&ov)[NV], int64_t row0, int64_t col0) {
    #pragma unroll
                for (int u = 0; u < NV; ++u) {
                    const int c = u * 64 + ln;
                    const int64_t gm = row0 + c / CH, gn = col0 + (c % CH) * 8;
                    uint16_t* dst = out + gm * a.ldo + gn;
                    if (full) {
                        __builtin_nontemporal_store(ov[u], reinterpret_cast<v4i*>(dst));
                    } else if (gm < a.m && gn < a.n) {
                        // edge tiles: element stores where a row ends inside a chunk
                        if (a.vec_store == 2 && gn + 8 <= a.n) {
                            *reinterpret_cast<v4i*>(dst) = ov[u];
                        } else {
                            for (int e = 0; e < 8 && gn + e < a.n; ++e)
                                dst[e] = (uint16_t)((uint32_t)ov[u][e >> 1] >> (16 * (e & 1)));
                        }
                    }
                }
            };
            v4i ov[NV];
            int64_t prow0 = 0, pcol0 = 0;
    #pragma unroll
            for (int i = 0; i < FM; ++i) {
                const float xsv = sc[wm * TM + i * 32 + r];
    #pragma unroll
                for (int jn = 0; jn < FN; ++jn) {
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float v[4];
    #pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = epilogue_value(acc[i][jn][4 * g + e], xsv, __int_as_float(wsr[jn][g][e]),
                                                  HB ? __int_as_float(bsr[jn][g][e]) : 0.0f, HB);
                        *reinterpret_cast<uint2*>(reg + r * RB + ((g ^ cx) << 4) + ((half ^ hx) << 3)) =
                            make_uint2(pack2<EPI>(v[0], v[1]), pack2<EPI>(v[2], v[3]));
                        const int e = (i * FN + jn) * 4 + g;
                        if (more && e < 2 * L) {
                            if (e < L) issue_one(e, 0, 0);          // stage 0 -> buffer 0
                            else issue_one(e - L, 1, stage1);       // stage 1 -> buffer 1
                        }
                    }
                    if (i + jn > 0) store_frag(ov, prow0, pcol0);  // the previous fragment
    #pragma unroll
                    for (int u = 0; u < NV; ++u) {
                        const int c = u * 64 + ln;
                        const int rr = c / CH, cc = c % CH;
                        v4i vv = *reinterpret_cast<const v4i*>(reg + rr * RB + ((cc ^ ((rr / RPW) % CH)) << 4));
                        if ((rr / (RPW * CH)) & 1) vv = v4i{vv[2], vv[3], vv[0], vv[1]};
                        ov[u] = vv;
                    }
                    prow0 = cm0 + wm * TM + i * 32;
                    pcol0 = cn0 + wn * TN + jn * 32;
                }
            }
            store_frag(ov, prow0, pcol0);
            stores_pending = full;
        }
        if (!more) break;
        tile = next;
        cur ^= 1;
    }
    if (sched_lane) claims_done(a.sched);
}

// ---------------------------------------------------------------------------
// Dequant-on-the-fly path (W8A16): bf16 x times the int8 weight, which is
// turned into bf16 (w * w_scale) on its way into LDS, on bf16 matrix cores
// ---------------------------------------------------------------------------
// #278 "int8_linear silently falls back ...", "Suggested fix": dequantise
// the int8 weight to the 16-bit compute type on the fly and multiply on the
// 16-bit matrix cores; x is not quantised and the weight stays int8 in HBM.
// The dequantised value is bf16(fp32(w) * w_scale[j]); products of two bf16
// values are exact in fp32 and v_mfma_f32_32x32x16_bf16 accumulates them in
// fp32; the epilogue adds the bias and rounds to the output type.
//
// Same block structure as gemm_dma_kernel with 128-byte stages: a stage is
// 64 K elements, i.e. 128 bytes of a bf16 x row (copied by direct-to-LDS
// loads into the same swizzled layout) and 64 bytes of an int8 W row.  W
// arrives by direct-to-LDS loads too, into a staging buffer; each lane then
// reads back the 16 bytes its own load wrote (so no barrier is needed),
// dequantises them and writes 32 bytes of bf16 into the W stage buffer, in
// the swizzled 128-byte layout.  A 16-byte fragment is then 8 bf16 of K and
// one MFMA step covers 16 K elements, so the fragment reads are the int8
// kernel's unchanged.  LDS: two stages of x and of bf16 W plus two int8
// staging buffers, 160 KiB for 256 x 256 blocks.  GemmArgs carries x as q
// with ldq in bytes (2 * ldx) and k in elements.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16 int8 weights times their row's scale, rounded to bf16: 32 bytes.
__device__ __forceinline__ void dequant16(const v4i w, float s, v4i& lo, v4i& hi)
{
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t u = (uint32_t)w[d];
        const float f0 = (float)(int8_t)(u & 0xffu) * s;
        const float f1 = (float)(int8_t)((u >> 8) & 0xffu) * s;
        const float f2 = (float)(int8_t)((u >> 16) & 0xffu) * s;
        const float f3 = (float)(int8_t)(u >> 24) * s;
        o[2 * d] = bf16x2_rne_bits(f0, f1);
        o[2 * d + 1] = bf16x2_rne_bits(f2, f3);
    }
    lo = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    hi = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
}

template <int FM, int FN>
__device__ __forceinline__ void mfma_bf16_frags(const Frags<FM, FN>& f, f32x16 (&acc)[FM][FN])
{
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, f.b[j]), __builtin_bit_cast(bf16x8, f.a[i]),
                acc[i][j], 0, 0, 0);
}

// Epilogue of the fp32 accumulators: out = round_out(acc + bias), stored
// straight from registers (four consecutive columns of one row per lane and
// group).
template <int FM, int FN, int TM, int TN, int EPI>
__device__ __forceinline__ void store_tile_f32(const GemmArgs& a, const f32x16 (&acc)[FM][FN],
                                               int64_t m0, int64_t n0, int wm, int wn, int lane)
{
    const int frag_row = lane & 31;
    const int col_off = 4 * (lane >> 5);
    const bool has_bias = a.bias != nullptr;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t gn = n0 + wn * TN + j * 32 + g * 8 + col_off;
            float bv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bv[e] = has_bias ? bias_at<EPI>(a.bias, gn + e < a.n ? gn + e : 0) : 0.0f;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int64_t gm = m0 + wm * TM + i * 32 + frag_row;
                if (gm >= a.m || gn >= a.n) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[i][j][4 * g + e];
                    if (has_bias) v[e] = v[e] + bv[e];
                }
                if constexpr (EPI == EPI_F32) {
                    float* orow = reinterpret_cast<float*>(a.out) + gm * a.ldo;
                    if (a.vec_store && gn + 3 < a.n) {
                        *reinterpret_cast<float4*>(orow + gn) = make_float4(v[0], v[1], v[2], v[3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (gn + e < a.n) orow[gn + e] = v[e];
                    }
                } else {
                    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + gm * a.ldo;
                    const uint32_t p0 = pack2<EPI>(v[0], v[1]), p1 = pack2<EPI>(v[2], v[3]);
                    if (a.vec_store && gn + 3 < a.n) {
                        *reinterpret_cast<uint2*>(orow + gn) = make_uint2(p0, p1);
                    } else {
                        const uint32_t h[4] = {p0 & 0xffffu, p0 >> 16, p1 & 0xffffu, p1 >> 16};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (gn + e < a.n) orow[gn + e] = (uint16_t)h[e];
                    }
                }
            }
        }
}

// 16-bit outputs of an interior tile through LDS: each wave packs its
// TM x TN sub-tile (bias added in fp32, as in store_tile_f32) into its own
// region of the freed stage buffers, rows of TN * 2 bytes with the 16-byte
// chunks swizzled as in the stage buffers, then reads it back a row segment
// at a time and stores whole segments (16 bytes per lane, TN * 2 bytes per
// row): stores straight from the accumulators write 16 bytes per row and
// instruction, and the memory side counted 3.6 times the output for them.
// Needs out rows 16-byte aligned (vec_store == 2).
template <int FM, int FN, int TM, int TN, int EPI>
__device__ __forceinline__ void store_tile_lds16(const GemmArgs& a, const f32x16 (&acc)[FM][FN],
                                                 int64_t m0, int64_t n0, int wm, int wn, int lane,
                                                 int8_t* region)
{
    constexpr int RB = TN * 2;               // bytes of a row segment
    constexpr int CPR = RB / 16;             // 16-byte chunks per row
    constexpr int RPS = 64 / CPR;            // rows per read-back instruction
    static_assert(TM % RPS == 0, "read-back rows");
    const int frag_row = lane & 31;
    const int half = lane >> 5;              // columns 4 * half .. + 3 of each group of 8
    const bool has_bias = a.bias != nullptr;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int col = j * 32 + g * 8 + 4 * half;
            float bv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bv[e] = has_bias ? bias_at<EPI>(a.bias, n0 + wn * TN + col + e) : 0.0f;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = i * 32 + frag_row;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[i][j][4 * g + e];
                    if (has_bias) v[e] = v[e] + bv[e];
                }
                const uint2 packed = make_uint2(pack2<EPI>(v[0], v[1]), pack2<EPI>(v[2], v[3]));
                *reinterpret_cast<uint2*>(region + row * RB + (((col >> 3) ^ swz_b<RB>(row)) << 4) +
                                          half * 8) = packed;
            }
        }
    const int c = lane % CPR;
    uint16_t* const out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
    for (int r0 = 0; r0 < TM; r0 += RPS) {
        const int row = r0 + lane / CPR;
        const v4i v = *reinterpret_cast<const v4i*>(region + row * RB + ((c ^ swz_b<RB>(row)) << 4));
        v4i* dst = reinterpret_cast<v4i*>(out + (m0 + wm * TM + row) * a.ldo + n0 + wn * TN + c * 8);
        if (a.stream_out) __builtin_nontemporal_store(v, dst);
        else *dst = v;
    }
}

constexpr int dq_lds_bytes(int bm, int bn) { return 2 * (bm + bn) * 128 + 2 * bn * 64; }

template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void dq_tile(const GemmArgs& a, int64_t m0, int64_t n0, int8_t* smem)
{
    constexpr int NW = WM * WN, NT = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int BKB = 128;                  // bytes of a stage row in LDS (64 bf16)
    constexpr int KE = 64;                    // K elements per stage
    constexpr int KS = 4;                     // 16-element MFMA steps per stage
    constexpr int CPR = 8, RPI = 8;           // x: 16-byte chunks per row, rows per 1-KiB load
    constexpr int A_LD = BM / RPI / NW;       // x loads per wave per stage
    constexpr int B_LD = BN / 16 / NW;        // W loads per wave per stage (16 rows x 64 bytes)
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(A_LD * NW * RPI == BM && A_LD >= 1, "x split");
    static_assert(B_LD * NW * 16 == BN && B_LD >= 1, "W split");

    // smem: 2 * (BM + BN) * 128 + 2 * BN * 64 bytes, 1 KiB aligned
    int8_t* const lds_a = smem;                           // 2 x [BM rows x 128 B]
    int8_t* const lds_b = smem + 2 * BM * BKB;            // 2 x [BN rows x 128 B] bf16
    int8_t* const lds_w = smem + 2 * (BM + BN) * BKB;     // 2 x [BN rows x 64 B] int8 staging

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int t = threadIdx.x;
    const int a_rows = (int)min<int64_t>(BM, a.m - m0);
    const int b_rows = (int)min<int64_t>(BN, a.n - n0);

    const int8_t* a_base = a.q + m0 * a.ldq;
    const int8_t* w_base = a.w + n0 * a.ldw;
    uint32_t a_off[A_LD], a_dst[A_LD], w_off[B_LD], w_dst[B_LD];
    int w_row[B_LD];
    float w_scl[B_LD];
    const uint32_t la0 = lds_addr(lds_a), lw0 = lds_addr(lds_w);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int blk = i * NW + wave;
        const int row = blk * RPI + lane / CPR;
        const int chunk = (lane % CPR) ^ swz_b<BKB>(row);
        a_off[i] = (uint32_t)(min(row, a_rows - 1) * a.ldq + chunk * 16);
        a_dst[i] = la0 + blk * 1024;
    }
    // W load i of this wave: rows 16*blk .. +15, lane L takes row 16*blk + L/4
    // and the 16 bytes (L%4)*16 of the stage, and writes them at blk*1024 + 16L.
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int blk = i * NW + wave;
        const int row = blk * 16 + lane / 4;
        const int grow = min(row, b_rows - 1);
        w_off[i] = (uint32_t)(grow * a.ldw + (lane % 4) * 16);
        w_dst[i] = lw0 + blk * 1024;
        w_row[i] = row;
        w_scl[i] = a.ws[(n0 + grow) * a.ws_stride];
    }
    auto issue_x = [&](int buf, int64_t stage) {
#pragma unroll
        for (int d = 0; d < A_LD; ++d)
            dma16(a_base, a_off[d] + (uint32_t)(stage * BKB), a_dst[d] + buf * (BM * BKB));
    };
    auto issue_w = [&](int buf, int64_t stage) {
#pragma unroll
        for (int d = 0; d < B_LD; ++d)
            dma16(w_base, w_off[d] + (uint32_t)(stage * KE), w_dst[d] + buf * (BN * KE));
    };
    // This lane's staged W bytes of buffer buf -> bf16 W stage buffer buf.
    auto convert = [&](int buf) {
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int blk = i * NW + wave;
            const v4i wv = *reinterpret_cast<const v4i*>(lds_w + buf * (BN * KE) + blk * 1024 + lane * 16);
            v4i lo, hi;
            dequant16(wv, w_scl[i], lo, hi);
            const int c0 = (lane % 4) * 2;
            int8_t* base = lds_b + buf * (BN * BKB);
            *reinterpret_cast<v4i*>(base + lds_off_b<BKB>(w_row[i], c0)) = lo;
            *reinterpret_cast<v4i*>(base + lds_off_b<BKB>(w_row[i], c0 + 1)) = hi;
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Loads run ahead of the products: x of stage j+2 goes out in the last
    // K step of stage j, W of stage j+2 in its first, right after W of stage
    // j+1 has been dequantised (not just before a barrier, where every wave
    // would do it at once); before the barrier that publishes stage j+1 a
    // wave waits for its x loads only.
    // A wave's loads complete in order, so each wait allows as many pending
    // loads as were issued after the one it needs; near the end of K, where
    // fewer follow, it waits for fewer.  Buffers: x and bf16 W of stage j in
    // s = j % 2; int8 W of stage j in staging buffer j % 2, which is free once
    // stage j has been dequantised and published.
    const int64_t nk = a.k / KE;
    if (nk > 0) {
        issue_w(0, 0);
        issue_x(0, 0);
        if (nk > 1) {
            issue_w(1, 1);
            wait_vmcnt<A_LD + B_LD>();                 // W of stage 0 landed
        } else {
            wait_vmcnt<A_LD>();
        }
        convert(0);
        if (nk > 1) wait_vmcnt<B_LD>();                // x of stage 0 landed
        else wait_vmcnt<0>();
        __syncthreads();                               // stage 0 published
        if (nk > 1) issue_x(1, 1);
        Frags<FM, FN> f[2];
        load_frags<FM, FN, TM, TN, BKB>(f[0], lds_a, lds_b, wm, wn, lane, 0);
        for (int64_t kt = 0; kt < nk; kt += 2) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int64_t j = kt + s;
                if (j < nk) {
                    const int8_t* la = lds_a + s * (BM * BKB);
                    const int8_t* lb = lds_b + s * (BN * BKB);
                    const int nb = s ^ 1;
                    const bool more1 = j + 1 < nk, more2 = j + 2 < nk;
#pragma unroll
                    for (int kk = 0; kk < KS - 1; ++kk) {
                        load_frags<FM, FN, TM, TN, BKB>(f[(kk + 1) & 1], la, lb, wm, wn, lane, kk + 1);
                        __builtin_amdgcn_sched_barrier(0);
                        mfma_bf16_frags(f[kk & 1], acc);
                        __builtin_amdgcn_sched_barrier(0);
                        if (kk == 0 && more1) {
                            // W of stage j+1; only x of stage j+1 came after
                            // it.  Then W of stage j+2 into staging buffer
                            // s, whose stage j was dequantised in stage j-1.
                            wait_vmcnt<A_LD>();
                            convert(nb);
                            __builtin_amdgcn_sched_barrier(0);
                            if (more2) issue_w(s, j + 2);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    if (more1) {
                        if (more2) wait_vmcnt<B_LD>();         // x of stage j+1 landed
                        else wait_vmcnt<0>();
                    }
                    __syncthreads();                   // stage j+1 published, stage j read
                    if (more1)
                        load_frags<FM, FN, TM, TN, BKB>(f[0], lds_a + nb * (BM * BKB),
                                                        lds_b + nb * (BN * BKB), wm, wn, lane, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    // Last K step of stage j, with x of stage j+2 into buffer s
                    // between the products.
                    const Frags<FM, FN>& fl = f[(KS - 1) & 1];
                    constexpr int NP = FM * FN, STRIDE = NP / A_LD > 0 ? NP / A_LD : 1;
                    int d = 0;
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        const int i = p / FN, jj = p % FN;
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, fl.b[jj]), __builtin_bit_cast(bf16x8, fl.a[i]),
                            acc[i][jj], 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        if (p % STRIDE == STRIDE - 1 && d < A_LD) {
                            if (more2)
                                dma16(a_base, a_off[d] + (uint32_t)((j + 2) * BKB),
                                      a_dst[d] + s * (BM * BKB));
                            ++d;
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
#pragma unroll
                    for (; d < A_LD; ++d) {
                        if (more2)
                            dma16(a_base, a_off[d] + (uint32_t)((j + 2) * BKB), a_dst[d] + s * (BM * BKB));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        wait_vmcnt<0>();
    }

    // K tail (k % 64 elements): one register-loaded stage in buffer 0, every
    // element at or past k zero.  x rows are 16-byte aligned and at least k
    // rounded up to 8 elements long, W rows k rounded up to 16 bytes.
    const int rem = (int)(a.k - nk * KE);
    if (rem > 0) {
        __syncthreads();
        const int64_t ka = nk * BKB, kw = nk * KE;
        for (int c = t; c < BM * CPR; c += NT) {
            const int row = c / CPR, ch = c % CPR;
            const int start = ch * 8;                       // elements
            v4i v = {0, 0, 0, 0};
            if (start < rem) {
                v = *reinterpret_cast<const v4i*>(a_base + (int64_t)min(row, a_rows - 1) * a.ldq + ka +
                                                  ch * 16);
                if (rem - start < 8) v = keep_bytes(v, 2 * (rem - start));
            }
            *reinterpret_cast<v4i*>(lds_a + lds_off_b<BKB>(row, ch)) = v;
        }
        for (int c = t; c < BN * 4; c += NT) {
            const int row = c >> 2, qtr = c & 3;
            const int start = qtr * 16;
            v4i v = {0, 0, 0, 0};
            const int64_t grow = n0 + min(row, b_rows - 1);
            if (start < rem) {
                v = *reinterpret_cast<const v4i*>(a.w + grow * a.ldw + kw + start);
                if (rem - start < 16) v = keep_bytes(v, rem - start);
            }
            v4i lo, hi;
            dequant16(v, a.ws[grow * a.ws_stride], lo, hi);
            *reinterpret_cast<v4i*>(lds_b + lds_off_b<BKB>(row, qtr * 2)) = lo;
            *reinterpret_cast<v4i*>(lds_b + lds_off_b<BKB>(row, qtr * 2 + 1)) = hi;
        }
        __syncthreads();
        const int steps = (rem + 15) / 16;
        for (int kk = 0; kk < steps; ++kk) {
            Frags<FM, FN> ft;
            load_frags<FM, FN, TM, TN, BKB>(ft, lds_a, lds_b, wm, wn, lane, kk);
            mfma_bf16_frags(ft, acc);
        }
    }
    if constexpr (EPI != EPI_F32) {
        static_assert(BM * BN * 2 <= dq_lds_bytes(BM, BN), "output staging fits the stage buffers");
        if (a.vec_store == 2 && m0 + BM <= a.m && n0 + BN <= a.n) {
            __syncthreads();                      // every wave is done with the stage buffers
            store_tile_lds16<FM, FN, TM, TN, EPI>(a, acc, m0, n0, wm, wn, lane,
                                                  smem + wave * (TM * TN * 2));
            return;
        }
    }
    store_tile_f32<FM, FN, TM, TN, EPI>(a, acc, m0, n0, wm, wn, lane);
}

// One block per tile.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dq_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(1024))) int8_t smem[dq_lds_bytes(BM, BN)];
    int64_t m0, n0;
    tile_origin<BM, BN>(a, m0, n0);
    dq_tile<BM, BN, WM, WN, EPI>(a, m0, n0, smem);
}

// One block per CU walking tiles claimed through a.sched (claim_start /
// claim_finish): the XCDs, which run at different clocks, finish together,
// and no block launch separates two tiles on a CU.  Thread 0 claims the next
// tile's id at the start of the current one and hands it over at its end
// through the first word of the second bf16 W stage buffer, which the next
// tile first writes after its first barrier.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dq_persist_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(1024))) int8_t smem[dq_lds_bytes(BM, BN)];
    int& next_id = *reinterpret_cast<int*>(smem + 2 * BM * 128 + BN * 128);
    const int num = a.tiles_m * a.tiles_n;
    const bool lead = threadIdx.x == 0;
    Claims claims{false, 0u};
    if (lead) next_id = claim_finish(a.sched, num, claim_start(a.sched, claims), claims);
    __syncthreads();
    int id = __builtin_amdgcn_readfirstlane(next_id);
    while (id >= 0) {
        unsigned pending = 0;
        if (lead) pending = claim_start(a.sched, claims);
        int64_t m0, n0;
        grouped_origin<BM, BN>(a, id, m0, n0);
        dq_tile<BM, BN, WM, WN, EPI>(a, m0, n0, smem);
        __syncthreads();                          // this tile's LDS is no longer read
        if (lead) next_id = claim_finish(a.sched, num, pending, claims);
        __syncthreads();
        id = __builtin_amdgcn_readfirstlane(next_id);
    }
    if (lead) claims_done(a.sched);
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Few rows (m <= 64): the same sum, bound by reading W.  A block owns 32
// columns (W rows n0 .. n0+31, two groups of 16) and splits K among its KW
// waves.  Every wave streams its columns and its part of K through a ring
// of its own in LDS (3 chunks of 64 K; 2 with 8 x loads, so that two
// 4-wave blocks share a CU, and where the rings would not fit otherwise),
// filled by direct-to-LDS loads, so no barrier is needed in the K loop; the
// loads of W read 64 contiguous bytes of each of 16 rows (four lanes a row,
// the stage buffers' swizzle), and x takes one load per 8 of its rows (XR =
// 1, 2, 4 or 8; lanes past m load the last row again).  The products are
// v_mfma_f32_16x16x32_bf16 into 16 x 16 accumulators, one per column group
// and 16 rows of x (MB = 1, 2 or 4 of those): lane l reads W row
// l % 16 of a group and x row l % 16 of a row block (the last row again past
// m; those outputs are dropped), both at the 16 K elements 16 (l / 16) ..
// +15 of the chunk, the first 8 for one product and the last 8 for the
// other, so both operands see one and the same order of K.  The partial
// sums meet in LDS once, at the end, summed over the waves in a fixed order.
//
// Reading W and x into registers instead (same products, a ring of 5 chunks
// per wave) measured 33 against 28 us at 1 x 28672 x 5376 and 49 against 31
// us at 16 rows: the vector L1 stalled the address units 45 % of the time,
// at its limit of lines in flight; the direct-to-LDS loads do not hold one.
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int KW, int XR>
__host__ __device__ constexpr int dq_few_slot_bytes() { return 2048 + XR * 1024; }
template <int KW, int XR>
__host__ __device__ constexpr int dqf_ahead()
{
    return XR < 8 && KW * 3 * dq_few_slot_bytes<KW, XR>() <= 163840 ? 3 : 2;
}
template <int KW, int XR>
__host__ __device__ constexpr int dq_few_ring_bytes() { return KW * dqf_ahead<KW, XR>() * dq_few_slot_bytes<KW, XR>(); }
// Blocks per CU: 4 waves per SIMD, or fewer where the rings fill the LDS.
template <int KW, int XR>
__host__ __device__ constexpr int dq_few_blocks()
{
    return 163840 / dq_few_ring_bytes<KW, XR>() < 16 / KW ? 163840 / dq_few_ring_bytes<KW, XR>() : 16 / KW;
}

template <int EPI, int KW, int XR>
__global__ __launch_bounds__(64 * KW, (dq_few_blocks<KW, XR>())) void gemm_dq_few_kernel(GemmArgs a)
{
    constexpr int MB = XR >= 2 ? XR / 2 : 1;             // 16-row blocks of x
    constexpr int SLOT = dq_few_slot_bytes<KW, XR>();    // one chunk: W of both groups, then x
    constexpr int L = 2 + XR;                            // loads per chunk and wave
    constexpr int AH = dqf_ahead<KW, XR>();
    constexpr int RING = dq_few_ring_bytes<KW, XR>();
    constexpr int NR = 8 * MB;                           // accumulator registers per lane
    constexpr int RED = KW * NR * 65 * 4;
    static_assert(RED <= RING && RING <= 163840, "the rings, then the sums, fit in LDS");
    __shared__ __attribute__((aligned(1024))) int8_t lds[RING];
    float* const red = reinterpret_cast<float*>(lds);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * 32;
    const int rows = (int)min<int64_t>(a.m, 16 * MB);
    const int grp = lane >> 4;                            // K group of the products
    const int rr = lane & 15;
    const float scale0 = a.ws[min<int64_t>(n0 + rr, a.n - 1) * a.ws_stride];
    const float scale1 = a.ws[min<int64_t>(n0 + 16 + rr, a.n - 1) * a.ws_stride];
    // Take the scales now: the compiler's wait for them counts only its own
    // loads, so later it would also wait for every direct-to-LDS load.
    asm volatile("" : : "v"(scale0), "v"(scale1));

    // Loads: lane l copies 16 bytes of W row l / 4 of a group (its 16-byte
    // piece chosen by the swizzle) and 16 bytes of x row 8 i + l / 8.
    const int wr = lane >> 2;
    const int wpiece = (lane & 3) ^ ((wr >> 2) & 3);
    const uint32_t w_off0 = (uint32_t)(min<int64_t>(n0 + wr, a.n - 1) - n0) * (uint32_t)a.ldw + wpiece * 16;
    const uint32_t w_off1 = (uint32_t)(min<int64_t>(n0 + 16 + wr, a.n - 1) - n0) * (uint32_t)a.ldw + wpiece * 16;
    const int8_t* const w_blk = a.w + n0 * a.ldw;
    uint32_t x_off[XR];
#pragma unroll
    for (int i = 0; i < XR; ++i)
        x_off[i] = (uint32_t)(min(8 * i + (lane >> 3), rows - 1) * a.ldq + (lane & 7) * 16);
    const int64_t nck = a.k / 64;
    const int64_t cb = nck * wave / KW, ce = nck * (wave + 1) / KW;
    const int nc = (int)(ce - cb);
    const uint32_t ring = lds_addr(lds) + wave * (AH * SLOT);
    auto issue = [&](int slot, int c) {
        const int64_t kc = cb + c;
        const uint32_t dst = ring + slot * SLOT;
        dma16(w_blk + kc * 64, w_off0, dst);
        dma16(w_blk + kc * 64, w_off1, dst + 1024);
#pragma unroll
        for (int i = 0; i < XR; ++i) dma16(a.q + kc * 128, x_off[i], dst + 2048 + i * 1024);
    };
    // Reads: W row l % 16 of a group, the 16 bytes of K group l / 16; x row
    // l % 16 of a row block, 32 bytes of that K group.
    const int w_rd = rr * 64 + ((grp ^ ((rr >> 2) & 3)) << 4);
    int x_rd[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) x_rd[b] = 2048 + min(16 * b + rr, rows - 1) * 128 + grp * 32;
    const int8_t* const my = lds + wave * (AH * SLOT);

    f32x4v acc[MB][2];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int g = 0; g < 2; ++g) acc[b][g] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    auto product = [&](const v4i& w0, const v4i& w1, const v4i (&x0)[MB], const v4i (&x1)[MB]) {
        v4i lo[2], hi[2];
        dequant16(w0, scale0, lo[0], hi[0]);
        dequant16(w1, scale1, lo[1], hi[1]);
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                acc[b][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, lo[g]), __builtin_bit_cast(bf16x8, x0[b]), acc[b][g], 0, 0, 0);
                acc[b][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, hi[g]), __builtin_bit_cast(bf16x8, x1[b]), acc[b][g], 0, 0, 0);
            }
    };
    auto consume = [&](int slot) {
        const int8_t* base = my + slot * SLOT;
        const v4i w0 = *reinterpret_cast<const v4i*>(base + w_rd);
        const v4i w1 = *reinterpret_cast<const v4i*>(base + 1024 + w_rd);
        v4i x0[MB], x1[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            x0[b] = *reinterpret_cast<const v4i*>(base + x_rd[b]);
            x1[b] = *reinterpret_cast<const v4i*>(base + x_rd[b] + 16);
        }
        product(w0, w1, x0, x1);
    };
    // Slot i holds chunk c + i; every slot is refilled right after its
    // products, always (past the last chunk with the last chunk again), so
    // each wait allows the loads of the AH - 1 chunks issued after the one it
    // needs; the last AH chunks drain with fewer.  The scheduling barriers
    // keep each chunk's reads, conversion and products together: left
    // alone, the compiler sinks all products to the end of the loop, holds
    // every slot's data at once and spills.
    if (nc > 0) {
#pragma unroll
        for (int i = 0; i < AH; ++i) issue(i, min(i, nc - 1));
        int c = 0;
        for (; c + 2 * AH <= nc; c += AH) {
#pragma unroll
            for (int i = 0; i < AH; ++i) {
                wait_vmcnt<(AH - 1) * L>();
                consume(i);
                __builtin_amdgcn_sched_barrier(0);
                issue(i, c + AH + i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < AH; ++i) {
            wait_vmcnt<(AH - 1) * L>();
            if (c + i < nc) consume(i);
            __builtin_amdgcn_sched_barrier(0);
            issue(i, min(c + AH + i, nc - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        // chunk c + AH + i has AH - 1 - i chunks of loads after it
        wait_vmcnt<(AH - 1) * L>();
        if (c + AH < nc) consume(0);
        if constexpr (AH == 3) {
            wait_vmcnt<L>();
            if (c + AH + 1 < nc) consume(1);
        }
        wait_vmcnt<0>();
        if (c + 2 * AH - 1 < nc) consume(AH - 1);
    }

    // K tail (k % 64 elements), in the last wave, through registers; elements
    // at or past k are zero in both operands (W rows are readable up to k
    // rounded up to 16 bytes, x rows up to k rounded up to 8 elements).
    const int rem = (int)(a.k - nck * 64);
    if (rem > 0 && wave == KW - 1) {
        const int start = grp * 16;
        const int64_t wn0 = min<int64_t>(n0 + rr, a.n - 1), wn1 = min<int64_t>(n0 + 16 + rr, a.n - 1);
        v4i w0 = {0, 0, 0, 0}, w1 = {0, 0, 0, 0}, x0[MB], x1[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) x0[b] = x1[b] = v4i{0, 0, 0, 0};
        if (start < rem) {
            w0 = *reinterpret_cast<const v4i*>(a.w + wn0 * a.ldw + nck * 64 + start);
            w1 = *reinterpret_cast<const v4i*>(a.w + wn1 * a.ldw + nck * 64 + start);
            if (rem - start < 16) {
                w0 = keep_bytes(w0, rem - start);
                w1 = keep_bytes(w1, rem - start);
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const int8_t* const xr = a.q + min(16 * b + rr, rows - 1) * a.ldq + nck * 128 + grp * 32;
                x0[b] = *reinterpret_cast<const v4i*>(xr);
                if (rem - start < 8) x0[b] = keep_bytes(x0[b], 2 * (rem - start));
                if (start + 8 < rem) {
                    x1[b] = *reinterpret_cast<const v4i*>(xr + 16);
                    if (rem - start - 8 < 8) x1[b] = keep_bytes(x1[b], 2 * (rem - start - 8));
                }
            }
        }
        product(w0, w1, x0, x1);
    }

    // Lane l, register r of accumulator (b, g): column (W row) 16 g +
    // 4 (l / 16) + r, x row 16 b + l % 16.  The sums overlay the rings, once
    // every wave is done with its own.
    __syncthreads();
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(wave * NR + (b * 2 + g) * 4 + r) * 65 + lane] = acc[b][g][r];
    __syncthreads();
    for (int o = threadIdx.x; o < rows * 32; o += 64 * KW) {
        const int j = o >> 5, i = o & 31;
        const int64_t gn = n0 + i;
        if (gn >= a.n) continue;
        const int ii = i & 15;
        const int at = (((j >> 4) * 2 + (i >> 4)) * 4 + (ii & 3)) * 65 + (j & 15) + 16 * (ii >> 2);
        float v = red[at];
#pragma unroll
        for (int w = 1; w < KW; ++w) v = v + red[w * NR * 65 + at];
        if (a.bias) v = v + bias_at<EPI>(a.bias, gn);
        if constexpr (EPI == EPI_F32) {
            reinterpret_cast<float*>(a.out)[j * a.ldo + gn] = v;
        } else {
            reinterpret_cast<uint16_t*>(a.out)[j * a.ldo + gn] = (uint16_t)(pack2<EPI>(v, 0.0f) & 0xffffu);
        }
    }
}

// ---------------------------------------------------------------------------
// Register-staged pipeline (any k % 16 == 0)
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int EPI, bool KTAIL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs a)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int CPR = kBK / 16;                       // 16-B chunks per row
    constexpr int A_LD = BM * CPR / NT, B_LD = BN * CPR / NT;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "load split");

    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][BM * kBK];
    __shared__ __attribute__((aligned(16))) int8_t lds_b[2][BN * kBK];

    int64_t m0, n0;
    tile_origin<BM, BN>(a, m0, n0);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;

    const int8_t* a_src[A_LD];
    int a_lds[A_LD], a_kc[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int c = tid + i * NT;
        const int row = c / CPR, kc = c % CPR;
        const int64_t gr = m0 + row < a.m ? m0 + row : a.m - 1;
        a_src[i] = a.q + gr * a.ldq + kc * 16;
        a_lds[i] = lds_off(row, kc);
        a_kc[i] = kc * 16;
    }
    const int8_t* b_src[B_LD];
    int b_lds[B_LD], b_kc[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int c = tid + i * NT;
        const int row = c / CPR, kc = c % CPR;
        const int64_t gr = n0 + row < a.n ? n0 + row : a.n - 1;
        b_src[i] = a.w + gr * a.ldw + kc * 16;
        b_lds[i] = lds_off(row, kc);
        b_kc[i] = kc * 16;
    }

    // Every call issues the same A_LD + B_LD loads, so the hardware's
    // in-order load counter always has the same number of loads in flight
    // per stage.  With KTAIL (k % 64 != 0), a chunk wholly at or past k is
    // read from the row's last 16-byte chunk instead and replaced by zeros,
    // and the chunk that straddles k keeps only its bytes before k.  Rows
    // are 16-byte aligned and at least kpad = k rounded up to 16 bytes long,
    // so every chunk read here is inside the row.
    const int64_t kpad = (a.k + 15) & ~(int64_t)15;
    auto tail_chunk = [&](const int8_t* src, int64_t k0, int kc) {
        const int64_t p = k0 + kc;
        const bool in = p < a.k;
        const v4i v = *reinterpret_cast<const v4i*>(src + (in ? k0 : kpad - 16 - kc));
        const int valid = in ? (int)min<int64_t>(a.k - p, 16) : 0;
        return valid >= 16 ? v : keep_bytes(v, valid);
    };
    auto load_stage = [&](v4i* ra, v4i* rb, int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ra[i] = KTAIL ? tail_chunk(a_src[i], k0, a_kc[i])
                          : *reinterpret_cast<const v4i*>(a_src[i] + k0);
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            rb[i] = KTAIL ? tail_chunk(b_src[i], k0, b_kc[i])
                          : *reinterpret_cast<const v4i*>(b_src[i] + k0);
    };
    auto store_stage = [&](int buf, const v4i* ra, const v4i* rb) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            *reinterpret_cast<v4i*>(&lds_a[buf][a_lds[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            *reinterpret_cast<v4i*>(&lds_b[buf][b_lds[i]]) = rb[i];
    };

    v16i acc[FM][FN];
    zero_acc(acc);

    // Two register sets: set 0 carries even stages, set 1 odd stages.
    // Prefetches past the last stage re-read the last stage (never used),
    // which keeps the loop free of branches around loads.
    v4i ra0[A_LD], rb0[B_LD], ra1[A_LD], rb1[B_LD];
    const int64_t nk = (a.k + kBK - 1) / kBK;
    const int64_t k_last = (nk - 1) * kBK;
    if (nk > 0) {
        load_stage(ra0, rb0, 0);
        store_stage(0, ra0, rb0);
        load_stage(ra1, rb1, nk > 1 ? kBK : 0);
    }
    __syncthreads();
    // Pairs of stages, so that both register sets and both LDS buffers are
    // fixed in the code; an odd last stage runs after the loop.
    int64_t kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        // stage kt (even) from LDS buffer 0; stage kt+1 is in set 1
        load_stage(ra0, rb0, min((kt + 2) * kBK, k_last));
        mma_stage<FM, FN, TM, TN>(lds_a[0], lds_b[0], wm, wn, lane, acc);
        store_stage(1, ra1, rb1);
        __syncthreads();
        // stage kt+1 (odd) from LDS buffer 1; stage kt+2 is in set 0
        load_stage(ra1, rb1, min((kt + 3) * kBK, k_last));
        mma_stage<FM, FN, TM, TN>(lds_a[1], lds_b[1], wm, wn, lane, acc);
        store_stage(0, ra0, rb0);
        __syncthreads();
    }
    if (kt < nk) mma_stage<FM, FN, TM, TN>(lds_a[0], lds_b[0], wm, wn, lane, acc);

    store_tile<FM, FN, TM, TN, EPI>(a, acc, m0, n0, wm, wn, lane);
}

// ===========================================================================
// Steps 1-3 in one kernel for few rows (decode and small batches)
// ===========================================================================
//
// With few rows the layer's time is the weight's stream plus the launch of
// a quantisation that has almost nothing to do.  Here each 64 x 64 output
// block quantises its own rows of x into LDS with the quantisation
// kernel's arithmetic, so codes and scales are identical to that kernel's,
// and keeps the codes there for the whole of K while the weight streams
// through four 4 KiB direct-to-LDS stages.  Blocks stay small so that
// many fit a compute unit: the stream needs the loads of many blocks in
// flight.  The first four stage loads go out once the first loads of x
// have been used, so the rest of the quantisation runs while they are in
// flight.  All four waves share the quantisation (below).  Blocks of the first column tile then copy the
// codes and scales to global memory, so the call leaves what the
// quantisation would.  Four waves, each a 32 x 32 product per 32-byte K
// step.
//
// LDS: weight stages (16 KiB), row scales and reciprocals, column scales
// and bias, 32 partial maxima per row, then the codes: K stage j of row
// slot r at (j * rows + r) * 64, its 16-byte chunks swizzled as in the GEMM
// stages.
constexpr int kLsBM = 64, kLsBN = 64, kLsS = 4, kLsBK = 64, kLsNB = 8;
constexpr int kLsHdr = kLsS * kLsBN * kLsBK + 1024;  // weight stages, row scales, reciprocals,
                                                     // column scales, bias

// bytes of the per-row partial maxima, rounded up to 256 so the codes keep
// the stage buffers' bank alignment
__host__ __device__ constexpr int layer_part_bytes(int rows) { return (rows * 128 + 255) & ~255; }

struct LayerArgs {
    const uint16_t* x;
    int8_t* q;
    float* xs;
    const int8_t* w;
    const float* ws;
    const void* bias;
    void* out;
    int64_t ldx, ldq, ldw, ldo;
    int64_t m, n, k;
    int tiles_m;
    int rows;        // row slots of codes in LDS: min(64, m)
    int ws_stride;   // 1: per-column w scale, 0: tensor-wide
    int vec_store;   // out rows allow 16-byte (fp32) or 8-byte (16-bit) stores (1) or not (0)
};

template <int EPI, bool PER_ROW>
__global__ __launch_bounds__(256) void layer_small_kernel(LayerArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) int8_t lsm[];
    constexpr int BK = kLsBK, CPR = BK / 16, RPI = 64 / CPR;   // 16 weight rows per 1 KiB load
    constexpr int WL = kLsBN / RPI / 4;                          // loads per wave and stage
    int8_t* const wst = lsm;
    float* const sxs = reinterpret_cast<float*>(lsm + kLsS * kLsBN * BK);   // row scales
    float* const srcp = sxs + kLsBM;                                        // their reciprocals
    float* const sws = srcp + kLsBM;                                        // column scales
    float* const sbs = sws + kLsBN;                                         // bias, as fp32
    uint32_t* const rpart = reinterpret_cast<uint32_t*>(lsm + kLsHdr);      // 32 partial maxima per row
    int8_t* const codes = lsm + kLsHdr + layer_part_bytes(a.rows);

    const int tm = (int)(blockIdx.x % (unsigned)a.tiles_m);
    const int tn = (int)(blockIdx.x / (unsigned)a.tiles_m);
    const int64_t m0 = (int64_t)tm * kLsBM, n0 = (int64_t)tn * kLsBN;
    const int R = (int)min<int64_t>(kLsBM, a.m - m0);          // rows of this block
    const int rows = a.rows;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;                    // 2 x 2 waves of 32 x 32
    const int64_t nk = a.k / BK;
    const int64_t nvec = a.k >> 3;                              // 8-element chunks per row

    // weight stages: wave w loads weight rows 16 w .. 16 w + 15
    const int8_t* w_base = a.w + n0 * a.ldw;
    const int b_rows = (int)min<int64_t>(kLsBN, a.n - n0);
    uint32_t w_off[WL], w_dst[WL];
#pragma unroll
    for (int i = 0; i < WL; ++i) {
        const int blk = i * 4 + wave;
        const int wrow = blk * RPI + lane / CPR;
        w_off[i] = (uint32_t)(min(wrow, b_rows - 1) * a.ldw + (((lane % CPR) ^ swz_b<BK>(wrow)) * 16));
        w_dst[i] = lds_addr(wst) + blk * 1024;
    }
    auto issue = [&](int buf, int64_t stage) {
#pragma unroll
        for (int i = 0; i < WL; ++i)
            dma16(w_base, w_off[i] + (uint32_t)(stage * BK), w_dst[i] + buf * (kLsBN * BK));
    };

    // codes of row r, 8-element chunk v, in the LDS layout
    auto code_off = [&](int r, int64_t v) {
        const int64_t kb = v * 8;
        return (int64_t)((kb >> 6) * rows + r) * 64 +
               ((((int)(kb >> 4) & 3) ^ swz_b<BK>(r)) << 4) + (int)(kb & 8);
    };
    // Quantisation of the block's R rows, spread over all 256 threads: the
    // R * k / 8 chunks are dealt out in batches of NB per thread (NB loads
    // in flight each).  Pass 1 folds each chunk's absmax into one of 32
    // partial maxima of its row in LDS (slot lane % 32, so the lanes of a
    // wave never wait on one address); one thread per row then folds the
    // 32 into the row's scale and reciprocal (one maximum for the tensor).
    // Pass 2 writes the codes, from the registers when the block's chunks
    // fit one batch, else reading x again.  The weight stages' loads go out
    // once the first batch's maxima are folded: the compiler cannot count
    // the per-lane conditional x loads and waits for every load of the wave
    // before using them, and a wave's loads complete in order, so stages
    // issued before would hold up the maxima until the weight arrived.
    const int t = threadIdx.x;
    // The block's column scales and bias, loaded first: their latency then
    // passes under the quantisation and the K loop instead of holding up
    // the epilogue, and loads issued before the weight stages' leave the
    // K loop's counted waits exact.  Columns past n repeat the last one.
    float t_ws = 0.0f, t_b = 0.0f;
    if (t < kLsBN) {
        const int64_t c = min<int64_t>(n0 + t, a.n - 1);
        t_ws = a.ws[c * a.ws_stride];
        if (a.bias) t_b = bias_at<EPI>(a.bias, c);
    }
    const int nv = (int)nvec;                                  // < 2^15 (k <= CK_MAX_K)
    const int total = R * nv;
    const int step_r = 256 / nv, step_v = 256 % nv;            // nv >= 8
    for (int i = t; i < rows * 32; i += 256) rpart[i] = 0u;
    __syncthreads();
    constexpr int NB = kLsNB;
    v4i c[NB];
    // phase 1: loads only; phase 2: maxima (pass 1) or codes (pass 2)
    auto batch = [&](int base, bool load, bool use, bool codes_pass) {
        int idx = base + t;
        int row = idx / nv;
        int v = idx - row * nv;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (idx < total) {
                if (load) c[i] = *reinterpret_cast<const v4i*>(a.x + (m0 + row) * a.ldx + (int64_t)v * 8);
                if (!use) {
                } else if (!codes_pass) {
                    atomicMax(&rpart[(PER_ROW ? row : 0) * 32 + (lane & 31)],
                              absmax_fold(absmax_pk(0u, c[i])));
                } else {
                    const float sc = sxs[PER_ROW ? row : 0], rc = srcp[PER_ROW ? row : 0];
                    const bool recip = sc > 0.0f && rc < 8.5070592e+37f;
                    *reinterpret_cast<uint2*>(codes + code_off(row, v)) = quant8_fast(c[i], sc, rc, recip);
                }
            }
            idx += 256;
            row += step_r;
            v += step_v;
            if (v >= nv) { v -= nv; ++row; }
        }
    };
    const bool one_batch = total <= 256 * NB;
    batch(0, true, false, false);
    batch(0, false, true, false);
#pragma unroll
    for (int st = 0; st < kLsS; ++st) issue(st, min<int64_t>(st, nk - 1));
    for (int base = 256 * NB; base < total; base += 256 * NB) batch(base, true, true, false);
    __syncthreads();
    if (t < (PER_ROW ? R : 1)) {
        uint32_t mb = 0;
        for (int i = 0; i < 32; ++i) mb = max(mb, rpart[t * 32 + i]);
        const float sc = bf16_bits_to_f32(mb) / 127.0f;
        sxs[t] = sc;
        srcp[t] = 1.0f / sc;
    }
    __syncthreads();
    if (one_batch) batch(0, false, true, true);
    else
        for (int base = 0; base < total; base += 256 * NB) batch(base, true, true, true);

    // K loop: one barrier per stage; after it, the buffer of stage j - 1 is
    // free and takes stage j + 3 (past the end, the last stage again, so
    // every wave issues WL loads per stage and the waits stay exact).
    v16i acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0;
    const int frag_row = lane & 31;
    const int arow = min(wm * 32 + frag_row, rows - 1);   // slots past the block's rows: never stored
    const int brow = wn * 32 + frag_row;
    for (int64_t j = 0; j < nk; ++j) {
        if (j == 0) wait_vmcnt<(kLsS - 1) * WL>();     // stage 0 landed
        else wait_vmcnt<(kLsS - 2) * WL>();            // stage j landed
        __syncthreads();
        if (j > 0) issue((int)((j - 1) % kLsS), min<int64_t>(j - 1 + kLsS, nk - 1));
        const int8_t* ab = codes + j * rows * 64;
        const int8_t* wb = wst + (j % kLsS) * (kLsBN * BK);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int chunk = kk * 2 + (lane >> 5);
            const v4i fa = *reinterpret_cast<const v4i*>(ab + lds_off_b<BK>(arow, chunk));
            const v4i fb = *reinterpret_cast<const v4i*>(wb + lds_off_b<BK>(brow, chunk));
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb, fa, acc, 0, 0, 0);
        }
    }
    wait_vmcnt<0>();            // no stage load may land in LDS after the block ends
    if (t < kLsBN) {
        sws[t] = t_ws;
        sbs[t] = t_b;
    }
    __syncthreads();

    // epilogue: lane holds row frag_row, four columns per group g
    const int64_t gm = m0 + wm * 32 + frag_row;
    const int col_off = 4 * (lane >> 5);
    const bool has_bias = a.bias != nullptr;
    const float xsv = sxs[PER_ROW ? min(wm * 32 + frag_row, R - 1) : 0];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t gn = n0 + wn * 32 + g * 8 + col_off;
        float wsv[4], bv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wsv[e] = sws[wn * 32 + g * 8 + col_off + e];
            bv[e] = sbs[wn * 32 + g * 8 + col_off + e];
        }
        if (gm >= a.m || gn >= a.n) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = epilogue_value(acc[4 * g + e], xsv, wsv[e], bv[e], has_bias);
        if constexpr (EPI == EPI_F32) {
            float* orow = reinterpret_cast<float*>(a.out) + gm * a.ldo;
            if (a.vec_store && gn + 3 < a.n) {
                *reinterpret_cast<float4*>(orow + gn) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (gn + e < a.n) orow[gn + e] = v[e];
            }
        } else {
            uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + gm * a.ldo;
            const uint32_t p0 = pack2<EPI>(v[0], v[1]), p1 = pack2<EPI>(v[2], v[3]);
            if (a.vec_store && gn + 3 < a.n) {
                *reinterpret_cast<uint2*>(orow + gn) = make_uint2(p0, p1);
            } else {
                const uint32_t h[4] = {p0 & 0xffffu, p0 >> 16, p1 & 0xffffu, p1 >> 16};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (gn + e < a.n) orow[gn + e] = (uint16_t)h[e];
            }
        }
    }

    // the first column tile leaves the codes and scales in global memory
    if (tn != 0) return;
    for (int r = wave; r < R; r += 4) {
        int8_t* qr = a.q + (m0 + r) * a.ldq;
        for (int64_t v = lane; v < nvec; v += 64)
            *reinterpret_cast<uint2*>(qr + v * 8) = *reinterpret_cast<const uint2*>(codes + code_off(r, v));
        if (PER_ROW && lane == 0) a.xs[m0 + r] = sxs[r];
    }
    if (!PER_ROW && threadIdx.x == 0) a.xs[0] = sxs[0];
}

// ===========================================================================
// Host side: validation, tile choice, launches
// ===========================================================================

namespace {

thread_local char g_err[512];

ck_status fail(ck_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

ck_status ok()
{
    g_err[0] = '\0';
    return CK_OK;
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];

ck_status check_device()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CK_ERR_HIP, "device id %d out of range", dev);
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        if (e != hipSuccess)
            return fail(CK_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
        if (st == 2)
            return fail(CK_ERR_WRONG_ARCH, "device %d is %s, this library runs on gfx950 only",
                        dev, p.gcnArchName);
    }
    if (st == 2) return fail(CK_ERR_WRONG_ARCH, "device %d is not gfx950", dev);
    return CK_OK;
}

ck_status launch(const void* fn, unsigned grid, unsigned block, void** args, hipStream_t stream,
                 const char* what)
{
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, stream);
    if (e != hipSuccess) return fail(CK_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return CK_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Row-quantisation kernel holding a whole row in registers when it fits
// (NC of 4, 8, 11 or 16 16-byte chunks per lane), without the loops for
// longer rows and a k % 8 tail when they are not needed.
template <bool PER_ROW, bool REST>
const void* quantize_row_fn_rest(int64_t chunks)
{
    if (chunks <= 4) return reinterpret_cast<const void*>(&quantize_rows_kernel<PER_ROW, 4, REST>);
    if (chunks <= 8) return reinterpret_cast<const void*>(&quantize_rows_kernel<PER_ROW, 8, REST>);
    if (chunks <= 11) return reinterpret_cast<const void*>(&quantize_rows_kernel<PER_ROW, 11, REST>);
    return reinterpret_cast<const void*>(&quantize_rows_kernel<PER_ROW, kQzRegChunks, REST>);
}

const void* quantize_row_fn(int64_t k, bool per_row)
{
    const int64_t chunks = (k / 8 + 63) / 64;      // 16-byte chunks per lane
    const bool rest = k % 8 != 0 || chunks > kQzRegChunks;
    if (per_row) return rest ? quantize_row_fn_rest<true, true>(chunks) : quantize_row_fn_rest<true, false>(chunks);
    return rest ? quantize_row_fn_rest<false, true>(chunks) : quantize_row_fn_rest<false, false>(chunks);
}

// Tensor-wide amax kernel for 16-byte aligned rows: 4, 8 or 16 chunks per
// lane and pass (rows past 16 chunks take several passes), with the k % 8
// tail loop only where k needs it.
const void* tensor_amax_rows_fn(int64_t k)
{
    const int64_t chunks = (k / 8 + 63) / 64;
    const bool tail = k % 8 != 0;
#define CK_AMAX_ROWS(R)                                                                  \
    (chunks <= 4   ? reinterpret_cast<const void*>(&tensor_amax_rows_kernel<4, R>)    \
     : chunks <= 8 ? reinterpret_cast<const void*>(&tensor_amax_rows_kernel<8, R>)    \
                   : reinterpret_cast<const void*>(&tensor_amax_rows_kernel<16, R>))
    return tail ? CK_AMAX_ROWS(true) : CK_AMAX_ROWS(false);
#undef CK_AMAX_ROWS
}

// Rotated-row kernel for a mode and block 2^lb, with the smallest
// register-resident chunk count of 4, 8, 12 or 16 that holds the row (rows
// past 16 chunks re-read the rest).  The rotated values stay in fp32, 8
// registers per chunk, so the count sets the waves a SIMD can hold: 12
// chunks (rows up to 6144 elements) take about 124 registers, four waves,
// where 16 take about 156, three.
template <int MODE, int NC>
const void* quantize_rot_fn_nc(int lb)
{
    switch (lb) {
    case 0: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 0>);
    case 1: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 1>);
    case 2: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 2>);
    case 3: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 3>);
    case 4: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 4>);
    case 5: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 5>);
    case 6: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 6>);
    case 7: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 7>);
    case 8: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 8>);
    default: return reinterpret_cast<const void*>(&quantize_rot_kernel<MODE, NC, 9>);
    }
}

template <int MODE>
const void* quantize_rot_fn_mode(int64_t k, int lb)
{
    const int64_t chunks = (k / 8 + 63) / 64;
    if (chunks <= 4) return quantize_rot_fn_nc<MODE, 4>(lb);
    if (chunks <= 8) return quantize_rot_fn_nc<MODE, 8>(lb);
    if (chunks <= 12) return quantize_rot_fn_nc<MODE, 12>(lb);
    return quantize_rot_fn_nc<MODE, 16>(lb);
}

// ---- compiled tile configurations
// Ids 0..3: block shapes on the direct-to-LDS kernel (k % 64 == 0; other k
// take the register-staged kernel of the same shape).  Ids 4..7: the same
// shapes, always on the register-staged kernel.
constexpr int kDmaStages = 4;

struct TileCfg {
    int bm, bn, threads;
    bool dma;
    int dma_bk;                        // bytes of K per DMA stage; a shorter K tail
                                       // takes one more, register-loaded stage
    const void* dma_fn[kNumEpi];       // direct-to-LDS main loop, by epilogue
    const void* reg_fn[kNumEpi];       // register-staged, k % 64 == 0
    const void* reg_tail_fn[kNumEpi];  // register-staged, any k
    const void* persist_fn[kNumEpi][2];   // persistent direct-to-LDS kernel, [epilogue][has
                                          // bias] (16-bit outputs and the int32 accumulators,
                                          // k a positive multiple of dma_bk), else null
};

template <int BM, int BN, int WM, int WN, bool IL, int BKB, int S, int EPI>
void set_epi(TileCfg& c)
{
    c.dma_fn[EPI] = reinterpret_cast<const void*>(&gemm_dma_kernel<BM, BN, WM, WN, EPI, S, IL, BKB>);
    c.reg_fn[EPI] = reinterpret_cast<const void*>(&gemm_kernel<BM, BN, WM, WN, EPI, false>);
    c.reg_tail_fn[EPI] = reinterpret_cast<const void*>(&gemm_kernel<BM, BN, WM, WN, EPI, true>);
}

template <int BM, int BN, int WM, int WN, bool IL = false, int BKB = 64, int S = kDmaStages>
TileCfg make_tile(bool dma)
{
    TileCfg c{BM, BN, 64 * WM * WN, dma, BKB, {}, {}, {}, {}};
    set_epi<BM, BN, WM, WN, IL, BKB, S, EPI_BF16>(c);
    set_epi<BM, BN, WM, WN, IL, BKB, S, EPI_I32>(c);
    set_epi<BM, BN, WM, WN, IL, BKB, S, EPI_F16>(c);
    set_epi<BM, BN, WM, WN, IL, BKB, S, EPI_F32>(c);
    return c;
}

template <int BM, int BN, int WM, int WN>
TileCfg make_persist_tile()
{
    TileCfg c = make_tile<BM, BN, WM, WN, true, 128, 2>(true);
    c.persist_fn[EPI_BF16][0] = reinterpret_cast<const void*>(&gemm_persist_kernel<BM, BN, WM, WN, EPI_BF16, false>);
    c.persist_fn[EPI_BF16][1] = reinterpret_cast<const void*>(&gemm_persist_kernel<BM, BN, WM, WN, EPI_BF16, true>);
    c.persist_fn[EPI_F16][0] = reinterpret_cast<const void*>(&gemm_persist_kernel<BM, BN, WM, WN, EPI_F16, false>);
    c.persist_fn[EPI_F16][1] = reinterpret_cast<const void*>(&gemm_persist_kernel<BM, BN, WM, WN, EPI_F16, true>);
    c.persist_fn[EPI_I32][0] = reinterpret_cast<const void*>(&gemm_persist_kernel<BM, BN, WM, WN, EPI_I32, false>);
    return c;
}

const TileCfg* tiles()
{
    static const TileCfg t[CK_NUM_TILES] = {
        make_tile<256, 256, 2, 2>(true),    // 0: 4 waves, 128 x 128 per wave
        make_tile<256, 128, 2, 2>(true),    // 1: 4 waves, 128 x 64 per wave
        make_tile<128, 128, 2, 2>(true),    // 2: 4 waves, 64 x 64 per wave
        make_tile<64, 64, 2, 2>(true),      // 3: 4 waves, 32 x 32 per wave
        make_tile<256, 256, 2, 2>(false),   // 4..7: same shapes, register-staged
        make_tile<256, 128, 2, 2>(false),
        make_tile<128, 128, 2, 2>(false),
        make_tile<64, 64, 2, 2>(false),
        make_tile<256, 256, 2, 4>(true),    // 8: 8 waves, 128 x 64 per wave
        make_tile<256, 256, 4, 2>(true),    // 9: 8 waves, 64 x 128 per wave
        make_tile<256, 256, 2, 2, true>(true),   // 10: as 0, refill loads spread over the products
        make_tile<256, 256, 2, 4, true>(true),   // 11: as 8, refill loads spread over the products
        make_tile<256, 256, 2, 4, true, 128, 2>(true),   // 12: as 11, 128-byte K stages, 2 buffers
        make_persist_tile<256, 256, 2, 4>(),     // 13: as 12, persistent (one block per CU)
    };
    return t;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kNumCUs = 256;

// Heuristic, from sweeps of the five workloads and of decode shapes
// (m = 1 .. 128 against n = 16384 / 28672):
//   - the 256 x 256 tile (id 12: 8 waves, 128-byte K stages, refill loads
//     spread over the products) when it gives every CU at least one tile;
//     with k not a multiple of 128 it still beat the 64-byte-stage tile
//     (tail stage included);
//   - else 128 x 128 (id 2) when that fills at least 3/4 of the CUs and
//     m > 16 (m = 128, n = 28672: 34 us against 48 us for 64 x 64);
//   - else 64 x 64 (id 3): small m streams W at 6.2-6.4 TB/s with it.
// group_m = 4 row tiles per launch-order group measured best or within 1 %.
void heuristic(int64_t m, int64_t n, int64_t k, int* tile, int* group_m)
{
    (void)k;
    const TileCfg* t = tiles();
    const auto count = [&](int id) { return cdiv(m, t[id].bm) * cdiv(n, t[id].bn); };
    if (count(12) > kNumCUs) *tile = 13;                   // persistent, with stealing
    else if (count(12) == kNumCUs) *tile = 12;
    else if (m > 16 && count(2) * 4 >= kNumCUs * 3) *tile = 2;
    else *tile = 3;
    *group_m = 4;
}

// ---- measured tile table, forced tile, path log (host state)
//
// PR #142 "What this does": a table of measured winners consulted before
// the heuristic for exact shape matches, a forced configuration for A/B
// runs that is never replaced by another, and a one-line log per unique
// shape of the path that ran.  Here the table is filled through the C ABI
// (the Python binding loads a JSON file written by its sweep tool, for
// gfx950 only); CK_INT8_FORCE_TILE and CK_INT8_LOG_PATH give the initial
// forced tile and log switch, which the ABI can change later.

std::mutex g_host_mu;
std::map<std::tuple<int64_t, int64_t, int64_t>, std::pair<int, int>> g_table;
std::set<std::tuple<int, int64_t, int64_t, int64_t, int, int, int>> g_logged;

int env_int(const char* name, int dflt)
{
    const char* v = getenv(name);
    if (!v || !*v) return dflt;
    char* end = nullptr;
    const long x = strtol(v, &end, 10);
    return (end && *end == '\0') ? (int)x : dflt;
}

std::atomic<int> g_forced_tile{-2};          // -2: not read from the environment yet
std::atomic<int> g_log_paths{-1};            // -1: not read yet

int forced_tile()
{
    int f = g_forced_tile.load(std::memory_order_acquire);
    if (f == -2) {
        f = env_int("CK_INT8_FORCE_TILE", -1);
        if (f < -1 || f >= CK_NUM_TILES) f = -1;
        int expect = -2;
        g_forced_tile.compare_exchange_strong(expect, f);
        f = g_forced_tile.load(std::memory_order_acquire);
    }
    return f;
}

bool log_paths()
{
    int v = g_log_paths.load(std::memory_order_acquire);
    if (v < 0) {
        v = env_int("CK_INT8_LOG_PATH", 0) != 0 ? 1 : 0;
        int expect = -1;
        g_log_paths.compare_exchange_strong(expect, v);
        v = g_log_paths.load(std::memory_order_acquire);
    }
    return v == 1;
}

enum Source { SRC_ARG = 0, SRC_FORCED = 1, SRC_TABLE = 2, SRC_HEURISTIC = 3 };
const char* const kSourceName[] = {"argument", "forced", "table", "heuristic"};

// Tile and group for a call: an explicit tile argument, else the forced
// tile, else a table entry for (m, n, k), else the heuristic.  A positive
// group_m argument always wins; otherwise the table's group (for a table
// pick) or the heuristic's.
void choose(int64_t m, int64_t n, int64_t k, int tile_arg, int group_arg, int* tile, int* group,
            Source* src)
{
    int ht, hg;
    heuristic(m, n, k, &ht, &hg);
    int t = ht, g = hg;
    Source so = SRC_HEURISTIC;
    if (tile_arg >= 0) {
        t = tile_arg;
        so = SRC_ARG;
    } else if (forced_tile() >= 0) {
        t = forced_tile();
        so = SRC_FORCED;
    } else {
        std::lock_guard<std::mutex> lk(g_host_mu);
        const auto it = g_table.find(std::make_tuple(m, n, k));
        if (it != g_table.end()) {
            t = it->second.first;
            g = it->second.second;
            so = SRC_TABLE;
        }
    }
    if (group_arg > 0) g = group_arg;
    *tile = t;
    *group = g;
    *src = so;
}

void log_once(int what, int64_t m, int64_t n, int64_t k, int a, int b, int c, const char* text)
{
    if (!log_paths()) return;
    std::lock_guard<std::mutex> lk(g_host_mu);
    if (!g_logged.insert(std::make_tuple(what, m, n, k, a, b, c)).second) return;
    fprintf(stderr, "ck_int8 path: %s\n", text);
    fflush(stderr);
}

ck_status check_gemm_args(const int8_t* q, int64_t ldq, const int8_t* w, int64_t ldw,
                          const void* out, int64_t ldo, int64_t m, int64_t n, int64_t k)
{
    if (m < 0 || n < 0 || k < 0) return fail(CK_ERR_INVALID_ARG, "negative size m=%lld n=%lld k=%lld",
                                             (long long)m, (long long)n, (long long)k);
    if (m == 0 || n == 0) return CK_OK;
    if (!out) return fail(CK_ERR_INVALID_ARG, "NULL out");
    if (ldo < n) return fail(CK_ERR_INVALID_ARG, "ldo smaller than n");
    if (k == 0) return CK_OK;            // q and w are never read
    if (!q || !w) return fail(CK_ERR_INVALID_ARG, "NULL q or w");
    if (ldq < k || ldw < k) return fail(CK_ERR_INVALID_ARG, "ldq/ldw smaller than k");
    if (k > CK_MAX_K) return fail(CK_ERR_UNSUPPORTED, "k=%lld > %d may overflow int32", (long long)k, CK_MAX_K);
    if (ldq % 16 != 0 || ldw % 16 != 0 || !aligned(q, 16) || !aligned(w, 16))
        return fail(CK_ERR_UNSUPPORTED,
                    "q and w need 16-byte aligned rows (ldq, ldw multiples of 16; pad rows "
                    "whose k is not)");
    return CK_OK;
}

const char* epi_name(int epi)
{
    return epi == EPI_BF16 ? "bf16" : epi == EPI_F16 ? "fp16" : epi == EPI_F32 ? "fp32" : "int32";
}

// ---------------------------------------------------------------------------
// Tile counters of the persistent kernel
// ---------------------------------------------------------------------------
// Every launch leaves its counters at zero, so launches on one stream can
// share them; launches on different streams may run at the same time, so
// each (device, stream) pair gets its own (hipStreamPerThread: each host
// thread its own).  A slot is cleared by a kernel on its stream, ordered
// before its first use.  Under graph capture no counters are handed out (a
// replay could run beside another launch that shares them) and the caller
// runs the non-persistent kernel instead.
//
// Words of a (device, stream) slot: [0, 10) the persistent kernels' tile
// claims, [12, 14) the two amax cells of the tensor-wide quantisation (the
// one the next call uses is zero).
//
// The slots live in a file-scope device array, so no call ever allocates
// device memory: the runtime places one copy of the array on each device
// when it loads this library's code there, and it stays until the process
// ends.  Host code reaches a device's copy only through the address
// hipGetSymbolAddress returns with that device current (the array's name
// on the host is a stand-in, not a device address).
constexpr int kSchedWords = 16;
constexpr int kSchedAmaxWord = 12;
constexpr int kSchedSlotsPerDevice = 1024;     // 64 KiB per device

static __device__ __align__(256) unsigned g_counter_pool[kSchedSlotsPerDevice * kSchedWords];

__global__ void zero_words_kernel(unsigned* p, int n)
{
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

struct SchedKey {
    int dev;
    hipStream_t stream;
    std::thread::id thread;
    bool operator<(const SchedKey& o) const
    {
        return std::tie(dev, stream, thread) < std::tie(o.dev, o.stream, o.thread);
    }
};
std::mutex g_sched_mu;
std::map<SchedKey, unsigned*> g_sched;   // slot of each (device, stream)
std::map<int, std::pair<unsigned*, int>> g_sched_pool;   // device -> (its pool copy, slots used)

unsigned* sched_counters(hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return nullptr;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    const SchedKey key{dev, stream,
                       stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
    std::lock_guard<std::mutex> lk(g_sched_mu);
    auto it = g_sched.find(key);
    if (it != g_sched.end()) return it->second;
    auto& pool = g_sched_pool[dev];
    if (!pool.first) {
        void* base = nullptr;
        if (hipGetSymbolAddress(&base, HIP_SYMBOL(g_counter_pool)) != hipSuccess || !base) {
            (void)hipGetLastError();
            return nullptr;
        }
        pool = {static_cast<unsigned*>(base), 0};
    }
    if (pool.second >= kSchedSlotsPerDevice) return nullptr;   // then the non-persistent kernel runs
    unsigned* p = pool.first + (size_t)pool.second++ * kSchedWords;
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, p, kSchedWords);
    if (hipGetLastError() != hipSuccess) return nullptr;       // the slot stays unused
    g_sched.emplace(key, p);
    return p;
}

// Which of a block's two amax cells the next tensor-wide quantisation on
// that stream uses.  The mutex is held across both launches of a call, so
// the cells are used in the order the calls are enqueued, also when several
// host threads share the stream.
std::mutex g_amax_mu;
std::map<const unsigned*, unsigned> g_amax_parity;

// ---------------------------------------------------------------------------
// Scratch of ck_int8_linear_noalloc
// ---------------------------------------------------------------------------
// One fixed array per device holds the persistent kernel's tile-claim
// counters for the allocation-free entry point: no per-stream slot, no
// host bookkeeping per call.  Every call of that entry point on a device
// shares the device's copy, which keeps the last call's contents; each call
// zeroes the counters it uses with a kernel on its own stream before the
// GEMM (a kernel, not a memset, so the call can be captured into a graph).
// Calls whose kernels overlap on one device (other streams, graph replays
// running at the same time) race on the counters.  The host reaches a
// device's copy only through the address hipGetSymbolAddress gives with
// that device current; the array's name on the host is a stand-in.
constexpr int kScratchBytes = 256;
constexpr int kClaimWords = 10;                  // sched[0..9] of the persistent kernel
static_assert(kClaimWords * sizeof(unsigned) <= (size_t)kScratchBytes, "claims fit the scratch");

static __device__ __align__(256) unsigned scratch[kScratchBytes / sizeof(unsigned)];

std::mutex g_scratch_mu;
std::atomic<unsigned*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on
// that device, with the device current).
ck_status scratch_on_device(unsigned** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CK_ERR_HIP, "device id %d out of range", dev);
    unsigned* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!p) {
            void* a = nullptr;
            e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !a)
                return fail(CK_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
            p = static_cast<unsigned*>(a);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return CK_OK;
}

// scratch_counters: the persistent kernel's counters come from there
// (cleared first on the stream) instead of the stream's slot.
ck_status run_gemm(GemmArgs& g, int tile, int group_m, int epi, Source src, hipStream_t stream,
                   unsigned* scratch_counters = nullptr)
{
    const TileCfg& t = tiles()[tile];
    const int64_t tm = cdiv(g.m, t.bm), tn = cdiv(g.n, t.bn);
    if (tm * tn > 0x7fffffffLL || tm > 0x7fffffffLL / 2)
        return fail(CK_ERR_UNSUPPORTED, "too many tiles (%lld)", (long long)(tm * tn));
    g.tiles_m = (int)tm;
    g.tiles_n = (int)tn;
    // A group never spans more row tiles than there are (so group_m *
    // tiles_n stays within the tile count, which fits in int).
    if (group_m > g.tiles_m) group_m = g.tiles_m;
    g.group_m = group_m;
    void* args[] = {&g};
    const bool tail = g.k % kBK != 0;
    // The DMA kernel keeps a tile's row offsets in 32 bits.
    const bool dma = t.dma && (int64_t)t.bm * g.ldq < (1LL << 31) &&
                     (int64_t)t.bn * g.ldw < (1LL << 31);
    const void* fn = dma ? t.dma_fn[epi] : tail ? t.reg_tail_fn[epi] : t.reg_fn[epi];
    g.stream_out = tm * tn > 2 * kNumCUs ? 1 : 0;
    // The persistent kernel runs one block per CU when there are more tiles
    // than CUs (with fewer it would be tile 12 with NT stores); blocks claim
    // tiles through per-stream counters (none under graph capture: then
    // tile 12's kernel runs).
    const void* pfn = t.persist_fn[epi][g.bias != nullptr ? 1 : 0];
    bool persist = dma && pfn && g.k > 0 && g.k % t.dma_bk == 0 && tm * tn > kNumCUs;
    if (persist && scratch_counters) {
        int nw = kClaimWords;
        void* zargs[] = {(void*)&scratch_counters, (void*)&nw};
        const ck_status z = launch(reinterpret_cast<const void*>(&zero_words_kernel), 1, 64, zargs,
                                   stream, "scratch clear");
        if (z != CK_OK) return z;
        g.sched = scratch_counters;
    } else {
        g.sched = persist ? sched_counters(stream) : nullptr;
    }
    persist = persist && g.sched;
    if (persist) fn = pfn;
    const int64_t blocks = persist ? kNumCUs : tm * tn;
    const ck_status s = launch(fn, (unsigned)blocks, (unsigned)t.threads, args, stream, "gemm");
    if (s == CK_OK && log_paths()) {
        char text[320];
        const int64_t step = dma ? t.dma_bk : kBK;
        snprintf(text, sizeof text,
                 "gemm %lldx%lldx%lld out=%s tile=%d (%dx%d, %d threads, %s%s %lld-byte K stages"
                 ", K tail %lld bytes) group_m=%d blocks=%lld stores=%s source=%s%s",
                 (long long)g.m, (long long)g.n, (long long)g.k, epi_name(epi), tile, t.bm, t.bn,
                 t.threads, persist ? "persistent " : "", dma ? "direct-to-LDS" : "register-staged",
                 (long long)step, (long long)(g.k % step), group_m, (long long)blocks,
                 g.stream_out ? "streaming" : "cached", kSourceName[src],
                 persist && scratch_counters ? " counters=scratch" : "");
        log_once(scratch_counters ? 4 : 0, g.m, g.n, g.k, epi, tile, group_m, text);
    }
    return s;
}

ck_status linear_impl(const int8_t* q, int64_t ldq, const float* x_scale, ck_scale_mode x_mode,
                      const int8_t* w, int64_t ldw, const float* w_scale, ck_scale_mode w_mode,
                      const void* bias, void* out, int64_t ldo, ck_out_dtype out_dtype,
                      int64_t m, int64_t n, int64_t k, int tile, int group_m, hipStream_t stream,
                      bool use_scratch = false)
{
    if (out_dtype != CK_OUT_BF16 && out_dtype != CK_OUT_FP16 && out_dtype != CK_OUT_FP32)
        return fail(CK_ERR_INVALID_ARG, "bad out_dtype");
    ck_status s = check_gemm_args(q, ldq, w, ldw, out, ldo, m, n, k);
    if (s != CK_OK) return s;
    if (x_mode != CK_SCALE_TENSOR && x_mode != CK_SCALE_ROW) return fail(CK_ERR_INVALID_ARG, "bad x_mode");
    if (w_mode != CK_SCALE_TENSOR && w_mode != CK_SCALE_ROW) return fail(CK_ERR_INVALID_ARG, "bad w_mode");
    if (tile < -1 || tile >= CK_NUM_TILES) return fail(CK_ERR_INVALID_ARG, "unknown tile %d", tile);
    if (group_m < 0) return fail(CK_ERR_INVALID_ARG, "group_m < 0");
    if (m == 0 || n == 0) return ok();
    if (!x_scale || !w_scale) return fail(CK_ERR_INVALID_ARG, "NULL x_scale or w_scale");
    const int esz = out_dtype == CK_OUT_FP32 ? 4 : 2;       // bytes per output / bias element
    if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(out, esz) ||
        (bias && !aligned(bias, esz)))
        return fail(CK_ERR_UNSUPPORTED, "misaligned scale, bias or out");
    Source src;
    choose(m, n, k, tile, group_m, &tile, &group_m, &src);
    if ((s = check_device()) != CK_OK) return s;
    GemmArgs g{};
    g.q = q; g.w = w; g.xs = x_scale; g.ws = w_scale; g.bias = bias; g.out = out;
    g.ldq = ldq; g.ldw = ldw; g.ldo = ldo; g.m = m; g.n = n; g.k = k;
    g.xs_stride = x_mode == CK_SCALE_ROW ? 1 : 0;
    g.ws_stride = w_mode == CK_SCALE_ROW ? 1 : 0;
    int epi;
    if (out_dtype == CK_OUT_FP32) {
        epi = EPI_F32;
        g.vec_store = (ldo % 4 == 0 && aligned(out, 16)) ? 1 : 0;
    } else {
        epi = out_dtype == CK_OUT_FP16 ? EPI_F16 : EPI_BF16;
        g.vec_store = (ldo % 8 == 0 && aligned(out, 16)) ? 2 : (ldo % 4 == 0 && aligned(out, 8)) ? 1 : 0;
    }
    unsigned* counters = nullptr;
    if (use_scratch && (s = scratch_on_device(&counters)) != CK_OK) return s;
    if ((s = run_gemm(g, tile, group_m, epi, src, stream, counters)) != CK_OK) return s;
    return ok();
}

// One-kernel layer for few rows (layer_small_kernel): whether the shape and
// layouts allow it, and whether the library takes it by itself.
constexpr int64_t kLdsBytes = 160 * 1024;

bool layer_small_ok(const uint16_t* x, int64_t ldx, int64_t ldq, ck_scale_mode x_mode, int64_t ldw,
                    int64_t m, int64_t n, int64_t k)
{
    if (m < 1 || n < 1 || k < kLsBK || k % kLsBK != 0 || k > CK_MAX_K) return false;
    if (!aligned(x, 16) || ldx % 8 != 0 || ldq % 8 != 0) return false;
    if (x_mode != CK_SCALE_ROW && m > kLsBM) return false;
    const int64_t rows = m < kLsBM ? m : kLsBM;
    if (kLsHdr + layer_part_bytes((int)rows) + k * rows > kLdsBytes) return false;
    if ((int64_t)kLsBN * ldw + k >= (1LL << 32)) return false;   // 32-bit weight offsets
    return ((m + kLsBM - 1) / kLsBM) * ((n + kLsBN - 1) / kLsBN) < (1LL << 31);
}

// Measured (one kernel against the quantisation kernel + the GEMM, per
// call, back to back): 1 or 2 rows gain 14-18 % (m = 1, 28672 x 5376:
// 25.9 against 30.6 us); 4 rows are even, 8 rows lose 22 %: every block
// quantising the rows again costs more than the launch it saves.
bool layer_small_preferred(int64_t m, int64_t n, int64_t k)
{
    (void)n; (void)k;
    return m <= 2;
}

template <int EPI>
const void* layer_small_fn(bool per_row)
{
    return per_row ? reinterpret_cast<const void*>(&layer_small_kernel<EPI, true>)
                   : reinterpret_cast<const void*>(&layer_small_kernel<EPI, false>);
}

ck_status layer_small(LayerArgs g, int epi, bool per_row, hipStream_t stream)
{
    const void* fn = epi == EPI_F32 ? layer_small_fn<EPI_F32>(per_row)
                   : epi == EPI_F16 ? layer_small_fn<EPI_F16>(per_row)
                                    : layer_small_fn<EPI_BF16>(per_row);
    const int64_t tm = (g.m + kLsBM - 1) / kLsBM, tn = (g.n + kLsBN - 1) / kLsBN;
    g.tiles_m = (int)tm;
    g.rows = (int)(g.m < kLsBM ? g.m : kLsBM);
    const size_t bytes = (size_t)kLsHdr + layer_part_bytes(g.rows) + (size_t)(g.k / kLsBK) * g.rows * kLsBK;
    // allow up to the whole LDS as dynamic shared memory (once per kernel)
    static std::mutex mu;
    static std::set<const void*> raised;
    {
        std::lock_guard<std::mutex> lk(mu);
        if (!raised.count(fn)) {
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)kLdsBytes);
            if (e != hipSuccess) return fail(CK_ERR_HIP, "layer: hipFuncSetAttribute: %s", hipGetErrorString(e));
            raised.insert(fn);
        }
    }
    void* args[] = {&g};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(tm * tn)), dim3(256), args, bytes, stream);
    if (e != hipSuccess) return fail(CK_ERR_HIP, "layer launch: %s", hipGetErrorString(e));
    if (log_paths()) {
        char text[256];
        snprintf(text, sizeof text,
                 "layer %lldx%lldx%lld out=%s x_scale=%s one kernel (quantisation in the GEMM "
                 "blocks, %d code rows in LDS, %zu bytes of LDS) blocks=%lld",
                 (long long)g.m, (long long)g.n, (long long)g.k, epi_name(epi),
                 per_row ? "row" : "tensor", g.rows, bytes, (long long)(tm * tn));
        log_once(5, g.m, g.n, g.k, epi, per_row ? 1 : 0, 0, text);
    }
    return CK_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

ck_status ck_quantize_int8_rowwise(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                                   int8_t* q, int64_t ldq, float* scale, ck_scale_mode mode,
                                   hipStream_t stream)
{
    if (mode != CK_SCALE_TENSOR && mode != CK_SCALE_ROW) return fail(CK_ERR_INVALID_ARG, "bad mode");
    if (m < 0 || k < 0) return fail(CK_ERR_INVALID_ARG, "negative size");
    if (!scale) return fail(CK_ERR_INVALID_ARG, "NULL scale");
    if (m > 0 && k > 0) {
        if (!x || !q) return fail(CK_ERR_INVALID_ARG, "NULL x or q");
        if (ldx < k || ldq < k) return fail(CK_ERR_INVALID_ARG, "ldx/ldq smaller than k");
        if (!aligned(x, 2)) return fail(CK_ERR_UNSUPPORTED, "misaligned x");
    }
    if (!aligned(scale, 4)) return fail(CK_ERR_UNSUPPORTED, "misaligned scale");
    if (mode == CK_SCALE_ROW && m == 0) return ok();
    if (m / kQzWaves + 1 > 0x7fffffffLL) return fail(CK_ERR_UNSUPPORTED, "m too large");
    ck_status s = check_device();
    if (s != CK_OK) return s;

    const unsigned qgrid = (unsigned)((m + kQzWaves - 1) / kQzWaves);
    // 16-byte x rows and 8-byte q rows take the vector kernels
    const bool vec = ldx % 8 == 0 && aligned(x, 16) && ldq % 8 == 0 && aligned(q, 8);
    const void* row_fn = vec ? quantize_row_fn(k, true)
                             : reinterpret_cast<const void*>(&quantize_rows_any_kernel<true>);
    const uint32_t* no_cell = nullptr;
    if (mode == CK_SCALE_ROW) {
        // k == 0 is handled by the row kernel itself: amax 0, scale 0
        void* args[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&q, (void*)&ldq,
                        (void*)&scale, (void*)&no_cell};
        s = launch(row_fn, qgrid, 64 * kQzWaves, args, stream, "quantize_rows");
        if (s == CK_OK && log_paths()) {
            char text[160];
            snprintf(text, sizeof text, "quantize %lldx%lld scales=per-row kernel=%s",
                     (long long)m, (long long)k, vec ? "vector" : "element-wise");
            log_once(1, m, k, 0, 1, vec, 0, text);
        }
        return s == CK_OK ? ok() : s;
    }
    // Tensor-wide: two launches through the stream's alternating amax cells
    // (the amax launch clears the other cell for the next call), or, without
    // counters (graph capture, empty input, unaligned rows), four launches
    // with scale[0] as the cell.
    // Aligned rows: two rows per wave (a multiple of 8 blocks, so that the
    // amax kernel places rows by XCD) up to AMAX_BLOCKS blocks, then more;
    // others: the element-wise kernel, 4 waves a block and at most 512
    // blocks.  One atomic per block either way.
    const int64_t amax_rows_blocks =
        std::min<int64_t>(((m + 2 * AMAX_WAVES - 1) / (2 * AMAX_WAVES) + 7) / 8 * 8, AMAX_BLOCKS);
    const int64_t amax_any_blocks = std::min<int64_t>((m + 3) / 4, 512);
    unsigned* slot = m > 0 && k > 0 && vec ? sched_counters(stream) : nullptr;
    if (slot) {
        std::lock_guard<std::mutex> lk(g_amax_mu);
        unsigned& parity = g_amax_parity[slot];
        uint32_t* cur = slot + kSchedAmaxWord + parity;
        uint32_t* other = slot + kSchedAmaxWord + (parity ^ 1u);
        {
            void* args[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&cur, (void*)&other};
            if ((s = launch(tensor_amax_rows_fn(k), (unsigned)amax_rows_blocks, 64 * AMAX_WAVES, args,
                            stream, "tensor_amax")) != CK_OK)
                return s;
        }
        parity ^= 1u;                              // cur is used, other is zero
        const uint32_t* ccur = cur;
        void* args[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&q, (void*)&ldq,
                        (void*)&scale, (void*)&ccur};
        if ((s = launch(quantize_row_fn(k, false), qgrid, 64 * kQzWaves, args, stream,
                        "quantize_rows_tensor")) != CK_OK)
            return s;
        if (log_paths()) {
            char text[160];
            snprintf(text, sizeof text, "quantize %lldx%lld scales=tensor-wide kernel=vector "
                     "amax=two launches", (long long)m, (long long)k);
            log_once(1, m, k, 0, 0, 1, 1, text);
        }
        return ok();
    }
    uint32_t* cell = reinterpret_cast<uint32_t*>(scale);
    uint32_t* no_clear = nullptr;
    {
        void* args[] = {(void*)&cell};
        if ((s = launch(reinterpret_cast<const void*>(&tensor_amax_zero_kernel), 1, 1, args, stream,
                        "tensor_amax_zero")) != CK_OK)
            return s;
    }
    if (m > 0 && k > 0) {
        void* args[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&cell, (void*)&no_clear};
        const void* fn = vec ? tensor_amax_rows_fn(k)
                             : reinterpret_cast<const void*>(&tensor_amax_kernel);
        if ((s = launch(fn, (unsigned)(vec ? amax_rows_blocks : amax_any_blocks), vec ? 64 * AMAX_WAVES : 256,
                        args, stream, "tensor_amax")) != CK_OK)
            return s;
    }
    {
        void* args[] = {(void*)&scale};
        if ((s = launch(reinterpret_cast<const void*>(&tensor_amax_final_kernel), 1, 1, args, stream,
                        "tensor_amax_final")) != CK_OK)
            return s;
    }
    if (m > 0) {
        void* args[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&q, (void*)&ldq,
                        (void*)&scale, (void*)&no_cell};
        const void* fn = vec ? quantize_row_fn(k, false)
                             : reinterpret_cast<const void*>(&quantize_rows_any_kernel<false>);
        if ((s = launch(fn, qgrid, 64 * kQzWaves, args, stream, "quantize_rows_tensor")) != CK_OK)
            return s;
    }
    if (log_paths()) {
        char text[160];
        snprintf(text, sizeof text, "quantize %lldx%lld scales=tensor-wide kernel=%s "
                 "amax=four launches", (long long)m, (long long)k, vec ? "vector" : "element-wise");
        log_once(1, m, k, 0, 0, vec, 0, text);
    }
    return ok();
}

ck_status ck_quantize_int8_rotated(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                                   int64_t block, int8_t* q, int64_t ldq, float* scale,
                                   ck_scale_mode mode, hipStream_t stream)
{
    if (mode != CK_SCALE_TENSOR && mode != CK_SCALE_ROW) return fail(CK_ERR_INVALID_ARG, "bad mode");
    if (m < 0 || k < 0) return fail(CK_ERR_INVALID_ARG, "negative size");
    if (!scale) return fail(CK_ERR_INVALID_ARG, "NULL scale");
    if (block < 1 || block > 512 || (block & (block - 1)) != 0)
        return fail(CK_ERR_INVALID_ARG, "block %lld is not a power of two in [1, 512]",
                    (long long)block);
    if (k % block != 0)
        return fail(CK_ERR_INVALID_ARG, "k=%lld is not a multiple of block %lld", (long long)k,
                    (long long)block);
    if (m > 0 && k > 0) {
        if (!x || !q) return fail(CK_ERR_INVALID_ARG, "NULL x or q");
        if (ldx < k || ldq < k) return fail(CK_ERR_INVALID_ARG, "ldx/ldq smaller than k");
        if (k % 8 != 0) return fail(CK_ERR_UNSUPPORTED, "rotated rows need k %% 8 == 0");
        if (ldx % 8 != 0 || !aligned(x, 16) || ldq % 8 != 0 || !aligned(q, 8))
            return fail(CK_ERR_UNSUPPORTED,
                        "rotated rows need 16-byte aligned x rows and 8-byte aligned q rows");
    }
    if (!aligned(scale, 4)) return fail(CK_ERR_UNSUPPORTED, "misaligned scale");
    if (mode == CK_SCALE_ROW && m == 0) return ok();
    if (m / kQzWaves + 1 > 0x7fffffffLL) return fail(CK_ERR_UNSUPPORTED, "m too large");
    ck_status s = check_device();
    if (s != CK_OK) return s;

    const unsigned grid = (unsigned)((m + kQzWaves - 1) / kQzWaves);
    // Amax pass, one atomic per block: past 512 row groups two groups per
    // block (a multiple of 8 blocks), at most ROT_AMAX_BLOCKS; fewer groups
    // keep a block each (300 x 1024: 7.3 us that way, 8.1 us with 40 blocks).
    const unsigned amax_half = ((grid + 1) / 2 + 7) / 8 * 8;
    const unsigned amax_grid = grid <= 512 ? grid : std::min(amax_half, (unsigned)ROT_AMAX_BLOCKS);
    int lb = 0;
    while ((1LL << lb) < block) ++lb;
    const float r = (float)(1.0 / sqrt((double)block));
    uint32_t* no_clear = nullptr;
    const uint32_t* no_cell = nullptr;
    void* args[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&q, (void*)&ldq,
                    (void*)&scale, (void*)&r, (void*)&no_clear, (void*)&no_cell};
    if (mode == CK_SCALE_ROW) {
        s = launch(quantize_rot_fn_mode<ROT_ROW>(k, lb), grid, 64 * kQzWaves, args, stream,
                   "quantize_rot_rows");
        if (s == CK_OK && log_paths()) {
            char text[160];
            snprintf(text, sizeof text, "quantize %lldx%lld scales=per-row rotation block=%lld",
                     (long long)m, (long long)k, (long long)block);
            log_once(2, m, k, block, 1, 0, 0, text);
        }
        return s == CK_OK ? ok() : s;
    }
    // Tensor-wide: two launches through the stream's amax cells, as in
    // ck_quantize_int8_rowwise, or four with scale[0] as the cell.
    unsigned* slot = m > 0 && k > 0 ? sched_counters(stream) : nullptr;
    if (slot) {
        std::lock_guard<std::mutex> lk(g_amax_mu);
        unsigned& parity = g_amax_parity[slot];
        uint32_t* cur = slot + kSchedAmaxWord + parity;
        uint32_t* other = slot + kSchedAmaxWord + (parity ^ 1u);
        float* cur_f = reinterpret_cast<float*>(cur);
        {
            void* a0[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&q, (void*)&ldq,
                          (void*)&cur_f, (void*)&r, (void*)&other, (void*)&no_cell};
            if ((s = launch(quantize_rot_fn_mode<ROT_TENSOR_AMAX>(k, lb), amax_grid, 64 * kQzWaves, a0,
                            stream, "quantize_rot_amax")) != CK_OK)
                return s;
        }
        parity ^= 1u;                              // cur is used, other is zero
        const uint32_t* ccur = cur;
        void* a1[] = {(void*)&x, (void*)&m, (void*)&k, (void*)&ldx, (void*)&q, (void*)&ldq,
                      (void*)&scale, (void*)&r, (void*)&no_clear, (void*)&ccur};
        if ((s = launch(quantize_rot_fn_mode<ROT_TENSOR_CODES>(k, lb), grid, 64 * kQzWaves, a1,
                        stream, "quantize_rot_codes")) != CK_OK)
            return s;
        if (log_paths()) {
            char text[160];
            snprintf(text, sizeof text, "quantize %lldx%lld scales=tensor-wide rotation block=%lld "
                     "amax=two launches", (long long)m, (long long)k, (long long)block);
            log_once(2, m, k, block, 0, 0, 1, text);
        }
        return ok();
    }
    uint32_t* cell = reinterpret_cast<uint32_t*>(scale);
    {
        void* a0[] = {(void*)&cell};
        if ((s = launch(reinterpret_cast<const void*>(&tensor_amax_zero_kernel), 1, 1, a0, stream,
                        "tensor_amax_zero")) != CK_OK)
            return s;
    }
    if (m > 0 && k > 0) {
        if ((s = launch(quantize_rot_fn_mode<ROT_TENSOR_AMAX>(k, lb), amax_grid, 64 * kQzWaves, args, stream,
                        "quantize_rot_amax")) != CK_OK)
            return s;
    }
    {
        void* a1[] = {(void*)&scale};
        if ((s = launch(reinterpret_cast<const void*>(&tensor_amax_final_kernel), 1, 1, a1, stream,
                        "tensor_amax_final")) != CK_OK)
            return s;
    }
    if (m > 0) {
        if ((s = launch(quantize_rot_fn_mode<ROT_TENSOR_CODES>(k, lb), grid, 64 * kQzWaves, args, stream,
                        "quantize_rot_codes")) != CK_OK)
            return s;
    }
    if (log_paths()) {
        char text[160];
        snprintf(text, sizeof text, "quantize %lldx%lld scales=tensor-wide rotation block=%lld "
                 "amax=four launches", (long long)m, (long long)k, (long long)block);
        log_once(2, m, k, block, 0, 0, 0, text);
    }
    return ok();
}

ck_status ck_int8_linear(const int8_t* q, int64_t ldq, const float* x_scale, ck_scale_mode x_mode,
                         const int8_t* w, int64_t ldw, const float* w_scale, ck_scale_mode w_mode,
                         const uint16_t* bias, uint16_t* out, int64_t ldo, int64_t m, int64_t n,
                         int64_t k, hipStream_t stream)
{
    return linear_impl(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                       CK_OUT_BF16, m, n, k, -1, 0, stream);
}

ck_status ck_int8_linear_tiled(const int8_t* q, int64_t ldq, const float* x_scale,
                               ck_scale_mode x_mode, const int8_t* w, int64_t ldw,
                               const float* w_scale, ck_scale_mode w_mode, const uint16_t* bias,
                               uint16_t* out, int64_t ldo, int64_t m, int64_t n, int64_t k,
                               int tile, int group_m, hipStream_t stream)
{
    return linear_impl(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                       CK_OUT_BF16, m, n, k, tile, group_m, stream);
}

ck_status ck_int8_linear_ex(const int8_t* q, int64_t ldq, const float* x_scale,
                            ck_scale_mode x_mode, const int8_t* w, int64_t ldw,
                            const float* w_scale, ck_scale_mode w_mode, const void* bias,
                            void* out, int64_t ldo, ck_out_dtype out_dtype, int64_t m, int64_t n,
                            int64_t k, int tile, int group_m, hipStream_t stream)
{
    return linear_impl(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                       out_dtype, m, n, k, tile, group_m, stream);
}

ck_status ck_int8_linear_noalloc(const int8_t* q, int64_t ldq, const float* x_scale,
                                 ck_scale_mode x_mode, const int8_t* w, int64_t ldw,
                                 const float* w_scale, ck_scale_mode w_mode, const void* bias,
                                 void* out, int64_t ldo, ck_out_dtype out_dtype, int64_t m,
                                 int64_t n, int64_t k, int tile, int group_m, hipStream_t stream)
{
    return linear_impl(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                       out_dtype, m, n, k, tile, group_m, stream, true);
}

ck_status ck_int8_layer(const uint16_t* x, int64_t ldx, int8_t* q, int64_t ldq, float* x_scale,
                        ck_scale_mode x_mode, const int8_t* w, int64_t ldw, const float* w_scale,
                        ck_scale_mode w_mode, const void* bias, void* out, int64_t ldo,
                        ck_out_dtype out_dtype, int64_t m, int64_t n, int64_t k, int fused,
                        hipStream_t stream)
{
    if (fused < -1 || fused > 1) return fail(CK_ERR_INVALID_ARG, "fused must be -1, 0 or 1");
    if (out_dtype != CK_OUT_BF16 && out_dtype != CK_OUT_FP16 && out_dtype != CK_OUT_FP32)
        return fail(CK_ERR_INVALID_ARG, "bad out_dtype");
    if (x_mode != CK_SCALE_TENSOR && x_mode != CK_SCALE_ROW) return fail(CK_ERR_INVALID_ARG, "bad x_mode");
    if (w_mode != CK_SCALE_TENSOR && w_mode != CK_SCALE_ROW) return fail(CK_ERR_INVALID_ARG, "bad w_mode");
    // every argument of both steps is checked before anything is launched
    ck_status s = check_gemm_args(q, ldq, w, ldw, out, ldo, m, n, k);
    if (s != CK_OK) return s;
    if (!x_scale) return fail(CK_ERR_INVALID_ARG, "NULL x_scale");
    if (m > 0 && k > 0) {
        if (!x || !q) return fail(CK_ERR_INVALID_ARG, "NULL x or q");
        if (ldx < k || ldq < k) return fail(CK_ERR_INVALID_ARG, "ldx/ldq smaller than k");
        if (!aligned(x, 2)) return fail(CK_ERR_UNSUPPORTED, "misaligned x");
    }
    const int esz = out_dtype == CK_OUT_FP32 ? 4 : 2;
    if (!aligned(x_scale, 4) || (m > 0 && n > 0 && (!w_scale || !aligned(w_scale, 4))) ||
        (m > 0 && n > 0 && (!aligned(out, esz) || (bias && !aligned(bias, esz)))))
        return fail(m > 0 && n > 0 && !w_scale ? CK_ERR_INVALID_ARG : CK_ERR_UNSUPPORTED,
                    "NULL w_scale, or misaligned scale, bias or out");
    const bool can = layer_small_ok(x, ldx, ldq, x_mode, ldw, m, n, k);
    if (fused == 1 && !can)
        return fail(CK_ERR_UNSUPPORTED, "one-kernel layer needs m, n >= 1, k a positive multiple of "
                    "64, 16-byte aligned x rows, per-row scales or m <= %d, and %d + 128 r (rounded "
                    "up to 256) + r k <= %lld bytes of LDS, r = min(m, %d)", kLsBM, kLsHdr,
                    (long long)kLdsBytes, kLsBM);
    if (!(can && (fused == 1 || (fused == -1 && layer_small_preferred(m, n, k))))) {
        if ((s = ck_quantize_int8_rowwise(x, m, k, ldx, q, ldq, x_scale, x_mode, stream)) != CK_OK) return s;
        return linear_impl(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                           out_dtype, m, n, k, -1, 0, stream);
    }
    if ((s = check_device()) != CK_OK) return s;
    LayerArgs g{};
    g.x = x; g.q = q; g.xs = x_scale; g.w = w; g.ws = w_scale; g.bias = bias; g.out = out;
    g.ldx = ldx; g.ldq = ldq; g.ldw = ldw; g.ldo = ldo; g.m = m; g.n = n; g.k = k;
    g.ws_stride = w_mode == CK_SCALE_ROW ? 1 : 0;
    int epi;
    if (out_dtype == CK_OUT_FP32) {
        epi = EPI_F32;
        g.vec_store = (ldo % 4 == 0 && aligned(out, 16)) ? 1 : 0;
    } else {
        epi = out_dtype == CK_OUT_FP16 ? EPI_F16 : EPI_BF16;
        g.vec_store = (ldo % 4 == 0 && aligned(out, 8)) ? 1 : 0;
    }
    if ((s = layer_small(g, epi, x_mode == CK_SCALE_ROW, stream)) != CK_OK) return s;
    return ok();
}

#ifndef DQ_FEW_ROWS
#define DQ_FEW_ROWS 64
#endif
ck_status ck_int8_linear_dequant(const uint16_t* x, int64_t ldx, const int8_t* w, int64_t ldw,
                                 const float* w_scale, ck_scale_mode w_mode, const void* bias,
                                 void* out, int64_t ldo, ck_out_dtype out_dtype, int64_t m,
                                 int64_t n, int64_t k, hipStream_t stream)
{
    if (out_dtype != CK_OUT_BF16 && out_dtype != CK_OUT_FP16 && out_dtype != CK_OUT_FP32)
        return fail(CK_ERR_INVALID_ARG, "bad out_dtype");
    if (w_mode != CK_SCALE_TENSOR && w_mode != CK_SCALE_ROW) return fail(CK_ERR_INVALID_ARG, "bad w_mode");
    if (m < 0 || n < 0 || k < 0) return fail(CK_ERR_INVALID_ARG, "negative size");
    if (m == 0 || n == 0) return ok();
    if (!out) return fail(CK_ERR_INVALID_ARG, "NULL out");
    if (ldo < n) return fail(CK_ERR_INVALID_ARG, "ldo smaller than n");
    if (!w_scale) return fail(CK_ERR_INVALID_ARG, "NULL w_scale");
    if (k > 0) {
        if (!x || !w) return fail(CK_ERR_INVALID_ARG, "NULL x or w");
        if (ldx < k || ldw < k) return fail(CK_ERR_INVALID_ARG, "ldx/ldw smaller than k");
        if (ldx % 8 != 0 || !aligned(x, 16))
            return fail(CK_ERR_UNSUPPORTED, "x rows must start 16 bytes apart (ldx %% 8 == 0)");
        if (ldw % 16 != 0 || !aligned(w, 16))
            return fail(CK_ERR_UNSUPPORTED, "w rows must start 16 bytes apart (ldw %% 16 == 0)");
    }
    const int esz = out_dtype == CK_OUT_FP32 ? 4 : 2;
    if (!aligned(w_scale, 4) || !aligned(out, esz) || (bias && !aligned(bias, esz)))
        return fail(CK_ERR_UNSUPPORTED, "misaligned scale, bias or out");
    const int epi = out_dtype == CK_OUT_FP32 ? EPI_F32 : out_dtype == CK_OUT_FP16 ? EPI_F16 : EPI_BF16;
    if (m <= DQ_FEW_ROWS) {
        // Few rows: one block per 32 columns, K split over 4 waves from 256
        // blocks (8192 columns) on and over 8 below (one row: 8192 x 8192 15
        // against 17 us, 4096 x 4096 9 against 8 us, 28672 x 5376 28 against
        // 29 us); 16 waves were slower on every shape measured.
        const int64_t blocks = cdiv(n, 32);
        if (blocks > 0x7fffffffLL) return fail(CK_ERR_UNSUPPORTED, "too many column blocks");
        // 32-bit lane offsets from the block's first W row (31 rows on) and
        // from x's first row (63 rows of 2 ldx bytes on)
        if (32 * ldw >= (1LL << 31) || 128 * ldx >= (1LL << 31))
            return fail(CK_ERR_UNSUPPORTED, "rows too long for 32-bit offsets");
        ck_status s = check_device();
        if (s != CK_OK) return s;
        GemmArgs g{};
        g.q = reinterpret_cast<const int8_t*>(x); g.w = w; g.ws = w_scale; g.bias = bias; g.out = out;
        g.ldq = 2 * ldx; g.ldw = ldw; g.ldo = ldo; g.m = m; g.n = n; g.k = k;
        g.ws_stride = w_mode == CK_SCALE_ROW ? 1 : 0;
        const int kw = blocks >= 256 ? 4 : 8;
        const int xr = m <= 8 ? 1 : m <= 16 ? 2 : m <= 32 ? 4 : 8;
#define CK_DQ_FEW_X(E, X) (kw == 4 ? reinterpret_cast<const void*>(&gemm_dq_few_kernel<E, 4, X>)    \
                                     : reinterpret_cast<const void*>(&gemm_dq_few_kernel<E, 8, X>))
#define CK_DQ_FEW(E) (xr == 1 ? CK_DQ_FEW_X(E, 1) : xr == 2 ? CK_DQ_FEW_X(E, 2)                     \
                      : xr == 4 ? CK_DQ_FEW_X(E, 4) : CK_DQ_FEW_X(E, 8))
        const void* fn = epi == EPI_F32 ? CK_DQ_FEW(EPI_F32) : epi == EPI_F16 ? CK_DQ_FEW(EPI_F16)
                                                                            : CK_DQ_FEW(EPI_BF16);
#undef CK_DQ_FEW
#undef CK_DQ_FEW_X
        void* args[] = {&g};
        s = launch(fn, (unsigned)blocks, 64u * kw, args, stream, "gemm_dequant");
        if (s == CK_OK && log_paths()) {
            char text[256];
            snprintf(text, sizeof text,
                     "gemm_dequant %lldx%lldx%lld out=%s few rows: 32 columns x %d K parts per block "
                     "(16x16 bf16 MFMA, W and x through per-wave LDS rings, K tail %lld elements) "
                     "blocks=%lld",
                     (long long)m, (long long)n, (long long)k, epi_name(epi), kw, (long long)(k % 64),
                     (long long)blocks);
            log_once(3, m, n, k, epi, 32, 0, text);
        }
        return s == CK_OK ? ok() : s;
    }
    const bool big = cdiv(m, 256) * cdiv(n, 256) >= kNumCUs;
    const int bm = big ? 256 : 64, bn = bm;
    if ((int64_t)bm * 2 * ldx >= (1LL << 31) || (int64_t)bn * ldw >= (1LL << 31))
        return fail(CK_ERR_UNSUPPORTED, "rows too long for 32-bit tile offsets");
    const int64_t tm = cdiv(m, bm), tn = cdiv(n, bn);
    if (tm * tn > 0x7fffffffLL) return fail(CK_ERR_UNSUPPORTED, "too many tiles");
    ck_status s = check_device();
    if (s != CK_OK) return s;
    GemmArgs g{};
    g.q = reinterpret_cast<const int8_t*>(x); g.w = w; g.ws = w_scale; g.bias = bias; g.out = out;
    g.ldq = 2 * ldx; g.ldw = ldw; g.ldo = ldo; g.m = m; g.n = n; g.k = k;
    g.ws_stride = w_mode == CK_SCALE_ROW ? 1 : 0;
    g.tiles_m = (int)tm; g.tiles_n = (int)tn; g.group_m = tm < 4 ? (int)tm : 4;
    // 16-bit outputs with 16-byte aligned rows go through the LDS-staged
    // epilogue (vec_store 2), non-temporally past two waves of tiles.
    if (out_dtype == CK_OUT_FP32) g.vec_store = (ldo % 4 == 0 && aligned(out, 16)) ? 1 : 0;
    else g.vec_store = (ldo % 8 == 0 && aligned(out, 16)) ? 2 : (ldo % 4 == 0 && aligned(out, 8)) ? 1 : 0;
    g.stream_out = tm * tn > 2 * kNumCUs ? 1 : 0;
    const void* fn;
    // More 256x256 tiles than CUs: one block per CU claims tiles (per-stream
    // counters; none under graph capture, then one block per tile).
    g.sched = big && tm * tn > kNumCUs ? sched_counters(stream) : nullptr;
    const bool persist = g.sched != nullptr;
    if (persist)
        fn = epi == EPI_F32 ? reinterpret_cast<const void*>(&gemm_dq_persist_kernel<256, 256, 2, 4, EPI_F32>)
           : epi == EPI_F16 ? reinterpret_cast<const void*>(&gemm_dq_persist_kernel<256, 256, 2, 4, EPI_F16>)
                            : reinterpret_cast<const void*>(&gemm_dq_persist_kernel<256, 256, 2, 4, EPI_BF16>);
    else if (big)
        fn = epi == EPI_F32 ? reinterpret_cast<const void*>(&gemm_dq_kernel<256, 256, 2, 4, EPI_F32>)
           : epi == EPI_F16 ? reinterpret_cast<const void*>(&gemm_dq_kernel<256, 256, 2, 4, EPI_F16>)
                            : reinterpret_cast<const void*>(&gemm_dq_kernel<256, 256, 2, 4, EPI_BF16>);
    else
        fn = epi == EPI_F32 ? reinterpret_cast<const void*>(&gemm_dq_kernel<64, 64, 2, 2, EPI_F32>)
           : epi == EPI_F16 ? reinterpret_cast<const void*>(&gemm_dq_kernel<64, 64, 2, 2, EPI_F16>)
                            : reinterpret_cast<const void*>(&gemm_dq_kernel<64, 64, 2, 2, EPI_BF16>);
    void* args[] = {&g};
    const int64_t blocks = persist ? kNumCUs : tm * tn;
    s = launch(fn, (unsigned)blocks, big ? 512u : 256u, args, stream, "gemm_dequant");
    if (s == CK_OK && log_paths()) {
        char text[256];
        snprintf(text, sizeof text,
                 "gemm_dequant %lldx%lldx%lld out=%s block=%dx%d (bf16 MFMA, W dequantised into "
                 "LDS, K tail %lld elements) %sblocks=%lld",
                 (long long)m, (long long)n, (long long)k, epi_name(epi), bm, bn,
                 (long long)(k % 64), persist ? "persistent " : "", (long long)blocks);
        log_once(3, m, n, k, epi, bm, 0, text);
    }
    return s == CK_OK ? ok() : s;
}

ck_status ck_int8_gemm_i32(const int8_t* q, int64_t ldq, const int8_t* w, int64_t ldw,
                           int32_t* acc, int64_t ldacc, int64_t m, int64_t n, int64_t k, int tile,
                           hipStream_t stream)
{
    ck_status s = check_gemm_args(q, ldq, w, ldw, acc, ldacc, m, n, k);
    if (s != CK_OK) return s;
    if (tile < -1 || tile >= CK_NUM_TILES) return fail(CK_ERR_INVALID_ARG, "unknown tile %d", tile);
    if (m == 0 || n == 0) return ok();
    if (!aligned(acc, 4)) return fail(CK_ERR_UNSUPPORTED, "misaligned acc");
    int group_m;
    Source src;
    choose(m, n, k, tile, 0, &tile, &group_m, &src);
    if ((s = check_device()) != CK_OK) return s;
    GemmArgs g{};
    g.q = q; g.w = w; g.out = acc;
    g.ldq = ldq; g.ldw = ldw; g.ldo = ldacc; g.m = m; g.n = n; g.k = k;
    g.vec_store = (ldacc % 4 == 0) && aligned(acc, 16);
    if ((s = run_gemm(g, tile, group_m, EPI_I32, src, stream)) != CK_OK) return s;
    return ok();
}

ck_status ck_int8_select_tile(int64_t m, int64_t n, int64_t k, int* tile, int* bm, int* bn,
                              int* group_m)
{
    if (m < 0 || n < 0 || k < 0) return fail(CK_ERR_INVALID_ARG, "negative size");
    int t, g;
    Source src;
    choose(m, n, k, -1, 0, &t, &g, &src);
    if (tile) *tile = t;
    if (bm) *bm = tiles()[t].bm;
    if (bn) *bn = tiles()[t].bn;
    if (group_m) *group_m = g;
    return ok();
}

ck_status ck_int8_tile_info(int tile, int* bm, int* bn, int* threads)
{
    if (tile < 0 || tile >= CK_NUM_TILES) return fail(CK_ERR_INVALID_ARG, "unknown tile %d", tile);
    const TileCfg& t = tiles()[tile];
    if (bm) *bm = t.bm;
    if (bn) *bn = t.bn;
    if (threads) *threads = t.threads;
    return ok();
}

ck_status ck_int8_table_set(int64_t m, int64_t n, int64_t k, int tile, int group_m)
{
    if (m < 0 || n < 0 || k < 0) return fail(CK_ERR_INVALID_ARG, "negative size");
    if (tile < -1 || tile >= CK_NUM_TILES) return fail(CK_ERR_INVALID_ARG, "unknown tile %d", tile);
    if (tile >= 0 && group_m < 1) return fail(CK_ERR_INVALID_ARG, "group_m must be >= 1");
    std::lock_guard<std::mutex> lk(g_host_mu);
    const auto key = std::make_tuple(m, n, k);
    if (tile < 0) g_table.erase(key);
    else g_table[key] = std::make_pair(tile, group_m);
    return ok();
}

ck_status ck_int8_table_clear(void)
{
    std::lock_guard<std::mutex> lk(g_host_mu);
    g_table.clear();
    return ok();
}

int64_t ck_int8_table_size(void)
{
    std::lock_guard<std::mutex> lk(g_host_mu);
    return (int64_t)g_table.size();
}

ck_status ck_int8_set_forced_tile(int tile)
{
    if (tile < -1 || tile >= CK_NUM_TILES) return fail(CK_ERR_INVALID_ARG, "unknown tile %d", tile);
    forced_tile();                            // consume the environment first
    g_forced_tile.store(tile, std::memory_order_release);
    return ok();
}

int ck_int8_forced_tile(void) { return forced_tile(); }

ck_status ck_int8_set_path_log(int on)
{
    log_paths();
    g_log_paths.store(on ? 1 : 0, std::memory_order_release);
    return ok();
}

ck_status ck_hbm_stream(const void* src, int64_t chunks, void* dst, int blocks, int unroll,
                        hipStream_t stream)
{
    if (chunks < 0) return fail(CK_ERR_INVALID_ARG, "negative chunk count");
    if (chunks == 0) return ok();
    if (!src || !dst) return fail(CK_ERR_INVALID_ARG, "NULL src or dst");
    if (!aligned(src, 16) || !aligned(dst, 8)) return fail(CK_ERR_UNSUPPORTED, "src needs 16-byte, dst 8-byte alignment");
    if (blocks < 1) return fail(CK_ERR_INVALID_ARG, "blocks < 1");
    const void* fn = unroll == 1   ? reinterpret_cast<const void*>(&hbm_stream_kernel<1>)
                     : unroll == 2 ? reinterpret_cast<const void*>(&hbm_stream_kernel<2>)
                     : unroll == 4 ? reinterpret_cast<const void*>(&hbm_stream_kernel<4>)
                     : unroll == 8 ? reinterpret_cast<const void*>(&hbm_stream_kernel<8>)
                                   : nullptr;
    if (!fn) return fail(CK_ERR_INVALID_ARG, "unroll must be 1, 2, 4 or 8");
    ck_status s = check_device();
    if (s != CK_OK) return s;
    const v4i* sp = static_cast<const v4i*>(src);
    uint2* dp = static_cast<uint2*>(dst);
    void* args[] = {(void*)&sp, (void*)&dp, (void*)&chunks};
    s = launch(fn, (unsigned)blocks, 256, args, stream, "hbm_stream");
    return s == CK_OK ? ok() : s;
}

ck_status ck_mfma_ceiling(int64_t iters, int mode, int32_t* out, uint32_t seed, hipStream_t stream)
{
    if (iters < 0) return fail(CK_ERR_INVALID_ARG, "negative iteration count");
    if (mode != 0 && mode != 1) return fail(CK_ERR_INVALID_ARG, "mode must be 0 or 1");
    if (!out) return fail(CK_ERR_INVALID_ARG, "NULL out");
    if (!aligned(out, 4)) return fail(CK_ERR_UNSUPPORTED, "misaligned out");
    ck_status s = check_device();
    if (s != CK_OK) return s;
    void* args[] = {(void*)&iters, (void*)&out, (void*)&seed};
    const void* fn = mode == 0 ? reinterpret_cast<const void*>(&mfma_ceiling_kernel<0>)
                               : reinterpret_cast<const void*>(&mfma_ceiling_kernel<1>);
    s = launch(fn, kNumCUs, 512, args, stream, "mfma_ceiling");
    return s == CK_OK ? ok() : s;
}

const char* ck_status_string(ck_status s)
{
    switch (s) {
    case CK_OK: return "CK_OK";
    case CK_ERR_INVALID_ARG: return "CK_ERR_INVALID_ARG";
    case CK_ERR_UNSUPPORTED: return "CK_ERR_UNSUPPORTED";
    case CK_ERR_HIP: return "CK_ERR_HIP";
    case CK_ERR_WRONG_ARCH: return "CK_ERR_WRONG_ARCH";
    }
    return "CK_ERR_UNKNOWN";
}

const char* ck_last_error(void) { return g_err; }

int ck_abi_version(void) { return CK_ABI_VERSION; }

}  // extern "C"
