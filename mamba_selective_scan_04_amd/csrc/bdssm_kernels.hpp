// bdssm_kernels.hpp -- gfx950 (CDNA4, wave64) kernels of the block-restricted
// bidirectional selective scan.  Device code only; the launch plans and the
// C ABI are in bdssm.hip, the launchers in launch_*.hip.
//
// Pages cited (arXiv 2607.02805, "Training Hybrid Block Diffusion Language
// Models with Partial Bidirectionality"):
//   [ABS]  the paper's abstract (newx.sg page, "Abstract").
//   [DE-M] gist.science German page, "Technische Zusammenfassung" > "Methodik".
//   [DE-P] same page, "Problemstellung".
//
// Recurrence (Mamba-1 selective scan, diagonal A; the pages print no formula):
//   forward  hf_t = exp(dt_t A) hf_{t-1} + dt_t B_t x_t      (whole sequence)
//   reverse  hr_t = exp(dt_t A) hr_{t+1} + dt_t B_t x_t      (inside one
//            L-token block, from zero) [ABS], [DE-M]
//   y_t = sum_n C_t[n] (hf_t + hr_t) + Dskip x_t
//
// Design notes (why the kernels look like this on MI355X):
// * The work is an elementwise recurrence, not a contraction, so there is no
//   MFMA.  Per (token, channel, state) it costs one v_exp_f32 (half rate on
//   gfx950), two multiplies and one FMA forward, plus three FMAs for the
//   in-block reverse and the output; at ~0.25-0.375 HBM bytes per element the
//   VALU, not HBM, is the roof.  Everything is arranged to spend VALU slots
//   only on those operations: exp2 with A pre-scaled by log2(e), dt*x formed
//   once per (token, channel), one discretisation shared by both directions,
//   bf16 widened by a shift, B and C broadcast through scalar registers.
// * Lanes map to channels, so every token row of x / dt / y is one coalesced
//   wave access, and B_t, C_t (shared by all channels) are wave-uniform
//   scalar loads.
// * Parallelism over time comes from chunking: chunk-local forward aggregates
//   (decay exponent sum S = sum dt and the local end state), a tiny carry
//   kernel that chains them, then a final pass that starts every chunk from
//   its exact incoming state.  Chunks are multiples of 16 tokens (of L for
//   other block lengths), so an L-block never straddles two chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bdssm_dev {

constexpr int kStates = 16;      // d_state of the register-resident wave kernels
constexpr int kWave = 64;        // gfx950 wavefront
constexpr int kGroup = 16;       // tokens per register-resident group in the bidirectional kernel
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- element io

__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);   // bf16 -> fp32 is exact
}

// A stream element held across loop iterations: bf16 bits zero-extended to 32
// bits.  Carried as 16-bit values, pairs of them get packed into one register
// (v_perm), and the pack waits for both loads as soon as they are issued,
// which undoes a software prefetch.
template <typename Tin> struct Staged { using type = Tin; };
template <> struct Staged<uint16_t> { using type = uint32_t; };
__device__ __forceinline__ float widen_staged(float v) { return v; }
__device__ __forceinline__ float widen_staged(uint32_t v) { return __uint_as_float(v << 16); }

template <typename Tin> __device__ __forceinline__ Tin narrow(float v);
template <> __device__ __forceinline__ float narrow<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t narrow<uint16_t>(float v) {
    __bf16 h = static_cast<__bf16>(v);                          // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// A full lane permutation by DPP (every lane reads a valid source lane: quad
// permutations, row rotations, row mirrors).  Written with a zero old value and
// bound_ctrl so that the compiler folds the move into the instruction that
// consumes it (v_add_f32_dpp and the like).
template <int kCtrl> __device__ __forceinline__ float dpp_perm(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane ^ 7 within 8
constexpr int kDppRor4 = 0x124;         // row_ror:4
constexpr int kDppRor8 = 0x128;         // row_ror:8: lane ^ 8 within a row of 16

// ------------------------------------------------- optional Mamba-1 fusions
// The step size may arrive raw: dt = dt_raw + bias (kDtBias), optionally
// through softplus (kDtSoftplus); the output may be gated by silu(z).
constexpr int kDtPlain = 0, kDtBias = 1, kDtSoftplus = 2;
constexpr float kLn2 = 0.6931471805599453f;

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|).  log1p(w) uses the
// hardware log2 with Goldberg's correction (1991, Theorem 4):
// u = fl(1 + w), log1p(w) = log(u) * w / (u - 1), and = w when u == 1; this
// keeps the relative accuracy for small w that log(1 + w) alone would lose.
__device__ __forceinline__ float softplus_f(float v) {
    const float w = fast_exp2(-__builtin_fabsf(v) * kLog2e);
    const float u = 1.f + w;
    const float l1p = (u == 1.f) ? w : __builtin_amdgcn_logf(u) * kLn2 * (w * __builtin_amdgcn_rcpf(u - 1.f));
    return __builtin_fmaxf(v, 0.f) + l1p;
}

template <int kDt> __device__ __forceinline__ float step_size(float raw, float bias) {
    if constexpr (kDt == kDtPlain) return raw;
    else if constexpr (kDt == kDtBias) return raw + bias;
    else return softplus_f(raw + bias);
}

// silu(z) = z / (1 + e^-z)
__device__ __forceinline__ float silu_f(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + fast_exp2(-z * kLog2e));
}

// Optional per-call features of the bidirectional pass (all may be null):
// the step-size transform (dt_mode, dt_bias), the output gate z, and separate
// reverse-direction operands (dt_r with its own bias dt_bias_r, B_r, C_r,
// A_r), which only the in-block reverse scan reads.
template <typename Tin> struct FuseArgs {
    const float *dt_bias;
    int dt_mode;
    const Tin *z;
    const Tin *dt_r, *B_r, *C_r;
    const float *A_r, *dt_bias_r;
};

// States 2q and 2q+1 of a B or C row.  The row is read as 32-bit words: with a
// wave-uniform address that lets the compiler use scalar loads (s_load_dwordxN)
// and unpack bf16 pairs on the scalar unit instead of spending VALU slots.
__device__ __forceinline__ void load_pair(const uint16_t *row, int q, float &lo, float &hi) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(row)[q];
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ void load_pair(const float *row, int q, float &lo, float &hi) {
    lo = row[2 * q];
    hi = row[2 * q + 1];
}

// Wave-uniform value kept in a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A wave-uniform pointer, asserted as such so that loads through it become
// scalar loads even when the compiler cannot prove uniformity by itself.
template <typename T> __device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)uniform((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)uniform((int)(uint32_t)(a >> 32));
    return reinterpret_cast<T *>(lo | (hi << 32));
}

// Rows of kN fp32 values (A rows, states): float4 accesses when kN % 4 == 0.
template <int kN> __device__ __forceinline__ void load_row(const float *p, float *v) {
    if constexpr (kN % 4 == 0) {
#pragma unroll
        for (int q = 0; q < kN / 4; ++q) {
            const float4 t = reinterpret_cast<const float4 *>(p)[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) v[n] = p[n];
    }
}
template <int kN> __device__ __forceinline__ void store_row(float *p, const float *v) {
    if constexpr (kN % 4 == 0) {
#pragma unroll
        for (int q = 0; q < kN / 4; ++q)
            reinterpret_cast<float4 *>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) p[n] = v[n];
    }
}

// ---------------------------------------------------------- token-row streams
//
// x, dt and y are [batch, T, D] with lanes on channels.  A chunk's rows are
// read and written through a raw buffer resource based at the chunk's first
// row: the lane's byte offset (channel * element size) sits in one VGPR for
// the whole kernel and the row offset (k * D * element size) in a scalar
// register, so streaming a row costs no VALU address arithmetic.  The launch
// plan keeps every chunk below 2^31 bytes per stream.
constexpr int32_t kRawBufferWord3 = 0x00020000;   // gfx9-family raw buffer descriptor
// A byte offset (0xFFFFFF00 as the unsigned 32-bit buffer offset) past any
// buffer range the launch plan creates (every range is below 2^31 bytes): a
// buffer load there is out of range and returns zero.
constexpr int32_t kOutOfRange = (int32_t)0xFFFFFF00u;

// One row of 64 elements from a raw buffer straight into LDS (lane i's element
// lands zero-extended in dword i of the destination).
typedef __attribute__((address_space(3))) void lds_void;
template <int kBytes>
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t rsrc, void *lds_dst, int voffset, int soffset) {
    static_assert(kBytes == 2 || kBytes == 4, "16- or 32-bit elements");
    if constexpr (kBytes == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)lds_dst, 2, voffset, soffset, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)lds_dst, 4, voffset, soffset, 0, 0);
}

template <typename Tin> struct Rows {
    __amdgpu_buffer_rsrc_t rsrc;
    int32_t lane_off;    // channel * sizeof(Tin)
    int32_t pitch;       // D * sizeof(Tin)

    __device__ __forceinline__ Rows(const Tin *first_row, int64_t nrows, int D, int d) {
        pitch = uniform(D * (int32_t)sizeof(Tin));
        lane_off = d * (int32_t)sizeof(Tin);
        // the base and size are wave-uniform; say so, so that the descriptor
        // is built in scalar registers (no per-lane waterfall)
        rsrc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<Tin *>(first_row)), 0,
                                                 uniform((int)(nrows * pitch)), kRawBufferWord3);
    }
    __device__ __forceinline__ Tin load(int k) const;
    __device__ __forceinline__ void store(int k, Tin v) const;
    // load / store at a byte offset of the lane's own choosing (an offset past
    // the rows reads zero / drops the store)
    __device__ __forceinline__ Tin load_at(int32_t off) const;
    __device__ __forceinline__ void store_at(int32_t off, Tin v) const;
};
template <> __device__ __forceinline__ uint16_t Rows<uint16_t>::load(int k) const {
    return __builtin_amdgcn_raw_buffer_load_b16(rsrc, lane_off, k * pitch, 0);
}
template <> __device__ __forceinline__ float Rows<float>::load(int k) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_off, k * pitch, 0));
}
template <> __device__ __forceinline__ void Rows<uint16_t>::store(int k, uint16_t v) const {
    __builtin_amdgcn_raw_buffer_store_b16(v, rsrc, lane_off, k * pitch, 0);
}
template <> __device__ __forceinline__ void Rows<float>::store(int k, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc, lane_off, k * pitch, 0);
}
template <> __device__ __forceinline__ uint16_t Rows<uint16_t>::load_at(int32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b16(rsrc, off, 0, 0);
}
template <> __device__ __forceinline__ float Rows<float>::load_at(int32_t off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0));
}
template <> __device__ __forceinline__ void Rows<uint16_t>::store_at(int32_t off, uint16_t v) const {
    __builtin_amdgcn_raw_buffer_store_b16(v, rsrc, off, 0, 0);
}
template <> __device__ __forceinline__ void Rows<float>::store_at(int32_t off, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc, off, 0, 0);
}

// ------------------------------------------------------------------------
// Chunk-local directional scan, one lane per channel, all 16 states in
// registers.  Used for
//   * aggregates (h0 == nullptr): the state reached from zero over the chunk
//     and S = sum of dt over the chunk, so the chunk acts on an incoming
//     state h as  h -> exp2(A' S) h + h_local;
//   * kDirect: a forward pass over one chunk from h0 (commit without output,
//     prefill of a short context), writing the final state (a separate
//     instantiation so profiles tell the two uses apart).
// kRev scans the chunk from its last token to its first (the reverse
// direction of the full-sequence baseline).
// Tokens stream through a register pipeline of 5-token stages: the loads of
// the next stage are issued before the arithmetic of the current one.
// grid = (ceil(D/64), chunks launched, batch), block = 64.
// hout / sout are indexed by chunk id c = c_first + blockIdx.y over n_chunks.
// kDt: how dt is formed from the dt stream (kDtPlain / kDtBias / kDtSoftplus,
// with the per-channel dt_bias, which may be null).
// Resident waves per SIMD the chunk scan is built for (the launch plans size
// their fine chunks to exactly one round of them): 7 leaves 72 VGPRs, room for
// two stages of 5 tokens without spills.
//
// kBoth (chunk_both_kernel, forward only): the same left-to-right pass also
// forms the chunk's reverse aggregate, the reverse-direction state at the
// chunk's first token from zero after its last,  r = sum_s P_s u_s  with
// P_s the product of the decays of the chunk's tokens before s (P = 1 at the
// first token; r += P u, then P *= dA), into rout; it shares the decays and
// injections of the forward recurrence (7 issue slots per state and token
// instead of 5 + 5 for two passes), and S serves both carries.
constexpr int kChunkWaves = 7;
template <typename Tin, bool kRev, bool kDirect, int kDt, int kN, bool kBoth>
__device__ __forceinline__ void chunk_scan_body(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const float *__restrict__ A, const float *h0, float *hout, float *__restrict__ sout,
    int64_t T, int D, int64_t Tc, int n_chunks, int c_first, const float *__restrict__ dt_bias,
    float *__restrict__ rout)
{
    static_assert(!kBoth || (!kRev && !kDirect), "the two-direction aggregates scan forward from zero");
    constexpr int U = 5;                      // tokens per pipeline stage
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = c_first + blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);   // >= 1

    float a2[kN], h[kN];
    load_row<kN>(A + (int64_t)d * kN, a2);
#pragma unroll
    for (int n = 0; n < kN; ++n) a2[n] *= kLog2e;
    if (kDirect && h0 != nullptr) {
        load_row<kN>(h0 + ((int64_t)b * D + d) * kN, h);
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.f;
    }
    float S = 0.f;
    // kBoth: the reverse aggregate and the running decay product
    float r[kBoth ? kN : 1], P[kBoth ? kN : 1];
    if constexpr (kBoth) {
#pragma unroll
        for (int n = 0; n < kN; ++n) { r[n] = 0.f; P[n] = 1.f; }
    }
    const float bias = (kDt != kDtPlain && dt_bias != nullptr) ? dt_bias[d] : 0.f;
    const int64_t first = (int64_t)b * T + t_begin;           // first row of the chunk
    const Rows<Tin> xs(x + first * D, len, D, d);
    const Rows<Tin> ds(dt + first * D, len, D, d);
    const Tin *bs = Bm + first * kN;
    // step k of the sweep visits row pos(k) of the chunk
    auto pos = [&](int k) -> int { return kRev ? len - 1 - k : k; };

    // Tokens stream through registers in stages of U: a stage's x and dt are
    // loaded one stage ahead into one of two buffers used in turn (the loop is
    // unrolled by two, so no copy between iterations forces an early wait),
    // held as 32-bit values (Staged).  Measured on MI355X at 65,536 tokens x 8
    // x 1536 channels (prefill): 1.735 ms with 5-token stages at 7 waves per
    // SIMD; 1.75 ms with 4 or 6 tokens at 8, 7 or 6 waves; 1.80 ms with 8
    // tokens at 5 waves; 1.89 ms with one 6-token buffer copied forward each
    // stage (the copy and a 16-bit packing of the staged values waited for
    // the loads at once); 1.95 ms with the rows staged in LDS by DMA.
    using St = typename Staged<Tin>::type;
    auto consume = [&](const St *xr, const St *dr, int k0, int count) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (i < count) {
                const float dl = step_size<kDt>(widen_staged(dr[i]), bias);
                const float dx = dl * widen_staged(xr[i]);
                S += dl;
                const Tin *brow = bs + (int64_t)pos(k0 + i) * kN;
#pragma unroll
                for (int q = 0; q < kN / 2; ++q) {
                    float b0, b1;
                    load_pair(brow, q, b0, b1);
                    const float e0 = fast_exp2(dl * a2[2 * q]), e1 = fast_exp2(dl * a2[2 * q + 1]);
                    const float u0 = dx * b0, u1 = dx * b1;
                    h[2 * q] = __builtin_fmaf(e0, h[2 * q], u0);
                    h[2 * q + 1] = __builtin_fmaf(e1, h[2 * q + 1], u1);
                    if constexpr (kBoth) {
                        r[2 * q] = __builtin_fmaf(P[2 * q], u0, r[2 * q]);
                        r[2 * q + 1] = __builtin_fmaf(P[2 * q + 1], u1, r[2 * q + 1]);
                        P[2 * q] *= e0;
                        P[2 * q + 1] *= e1;
                    }
                }
            }
        }
    };
    // count < U: the rows past the chunk re-read its last row
    auto load_stage = [&](int k0, int count, St *xo, St *dout) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int k = pos(k0 + (i < count ? i : count - 1));
            xo[i] = xs.load(k);
            dout[i] = ds.load(k);
        }
    };

    // full stages in the loop (a constant token count, so no per-token
    // branches), the partial one after it
    const int n_full = len / U;
    const int rem = len - n_full * U;
    St xa[U], da[U], xb[U], db[U];
    if (n_full > 0) load_stage(0, U, xa, da);
    int g = 0;
    for (; g + 1 < n_full; g += 2) {
        load_stage((g + 1) * U, U, xb, db);
        consume(xa, da, g * U, U);
        if (g + 2 < n_full) load_stage((g + 2) * U, U, xa, da);
        consume(xb, db, (g + 1) * U, U);
    }
    if (g < n_full) consume(xa, da, g * U, U);       // an odd number of full stages: the last is in xa
    if (rem > 0) {
        load_stage(n_full * U, rem, xb, db);
        consume(xb, db, n_full * U, rem);
    }
    if (live) {
        store_row<kN>(hout + (((int64_t)b * n_chunks + c) * D + d) * kN, h);
        if (!kDirect && sout != nullptr) sout[((int64_t)b * n_chunks + c) * D + d] = S;
        if constexpr (kBoth) store_row<kN>(rout + (((int64_t)b * n_chunks + c) * D + d) * kN, r);
    }
}

template <typename Tin, bool kRev, bool kDirect, int kDt = kDtPlain, int kN = kStates>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(kN > 16 ? 4 : kChunkWaves))) void chunk_state_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const float *__restrict__ A, const float *h0, float *hout, float *__restrict__ sout,
    int64_t T, int D, int64_t Tc, int n_chunks, int c_first, const float *__restrict__ dt_bias)
{
    chunk_scan_body<Tin, kRev, kDirect, kDt, kN, false>(x, dt, Bm, A, h0, hout, sout, T, D, Tc, n_chunks,
                                                         c_first, dt_bias, nullptr);
}

// Forward and reverse aggregates of every chunk in one forward pass (the
// full-sequence baseline with shared operands): hout / sout as for
// chunk_state_kernel, rout the reverse aggregates [batch, n_chunks, D, kN].
// Three state arrays and the decay rows fill the registers: four waves per
// SIMD at 16 states (five spilled).
template <typename Tin, int kDt = kDtPlain, int kN = kStates>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(kN > 16 ? 2 : 4))) void chunk_both_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const float *__restrict__ A, float *hout, float *__restrict__ sout, float *__restrict__ rout,
    int64_t T, int D, int64_t Tc, int n_chunks, const float *__restrict__ dt_bias)
{
    chunk_scan_body<Tin, false, false, kDt, kN, true>(x, dt, Bm, A, nullptr, hout, sout, T, D, Tc, n_chunks, 0,
                                                       dt_bias, rout);
}

// Carry across chunks: one thread per (b, d, n) (n < n_states), sequential
// over chunks.
// Forward: h starts at h_init (or 0); for chunk c < n_agg, h_in[c] = h, then
// h <- exp2(A' S_c) h + h_local_c.  Writes h_in[n_agg] too when requested,
// and the final state.  Reverse (kRev): h starts at 0 on the right, walks
// chunks n_chunks-1 .. c_low, h_in[c] = h (the state entering chunk c from its
// right end), then folds chunk c (aggregates exist for c > c_low).
template <bool kRev>
__global__ __launch_bounds__(256) void carry_kernel(
    const float *__restrict__ agg_h, const float *__restrict__ agg_s, const float *__restrict__ A,
    const float *h_init, float *__restrict__ h_in, float *h_final,
    int batch, int D, int n_states, int n_chunks, int n_agg, int c_low)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)batch * D * n_states;
    if (i >= total) return;
    const int n = (int)(i % n_states);
    const int64_t bd = i / n_states;
    const int d = (int)(bd % D);
    const int64_t b = bd / D;
    const float a2 = A[(int64_t)d * n_states + n] * kLog2e;
    const int64_t cs = (int64_t)D * n_states;     // chunk stride in agg_h / h_in
    const int64_t base_h = b * n_chunks * cs + (int64_t)d * n_states + n;
    const int64_t base_s = b * n_chunks * (int64_t)D + d;
    float h = (h_init != nullptr && !kRev) ? h_init[i] : 0.f;
    if (!kRev) {
        // Groups of 8 chunks: the 16 loads and 8 decays of a group do not
        // depend on h, so only the 8 FMAs form the serial chain.
        int c = 0;
        for (; c + 8 <= n_agg; c += 8) {
            float g[8], l[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                g[k] = fast_exp2(a2 * agg_s[base_s + (int64_t)(c + k) * D]);
                l[k] = agg_h[base_h + (c + k) * cs];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (h_in) h_in[base_h + (c + k) * cs] = h;
                h = __builtin_fmaf(g[k], h, l[k]);
            }
        }
        for (; c < n_agg; ++c) {
            if (h_in) h_in[base_h + c * cs] = h;
            const float s = agg_s[base_s + (int64_t)c * D];
            h = __builtin_fmaf(fast_exp2(a2 * s), h, agg_h[base_h + c * cs]);
        }
        if (h_in && n_agg < n_chunks) h_in[base_h + (int64_t)n_agg * cs] = h;
        if (h_final) h_final[i] = h;
    } else {
        for (int c = n_chunks - 1; c >= c_low; --c) {
            h_in[base_h + c * cs] = h;
            if (c == c_low) break;
            const float s = agg_s[base_s + (int64_t)c * D];
            h = __builtin_fmaf(fast_exp2(a2 * s), h, agg_h[base_h + c * cs]);
        }
    }
}

// The same carry with the chunk sequence cut into W segments, one wave per
// segment (W = blockDim.x / 64, at most 16; lanes: 64 consecutive (b, d, n)).  Each wave
// folds its segment from zero into an affine map (S = sum of the step-size
// sums, H = the segment's state from zero); the maps of the waves before it,
// through LDS, give the state entering its segment; with h_in requested the
// wave walks its segment again from that state and writes the states
// entering its chunks (the reloads hit the cache).  Same outputs as
// carry_kernel; only the rounding order differs (a segment's decay is
// exp2(A' S) of the summed S, not the product of its chunks' decays).
// k counts fold steps: chunk k forward, chunk n_chunks - 1 - k reverse; K =
// n_agg forward, n_chunks - 1 - c_low reverse.
template <bool kRev>
__global__ __launch_bounds__(1024) void carry_tree_kernel(
    const float *__restrict__ agg_h, const float *__restrict__ agg_s, const float *__restrict__ A,
    const float *h_init, float *__restrict__ h_in, float *h_final,
    int batch, int D, int n_states, int n_chunks, int n_agg, int c_low)
{
    __shared__ float seg_h[16][kWave], seg_s[16][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int W = uniform((int)(blockDim.x >> 6));
    const int w = uniform((int)(threadIdx.x >> 6));
    const int64_t total = (int64_t)batch * D * n_states;
    const int64_t i_raw = (int64_t)blockIdx.x * kWave + lane;
    const bool live = i_raw < total;
    const int64_t i = live ? i_raw : total - 1;
    const int n = (int)(i % n_states);
    const int64_t bd = i / n_states;
    const int d = (int)(bd % D);
    const int64_t b = bd / D;
    const float a2 = A[(int64_t)d * n_states + n] * kLog2e;
    const int64_t cs = (int64_t)D * n_states;
    const int64_t base_h = b * n_chunks * cs + (int64_t)d * n_states + n;
    const int64_t base_s = b * n_chunks * (int64_t)D + d;
    const int K = kRev ? n_chunks - 1 - c_low : n_agg;
    const int k0 = (int)((int64_t)K * w / W), k1 = (int)((int64_t)K * (w + 1) / W);
    auto chunk = [&](int k) { return kRev ? n_chunks - 1 - k : k; };

    // the segment from zero: 8 chunks' loads and decays ahead of their FMAs
    float h = 0.f, S = 0.f;
    int k = k0;
    for (; k + 8 <= k1; k += 8) {
        float s[8], l[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            s[j] = agg_s[base_s + (int64_t)chunk(k + j) * D];
            l[j] = agg_h[base_h + chunk(k + j) * cs];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h = __builtin_fmaf(fast_exp2(a2 * s[j]), h, l[j]);
            S += s[j];
        }
    }
    for (; k < k1; ++k) {
        const float s = agg_s[base_s + (int64_t)chunk(k) * D];
        h = __builtin_fmaf(fast_exp2(a2 * s), h, agg_h[base_h + chunk(k) * cs]);
        S += s;
    }
    seg_h[w][lane] = h;
    seg_s[w][lane] = S;
    __syncthreads();
    // the state entering this wave's segment
    float hin = (!kRev && h_init != nullptr) ? h_init[i] : 0.f;
    for (int j = 0; j < w; ++j) hin = __builtin_fmaf(fast_exp2(a2 * seg_s[j][lane]), hin, seg_h[j][lane]);
    float fin = __builtin_fmaf(fast_exp2(a2 * S), hin, h);
    if (h_in != nullptr) {
        float hh = hin;
        int kk = k0;
        for (; kk + 8 <= k1; kk += 8) {
            float s[8], l[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                s[j] = agg_s[base_s + (int64_t)chunk(kk + j) * D];
                l[j] = agg_h[base_h + chunk(kk + j) * cs];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (live) h_in[base_h + chunk(kk + j) * cs] = hh;
                hh = __builtin_fmaf(fast_exp2(a2 * s[j]), hh, l[j]);
            }
        }
        for (; kk < k1; ++kk) {
            if (live) h_in[base_h + chunk(kk) * cs] = hh;
            const float s = agg_s[base_s + (int64_t)chunk(kk) * D];
            hh = __builtin_fmaf(fast_exp2(a2 * s), hh, agg_h[base_h + chunk(kk) * cs]);
        }
        fin = hh;
    }
    if (w == W - 1 && live) {
        if (h_in != nullptr && (kRev || K < n_chunks)) h_in[base_h + chunk(K) * cs] = fin;
        if (h_final != nullptr) h_final[i] = fin;
    }
}

// ------------------------------------------------------------------------
// Bidirectional kernel: forward scan from the chunk's incoming state, reverse
// scan restricted to each L-token block, fused output.
//
// One wave owns 16 channels completely: lane l handles channel l / 4 and
// states 4 (l % 4) .. 4 (l % 4) + 3, so the four lanes of a DPP quad hold the
// 16 states of one channel.  Nothing is shared between waves, so there is no
// barrier at all:
//   * each wave loads its own 16 channels' x / dt rows and the group's B / C
//     rows straight into its own LDS region (lane-varying buffer offsets pack
//     4 tokens x 16 channels, or 4 tokens x 16 states, into one 64-lane load),
//     one group ahead, double-buffered in distinct arrays;
//   * after waiting for its own loads it widens B / C to fp32 in LDS; lanes
//     read x, dt and their 4 states of B / C back as LDS broadcasts;
//   * the output sum over a channel's 16 states is a reduce-scatter inside the
//     quad (two DPP exchange steps), after which each lane owns 4 tokens of
//     its channel.
// The decays of 16 tokens x 4 states stay in VGPRs between the forward pass
// and the in-block reverse pass; dt * x is kept per token and the injections
// are formed again in the reverse pass.  Tokens past the chunk end inside the
// last group re-read the last valid row and are neutralised with dt = 0
// (decay 1, injection 0); they are not stored.
//
// hin: incoming state of chunk c at hin[b*hin_bs + c*hin_cs + d*16 + n].
// kBlockInit (two-stream training form): instead of carrying the forward
// state across blocks, every L-block k starts from h0_blocks[b, k, d, :]
// ([batch, T/L+1, D, 16], the layout of bounds); hin is then unused.
// bounds (optional): forward state at every multiple of L, [batch,T/L+1,D,16].
// hout (optional): forward state after token T-1 (written by the last chunk;
// may alias hin when there is a single chunk: each lane reads its own states
// before it writes them).
// kFuse (optional layer features, FuseArgs; 1: step size and gate, 2: also
// separate reverse operands, a variant of its own so that the others do not
// carry its registers and LDS): dt is formed from the dt stream as
// step_size<dt_mode> with dt_bias (each lane transforms the 4 dt values it
// loaded, in LDS, once per token and channel); when z is given the output is
// multiplied by silu(z) (z rows are loaded with x and dt); when dt_r is given
// the reverse scan takes its own operands (dt_r, B_r, C_r rows staged beside
// the forward ones, decays exp2(dt_r A_r') computed in the reverse pass).
// grid = (ceil(D/64), chunks, batch), block = 256 (4 independent waves).
template <typename Tin, int L, bool kBlockInit, int kFuse = 0>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(2))) void bidir_wave_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    const float *hin, int64_t hin_bs, int64_t hin_cs,
    Tin *__restrict__ y, float *__restrict__ bounds, float *hout,
    int64_t T, int D, int64_t Tc, const float *__restrict__ h0_blocks, FuseArgs<Tin> fz)
{
    constexpr int P = 4;                      // states per lane
    constexpr int CW = kWave / P;             // channels per wave (16)
    constexpr int ES = sizeof(Tin);
    constexpr bool kSep = kFuse == 2;         // separate reverse operands
    constexpr int NS = kSep ? 4 : kFuse ? 3 : 2;   // token-row streams: x, dt (, z (, dt_r))
    constexpr int NR = kSep ? 4 : 2;               // per-token rows: B, C (, B_r, C_r)
    static_assert(kGroup % L == 0, "block length must divide the token group");
    // per wave: token rows [stream][4 loads][64], raw B/C rows [row][4 loads][64]
    // (both double buffered: the next group's loads are in flight), and fp32
    // B/C rows [token][row][16] (single buffer: written after this wave's last
    // read of the previous group, in program order)
    __shared__ uint32_t xdA[4][NS][4][kWave], xdB[4][NS][4][kWave];
    __shared__ uint32_t bcrA[4][NR][4][kWave], bcrB[4][NR][4][kWave];
    __shared__ float bcf[4][kGroup][NR][kStates];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform(threadIdx.x >> 6);
    const int cl = lane >> 2;                 // channel within the wave
    const int g = lane & 3;                   // state group
    const int s0 = P * g;
    const int d_raw = blockIdx.x * kWave + w * CW + cl;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);

    float a2[P], hf[P];
    {
        const float4 av = *reinterpret_cast<const float4 *>(A + (int64_t)d * kStates + s0);
        a2[0] = av.x * kLog2e; a2[1] = av.y * kLog2e; a2[2] = av.z * kLog2e; a2[3] = av.w * kLog2e;
        if (hin != nullptr) {
            const float4 hv = *reinterpret_cast<const float4 *>(
                hin + (int64_t)b * hin_bs + (int64_t)c * hin_cs + (int64_t)d * kStates + s0);
            hf[0] = hv.x; hf[1] = hv.y; hf[2] = hv.z; hf[3] = hv.w;
        } else {
            hf[0] = hf[1] = hf[2] = hf[3] = 0.f;
        }
    }
    const float dsk = Dskip[d];
    const int64_t nbl = T / L;
    auto store_state = [&](float *dst) {
        *reinterpret_cast<float4 *>(dst + s0) = make_float4(hf[0], hf[1], hf[2], hf[3]);
    };
    if (bounds != nullptr && c == 0 && live)
        store_state(bounds + ((int64_t)b * (nbl + 1) * D + d) * kStates);

    const int64_t first = (int64_t)b * T + t_begin;
    // the wave's 16 channels start at channel d_w0 (clamped lanes re-read D-1)
    const int d_w0 = blockIdx.x * kWave + w * CW;
    const Rows<Tin> xs(x + first * D, len, D, 0);
    const Rows<Tin> ds(dt + first * D, len, D, 0);
    __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Bm + first * kStates)), 0, uniform(len * kStates * ES), kRawBufferWord3);
    __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Cm + first * kStates)), 0, uniform(len * kStates * ES), kRawBufferWord3);
    // load j of a group covers tokens 4j .. 4j+3: lane l takes token 4j + l/16
    // and channel (or state) l % 16
    const int ld_tok = lane >> 4, ld_col = lane & 15;
    const int ld_ch = (d_w0 + ld_col < D) ? d_w0 + ld_col : D - 1;
    const bool gate = kFuse && fz.z != nullptr;
    const bool sep = kSep && fz.dt_r != nullptr;
    const Rows<Tin> zs((gate ? fz.z : x) + first * D, len, D, 0);
    const Rows<Tin> rds((sep ? fz.dt_r : x) + first * D, len, D, 0);
    __amdgpu_buffer_rsrc_t rbrs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>((sep ? fz.B_r : Bm) + first * kStates)), 0, uniform(len * kStates * ES), kRawBufferWord3);
    __amdgpu_buffer_rsrc_t rcrs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>((sep ? fz.C_r : Cm) + first * kStates)), 0, uniform(len * kStates * ES), kRawBufferWord3);
    const float ld_bias = (kFuse && fz.dt_bias != nullptr) ? fz.dt_bias[ld_ch] : 0.f;
    const float ld_bias_r = (kSep && sep && fz.dt_bias_r != nullptr) ? fz.dt_bias_r[ld_ch] : 0.f;
    float a2r[P] = {0.f, 0.f, 0.f, 0.f};
    if (kSep && sep) {
        const float4 av = *reinterpret_cast<const float4 *>(fz.A_r + (int64_t)d * kStates + s0);
        a2r[0] = av.x * kLog2e; a2r[1] = av.y * kLog2e; a2r[2] = av.z * kLog2e; a2r[3] = av.w * kLog2e;
    }

    auto issue = [&](auto &xd, auto &bcr, int k0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int k = k0 + 4 * j + ld_tok;
            k = k < len ? k : len - 1;
            load_to_lds<ES>(xs.rsrc, &xd[w][0][j][0], ld_ch * ES + k * xs.pitch, 0);
            load_to_lds<ES>(ds.rsrc, &xd[w][1][j][0], ld_ch * ES + k * ds.pitch, 0);
            load_to_lds<ES>(brs, &bcr[w][0][j][0], (k * kStates + ld_col) * ES, 0);
            load_to_lds<ES>(crs, &bcr[w][1][j][0], (k * kStates + ld_col) * ES, 0);
            if constexpr (kFuse != 0) {
                if (gate) load_to_lds<ES>(zs.rsrc, &xd[w][2][j][0], ld_ch * ES + k * zs.pitch, 0);
            }
            if constexpr (kSep) {
                if (sep) {
                    load_to_lds<ES>(rds.rsrc, &xd[w][3][j][0], ld_ch * ES + k * rds.pitch, 0);
                    load_to_lds<ES>(rbrs, &bcr[w][2][j][0], (k * kStates + ld_col) * ES, 0);
                    load_to_lds<ES>(rcrs, &bcr[w][3][j][0], (k * kStates + ld_col) * ES, 0);
                }
            }
        }
    };
    auto elem = [&](uint32_t v) -> float {
        return ES == 2 ? __uint_as_float(v << 16) : __uint_as_float(v);
    };
    // wait for this wave's own LDS loads (vmcnt = 0), then widen B / C (and,
    // with kFuse, turn the lane's own 4 raw dt (and dt_r) values into fp32 dt)
    auto form_dt = [&](float raw, float bias) -> float {
        if (fz.dt_mode == kDtSoftplus) return step_size<kDtSoftplus>(raw, bias);
        if (fz.dt_mode == kDtBias) return step_size<kDtBias>(raw, bias);
        return raw;
    };
    auto widen_bc = [&](auto &bcr, auto &xd) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
        for (int which = 0; which < 2; ++which)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bcf[w][4 * j + ld_tok][which][ld_col] = elem(bcr[w][which][j][lane]);
        if constexpr (kFuse != 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xd[w][1][j][lane] = __float_as_uint(form_dt(elem(xd[w][1][j][lane]), ld_bias));
        }
        if constexpr (kSep) {
            if (sep) {
#pragma unroll
                for (int which = 2; which < 4; ++which)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        bcf[w][4 * j + ld_tok][which][ld_col] = elem(bcr[w][which][j][lane]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xd[w][3][j][lane] = __float_as_uint(form_dt(elem(xd[w][3][j][lane]), ld_bias_r));
            }
        }
    };
    // dt as stored in LDS: raw stream bits, or fp32 after the fusion transform
    auto dt_elem = [&](uint32_t v) -> float { return kFuse != 0 ? __uint_as_float(v) : elem(v); };
    // quad reduce-scatter helpers (DPP within groups of 4 lanes)
    auto xor2 = [](float v) {
        return dpp_perm<kDppXor2>(v);
    };
    auto xor1 = [](float v) {
        return dpp_perm<kDppXor1>(v);
    };
    Tin *ylane = y + first * D + d;
    const bool hi2 = (g & 2) != 0, hi1 = (g & 1) != 0;

    // two-stream form: the block start states of a group are loaded one group
    // ahead, with that group's rows, so that the wait for the rows at the end
    // of the previous group covers them too (the vector-memory counter is in
    // order: a wait for them placed after a later DMA would wait for the DMA)
    // (for L >= 8; with more blocks per group the states would not fit the
    // registers, and the group loads them itself)
    constexpr int NBk = kBlockInit ? kGroup / L : 1;
    constexpr bool kAhead = kBlockInit && L >= 8;
    float hbn[NBk][P];
    auto load_hb = [&](int k0n) {
        if constexpr (kBlockInit) {
            const int nv = (len - k0n < kGroup) ? len - k0n : kGroup;
#pragma unroll
            for (int q = 0; q < NBk; ++q) {
                const int i = q * L < nv ? q * L : 0;
                const int64_t blk = (t_begin + k0n + i) / L;
                const float4 v = *reinterpret_cast<const float4 *>(
                    h0_blocks + (((int64_t)b * (nbl + 1) + blk) * D + d) * kStates + s0);
                hbn[q][0] = v.x; hbn[q][1] = v.y; hbn[q][2] = v.z; hbn[q][3] = v.w;
            }
        }
    };

    auto group = [&](auto &xd, auto &xdn, auto &bcrn, int k0) {
        const int nvalid = (len - k0 < kGroup) ? len - k0 : kGroup;   // uniform
        const bool more = k0 + kGroup < len;
        if constexpr (kBlockInit && !kAhead) load_hb(k0);
        float hb[NBk][P];
#pragma unroll
        for (int q = 0; q < NBk; ++q)
#pragma unroll
            for (int j = 0; j < P; ++j) hb[q][j] = hbn[q][j];
        if (more) {
            if constexpr (kAhead) load_hb(k0 + kGroup);
            issue(xdn, bcrn, k0 + kGroup);
        }
        float dx[kGroup], dl[kGroup], ya[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const float xv = elem(xd[w][0][i >> 2][(i & 3) * CW + cl]);
            const float dv = dt_elem(xd[w][1][i >> 2][(i & 3) * CW + cl]);
            dl[i] = i < nvalid ? dv : 0.f;
            dx[i] = dl[i] * xv;
            ya[i] = 0.f;
        }
        float dA[kGroup][P];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            if constexpr (kBlockInit) {
                if (i % L == 0) {
#pragma unroll
                    for (int j = 0; j < P; ++j) hf[j] = hb[i / L][j];
                }
            }
            const float4 b4 = *reinterpret_cast<const float4 *>(&bcf[w][i][0][s0]);
            const float4 c4 = *reinterpret_cast<const float4 *>(&bcf[w][i][1][s0]);
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
            float acc = ya[i];
#pragma unroll
            for (int j = 0; j < P; ++j) {
                dA[i][j] = fast_exp2(dl[i] * a2[j]);
                hf[j] = __builtin_fmaf(dA[i][j], hf[j], dx[i] * bv[j]);
                acc = __builtin_fmaf(cv[j], hf[j], acc);
            }
            ya[i] = acc;
            if ((i & 3) == 3) asm volatile("" ::: "memory");
            if ((i + 1) % L == 0 && bounds != nullptr && i < nvalid && live) {
                const int64_t kb = (t_begin + k0 + i + 1) / L;
                store_state(bounds + (((int64_t)b * (nbl + 1) + kb) * D + d) * kStates);
            }
        }
        asm volatile("" ::: "memory");
        float hr[P] = {0.f, 0.f, 0.f, 0.f};
        if (!sep) {
            // shared operands: the forward's decays and injections
#pragma unroll
            for (int i = kGroup - 1; i >= 0; --i) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&bcf[w][i][0][s0]);
                const float4 c4 = *reinterpret_cast<const float4 *>(&bcf[w][i][1][s0]);
                const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
                const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
                if ((i + 1) % L == 0) { hr[0] = hr[1] = hr[2] = hr[3] = 0.f; }
                float acc = ya[i];
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    hr[j] = __builtin_fmaf(dA[i][j], hr[j], dx[i] * bv[j]);
                    acc = __builtin_fmaf(cv[j], hr[j], acc);
                }
                ya[i] = acc;
                if ((i & 3) == 0) asm volatile("" ::: "memory");
            }
        } else if constexpr (kSep) {
            // the reverse scan's own operands: dt_r, B_r, C_r, A_r
#pragma unroll
            for (int i = kGroup - 1; i >= 0; --i) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&bcf[w][i][2][s0]);
                const float4 c4 = *reinterpret_cast<const float4 *>(&bcf[w][i][3][s0]);
                const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
                const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
                if ((i + 1) % L == 0) { hr[0] = hr[1] = hr[2] = hr[3] = 0.f; }
                const float dlr = i < nvalid ? dt_elem(xd[w][3][i >> 2][(i & 3) * CW + cl]) : 0.f;
                const float dxr = dlr * elem(xd[w][0][i >> 2][(i & 3) * CW + cl]);
                float acc = ya[i];
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    hr[j] = __builtin_fmaf(fast_exp2(dlr * a2r[j]), hr[j], dxr * bv[j]);
                    acc = __builtin_fmaf(cv[j], hr[j], acc);
                }
                ya[i] = acc;
                if ((i & 3) == 0) asm volatile("" ::: "memory");
            }
        }
        // reduce-scatter over the quad: after step 1 the lanes with g & 2
        // hold tokens 8..15, the others 0..7; after step 2 lane g holds
        // tokens 4g .. 4g+3 summed over the channel's 16 states
        float r8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float keep = hi2 ? ya[k + 8] : ya[k];
            const float send = hi2 ? ya[k] : ya[k + 8];
            r8[k] = keep + xor2(send);
        }
        float r4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float keep = hi1 ? r8[k + 4] : r8[k];
            const float send = hi1 ? r8[k] : r8[k + 4];
            r4[k] = keep + xor1(send);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * g + q;
            const float xv = elem(xd[w][0][g][q * CW + cl]);
            float tot = __builtin_fmaf(dsk, xv, r4[q]);
            if constexpr (kFuse != 0) {
                if (gate) tot *= silu_f(elem(xd[w][2][g][q * CW + cl]));
            }
            if (live && i < nvalid) ylane[(int64_t)(k0 + i) * D] = narrow<Tin>(tot);
        }
        if (more) widen_bc(bcrn, xdn);
    };

    if constexpr (kAhead) load_hb(0);
    issue(xdA, bcrA, 0);
    widen_bc(bcrA, xdA);
    for (int k0 = 0; k0 < len; k0 += 2 * kGroup) {
        group(xdA, xdB, bcrB, k0);
        if (k0 + kGroup < len) group(xdB, xdA, bcrA, k0 + kGroup);
    }
    if (hout != nullptr && t_end == T && live) store_state(hout + ((int64_t)b * D + d) * kStates);
}

// ------------------------------------------------------------------------
// Bidirectional kernel, two states per lane (the shared-operand passes: plain
// and with the step-size / gate fusions), for kN = 4, 8, 16 or 32 states:
// lane = P * channel + state pair (states 2g, 2g + 1), P = kN / 2 lanes per
// channel, CW = 64 / P channels per wave, 4 waves (4 CW channels) per
// workgroup.  A 16-token group's decays and injections then take 64
// registers per lane at any state count, and the kernel runs three waves per
// SIMD, where bidir_wave_kernel's four-state lanes wait on latency at two.
// Per group, staged as in bwd_pair_kernel (the x / dt (/ z) rows of the
// wave's CW channels DMA'd into the wave's LDS slice, the group's B / C rows
// shared by the workgroup, their loads spread over the waves; one group
// ahead, widened in place by the lane that loaded them; one barrier per
// group; at 16 and 32 states with blocks of at most 16 tokens (except the
// two-stream form at L = 4), two groups per barrier with the next two
// groups' rows in flight, so that the loads have two groups' work to land
// in):
//   forward, left to right: a = exp2(dt A'), u = dt x B, hf = a hf + u, the
//     lane's output partial C . hf over its two states; the group's decays
//     and injections stay in registers (64 per lane), so the reverse pass
//     forms neither again;
//   reverse, right to left, reset where a block ends: hr = a hr + u,
//     partial += C . hr;
//   output: the 16 tokens' partials are summed over the channel's P lanes by
//     a reduce-scatter over the lane bits of g, from the top bit down (row
//     rotation by 8 for bit 3, half-row mirror for bit 2, the quad exchanges
//     for bits 1 and 0), after which lane g holds tokens 16 g / P .. of its
//     channel; + Dskip x, times silu(z) with the gate, stored through buffer
//     stores whose out-of-range offsets drop dead channels and tokens past the
//     chunk.
// dt of tokens past the chunk end and of channels past D reads zero (an
// out-of-range DMA offset; after the step-size transform it is set to zero
// again): such tokens decay by 1 and inject nothing.
// L = 0 (long blocks: Lr tokens, a multiple of 16 from 32 to kLongMax; chunks
// are whole blocks): each block's groups are first walked right to left with
// the reverse recurrence alone (groups kb - 1 .. 1, kb = Lr / 16), keeping the
// reverse state entering each group from its right in LDS; then the groups run
// left to right as above, each reverse pass starting from its saved state.
// The walk reads the group's rows a second time and costs about half the
// forward pass's issue slots per element, over (kb - 1) / kb of the tokens.
// Arguments as in bidir_wave_kernel, with states [.., kN] and the block length
// Lr (L = 0 only); separate reverse operands run bidir_wave_kernel<..., 2>
// (16 states) or block_bidir_kernel.
// grid = (ceil(D / (4 CW)), chunks, batch), block = 256.
template <int kN> constexpr int pair_channels() { return 4 * (2 * kWave / kN); }

// Workgroup -> (channel tile, chunk, batch row) for the two-state kernels,
// whose 16-state tile is 32 channels, 64 bytes of each bf16 stream row.  The
// hardware hands workgroups to the 8 XCDs in turn (linear id mod 8), each
// with its own L2, and a 128-byte line spans two tiles: mapped in order, the
// two tiles of a line run on different XCDs and the line is fetched from HBM
// twice.  Within every run of 16 linear ids this pairs tiles 2j and 2j + 1 on
// one XCD, dispatched 8 apart (ids 16q + i and 16q + 8 + i take tiles 16q +
// 2i and 16q + 2i + 1); an incomplete last run keeps the plain order.
struct BlockPos {
    int tile, c, b;
};
// The remapped id differs from the linear one by less than 16, so with at
// least 16 tiles per row it moves the tile by that much and carries into the
// chunk and batch indices at most once (no integer division); narrower grids
// keep the plain order, and so do single-chunk launches (the latency-bound
// block step and commit, whose 16 rows per workgroup gain nothing from the
// shared lines: 3.9 us plain against 4.0-4.1 us paired at 65K b8).
__device__ __forceinline__ BlockPos xcd_paired_block() {
    const int nx = gridDim.x, ny = gridDim.y;
    int t = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
    const int lin = t + nx * (c + ny * b);
    if (nx >= 16 && ny > 1 && (lin | 15) < nx * ny * (int)gridDim.z) {
        t += (((lin & 7) << 1) | ((lin >> 3) & 1)) - (lin & 15);
        if (t >= nx) {
            t -= nx;
            if (++c == ny) { c = 0; ++b; }
        } else if (t < 0) {
            t += nx;
            if (--c < 0) { c = ny - 1; --b; }
        }
    }
    return BlockPos{t, c, b};
}
// The longest block the two-state forward takes (multiples of 16 from 32):
// its right-to-left walk keeps Lr / 16 - 1 reverse states per lane in LDS.
constexpr int kLongMax = 256;
// dynamic LDS of bidir_pair_kernel's long-block mode
inline size_t pair_long_lds(int64_t Lr) { return (size_t)4 * (Lr / kGroup - 1) * kWave * 2 * sizeof(float); }
constexpr int kPairChannels = pair_channels<kStates>();   // 32: the 16-state two-state kernels

// One step of the output reduce-scatter: lanes whose bit kBit of g is set
// keep the upper half of the values, the others the lower half, each adding
// its partner's (the lane that differs in bit kBit; below bit 3 a DPP
// pattern that flips it within the same aligned group).
template <int kBit, int kV>
__device__ __forceinline__ void pair_scatter(const float (&in)[2 * kV], float (&out)[kV], bool hi) {
#pragma unroll
    for (int k = 0; k < kV; ++k) {
        const float keep = hi ? in[k + kV] : in[k];
        const float send = hi ? in[k] : in[k + kV];
        if constexpr (kBit == 3) out[k] = keep + dpp_perm<kDppRor8>(send);
        else if constexpr (kBit == 2) out[k] = keep + dpp_perm<kDppHalfMirror>(send);
        else if constexpr (kBit == 1) out[k] = keep + dpp_perm<kDppXor2>(send);
        else out[k] = keep + dpp_perm<kDppXor1>(send);
    }
}

template <typename Tin, int kN, int L, bool kBlockInit, int kFuse = 0>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(L == 1 ? 2 : 3))) void bidir_pair_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    const float *hin, int64_t hin_bs, int64_t hin_cs,
    Tin *__restrict__ y, float *__restrict__ bounds, float *hout,
    int64_t T, int D, int64_t Tc, const float *__restrict__ h0_blocks, FuseArgs<Tin> fz, int Lr)
{
    static_assert(kFuse == 0 || kFuse == 1, "separate reverse operands run bidir_wave_kernel");
    // L = 0: blocks of Lr tokens (a multiple of 16 from 32 to kLongMax)
    constexpr bool kLong = L == 0;
    static_assert(kLong || kGroup % L == 0, "block length must divide the token group");
    static_assert(kN == 4 || kN == 8 || kN == 16 || kN == 32, "state counts 4, 8, 16, 32");
    constexpr int P = kN / 2;                 // lanes per channel
    constexpr int CW = kWave / P;             // channels per wave
    constexpr int ES = sizeof(Tin);
    constexpr int G = kGroup;                 // 16 tokens per group
    constexpr int NS = kFuse ? 3 : 2;         // row streams: x, dt (, z)
    constexpr int XL = G * CW / kWave;        // x / dt loads per group and stream (P tokens each)
    constexpr int BL = G * kN / kWave;        // B / C loads per group and stream (64 / kN tokens each)
    constexpr int BT = kWave / kN;            // tokens per B / C load
    constexpr int NV = G / P;                 // output tokens per lane
    constexpr int LB = kLong ? G : L;         // block length as seen inside one group
    // double buffers as distinct arrays (the loads in flight into one are told
    // apart from the reads of the other): [wave][stream][token][channel] and
    // [B, C][token][state]
    __shared__ __attribute__((aligned(16))) uint32_t xdA[4][NS][G][CW], xdB[4][NS][G][CW];
    __shared__ __attribute__((aligned(16))) uint32_t bcA[2][G][kN], bcB[2][G][kN];
    // long blocks: the reverse state entering each group of the block from
    // its right, formed by the block's right-to-left state walk (per lane),
    // [wave][Lr / 16 - 1][lane] in dynamic LDS
    extern __shared__ float2 rsv[];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform(threadIdx.x >> 6);
    const int cl = lane / P;                  // channel within the wave
    const int g = lane % P;                   // state pair
    const int s0 = 2 * g;
    const BlockPos pos = xcd_paired_block();
    const int d_w0 = pos.tile * (4 * CW) + w * CW;
    const int d_raw = d_w0 + cl;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = pos.c;
    const int b = pos.b;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);
    const int Lb = kLong ? Lr : L;            // block length
    const int64_t nbl = T / Lb;

    float a2[2], hf[2] = {0.f, 0.f};
    {
        const float2 av = *reinterpret_cast<const float2 *>(A + (int64_t)d * kN + s0);
        a2[0] = av.x * kLog2e; a2[1] = av.y * kLog2e;
        if (hin != nullptr) {
            const float2 hv = *reinterpret_cast<const float2 *>(
                hin + (int64_t)b * hin_bs + (int64_t)c * hin_cs + (int64_t)d * kN + s0);
            hf[0] = hv.x; hf[1] = hv.y;
        }
    }
    const float dsk = Dskip[d];
    auto store_state = [&](float *dst) {
        *reinterpret_cast<float2 *>(dst + s0) = make_float2(hf[0], hf[1]);
    };
    if (bounds != nullptr && c == 0 && live)
        store_state(bounds + ((int64_t)b * (nbl + 1) * D + d) * kN);

    const int64_t first = (int64_t)b * T + t_begin;
    const Rows<Tin> xs(x + first * D, len, D, 0);
    const Rows<Tin> ds(dt + first * D, len, D, 0);
    const Rows<Tin> ys(y + first * D, len, D, 0);
    __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Bm + first * kN)), 0, uniform(len * kN * ES), kRawBufferWord3);
    __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Cm + first * kN)), 0, uniform(len * kN * ES), kRawBufferWord3);
    // DMA lanes: x / dt (/ z) load j covers tokens P j .. P j + P - 1 (lane:
    // token l / CW, channel l % CW); B / C load j (taken by wave j % 4) covers
    // tokens BT j .. (lane: token l / kN, state l % kN)
    const int ld_tok = lane / CW, ld_col = lane % CW;
    const bool ld_live = d_w0 + ld_col < D;
    const int ld_ch = ld_live ? d_w0 + ld_col : D - 1;
    const int bc_tok = lane / kN, bc_col = lane % kN;
    const bool gate = kFuse && fz.z != nullptr;
    const float ld_bias = (kFuse && fz.dt_bias != nullptr) ? fz.dt_bias[ld_ch] : 0.f;
    const Rows<Tin> zs((gate ? fz.z : x) + first * D, len, D, 0);

    auto issue = [&](auto &xd, auto &bc, int k0) {
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int kr = k0 + P * j + ld_tok;
            const int k = kr < len ? kr : len - 1;
            const int zoff = (kr < len && ld_live) ? ld_ch * ES + k * ds.pitch : kOutOfRange;
            load_to_lds<ES>(xs.rsrc, &xd[w][0][P * j][0], ld_ch * ES + k * xs.pitch, 0);
            load_to_lds<ES>(ds.rsrc, &xd[w][1][P * j][0], zoff, 0);
            if constexpr (kFuse) {
                if (gate) load_to_lds<ES>(zs.rsrc, &xd[w][2][P * j][0], zoff, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < BL; j += 4) {
            if (BL % 4 == 0 || j + w < BL) {
                const int kt = k0 + BT * (j + w) + bc_tok;
                const int kb = kt < len ? kt : len - 1;
                load_to_lds<ES>(brs, &bc[0][BT * (j + w)][0], (kb * kN + bc_col) * ES, 0);
                load_to_lds<ES>(crs, &bc[1][BT * (j + w)][0], (kb * kN + bc_col) * ES, 0);
            }
        }
    };
    // after this wave's own loads have landed, widen the dwords this lane
    // loaded to fp32 in place; with the fusions, form the step size (zero
    // again past the chunk end) and silu(z)
    auto widen = [&](auto &xd, auto &bc, int k0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if constexpr (ES == 2) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int j = 0; j < XL; ++j) {
                    if (s == 2 && !gate) continue;
                    uint32_t &v = (&xd[w][s][P * j][0])[lane];
                    v <<= 16;
                }
#pragma unroll
            for (int j = 0; j < BL; j += 4) {
                if (BL % 4 == 0 || j + w < BL) {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        uint32_t &v = (&bc[s][BT * (j + w)][0])[lane];
                        v <<= 16;
                    }
                }
            }
        }
        if constexpr (kFuse) {
#pragma unroll
            for (int j = 0; j < XL; ++j) {
                uint32_t &dv = (&xd[w][1][P * j][0])[lane];
                const float raw = __uint_as_float(dv);
                float dl = raw;
                if (fz.dt_mode == kDtSoftplus) dl = step_size<kDtSoftplus>(raw, ld_bias);
                else if (fz.dt_mode == kDtBias) dl = step_size<kDtBias>(raw, ld_bias);
                dv = __float_as_uint(k0 + P * j + ld_tok < len ? dl : 0.f);
                if (gate) {
                    uint32_t &zv = (&xd[w][2][P * j][0])[lane];
                    zv = __float_as_uint(silu_f(__uint_as_float(zv)));
                }
            }
        }
    };
    auto f32 = [](uint32_t v) { return __uint_as_float(v); };
    auto bcv = [&](auto &bc, int which, int i) {
        const uint2 v = *reinterpret_cast<const uint2 *>(&bc[which][i][s0]);
        return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
    };

    // two-stream form: the block start states of a group, loaded one group
    // ahead with its rows for L >= 4 (at most 4 blocks per group)
    constexpr int NB = kBlockInit ? G / LB : 1;
    constexpr bool kAhead = kBlockInit && (kLong || L >= 4);
    float2 hbn[NB];
    auto load_hb_into = [&](float2 (&dst)[NB], int k0n) {
        if constexpr (kBlockInit) {
            const int nv = (len - k0n < G) ? len - k0n : G;
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int i = q * LB < nv ? q * LB : 0;
                const int64_t blk = (t_begin + k0n + i) / Lb;
                dst[q] = *reinterpret_cast<const float2 *>(
                    h0_blocks + (((int64_t)b * (nbl + 1) + blk) * D + d) * kN + s0);
            }
        }
    };
    auto load_hb = [&](int k0n) { load_hb_into(hbn, k0n); };

    // long blocks: gsb / geb, whether the group starts / ends its block, and
    // hri, the reverse state entering it from the right
    auto group = [&](auto &xd, auto &bc, int k0, const float2 *hb, float2 hri = make_float2(0.f, 0.f),
                     bool gsb = true, bool geb = true) __attribute__((always_inline)) {
        const int nvalid = (len - k0 < G) ? len - k0 : G;   // uniform
        // injections kept per state (at 4 states dt x per token: the
        // registers of the wider x / dt staging leave no room for more)
        constexpr int KU = kN == 4 ? 1 : 2;
        float dA[G][2], us[G][KU], ya[G];
        // forward, left to right
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if constexpr (kBlockInit) {
                if (i % LB == 0 && gsb) { hf[0] = hb[i / LB].x; hf[1] = hb[i / LB].y; }
            }
            const float dl = f32(xd[w][1][i][cl]);
            const float dxv = dl * f32(xd[w][0][i][cl]);
            const float2 bv = bcv(bc, 0, i), cv = bcv(bc, 1, i);
            const float a0 = fast_exp2(dl * a2[0]), a1 = fast_exp2(dl * a2[1]);
            dA[i][0] = a0; dA[i][1] = a1;
            const float u0 = dxv * bv.x, u1 = dxv * bv.y;
            if constexpr (KU == 2) {
                us[i][0] = u0;
                us[i][KU - 1] = u1;
            } else {
                us[i][0] = dxv;
            }
            hf[0] = __builtin_fmaf(a0, hf[0], u0);
            hf[1] = __builtin_fmaf(a1, hf[1], u1);
            ya[i] = __builtin_fmaf(cv.y, hf[1], cv.x * hf[0]);
            if ((i + 1) % LB == 0 && geb && bounds != nullptr && i < nvalid && live) {
                const int64_t kb = (t_begin + k0 + i + 1) / Lb;
                store_state(bounds + (((int64_t)b * (nbl + 1) + kb) * D + d) * kN);
            }
            if ((i & 3) == 3) {
                // 4-token batches: the batch's arithmetic completes before the
                // next batch's LDS reads are issued (register pressure)
                asm volatile("" : "+v"(hf[0]), "+v"(hf[1]), "+v"(ya[i]), "+v"(ya[i - 1]), "+v"(ya[i - 2]),
                             "+v"(ya[i - 3]) :: "memory");
            }
        }
        // reverse, right to left, from zero at every block end (long blocks:
        // from the state entering the group from its right)
        float hr[2] = {hri.x, hri.y};
#pragma unroll
        for (int i = G - 1; i >= 0; --i) {
            if (!kLong && (i + 1) % LB == 0) { hr[0] = hr[1] = 0.f; }
            const float2 cv = bcv(bc, 1, i);
            float u0 = us[i][0], u1 = us[i][KU - 1];
            if constexpr (KU == 1) {
                const float2 bv = bcv(bc, 0, i);
                u0 *= bv.x;
                u1 *= bv.y;
            }
            hr[0] = __builtin_fmaf(dA[i][0], hr[0], u0);
            hr[1] = __builtin_fmaf(dA[i][1], hr[1], u1);
            ya[i] = __builtin_fmaf(cv.y, hr[1], __builtin_fmaf(cv.x, hr[0], ya[i]));
            if ((i & 3) == 0) {
                asm volatile("" : "+v"(hr[0]), "+v"(hr[1]), "+v"(ya[i]), "+v"(ya[i + 1]), "+v"(ya[i + 2]),
                             "+v"(ya[i + 3]) :: "memory");
            }
        }
        // the channel's sum over its P lanes, from the top bit of g down: lane
        // g ends with tokens NV g .. NV g + NV - 1
        float r[NV];
        if constexpr (P == 16) {
            float r8[8], r4[4], r2[2];
            pair_scatter<3, 8>(ya, r8, (g & 8) != 0);
            pair_scatter<2, 4>(r8, r4, (g & 4) != 0);
            pair_scatter<1, 2>(r4, r2, (g & 2) != 0);
            pair_scatter<0, 1>(r2, r, (g & 1) != 0);
        } else if constexpr (P == 8) {
            float r8[8], r4[4];
            pair_scatter<2, 8>(ya, r8, (g & 4) != 0);
            pair_scatter<1, 4>(r8, r4, (g & 2) != 0);
            pair_scatter<0, 2>(r4, r, (g & 1) != 0);
        } else if constexpr (P == 4) {
            float r8[8];
            pair_scatter<1, 8>(ya, r8, (g & 2) != 0);
            pair_scatter<0, 4>(r8, r, (g & 1) != 0);
        } else {
            pair_scatter<0, 8>(ya, r, (g & 1) != 0);
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int t = NV * g + k;
            float tot = __builtin_fmaf(dsk, f32(xd[w][0][t][cl]), r[k]);
            if constexpr (kFuse) {
                if (gate) tot *= f32(xd[w][2][t][cl]);
            }
            const int32_t off = (live && t < nvalid) ? (k0 + t) * ys.pitch + d * ES : kOutOfRange;
            ys.store_at(off, narrow<Tin>(tot));
        }
    };

    // one group: the next group's loads go out first, then this group's
    // passes, then the next group's widening; the barrier keeps every wave's
    // reads of this group's B / C rows ahead of the loads that overwrite them
    auto step = [&](auto &xd, auto &bc, auto &xdn, auto &bcn, int k0) {
        const bool more = k0 + G < len;
        float2 hb[NB];
        if constexpr (kBlockInit && !kAhead) load_hb(k0);
#pragma unroll
        for (int q = 0; q < NB; ++q) hb[q] = hbn[q];
        if (more) {
            if constexpr (kAhead) load_hb(k0 + G);
            issue(xdn, bcn, k0 + G);
        }
        group(xd, bc, k0, hb);
        if (more) widen(xdn, bcn, k0 + G);
        __syncthreads();
    };
    if constexpr (kLong) {
        // Long blocks (chunks are whole blocks): per block of kb groups, a
        // right-to-left state walk over groups kb - 1 .. 1 leaves the reverse
        // state entering each group from its right in rsv; then the groups
        // run left to right as above, each reverse pass starting from its
        // saved state (zero in the block's last group).  Schedule entry s of
        // block s / (2 kb - 1): walk steps first, then the groups in order.
        const int kb = Lr / G;
        const int per = 2 * kb - 1;
        const int nsched = (len / Lr) * per;
        auto sched_k0 = [&](int s) {
            const int r = s % per;
            return (s / per) * Lr + (r < kb - 1 ? kb - 1 - r : r - (kb - 1)) * G;
        };
        float2 hrw = make_float2(0.f, 0.f);   // the walk's state
        // the walk over one group, right to left
        auto walk = [&](auto &xd, auto &bc) {
#pragma unroll
            for (int i = G - 1; i >= 0; --i) {
                const float dl = f32(xd[w][1][i][cl]);
                const float dxv = dl * f32(xd[w][0][i][cl]);
                const float2 bv = bcv(bc, 0, i);
                hrw.x = __builtin_fmaf(fast_exp2(dl * a2[0]), hrw.x, dxv * bv.x);
                hrw.y = __builtin_fmaf(fast_exp2(dl * a2[1]), hrw.y, dxv * bv.y);
                if ((i & 3) == 0) asm volatile("" : "+v"(hrw.x), "+v"(hrw.y) :: "memory");
            }
        };
        auto lstep = [&](auto &xd, auto &bc, auto &xdn, auto &bcn, int s) {
            const bool more = s + 1 < nsched;
            const int k0 = sched_k0(s), r = s % per;
            float2 hb[NB];
#pragma unroll
            for (int q = 0; q < NB; ++q) hb[q] = hbn[q];
            if (more) {
                if constexpr (kAhead) load_hb(sched_k0(s + 1));
                issue(xdn, bcn, sched_k0(s + 1));
            }
            if (r < kb - 1) {
                const int j = kb - 1 - r;             // walk over group j
                if (j == kb - 1) hrw = make_float2(0.f, 0.f);
                walk(xd, bc);
                rsv[(w * (kb - 1) + j - 1) * kWave + lane] = hrw;
            } else {
                const int j = r - (kb - 1);
                group(xd, bc, k0, hb, j == kb - 1 ? make_float2(0.f, 0.f) : rsv[(w * (kb - 1) + j) * kWave + lane],
                      j == 0, j == kb - 1);
            }
            if (more) widen(xdn, bcn, sched_k0(s + 1));
            __syncthreads();
        };
        if (nsched > 0) {
            if constexpr (kAhead) load_hb(sched_k0(0));
            issue(xdA, bcA, sched_k0(0));
            widen(xdA, bcA, sched_k0(0));
            __syncthreads();
        }
        for (int s = 0; s < nsched; s += 2) {
            lstep(xdA, bcA, xdB, bcB, s);
            if (s + 1 < nsched) lstep(xdB, bcB, xdA, bcA, s + 1);
        }
    } else if constexpr (kN >= 16 && !(kBlockInit && L == 4)) {
        // two groups per barrier, the next two groups' rows loading meanwhile
        // (four row buffers; not for the two-stream form at L = 4, whose
        // second group's four block start states would spill)
        __shared__ __attribute__((aligned(16))) uint32_t xdC[4][NS][G][CW], xdD[4][NS][G][CW];
        __shared__ __attribute__((aligned(16))) uint32_t bcC[2][G][kN], bcD[2][G][kN];
        float2 hbn2[NB];
        auto macro = [&](auto &x0, auto &b0, auto &x1, auto &b1, auto &n0, auto &nb0, auto &n1, auto &nb1,
                         int k0) {
            const bool has1 = k0 + G < len;
            const bool more0 = k0 + 2 * G < len, more1 = k0 + 3 * G < len;
            float2 hA[NB], hB[NB];
            if constexpr (kBlockInit && !kAhead) load_hb_into(hA, k0);
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                if constexpr (kAhead) hA[q] = hbn[q];
                hB[q] = hbn2[q];
            }
            if (more0) {
                if constexpr (kAhead) load_hb_into(hbn, k0 + 2 * G);
                issue(n0, nb0, k0 + 2 * G);
            }
            if (more1) {
                if constexpr (kAhead) load_hb_into(hbn2, k0 + 3 * G);
                issue(n1, nb1, k0 + 3 * G);
            }
            group(x0, b0, k0, hA);
            if (has1) {
                if constexpr (kBlockInit && !kAhead) load_hb_into(hB, k0 + G);
                group(x1, b1, k0 + G, hB);
            }
            if (more0) widen(n0, nb0, k0 + 2 * G);
            if (more1) widen(n1, nb1, k0 + 3 * G);
            __syncthreads();
        };
        if constexpr (kAhead) {
            load_hb_into(hbn, 0);
            if (G < len) load_hb_into(hbn2, G);
        }
        issue(xdA, bcA, 0);
        if (G < len) issue(xdB, bcB, G);
        widen(xdA, bcA, 0);
        if (G < len) widen(xdB, bcB, G);
        __syncthreads();
        for (int k0 = 0; k0 < len; k0 += 4 * G) {
            macro(xdA, bcA, xdB, bcB, xdC, bcC, xdD, bcD, k0);
            if (k0 + 2 * G < len) macro(xdC, bcC, xdD, bcD, xdA, bcA, xdB, bcB, k0 + 2 * G);
        }
    } else {
        if constexpr (kAhead) load_hb(0);
        issue(xdA, bcA, 0);
        widen(xdA, bcA, 0);
        __syncthreads();
        for (int k0 = 0; k0 < len; k0 += 2 * G) {
            step(xdA, bcA, xdB, bcB, k0);
            if (k0 + G < len) step(xdB, bcB, xdA, bcA, k0 + G);
        }
    }
    if (hout != nullptr && t_end == T && live) store_state(hout + ((int64_t)b * D + d) * kN);
}

// ------------------------------------------------------------------------
// One block from the cache, for the latency-bound single-block calls
// (block_step, commit; L <= 16, shared operands): one lane per (channel,
// state), 64 / kN channels per wave, four independent waves per workgroup, so a block
// spreads over kN times the waves of a one-lane-per-channel layout and each
// lane runs one state's recurrence.  Every load of the block is issued up
// front.  The per-channel rows (x, dt, z) are loaded once per element by the
// channel's lanes in turn, the step size and silu(z) formed there, and shared
// through LDS; each lane loads its state's B and C.  The lane runs the forward
// recurrence from the cache and, when y is wanted, the in-block reverse; the
// per-token outputs are summed over the channel's kN lanes through LDS, plus
// Dskip x, times silu(z).  kCommit writes the forward state after the block
// back to h_cache (each lane reads, then writes, its own entry).
// grid = (ceil(D / (256 / kN)), batch), block = 256.
template <typename Tin, int kN, bool kCommit, bool kFuse>
__global__ __launch_bounds__(4 * kWave) void block_lane_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    float *h_cache, Tin *__restrict__ y, int D, int L, FuseArgs<Tin> fz)
{
    constexpr int CW = kWave / kN;            // channels per wave
    constexpr int G = kGroup;                 // L <= 16
    __shared__ float part_s[4][G][kWave];     // per-lane output partials
    __shared__ float xs_s[4][G][CW], dls_s[4][G][CW], gz_s[4][G][CW];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform(threadIdx.x >> 6);
    auto &part = part_s[w];
    auto &xs = xs_s[w];
    auto &dls = dls_s[w];
    auto &gz = gz_s[w];
    const int cl = lane / kN, n = lane % kN;
    const int d0 = (blockIdx.x * 4 + w) * CW;
    const int d_raw = d0 + cl;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int b = blockIdx.y;
    const int64_t row0 = (int64_t)b * L;
    const bool with_y = y != nullptr;
    const bool gate = kFuse && with_y && fz.z != nullptr;
    // output lanes: channel lane % CW (CW divides 64)
    const int c_out = lane % CW;
    const bool out_live = d0 + c_out < D;
    const float dsk_out = with_y ? Dskip[out_live ? d0 + c_out : D - 1] : 0.f;   // Dskip may be null without y

    const int64_t hidx = ((int64_t)b * D + d) * kN + n;
    float h = h_cache[hidx];
    const float a2 = A[(int64_t)d * kN + n] * kLog2e;
    const float bias = (kFuse && fz.dt_bias != nullptr) ? fz.dt_bias[d] : 0.f;

    // every load first (one memory round trip): the channel's rows, lane
    // (cl, n) taking tokens n, n + kN, ..., and the lane's B and C
    // (rows past L re-read row L - 1: unconditional loads go out back to back)
    constexpr int NT = (G + kN - 1) / kN;
    Tin rx[NT], rd[NT], rz[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = j * kN + n;
        const int64_t r = (row0 + (t < L ? t : L - 1)) * D + d;
        rx[j] = x[r];
        rd[j] = dt[r];
        rz[j] = gate ? fz.z[r] : rx[j];
    }
    const Tin *crow = with_y ? Cm : Bm;       // C may be null without y
    Tin rb[G], rc[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int64_t r = (row0 + (t < L ? t : L - 1)) * kN + n;
        rb[t] = Bm[r];
        rc[t] = crow[r];
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int t = j * kN + n;
        if (t < L) {
            float dv = widen(rd[j]);
            if constexpr (kFuse) {
                if (fz.dt_mode == kDtSoftplus) dv = step_size<kDtSoftplus>(dv, bias);
                else if (fz.dt_mode == kDtBias) dv = step_size<kDtBias>(dv, bias);
            }
            xs[t][cl] = widen(rx[j]);
            dls[t][cl] = dv;
            if (gate) gz[t][cl] = silu_f(widen(rz[j]));
        }
    }
    float bv[G], cv[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
        if (t < L) {
            bv[t] = widen(rb[t]);
            cv[t] = with_y ? widen(rc[t]) : 0.f;
        }
    }
    asm volatile("" ::: "memory");
    float a[G], u[G], yp[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
        if (t < L) {
            const float dv = dls[t][cl];
            a[t] = fast_exp2(dv * a2);
            u[t] = dv * xs[t][cl] * bv[t];
            h = __builtin_fmaf(a[t], h, u[t]);
            yp[t] = cv[t] * h;
        }
    }
    if (kCommit && live) h_cache[hidx] = h;
    if (!with_y) return;
    float hr = 0.f;
#pragma unroll
    for (int t = G - 1; t >= 0; --t) {
        if (t < L) {
            hr = __builtin_fmaf(a[t], hr, u[t]);
            part[t][lane] = __builtin_fmaf(cv[t], hr, yp[t]);
        }
    }
    asm volatile("" ::: "memory");
    for (int o = lane; o < L * CW; o += kWave) {
        const int t = o / CW;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < kN; k += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(&part[t][c_out * kN + k]);
            s += (v.x + v.y) + (v.z + v.w);
        }
        float tot = __builtin_fmaf(dsk_out, xs[t][c_out], s);
        if (gate) tot *= gz[t][c_out];
        if (out_live) y[(row0 + t) * D + d0 + c_out] = narrow<Tin>(tot);
    }
}

// ------------------------------------------------------------------------
// Directional output sweep for the full-sequence baseline: one lane per
// channel, 16 states.  Forward (kRev = false): from the chunk's incoming
// forward state, writes yf_t = sum_n C_t h_t to an fp32 buffer.  Reverse:
// from the state entering the chunk from its right end, walks the chunk
// backwards and writes y_t = yf_t + sum_n C_t h_t + Dskip x_t (times silu(z_t)
// when the gate z is given).  kDt / dt_bias form dt as in chunk_state_kernel.
// grid = (ceil(D/64), chunks, batch), block = 64.
template <typename Tin, bool kRev, int kDt = kDtPlain, int kN = kStates>
__global__ __launch_bounds__(kWave) void sweep_output_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    const float *__restrict__ hin, float *__restrict__ yf, Tin *__restrict__ y,
    int64_t T, int D, int64_t Tc, int n_chunks, const float *__restrict__ dt_bias,
    const Tin *__restrict__ z)
{
    constexpr int U = 6;                      // tokens per pipeline stage
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);

    float a2[kN], h[kN];
    load_row<kN>(A + (int64_t)d * kN, a2);
#pragma unroll
    for (int n = 0; n < kN; ++n) a2[n] *= kLog2e;
    load_row<kN>(hin + (((int64_t)b * n_chunks + c) * D + d) * kN, h);
    const float dsk = Dskip[d];
    const float bias = (kDt != kDtPlain && dt_bias != nullptr) ? dt_bias[d] : 0.f;
    const bool gate = kRev && z != nullptr;
    const int64_t first = (int64_t)b * T + t_begin;
    const Rows<Tin> xs(x + first * D, len, D, d);
    const Rows<Tin> ds(dt + first * D, len, D, d);
    const Rows<Tin> ys(y + first * D, len, D, d);
    const Rows<Tin> zs((gate ? z : x) + first * D, len, D, d);
    const Rows<float> fs(yf + first * D, len, D, d);
    const Tin *bs = Bm + first * kN;
    const Tin *cs = Cm + first * kN;
    auto pos = [&](int k) -> int { return kRev ? len - 1 - k : k; };

    auto consume = [&](const Tin *xr, const Tin *dr, const float *yr, int k0, int count) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (i < count) {
                const int p = pos(k0 + i);
                const float xv = widen(xr[i]);
                const float dl = step_size<kDt>(widen(dr[i]), bias);
                const float dx = dl * xv;
                const Tin *brow = bs + (int64_t)p * kN;
                const Tin *crow = cs + (int64_t)p * kN;
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < kN / 2; ++q) {
                    float b0, b1, c0, c1;
                    load_pair(brow, q, b0, b1);
                    load_pair(crow, q, c0, c1);
                    h[2 * q] = __builtin_fmaf(fast_exp2(dl * a2[2 * q]), h[2 * q], dx * b0);
                    h[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2[2 * q + 1]), h[2 * q + 1], dx * b1);
                    acc = __builtin_fmaf(c0, h[2 * q], acc);
                    acc = __builtin_fmaf(c1, h[2 * q + 1], acc);
                }
                if (!kRev) {
                    if (live) fs.store(p, acc);
                } else {
                    float tot = yr[i] + acc + dsk * xv;
                    if (gate) tot *= silu_f(widen(zs.load(p)));
                    if (live) ys.store(p, narrow<Tin>(tot));
                }
            }
        }
    };

    const int n_full = len / U;
    const int rem = len - n_full * U;
    Tin xr[U], dr[U];
    float yr[U];
    auto load_stage = [&](int k0, int count, Tin *xo, Tin *dout, float *yo) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int p = pos(k0 + (i < count ? i : count - 1));
            xo[i] = xs.load(p);
            dout[i] = ds.load(p);
            if (kRev) yo[i] = fs.load(p);
        }
    };
    if (n_full > 0) load_stage(0, U, xr, dr, yr);
    for (int g = 0; g < n_full; ++g) {
        Tin xn[U], dn[U];
        float yn[U];
        if (g + 1 < n_full) load_stage((g + 1) * U, U, xn, dn, yn);
        consume(xr, dr, yr, g * U, U);
#pragma unroll
        for (int i = 0; i < U; ++i) { xr[i] = xn[i]; dr[i] = dn[i]; yr[i] = yn[i]; }
    }
    if (rem > 0) {
        load_stage(n_full * U, rem, xr, dr, yr);
        consume(xr, dr, yr, n_full * U, rem);
    }
}

// ------------------------------------------------------------------------
// Bidirectional pass for any block length up to kMaxLdsBlock (T % L == 0)
// and any even state count kN: one lane per channel, the kN states of the
// forward and of the reverse scan in registers, one wave per workgroup.
// Every L-block of the chunk is walked twice:
//   * left to right with the forward state (carried across the chunk's
//     blocks; kBlockInit: restarted from h0_blocks at every block), the
//     per-token forward output yf_t = sum_n C_t hf_t going to LDS;
//   * right to left with the reverse state from zero, adding yr_t + Dskip x_t
//     to yf_t and storing y (times silu(z_t) when the gate is given).
// The second walk forms its decays again: a block may be longer than the
// registers can hold, and the rows it re-reads are the block's own, still in
// L2.  LDS holds one fp32 value per token and channel of a block (of a
// segment, for blocks longer than seg): 256 * min(L, seg) bytes of dynamic
// shared memory.
// Chunks are whole numbers of blocks (Tc % L == 0).  hin, bounds, hout and the
// fusions as in bidir_wave_kernel (states are [.., kN] instead of [.., 16]);
// with separate reverse operands the reverse walk reads dt_r (with dt_bias_r,
// same transform), B_r, C_r and A_r.
// grid = (ceil(D/64), chunks, batch), block = 64.
constexpr int kMaxLdsBlock = 256;
// Blocks longer than seg tokens are finished in segments of seg tokens (the
// LDS then holds one segment's outputs, 256 seg bytes: 8 KB at seg = 32
// rather than 64 KB for a whole 256-token block, which let only two
// workgroups share a CU): the reverse state entering a
// segment from the right is formed again by a state-only reverse walk from
// the block's end (an exp and two FMAs per state and token, no C, no output),
// which adds (L / seg - 1) / 2 state-only walks of the block.

template <typename Tin, int kN, bool kBlockInit, int kDt>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(kN <= 16 ? 4 : 1))) void block_bidir_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    const float *hin, int64_t hin_bs, int64_t hin_cs, Tin *__restrict__ y,
    float *__restrict__ bounds, float *hout, int64_t T, int D, int L, int64_t Tc,
    const float *__restrict__ h0_blocks, FuseArgs<Tin> fz, int seg)
{
    static_assert(kN % 2 == 0, "B and C rows are read in pairs");
    extern __shared__ float yf_lds[];             // [min(L, seg)][64]
    constexpr int U = 4;                          // tokens per pipeline stage
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);      // a multiple of L
    const int64_t nbl = T / L;
    const bool gate = fz.z != nullptr;
    const bool sep = fz.dt_r != nullptr;

    float a2[kN], a2r[kN], h[kN], hr[kN];
    load_row<kN>(A + (int64_t)d * kN, a2);
    load_row<kN>((sep ? fz.A_r : A) + (int64_t)d * kN, a2r);
#pragma unroll
    for (int n = 0; n < kN; ++n) { a2[n] *= kLog2e; a2r[n] *= kLog2e; }
    if (!kBlockInit && hin != nullptr) {
        load_row<kN>(hin + (int64_t)b * hin_bs + (int64_t)c * hin_cs + (int64_t)d * kN, h);
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.f;
    }
    const float dsk = Dskip[d];
    const float bias = (kDt != kDtPlain && fz.dt_bias != nullptr) ? fz.dt_bias[d] : 0.f;
    const float bias_r = sep ? ((kDt != kDtPlain && fz.dt_bias_r != nullptr) ? fz.dt_bias_r[d] : 0.f) : bias;

    const int64_t first = (int64_t)b * T + t_begin;
    const Rows<Tin> xs(x + first * D, len, D, d);
    const Rows<Tin> ds(dt + first * D, len, D, d);
    const Rows<Tin> rds((sep ? fz.dt_r : dt) + first * D, len, D, d);
    const Rows<Tin> zs((gate ? fz.z : x) + first * D, len, D, d);
    const Rows<Tin> ys(y + first * D, len, D, d);
    const Tin *bs = Bm + first * kN, *cs = Cm + first * kN;
    const Tin *rbs = (sep ? fz.B_r : Bm) + first * kN, *rcs = (sep ? fz.C_r : Cm) + first * kN;

    // one token of the forward walk (row p of the chunk, row r of the block)
    auto fwd_tok = [&](int p, int r, float xv, float dl) {
        const float dx = dl * xv;
        const Tin *brow = bs + (int64_t)p * kN, *crow = cs + (int64_t)p * kN;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int q = 0; q < kN / 2; ++q) {
            float b0, b1, c0, c1;
            load_pair(brow, q, b0, b1);
            load_pair(crow, q, c0, c1);
            h[2 * q] = __builtin_fmaf(fast_exp2(dl * a2[2 * q]), h[2 * q], dx * b0);
            h[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2[2 * q + 1]), h[2 * q + 1], dx * b1);
            acc0 = __builtin_fmaf(c0, h[2 * q], acc0);
            acc1 = __builtin_fmaf(c1, h[2 * q + 1], acc1);
        }
        yf_lds[r * kWave + lane] = acc0 + acc1;
    };
    // one token of the reverse walk that only carries the state (a segment
    // right of the one being finished)
    auto rev_state_tok = [&](int p, float xv, float dl) {
        const float dx = dl * xv;
        const Tin *brow = rbs + (int64_t)p * kN;
#pragma unroll
        for (int q = 0; q < kN / 2; ++q) {
            float b0, b1;
            load_pair(brow, q, b0, b1);
            hr[2 * q] = __builtin_fmaf(fast_exp2(dl * a2r[2 * q]), hr[2 * q], dx * b0);
            hr[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2r[2 * q + 1]), hr[2 * q + 1], dx * b1);
        }
    };
    // one token of the reverse walk
    auto rev_tok = [&](int p, int r, float xv, float dl, float zv) {
        const float dx = dl * xv;
        const Tin *brow = rbs + (int64_t)p * kN, *crow = rcs + (int64_t)p * kN;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int q = 0; q < kN / 2; ++q) {
            float b0, b1, c0, c1;
            load_pair(brow, q, b0, b1);
            load_pair(crow, q, c0, c1);
            hr[2 * q] = __builtin_fmaf(fast_exp2(dl * a2r[2 * q]), hr[2 * q], dx * b0);
            hr[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2r[2 * q + 1]), hr[2 * q + 1], dx * b1);
            acc0 = __builtin_fmaf(c0, hr[2 * q], acc0);
            acc1 = __builtin_fmaf(c1, hr[2 * q + 1], acc1);
        }
        float tot = __builtin_fmaf(dsk, xv, yf_lds[r * kWave + lane] + (acc0 + acc1));
        if (gate) tot *= silu_f(zv);
        if (live) ys.store(p, narrow<Tin>(tot));
    };
    // walk rows k0 .. k0 + n - 1 of the chunk, forward (mode 0) or reverse
    // (mode 1: with the output, LDS row p - r0; mode 2: the state alone); the
    // rows of the next U tokens are loaded before the arithmetic of the
    // current U
    auto walk = [&](auto mode_tag, int k0, int n, int r0) {
        constexpr int M = decltype(mode_tag)::value;
        constexpr bool R = M != 0;
        const Rows<Tin> &dsrc = R ? rds : ds;
        const int nst = (n + U - 1) / U;
        auto pos = [&](int k) { return R ? k0 + n - 1 - k : k0 + k; };
        auto stage = [&](int s, Tin *xo, Tin *dout, Tin *zo) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int k = (s * U + i < n) ? s * U + i : n - 1;
                const int p = pos(k);
                xo[i] = xs.load(p);
                dout[i] = dsrc.load(p);
                zo[i] = (M == 1 && gate) ? zs.load(p) : xo[i];
            }
        };
        Tin xr[U], dr[U], zr[U];
        stage(0, xr, dr, zr);
        for (int s = 0; s < nst; ++s) {
            Tin xn[U], dn[U], zn[U];
            if (s + 1 < nst) stage(s + 1, xn, dn, zn);
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int k = s * U + i;
                if (k < n) {
                    const int p = pos(k);
                    if constexpr (M == 2)
                        rev_state_tok(p, widen(xr[i]), step_size<kDt>(widen(dr[i]), bias_r));
                    else if constexpr (M == 1)
                        rev_tok(p, p - r0, widen(xr[i]), step_size<kDt>(widen(dr[i]), bias_r), widen(zr[i]));
                    else
                        fwd_tok(p, p - r0, widen(xr[i]), step_size<kDt>(widen(dr[i]), bias));
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i) { xr[i] = xn[i]; dr[i] = dn[i]; zr[i] = zn[i]; }
        }
    };

    for (int k0 = 0; k0 < len; k0 += L) {
        const int64_t blk = (t_begin + k0) / L;
        if constexpr (kBlockInit) {
            load_row<kN>(h0_blocks + (((int64_t)b * (nbl + 1) + blk) * D + d) * kN, h);
        } else if (bounds != nullptr && live) {
            store_row<kN>(bounds + (((int64_t)b * (nbl + 1) + blk) * D + d) * kN, h);
        }
        // segments of at most seg tokens, left to right: the forward walk
        // stages the segment's outputs; the reverse state entering it from the
        // right is formed again from the block's end (state only), then the
        // reverse walk over the segment finishes y
        for (int s0 = 0; s0 < L; s0 += seg) {
            const int sl = (L - s0 < seg) ? L - s0 : seg;
            walk(std::integral_constant<int, 0>{}, k0 + s0, sl, k0 + s0);
#pragma unroll
            for (int n = 0; n < kN; ++n) hr[n] = 0.f;
            if (s0 + sl < L) walk(std::integral_constant<int, 2>{}, k0 + s0 + sl, L - s0 - sl, 0);
            walk(std::integral_constant<int, 1>{}, k0 + s0, sl, k0 + s0);
        }
    }
    if (t_end == T && live) {
        if (!kBlockInit && bounds != nullptr)
            store_row<kN>(bounds + (((int64_t)b * (nbl + 1) + nbl) * D + d) * kN, h);
        if (hout != nullptr) store_row<kN>(hout + ((int64_t)b * D + d) * kN, h);
    }
}

// One block per batch row (the block step, the commit with outputs), block
// lengths above 16, up to 16 states: block_bidir_kernel would walk the whole
// block in one wave per 64 channels (batch * D / 64 waves in all).  Here the
// block's tokens are split over the NW waves of the workgroup (segments of
// ceil(L / NW) <= kSplitSeg tokens), all on the same 64 channels (lane =
// channel):
//   1. each wave walks its segment forward from a zero state, state only, and
//      leaves the local state and the sum of its step sizes in LDS (the decay
//      over a segment is exp2(A' sum dt)); each wave combines hin with the
//      segments left of it into the state entering its segment;
//   2. the same in reverse: local states from zero at the segment's right
//      end, combined over the segments right of it (zero at the block's end);
//   3. each wave walks its segment forward, keeping sum_n C hf per token in
//      registers, then in reverse, adding sum_n C hr + Dskip x (times
//      silu(z)) and storing y; the last wave stores the final forward state
//      in hout.
// hout may alias hin (commit): every wave reads hin before the barriers that
// precede the store.  Fusions and separate reverse operands as in
// block_bidir_kernel.  LDS: NW (kN + 1) 256 bytes (one direction at a time).
// grid = (ceil(D/64), 1, batch), block = 64 NW (NW <= 8).
constexpr int kSplitSeg = 32;

template <typename Tin, int kN, int kDt>
__global__ __launch_bounds__(8 * kWave) void block_split_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    const float *hin, int64_t hin_bs, Tin *__restrict__ y, float *hout, int D, int L,
    FuseArgs<Tin> fz)
{
    static_assert(kN % 2 == 0 && kN <= 16, "B and C rows are read in pairs; registers");
    extern __shared__ float lds_split[];          // [NW][kN + 1][64]
    const int NW = blockDim.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int b = blockIdx.z;
    const int SL = (L + NW - 1) / NW;
    const int s0 = (w * SL < L) ? w * SL : L;
    const int ns = ((s0 + SL < L) ? s0 + SL : L) - s0;       // tokens of this segment (uniform)
    auto slot = [&](int k, int n) -> float & { return lds_split[((size_t)k * (kN + 1) + n) * kWave + lane]; };

    const bool gate = fz.z != nullptr;
    const bool sep = fz.dt_r != nullptr;
    float a2[kN], a2r[kN], h[kN], hr[kN];
    load_row<kN>(A + (int64_t)d * kN, a2);
    load_row<kN>((sep ? fz.A_r : A) + (int64_t)d * kN, a2r);
#pragma unroll
    for (int n = 0; n < kN; ++n) { a2[n] *= kLog2e; a2r[n] *= kLog2e; }
    const float dsk = Dskip[d];
    const float bias = (kDt != kDtPlain && fz.dt_bias != nullptr) ? fz.dt_bias[d] : 0.f;
    const float bias_r = sep ? ((kDt != kDtPlain && fz.dt_bias_r != nullptr) ? fz.dt_bias_r[d] : 0.f) : bias;
    const int64_t first = (int64_t)b * L;
    const Rows<Tin> xs(x + first * D, L, D, d);
    const Rows<Tin> ds(dt + first * D, L, D, d);
    const Rows<Tin> rds((sep ? fz.dt_r : dt) + first * D, L, D, d);
    const Rows<Tin> zs((gate ? fz.z : x) + first * D, L, D, d);
    const Rows<Tin> ys(y + first * D, L, D, d);
    const Tin *bs = Bm + first * kN, *cs = Cm + first * kN;
    const Tin *rbs = (sep ? fz.B_r : Bm) + first * kN, *rcs = (sep ? fz.C_r : Cm) + first * kN;

    // one state-only token: st <- exp2(dl a) st + dl x B
    auto state_tok = [&](float *st, const float *aa, const Tin *brow, float dl, float xv) {
        const float dx = dl * xv;
#pragma unroll
        for (int q = 0; q < kN / 2; ++q) {
            float b0, b1;
            load_pair(brow, q, b0, b1);
            st[2 * q] = __builtin_fmaf(fast_exp2(dl * aa[2 * q]), st[2 * q], dx * b0);
            st[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * aa[2 * q + 1]), st[2 * q + 1], dx * b1);
        }
    };

    // 1. forward: local state of the segment, then the state entering it
    {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.f;
        float S = 0.f;
        for (int i = 0; i < ns; ++i) {
            const int p = s0 + i;
            const float dl = step_size<kDt>(widen(ds.load(p)), bias);
            S += dl;
            state_tok(h, a2, bs + (int64_t)p * kN, dl, widen(xs.load(p)));
        }
#pragma unroll
        for (int n = 0; n < kN; ++n) slot(w, n) = h[n];
        slot(w, kN) = S;
    }
    __syncthreads();
    if (hin != nullptr) {
        load_row<kN>(hin + (int64_t)b * hin_bs + (int64_t)d * kN, h);
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.f;
    }
    for (int k = 0; k < w; ++k) {
        const float S = slot(k, kN);
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = __builtin_fmaf(fast_exp2(S * a2[n]), h[n], slot(k, n));
    }
    __syncthreads();          // the slots are reused; every read of hin precedes the store to hout
    // 2. reverse: local state of the segment, then the state entering it from the right
    {
#pragma unroll
        for (int n = 0; n < kN; ++n) hr[n] = 0.f;
        float S = 0.f;
        for (int i = ns - 1; i >= 0; --i) {
            const int p = s0 + i;
            const float dl = step_size<kDt>(widen(rds.load(p)), bias_r);
            S += dl;
            state_tok(hr, a2r, rbs + (int64_t)p * kN, dl, widen(xs.load(p)));
        }
#pragma unroll
        for (int n = 0; n < kN; ++n) slot(w, n) = hr[n];
        slot(w, kN) = S;
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kN; ++n) hr[n] = 0.f;
    for (int k = NW - 1; k > w; --k) {
        const float S = slot(k, kN);
#pragma unroll
        for (int n = 0; n < kN; ++n) hr[n] = __builtin_fmaf(fast_exp2(S * a2r[n]), hr[n], slot(k, n));
    }
    // 3. the outputs of the segment
    float yf[kSplitSeg];
#pragma unroll
    for (int i = 0; i < kSplitSeg; ++i) {
        if (i < ns) {
            const int p = s0 + i;
            const float dl = step_size<kDt>(widen(ds.load(p)), bias);
            const float dx = dl * widen(xs.load(p));
            const Tin *brow = bs + (int64_t)p * kN, *crow = cs + (int64_t)p * kN;
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int q = 0; q < kN / 2; ++q) {
                float b0, b1, c0, c1;
                load_pair(brow, q, b0, b1);
                load_pair(crow, q, c0, c1);
                h[2 * q] = __builtin_fmaf(fast_exp2(dl * a2[2 * q]), h[2 * q], dx * b0);
                h[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2[2 * q + 1]), h[2 * q + 1], dx * b1);
                acc0 = __builtin_fmaf(c0, h[2 * q], acc0);
                acc1 = __builtin_fmaf(c1, h[2 * q + 1], acc1);
            }
            yf[i] = acc0 + acc1;
        }
    }
    if (w == NW - 1 && hout != nullptr && live) store_row<kN>(hout + ((int64_t)b * D + d) * kN, h);
#pragma unroll
    for (int i = kSplitSeg - 1; i >= 0; --i) {
        if (i < ns) {
            const int p = s0 + i;
            const float xv = widen(xs.load(p));
            const float dl = step_size<kDt>(widen(rds.load(p)), bias_r);
            const float dx = dl * xv;
            const Tin *brow = rbs + (int64_t)p * kN, *crow = rcs + (int64_t)p * kN;
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int q = 0; q < kN / 2; ++q) {
                float b0, b1, c0, c1;
                load_pair(brow, q, b0, b1);
                load_pair(crow, q, c0, c1);
                hr[2 * q] = __builtin_fmaf(fast_exp2(dl * a2r[2 * q]), hr[2 * q], dx * b0);
                hr[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2r[2 * q + 1]), hr[2 * q + 1], dx * b1);
                acc0 = __builtin_fmaf(c0, hr[2 * q], acc0);
                acc1 = __builtin_fmaf(c1, hr[2 * q + 1], acc1);
            }
            float tot = __builtin_fmaf(dsk, xv, yf[i] + (acc0 + acc1));
            if (gate) tot *= silu_f(widen(zs.load(p)));
            if (live) ys.store(p, narrow<Tin>(tot));
        }
    }
}

// dst[i] = src[i], or 0 when src is null.  A kernel rather than a memset or
// memcpy node so that callers may capture the entry points in a HIP graph.
static __global__ __attribute__((unused)) __launch_bounds__(256) void copy_or_zero_kernel(const float *src, float *dst, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src != nullptr ? src[i] : 0.f;
}

}  // namespace bdssm_dev
