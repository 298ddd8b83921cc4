// bdssm_kernels.hpp -- gfx950 (CDNA4, wave64) kernels of the block-restricted
// bidirectional selective scan.  Device code only; the launch policy and the
// C ABI are in bdssm.hip.
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
//   its exact incoming state.  Chunks are multiples of 16 tokens, so an
//   L-block (L | 16) never straddles two chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdssm_dev {

constexpr int kStates = 16;      // d_state handled by this build
constexpr int kWave = 64;        // gfx950 wavefront
constexpr int kGroup = 16;       // tokens per register-resident group in the bidirectional kernel
constexpr int kWavesBidir = 4;   // waves per workgroup of the bidirectional kernel (4 states each)
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- element io

__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);   // bf16 -> fp32 is exact
}

template <typename Tin> __device__ __forceinline__ Tin narrow(float v);
template <> __device__ __forceinline__ float narrow<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t narrow<uint16_t>(float v) {
    __bf16 h = static_cast<__bf16>(v);                          // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

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

// ------------------------------------------------------------------------
// Chunk-local directional scan, one lane per channel, all 16 states in
// registers.  Used for
//   * aggregates (h0 == nullptr): the state reached from zero over the chunk
//     and S = sum of dt over the chunk, so the chunk acts on an incoming
//     state h as  h -> exp2(A' S) h + h_local;
//   * kDirect: a forward pass over one chunk from h0 (commit without output,
//     prefill of a short context), writing the final state (a separate
//     instantiation so profiles tell the two uses apart).
// Tokens stream through a 6-deep register pipeline: the loads of the next 6
// tokens are issued before the arithmetic of the current 6 (6 keeps the bf16
// kernel at <= 64 VGPRs, i.e. 8 waves per SIMD).
// kRev scans the chunk from its last token to its first (the reverse
// direction of the full-sequence baseline).
// grid = (ceil(D/64), chunks launched, batch), block = 64.
// hout / sout are indexed by chunk id c = c_first + blockIdx.y over n_chunks.
template <typename Tin, bool kRev, bool kDirect>
__global__ __launch_bounds__(kWave) void chunk_state_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const float *__restrict__ A, const float *h0, float *hout, float *__restrict__ sout,
    int64_t T, int D, int64_t Tc, int n_chunks, int c_first)
{
    constexpr int U = 6;                      // tokens per pipeline stage
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = c_first + blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int64_t len = t_end - t_begin;      // >= 1

    float a2[kStates], h[kStates];
    {
        const float4 *ar = reinterpret_cast<const float4 *>(A + (int64_t)d * kStates);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 v = ar[q];
            a2[4 * q + 0] = v.x * kLog2e; a2[4 * q + 1] = v.y * kLog2e;
            a2[4 * q + 2] = v.z * kLog2e; a2[4 * q + 3] = v.w * kLog2e;
        }
    }
    if (kDirect && h0 != nullptr) {
        const float4 *hr = reinterpret_cast<const float4 *>(h0 + ((int64_t)b * D + d) * kStates);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 v = hr[q];
            h[4 * q + 0] = v.x; h[4 * q + 1] = v.y; h[4 * q + 2] = v.z; h[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int n = 0; n < kStates; ++n) h[n] = 0.f;
    }
    float S = 0.f;
    // Step k of the sweep is token t_first + k * step.  Row pointers are
    // wave-uniform (scalar registers); lanes index them by channel, so the
    // loads need no per-lane address arithmetic.
    const int64_t step = kRev ? -(int64_t)D : (int64_t)D;
    const int64_t t_first = kRev ? t_end - 1 : t_begin;
    const Tin *xs = x + ((int64_t)b * T + t_first) * D;
    const Tin *ds = dt + ((int64_t)b * T + t_first) * D;
    const Tin *bs = Bm + ((int64_t)b * T + t_first) * kStates;
    const int64_t bstep = kRev ? -kStates : kStates;

    auto consume = [&](const Tin *xr, const Tin *dr, int64_t k0, int count) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (i < count) {
                const float dl = widen(dr[i]);
                const float dx = dl * widen(xr[i]);
                S += dl;
                const Tin *brow = bs + (k0 + i) * bstep;
#pragma unroll
                for (int q = 0; q < kStates / 2; ++q) {
                    float b0, b1;
                    load_pair(brow, q, b0, b1);
                    h[2 * q] = __builtin_fmaf(fast_exp2(dl * a2[2 * q]), h[2 * q], dx * b0);
                    h[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2[2 * q + 1]), h[2 * q + 1], dx * b1);
                }
            }
        }
    };

    const int64_t n_full = len / U;
    const int rem = (int)(len - n_full * U);
    Tin xr[U], dr[U];
    if (n_full > 0) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            xr[i] = xs[i * step + d];
            dr[i] = ds[i * step + d];
        }
    }
    for (int64_t g = 0; g < n_full; ++g) {
        // issue the next stage's loads before this stage's arithmetic
        Tin xn[U], dn[U];
        const int64_t kn = (g + 1) * U;
        if (g + 1 < n_full) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                xn[i] = xs[(kn + i) * step + d];
                dn[i] = ds[(kn + i) * step + d];
            }
        }
        consume(xr, dr, g * U, U);
#pragma unroll
        for (int i = 0; i < U; ++i) { xr[i] = xn[i]; dr[i] = dn[i]; }
    }
    if (rem > 0) {
        const int64_t k0 = n_full * U;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t k = k0 + (i < rem ? i : rem - 1);
            xr[i] = xs[k * step + d];
            dr[i] = ds[k * step + d];
        }
        consume(xr, dr, k0, rem);
    }
    if (live) {
        float4 *o = reinterpret_cast<float4 *>(hout + (((int64_t)b * n_chunks + c) * D + d) * kStates);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = make_float4(h[4 * q + 0], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
        if (!kDirect && sout != nullptr) sout[((int64_t)b * n_chunks + c) * D + d] = S;
    }
}

// ------------------------------------------------------------------------
// Carry across chunks: one thread per (b, d, n), sequential over chunks.
// Forward: h starts at h_init (or 0); for chunk c < n_agg, h_in[c] = h, then
// h <- exp2(A' S_c) h + h_local_c.  Writes h_in[n_agg] too when requested,
// and the final state.  Reverse (kRev): h starts at 0 on the right, walks
// chunks n_chunks-1 .. 0, h_in[c] = h (the state entering chunk c from its
// right end), then folds chunk c (aggregates exist for c >= 1).
template <bool kRev>
__global__ __launch_bounds__(256) void carry_kernel(
    const float *__restrict__ agg_h, const float *__restrict__ agg_s, const float *__restrict__ A,
    const float *h_init, float *__restrict__ h_in, float *h_final,
    int batch, int D, int n_chunks, int n_agg)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)batch * D * kStates;
    if (i >= total) return;
    const int n = (int)(i % kStates);
    const int64_t bd = i / kStates;
    const int d = (int)(bd % D);
    const int64_t b = bd / D;
    const float a2 = A[(int64_t)d * kStates + n] * kLog2e;
    const int64_t cs = (int64_t)D * kStates;      // chunk stride in agg_h / h_in
    const int64_t base_h = b * n_chunks * cs + (int64_t)d * kStates + n;
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
        for (int c = n_chunks - 1; c >= 0; --c) {
            h_in[base_h + c * cs] = h;
            if (c == 0) break;
            const float s = agg_s[base_s + (int64_t)c * D];
            h = __builtin_fmaf(fast_exp2(a2 * s), h, agg_h[base_h + c * cs]);
        }
    }
}

// ------------------------------------------------------------------------
// Bidirectional block kernel: forward scan from the chunk's incoming state,
// reverse scan restricted to each L-token block, fused output.
//
// Workgroup = 4 waves x 64 lanes; lane = channel, wave w = states 4w..4w+3.
// Tokens are processed in register-resident groups of 16: the discretisation
// (decay and injection for 16 tokens x 4 states) is computed once, kept in
// VGPRs, and consumed by the forward pass (ascending) and then the in-block
// reverse pass (descending).  Each wave's partial output sums over its 4
// states go through LDS (double-buffered, one barrier per group) and each
// wave finishes 4 of the 16 tokens.  Dskip * x is folded into wave 0's
// partial.  Tokens past the chunk end inside the last group are neutral
// (dt = 0 gives decay 1 and injection 0) and are not stored.
//
// hin: incoming state of chunk c at hin[b*hin_bs + c*hin_cs + d*16 + n].
// bounds (optional): forward state at every multiple of L, [batch,T/L+1,D,16].
// hout (optional): forward state after token T-1 (written by the last chunk;
// may alias hin when there is a single chunk: each thread reads its own
// states before it writes them).
// grid = (ceil(D/64), chunks, batch), block = 256.
template <typename Tin, int L>
__global__ __launch_bounds__(kWave * kWavesBidir) void bidir_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    const float *hin, int64_t hin_bs, int64_t hin_cs,
    Tin *__restrict__ y, float *__restrict__ bounds, float *hout,
    int64_t T, int D, int64_t Tc)
{
    static_assert(kGroup % L == 0, "block length must divide the token group");
    __shared__ float red[2][kWavesBidir][kGroup][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform(threadIdx.x >> 6);
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int64_t row = (int64_t)b * T;
    const int s0 = 4 * w;                  // first state of this wave

    float a2[4], hf[4];
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
    const int64_t nbl = T / L;             // number of L-blocks (T % L == 0)
    if (bounds != nullptr && c == 0 && live) {
        *reinterpret_cast<float4 *>(bounds + ((int64_t)b * (nbl + 1) * D + d) * kStates + s0) =
            make_float4(hf[0], hf[1], hf[2], hf[3]);
    }

    int buf = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kGroup) {
        const int nvalid = (int)((t_end - t0 < kGroup) ? (t_end - t0) : kGroup);   // uniform
        float xv[kGroup], dl[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int ii = i < nvalid ? i : nvalid - 1;
            const int64_t ix = (row + t0 + ii) * D + d;
            xv[i] = widen(x[ix]);
            dl[i] = i < nvalid ? widen(dt[ix]) : 0.f;
        }
        float dA[kGroup][4], u[kGroup][4], ya[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int ii = i < nvalid ? i : nvalid - 1;
            const Tin *brow = Bm + (row + t0 + ii) * kStates + s0;
            const float dx = dl[i] * xv[i];
            float bv[4];
            load_pair(brow, 0, bv[0], bv[1]);
            load_pair(brow, 1, bv[2], bv[3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dA[i][j] = fast_exp2(dl[i] * a2[j]);
                u[i][j] = dx * bv[j];
            }
        }
        // forward, ascending
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int ii = i < nvalid ? i : nvalid - 1;
            const Tin *crow = Cm + (row + t0 + ii) * kStates + s0;
            float cv[4];
            load_pair(crow, 0, cv[0], cv[1]);
            load_pair(crow, 1, cv[2], cv[3]);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hf[j] = __builtin_fmaf(dA[i][j], hf[j], u[i][j]);
                acc = __builtin_fmaf(cv[j], hf[j], acc);
            }
            ya[i] = acc;
            if ((i + 1) % L == 0 && bounds != nullptr && i < nvalid && live) {
                const int64_t k = (t0 + i + 1) / L;
                *reinterpret_cast<float4 *>(bounds + (((int64_t)b * (nbl + 1) + k) * D + d) * kStates + s0) =
                    make_float4(hf[0], hf[1], hf[2], hf[3]);
            }
        }
        // reverse inside each L-block, descending, from zero at the block end
        float hr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = kGroup - 1; i >= 0; --i) {
            const int ii = i < nvalid ? i : nvalid - 1;
            const Tin *crow = Cm + (row + t0 + ii) * kStates + s0;
            float cv[4];
            load_pair(crow, 0, cv[0], cv[1]);
            load_pair(crow, 1, cv[2], cv[3]);
            if ((i + 1) % L == 0) { hr[0] = hr[1] = hr[2] = hr[3] = 0.f; }
            float acc = ya[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hr[j] = __builtin_fmaf(dA[i][j], hr[j], u[i][j]);
                acc = __builtin_fmaf(cv[j], hr[j], acc);
            }
            ya[i] = acc;
        }
        if (w == 0) {
#pragma unroll
            for (int i = 0; i < kGroup; ++i) ya[i] = __builtin_fmaf(dsk, xv[i], ya[i]);
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) red[buf][w][i][lane] = ya[i];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * w + q;
            const float s = red[buf][0][i][lane] + red[buf][1][i][lane] + red[buf][2][i][lane] +
                            red[buf][3][i][lane];
            if (live && i < nvalid) y[(row + t0 + i) * D + d] = narrow<Tin>(s);
        }
        buf ^= 1;
    }
    if (hout != nullptr && t_end == T && live) {
        *reinterpret_cast<float4 *>(hout + ((int64_t)b * D + d) * kStates + s0) =
            make_float4(hf[0], hf[1], hf[2], hf[3]);
    }
}

// ------------------------------------------------------------------------
// Directional output sweep for the full-sequence baseline: one lane per
// channel, 16 states.  Forward (kRev = false): from the chunk's incoming
// forward state, writes yf_t = sum_n C_t h_t to an fp32 buffer.  Reverse:
// from the state entering the chunk from its right end, walks the chunk
// backwards and writes y_t = yf_t + sum_n C_t h_t + Dskip x_t.
// grid = (ceil(D/64), chunks, batch), block = 64.
template <typename Tin, bool kRev>
__global__ __launch_bounds__(kWave) void sweep_output_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const float *__restrict__ A, const float *__restrict__ Dskip,
    const float *__restrict__ hin, float *__restrict__ yf, Tin *__restrict__ y,
    int64_t T, int D, int64_t Tc, int n_chunks)
{
    constexpr int U = 4;                      // tokens per pipeline stage
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int64_t len = t_end - t_begin;

    float a2[kStates], h[kStates];
    {
        const float4 *ar = reinterpret_cast<const float4 *>(A + (int64_t)d * kStates);
        const float4 *hr = reinterpret_cast<const float4 *>(hin + (((int64_t)b * n_chunks + c) * D + d) * kStates);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 v = ar[q];
            a2[4 * q + 0] = v.x * kLog2e; a2[4 * q + 1] = v.y * kLog2e;
            a2[4 * q + 2] = v.z * kLog2e; a2[4 * q + 3] = v.w * kLog2e;
            float4 g = hr[q];
            h[4 * q + 0] = g.x; h[4 * q + 1] = g.y; h[4 * q + 2] = g.z; h[4 * q + 3] = g.w;
        }
    }
    const float dsk = Dskip[d];
    const int64_t step = kRev ? -(int64_t)D : (int64_t)D;
    const int64_t t_first = kRev ? t_end - 1 : t_begin;
    const int64_t o_first = ((int64_t)b * T + t_first) * D;
    const Tin *xs = x + o_first;
    const Tin *ds = dt + o_first;
    float *yfs = yf + o_first;
    Tin *ys = y + o_first;
    const Tin *bs = Bm + ((int64_t)b * T + t_first) * kStates;
    const Tin *cs = Cm + ((int64_t)b * T + t_first) * kStates;
    const int64_t bstep = kRev ? -kStates : kStates;

    auto consume = [&](const Tin *xr, const Tin *dr, const float *yr, int64_t k0, int count) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (i < count) {
                const float xv = widen(xr[i]);
                const float dl = widen(dr[i]);
                const float dx = dl * xv;
                const Tin *brow = bs + (k0 + i) * bstep;
                const Tin *crow = cs + (k0 + i) * bstep;
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < kStates / 2; ++q) {
                    float b0, b1, c0, c1;
                    load_pair(brow, q, b0, b1);
                    load_pair(crow, q, c0, c1);
                    h[2 * q] = __builtin_fmaf(fast_exp2(dl * a2[2 * q]), h[2 * q], dx * b0);
                    h[2 * q + 1] = __builtin_fmaf(fast_exp2(dl * a2[2 * q + 1]), h[2 * q + 1], dx * b1);
                    acc = __builtin_fmaf(c0, h[2 * q], acc);
                    acc = __builtin_fmaf(c1, h[2 * q + 1], acc);
                }
                const int64_t o = (k0 + i) * step + d;
                if (!kRev) {
                    if (live) yfs[o] = acc;
                } else {
                    const float tot = yr[i] + acc + dsk * xv;
                    if (live) ys[o] = narrow<Tin>(tot);
                }
            }
        }
    };

    const int64_t n_full = len / U;
    const int rem = (int)(len - n_full * U);
    Tin xr[U], dr[U];
    float yr[U];
    auto load_stage = [&](int64_t k0, int count, Tin *xo, Tin *dout, float *yo) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t k = k0 + (i < count ? i : count - 1);
            xo[i] = xs[k * step + d];
            dout[i] = ds[k * step + d];
            if (kRev) yo[i] = yfs[k * step + d];
        }
    };
    if (n_full > 0) load_stage(0, U, xr, dr, yr);
    for (int64_t g = 0; g < n_full; ++g) {
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

// dst[i] = src[i], or 0 when src is null.  A kernel rather than a memset or
// memcpy node so that callers may capture the entry points in a HIP graph.
__global__ __launch_bounds__(256) void copy_or_zero_kernel(const float *src, float *dst, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src != nullptr ? src[i] : 0.f;
}

}  // namespace bdssm_dev
