// bdssm_bwd_kernels.hpp -- gfx950 kernels of the backward pass (reverse-mode
// gradients) of the all-block training forms.  Device code only; the launch
// plans and the C ABI are in bdssm.hip, the launchers in launch_bwd*.hip.
//
// Page cited: gist.science German page on arXiv 2607.02805, "Technische
// Zusammenfassung" > "Methodik" [DE-M]: the all-block objective lets the
// downstream block losses train the prefix scan, i.e. gradients flow through
// the forward recurrence across blocks and, in the two-stream form, from the
// noisy blocks back into the clean stream's block-start states.
//
// For one (batch, channel) row and state n, with a_t = exp(dt_t A) and
// u_t = dt_t B_t x_t, the forward training scan is
//   hf_t = a_t hf_{t-1} + u_t,  hr_t = a_t hr_{t+1} + u_t (inside a block),
//   y_t = sum_n C_t (hf_t + hr_t) + Dskip x_t.
// Given dy, the adjoints are
//   gf_t = dy_t C_t + q_{t+1},  q_t = a_t gf_t   (q runs right to left over the
//          whole row; + dbounds at block ends when the block states feed
//          another computation)
//   gr_t = dy_t C_t + a_{t-1} gr_{t-1}          (left to right inside a block)
// and with du = gf + gr, da = gf hf_{t-1} + gr hr_{t+1}:
//   ddt += du B x + da a A,  dx += du dt B (+ dy Dskip),  dB += du dt x,
//   dC += dy (hf + hr),      dA += da a dt,               dDskip += dy x.
//
// Pipeline (continuous form): adjoint_chunk_kernel (chunk-local q from zero
// and S = sum dt, right to left), carry_kernel<true> (q entering every chunk
// from its right end), bwd_wave_kernel (one coarse chunk per workgroup column,
// walking 16-token groups right to left from the carried q, with the forward
// state at each group start taken from the forward pass's saved block states),
// then bc_reduce_kernel and param_reduce_kernel for the sums over channels,
// batch and chunks.  The two-stream form needs no carry: every block starts
// from its given state and its adjoint starts from zero at its end.
#pragma once

#include "bdssm_kernels.hpp"

namespace bdssm_dev {

// ------------------------------------------------------------------------
// Chunk-local adjoint of the forward state, one lane per channel, 16 states
// in registers, walking the chunk from its last token to its first:
//   q <- a_t (dy_t C_t + q)      (+ dbounds[(t+1)/L] added to q at block ends)
// Starting from q = 0 at the chunk's right end, the value reached at its left
// end and S = sum dt over the chunk describe the chunk's action on an
// incoming q:  q_left = exp2(A' S) q_right + q_local.
// grid = (ceil(D/64), chunks launched, batch), block = 64; chunk c = c_first +
// blockIdx.y.  L divides 16 and chunks are whole 16-token groups, so block
// ends sit at chunk-local rows p with (p + 1) % L == 0 (masks and shifts).
// Fusions: dt is formed as step_size<kDt>(dt stream, dt_bias) and, with the
// gate z (may be null), dy enters as dy silu(z), as in the forward.
template <typename Tin, int L, int kDt = kDtPlain>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(6))) void adjoint_chunk_kernel(
    const Tin *__restrict__ dt, const Tin *__restrict__ dy, const Tin *__restrict__ Cm,
    const float *__restrict__ A, const float *__restrict__ dbounds, float *__restrict__ qout,
    float *__restrict__ sout, int64_t T, int D, int64_t Tc, int n_chunks, int c_first,
    const float *__restrict__ dt_bias, const Tin *__restrict__ z)
{
    static_assert(kGroup % L == 0, "block length must divide the token group");
    constexpr int U = 4;                      // tokens per pipeline stage
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = c_first + blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);
    const int64_t nbl = T / L;
    const int64_t blk0 = t_begin / L;           // block index of the chunk's first row

    float a2[kStates], q[kStates];
    {
        const float4 *ar = reinterpret_cast<const float4 *>(A + (int64_t)d * kStates);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float4 v = ar[k];
            a2[4 * k + 0] = v.x * kLog2e; a2[4 * k + 1] = v.y * kLog2e;
            a2[4 * k + 2] = v.z * kLog2e; a2[4 * k + 3] = v.w * kLog2e;
        }
    }
#pragma unroll
    for (int n = 0; n < kStates; ++n) q[n] = 0.f;
    float S = 0.f;
    const int64_t first = (int64_t)b * T + t_begin;
    const Rows<Tin> ds(dt + first * D, len, D, d);
    const Rows<Tin> ys(dy + first * D, len, D, d);
    const bool gate = z != nullptr;
    const Rows<Tin> zs((gate ? z : dy) + first * D, len, D, d);
    const float bias = (kDt != kDtPlain && dt_bias != nullptr) ? dt_bias[d] : 0.f;
    const Tin *cs = Cm + first * kStates;

    // Tokens stream through registers in stages of U as in chunk_state_kernel:
    // a stage's dt and dy are loaded one stage ahead into one of two buffers
    // used in turn (the loop unrolled by two, so no copy between iterations
    // forces an early wait), held as 32-bit values; the gate z is read where
    // it is used.
    using St = typename Staged<Tin>::type;
    auto consume = [&](const St *dr, const St *yr, int k0, int count) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (i < count) {
                const int p = len - 1 - (k0 + i);            // row within the chunk
                if (dbounds != nullptr && (p + 1) % L == 0) {
                    const float4 *r = reinterpret_cast<const float4 *>(
                        dbounds + (((int64_t)b * (nbl + 1) + blk0 + (p + 1) / L) * D + d) * kStates);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float4 v = r[k];
                        q[4 * k + 0] += v.x; q[4 * k + 1] += v.y;
                        q[4 * k + 2] += v.z; q[4 * k + 3] += v.w;
                    }
                }
                const float dl = step_size<kDt>(widen_staged(dr[i]), bias);
                float gy = live ? widen_staged(yr[i]) : 0.f;
                if (gate) gy *= silu_f(widen(zs.load(p)));
                S += dl;
                const Tin *crow = cs + (int64_t)p * kStates;
#pragma unroll
                for (int k = 0; k < kStates / 2; ++k) {
                    float c0, c1;
                    load_pair(crow, k, c0, c1);
                    q[2 * k] = fast_exp2(dl * a2[2 * k]) * __builtin_fmaf(gy, c0, q[2 * k]);
                    q[2 * k + 1] = fast_exp2(dl * a2[2 * k + 1]) * __builtin_fmaf(gy, c1, q[2 * k + 1]);
                }
            }
        }
    };
    // count < U: the rows past the stage re-read its last row
    auto load_stage = [&](int k0, int count, St *dout, St *yo) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int p = len - 1 - (k0 + (i < count ? i : count - 1));
            dout[i] = ds.load(p);
            yo[i] = ys.load(p);
        }
    };
    const int n_full = len / U;
    const int rem = len - n_full * U;
    St da[U], ya[U], db[U], yb[U];
    if (n_full > 0) load_stage(0, U, da, ya);
    int g = 0;
    for (; g + 1 < n_full; g += 2) {
        load_stage((g + 1) * U, U, db, yb);
        consume(da, ya, g * U, U);
        if (g + 2 < n_full) load_stage((g + 2) * U, U, da, ya);
        consume(db, yb, (g + 1) * U, U);
    }
    if (g < n_full) consume(da, ya, g * U, U);       // an odd number of full stages: the last is in da
    if (rem > 0) {
        load_stage(n_full * U, rem, db, yb);
        consume(db, yb, n_full * U, rem);
    }
    if (live) {
        float4 *o = reinterpret_cast<float4 *>(qout + (((int64_t)b * n_chunks + c) * D + d) * kStates);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o[k] = make_float4(q[4 * k + 0], q[4 * k + 1], q[4 * k + 2], q[4 * k + 3]);
        sout[((int64_t)b * n_chunks + c) * D + d] = S;
    }
}

// Cross-lane exchanges used by the channel reduction (partner = lane ^ mask).
__device__ __forceinline__ float xchg8(float v) {        // DPP row_ror:8 == lane ^ 8 in a row of 16
    return dpp_perm<kDppRor8>(v);
}
__device__ __forceinline__ float xchg4(float v) {        // ds_swizzle bit mode: xor_mask 4
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (4 << 10) | 0x1F));
}
__device__ __forceinline__ float xchg16(float v) {       // ds_swizzle bit mode: xor_mask 16
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (16 << 10) | 0x1F));
}
__device__ __forceinline__ float xchg32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v)));
}
// Two-value folds with the gfx950 lane swaps (VALU instructions, no LDS pipe):
// fold32(a, b) is a[l] + a[l + 32] in lanes l < 32 and b[l - 32] + b[l] in lanes
// l >= 32; fold16(a, b) is, per 16-lane row r, the sum of rows r and r ^ 1 of a
// in the even rows and of b in the odd rows.
__device__ __forceinline__ float fold32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fold16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------------
// Backward of the bidirectional pass over one coarse chunk.  Same lane layout
// as bidir_wave_kernel: lane = 4 * channel + state group, 16 channels per wave,
// 4 waves per workgroup (64 channels), 4 states per lane.  16-token groups are
// visited from the chunk's last to its first; each group's x / dt / dy rows
// and B / C rows are DMA'd into the wave's LDS slice one group ahead.
//
// Per group:
//   pass A (left to right): the forward state from the group's start state
//     (continuous form: the saved block state at the group start; two-stream
//     form: the given state at every block start), keeping hf_{t-1} per token,
//     and the reverse scan's adjoint gr, reset at block starts;
//   pass B (right to left): the in-block reverse state hr and the forward
//     adjoint gf (q carried across groups; two-stream form: reset at block
//     ends), and every gradient term.
// Reductions:
//   * ddt and dx sum over the channel's 16 states: quad reduce-scatter (DPP),
//     after which each lane owns 4 tokens of its channel and stores them;
//   * dB and dC sum over channels: for every token the 8 values of a lane
//     ({B, C} x 4 states) are reduce-scattered over the wave's 16 channels
//     (exchanges with lanes ^ 8, ^ 4, ^ 16, then a sum with lane ^ 32), leaving
//     one value per lane pair; the four waves' results meet in LDS (one barrier per
//     group) and are summed in a fixed order into part_bc [batch, ceil(D/64),
//     T, 32] (32 = dB's 16 states then dC's), reduced over channel blocks by
//     bc_reduce_kernel;
//   * dA and dDskip accumulate in registers over the chunk and are written
//     per (batch, chunk) to part_a [batch, chunks, D, 16] and part_d
//     [batch, chunks, D].
// Lanes past the last channel read dt = dy = 0 and start from a zero
// adjoint, so every gradient term they form is zero.
//
// h_start: continuous form: the forward's saved block states h_bounds
//          [batch, T/L+1, D, 16] (read at group starts); two-stream form
//          (kBlockInit): the block start states h0_blocks, same layout.
// qin: continuous form, adjoint entering coarse chunk c from its right end at
//      qin[b*qin_bs + c*qin_cs + d*16 + n]; nullptr = zero (also ignored for
//      the chunk that ends the sequence).
// dbounds: continuous form only (may be null): dJ/dh_bounds.
// dh0: continuous form: dJ/dh_init [batch, D, 16] (may be null), written by
//      chunk 0; two-stream form: dJ/dh0_blocks [batch, T/L+1, D, 16] (may be
//      null; entry T/L is written as zero).
// grid = (ceil(D/64), chunks, batch), block = 256.
template <typename Tin, int L, bool kBlockInit>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(2))) void bwd_wave_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const Tin *__restrict__ dy, const float *__restrict__ A,
    const float *__restrict__ Dskip, const float *__restrict__ h_start, const float *qin,
    int64_t qin_bs, int64_t qin_cs, const float *__restrict__ dbounds, Tin *__restrict__ dx,
    Tin *__restrict__ ddt, float *__restrict__ part_bc, float *__restrict__ part_a,
    float *__restrict__ part_d, float *__restrict__ dh0, int64_t T, int D, int64_t Tc)
{
    constexpr int P = 4;
    constexpr int CW = kWave / P;
    constexpr int ES = sizeof(Tin);
    static_assert(kGroup % L == 0, "block length must divide the token group");
    __shared__ uint32_t xdA[4][3][4][kWave], xdB[4][3][4][kWave];
    __shared__ uint32_t bcrA[4][2][4][kWave], bcrB[4][2][4][kWave];
    __shared__ float bcfA[4][kGroup][2][kStates], bcfB[4][kGroup][2][kStates];
    __shared__ float redA[4][kGroup * 2 * kStates], redB[4][kGroup * 2 * kStates];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform(threadIdx.x >> 6);
    const int cl = lane >> 2;
    const int g = lane & 3;
    const int s0 = P * g;
    const int d_raw = blockIdx.x * kWave + w * CW + cl;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);
    const int64_t nbl = T / L;

    float a2[P], ar[P], q[P];
    {
        const float4 av = *reinterpret_cast<const float4 *>(A + (int64_t)d * kStates + s0);
        ar[0] = av.x; ar[1] = av.y; ar[2] = av.z; ar[3] = av.w;
#pragma unroll
        for (int j = 0; j < P; ++j) a2[j] = ar[j] * kLog2e;
        q[0] = q[1] = q[2] = q[3] = 0.f;
        if (!kBlockInit && qin != nullptr && t_end < T && live) {
            const float4 v = *reinterpret_cast<const float4 *>(
                qin + (int64_t)b * qin_bs + (int64_t)c * qin_cs + (int64_t)d * kStates + s0);
            q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
        }
    }
    const float dsk = Dskip[d];
    float dA_acc[P] = {0.f, 0.f, 0.f, 0.f};
    float dD_acc = 0.f;
    auto state_at = [&](const float *base, int64_t blk) -> float4 {
        return *reinterpret_cast<const float4 *>(base + (((int64_t)b * (nbl + 1) + blk) * D + d) * kStates + s0);
    };
    if (kBlockInit && dh0 != nullptr && t_end == T && live)
        *reinterpret_cast<float4 *>(dh0 + (((int64_t)b * (nbl + 1) + nbl) * D + d) * kStates + s0) =
            make_float4(0.f, 0.f, 0.f, 0.f);

    const int64_t first = (int64_t)b * T + t_begin;
    const int d_w0 = blockIdx.x * kWave + w * CW;
    const Rows<Tin> xs(x + first * D, len, D, 0);
    const Rows<Tin> ds(dt + first * D, len, D, 0);
    const Rows<Tin> ys(dy + first * D, len, D, 0);
    __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Bm + first * kStates)), 0, uniform(len * kStates * ES), kRawBufferWord3);
    __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Cm + first * kStates)), 0, uniform(len * kStates * ES), kRawBufferWord3);
    const int ld_tok = lane >> 4, ld_col = lane & 15;
    const int ld_ch = (d_w0 + ld_col < D) ? d_w0 + ld_col : D - 1;

    // dt and dy of tokens past the chunk end and of channels past D are read
    // at an offset beyond the buffer's range, which the buffer unit returns
    // as zero: such tokens then decay by 1 and inject nothing, and dead lanes
    // form no gradient terms, without any masking in the arithmetic
    const bool ld_live = d_w0 + ld_col < D;
    auto issue = [&](auto &xd, auto &bcr, int k0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kr = k0 + 4 * j + ld_tok;
            const int k = kr < len ? kr : len - 1;
            const int zoff = (kr < len && ld_live) ? ld_ch * ES + k * ds.pitch : kOutOfRange;
            load_to_lds<ES>(xs.rsrc, &xd[w][0][j][0], ld_ch * ES + k * xs.pitch, 0);
            load_to_lds<ES>(ds.rsrc, &xd[w][1][j][0], zoff, 0);
            load_to_lds<ES>(ys.rsrc, &xd[w][2][j][0], zoff, 0);
            load_to_lds<ES>(brs, &bcr[w][0][j][0], (k * kStates + ld_col) * ES, 0);
            load_to_lds<ES>(crs, &bcr[w][1][j][0], (k * kStates + ld_col) * ES, 0);
        }
    };
    auto elem = [&](uint32_t v) -> float {
        return ES == 2 ? __uint_as_float(v << 16) : __uint_as_float(v);
    };
    auto widen_bc = [&](auto &bcr, auto &bcf) {
        __builtin_amdgcn_s_waitcnt(0x0F70);     // this wave's own LDS loads have landed
#pragma unroll
        for (int which = 0; which < 2; ++which)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bcf[w][4 * j + ld_tok][which][ld_col] = elem(bcr[w][which][j][lane]);
    };
    auto xor2 = [](float v) {
        return dpp_perm<kDppXor2>(v);
    };
    auto xor1 = [](float v) {
        return dpp_perm<kDppXor1>(v);
    };
    const bool hi2 = (g & 2) != 0, hi1 = (g & 1) != 0;
    const bool b2 = (lane & 4) != 0, b3 = (lane & 8) != 0, b4 = (lane & 16) != 0, b5 = (lane & 32) != 0;
    // slot of this lane's reduced dB / dC value within a token's 32: dB (b5
    // clear) or dC, state 4g + 2 b4 + b3
    const int red_slot = (b5 ? kStates : 0) + s0 + (b4 ? 2 : 0) + (b3 ? 1 : 0);
    const int nblk64 = gridDim.x;
    float *pbc = part_bc + ((int64_t)b * nblk64 + blockIdx.x) * T * 32;
    Tin *dxl = dx + first * D + d;
    Tin *dtl = ddt + first * D + d;

    auto group = [&](auto &xd, auto &bcf, auto &red, auto &xdn, auto &bcrn, auto &bcfn, int k0) {
        const int nvalid = (len - k0 < kGroup) ? len - k0 : kGroup;   // uniform
        const bool more = k0 > 0;
        if (more) issue(xdn, bcrn, k0 - kGroup);
        auto xval = [&](int i) { return elem(xd[w][0][i >> 2][(i & 3) * CW + cl]); };
        auto dval = [&](int i) { return elem(xd[w][1][i >> 2][(i & 3) * CW + cl]); };
        auto yval = [&](int i) { return elem(xd[w][2][i >> 2][(i & 3) * CW + cl]); };

        // One 4-token segment at a time from the right.  For each segment,
        // first the forward quantities: the forward state is known at every
        // block start (the saved block states, or the given block starts of the
        // two-stream form) and the reverse adjoint is zero there, so the forward
        // scan runs from the segment's block start up to the segment and then
        // over it, keeping the decays, hf_{t-1} and gr_t of its 4 tokens.  Then
        // the segment is walked right to left with the reverse state and the
        // forward adjoint.  (Recomputing instead of storing all 16 tokens keeps
        // the kernel within 256 registers, i.e. two waves per SIMD.)
        constexpr int kSeg = 4, nSeg = kGroup / kSeg;
        auto step_fwd = [&](int i, float *hf, float *pr, float *a_o, float *hp_o, float *gr_o) {
            const float dl = dval(i), dxv = dl * xval(i), gy = yval(i);
            const float4 b4v = *reinterpret_cast<const float4 *>(&bcf[w][i][0][s0]);
            const float4 c4v = *reinterpret_cast<const float4 *>(&bcf[w][i][1][s0]);
            const float bv[4] = {b4v.x, b4v.y, b4v.z, b4v.w};
            const float cv[4] = {c4v.x, c4v.y, c4v.z, c4v.w};
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const float a = fast_exp2(dl * a2[j]);
                const float gr_j = __builtin_fmaf(gy, cv[j], pr[j]);
                if (a_o != nullptr) { a_o[j] = a; hp_o[j] = hf[j]; gr_o[j] = gr_j; }
                hf[j] = __builtin_fmaf(a, hf[j], dxv * bv[j]);
                pr[j] = a * gr_j;
            }
        };
        float hr[P] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sg = nSeg - 1; sg >= 0; --sg) {
            float a4[kSeg][P], hp4[kSeg][P], gr4[kSeg][P];
            {
                const int i0 = sg * kSeg;
                const int r = (i0 / L) * L;                 // block start at or before i0
                float hf[P], pr[P] = {0.f, 0.f, 0.f, 0.f};
                {
                    const int rv = r < nvalid ? r : 0;      // past the end: any valid state
                    const float4 v = state_at(h_start, (t_begin + k0 + rv) / L);
                    hf[0] = v.x; hf[1] = v.y; hf[2] = v.z; hf[3] = v.w;
                }
#pragma unroll
                for (int i = r; i < i0; ++i) {
                    step_fwd(i, hf, pr, nullptr, nullptr, nullptr);
                    if ((i & 3) == 3) asm volatile("" ::: "memory");
                }
#pragma unroll
                for (int k = 0; k < kSeg; ++k) {
                    const int i = i0 + k;
                    if (i % L == 0 && i != r) {
                        if constexpr (kBlockInit) {
                            const int ib = i < nvalid ? i : 0;
                            const float4 v = state_at(h_start, (t_begin + k0 + ib) / L);
                            hf[0] = v.x; hf[1] = v.y; hf[2] = v.z; hf[3] = v.w;
                        }
                        pr[0] = pr[1] = pr[2] = pr[3] = 0.f;
                    }
                    step_fwd(i, hf, pr, a4[k], hp4[k], gr4[k]);
                }
            }
            asm volatile("" ::: "memory");
            float sdt[kSeg], sdx[kSeg];
#pragma unroll
            for (int k = kSeg - 1; k >= 0; --k) {
                const int i = sg * kSeg + k;
                if ((i + 1) % L == 0) {
                    hr[0] = hr[1] = hr[2] = hr[3] = 0.f;
                    if constexpr (kBlockInit) {
                        q[0] = q[1] = q[2] = q[3] = 0.f;
                    } else {
                        const int64_t tb = t_begin + k0 + i + 1;
                        if (dbounds != nullptr && i < nvalid && live) {
                            const float4 v = state_at(dbounds, tb / L);
                            q[0] += v.x; q[1] += v.y; q[2] += v.z; q[3] += v.w;
                        }
                    }
                }
                const float xv = xval(i), dl = dval(i), gy = yval(i);
                const float dxv = dl * xv;
                const float4 b4v = *reinterpret_cast<const float4 *>(&bcf[w][i][0][s0]);
                const float4 c4v = *reinterpret_cast<const float4 *>(&bcf[w][i][1][s0]);
                const float bv[4] = {b4v.x, b4v.y, b4v.z, b4v.w};
                const float cv[4] = {c4v.x, c4v.y, c4v.z, c4v.w};
                float s1 = 0.f, s2 = 0.f;
                float tokv[8];                          // dB then dC of the lane's 4 states
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const float a = a4[k][j];
                    const float u = dxv * bv[j];
                    const float hr1 = hr[j];
                    hr[j] = __builtin_fmaf(a, hr1, u);
                    const float gf = __builtin_fmaf(gy, cv[j], q[j]);
                    const float du = gf + gr4[k][j];
                    const float da = __builtin_fmaf(gf, hp4[k][j], gr4[k][j] * hr1);
                    q[j] = a * gf;
                    s1 = __builtin_fmaf(du, bv[j], s1);
                    const float daa = da * a;
                    s2 = __builtin_fmaf(daa, ar[j], s2);
                    dA_acc[j] = __builtin_fmaf(daa, dl, dA_acc[j]);
                    tokv[j] = du * dxv;                                              // dB
                    tokv[4 + j] = gy * (__builtin_fmaf(a, hp4[k][j], u) + hr[j]);     // dC
                }
                sdt[k] = __builtin_fmaf(xv, s1, s2);
                sdx[k] = dl * s1;
                if constexpr (kBlockInit) {
                    if (i % L == 0 && dh0 != nullptr && i < nvalid && live)
                        *reinterpret_cast<float4 *>(dh0 + (((int64_t)b * (nbl + 1) + (t_begin + k0 + i) / L) * D + d) * kStates + s0) =
                            make_float4(q[0], q[1], q[2], q[3]);
                }
                {
                    // reduce the token's 8 values (dB, dC x 4 states) over the
                    // wave's 16 channels: reduce-scatter over lane bit 5 (dB /
                    // dC) and bit 4 (states j, j + 2) by lane-swap folds, over
                    // bit 3 (states j, j + 1) by a row rotation, then a plain
                    // sum over bit 2 (both lanes hold it)
                    float f4[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) f4[m] = fold32(tokv[m], tokv[m + 4]);
                    const float e0 = fold16(f4[0], f4[2]), e1 = fold16(f4[1], f4[3]);
                    float r1 = (b3 ? e1 : e0) + xchg8(b3 ? e0 : e1);
                    r1 += xchg4(r1);
                    if (!b2) red[w][i * 2 * kStates + red_slot] = r1;
                }
            }
            // ddt and dx of the segment: quad reduce-scatter over the channel's
            // 16 states; lane g ends with token 2 (g & 1) + {0, 1} of ddt (g < 2)
            // or dx (g >= 2)
            float v4[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float keep = hi2 ? sdx[m] : sdt[m];
                const float send = hi2 ? sdt[m] : sdx[m];
                v4[m] = keep + xor2(send);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float keep = hi1 ? v4[m + 2] : v4[m];
                const float send = hi1 ? v4[m] : v4[m + 2];
                const float tot = keep + xor1(send);
                const int i = sg * kSeg + (hi1 ? 2 : 0) + m;
                const float xv = xval(i), gy = yval(i);
                if (!hi2) dD_acc = __builtin_fmaf(gy, xv, dD_acc);
                if (live && i < nvalid) {
                    if (hi2) dxl[(int64_t)(k0 + i) * D] = narrow<Tin>(__builtin_fmaf(gy, dsk, tot));
                    else dtl[(int64_t)(k0 + i) * D] = narrow<Tin>(tot);
                }
            }
            asm volatile("" ::: "memory");
        }

        // the four waves' dB / dC partials: sum in a fixed order
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int o = threadIdx.x + h * 256;
            const float v = ((red[0][o] + red[1][o]) + red[2][o]) + red[3][o];
            if ((o >> 5) < nvalid) pbc[(t_begin + k0) * 32 + o] = v;
        }
        if (more) widen_bc(bcrn, bcfn);
    };

    const int k_last = ((len - 1) / kGroup) * kGroup;
    issue(xdA, bcrA, k_last);
    widen_bc(bcrA, bcfA);
    for (int k0 = k_last; k0 >= 0; k0 -= 2 * kGroup) {
        group(xdA, bcfA, redA, xdB, bcrB, bcfB, k0);
        if (k0 - kGroup >= 0) group(xdB, bcfB, redB, xdA, bcrA, bcfA, k0 - kGroup);
    }

    // continuous form: gradient of the start state (chunk 0)
    if (!kBlockInit && c == 0 && dh0 != nullptr && live) {
        float v[P] = {q[0], q[1], q[2], q[3]};
        if (dbounds != nullptr) {
            const float4 e = state_at(dbounds, 0);
            v[0] += e.x; v[1] += e.y; v[2] += e.z; v[3] += e.w;
        }
        *reinterpret_cast<float4 *>(dh0 + ((int64_t)b * D + d) * kStates + s0) = make_float4(v[0], v[1], v[2], v[3]);
    }
    // dA and dDskip partials of this (batch, chunk)
    if (live) {
        const int64_t pc = (int64_t)b * gridDim.y + c;
        *reinterpret_cast<float4 *>(part_a + (pc * D + d) * kStates + s0) =
            make_float4(dA_acc[0], dA_acc[1], dA_acc[2], dA_acc[3]);
    }
    dD_acc += xor2(dD_acc);
    dD_acc += xor1(dD_acc);
    if (live && g == 0) part_d[((int64_t)b * gridDim.y + c) * D + d] = dD_acc;
}

// ------------------------------------------------------------------------
// Backward of the bidirectional pass over one coarse chunk, two states per
// lane, for kN = 4, 8, 16 or 32 states: lane = P * channel + state pair
// (states 2g, 2g+1), P = kN / 2 lanes per channel, CW = 64 / P channels per
// wave, 4 waves per workgroup (4 CW channels: 32 at 16 states).  With two
// states per lane the forward states before each token and the reverse
// adjoints of a whole 16-token group fit in 64 VGPRs at any state count, so
// the forward state and the reverse adjoint are formed once per token (no
// segment recomputation):
//   pass A (left to right over the group): hf from the group's block start
//     state, gr reset at block starts; keeps hf_{t-1}, gr_t per token, and
//     the decays of the group's last KA tokens (up to 12: what the registers
//     left over hold without spilling);
//   pass B (right to left): hr (reset at block ends), gf (q carried across
//     groups; + dbounds or reset at block ends), every gradient term; the
//     decays of the other tokens and the injections are formed again.
// Reductions stay in registers (VALU lane exchanges, no LDS round trip):
//   * dB / dC: per token the lane's 4 values are summed over the wave's CW
//     channels by two 32-lane folds (permlane32 swaps) and one 16-lane fold
//     (permlane16 swap), which leave lane l with dB or dC (bit 5) of state
//     2g + (bit 4); the channel bits below bit 4 (none at 32 states) are
//     summed by a DPP row rotation over a token pair (16 states) or by row
//     rotations and quad exchanges with one lane of each duplicate storing;
//     the wave's sums meet the other waves' in red (one barrier per group) and
//     are added in a fixed order into part_bc [batch, ceil(D/(4 CW)), T, 2 kN],
//     reduced over channel blocks by bc_reduce_kernel;
//   * dt and x: per token the lane's two partial sums are summed over the
//     channel's P state pairs by an exchange over the top bit of g (dt kept
//     in lanes g < P/2, x in the others) and exchanges over the lower bits;
//     each lane keeps one token of every P/2, so that after P/2 tokens the
//     64 lanes hold (token, dt or x, channel) and store them together.
// Staging: x / dt / dy rows of the wave's CW channels and the group's B / C
// rows (shared by the workgroup, their loads spread over the waves) are DMA'd
// into LDS one group ahead and widened to fp32 in place by the lane that
// loaded them.  Arguments and the other partial outputs as in bwd_wave_kernel.
//
// L = 0 (long blocks: Lr tokens, a multiple of 16 above 16): a block spans
// several groups.  Groups are still walked right to left, so hr and the
// forward adjoint carry from a group into the one on its left and restart
// only where a block ends; the forward state and the reverse adjoint's carry
// at a group start inside a block come from group_state_kernel (gstate), at a
// block start from the block state and zero.  Chunks are whole blocks.
//
// kFuse (the gradients of the forward's fusions, BwdFuse): the dt rows are
// turned into the step size of the forward (step_size<dt_mode> with dt_bias)
// as they are widened; with the gate z (staged as a fourth row stream), dy
// becomes dy silu(z), the gradient of the ungated output, and the z row holds
// dy silu'(z).  Pass B also forms y_pre = sum_n C (hf + hr) + Dskip x of each
// token (summed over the channel's P lanes by DPP) and parks it in the
// token's x slot, and the flush parks the dt partial total in the dy slot
// (pass B no longer reads either).  After pass B, when the group's state
// arrays are dead, an epilogue turns the parked values into the dt stream's
// gradient (the step size's gradient times softplus'(v) = s(v), s the
// logistic function, taken from the step size as s(v) = 1 - exp(-softplus(v)))
// and dz = dy silu'(z) y_pre, with masked buffer stores; the dt-stream
// gradient's sums over the chunk's tokens go to part_bias [batch, chunks, D]
// for the gradient of dt_bias.  (Done inside pass B, the same work spills.)
// grid = (ceil(D/(4 CW)), chunks, batch), block = 256.

template <typename Tin> struct BwdFuse {
    const float *dt_bias;   // [D] or null
    int dt_mode;            // kDtPlain / kDtBias / kDtSoftplus
    const Tin *z;           // gate [batch, T, D] or null
    Tin *dz;                // [batch, T, D], written when z is given
    float *part_bias;       // [batch, chunks, D] or null
    // separate reverse-direction operands (bwd_general_kernel<..., 2> only):
    // inputs, the reverse dt stream's gradient and the reverse partials
    const Tin *dt_r, *B_r, *C_r;
    const float *A_r, *dt_bias_r;
    Tin *ddt_r;
    float *part_bc_r, *part_a_r, *part_bias_r;
};

// The logistic function of v from softplus(v) = sp: 1 - exp(-sp), with the
// series sp - sp^2/2 + sp^3/6 where the subtraction would cancel (sp < 1/32).
__device__ __forceinline__ float sigmoid_from_softplus(float sp) {
    if (sp < 0.03125f) return sp * (1.f - sp * (0.5f - sp * (1.f / 6.f)));
    return 1.f - fast_exp2(-sp * kLog2e);
}

template <typename Tin, int kN, int L, bool kBlockInit, bool kFuse = false>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(kN == 4 ? 2 : 3))) void bwd_pair_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const Tin *__restrict__ dy, const float *__restrict__ A,
    const float *__restrict__ Dskip, const float *__restrict__ h_start, const float *qin,
    int64_t qin_bs, int64_t qin_cs, const float *__restrict__ dbounds, Tin *__restrict__ dx,
    Tin *__restrict__ ddt, float *__restrict__ part_bc, float *__restrict__ part_a,
    float *__restrict__ part_d, float *__restrict__ dh0, int64_t T, int D, int64_t Tc,
    BwdFuse<Tin> fz, const float *__restrict__ gstate, int Lr)
{
    static_assert(kN == 4 || kN == 8 || kN == 16 || kN == 32, "state counts 4, 8, 16, 32");
    constexpr int P = kN / 2;                 // lanes per channel
    constexpr int CW = kWave / P;             // channels per wave
    constexpr int ES = sizeof(Tin);
    constexpr int G = kGroup;                 // 16 tokens per group
    constexpr int XL = G * CW / kWave;        // x / dt / dy loads per group and stream (P tokens each)
    constexpr int BL = G * kN / kWave;        // B / C loads per group and stream (BT tokens each)
    constexpr int BT = kWave / kN;
    constexpr int TK = P / 2;                 // tokens per dt / x flush
    constexpr int EV = CW / 4;                // the fused epilogue's values per lane
    constexpr int NSB = kFuse ? 4 : 3;        // row streams: x, dt, dy (, z)
    // decays kept from pass A for pass B, per group: as many tokens as the
    // registers hold without spilling at three waves per SIMD (two at 4
    // states); the others are formed again in pass B.  With the fusions only
    // the two-stream form at 16 states and L = 16 has room (4 tokens; the
    // continuous form spilled at 4, the two-stream form at 8)
    constexpr int KA = kFuse ? ((kN == 16 && L == 16 && kBlockInit) ? 4 : 0)
                       : kN == 4 ? 12
                       : (L == 1 || L == 2) ? 0
                       : kN == 8 ? (L == 16 ? 8 : 0)
                       : (L == 0 || L == 4) ? 8 : 12;
    // L = 0: blocks of Lr tokens, a multiple of 16 above 16, spanning several
    // groups; gstate holds the forward state and the reverse adjoint's carry
    // at every group start ([batch, T/16, 2, D, 16], group_state_kernel)
    constexpr bool kLong = L == 0;
    static_assert(!kLong || kN == kStates, "long blocks at 16 states");
    constexpr int LB = kLong ? G : L;         // block length as seen inside one group
    static_assert(kLong || G % L == 0, "block length must divide the token group");
    // Double buffers as distinct arrays (A / B), so that the compiler can tell
    // the loads in flight into one buffer from the reads of the other and
    // does not wait for them: [wave][stream x, dt, dy (, z)][token][channel]
    // and [B, C][token][state]
    __shared__ __attribute__((aligned(16))) uint32_t xdA[4][NSB][G][CW], xdB[4][NSB][G][CW];
    __shared__ __attribute__((aligned(16))) uint32_t bcA[2][G][kN], bcB[2][G][kN];
    __shared__ __attribute__((aligned(16))) float redA[4][G * 2 * kN], redB[4][G * 2 * kN];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform(threadIdx.x >> 6);
    const int cl = lane / P;                  // channel within the wave
    const int g = lane % P;                   // state pair
    const int s0 = 2 * g;
    const BlockPos pos = xcd_paired_block();   // (channel tile, chunk, batch row)
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

    float a2[2], ar[2], q[2];
    {
        const float2 av = *reinterpret_cast<const float2 *>(A + (int64_t)d * kN + s0);
        ar[0] = av.x; ar[1] = av.y;
        a2[0] = av.x * kLog2e; a2[1] = av.y * kLog2e;
        q[0] = q[1] = 0.f;
        if (!kBlockInit && qin != nullptr && t_end < T && live) {
            const float2 v = *reinterpret_cast<const float2 *>(
                qin + (int64_t)b * qin_bs + (int64_t)c * qin_cs + (int64_t)d * kN + s0);
            q[0] = v.x; q[1] = v.y;
        }
    }
    float dA_acc[2] = {0.f, 0.f};
    float dD_acc = 0.f;
    auto state_at = [&](const float *base, int64_t blk) -> float2 {
        return *reinterpret_cast<const float2 *>(base + (((int64_t)b * (nbl + 1) + blk) * D + d) * kN + s0);
    };
    if (kBlockInit && dh0 != nullptr && t_end == T && live)
        *reinterpret_cast<float2 *>(dh0 + (((int64_t)b * (nbl + 1) + nbl) * D + d) * kN + s0) =
            make_float2(0.f, 0.f);

    // after the per-token channel sums: lane l holds dB (bit 5 clear) or dC of
    // state 2g + (bit 4) of its state pair g, i.e. entry bc_idx of the
    // token's 2 kN (dB by state, then dC)
    const int bc_idx = ((lane >> 5) ? kN : 0) + s0 + ((lane >> 4) & 1);
    // 16 states: a token pair's sums, lanes with bit 3 clear holding token
    // i + 1 and the others token i
    const bool b3 = (lane & 8) != 0;
    const int red_lane = (P == 8 && !b3 ? 2 * kN : 0) + bc_idx;
    // below 16 states the sums end duplicated over the lane bits 1 .. 3 below
    // the channel bits that the folds leave; one lane of each writes them
    constexpr int kDupMask = P == 4 ? 12 : P == 2 ? 14 : 0;
    // the dt / x sums of a TK-token segment: lane l holds token TK s + g % TK
    // of quantity g / TK (0: dt, 1: x) of its own channel cl
    const int o_tok = g % TK, o_q = g / TK;
    // Dskip dy enters the x sum once per channel, in lane g == 0
    const float dskg = (g == 0) ? Dskip[d] : 0.f;
    // the fused epilogue's lanes: tokens l / CW + P h (h < EV), channel l % CW
    const int o_ch = lane % CW;
    const bool o_live = d_w0 + o_ch < D;

    const int64_t first = (int64_t)b * T + t_begin;
    const Rows<Tin> xs(x + first * D, len, D, 0);
    const Rows<Tin> ds(dt + first * D, len, D, 0);
    const Rows<Tin> ys(dy + first * D, len, D, 0);
    __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Bm + first * kN)), 0, uniform(len * kN * ES), kRawBufferWord3);
    __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<Tin *>(Cm + first * kN)), 0, uniform(len * kN * ES), kRawBufferWord3);
    // DMA lanes: x / dt / dy load j covers tokens P j .. P j + P - 1 (lane:
    // token l / CW, channel l % CW); B / C load j (taken by wave j % 4) covers
    // tokens BT j .. (lane: token l / kN, state l % kN)
    const int ld_tok = lane / CW, ld_col = lane % CW;
    const bool ld_live = d_w0 + ld_col < D;
    const int ld_ch = ld_live ? d_w0 + ld_col : D - 1;
    const int bc_tok = lane / kN, bc_col = lane % kN;
    const bool gate = kFuse && fz.z != nullptr;
    const bool sp_mode = kFuse && fz.dt_mode == kDtSoftplus;
    const float ld_bias = (kFuse && fz.dt_bias != nullptr) ? fz.dt_bias[ld_ch] : 0.f;
    const Rows<Tin> zs((gate ? fz.z : dy) + first * D, len, D, 0);
    float bias_acc = 0.f;                     // this lane's share of the dt-stream gradient sum
    const float dsk = kFuse ? Dskip[d] : 0.f;
    // the fused epilogue's outputs (no gate: an empty range, every store dropped)
    const Rows<Tin> dts(ddt + first * D, len, D, 0);
    const Rows<Tin> dzs(gate ? fz.dz + first * D : ddt, gate ? len : 0, D, 0);

    // dt and dy of tokens past the chunk end and of channels past D are read
    // at an offset beyond the buffer's range, which returns zero: such tokens
    // decay by 1 and inject nothing, and dead channels form no gradient terms
    auto issue = [&](auto &xd, auto &bc, int k0) {
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int kr = k0 + P * j + ld_tok;
            const int k = kr < len ? kr : len - 1;
            const int zoff = (kr < len && ld_live) ? ld_ch * ES + k * ds.pitch : kOutOfRange;
            load_to_lds<ES>(xs.rsrc, &xd[w][0][P * j][0], ld_ch * ES + k * xs.pitch, 0);
            load_to_lds<ES>(ds.rsrc, &xd[w][1][P * j][0], zoff, 0);
            load_to_lds<ES>(ys.rsrc, &xd[w][2][P * j][0], zoff, 0);
            if constexpr (kFuse) {
                if (gate) load_to_lds<ES>(zs.rsrc, &xd[w][NSB - 1][P * j][0], zoff, 0);
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
    // loaded to fp32 in place (bf16 only)
    auto widen = [&](auto &xd, auto &bc) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if constexpr (ES == 2) {
#pragma unroll
            for (int s = 0; s < NSB; ++s)
#pragma unroll
                for (int j = 0; j < XL; ++j) {
                    if (s == 3 && !gate) continue;
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
            // the step size of the forward, and the gate's two factors of dy
#pragma unroll
            for (int j = 0; j < XL; ++j) {
                uint32_t &dv = (&xd[w][1][P * j][0])[lane];
                const float raw = __uint_as_float(dv);
                float dl = raw;
                if (fz.dt_mode == kDtSoftplus) dl = step_size<kDtSoftplus>(raw, ld_bias);
                else if (fz.dt_mode == kDtBias) dl = step_size<kDtBias>(raw, ld_bias);
                dv = __float_as_uint(dl);
                if (gate) {
                    uint32_t &yv = (&xd[w][2][P * j][0])[lane];
                    uint32_t &zv = (&xd[w][3][P * j][0])[lane];
                    const float zf = __uint_as_float(zv), gy = __uint_as_float(yv);
                    const float sg = __builtin_amdgcn_rcpf(1.f + fast_exp2(-zf * kLog2e));
                    yv = __float_as_uint(gy * (zf * sg));                         // dy silu(z)
                    zv = __float_as_uint(gy * (sg * __builtin_fmaf(zf, 1.f - sg, 1.f)));   // dy silu'(z)
                }
            }
        }
    };
    auto f32 = [](uint32_t v) { return __uint_as_float(v); };

    float *pbc = part_bc + ((int64_t)b * gridDim.x + pos.tile) * T * (2 * kN);
    Tin *dxw = dx + first * D;
    Tin *dtw = ddt + first * D;

    constexpr int NB = G / LB;                // blocks per group (1 for kLong)
    constexpr int NH = kLong ? 2 : (kBlockInit ? NB : 1);   // group-start values
    constexpr int ND = kLong ? 1 : (kBlockInit ? 1 : NB);   // d_bounds entries
    float hrc[2] = {0.f, 0.f};                // kLong: the reverse state carried between groups
    // hst: forward state at the group start (two-stream form: at each block
    // start of the group); dbd: dbounds at each block end of the group
    // (continuous form; zero past the chunk end or without dbounds)
    auto group = [&](auto &xd, auto &bc, auto &red, int k0, const float2 *hst, const float2 *dbd) {
        const int nvalid = (len - k0 < G) ? len - k0 : G;   // uniform
        auto xval = [&](int i) { return f32(xd[w][0][i][cl]); };
        auto dval = [&](int i) { return f32(xd[w][1][i][cl]); };
        auto yval = [&](int i) { return f32(xd[w][2][i][cl]); };
        auto bcv = [&](int which, int i) {
            const uint2 v = *reinterpret_cast<const uint2 *>(&bc[which][i][s0]);
            return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
        };

        // pass A: forward state and reverse adjoint, left to right
        float hp_s[G][2], gr_s[G][2];
        // the decays of the group's last KA tokens, kept for pass B (which
        // takes those tokens first, so their registers free early); the rest
        // pass B forms again
        float a_s[KA > 0 ? KA : 1][2];
        float hf[2] = {hst[0].x, hst[0].y}, pr[2] = {0.f, 0.f};
        if constexpr (kLong) {
            pr[0] = hst[NH - 1].x; pr[1] = hst[NH - 1].y;
        }
        // kLong: whether this group starts / ends a block (uniform; chunks
        // are whole blocks, so the chunk's end ends one)
        const bool gsb = !kLong || k0 % Lb == 0;
        const bool geb = !kLong || (k0 + G) % Lb == 0 || k0 + G >= len;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if (i % LB == 0 && i != 0) {
                if constexpr (kBlockInit) {
                    hf[0] = hst[i / LB].x; hf[1] = hst[i / LB].y;
                }
                pr[0] = pr[1] = 0.f;
            }
            const float dl = dval(i), dxv = dl * xval(i), gy = yval(i);
            const float2 bv = bcv(0, i), cv = bcv(1, i);
            const float bb[2] = {bv.x, bv.y}, cc[2] = {cv.x, cv.y};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float a = fast_exp2(dl * a2[j]);
                if (i >= G - KA) a_s[i - (G - KA)][j] = a;
                const float gr_j = __builtin_fmaf(gy, cc[j], pr[j]);
                hp_s[i][j] = hf[j];
                gr_s[i][j] = gr_j;
                hf[j] = __builtin_fmaf(a, hf[j], dxv * bb[j]);
                pr[j] = a * gr_j;
            }
            // 4-token batches: the batch's arithmetic completes before the
            // next batch's rows are read (register pressure)
            if ((i & 3) == 3)
                asm volatile("" : "+v"(hf[0]), "+v"(hf[1]), "+v"(pr[0]), "+v"(pr[1]), "+v"(gr_s[i][0]),
                             "+v"(gr_s[i][1]), "+v"(gr_s[i - 1][0]), "+v"(gr_s[i - 1][1]), "+v"(gr_s[i - 2][0]),
                             "+v"(gr_s[i - 2][1]), "+v"(gr_s[i - 3][0]), "+v"(gr_s[i - 3][1]) :: "memory");
        }

        // read the token rows again in pass B rather than keeping pass A's
        // values live across the group
        asm volatile("" ::: "memory");
        // pass B: reverse state and forward adjoint, right to left
        float hr[2] = {0.f, 0.f};
        if constexpr (kLong) {
            hr[0] = hrc[0]; hr[1] = hrc[1];
        }
        float tsum = 0.f;                     // this lane's token of the current 4-token segment
        float s16_next = 0.f;                 // the 16-lane fold of token i + 1 (i even)
#pragma unroll
        for (int i = G - 1; i >= 0; --i) {
            if ((i + 1) % LB == 0 && geb) {
                hr[0] = hr[1] = 0.f;
                if constexpr (kBlockInit) {
                    q[0] = q[1] = 0.f;
                } else {
                    q[0] += dbd[i / LB].x; q[1] += dbd[i / LB].y;
                }
            }
            const float xv = xval(i), dl = dval(i), gy = yval(i);
            const float dxv = dl * xv;
            const float2 bv = bcv(0, i), cv = bcv(1, i);
            const float bb[2] = {bv.x, bv.y}, cc[2] = {cv.x, cv.y};
            float s1 = 0.f, s2 = 0.f, vb[2], vc[2], yp = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float a = (i >= G - KA) ? a_s[i - (G - KA)][j] : fast_exp2(dl * a2[j]);
                const float u = dxv * bb[j];
                const float hr1 = hr[j];
                hr[j] = __builtin_fmaf(a, hr1, u);
                const float gf = __builtin_fmaf(gy, cc[j], q[j]);
                const float du = gf + gr_s[i][j];
                const float da = __builtin_fmaf(gf, hp_s[i][j], gr_s[i][j] * hr1);
                q[j] = a * gf;
                s1 = __builtin_fmaf(du, bb[j], s1);
                const float daa = da * a;
                s2 = __builtin_fmaf(daa, ar[j], s2);
                dA_acc[j] = __builtin_fmaf(daa, dl, dA_acc[j]);
                // forward state after token i: kept as the state before token
                // i + 1, except where the two-stream form restarts a block
                const float hf_t = (i == G - 1) ? hf[j]
                                   : (kBlockInit && (i + 1) % LB == 0) ? __builtin_fmaf(a, hp_s[i][j], u)
                                                                      : hp_s[i + 1][j];
                vb[j] = du * dxv;                     // dB
                vc[j] = gy * (hf_t + hr[j]);          // dC
                if constexpr (kFuse) yp = __builtin_fmaf(cc[j], hf_t + hr[j], yp);
            }
            dD_acc = __builtin_fmaf(gy, xv, dD_acc);   // every lane; lane g == 0's total is stored
            if constexpr (kFuse) {
                // y_pre of the token: the lane's C (hf + hr) summed over the
                // channel's P state pairs (quad exchanges, then the half-row
                // mirror or the row rotations by 4 and 8), + Dskip x, into the
                // token's x slot (pass B is done with it)
                yp += dpp_perm<kDppXor1>(yp);
                if constexpr (P >= 4) yp += dpp_perm<kDppXor2>(yp);
                if constexpr (P == 8) yp += dpp_perm<kDppHalfMirror>(yp);
                if constexpr (P == 16) {
                    yp += dpp_perm<kDppRor4>(yp);
                    yp += dpp_perm<kDppRor8>(yp);
                }
                xd[w][0][i][cl] = __float_as_uint(__builtin_fmaf(dsk, xv, yp));
            }
            if constexpr (kBlockInit) {
                if (i % LB == 0 && gsb && dh0 != nullptr && i < nvalid && live) {
                    const int64_t blk = kLong ? t_begin / Lb + k0 / Lb : (t_begin + k0 + i) / LB;
                    *reinterpret_cast<float2 *>(dh0 + (((int64_t)b * (nbl + 1) + blk) * D + d) * kN + s0) =
                        make_float2(q[0], q[1]);
                }
            }
            // dB / dC of the token summed over the wave's CW channels (lanes
            // g, g + P, ...): the 32-lane folds sum lane bit 5, the 16-lane
            // fold bit 4, which completes the sum at 32 states.  At 16 states
            // the last channel bit (3, a row rotation by 8) takes two tokens
            // at once, lanes with bit 3 clear keeping token i + 1 and the
            // others token i, so that all 64 lanes store a distinct sum;
            // below, the channel bits left (3 and 2, and 1) are summed by row
            // rotations (and a quad exchange) and one lane of each duplicate
            // stores.  The sums meet the other waves' in red.
            {
                const float f0 = fold32(vb[0], vc[0]);
                const float f1 = fold32(vb[1], vc[1]);
                float s16 = fold16(f0, f1);
                if constexpr (P == 16) {
                    red[w][i * 2 * kN + red_lane] = s16;
                } else if constexpr (P == 8) {
                    if (i & 1) {
                        s16_next = s16;
                    } else {
                        float keep = b3 ? s16 : s16_next;
                        const float snd = b3 ? s16_next : s16;
                        keep += xchg8(snd);
                        red[w][i * 2 * kN + red_lane] = keep;
                    }
                } else {
                    if constexpr (P == 2) s16 += dpp_perm<kDppXor2>(s16);
                    s16 += dpp_perm<kDppRor4>(s16);
                    s16 += dpp_perm<kDppRor8>(s16);
                    if ((lane & kDupMask) == 0) red[w][i * 2 * kN + red_lane] = s16;
                }
            }
            // dt and x partials of the token summed over the channel's P state
            // pairs: an exchange over the top bit of g (row rotation by 8,
            // half-row mirror, or a quad exchange) leaves the dt sum's pairs in
            // lanes g < TK and the x sum's in lanes g >= TK, exchanges over
            // the lower bits complete them; lane g keeps token i where
            // g % TK == i % TK
            {
                const float pa = __builtin_fmaf(xv, s1, s2);
                const float pb = __builtin_fmaf(dskg, gy, dl * s1);
                float v = o_q ? pb : pa;
                const float snd = o_q ? pa : pb;
                if constexpr (P == 16) v += dpp_perm<kDppRor8>(snd);
                else if constexpr (P == 8) v += dpp_perm<kDppHalfMirror>(snd);
                else if constexpr (P == 4) v += dpp_perm<kDppXor2>(snd);
                else v += dpp_perm<kDppXor1>(snd);
                if constexpr (P >= 4) v += dpp_perm<kDppXor1>(v);
                if constexpr (P >= 8) v += dpp_perm<kDppXor2>(v);
                if constexpr (P == 16) v += dpp_perm<kDppHalfMirror>(v);
                if (o_tok == i % TK) tsum = v;
            }
            if ((i & 3) == 0)
                asm volatile("" : "+v"(hr[0]), "+v"(hr[1]), "+v"(q[0]), "+v"(q[1]), "+v"(dA_acc[0]),
                             "+v"(dA_acc[1]), "+v"(tsum), "+v"(dD_acc) :: "memory");
            if (i % TK == 0) {
                const int it = i + o_tok;
                if constexpr (kFuse) {
                    // dx is final here; the dt-stream gradient before the
                    // softplus factor goes to the token's dy slot for the
                    // group's epilogue
                    if (o_q) {
                        if (live && it < nvalid) dxw[(int64_t)(k0 + it) * D + d] = narrow<Tin>(tsum);
                    } else {
                        xd[w][2][it][cl] = __float_as_uint(tsum);
                    }
                } else {
                    if (live && it < nvalid) (o_q ? dxw : dtw)[(int64_t)(k0 + it) * D + d] = narrow<Tin>(tsum);
                }
            }
        }
        if constexpr (kLong) {
            hrc[0] = hr[0]; hrc[1] = hr[1];
        }
        if constexpr (kFuse) {
            // epilogue of the group: lane (tokens l / CW + P h, channel l % CW)
            // applies softplus'(v) = s(v) to the dt-stream gradient, adds it
            // to the bias sum and stores it, and stores dz = dy silu'(z) y_pre
#pragma unroll
            for (int h = 0; h < EV; ++h) {
                const int t = lane / CW + P * h;
                const bool ok = o_live && t < nvalid;
                // stores of dead channels and tokens past the group go to an
                // offset beyond the buffer's range, which drops them
                const int32_t off = ok ? (k0 + t) * dts.pitch + (d_w0 + o_ch) * ES : kOutOfRange;
                float gdt = f32(xd[w][2][t][o_ch]);
                if (sp_mode) gdt *= sigmoid_from_softplus(f32(xd[w][1][t][o_ch]));
                bias_acc += ok ? gdt : 0.f;
                dts.store_at(off, narrow<Tin>(gdt));
                dzs.store_at(off, narrow<Tin>(f32(xd[w][3][t][o_ch]) * f32(xd[w][0][t][o_ch])));
            }
        }
    };

    // The global loads of a group (its start states, its d_bounds entries)
    // are issued one group ahead, together with that group's rows, so that
    // the wait for the rows at the end of the previous group covers them (the
    // vector-memory counter is in order: a wait for them placed after a later
    // DMA would wait for the DMA as well).
    float2 hstn[NH], dbdn[ND];
    auto load_group = [&](int k0n) {
        const int nv = (len - k0n < G) ? len - k0n : G;
        if constexpr (kLong) {
            // a block's first group starts from the block state and a zero
            // reverse adjoint, the others from the group-state pre-pass
            if (k0n % Lb == 0) {
                hstn[0] = state_at(h_start, t_begin / Lb + k0n / Lb);
                hstn[1] = make_float2(0.f, 0.f);
            } else {
                const int64_t ng = (T + G - 1) / G;
                const float *gs = gstate + ((((int64_t)b * ng + (t_begin + k0n) / G) * 2) * D + d) * kStates + s0;
                hstn[0] = *reinterpret_cast<const float2 *>(gs);
                const float2 v = *reinterpret_cast<const float2 *>(gs + (int64_t)D * kStates);
                // a dead channel carries no adjoint (its step size need not be
                // zero under the softplus transform, so it would reach dB)
                hstn[1] = live ? v : make_float2(0.f, 0.f);
            }
            dbdn[0] = make_float2(0.f, 0.f);
            if (!kBlockInit && dbounds != nullptr && (k0n + G) % Lb == 0 && k0n + G <= len) {
                const float2 v = state_at(dbounds, t_begin / Lb + (k0n + G) / Lb);
                if (live) dbdn[0] = v;
            }
        } else if constexpr (kBlockInit) {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int ib = k * L < nv ? k * L : 0;
                hstn[k] = state_at(h_start, (t_begin + k0n + ib) / L);
            }
            dbdn[0] = make_float2(0.f, 0.f);
        } else {
            hstn[0] = state_at(h_start, (t_begin + k0n) / L);
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int ie = k * L + L - 1;          // the block's last token
                dbdn[k] = make_float2(0.f, 0.f);
                if (dbounds != nullptr && ie < nv) {
                    const float2 v = state_at(dbounds, (t_begin + k0n + ie + 1) / L);
                    if (live) dbdn[k] = v;
                }
            }
        }
    };
    // one group: the next group's loads go out first, then this group's
    // passes; after the barrier the four waves' dB / dC sums of the group are
    // added in a fixed order
    auto step = [&](auto &xd, auto &bc, auto &red, auto &xdn, auto &bcn, int k0) {
        const bool more = k0 > 0;
        float2 hst[NH], dbd[ND];
#pragma unroll
        for (int k = 0; k < NH; ++k) hst[k] = hstn[k];
#pragma unroll
        for (int k = 0; k < ND; ++k) dbd[k] = dbdn[k];
        if (more) {
            load_group(k0 - G);
            issue(xdn, bcn, k0 - G);
        }
        group(xd, bc, red, k0, hst, dbd);
        if (more) widen(xdn, bcn);
        __syncthreads();
        const int nvalid = (len - k0 < G) ? len - k0 : G;
        constexpr int NR = G * 2 * kN;        // the group's sums, NR / 256 or fewer per thread
#pragma unroll
        for (int h = 0; h < (NR + 4 * kWave - 1) / (4 * kWave); ++h) {
            const int o = threadIdx.x + h * 4 * kWave;
            if (NR % (4 * kWave) == 0 || o < NR) {
                const float v = ((red[0][o] + red[1][o]) + red[2][o]) + red[3][o];
                if (o / (2 * kN) < nvalid) pbc[(t_begin + k0) * (2 * kN) + o] = v;
            }
        }
    };
    const int k_last = ((len - 1) / G) * G;
    load_group(k_last);
    issue(xdA, bcA, k_last);
    widen(xdA, bcA);
    __syncthreads();
    for (int k0 = k_last; k0 >= 0; k0 -= 2 * G) {
        step(xdA, bcA, redA, xdB, bcB, k0);
        if (k0 - G >= 0) step(xdB, bcB, redB, xdA, bcA, k0 - G);
    }

    // continuous form: gradient of the start state (chunk 0)
    if (!kBlockInit && c == 0 && dh0 != nullptr && live) {
        float v0 = q[0], v1 = q[1];
        if (dbounds != nullptr) {
            const float2 e = state_at(dbounds, 0);
            v0 += e.x; v1 += e.y;
        }
        *reinterpret_cast<float2 *>(dh0 + ((int64_t)b * D + d) * kN + s0) = make_float2(v0, v1);
    }
    // dA and dDskip partials of this (batch, chunk)
    if (live) {
        const int64_t pc = (int64_t)b * gridDim.y + c;
        *reinterpret_cast<float2 *>(part_a + (pc * D + d) * kN + s0) = make_float2(dA_acc[0], dA_acc[1]);
        if (g == 0) part_d[pc * D + d] = dD_acc;
    }
    if constexpr (kFuse) {
        // the dt-stream gradient summed over the chunk: the token lanes of
        // each output channel (lanes ch, ch + CW, ...: the lane bits from
        // log2 CW up), in a fixed order
        if constexpr (CW <= 4) {
            bias_acc += dpp_perm<kDppRor4>(bias_acc);
            bias_acc += dpp_perm<kDppRor8>(bias_acc);
        } else if constexpr (CW == 8) {
            bias_acc += xchg8(bias_acc);
        }
        if constexpr (CW <= 16) bias_acc = fold16(bias_acc, bias_acc);
        bias_acc = fold32(bias_acc, bias_acc);
        if (fz.part_bias != nullptr && lane < CW && o_live)
            fz.part_bias[((int64_t)b * gridDim.y + c) * D + d_w0 + lane] = bias_acc;
    }
}

// ------------------------------------------------------------------------
// The general backward: block lengths outside {1, 2, 4, 8, 16} (up to
// kMaxLdsBlock) and state counts other than 16, the gradients of bwd_pair_kernel.

// Chunk-local adjoint for kN states and any block length L (adjoint_chunk_kernel's
// job).  Chunks are whole blocks, so the chunk's last row ends a block; block
// ends are counted from the right end.  grid = (ceil(D/64), chunks launched,
// batch), block = 64; chunk c = c_first + blockIdx.y.
template <typename Tin, int kN, int kDt = kDtPlain>
__global__ __launch_bounds__(kWave) void adjoint_general_kernel(
    const Tin *__restrict__ dt, const Tin *__restrict__ dy, const Tin *__restrict__ Cm,
    const float *__restrict__ A, const float *__restrict__ dbounds, float *__restrict__ qout,
    float *__restrict__ sout, int64_t T, int D, int L, int64_t Tc, int n_chunks, int c_first,
    const float *__restrict__ dt_bias, const Tin *__restrict__ z)
{
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = c_first + blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);
    const int64_t nbl = T / L;
    const int64_t blk0 = t_begin / L;

    float a2[kN], q[kN];
    load_row<kN>(A + (int64_t)d * kN, a2);
#pragma unroll
    for (int n = 0; n < kN; ++n) { a2[n] *= kLog2e; q[n] = 0.f; }
    float S = 0.f;
    const int64_t first = (int64_t)b * T + t_begin;
    const Rows<Tin> ds(dt + first * D, len, D, d);
    const Rows<Tin> ys(dy + first * D, len, D, d);
    const bool gate = z != nullptr;
    const Rows<Tin> zs((gate ? z : dy) + first * D, len, D, d);
    const float bias = (kDt != kDtPlain && dt_bias != nullptr) ? dt_bias[d] : 0.f;
    const Tin *cs = Cm + first * kN;
    // Tokens stream through registers in stages of U as in adjoint_chunk_kernel
    // (two named 32-bit buffers, the loop unrolled by two).
    constexpr int U = 4;
    using St = typename Staged<Tin>::type;
    int kb = 0;                                   // rows walked since the last block end
    auto consume = [&](const St *dr, const St *yr, int k0, int count) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (i < count) {
                const int p = len - 1 - (k0 + i);        // row within the chunk
                if (dbounds != nullptr && kb == 0) {
                    float v[kN];
                    load_row<kN>(dbounds + (((int64_t)b * (nbl + 1) + blk0 + (p + 1) / L) * D + d) * kN, v);
#pragma unroll
                    for (int n = 0; n < kN; ++n) q[n] += v[n];
                }
                const float dl = step_size<kDt>(widen_staged(dr[i]), bias);
                float gy = live ? widen_staged(yr[i]) : 0.f;
                if (gate) gy *= silu_f(widen(zs.load(p)));
                S += dl;
                const Tin *crow = cs + (int64_t)p * kN;
#pragma unroll
                for (int k = 0; k < kN / 2; ++k) {
                    float c0, c1;
                    load_pair(crow, k, c0, c1);
                    q[2 * k] = fast_exp2(dl * a2[2 * k]) * __builtin_fmaf(gy, c0, q[2 * k]);
                    q[2 * k + 1] = fast_exp2(dl * a2[2 * k + 1]) * __builtin_fmaf(gy, c1, q[2 * k + 1]);
                }
                kb = (kb + 1 == L) ? 0 : kb + 1;
            }
        }
    };
    // count < U: the rows past the stage re-read its last row
    auto load_stage = [&](int k0, int count, St *dout, St *yo) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int p = len - 1 - (k0 + (i < count ? i : count - 1));
            dout[i] = ds.load(p);
            yo[i] = ys.load(p);
        }
    };
    const int n_full = len / U;
    const int rem = len - n_full * U;
    St da[U], ya[U], db[U], yb[U];
    if (n_full > 0) load_stage(0, U, da, ya);
    int g = 0;
    for (; g + 1 < n_full; g += 2) {
        load_stage((g + 1) * U, U, db, yb);
        consume(da, ya, g * U, U);
        if (g + 2 < n_full) load_stage((g + 2) * U, U, da, ya);
        consume(db, yb, (g + 1) * U, U);
    }
    if (g < n_full) consume(da, ya, g * U, U);       // an odd number of full stages: the last is in da
    if (rem > 0) {
        load_stage(n_full * U, rem, db, yb);
        consume(db, yb, n_full * U, rem);
    }
    if (live) {
        store_row<kN>(qout + (((int64_t)b * n_chunks + c) * D + d) * kN, q);
        sout[((int64_t)b * n_chunks + c) * D + d] = S;
    }
}

// Group states for bwd_pair_kernel's long blocks (block lengths that are
// multiples of 16 above 16, 16 states): the forward state and the reverse
// adjoint's carry (a * gr, the adjoint of the in-block reverse recurrence,
// which runs left to right from zero at the block start) at every 16-token
// group start that lies inside a block, not at its start, into gstate
// [batch, ceil(T/16), 2, D, 16] (entries at block starts are not written).
// Walks each block from its start state up to its last group start, with the
// pair kernel's pass-A recurrences.  One lane per channel, the 16 states in
// registers; grid = (ceil(D/64), min(blocks, 65535), batch), block = 64.
template <typename Tin, int kDt>
__global__ __launch_bounds__(kWave) void group_state_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const Tin *__restrict__ dy, const float *__restrict__ A,
    const float *__restrict__ h_start, float *__restrict__ gstate, int64_t T, int D, int L,
    const float *__restrict__ dt_bias, const Tin *__restrict__ z)
{
    constexpr int G = kGroup;
    constexpr int U = 4;                      // tokens per pipeline stage (divides G)
    using St = typename Staged<Tin>::type;
    const int lane = threadIdx.x;
    const int d_raw = blockIdx.x * kWave + lane;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int b = blockIdx.z;
    const int64_t nbl = T / L, nbt = (T + L - 1) / L, ng = (T + G - 1) / G;
    float a2[kStates];
    load_row<kStates>(A + (int64_t)d * kStates, a2);
#pragma unroll
    for (int n = 0; n < kStates; ++n) a2[n] *= kLog2e;
    const bool gate = z != nullptr;
    const float bias = (kDt != kDtPlain && dt_bias != nullptr) ? dt_bias[d] : 0.f;
    const int64_t row0 = (int64_t)b * T;
    for (int64_t blk = blockIdx.y; blk < nbt; blk += gridDim.y) {
        const int64_t t0 = blk * L;
        const int64_t pend = (t0 + L < T) ? t0 + L : T;
        if (t0 + G >= pend) continue;                  // one group: nothing to hand over
        float hf[kStates], pr[kStates];
        load_row<kStates>(h_start + (((int64_t)b * (nbl + 1) + blk) * D + d) * kStates, hf);
#pragma unroll
        for (int n = 0; n < kStates; ++n) pr[n] = 0.f;
        // the tokens before the block's last group (a multiple of 16), through
        // a register pipeline of U-token stages (two named 32-bit buffers, the
        // loop unrolled by two, as in chunk_state_kernel)
        const int nwalk = (int)(((pend - t0 - 1) / G) * G);
        const int64_t first = row0 + t0;
        const Rows<Tin> xs(x + first * D, nwalk, D, d);
        const Rows<Tin> ds(dt + first * D, nwalk, D, d);
        const Rows<Tin> ys(dy + first * D, nwalk, D, d);
        const Rows<Tin> zs((gate ? z : dy) + first * D, nwalk, D, d);
        const Tin *bs = Bm + first * kStates, *cs = Cm + first * kStates;
        auto consume = [&](const St *xr, const St *dr, const St *yr, int k0) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int k = k0 + i;
                const float dl = step_size<kDt>(widen_staged(dr[i]), bias);
                const float dxv = dl * widen_staged(xr[i]);
                float gy = widen_staged(yr[i]);
                if (gate) gy *= silu_f(widen(zs.load(k)));
                const Tin *brow = bs + (int64_t)k * kStates, *crow = cs + (int64_t)k * kStates;
#pragma unroll
                for (int q = 0; q < kStates / 2; ++q) {
                    float b0, b1, c0, c1;
                    load_pair(brow, q, b0, b1);
                    load_pair(crow, q, c0, c1);
                    const float bb[2] = {b0, b1}, cc[2] = {c0, c1};
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int n = 2 * q + j;
                        const float a = fast_exp2(dl * a2[n]);
                        const float gr = __builtin_fmaf(gy, cc[j], pr[n]);
                        hf[n] = __builtin_fmaf(a, hf[n], dxv * bb[j]);
                        pr[n] = a * gr;
                    }
                }
                // after each group: the state at the next group's start
                if ((k + 1) % G == 0 && live) {
                    float *o = gstate + ((((int64_t)b * ng + (t0 + k + 1) / G) * 2) * D + d) * kStates;
                    store_row<kStates>(o, hf);
                    store_row<kStates>(o + (int64_t)D * kStates, pr);
                }
            }
        };
        auto load_stage = [&](int k0, St *xo, St *dout, St *yo) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                xo[i] = xs.load(k0 + i);
                dout[i] = ds.load(k0 + i);
                yo[i] = ys.load(k0 + i);
            }
        };
        const int nst = nwalk / U;                 // G is a multiple of U: whole stages
        St xa[U], da[U], ya[U], xb[U], db[U], yb[U];
        load_stage(0, xa, da, ya);
        int g = 0;
        for (; g + 1 < nst; g += 2) {
            load_stage((g + 1) * U, xb, db, yb);
            consume(xa, da, ya, g * U);
            if (g + 2 < nst) load_stage((g + 2) * U, xa, da, ya);
            consume(xb, db, yb, (g + 1) * U);
        }
        if (g < nst) consume(xa, da, ya, g * U);
    }
}

// v summed with the lane v ^ kMask holds (all lanes active)
template <int kMask> __device__ __forceinline__ float xor_add(float v, int lane) {
    if constexpr (kMask == 1)
        return v + dpp_perm<kDppXor1>(v);
    else if constexpr (kMask == 2)
        return v + dpp_perm<kDppXor2>(v);
    else if constexpr (kMask == 4) return v + xchg4(v);
    else if constexpr (kMask == 8) return v + xchg8(v);
    else if constexpr (kMask == 16) return fold16(v, v);
    else return fold32(v, v);
}
// butterfly sum over the lane-index bits kFrom, 2 kFrom, ... below kTo
template <int kFrom, int kTo> __device__ __forceinline__ float lane_sum(float v, int lane) {
    if constexpr (kFrom >= kTo) {
        return v;
    } else if constexpr (kFrom == 4 && kTo >= 16) {
        // bits 2 and 3 together: row rotations by 4 and 8 add up the four
        // lanes of a 16-lane row that agree in bits 0 and 1
        v += dpp_perm<kDppRor4>(v);
        v += dpp_perm<kDppRor8>(v);
        return lane_sum<16, kTo>(v, lane);
    } else {
        return lane_sum<2 * kFrom, kTo>(xor_add<kFrom>(v, lane), lane);
    }
}

// The sum over each aligned group of kN lanes, in every lane of the group,
// with DPP alone for kN <= 16 (no LDS-pipe swizzles): quad exchanges, then
// half-row mirror (kN = 8) or row rotations by 4 and 8 (kN = 16: after the
// quad sums, rotating a 16-lane row by 4 and then 8 adds up its four quads).
template <int kN> __device__ __forceinline__ float group_sum(float v, int lane) {
    v += dpp_perm<kDppXor1>(v);
    if constexpr (kN >= 4) v += dpp_perm<kDppXor2>(v);
    if constexpr (kN == 8) v += dpp_perm<kDppHalfMirror>(v);
    if constexpr (kN >= 16) {
        v += dpp_perm<kDppRor4>(v);
        v += dpp_perm<kDppRor8>(v);
    }
    if constexpr (kN >= 32) v = fold16(v, v);
    (void)lane;
    return v;
}

// Block-local backward of the general path, one lane per (channel, state):
// lane = kN cl + n, CW = 64 / kN channels per wave, NW waves per workgroup.
// Each block of the chunk (right to left) is walked twice: left to right for
// hf and the reverse adjoint gr, keeping both at every 16-token segment start
// (LDS, dynamic size NW / 2 KB per segment), then segment by segment right to
// left: the segment's hf before each token and gr are formed again from its
// checkpoint into registers, and the right-to-left walk runs hr and the
// forward adjoint with every gradient term, as in bwd_pair_kernel.  The
// token rows of a segment are staged in LDS (x, dt, dy per wave, B and C
// shared by the workgroup; widened, the step size and the gate's factors
// formed once per element).  Sums: over the channel's kN lanes by butterfly
// (dt, x, and y_pre for the gate), over the wave's channels by butterfly and
// over the NW waves in LDS (dB, dC: part_bc [batch, ceil(D / (NW CW)), T,
// 2 kN]).  Arguments as in bwd_pair_kernel.
// kFuse: 0 plain, 1 the fusions (BwdFuse), 2 the fusions and separate reverse
// operands: the reverse recurrence and its adjoint run on dt_r (own bias),
// B_r, C_r, A_r, and every gradient term splits by direction (the reverse
// operands' gradients go to ddt_r and the _r partials); two waves per
// workgroup keep its LDS below 64 KB at kN = 32 and L = 256.
// grid = (ceil(D / (NW CW)), chunks, batch), block = 64 NW.
template <int kFuse> constexpr int bwd_general_waves() { return kFuse == 2 ? 2 : 4; }
// At 32 states the registers are held to 128 (four waves per SIMD; some
// spills): measured 17% faster at the 87M shape.  At 4 and 8 states the same
// bound spills the token loop and is slower, so they keep three.

template <typename Tin, int kN, bool kBlockInit, int kFuse>
__global__ __launch_bounds__(bwd_general_waves<kFuse>() * kWave) __attribute__((amdgpu_waves_per_eu(kN == 32 ? 4 : 1))) void bwd_general_kernel(
    const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ Bm,
    const Tin *__restrict__ Cm, const Tin *__restrict__ dy, const float *__restrict__ A,
    const float *__restrict__ Dskip, const float *__restrict__ h_start, const float *qin,
    int64_t qin_bs, int64_t qin_cs, const float *__restrict__ dbounds, Tin *__restrict__ dx,
    Tin *__restrict__ ddt, float *__restrict__ part_bc, float *__restrict__ part_a,
    float *__restrict__ part_d, float *__restrict__ dh0, int64_t T, int D, int L, int64_t Tc,
    BwdFuse<Tin> fz)
{
    constexpr int NW = bwd_general_waves<kFuse>();
    constexpr bool kSep = kFuse == 2;
    constexpr int NR = kSep ? 2 : 1;          // B / C row sets: forward (, reverse)
    constexpr int CW = kWave / kN;            // channels per wave
    constexpr int G = 16;                     // segment length
    constexpr int ES = sizeof(Tin);
    constexpr int NE = (G * CW + kWave - 1) / kWave;   // token-row elements per lane per stream
    __shared__ float tx[NW][G][CW], tdl[NW][G][CW], tgy[NW][G][CW], tzv[NW][G][CW], tdr[NW][kSep ? G : 1][CW];
    __shared__ float tb[NR][G][kN], tc[NR][G][kN];   // B / C rows, shared by the waves
    __shared__ float red[NR][NW][G][2 * kN];
    extern __shared__ float ck[];             // [segments][NW waves][2][64]: hf, pr at segment starts

    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform(threadIdx.x >> 6);
    const int cl = lane / kN;
    const int n = lane % kN;
    const int d_w0 = blockIdx.x * NW * CW + w * CW;
    const int d_raw = d_w0 + cl;
    const bool live = d_raw < D;
    const int d = live ? d_raw : D - 1;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)c * Tc;
    const int64_t t_end = (t_begin + Tc < T) ? t_begin + Tc : T;
    const int len = (int)(t_end - t_begin);
    const int64_t nbl = T / L;
    const int nseg = (L + G - 1) / G;

    const float ar = A[(int64_t)d * kN + n];
    const float a2 = ar * kLog2e;
    const float arr = kSep ? fz.A_r[(int64_t)d * kN + n] : 0.f;
    const float a2r = arr * kLog2e;
    const float dsk = Dskip[d];
    float q = 0.f;
    if (!kBlockInit && qin != nullptr && t_end < T)
        q = qin[(int64_t)b * qin_bs + (int64_t)c * qin_cs + (int64_t)d * kN + n];
    float dA_acc = 0.f, dD_acc = 0.f, bias_acc = 0.f, dAr_acc = 0.f, bias_r_acc = 0.f;
    auto state_idx = [&](int64_t blk) { return (((int64_t)b * (nbl + 1) + blk) * D + d) * kN + n; };
    if (kBlockInit && dh0 != nullptr && t_end == T && live) dh0[state_idx(nbl)] = 0.f;

    const int64_t first = (int64_t)b * T + t_begin;
    const Rows<Tin> xs(x + first * D, len, D, 0);
    const Rows<Tin> dts(dt + first * D, len, D, 0);
    const Rows<Tin> ys(dy + first * D, len, D, 0);
    const bool gate = kFuse != 0 && fz.z != nullptr;
    const Rows<Tin> zs((gate ? fz.z : dy) + first * D, len, D, 0);
    const Rows<Tin> drs((kSep ? fz.dt_r : dt) + first * D, len, D, 0);
    const Rows<Tin> bs(Bm + first * kN, len, kN, 0);
    const Rows<Tin> cs(Cm + first * kN, len, kN, 0);
    const Rows<Tin> brs((kSep ? fz.B_r : Bm) + first * kN, len, kN, 0);
    const Rows<Tin> crs((kSep ? fz.C_r : Cm) + first * kN, len, kN, 0);
    const bool sp_mode = kFuse != 0 && fz.dt_mode == kDtSoftplus;
    auto step_of = [&](float raw, float bias, bool ok) -> float {
        if constexpr (kFuse != 0) {
            if (fz.dt_mode == kDtSoftplus) return ok ? step_size<kDtSoftplus>(raw, bias) : 0.f;
            if (fz.dt_mode == kDtBias) return ok ? step_size<kDtBias>(raw, bias) : 0.f;
        }
        return raw;
    };

    // stage the rows of tokens k0 .. k0 + cnt - 1 (chunk-local)
    auto stage = [&](int k0, int cnt) {
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            const int e = lane + kWave * j;
            if (e < G * CW) {
                const int i = e / CW, ch = e % CW;
                const bool ok = i < cnt && d_w0 + ch < D;
                const int32_t off = ok ? (d_w0 + ch) * ES + (k0 + i) * xs.pitch : kOutOfRange;
                const float xv = widen(xs.load_at(off));
                float dl = widen(dts.load_at(off));
                float gy = widen(ys.load_at(off));
                float zv = 0.f;
                if constexpr (kFuse != 0) {
                    dl = step_of(dl, (fz.dt_bias != nullptr && ok) ? fz.dt_bias[d_w0 + ch] : 0.f, ok);
                    if (gate) {
                        const float zf = widen(zs.load_at(off));
                        const float sg = __builtin_amdgcn_rcpf(1.f + fast_exp2(-zf * kLog2e));
                        zv = gy * (sg * __builtin_fmaf(zf, 1.f - sg, 1.f));     // dy silu'(z)
                        gy = gy * (zf * sg);                                     // dy silu(z)
                    }
                }
                if constexpr (kSep) {
                    tdr[w][i][ch] = step_of(widen(drs.load_at(off)),
                                            (fz.dt_bias_r != nullptr && ok) ? fz.dt_bias_r[d_w0 + ch] : 0.f, ok);
                }
                tx[w][i][ch] = xv;
                tdl[w][i][ch] = dl;
                tgy[w][i][ch] = gy;
                tzv[w][i][ch] = zv;
            }
        }
#pragma unroll
        for (int j = 0; j < (G * kN + NW * kWave - 1) / (NW * kWave); ++j) {
            const int e = threadIdx.x + NW * kWave * j;
            if (e < G * kN) {
                const int i = e / kN, col = e % kN;
                const int32_t off = i < cnt ? col * ES + (k0 + i) * bs.pitch : kOutOfRange;
                tb[0][i][col] = widen(bs.load_at(off));
                tc[0][i][col] = widen(cs.load_at(off));
                if constexpr (kSep) {
                    tb[NR - 1][i][col] = widen(brs.load_at(off));
                    tc[NR - 1][i][col] = widen(crs.load_at(off));
                }
            }
        }
        __syncthreads();                              // the shared B / C rows are complete
    };
    // the reverse recurrence's step and rows (the forward's without kSep)
    auto rdl = [&](int i) { return kSep ? tdr[w][i & (kSep ? G - 1 : 0)][cl] : tdl[w][i][cl]; };

    float *pbc = part_bc + ((int64_t)b * gridDim.x + blockIdx.x) * T * (2 * kN);
    float *pbcr = kSep ? fz.part_bc_r + ((int64_t)b * gridDim.x + blockIdx.x) * T * (2 * kN) : nullptr;
    float *ckw = ck + (int64_t)w * 2 * kWave;     // + seg * NW * 2 * 64

    for (int kb0 = len - L; kb0 >= 0; kb0 -= L) {            // blocks, right to left
        const int64_t blk = (t_begin + kb0) / L;
        // pass 1: hf and the reverse adjoint's carried pr = a_r gr, left to right
        float hf = h_start[state_idx(blk)];
        float pr = 0.f;
        for (int sg = 0; sg < nseg; ++sg) {
            const int k0 = kb0 + sg * G;
            const int cnt = (L - sg * G < G) ? L - sg * G : G;
            ckw[sg * NW * 2 * kWave + lane] = hf;
            ckw[sg * NW * 2 * kWave + kWave + lane] = pr;
            if (sg == nseg - 1) break;                      // the last segment is formed again in pass 2
            __syncthreads();                                 // every wave is done with the last rows
            stage(k0, cnt);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float dl = tdl[w][i][cl], xv = tx[w][i][cl], gy = tgy[w][i][cl];
                const float a = fast_exp2(dl * a2);
                const float a_r = kSep ? fast_exp2(rdl(i) * a2r) : a;
                const float grv = __builtin_fmaf(gy, tc[NR - 1][i][n], pr);
                hf = __builtin_fmaf(a, hf, dl * xv * tb[0][i][n]);
                pr = a_r * grv;
            }
            asm volatile("" ::: "memory");
        }
        // pass 2: segments right to left
        float hr = 0.f;
        if (kBlockInit) q = 0.f;
        else if (dbounds != nullptr) q += dbounds[state_idx(blk + 1)];
        for (int sg = nseg - 1; sg >= 0; --sg) {
            const int k0 = kb0 + sg * G;
            const int cnt = (L - sg * G < G) ? L - sg * G : G;
            __syncthreads();                                 // rows and red of the last segment consumed
            stage(k0, cnt);
            float hp[G], gs[G];
            float h = ckw[sg * NW * 2 * kWave + lane];
            float p2 = ckw[sg * NW * 2 * kWave + kWave + lane];
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float dl = tdl[w][i][cl], xv = tx[w][i][cl], gy = tgy[w][i][cl];
                const float a = fast_exp2(dl * a2);
                const float a_r = kSep ? fast_exp2(rdl(i) * a2r) : a;
                hp[i] = h;
                gs[i] = __builtin_fmaf(gy, tc[NR - 1][i][n], p2);
                h = __builtin_fmaf(a, h, dl * xv * tb[0][i][n]);
                p2 = a_r * gs[i];
            }
            // rows past cnt carry dt = 0, x = dy = 0: their decay is 1 and they
            // inject nothing, so h after the last row is the state after row cnt - 1
#pragma unroll
            for (int i = G - 1; i >= 0; --i) {
                if (i < cnt) {
                    const float dl = tdl[w][i][cl], xv = tx[w][i][cl], gy = tgy[w][i][cl];
                    const float bv = tb[0][i][n], cv = tc[0][i][n];
                    const float a = fast_exp2(dl * a2);
                    // the state after token i (rows past cnt leave it unchanged)
                    const float hf_t = (i == G - 1) ? h : hp[(i + 1) & (G - 1)];
                    const float gf = __builtin_fmaf(gy, cv, q);
                    float sdt_l, sx_l, yp_l, vb_l, vc_l, sdtr_l = 0.f, vbr_l = 0.f, vcr_l = 0.f;
                    if constexpr (kSep) {
                        const float dlr = rdl(i), bvr = tb[NR - 1][i][n], cvr = tc[NR - 1][i][n];
                        const float a_r = fast_exp2(dlr * a2r);
                        const float hr1 = hr;
                        hr = __builtin_fmaf(a_r, hr1, dlr * xv * bvr);
                        const float daa = gf * hp[i] * a;               // forward operands
                        dA_acc = __builtin_fmaf(daa, dl, dA_acc);
                        sdt_l = __builtin_fmaf(gf * bv, xv, daa * ar);
                        vb_l = gf * dl * xv;
                        vc_l = gy * hf_t;
                        const float daar = gs[i] * hr1 * a_r;           // reverse operands
                        dAr_acc = __builtin_fmaf(daar, dlr, dAr_acc);
                        sdtr_l = __builtin_fmaf(gs[i] * bvr, xv, daar * arr);
                        vbr_l = gs[i] * dlr * xv;
                        vcr_l = gy * hr;
                        sx_l = __builtin_fmaf(gf * bv, dl, gs[i] * bvr * dlr);
                        yp_l = __builtin_fmaf(cv, hf_t, cvr * hr);
                    } else {
                        const float u = dl * xv * bv;
                        const float hr1 = hr;
                        hr = __builtin_fmaf(a, hr1, u);
                        const float du = gf + gs[i];
                        const float daa = __builtin_fmaf(gf, hp[i], gs[i] * hr1) * a;
                        dA_acc = __builtin_fmaf(daa, dl, dA_acc);
                        const float hsum = hf_t + hr;
                        sdt_l = __builtin_fmaf(du * bv, xv, daa * ar);
                        sx_l = du * bv * dl;
                        yp_l = cv * hsum;
                        vb_l = du * dl * xv;
                        vc_l = gy * hsum;
                    }
                    q = a * gf;
                    // sums over the channel's kN lanes
                    float sdt = group_sum<kN>(sdt_l, lane);
                    const float sx = group_sum<kN>(sx_l, lane);
                    float yp = 0.f;
                    if constexpr (kFuse != 0) yp = group_sum<kN>(yp_l, lane);
                    float sdtr = 0.f;
                    if constexpr (kSep) sdtr = group_sum<kN>(sdtr_l, lane);
                    // dB, dC of the token: sums over the wave's channels
                    const float vb = lane_sum<kN, kWave>(vb_l, lane);
                    const float vc = lane_sum<kN, kWave>(vc_l, lane);
                    if (cl == 0) {
                        red[0][w][i][n] = vb;
                        red[0][w][i][kN + n] = vc;
                    }
                    if constexpr (kSep) {
                        const float vbr = lane_sum<kN, kWave>(vbr_l, lane);
                        const float vcr = lane_sum<kN, kWave>(vcr_l, lane);
                        if (cl == 0) {
                            red[NR - 1][w][i][n] = vbr;
                            red[NR - 1][w][i][kN + n] = vcr;
                        }
                    }
                    const int64_t row = (first + k0 + i) * D + d;
                    if (n == 0 && live) {
                        dD_acc = __builtin_fmaf(gy, xv, dD_acc);
                        dx[row] = narrow<Tin>(__builtin_fmaf(gy, dsk, sx));
                        if constexpr (kFuse != 0) {
                            if (sp_mode) sdt *= sigmoid_from_softplus(dl);
                            bias_acc += sdt;
                            if (gate) fz.dz[row] = narrow<Tin>(tzv[w][i][cl] * __builtin_fmaf(dsk, xv, yp));
                        }
                        if constexpr (kSep) {
                            if (sp_mode) sdtr *= sigmoid_from_softplus(rdl(i));
                            bias_r_acc += sdtr;
                            fz.ddt_r[row] = narrow<Tin>(sdtr);
                        }
                        ddt[row] = narrow<Tin>(sdt);
                    }
                    if (kBlockInit && sg == 0 && i == 0 && dh0 != nullptr && live) dh0[state_idx(blk)] = q;
                }
            }
            __syncthreads();
            // dB / dC of the segment: the waves' sums in order
            for (int o = threadIdx.x; o < cnt * 2 * kN; o += NW * kWave) {
                const int i = o / (2 * kN), j = o % (2 * kN);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    float sum = red[r][0][i][j];
#pragma unroll
                    for (int v = 1; v < NW; ++v) sum += red[r][v][i][j];
                    (r == 0 ? pbc : pbcr)[(t_begin + k0 + i) * (2 * kN) + j] = sum;
                }
            }
        }
    }
    // continuous form: the start state's gradient (chunk 0)
    if (!kBlockInit && c == 0 && dh0 != nullptr && live)
        dh0[((int64_t)b * D + d) * kN + n] = q + (dbounds != nullptr ? dbounds[state_idx(0)] : 0.f);
    if (live) {
        const int64_t pc = (int64_t)b * gridDim.y + c;
        part_a[(pc * D + d) * kN + n] = dA_acc;
        if constexpr (kSep) fz.part_a_r[(pc * D + d) * kN + n] = dAr_acc;
        if (n == 0) {
            part_d[pc * D + d] = dD_acc;
            if (kFuse != 0 && fz.part_bias != nullptr) fz.part_bias[pc * D + d] = bias_acc;
            if (kSep && fz.part_bias_r != nullptr) fz.part_bias_r[pc * D + d] = bias_r_acc;
        }
    }
}

// dB and dC: sum the channel-block partials in order.  One thread per four
// consecutive columns of one (batch, token) row (16-byte loads; 2N is a
// multiple of 4), j < N -> dB states j .. j + 3, else dC states j - N ..;
// eight channel blocks' loads in flight, each column summed over the blocks
// in increasing order.  grid = ceil(batch T 2N / 4 / 256), block = 256.
template <typename Tin>
__global__ __launch_bounds__(256) void bc_reduce_kernel(const float *__restrict__ part_bc, Tin *__restrict__ dB,
                                                        Tin *__restrict__ dC, int batch, int64_t T, int nblk,
                                                        int N)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int ncol = 2 * N;
    if (i >= (int64_t)batch * T * ncol) return;
    const int j = (int)(i % ncol);
    const int64_t bt = i / ncol;
    const int64_t b = bt / T, t = bt % T;
    const float4 *p = reinterpret_cast<const float4 *>(part_bc + (b * nblk * T + t) * ncol + j);
    const int64_t stride = T * ncol / 4;          // one channel block, in float4
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int kU = 8;
    int k = 0;
    for (; k + kU <= nblk; k += kU) {
        float4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = p[(int64_t)(k + u) * stride];
#pragma unroll
        for (int u = 0; u < kU; ++u) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
    }
    for (; k < nblk; ++k) {
        const float4 v = p[(int64_t)k * stride];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    Tin *o = (j < N) ? dB + bt * N + j : dC + bt * N + j - N;
    o[0] = narrow<Tin>(s.x);
    o[1] = narrow<Tin>(s.y);
    o[2] = narrow<Tin>(s.z);
    o[3] = narrow<Tin>(s.w);
}

// dA [D,N], dDskip [D] (when part_d is given) and (when part_bias is given)
// the dt_bias gradient [D]: sums of the (batch, chunk) partials.  A workgroup
// covers 64 outputs; its four waves sum interleaved quarters of the partials
// (k = w, w + 4, ...; eight loads in flight per lane), and wave 0 adds the four
// in a fixed order, so the result does not depend on timing.
// grid = ceil((D N + 2 D) / 64) (or D N + D without the bias), block = 256.
static __global__ __attribute__((unused)) __launch_bounds__(256) void param_reduce_kernel(const float *__restrict__ part_a,
                                                           const float *__restrict__ part_d,
                                                           float *__restrict__ dA, float *__restrict__ dDskip,
                                                           int D, int n_parts,
                                                           const float *__restrict__ part_bias,
                                                           float *__restrict__ d_bias, int N)
{
    __shared__ float acc[4][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * kWave + lane;
    const int64_t na = (int64_t)D * N;
    // which array this output sums, its stride between partials and its index
    const float *src = nullptr;
    float *dst = nullptr;
    int64_t stride = 0, j = 0;
    if (i < na) {
        src = part_a; dst = dA; stride = na; j = i;
    } else if (i < na + D) {
        if (part_d != nullptr && dDskip != nullptr) { src = part_d; dst = dDskip; stride = D; j = i - na; }
    } else if (i < na + 2 * D) {
        if (part_bias != nullptr && d_bias != nullptr) { src = part_bias; dst = d_bias; stride = D; j = i - na - D; }
    }
    float s = 0.f;
    if (src != nullptr) {
        constexpr int kU = 8;
        int k = w;
        for (; k + 4 * (kU - 1) < n_parts; k += 4 * kU) {
            float v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) v[u] = src[(int64_t)(k + 4 * u) * stride + j];
#pragma unroll
            for (int u = 0; u < kU; ++u) s += v[u];
        }
        for (; k < n_parts; k += 4) s += src[(int64_t)k * stride + j];
    }
    acc[w][lane] = s;
    __syncthreads();
    if (w == 0 && dst != nullptr) dst[j] = ((acc[0][lane] + acc[1][lane]) + acc[2][lane]) + acc[3][lane];
}

}  // namespace bdssm_dev
