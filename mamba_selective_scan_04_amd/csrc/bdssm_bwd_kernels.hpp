// bdssm_bwd_kernels.hpp -- gfx950 kernels of the backward pass (reverse-mode
// gradients) of the all-block training forms.  Device code only; launch
// policy and the C ABI are in bdssm.hip.
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
// blockIdx.y.
template <typename Tin>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(8))) void adjoint_chunk_kernel(
    const Tin *__restrict__ dt, const Tin *__restrict__ dy, const Tin *__restrict__ Cm,
    const float *__restrict__ A, const float *__restrict__ dbounds, float *__restrict__ qout,
    float *__restrict__ sout, int64_t T, int D, int L, int64_t Tc, int n_chunks, int c_first)
{
    constexpr int U = 4;
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
    const Tin *cs = Cm + first * kStates;

    auto consume = [&](const Tin *dr, const Tin *yr, int k0, int count) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (i < count) {
                const int p = len - 1 - (k0 + i);            // row within the chunk
                const int64_t t = t_begin + p;
                if (dbounds != nullptr && (t + 1) % L == 0) {
                    const float4 *r = reinterpret_cast<const float4 *>(
                        dbounds + (((int64_t)b * (nbl + 1) + (t + 1) / L) * D + d) * kStates);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float4 v = r[k];
                        q[4 * k + 0] += v.x; q[4 * k + 1] += v.y;
                        q[4 * k + 2] += v.z; q[4 * k + 3] += v.w;
                    }
                }
                const float dl = widen(dr[i]);
                const float gy = live ? widen(yr[i]) : 0.f;
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
    auto load_stage = [&](int k0, int count, Tin *dout, Tin *yo) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int p = len - 1 - (k0 + (i < count ? i : count - 1));
            dout[i] = ds.load(p);
            yo[i] = ys.load(p);
        }
    };
    const int n_full = len / U;
    const int rem = len - n_full * U;
    Tin dr[U], yr[U];
    if (n_full > 0) load_stage(0, U, dr, yr);
    for (int g = 0; g < n_full; ++g) {
        Tin dn[U], yn[U];
        if (g + 1 < n_full) load_stage((g + 1) * U, U, dn, yn);
        consume(dr, yr, g * U, U);
#pragma unroll
        for (int i = 0; i < U; ++i) { dr[i] = dn[i]; yr[i] = yn[i]; }
    }
    if (rem > 0) {
        load_stage(n_full * U, rem, dr, yr);
        consume(dr, yr, n_full * U, rem);
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
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
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
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    };
    auto xor1 = [](float v) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    };
    const bool hi2 = (g & 2) != 0, hi1 = (g & 1) != 0;
    const bool b2 = (lane & 4) != 0, b3 = (lane & 8) != 0, b4 = (lane & 16) != 0, b5 = (lane & 32) != 0;
    // slot of this lane's reduced dB / dC value within a token's 32
    const int red_slot = (b3 ? kStates : 0) + s0 + (b2 ? 2 : 0) + (b4 ? 1 : 0);
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
                    // wave's 16 channels: reduce-scatter over lanes ^ 8, ^ 4, ^ 16,
                    // then a plain sum over lanes ^ 32 (both halves hold it)
                    float r4[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float keep = b3 ? tokv[m + 4] : tokv[m];
                        const float send = b3 ? tokv[m] : tokv[m + 4];
                        r4[m] = keep + xchg8(send);
                    }
                    float r2[2];
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const float keep = b2 ? r4[m + 2] : r4[m];
                        const float send = b2 ? r4[m] : r4[m + 2];
                        r2[m] = keep + xchg4(send);
                    }
                    const float keep = b4 ? r2[1] : r2[0];
                    const float send = b4 ? r2[0] : r2[1];
                    float r1 = keep + xchg16(send);
                    r1 += xchg32(r1, lane);
                    // slot: dB (b3 = 0) or dC (b3 = 1), state 4g + 2 b2 + b4
                    if (!b5) red[w][i * 2 * kStates + red_slot] = r1;
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

// dB and dC: sum the channel-block partials in order.  One thread per
// (batch, token, j), j < 16 -> dB state j, j >= 16 -> dC state j - 16.
template <typename Tin>
__global__ __launch_bounds__(256) void bc_reduce_kernel(const float *__restrict__ part_bc, Tin *__restrict__ dB,
                                                        Tin *__restrict__ dC, int batch, int64_t T, int nblk64)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)batch * T * 32) return;
    const int j = (int)(i & 31);
    const int64_t bt = i >> 5;
    const int64_t b = bt / T, t = bt % T;
    const float *p = part_bc + (b * nblk64 * T + t) * 32 + j;
    float s = 0.f;
    for (int k = 0; k < nblk64; ++k) s += p[(int64_t)k * T * 32];
    if (j < kStates) dB[bt * kStates + j] = narrow<Tin>(s);
    else dC[bt * kStates + j - kStates] = narrow<Tin>(s);
}

// dA [D,16] and dDskip [D]: sum the (batch, chunk) partials in order.
__global__ __launch_bounds__(256) void param_reduce_kernel(const float *__restrict__ part_a,
                                                           const float *__restrict__ part_d,
                                                           float *__restrict__ dA, float *__restrict__ dDskip,
                                                           int D, int n_parts)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t na = (int64_t)D * kStates;
    if (i < na) {
        float s = 0.f;
        for (int k = 0; k < n_parts; ++k) s += part_a[(int64_t)k * na + i];
        dA[i] = s;
    } else if (i < na + D) {
        const int64_t dd = i - na;
        float s = 0.f;
        for (int k = 0; k < n_parts; ++k) s += part_d[(int64_t)k * D + dd];
        dDskip[dd] = s;
    }
}

}  // namespace bdssm_dev
