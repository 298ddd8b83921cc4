// launch_bwd.hip -- launchers of the backward's register-resident kernels
// (adjoint_chunk_kernel, bwd_pair_kernel, bwd_wave_kernel, group_state_kernel)
// and of the ordered gradient reductions.
// Compiled once per stream type (BDSSM_TIN = float, or uint16_t for bf16).
#include "bdssm_launch.hpp"

#ifndef BDSSM_TIN
#error "compiled once per stream type: -DBDSSM_TIN=float or -DBDSSM_TIN=uint16_t"
#endif

namespace bdssm_host {

template <typename Tin, int kDt>
void launch_adjoint_chunk_k(const void *dt, const void *dy, const void *C, const float *A,
                            const float *dbounds, float *qout, float *sout, int64_t batch, int64_t T,
                            int64_t D, int64_t L, int64_t Tc, int n_chunks, int c_first, int n_launch,
                            const float *dt_bias, const void *z, hipStream_t st) {
#define BDSSM_ADJ(LL)                                                                              \
    hipLaunchKernelGGL((adjoint_chunk_kernel<Tin, LL, kDt>), grid3(D, n_launch, batch), dim3(kWave), 0, \
                       st, (const Tin *)dt, (const Tin *)dy, (const Tin *)C, A, dbounds, qout, sout, T, \
                       (int)D, Tc, n_chunks, c_first, dt_bias, (const Tin *)z)
    switch (L) {
    case 1: BDSSM_ADJ(1); break;
    case 2: BDSSM_ADJ(2); break;
    case 4: BDSSM_ADJ(4); break;
    case 8: BDSSM_ADJ(8); break;
    default: BDSSM_ADJ(16); break;
    }
#undef BDSSM_ADJ
}

// Adjoint aggregates of n_launch fine chunks; the step size and gate of the
// fused forward when given.
template <typename Tin>
void launch_adjoint_chunk(const void *dt, const void *dy, const void *C, const float *A,
                          const float *dbounds, float *qout, float *sout, int64_t batch, int64_t T,
                          int64_t D, int64_t L, int64_t Tc, int n_chunks, int c_first, int n_launch,
                          hipStream_t st, int dt_mode, const float *dt_bias,
                          const void *z) {
    if (n_launch <= 0) return;
    switch (dt_mode) {
    case kDtSoftplus:
        launch_adjoint_chunk_k<Tin, kDtSoftplus>(dt, dy, C, A, dbounds, qout, sout, batch, T, D, L, Tc,
                                                 n_chunks, c_first, n_launch, dt_bias, z, st);
        break;
    case kDtBias:
        launch_adjoint_chunk_k<Tin, kDtBias>(dt, dy, C, A, dbounds, qout, sout, batch, T, D, L, Tc,
                                             n_chunks, c_first, n_launch, dt_bias, z, st);
        break;
    default:
        launch_adjoint_chunk_k<Tin, kDtPlain>(dt, dy, C, A, dbounds, qout, sout, batch, T, D, L, Tc,
                                              n_chunks, c_first, n_launch, dt_bias, z, st);
        break;
    }
}

template <typename Tin, int kN, int L, bool kBlockInit>
void launch_bwd_L(const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t Tc, int nc,
                  hipStream_t st) {
    if constexpr (kN == kStates) {
        if (bwd_use_wave(L, a.fused, kN)) {
            hipLaunchKernelGGL((bwd_wave_kernel<Tin, L, kBlockInit>), grid3(D, nc, batch), dim3(4 * kWave), 0,
                               st, (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                               (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                               a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0, T,
                               (int)D, Tc);
            return;
        }
    }
    const dim3 g((unsigned)ceil_div(D, pair_channels<kN>()), (unsigned)nc, (unsigned)batch);
    const BwdFuse<Tin> fz{a.dt_bias, a.dt_mode, (const Tin *)a.z, (Tin *)a.dz, a.part_bias};
    if (a.fused)
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, kN, L, kBlockInit, true>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)nullptr, 0);
    else
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, kN, L, kBlockInit, false>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)nullptr, 0);
}

template <typename Tin, int kN, bool kBlockInit>
void launch_bwd_n(int64_t L, const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t Tc, int nc,
                  hipStream_t st) {
    switch (L) {
    case 1: launch_bwd_L<Tin, kN, 1, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    case 2: launch_bwd_L<Tin, kN, 2, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    case 4: launch_bwd_L<Tin, kN, 4, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    case 8: launch_bwd_L<Tin, kN, 8, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    default: launch_bwd_L<Tin, kN, 16, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    }
}

template <typename Tin, bool kBlockInit>
void launch_bwd(int64_t L, int64_t N, const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t Tc,
                int nc, hipStream_t st) {
    with_states(N, [&](auto n) {
        launch_bwd_n<Tin, decltype(n)::value, kBlockInit>(L, a, batch, T, D, Tc, nc, st);
    });
}

template <typename Tin, int kDt>
void launch_group_state_k(const BwdArgs &a, float *gstate, int64_t batch, int64_t T, int64_t D, int64_t L,
                          hipStream_t st) {
    const int64_t nbt = ceil_div(T, L);
    hipLaunchKernelGGL((group_state_kernel<Tin, kDt>),
                       dim3((unsigned)ceil_div(D, kWave), (unsigned)(nbt < 65535 ? nbt : 65535), (unsigned)batch),
                       dim3(kWave), 0, st, (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B,
                       (const Tin *)a.C, (const Tin *)a.dy, a.A, a.h_start, gstate, T, (int)D, (int)L,
                       a.dt_bias, (const Tin *)a.z);
}

// long blocks: the group states, then bwd_pair_kernel over groups that
// continue a block (chunks are whole blocks)
template <typename Tin, bool kBlockInit>
void launch_bwd_long(const BwdArgs &a, float *gstate, int64_t batch, int64_t T, int64_t D, int64_t L,
                     int64_t Tc, int nc, hipStream_t st) {
    if (a.dt_mode == kDtSoftplus) launch_group_state_k<Tin, kDtSoftplus>(a, gstate, batch, T, D, L, st);
    else if (a.dt_mode == kDtBias) launch_group_state_k<Tin, kDtBias>(a, gstate, batch, T, D, L, st);
    else launch_group_state_k<Tin, kDtPlain>(a, gstate, batch, T, D, L, st);
    const dim3 g((unsigned)ceil_div(D, kPairChannels), (unsigned)nc, (unsigned)batch);
    const BwdFuse<Tin> fz{a.dt_bias, a.dt_mode, (const Tin *)a.z, (Tin *)a.dz, a.part_bias};
    if (a.fused)
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, kStates, 0, kBlockInit, true>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)gstate, (int)L);
    else
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, kStates, 0, kBlockInit, false>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)gstate, (int)L);
}

template <typename Tin>
void launch_bwd_reduce(const BwdWorkspace &w, void *dB, void *dC, float *dA, float *dDskip,
                       int64_t batch, int64_t T, int64_t D, int64_t L, int64_t N, int64_t nc,
                       hipStream_t st, bool fused, float *d_bias,
                       const bdssm_fusion_grads *gr) {
    const bool sep = gr != nullptr;
    const int64_t nbc = batch * T * 2 * N;
    const int nblk = (int)ceil_div(D, bwd_channels(L, N, fused, sep));
    hipLaunchKernelGGL((bc_reduce_kernel<Tin>), dim3((unsigned)ceil_div(nbc / 4, 256)), dim3(256), 0, st,
                       w.part_bc, (Tin *)dB, (Tin *)dC, (int)batch, T, nblk, (int)N);
    const bool nb = fused && d_bias != nullptr;
    hipLaunchKernelGGL(param_reduce_kernel, dim3((unsigned)ceil_div(D * (N + (nb ? 2 : 1)), kWave)),
                       dim3(256), 0, st, w.part_a, w.part_d, dA, dDskip, (int)D, (int)(batch * nc),
                       nb ? w.part_bias : nullptr, nb ? d_bias : nullptr, (int)N);
    if (sep) {
        // the reverse operands' dB_r, dC_r, dA_r (and their bias gradient)
        hipLaunchKernelGGL((bc_reduce_kernel<Tin>), dim3((unsigned)ceil_div(nbc / 4, 256)), dim3(256), 0, st,
                           w.part_bc_r, (Tin *)gr->dB_rev, (Tin *)gr->dC_rev, (int)batch, T, nblk, (int)N);
        const bool nbr = gr->d_dt_bias_rev != nullptr;
        hipLaunchKernelGGL(param_reduce_kernel, dim3((unsigned)ceil_div(D * (N + 2), kWave)), dim3(256), 0, st,
                           w.part_a_r, nullptr, gr->dA_rev, nullptr, (int)D, (int)(batch * nc),
                           nbr ? w.part_bias_r : nullptr, nbr ? gr->d_dt_bias_rev : nullptr, (int)N);
    }
}

// ------------------------------------------------ explicit instantiations

template void launch_adjoint_chunk<BDSSM_TIN>(const void *, const void *, const void *, const float *,
                                            const float *, float *, float *, int64_t, int64_t, int64_t,
                                            int64_t, int64_t, int, int, int, hipStream_t, int, const float *,
                                            const void *);
template void launch_bwd<BDSSM_TIN, false>(int64_t, int64_t, const BwdArgs &, int64_t, int64_t, int64_t, int64_t,
                                        int, hipStream_t);
template void launch_bwd<BDSSM_TIN, true>(int64_t, int64_t, const BwdArgs &, int64_t, int64_t, int64_t, int64_t,
                                       int, hipStream_t);
template void launch_bwd_long<BDSSM_TIN, false>(const BwdArgs &, float *, int64_t, int64_t, int64_t, int64_t,
                                             int64_t, int, hipStream_t);
template void launch_bwd_long<BDSSM_TIN, true>(const BwdArgs &, float *, int64_t, int64_t, int64_t, int64_t,
                                            int64_t, int, hipStream_t);
template void launch_bwd_reduce<BDSSM_TIN>(const BwdWorkspace &, void *, void *, float *, float *, int64_t,
                                         int64_t, int64_t, int64_t, int64_t, int64_t, hipStream_t, bool,
                                         float *, const bdssm_fusion_grads *);

}  // namespace bdssm_host
