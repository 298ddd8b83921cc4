// launch_bwd_general.hip -- launchers of the backward's general path
// (bwd_general_kernel, adjoint_general_kernel).
// Compiled once per stream type (BDSSM_TIN = float, or uint16_t for bf16).
#include "bdssm_launch.hpp"

#ifndef BDSSM_TIN
#error "compiled once per stream type: -DBDSSM_TIN=float or -DBDSSM_TIN=uint16_t"
#endif

namespace bdssm_host {

template <typename Tin, int kN, bool kBlockInit, int kF>
void launch_bwd_general_v(const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t L, int64_t Tc,
                          int nc, hipStream_t st) {
    constexpr int NW = bwd_general_waves<kF>();
    const dim3 g((unsigned)ceil_div(D, NW * kWave / kN), (unsigned)nc, (unsigned)batch);
    const BwdFuse<Tin> fz{a.dt_bias, a.dt_mode, (const Tin *)a.z, (Tin *)a.dz, a.part_bias,
                          (const Tin *)a.dt_r, (const Tin *)a.B_r, (const Tin *)a.C_r, a.A_r, a.dt_bias_r,
                          (Tin *)a.ddt_r, a.part_bc_r, a.part_a_r, a.part_bias_r};
    hipLaunchKernelGGL((bwd_general_kernel<Tin, kN, kBlockInit, kF>), g, dim3(NW * kWave),
                       bwd_general_lds(L, NW), st, (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B,
                       (const Tin *)a.C, (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs,
                       a.qin_cs, a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                       T, (int)D, (int)L, Tc, fz);
}

template <typename Tin, int kN, bool kBlockInit>
void launch_bwd_general_k(const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t L, int64_t Tc,
                          int nc, hipStream_t st) {
    if (a.sep) launch_bwd_general_v<Tin, kN, kBlockInit, 2>(a, batch, T, D, L, Tc, nc, st);
    else if (a.fused) launch_bwd_general_v<Tin, kN, kBlockInit, 1>(a, batch, T, D, L, Tc, nc, st);
    else launch_bwd_general_v<Tin, kN, kBlockInit, 0>(a, batch, T, D, L, Tc, nc, st);
}

template <typename Tin, bool kBlockInit>
void launch_bwd_general(int64_t N, const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t L,
                        int64_t Tc, int nc, hipStream_t st) {
    with_states(N, [&](auto kn) {
        launch_bwd_general_k<Tin, decltype(kn)::value, kBlockInit>(a, batch, T, D, L, Tc, nc, st);
    });
}

template <typename Tin, int kN, int kDt>
void launch_adjoint_general_k(const void *dt, const void *dy, const void *C, const float *A,
                              const float *dbounds, float *qout, float *sout, int64_t batch, int64_t T,
                              int64_t D, int64_t L, int64_t Tc, int n_chunks, int c_first, int n_launch,
                              const float *dt_bias, const void *z, hipStream_t st) {
    hipLaunchKernelGGL((adjoint_general_kernel<Tin, kN, kDt>),
                       dim3((unsigned)ceil_div(D, kWave), (unsigned)n_launch, (unsigned)batch), dim3(kWave),
                       0, st, (const Tin *)dt, (const Tin *)dy, (const Tin *)C, A, dbounds, qout, sout, T,
                       (int)D, (int)L, Tc, n_chunks, c_first, dt_bias, (const Tin *)z);
}

// chunk-local adjoints of the general path (chunks c_first .. c_first + n_launch - 1)
template <typename Tin>
void launch_adjoint_general(int64_t N, const void *dt, const void *dy, const void *C, const float *A,
                            const float *dbounds, float *qout, float *sout, int64_t batch, int64_t T,
                            int64_t D, int64_t L, int64_t Tc, int n_chunks, int c_first, int n_launch,
                            int dt_mode, const float *dt_bias, const void *z, hipStream_t st) {
    if (n_launch <= 0) return;
    with_states(N, [&](auto kn) {
        constexpr int K = decltype(kn)::value;
        if (dt_mode == kDtSoftplus)
            launch_adjoint_general_k<Tin, K, kDtSoftplus>(dt, dy, C, A, dbounds, qout, sout, batch, T, D, L, Tc,
                                                          n_chunks, c_first, n_launch, dt_bias, z, st);
        else if (dt_mode == kDtBias)
            launch_adjoint_general_k<Tin, K, kDtBias>(dt, dy, C, A, dbounds, qout, sout, batch, T, D, L, Tc,
                                                      n_chunks, c_first, n_launch, dt_bias, z, st);
        else
            launch_adjoint_general_k<Tin, K, kDtPlain>(dt, dy, C, A, dbounds, qout, sout, batch, T, D, L, Tc,
                                                       n_chunks, c_first, n_launch, dt_bias, z, st);
    });
}

// ------------------------------------------------ explicit instantiations

template void launch_bwd_general<BDSSM_TIN, false>(int64_t, const BwdArgs &, int64_t, int64_t, int64_t, int64_t,
                                                int64_t, int, hipStream_t);
template void launch_bwd_general<BDSSM_TIN, true>(int64_t, const BwdArgs &, int64_t, int64_t, int64_t, int64_t,
                                               int64_t, int, hipStream_t);
template void launch_adjoint_general<BDSSM_TIN>(int64_t, const void *, const void *, const void *, const float *,
                                              const float *, float *, float *, int64_t, int64_t, int64_t,
                                              int64_t, int64_t, int, int, int, int, const float *, const void *,
                                              hipStream_t);

}  // namespace bdssm_host
