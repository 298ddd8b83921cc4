// launch_chunk.hip -- launchers of the one-lane-per-channel chunk scans (prefill
// aggregates, direct passes) and of the baseline's output sweeps.
// Compiled once per stream type (BDSSM_TIN = float, or uint16_t for bf16).
#include "bdssm_launch.hpp"

#ifndef BDSSM_TIN
#error "compiled once per stream type: -DBDSSM_TIN=float or -DBDSSM_TIN=uint16_t"
#endif

namespace bdssm_host {

template <typename Tin, bool kRev, bool kDirect, int kN>
void launch_chunk_state_k(int dt_mode, dim3 g, const Tin *xp, const Tin *dp, const Tin *bp,
                          const float *A, const float *h0, float *hout, float *sout, int64_t T,
                          int64_t D, int64_t Tc, int n_chunks, int c_first, const float *bias,
                          hipStream_t st) {
    switch (dt_mode) {
    case kDtSoftplus:
        hipLaunchKernelGGL((chunk_state_kernel<Tin, kRev, kDirect, kDtSoftplus, kN>), g, dim3(kWave), 0, st,
                           xp, dp, bp, A, h0, hout, sout, T, (int)D, Tc, n_chunks, c_first, bias);
        break;
    case kDtBias:
        hipLaunchKernelGGL((chunk_state_kernel<Tin, kRev, kDirect, kDtBias, kN>), g, dim3(kWave), 0, st,
                           xp, dp, bp, A, h0, hout, sout, T, (int)D, Tc, n_chunks, c_first, bias);
        break;
    default:
        hipLaunchKernelGGL((chunk_state_kernel<Tin, kRev, kDirect, kDtPlain, kN>), g, dim3(kWave), 0, st,
                           xp, dp, bp, A, h0, hout, sout, T, (int)D, Tc, n_chunks, c_first, bias);
        break;
    }
}

// Chunk-local scans of n_launch chunks (N states per channel).
template <typename Tin>
void launch_chunk_state(bool rev, const void *x, const void *dt, const void *B, const float *A,
                        const float *h0, float *hout, float *sout, int64_t batch, int64_t T,
                        int64_t D, int64_t N, int64_t Tc, int n_chunks, int c_first, int n_launch,
                        hipStream_t st, const Fuse &f) {
    if (n_launch <= 0) return;
    const dim3 g = grid3(D, n_launch, batch);
    const Tin *xp = (const Tin *)x, *dp = (const Tin *)dt, *bp = (const Tin *)B;
    with_states(N, [&](auto kn) {
        constexpr int kN = decltype(kn)::value;
        if (sout == nullptr)   // direct pass from h0 into hout (one chunk)
            launch_chunk_state_k<Tin, false, true, kN>(f.dt_mode, g, xp, dp, bp, A, h0, hout, sout, T, D,
                                                       Tc, n_chunks, c_first, f.dt_bias, st);
        else if (rev)
            launch_chunk_state_k<Tin, true, false, kN>(f.dt_mode, g, xp, dp, bp, A, h0, hout, sout, T, D,
                                                       Tc, n_chunks, c_first, f.dt_bias, st);
        else
            launch_chunk_state_k<Tin, false, false, kN>(f.dt_mode, g, xp, dp, bp, A, h0, hout, sout, T,
                                                        D, Tc, n_chunks, c_first, f.dt_bias, st);
    });
}

// Forward and reverse aggregates of all n_chunks chunks in one pass
// (chunk_both_kernel; shared operands).
template <typename Tin>
void launch_chunk_both(const void *x, const void *dt, const void *B, const float *A, float *hout, float *sout,
                       float *rout, int64_t batch, int64_t T, int64_t D, int64_t N, int64_t Tc, int n_chunks,
                       hipStream_t st, const Fuse &f) {
    if (n_chunks <= 0) return;
    const dim3 g = grid3(D, n_chunks, batch);
    const Tin *xp = (const Tin *)x, *dp = (const Tin *)dt, *bp = (const Tin *)B;
    with_states(N, [&](auto kn) {
        constexpr int kN = decltype(kn)::value;
#define BDSSM_BOTH(KDT)                                                                                 \
        hipLaunchKernelGGL((chunk_both_kernel<Tin, KDT, kN>), g, dim3(kWave), 0, st, xp, dp, bp, A, hout, sout, \
                           rout, T, (int)D, Tc, n_chunks, f.dt_bias)
        switch (f.dt_mode) {
        case kDtSoftplus: BDSSM_BOTH(kDtSoftplus); break;
        case kDtBias: BDSSM_BOTH(kDtBias); break;
        default: BDSSM_BOTH(kDtPlain); break;
        }
#undef BDSSM_BOTH
    });
}

template <typename Tin, bool kRev, int kN>
void launch_sweep_k(dim3 g, const void *x, const void *dt, const void *B, const void *C,
                    const float *A, const float *Dskip, const float *hin, float *yf, void *y,
                    int64_t T, int64_t D, int64_t Tc, int n_chunks, const Fuse &f, hipStream_t st) {
    const Tin *zp = (const Tin *)f.z;
#define BDSSM_SWEEP(KDT)                                                                          \
    hipLaunchKernelGGL((sweep_output_kernel<Tin, kRev, KDT, kN>), g, dim3(kWave), 0, st, (const Tin *)x, \
                       (const Tin *)dt, (const Tin *)B, (const Tin *)C, A, Dskip, hin, yf, (Tin *)y, \
                       T, (int)D, Tc, n_chunks, f.dt_bias, zp)
    switch (f.dt_mode) {
    case kDtSoftplus: BDSSM_SWEEP(kDtSoftplus); break;
    case kDtBias: BDSSM_SWEEP(kDtBias); break;
    default: BDSSM_SWEEP(kDtPlain); break;
    }
#undef BDSSM_SWEEP
}

template <typename Tin>
void launch_sweep(bool rev, const void *x, const void *dt, const void *B, const void *C,
                  const float *A, const float *Dskip, const float *hin, float *yf, void *y,
                  int64_t batch, int64_t T, int64_t D, int64_t N, int64_t Tc, int n_chunks,
                  hipStream_t st, const Fuse &f) {
    const dim3 g = grid3(D, n_chunks, batch);
    with_states(N, [&](auto kn) {
        constexpr int kN = decltype(kn)::value;
        if (rev) launch_sweep_k<Tin, true, kN>(g, x, dt, B, C, A, Dskip, hin, yf, y, T, D, Tc, n_chunks, f, st);
        else launch_sweep_k<Tin, false, kN>(g, x, dt, B, C, A, Dskip, hin, yf, y, T, D, Tc, n_chunks, f, st);
    });
}

// ------------------------------------------------ explicit instantiations

template void launch_chunk_state<BDSSM_TIN>(bool, const void *, const void *, const void *, const float *,
                                          const float *, float *, float *, int64_t, int64_t, int64_t,
                                          int64_t, int64_t, int, int, int, hipStream_t, const Fuse &);
template void launch_chunk_both<BDSSM_TIN>(const void *, const void *, const void *, const float *, float *,
                                         float *, float *, int64_t, int64_t, int64_t, int64_t, int64_t, int,
                                         hipStream_t, const Fuse &);
template void launch_sweep<BDSSM_TIN>(bool, const void *, const void *, const void *, const void *, const float *,
                                    const float *, const float *, float *, void *, int64_t, int64_t, int64_t,
                                    int64_t, int64_t, int, hipStream_t, const Fuse &);

}  // namespace bdssm_host
