// launch_bidir.hip -- launchers of the register-resident bidirectional kernels
// (bidir_pair_kernel: block lengths 1, 2, 4, 8, 16 and multiples of 16 up to
// 256 at 4, 8, 16 or 32 states; bidir_wave_kernel for separate reverse
// operands at 16 states).
// Compiled once per stream type (BDSSM_TIN = float, or uint16_t for bf16).
#include "bdssm_launch.hpp"

#ifndef BDSSM_TIN
#error "compiled once per stream type: -DBDSSM_TIN=float or -DBDSSM_TIN=uint16_t"
#endif

namespace bdssm_host {

template <typename Tin, int L, bool kInit, int kFuse>
void launch_bidir_k(dim3 g, const void *x, const void *dt, const void *B, const void *C,
                    const float *A, const float *Dskip, const float *hin, int64_t hin_bs,
                    int64_t hin_cs, void *y, float *bounds, float *hout, int64_t T, int64_t D,
                    int64_t Tc, const float *h0_blocks, const Fuse &f, hipStream_t st) {
    hipLaunchKernelGGL((bidir_wave_kernel<Tin, L, kInit, kFuse>), g, dim3(4 * kWave), 0, st,
                       (const Tin *)x, (const Tin *)dt, (const Tin *)B, (const Tin *)C, A, Dskip,
                       hin, hin_bs, hin_cs, (Tin *)y, bounds, hout, T, (int)D, Tc, h0_blocks,
                       f.args<Tin>());
}

template <typename Tin, int kN, int L, bool kInit, int kFuse>
void launch_pair_k(dim3 g, const void *x, const void *dt, const void *B, const void *C,
                   const float *A, const float *Dskip, const float *hin, int64_t hin_bs,
                   int64_t hin_cs, void *y, float *bounds, float *hout, int64_t T, int64_t D,
                   int64_t Tc, const float *h0_blocks, const Fuse &f, hipStream_t st, int64_t Lr) {
    hipLaunchKernelGGL((bidir_pair_kernel<Tin, kN, L, kInit, kFuse>), g, dim3(4 * kWave),
                       L == 0 ? pair_long_lds(Lr) : 0, st,
                       (const Tin *)x, (const Tin *)dt, (const Tin *)B, (const Tin *)C, A, Dskip,
                       hin, hin_bs, hin_cs, (Tin *)y, bounds, hout, T, (int)D, Tc, h0_blocks,
                       f.args<Tin>(), (int)Lr);
}

// bidir_pair_kernel at kN states and block length L (shared operands; L = 0:
// long blocks of Lr tokens)
template <typename Tin, int kN, int L>
void launch_pair_L(const void *x, const void *dt, const void *B, const void *C, const float *A,
                   const float *Dskip, const float *hin, int64_t hin_bs, int64_t hin_cs, void *y,
                   float *bounds, float *hout, int64_t batch, int64_t T, int64_t D, int64_t Tc,
                   int n_chunks, const float *h0_blocks, const Fuse &f, hipStream_t st, int64_t Lr = 0) {
    const dim3 g((unsigned)ceil_div(D, pair_channels<kN>()), (unsigned)n_chunks, (unsigned)batch);
    const bool fused = f.any();
#define BDSSM_PAIR(INIT, FV)                                                                         \
    launch_pair_k<Tin, kN, L, INIT, FV>(g, x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, T, D, \
                                        Tc, h0_blocks, f, st, Lr)
    if (h0_blocks != nullptr) {
        if (fused) BDSSM_PAIR(true, 1);
        else BDSSM_PAIR(true, 0);
    } else {
        if (fused) BDSSM_PAIR(false, 1);
        else BDSSM_PAIR(false, 0);
    }
#undef BDSSM_PAIR
}

template <typename Tin, int kN>
void launch_pair(int64_t L, const void *x, const void *dt, const void *B, const void *C, const float *A,
                 const float *Dskip, const float *hin, int64_t hin_bs, int64_t hin_cs, void *y,
                 float *bounds, float *hout, int64_t batch, int64_t T, int64_t D, int64_t Tc,
                 int n_chunks, const float *h0_blocks, const Fuse &f, hipStream_t st) {
    if (L > kGroup) {
        launch_pair_L<Tin, kN, 0>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc,
                                  n_chunks, h0_blocks, f, st, L);
        return;
    }
    switch (L) {
    case 1: launch_pair_L<Tin, kN, 1>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    case 2: launch_pair_L<Tin, kN, 2>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    case 4: launch_pair_L<Tin, kN, 4>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    case 8: launch_pair_L<Tin, kN, 8>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    default: launch_pair_L<Tin, kN, 16>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    }
}

// bidir_wave_kernel (16 states): separate reverse operands, or forced
template <typename Tin, int L>
void launch_bidir_L(const void *x, const void *dt, const void *B, const void *C, const float *A,
                    const float *Dskip, const float *hin, int64_t hin_bs, int64_t hin_cs, void *y,
                    float *bounds, float *hout, int64_t batch, int64_t T, int64_t D, int64_t Tc,
                    int n_chunks, const float *h0_blocks, const Fuse &f, hipStream_t st) {
    const dim3 g = grid3(D, n_chunks, batch);
    // kernel variant: 0 plain, 1 fused step size / gate, 2 also separate
    // reverse operands
    const int fv = f.dt_r != nullptr ? 2 : f.any() ? 1 : 0;
#define BDSSM_BIDIR(INIT, FV)                                                                       \
    launch_bidir_k<Tin, L, INIT, FV>(g, x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, T, D, \
                                     Tc, h0_blocks, f, st)
    if (h0_blocks != nullptr) {
        if (fv == 2) BDSSM_BIDIR(true, 2);
        else if (fv == 1) BDSSM_BIDIR(true, 1);
        else BDSSM_BIDIR(true, 0);
    } else {
        if (fv == 2) BDSSM_BIDIR(false, 2);
        else if (fv == 1) BDSSM_BIDIR(false, 1);
        else BDSSM_BIDIR(false, 0);
    }
#undef BDSSM_BIDIR
}

// The bidirectional pass: for L | 16 and for multiples of 16 up to 256
// (chunks of whole blocks, several blocks per row), bidir_pair_kernel at any
// supported state count (shared operands); bidir_wave_kernel for separate
// reverse operands at 16 states and L | 16; everything else on
// block_bidir_kernel or block_split_kernel (Tc then a multiple of L).
template <typename Tin>
void launch_bidir(int64_t L, const void *x, const void *dt, const void *B, const void *C,
                  const float *A, const float *Dskip, const float *hin, int64_t hin_bs,
                  int64_t hin_cs, void *y, float *bounds, float *hout, int64_t batch, int64_t T,
                  int64_t D, int64_t N, int64_t Tc, int n_chunks, hipStream_t st,
                  const float *h0_blocks, const Fuse &f) {
    const bool sep = f.dt_r != nullptr;
    // long blocks: one block per row (block step, commit) stays on
    // block_split_kernel / block_bidir_kernel, whose waves share the block
    const bool lng = pair_long(L, N) && !(n_chunks == 1 && T == L);
    if ((pair_path(L, N) || lng) && !sep && pair_bidir()) {
        with_states(N, [&](auto n) {
            launch_pair<Tin, decltype(n)::value>(L, x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout,
                                                 batch, T, D, Tc, n_chunks, h0_blocks, f, st);
        });
        return;
    }
    if (!wave_path(L, N)) {
        launch_block_bidir_any<Tin>(N, L, x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout,
                                    batch, T, D, Tc, n_chunks, h0_blocks, f, st);
        return;
    }
    switch (L) {
    case 1: launch_bidir_L<Tin, 1>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    case 2: launch_bidir_L<Tin, 2>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    case 4: launch_bidir_L<Tin, 4>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    case 8: launch_bidir_L<Tin, 8>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    default: launch_bidir_L<Tin, 16>(x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st); break;
    }
}

// ------------------------------------------------ explicit instantiations

template void launch_bidir<BDSSM_TIN>(int64_t, const void *, const void *, const void *, const void *,
                                    const float *, const float *, const float *, int64_t, int64_t, void *,
                                    float *, float *, int64_t, int64_t, int64_t, int64_t, int64_t, int,
                                    hipStream_t, const float *, const Fuse &);

}  // namespace bdssm_host
