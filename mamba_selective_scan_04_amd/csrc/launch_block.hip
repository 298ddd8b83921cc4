// launch_block.hip -- launchers of the one-lane-per-channel block kernels
// (block_bidir_kernel, block_split_kernel) and of block_lane_kernel.
// Compiled once per stream type (BDSSM_TIN = float, or uint16_t for bf16).
#include "bdssm_launch.hpp"

#ifndef BDSSM_TIN
#error "compiled once per stream type: -DBDSSM_TIN=float or -DBDSSM_TIN=uint16_t"
#endif

namespace bdssm_host {

// One block from the cache on block_lane_kernel (block_step: kCommit false;
// commit: true, y optional).  Used for L <= 16 with shared reverse operands.
template <typename Tin, bool kCommit>
void launch_block_lane(int64_t N, const void *x, const void *dt, const void *B, const void *C,
                       const float *A, const float *Dskip, float *h_cache, void *y, int64_t batch,
                       int64_t D, int64_t L, const Fuse &f, hipStream_t st) {
    with_states(N, [&](auto kn) {
        constexpr int K = decltype(kn)::value;
        const dim3 g((unsigned)ceil_div(D, 4 * kWave / K), (unsigned)batch);
        if (f.any())
            hipLaunchKernelGGL((block_lane_kernel<Tin, K, kCommit, true>), g, dim3(4 * kWave), 0, st,
                               (const Tin *)x, (const Tin *)dt, (const Tin *)B, (const Tin *)C, A, Dskip,
                               h_cache, (Tin *)y, (int)D, (int)L, f.args<Tin>());
        else
            hipLaunchKernelGGL((block_lane_kernel<Tin, K, kCommit, false>), g, dim3(4 * kWave), 0, st,
                               (const Tin *)x, (const Tin *)dt, (const Tin *)B, (const Tin *)C, A, Dskip,
                               h_cache, (Tin *)y, (int)D, (int)L, f.args<Tin>());
    });
}

// Segment length of block_bidir_kernel for block length L and N states: small
// enough that the staged outputs (256 bytes per token) do not limit the
// workgroups per CU below what the registers allow (16 waves per CU at
// N <= 16: 32 tokens; 8 at N = 32: 64), no smaller, since every segment
// boundary adds state-only reverse work (measured on MI355X at the 87M
// training shape).  BDSSM_SEG overrides (tuning, tests).
static int block_seg(int64_t L, int64_t N) {
    const int64_t forced = env_int("BDSSM_SEG", 0);
    const int64_t s = forced > 0 ? forced : (N >= 32 ? 64 : 32);
    return (int)(L < s ? L : s);
}

template <typename Tin, int kN, bool kInit, int kDt>
void launch_block_bidir_k(dim3 g, int64_t L, const void *x, const void *dt, const void *B,
                          const void *C, const float *A, const float *Dskip, const float *hin,
                          int64_t hin_bs, int64_t hin_cs, void *y, float *bounds, float *hout,
                          int64_t T, int64_t D, int64_t Tc, const float *h0_blocks, const Fuse &f,
                          hipStream_t st) {
    const int seg = block_seg(L, kN);
    const size_t lds = (size_t)seg * kWave * sizeof(float);
    hipLaunchKernelGGL((block_bidir_kernel<Tin, kN, kInit, kDt>), g, dim3(kWave), lds, st,
                       (const Tin *)x, (const Tin *)dt, (const Tin *)B, (const Tin *)C, A, Dskip,
                       hin, hin_bs, hin_cs, (Tin *)y, bounds, hout, T, (int)D, (int)L, Tc,
                       h0_blocks, f.args<Tin>(), seg);
}

// A single block per batch row (T == L, one chunk, no block states) above 32
// tokens at up to 16 states: block_split_kernel spreads the block's tokens
// over up to 8 waves (at 8 x 1536 channels: 35 / 50 / 89 us at L = 64 / 128 /
// 256 against 65 / 165 / 469 us on block_bidir_kernel; at L = 32 the latter
// is slightly faster).  BDSSM_SPLIT=0 keeps block_bidir_kernel (tests).
static bool use_split(int64_t L, int64_t N, int64_t T, int n_chunks, const float *bounds, const float *h0_blocks) {
    if (N > 16 || L <= 2 * kGroup || T != L || n_chunks != 1 || bounds != nullptr || h0_blocks != nullptr) return false;
    const char *v = getenv("BDSSM_SPLIT");
    return !(v != nullptr && v[0] == '0');
}

template <typename Tin, int kN>
void launch_block_split(int64_t L, const void *x, const void *dt, const void *B, const void *C,
                        const float *A, const float *Dskip, const float *hin, int64_t hin_bs, void *y,
                        float *hout, int64_t batch, int64_t D, const Fuse &f, hipStream_t st) {
    if constexpr (kN <= 16) {
        const int nw = (int)(ceil_div(L, kGroup) < 8 ? ceil_div(L, kGroup) : 8);   // segments <= kSplitSeg
        const size_t lds = (size_t)nw * (kN + 1) * kWave * sizeof(float);
        const dim3 g((unsigned)ceil_div(D, kWave), 1u, (unsigned)batch);
#define BDSSM_SPLIT_K(KDT)                                                                                   \
    hipLaunchKernelGGL((block_split_kernel<Tin, kN, KDT>), g, dim3(nw * kWave), lds, st, (const Tin *)x,    \
                       (const Tin *)dt, (const Tin *)B, (const Tin *)C, A, Dskip, hin, hin_bs, (Tin *)y, hout, \
                       (int)D, (int)L, f.args<Tin>())
        switch (f.dt_mode) {
        case kDtSoftplus: BDSSM_SPLIT_K(kDtSoftplus); break;
        case kDtBias: BDSSM_SPLIT_K(kDtBias); break;
        default: BDSSM_SPLIT_K(kDtPlain); break;
        }
#undef BDSSM_SPLIT_K
    }
}

// Bidirectional pass with block_bidir_kernel (any L <= kMaxLdsBlock; Tc a
// multiple of L), or block_split_kernel for a single block per row.
template <typename Tin, int kN>
void launch_block_bidir(int64_t L, const void *x, const void *dt, const void *B, const void *C,
                        const float *A, const float *Dskip, const float *hin, int64_t hin_bs,
                        int64_t hin_cs, void *y, float *bounds, float *hout, int64_t batch,
                        int64_t T, int64_t D, int64_t Tc, int n_chunks, const float *h0_blocks,
                        const Fuse &f, hipStream_t st) {
    if (use_split(L, kN, T, n_chunks, bounds, h0_blocks)) {
        launch_block_split<Tin, kN>(L, x, dt, B, C, A, Dskip, hin, hin_bs, y, hout, batch, D, f, st);
        return;
    }
    const dim3 g = grid3(D, n_chunks, batch);
#define BDSSM_BLOCK(INIT, KDT)                                                                       \
    launch_block_bidir_k<Tin, kN, INIT, KDT>(g, L, x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds, \
                                             hout, T, D, Tc, h0_blocks, f, st)
    if (h0_blocks != nullptr) {
        switch (f.dt_mode) {
        case kDtSoftplus: BDSSM_BLOCK(true, kDtSoftplus); break;
        case kDtBias: BDSSM_BLOCK(true, kDtBias); break;
        default: BDSSM_BLOCK(true, kDtPlain); break;
        }
    } else {
        switch (f.dt_mode) {
        case kDtSoftplus: BDSSM_BLOCK(false, kDtSoftplus); break;
        case kDtBias: BDSSM_BLOCK(false, kDtBias); break;
        default: BDSSM_BLOCK(false, kDtPlain); break;
        }
    }
#undef BDSSM_BLOCK
}


template <typename Tin>
void launch_block_bidir_any(int64_t N, int64_t L, const void *x, const void *dt, const void *B,
                            const void *C, const float *A, const float *Dskip, const float *hin,
                            int64_t hin_bs, int64_t hin_cs, void *y, float *bounds, float *hout,
                            int64_t batch, int64_t T, int64_t D, int64_t Tc, int n_chunks,
                            const float *h0_blocks, const Fuse &f, hipStream_t st) {
    with_states(N, [&](auto kn) {
        launch_block_bidir<Tin, decltype(kn)::value>(L, x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs, y, bounds,
                                                     hout, batch, T, D, Tc, n_chunks, h0_blocks, f, st);
    });
}

// ------------------------------------------------ explicit instantiations

template void launch_block_bidir_any<BDSSM_TIN>(int64_t, int64_t, const void *, const void *, const void *,
                                              const void *, const float *, const float *, const float *,
                                              int64_t, int64_t, void *, float *, float *, int64_t, int64_t,
                                              int64_t, int64_t, int, const float *, const Fuse &, hipStream_t);
template void launch_block_lane<BDSSM_TIN, false>(int64_t, const void *, const void *, const void *, const void *,
                                               const float *, const float *, float *, void *, int64_t, int64_t,
                                               int64_t, const Fuse &, hipStream_t);
template void launch_block_lane<BDSSM_TIN, true>(int64_t, const void *, const void *, const void *, const void *,
                                              const float *, const float *, float *, void *, int64_t, int64_t,
                                              int64_t, const Fuse &, hipStream_t);

}  // namespace bdssm_host
