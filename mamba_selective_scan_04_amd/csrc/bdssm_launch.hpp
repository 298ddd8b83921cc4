// bdssm_launch.hpp -- host-side launch policy shared by the translation
// units of libbdssm: chunk plans, workspace layouts, the resolved fusion
// arguments and the launchers of each kernel family.  The launchers are
// defined in launch_*.hip (each compiled once per stream type, float and
// bf16 stored as uint16_t) and called by the entry points in bdssm.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "bdssm.h"
#include "bdssm_bwd_kernels.hpp"
#include "bdssm_kernels.hpp"

namespace bdssm_host {

using namespace bdssm_dev;

// 256 CUs x 4 SIMDs x the chunk kernel's resident waves per SIMD
constexpr int64_t kFineWaves = 256 * 4 * kChunkWaves;
// workgroups of the bidirectional kernel resident at once (two 4-wave
// workgroups per CU at its register use)
constexpr int64_t kCoarseGroups = 512;
// issue slots of the adjoint pre-pass per token relative to the backward pass
constexpr double kBwdPrepassWeight = 0.2;

// ------------------------------------------------------------ launch policy
//
// Chunking of the time axis.  The per-token loop is sequential per channel,
// so a launch has batch * ceil(D/64) waves per chunk; long sequences are cut
// into chunks until the chip is full.
//   fine chunks  (one wave per 64 channels, 16 states per lane): at most
//                kFineWaves waves, the number resident at once (kChunkWaves per SIMD),
//                so the launch runs in a single round with no tail.
//   coarse chunks (bidirectional pass, 4 independent waves per 64
//                channels): count chosen by a small cost model (below) against
//                kCoarseGroups resident workgroups; each is a whole number of
//                fine chunks so its incoming state is a fine-chunk boundary.
// Every chunk is a multiple of 16 tokens, so blocks of L | 16 never straddle.
// BDSSM_FINE_WAVES / BDSSM_COARSE_GROUPS / BDSSM_CHUNK (fine chunk length in
// tokens) / BDSSM_COARSE_CHUNKS override the targets; they exist for tuning
// sweeps and for the chunk-invariance tests.
struct Plan {
    int64_t fine_len;    // tokens per fine chunk (multiple of 16)
    int n_fine;          // number of fine chunks
    int per_coarse;      // fine chunks per coarse chunk
    int n_coarse;        // number of coarse chunks
};

inline int64_t env_int(const char *name, int64_t dflt) {
    const char *s = getenv(name);
    if (s == nullptr || *s == 0) return dflt;
    char *end = nullptr;
    long long v = strtoll(s, &end, 10);
    return (end != s && v > 0) ? (int64_t)v : dflt;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// prepass_weight: issue slots of the chunk pre-pass per token relative to
// the main pass (forward aggregates vs the bidirectional pass ~0.45; adjoint
// aggregates vs the backward pass ~0.2).
// coarse_ch / coarse_cap: channels per workgroup of the coarse pass and how
// many of its workgroups are resident at once (the forward wave kernel: 64,
// 512; bwd_pair_kernel: 32, 768).
// fill_prepass (the training forms): with several coarse chunks the pre-pass
// covers only (nc - 1) / nc of the fine chunks, so the fine chunks are cut
// shorter until the pre-pass alone fills one round of resident waves.
inline Plan make_plan(int64_t batch, int64_t D, int64_t T, double prepass_weight = 0.45,
               int64_t coarse_ch = kWave, int64_t coarse_cap = kCoarseGroups, bool one_round = false,
               bool fill_prepass = false) {
    Plan p{};
    const int64_t groups = batch * ceil_div(D, kWave);          // fine pass: one wave per 64 channels
    const int64_t cgroups = batch * ceil_div(D, coarse_ch);     // coarse pass workgroups per chunk
    const int64_t ngroups16 = ceil_div(T, kGroup);
    if (T == 0 || groups == 0) {
        p.fine_len = kGroup; p.n_fine = 1; p.per_coarse = 1; p.n_coarse = 1;
        return p;
    }
    const int64_t fine_waves = env_int("BDSSM_FINE_WAVES", kFineWaves);
    const int64_t coarse_groups = env_int("BDSSM_COARSE_GROUPS", coarse_cap);
    // one round of resident waves: never more chunks than fit at once
    int64_t nf = fine_waves / groups;
    if (nf > ngroups16) nf = ngroups16;
    if (nf < 1) nf = 1;
    int64_t fl = ceil_div(ngroups16, nf) * kGroup;
    const int64_t forced = env_int("BDSSM_CHUNK", 0);
    if (forced > 0) fl = ceil_div(forced, kGroup) * kGroup;
    if (ceil_div(T, fl) > 65535) fl = ceil_div(ceil_div(T, 65535), kGroup) * kGroup;
    // every chunk's rows of one stream must stay below 2^31 bytes (32-bit
    // buffer offsets); 4 bytes per element covers both dtypes
    const int64_t max_tok = ((((int64_t)1 << 31) - 1) / (D * 4)) / kGroup * kGroup;
    if (fl > max_tok) fl = max_tok;
    nf = ceil_div(T, fl);
    // Coarse chunk count: each extra chunk adds parallelism to the
    // bidirectional pass but costs a forward pre-pass over its tokens.
    // Estimated time, in units of "one resident wave of workgroups scanning
    // the whole sequence": ceil(groups * nc / capacity) / nc for the pass
    // itself, plus the pre-pass over (nc - 1) / nc of the tokens at full
    // occupancy, weighted by its share of issue slots (~0.45).
    int64_t nc = 1;
    double best = 1e30;
    for (int64_t cand = 1; cand <= 32 && cand <= nf; ++cand) {
        const double rounds = (double)ceil_div(cgroups * cand, coarse_groups);
        const double est = rounds / cand + prepass_weight * (double)(cand - 1) / cand * (double)cgroups / coarse_groups;
        if (est < best - 1e-9) { best = est; nc = cand; }
    }
    // one_round: the most coarse chunks whose workgroups are all resident at
    // once (a pass that keeps its SIMDs busy at three of its four resident
    // workgroups per CU loses more to a partly filled second round than it
    // gains from the extra ones)
    if (one_round && cgroups <= coarse_groups) {
        nc = coarse_groups / cgroups;
        if (nc > 32) nc = 32;
        if (nc > nf) nc = nf;
    }
    const int64_t forced_nc = env_int("BDSSM_COARSE_CHUNKS", 0);
    if (forced_nc > 0) nc = forced_nc < nf ? forced_nc : nf;
    // BDSSM_FILL_PREPASS=0 keeps the inference plan's fine chunks (tests)
    const char *fp = getenv("BDSSM_FILL_PREPASS");
    if (fill_prepass && nc > 1 && forced == 0 && !(fp != nullptr && fp[0] == '0')) {
        int64_t nf2 = ceil_div(fine_waves * nc, (nc - 1) * groups);
        if (nf2 > ngroups16) nf2 = ngroups16;
        if (nf2 > nf) {
            const int64_t fl2 = ceil_div(ngroups16, nf2) * kGroup;
            if (ceil_div(T, fl2) <= 65535) {
                fl = fl2;
                nf = ceil_div(T, fl);
            }
        }
    }
    int64_t per = ceil_div(nf, nc);
    if (per * fl > max_tok) per = max_tok / fl;
    nc = ceil_div(nf, per);
    p.fine_len = fl;
    p.n_fine = (int)nf;
    p.per_coarse = (int)per;
    p.n_coarse = (int)nc;
    return p;
}

// Block lengths the register-resident wave kernels take (L divides their
// 16-token group); every other L up to kMaxLdsBlock goes to block_bidir_kernel.
inline bool wave_block(int64_t L) { return L == 1 || L == 2 || L == 4 || L == 8 || L == 16; }

// State counts the library is built for.  16 runs everything; the others run
// the one-lane-per-channel kernels (chunk scan, carry, block_bidir_kernel,
// the baseline's sweeps), whose templates are instantiated for each.
inline bool supported_states(int64_t N) { return N == 4 || N == 8 || N == 16 || N == 32; }

// Whether a bidirectional pass runs the register-resident wave kernels.
inline bool wave_path(int64_t L, int64_t N) { return N == kStates && wave_block(L); }

// The register-resident bidirectional pass with shared operands runs
// bidir_pair_kernel (two states per lane); BDSSM_BIDIR_KERNEL=wave keeps it on
// bidir_wave_kernel (four states per lane; tests).  Separate reverse operands
// always take bidir_wave_kernel<..., 2>.
inline bool pair_bidir() {
    const char *v = getenv("BDSSM_BIDIR_KERNEL");
    return !(v != nullptr && v[0] == 'w');
}
// workgroups of bidir_pair_kernel resident at once (three per CU: its
// registers)
constexpr int64_t kPairGroups = 3 * 256;
// Whether a bidirectional pass with shared operands can run bidir_pair_kernel
// (block lengths dividing the 16-token group, any supported state count), and
// its channels per workgroup (4 waves x 64 lanes / (N / 2) lanes per channel).
inline bool pair_path(int64_t L, int64_t N) { return wave_block(L) && supported_states(N); }
// Long blocks in bidir_pair_kernel (L = 0 mode, chunks of whole blocks):
// multiples of 16 from 32 to kLongMax, any supported state count.
inline bool pair_long(int64_t L, int64_t N) {
    return L > kGroup && L <= kLongMax && L % kGroup == 0 && supported_states(N);
}
inline int64_t pair_channels_of(int64_t N) { return 8 * kWave / N; }

// f(std::integral_constant<int, N>) for a supported state count N.
template <typename F> void with_states(int64_t N, F &&f) {
    switch (N) {
    case 4: f(std::integral_constant<int, 4>()); break;
    case 8: f(std::integral_constant<int, 8>()); break;
    case 32: f(std::integral_constant<int, 32>()); break;
    default: f(std::integral_constant<int, 16>()); break;
    }
}

// Chunking of the two-stream forms: blocks are independent, so chunks only
// add parallelism (no carry); aim for about four rounds of resident
// workgroups.  Returns false if the chunk count exceeds the grid limit.
// Block lengths outside the wave kernels' set round the chunk up to whole
// blocks (one wave per 64 channels there, so four times the chunks).
inline bool blocks_plan(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, int64_t *tc_out,
                 int64_t *nc_out, int64_t coarse_ch = kWave, int64_t coarse_cap = kCoarseGroups) {
    const bool wave = pair_path(L, N) || (pair_long(L, N) && coarse_ch == pair_channels_of(N));
    const int64_t unit = pair_path(L, N) ? kGroup : L;
    const int64_t groups = batch * ceil_div(D, coarse_ch);
    const int64_t nunits = ceil_div(T, unit);
    int64_t nc = ceil_div((wave ? 4 : 16) * coarse_cap, groups);
    if (nc > nunits) nc = nunits;
    if (nc < 1) nc = 1;
    int64_t tc = ceil_div(nunits, nc) * unit;
    const int64_t max_tok = ((((int64_t)1 << 31) - 1) / (D * 4)) / unit * unit;
    if (max_tok < unit) return false;
    if (tc > max_tok) tc = max_tok;
    nc = ceil_div(T, tc);
    *tc_out = tc;
    *nc_out = nc;
    return nc <= 65535;
}

// Chunking for the other block lengths: chunks are whole numbers of blocks,
// about as long as make_plan's fine chunks, all aggregated by the forward
// pre-pass and each scanned by one block_bidir_kernel workgroup column.
// Returns false if no such chunking fits the grid or the 32-bit offsets.
inline bool plan_general(int64_t batch, int64_t D, int64_t T, int64_t L, Plan *out) {
    const Plan base = make_plan(batch, D, T);
    int64_t tc = ceil_div(base.fine_len, L) * L;
    const int64_t max_tok = (((int64_t)1 << 31) - 1) / (D * 4);
    if (tc > max_tok) tc = (max_tok / L) * L;
    if (tc < L || T == 0) { if (T != 0) return false; tc = L; }
    const int64_t n = T == 0 ? 1 : ceil_div(T, tc);
    if (n > 65535) return false;
    out->fine_len = tc;
    out->n_fine = (int)n;
    out->per_coarse = 1;
    out->n_coarse = (int)n;
    return true;
}

// The long-block pair plan: the pair kernel's coarse chunk count (one round
// of resident workgroups), every fine chunk a whole number of blocks, so that
// the coarse chunks are too.  Returns false if the chunking does not fit the
// grid or the 32-bit offsets.
inline int64_t pair_long_capacity(int64_t L, int64_t N) {
    // workgroups per CU by LDS: the rows (x, dt, z double-buffered per wave;
    // B, C double-buffered) and the walk's saved states, at most three (the
    // registers)
    const int64_t lds = 1536 * (8 * kWave / N / 4) + 256 * N + (int64_t)pair_long_lds(L);
    int64_t per_cu = (160 * 1024) / lds;
    if (per_cu > 3) per_cu = 3;
    if (per_cu < 1) per_cu = 1;
    return per_cu * 256;
}
inline bool plan_long(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, Plan *out) {
    const Plan base = make_plan(batch, D, T, 0.45, pair_channels_of(N), pair_long_capacity(L, N), true);
    if (T == 0) { *out = base; return true; }
    const int64_t max_tok = ((((int64_t)1 << 31) - 1) / (D * 4)) / L * L;
    int64_t fl = ceil_div(base.fine_len, L) * L;
    if (fl > max_tok) fl = max_tok;
    if (fl < L) return false;
    const int64_t nf = ceil_div(T, fl);
    int64_t per = ceil_div(nf, base.n_coarse);
    if (per * fl > max_tok) per = max_tok / fl;
    if (per < 1) per = 1;
    const int64_t nc = ceil_div(nf, per);
    if (nf > 65535 || nc > 65535) return false;
    out->fine_len = fl;
    out->n_fine = (int)nf;
    out->per_coarse = (int)per;
    out->n_coarse = (int)nc;
    return true;
}

// The plan of the forward entry points for block length L, N states.
inline bool plan_for(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, Plan *out, bool train = false) {
    if (pair_path(L, N)) {
        // the training plans' shorter pre-pass chunks: measured faster at 8 to 32
        // states, slower at 4 (1.035 against 1.020 ms for the 87M all-block step)
        *out = make_plan(batch, D, T, 0.45, pair_channels_of(N), kPairGroups, true, train && N >= 8);
        return true;
    }
    if (pair_long(L, N) && pair_bidir()) return plan_long(batch, D, T, L, N, out);
    return plan_general(batch, D, T, L, out);
}

// Workspace layout (fp32 arrays, each 256-byte aligned):
//   agg_h [batch, n_fine, D, N], agg_s [batch, n_fine, D], h_in [batch, n_fine, D, N]
//   full scan adds ragg_h, ragg_s, hr_in (same sizes) and yf [batch, T, D].
struct Workspace {
    float *agg_h, *agg_s, *h_in, *ragg_h, *ragg_s, *hr_in, *yf;
    size_t bytes;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Backward workspace (fp32, 256-byte aligned):
//   continuous form with several coarse chunks: agg_q [batch, n_fine, D, N],
//     agg_s [batch, n_fine, D], q_in [batch, n_fine, D, N];
//   both forms: part_bc [batch, nblk, T, 2N] (nblk = channel blocks of the
//     block-local kernel), part_a [batch, nc, D, N],
//     part_bias [batch, nc, D] (the dt_bias gradient of the fused backward),
//     part_d [batch, nc, D]   (nc = coarse chunks of the backward pass);
//   separate reverse operands: part_bc_r, part_a_r, part_bias_r (sizes as above);
//   long blocks (L a multiple of 16 above 16, 16 states): gstate
//     [batch, ceil(T/16), 2, D, 16] (group_state_kernel).
struct BwdWorkspace {
    float *agg_q, *agg_s, *q_in, *part_bc, *part_a, *part_d, *part_bias;
    float *part_bc_r, *part_a_r, *part_bias_r;    // separate reverse operands only
    float *gstate;                                // long blocks only
    size_t bytes;
};

// block lengths that bwd_pair_kernel<..., 0, ...> takes: multiples of the
// 16-token group above it, 16 states, shared operands
inline bool long_block(int64_t L, int64_t N, bool sep = false) {
    return !sep && N == kStates && L > kGroup && L % kGroup == 0;
}

inline BwdWorkspace layout_bwd(void *base, int64_t batch, int64_t D, int64_t T, int64_t n_fine,
                        int64_t nc, bool carry, int64_t N, int64_t nblk, bool sep = false,
                        int64_t L = 0) {
    BwdWorkspace w{};
    size_t off = 0;
    auto take = [&](size_t n) -> float * {
        float *r = base ? reinterpret_cast<float *>(static_cast<char *>(base) + off) : nullptr;
        off += align256(n);
        return r;
    };
    if (carry) {
        const size_t nh = (size_t)batch * n_fine * D * N * sizeof(float);
        w.agg_q = take(nh);
        w.agg_s = take((size_t)batch * n_fine * D * sizeof(float));
        w.q_in = take(nh);
    }
    w.part_bc = take((size_t)batch * nblk * T * 2 * N * sizeof(float));
    w.part_a = take((size_t)batch * nc * D * N * sizeof(float));
    w.part_d = take((size_t)batch * nc * D * sizeof(float));
    w.part_bias = take((size_t)batch * nc * D * sizeof(float));
    if (sep) {
        w.part_bc_r = take((size_t)batch * nblk * T * 2 * N * sizeof(float));
        w.part_a_r = take((size_t)batch * nc * D * N * sizeof(float));
        w.part_bias_r = take((size_t)batch * nc * D * sizeof(float));
    }
    if (long_block(L, N, sep)) w.gstate = take((size_t)batch * ceil_div(T, kGroup) * 2 * D * kStates * sizeof(float));
    w.bytes = off;
    return w;
}

inline Workspace layout_ws(void *base, int64_t batch, int64_t D, int64_t N, int64_t T, const Plan &p,
                    int op) {
    Workspace w{};
    const size_t nh = (size_t)batch * p.n_fine * D * N * sizeof(float);
    const size_t ns = (size_t)batch * p.n_fine * D * sizeof(float);
    size_t off = 0;
    auto take = [&](size_t n) -> float * {
        float *r = base ? reinterpret_cast<float *>(static_cast<char *>(base) + off) : nullptr;
        off += align256(n);
        return r;
    };
    const bool chunked = p.n_fine > 1;
    if (op == BDSSM_OP_PREFILL || op == BDSSM_OP_TRAIN) {
        if (chunked) { w.agg_h = take(nh); w.agg_s = take(ns); w.h_in = take(nh); }
    } else if (op == BDSSM_OP_FULL) {
        w.agg_h = take(nh); w.agg_s = take(ns); w.h_in = take(nh);
        w.ragg_h = take(nh); w.ragg_s = take(ns); w.hr_in = take(nh);
        w.yf = take((size_t)batch * T * D * sizeof(float));
    }
    w.bytes = off;
    return w;
}

inline dim3 grid3(int64_t D, int64_t chunks, int64_t batch) {
    return dim3((unsigned)ceil_div(D, kWave), (unsigned)chunks, (unsigned)batch);
}


// ---------------------------------------------------------------- launchers

// The optional Mamba-1 fusions of one call, resolved from bdssm_fusion.
struct Fuse {
    const float *dt_bias = nullptr;
    int dt_mode = kDtPlain;
    const void *z = nullptr;
    // separate reverse-direction operands (dt_r == nullptr: shared)
    const void *dt_r = nullptr, *B_r = nullptr, *C_r = nullptr;
    const float *A_r = nullptr, *dt_bias_r = nullptr;
    bool any() const { return dt_mode != kDtPlain || z != nullptr || dt_r != nullptr; }
    template <typename Tin> FuseArgs<Tin> args() const {
        return FuseArgs<Tin>{dt_bias, dt_mode, (const Tin *)z, (const Tin *)dt_r,
                             (const Tin *)B_r, (const Tin *)C_r, A_r, dt_bias_r};
    }
    // the operands of the reverse direction, as a plain (unfused-reverse) Fuse
    // for the baseline's reverse passes: its own bias, the same transform
    Fuse reverse() const {
        Fuse r = *this;
        if (dt_r != nullptr) {
            r.dt_bias = dt_bias_r;
            r.dt_mode = dt_mode == kDtSoftplus ? kDtSoftplus : (dt_bias_r != nullptr ? kDtBias : kDtPlain);
        }
        r.dt_r = r.B_r = r.C_r = nullptr;
        r.A_r = r.dt_bias_r = nullptr;
        return r;
    }
};

inline Fuse resolve_fusion(const bdssm_fusion *f, bool with_y) {
    Fuse r;
    if (f == nullptr) return r;
    r.dt_bias = f->dt_bias;
    r.dt_mode = f->dt_softplus ? kDtSoftplus : (f->dt_bias != nullptr ? kDtBias : kDtPlain);
    r.z = with_y ? f->z : nullptr;
    if (with_y && f->dt_rev != nullptr) {
        r.dt_r = f->dt_rev; r.B_r = f->B_rev; r.C_r = f->C_rev;
        r.A_r = f->A_rev; r.dt_bias_r = f->dt_bias_rev;
        // a reverse bias needs the biased transform even when the forward
        // direction has none (its bias then reads as zero)
        if (r.dt_mode == kDtPlain && r.dt_bias_r != nullptr) r.dt_mode = kDtBias;
    }
    return r;
}

// Whether a single-block call runs block_lane_kernel.  Measured on MI355X
// (65K context, batch 8, graph replays): the state-only commit takes 4.5 us
// there against 5.8 us on the one-lane-per-channel chunk kernel, but the block
// step takes 5.1 us against 4.3 us on bidir_wave_kernel, whose row DMA beats
// the lane kernel's per-lane loads; so only the state-only commit uses it.
// BDSSM_BLOCK_KERNEL=lane / wave forces one path (comparison and tests).
inline bool block_lane_path(int64_t L, const Fuse &f, bool with_y) {
    if (L > kGroup || f.dt_r != nullptr) return false;
    const char *v = getenv("BDSSM_BLOCK_KERNEL");
    if (v != nullptr && v[0] == 'w') return false;
    if (v != nullptr && v[0] == 'l') return true;
    return !with_y;
}

struct BwdArgs {
    const void *x, *dt, *B, *C, *dy;
    const float *A, *Dskip, *h_start, *qin, *dbounds;
    int64_t qin_bs, qin_cs;
    void *dx, *ddt;
    float *part_bc, *part_a, *part_d, *dh0;
    // the fused forward's gradients (fused: any of them in use)
    bool fused = false;
    const float *dt_bias = nullptr;
    int dt_mode = kDtPlain;
    const void *z = nullptr;
    void *dz = nullptr;
    float *part_bias = nullptr;
    // separate reverse operands (sep), their gradients and partials
    bool sep = false;
    const void *dt_r = nullptr, *B_r = nullptr, *C_r = nullptr;
    const float *A_r = nullptr, *dt_bias_r = nullptr;
    void *ddt_r = nullptr;
    float *part_bc_r = nullptr, *part_a_r = nullptr, *part_bias_r = nullptr;
};

// BDSSM_BWD_KERNEL=general keeps every backward on bwd_general_kernel (tests).
inline bool bwd_force_general() {
    const char *v = getenv("BDSSM_BWD_KERNEL");
    return v != nullptr && v[0] == 'g';
}

// The backward's block-local kernel for L | 16.  bwd_pair_kernel (two states
// per lane, the whole 16-token group held in registers, 512 / N channels per
// workgroup) takes every supported state count; at 16 states and L <= 4 the
// four-state bwd_wave_kernel (segment recomputation, 64 channels per
// workgroup) is faster, since the pair kernel's per-block loads spill there
// (measured on MI355X).  BDSSM_BWD_KERNEL=wave / pair forces one of them at
// 16 states (tuning and tests).
inline bool bwd_use_wave(int64_t L, bool fused = false, int64_t N = kStates) {
    if (fused || N != kStates) return false;   // only bwd_pair_kernel has the fused variant and N != 16
    const char *v = getenv("BDSSM_BWD_KERNEL");
    if (v != nullptr && v[0] == 'w') return true;
    if (v != nullptr && v[0] == 'p') return false;
    return L < 8;
}

// channels per workgroup of the chosen kernel (the dB / dC partial blocks)
inline int64_t bwd_block_channels(int64_t L, bool fused = false, int64_t N = kStates) {
    return bwd_use_wave(L, fused, N) ? kWave : pair_channels_of(N);
}

// workgroups of the chosen kernel resident at once: bwd_pair_kernel fits
// three per CU (148-168 registers, 32-48 KB LDS at 16 states), bwd_wave_kernel
// two
inline int64_t bwd_block_capacity(int64_t L, bool fused = false, int64_t N = kStates) {
    return bwd_use_wave(L, fused, N) ? kCoarseGroups : 3 * 256;
}

// Long blocks (multiples of 16 above 16 at 16 states) take bwd_pair_kernel
// with group states from group_state_kernel.
inline bool bwd_long(int64_t L, int64_t N, bool sep = false) {
    return long_block(L, N, sep) && !bwd_force_general();
}

// The general backward path (bwd_general_kernel): block lengths outside the
// 16-token group's divisors and its multiples, and multiples of 16 at state
// counts other than 16.  Separate reverse operands always take it
// (bwd_general_kernel<..., 2>).
inline bool bwd_general(int64_t L, int64_t N, bool sep = false) {
    return sep || bwd_force_general() || (!(wave_block(L) && supported_states(N)) && !bwd_long(L, N));
}

// channels per workgroup of the block-local kernel (the dB / dC partial blocks)
inline int64_t bwd_channels(int64_t L, int64_t N, bool fused, bool sep = false) {
    if (sep) return bwd_general_waves<2>() * kWave / N;
    if (bwd_long(L, N)) return kPairChannels;
    return bwd_general(L, N) ? bwd_general_waves<0>() * kWave / N : bwd_block_channels(L, fused, N);
}

// chunk plans of the two backward forms, for the chosen kernel's geometry.
// The general path's chunks are whole blocks (its own adjoint pre-pass and
// the carry join them), as in the forward's general plan.
inline bool bwd_plan(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, bool fused, Plan *p,
              bool sep = false) {
    if (bwd_general(L, N, sep) || bwd_long(L, N, sep)) return plan_general(batch, D, T, L, p);
    *p = make_plan(batch, D, T, kBwdPrepassWeight, bwd_block_channels(L, fused, N),
                   bwd_block_capacity(L, fused, N), false, N >= 8);
    return true;
}
inline bool bwd_blocks_plan(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, int64_t *tc,
                     int64_t *nc, bool fused, bool sep = false) {
    if (bwd_general(L, N, sep) || bwd_long(L, N, sep))
        return blocks_plan(batch, D, T, L, N, tc, nc, bwd_channels(L, N, fused, sep), 3 * 256);
    return blocks_plan(batch, D, T, L, N, tc, nc, bwd_block_channels(L, fused, N),
                       bwd_block_capacity(L, fused, N));
}

// dynamic LDS of bwd_general_kernel: hf and pr at every 16-token segment start
inline size_t bwd_general_lds(int64_t L, int nw) { return (size_t)ceil_div(L, kGroup) * nw * 2 * kWave * sizeof(float); }

// ---------------------------------------------------------------- launchers
// (definitions in launch_*.hip; explicit instantiations for float and uint16_t)

// Chunk-local scans of n_launch chunks (N states per channel); sout == nullptr
// is the direct pass from h0 into hout (one chunk).          launch_chunk.hip
template <typename Tin>
void launch_chunk_state(bool rev, const void *x, const void *dt, const void *B, const float *A,
                        const float *h0, float *hout, float *sout, int64_t batch, int64_t T,
                        int64_t D, int64_t N, int64_t Tc, int n_chunks, int c_first, int n_launch,
                        hipStream_t st, const Fuse &f = Fuse());

// Forward and reverse chunk aggregates in one pass (the baseline with shared
// operands; sout serves both carries).                      launch_chunk.hip
template <typename Tin>
void launch_chunk_both(const void *x, const void *dt, const void *B, const float *A, float *hout, float *sout,
                       float *rout, int64_t batch, int64_t T, int64_t D, int64_t N, int64_t Tc, int n_chunks,
                       hipStream_t st, const Fuse &f = Fuse());

// The baseline's output sweeps.                               launch_chunk.hip
template <typename Tin>
void launch_sweep(bool rev, const void *x, const void *dt, const void *B, const void *C,
                  const float *A, const float *Dskip, const float *hin, float *yf, void *y,
                  int64_t batch, int64_t T, int64_t D, int64_t N, int64_t Tc, int n_chunks,
                  hipStream_t st, const Fuse &f = Fuse());

// Carry of chunk aggregates (forward, or the adjoint's reverse).  bdssm.hip
void launch_carry(bool rev, const float *agg_h, const float *agg_s, const float *A,
                  const float *h_init, float *h_in, float *h_final, int64_t batch, int64_t D,
                  int64_t N, int n_chunks, int n_agg, hipStream_t st, int c_low = 0);

// The bidirectional pass: the wave kernels for N = 16 and L | 16, else
// launch_block_bidir_any (Tc then a multiple of L).           launch_bidir.hip
template <typename Tin>
void launch_bidir(int64_t L, const void *x, const void *dt, const void *B, const void *C,
                  const float *A, const float *Dskip, const float *hin, int64_t hin_bs,
                  int64_t hin_cs, void *y, float *bounds, float *hout, int64_t batch, int64_t T,
                  int64_t D, int64_t N, int64_t Tc, int n_chunks, hipStream_t st,
                  const float *h0_blocks = nullptr, const Fuse &f = Fuse());

// Bidirectional pass of the one-lane-per-channel kernels (any L up to
// kMaxLdsBlock, N states), or block_split_kernel for one block per row.
//                                                             launch_block.hip
template <typename Tin>
void launch_block_bidir_any(int64_t N, int64_t L, const void *x, const void *dt, const void *B,
                            const void *C, const float *A, const float *Dskip, const float *hin,
                            int64_t hin_bs, int64_t hin_cs, void *y, float *bounds, float *hout,
                            int64_t batch, int64_t T, int64_t D, int64_t Tc, int n_chunks,
                            const float *h0_blocks, const Fuse &f, hipStream_t st);

// One block from the cache on block_lane_kernel.              launch_block.hip
template <typename Tin, bool kCommit>
void launch_block_lane(int64_t N, const void *x, const void *dt, const void *B, const void *C,
                       const float *A, const float *Dskip, float *h_cache, void *y, int64_t batch,
                       int64_t D, int64_t L, const Fuse &f, hipStream_t st);

// Adjoint aggregates of n_launch fine chunks.                 launch_bwd.hip
template <typename Tin>
void launch_adjoint_chunk(const void *dt, const void *dy, const void *C, const float *A,
                          const float *dbounds, float *qout, float *sout, int64_t batch, int64_t T,
                          int64_t D, int64_t L, int64_t Tc, int n_chunks, int c_first, int n_launch,
                          hipStream_t st, int dt_mode = kDtPlain, const float *dt_bias = nullptr,
                          const void *z = nullptr);

// The block-local backward kernels (L | 16, N states).         launch_bwd.hip
template <typename Tin, bool kBlockInit>
void launch_bwd(int64_t L, int64_t N, const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t Tc,
                int nc, hipStream_t st);

// Long blocks: group states, then bwd_pair_kernel.            launch_bwd.hip
template <typename Tin, bool kBlockInit>
void launch_bwd_long(const BwdArgs &a, float *gstate, int64_t batch, int64_t T, int64_t D, int64_t L,
                     int64_t Tc, int nc, hipStream_t st);

// Ordered reductions of the dB / dC and parameter partials.  launch_bwd.hip
template <typename Tin>
void launch_bwd_reduce(const BwdWorkspace &w, void *dB, void *dC, float *dA, float *dDskip,
                       int64_t batch, int64_t T, int64_t D, int64_t L, int64_t N, int64_t nc,
                       hipStream_t st, bool fused = false, float *d_bias = nullptr,
                       const bdssm_fusion_grads *gr = nullptr);

// The general backward kernel.                          launch_bwd_general.hip
template <typename Tin, bool kBlockInit>
void launch_bwd_general(int64_t N, const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t L,
                        int64_t Tc, int nc, hipStream_t st);

// Chunk-local adjoints of the general path.             launch_bwd_general.hip
template <typename Tin>
void launch_adjoint_general(int64_t N, const void *dt, const void *dy, const void *C, const float *A,
                            const float *dbounds, float *qout, float *sout, int64_t batch, int64_t T,
                            int64_t D, int64_t L, int64_t Tc, int n_chunks, int c_first, int n_launch,
                            int dt_mode, const float *dt_bias, const void *z, hipStream_t st);

}  // namespace bdssm_host
