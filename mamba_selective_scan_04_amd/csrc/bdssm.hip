// bdssm.hip -- C ABI, argument checks and launch policy of the
// block-restricted bidirectional selective scan on MI355X (gfx950).
//
// Pages cited (arXiv 2607.02805, "Training Hybrid Block Diffusion Language
// Models with Partial Bidirectionality"):
//   [ABS]  the paper's abstract (newx.sg page, "Abstract").
//   [DE-M] gist.science German page, "Technische Zusammenfassung" > "Methodik".
//   [DE-P] same page, "Problemstellung".
//
// Each entry point validates every argument on the host before the first HIP
// call, then enqueues a fixed sequence of kernels on the caller's stream:
//   prefill (state only): chunk aggregates + carry            [DE-M] cache built
//                                                             from the clean prefix
//   prefill (with y), train_scan: chunk aggregates + carry + bidirectional pass
//   block_step: one bidirectional pass over one block from the cache [ABS]
//   commit: one forward pass over one block, cache updated in place [DE-M]
//   full_scan (baseline): forward and reverse aggregates + both carries +
//                         a forward output sweep + a reverse output sweep [DE-P]
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <initializer_list>
#include <type_traits>

#include "bdssm.h"
#include "bdssm_bwd_kernels.hpp"
#include "bdssm_kernels.hpp"



using namespace bdssm_dev;

namespace {

constexpr int kVersion = 10600;   // 1.6.0

// 256 CUs x 4 SIMDs x 8 resident waves (the chunk kernel fits in 64 VGPRs)
constexpr int64_t kFineWaves = 256 * 4 * 8;
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
//                kFineWaves waves, the number resident at once (8 per SIMD),
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

int64_t env_int(const char *name, int64_t dflt) {
    const char *s = getenv(name);
    if (s == nullptr || *s == 0) return dflt;
    char *end = nullptr;
    long long v = strtoll(s, &end, 10);
    return (end != s && v > 0) ? (int64_t)v : dflt;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// prepass_weight: issue slots of the chunk pre-pass per token relative to
// the main pass (forward aggregates vs the bidirectional pass ~0.45; adjoint
// aggregates vs the backward pass ~0.2).
// coarse_ch / coarse_cap: channels per workgroup of the coarse pass and how
// many of its workgroups are resident at once (the forward wave kernel: 64,
// 512; bwd_pair_kernel: 32, 768).
Plan make_plan(int64_t batch, int64_t D, int64_t T, double prepass_weight = 0.45,
               int64_t coarse_ch = kWave, int64_t coarse_cap = kCoarseGroups) {
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
    const int64_t forced_nc = env_int("BDSSM_COARSE_CHUNKS", 0);
    if (forced_nc > 0) nc = forced_nc < nf ? forced_nc : nf;
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
bool wave_block(int64_t L) { return L == 1 || L == 2 || L == 4 || L == 8 || L == 16; }

// State counts the library is built for.  16 runs everything; the others run
// the one-lane-per-channel kernels (chunk scan, carry, block_bidir_kernel,
// the baseline's sweeps), whose templates are instantiated for each.
bool supported_states(int64_t N) { return N == 4 || N == 8 || N == 16 || N == 32; }

// Whether a bidirectional pass runs the register-resident wave kernels.
bool wave_path(int64_t L, int64_t N) { return N == kStates && wave_block(L); }

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
bool blocks_plan(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, int64_t *tc_out,
                 int64_t *nc_out, int64_t coarse_ch = kWave, int64_t coarse_cap = kCoarseGroups) {
    const bool wave = wave_path(L, N);
    const int64_t unit = wave ? kGroup : L;
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
bool plan_general(int64_t batch, int64_t D, int64_t T, int64_t L, Plan *out) {
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

// The plan of the forward entry points for block length L, N states.
bool plan_for(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, Plan *out) {
    if (wave_path(L, N)) { *out = make_plan(batch, D, T); return true; }
    return plan_general(batch, D, T, L, out);
}

// Workspace layout (fp32 arrays, each 256-byte aligned):
//   agg_h [batch, n_fine, D, N], agg_s [batch, n_fine, D], h_in [batch, n_fine, D, N]
//   full scan adds ragg_h, ragg_s, hr_in (same sizes) and yf [batch, T, D].
struct Workspace {
    float *agg_h, *agg_s, *h_in, *ragg_h, *ragg_s, *hr_in, *yf;
    size_t bytes;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

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
bool long_block(int64_t L, int64_t N, bool sep = false) {
    return !sep && N == kStates && L > kGroup && L % kGroup == 0;
}

BwdWorkspace layout_bwd(void *base, int64_t batch, int64_t D, int64_t T, int64_t n_fine,
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

Workspace layout_ws(void *base, int64_t batch, int64_t D, int64_t N, int64_t T, const Plan &p,
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

// ---------------------------------------------------------------- checking

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range { const void *p; size_t n; };

bool overlaps(Range a, Range b) {
    if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

int check_shape(const bdssm_shape *s) {
    if (s == nullptr) return BDSSM_ERR_NULL;
    if (s->dtype != BDSSM_F32 && s->dtype != BDSSM_BF16) return BDSSM_ERR_DTYPE;
    if (s->batch < 0 || s->d_inner < 0) return BDSSM_ERR_SHAPE;
    if (!supported_states(s->d_state)) return BDSSM_ERR_SHAPE;
    const int64_t L = s->block_len;
    if (L < 1 || (!wave_block(L) && L > kMaxLdsBlock)) return BDSSM_ERR_SHAPE;
    // d_inner bound keeps a 16-token group of one stream within 32-bit buffer offsets
    if (s->d_inner > (int64_t)1 << 24 || s->batch > 65535) return BDSSM_ERR_SHAPE;
    return BDSSM_OK;
}

size_t esize(const bdssm_shape *s) { return s->dtype == BDSSM_BF16 ? 2 : 4; }

// Shared checks of the per-token streams of one call covering T tokens.
int check_streams(const bdssm_shape *s, int64_t T, const void *x, const void *dt, const void *B,
                  const void *C, bool need_c, const float *A, const float *Dskip, bool need_dskip) {
    const bool nonempty = s->batch > 0 && s->d_inner > 0 && T > 0;
    if (!nonempty) return BDSSM_OK;
    if (!x || !dt || !B || !A || (need_c && !C) || (need_dskip && !Dskip)) return BDSSM_ERR_NULL;
    const void *ps[] = {x, dt, B, C, A, Dskip};
    for (const void *p : ps)
        if (p && !aligned16(p)) return BDSSM_ERR_ALIGN;
    if (T > ((int64_t)1 << 40) / (s->batch * s->d_inner)) return BDSSM_ERR_SHAPE;
    if (s->d_inner * ceil_div(T, kGroup) > ((int64_t)1 << 40)) return BDSSM_ERR_SHAPE;
    return BDSSM_OK;
}

// Outputs must not overlap any input.
int check_alias(const bdssm_shape *s, int64_t T, const void *x, const void *dt, const void *B,
                const void *C, const float *A, const float *Dskip, const float *h_src,
                std::initializer_list<Range> outs) {
    const size_t e = esize(s);
    const size_t nx = (size_t)s->batch * T * s->d_inner * e;
    const size_t N = (size_t)s->d_state;
    const size_t nb = (size_t)s->batch * T * N * e;
    const Range ins[] = {{x, nx}, {dt, nx}, {B, nb}, {C, nb},
                         {A, (size_t)s->d_inner * N * 4}, {Dskip, (size_t)s->d_inner * 4},
                         {h_src, (size_t)s->batch * s->d_inner * N * 4}};
    for (const Range &o : outs) {
        for (const Range &i : ins)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
    }
    // outputs among themselves
    const Range *ob = outs.begin();
    for (size_t i = 0; i < outs.size(); ++i)
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(ob[i], ob[j])) return BDSSM_ERR_ALIAS;
    return BDSSM_OK;
}

// Checks of the optional fusion arguments: 16-byte alignment, and no output
// may overlap dt_bias or z (z is read only when the call produces y).
int check_fusion(const bdssm_fusion *f, const bdssm_shape *s, int64_t T, bool with_y,
                 std::initializer_list<Range> outs) {
    if (f == nullptr) return BDSSM_OK;
    const bool rev = with_y && f->dt_rev != nullptr;
    if (rev && (f->B_rev == nullptr || f->C_rev == nullptr || f->A_rev == nullptr))
        return BDSSM_ERR_NULL;
    const void *ps[] = {f->dt_bias, with_y ? f->z : nullptr, rev ? f->dt_rev : nullptr,
                        rev ? f->B_rev : nullptr, rev ? f->C_rev : nullptr,
                        rev ? f->A_rev : nullptr, rev ? f->dt_bias_rev : nullptr};
    for (const void *p : ps)
        if (!aligned16(p)) return BDSSM_ERR_ALIGN;
    const size_t ntok = (size_t)s->batch * T * s->d_inner * esize(s);
    const size_t nbc = (size_t)s->batch * T * s->d_state * esize(s);
    const Range ins[] = {{f->dt_bias, (size_t)s->d_inner * 4},
                         {with_y ? f->z : nullptr, ntok},
                         {rev ? f->dt_rev : nullptr, ntok}, {rev ? f->B_rev : nullptr, nbc},
                         {rev ? f->C_rev : nullptr, nbc},
                         {rev ? f->A_rev : nullptr, (size_t)s->d_inner * s->d_state * 4},
                         {rev ? f->dt_bias_rev : nullptr, (size_t)s->d_inner * 4}};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
    return BDSSM_OK;
}

int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? BDSSM_OK : BDSSM_ERR_HIP;
}

// dst <- src (or zeros); src may equal dst.
int copy_or_zero(const float *src, float *dst, int64_t n, hipStream_t st) {
    (void)hipGetLastError();
    if (src == dst || n == 0) return BDSSM_OK;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, src,
                       dst, n);
    return launch_status();
}

dim3 grid3(int64_t D, int64_t chunks, int64_t batch) {
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

Fuse resolve_fusion(const bdssm_fusion *f, bool with_y) {
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
                        hipStream_t st, const Fuse &f = Fuse()) {
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

void launch_carry(bool rev, const float *agg_h, const float *agg_s, const float *A,
                  const float *h_init, float *h_in, float *h_final, int64_t batch, int64_t D,
                  int64_t N, int n_chunks, int n_agg, hipStream_t st, int c_low = 0) {
    const int64_t total = batch * D * N;
    const dim3 g((unsigned)ceil_div(total, 256));
    if (rev)
        hipLaunchKernelGGL((carry_kernel<true>), g, dim3(256), 0, st, agg_h, agg_s, A, h_init, h_in,
                           h_final, (int)batch, (int)D, (int)N, n_chunks, n_agg, c_low);
    else
        hipLaunchKernelGGL((carry_kernel<false>), g, dim3(256), 0, st, agg_h, agg_s, A, h_init, h_in,
                           h_final, (int)batch, (int)D, (int)N, n_chunks, n_agg, c_low);
}

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

// Whether a single-block call runs block_lane_kernel.  Measured on MI355X
// (65K context, batch 8, graph replays): the state-only commit takes 4.5 us
// there against 5.8 us on the one-lane-per-channel chunk kernel, but the block
// step takes 5.1 us against 4.3 us on bidir_wave_kernel, whose row DMA beats
// the lane kernel's per-lane loads; so only the state-only commit uses it.
// BDSSM_BLOCK_KERNEL=lane / wave forces one path (comparison and tests).
bool block_lane_path(int64_t L, const Fuse &f, bool with_y) {
    if (L > kGroup || f.dt_r != nullptr) return false;
    const char *v = getenv("BDSSM_BLOCK_KERNEL");
    if (v != nullptr && v[0] == 'w') return false;
    if (v != nullptr && v[0] == 'l') return true;
    return !with_y;
}

// Segment length of block_bidir_kernel for block length L and N states: small
// enough that the staged outputs (256 bytes per token) do not limit the
// workgroups per CU below what the registers allow (16 waves per CU at
// N <= 16: 32 tokens; 8 at N = 32: 64), no smaller, since every segment
// boundary adds state-only reverse work (measured on MI355X at the 87M
// training shape).  BDSSM_SEG overrides (tuning, tests).
int block_seg(int64_t L, int64_t N) {
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
bool use_split(int64_t L, int64_t N, int64_t T, int n_chunks, const float *bounds, const float *h0_blocks) {
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

// The bidirectional pass: the wave kernels for N = 16 and L | 16, else
// block_bidir_kernel (Tc then a multiple of L).
template <typename Tin>
void launch_bidir(int64_t L, const void *x, const void *dt, const void *B, const void *C,
                  const float *A, const float *Dskip, const float *hin, int64_t hin_bs,
                  int64_t hin_cs, void *y, float *bounds, float *hout, int64_t batch, int64_t T,
                  int64_t D, int64_t N, int64_t Tc, int n_chunks, hipStream_t st,
                  const float *h0_blocks = nullptr, const Fuse &f = Fuse()) {
    if (!wave_path(L, N)) {
        with_states(N, [&](auto kn) {
            launch_block_bidir<Tin, decltype(kn)::value>(L, x, dt, B, C, A, Dskip, hin, hin_bs, hin_cs,
                                                         y, bounds, hout, batch, T, D, Tc, n_chunks,
                                                         h0_blocks, f, st);
        });
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
                  hipStream_t st, const Fuse &f = Fuse()) {
    const dim3 g = grid3(D, n_chunks, batch);
    with_states(N, [&](auto kn) {
        constexpr int kN = decltype(kn)::value;
        if (rev) launch_sweep_k<Tin, true, kN>(g, x, dt, B, C, A, Dskip, hin, yf, y, T, D, Tc, n_chunks, f, st);
        else launch_sweep_k<Tin, false, kN>(g, x, dt, B, C, A, Dskip, hin, yf, y, T, D, Tc, n_chunks, f, st);
    });
}

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
                          hipStream_t st, int dt_mode = kDtPlain, const float *dt_bias = nullptr,
                          const void *z = nullptr) {
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

// The backward's block-local kernel.  bwd_pair_kernel (two states per lane,
// the whole 16-token group held in registers, 32 channels per workgroup) is
// the faster for L = 8 and 16; for L <= 4 its per-block loads spill and the
// four-state bwd_wave_kernel (segment recomputation, 64 channels per
// workgroup) is faster (measured on MI355X).  BDSSM_BWD_KERNEL=wave / pair
// forces one of them (tuning and tests).
bool bwd_use_wave(int64_t L, bool fused = false) {
    if (fused) return false;                 // only bwd_pair_kernel has the fused variant
    const char *v = getenv("BDSSM_BWD_KERNEL");
    if (v != nullptr && v[0] == 'w') return true;
    if (v != nullptr && v[0] == 'p') return false;
    return L < 8;
}

// channels per workgroup of the chosen kernel (the dB / dC partial blocks)
int64_t bwd_block_channels(int64_t L, bool fused = false) {
    return bwd_use_wave(L, fused) ? kWave : kPairChannels;
}

// workgroups of the chosen kernel resident at once: bwd_pair_kernel fits
// three per CU (168 registers, 44 KB LDS; 48 KB with the fused streams),
// bwd_wave_kernel two
int64_t bwd_block_capacity(int64_t L, bool fused = false) {
    return bwd_use_wave(L, fused) ? kCoarseGroups : 3 * 256;
}

// Long blocks (multiples of 16 above 16 at 16 states) take bwd_pair_kernel
// with group states from group_state_kernel; BDSSM_BWD_KERNEL=general sends
// them to bwd_general_kernel instead (tests).
bool bwd_long(int64_t L, int64_t N, bool sep = false) {
    if (!long_block(L, N, sep)) return false;
    const char *v = getenv("BDSSM_BWD_KERNEL");
    return !(v != nullptr && v[0] == 'g');
}

// The general backward path (bwd_general_kernel): block lengths outside the
// 16-token group's divisors and its multiples, and state counts other than 16.
// Separate reverse operands always take it (bwd_general_kernel<..., 2>).
bool bwd_general(int64_t L, int64_t N, bool sep = false) {
    return sep || (!(wave_block(L) && N == kStates) && !bwd_long(L, N));
}

// channels per workgroup of the block-local kernel (the dB / dC partial blocks)
int64_t bwd_channels(int64_t L, int64_t N, bool fused, bool sep = false) {
    if (sep) return bwd_general_waves<2>() * kWave / N;
    if (bwd_long(L, N)) return kPairChannels;
    return bwd_general(L, N) ? bwd_general_waves<0>() * kWave / N : bwd_block_channels(L, fused);
}

// chunk plans of the two backward forms, for the chosen kernel's geometry.
// The general path's chunks are whole blocks (its own adjoint pre-pass and
// the carry join them), as in the forward's general plan.
bool bwd_plan(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, bool fused, Plan *p,
              bool sep = false) {
    if (bwd_general(L, N, sep) || bwd_long(L, N, sep)) return plan_general(batch, D, T, L, p);
    *p = make_plan(batch, D, T, kBwdPrepassWeight, bwd_block_channels(L, fused),
                   bwd_block_capacity(L, fused));
    return true;
}
bool bwd_blocks_plan(int64_t batch, int64_t D, int64_t T, int64_t L, int64_t N, int64_t *tc,
                     int64_t *nc, bool fused, bool sep = false) {
    if (bwd_general(L, N, sep) || bwd_long(L, N, sep))
        return blocks_plan(batch, D, T, L, N, tc, nc, bwd_channels(L, N, fused, sep), 3 * 256);
    return blocks_plan(batch, D, T, L, kStates, tc, nc, bwd_block_channels(L, fused),
                       bwd_block_capacity(L, fused));
}

// dynamic LDS of bwd_general_kernel: hf and pr at every 16-token segment start
size_t bwd_general_lds(int64_t L, int nw) { return (size_t)ceil_div(L, kGroup) * nw * 2 * kWave * sizeof(float); }

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

template <typename Tin, int L, bool kBlockInit>
void launch_bwd_L(const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t Tc, int nc,
                  hipStream_t st) {
    if (bwd_use_wave(L, a.fused)) {
        hipLaunchKernelGGL((bwd_wave_kernel<Tin, L, kBlockInit>), grid3(D, nc, batch), dim3(4 * kWave), 0,
                           st, (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0, T,
                           (int)D, Tc);
        return;
    }
    const dim3 g((unsigned)ceil_div(D, kPairChannels), (unsigned)nc, (unsigned)batch);
    const BwdFuse<Tin> fz{a.dt_bias, a.dt_mode, (const Tin *)a.z, (Tin *)a.dz, a.part_bias};
    if (a.fused)
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, L, kBlockInit, true>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)nullptr, 0);
    else
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, L, kBlockInit, false>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)nullptr, 0);
}

template <typename Tin, bool kBlockInit>
void launch_bwd(int64_t L, const BwdArgs &a, int64_t batch, int64_t T, int64_t D, int64_t Tc,
                int nc, hipStream_t st) {
    switch (L) {
    case 1: launch_bwd_L<Tin, 1, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    case 2: launch_bwd_L<Tin, 2, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    case 4: launch_bwd_L<Tin, 4, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    case 8: launch_bwd_L<Tin, 8, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    default: launch_bwd_L<Tin, 16, kBlockInit>(a, batch, T, D, Tc, nc, st); break;
    }
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
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, 0, kBlockInit, true>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)gstate, (int)L);
    else
        hipLaunchKernelGGL((bwd_pair_kernel<Tin, 0, kBlockInit, false>), g, dim3(4 * kWave), 0, st,
                           (const Tin *)a.x, (const Tin *)a.dt, (const Tin *)a.B, (const Tin *)a.C,
                           (const Tin *)a.dy, a.A, a.Dskip, a.h_start, a.qin, a.qin_bs, a.qin_cs,
                           a.dbounds, (Tin *)a.dx, (Tin *)a.ddt, a.part_bc, a.part_a, a.part_d, a.dh0,
                           T, (int)D, Tc, fz, (const float *)gstate, (int)L);
}

template <typename Tin>
void launch_bwd_reduce(const BwdWorkspace &w, void *dB, void *dC, float *dA, float *dDskip,
                       int64_t batch, int64_t T, int64_t D, int64_t L, int64_t N, int64_t nc,
                       hipStream_t st, bool fused = false, float *d_bias = nullptr,
                       const bdssm_fusion_grads *gr = nullptr) {
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

// Forward state only over T tokens from h_init: h_final <- state after T.
template <typename Tin>
void run_state_only(const bdssm_shape *s, int64_t T, const void *x, const void *dt, const void *B,
                    const float *A, const float *h_init, float *h_final, const Workspace &w,
                    const Plan &p, hipStream_t st, const Fuse &f = Fuse()) {
    const int64_t batch = s->batch, D = s->d_inner, N = s->d_state;
    if (p.n_fine == 1) {
        // one chunk: scan directly from h_init into h_final (same-lane read then write)
        launch_chunk_state<Tin>(false, x, dt, B, A, h_init, h_final, nullptr, batch, T, D, N,
                                p.fine_len, 1, 0, 1, st, f);
        return;
    }
    launch_chunk_state<Tin>(false, x, dt, B, A, nullptr, w.agg_h, w.agg_s, batch, T, D, N,
                            p.fine_len, p.n_fine, 0, p.n_fine, st, f);
    launch_carry(false, w.agg_h, w.agg_s, A, h_init, nullptr, h_final, batch, D, N, p.n_fine,
                 p.n_fine, st);
}

// Forward over T tokens from h_init with the in-block reverse and the output.
template <typename Tin>
void run_bidirectional(const bdssm_shape *s, int64_t T, const void *x, const void *dt,
                       const void *B, const void *C, const float *A, const float *Dskip,
                       const float *h_init, void *y, float *bounds, float *h_final,
                       const Workspace &w, const Plan &p, hipStream_t st, const Fuse &f = Fuse()) {
    const int64_t batch = s->batch, D = s->d_inner, N = s->d_state;
    const int64_t hs = D * N;
    if (p.n_coarse == 1) {
        launch_bidir<Tin>(s->block_len, x, dt, B, C, A, Dskip, h_init, hs, 0, y, bounds, h_final,
                          batch, T, D, N, p.fine_len * p.n_fine, 1, st, nullptr, f);
        return;
    }
    // aggregates of every fine chunk before the last coarse chunk, then the carry
    const int n_agg = (p.n_coarse - 1) * p.per_coarse;
    launch_chunk_state<Tin>(false, x, dt, B, A, nullptr, w.agg_h, w.agg_s, batch, T, D, N,
                            p.fine_len, p.n_fine, 0, n_agg, st, f);
    launch_carry(false, w.agg_h, w.agg_s, A, h_init, w.h_in, nullptr, batch, D, N, p.n_fine, n_agg,
                 st);
    launch_bidir<Tin>(s->block_len, x, dt, B, C, A, Dskip, w.h_in, (int64_t)p.n_fine * hs,
                      (int64_t)p.per_coarse * hs, y, bounds, h_final, batch, T, D, N,
                      p.fine_len * p.per_coarse, p.n_coarse, st, nullptr, f);
}

template <typename Tin>
void run_full(const bdssm_shape *s, int64_t T, const void *x, const void *dt, const void *B,
              const void *C, const float *A, const float *Dskip, void *y, const Workspace &w,
              const Plan &p, hipStream_t st, const Fuse &f = Fuse()) {
    const int64_t batch = s->batch, D = s->d_inner, N = s->d_state;
    const int nf = p.n_fine;
    // forward: aggregates of chunks 0..nf-2, incoming states of all chunks
    launch_chunk_state<Tin>(false, x, dt, B, A, nullptr, w.agg_h, w.agg_s, batch, T, D, N,
                            p.fine_len, nf, 0, nf - 1, st, f);
    launch_carry(false, w.agg_h, w.agg_s, A, nullptr, w.h_in, nullptr, batch, D, N, nf, nf - 1, st);
    // reverse (with its own operands when given): aggregates of chunks
    // 1..nf-1 (scanned right to left), incoming states
    const bool sep = f.dt_r != nullptr;
    const void *rdt = sep ? f.dt_r : dt, *rB = sep ? f.B_r : B, *rC = sep ? f.C_r : C;
    const float *rA = sep ? f.A_r : A;
    const Fuse fr = f.reverse();
    launch_chunk_state<Tin>(true, x, rdt, rB, rA, nullptr, w.ragg_h, w.ragg_s, batch, T, D, N,
                            p.fine_len, nf, 1, nf - 1, st, fr);
    launch_carry(true, w.ragg_h, w.ragg_s, rA, nullptr, w.hr_in, nullptr, batch, D, N, nf, nf, st);
    Fuse ff = f;
    ff.z = nullptr;             // the gate multiplies the final output only
    launch_sweep<Tin>(false, x, dt, B, C, A, Dskip, w.h_in, w.yf, y, batch, T, D, N, p.fine_len, nf, st, ff);
    launch_sweep<Tin>(true, x, rdt, rB, rC, rA, Dskip, w.hr_in, w.yf, y, batch, T, D, N, p.fine_len, nf, st, fr);
}

}  // namespace

// ====================================================================== ABI

extern "C" {

int bdssm_version(void) { return kVersion; }

const char *bdssm_status_str(int status) {
    switch (status) {
    case BDSSM_OK: return "ok";
    case BDSSM_ERR_NULL: return "a required pointer is NULL";
    case BDSSM_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case BDSSM_ERR_DTYPE: return "unknown dtype";
    case BDSSM_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case BDSSM_ERR_WORKSPACE: return "workspace missing or too small";
    case BDSSM_ERR_HIP: return "HIP launch or runtime error";
    case BDSSM_ERR_ALIAS: return "an output overlaps an input";
    default: return "unknown status";
    }
}

size_t bdssm_workspace_bytes(const bdssm_shape *shape, int64_t T, int op) {
    if (check_shape(shape) != BDSSM_OK || T < 0 || T % shape->block_len != 0) return (size_t)-1;
    if (op < BDSSM_OP_PREFILL || op > BDSSM_OP_BLOCKS_BWD_REV) return (size_t)-1;
    const int64_t batch = shape->batch, D = shape->d_inner;
    if (batch == 0 || D == 0 || T == 0) return 0;
    const int64_t N = shape->d_state, L = shape->block_len;
    // the backward's plan depends on the kernel, which a fusion can change:
    // size for the larger of the two
    if (op == BDSSM_OP_TRAIN_BWD || op == BDSSM_OP_TRAIN_BWD_REV) {
        const bool sep = op == BDSSM_OP_TRAIN_BWD_REV;
        size_t n = 0;
        for (int fused = sep ? 1 : 0; fused < 2; ++fused) {
            Plan p;
            if (!bwd_plan(batch, D, T, L, N, fused != 0, &p, sep)) return (size_t)-1;
            const size_t m = layout_bwd(nullptr, batch, D, T, p.n_fine, p.n_coarse, p.n_coarse > 1, N,
                                        ceil_div(D, bwd_channels(L, N, fused != 0, sep)), sep, L).bytes;
            n = m > n ? m : n;
        }
        return n;
    }
    if (op == BDSSM_OP_BLOCKS_BWD || op == BDSSM_OP_BLOCKS_BWD_REV) {
        const bool sep = op == BDSSM_OP_BLOCKS_BWD_REV;
        size_t n = 0;
        for (int fused = sep ? 1 : 0; fused < 2; ++fused) {
            int64_t tc, nc;
            if (!bwd_blocks_plan(batch, D, T, L, N, &tc, &nc, fused != 0, sep)) return (size_t)-1;
            const size_t m = layout_bwd(nullptr, batch, D, T, 1, nc, false, N,
                                        ceil_div(D, bwd_channels(L, N, fused != 0, sep)), sep, L).bytes;
            n = m > n ? m : n;
        }
        return n;
    }
    Plan p;
    if (op == BDSSM_OP_FULL) p = make_plan(batch, D, T);
    else if (!plan_for(batch, D, T, shape->block_len, shape->d_state, &p)) return (size_t)-1;
    return layout_ws(nullptr, batch, D, shape->d_state, T, p, op).bytes;
}

int bdssm_prefill(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                  const void *B, const void *C, const float *A, const float *Dskip,
                  const float *h_init, float *h_cache, void *y, void *ws, size_t ws_bytes,
                  const bdssm_fusion *fusion, void *stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (t_ctx < 0 || t_ctx % shape->block_len != 0) return BDSSM_ERR_SHAPE;
    const bool with_y = y != nullptr;
    rc = check_streams(shape, t_ctx, x, dt, B, C, with_y, A, Dskip, with_y);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, N = shape->d_state;
    if (batch == 0 || D == 0) return BDSSM_OK;
    if (h_cache == nullptr) return BDSSM_ERR_NULL;
    if (!aligned16(h_cache) || !aligned16(h_init) || !aligned16(y) || !aligned16(ws))
        return BDSSM_ERR_ALIGN;
    const size_t nstate = (size_t)batch * D * N * 4;
    const size_t ny = (size_t)batch * t_ctx * D * esize(shape);
    rc = check_alias(shape, t_ctx, x, dt, B, C, A, Dskip, nullptr,
                     {Range{h_cache, nstate}, Range{y, ny}});
    if (rc) return rc;
    if (h_init && h_init != h_cache && overlaps({h_init, nstate}, {h_cache, nstate}))
        return BDSSM_ERR_ALIAS;
    if (h_init && overlaps({h_init, nstate}, {y, ny})) return BDSSM_ERR_ALIAS;
    rc = check_fusion(fusion, shape, t_ctx, with_y, {Range{h_cache, nstate}, Range{y, ny}, Range{ws, ws_bytes}});
    if (rc) return rc;
    const Fuse f = resolve_fusion(fusion, with_y);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (t_ctx == 0) return copy_or_zero(h_init, h_cache, batch * D * N, st);
    Plan p;
    if (!plan_for(batch, D, t_ctx, shape->block_len, N, &p)) return BDSSM_ERR_SHAPE;
    const Workspace probe = layout_ws(nullptr, batch, D, N, t_ctx, p, BDSSM_OP_PREFILL);
    if (probe.bytes > 0 && (ws == nullptr || ws_bytes < probe.bytes)) return BDSSM_ERR_WORKSPACE;
    if (probe.bytes > 0) {
        rc = check_alias(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, {Range{ws, probe.bytes}});
        if (rc) return rc;
        if (overlaps({ws, probe.bytes}, {y, ny}) || overlaps({ws, probe.bytes}, {h_cache, nstate}))
            return BDSSM_ERR_ALIAS;
    }
    const Workspace w = layout_ws(ws, batch, D, N, t_ctx, p, BDSSM_OP_PREFILL);
    (void)hipGetLastError();
    if (shape->dtype == BDSSM_BF16) {
        if (with_y) run_bidirectional<uint16_t>(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, y, nullptr, h_cache, w, p, st, f);
        else run_state_only<uint16_t>(shape, t_ctx, x, dt, B, A, h_init, h_cache, w, p, st, f);
    } else {
        if (with_y) run_bidirectional<float>(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, y, nullptr, h_cache, w, p, st, f);
        else run_state_only<float>(shape, t_ctx, x, dt, B, A, h_init, h_cache, w, p, st, f);
    }
    return launch_status();
}

int bdssm_block_step(const bdssm_shape *shape, const float *h_cache, const void *x,
                     const void *dt, const void *B, const void *C, const float *A,
                     const float *Dskip, void *y, const bdssm_fusion *fusion, void *stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    const int64_t L = shape->block_len;
    rc = check_streams(shape, L, x, dt, B, C, true, A, Dskip, true);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, N = shape->d_state;
    if (batch == 0 || D == 0) return BDSSM_OK;
    if (h_cache == nullptr || y == nullptr) return BDSSM_ERR_NULL;
    if (!aligned16(h_cache) || !aligned16(y)) return BDSSM_ERR_ALIGN;
    rc = check_alias(shape, L, x, dt, B, C, A, Dskip, h_cache,
                     {Range{y, (size_t)batch * L * D * esize(shape)}});
    if (rc) return rc;
    rc = check_fusion(fusion, shape, L, true, {Range{y, (size_t)batch * L * D * esize(shape)}});
    if (rc) return rc;
    const Fuse f = resolve_fusion(fusion, true);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (block_lane_path(L, f, true)) {
        if (shape->dtype == BDSSM_BF16)
            launch_block_lane<uint16_t, false>(N, x, dt, B, C, A, Dskip, const_cast<float *>(h_cache), y, batch, D, L, f, st);
        else
            launch_block_lane<float, false>(N, x, dt, B, C, A, Dskip, const_cast<float *>(h_cache), y, batch, D, L, f, st);
    } else if (shape->dtype == BDSSM_BF16) {
        launch_bidir<uint16_t>(L, x, dt, B, C, A, Dskip, h_cache, D * N, 0, y, nullptr, nullptr, batch, L, D, N, L, 1, st, nullptr, f);
    } else {
        launch_bidir<float>(L, x, dt, B, C, A, Dskip, h_cache, D * N, 0, y, nullptr, nullptr, batch, L, D, N, L, 1, st, nullptr, f);
    }
    return launch_status();
}

int bdssm_commit(const bdssm_shape *shape, float *h_cache, const void *x, const void *dt,
                 const void *B, const void *C, const float *A, const float *Dskip, void *y,
                 const bdssm_fusion *fusion, void *stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    const int64_t L = shape->block_len;
    const bool with_y = y != nullptr;
    rc = check_streams(shape, L, x, dt, B, C, with_y, A, Dskip, with_y);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, N = shape->d_state;
    if (batch == 0 || D == 0) return BDSSM_OK;
    if (h_cache == nullptr) return BDSSM_ERR_NULL;
    if (!aligned16(h_cache) || !aligned16(y)) return BDSSM_ERR_ALIGN;
    rc = check_alias(shape, L, x, dt, B, C, A, Dskip, nullptr,
                     {Range{h_cache, (size_t)batch * D * N * 4},
                      Range{y, (size_t)batch * L * D * esize(shape)}});
    if (rc) return rc;
    rc = check_fusion(fusion, shape, L, with_y, {Range{h_cache, (size_t)batch * D * N * 4},
                                                 Range{y, (size_t)batch * L * D * esize(shape)}});
    if (rc) return rc;
    const Fuse f = resolve_fusion(fusion, with_y);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (block_lane_path(L, f, with_y)) {
        if (shape->dtype == BDSSM_BF16)
            launch_block_lane<uint16_t, true>(N, x, dt, B, C, A, Dskip, h_cache, y, batch, D, L, f, st);
        else
            launch_block_lane<float, true>(N, x, dt, B, C, A, Dskip, h_cache, y, batch, D, L, f, st);
    } else if (shape->dtype == BDSSM_BF16) {
        if (with_y) launch_bidir<uint16_t>(L, x, dt, B, C, A, Dskip, h_cache, D * N, 0, y, nullptr, h_cache, batch, L, D, N, L, 1, st, nullptr, f);
        else launch_chunk_state<uint16_t>(false, x, dt, B, A, h_cache, h_cache, nullptr, batch, L, D, N, L, 1, 0, 1, st, f);
    } else {
        if (with_y) launch_bidir<float>(L, x, dt, B, C, A, Dskip, h_cache, D * N, 0, y, nullptr, h_cache, batch, L, D, N, L, 1, st, nullptr, f);
        else launch_chunk_state<float>(false, x, dt, B, A, h_cache, h_cache, nullptr, batch, L, D, N, L, 1, 0, 1, st, f);
    }
    return launch_status();
}

int bdssm_train_scan(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                     const void *B, const void *C, const float *A, const float *Dskip,
                     const float *h_init, void *y, float *h_bounds, void *ws, size_t ws_bytes,
                     const bdssm_fusion *fusion, void *stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (T < 0 || T % shape->block_len != 0) return BDSSM_ERR_SHAPE;
    rc = check_streams(shape, T, x, dt, B, C, true, A, Dskip, true);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, L = shape->block_len, N = shape->d_state;
    if (batch == 0 || D == 0) return BDSSM_OK;
    if (T > 0 && y == nullptr) return BDSSM_ERR_NULL;
    if (!aligned16(h_init) || !aligned16(y) || !aligned16(h_bounds) || !aligned16(ws))
        return BDSSM_ERR_ALIGN;
    const size_t nbnd = (size_t)batch * (T / L + 1) * D * N * 4;
    Plan p;
    if (!plan_for(batch, D, T, L, N, &p)) return BDSSM_ERR_SHAPE;
    const Workspace probe = layout_ws(nullptr, batch, D, N, T, p, BDSSM_OP_TRAIN);
    rc = check_alias(shape, T, x, dt, B, C, A, Dskip, h_init,
                     {Range{y, (size_t)batch * T * D * esize(shape)}, Range{h_bounds, nbnd},
                      Range{T > 0 ? ws : nullptr, probe.bytes}});
    if (rc) return rc;
    rc = check_fusion(fusion, shape, T, true, {Range{y, (size_t)batch * T * D * esize(shape)},
                                               Range{h_bounds, nbnd}, Range{T > 0 ? ws : nullptr, probe.bytes}});
    if (rc) return rc;
    const Fuse f = resolve_fusion(fusion, true);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) {
        if (h_bounds == nullptr) return BDSSM_OK;
        return copy_or_zero(h_init, h_bounds, batch * D * N, st);
    }
    if (probe.bytes > 0 && (ws == nullptr || ws_bytes < probe.bytes)) return BDSSM_ERR_WORKSPACE;
    const Workspace w = layout_ws(ws, batch, D, N, T, p, BDSSM_OP_TRAIN);
    (void)hipGetLastError();
    if (shape->dtype == BDSSM_BF16)
        run_bidirectional<uint16_t>(shape, T, x, dt, B, C, A, Dskip, h_init, y, h_bounds, nullptr, w, p, st, f);
    else
        run_bidirectional<float>(shape, T, x, dt, B, C, A, Dskip, h_init, y, h_bounds, nullptr, w, p, st, f);
    return launch_status();
}

int bdssm_train_scan_blocks(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                            const void *B, const void *C, const float *A, const float *Dskip,
                            const float *h0_blocks, void *y, const bdssm_fusion *fusion,
                            void *stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (T < 0 || T % shape->block_len != 0) return BDSSM_ERR_SHAPE;
    rc = check_streams(shape, T, x, dt, B, C, true, A, Dskip, true);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, L = shape->block_len, N = shape->d_state;
    if (batch == 0 || D == 0 || T == 0) return BDSSM_OK;
    if (y == nullptr || h0_blocks == nullptr) return BDSSM_ERR_NULL;
    if (!aligned16(y) || !aligned16(h0_blocks)) return BDSSM_ERR_ALIGN;
    const size_t nb0 = (size_t)batch * (T / L + 1) * D * N * 4;
    rc = check_alias(shape, T, x, dt, B, C, A, Dskip, nullptr,
                     {Range{y, (size_t)batch * T * D * esize(shape)}});
    if (rc) return rc;
    if (overlaps({y, (size_t)batch * T * D * esize(shape)}, {h0_blocks, nb0})) return BDSSM_ERR_ALIAS;
    rc = check_fusion(fusion, shape, T, true, {Range{y, (size_t)batch * T * D * esize(shape)}});
    if (rc) return rc;
    const Fuse f = resolve_fusion(fusion, true);
    int64_t tc, nc;
    if (!blocks_plan(batch, D, T, L, N, &tc, &nc)) return BDSSM_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (shape->dtype == BDSSM_BF16)
        launch_bidir<uint16_t>(L, x, dt, B, C, A, Dskip, nullptr, 0, 0, y, nullptr, nullptr, batch, T, D, N, tc, (int)nc, st, h0_blocks, f);
    else
        launch_bidir<float>(L, x, dt, B, C, A, Dskip, nullptr, 0, 0, y, nullptr, nullptr, batch, T, D, N, tc, (int)nc, st, h0_blocks, f);
    return launch_status();
}

int bdssm_full_scan(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                    const void *B, const void *C, const float *A, const float *Dskip, void *y,
                    void *ws, size_t ws_bytes, const bdssm_fusion *fusion, void *stream) {
    if (shape == nullptr) return BDSSM_ERR_NULL;
    // the block length does not apply; validate the rest with L = 1
    bdssm_shape s1 = *shape;
    s1.block_len = 1;
    int rc = check_shape(&s1);
    if (rc) return rc;
    if (T < 0) return BDSSM_ERR_SHAPE;
    rc = check_streams(&s1, T, x, dt, B, C, true, A, Dskip, true);
    if (rc) return rc;
    const int64_t batch = s1.batch, D = s1.d_inner;
    if (batch == 0 || D == 0 || T == 0) return BDSSM_OK;
    if (y == nullptr) return BDSSM_ERR_NULL;
    if (!aligned16(y) || !aligned16(ws)) return BDSSM_ERR_ALIGN;
    const Plan p = make_plan(batch, D, T);
    const Workspace probe = layout_ws(nullptr, batch, D, s1.d_state, T, p, BDSSM_OP_FULL);
    if (ws == nullptr || ws_bytes < probe.bytes) return BDSSM_ERR_WORKSPACE;
    rc = check_alias(&s1, T, x, dt, B, C, A, Dskip, nullptr,
                     {Range{y, (size_t)batch * T * D * esize(&s1)}, Range{ws, probe.bytes}});
    if (rc) return rc;
    rc = check_fusion(fusion, &s1, T, true, {Range{y, (size_t)batch * T * D * esize(&s1)}, Range{ws, probe.bytes}});
    if (rc) return rc;
    const Fuse f = resolve_fusion(fusion, true);
    const Workspace w = layout_ws(ws, batch, D, s1.d_state, T, p, BDSSM_OP_FULL);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (s1.dtype == BDSSM_BF16) run_full<uint16_t>(&s1, T, x, dt, B, C, A, Dskip, y, w, p, st, f);
    else run_full<float>(&s1, T, x, dt, B, C, A, Dskip, y, w, p, st, f);
    return launch_status();
}

}  // extern "C"

// ---------------------------------------------------------------- backward

namespace {

// Argument checks shared by the two backward entry points; on success fills
// the byte sizes used by the caller.
int check_bwd(const bdssm_shape *shape, int64_t T, const void *x, const void *dt, const void *B,
              const void *C, const float *A, const float *Dskip, const float *h_states,
              const void *dy, const float *dbounds, void *dx, void *ddt, void *dB, void *dC,
              float *dA, float *dDskip, float *dh, size_t dh_bytes) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (T < 0 || T % shape->block_len != 0) return BDSSM_ERR_SHAPE;
    // the general path's checkpoints cover blocks up to kMaxLdsBlock tokens
    if (shape->block_len > kMaxLdsBlock) return BDSSM_ERR_SHAPE;
    rc = check_streams(shape, T, x, dt, B, C, true, A, Dskip, true);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, L = shape->block_len, N = shape->d_state;
    if (D > 0 && (dA == nullptr || dDskip == nullptr)) return BDSSM_ERR_NULL;
    const bool work = batch > 0 && D > 0 && T > 0;
    if (work && (!h_states || !dy || !dx || !ddt || !dB || !dC)) return BDSSM_ERR_NULL;
    const void *ps[] = {h_states, dy, dbounds, dx, ddt, dB, dC, dA, dDskip, dh};
    for (const void *p : ps)
        if (p && !aligned16(p)) return BDSSM_ERR_ALIGN;
    const size_t e = esize(shape);
    const size_t ntok = (size_t)batch * T * D * e, nbc = (size_t)batch * T * N * e;
    const size_t nbnd = (size_t)batch * (T / L + 1) * D * N * 4;
    const Range outs[] = {{dx, ntok}, {ddt, ntok}, {dB, nbc}, {dC, nbc},
                          {dA, (size_t)D * N * 4}, {dDskip, (size_t)D * 4}, {dh, dh_bytes}};
    const Range ins[] = {{x, ntok}, {dt, ntok}, {B, nbc}, {C, nbc}, {A, (size_t)D * N * 4},
                         {Dskip, (size_t)D * 4}, {h_states, nbnd}, {dy, ntok}, {dbounds, nbnd}};
    for (const Range &o : outs) {
        for (const Range &i : ins)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
        for (const Range &o2 : outs)
            if (&o2 != &o && overlaps(o, o2)) return BDSSM_ERR_ALIAS;
    }
    return BDSSM_OK;
}

// Zero the reverse operands' parameter gradients of an empty call.
int zero_bwd_rev(const bdssm_fusion_grads *g, int64_t D, int64_t N, hipStream_t st) {
    int rc = copy_or_zero(nullptr, g->dA_rev, D * N, st);
    if (!rc && g->d_dt_bias_rev) rc = copy_or_zero(nullptr, g->d_dt_bias_rev, D, st);
    return rc;
}

// Zero the parameter gradients (and the start-state gradient) of an empty call.
int zero_bwd(int64_t D, int64_t N, float *dA, float *dDskip, float *dh, int64_t dh_n, hipStream_t st) {
    int rc = D > 0 ? copy_or_zero(nullptr, dA, D * N, st) : BDSSM_OK;
    if (!rc && D > 0) rc = copy_or_zero(nullptr, dDskip, D, st);
    if (!rc && dh && dh_n > 0) rc = copy_or_zero(nullptr, dh, dh_n, st);
    return rc;
}

bool ws_clear(void *ws, size_t bytes, std::initializer_list<Range> others) {
    for (const Range &o : others)
        if (overlaps({ws, bytes}, o)) return false;
    return true;
}

// The fused forward's gradients requested from a backward call: resolves the
// fusion and checks the extra arguments (alignment; dz and d_dt_bias are
// outputs, z and dt_bias inputs; separate reverse operands are rejected).
int resolve_bwd_fusion(const bdssm_fusion *f, bdssm_fusion_grads *g, const bdssm_shape *s,
                       int64_t T, std::initializer_list<Range> ins, std::initializer_list<Range> outs,
                       BwdArgs *a) {
    a->fused = false;
    a->sep = false;
    const float *bias = f ? f->dt_bias : nullptr;
    // a reverse bias alone also selects the bias form (the forward's bias is then zero)
    const bool rbias = f && f->dt_rev != nullptr && f->dt_bias_rev != nullptr;
    const int mode = (f && f->dt_softplus) ? kDtSoftplus : ((bias || rbias) ? kDtBias : kDtPlain);
    const void *z = f ? f->z : nullptr;
    void *dz = g ? g->dz : nullptr;
    float *dbias = g ? g->d_dt_bias : nullptr;
    if (z != nullptr && dz == nullptr) return BDSSM_ERR_NULL;
    if (z == nullptr) dz = nullptr;
    const void *ps[] = {bias, z, dz, dbias};
    for (const void *p : ps)
        if (!aligned16(p)) return BDSSM_ERR_ALIGN;
    const size_t ntok = (size_t)s->batch * T * s->d_inner * esize(s);
    const Range fin[] = {{bias, (size_t)s->d_inner * 4}, {z, ntok}};
    const Range fout[] = {{dz, ntok}, {dbias, (size_t)s->d_inner * 4}};
    for (const Range &o : fout) {
        for (const Range &i : ins)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
        for (const Range &i : fin)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
        for (const Range &o2 : outs)
            if (overlaps(o, o2)) return BDSSM_ERR_ALIAS;
    }
    if (overlaps(fout[0], fout[1])) return BDSSM_ERR_ALIAS;
    for (const Range &o : outs)
        for (const Range &i : fin)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
    a->fused = mode != kDtPlain || z != nullptr || dbias != nullptr;
    a->dt_bias = bias;
    a->dt_mode = mode;
    a->z = z;
    a->dz = dz;
    if (f == nullptr || f->dt_rev == nullptr) return BDSSM_OK;
    // separate reverse operands: their inputs and the gradients they need
    if (f->B_rev == nullptr || f->C_rev == nullptr || f->A_rev == nullptr) return BDSSM_ERR_NULL;
    if (g == nullptr || g->ddt_rev == nullptr || g->dB_rev == nullptr || g->dC_rev == nullptr ||
        g->dA_rev == nullptr)
        return BDSSM_ERR_NULL;
    const size_t nbc = (size_t)s->batch * T * s->d_state * esize(s);
    const size_t npar = (size_t)s->d_inner * s->d_state * 4;
    const void *pr[] = {f->dt_rev, f->B_rev, f->C_rev, f->A_rev, f->dt_bias_rev, g->ddt_rev, g->dB_rev,
                        g->dC_rev, g->dA_rev, g->d_dt_bias_rev};
    for (const void *p : pr)
        if (!aligned16(p)) return BDSSM_ERR_ALIGN;
    const Range rin[] = {{f->dt_rev, ntok}, {f->B_rev, nbc}, {f->C_rev, nbc}, {f->A_rev, npar},
                         {f->dt_bias_rev, (size_t)s->d_inner * 4}};
    const Range rout[] = {{g->ddt_rev, ntok}, {g->dB_rev, nbc}, {g->dC_rev, nbc}, {g->dA_rev, npar},
                          {g->d_dt_bias_rev, (size_t)s->d_inner * 4}};
    for (const Range &o : rout) {
        for (const Range &i : ins)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
        for (const Range &i : fin)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
        for (const Range &i : rin)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
        for (const Range &o2 : outs)
            if (overlaps(o, o2)) return BDSSM_ERR_ALIAS;
        for (const Range &o2 : fout)
            if (overlaps(o, o2)) return BDSSM_ERR_ALIAS;
        for (const Range &o2 : rout)
            if (&o2 != &o && overlaps(o, o2)) return BDSSM_ERR_ALIAS;
    }
    for (const Range &i : rin) {
        for (const Range &o : outs)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
        for (const Range &o : fout)
            if (overlaps(o, i)) return BDSSM_ERR_ALIAS;
    }
    a->sep = true;
    a->fused = true;
    a->dt_r = f->dt_rev;
    a->B_r = f->B_rev;
    a->C_r = f->C_rev;
    a->A_r = f->A_rev;
    a->dt_bias_r = f->dt_bias_rev;
    a->ddt_r = g->ddt_rev;
    return BDSSM_OK;
}

}  // namespace

extern "C" {

int bdssm_train_scan_bwd(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                         const void *B, const void *C, const float *A, const float *Dskip,
                         const float *h_bounds, const void *dy, const float *d_bounds, void *dx,
                         void *ddt, void *dB, void *dC, float *dA, float *dDskip, float *dh_init,
                         void *ws, size_t ws_bytes, const bdssm_fusion *fusion,
                         bdssm_fusion_grads *grads, void *stream) {
    const size_t nstate = shape ? (size_t)(shape->batch > 0 ? shape->batch : 0) *
                                      (shape->d_inner > 0 ? shape->d_inner : 0) *
                                      (shape->d_state > 0 ? shape->d_state : 0) * 4 : 0;
    int rc = check_bwd(shape, T, x, dt, B, C, A, Dskip, h_bounds, dy, d_bounds, dx, ddt, dB, dC, dA,
                       dDskip, dh_init, nstate);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, L = shape->block_len, N = shape->d_state;
    BwdArgs a{x, dt, B, C, dy, A, Dskip, h_bounds, nullptr, d_bounds, 0, 0, dx, ddt,
              nullptr, nullptr, nullptr, dh_init};
    const size_t e = esize(shape);
    const size_t ntok = (size_t)batch * T * D * e, nbc = (size_t)batch * T * N * e;
    const size_t nbnd = (size_t)batch * (T / L + 1) * D * N * 4;
    const size_t npar = (size_t)D * N * 4;
    rc = resolve_bwd_fusion(fusion, grads, shape, T,
                            {{x, ntok}, {dt, ntok}, {B, nbc}, {C, nbc}, {dy, ntok}, {h_bounds, nbnd},
                             {d_bounds, nbnd}, {A, npar}, {Dskip, (size_t)D * 4}},
                            {{dx, ntok}, {ddt, ntok}, {dB, nbc}, {dC, nbc}, {dA, npar},
                             {dDskip, (size_t)D * 4}, {dh_init, nstate}, {ws, ws_bytes}},
                            &a);
    if (rc) return rc;
    float *d_bias = grads ? grads->d_dt_bias : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (batch == 0 || D == 0 || T == 0) {
        rc = zero_bwd(D, N, dA, dDskip, dh_init, batch * D * N, st);
        if (!rc && d_bias && D > 0) rc = copy_or_zero(nullptr, d_bias, D, st);
        if (!rc && a.sep && D > 0) rc = zero_bwd_rev(grads, D, N, st);
        if (rc || dh_init == nullptr || d_bounds == nullptr || batch == 0 || D == 0) return rc;
        // T == 0: the only gradient of the start state is its own bound
        return copy_or_zero(d_bounds, dh_init, batch * D * N, st);
    }
    if (!aligned16(ws)) return BDSSM_ERR_ALIGN;
    const bool general = bwd_general(L, N, a.sep), lng = bwd_long(L, N, a.sep);
    Plan p;
    if (!bwd_plan(batch, D, T, L, N, a.fused, &p, a.sep)) return BDSSM_ERR_SHAPE;
    const bool carry = p.n_coarse > 1;
    const int64_t nblk = ceil_div(D, bwd_channels(L, N, a.fused, a.sep));
    const BwdWorkspace probe = layout_bwd(nullptr, batch, D, T, p.n_fine, p.n_coarse, carry, N, nblk, a.sep, L);
    if (ws == nullptr || ws_bytes < probe.bytes) return BDSSM_ERR_WORKSPACE;
    if (!ws_clear(ws, probe.bytes, {{x, ntok}, {dt, ntok}, {B, nbc}, {C, nbc}, {dy, ntok},
                                    {h_bounds, nbnd}, {d_bounds, nbnd}, {dx, ntok}, {ddt, ntok},
                                    {dB, nbc}, {dC, nbc}, {dA, npar}, {dDskip, (size_t)D * 4},
                                    {dh_init, nstate}, {A, npar}, {Dskip, (size_t)D * 4}}))
        return BDSSM_ERR_ALIAS;
    const BwdWorkspace w = layout_bwd(ws, batch, D, T, p.n_fine, p.n_coarse, carry, N, nblk, a.sep, L);
    const int64_t hs = D * N;
    a.part_bc = w.part_bc;
    a.part_a = w.part_a;
    a.part_d = w.part_d;
    a.part_bias = w.part_bias;
    a.part_bc_r = w.part_bc_r;
    a.part_a_r = w.part_a_r;
    a.part_bias_r = w.part_bias_r;
    const int64_t Tc = carry ? p.fine_len * p.per_coarse : p.fine_len * p.n_fine;
    const bool bf = shape->dtype == BDSSM_BF16;
    if (carry) {
        // adjoint aggregates of the fine chunks right of the first coarse chunk,
        // then the adjoint entering each fine chunk from its right end
        const int c_first = p.per_coarse, n_launch = p.n_fine - p.per_coarse;
        if (general || lng) {
            if (bf)
                launch_adjoint_general<uint16_t>(N, dt, dy, C, A, d_bounds, w.agg_q, w.agg_s, batch, T, D, L,
                                                 p.fine_len, p.n_fine, c_first, n_launch, a.dt_mode, a.dt_bias,
                                                 a.z, st);
            else
                launch_adjoint_general<float>(N, dt, dy, C, A, d_bounds, w.agg_q, w.agg_s, batch, T, D, L,
                                              p.fine_len, p.n_fine, c_first, n_launch, a.dt_mode, a.dt_bias,
                                              a.z, st);
        } else if (bf) {
            launch_adjoint_chunk<uint16_t>(dt, dy, C, A, d_bounds, w.agg_q, w.agg_s, batch, T, D, L,
                                           p.fine_len, p.n_fine, c_first, n_launch, st, a.dt_mode, a.dt_bias,
                                           a.z);
        } else {
            launch_adjoint_chunk<float>(dt, dy, C, A, d_bounds, w.agg_q, w.agg_s, batch, T, D, L,
                                        p.fine_len, p.n_fine, c_first, n_launch, st, a.dt_mode, a.dt_bias,
                                        a.z);
        }
        launch_carry(true, w.agg_q, w.agg_s, A, nullptr, w.q_in, nullptr, batch, D, N, p.n_fine,
                     p.n_fine, st, p.per_coarse - 1);
        a.qin = w.q_in + (int64_t)(p.per_coarse - 1) * hs;
        a.qin_bs = (int64_t)p.n_fine * hs;
        a.qin_cs = (int64_t)p.per_coarse * hs;
    }
    const int nc = carry ? p.n_coarse : 1;
    if (bf) {
        if (general) launch_bwd_general<uint16_t, false>(N, a, batch, T, D, L, Tc, nc, st);
        else if (lng) launch_bwd_long<uint16_t, false>(a, w.gstate, batch, T, D, L, Tc, nc, st);
        else launch_bwd<uint16_t, false>(L, a, batch, T, D, Tc, nc, st);
        launch_bwd_reduce<uint16_t>(w, dB, dC, dA, dDskip, batch, T, D, L, N, nc, st, a.fused, d_bias,
                                    a.sep ? grads : nullptr);
    } else {
        if (general) launch_bwd_general<float, false>(N, a, batch, T, D, L, Tc, nc, st);
        else if (lng) launch_bwd_long<float, false>(a, w.gstate, batch, T, D, L, Tc, nc, st);
        else launch_bwd<float, false>(L, a, batch, T, D, Tc, nc, st);
        launch_bwd_reduce<float>(w, dB, dC, dA, dDskip, batch, T, D, L, N, nc, st, a.fused, d_bias,
                                 a.sep ? grads : nullptr);
    }
    return launch_status();
}

int bdssm_train_scan_blocks_bwd(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                                const void *B, const void *C, const float *A, const float *Dskip,
                                const float *h0_blocks, const void *dy, void *dx, void *ddt,
                                void *dB, void *dC, float *dA, float *dDskip, float *dh0_blocks,
                                void *ws, size_t ws_bytes, const bdssm_fusion *fusion,
                                bdssm_fusion_grads *grads, void *stream) {
    size_t nbnd = 0;
    if (shape && shape->block_len > 0 && T >= 0 && shape->batch > 0 && shape->d_inner > 0 &&
        shape->d_state > 0)
        nbnd = (size_t)shape->batch * (T / shape->block_len + 1) * shape->d_inner * shape->d_state * 4;
    int rc = check_bwd(shape, T, x, dt, B, C, A, Dskip, h0_blocks, dy, nullptr, dx, ddt, dB, dC, dA,
                       dDskip, dh0_blocks, nbnd);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, L = shape->block_len, N = shape->d_state;
    BwdArgs a{x, dt, B, C, dy, A, Dskip, h0_blocks, nullptr, nullptr, 0, 0, dx, ddt,
              nullptr, nullptr, nullptr, dh0_blocks};
    const size_t e = esize(shape);
    const size_t ntok = (size_t)batch * T * D * e, nbc = (size_t)batch * T * N * e;
    const size_t npar = (size_t)D * N * 4;
    rc = resolve_bwd_fusion(fusion, grads, shape, T,
                            {{x, ntok}, {dt, ntok}, {B, nbc}, {C, nbc}, {dy, ntok}, {h0_blocks, nbnd},
                             {A, npar}, {Dskip, (size_t)D * 4}},
                            {{dx, ntok}, {ddt, ntok}, {dB, nbc}, {dC, nbc}, {dA, npar},
                             {dDskip, (size_t)D * 4}, {dh0_blocks, nbnd}, {ws, ws_bytes}},
                            &a);
    if (rc) return rc;
    float *d_bias = grads ? grads->d_dt_bias : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (batch == 0 || D == 0 || T == 0) {
        rc = zero_bwd(D, N, dA, dDskip, dh0_blocks, batch * D * N, st);
        if (!rc && d_bias && D > 0) rc = copy_or_zero(nullptr, d_bias, D, st);
        if (!rc && a.sep && D > 0) rc = zero_bwd_rev(grads, D, N, st);
        return rc;
    }
    if (!aligned16(ws)) return BDSSM_ERR_ALIGN;
    const bool general = bwd_general(L, N, a.sep), lng = bwd_long(L, N, a.sep);
    int64_t tc, nc;
    if (!bwd_blocks_plan(batch, D, T, L, N, &tc, &nc, a.fused, a.sep)) return BDSSM_ERR_SHAPE;
    const int64_t nblk = ceil_div(D, bwd_channels(L, N, a.fused, a.sep));
    const BwdWorkspace probe = layout_bwd(nullptr, batch, D, T, 1, nc, false, N, nblk, a.sep, L);
    if (ws == nullptr || ws_bytes < probe.bytes) return BDSSM_ERR_WORKSPACE;
    if (!ws_clear(ws, probe.bytes, {{x, ntok}, {dt, ntok}, {B, nbc}, {C, nbc}, {dy, ntok},
                                    {h0_blocks, nbnd}, {dx, ntok}, {ddt, ntok}, {dB, nbc},
                                    {dC, nbc}, {dA, npar}, {dDskip, (size_t)D * 4}, {dh0_blocks, nbnd},
                                    {A, npar}, {Dskip, (size_t)D * 4}}))
        return BDSSM_ERR_ALIAS;
    const BwdWorkspace w = layout_bwd(ws, batch, D, T, 1, nc, false, N, nblk, a.sep, L);
    a.part_bc = w.part_bc;
    a.part_a = w.part_a;
    a.part_d = w.part_d;
    a.part_bias = w.part_bias;
    a.part_bc_r = w.part_bc_r;
    a.part_a_r = w.part_a_r;
    a.part_bias_r = w.part_bias_r;
    if (shape->dtype == BDSSM_BF16) {
        if (general) launch_bwd_general<uint16_t, true>(N, a, batch, T, D, L, tc, (int)nc, st);
        else if (lng) launch_bwd_long<uint16_t, true>(a, w.gstate, batch, T, D, L, tc, (int)nc, st);
        else launch_bwd<uint16_t, true>(L, a, batch, T, D, tc, (int)nc, st);
        launch_bwd_reduce<uint16_t>(w, dB, dC, dA, dDskip, batch, T, D, L, N, nc, st, a.fused, d_bias,
                                    a.sep ? grads : nullptr);
    } else {
        if (general) launch_bwd_general<float, true>(N, a, batch, T, D, L, tc, (int)nc, st);
        else if (lng) launch_bwd_long<float, true>(a, w.gstate, batch, T, D, L, tc, (int)nc, st);
        else launch_bwd<float, true>(L, a, batch, T, D, tc, (int)nc, st);
        launch_bwd_reduce<float>(w, dB, dC, dA, dDskip, batch, T, D, L, N, nc, st, a.fused, d_bias,
                                 a.sep ? grads : nullptr);
    }
    return launch_status();
}

}  // extern "C"
