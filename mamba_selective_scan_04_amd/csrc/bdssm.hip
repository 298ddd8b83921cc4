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

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "bdssm.h"
#include "bdssm_launch.hpp"

using namespace bdssm_host;

namespace {

constexpr int kVersion = 10700;   // 1.7.0

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

// The single-block kernels address one block's rows of a stream with 32-bit
// buffer offsets (L rows of D elements); 4 bytes per element covers both
// dtypes, as in the chunk plans.
bool block_rows_fit(const bdssm_shape *s) {
    return s->block_len * s->d_inner * 4 < ((int64_t)1 << 31);
}

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

}  // namespace

namespace bdssm_host {

void launch_carry(bool rev, const float *agg_h, const float *agg_s, const float *A,
                  const float *h_init, float *h_in, float *h_final, int64_t batch, int64_t D,
                  int64_t N, int n_chunks, int n_agg, hipStream_t st, int c_low) {
    const int64_t total = batch * D * N;
    // long chunk sequences (more than 64 fold steps; at fewer the one-thread
    // walk measured as fast): one wave per segment of about 12 fold steps, at
    // most 16 segments (batches of 16 loads per lane measured slower).
    // BDSSM_CARRY=serial keeps the one-thread walk, BDSSM_CARRY=tree takes
    // the segments from 2 steps on (tests)
    const int64_t K = rev ? n_chunks - 1 - c_low : n_agg;
    const char *cv = getenv("BDSSM_CARRY");
    const char mode = cv != nullptr ? cv[0] : 0;
    int64_t W = mode == 's' ? 1 : (K > 64 || (mode == 't' && K > 1)) ? ceil_div(K, 12) : 1;
    if (W < 2 && mode == 't' && K > 1) W = 2;
    if (W > 16) W = 16;
    if (W >= 2 && ceil_div(total, kWave) * kWave * W < ((int64_t)1 << 31)) {
        const dim3 gt((unsigned)ceil_div(total, kWave));
        if (rev)
            hipLaunchKernelGGL((carry_tree_kernel<true>), gt, dim3((unsigned)(kWave * W)), 0, st, agg_h, agg_s, A,
                               h_init, h_in, h_final, (int)batch, (int)D, (int)N, n_chunks, n_agg, c_low);
        else
            hipLaunchKernelGGL((carry_tree_kernel<false>), gt, dim3((unsigned)(kWave * W)), 0, st, agg_h, agg_s,
                               A, h_init, h_in, h_final, (int)batch, (int)D, (int)N, n_chunks, n_agg, c_low);
        return;
    }
    const dim3 g((unsigned)ceil_div(total, 256));
    if (rev)
        hipLaunchKernelGGL((carry_kernel<true>), g, dim3(256), 0, st, agg_h, agg_s, A, h_init, h_in,
                           h_final, (int)batch, (int)D, (int)N, n_chunks, n_agg, c_low);
    else
        hipLaunchKernelGGL((carry_kernel<false>), g, dim3(256), 0, st, agg_h, agg_s, A, h_init, h_in,
                           h_final, (int)batch, (int)D, (int)N, n_chunks, n_agg, c_low);
}

}  // namespace bdssm_host

namespace {

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
    const bool sep = f.dt_r != nullptr;
    const void *rdt = sep ? f.dt_r : dt, *rB = sep ? f.B_r : B, *rC = sep ? f.C_r : C;
    const float *rA = sep ? f.A_r : A;
    const Fuse fr = f.reverse();
    // shared operands: both directions' aggregates of every chunk in one
    // forward pass (BDSSM_FULL_AGG=separate: one pass per direction)
    const char *fa = getenv("BDSSM_FULL_AGG");
    if (!sep && !(fa != nullptr && fa[0] == 's')) {
        if (nf > 1)
            launch_chunk_both<Tin>(x, dt, B, A, w.agg_h, w.agg_s, w.ragg_h, batch, T, D, N, p.fine_len, nf, st, f);
        launch_carry(false, w.agg_h, w.agg_s, A, nullptr, w.h_in, nullptr, batch, D, N, nf, nf - 1, st);
        launch_carry(true, w.ragg_h, w.agg_s, A, nullptr, w.hr_in, nullptr, batch, D, N, nf, nf, st);
    } else {
        // forward: aggregates of chunks 0..nf-2, incoming states of all chunks
        launch_chunk_state<Tin>(false, x, dt, B, A, nullptr, w.agg_h, w.agg_s, batch, T, D, N,
                                p.fine_len, nf, 0, nf - 1, st, f);
        launch_carry(false, w.agg_h, w.agg_s, A, nullptr, w.h_in, nullptr, batch, D, N, nf, nf - 1, st);
        // reverse (with its own operands when given): aggregates of chunks
        // 1..nf-1 (scanned right to left), incoming states
        launch_chunk_state<Tin>(true, x, rdt, rB, rA, nullptr, w.ragg_h, w.ragg_s, batch, T, D, N,
                                p.fine_len, nf, 1, nf - 1, st, fr);
        launch_carry(true, w.ragg_h, w.ragg_s, rA, nullptr, w.hr_in, nullptr, batch, D, N, nf, nf, st);
    }
    Fuse ff = f;
    ff.z = nullptr;             // the gate multiplies the final output only
    launch_sweep<Tin>(false, x, dt, B, C, A, Dskip, w.h_in, w.yf, y, batch, T, D, N, p.fine_len, nf, st, ff);
    launch_sweep<Tin>(true, x, rdt, rB, rC, rA, Dskip, w.hr_in, w.yf, y, batch, T, D, N, p.fine_len, nf, st, fr);
}

// ---------------------------------------------------------------- prefill
//
// What bdssm_prefill and bdssm_prefill_noalloc share: the argument checks,
// the plan with the workspace it needs, and the launches.  They differ only
// in where the workspace comes from (the caller's buffer, or the library's
// scratch array).

struct PrefillPlan {
    Fuse f;
    Plan p{};
    size_t ws_bytes = 0;   // workspace the plan needs (0: none)
    bool empty = false;    // no rows: nothing to enqueue
};

// Argument checks in the order of the C ABI's contract (ws / ws_bytes: the
// caller's workspace, or nullptr / 0), then the plan.
int prefill_prepare(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                    const void *B, const void *C, const float *A, const float *Dskip,
                    const float *h_init, float *h_cache, void *y, void *ws, size_t ws_bytes,
                    const bdssm_fusion *fusion, PrefillPlan *out) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (t_ctx < 0 || t_ctx % shape->block_len != 0) return BDSSM_ERR_SHAPE;
    const bool with_y = y != nullptr;
    rc = check_streams(shape, t_ctx, x, dt, B, C, with_y, A, Dskip, with_y);
    if (rc) return rc;
    const int64_t batch = shape->batch, D = shape->d_inner, N = shape->d_state;
    if (batch == 0 || D == 0) { out->empty = true; return BDSSM_OK; }
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
    out->f = resolve_fusion(fusion, with_y);
    if (t_ctx == 0) return BDSSM_OK;
    if (!plan_for(batch, D, t_ctx, shape->block_len, N, &out->p)) return BDSSM_ERR_SHAPE;
    out->ws_bytes = layout_ws(nullptr, batch, D, N, t_ctx, out->p, BDSSM_OP_PREFILL).bytes;
    return BDSSM_OK;
}

int prefill_launch(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt, const void *B,
                   const void *C, const float *A, const float *Dskip, const float *h_init, float *h_cache,
                   void *y, void *ws, const PrefillPlan &pp, hipStream_t st) {
    const int64_t batch = shape->batch, D = shape->d_inner, N = shape->d_state;
    if (t_ctx == 0) return copy_or_zero(h_init, h_cache, batch * D * N, st);
    const Workspace w = layout_ws(ws, batch, D, N, t_ctx, pp.p, BDSSM_OP_PREFILL);
    const bool with_y = y != nullptr;
    (void)hipGetLastError();
    if (shape->dtype == BDSSM_BF16) {
        if (with_y) run_bidirectional<uint16_t>(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, y, nullptr, h_cache, w, pp.p, st, pp.f);
        else run_state_only<uint16_t>(shape, t_ctx, x, dt, B, A, h_init, h_cache, w, pp.p, st, pp.f);
    } else {
        if (with_y) run_bidirectional<float>(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, y, nullptr, h_cache, w, pp.p, st, pp.f);
        else run_state_only<float>(shape, t_ctx, x, dt, B, A, h_init, h_cache, w, pp.p, st, pp.f);
    }
    return launch_status();
}

// ------------------------------------------------ the allocation-free scratch
//
// bdssm_prefill_noalloc takes its workspace from this array instead of a
// caller's buffer.  Each device the library runs on holds its own copy for
// the life of the process.  Its address is looked up once per device, with
// that device current, on the first call there; host code uses only that
// address (the array's name in host code is not a device address).  Every
// call on one device shares the array: calls that overlap in time on one
// device (different streams, or threads) race.  Nothing in it needs to start
// at zero: every workspace array of the prefill is written before it is read.
constexpr size_t kScratchBytes = BDSSM_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address (looked up on the first call there).
int scratch_ptr(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return BDSSM_ERR_HIP;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return BDSSM_ERR_HIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BDSSM_OK;
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

size_t bdssm_workspace_bytes_op(const bdssm_shape *shape, int64_t T, int op) {
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
    else if (!plan_for(batch, D, T, shape->block_len, shape->d_state, &p, op == BDSSM_OP_TRAIN)) return (size_t)-1;
    return layout_ws(nullptr, batch, D, shape->d_state, T, p, op).bytes;
}

size_t bdssm_workspace_bytes(const bdssm_shape *shape, int64_t T) {
    size_t n = 0;
    for (int op : {BDSSM_OP_PREFILL, BDSSM_OP_TRAIN, BDSSM_OP_FULL}) {
        const size_t m = bdssm_workspace_bytes_op(shape, T, op);
        if (m == (size_t)-1) return m;
        n = m > n ? m : n;
    }
    return n;
}

int bdssm_prefill_ex(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                  const void *B, const void *C, const float *A, const float *Dskip,
                  const float *h_init, float *h_cache, void *y, void *ws, size_t ws_bytes,
                  const bdssm_fusion *fusion, hipStream_t stream) {
    PrefillPlan pp;
    int rc = prefill_prepare(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, h_cache, y, ws, ws_bytes, fusion,
                             &pp);
    if (rc || pp.empty) return rc;
    if (pp.ws_bytes > 0) {
        if (ws == nullptr || ws_bytes < pp.ws_bytes) return BDSSM_ERR_WORKSPACE;
        rc = check_alias(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, {Range{ws, pp.ws_bytes}});
        if (rc) return rc;
        const size_t nstate = (size_t)shape->batch * shape->d_inner * shape->d_state * 4;
        const size_t ny = (size_t)shape->batch * t_ctx * shape->d_inner * esize(shape);
        if (overlaps({ws, pp.ws_bytes}, {y, ny}) || overlaps({ws, pp.ws_bytes}, {h_cache, nstate}))
            return BDSSM_ERR_ALIAS;
    }
    return prefill_launch(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, h_cache, y, ws, pp,
                          stream);
}

int bdssm_prefill_noalloc(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                          const void *B, const void *C, const float *A, const float *Dskip,
                          const float *h_init, float *h_cache, void *y, const bdssm_fusion *fusion,
                          hipStream_t stream) {
    PrefillPlan pp;
    int rc = prefill_prepare(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, h_cache, y, nullptr, 0, fusion, &pp);
    if (rc || pp.empty) return rc;
    if (pp.ws_bytes > kScratchBytes) return BDSSM_ERR_WORKSPACE;
    void *ws = nullptr;
    if (pp.ws_bytes > 0) {
        rc = scratch_ptr(&ws);
        if (rc) return rc;
    }
    return prefill_launch(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, h_cache, y, ws, pp,
                          stream);
}

int bdssm_block_step_ex(const bdssm_shape *shape, const float *h_cache, const void *x,
                     const void *dt, const void *B, const void *C, const float *A,
                     const float *Dskip, void *y, const bdssm_fusion *fusion, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    const int64_t L = shape->block_len;
    rc = check_streams(shape, L, x, dt, B, C, true, A, Dskip, true);
    if (rc) return rc;
    if (!block_rows_fit(shape)) return BDSSM_ERR_SHAPE;
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
    hipStream_t st = stream;
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

int bdssm_commit_ex(const bdssm_shape *shape, float *h_cache, const void *x, const void *dt,
                 const void *B, const void *C, const float *A, const float *Dskip, void *y,
                 const bdssm_fusion *fusion, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    const int64_t L = shape->block_len;
    const bool with_y = y != nullptr;
    rc = check_streams(shape, L, x, dt, B, C, with_y, A, Dskip, with_y);
    if (rc) return rc;
    if (!block_rows_fit(shape)) return BDSSM_ERR_SHAPE;
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
    hipStream_t st = stream;
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

int bdssm_train_scan_ex(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                     const void *B, const void *C, const float *A, const float *Dskip,
                     const float *h_init, void *y, float *h_bounds, void *ws, size_t ws_bytes,
                     const bdssm_fusion *fusion, hipStream_t stream) {
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
    if (!plan_for(batch, D, T, L, N, &p, true)) return BDSSM_ERR_SHAPE;
    const Workspace probe = layout_ws(nullptr, batch, D, N, T, p, BDSSM_OP_TRAIN);
    rc = check_alias(shape, T, x, dt, B, C, A, Dskip, h_init,
                     {Range{y, (size_t)batch * T * D * esize(shape)}, Range{h_bounds, nbnd},
                      Range{T > 0 ? ws : nullptr, probe.bytes}});
    if (rc) return rc;
    rc = check_fusion(fusion, shape, T, true, {Range{y, (size_t)batch * T * D * esize(shape)},
                                               Range{h_bounds, nbnd}, Range{T > 0 ? ws : nullptr, probe.bytes}});
    if (rc) return rc;
    const Fuse f = resolve_fusion(fusion, true);
    hipStream_t st = stream;
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
                            hipStream_t stream) {
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
    const bool pair = pair_path(L, N) || (pair_long(L, N) && pair_bidir());
    if (!blocks_plan(batch, D, T, L, N, &tc, &nc, pair ? pair_channels_of(N) : kWave,
                     pair ? (pair_path(L, N) ? kPairGroups : pair_long_capacity(L, N)) : kCoarseGroups))
        return BDSSM_ERR_SHAPE;
    hipStream_t st = stream;
    (void)hipGetLastError();
    if (shape->dtype == BDSSM_BF16)
        launch_bidir<uint16_t>(L, x, dt, B, C, A, Dskip, nullptr, 0, 0, y, nullptr, nullptr, batch, T, D, N, tc, (int)nc, st, h0_blocks, f);
    else
        launch_bidir<float>(L, x, dt, B, C, A, Dskip, nullptr, 0, 0, y, nullptr, nullptr, batch, T, D, N, tc, (int)nc, st, h0_blocks, f);
    return launch_status();
}

int bdssm_full_scan_ex(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                    const void *B, const void *C, const float *A, const float *Dskip, void *y,
                    void *ws, size_t ws_bytes, const bdssm_fusion *fusion, hipStream_t stream) {
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
    hipStream_t st = stream;
    (void)hipGetLastError();
    if (s1.dtype == BDSSM_BF16) run_full<uint16_t>(&s1, T, x, dt, B, C, A, Dskip, y, w, p, st, f);
    else run_full<float>(&s1, T, x, dt, B, C, A, Dskip, y, w, p, st, f);
    return launch_status();
}

// The five entry points without the fusions: the same calls with fusion NULL.
int bdssm_prefill(const bdssm_shape *shape, int64_t t_ctx, const void *x, const void *dt,
                  const void *B, const void *C, const float *A, const float *Dskip,
                  const float *h_init, float *h_cache, void *y, void *ws, size_t ws_bytes,
                  hipStream_t stream) {
    return bdssm_prefill_ex(shape, t_ctx, x, dt, B, C, A, Dskip, h_init, h_cache, y, ws, ws_bytes, nullptr,
                            stream);
}

int bdssm_block_step(const bdssm_shape *shape, const float *h_cache, const void *x, const void *dt,
                     const void *B, const void *C, const float *A, const float *Dskip, void *y,
                     hipStream_t stream) {
    return bdssm_block_step_ex(shape, h_cache, x, dt, B, C, A, Dskip, y, nullptr, stream);
}

int bdssm_commit(const bdssm_shape *shape, float *h_cache, const void *x, const void *dt,
                 const void *B, const void *C, const float *A, const float *Dskip, void *y,
                 hipStream_t stream) {
    return bdssm_commit_ex(shape, h_cache, x, dt, B, C, A, Dskip, y, nullptr, stream);
}

int bdssm_train_scan(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                     const void *B, const void *C, const float *A, const float *Dskip,
                     const float *h_init, void *y, float *h_bounds, void *ws, size_t ws_bytes,
                     hipStream_t stream) {
    return bdssm_train_scan_ex(shape, T, x, dt, B, C, A, Dskip, h_init, y, h_bounds, ws, ws_bytes, nullptr,
                               stream);
}

int bdssm_full_scan(const bdssm_shape *shape, int64_t T, const void *x, const void *dt,
                    const void *B, const void *C, const float *A, const float *Dskip, void *y,
                    void *ws, size_t ws_bytes, hipStream_t stream) {
    return bdssm_full_scan_ex(shape, T, x, dt, B, C, A, Dskip, y, ws, ws_bytes, nullptr, stream);
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
                         bdssm_fusion_grads *grads, hipStream_t stream) {
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
    hipStream_t st = stream;
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
        if (general || lng || N != kStates) {
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
        else launch_bwd<uint16_t, false>(L, N, a, batch, T, D, Tc, nc, st);
        launch_bwd_reduce<uint16_t>(w, dB, dC, dA, dDskip, batch, T, D, L, N, nc, st, a.fused, d_bias,
                                    a.sep ? grads : nullptr);
    } else {
        if (general) launch_bwd_general<float, false>(N, a, batch, T, D, L, Tc, nc, st);
        else if (lng) launch_bwd_long<float, false>(a, w.gstate, batch, T, D, L, Tc, nc, st);
        else launch_bwd<float, false>(L, N, a, batch, T, D, Tc, nc, st);
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
                                bdssm_fusion_grads *grads, hipStream_t stream) {
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
    hipStream_t st = stream;
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
        else launch_bwd<uint16_t, true>(L, N, a, batch, T, D, tc, (int)nc, st);
        launch_bwd_reduce<uint16_t>(w, dB, dC, dA, dDskip, batch, T, D, L, N, nc, st, a.fused, d_bias,
                                    a.sep ? grads : nullptr);
    } else {
        if (general) launch_bwd_general<float, true>(N, a, batch, T, D, L, tc, (int)nc, st);
        else if (lng) launch_bwd_long<float, true>(a, w.gstate, batch, T, D, L, tc, (int)nc, st);
        else launch_bwd<float, true>(L, N, a, batch, T, D, tc, (int)nc, st);
        launch_bwd_reduce<float>(w, dB, dC, dA, dDskip, batch, T, D, L, N, nc, st, a.fused, d_bias,
                                 a.sep ? grads : nullptr);
    }
    return launch_status();
}

}  // extern "C"

