// api.hip -- the extern "C" entry points of libsla (declared in include/sla.h).
//
// Host-side only: argument checks, per-row counts, workspace carving and the
// launch sequence pool -> classify -> block states -> assemble -> fused, all
// on the caller's stream.  No host synchronisation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <string>
#include <vector>

#include "sla.h"
#include "sla_launch.h"

namespace {

thread_local std::string g_err;

sla_status fail(sla_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
sla_status fail(sla_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

sla_status device_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return SLA_OK;
    return fail(SLA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int MAX_NB = 2432;        // score-based masks (the selection holds a row of scores per wave)
constexpr int MAX_NB_LISTS = 4095;  // masks from lists or frame sets: 12-bit block indices in the slots

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
long round_up(long x, long m) { return (x + m - 1) / m * m; }

sla_status counts_impl(long Nb, double rc, double rn, int *kc, int *kn) {
    if (!(rc >= 0.0 && rc <= 1.0) || !(rn >= 0.0 && rn <= 1.0) || rc + rn > 1.0 + 1e-12)
        return fail(SLA_ERR_INVALID_ARG, "fractions must lie in [0,1] and sum to at most 1 (got %g, %g)", rc, rn);
    double c = ceil(rc * (double)Nb - 1e-9);
    double n = floor(rn * (double)Nb + 1e-9);
    if (c < 0) c = 0;
    if (c > (double)Nb) c = (double)Nb;
    if (n < 0) n = 0;
    if (n > (double)Nb - c) n = (double)Nb - c;
    *kc = (int)c;
    *kn = (int)n;
    return SLA_OK;
}

sla_status check_shape(int B, int H, int N, int d, int block, int max_nb = MAX_NB) {
    if (B < 1 || H < 1 || N < 1) return fail(SLA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
    if (d != 64 && d != 128) return fail(SLA_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", d);
    if (block != 64) return fail(SLA_ERR_UNSUPPORTED, "block size %d not supported (64)", block);
    const long Nb = (N + 63) / 64;
    if (Nb > max_nb) return fail(SLA_ERR_UNSUPPORTED, "N = %d gives %ld blocks; at most %d are supported", N, Nb, max_nb);
    return SLA_OK;
}

struct Layout {
    size_t qp, kp, kpack, mask, crit, marg, mbits, mcount, ulist, ucount, wst, hs, hhat, total;
    int Nb, Nbc, Nbp, Lp, kc, kn;
};

Layout make_layout(int B, int H, int N, int d, bool f32, int kc, int kn) {
    Layout L;
    const long BH = (long)B * H;
    L.Nb = (N + 63) / 64;
    L.Nbc = (int)round_up(L.Nb, 64);
    L.Nbp = (int)round_up(L.Nb, 512);
    L.Lp = (int)round_up((long)d * d + d, 256);
    L.kc = kc;
    L.kn = kn;
    const size_t es = f32 ? 4 : 2;   // state element size
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    L.qp = take(sizeof(float) * BH * L.Nb * d);
    L.kp = take(sizeof(float) * BH * L.Nb * d);
    L.kpack = take(sizeof(float) * BH * sla::classify_packed_keys(L.Nb) * d);
    L.mask = take((size_t)BH * L.Nb * L.Nb);
    L.crit = take(sizeof(int32_t) * BH * L.Nb * (kc > 0 ? kc : 1));
    L.mcount = take(sizeof(int32_t) * BH * L.Nb);
    const long Np = (L.Nb + 1) / 2;
    // float inputs: union of each row pair's critical lists (16-bit inputs read the critical lists)
    L.ulist = take(f32 ? sizeof(uint32_t) * BH * Np * 2 * (kc > 0 ? kc : 1) : 0);
    L.ucount = take(f32 ? sizeof(int32_t) * BH * Np : 0);
    const bool states = kc + kn < L.Nb;
    // marginal indicator: float rows for float inputs, bits for 16-bit inputs
    L.marg = take(states && f32 ? sizeof(float) * BH * L.Nb * L.Nbc : 0);
    L.mbits = take(states && !f32 ? sizeof(uint32_t) * BH * (L.Nbc / 32) * L.Nbp : 0);
    L.wst = take(states ? es * d * d : 0);
    L.hs = take(states ? es * BH * L.Nbc * L.Lp : 0);     // one row per key block, padded to Nbc rows
    L.hhat = take(states ? es * BH * L.Nb * L.Lp : 0);
    L.total = off;
    return L;
}

// Per-thread stage timing (sla_set_stage_timing / sla_stage_times): a start
// and an end event per stage, recorded on the stream the stage runs on.
typedef std::array<hipEvent_t, 2 * SLA_NUM_STAGES> StageEvents;
struct StageTimer {
    bool on = false;
    std::vector<hipEvent_t> pool;      // created events, reused
    size_t used = 0;
    std::vector<StageEvents> calls;

    hipEvent_t next() {
        if (used == pool.size()) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return nullptr;
            pool.push_back(e);
        }
        return pool[used++];
    }
};
thread_local StageTimer g_timer;

// Records the start (end = 0) or the end (end = 1) of stage `i` of the current call.
void mark_stage(StageEvents *ev, int i, int end, hipStream_t s) {
    if (ev && (*ev)[2 * i + end]) (void)hipEventRecord((*ev)[2 * i + end], s);   // timing only: a failed record is not an error of the call
}

// The event set of a new call while timing is on, else nullptr.
StageEvents *timed_call() {
    if (!g_timer.on) return nullptr;
    StageEvents set;
    for (auto &e : set) e = g_timer.next();
    g_timer.calls.push_back(set);
    return &g_timer.calls.back();
}

// Calls over a given block schedule: stage 1 is building the schedule, stage
// 4 the attention kernel, stage 3 the merge of its shares (when it runs in
// shares); pool and states do not run (zero time).
void mark_unused_stages(StageEvents *ev, hipStream_t s) {
    for (int i : {0, 2}) {
        mark_stage(ev, i, 0, s);
        mark_stage(ev, i, 1, s);
    }
}

}  // namespace

namespace sla {
// Sets the thread's error text (sla_last_error) for entry points defined in
// other source files, and returns st.
sla_status set_error(sla_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}
}  // namespace sla

extern "C" {

sla_status sla_set_stage_timing(int enable) {
    g_timer.on = enable != 0;
    return SLA_OK;
}

sla_status sla_stage_times(float *ms, int *calls) {
    if (!ms || !calls) return fail(SLA_ERR_INVALID_ARG, "ms and calls must not be NULL");
    for (int i = 0; i < SLA_NUM_STAGES; ++i) ms[i] = 0.f;
    *calls = (int)g_timer.calls.size();
    for (auto &ev : g_timer.calls) {
        for (int i = 0; i < SLA_NUM_STAGES; ++i) {
            hipError_t e = hipEventSynchronize(ev[2 * i + 1]);
            if (e != hipSuccess) return device_status(e, "stage timing");
            float t = 0.f;
            e = hipEventElapsedTime(&t, ev[2 * i], ev[2 * i + 1]);
            if (e != hipSuccess) return device_status(e, "stage timing");
            ms[i] += t;
        }
    }
    g_timer.calls.clear();
    g_timer.used = 0;
    return SLA_OK;
}

int sla_version(void) { return 100; }

// Long slot schedules run in shares (each workgroup one share of its row
// pair's slots, share-major order, so that the workgroups resident on an
// XCD use one share's tiles through its L2), merged by their log-sum-exp.
// (from 256 slots per row: shorter schedules, such as the sliding tiles', ran
// slower in shares, their tiles staying in L2 without them)
static int slot_nchunk(int kmax) { return kmax >= 256 ? 4 : 1; }
// fp16 partial outputs (normalized per share, so |values| <= max |V|; sized
// for d = 128, the largest d) and float log-sum-exps
static size_t slot_chunk_bytes(long BH, int Nb, int nchunk) {
    if (nchunk <= 1) return 0;
    return align256(sizeof(uint16_t) * (size_t)nchunk * BH * 64 * Nb * 128) +
           align256(sizeof(float) * (size_t)nchunk * BH * 64 * Nb);
}
// the fused launch over a slot schedule, in shares when it is long enough;
// the partial buffers follow `tail` in the workspace
static sla_status slots_attention(sla::FusedArgs fa, int kmax, char *tail, void *out, bool bf16_out, hipStream_t s,
                                  StageEvents *ev) {
    const int nchunk = slot_nchunk(kmax);
    _Float16 *part = nullptr;
    float *plse = nullptr;
    if (nchunk > 1) {
        part = (_Float16 *)tail;
        plse = (float *)(tail + align256(sizeof(uint16_t) * (size_t)nchunk * fa.BH * 64 * fa.Nb * 128));
        fa.nchunk = nchunk;
        fa.out = part; fa.lse = plse; fa.bf16_out = false;
    }
    mark_stage(ev, 4, 0, s);
    sla_status st = device_status(sla::launch_fused16s(fa, s), "fused launch");
    mark_stage(ev, 4, 1, s);
    mark_stage(ev, 3, 0, s);
    if (st == SLA_OK && nchunk > 1)
        st = device_status(sla::launch_chunk_merge(part, plse, nchunk, fa.BH, fa.N, fa.Nb, fa.D, out, bf16_out, s),
                           "chunk merge launch");
    mark_stage(ev, 3, 1, s);
    return st;
}

sla_status sla_lists_workspace_size(int B, int H, int N, int kmax, size_t *bytes) {
    if (!bytes) return fail(SLA_ERR_INVALID_ARG, "bytes must not be NULL");
    sla_status st = check_shape(B, H, N, 128, 64, MAX_NB_LISTS);
    if (st != SLA_OK) return st;
    const int Nb = (N + 63) / 64;
    if (kmax < 1 || kmax > Nb) return fail(SLA_ERR_INVALID_ARG, "kmax must lie in [1, Nb] (got %d, Nb = %d)", kmax, Nb);
    const size_t pairs = (size_t)B * H * ((Nb + 1) / 2);
    *bytes = align256(sizeof(uint32_t) * pairs * kmax) + align256(sizeof(int32_t) * pairs) +
             slot_chunk_bytes((long)B * H, Nb, slot_nchunk(kmax));
    return SLA_OK;
}

sla_status sla_forward_lists(const void *q, const void *k, const void *v, sla_dtype in_dtype, sla_dtype out_dtype,
                             int B, int H, int N, int d, int block, const int32_t *lists, const int32_t *counts,
                             int kmax, void *out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !lists || !counts || !out) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    sla_status st = check_shape(B, H, N, d, block, MAX_NB_LISTS);
    if (st != SLA_OK) return st;
    if (in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "attention over given lists takes bf16 inputs");
    if (out_dtype != SLA_F32 && out_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "output dtype must be F32 or BF16");
    size_t need = 0;
    st = sla_lists_workspace_size(B, H, N, kmax, &need);
    if (st != SLA_OK) return st;
    if (!workspace) return fail(SLA_ERR_INVALID_ARG, "null workspace");
    if (workspace_bytes < need)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if (((uintptr_t)workspace & 255) != 0) return fail(SLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const long BH = (long)B * H;
    const int Nb = (N + 63) / 64;
    uint32_t *slots = (uint32_t *)workspace;
    int32_t *pcount = (int32_t *)((char *)workspace + align256(sizeof(uint32_t) * (size_t)BH * ((Nb + 1) / 2) * kmax));
    StageEvents *ev = timed_call();
    mark_unused_stages(ev, s);
    mark_stage(ev, 1, 0, s);
    st = device_status(sla::launch_lists_to_slots(lists, counts, kmax, BH, Nb, slots, pcount, s), "slot schedule launch");
    mark_stage(ev, 1, 1, s);
    if (st != SLA_OK) return st;
    sla::FusedArgs fa{};
    fa.q = q; fa.k = k; fa.v = v; fa.slots = slots; fa.kc = kmax; fa.pcount = pcount;
    fa.out = out; fa.BH = BH; fa.N = N; fa.Nb = Nb; fa.D = d;
    fa.bf16_in = true; fa.bf16_out = out_dtype == SLA_BF16;
    return slots_attention(fa, kmax, (char *)pcount + align256(sizeof(int32_t) * (size_t)BH * ((Nb + 1) / 2)), out,
                           out_dtype == SLA_BF16, s, ev);
}

// ---- LVSA frame-level sets --------------------------------------------------

static sla_status lvsa_params(int T, int C, int W, int step, sla::LvsaParams *p, int *frames_per_set) {
    if (T < 1) return fail(SLA_ERR_INVALID_ARG, "T must be >= 1 (got %d)", T);
    if (W < 0 || step < 0) return fail(SLA_ERR_INVALID_ARG, "W and step must be >= 0 (got %d, %d)", W, step);
    if (C - (2 * W + 1) < 1) return fail(SLA_ERR_INVALID_ARG, "the budget C = %d must exceed the window 2W + 1 = %d", C, 2 * W + 1);
    const int K = C - (2 * W + 1);
    p->T = T; p->W = W; p->s = step;
    p->Tper = (T + K - 1) / K;
    p->m = (T + p->Tper - 1) / p->Tper;
    *frames_per_set = p->m + std::min(2 * W + 1, T - p->m);
    return SLA_OK;
}

sla_status sla_lvsa_plan(int T, int C, int W, int *t_per, int *n_global, int *frames_per_set) {
    if (!t_per || !n_global || !frames_per_set) return fail(SLA_ERR_INVALID_ARG, "null output pointer");
    sla::LvsaParams p;
    int f;
    sla_status st = lvsa_params(T, C, W, 0, &p, &f);
    if (st != SLA_OK) return st;
    *t_per = p.Tper; *n_global = p.m; *frames_per_set = f;
    return SLA_OK;
}

sla_status sla_lvsa_sets(int T, int C, int W, int step, int32_t *sets, int32_t *counts, int max_frames,
                         void *stream) {
    if (!sets || !counts) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    sla::LvsaParams p;
    int f;
    sla_status st = lvsa_params(T, C, W, step, &p, &f);
    if (st != SLA_OK) return st;
    if (max_frames < f) return fail(SLA_ERR_INVALID_ARG, "max_frames = %d is below the set size %d", max_frames, f);
    return device_status(sla::launch_lvsa_frames(p, nullptr, sets, counts, max_frames, (hipStream_t)stream),
                         "frame set launch");
}

// slots per pair: a row takes the key blocks touched by at most two frames' sets
static int lvsa_kmax(int Nb, int P, int frames_per_set) {
    const long bound = 2L * frames_per_set * ((P + 63) / 64 + 1);
    return (int)std::min<long>(Nb, bound);
}

static sla_status lvsa_shape(int B, int H, int N, int d, int block, int T, int *P) {
    sla_status st = check_shape(B, H, N, d, block, MAX_NB_LISTS);
    if (st != SLA_OK) return st;
    if (T < 1 || N % T != 0) return fail(SLA_ERR_INVALID_ARG, "N = %d is not T = %d frames of equal size", N, T);
    *P = N / T;
    if (*P < 64) return fail(SLA_ERR_UNSUPPORTED, "frames of %d tokens: at least 64 are needed", *P);
    return SLA_OK;
}

sla_status sla_lvsa_workspace_size(int B, int H, int N, int T, int C, int W, size_t *bytes) {
    if (!bytes) return fail(SLA_ERR_INVALID_ARG, "bytes must not be NULL");
    int P, f;
    sla_status st = lvsa_shape(B, H, N, 128, 64, T, &P);
    if (st != SLA_OK) return st;
    sla::LvsaParams p;
    st = lvsa_params(T, C, W, 0, &p, &f);
    if (st != SLA_OK) return st;
    const int Nb = (N + 63) / 64, Np = (Nb + 1) / 2;
    const int kmax = lvsa_kmax(Nb, P, f);
    *bytes = align256(sizeof(int32_t) * 2 * (size_t)T) + align256(sizeof(uint32_t) * (size_t)Np * kmax) +
             align256(sizeof(int32_t) * (size_t)Np) + slot_chunk_bytes((long)B * H, Nb, slot_nchunk(kmax));
    return SLA_OK;
}

sla_status sla_forward_lvsa(const void *q, const void *k, const void *v, sla_dtype in_dtype, sla_dtype out_dtype,
                            int B, int H, int N, int d, int block, int T, int C, int W, int step, void *out,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !out) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    int P, f;
    sla_status st = lvsa_shape(B, H, N, d, block, T, &P);
    if (st != SLA_OK) return st;
    if (in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "LVSA attention takes bf16 inputs");
    if (out_dtype != SLA_F32 && out_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "output dtype must be F32 or BF16");
    sla::LvsaParams p;
    st = lvsa_params(T, C, W, step, &p, &f);
    if (st != SLA_OK) return st;
    size_t need = 0;
    st = sla_lvsa_workspace_size(B, H, N, T, C, W, &need);
    if (st != SLA_OK) return st;
    if (!workspace) return fail(SLA_ERR_INVALID_ARG, "null workspace");
    if (workspace_bytes < need)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if (((uintptr_t)workspace & 255) != 0) return fail(SLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int Nb = (N + 63) / 64, Np = (Nb + 1) / 2;
    const int kmax = lvsa_kmax(Nb, P, f);
    char *w = (char *)workspace;
    int32_t *lohi = (int32_t *)w;
    uint32_t *slots = (uint32_t *)(w + align256(sizeof(int32_t) * 2 * (size_t)T));
    int32_t *pcount = (int32_t *)((char *)slots + align256(sizeof(uint32_t) * (size_t)Np * kmax));
    StageEvents *ev = timed_call();
    mark_unused_stages(ev, s);
    mark_stage(ev, 1, 0, s);
    st = device_status(sla::launch_lvsa_frames(p, lohi, nullptr, nullptr, 0, s), "frame window launch");
    if (st == SLA_OK)
        st = device_status(sla::launch_lvsa_slots(p, P, N, Nb, lohi, kmax, slots, pcount, s), "slot schedule launch");
    mark_stage(ev, 1, 1, s);
    if (st != SLA_OK) return st;
    sla::FusedArgs fa{};
    fa.q = q; fa.k = k; fa.v = v; fa.slots = slots; fa.kc = kmax; fa.pcount = pcount; fa.bcast = true; fa.fp = P;
    fa.out = out; fa.BH = (long)B * H; fa.N = N; fa.Nb = Nb; fa.D = d;
    fa.bf16_in = true; fa.bf16_out = out_dtype == SLA_BF16;
    return slots_attention(fa, kmax, (char *)pcount + align256(sizeof(int32_t) * (size_t)Np), out,
                           out_dtype == SLA_BF16, s, ev);
}

// ---- STA tiles -----------------------------------------------------------

struct StaShape {
    sla::StaParams p;
    int N, Nb, kmax;
};

static sla_status sta_shape(int F, int Hh, int Ww, int tf, int th, int tw, int wf, int wh, int ww, StaShape *o) {
    if (F < 1 || Hh < 1 || Ww < 1) return fail(SLA_ERR_INVALID_ARG, "grid must be >= 1 on every axis (got %d, %d, %d)", F, Hh, Ww);
    if (tf < 1 || th < 1 || tw < 1 || F % tf || Hh % th || Ww % tw)
        return fail(SLA_ERR_INVALID_ARG, "tiles (%d, %d, %d) must divide the grid (%d, %d, %d)", tf, th, tw, F, Hh, Ww);
    if (wf < 1 || wh < 1 || ww < 1) return fail(SLA_ERR_INVALID_ARG, "windows must be >= 1 (got %d, %d, %d)", wf, wh, ww);
    const long vol = (long)tf * th * tw;
    if (vol % 64) return fail(SLA_ERR_UNSUPPORTED, "a tile of %ld tokens is not whole 64-token blocks", vol);
    const long N = (long)F * Hh * Ww;
    if (N > 64L * MAX_NB_LISTS) return fail(SLA_ERR_UNSUPPORTED, "N = %ld gives more than %d blocks", N, MAX_NB_LISTS);
    sla::StaParams &p = o->p;
    p.tf = tf; p.th = th; p.tw = tw; p.wf = wf; p.wh = wh; p.ww = ww;
    p.gf = F / tf; p.gh = Hh / th; p.gw = Ww / tw; p.vol = (int)vol;
    p.rf = std::min(wf / (2 * tf) + 1, p.gf);
    p.rh = std::min(wh / (2 * th) + 1, p.gh);
    p.rw = std::min(ww / (2 * tw) + 1, p.gw);
    // kept tile offsets per axis: 2*delta*t in (-W, W]
    auto count = [](int t, int W, int r) {
        int c = 0;
        for (int d = -r; d <= r; ++d) c += (2 * d * t > -W && 2 * d * t <= W);
        return c;
    };
    const long tiles = (long)count(tf, wf, p.rf) * count(th, wh, p.rh) * count(tw, ww, p.rw);
    o->N = (int)N;
    o->Nb = (int)(N / 64);
    o->kmax = (int)std::max<long>(1, std::min<long>(o->Nb, tiles * (vol / 64)));
    return SLA_OK;
}

sla_status sla_sta_tile_order(int F, int Hh, int Ww, int tf, int th, int tw, int32_t *perm) {
    if (!perm) return fail(SLA_ERR_INVALID_ARG, "perm must not be NULL");
    if (F < 1 || Hh < 1 || Ww < 1 || tf < 1 || th < 1 || tw < 1 || F % tf || Hh % th || Ww % tw)
        return fail(SLA_ERR_INVALID_ARG, "tiles (%d, %d, %d) must divide the grid (%d, %d, %d)", tf, th, tw, F, Hh, Ww);
    const int gh = Hh / th, gw = Ww / tw;
    long m = 0;
    for (int gf_ = 0; gf_ < F / tf; ++gf_)
        for (int gh_ = 0; gh_ < gh; ++gh_)
            for (int gw_ = 0; gw_ < gw; ++gw_)
                for (int f = 0; f < tf; ++f)
                    for (int h = 0; h < th; ++h)
                        for (int w = 0; w < tw; ++w)
                            perm[m++] = (int32_t)(((long)(gf_ * tf + f) * Hh + gh_ * th + h) * Ww + gw_ * tw + w);
    return SLA_OK;
}

sla_status sla_sta_workspace_size(int B, int H, int F, int Hh, int Ww, int tf, int th, int tw, int wf, int wh, int ww,
                                  size_t *bytes) {
    if (!bytes) return fail(SLA_ERR_INVALID_ARG, "bytes must not be NULL");
    if (B < 1 || H < 1) return fail(SLA_ERR_INVALID_ARG, "B, H must be >= 1 (got %d, %d)", B, H);
    StaShape sh;
    sla_status st = sta_shape(F, Hh, Ww, tf, th, tw, wf, wh, ww, &sh);
    if (st != SLA_OK) return st;
    const size_t Np = (size_t)(sh.Nb + 1) / 2;
    *bytes = align256(sizeof(uint32_t) * Np * sh.kmax) + align256(sizeof(int32_t) * Np) +
             slot_chunk_bytes((long)B * H, sh.Nb, slot_nchunk(sh.kmax));
    return SLA_OK;
}

sla_status sla_forward_sta(const void *q, const void *k, const void *v, sla_dtype in_dtype, sla_dtype out_dtype,
                           int B, int H, int d, int block, int F, int Hh, int Ww, int tf, int th, int tw, int wf,
                           int wh, int ww, void *out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !out) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    StaShape sh;
    sla_status st = sta_shape(F, Hh, Ww, tf, th, tw, wf, wh, ww, &sh);
    if (st != SLA_OK) return st;
    st = check_shape(B, H, sh.N, d, block, MAX_NB_LISTS);
    if (st != SLA_OK) return st;
    if (in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "sliding tile attention takes bf16 inputs");
    if (out_dtype != SLA_F32 && out_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "output dtype must be F32 or BF16");
    size_t need = 0;
    st = sla_sta_workspace_size(B, H, F, Hh, Ww, tf, th, tw, wf, wh, ww, &need);
    if (st != SLA_OK) return st;
    if (!workspace) return fail(SLA_ERR_INVALID_ARG, "null workspace");
    if (workspace_bytes < need)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if (((uintptr_t)workspace & 255) != 0) return fail(SLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int Np = (sh.Nb + 1) / 2;
    uint32_t *slots = (uint32_t *)workspace;
    int32_t *pcount = (int32_t *)((char *)workspace + align256(sizeof(uint32_t) * (size_t)Np * sh.kmax));
    StageEvents *ev = timed_call();
    mark_unused_stages(ev, s);
    mark_stage(ev, 1, 0, s);
    st = device_status(sla::launch_sta_slots(sh.p, sh.Nb, sh.kmax, slots, pcount, s), "slot schedule launch");
    mark_stage(ev, 1, 1, s);
    if (st != SLA_OK) return st;
    sla::FusedArgs fa{};
    fa.q = q; fa.k = k; fa.v = v; fa.slots = slots; fa.kc = sh.kmax; fa.pcount = pcount; fa.bcast = true;
    fa.out = out; fa.BH = (long)B * H; fa.N = sh.N; fa.Nb = sh.Nb; fa.D = d;
    fa.bf16_in = true; fa.bf16_out = out_dtype == SLA_BF16;
    return slots_attention(fa, sh.kmax, (char *)pcount + align256(sizeof(int32_t) * (size_t)Np), out,
                           out_dtype == SLA_BF16, s, ev);
}

sla_status sla_block_mass(const void *q, const void *k, sla_dtype in_dtype, int B, int H, int N, int d, int block,
                          float *mass, void *stream) {
    if (!q || !k || !mass) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    sla_status st = check_shape(B, H, N, d, block);
    if (st != SLA_OK) return st;
    if (in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "block mass takes bf16 inputs");
    sla::MassArgs a{};
    a.q = q; a.k = k; a.BH = (long)B * H; a.N = N; a.Nb = (N + 63) / 64; a.D = d; a.mass = mass;
    return device_status(sla::launch_block_mass(a, (hipStream_t)stream), "block mass launch");
}

sla_status sla_mask_stats(const float *mass, const int8_t *mask, long rows, int Nb, float *stats, void *stream) {
    if (!mass || !mask || !stats) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    if (rows < 1 || Nb < 1) return fail(SLA_ERR_INVALID_ARG, "rows and Nb must be >= 1");
    if (Nb > MAX_NB) return fail(SLA_ERR_UNSUPPORTED, "Nb = %d exceeds the supported %d", Nb, MAX_NB);
    return device_status(sla::launch_mask_stats(mass, mask, rows, Nb, stats, (hipStream_t)stream), "mask stats launch");
}

const char *sla_last_error(void) { return g_err.c_str(); }

sla_status sla_counts(int Nb, double crit_frac, double negl_frac, int *k_c, int *k_n) {
    if (!k_c || !k_n) return fail(SLA_ERR_INVALID_ARG, "k_c and k_n must not be NULL");
    if (Nb < 1) return fail(SLA_ERR_INVALID_ARG, "Nb must be >= 1 (got %d)", Nb);
    return counts_impl(Nb, crit_frac, negl_frac, k_c, k_n);
}

sla_status sla_workspace_size(int B, int H, int N, int d, int block, sla_dtype in_dtype, double crit_frac,
                              double negl_frac, size_t *bytes) {
    if (!bytes) return fail(SLA_ERR_INVALID_ARG, "bytes must not be NULL");
    sla_status st = check_shape(B, H, N, d, block);
    if (st != SLA_OK) return st;
    if (in_dtype != SLA_F32 && in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "input dtype %d not supported", (int)in_dtype);
    int kc, kn;
    st = counts_impl((N + 63) / 64, crit_frac, negl_frac, &kc, &kn);
    if (st != SLA_OK) return st;
    *bytes = make_layout(B, H, N, d, in_dtype == SLA_F32, kc, kn).total;
    return SLA_OK;
}

sla_status sla_pool(const void *q, const void *k, sla_dtype in_dtype, int B, int H, int N, int d, int block,
                    float *q_pool, float *k_pool, void *stream) {
    if (!q || !k || !q_pool || !k_pool) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    sla_status st = check_shape(B, H, N, d, block);
    if (st != SLA_OK) return st;
    if (in_dtype != SLA_F32 && in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "input dtype %d not supported", (int)in_dtype);
    const int Nb = (N + 63) / 64;
    return device_status(sla::launch_pool(in_dtype == SLA_BF16, d, q, k, q_pool, k_pool, nullptr, (long)B * H, N, Nb, 64,
                                          (hipStream_t)stream),
                         "pool launch");
}

sla_status sla_classify(const float *q_pool, const float *k_pool, int B, int H, int Nb, int d, double crit_frac,
                        double negl_frac, int8_t *mask, int32_t *crit_idx, int32_t *excl_idx, float *p_c,
                        void *stream) {
    if (!q_pool || !k_pool || !mask) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    if (B < 1 || H < 1 || Nb < 1) return fail(SLA_ERR_INVALID_ARG, "B, H, Nb must be >= 1");
    if (d != 64 && d != 128) return fail(SLA_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", d);
    if (Nb > MAX_NB) return fail(SLA_ERR_UNSUPPORTED, "Nb = %d exceeds the supported %d", Nb, MAX_NB);
    int kc, kn;
    sla_status st = counts_impl(Nb, crit_frac, negl_frac, &kc, &kn);
    if (st != SLA_OK) return st;
    if (kc > 0 && !crit_idx) return fail(SLA_ERR_INVALID_ARG, "crit_idx must not be NULL when k_c > 0");
    sla::ClassifyArgs a{};
    a.qp = q_pool; a.kp = k_pool; a.BH = (long)B * H; a.Nb = Nb; a.D = d; a.kc = kc; a.kn = kn;
    a.mask = mask; a.crit = crit_idx; a.excl = excl_idx; a.pc = p_c;
    a.marg = nullptr; a.mbits = nullptr; a.Nbc = 0; a.Nbp = 0; a.mcount = nullptr; a.n_last = 64;
    a.ulist = nullptr; a.ucount = nullptr;
    a.inv_sqrt_d = 1.0 / sqrt((double)d);
    return device_status(sla::launch_classify(a, (hipStream_t)stream), "classify launch");
}

// The forward pass; with lse_out the fused kernel also writes each row's
// log-sum-exp, with os_out the sparse part of the output alone (float32),
// and with linear_off it leaves the linear branch out of `out` (the states
// and the marginal sums are still formed), as the backward needs.
static sla_status forward_impl(const void *q, const void *k, const void *v, const float *w_proj, sla_dtype in_dtype,
                               sla_dtype out_dtype, int B, int H, int N, int d, int block, double crit_frac,
                               double negl_frac, sla_phi phi, void *out, int8_t *mask_out, void *workspace,
                               size_t workspace_bytes, void *stream, float *lse_out, bool linear_off,
                               bool timed = true, float *os_out = nullptr) {
    if (!q || !k || !v || !w_proj || !out) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    sla_status st = check_shape(B, H, N, d, block);
    if (st != SLA_OK) return st;
    if (in_dtype != SLA_F32 && in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "input dtype %d not supported", (int)in_dtype);
    if (out_dtype != SLA_F32 && out_dtype != in_dtype)
        return fail(SLA_ERR_UNSUPPORTED, "output dtype must be F32 or the input dtype");
    if (phi != SLA_PHI_SOFTMAX) return fail(SLA_ERR_UNSUPPORTED, "feature map %d not supported", (int)phi);
    int kc, kn;
    const int Nb = (N + 63) / 64;
    st = counts_impl(Nb, crit_frac, negl_frac, &kc, &kn);
    if (st != SLA_OK) return st;
    const bool f32 = in_dtype == SLA_F32;
    const Layout L = make_layout(B, H, N, d, f32, kc, kn);
    if (!workspace && L.total > 0) return fail(SLA_ERR_INVALID_ARG, "null workspace");
    if (workspace_bytes < L.total)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, L.total);
    if (((uintptr_t)workspace & 255) != 0) return fail(SLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    char *ws = (char *)workspace;
    hipStream_t s = (hipStream_t)stream;
    const long BH = (long)B * H;
    const bool states = kc + kn < Nb;
    float *qp = (float *)(ws + L.qp), *kp = (float *)(ws + L.kp);
    int8_t *mask = mask_out ? mask_out : (int8_t *)(ws + L.mask);
    int32_t *crit = (int32_t *)(ws + L.crit);
    int32_t *mcount = (int32_t *)(ws + L.mcount);

    StageEvents *ev = timed ? timed_call() : nullptr;
    mark_stage(ev, 0, 0, s);
    float *kpack = (float *)(ws + L.kpack);
    st = device_status(sla::launch_pool(!f32, d, q, k, qp, kp, kpack, BH, N, Nb, 64, s), "pool launch");
    if (st != SLA_OK) return st;
    mark_stage(ev, 0, 1, s);

    sla::ClassifyArgs ca{};
    ca.qp = qp; ca.kp = kp; ca.kpack = kpack; ca.BH = BH; ca.Nb = Nb; ca.D = d; ca.kc = kc; ca.kn = kn;
    ca.mask = mask; ca.crit = crit; ca.excl = nullptr; ca.pc = nullptr;
    ca.marg = states && f32 ? (float *)(ws + L.marg) : nullptr;
    ca.mbits = states && !f32 ? (uint32_t *)(ws + L.mbits) : nullptr;
    ca.Nbc = L.Nbc; ca.Nbp = L.Nbp;
    ca.mcount = mcount; ca.n_last = N - 64 * (Nb - 1);
    ca.ulist = f32 ? (uint32_t *)(ws + L.ulist) : nullptr;
    ca.ucount = f32 ? (int32_t *)(ws + L.ucount) : nullptr;
    ca.inv_sqrt_d = 1.0 / sqrt((double)d);
    mark_stage(ev, 1, 0, s);
    st = device_status(sla::launch_classify(ca, s), "classify launch");
    if (st != SLA_OK) return st;
    mark_stage(ev, 1, 1, s);

    // block states (they need only K, V and W).  They run after pool and
    // classify rather than beside them: the state kernel's persistent
    // workgroups fill every compute unit's registers, so nothing would run
    // next to them anyway.
    if (states) {
        sla::StateArgs sa{};
        sa.k = k; sa.v = v; sa.w = w_proj; sa.BH = BH; sa.N = N; sa.Nb = Nb; sa.D = d; sa.Lp = L.Lp; sa.Nbc = L.Nbc;
        sa.hs = ws + L.hs; sa.wstate = ws + L.wst; sa.bf16_in = !f32;
        mark_stage(ev, 2, 0, s);
        st = device_status(sla::launch_state(sa, s), "state launch");
        mark_stage(ev, 2, 1, s);
        if (st != SLA_OK) return st;
    } else {
        mark_stage(ev, 2, 0, s);
        mark_stage(ev, 2, 1, s);
    }
    mark_stage(ev, 3, 0, s);
    if (states) {
        sla::AssembleArgs aa{};
        aa.marg = ws + L.marg; aa.mbits = (const uint32_t *)(ws + L.mbits); aa.hs = ws + L.hs; aa.mcount = mcount; aa.hhat = ws + L.hhat;
        aa.BH = BH; aa.Nb = Nb; aa.Nbc = L.Nbc; aa.Nbp = L.Nbp; aa.Lp = L.Lp; aa.f32 = f32;
        st = device_status(sla::launch_assemble(aa, s), "assemble launch");
        if (st != SLA_OK) return st;
    }
    mark_stage(ev, 3, 1, s);
    mark_stage(ev, 4, 0, s);
    sla::FusedArgs fa{};
    fa.q = q; fa.k = k; fa.v = v; fa.ulist = (const uint32_t *)(ws + L.ulist);
    fa.ucount = (const int32_t *)(ws + L.ucount); fa.kc = kc;
    fa.hhat = ws + L.hhat; fa.mcount = states && !linear_off ? mcount : nullptr; fa.Lp = L.Lp;
    fa.out = out; fa.BH = BH; fa.N = N; fa.Nb = Nb; fa.D = d; fa.lse = lse_out; fa.os = os_out;
    fa.bf16_in = !f32; fa.bf16_out = out_dtype == SLA_BF16;
    fa.crit = (const int32_t *)(ws + L.crit);
    st = device_status(f32 ? sla::launch_fused(fa, s) : sla::launch_fused16s(fa, s), "fused launch");
    mark_stage(ev, 4, 1, s);
    return st;
}

sla_status sla_forward(const void *q, const void *k, const void *v, const float *w_proj, sla_dtype in_dtype,
                       sla_dtype out_dtype, int B, int H, int N, int d, int block, double crit_frac,
                       double negl_frac, sla_phi phi, void *out, int8_t *mask_out, void *workspace,
                       size_t workspace_bytes, void *stream) {
    return forward_impl(q, k, v, w_proj, in_dtype, out_dtype, B, H, N, d, block, crit_frac, negl_frac, phi, out,
                        mask_out, workspace, workspace_bytes, stream, nullptr, false);
}

// ---- backward ----------------------------------------------------------------

struct BwdLayout {
    size_t fwd, o_s, lse, dbuf, tlist, tcnt, mbitsT, dhr, dexp, kbyte, hexp, dhs, dwp, total;
};

static sla_status bwd_layout(int B, int H, int N, int d, int block, double crit_frac, double negl_frac,
                             BwdLayout *o, Layout *L, int *kc, int *kn) {
    sla_status st = check_shape(B, H, N, d, block);
    if (st != SLA_OK) return st;
    const int Nb = (N + 63) / 64;
    st = counts_impl(Nb, crit_frac, negl_frac, kc, kn);
    if (st != SLA_OK) return st;
    *L = make_layout(B, H, N, d, false, *kc, *kn);
    const size_t BH = (size_t)B * H;
    size_t off = align256(L->total);
    auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
    o->fwd = 0;
    o->o_s = take(sizeof(float) * BH * N * d);
    o->lse = take(sizeof(float) * BH * 64 * Nb);       // rows padded to whole blocks (aligned runs)
    o->dbuf = take(sizeof(float) * BH * 64 * Nb);
    o->tlist = take(sizeof(int32_t) * BH * Nb * Nb);
    o->tcnt = take(sizeof(int32_t) * BH * Nb);
    o->mbitsT = take(sizeof(uint32_t) * BH * (L->Nbc / 32) * L->Nbp);
    o->dhr = take(sizeof(uint16_t) * BH * L->Nbc * L->Lp);
    o->dexp = take(sizeof(int32_t) * BH * L->Nbc);
    o->kbyte = take(BH * L->Nbc);
    o->hexp = take(sizeof(int32_t) * BH);
    o->dhs = take(sizeof(uint16_t) * BH * Nb * L->Lp);
    o->dwp = take(sizeof(float) * sla::backward_key_groups((long)BH, Nb, d) * d * d);
    o->total = off;
    return SLA_OK;
}

sla_status sla_backward_workspace_size(int B, int H, int N, int d, int block, double crit_frac, double negl_frac,
                                       size_t *bytes) {
    if (!bytes) return fail(SLA_ERR_INVALID_ARG, "bytes must not be NULL");
    BwdLayout o;
    Layout L;
    int kc, kn;
    sla_status st = bwd_layout(B, H, N, d, block, crit_frac, negl_frac, &o, &L, &kc, &kn);
    if (st != SLA_OK) return st;
    *bytes = o.total;
    return SLA_OK;
}

// Checks shared by the backward entry points; the layout of the workspace.
static sla_status backward_checks(const void *q, const void *k, const void *v, const float *w_proj, const void *dout,
                                  sla_dtype in_dtype, int B, int H, int N, int d, int block, double crit_frac,
                                  double negl_frac, sla_phi phi, const float *dq, const float *dk, const float *dv,
                                  const float *dw, const void *workspace, size_t workspace_bytes, BwdLayout *o,
                                  Layout *L, int *kc, int *kn) {
    if (!q || !k || !v || !w_proj || !dout || !dq || !dk || !dv || !dw)
        return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    if (in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "the backward pass takes bf16 inputs");
    if (phi != SLA_PHI_SOFTMAX) return fail(SLA_ERR_UNSUPPORTED, "feature map %d not supported", (int)phi);
    sla_status st = bwd_layout(B, H, N, d, block, crit_frac, negl_frac, o, L, kc, kn);
    if (st != SLA_OK) return st;
    if (!workspace) return fail(SLA_ERR_INVALID_ARG, "null workspace");
    if (workspace_bytes < o->total)
        return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, o->total);
    if (((uintptr_t)workspace & 255) != 0) return fail(SLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return SLA_OK;
}

// The gradient stages, from the forward's labels, lists, marginal states,
// sparse output and log-sum-exp in the workspace (timed as stages 1-4).
static sla_status backward_grads(const void *q, const void *k, const void *v, const float *w_proj, const void *dout,
                                 int B, int H, int N, int d, float *dq, float *dk, float *dv, float *dw, char *ws,
                                 const BwdLayout &o, const Layout &L, int kc, int kn, hipStream_t s, StageEvents *ev) {
    const int Nb = (N + 63) / 64;
    sla::BackwardArgs a{};
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.w = w_proj;
    a.o_s = (const float *)(ws + o.o_s); a.lse = (const float *)(ws + o.lse);
    a.crit = (const int32_t *)(ws + L.crit); a.kc = kc; a.mask = (const int8_t *)(ws + L.mask);
    a.hhat = ws + L.hhat; a.mcount = (const int32_t *)(ws + L.mcount);
    a.dq = dq; a.dk = dk; a.dv = dv; a.dw = dw; a.dbuf = (float *)(ws + o.dbuf);
    a.tlist = (int32_t *)(ws + o.tlist); a.tcnt = (int32_t *)(ws + o.tcnt);
    a.mbitsT = (uint32_t *)(ws + o.mbitsT); a.dhr = ws + o.dhr; a.dexp = (int32_t *)(ws + o.dexp);
    a.kbyte = (uint8_t *)(ws + o.kbyte); a.hexp = (int32_t *)(ws + o.hexp);
    a.dhs = ws + o.dhs; a.dwp = (float *)(ws + o.dwp);
    a.BH = (long)B * H; a.N = N; a.Nb = Nb; a.Nbc = L.Nbc; a.Nbp = L.Nbp; a.Lp = L.Lp; a.D = d;
    mark_stage(ev, 1, 0, s);
    sla_status st = device_status(sla::launch_backward_dq(a, s), "backward dq launch");
    mark_stage(ev, 1, 1, s);
    if (st != SLA_OK) return st;
    mark_stage(ev, 2, 0, s);
    st = device_status(sla::launch_backward_dkv(a, s), "backward dk/dv launch");
    mark_stage(ev, 2, 1, s);
    if (st != SLA_OK) return st;
    const bool linear = kc + kn < Nb;
    mark_stage(ev, 3, 0, s);
    st = device_status(linear ? sla::launch_backward_lin_rows(a, s) : sla::launch_zero(dw, (long)d * d, s),
                       "backward linear rows launch");
    mark_stage(ev, 3, 1, s);
    if (st != SLA_OK) return st;
    mark_stage(ev, 4, 0, s);
    if (linear) st = device_status(sla::launch_backward_lin_keys(a, s), "backward linear keys launch");
    mark_stage(ev, 4, 1, s);
    return st;
}

sla_status sla_backward(const void *q, const void *k, const void *v, const float *w_proj, const void *dout,
                        sla_dtype in_dtype, int B, int H, int N, int d, int block, double crit_frac,
                        double negl_frac, sla_phi phi, float *dq, float *dk, float *dv, float *dw, void *workspace,
                        size_t workspace_bytes, void *stream) {
    BwdLayout o;
    Layout L;
    int kc, kn;
    sla_status st = backward_checks(q, k, v, w_proj, dout, in_dtype, B, H, N, d, block, crit_frac, negl_frac, phi, dq,
                                    dk, dv, dw, workspace, workspace_bytes, &o, &L, &kc, &kn);
    if (st != SLA_OK) return st;
    char *ws = (char *)workspace;
    hipStream_t s = (hipStream_t)stream;
    StageEvents *ev = timed_call();
    // the forward again: labels, critical lists, marginal states, and the
    // sparse output with its log-sum-exp
    mark_stage(ev, 0, 0, s);
    st = forward_impl(q, k, v, w_proj, SLA_BF16, SLA_F32, B, H, N, d, block, crit_frac, negl_frac, phi,
                      ws + o.o_s, nullptr, ws, L.total, stream, (float *)(ws + o.lse), true, false);
    mark_stage(ev, 0, 1, s);
    if (st != SLA_OK) return st;
    return backward_grads(q, k, v, w_proj, dout, B, H, N, d, dq, dk, dv, dw, ws, o, L, kc, kn, s, ev);
}

sla_status sla_forward_save(const void *q, const void *k, const void *v, const float *w_proj, sla_dtype in_dtype,
                            sla_dtype out_dtype, int B, int H, int N, int d, int block, double crit_frac,
                            double negl_frac, sla_phi phi, void *out, int8_t *mask_out, void *saved,
                            size_t saved_bytes, void *stream) {
    if (!q || !k || !v || !w_proj || !out) return fail(SLA_ERR_INVALID_ARG, "null tensor pointer");
    if (in_dtype != SLA_BF16) return fail(SLA_ERR_UNSUPPORTED, "the backward pass takes bf16 inputs");
    if (out_dtype != SLA_F32 && out_dtype != SLA_BF16)
        return fail(SLA_ERR_UNSUPPORTED, "output dtype must be F32 or the input dtype");
    if (phi != SLA_PHI_SOFTMAX) return fail(SLA_ERR_UNSUPPORTED, "feature map %d not supported", (int)phi);
    BwdLayout o;
    Layout L;
    int kc, kn;
    sla_status st = bwd_layout(B, H, N, d, block, crit_frac, negl_frac, &o, &L, &kc, &kn);
    if (st != SLA_OK) return st;
    if (!saved) return fail(SLA_ERR_INVALID_ARG, "null saved-state buffer");
    if (saved_bytes < o.total)
        return fail(SLA_ERR_WORKSPACE, "saved-state buffer of %zu bytes is smaller than the %zu required", saved_bytes,
                    o.total);
    if (((uintptr_t)saved & 255) != 0) return fail(SLA_ERR_INVALID_ARG, "saved-state buffer must be 256-byte aligned");
    char *ws = (char *)saved;
    hipStream_t s = (hipStream_t)stream;
    // the labels stay in the buffer (the backward reads them there); a
    // caller's mask_out gets a copy
    st = forward_impl(q, k, v, w_proj, in_dtype, out_dtype, B, H, N, d, block, crit_frac, negl_frac, phi, out, nullptr,
                      ws, L.total, stream, (float *)(ws + o.lse), false, true, (float *)(ws + o.o_s));
    if (st != SLA_OK || !mask_out) return st;
    const size_t mask_bytes = (size_t)B * H * ((N + 63) / 64) * ((N + 63) / 64);
    return device_status(hipMemcpyAsync(mask_out, ws + L.mask, mask_bytes, hipMemcpyDeviceToDevice, s),
                         "mask copy");
}

sla_status sla_backward_saved(const void *q, const void *k, const void *v, const float *w_proj, const void *dout,
                              sla_dtype in_dtype, int B, int H, int N, int d, int block, double crit_frac,
                              double negl_frac, sla_phi phi, float *dq, float *dk, float *dv, float *dw, void *saved,
                              size_t saved_bytes, void *stream) {
    BwdLayout o;
    Layout L;
    int kc, kn;
    sla_status st = backward_checks(q, k, v, w_proj, dout, in_dtype, B, H, N, d, block, crit_frac, negl_frac, phi, dq,
                                    dk, dv, dw, saved, saved_bytes, &o, &L, &kc, &kn);
    if (st != SLA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    StageEvents *ev = timed_call();
    mark_stage(ev, 0, 0, s);                             // no forward stage
    mark_stage(ev, 0, 1, s);
    return backward_grads(q, k, v, w_proj, dout, B, H, N, d, dq, dk, dv, dw, (char *)saved, o, L, kc, kn, s, ev);
}

}  // extern "C"
